// Fused recurrent form for gfx950: the decode step (one token) and the
// multi-token call (T tokens per sequence in one launch).
//
// Per token, the decay, the erase read, the delta write and the read-out of
// the updated state (Gated DeltaNet-2 analysis, iplexlaw.co.kr, "Independent
// decisions on two axes") are fused, and the FP32 state stays in registers
// across the call's tokens: it is streamed from HBM once and written back
// once per call.  alpha is clamped to [2^-15, 1] as in the chunkwise kernels.
// With ae = alpha (.) e and aq = alpha (.) q:
//     r = S^T ae,  s = S^T aq,  u = z - r,  o = s + (k . q) u,
//     S <- Diag(alpha) S + k u^T
// (o = S_new^T q expands to S^T (alpha (.) q) + u (k^T q)).
//
// Work split: one 256-thread workgroup per (sequence, head).  Thread t owns
// four adjacent value columns (one float4) in rows t / (DV/4) + RPP * i, so a
// wavefront reads whole contiguous rows (coalesced dwordx4).  The tile stays
// in VGPRs between the two column reductions and the write-back: no re-read.
// The token vectors go through LDS in two buffers (token parity), and the
// next token's are loaded into registers while the current one is computed.
// There is no matrix work here (0.75 flop per state byte per token), so no
// MFMA.
#include "gdn2_device.hpp"
#include "launch.hpp"

namespace gdn2 {
namespace {

constexpr int kStepThreads = 256;

// One token's inputs as loaded by this thread: key channel c = tid (q, k, b,
// alpha; tid < DK) and value column j = tid (v, w; tid < DV).
struct TokenRegs {
    float q, k, b, a, v, w;
};

template <typename T, int DK, int DV>
__device__ __forceinline__ void load_token(TokenRegs& x, const StepArgs& a, int64_t row, int tid)
{
    // A scalar gate (one value per token and head) is read with stride 0 over
    // its channels; a tied write gate is the scalar erase gate.
    const bool sb = a.gates & kScalarErase, sa = a.gates & kScalarDecay;
    if (tid < DK) {
        x.q = load_as_f32(static_cast<const T*>(a.q), row * DK + tid);
        x.k = load_as_f32(static_cast<const T*>(a.k), row * DK + tid);
        x.b = load_as_f32(static_cast<const T*>(a.b), sb ? row : row * DK + tid);
        x.a = __builtin_amdgcn_fmed3f(a.alpha[sa ? row : row * DK + tid], 0x1p-15f, 1.0f);  // as the chunk kernels
    }
    if (tid < DV) {
        x.v = load_as_f32(static_cast<const T*>(a.v), row * DV + tid);
        x.w = a.gates & kTied         ? load_as_f32(static_cast<const T*>(a.b), row)
              : a.gates & kScalarWrite ? load_as_f32(static_cast<const T*>(a.w), row)
                                       : load_as_f32(static_cast<const T*>(a.w), row * DV + tid);
    }
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(kStepThreads) void recurrent_kernel(StepArgs a)
{
    constexpr int TPR = DV / 4;               // threads per state row
    constexpr int RPP = kStepThreads / TPR;   // rows per pass
    constexpr int NP = DK / RPP;              // float4s per thread
    static_assert(DK % RPP == 0 && NP >= 1, "tile does not divide the state");
    static_assert(TPR <= 64 && 64 % TPR == 0, "row must fit in a wavefront");
    static_assert(DK <= kStepThreads && DV <= kStepThreads, "one thread per channel");

    __shared__ float s_alpha[2][DK], s_ae[2][DK], s_aq[2][DK], s_k[2][DK], s_q[2][DK];
    __shared__ float s_z[2][DV];
    __shared__ float4 s_red[2][kStepThreads / 64][TPR];

    const int head = blockIdx.x;  // n * H + h
    const int tid = threadIdx.x;
    const int col4 = tid % TPR;
    const int row0 = tid / TPR;
    const int wave = tid / 64, lane = tid % 64;
    const int64_t n = head / a.H, h = head % a.H;
    float* S = a.state + int64_t(head) * DK * DV;

    float4 st[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i)
        st[i] = reinterpret_cast<const float4*>(S + int64_t(row0 + RPP * i) * DV)[col4];

    TokenRegs x;
    if (a.T > 0) load_token<T, DK, DV>(x, a, n * a.T * a.H + h, tid);
    for (int t = 0; t < a.T; ++t) {
        const int buf = t & 1;
        const int64_t row = (n * a.T + t) * a.H + h;  // token t of this (sequence, head)
        if (tid < DK) {
            s_alpha[buf][tid] = x.a;
            s_ae[buf][tid] = x.a * (x.b * x.k);
            s_aq[buf][tid] = x.a * x.q;
            s_k[buf][tid] = x.k;
            s_q[buf][tid] = x.q;
        }
        if (tid < DV) s_z[buf][tid] = x.w * x.v;
        if (t + 1 < a.T) load_token<T, DK, DV>(x, a, row + a.H, tid);  // in flight during this token
        __syncthreads();

        // k . q, computed redundantly by every wavefront
        float kq = 0.f;
        for (int c = lane; c < DK; c += 64) kq += s_k[buf][c] * s_q[buf][c];
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) kq += __shfl_xor(kq, off, 64);

        float4 r = make_float4(0.f, 0.f, 0.f, 0.f), s = r;
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int c = row0 + RPP * i;
            const float ae = s_ae[buf][c], aq = s_aq[buf][c];
            r.x += st[i].x * ae; r.y += st[i].y * ae; r.z += st[i].z * ae; r.w += st[i].w * ae;
            s.x += st[i].x * aq; s.y += st[i].y * aq; s.z += st[i].z * aq; s.w += st[i].w * aq;
        }
        // reduce over the row groups inside the wavefront ...
#pragma unroll
        for (int off = TPR; off < 64; off <<= 1) {
            r.x += __shfl_xor(r.x, off, 64); r.y += __shfl_xor(r.y, off, 64);
            r.z += __shfl_xor(r.z, off, 64); r.w += __shfl_xor(r.w, off, 64);
            s.x += __shfl_xor(s.x, off, 64); s.y += __shfl_xor(s.y, off, 64);
            s.z += __shfl_xor(s.z, off, 64); s.w += __shfl_xor(s.w, off, 64);
        }
        // ... and across wavefronts through LDS
        if (lane < TPR) {
            s_red[0][wave][lane] = r;
            s_red[1][wave][lane] = s;
        }
        __syncthreads();
        r = s_red[0][0][col4];
        s = s_red[1][0][col4];
#pragma unroll
        for (int wv = 1; wv < kStepThreads / 64; ++wv) {
            const float4 r2 = s_red[0][wv][col4], s2 = s_red[1][wv][col4];
            r.x += r2.x; r.y += r2.y; r.z += r2.z; r.w += r2.w;
            s.x += s2.x; s.y += s2.y; s.z += s2.z; s.w += s2.w;
        }
        const float* z = s_z[buf] + 4 * col4;
        const float4 u = make_float4(z[0] - r.x, z[1] - r.y, z[2] - r.z, z[3] - r.w);
        if (row0 == 0) {
            T* o = static_cast<T*>(a.o) + row * DV + 4 * col4;
            store_from_f32(o, 0, s.x + kq * u.x);
            store_from_f32(o, 1, s.y + kq * u.y);
            store_from_f32(o, 2, s.z + kq * u.z);
            store_from_f32(o, 3, s.w + kq * u.w);
        }
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int c = row0 + RPP * i;
            const float aa = s_alpha[buf][c], kk = s_k[buf][c];
            st[i].x = aa * st[i].x + kk * u.x;
            st[i].y = aa * st[i].y + kk * u.y;
            st[i].z = aa * st[i].z + kk * u.z;
            st[i].w = aa * st[i].w + kk * u.w;
        }
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) reinterpret_cast<float4*>(S + int64_t(row0 + RPP * i) * DV)[col4] = st[i];
}

template <typename T, int DK, int DV>
hipError_t launch_dkdv(const StepArgs& a, hipStream_t stream)
{
    const int64_t blocks = int64_t(a.N) * a.H;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((recurrent_kernel<T, DK, DV>), dim3(unsigned(blocks)), dim3(kStepThreads),
                       0, stream, a);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_typed(const StepArgs& a, hipStream_t stream)
{
#define GDN2_STEP_CASE(DK_, DV_) \
    if (a.dk == DK_ && a.dv == DV_) return launch_dkdv<T, DK_, DV_>(a, stream);
    GDN2_STEP_CASE(32, 32) GDN2_STEP_CASE(32, 64) GDN2_STEP_CASE(32, 128)
    GDN2_STEP_CASE(64, 32) GDN2_STEP_CASE(64, 64) GDN2_STEP_CASE(64, 128)
    GDN2_STEP_CASE(128, 32) GDN2_STEP_CASE(128, 64) GDN2_STEP_CASE(128, 128)
#undef GDN2_STEP_CASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_recurrent(const StepArgs& a, bool bf16, hipStream_t stream)
{
    return bf16 ? launch_typed<bf16raw>(a, stream) : launch_typed<float>(a, stream);
}

}  // namespace gdn2
