// Fused recurrent decode step for gfx950.
//
// One token per (sequence, head): the decay, the erase read, the delta write
// and the read-out of the updated state (Gated DeltaNet-2 analysis,
// iplexlaw.co.kr, "Independent decisions on two axes") fused so that the FP32
// state is streamed from HBM once and written back once.  With
// ae = alpha (.) e and aq = alpha (.) q:
//     r = S^T ae,  s = S^T aq,  u = z - r,  o = s + (k . q) u,
//     S <- Diag(alpha) S + k u^T
// (o = S_new^T q expands to S^T (alpha (.) q) + u (k^T q)).
//
// Work split: one 256-thread workgroup per (sequence, head).  Thread t owns
// four adjacent value columns (one float4) in rows t / (DV/4) + RPP * i, so a
// wavefront reads whole contiguous rows (coalesced dwordx4).  The tile stays
// in VGPRs between the two column reductions and the write-back: no re-read.
// There is no matrix work here (0.75 flop per byte), so no MFMA.
#include "gdn2_device.hpp"
#include "launch.hpp"

namespace gdn2 {
namespace {

constexpr int kStepThreads = 256;

template <typename T, int DK, int DV>
__global__ __launch_bounds__(kStepThreads) void recurrent_step_kernel(StepArgs a)
{
    constexpr int TPR = DV / 4;               // threads per state row
    constexpr int RPP = kStepThreads / TPR;   // rows per pass
    constexpr int NP = DK / RPP;              // float4s per thread
    static_assert(DK % RPP == 0 && NP >= 1, "tile does not divide the state");
    static_assert(TPR <= 64 && 64 % TPR == 0, "row must fit in a wavefront");

    __shared__ float s_alpha[DK], s_ae[DK], s_aq[DK], s_k[DK], s_q[DK];
    __shared__ float s_z[DV];
    __shared__ float4 s_red[2][kStepThreads / 64][TPR];

    const int head = blockIdx.x;  // n * H + h
    const int tid = threadIdx.x;
    const int col4 = tid % TPR;
    const int row0 = tid / TPR;
    float* S = a.state + int64_t(head) * DK * DV;

    float4 st[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i)
        st[i] = reinterpret_cast<const float4*>(S + int64_t(row0 + RPP * i) * DV)[col4];

    const T* q = static_cast<const T*>(a.q) + int64_t(head) * DK;
    const T* k = static_cast<const T*>(a.k) + int64_t(head) * DK;
    // A scalar gate (one value per head) is read with stride 0 over its
    // channels; a tied write gate is the scalar erase gate.
    const int bst = a.gates & kScalarErase ? 0 : 1, ast = a.gates & kScalarDecay ? 0 : 1;
    const int wst = a.gates & (kScalarWrite | kTied) ? 0 : 1;
    const T* b = static_cast<const T*>(a.b) + int64_t(head) * (bst ? DK : 1);
    const T* v = static_cast<const T*>(a.v) + int64_t(head) * DV;
    const T* w = a.gates & kTied ? b : static_cast<const T*>(a.w) + int64_t(head) * (wst ? DV : 1);
    const float* al = a.alpha + int64_t(head) * (ast ? DK : 1);
    for (int c = tid; c < DK; c += kStepThreads) {
        const float kk = load_as_f32(k, c), qq = load_as_f32(q, c), aa = al[c * ast];
        s_alpha[c] = aa;
        s_ae[c] = aa * (load_as_f32(b, c * bst) * kk);
        s_aq[c] = aa * qq;
        s_k[c] = kk;
        s_q[c] = qq;
    }
    for (int j = tid; j < DV; j += kStepThreads) s_z[j] = load_as_f32(w, j * wst) * load_as_f32(v, j);
    __syncthreads();

    // k . q, computed redundantly by every wavefront
    float kq = 0.f;
    for (int c = tid % 64; c < DK; c += 64) kq += s_k[c] * s_q[c];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) kq += __shfl_xor(kq, off, 64);

    float4 r = make_float4(0.f, 0.f, 0.f, 0.f), s = r;
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int row = row0 + RPP * i;
        const float ae = s_ae[row], aq = s_aq[row];
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
    const int wave = tid / 64, lane = tid % 64;
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
    const float4 u = make_float4(s_z[4 * col4 + 0] - r.x, s_z[4 * col4 + 1] - r.y,
                                 s_z[4 * col4 + 2] - r.z, s_z[4 * col4 + 3] - r.w);
    if (row0 == 0) {
        T* o = static_cast<T*>(a.o) + int64_t(head) * DV + 4 * col4;
        store_from_f32(o, 0, s.x + kq * u.x);
        store_from_f32(o, 1, s.y + kq * u.y);
        store_from_f32(o, 2, s.z + kq * u.z);
        store_from_f32(o, 3, s.w + kq * u.w);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
        const int row = row0 + RPP * i;
        const float aa = s_alpha[row], kk = s_k[row];
        float4 x;
        x.x = aa * st[i].x + kk * u.x;
        x.y = aa * st[i].y + kk * u.y;
        x.z = aa * st[i].z + kk * u.z;
        x.w = aa * st[i].w + kk * u.w;
        reinterpret_cast<float4*>(S + int64_t(row) * DV)[col4] = x;
    }
}

template <typename T, int DK, int DV>
hipError_t launch_dkdv(const StepArgs& a, hipStream_t stream)
{
    const int64_t blocks = int64_t(a.N) * a.H;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((recurrent_step_kernel<T, DK, DV>), dim3(unsigned(blocks)), dim3(kStepThreads),
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

hipError_t launch_recurrent_step(const StepArgs& a, bool bf16, hipStream_t stream)
{
    return bf16 ? launch_typed<bf16raw>(a, stream) : launch_typed<float>(a, stream);
}

}  // namespace gdn2
