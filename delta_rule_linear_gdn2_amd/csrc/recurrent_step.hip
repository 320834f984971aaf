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
// Work split: column j of the state evolves with column j of z, r and s
// alone, so a (sequence, head) splits into independent 32-column quarters.
// One wavefront (a one-wave workgroup) owns one quarter: lane l holds the
// four columns 4 (l & 7) .. + 3 of the rows g NP .. g NP + NP - 1, g = l >> 3,
// NP = dk / 8, in VGPRs.  The column sums over dk are a register sum over the
// lane's NP rows and three lane-exchange steps across the eight row groups
// (on the vector ALU: a DPP rotate and two lane swaps): no workgroup barrier,
// no LDS and no cross-wave exchange, so a wavefront never waits for another.
// The token vectors go through the wave's own LDS (two buffers, token
// parity); the next token's are loaded into registers while the current one
// is computed.  The quarters of one head share blockIdx mod 8, hence one
// XCD, so the token vectors that every quarter reads come from that XCD's L2.
//
// The state is streamed: the loads carry the non-temporal hint and the stores
// the non-temporal and system-scope hints.  On MI355X with 256 sequences x 16
// heads of 128 x 128 FP32 state (268 MB, beyond the 256 MB Infinity Cache),
// that policy measured 95-96 us per step both in place and with the state
// last touched several steps earlier; the default policy took 82 us in place
// (partly served from the cache) but 108 us on a cold state.  A decode loop
// over a model's layers touches every layer's state between two steps of one
// layer, so the cold figure is the one that matters.
//
// There is no matrix work here (0.75 flop per state byte per token), so no
// MFMA.
#include "gdn2_device.hpp"
#include "launch.hpp"

namespace gdn2 {
namespace {

constexpr int kCols = 32;          // value columns per wavefront
constexpr int kAuxLoad = 2;        // buffer cache policy of the state loads: nt
constexpr int kAuxStore = 2 | 16;  // of the state stores: nt, sc1

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}
__device__ __forceinline__ float4 ld_state(rsrc_t r, uint32_t off)
{
    const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, kAuxLoad);
    return make_float4(__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]), __uint_as_float(x[3]));
}
__device__ __forceinline__ void st_state(rsrc_t r, uint32_t off, float4 v)
{
    const u32x4 x = {__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z), __float_as_uint(v.w)};
    __builtin_amdgcn_raw_buffer_store_b128(x, r, int(off), 0, kAuxStore);
}

__device__ __forceinline__ void store_o4(float* o, float4 x) { *reinterpret_cast<float4*>(o) = x; }
__device__ __forceinline__ void store_o4(bf16raw* o, float4 x)
{
    *reinterpret_cast<uint2*>(o) = make_uint2(f32x2_to_bf16x2(x.x, x.y), f32x2_to_bf16x2(x.z, x.w));
}

// One token's inputs as loaded by a lane: key channels lane + 64 i (q, k, b,
// alpha) and value column lane of the quarter (v, w; lanes < 32).  A scalar
// gate (one value per token and head) is read with stride 0 over its
// channels; a tied write gate is the scalar erase gate.
template <int DK>
struct TokenRegs {
    static constexpr int KI = (DK + 63) / 64;
    float q[KI], k[KI], b[KI], a[KI];
    float v, w;
};

template <typename T, int DK, int DV>
__device__ __forceinline__ void load_token(TokenRegs<DK>& x, const StepArgs& a, int64_t row, int col0, int lane)
{
    const bool sb = a.gates & kScalarErase, sa = a.gates & kScalarDecay;
#pragma unroll
    for (int i = 0; i < TokenRegs<DK>::KI; ++i) {
        const int c = lane + 64 * i;
        if (c < DK) {
            x.q[i] = load_as_f32(static_cast<const T*>(a.q), row * DK + c);
            x.k[i] = load_as_f32(static_cast<const T*>(a.k), row * DK + c);
            x.b[i] = load_as_f32(static_cast<const T*>(a.b), sb ? row : row * DK + c);
            x.a[i] = a.alpha[sa ? row : row * DK + c];
        }
    }
    if (lane < kCols) {
        const int64_t j = row * DV + col0 + lane;
        x.v = load_as_f32(static_cast<const T*>(a.v), j);
        x.w = a.gates & kTied         ? load_as_f32(static_cast<const T*>(a.b), row)
              : a.gates & kScalarWrite ? load_as_f32(static_cast<const T*>(a.w), row)
                                       : load_as_f32(static_cast<const T*>(a.w), j);
    }
}

// Cross-lane sums on the vector ALU (no LDS traffic): every lane receives x
// plus the value of lane ^ 8 (DPP rotate by 8 inside each row of 16 lanes),
// lane ^ 16 and lane ^ 32.  A lane-swap instruction given the same register
// twice returns the two halves exchanged; their sum is the pairwise sum in
// every lane.
template <int CTRL>
__device__ __forceinline__ float dpp_row(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;
__device__ __forceinline__ float sum_xor8(float x) { return x + dpp_row<kRowRor8>(x); }
__device__ __forceinline__ float sum_xor16(float x)
{
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor32(float x)
{
    const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
// Sum over the whole wavefront, in every lane.
__device__ __forceinline__ float wave_sum(float x)
{
    x += dpp_row<kRowRor8>(x);
    x += dpp_row<kRowRor4>(x);
    x += dpp_row<kRowRor2>(x);
    x += dpp_row<kRowRor1>(x);
    return sum_xor32(sum_xor16(x));
}
// Sum over the eight row groups (lanes 8 apart), in every lane.
__device__ __forceinline__ float rowgroup_sum(float x) { return sum_xor32(sum_xor16(sum_xor8(x))); }

// The wave's own LDS writes are complete (it is the only wave of its
// workgroup, so no s_barrier); global loads stay in flight.
__device__ __forceinline__ void wave_lds_fence()
{
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
    __asm__ volatile("" ::: "memory");
}

template <typename T, int DK, int DV>
__global__ __launch_bounds__(64) void recurrent_kernel(StepArgs a)
{
    constexpr int NQ = DV / kCols;   // quarters per head
    constexpr int NP = DK / 8;       // rows per lane
    static_assert(DV % kCols == 0 && NP % 4 == 0, "tile does not divide the state");

    __shared__ __attribute__((aligned(16))) float s_al[2][DK], s_ae[2][DK], s_aq[2][DK], s_k[2][DK];
    __shared__ __attribute__((aligned(16))) float s_z[2][kCols];

    // blockIdx -> (head, quarter): the NQ quarters of a head are 8 blocks apart
    const int blk = blockIdx.x;
    const int quarter = (blk % (8 * NQ)) / 8;
    const int64_t head = int64_t(blk / (8 * NQ)) * 8 + (blk & 7);  // n * H + h
    if (head >= int64_t(a.N) * a.H) return;
    const int lane = threadIdx.x;
    const int col4 = lane & 7, g = lane >> 3;
    const int64_t n = head / a.H, h = head % a.H;
    const int col0 = quarter * kCols;
    const int c0 = col0 + 4 * col4;  // this lane's first column

    // token 0's inputs first: they land before the state and are staged while
    // the state is still in flight
    TokenRegs<DK> x;
    if (a.T > 0) load_token<T, DK, DV>(x, a, n * a.T * a.H + h, col0, lane);

    const rsrc_t rs = make_rsrc(a.state + head * DK * DV, DK * DV * 4);
    float4 st[NP];
#pragma unroll
    for (int i = 0; i < NP; ++i) st[i] = ld_state(rs, uint32_t((g * NP + i) * DV + c0) * 4);

    for (int t = 0; t < a.T; ++t) {
        const int buf = t & 1;
        const int64_t row = (n * a.T + t) * a.H + h;  // token t of this (sequence, head)
        float kq = 0.f;
#pragma unroll
        for (int i = 0; i < TokenRegs<DK>::KI; ++i) {
            const int c = lane + 64 * i;
            if (c < DK) {
                const float al = __builtin_amdgcn_fmed3f(x.a[i], 0x1p-15f, 1.0f);
                s_al[buf][c] = al;
                s_ae[buf][c] = al * (x.b[i] * x.k[i]);
                s_aq[buf][c] = al * x.q[i];
                s_k[buf][c] = x.k[i];
                kq += x.k[i] * x.q[i];
            }
        }
        if (lane < kCols) s_z[buf][lane] = x.w * x.v;
        if (t + 1 < a.T) load_token<T, DK, DV>(x, a, row + a.H, col0, lane);  // in flight during this token
        kq = wave_sum(kq);
        wave_lds_fence();

        float4 r = make_float4(0.f, 0.f, 0.f, 0.f), s = r;
#pragma unroll
        for (int i4 = 0; i4 < NP / 4; ++i4) {
            const float4 ae = *reinterpret_cast<const float4*>(&s_ae[buf][g * NP + 4 * i4]);
            const float4 aq = *reinterpret_cast<const float4*>(&s_aq[buf][g * NP + 4 * i4]);
            const float aev[4] = {ae.x, ae.y, ae.z, ae.w}, aqv[4] = {aq.x, aq.y, aq.z, aq.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 y = st[4 * i4 + j];
                r.x += y.x * aev[j]; r.y += y.y * aev[j]; r.z += y.z * aev[j]; r.w += y.w * aev[j];
                s.x += y.x * aqv[j]; s.y += y.y * aqv[j]; s.z += y.z * aqv[j]; s.w += y.w * aqv[j];
            }
        }
        // sum over the eight row groups (lanes 8 apart)
        r = make_float4(rowgroup_sum(r.x), rowgroup_sum(r.y), rowgroup_sum(r.z), rowgroup_sum(r.w));
        s = make_float4(rowgroup_sum(s.x), rowgroup_sum(s.y), rowgroup_sum(s.z), rowgroup_sum(s.w));
        const float4 z = *reinterpret_cast<const float4*>(&s_z[buf][4 * col4]);
        const float4 u = make_float4(z.x - r.x, z.y - r.y, z.z - r.z, z.w - r.w);
        if (g == 0)
            store_o4(static_cast<T*>(a.o) + row * DV + c0,
                     make_float4(s.x + kq * u.x, s.y + kq * u.y, s.z + kq * u.z, s.w + kq * u.w));
#pragma unroll
        for (int i4 = 0; i4 < NP / 4; ++i4) {
            const float4 al = *reinterpret_cast<const float4*>(&s_al[buf][g * NP + 4 * i4]);
            const float4 kk = *reinterpret_cast<const float4*>(&s_k[buf][g * NP + 4 * i4]);
            const float alv[4] = {al.x, al.y, al.z, al.w}, kv[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                float4& y = st[4 * i4 + j];
                y.x = alv[j] * y.x + kv[j] * u.x;
                y.y = alv[j] * y.y + kv[j] * u.y;
                y.z = alv[j] * y.z + kv[j] * u.z;
                y.w = alv[j] * y.w + kv[j] * u.w;
            }
        }
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) st_state(rs, uint32_t((g * NP + i) * DV + c0) * 4, st[i]);
}

template <typename T, int DK, int DV>
hipError_t launch_dkdv(const StepArgs& a, hipStream_t stream)
{
    constexpr int NQ = DV / kCols;
    const int64_t heads = int64_t(a.N) * a.H;
    const int64_t blocks = (heads + 7) / 8 * 8 * NQ;  // padded to whole groups of eight heads
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((recurrent_kernel<T, DK, DV>), dim3(unsigned(blocks)), dim3(64), 0, stream, a);
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
