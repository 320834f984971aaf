// Sequence segments for few-chain chunkwise calls: the combine step.
//
// The recurrence of one (sequence, head) is affine in its incoming state:
// over a segment of tokens, S_out = M S_in + N, where M (dk x dk) is what the
// segment does to a state (its per-token decays and erase corrections
// composed) and N is the segment run from a zero state.  This is the same
// fact that lets the chunkwise form hand its state from chunk to chunk
// (Gated DeltaNet-2 analysis, iplexlaw.co.kr, "Token processing and parallel
// training"), applied to runs of chunks.  The chunk kernel computes N and M
// of every segment but the last in one launch (M as extra value columns that
// start from the identity with z = 0).  This kernel then forms the true
// incoming state of every later segment in order:
//     S_in(1) = S_out(0),   S_in(p + 1) = M_p S_in(p) + N_p,
// and a second chunk-kernel launch re-runs segments 1 .. P - 1 from them.
//
// Work split: the columns of S evolve independently (M acts on the rows), so
// one workgroup of 256 threads takes eight columns of one (row, head):
// thread (r, g) computes row r of columns 4 g .. 4 g + 3, with S_in(p) and M_p
// staged in LDS (rows of M padded by four floats, so that 16 lanes reading 16
// rows at one column hit distinct banks).  The steps are latency-bound, so
// the loads of M_(p+1) and N_p are issued before step p's products and land
// while they run; each M_p then costs one LDS store per thread, not a round
// trip to memory per row.  FP32 throughout.
#include "gdn2_device.hpp"
#include "launch.hpp"

namespace gdn2 {
namespace {

constexpr int kCombDK = 128;
constexpr int kCombCols = 8;                       // columns per workgroup
constexpr int kCombThreads = kCombDK * kCombCols / 4;  // one row of four columns per thread
constexpr int kCombPad = kCombDK + 4;              // floats per LDS row of M
constexpr int kCombLoads = kCombDK * kCombDK / 4 / kCombThreads;  // float4 loads of M per thread
constexpr int kCombLds = (kCombDK * kCombPad + kCombDK * kCombCols) * 4;

// Workgroup barrier for LDS traffic only: waits for this wave's LDS accesses
// (lgkmcnt = 0), not for its global loads, so the prefetch of the next map
// stays in flight across it (a full __syncthreads() fence would drain it).
__device__ __forceinline__ void comb_barrier()
{
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// One thread's share of a map M (kCombLoads float4 of the 4096 in a 128 x
// 128 map): float4 i = tid + kCombThreads j, row i / 32, columns 4 (i % 32)
// .. + 3, so consecutive threads read consecutive 16 bytes of a row.  Held as
// a native vector type: HIP's float4, whose copies lower to memory copies,
// would keep the registers in scratch.
typedef float comb_f4 __attribute__((ext_vector_type(4)));
struct CombRegs {
    comb_f4 v[kCombLoads];
};
__device__ __forceinline__ int comb_src(int tid, int j, int64_t wout)
{
    const int i = tid + kCombThreads * j;
    return int((i / (kCombDK / 4)) * wout + 4 * (i % (kCombDK / 4)));
}
__device__ __forceinline__ int comb_dst(int tid, int j)
{
    const int i = tid + kCombThreads * j;
    return (i / (kCombDK / 4)) * kCombPad + 4 * (i % (kCombDK / 4));
}
__device__ __forceinline__ void comb_load(CombRegs& m, const float* mp, int tid, int64_t wout)
{
    const comb_f4* f = reinterpret_cast<const comb_f4*>(mp);
#pragma unroll
    for (int j = 0; j < kCombLoads; ++j) m.v[j] = f[comb_src(tid, j, wout) / 4];
}
__device__ __forceinline__ void comb_store(float* s_m, const CombRegs& m, int tid)
{
    comb_f4* f = reinterpret_cast<comb_f4*>(s_m);
#pragma unroll
    for (int j = 0; j < kCombLoads; ++j) f[comb_dst(tid, j) / 4] = m.v[j];
}
static_assert(kCombLoads * kCombThreads * 4 == kCombDK * kCombDK, "every element of M loaded once");

// out: [B][P][H][dk][dv + dk] final states of segments 0 .. P - 2 (N_p in
// columns < dv, M_p in columns dv .. dv + dk - 1); in: [B][P][H][dk][dv]
// receives S_in(p) for p = 1 .. P - 1.
__global__ __launch_bounds__(kCombThreads) void segment_combine_kernel(const float* __restrict__ out,
                                                                       float* __restrict__ in, int B, int H, int dv,
                                                                       int P)
{
    constexpr int DK = kCombDK;
    extern __shared__ __align__(16) unsigned char comb_lds[];
    float* s_m = reinterpret_cast<float*>(comb_lds);                          // [DK][kCombPad]
    float4* s_state = reinterpret_cast<float4*>(comb_lds + DK * kCombPad * 4);  // [DK][kCombCols / 4]
    // XCD-aware mapping: the column slices of one (row, head) share blockIdx
    // mod 8, hence an XCD, so its maps come from HBM once and from that XCD's
    // L2 for the other slices
    const int slices = dv / kCombCols;
    const int blk = blockIdx.x;
    const int xcd = blk & 7, slot = blk >> 3;
    const int slice = slot % slices;
    const int bh = (slot / slices) * 8 + xcd;  // b * H + h
    if (bh >= B * H) return;
    const int64_t b = bh / H, h = bh % H;
    const int tid = threadIdx.x;
    const int r = tid % DK, g = tid / DK;  // state row, group of four columns
    const int c0 = slice * kCombCols + 4 * g;
    const int64_t wout = int64_t(dv) + DK;  // columns of a segment's final state
    const int64_t seg_out = int64_t(H) * DK * wout, seg_in = int64_t(H) * DK * dv;
    const float* o0 = out + (b * P * H + h) * DK * wout;  // segment 0 of this (row, head)
    float* i0 = in + (b * P * H + h) * DK * dv;

    const float* mbase = o0 + dv;  // M_0; M_p at mbase + p * seg_out
    // S_in(1) = S_out(0): the real columns of segment 0's final state
    float4 x = *reinterpret_cast<const float4*>(o0 + r * wout + c0);
    *reinterpret_cast<float4*>(i0 + 1 * seg_in + r * dv + c0) = x;
    if (P > 2) {  // M_1 and S_in(1) into LDS
        CombRegs m1;
        comb_load(m1, mbase + seg_out, tid, wout);
        comb_store(s_m, m1, tid);
        s_state[r * (kCombCols / 4) + g] = x;
    }
    for (int p = 1; p + 1 < P; ++p) {  // LDS holds M_p and S_in(p)
        const float* op = o0 + p * seg_out;
        const float4 np = *reinterpret_cast<const float4*>(op + r * wout + c0);  // N_p, added after the products
        const bool more = p + 2 < P;
        CombRegs mn;  // M_(p+1), in flight during this step's products
        if (more) comb_load(mn, mbase + (p + 1) * seg_out, tid, wout);
        comb_barrier();
        const float* mrow = s_m + r * kCombPad;  // row r of M_p
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
        for (int k = 0; k < DK; k += 4) {
            const float4 m = *reinterpret_cast<const float4*>(mrow + k);
            const float4 s0 = s_state[(k + 0) * (kCombCols / 4) + g], s1 = s_state[(k + 1) * (kCombCols / 4) + g];
            const float4 s2 = s_state[(k + 2) * (kCombCols / 4) + g], s3 = s_state[(k + 3) * (kCombCols / 4) + g];
            acc.x += m.x * s0.x + m.y * s1.x + m.z * s2.x + m.w * s3.x;
            acc.y += m.x * s0.y + m.y * s1.y + m.z * s2.y + m.w * s3.y;
            acc.z += m.x * s0.z + m.y * s1.z + m.z * s2.z + m.w * s3.z;
            acc.w += m.x * s0.w + m.y * s1.w + m.z * s2.w + m.w * s3.w;
        }
        comb_barrier();  // every thread has read M_p and S_in(p) before they are replaced
        x = make_float4(acc.x + np.x, acc.y + np.y, acc.z + np.z, acc.w + np.w);
        *reinterpret_cast<float4*>(i0 + (p + 1) * seg_in + r * dv + c0) = x;
        if (more) {
            comb_store(s_m, mn, tid);
            s_state[r * (kCombCols / 4) + g] = x;
        }
    }
}

}  // namespace

hipError_t launch_segment_combine(const float* seg_out, float* seg_in, int B, int H, int dk, int dv, int P,
                                  hipStream_t stream)
{
    if (dk != kCombDK || dv % kCombCols != 0 || P < 2) return hipErrorInvalidValue;
    // Allow the kernel its > 64 KiB of dynamic LDS (thread-safe one-time call).
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(segment_combine_kernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kCombLds);
    if (attr != hipSuccess) return attr;
    const int64_t blocks = (int64_t(B) * H + 7) / 8 * 8 * (dv / kCombCols);  // whole groups of eight (row, head)
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(segment_combine_kernel, dim3(unsigned(blocks)), dim3(kCombThreads), kCombLds, stream, seg_out,
                       seg_in, B, H, dv, P);
    return hipGetLastError();
}

}  // namespace gdn2
