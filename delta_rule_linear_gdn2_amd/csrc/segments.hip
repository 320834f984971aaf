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
// one workgroup takes four columns of one (row, head); thread r computes row
// r of those four columns, with S_in(p) staged in LDS and M_p loaded into LDS
// once per step with coalesced 16-byte loads (rows padded by four floats, so
// that 16 lanes reading 16 rows at one column hit distinct banks).  FP32
// throughout.
#include "gdn2_device.hpp"
#include "launch.hpp"

namespace gdn2 {
namespace {

constexpr int kCombCols = 4;

// out: [B][P][H][dk][dv + dk] final states of segments 0 .. P - 2 (N_p in
// columns < dv, M_p in columns dv .. dv + dk - 1); in: [B][P][H][dk][dv]
// receives S_in(p) for p = 1 .. P - 1.
template <int DK>
__global__ __launch_bounds__(DK) void segment_combine_kernel(const float* __restrict__ out, float* __restrict__ in,
                                                             int H, int dv, int P)
{
    constexpr int kPad = DK + 4;  // floats per LDS row of M
    __shared__ float4 s_state[DK];
    __shared__ __attribute__((aligned(16))) float s_m[DK * kPad];
    const int slices = dv / kCombCols;
    const int blk = blockIdx.x;
    const int slice = blk % slices;
    const int bh = blk / slices;           // b * H + h
    const int64_t b = bh / H, h = bh % H;
    const int r = threadIdx.x;             // state row
    const int c0 = slice * kCombCols;
    const int64_t wout = int64_t(dv) + DK;  // columns of a segment's final state
    const int64_t seg_out = int64_t(H) * DK * wout, seg_in = int64_t(H) * DK * dv;
    const float* o0 = out + (b * P * H + h) * DK * wout;  // segment 0 of this (row, head)
    float* i0 = in + (b * P * H + h) * DK * dv;

    // S_in(1) = S_out(0): the real columns of segment 0's final state
    float4 x = *reinterpret_cast<const float4*>(o0 + r * wout + c0);
    *reinterpret_cast<float4*>(i0 + 1 * seg_in + r * dv + c0) = x;
    for (int p = 1; p + 1 < P; ++p) {
        const float* op = o0 + p * seg_out;
        // M_p into LDS: DK rows of DK floats, DK / 4 threads per row
#pragma unroll 4
        for (int i = r; i < DK * DK / 4; i += DK) {
            const int row = i / (DK / 4), c4 = i % (DK / 4);
            *reinterpret_cast<float4*>(s_m + row * kPad + 4 * c4) =
                *reinterpret_cast<const float4*>(op + row * wout + dv + 4 * c4);
        }
        s_state[r] = x;
        float4 acc = *reinterpret_cast<const float4*>(op + r * wout + c0);  // N_p
        __syncthreads();
        const float* mrow = s_m + r * kPad;  // row r of M_p
#pragma unroll 8
        for (int k = 0; k < DK; k += 4) {
            const float4 m = *reinterpret_cast<const float4*>(mrow + k);
            const float mk[4] = {m.x, m.y, m.z, m.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float4 sv = s_state[k + j];
                acc.x += mk[j] * sv.x;
                acc.y += mk[j] * sv.y;
                acc.z += mk[j] * sv.z;
                acc.w += mk[j] * sv.w;
            }
        }
        __syncthreads();  // every thread has read M_p and S_in(p) before they are replaced
        x = acc;
        *reinterpret_cast<float4*>(i0 + (p + 1) * seg_in + r * dv + c0) = x;
    }
}

}  // namespace

hipError_t launch_segment_combine(const float* seg_out, float* seg_in, int B, int H, int dk, int dv, int P,
                                  hipStream_t stream)
{
    if (dk != 128 || dv % kCombCols != 0 || P < 2) return hipErrorInvalidValue;
    const int64_t blocks = int64_t(B) * H * (dv / kCombCols);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((segment_combine_kernel<128>), dim3(unsigned(blocks)), dim3(128), 0, stream, seg_out, seg_in,
                       H, dv, P);
    return hipGetLastError();
}

}  // namespace gdn2
