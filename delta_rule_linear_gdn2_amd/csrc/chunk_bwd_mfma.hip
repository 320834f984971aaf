// Chunkwise backward pass on gfx950 matrix cores (bf16 inputs, dk = dv = 128,
// 64-token chunks).
//
// The gate-aware backward of the Gated DeltaNet-2 analysis (iplexlaw.co.kr,
// "Token processing and parallel training"): the channel-wise decay and the
// erase gate stay inside the sums.  Per chunk of L tokens with incoming state
// S, outgoing-state gradient dS' and, per key channel, G_i = sum_{m<=i}
// log2 alpha_m:
//   Et = e 2^G,  Qt = q 2^G,  Kd = k 2^-G,  Kb = k 2^(G_L - G)   (e = b k)
//   A = strict_lower(Et Kd^T),  P = lower(Qt Kd^T)
//   X = Z - Et S,  U = (I + A)^-1 X,  S' = 2^G_L S + Kb^T U          (forward)
//   dU = Kb dS' + P^T dO,  dX = (I + A)^-T dU,  dZ = dX
//   dS = 2^G_L dS' + Qt^T dO - Et^T dX                              (into the chunk before)
//   dA = -strict_lower(dX U^T),  dP = lower(dO U^T)
//   dEt = -dX S^T,  dQt = dO S^T,  dKb = U dS'^T
// and through the factors, per channel:
//   de = 2^G (dA Kd + dEt),  dq = 2^G (dP Kd + dQt)
//   dk = 2^-G (dA^T Et + dP^T Qt) + 2^(G_L - G) dKb + b de,  db = k de
//   dg = e 2^G (dA Kd) + q 2^G (dP Kd) - k 2^-G (dA^T Et + dP^T Qt)
//        + Et dEt + Qt dQt - Kb dKb,    dg_L += sum_j Kb_j dKb_j + 2^G_L rowsum(dS' . S)
//   dlog(alpha_m) = sum_{i>=m} dg_i,  dalpha = dlog(alpha) / alpha,  dv = dX w,  dw = dX v.
// Splitting the pairwise factor 2^(G_i - G_j) = 2^G_i 2^-G_j turns the
// pairwise sums into matrix products; it stays inside the FP32 and bf16 range
// while every channel decays by at least 2^-64 over the chunk.  The first
// kernel checks that for every chunk and raises a flag otherwise; the two
// later kernels then do nothing and the FP32 backward (chunk_bwd.hip, exact
// pairwise factors) runs instead, on the same workspace.
//
// Three kernels (products v_mfma_f32_16x16x32_bf16 and _16x16x16 with FP32
// accumulation; the diagonal blocks of (I + A)^-1 in FP32 with
// v_mfma_f32_16x16x4_f32):
//   bwd_fstate  (chain x 64-column value tile, chunks in order)    S of every
//               chunk start and the U rows, both bf16, into the workspace;
//   bwd_bstate  (chain x value tile, chunks in reverse)            dS' of every
//               chunk end and the dX rows (bf16) into the workspace; dv, dw, dS0;
//   bwd_grads   (chunk x head, all parallel)                      dq, dk, db, dalpha.
// The sequential kernels run eight wavefronts: four value waves (16 value
// columns each, the FP32 state slice in accumulators) and four key waves that
// prepare the next chunk (decay scan, factor tiles, A and P, the inverses of
// the diagonal blocks of I + A) while the value waves work, two barriers per
// chunk.  The key waves take one token per lane, so the running decay is a
// wavefront prefix sum.
#include "gdn2_device.hpp"
#include "launch.hpp"

namespace gdn2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 64;          // tokens per chunk
constexpr int kD = 128;         // key and value head size
constexpr int kTileV = 64;      // value columns per workgroup of the sequential kernels
constexpr int kThreads = 512;   // eight wavefronts
constexpr float kRangeLog2 = -64.f;  // smallest decay over a chunk (log2) the split factors take

__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(uint2 a, uint2 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
}
__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ float pow2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ bf16x8 as8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ uint32_t pk2(float a, float b) { return f32x2_to_bf16x2(a, b); }
// B operand of a 32-deep K step from two accumulator blocks: rows 4g..4g+3
// of each, so the K indices of lane group g are {4g..4g+3} and {16+4g..+3}.
__device__ __forceinline__ bf16x8 pk_pair(f32x4 lo, f32x4 hi)
{
    return as8(make_uint4(pk2(lo[0], lo[1]), pk2(lo[2], lo[3]), pk2(hi[0], hi[1]), pk2(hi[2], hi[3])));
}
// B operand of a 16-deep K step from one accumulator block.
__device__ __forceinline__ uint2 pk_blk(f32x4 v) { return make_uint2(pk2(v[0], v[1]), pk2(v[2], v[3])); }
__device__ __forceinline__ float lo_f(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float hi_f(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// ---- LDS tiles ---------------------------------------------------------------
// bf16 tiles of RB-byte rows; the 16-byte granules of a row are XOR-swizzled by
// the row's low bits, so 16 rows read at one granule column fall in distinct
// banks.
template <int RB>
__device__ __forceinline__ int toff(int row, int e)
{
    constexpr int NG = RB / 16;
    const int byte = 2 * e;
    return row * RB + ((((byte >> 4) ^ row) & (NG - 1)) << 4) + (byte & 15);
}
template <typename V>
__device__ __forceinline__ V ldsr(const unsigned char* s, int off)
{
    return *reinterpret_cast<const V*>(s + off);
}
template <typename V>
__device__ __forceinline__ void ldsw(unsigned char* s, int off, V v)
{
    *reinterpret_cast<V*>(s + off) = v;
}
// Operand row `row` of a tile at `base`, K step ks (32 deep), lane group g:
// elements 32 ks + 8 g .. + 7 (both operands from LDS) ...
template <int RB>
__device__ __forceinline__ bf16x8 op_nat(const unsigned char* s, int base, int row, int ks, int g)
{
    return as8(ldsr<uint4>(s, base + toff<RB>(row, 32 * ks + 8 * g)));
}
// ... or 32 ks + 4 g .. + 3 and 32 ks + 16 + 4 g .. + 3 (the partner of an
// accumulator-sourced operand, see pk_pair).
template <int RB>
__device__ __forceinline__ bf16x8 op_split(const unsigned char* s, int base, int row, int ks, int g)
{
    const uint2 lo = ldsr<uint2>(s, base + toff<RB>(row, 32 * ks + 4 * g));
    const uint2 hi = ldsr<uint2>(s, base + toff<RB>(row, 32 * ks + 16 + 4 * g));
    return as8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// 16 x 16 FP32 blocks (diagonal blocks of A and their inverses), rows padded.
constexpr int kTRow = 17;
constexpr int kTBlk = 16 * kTRow * 4;  // bytes per block
__device__ __forceinline__ int tb_off(int m, int i, int j) { return m * kTBlk + (i * kTRow + j) * 4; }

// The FP32 products of the solves take their B operand straight from the
// accumulators of the bf16 products that formed it.  On gfx950 the wait the
// compiler puts between the two was too short after v_mfma_f32_16x16x16_bf16
// (tests showed stale rows), so y passes through an explicit wait first; y is
// an operand of the statement, so the products cannot move above it.
__device__ __forceinline__ void mfma_src_wait(f32x4& y)
{
    __asm__ volatile("s_nop 7\n\ts_nop 7" : "+v"(y));
}

// A wave waits for its own LDS accesses (before it reads what its lanes wrote).
__device__ __forceinline__ void wave_lds_fence()
{
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
    __builtin_amdgcn_wave_barrier();
    __asm__ volatile("" ::: "memory");
}
// Workgroup barrier that waits for LDS accesses only: global loads issued for
// the next chunk stay in flight.
__device__ __forceinline__ void lds_sync()
{
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// Inclusive prefix sum over the 64 lanes: rows of 16 lanes by DPP shifts
// (lanes shifted in from outside the row read 0), then the row totals.
template <int N>
__device__ __forceinline__ float row_shr(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xF, 0xF, true));
}
__device__ __forceinline__ float readlane_f(float x, int l)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}
__device__ __forceinline__ float wave_scan(float x, int lane)
{
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x += row_shr<8>(x);
    const float t0 = readlane_f(x, 15), t1 = readlane_f(x, 31), t2 = readlane_f(x, 47);
    const int rw = lane >> 4;
    return x + ((rw >= 1 ? t0 : 0.f) + (rw >= 2 ? t1 : 0.f) + (rw >= 3 ? t2 : 0.f));
}

// Inclusive suffix sum over the 64 lanes (lane l gets the sum over lanes >= l).
template <int N>
__device__ __forceinline__ float row_shl(float x)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 + N, 0xF, 0xF, true));
}
__device__ __forceinline__ float wave_rscan(float x, int lane)
{
    x += row_shl<1>(x);
    x += row_shl<2>(x);
    x += row_shl<4>(x);
    x += row_shl<8>(x);
    const float t1 = readlane_f(x, 16), t2 = readlane_f(x, 32), t3 = readlane_f(x, 48);
    const int rw = lane >> 4;
    return x + ((rw <= 2 ? t3 : 0.f) + (rw <= 1 ? t2 : 0.f) + (rw <= 0 ? t1 : 0.f));
}

// XCD-aware block order: the two value tiles of a chain get the same blockIdx
// mod 8, so they run on one XCD and share its L2.
__device__ __forceinline__ void xcd_pair(int64_t bid, int64_t& group, int& member)
{
    const int64_t q = bid >> 3;
    member = int(q & 1);
    group = (q >> 1) * 8 + (bid & 7);
}
inline int64_t xcd_pair_grid(int64_t groups) { return (groups + 7) / 8 * 16; }

// Workspace tile index of chunk m of sequence n (its 64-token slot).
__device__ __forceinline__ int64_t tile64(const BwdArgs& a, int n, int64_t bos, int m)
{
    return a.cu_seqlens ? (bos + int64_t(m) * kC) / kC + n : int64_t(n) * a.slots64 + m;
}

// ---- the key-side preparation (one token per lane) ---------------------------
// One token's key-side inputs for NC channels starting at c0.
template <int NC>
struct KeyIn {
    float al[NC];
    uint32_t k[NC / 2], b[NC / 2], q[NC / 2];
};

template <int NC, bool WQ>
__device__ __forceinline__ void load_keys(KeyIn<NC>& x, const BwdArgs& a, int64_t off, bool valid)
{
    if (valid) {
        const float* al = a.alpha + off;
        const bf16raw* kp = static_cast<const bf16raw*>(a.k) + off;
        const bf16raw* bp = static_cast<const bf16raw*>(a.b) + off;
        const bf16raw* qp = static_cast<const bf16raw*>(a.q) + off;
#pragma unroll
        for (int j = 0; j < NC / 4; ++j) *reinterpret_cast<float4*>(&x.al[4 * j]) = reinterpret_cast<const float4*>(al)[j];
#pragma unroll
        for (int j = 0; j < NC / 8; ++j) {
            *reinterpret_cast<uint4*>(&x.k[4 * j]) = reinterpret_cast<const uint4*>(kp)[j];
            *reinterpret_cast<uint4*>(&x.b[4 * j]) = reinterpret_cast<const uint4*>(bp)[j];
            if (WQ) *reinterpret_cast<uint4*>(&x.q[4 * j]) = reinterpret_cast<const uint4*>(qp)[j];
        }
    } else {
#pragma unroll
        for (int c = 0; c < NC; ++c) x.al[c] = 1.f;
#pragma unroll
        for (int c = 0; c < NC / 2; ++c) x.k[c] = x.b[c] = x.q[c] = 0u;
    }
}
template <int NC>
__device__ __forceinline__ float kv(const uint32_t* w, int c)
{
    return (c & 1) ? hi_f(w[c >> 1]) : lo_f(w[c >> 1]);
}

// Running log2 decay G of the lane's token for each channel, its value at the
// chunk's last token (lane 63; padding tokens have alpha = 1), and whether
// every channel stays in the split range.
template <int NC>
__device__ __forceinline__ bool decay_scan(const KeyIn<NC>& x, int lane, float* G, float* GL)
{
    bool ok = true;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
        G[c] = wave_scan(log2_decay(x.al[c]), lane);
        GL[c] = readlane_f(G[c], 63);
        ok = ok && GL[c] >= kRangeLog2;
    }
    return ok;
}

// T = (I + L)^-1 for a strictly lower 16 x 16 FP32 block L on the FP32
// matrix cores: L is nilpotent (L^16 = 0), so
//     (I + L)^-1 = (I - L)(I + L^2)(I + L^4)(I + L^8).
// An accumulator block holding a matrix P (lane rows 4g..4g+3, column r)
// serves as the A operand of P^T (K index 4g + s in step s) and as the B
// operand of P, so mm(P, Q) = P^T Q needs no data movement; the chain keeps L
// and L^T (both read from the block's FP32 copy at ad, rows padded) and works
// on T^T.  Each product reads accumulators of the one before: the explicit
// wait covers that on gfx950.  Lanes write T (rows i, columns j) at t.
__device__ __forceinline__ f32x4 mm(f32x4 p, f32x4 q)
{
    mfma_src_wait(p);
    mfma_src_wait(q);
    f32x4 d = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s) d = mma4(p[s], q[s], d);
    return d;
}
__device__ __forceinline__ void diag_inverse(unsigned char* lds, int ad, int t, int g, int r)
{
    f32x4 L, LT;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        L[e] = ldsr<float>(lds, ad + ((4 * g + e) * kTRow + r) * 4);   // L[4g + e][r]
        LT[e] = ldsr<float>(lds, ad + (r * kTRow + 4 * g + e) * 4);   // L^T[4g + e][r]
    }
    const f32x4 L2 = mm(LT, L), L2T = mm(L, LT);
    const f32x4 L4 = mm(L2T, L2), L4T = mm(L2, L2T);
    const f32x4 L8 = mm(L4T, L4);
    f32x4 M = -LT;  // (I - L)^T
#pragma unroll
    for (int e = 0; e < 4; ++e) M[e] += (4 * g + e == r) ? 1.f : 0.f;
    M += mm(L2, M);
    M += mm(L4, M);
    M += mm(L8, M);  // T^T: lane holds T[r][4g + e]
#pragma unroll
    for (int e = 0; e < 4; ++e) ldsw<float>(lds, t + (r * kTRow + 4 * g + e) * 4, M[e]);
}

// Stage an accumulator tile set (NB blocks of 16 rows x 16 columns, lane rows
// 4g..4g+3 of column r) as bf16 through the wave's LDS region (48-byte rows)
// and store it as 16-byte row pieces: dst + row * stride.
template <int NB>
__device__ __forceinline__ void stage_store(unsigned char* lds, int stg, const f32x4* blk, int g, int r, int lane,
                                            bf16raw* dst, int64_t stride)
{
#pragma unroll
    for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) ldsw<bf16raw>(lds, stg + (16 * b + 4 * g + e) * 48 + 2 * r, f32_to_bf16(blk[b][e]));
    wave_lds_fence();
#pragma unroll
    for (int it = 0; it < NB / 2; ++it) {
        const int p = lane + 64 * it, row = p >> 1, half = p & 1;
        const uint4 v = ldsr<uint4>(lds, stg + row * 48 + 16 * half);
        *reinterpret_cast<uint4*>(dst + row * stride + 8 * half) = v;
    }
    wave_lds_fence();
}

// =============================================================================
// bwd_fstate: the forward state pass.
// LDS map (bytes).
constexpr int kF_E = 0;                      // [2][64][128] bf16 Et (chunk in work, chunk in preparation)
constexpr int kF_KD = 32768;                 // [64][128] bf16 Kd (preparation)
constexpr int kF_KBT = 49152;                // [128][64] bf16 Kb^T
constexpr int kF_AN = 65536;                 // [64][64] bf16 -A (rows i), blocks below the diagonal
constexpr int kF_T = 73728;                  // [4] FP32 blocks T_m = (I + A_mm)^-1
constexpr int kF_AD = kF_T + 4 * kTBlk;      // [4] FP32 blocks A_mm (preparation)
constexpr int kF_GL = kF_AD + 4 * kTBlk;     // [2][128] f32 2^G_L (chunk in work, chunk in preparation)
constexpr int kF_Z = kF_GL + 1024;           // [4 value waves][16 columns][64 tokens] f32, z = w v
constexpr int kF_STG = kF_Z + 4 * 4096;      // [4 value waves][128][48 B] staging
constexpr int kF_Bytes = kF_STG + 4 * 128 * 48;
static_assert(kF_Bytes <= 160 * 1024, "LDS budget");

__device__ __forceinline__ int zoff(int col, int tok)
{
    return col * 256 + ((((tok >> 2) ^ col) & 15) << 4) + ((tok & 3) << 2);
}

// Key waves, first half of the preparation of chunk c: the decay scan, the
// tiles Et and Kd (rows = tokens), and Kb kept in registers for later.
struct FPrep {
    KeyIn<32> in;
    uint32_t kb[16];  // Kb of the lane's token, 32 channels, bf16 pairs
};

__global__ __launch_bounds__(kThreads) void bwd_fstate_kernel(BwdArgs a)
{
    extern __shared__ __align__(16) unsigned char lds[];
    int64_t chain;
    int tile;
    xcd_pair(blockIdx.x, chain, tile);
    if (chain >= int64_t(a.N) * a.H) return;
    const int n = int(chain / a.H), h = int(chain % a.H);
    int64_t bos, eos, brow;
    sequence_bounds(a.cu_seqlens, n, a.T, bos, eos, brow);
    const int nch = int((eos - bos + kC - 1) / kC);
    if (nch == 0) return;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const bool value = wave < 4;
    const int64_t rowbase = brow * a.T + bos;  // token row of the sequence's first token
    const bf16raw* vp = static_cast<const bf16raw*>(a.v);
    const bf16raw* wp = static_cast<const bf16raw*>(a.w);

    if (value) {
        // ---- value waves: 16 columns each ----
        const int col0 = tile * kTileV + wave * 16;
        const int zw = kF_Z + wave * 4096, stg = kF_STG + wave * 128 * 48;
        f32x4 S[8];
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[cb][e] = a.initial_state
                               ? a.initial_state[((int64_t(n) * a.H + h) * kD + 16 * cb + 4 * g + e) * kD + col0 + r]
                               : 0.f;
        // z = w v of the chunk's tokens, lane = token, 16 columns
        uint4 zv[2], zw4[2];
        auto load_z = [&](int c) {
            const int64_t t = int64_t(c) * kC + lane;
            if (t < eos - bos) {
                const int64_t off = ((rowbase + t) * a.H + h) * kD + col0;
                zv[0] = *reinterpret_cast<const uint4*>(vp + off);
                zv[1] = *reinterpret_cast<const uint4*>(vp + off + 8);
                zw4[0] = *reinterpret_cast<const uint4*>(wp + off);
                zw4[1] = *reinterpret_cast<const uint4*>(wp + off + 8);
            } else {
                zv[0] = zv[1] = zw4[0] = zw4[1] = make_uint4(0, 0, 0, 0);
            }
        };
        load_z(0);
        lds_sync();  // preparation of chunk 0, first half
        lds_sync();  // second half
        for (int c = 0; c < nch; ++c) {
            // z of this chunk into LDS ([column][token], FP32), then the next chunk's loads
            {
                const uint32_t vv[8] = {zv[0].x, zv[0].y, zv[0].z, zv[0].w, zv[1].x, zv[1].y, zv[1].z, zv[1].w};
                const uint32_t ww[8] = {zw4[0].x, zw4[0].y, zw4[0].z, zw4[0].w, zw4[1].x, zw4[1].y, zw4[1].z, zw4[1].w};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    ldsw<float>(lds, zw + zoff(2 * j, lane), lo_f(vv[j]) * lo_f(ww[j]));
                    ldsw<float>(lds, zw + zoff(2 * j + 1, lane), hi_f(vv[j]) * hi_f(ww[j]));
                }
            }
            const int64_t tl = tile64(a, n, bos, c);
            // the chunk-start state, bf16, [dk][dv]
            stage_store<8>(lds, stg, S, g, r, lane, a.ws_s16 + (tl * a.H + h) * kD * kD + col0, kD);
            bf16x8 sb[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) sb[s] = pk_pair(S[2 * s], S[2 * s + 1]);
            const int eb = kF_E + (c & 1) * 16384;
            // X = Z - Et S, then the blocked solve U = (I + A)^-1 X
            f32x4 U[4];
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                f32x4 acc = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s) acc = mma32(op_split<256>(lds, eb, 16 * m + r, s, g), sb[s], acc);
                const float4 z = ldsr<float4>(lds, zw + zoff(r, 16 * m + 4 * g));
                f32x4 y = f32x4{z.x, z.y, z.z, z.w} - acc;
#pragma unroll
                for (int k = 0; k < m; ++k)
                    y = mma16(ldsr<uint2>(lds, kF_AN + toff<128>(16 * m + r, 16 * k + 4 * g)), pk_blk(U[k]), y);
                mfma_src_wait(y);
                f32x4 u = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s) u = mma4(ldsr<float>(lds, kF_T + tb_off(m, r, 4 * g + s)), y[s], u);
                U[m] = u;
            }
            stage_store<4>(lds, stg, U, g, r, lane, a.ws_u16 + (tl * a.H + h) * kC * kD + col0, kD);
            if (c + 1 < nch) {
                // S <- 2^G_L S + Kb^T U
                bf16x8 ub[2];
#pragma unroll
                for (int s = 0; s < 2; ++s) ub[s] = pk_pair(U[2 * s], U[2 * s + 1]);
#pragma unroll
                for (int cb = 0; cb < 8; ++cb) {
                    const float4 gl = ldsr<float4>(lds, kF_GL + 512 * (c & 1) + (16 * cb + 4 * g) * 4);
                    f32x4 acc = S[cb] * f32x4{gl.x, gl.y, gl.z, gl.w};
#pragma unroll
                    for (int s = 0; s < 2; ++s) acc = mma32(op_split<128>(lds, kF_KBT, 16 * cb + r, s, g), ub[s], acc);
                    S[cb] = acc;
                }
            }
            if (c + 1 < nch) load_z(c + 1);  // completes while the key waves finish the next chunk
            lds_sync();  // B1: the key waves prepared the next chunk's first half
            lds_sync();  // B0: and its second half
        }
    } else {
        // ---- key waves: channels 32 p .. 32 p + 31, one token per lane ----
        const int p = wave - 4, c0 = 32 * p;
        FPrep pr;
        auto load = [&](int c) {
            const int64_t t = int64_t(c) * kC + lane;
            load_keys<32, false>(pr.in, a, ((rowbase + t) * a.H + h) * kD + c0, t < eos - bos);
        };
        // first half: scan, Et and Kd tiles, Kb and 2^G_L in registers
        auto half1 = [&](int c) {
            const int eb = kF_E + (c & 1) * 16384;
            bool ok = true;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // eight channels at a time: running decay, its chunk total, the factor tiles
                uint32_t et[4], kd[4];
                float gl8[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float ev[2], kdv[2], kbv[2];
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int ch = 8 * j + 2 * i + h2;
                        const float G = wave_scan(log2_decay(pr.in.al[ch]), lane);
                        const float GL = readlane_f(G, 63);
                        ok = ok && GL >= kRangeLog2;
                        gl8[2 * i + h2] = GL;
                        const float kf = kv<32>(pr.in.k, ch), bf = kv<32>(pr.in.b, ch);
                        ev[h2] = bf * kf * pow2(G);
                        kdv[h2] = kf * pow2(-G);
                        kbv[h2] = kf * pow2(GL - G);
                    }
                    et[i] = pk2(ev[0], ev[1]);
                    kd[i] = pk2(kdv[0], kdv[1]);
                    pr.kb[4 * j + i] = pk2(kbv[0], kbv[1]);
                }
                ldsw<uint4>(lds, eb + toff<256>(lane, c0 + 8 * j), make_uint4(et[0], et[1], et[2], et[3]));
                ldsw<uint4>(lds, kF_KD + toff<256>(lane, c0 + 8 * j), make_uint4(kd[0], kd[1], kd[2], kd[3]));
                if (lane == 63) {
                    ldsw<float4>(lds, kF_GL + 512 * (c & 1) + (c0 + 8 * j) * 4,
                                 make_float4(pow2(gl8[0]), pow2(gl8[1]), pow2(gl8[2]), pow2(gl8[3])));
                    ldsw<float4>(lds, kF_GL + 512 * (c & 1) + (c0 + 8 * j + 4) * 4,
                                 make_float4(pow2(gl8[4]), pow2(gl8[5]), pow2(gl8[6]), pow2(gl8[7])));
                }
            }
            if (!ok && lane == 0) atomicOr(a.range_flag, 1);
        };
        // second half: A^T blocks of row block p (-A below the diagonal, the
        // diagonal block inverted), Kb^T and 2^G_L
        auto half2 = [&](int c) {
            const int eb = kF_E + (c & 1) * 16384;
            const int m = p;
            for (int nb = 0; nb <= m; ++nb) {
                f32x4 acc = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s)
                    acc = mma32(op_nat<256>(lds, kF_KD, 16 * nb + r, s, g), op_nat<256>(lds, eb, 16 * m + r, s, g), acc);
                // acc: rows j = 16 nb + 4g + e, column i = 16 m + r of A^T
                if (nb < m) {
                    ldsw<uint2>(lds, kF_AN + toff<128>(16 * m + r, 16 * nb + 4 * g),
                                make_uint2(pk2(-acc[0], -acc[1]), pk2(-acc[2], -acc[3])));
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        ldsw<float>(lds, kF_AD + tb_off(m, r, 4 * g + e), r > 4 * g + e ? acc[e] : 0.f);
                }
            }
            wave_lds_fence();
            diag_inverse(lds, kF_AD + m * kTBlk, kF_T + m * kTBlk, g, r);
#pragma unroll
            for (int ch = 0; ch < 32; ++ch) {
                const uint32_t w = pr.kb[ch >> 1];
                ldsw<bf16raw>(lds, kF_KBT + toff<128>(c0 + ch, lane), bf16raw((ch & 1) ? (w >> 16) : (w & 0xffffu)));
            }
        };
        load(0);
        half1(0);
        lds_sync();
        half2(0);
        if (nch > 1) load(1);
        lds_sync();
        for (int c = 0; c < nch; ++c) {
            if (c + 1 < nch) half1(c + 1);
            lds_sync();
            if (c + 1 < nch) {
                half2(c + 1);
                if (c + 2 < nch) load(c + 2);
            }
            lds_sync();
        }
    }
}

// =============================================================================
// bwd_bstate: the reverse state-gradient pass.
constexpr int kB_KB = 0;                    // [64][128] bf16 Kb (rows tokens)
constexpr int kB_QT = 16384;                // [128][64] bf16 Qt^T
constexpr int kB_ET = 32768;                // [128][64] bf16 -Et^T
constexpr int kB_SE = 49152;                // [64][128] bf16 Et (preparation)
constexpr int kB_SQ = 65536;                // [64][128] bf16 Qt (preparation)
constexpr int kB_SKD = 81920;               // [64][128] bf16 Kd (preparation)
constexpr int kB_AT = 98304;                // [64][64] bf16 -A^T (rows j), blocks above the diagonal
constexpr int kB_PT = 106496;               // [64][64] bf16 P^T (rows j)
constexpr int kB_T = 114688;                // [4] FP32 blocks T_m
constexpr int kB_AD = kB_T + 4 * kTBlk;     // [4] FP32 blocks A_mm (preparation)
constexpr int kB_GL = kB_AD + 4 * kTBlk;    // [2][128] f32 2^G_L (chunk in work, chunk in preparation)
constexpr int kB_DO = kB_GL + 1024;         // [4 value waves][16 columns][64 tokens] bf16 dO
constexpr int kB_STG = kB_DO + 4 * 2048;    // [4 value waves] staging (dS' bf16, dX FP32)
constexpr int kB_StgWave = 128 * 48;
constexpr int kB_Bytes = kB_STG + 4 * kB_StgWave;
static_assert(kB_Bytes <= 160 * 1024, "LDS budget");
static_assert(64 * 80 <= kB_StgWave, "dX staging");

// One chunk's value-side rows of a value wave: dO (lane = token, 16
// columns) and w, v (two (token, 8 columns) pieces per lane, tokens lane / 2
// and lane / 2 + 32).
struct RowsB {
    uint4 d0, d1, w0, w1, v0, v1;
};
__device__ __forceinline__ void load_rows_b(const BwdArgs& a, RowsB& x, const bf16raw* dop, const bf16raw* wp,
                                            const bf16raw* vp, int64_t rowbase, int h, int col0, int c, int64_t L,
                                            int lane)
{
    const uint4 z = make_uint4(0, 0, 0, 0);
    const int64_t t = int64_t(c) * kC + lane;
    const int64_t off = ((rowbase + t) * a.H + h) * kD + col0;
    x.d0 = t < L ? *reinterpret_cast<const uint4*>(dop + off) : z;
    x.d1 = t < L ? *reinterpret_cast<const uint4*>(dop + off + 8) : z;
    const int64_t t0 = int64_t(c) * kC + (lane >> 1), t1 = t0 + 32;
    const int64_t o0 = ((rowbase + t0) * a.H + h) * kD + col0 + 8 * (lane & 1);
    const int64_t o1 = ((rowbase + t1) * a.H + h) * kD + col0 + 8 * (lane & 1);
    x.w0 = t0 < L ? *reinterpret_cast<const uint4*>(wp + o0) : z;
    x.v0 = t0 < L ? *reinterpret_cast<const uint4*>(vp + o0) : z;
    x.w1 = t1 < L ? *reinterpret_cast<const uint4*>(wp + o1) : z;
    x.v1 = t1 < L ? *reinterpret_cast<const uint4*>(vp + o1) : z;
}

// T_m^T y for the FP32 diagonal block T_m (K index 4g + s in step s).
__device__ __forceinline__ f32x4 tmul_t(const unsigned char* lds, int tbase, int m, int g, int r, f32x4 y)
{
    mfma_src_wait(y);
    f32x4 x = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s) x = mma4(ldsr<float>(lds, tbase + tb_off(m, 4 * g + s, r)), y[s], x);
    return x;
}

// dv = dX w, dw = dX v and the bf16 dX row piece of token lane / 2 + 32 it
// (columns 8 (lane & 1) .. + 7 of the wave's 16), from the FP32 staging.
__device__ __forceinline__ void store_dvdw(const BwdArgs& a, const unsigned char* lds, int stg, int lane, int64_t tl,
                                           int h, int col0, int c, int64_t L, int64_t rowbase, uint4 wq, uint4 vq,
                                           int it)
{
    const int tok = (lane >> 1) + 32 * it, half = lane & 1;
    const float4 x0 = ldsr<float4>(lds, stg + tok * 80 + 32 * half);
    const float4 x1 = ldsr<float4>(lds, stg + tok * 80 + 32 * half + 16);
    const float xs[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    const uint32_t w4[4] = {wq.x, wq.y, wq.z, wq.w}, v4[4] = {vq.x, vq.y, vq.z, vq.w};
    uint32_t odv[4], odw[4], odx[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        odv[j] = pk2(xs[2 * j] * lo_f(w4[j]), xs[2 * j + 1] * hi_f(w4[j]));
        odw[j] = pk2(xs[2 * j] * lo_f(v4[j]), xs[2 * j + 1] * hi_f(v4[j]));
        odx[j] = pk2(xs[2 * j], xs[2 * j + 1]);
    }
    const int64_t t = int64_t(c) * kC + tok;
    *reinterpret_cast<uint4*>(a.ws_dx16 + ((tl * a.H + h) * kC + tok) * kD + col0 + 8 * half) =
        make_uint4(odx[0], odx[1], odx[2], odx[3]);
    if (t < L) {
        const int64_t off = ((rowbase + t) * a.H + h) * kD + col0 + 8 * half;
        *reinterpret_cast<uint4*>(static_cast<bf16raw*>(a.dv) + off) = make_uint4(odv[0], odv[1], odv[2], odv[3]);
        *reinterpret_cast<uint4*>(static_cast<bf16raw*>(a.dw) + off) = make_uint4(odw[0], odw[1], odw[2], odw[3]);
    }
}

struct BPrep {
    KeyIn<32> in;
    uint32_t kb[16];
};

__global__ __launch_bounds__(kThreads) void bwd_bstate_kernel(BwdArgs a)
{
    extern __shared__ __align__(16) unsigned char lds[];
    if (*a.range_flag != 0) return;
    int64_t chain;
    int tile;
    xcd_pair(blockIdx.x, chain, tile);
    if (chain >= int64_t(a.N) * a.H) return;
    const int n = int(chain / a.H), h = int(chain % a.H);
    int64_t bos, eos, brow;
    sequence_bounds(a.cu_seqlens, n, a.T, bos, eos, brow);
    const int nch = int((eos - bos + kC - 1) / kC);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, g = lane >> 4, r = lane & 15;
    const bool value = wave < 4;
    const int64_t rowbase = brow * a.T + bos;
    const int64_t L = eos - bos;

    if (value) {
        const int col0 = tile * kTileV + wave * 16;
        const int dw_ = kB_DO + wave * 2048, stg = kB_STG + wave * kB_StgWave;
        const bf16raw* dop = static_cast<const bf16raw*>(a.d_o);
        const bf16raw* vp = static_cast<const bf16raw*>(a.v);
        const bf16raw* wp = static_cast<const bf16raw*>(a.w);
        f32x4 S[8];  // dS', then dS
        const int64_t sbase = (int64_t(n) * a.H + h) * kD * kD + col0 + r;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int e = 0; e < 4; ++e)
                S[cb][e] = a.d_final_state ? a.d_final_state[sbase + (16 * cb + 4 * g + e) * kD] : 0.f;
        // dO: lane = token, 16 columns; w, v: two (token, 8 columns) pieces per lane
        RowsB cur, nxt;
        if (nch > 0) load_rows_b(a, cur, dop, wp, vp, rowbase, h, col0, nch - 1, L, lane);
        lds_sync();
        lds_sync();
        for (int c = nch - 1; c >= 0; --c) {
            // dO of this chunk into LDS ([column][token])
            {
                const uint32_t d8[8] = {cur.d0.x, cur.d0.y, cur.d0.z, cur.d0.w, cur.d1.x, cur.d1.y, cur.d1.z, cur.d1.w};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    ldsw<bf16raw>(lds, dw_ + toff<128>(2 * j, lane), bf16raw(d8[j] & 0xffffu));
                    ldsw<bf16raw>(lds, dw_ + toff<128>(2 * j + 1, lane), bf16raw(d8[j] >> 16));
                }
            }
            const int64_t tl = tile64(a, n, bos, c);
            // the chunk-end state gradient, bf16, [dk][dv]
            stage_store<8>(lds, stg, S, g, r, lane, a.ws_ds16 + (tl * a.H + h) * kD * kD + col0, kD);
            bf16x8 sb[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) sb[s] = pk_pair(S[2 * s], S[2 * s + 1]);
            const bf16x8 dob0 = op_nat<128>(lds, dw_, r, 0, g), dob1 = op_nat<128>(lds, dw_, r, 1, g);
            // dU = Kb dS' + P^T dO (P^T is zero left of the diagonal blocks)
            f32x4 du0 = zero4(), du1 = zero4(), du2 = zero4(), du3 = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                du0 = mma32(op_split<256>(lds, kB_KB, r, s, g), sb[s], du0);
                du1 = mma32(op_split<256>(lds, kB_KB, 16 + r, s, g), sb[s], du1);
                du2 = mma32(op_split<256>(lds, kB_KB, 32 + r, s, g), sb[s], du2);
                du3 = mma32(op_split<256>(lds, kB_KB, 48 + r, s, g), sb[s], du3);
            }
            du0 = mma32(op_nat<128>(lds, kB_PT, r, 0, g), dob0, du0);
            du1 = mma32(op_nat<128>(lds, kB_PT, 16 + r, 0, g), dob0, du1);
            du0 = mma32(op_nat<128>(lds, kB_PT, r, 1, g), dob1, du0);
            du1 = mma32(op_nat<128>(lds, kB_PT, 16 + r, 1, g), dob1, du1);
            du2 = mma32(op_nat<128>(lds, kB_PT, 32 + r, 1, g), dob1, du2);
            du3 = mma32(op_nat<128>(lds, kB_PT, 48 + r, 1, g), dob1, du3);
            // dX = (I + A)^-T dU, blocks from the last:
            // dX_m = T_m^T (dU_m - sum_{k>m} A_km^T dX_k)
            const f32x4 dx3 = tmul_t(lds, kB_T, 3, g, r, du3);
            du2 = mma16(ldsr<uint2>(lds, kB_AT + toff<128>(32 + r, 48 + 4 * g)), pk_blk(dx3), du2);
            const f32x4 dx2 = tmul_t(lds, kB_T, 2, g, r, du2);
            du1 = mma16(ldsr<uint2>(lds, kB_AT + toff<128>(16 + r, 32 + 4 * g)), pk_blk(dx2), du1);
            du1 = mma16(ldsr<uint2>(lds, kB_AT + toff<128>(16 + r, 48 + 4 * g)), pk_blk(dx3), du1);
            const f32x4 dx1 = tmul_t(lds, kB_T, 1, g, r, du1);
            du0 = mma16(ldsr<uint2>(lds, kB_AT + toff<128>(r, 16 + 4 * g)), pk_blk(dx1), du0);
            du0 = mma16(ldsr<uint2>(lds, kB_AT + toff<128>(r, 32 + 4 * g)), pk_blk(dx2), du0);
            du0 = mma16(ldsr<uint2>(lds, kB_AT + toff<128>(r, 48 + 4 * g)), pk_blk(dx3), du0);
            const f32x4 dx0 = tmul_t(lds, kB_T, 0, g, r, du0);
            // dv = dX w, dw = dX v and the dX rows (bf16), through FP32 staging
            const f32x4 dX[4] = {dx0, dx1, dx2, dx3};
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int e = 0; e < 4; ++e) ldsw<float>(lds, stg + (16 * b + 4 * g + e) * 80 + 4 * r, dX[b][e]);
            wave_lds_fence();
            store_dvdw(a, lds, stg, lane, tl, h, col0, c, L, rowbase, cur.w0, cur.v0, 0);
            store_dvdw(a, lds, stg, lane, tl, h, col0, c, L, rowbase, cur.w1, cur.v1, 1);
            wave_lds_fence();
            // dS = 2^G_L dS' + Qt^T dO - Et^T dX
            const bf16x8 xb0 = pk_pair(dx0, dx1), xb1 = pk_pair(dx2, dx3);
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) {
                const float4 gl = ldsr<float4>(lds, kB_GL + 512 * (c & 1) + (16 * cb + 4 * g) * 4);
                f32x4 acc = S[cb] * f32x4{gl.x, gl.y, gl.z, gl.w};
                acc = mma32(op_nat<128>(lds, kB_QT, 16 * cb + r, 0, g), dob0, acc);
                acc = mma32(op_split<128>(lds, kB_ET, 16 * cb + r, 0, g), xb0, acc);
                acc = mma32(op_nat<128>(lds, kB_QT, 16 * cb + r, 1, g), dob1, acc);
                acc = mma32(op_split<128>(lds, kB_ET, 16 * cb + r, 1, g), xb1, acc);
                S[cb] = acc;
            }
            // the next chunk's rows: the loads complete while the key waves
            // finish its preparation
            if (c > 0) load_rows_b(a, nxt, dop, wp, vp, rowbase, h, col0, c - 1, L, lane);
            lds_sync();
            lds_sync();
            if (c > 0) cur = nxt;
        }
        if (a.d_initial_state) {
#pragma unroll
            for (int cb = 0; cb < 8; ++cb)
#pragma unroll
                for (int e = 0; e < 4; ++e) a.d_initial_state[sbase + (16 * cb + 4 * g + e) * kD] = S[cb][e];
        }
    } else {
        const int p = wave - 4, c0 = 32 * p;
        // P^T blocks above the diagonal are read as zeros
        for (int i = threadIdx.x - 256; i < 8192 / 16; i += 256) ldsw<uint4>(lds, kB_PT + 16 * i, make_uint4(0, 0, 0, 0));
        BPrep pr;
        auto load = [&](int c) {
            const int64_t t = int64_t(c) * kC + lane;
            load_keys<32, true>(pr.in, a, ((rowbase + t) * a.H + h) * kD + c0, t < L);
        };
        // first half: scan, the Et, Qt, Kd tiles (rows = tokens), Kb in
        // registers, 2^G_L into the buffer of chunk c
        auto half1 = [&](int c) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                uint32_t kd[4], et[4], qt[4];
                float gl8[8];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float ev[2], kdv[2], kbv[2], qv[2];
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int ch = 8 * j + 2 * i + h2;
                        const float G = wave_scan(log2_decay(pr.in.al[ch]), lane);
                        const float GL = readlane_f(G, 63);
                        gl8[2 * i + h2] = GL;
                        const float kf = kv<32>(pr.in.k, ch), bf = kv<32>(pr.in.b, ch), qf = kv<32>(pr.in.q, ch);
                        const float up = pow2(G);
                        ev[h2] = bf * kf * up;
                        qv[h2] = qf * up;
                        kdv[h2] = kf * pow2(-G);
                        kbv[h2] = kf * pow2(GL - G);
                    }
                    et[i] = pk2(ev[0], ev[1]);
                    qt[i] = pk2(qv[0], qv[1]);
                    kd[i] = pk2(kdv[0], kdv[1]);
                    pr.kb[4 * j + i] = pk2(kbv[0], kbv[1]);
                }
                ldsw<uint4>(lds, kB_SE + toff<256>(lane, c0 + 8 * j), make_uint4(et[0], et[1], et[2], et[3]));
                ldsw<uint4>(lds, kB_SQ + toff<256>(lane, c0 + 8 * j), make_uint4(qt[0], qt[1], qt[2], qt[3]));
                ldsw<uint4>(lds, kB_SKD + toff<256>(lane, c0 + 8 * j), make_uint4(kd[0], kd[1], kd[2], kd[3]));
                if (lane == 63) {
                    ldsw<float4>(lds, kB_GL + 512 * (c & 1) + (c0 + 8 * j) * 4,
                                 make_float4(pow2(gl8[0]), pow2(gl8[1]), pow2(gl8[2]), pow2(gl8[3])));
                    ldsw<float4>(lds, kB_GL + 512 * (c & 1) + (c0 + 8 * j + 4) * 4,
                                 make_float4(pow2(gl8[4]), pow2(gl8[5]), pow2(gl8[6]), pow2(gl8[7])));
                }
            }
        };
        auto half2 = [&](int c) {
            (void)c;
            const int m = p;
            for (int nb = 0; nb <= m; ++nb) {
                f32x4 accA = zero4(), accP = zero4();
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const bf16x8 kd = op_nat<256>(lds, kB_SKD, 16 * nb + r, s, g);
                    accA = mma32(op_nat<256>(lds, kB_SE, 16 * m + r, s, g), kd, accA);
                    accP = mma32(op_nat<256>(lds, kB_SQ, 16 * m + r, s, g), kd, accP);
                }
                // acc: rows i = 16 m + 4g + e, column j = 16 nb + r
                if (nb < m) {
                    ldsw<uint2>(lds, kB_AT + toff<128>(16 * nb + r, 16 * m + 4 * g),
                                make_uint2(pk2(-accA[0], -accA[1]), pk2(-accA[2], -accA[3])));
                    ldsw<uint2>(lds, kB_PT + toff<128>(16 * nb + r, 16 * m + 4 * g),
                                make_uint2(pk2(accP[0], accP[1]), pk2(accP[2], accP[3])));
                } else {
                    f32x4 pm;
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const int i = 4 * g + e;
                        pm[e] = i >= r ? accP[e] : 0.f;
                        ldsw<float>(lds, kB_AD + tb_off(m, i, r), i > r ? accA[e] : 0.f);
                    }
                    ldsw<uint2>(lds, kB_PT + toff<128>(16 * nb + r, 16 * m + 4 * g),
                                make_uint2(pk2(pm[0], pm[1]), pk2(pm[2], pm[3])));
                }
            }
            wave_lds_fence();
            diag_inverse(lds, kB_AD + m * kTBlk, kB_T + m * kTBlk, g, r);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                ldsw<uint4>(lds, kB_KB + toff<256>(lane, c0 + 8 * j),
                            make_uint4(pr.kb[4 * j], pr.kb[4 * j + 1], pr.kb[4 * j + 2], pr.kb[4 * j + 3]));
            // Qt^T and -Et^T (rows = channels) from the lane's own token rows
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint4 e4 = ldsr<uint4>(lds, kB_SE + toff<256>(lane, c0 + 8 * j));
                const uint4 q4 = ldsr<uint4>(lds, kB_SQ + toff<256>(lane, c0 + 8 * j));
                const uint32_t ew[4] = {e4.x, e4.y, e4.z, e4.w}, qw[4] = {q4.x, q4.y, q4.z, q4.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int ch = c0 + 8 * j + i, sh = (i & 1) ? 16 : 0;
                    ldsw<bf16raw>(lds, kB_QT + toff<128>(ch, lane), bf16raw(qw[i >> 1] >> sh));
                    ldsw<bf16raw>(lds, kB_ET + toff<128>(ch, lane), bf16raw((ew[i >> 1] >> sh) ^ 0x8000u));
                }
            }
        };
        if (nch > 0) {
            load(nch - 1);
            half1(nch - 1);
        }
        lds_sync();
        if (nch > 0) {
            half2(nch - 1);
            if (nch > 1) load(nch - 2);
        }
        lds_sync();
        for (int c = nch - 1; c >= 0; --c) {
            if (c > 0) half1(c - 1);
            lds_sync();
            if (c > 0) {
                half2(c - 1);
                if (c > 1) load(c - 2);
            }
            lds_sync();
        }
    }
}

// =============================================================================
// bwd_grads: per (chunk, head, half of the key channels), everything that
// needs S, dS', U and dX.  A workgroup takes 64 key channels, so that its LDS
// stays at 80 KB and two workgroups share a CU: one's loads overlap the
// other's products.  The products over value columns that do not involve the
// key channels (dA, dP and their transposes) are formed by both halves.
// LDS map (bytes).  Phase 1 (the products over value columns):
constexpr int kG_U = 0;         // [64][128] bf16 U
constexpr int kG_DX = 16384;    // [64][128] bf16 dX
constexpr int kG_DO = 32768;    // [64][128] bf16 dO
constexpr int kG_S = 49152;     // [64][128] bf16 S, the half's key channels
constexpr int kG_DS = 65536;    // [64][128] bf16 dS'
constexpr int kG_Phase1 = 81920;
// phases 2 to 4 (the products over tokens and the epilogue), over the same memory:
constexpr int kGRow = 65;                   // floats per row of the [channel][token] FP32 array
constexpr int kG_G = 0;                     // [64][65] f32 G
constexpr int kG_KDT = 16640;               // [64][64] bf16 Kd^T
constexpr int kG_ETT = kG_KDT + 8192;       // [64][64] bf16 Et^T
constexpr int kG_QTT = kG_ETT + 8192;       // [64][64] bf16 Qt^T
constexpr int kG_RQ = kG_QTT + 8192;        // [64][64] bf16 q (rows tokens)
constexpr int kG_RK = kG_RQ + 8192;         // [64][64] bf16 k
constexpr int kG_RB = kG_RK + 8192;         // [64][64] bf16 b
constexpr int kG_CL = kG_RB + 8192;         // [64][64] u8: alpha outside [2^-15, 1]
constexpr int kG_BT = kG_CL + 4096;         // [2][4][64] f32: per 16-token block, sums of dg and of Kb dKb
constexpr int kG_RS = kG_BT + 2048;         // [64] f32 rowsum(dS' . S)
constexpr int kG_GL = kG_RS + 256;          // [64] f32 G_L
constexpr int kG_Bytes = kG_Phase1;
static_assert(kG_GL + 256 <= kG_Bytes && 2 * kG_Bytes <= 160 * 1024, "LDS budget: two workgroups per CU");

// Suffix sums within each row of 16 lanes (lane r gets the sum over r' >= r).
__device__ __forceinline__ float row_rscan16(float x)
{
    x += row_shl<1>(x);
    x += row_shl<2>(x);
    x += row_shl<4>(x);
    x += row_shl<8>(x);
    return x;
}

// The chunk that owns workspace tile `tile` (false for an unused slot).
__device__ bool chunk_of_tile(const BwdArgs& a, int64_t tile, int& n, int& m, int64_t& bos, int64_t& eos,
                              int64_t& brow)
{
    if (!a.cu_seqlens) {
        n = int(tile / a.slots64);
        m = int(tile % a.slots64);
        sequence_bounds(nullptr, n, a.T, bos, eos, brow);
        return int64_t(m) * kC < eos;
    }
    // first slot of sequence s: bos_s / 64 + s, increasing in s
    int lo = 0, hi = a.N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        int64_t mb, me, mr;
        sequence_bounds(a.cu_seqlens, mid, a.T, mb, me, mr);
        if (mb / kC + mid <= tile) lo = mid; else hi = mid - 1;
    }
    n = lo;
    sequence_bounds(a.cu_seqlens, n, a.T, bos, eos, brow);
    const int64_t first = bos / kC + n;
    if (tile < first) return false;
    m = int(tile - first);
    return bos + int64_t(m) * kC < eos && tile64(a, n, bos, m) == tile;
}

__global__ __launch_bounds__(kThreads, 4) void bwd_grads_kernel(BwdArgs a)
{
    extern __shared__ __align__(16) unsigned char lds[];
    if (*a.range_flag != 0) return;
    int64_t ch_idx;  // (tile, head)
    int half;
    xcd_pair(blockIdx.x, ch_idx, half);
    if (ch_idx >= int64_t(a.B) * a.slots64 * a.H) return;
    const int h = int(ch_idx % a.H);
    const int64_t tile = ch_idx / a.H;
    int n, m;
    int64_t bos, eos, brow;
    if (!chunk_of_tile(a, tile, n, m, bos, eos, brow)) return;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
    const int64_t t0 = bos + int64_t(m) * kC;  // first token of the chunk
    const int L = int(eos - t0 < kC ? eos - t0 : kC);
    const int64_t rowbase = brow * a.T + t0;
    const int hc = 64 * half;                  // first key channel of this workgroup
    const bf16raw* dop = static_cast<const bf16raw*>(a.d_o);

    // ---- phase 0: U, dX, dO and the half's rows of S and dS' into LDS; the
    // key inputs (one token per lane, eight channels per wave) into registers
    {
        const bf16raw* us = a.ws_u16 + (tile * a.H + h) * kC * kD;
        const bf16raw* xs = a.ws_dx16 + (tile * a.H + h) * kC * kD;
        const bf16raw* ss = a.ws_s16 + ((tile * a.H + h) * kD + hc) * kD;
        const bf16raw* ds = a.ws_ds16 + ((tile * a.H + h) * kD + hc) * kD;
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int p = tid + kThreads * it, row = p >> 4, gr = p & 15;
            const uint4 u = reinterpret_cast<const uint4*>(us)[p];
            const uint4 x = reinterpret_cast<const uint4*>(xs)[p];
            uint4 d = make_uint4(0, 0, 0, 0);
            if (row < L) d = *reinterpret_cast<const uint4*>(dop + ((rowbase + row) * a.H + h) * kD + 8 * gr);
            const uint4 sv = reinterpret_cast<const uint4*>(ss)[p];
            const uint4 dv4 = reinterpret_cast<const uint4*>(ds)[p];
            ldsw<uint4>(lds, kG_U + toff<256>(row, 8 * gr), u);
            ldsw<uint4>(lds, kG_DX + toff<256>(row, 8 * gr), x);
            ldsw<uint4>(lds, kG_DO + toff<256>(row, 8 * gr), d);
            ldsw<uint4>(lds, kG_S + toff<256>(row, 8 * gr), sv);
            ldsw<uint4>(lds, kG_DS + toff<256>(row, 8 * gr), dv4);
        }
    }
    KeyIn<8> kin;
    const int c0 = 8 * wave;  // the wave's key channels within the half
    load_keys<8, true>(kin, a, ((rowbase + lane) * a.H + h) * kD + hc + c0, lane < L);
    __syncthreads();

    // ---- phase 1: rowsum(dS' . S) (kept in a register until phase 4) and the
    // products over value columns
    float rs_val;
    {
        const int ch = tid >> 3, qq = tid & 7;  // 8 threads per channel, 16 columns each
        float acc = 0.f;
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const uint4 s4 = ldsr<uint4>(lds, kG_S + toff<256>(ch, 16 * qq + 8 * j));
            const uint4 d4 = ldsr<uint4>(lds, kG_DS + toff<256>(ch, 16 * qq + 8 * j));
            const uint32_t sw[4] = {s4.x, s4.y, s4.z, s4.w}, dw[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) acc += lo_f(sw[i]) * lo_f(dw[i]) + hi_f(sw[i]) * hi_f(dw[i]);
        }
        acc += __shfl_xor(acc, 1);
        acc += __shfl_xor(acc, 2);
        acc += __shfl_xor(acc, 4);
        rs_val = acc;  // lanes with qq == 0 hold channel ch's sum
    }
    const int tb = wave & 3, cq = wave >> 2;  // token block; pair of channel blocks (2 cq, 2 cq + 1)
    f32x4 dAt[4], dA[4], dPt[4], dP[4], dEt[2], dQt[2], dKb[2];
#pragma unroll
    for (int b = 0; b < 4; ++b) dAt[b] = dA[b] = dPt[b] = dP[b] = zero4();
#pragma unroll
    for (int b = 0; b < 2; ++b) dEt[b] = dQt[b] = dKb[b] = zero4();
    // block by block, the K steps inside (shared operands are read again per
    // block: that keeps the live registers to the accumulators)
#pragma unroll
    for (int b = 0; b < 4; ++b) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const bf16x8 xt = op_nat<256>(lds, kG_DX, 16 * tb + r, s, g);
            const bf16x8 ut = op_nat<256>(lds, kG_U, 16 * tb + r, s, g);
            const bf16x8 ot = op_nat<256>(lds, kG_DO, 16 * tb + r, s, g);
            if (b <= tb) {
                const bf16x8 ub = op_nat<256>(lds, kG_U, 16 * b + r, s, g);
                dAt[b] = mma32(ub, xt, dAt[b]);
                dPt[b] = mma32(ub, ot, dPt[b]);
            }
            if (b >= tb) {
                dA[b] = mma32(op_nat<256>(lds, kG_DX, 16 * b + r, s, g), ut, dA[b]);
                dP[b] = mma32(op_nat<256>(lds, kG_DO, 16 * b + r, s, g), ut, dP[b]);
            }
            if (b < 2) {
                const int cb = 2 * cq + b;  // channel block within the half
                const bf16x8 sr = op_nat<256>(lds, kG_S, 16 * cb + r, s, g);
                dEt[b] = mma32(sr, xt, dEt[b]);
                dQt[b] = mma32(sr, ot, dQt[b]);
                dKb[b] = mma32(op_nat<256>(lds, kG_DS, 16 * cb + r, s, g), ut, dKb[b]);
            }
        }
        __builtin_amdgcn_sched_barrier(0);  // one block at a time: bounds the live operands
    }
    // masks and signs: dA = -strict_lower(dX U^T), dP = lower(dO U^T), dEt = -dX S^T
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int lr = 16 * b + 4 * g + e, lc = 16 * tb + r;  // accumulator row, column
            dAt[b][e] = lr < lc ? -dAt[b][e] : 0.f;   // rows j, columns i: j < i
            dPt[b][e] = lr <= lc ? dPt[b][e] : 0.f;
            dA[b][e] = lr > lc ? -dA[b][e] : 0.f;     // rows i, columns j: i > j
            dP[b][e] = lr >= lc ? dP[b][e] : 0.f;
        }
#pragma unroll
    for (int b = 0; b < 2; ++b) dEt[b] = -dEt[b];
    // dA, dP and their transposes as bf16 B operands over tokens (half the registers)
    bf16x8 bAt[2], bPt[2], bA[2], bP[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        bAt[s] = pk_pair(dAt[2 * s], dAt[2 * s + 1]);
        bPt[s] = pk_pair(dPt[2 * s], dPt[2 * s + 1]);
        bA[s] = pk_pair(dA[2 * s], dA[2 * s + 1]);
        bP[s] = pk_pair(dP[2 * s], dP[2 * s + 1]);
    }
    __syncthreads();

    // ---- phase 2: the key side of this chunk: G, the factor tiles and the
    // clamp flags [channel][token], the raw q, k, b [token][channel]
    {
        float G[8], GL[8];
        decay_scan<8>(kin, lane, G, GL);
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int ch = c0 + c;  // within the half
            const float kf = kv<8>(kin.k, c), bf = kv<8>(kin.b, c), qf = kv<8>(kin.q, c);
            const float up = pow2(G[c]);
            ldsw<float>(lds, kG_G + (ch * kGRow + lane) * 4, G[c]);
            ldsw<bf16raw>(lds, kG_KDT + toff<128>(ch, lane), f32_to_bf16(kf * pow2(-G[c])));
            ldsw<bf16raw>(lds, kG_ETT + toff<128>(ch, lane), f32_to_bf16(bf * kf * up));
            ldsw<bf16raw>(lds, kG_QTT + toff<128>(ch, lane), f32_to_bf16(qf * up));
            const float lg = __log2f(kin.al[c]);
            ldsw<unsigned char>(lds, kG_CL + ch * 64 + lane, (lg >= kLog2AlphaFloor && lg <= 0.f) ? 0 : 1);
        }
        ldsw<uint4>(lds, kG_RQ + toff<128>(lane, c0), make_uint4(kin.q[0], kin.q[1], kin.q[2], kin.q[3]));
        ldsw<uint4>(lds, kG_RK + toff<128>(lane, c0), make_uint4(kin.k[0], kin.k[1], kin.k[2], kin.k[3]));
        ldsw<uint4>(lds, kG_RB + toff<128>(lane, c0), make_uint4(kin.b[0], kin.b[1], kin.b[2], kin.b[3]));
        if (lane == 63) {
#pragma unroll
            for (int c = 0; c < 8; ++c) ldsw<float>(lds, kG_GL + 4 * (c0 + c), GL[c]);
        }
        if ((tid & 7) == 0) ldsw<float>(lds, kG_RS + 4 * (tid >> 3), rs_val);
    }
    const int tok = 16 * tb + r;
    __syncthreads();

    // ---- phase 3: products over tokens and the epilogue
    bf16raw* dq_out = static_cast<bf16raw*>(a.dq);
    bf16raw* dk_out = static_cast<bf16raw*>(a.dk);
    bf16raw* db_out = static_cast<bf16raw*>(a.db);
    f32x4 dgs[2];  // dg summed over this and the later tokens of the lane's 16-token block
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int cb = 2 * cq + b;
        f32x4 de = zero4(), dq = zero4(), dk = zero4();
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const bf16x8 kdt = op_split<128>(lds, kG_KDT, 16 * cb + r, s, g);
            de = mma32(kdt, bAt[s], de);
            dq = mma32(kdt, bPt[s], dq);
            dk = mma32(op_split<128>(lds, kG_ETT, 16 * cb + r, s, g), bA[s], dk);
            dk = mma32(op_split<128>(lds, kG_QTT, 16 * cb + r, s, g), bP[s], dk);
        }
        const uint2 rq = ldsr<uint2>(lds, kG_RQ + toff<128>(tok, 16 * cb + 4 * g));
        const uint2 rk = ldsr<uint2>(lds, kG_RK + toff<128>(tok, 16 * cb + 4 * g));
        const uint2 rb = ldsr<uint2>(lds, kG_RB + toff<128>(tok, 16 * cb + 4 * g));
        const uint32_t qw[2] = {rq.x, rq.y}, kw[2] = {rk.x, rk.y}, bw[2] = {rb.x, rb.y};
        float oq[4], ok[4], ob[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ch = 16 * cb + 4 * g + e;  // within the half
            const float G = ldsr<float>(lds, kG_G + (ch * kGRow + tok) * 4);
            const float gl = ldsr<float>(lds, kG_GL + 4 * ch);
            const float up = pow2(G), dn = pow2(-G), kbf = pow2(gl - G);
            const float qf = (e & 1) ? hi_f(qw[e >> 1]) : lo_f(qw[e >> 1]);
            const float kf = (e & 1) ? hi_f(kw[e >> 1]) : lo_f(kw[e >> 1]);
            const float bf = (e & 1) ? hi_f(bw[e >> 1]) : lo_f(bw[e >> 1]);
            const float ef = bf * kf;
            const float dep = up * de[e], dqp = up * dq[e], dkp = dn * dk[e];
            const float dEtv = dEt[b][e], dQtv = dQt[b][e], dKbv = dKb[b][e];
            const float dev = dep + up * dEtv;
            oq[e] = dqp + up * dQtv;
            ok[e] = dkp + kbf * dKbv + dev * bf;
            ob[e] = dev * kf;
            const float kbd = kf * kbf * dKbv;
            const float dg = ef * dep + qf * dqp - kf * dkp + ef * up * dEtv + qf * up * dQtv - kbd;
            // sums over the block's tokens: lane r = 0 of the row holds the block's total
            dgs[b][e] = row_rscan16(dg);
            const float kbs = row_rscan16(kbd);
            if (r == 0) {
                ldsw<float>(lds, kG_BT + (tb * 64 + ch) * 4, dgs[b][e]);
                ldsw<float>(lds, kG_BT + 1024 + (tb * 64 + ch) * 4, kbs);
            }
        }
        if (tok < L) {
            const int64_t off = ((rowbase + tok) * a.H + h) * kD + hc + 16 * cb + 4 * g;
            *reinterpret_cast<uint2*>(dq_out + off) = make_uint2(pk2(oq[0], oq[1]), pk2(oq[2], oq[3]));
            *reinterpret_cast<uint2*>(dk_out + off) = make_uint2(pk2(ok[0], ok[1]), pk2(ok[2], ok[3]));
            *reinterpret_cast<uint2*>(db_out + off) = make_uint2(pk2(ob[0], ob[1]), pk2(ob[2], ob[3]));
        }
        __builtin_amdgcn_sched_barrier(0);  // one tile at a time: bounds the live registers
    }
    __syncthreads();

    // ---- phase 4: dlog(alpha_m) = the sum of dg over tokens >= m plus the
    // chunk-end terms (2^G_L rowsum(dS' . S) and the sum of Kb dKb);
    // dalpha = dlog(alpha) / alpha, with alpha = 2^(G_m - G_(m-1)) (zero
    // where the clamp is active)
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        const int cb = 2 * cq + b;
        float da[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ch = 16 * cb + 4 * g + e;
            float later = 0.f, kbsum = 0.f;
#pragma unroll
            for (int t2 = 0; t2 < 4; ++t2) {
                const float bt = ldsr<float>(lds, kG_BT + (t2 * 64 + ch) * 4);
                later += t2 > tb ? bt : 0.f;
                kbsum += ldsr<float>(lds, kG_BT + 1024 + (t2 * 64 + ch) * 4);
            }
            const float end = pow2(ldsr<float>(lds, kG_GL + 4 * ch)) * ldsr<float>(lds, kG_RS + 4 * ch) + kbsum;
            const float G = ldsr<float>(lds, kG_G + (ch * kGRow + tok) * 4);
            const float Gp = tok > 0 ? ldsr<float>(lds, kG_G + (ch * kGRow + tok - 1) * 4) : 0.f;
            const float dl = dgs[b][e] + later + end;
            da[e] = ldsr<unsigned char>(lds, kG_CL + ch * 64 + tok) ? 0.f : dl / pow2(G - Gp);
        }
        if (tok < L)
            *reinterpret_cast<float4*>(a.dalpha + ((rowbase + tok) * a.H + h) * kD + hc + 16 * cb + 4 * g) =
                make_float4(da[0], da[1], da[2], da[3]);
        __builtin_amdgcn_sched_barrier(0);
    }
}

__global__ void bwd_flag_clear_kernel(int32_t* f) { f[threadIdx.x] = 0; }

}  // namespace

hipError_t launch_chunk_bwd_mfma(const BwdArgs& a, hipStream_t stream)
{
    if (a.dk_ != kD || a.dv_ != kD || !a.range_flag) return hipErrorInvalidValue;
    // more than 64 KiB of dynamic LDS (thread-safe one-time calls)
    static const hipError_t attr[3] = {
        hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_fstate_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kF_Bytes),
        hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_bstate_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kB_Bytes),
        hipFuncSetAttribute(reinterpret_cast<const void*>(bwd_grads_kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kG_Bytes)};
    for (hipError_t x : attr)
        if (x != hipSuccess) return x;
    hipLaunchKernelGGL(bwd_flag_clear_kernel, dim3(1), dim3(1), 0, stream, a.range_flag);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.T == 0) return e;
    const int64_t chains = xcd_pair_grid(int64_t(a.N) * a.H);
    const int64_t tiles = int64_t(a.B) * a.slots64 * a.H;
    if (chains > 0x7fffffff || tiles > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(bwd_fstate_kernel, dim3(unsigned(chains)), dim3(kThreads), kF_Bytes, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    // the FP32 path, gated on the range flag, then this path's last two kernels
    BwdArgs f = a;
    f.gate = a.range_flag;
    e = launch_chunk_bwd(f, true, stream);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(bwd_bstate_kernel, dim3(unsigned(chains)), dim3(kThreads), kB_Bytes, stream, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (tiles > 0) {
        const int64_t gblocks = xcd_pair_grid(tiles);  // the two channel halves of a (chunk, head) share an XCD
        if (gblocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL(bwd_grads_kernel, dim3(unsigned(gblocks)), dim3(kThreads), kG_Bytes, stream, a);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace gdn2
