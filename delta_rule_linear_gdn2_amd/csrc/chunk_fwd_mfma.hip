// Chunkwise forward on gfx950 matrix cores (bf16 inputs, dk = 128, value
// tiles of 64 columns).
//
// The chunkwise WY form (Gated DeltaNet-2 analysis, iplexlaw.co.kr, "Token
// processing and parallel training"): per chunk the cumulative channel-wise
// decay is absorbed into asymmetric factors, leaving a lower-triangular solve
// and dense products; FP32 is kept for the decay, the solve and the carried
// state.  With incoming state S, per key channel the running decay
// c_i = prod_{m<=i} alpha_m inside the chunk, e = b k and z = w v:
//     Et_i = e_i c_i     Qt_i = q_i c_i     Kt_j = k_j / c_j     Kb_j = Kt_j c_last
//     A = strict_lower(Et Kt^T)     P = lower(Qt Kt^T)
//     U = (I + A)^-1 (Z - Et S)     O = Qt S + P U     S <- Diag(c_last) S + Kb^T U
//
// Range.  alpha is clamped to [2^-15, 1].  A chunk is cut short when some
// channel decays below 2^-120 across it: it then covers 32, 16 or 8 tokens,
// the longest prefix whose decay stays at or above 2^-120 in every channel (8
// tokens always do).  Hence every factor c_i and 1 / c_j lies in
// [2^-120, 2^120], which FP32 and bf16 represent, and all factors are plain
// products of alpha (one reciprocal per element).  All waves take the decision
// from the same exchanged products, so it is uniform across the workgroup.
//
// Pipeline.  One workgroup of eight wavefronts (two per SIMD) per (sequence,
// head, 64-column value tile).  Waves 0..3 (value waves) own 16 value columns
// each and keep that 128 x 16 slice of the FP32 state in MFMA accumulators for
// the whole sequence; waves 4..7 (key waves) prepare the chunks.  Each period
// of three barriers B0, B1, B2 advances two chunks: the value waves form
// X = Z - Et S and (Qt S)^T of chunk c before B1, and its blocked solve,
// output rows and state update between B1 and B2; meanwhile the key waves
// compute the decay products of chunk c + 1 before B1 and its operand tiles
// between B1 and B2.  After B2, wave 3 forms the diagonal blocks of A of
// chunk c + 1 and their inverses, waves 0..2 its other A and P blocks, and the
// key waves issue the loads of chunk c + 2.  Tiles the value
// waves read between B1 and B2 are double-buffered; Et, Qt, Kt, the products
// and z are consumed before their next write and stay single.  Each wave loads
// its next inputs with 16-byte loads as soon as it has consumed the current
// ones.  Workgroups of one chain share an XCD, so the second value tile
// re-reads the key-side inputs from L2.
//
// Matrix products (v_mfma_f32_16x16x32_bf16, FP32 accumulate): lane
// l = 16 g + r provides row/column r and a group of eight K indices chosen by
// g; the accumulator holds rows 4g..4g+3 of column r.  A and B only need to
// agree on the K order, so for a K-step over 32 channels or tokens group g may
// take {4g..4g+3} U {16+4g..16+4g+3}: exactly the rows a lane holds in two
// adjacent accumulator blocks.  An accumulator tile therefore serves directly
// as a B operand, and as an A operand of the transposed product
// (X Y)^T = Y^T X^T; transposed products leave four consecutive columns of one
// row in each lane, so the stores of A, P and O are contiguous.  The diagonal
// blocks of the solve apply T_II = (I + A_II)^-1 in FP32
// (v_mfma_f32_16x16x4_f32).
#include "gdn2_device.hpp"
#include "launch.hpp"

namespace gdn2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kDK = 128;          // key head size
constexpr int kC = 64;            // chunk
constexpr int kDVT = 64;          // value columns per workgroup
constexpr int kWaves = 8;         // wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kValueWaves = 4;    // waves 0..3: 16 value columns each
constexpr int kTWave = 3;         // diagonal blocks of A and their inverses (a value wave)
constexpr float kAlphaMin = 0x1p-15f;
constexpr float kRangeMin = 0x1p-120f;

// ---- LDS map (bytes) -------------------------------------------------------
constexpr int kOffEt = 0;          // [64][128] bf16, single
constexpr int kOffQt = 16384;      // [64][128] bf16, single
constexpr int kOffKt = 32768;      // [64][128] bf16, single
constexpr int kOffKbT = 49152;     // [2][128][64] bf16
constexpr int kOffAneg = 81920;    // [2][64][64] bf16 (-A below the diagonal blocks)
constexpr int kOffP = 98304;       // [2][64][64] bf16
constexpr int kT16 = 20;            // floats per row of a 16 x 16 FP32 block (padded)
constexpr int kTBlk = 16 * kT16 + 16;  // floats per padded block (the next block shifts by 16 banks)
constexpr int kOffT = 114688;      // [2][4][kTBlk] f32, T_II row major
constexpr int kOffGam = kOffT + 2 * 4 * kTBlk * 4;  // [2][128] f32 (chunk decay per channel)
constexpr int kOffPh = kOffGam + 1024;  // [8][128] f32: decay over tokens 16 j .. 16 j + 15 (rows j < 4),
                                        // over 0..7 (row 4), per-block channel minima (row 5)
constexpr int kOffAd = kOffPh + 4096;   // [4][kTBlk] f32, diagonal blocks of A, column major
constexpr int kOffZs = kOffAd + 4 * kTBlk * 4;  // [64 columns][kZsStride] f32, z = w v
constexpr int kZsStride = 68;
constexpr int kLdsBytes = kOffZs + kDVT * kZsStride * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
static_assert(kOffP == kOffAneg + 2 * 8192 && kOffT == kOffP + 2 * 8192, "Aneg and P are cleared as one range");

// [64][128] bf16 tiles Et, Qt, Kt.  Channels are stored permuted within each
// group of 32 so that the split K groups of the matrix products, channels
// {32 s + 4 g .. + 3} U {32 s + 16 + 4 g .. + 3}, occupy the 16 contiguous bytes
// at position 32 s + 8 g; the 16-byte granules are XOR-swizzled by a linear
// map of the low four row bits, under which the prep stores (two 8-byte
// pieces per lane) and the operand reads (16 rows at one granule column) are
// free of bank conflicts.
__device__ __forceinline__ int chan_pos(int ch)
{
    return (ch & ~31) | ((ch & 12) << 1) | ((ch & 16) >> 2) | (ch & 3);
}
__device__ __forceinline__ int parity(int x) { return __builtin_popcount(x) & 1; }
__device__ __forceinline__ int tile_swz(int row)
{
    return parity(row & 11) | (parity(row & 9) << 1) | (parity(row & 7) << 2) | (parity(row & 13) << 3);
}
__device__ __forceinline__ int off_t128(int row, int pos)  // pos: permuted position
{
    return row * 256 + ((((pos >> 3) ^ tile_swz(row)) & 15) << 4) + ((pos & 7) << 1);
}
// [64][64] bf16 tiles Aneg, P: 8-byte pieces XOR-swizzled by the low row bits.
__device__ __forceinline__ int off_rc64(int row, int col)
{
    return row * 128 + ((((col >> 2) ^ row) & 15) << 3) + ((col & 3) << 1);
}
// [128][64] bf16 tile Kb^T (channel rows, token columns): 8-byte pieces
// XOR-swizzled by a linear map of the row bits (prep stores hit 16 channels
// eight apart, reads 16 consecutive channels).
__device__ __forceinline__ int kbt_swz(int row)
{
    return parity(row & 40) | (parity(row & 6) << 1) | (parity(row & 20) << 2) | (parity(row & 9) << 3);
}
__device__ __forceinline__ int off_kbt(int row, int col)
{
    return row * 128 + ((((col >> 2) ^ kbt_swz(row)) & 15) << 3) + ((col & 3) << 1);
}
// Float index of (column, token) in Zs: tokens rotated by 16 per group of 16
// columns so that the column-wise stores of z spread over the banks.
__device__ __forceinline__ int zs_index(int col, int tok) { return col * kZsStride + ((tok + 16 * (col >> 4)) & 63); }

__device__ __forceinline__ uint32_t pack2(float a, float b)
{
    bf16x2 v;
    v[0] = static_cast<__bf16>(a);
    v[1] = static_cast<__bf16>(b);
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <typename V>
__device__ __forceinline__ V lds_ld(const unsigned char* lds, int off)
{
    return *reinterpret_cast<const V*>(lds + off);
}
template <typename V>
__device__ __forceinline__ void lds_st(unsigned char* lds, int off, V v)
{
    *reinterpret_cast<V*>(lds + off) = v;
}

// Per-lane byte offsets of the operand reads.  For a tile row 16 k + r the
// swizzle terms depend on r only, so every read is one of these plus a
// compile-time constant (tile base and 16 k rows) -- except in Kb^T, whose
// swizzle also takes the block index (a constant XOR, see ld_kbt).
struct LaneOffs {
    int c128[4];     // [64][128] tile, positions 32 s + 8 g .. + 7 (16 bytes)
    int s64[2][2];   // [64][64] tile, columns 32 s + 16 h + 4 g .. + 3 (8 bytes)
    int kbt_row;     // Kb^T: r * 128
    int kbt_sl;      // Kb^T: 8-byte slot g ^ swizzle(r)
};

__device__ __forceinline__ LaneOffs lane_offsets(int r, int g)
{
    LaneOffs o;
#pragma unroll
    for (int s = 0; s < 4; ++s) o.c128[s] = off_t128(r, 32 * s + 8 * g);
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        o.s64[s][0] = off_rc64(r, 32 * s + 4 * g);
        o.s64[s][1] = off_rc64(r, 32 * s + 16 + 4 * g);
    }
    o.kbt_row = r * 128;
    o.kbt_sl = (g ^ kbt_swz(r)) & 15;
    return o;
}

// Row 16 k + r of a [64][128] tile: the split K group of K-step s.
__device__ __forceinline__ bf16x8 ld_c128(const unsigned char* lds, const LaneOffs& o, int base, int k, int s)
{
    return as_bf16x8(lds_ld<uint4>(lds, base + 16 * k * 256 + o.c128[s]));
}
// Split K groups, row 16 k + r of a [64][64] tile.
__device__ __forceinline__ bf16x8 ld_s64(const unsigned char* lds, const LaneOffs& o, int base, int k, int s)
{
    const uint2 lo = lds_ld<uint2>(lds, base + 16 * k * 128 + o.s64[s][0]);
    const uint2 hi = lds_ld<uint2>(lds, base + 16 * k * 128 + o.s64[s][1]);
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}
// Split K groups, channel row 16 cb + r of Kb^T (tokens 32 s + 4 g .. + 3 and
// 32 s + 16 + 4 g .. + 3): slot (8 s + 4 h + g) ^ swizzle(16 cb + r), and the
// swizzle is linear, so the block part is a constant.
__device__ __forceinline__ bf16x8 ld_kbt(const unsigned char* lds, const LaneOffs& o, int base, int cb, int s)
{
    const int c0 = ((8 * s) ^ kbt_swz(16 * cb)) & 15, c1 = ((8 * s + 4) ^ kbt_swz(16 * cb)) & 15;
    const uint2 lo = lds_ld<uint2>(lds, base + 16 * cb * 128 + o.kbt_row + ((o.kbt_sl ^ c0) << 3));
    const uint2 hi = lds_ld<uint2>(lds, base + 16 * cb * 128 + o.kbt_row + ((o.kbt_sl ^ c1) << 3));
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}
// Operand from two accumulator blocks held by this lane (rows 4g..4g+3 of
// blocks 2s and 2s+1), rounded to bf16.
__device__ __forceinline__ bf16x8 pack_acc_pair(f32x4 lo, f32x4 hi)
{
    return as_bf16x8(make_uint4(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(hi[0], hi[1]),
                                pack2(hi[2], hi[3])));
}

__device__ __forceinline__ float lo_f(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float hi_f(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }
__device__ __forceinline__ void unpack8(const uint4 x, float* f)
{
    f[0] = lo_f(x.x);
    f[1] = hi_f(x.x);
    f[2] = lo_f(x.y);
    f[3] = hi_f(x.y);
    f[4] = lo_f(x.z);
    f[5] = hi_f(x.z);
    f[6] = lo_f(x.w);
    f[7] = hi_f(x.w);
}

// DPP moves on 32-bit values (all lanes read valid sources).
template <int CTRL>
__device__ __forceinline__ float dpp(float x)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadPrev = 0x90;   // quad_perm(0, 0, 1, 2): lane i <- lane i - 1 (lane 0 <- itself)
constexpr int kQuadPrev2 = 0x40;  // quad_perm(0, 0, 0, 1): lanes 2, 3 <- lanes 0, 1
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

// Minimum over the wavefront, returned as a wave-uniform value.
__device__ __forceinline__ float wave_min(float x)
{
    x = fminf(x, dpp<kRowRor8>(x));
    x = fminf(x, dpp<kRowRor4>(x));
    x = fminf(x, dpp<kRowRor2>(x));
    x = fminf(x, dpp<kRowRor1>(x));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 48));
    return fminf(fminf(r0, r1), fminf(r2, r3));
}

// Workgroup barrier for LDS traffic only.  The waves exchange data through
// LDS alone, so a wave waits for its own LDS accesses (lgkmcnt = 0) and meets
// the others at s_barrier; its global loads stay in flight across the barrier
// (a full __syncthreads() fence would also wait for them, draining the
// prefetch of the next chunk at every barrier).  The empty asm statements keep
// the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_barrier()
{
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// Raw buffer resources: one descriptor per tensor window, 32-bit per-lane
// offsets.  Reads past the window return zero and stores past it are dropped;
// the windows end at the last valid token of the chunk.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;  // 32-bit raw buffer, gfx9 family

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), kRsrcFlags);
}
__device__ __forceinline__ uint4 ld_b128(rsrc_t r, uint32_t off)
{
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0);
    return make_uint4(x[0], x[1], x[2], x[3]);
}

// One key wavefront's share of a chunk's inputs: key wavefront kw prepares
// tokens 16 kw .. 16 kw + 15; lane l takes tokens 16 kw + 4 (l & 3) + {0..3}
// and channels 8 (l >> 2) .. + 7 (a quad holds the wavefront's 16 tokens).
struct RawK {
    uint4 q[4], k[4], b[4];  // 8 bf16 channels per token
    uint4 a[4][2];           // alpha, 8 FP32 channels per token
};
// A value wavefront's share of v and w: wavefront w loads tokens 16 w + (l & 15),
// columns 16 (l >> 4) .. + 15 of the tile.
struct RawV {
    uint4 v[2], w[2];
};

// Global row of (token t0, head h) in [B*T, H] order.
__device__ __forceinline__ int64_t token_row(const ChunkArgs& a, int64_t brow, int64_t t0, int h)
{
    return (brow * a.T + t0) * a.H + h;
}

// Buffer windows of a chunk's key-side inputs (L valid tokens from row0).
struct RawSrc {
    rsrc_t q, k, b, a;
    uint32_t kstride;  // bytes per token, bf16 key rows
};
__device__ __forceinline__ RawSrc raw_src(const ChunkArgs& a, int64_t row0, int L)
{
    RawSrc s;
    s.kstride = uint32_t(a.H) * kDK * 2;
    const uint32_t win = uint32_t(L - 1) * s.kstride + kDK * 2;
    s.q = make_rsrc(static_cast<const bf16raw*>(a.q) + row0 * kDK, win);
    s.k = make_rsrc(static_cast<const bf16raw*>(a.k) + row0 * kDK, win);
    s.b = make_rsrc(static_cast<const bf16raw*>(a.b) + row0 * kDK, win);
    s.a = make_rsrc(a.alpha + row0 * kDK, 2 * win);
    return s;
}
// Loads this lane's token t (of four) of a chunk.
__device__ __forceinline__ void load_token(RawK& R, const RawSrc& s, int t, int kw, int lane)
{
    const int tp = lane & 3, cg = lane >> 2;
    const uint32_t tok = uint32_t(16 * kw + 4 * tp + t);
    const uint32_t off = tok * s.kstride + 16 * cg;
    R.q[t] = ld_b128(s.q, off);
    R.k[t] = ld_b128(s.k, off);
    R.b[t] = ld_b128(s.b, off);
    R.a[t][0] = ld_b128(s.a, 2 * tok * s.kstride + 32 * cg);
    R.a[t][1] = ld_b128(s.a, 2 * tok * s.kstride + 32 * cg + 16);
}

__device__ __forceinline__ void load_rawv(RawV& V, const ChunkArgs& a, int64_t row0, int L, int j0, int wave,
                                          int lane)
{
    const uint32_t vstride = uint32_t(a.H) * uint32_t(a.dv) * 2;
    const uint32_t win = uint32_t(L - 1) * vstride + kDVT * 2;
    const int64_t base = row0 * a.dv + j0;
    const rsrc_t rv = make_rsrc(static_cast<const bf16raw*>(a.v) + base, win);
    const rsrc_t rw = make_rsrc(static_cast<const bf16raw*>(a.w) + base, win);
    const uint32_t off = uint32_t(16 * wave + (lane & 15)) * vstride + 32 * (lane >> 4);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        V.v[u] = ld_b128(rv, off + 16 * u);
        V.w[u] = ld_b128(rw, off + 16 * u);
    }
}

// Alpha of channel c of token t of this lane (as prepared by decay_pass1).
__device__ __forceinline__ float alpha_at(const RawK& R, int t, int c)
{
    const uint4 x = R.a[t][c >> 2];
    return __uint_as_float((c & 3) == 0 ? x.x : (c & 3) == 1 ? x.y : (c & 3) == 2 ? x.z : x.w);
}

// First half of the key prep: decay products along the wavefront's 16 tokens
// (in lane, then a quad scan).  Writes the product over the 16 tokens to
// Ph[kw] (and wavefront 0 the product over tokens 0..7 to Ph[4]); returns in
// ex the product over the wavefront's tokens before this lane's four.
__device__ __forceinline__ void decay_pass1(unsigned char* lds, RawK& R, float* ex, int L, int kw, int lane)
{
    const int tp = lane & 3, cg = lane >> 2;
    // alpha clamped to [2^-15, 1], and 1 past the sequence end, written back
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const bool live = 16 * kw + 4 * tp + t < L;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            uint4& x = R.a[t][h];
            x.x = __float_as_uint(live ? __builtin_amdgcn_fmed3f(__uint_as_float(x.x), kAlphaMin, 1.0f) : 1.0f);
            x.y = __float_as_uint(live ? __builtin_amdgcn_fmed3f(__uint_as_float(x.y), kAlphaMin, 1.0f) : 1.0f);
            x.z = __float_as_uint(live ? __builtin_amdgcn_fmed3f(__uint_as_float(x.z), kAlphaMin, 1.0f) : 1.0f);
            x.w = __float_as_uint(live ? __builtin_amdgcn_fmed3f(__uint_as_float(x.w), kAlphaMin, 1.0f) : 1.0f);
        }
    }
    float inc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        float p = 1.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) p *= alpha_at(R, t, c);
        const float y = dpp<kQuadPrev>(p);
        const float x1 = tp >= 1 ? p * y : p;
        const float z = dpp<kQuadPrev2>(x1);
        inc[c] = tp >= 2 ? x1 * z : x1;  // tokens 16 kw .. 16 kw + 4 tp + 3
        const float e = dpp<kQuadPrev>(inc[c]);
        ex[c] = tp >= 1 ? e : 1.0f;      // tokens 16 kw .. 16 kw + 4 tp - 1
    }
    float* ph = reinterpret_cast<float*>(lds + kOffPh);
    if (tp == 3 || (kw == 0 && tp == 1)) {
        float* dst = ph + (tp == 3 ? kw : 4) * 128 + 8 * cg;
        *reinterpret_cast<float4*>(dst) = make_float4(inc[0], inc[1], inc[2], inc[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(inc[4], inc[5], inc[6], inc[7]);
    }
    // smallest decay over the 16 tokens among all channels (products are <= 1)
    float m = 1.0f;
    if (tp == 3) {
#pragma unroll
        for (int c = 0; c < 8; ++c) m = fminf(m, inc[c]);
    }
    m = wave_min(m);
    if (lane == 0) ph[5 * 128 + kw] = m;
}

// Chunk length (identical in every wavefront: the same four values in the
// same order): with m_j the smallest decay over block j (tokens 16 j ..
// 16 j + 15) among all channels, the longest of 64, 32, 16 tokens for which
// m_0 m_1 ... stays >= 2^-120, else 8; at most L.  The product of the minima
// bounds every channel's decay from below, so all factors of the chunk stay
// within [2^-120, 2^120].
__device__ __forceinline__ int chunk_step(const unsigned char* lds, int L)
{
    const float* pm = reinterpret_cast<const float*>(lds + kOffPh) + 5 * 128;
    const float g16 = pm[0], g32 = g16 * pm[1], g64 = g32 * pm[2] * pm[3];
    const int leff = g64 >= kRangeMin ? 64 : g32 >= kRangeMin ? 32 : g16 >= kRangeMin ? 16 : 8;
    return leff < L ? leff : L;
}

// Stores channels 8 cg .. 8 cg + 7 of one row of a [64][128] tile: two
// 8-byte pieces at their permuted positions.
__device__ __forceinline__ void st_row8(unsigned char* lds, int base, int row, int cg, uint4 v)
{
    lds_st<uint2>(lds, base + off_t128(row, chan_pos(8 * cg)), make_uint2(v.x, v.y));
    lds_st<uint2>(lds, base + off_t128(row, chan_pos(8 * cg + 4)), make_uint2(v.z, v.w));
}

// Zero rows of Et, Qt, Kt and zero columns of Kb^T for the four tokens from tok0.
__device__ __forceinline__ void zero_rows(unsigned char* lds, int kbt, int tok0, int cg)
{
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        st_row8(lds, kOffEt, tok0 + t, cg, zero);
        st_row8(lds, kOffQt, tok0 + t, cg, zero);
        st_row8(lds, kOffKt, tok0 + t, cg, zero);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) lds_st<uint2>(lds, kbt + off_kbt(8 * cg + c, tok0), make_uint2(0u, 0u));
}

// Rows of Et, Qt, Kt and columns of Kb^T for this lane's four tokens, given
// the decay before them (cum) and the chunk decay (gam).
__device__ __forceinline__ void prep_rows(unsigned char* lds, const RawK& R, float* cum, const float* gam, int kbt,
                                          int tok0, int cg)
{
    uint32_t kbp[2][8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        float q[8], k[8], b[8];
        unpack8(R.q[t], q);
        unpack8(R.k[t], k);
        unpack8(R.b[t], b);
        float et[8], qt[8], kt[8], kb[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            cum[c] *= alpha_at(R, t, c);  // 1 past the sequence end (decay_pass1)
            const float rc = __builtin_amdgcn_rcpf(cum[c]);
            et[c] = b[c] * k[c] * cum[c];
            qt[c] = q[c] * cum[c];
            kt[c] = k[c] * rc;
            kb[c] = kt[c] * gam[c];
        }
        st_row8(lds, kOffEt, tok0 + t, cg, make_uint4(pack2(et[0], et[1]), pack2(et[2], et[3]),
                                                         pack2(et[4], et[5]), pack2(et[6], et[7])));
        st_row8(lds, kOffQt, tok0 + t, cg, make_uint4(pack2(qt[0], qt[1]), pack2(qt[2], qt[3]),
                                                         pack2(qt[4], qt[5]), pack2(qt[6], qt[7])));
        st_row8(lds, kOffKt, tok0 + t, cg, make_uint4(pack2(kt[0], kt[1]), pack2(kt[2], kt[3]),
                                                         pack2(kt[4], kt[5]), pack2(kt[6], kt[7])));
        if (t & 1) {
#pragma unroll
            for (int c = 0; c < 8; ++c) kbp[t >> 1][c] = pack2(__uint_as_float(kbp[t >> 1][c]), kb[c]);
        } else {
#pragma unroll
            for (int c = 0; c < 8; ++c) kbp[t >> 1][c] = __float_as_uint(kb[c]);
        }
        __builtin_amdgcn_sched_barrier(0);  // one token's temporaries at a time
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) lds_st<uint2>(lds, kbt + off_kbt(8 * cg + c, tok0), make_uint2(kbp[0][c], kbp[1][c]));
}

// Decay factors and operand rows of this lane's four tokens (wavefront not
// entirely past the chunk); the chunk decay gamma (wavefront 4 writes it).
__device__ __forceinline__ void prep_factors_rows(unsigned char* lds, const RawK& R, const float* ex, int step,
                                                  int kbuf, int kw, int lane)
{
    const int tp = lane & 3, cg = lane >> 2;
    const float* ph = reinterpret_cast<const float*>(lds + kOffPh) + 8 * cg;
    const int tok0 = 16 * kw + 4 * tp;
    const int kbt = kOffKbT + kbuf * 16384;
    // gamma over the tokens the chunk covers; cum: decay before this lane's tokens
    // products of blocks 0 .. nw - 1 (gamma) and 0 .. kw - 1 (prefix), as
    // multiplications by 1 past the bound (no data-dependent loads)
    const int nw = step <= 8 ? 0 : (step + 15) >> 4;  // 0: the chunk ends inside tokens 0..7
    float gam[8], cum[8];
    const float4* p4 = reinterpret_cast<const float4*>(ph);  // row j, channels 8 cg ..: p4[32 j], p4[32 j + 1]
    const auto block = [&](int j, float* v) {
        const float4 a = p4[32 * j], b = p4[32 * j + 1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    };
#pragma unroll
    for (int c = 0; c < 8; ++c) gam[c] = cum[c] = 1.0f;
    if (nw == 0) block(4, gam);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (j < nw || j < kw) {  // uniform
            float v[8];
            block(j, v);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                if (j < nw) gam[c] *= v[c];
                if (j < kw) cum[c] *= v[c];
            }
        }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) cum[c] *= ex[c];
    if (kw == 0 && tp == 0) {
        float* gp = reinterpret_cast<float*>(lds + kOffGam) + kbuf * 128 + 8 * cg;
        *reinterpret_cast<float4*>(gp) = make_float4(gam[0], gam[1], gam[2], gam[3]);
        *reinterpret_cast<float4*>(gp + 4) = make_float4(gam[4], gam[5], gam[6], gam[7]);
    }
    // A chunk cut short (step < L) ends at a multiple of 8, so each lane's four
    // tokens are either all in it or all past it; the lanes past it write
    // zero rows (their decay factors are not formed).  Past the sequence end
    // (step = L) the inputs read as zero and alpha as 1, which gives zero rows.
    if (tok0 >= step)
        zero_rows(lds, kbt, tok0, cg);
    else
        prep_rows(lds, R, cum, gam, kbt, tok0, cg);
}

// Second half of the key prep: decay factors and the operand tiles of this
// lane's four tokens; the chunk decay gamma (wavefront 4 writes it).
__device__ __forceinline__ void prep_tiles(unsigned char* lds, const RawK& R, const float* ex, int step, int kbuf,
                                           int kw, int lane)
{
    const int tp = lane & 3, cg = lane >> 2;
    const int tok0 = 16 * kw + 4 * tp;
    const int kbt = kOffKbT + kbuf * 16384;
    if (16 * kw >= step)  // the whole wavefront lies past the chunk
        zero_rows(lds, kbt, tok0, cg);
    else
        prep_factors_rows(lds, R, ex, step, kbuf, kw, lane);
}

// z = w v of the chunk into Zs (rows past the chunk are masked when read).
__device__ __forceinline__ void prep_z(unsigned char* lds, const RawV& V, int wave, int lane)
{
    const int tok = 16 * wave + (lane & 15), cq = lane >> 4;
    float* zs = reinterpret_cast<float*>(lds + kOffZs);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        float v[8], w[8];
        unpack8(V.v[u], v);
        unpack8(V.w[u], w);
#pragma unroll
        for (int m = 0; m < 8; ++m) zs[zs_index(16 * cq + 8 * u + m, tok)] = v[m] * w[m];
    }
}

// One block of A or P (16 x 16 over K = 128 channels), formed transposed:
// D = Kt_J Row_I^T, which leaves row 16 I + r, columns 16 J + 4 g .. + 3 in
// each lane.
template <int KIND, int I, int J>  // KIND 0: A (rows Et), 1: P (rows Qt)
__device__ __forceinline__ void ap_block(unsigned char* lds, const LaneOffs& o, int buf, int r, int g)
{
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s)
        acc = mfma_bf16(ld_c128(lds, o, kOffKt, J, s), ld_c128(lds, o, KIND == 0 ? kOffEt : kOffQt, I, s), acc);
    const int row = 16 * I + r, col = 16 * J + 4 * g;
    if (KIND == 0) {
        lds_st<uint2>(lds, kOffAneg + buf * 8192 + off_rc64(row, col),
                      make_uint2(pack2(-acc[0], -acc[1]), pack2(-acc[2], -acc[3])));
    } else {
        float p[4] = {acc[0], acc[1], acc[2], acc[3]};
        if (I == J) {
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = col + i <= row ? p[i] : 0.f;
        }
        lds_st<uint2>(lds, kOffP + buf * 8192 + off_rc64(row, col), make_uint2(pack2(p[0], p[1]), pack2(p[2], p[3])));
    }
    __builtin_amdgcn_sched_barrier(0);  // one block's operands in flight at a time
}

// The six A blocks below the diagonal blocks and the ten P blocks on and below
// them, over value wavefronts 0..2 (grouped by shared operands).
__device__ __forceinline__ void ap_work(unsigned char* lds, const LaneOffs& o, int buf, int slot, int r, int g)
{
    switch (slot) {
        case 0:
            ap_block<1, 3, 3>(lds, o, buf, r, g);
            ap_block<1, 3, 2>(lds, o, buf, r, g);
            ap_block<1, 3, 1>(lds, o, buf, r, g);
            ap_block<1, 3, 0>(lds, o, buf, r, g);
            ap_block<0, 3, 2>(lds, o, buf, r, g);
            break;
        case 1:
            ap_block<1, 2, 2>(lds, o, buf, r, g);
            ap_block<1, 2, 1>(lds, o, buf, r, g);
            ap_block<1, 2, 0>(lds, o, buf, r, g);
            ap_block<0, 3, 1>(lds, o, buf, r, g);
            ap_block<0, 3, 0>(lds, o, buf, r, g);
            break;
        default:
            ap_block<1, 1, 1>(lds, o, buf, r, g);
            ap_block<1, 1, 0>(lds, o, buf, r, g);
            ap_block<1, 0, 0>(lds, o, buf, r, g);
            ap_block<0, 2, 1>(lds, o, buf, r, g);
            ap_block<0, 2, 0>(lds, o, buf, r, g);
            ap_block<0, 1, 0>(lds, o, buf, r, g);
            break;
    }
}

// Wavefront kTWave: the diagonal blocks A_II (strictly lower, FP32) and
// T_II = (I + A_II)^-1 by forward substitution; lane group g takes block g,
// lane r its column r.
__device__ __forceinline__ void t_work(unsigned char* lds, const LaneOffs& o, int buf, int r, int g)
{
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc = mfma_bf16(ld_c128(lds, o, kOffEt, I, s), ld_c128(lds, o, kOffKt, I, s), acc);
        // acc[i] = A_II[4g + i][r]: column r, rows 4g..4g+3, strictly lower part
        float4 v;
        v.x = 4 * g + 0 > r ? acc[0] : 0.f;
        v.y = 4 * g + 1 > r ? acc[1] : 0.f;
        v.z = 4 * g + 2 > r ? acc[2] : 0.f;
        v.w = 4 * g + 3 > r ? acc[3] : 0.f;
        lds_st<float4>(lds, kOffAd + (I * kTBlk + r * kT16 + 4 * g) * 4, v);
        __builtin_amdgcn_sched_barrier(0);
    }
    // Other lanes of this wavefront read the columns back: LDS accesses of one
    // wavefront complete in order; this keeps the compiler from reordering.
    __asm__ volatile("" ::: "memory");
    const float* adc = reinterpret_cast<const float*>(lds + kOffAd) + g * kTBlk;  // column j at adc + j * kT16
    const auto adt = [&](int j, int q4) { return *reinterpret_cast<const float4*>(adc + j * kT16 + 4 * q4); };
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = i == r ? 1.f : 0.f;
    float4 c0[4], c1[4];  // columns j and j + 1; column j + 2 is read during step j
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
        c0[q4] = adt(0, q4);
        c1[q4] = adt(1, q4);
    }
#pragma unroll
    for (int j = 0; j < 15; ++j) {
        float4 c2[4];
        if (j < 13)
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) c2[q4] = adt(j + 2, q4);
        const float col[16] = {c0[0].x, c0[0].y, c0[0].z, c0[0].w, c0[1].x, c0[1].y, c0[1].z, c0[1].w,
                               c0[2].x, c0[2].y, c0[2].z, c0[2].w, c0[3].x, c0[3].y, c0[3].z, c0[3].w};
#pragma unroll
        for (int i = j + 1; i < 16; ++i) t[i] -= col[i] * t[j];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
            c0[q4] = c1[q4];
            if (j < 13) c1[q4] = c2[q4];
        }
        __asm__ volatile("" ::: "memory");  // two columns ahead, no further
    }
    float* T = reinterpret_cast<float*>(lds + kOffT) + (buf * 4 + g) * kTBlk;
#pragma unroll
    for (int i = 0; i < 16; ++i) T[i * kT16 + r] = t[i];
}

// Value wavefront, chunk of lv tokens: X = Z - Et S (direct, rows past the
// chunk zero) and OT = (Qt S)^T.
__device__ __forceinline__ void value_xo(const unsigned char* lds, const LaneOffs& o, const f32x4* S, f32x4* X,
                                         f32x4* OT, int lv, int wave, int r, int g)
{
    bf16x8 sb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) sb[s] = pack_acc_pair(S[2 * s], S[2 * s + 1]);
    const float* zs = reinterpret_cast<const float*>(lds + kOffZs);
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        f32x4 xe = f32x4{0.f, 0.f, 0.f, 0.f}, xq = xe;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            xe = mfma_bf16(ld_c128(lds, o, kOffEt, I, s), sb[s], xe);
            xq = mfma_bf16(sb[s], ld_c128(lds, o, kOffQt, I, s), xq);
        }
        const float4 z = *reinterpret_cast<const float4*>(zs + zs_index(16 * wave + r, 16 * I + 4 * g));
        const int t0 = 16 * I + 4 * g;
        X[I] = f32x4{t0 + 0 < lv ? z.x - xe[0] : 0.f, t0 + 1 < lv ? z.y - xe[1] : 0.f,
                     t0 + 2 < lv ? z.z - xe[2] : 0.f, t0 + 3 < lv ? z.w - xe[3] : 0.f};
        OT[I] = xq;
    }
}

// Value wavefront, rest of the chunk: blocked solve, output rows and state
// update, from the tiles of buffer vbuf.
__device__ __forceinline__ void value_solve(const unsigned char* lds, const LaneOffs& o, f32x4* S, const f32x4* X,
                                            const f32x4* OT, int vbuf, rsrc_t ro, int ostride, int lv, int wave, int r,
                                            int g)
{
    const int aneg = kOffAneg + vbuf * 8192, pb = kOffP + vbuf * 8192;
    const int tb = kOffT + vbuf * 4 * kTBlk * 4, kbt = kOffKbT + vbuf * 16384;
    // ---- blocked solve: R_I = X_I - sum_J A_IJ U_J ; U_I = T_II R_I
    f32x4 U[4];
    bf16x8 ub[2];
    const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        f32x4 R_ = X[I];
        if (I >= 1) R_ = mfma_bf16(ld_s64(lds, o, aneg, I, 0), ub[0], R_);
        if (I >= 3) R_ = mfma_bf16(ld_s64(lds, o, aneg, I, 1), ub[1], R_);
        const float4 tr = lds_ld<float4>(lds, tb + (I * kTBlk + r * kT16 + 4 * g) * 4);
        f32x4 u = zero4;
        u = mfma_f32(tr.x, R_[0], u);
        u = mfma_f32(tr.y, R_[1], u);
        u = mfma_f32(tr.z, R_[2], u);
        u = mfma_f32(tr.w, R_[3], u);
        U[I] = u;
        // operands over tokens 0..31 and 32..63; blocks not solved yet stay zero
        if (I == 0) ub[0] = pack_acc_pair(U[0], zero4);
        if (I == 1) ub[0] = pack_acc_pair(U[0], U[1]);
        if (I == 2) ub[1] = pack_acc_pair(U[2], zero4);
        if (I == 3) ub[1] = pack_acc_pair(U[2], U[3]);
    }
    // ---- O^T = (Qt S)^T + U^T P^T; lane holds token 16 I + r, columns 4g..4g+3
    const int o_vo = r * ostride + (16 * wave + 4 * g) * 2;
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        f32x4 acc2 = OT[I];
        acc2 = mfma_bf16(ub[0], ld_s64(lds, o, pb, I, 0), acc2);
        if (I >= 2) acc2 = mfma_bf16(ub[1], ld_s64(lds, o, pb, I, 1), acc2);
        if (16 * I + r < lv) {
            u32x2 pk;
            pk[0] = pack2(acc2[0], acc2[1]);
            pk[1] = pack2(acc2[2], acc2[3]);
            __builtin_amdgcn_raw_buffer_store_b64(pk, ro, o_vo, 16 * I * ostride, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    // ---- S <- Diag(gamma) S + Kb^T U
    const float* gam = reinterpret_cast<const float*>(lds + kOffGam) + vbuf * 128;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
        const float4 gm = *reinterpret_cast<const float4*>(gam + 16 * cb + 4 * g);
        f32x4 acc3 = f32x4{S[cb][0] * gm.x, S[cb][1] * gm.y, S[cb][2] * gm.z, S[cb][3] * gm.w};
        acc3 = mfma_bf16(ld_kbt(lds, o, kbt, cb, 0), ub[0], acc3);
        acc3 = mfma_bf16(ld_kbt(lds, o, kbt, cb, 1), ub[1], acc3);
        S[cb] = acc3;
        if (cb & 1) __builtin_amdgcn_sched_barrier(0);
    }
}

__global__ __launch_bounds__(kThreads) void chunk_fwd_mfma_kernel(ChunkArgs a, int ntiles, int nchains)
{
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane0 = tid & 63;
    const int g0 = lane0 >> 4, r0 = lane0 & 15;
    const bool vwave = wave < kValueWaves;
    const int kw = wave - kValueWaves;

    // XCD-aware mapping: all tiles of a chain share blockIdx.x % 8.
    const int bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int tile = slot % ntiles;
    const int chain = (slot / ntiles) * 8 + xcd;
    if (chain >= nchains) return;
    const int n = chain / a.H, h = chain % a.H;
    const int j0 = tile * kDVT;
    const int64_t dv = a.dv;

    int64_t bos, eos, brow;
    sequence_bounds(a.cu_seqlens, n, a.T, bos, eos, brow);

    // The blocks the solve and the output read as zero (A on the diagonal, P
    // right of it) are never written: clear Aneg and P, both buffers, once.
    {
        uint4* z = reinterpret_cast<uint4*>(lds + kOffAneg);
        const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int i = 0; i < 4; ++i) z[tid + i * kThreads] = zero;  // 4 x 512 x 16 = 32768 bytes
    }

    // Both roles run the same sequence of periods (the loop control is
    // computed identically) and meet at the same three barriers per period;
    // separate loops keep each role's registers apart.
    int64_t tk = bos;  // chunk the key side prepares this period
    int64_t tv = -1;   // chunk the value side finishes this period (< 0: none)
    int kbuf = 0;      // buffer the key side writes this period; the value side reads kbuf ^ 1
    if (vwave) {
        // state slice of a value wavefront: channels 16 cb + 4 g + i, column j0 + 16 wave + r
        f32x4 S[8];
        const int64_t sbase = (int64_t(n) * a.H + h) * kDK * dv + j0;
        const uint32_t sbytes = uint32_t(kDK * dv * 4);
        const int s_vo = ((4 * g0) * int(dv) + 16 * wave + r0) * 4;
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) S[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (a.initial_state) {
            const rsrc_t rs = make_rsrc(a.initial_state + sbase, sbytes);
#pragma unroll
            for (int cb = 0; cb < 8; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[cb][i] = __uint_as_float(
                        __builtin_amdgcn_raw_buffer_load_b32(rs, s_vo, (16 * cb + i) * int(dv) * 4, 0));
        }

        bf16raw* o = static_cast<bf16raw*>(a.o);
        const int ostride = a.H * int(dv) * 2;
        RawV V;
        int lv = 0;  // length of chunk tv
        if (tk < eos) load_rawv(V, a, token_row(a, brow, tk, h), int(eos - tk < kC ? eos - tk : kC), j0, wave, lane0);
        while (tk < eos || tv >= 0) {
            const bool has_k = tk < eos, has_v = tv >= 0;
            const int L = has_k ? int(eos - tk < kC ? eos - tk : kC) : 0;
            lds_barrier();  // B0: z and all tiles of chunk tv visible
            // Lane indices made opaque per period, so that the LDS addresses
            // derived from them are recomputed here rather than held in
            // registers across the whole loop.
            int r = r0, g = g0, lane = lane0;
            __asm__ volatile("" : "+v"(r), "+v"(g), "+v"(lane));
            f32x4 X[4], OT[4];  // per period (not carried across periods)
            if (has_v) value_xo(lds, lane_offsets(r, g), S, X, OT, lv, wave, r, g);
            lds_barrier();  // B1: decay products visible; Et, Qt and z of chunk tv consumed
            int step = 0;
            if (has_k) step = chunk_step(lds, L);
            if (has_v) {
                const rsrc_t ro = make_rsrc(o + token_row(a, brow, tv, h) * dv + j0,
                                            uint32_t(lv - 1) * uint32_t(ostride) + kDVT * 2);
                value_solve(lds, lane_offsets(r, g), S, X, OT, kbuf ^ 1, ro, ostride, lv, wave, r, g);
            }
            if (has_k) {
                prep_z(lds, V, wave, lane);
                const int64_t tn = tk + step;  // v, w of the next chunk
                if (tn < eos)
                    load_rawv(V, a, token_row(a, brow, tn, h), int(eos - tn < kC ? eos - tn : kC), j0, wave, lane);
            }
            lds_barrier();  // B2: tiles of chunk tk visible
            if (has_k) {
                const LaneOffs lk = lane_offsets(r, g);
                if (wave == kTWave)
                    t_work(lds, lk, kbuf, r, g);
                else
                    ap_work(lds, lk, kbuf, wave, r, g);
            }
            tv = has_k ? tk : -1;
            lv = step;
            tk = has_k ? tk + step : eos;
            kbuf ^= 1;
        }
        if (a.final_state) {
            const rsrc_t rs = make_rsrc(a.final_state + sbase, sbytes);
#pragma unroll
            for (int cb = 0; cb < 8; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[cb][i]), rs, s_vo,
                                                          (16 * cb + i) * int(dv) * 4, 0);
        }
    } else {
        RawK R;
        if (tk < eos) {
            const RawSrc src = raw_src(a, token_row(a, brow, tk, h), int(eos - tk < kC ? eos - tk : kC));
#pragma unroll
            for (int t = 0; t < 4; ++t) load_token(R, src, t, kw, lane0);
        }
        while (tk < eos || tv >= 0) {
            const bool has_k = tk < eos;
            const int L = has_k ? int(eos - tk < kC ? eos - tk : kC) : 0;
            lds_barrier();  // B0
            int r = r0, g = g0, lane = lane0;  // opaque per period (see the value loop)
            __asm__ volatile("" : "+v"(r), "+v"(g), "+v"(lane));
            float ex[8];  // per period
            if (has_k) decay_pass1(lds, R, ex, L, kw, lane);
            lds_barrier();  // B1
            int step = 0;
            if (has_k) {
                step = chunk_step(lds, L);
                prep_tiles(lds, R, ex, step, kbuf, kw, lane);
            }
            lds_barrier();  // B2
            // The next chunk's inputs, issued while the value waves form its
            // matrix blocks; they stay in flight until decay_pass1.
            const int64_t tn = tk + step;
            if (has_k && tn < eos) {
                const RawSrc nxt = raw_src(a, token_row(a, brow, tn, h), int(eos - tn < kC ? eos - tn : kC));
#pragma unroll
                for (int t = 0; t < 4; ++t) load_token(R, nxt, t, kw, lane);
            }
            tv = has_k ? tk : -1;
            tk = has_k ? tk + step : eos;
            kbuf ^= 1;
        }
    }

}

}  // namespace

bool chunk_fwd_mfma_supported(const ChunkArgs& a, bool bf16)
{
    return bf16 && a.dk == kDK && a.dv % kDVT == 0;
}

hipError_t launch_chunk_fwd_mfma(const ChunkArgs& a, hipStream_t stream)
{
    // Allow the kernel its > 64 KiB of dynamic LDS (thread-safe one-time call).
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_fwd_mfma_kernel),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (attr != hipSuccess) return attr;
    const int ntiles = a.dv / kDVT;
    const int64_t chains = int64_t(a.N) * a.H;
    const int64_t blocks = (chains + 7) / 8 * 8 * ntiles;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(chunk_fwd_mfma_kernel, dim3(unsigned(blocks)), dim3(kThreads), kLdsBytes, stream, a, ntiles,
                       int(chains));
    return hipGetLastError();
}

}  // namespace gdn2
