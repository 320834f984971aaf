// Chunkwise forward on gfx950 matrix cores (bf16 inputs, dk = 128, value
// tiles of 64 columns).
//
// The chunkwise WY form (Gated DeltaNet-2 analysis, iplexlaw.co.kr, "Token
// processing and parallel training"): inside a chunk the running product of
// each key channel's decay is folded into the row factors and, inverted, into
// the column factors, so one lower-triangular solve and a few dense products
// remain; the decay, the solve and the carried state stay in FP32.  With incoming state S, per key channel the running decay
// c_i = prod_{m<=i} alpha_m inside the chunk, e = b k and z = w v:
//     Et_i = e_i c_i     Qt_i = q_i c_i     Kt_j = k_j / c_j     gamma = c_last
//     A = strict_lower(Et Kt^T)     P = lower(Qt Kt^T)
//     U = (I + A)^-1 (Z - Et S)     O = Qt S + P U     S <- Diag(gamma) (S + Kt^T U)
// (the last is Diag(gamma) S + Kb^T U with Kb_j = Kt_j gamma, the form the
// pages' decayed keys take).
//
// Range.  alpha is clamped to [2^-15, 1].  A chunk is cut short when some
// channel decays below 2^-64 across it: it then covers 32, 16 or 8 tokens,
// the longest prefix whose decay stays at or above 2^-64 in every channel (8
// tokens always do).  Hence every factor c_i and 1 / c_j lies in
// [2^-64, 2^64], which FP32 and bf16 represent, S + Kt^T U stays far below the
// FP32 range, and all factors are plain products of alpha (one reciprocal per
// channel and lane).  All waves take the decision from the same exchanged
// products, so it is uniform across the workgroup.
//
// Pipeline.  One workgroup of twelve wavefronts (three per SIMD) per
// (sequence, head, 64-column value tile).  Waves 0..3 (value waves) own 16
// value columns each and keep that 128 x 16 slice of the FP32 state in MFMA
// accumulators for the whole sequence; waves 4..11 (key waves) prepare the
// chunks, each 16 tokens x 64 channels.  Each period of two barriers B0, B1
// advances two chunks.  Between B0 and B1 the value waves finish chunk c - 1
// block by block (X = Z - Et S, the blocked solve, the output rows, (Qt S)^T)
// and update the state, while the key waves form the tiles Et, Qt, Kt of chunk
// c; after B1 the value waves form the A and P blocks of chunk c and the
// inverses of its diagonal blocks, while the key waves store its z = w v and
// form the decay products of chunk c + 1, so that its length is known at the
// next B0.  Et, Qt, Kt, z and gamma are double-buffered (the state update
// reads the previous chunk's Kt as Kt^T, through the transposing LDS load);
// A, P and T are written and read in different halves of the period and stay
// single.  Global loads go out in both halves so that the memory pipe stays
// busy: alpha and q of the next chunk during the prep, as registers free up,
// and its k, b, v and w after B1.  Workgroups of one chain share an XCD, so
// the second value tile re-reads the key-side inputs from L2.
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
typedef __attribute__((address_space(3))) f32x4 lds_f4;  // four floats in LDS
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;  // four 16-bit values in LDS

constexpr int kDK = 128;          // key head size
constexpr int kC = 64;            // chunk
constexpr int kDVT = 64;          // value columns per workgroup
constexpr int kWaves = 12;        // wavefronts per workgroup (three per SIMD)
constexpr int kThreads = 64 * kWaves;
constexpr int kValueWaves = 4;    // waves 0..3: 16 value columns each
constexpr int kKeyWaves = 8;      // waves 4..11: 16 tokens x 64 channels each
constexpr int kTWave = 3;         // diagonal blocks of A and their inverses (a value wave)
constexpr float kAlphaMin = 0x1p-15f;
constexpr float kRangeMin = 0x1p-64f;

// ---- LDS map (bytes) -------------------------------------------------------
constexpr int kOffEt = 0;          // [2][64][128] bf16
constexpr int kOffQt = 32768;      // [2][64][128] bf16
constexpr int kOffKt = 65536;      // [2][64][128] bf16
constexpr int kOffAneg = 98304;    // [64][64] bf16 (-A below the diagonal blocks)
constexpr int kOffP = 106496;      // [64][64] bf16
constexpr int kT16 = 20;            // floats per row of a 16 x 16 FP32 block (padded)
constexpr int kTBlk = 16 * kT16 + 16;  // floats per padded block (the next block shifts by 16 banks)
constexpr int kOffT = 114688;      // [4][kTBlk] f32, T_II row major
constexpr int kOffAd = kOffT;   // [4][kTBlk] f32, diagonal blocks of A, column major; the same wave
                                // reads them all before it overwrites them with T
constexpr int kOffGam = kOffT + 4 * kTBlk * 4;  // [2][128] f32 (chunk decay per channel)
constexpr int kOffPh = kOffGam + 1024;  // [7][128] f32: decay over tokens 16 j .. 16 j + 15 (rows j < 4),
                                        // over 0..7 (row 4), per-block channel minima (row 5), ones (row 6)
constexpr int kPhOnes = 6;
constexpr int kOffZs = kOffPh + 3584;   // [2][value wavefront][16 columns][64 tokens] f32 (zs_off), z = w v
constexpr int kZsWave = 16 * 64 * 4;
constexpr int kZsBuf = kValueWaves * kZsWave;
constexpr int kLdsBytes = kOffZs + 2 * kZsBuf;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
static_assert(kOffP == kOffAneg + 8192 && kOffT == kOffP + 8192, "Aneg and P are cleared as one range");
static_assert(kOffZs % 16 == 0 && kZsWave % 256 == 0 && kZsBuf % 256 == 0 && (kOffZs & 0xF0) == 0,
              "16-byte aligned z rows; granule bits of the z base clear (store_z)");

// [64][128] bf16 tiles Et, Qt, Kt.  Channels are stored permuted within each
// group of 32 so that the split K groups of the matrix products, channels
// {32 s + 4 g .. + 3} U {32 s + 16 + 4 g .. + 3}, occupy the 16 contiguous bytes
// at position 32 s + 8 g; the 16-byte granules are XOR-swizzled by a linear
// map of the low four row bits.  Measured on gfx950: 16-byte reads of 16 rows
// at one granule column stay free of bank conflicts only when neighbouring
// lanes (rows 2j, 2j + 1) land on granules that differ in bit 0 alone, and the
// prep stores (two 8-byte pieces per lane, rows 4 apart across a quad) need
// the images of rows 4 and 8 to stay apart; the map row ^ (bit 2 ^ bit 3)
// meets both.
__device__ __forceinline__ int chan_pos(int ch)
{
    return (ch & ~31) | ((ch & 12) << 1) | ((ch & 16) >> 2) | (ch & 3);
}
__device__ __forceinline__ int tile_swz(int row)
{
    return (row ^ (((row >> 2) ^ (row >> 3)) & 1)) & 15;
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

// Byte offset of (column, token) in a value wavefront's z: the 16-byte token
// granules XOR-swizzled by the column, so that the token-wise stores (b32, one
// column) and the column-wise operand reads (16 columns at one granule, b128)
// are free of bank conflicts.
__device__ __forceinline__ int zs_off(int col, int tok)
{
    return col * 256 + ((((tok >> 2) ^ col) & 15) << 4) + ((tok & 3) << 2);
}

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
// compile-time constant (tile base and 16 k rows) -- except in the transposed
// reads of Kt, whose granule also takes the channel block (a constant XOR,
// see ld_ktr).
struct LaneOffs {
    int c128[4];     // [64][128] tile, positions 32 s + 8 g .. + 7 (16 bytes)
    int s64[2][2];   // [64][64] tile, columns 32 s + 16 h + 4 g .. + 3 (8 bytes)
    int ktr;         // Kt read transposed: row 4 g + (r >> 2), piece r & 3 (see ld_ktr)
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
    {
        const int row = 4 * g + (r >> 2);
        o.ktr = row * 256 + ((((r & 3) ^ tile_swz(row)) & 15) << 4);
    }
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
// Split K groups of Kt^T, channel row 16 cb + r (tokens 32 s + 4 g .. + 3 and
// 32 s + 16 + 4 g .. + 3), read straight from the token-major Kt tile with
// gfx950's transposing LDS load (ds_read_b64_tr_b16): in each group of 16
// lanes, lane 4 j + q reads the eight bytes of row t0 + j that hold
// channels 16 cb + 4 q .. + 3, and lane r receives channel 16 cb + r of those
// four rows (lane layout checked on the GPU with an in-bounds probe).  Those
// four channels sit at positions 32 (cb >> 1) + 8 q + 4 (cb & 1) .. + 3, in
// granule (4 (cb >> 1) + q) ^ tile_swz(row), and tile_swz(row) depends only
// on row & 15 = 4 g + j: the channel block enters as a constant XOR on the
// granule bits.
__device__ __forceinline__ bf16x8 ld_ktr(const unsigned char* lds, const LaneOffs& o, int base, int cb, int s)
{
    const int off = base + (o.ktr ^ ((cb >> 1) << 6)) + 8 * (cb & 1) + 32 * s * 256;
    const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds + off));
    const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(lds + off + 16 * 256));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}
// Operand from two accumulator blocks held by this lane (rows 4g..4g+3 of
// blocks 2s and 2s+1), rounded to bf16.
__device__ __forceinline__ bf16x8 pack_acc_pair(f32x4 lo, f32x4 hi)
{
    return as_bf16x8(make_uint4(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(hi[0], hi[1]),
                                pack2(hi[2], hi[3])));
}
// The same, keeping the lower block of an existing operand (its first four
// elements) and replacing the upper block.
__device__ __forceinline__ bf16x8 pack_acc_pair_hi(bf16x8 keep, f32x4 hi)
{
    const uint4 k = __builtin_bit_cast(uint4, keep);
    return as_bf16x8(make_uint4(k.x, k.y, pack2(hi[0], hi[1]), pack2(hi[2], hi[3])));
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
constexpr int kRowRor1 = 0x121, kRowRor2 = 0x122, kRowRor4 = 0x124, kRowRor8 = 0x128;

// x <- x * x[lane - K] within the row of 16 lanes; a lane whose source lies
// outside its row keeps x (bound control off: the DPP result is not written
// there).  A DPP operand that a vector instruction has just written needs two
// wait states.
template <int K>
__device__ __forceinline__ void scan_mul(float& x)
{
    static_assert(K == 2 || K == 4 || K == 8, "row shift");
    if (K == 2) __asm__ volatile("s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shr:2 row_mask:0xf bank_mask:0xf" : "+v"(x));
    if (K == 4) __asm__ volatile("s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shr:4 row_mask:0xf bank_mask:0xf" : "+v"(x));
    if (K == 8) __asm__ volatile("s_nop 1\n\tv_mul_f32_dpp %0, %0, %0 row_shr:8 row_mask:0xf bank_mask:0xf" : "+v"(x));
}
// x[lane - 2] within the row of 16 lanes, or 1 where that lies outside it.
__device__ __forceinline__ float scan_prev(float x)
{
    float e = 1.0f;
    __asm__ volatile("s_nop 1\n\tv_mov_b32_dpp %0, %1 row_shr:2 row_mask:0xf bank_mask:0xf" : "+v"(e) : "v"(x));
    return e;
}

// The smaller of two decay products.  These are non-negative and finite (the
// clamped alpha and products of it, possibly denormal or zero), and for such
// floats the order of the bit patterns as unsigned integers is the numeric
// order: one integer minimum, without the NaN canonicalisation of fminf.
__device__ __forceinline__ float min_decay(float a, float b)
{
    return __uint_as_float(min(__float_as_uint(a), __float_as_uint(b)));
}
// Minimum of decay products over the wavefront, returned as a wave-uniform
// value (integer minima as in min_decay; the last four on the scalar unit).
__device__ __forceinline__ float wave_min(float x)
{
    uint32_t u = __float_as_uint(x);
    u = min(u, uint32_t(__builtin_amdgcn_mov_dpp(int(u), kRowRor8, 0xF, 0xF, true)));
    u = min(u, uint32_t(__builtin_amdgcn_mov_dpp(int(u), kRowRor4, 0xF, 0xF, true)));
    u = min(u, uint32_t(__builtin_amdgcn_mov_dpp(int(u), kRowRor2, 0xF, 0xF, true)));
    u = min(u, uint32_t(__builtin_amdgcn_mov_dpp(int(u), kRowRor1, 0xF, 0xF, true)));
    const uint32_t r0 = __builtin_amdgcn_readlane(int(u), 0), r1 = __builtin_amdgcn_readlane(int(u), 16);
    const uint32_t r2 = __builtin_amdgcn_readlane(int(u), 32), r3 = __builtin_amdgcn_readlane(int(u), 48);
    return __uint_as_float(min(min(r0, r1), min(r2, r3)));
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

// Every window in this kernel is the same in all lanes of a wavefront (it
// depends on the chain, the chunk and the wavefront's role only); taking the
// first lane's value keeps the descriptor in scalar registers, where the
// buffer instructions need it, instead of a per-lane loop over descriptors.
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(p)), hi = __builtin_amdgcn_readfirstlane(uint32_t(p >> 32));
    void* pu = reinterpret_cast<void*>((uint64_t(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(pu, (short)0, int(__builtin_amdgcn_readfirstlane(bytes)), kRsrcFlags);
}
__device__ __forceinline__ uint4 ld_b128(rsrc_t r, uint32_t off)
{
    const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, int(off), 0, 0);
    return make_uint4(x[0], x[1], x[2], x[3]);
}

// One key wavefront's share of a chunk's inputs: key wavefront kw prepares
// tokens 16 tb .. 16 tb + 15 (tb = kw & 3) in channels 64 ch .. 64 ch + 63
// (ch = kw >> 2); lane l takes tokens 16 tb + 2 tp + {0, 1} and channels
// 64 ch + 8 cg .. + 7 with tp = (l >> 1) & 7 and cg = (l & 1) + 2 (l >> 4):
// each row of 16 lanes holds the block's 16 tokens of two channel groups,
// interleaved (see decay_pass1), and each half-wavefront the same tokens and
// channel groups as with consecutive lanes, so the loads and the prep's LDS
// stores touch the same addresses per half-wavefront.
//
// Gate layouts (template parameter G, gdn2_gate_flags): a scalar gate is one
// value per token and head, read once per token and applied to every channel
// of its axis.  A scalar erase gate sits in b[t].x (bf16 bits), a scalar or
// tied write gate in w.x of RawVK, a scalar decay in a[t][0].x.
struct RawK {
    uint4 q[2], k[2], b[2];  // 8 bf16 channels per token
    uint4 a[2][2];           // alpha, 8 FP32 channels per token
};
// v and w of 32 of the workgroup's 64 value columns, loaded by every key
// wavefront (its channel half ch picks the 32-column block u = ch, so that the
// two key wavefronts of a SIMD carry the same work and issue the same loads):
// tokens 16 tb + (l & 15), columns 32 u + 8 (l >> 4) .. + 7 of the tile.
struct RawVK {
    uint4 v, w;
};
struct KeyLane {
    int tb, ch, tp, cg;
    int tok0;  // 16 tb + 2 tp
    int c0;    // first channel: 64 ch + 8 cg
};
__device__ __forceinline__ KeyLane key_lane(int kw, int lane)
{
    KeyLane k;
    k.tb = kw & 3;
    k.ch = kw >> 2;
    k.tp = (lane >> 1) & 7;                   // the two channel groups of a
    k.cg = (lane & 1) | ((lane >> 4) << 1);   // row of 16 lanes interleave
    k.tok0 = 16 * k.tb + 2 * k.tp;
    k.c0 = 64 * k.ch + 8 * k.cg;
    return k;
}

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
template <int G>
__device__ __forceinline__ RawSrc raw_src(const ChunkArgs& a, int64_t row0, int L)
{
    RawSrc s;
    s.kstride = uint32_t(a.H) * kDK * 2;
    const uint32_t win = L > 0 ? uint32_t(L - 1) * s.kstride + kDK * 2 : 0u;  // 0: every load reads zero
    const uint32_t rows = L > 0 ? uint32_t(L - 1) * uint32_t(a.H) + 1 : 0u;   // per-token scalars
    s.q = make_rsrc(static_cast<const bf16raw*>(a.q) + row0 * kDK, win);
    s.k = make_rsrc(static_cast<const bf16raw*>(a.k) + row0 * kDK, win);
    if (G & kScalarErase)
        s.b = make_rsrc(static_cast<const bf16raw*>(a.b) + row0, 2 * rows);
    else
        s.b = make_rsrc(static_cast<const bf16raw*>(a.b) + row0 * kDK, win);
    if (G & kScalarDecay)
        s.a = make_rsrc(a.alpha + row0, 4 * rows);
    else
        s.a = make_rsrc(a.alpha + row0 * kDK, 2 * win);
    return s;
}
// Loads token t (of two) of this lane: q, k, b, and alpha.
__device__ __forceinline__ void load_q(RawK& R, const RawSrc& s, int t, const KeyLane& K)
{
    R.q[t] = ld_b128(s.q, uint32_t(K.tok0 + t) * s.kstride + 2 * K.c0);
}
template <int G>
__device__ __forceinline__ void load_kb(RawK& R, const RawSrc& s, int t, const KeyLane& K)
{
    const uint32_t off = uint32_t(K.tok0 + t) * s.kstride + 2 * K.c0;
    R.k[t] = ld_b128(s.k, off);
    if (G & kScalarErase)  // one bf16 per token (the token stride of a scalar row is kstride / 128)
        R.b[t].x = __builtin_amdgcn_raw_buffer_load_b16(s.b, int(uint32_t(K.tok0 + t) * (s.kstride >> 7)), 0, 0);
    else
        R.b[t] = ld_b128(s.b, off);
}
template <int G>
__device__ __forceinline__ void load_alpha(RawK& R, const RawSrc& s, int t, const KeyLane& K)
{
    if (G & kScalarDecay) {  // one FP32 decay per token
        R.a[t][0].x = __builtin_amdgcn_raw_buffer_load_b32(s.a, int(uint32_t(K.tok0 + t) * (s.kstride >> 6)), 0, 0);
        return;
    }
    const uint32_t off = 2 * uint32_t(K.tok0 + t) * s.kstride + 4 * K.c0;
    R.a[t][0] = ld_b128(s.a, off);
    R.a[t][1] = ld_b128(s.a, off + 16);
}

template <int G, bool SEG>
__device__ __forceinline__ void load_vk(RawVK& V, const ChunkArgs& a, int64_t row0, int L, int j0, int kw, int lane)
{
    const int u = kw >> 2;  // 32-column block
    const int dvio = SEG && a.dv_io > 0 ? a.dv_io : a.dv;
    const bool real = !SEG || j0 < dvio;
    const uint32_t vstride = uint32_t(a.H) * uint32_t(dvio) * 2;
    // map columns (j0 >= dv_io) have no v, w: an empty window reads zeros, so z = 0
    const uint32_t win = L > 0 && real ? uint32_t(L - 1) * vstride + kDVT * 2 : 0u;
    const int64_t base = row0 * dvio + (real ? j0 : 0);
    const uint32_t tok = uint32_t(16 * (kw & 3) + (lane & 15));
    const rsrc_t rv = make_rsrc(static_cast<const bf16raw*>(a.v) + base, win);
    const uint32_t off = tok * vstride + 2 * (8 * (lane >> 4)) + 64 * u;
    if (G & (kTied | kScalarWrite)) {  // the token's scalar write gate (tied: its erase gate)
        const uint32_t rows = L > 0 && real ? uint32_t(L - 1) * uint32_t(a.H) + 1 : 0u;
        const rsrc_t rg = make_rsrc(static_cast<const bf16raw*>(G & kTied ? a.b : a.w) + row0, 2 * rows);
        V.v = ld_b128(rv, off);
        V.w.x = __builtin_amdgcn_raw_buffer_load_b16(rg, int(tok * uint32_t(a.H) * 2), 0, 0);
    } else {
        const rsrc_t rw = make_rsrc(static_cast<const bf16raw*>(a.w) + base, win);
        V.v = ld_b128(rv, off);
        V.w = ld_b128(rw, off);
    }
}
// z = w v of this key lane's eight columns into buffer buf of the z of the
// value wavefront that owns them (rows past the chunk are masked when read).
//
// The lane's columns are c8 + m (c8 = 0 or 8, m < 8), so zs_off(c8 + m, tok)
// = base + 256 m + (((tok >> 2) ^ c8 ^ m) << 4) with base free of bits 4..7:
// one XOR with a constant per store, the column step in the offset field.
template <int G>
__device__ __forceinline__ void store_z(unsigned char* lds, const RawVK& V, int buf, int kw, int lane)
{
    const int tok = 16 * (kw & 3) + (lane & 15);
    const int c8 = 8 * ((lane >> 4) & 1);
    // zs_off(c8, tok) in the z of value wavefront 2 u + (lane >> 5), the owner
    // of columns 32 u + 8 (lane >> 4) .. + 7
    const int base = kOffZs + buf * kZsBuf + (2 * (kw >> 2) + (lane >> 5)) * kZsWave + c8 * 256 +
                     ((tok & 3) << 2) + ((((tok >> 2) ^ c8) & 15) << 4);
    float v[8], w[8];
    unpack8(V.v, v);
    if (G & (kTied | kScalarWrite)) {
#pragma unroll
        for (int m = 0; m < 8; ++m) w[m] = lo_f(V.w.x);
    } else {
        unpack8(V.w, w);
    }
#pragma unroll
    for (int m = 0; m < 8; ++m) lds_st<float>(lds + 256 * m, base ^ (m << 4), v[m] * w[m]);
}

// Alpha of channel c of token t of this lane, as loaded.
template <int G>
__device__ __forceinline__ float raw_alpha(const RawK& R, int t, int c)
{
    if (G & kScalarDecay) return __uint_as_float(R.a[t][0].x);
    const uint4 x = R.a[t][c >> 2];
    return __uint_as_float((c & 3) == 0 ? x.x : (c & 3) == 1 ? x.y : (c & 3) == 2 ? x.z : x.w);
}

// Decay products of a chunk along the key wavefront's 16 tokens (in lane,
// then a scan over the eight lanes of a channel group).  Writes the product
// over the block to Ph[tb] (and, for block 0, the product over tokens 0..7 to
// Ph[4]) for this wavefront's channels and its smallest block product to
// Ph[5][2 tb + ch]; returns the clamped alpha in al and in ex the product over
// the block's tokens before this lane's two.
template <int G>
__device__ __forceinline__ void decay_pass1(unsigned char* lds, const RawK& R, float (*al)[8], float* ex, int L,
                                            const KeyLane& K, int lane)
{
    // alpha clamped to [2^-15, 1], and 1 past the sequence end: the lower
    // clamp bound is 1 for a token past it (med3(x, 1, 1) = 1), so a chunk
    // of any length takes the same instructions
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const float lo = K.tok0 + t < L ? kAlphaMin : 1.0f;
#pragma unroll
        for (int c = 0; c < 8; ++c) al[t][c] = __builtin_amdgcn_fmed3f(raw_alpha<G>(R, t, c), lo, 1.0f);
    }
    const int tp = K.tp;
    float inc[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) inc[c] = al[0][c] * al[1][c];
    // The eight lanes of a channel group sit two apart in their row of 16, so
    // a row shift by 2 k reaches position tp - k of the same group, and
    // positions tp < k read from outside the row: with bound control off such
    // a lane is not written by the DPP multiply, which leaves its partial
    // product as it is (lane layout and result checked on the GPU with an
    // in-bounds probe).  Three in-place multiplies per channel form the
    // inclusive scan.
#pragma unroll
    for (int c = 0; c < 8; ++c) scan_mul<2>(inc[c]);
#pragma unroll
    for (int c = 0; c < 8; ++c) scan_mul<4>(inc[c]);
#pragma unroll
    for (int c = 0; c < 8; ++c) scan_mul<8>(inc[c]);  // tokens 16 tb .. 16 tb + 2 tp + 1
#pragma unroll
    for (int c = 0; c < 8; ++c) ex[c] = scan_prev(inc[c]);  // tokens 16 tb .. 16 tb + 2 tp - 1
    float* ph = reinterpret_cast<float*>(lds + kOffPh);
    if (tp == 7 || (K.tb == 0 && tp == 3)) {
        float* dst = ph + (tp == 7 ? K.tb : 4) * 128 + K.c0;
        *reinterpret_cast<float4*>(dst) = make_float4(inc[0], inc[1], inc[2], inc[3]);
        *reinterpret_cast<float4*>(dst + 4) = make_float4(inc[4], inc[5], inc[6], inc[7]);
    }
    // smallest decay over the 16 tokens among this wavefront's channels
    float m = 1.0f;
    if (tp == 7) {
#pragma unroll
        for (int c = 0; c < 8; ++c) m = min_decay(m, inc[c]);
    }
    m = wave_min(m);
    if (lane == 0) ph[5 * 128 + 2 * K.tb + K.ch] = m;
}

// Chunk length (identical in every wavefront: the same eight values in the
// same order): with m_j the smallest decay over block j (tokens 16 j ..
// 16 j + 15) among all channels (the smaller of its two channel halves), the longest of 64, 32, 16 tokens for which
// m_0 m_1 ... stays >= 2^-64, else 8; at most L.  The product of the minima
// bounds every channel's decay from below, so all factors of the chunk stay
// within [2^-64, 2^64].
__device__ __forceinline__ int chunk_step(const unsigned char* lds, int L)
{
    const float* pm = reinterpret_cast<const float*>(lds + kOffPh) + 5 * 128;
    const float m0 = min_decay(pm[0], pm[1]), m1 = min_decay(pm[2], pm[3]), m2 = min_decay(pm[4], pm[5]),
                m3 = min_decay(pm[6], pm[7]);
    const float g16 = m0, g32 = g16 * m1, g64 = g32 * m2 * m3;
    const int leff = g64 >= kRangeMin ? 64 : g32 >= kRangeMin ? 32 : g16 >= kRangeMin ? 16 : 8;
    // every lane read the same values: a scalar, so that the buffer windows
    // built from it stay scalar too
    return __builtin_amdgcn_readfirstlane(leff < L ? leff : L);
}

// Store offsets of the key prep for one lane (tokens tok0, tok0 + 1 with tok0
// even, channels c0 .. c0 + 7 with c0 a multiple of 8).  The swizzle is
// linear in the row bits over GF(2), so row tok0 + t of a [64][128] tile lies
// at (base ^ (tile_swz(t) << 4)) + 256 t: the XOR only touches the granule
// bits.
struct PrepOffs {
    int t128[2];  // row tok0 of a [64][128] tile, channels c0 .. + 3 and c0 + 4 .. + 7
};
__device__ __forceinline__ PrepOffs prep_offsets(int tok0, int c0)
{
    PrepOffs o;
    o.t128[0] = off_t128(tok0, chan_pos(c0));
    o.t128[1] = off_t128(tok0, chan_pos(c0 + 4));
    return o;
}
// Channels 8 cg .. 8 cg + 7 of row tok0 + t of the tile at byte offset tile.
__device__ __forceinline__ void st_tok(unsigned char* lds, const PrepOffs& o, int tile, int t, uint4 v)
{
    const int x = tile_swz(t) << 4;
    lds_st<uint2>(lds, tile + ((o.t128[0] ^ x) + 256 * t), make_uint2(v.x, v.y));
    lds_st<uint2>(lds, tile + ((o.t128[1] ^ x) + 256 * t), make_uint2(v.z, v.w));
}

// Key prep of a chunk, after its decay products (decay_pass1) and length
// (chunk_step) are known: the rows of Et, Qt and Kt (buffer ebuf).  Token by
// token, as their registers are consumed, the inputs of the next chunk are
// loaded into R.
//
// A chunk cut short (step < L) ends at a multiple of 8, so each lane's two
// tokens are both in it or both past it; lanes past it (kAllLive false) form
// zero rows from zeroed q and k with a running decay of 1 (their own decay
// factors are never formed).  Past the sequence end (step = L) the inputs
// read as zero and alpha as 1, which gives zero rows as well.
template <int G, bool kAllLive>
__device__ __forceinline__ void prep_tiles(unsigned char* lds, RawK& R, const RawSrc& nxt, const float (*al)[8],
                                           const float* ex, int step, int ebuf, const KeyLane& K)
{
    const bool live = kAllLive || K.tok0 < step;
    // decay before this lane's tokens: blocks 0 .. tb - 1 (the row of ones
    // stands in for the others), then the part of its own block before it
    float cum[8];
    {
        const float4* p4 = reinterpret_cast<const float4*>(lds + kOffPh) + (K.c0 >> 2);  // row j: p4[32 j], p4[32 j + 1]
        const int j0 = K.tb > 0 ? 0 : kPhOnes, j1 = K.tb > 1 ? 1 : kPhOnes, j2 = K.tb > 2 ? 2 : kPhOnes;
        const float4 a0 = p4[32 * j0], b0 = p4[32 * j0 + 1], a1 = p4[32 * j1], b1 = p4[32 * j1 + 1];
        const float4 a2 = p4[32 * j2], b2 = p4[32 * j2 + 1];
        const float x0[8] = {a0.x, a0.y, a0.z, a0.w, b0.x, b0.y, b0.z, b0.w};
        const float x1[8] = {a1.x, a1.y, a1.z, a1.w, b1.x, b1.y, b1.z, b1.w};
        const float x2[8] = {a2.x, a2.y, a2.z, a2.w, b2.x, b2.y, b2.z, b2.w};
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            cum[c] = x0[c] * x1[c] * x2[c] * ex[c];
            if (!kAllLive) cum[c] = live ? cum[c] : 1.0f;
        }
    }
    // 1 / (decay through token t): one reciprocal of the decay through the
    // lane's second token, then back through alpha
    float rc[2][8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        rc[1][c] = __builtin_amdgcn_rcpf(cum[c] * al[0][c] * al[1][c]);
        rc[0][c] = rc[1][c] * al[1][c];
    }
    const PrepOffs po = prep_offsets(K.tok0, K.c0);
    const int et_base = kOffEt + ebuf * 16384, qt_base = kOffQt + ebuf * 16384;
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        load_alpha<G>(R, nxt, t, K);  // alpha of token t of the next chunk (clamped copy in al)
        float q[8], k[8], b[8];
        unpack8(kAllLive || live ? R.q[t] : zero, q);
        unpack8(kAllLive || live ? R.k[t] : zero, k);
        if (G & kScalarErase) {
#pragma unroll
            for (int c = 0; c < 8; ++c) b[c] = lo_f(R.b[t].x);
        } else {
            unpack8(R.b[t], b);
        }
        float et[8], qt[8], kt[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            cum[c] *= al[t][c];  // 1 past the sequence end
            et[c] = b[c] * k[c] * cum[c];
            qt[c] = q[c] * cum[c];
            kt[c] = k[c] * rc[t][c];
        }
        st_tok(lds, po, et_base, t, make_uint4(pack2(et[0], et[1]), pack2(et[2], et[3]), pack2(et[4], et[5]),
                                               pack2(et[6], et[7])));
        st_tok(lds, po, qt_base, t, make_uint4(pack2(qt[0], qt[1]), pack2(qt[2], qt[3]), pack2(qt[4], qt[5]),
                                               pack2(qt[6], qt[7])));
        st_tok(lds, po, kOffKt + ebuf * 16384, t, make_uint4(pack2(kt[0], kt[1]), pack2(kt[2], kt[3]),
                                                             pack2(kt[4], kt[5]), pack2(kt[6], kt[7])));
        load_q(R, nxt, t, K);  // q of token t of the next chunk (k and b follow after B1)
        __builtin_amdgcn_sched_barrier(0);  // one token's temporaries at a time
    }
}


// One block of A or P (16 x 16 over K = 128 channels), formed transposed:
// D = Kt_J Row_I^T, which leaves row 16 I + r, columns 16 J + 4 g .. + 3 in
// each lane.
template <int KIND, int I, int J>  // KIND 0: A (rows Et), 1: P (rows Qt)
__device__ __forceinline__ void ap_block(unsigned char* lds, const LaneOffs& o, int ebuf, int r, int g)
{
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    const int rows = (KIND == 0 ? kOffEt : kOffQt) + ebuf * 16384;
    bf16x8 ka[4], ra[4];  // operands issued together so that their latency overlaps
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        ka[s] = ld_c128(lds, o, kOffKt + ebuf * 16384, J, s);
        ra[s] = ld_c128(lds, o, rows, I, s);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) acc = mfma_bf16(ka[s], ra[s], acc);
    const int row = 16 * I + r, col = 16 * J + 4 * g;
    if (KIND == 0) {
        lds_st<uint2>(lds, kOffAneg + off_rc64(row, col),
                      make_uint2(pack2(-acc[0], -acc[1]), pack2(-acc[2], -acc[3])));
    } else {
        float p[4] = {acc[0], acc[1], acc[2], acc[3]};
        if (I == J) {
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = col + i <= row ? p[i] : 0.f;
        }
        lds_st<uint2>(lds, kOffP + off_rc64(row, col), make_uint2(pack2(p[0], p[1]), pack2(p[2], p[3])));
    }
    __builtin_amdgcn_sched_barrier(0);  // one block's operands in flight at a time
}

// The six A blocks below the diagonal blocks and the ten P blocks on and below
// them, over value wavefronts 0..2 (grouped by shared operands).
__device__ __forceinline__ void ap_work(unsigned char* lds, const LaneOffs& o, int ebuf, int slot, int r, int g)
{
    // the store offsets are formed here each period, not held across the
    // loop (register budget of the value side's merged chunk sequence)
    __asm__ volatile("" : "+v"(r), "+v"(g));
    switch (slot) {
        case 0:
            ap_block<1, 3, 3>(lds, o, ebuf, r, g);
            ap_block<1, 3, 2>(lds, o, ebuf, r, g);
            ap_block<1, 3, 1>(lds, o, ebuf, r, g);
            ap_block<1, 3, 0>(lds, o, ebuf, r, g);
            ap_block<0, 3, 2>(lds, o, ebuf, r, g);
            break;
        case 1:
            ap_block<1, 2, 2>(lds, o, ebuf, r, g);
            ap_block<1, 2, 1>(lds, o, ebuf, r, g);
            ap_block<1, 2, 0>(lds, o, ebuf, r, g);
            ap_block<0, 3, 1>(lds, o, ebuf, r, g);
            ap_block<0, 3, 0>(lds, o, ebuf, r, g);
            break;
        default:
            ap_block<1, 1, 1>(lds, o, ebuf, r, g);
            ap_block<1, 1, 0>(lds, o, ebuf, r, g);
            ap_block<1, 0, 0>(lds, o, ebuf, r, g);
            ap_block<0, 2, 1>(lds, o, ebuf, r, g);
            ap_block<0, 2, 0>(lds, o, ebuf, r, g);
            ap_block<0, 1, 0>(lds, o, ebuf, r, g);
            break;
    }
}

// Wavefront kTWave: the diagonal blocks A_II (strictly lower, FP32) and
// T_II = (I + A_II)^-1 by forward substitution; lane group g takes block g,
// lane r its column r.
__device__ __forceinline__ void t_work(unsigned char* lds, const LaneOffs& o, int ebuf, int r, int g)
{
    __asm__ volatile("" : "+v"(r), "+v"(g));  // no part of this work moves above the barrier before it
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        bf16x8 ea[4], ka[4];  // operands issued together so that their latency overlaps
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            ea[s] = ld_c128(lds, o, kOffEt + ebuf * 16384, I, s);
            ka[s] = ld_c128(lds, o, kOffKt + ebuf * 16384, I, s);
        }
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma_bf16(ea[s], ka[s], acc);
        // acc[i] = (Et Kt^T)_II[4g + i][r]: column r, rows 4g..4g+3.  Only the
        // part below the diagonal, A_II, is read back (step j of the
        // substitution reads rows j + 1 .. 15 of column j), so the rest needs
        // no masking.
        lds_st<float4>(lds, kOffAd + (I * kTBlk + r * kT16 + 4 * g) * 4, make_float4(acc[0], acc[1], acc[2], acc[3]));
        __builtin_amdgcn_sched_barrier(0);
    }
    // Other lanes of this wavefront read the columns back: LDS accesses of one
    // wavefront complete in order; this keeps the compiler from reordering.
    __asm__ volatile("" ::: "memory");
    // column 0 of this lane group's block, as a local-memory pointer so that
    // it can be made opaque without leaving LDS addressing; column j at + j * kT16 / 4
    lds_f4* adc = (lds_f4*)(lds + kOffAd + g * kTBlk * 4);
    float t[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) t[i] = i == r ? 1.f : 0.f;
    // Step j needs rows j + 1 .. 15 of column j (the 16-byte pieces from
    // (j + 1) / 4 on).  Column j + kAhead is requested at step j, once t[j]
    // is final (the column pointer is made opaque there; the column offset is
    // the instruction's constant), so that kAhead columns are in flight and
    // none is read earlier (register budget).
    constexpr int kAhead = 2;
    f32x4 cb[kAhead + 1][4];
#pragma unroll
    for (int j = 0; j < kAhead; ++j)
#pragma unroll
        for (int q4 = (j + 1) >> 2; q4 < 4; ++q4) cb[j][q4] = adc[j * kT16 / 4 + q4];
#pragma unroll
    for (int j = 0; j < 15; ++j) {
        if (j + kAhead < 15) {
            const int jn = j + kAhead;
            __asm__ volatile("" : "+v"(adc) : "v"(t[j]) : "memory");  // after t[j] is final
#pragma unroll
            for (int q4 = (jn + 1) >> 2; q4 < 4; ++q4) cb[jn % (kAhead + 1)][q4] = adc[jn * kT16 / 4 + q4];
        }
        const f32x4* c = cb[j % (kAhead + 1)];
#pragma unroll
        for (int i = j + 1; i < 16; ++i) {
            const float a = c[i >> 2][i & 3];
            t[i] -= a * t[j];
        }
    }
    float* T = reinterpret_cast<float*>(lds + kOffT) + g * kTBlk;
#pragma unroll
    for (int i = 0; i < 16; ++i) T[i * kT16 + r] = t[i];
}

// Chunk decay gamma per channel (the decay through the chunk's last token)
// into buffer buf, from the decay products: blocks 0 .. nw - 1, or tokens
// 0..7 (row 4) when the chunk ends inside them.  One wavefront, two channels
// per lane.
__device__ __forceinline__ void value_gamma(unsigned char* lds, int step, int buf, int lane)
{
    const float2* ph = reinterpret_cast<const float2*>(lds + kOffPh) + lane;  // row j: ph[64 j]
    const int nw = step <= 8 ? 0 : (step + 15) >> 4;
    const int j1 = nw > 1 ? 1 : kPhOnes, j2 = nw > 2 ? 2 : kPhOnes, j3 = nw > 3 ? 3 : kPhOnes;
    const float2 x0 = ph[64 * (nw == 0 ? 4 : 0)], x1 = ph[64 * j1], x2 = ph[64 * j2], x3 = ph[64 * j3];
    reinterpret_cast<float2*>(lds + kOffGam)[buf * 64 + lane] =
        make_float2(x0.x * x1.x * x2.x * x3.x, x0.y * x1.y * x2.y * x3.y);
}

// Value wavefront, one chunk of lv tokens (tiles of buffer ebuf, chunk decay
// of buffer ebuf), block by block: X_I = Z_I - Et_I S (rows past the chunk
// zero), the blocked solve R_I = X_I - sum_{J<I} A_IJ U_J, U_I = T_II R_I, and
// the output rows O_I^T = (Qt_I S)^T + U^T P_I^T (P is lower triangular, so
// only U_0 .. U_I enter); then the state update.  Every product reads the
// state as it was at the chunk start.
__device__ __forceinline__ void value_chunk(const unsigned char* lds, const LaneOffs& o, f32x4* S, int lv, int ebuf,
                                            rsrc_t ro, int ostride, int wave, int r, int g)
{
    bf16x8 sb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) sb[s] = pack_acc_pair(S[2 * s], S[2 * s + 1]);
    const unsigned char* zs = lds + kOffZs + ebuf * kZsBuf + wave * kZsWave;
    const int et = kOffEt + ebuf * 16384, qt = kOffQt + ebuf * 16384;
    const int o_vo = r * ostride + (16 * wave + 4 * g) * 2;
    const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 ub[2];  // U as an operand over tokens 0..31 and 32..63; blocks not solved yet are zero
#pragma unroll
    for (int I = 0; I < 4; ++I) {
        // this block's operands, issued together so that their latency overlaps
        bf16x8 ea[4], qa[4], an[2], pa[2];
#pragma unroll
        for (int s = 0; s < 4; ++s) ea[s] = ld_c128(lds, o, et, I, s);
#pragma unroll
        for (int s = 0; s < 4; ++s) qa[s] = ld_c128(lds, o, qt, I, s);
        if (I >= 1) an[0] = ld_s64(lds, o, kOffAneg, I, 0);
        if (I >= 3) an[1] = ld_s64(lds, o, kOffAneg, I, 1);
        pa[0] = ld_s64(lds, o, kOffP, I, 0);
        if (I >= 2) pa[1] = ld_s64(lds, o, kOffP, I, 1);
        const float4 z = lds_ld<float4>(zs, zs_off(r, 16 * I + 4 * g));
        const float4 tr = lds_ld<float4>(lds, kOffT + (I * kTBlk + r * kT16 + 4 * g) * 4);
        f32x4 xe = zero4, xq = zero4;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            xe = mfma_bf16(ea[s], sb[s], xe);
            xq = mfma_bf16(sb[s], qa[s], xq);
        }
        const int t0 = 16 * I + 4 * g;
        f32x4 R_ = f32x4{t0 + 0 < lv ? z.x - xe[0] : 0.f, t0 + 1 < lv ? z.y - xe[1] : 0.f,
                         t0 + 2 < lv ? z.z - xe[2] : 0.f, t0 + 3 < lv ? z.w - xe[3] : 0.f};
        if (I >= 1) R_ = mfma_bf16(an[0], ub[0], R_);
        if (I >= 3) R_ = mfma_bf16(an[1], ub[1], R_);
        f32x4 u = zero4;
        u = mfma_f32(tr.x, R_[0], u);
        u = mfma_f32(tr.y, R_[1], u);
        u = mfma_f32(tr.z, R_[2], u);
        u = mfma_f32(tr.w, R_[3], u);
        if (I == 0) ub[0] = pack_acc_pair(u, zero4);
        if (I == 1) ub[0] = pack_acc_pair_hi(ub[0], u);
        if (I == 2) ub[1] = pack_acc_pair(u, zero4);
        if (I == 3) ub[1] = pack_acc_pair_hi(ub[1], u);
        f32x4 acc2 = mfma_bf16(ub[0], pa[0], xq);
        if (I >= 2) acc2 = mfma_bf16(ub[1], pa[1], acc2);
        {  // lane holds token 16 I + r, columns 4g..4g+3; tokens past the chunk
           // lie past the window ro (their offset is at least lv rows), so the
           // store drops them, with no branch splitting the block sequence
            u32x2 pk;
            pk[0] = pack2(acc2[0], acc2[1]);
            pk[1] = pack2(acc2[2], acc2[3]);
            __builtin_amdgcn_raw_buffer_store_b64(pk, ro, o_vo, 16 * I * ostride, 0);
        }
    }
    // ---- S <- Diag(gamma) (S + Kt^T U)  (= Diag(gamma) S + Kb^T U with Kb = Kt gamma)
    const float* gam = reinterpret_cast<const float*>(lds + kOffGam) + ebuf * 128;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) {
        const float4 gm = *reinterpret_cast<const float4*>(gam + 16 * cb + 4 * g);
        f32x4 acc3 = S[cb];
        acc3 = mfma_bf16(ld_ktr(lds, o, kOffKt + ebuf * 16384, cb, 0), ub[0], acc3);
        acc3 = mfma_bf16(ld_ktr(lds, o, kOffKt + ebuf * 16384, cb, 1), ub[1], acc3);
        S[cb] = f32x4{acc3[0] * gm.x, acc3[1] * gm.y, acc3[2] * gm.z, acc3[3] * gm.w};
        if (cb & 1) __builtin_amdgcn_sched_barrier(0);
    }
}

template <int G, bool SEG>
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
    const int64_t dv = a.dv;  // columns of the carried state
    // segment mode (SEG): columns of v, w, o and the caller's states, and
    // whether this tile holds state-map columns (identity start, z = 0, no output)
    const int64_t dvio = SEG && a.dv_io > 0 ? a.dv_io : a.dv;
    const bool map_tile = SEG && j0 >= dvio;

    int64_t bos, eos, brow;
    int seg = 0;  // segment of the row (segment mode)
    if (SEG) {
        brow = n / a.seg_count;
        seg = a.seg_first + n % a.seg_count;
        bos = int64_t(seg) * a.seg_len;
        eos = bos + a.seg_len < a.T ? bos + a.seg_len : a.T;
        if (bos > eos) bos = eos;
    } else {
        sequence_bounds(a.cu_seqlens, n, a.T, bos, eos, brow);
    }

    // The blocks the solve and the output read as zero (A on the diagonal, P
    // right of it) are never written: clear Aneg and P once.
    {
        uint4* z = reinterpret_cast<uint4*>(lds + kOffAneg);
        const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int i = tid; i < 1024; i += kThreads) z[i] = zero;  // 1024 x 16 = 16384 bytes
    }

    // Both roles run the same sequence of periods (the loop control is
    // computed identically) and meet at the same two barriers per period;
    // separate loops keep each role's registers apart.
    int64_t tk = bos;  // chunk the key side prepares this period
    int64_t tv = -1;   // chunk the value side finishes this period (< 0: none)
    int kbuf = 0;      // Et, Qt, gamma buffer the key side writes this period; the value side reads kbuf ^ 1
    if (vwave) {
        // state slice of a value wavefront: channels 16 cb + 4 g + i, column j0 + 16 wave + r
        f32x4 S[8];
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) S[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
        // the initial state: a [..][dk][dv_io] FP32 array, columns j0 .. j0 + 63
        const float* sin = nullptr;
        if (map_tile) {  // identity: column j0 + 16 wave + r holds e_(j0 - dv_io + 16 wave + r)
            const int d = int(j0 - dvio) + 16 * wave + r0;
#pragma unroll
            for (int cb = 0; cb < 8; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i) S[cb][i] = 16 * cb + 4 * g0 + i == d ? 1.f : 0.f;
        } else if (SEG && a.seg_states_in) {
            sin = a.seg_states_in + ((int64_t(brow) * a.seg_total + seg) * a.H + h) * kDK * dvio + j0;
        } else if (!SEG || seg == 0) {
            sin = a.initial_state ? a.initial_state + (int64_t(SEG ? brow : n) * a.H + h) * kDK * dvio + j0 : nullptr;
        }
        if (sin) {
            const int win = int(dvio);
            const rsrc_t rs = make_rsrc(sin, uint32_t(kDK * win * 4));
            const int s_vo = ((4 * g0) * win + 16 * wave + r0) * 4;
#pragma unroll
            for (int cb = 0; cb < 8; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    S[cb][i] = __uint_as_float(
                        __builtin_amdgcn_raw_buffer_load_b32(rs, s_vo, (16 * cb + i) * win * 4, 0));
        }

        // outputs: real columns only, and in segment mode per seg_o_all; token
        // tv of this (row, head) at obase + tv * H * dv_io
        const bool store_o = !SEG || (!map_tile && (a.seg_o_all || seg == 0));
        bf16raw* o = static_cast<bf16raw*>(a.o);
        const int ostride = a.H * int(dvio) * 2;
        const uint32_t o_on = store_o ? ~0u : 0u;
        int lv = 0;  // length of chunk tv
        while (tk < eos || tv >= 0) {
            const bool has_k = tk < eos, has_v = tv >= 0;
            const int L = has_k ? int(eos - tk < kC ? eos - tk : kC) : 0;
            lds_barrier();  // B0: tiles of chunk tv, decay products of chunk tk visible
            const int r = r0, g = g0, lane = lane0;
            const int step = has_k ? chunk_step(lds, L) : 0;
            if (has_k && wave == 0) value_gamma(lds, step, kbuf, lane);  // read by the next period's update

            if (has_v) {
                const rsrc_t ro = make_rsrc(o + token_row(a, brow, tv, h) * dvio + j0,
                                            SEG ? o_on & (uint32_t(lv - 1) * uint32_t(ostride) + kDVT * 2)
                                                : uint32_t(lv - 1) * uint32_t(ostride) + kDVT * 2);
                value_chunk(lds, lane_offsets(r, g), S, lv, kbuf ^ 1, ro, ostride, wave, r, g);
            }
            const int64_t tn = tk + step;

            lds_barrier();  // B1: tiles of chunk tk visible; A, P and T of chunk tv consumed
            if (has_k) {

                const LaneOffs lk = lane_offsets(r, g);
                if (wave == kTWave)
                    t_work(lds, lk, kbuf, r, g);
                else
                    ap_work(lds, lk, kbuf, wave, r, g);
            }
            tv = has_k ? tk : -1;
            lv = step;
            tk = has_k ? tn : eos;
            kbuf ^= 1;
        }
        float* sout = nullptr;
        int wout = int(dvio);
        if (SEG && a.seg_states_out) {
            sout = a.seg_states_out + ((int64_t(brow) * a.seg_total + seg) * a.H + h) * kDK * dv + j0;
            wout = int(dv);
        } else if (!map_tile && a.final_state && (!SEG || seg == a.seg_total - 1)) {
            sout = a.final_state + (int64_t(SEG ? brow : n) * a.H + h) * kDK * dvio + j0;
        }
        if (sout) {
            const rsrc_t rs = make_rsrc(sout, uint32_t(kDK * wout * 4));
            const int s_vo = ((4 * g0) * wout + 16 * wave + r0) * 4;
#pragma unroll
            for (int cb = 0; cb < 8; ++cb)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[cb][i]), rs, s_vo,
                                                          (16 * cb + i) * wout * 4, 0);
        }
    } else {
        // Key side.  The decay products of a chunk are formed after B1 of the
        // period before the one that prepares it, so its length is known at
        // B0; its tiles are formed between B0 and B1 (Et, Qt and Kt into the
        // buffers the value side does not read this period) and its z after
        // B1.  The next chunk's inputs are loaded during the prep and stay in
        // flight until its decay products and prep.
        if (kw == 0) {  // the row of ones of the decay products
            const float4 one = make_float4(1.f, 1.f, 1.f, 1.f);
            if (lane0 < 32) reinterpret_cast<float4*>(lds + kOffPh)[kPhOnes * 32 + lane0] = one;
        }
        RawK R;
        RawVK V;                // v, w of chunk tk, loaded in the period before
        float al[2][8], ex[8];  // clamped alpha and decay products of chunk tk
        if (tk < eos) {
            const int L = int(eos - tk < kC ? eos - tk : kC);
            const RawSrc src = raw_src<G>(a, token_row(a, brow, tk, h), L);
            const KeyLane K = key_lane(kw, lane0);
#pragma unroll
            for (int t = 0; t < 2; ++t) load_alpha<G>(R, src, t, K);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                load_q(R, src, t, K);
                load_kb<G>(R, src, t, K);
            }
            load_vk<G, SEG>(V, a, token_row(a, brow, tk, h), L, j0, kw, lane0);
            decay_pass1<G>(lds, R, al, ex, L, K, lane0);
        }
        while (tk < eos || tv >= 0) {
            const bool has_k = tk < eos;
            const int L = has_k ? int(eos - tk < kC ? eos - tk : kC) : 0;
            lds_barrier();  // B0
            if (kw >= 4) __builtin_amdgcn_s_setprio(1);
            int lane = lane0;  // opaque per period (see the value loop)
            __asm__ volatile("" : "+v"(lane));
            const KeyLane K = key_lane(kw, lane);
            const int step = has_k ? chunk_step(lds, L) : 0;
            const int64_t tn = tk + step;
            const int Ln = has_k && tn < eos ? int(eos - tn < kC ? eos - tn : kC) : 0;
            // the next chunk's window (empty past the sequence end: loads read zero)
            const RawSrc nxt = raw_src<G>(a, token_row(a, brow, Ln > 0 ? tn : tk, h), Ln);
            if (has_k) {
                if (16 * K.tb + 16 <= step)
                    prep_tiles<G, true>(lds, R, nxt, al, ex, step, kbuf, K);
                else
                    prep_tiles<G, false>(lds, R, nxt, al, ex, step, kbuf, K);
            }
            lds_barrier();  // B1
            if (kw >= 4) __builtin_amdgcn_s_setprio(0);
            if (has_k) {
                // k and b of the next chunk: issued here so that the memory pipe
                // stays busy in this half of the period as well
#pragma unroll
                for (int t = 0; t < 2; ++t) load_kb<G>(R, nxt, t, K);
                // z of chunk tk (read by the value side next period), then v, w of the next chunk
                store_z<G>(lds, V, kbuf, kw, lane);
                load_vk<G, SEG>(V, a, token_row(a, brow, Ln > 0 ? tn : tk, h), Ln, j0, kw, lane);
            }
            if (Ln > 0) decay_pass1<G>(lds, R, al, ex, Ln, K, lane);
            tv = has_k ? tk : -1;
            tk = has_k ? tn : eos;
            kbuf ^= 1;
        }
    }

}

}  // namespace

bool chunk_fwd_mfma_supported(const ChunkArgs& a, bool bf16)
{
    return bf16 && a.dk == kDK && a.dv % kDVT == 0;
}

namespace {

template <int G, bool SEG>
hipError_t launch_mode(const ChunkArgs& a, hipStream_t stream)
{
    // Allow the kernel its > 64 KiB of dynamic LDS (thread-safe one-time call).
    static const hipError_t attr =
        hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_fwd_mfma_kernel<G, SEG>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    if (attr != hipSuccess) return attr;
    const int ntiles = a.dv / kDVT;
    const int64_t chains = int64_t(a.N) * a.H;
    const int64_t blocks = (chains + 7) / 8 * 8 * ntiles;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((chunk_fwd_mfma_kernel<G, SEG>), dim3(unsigned(blocks)), dim3(kThreads), kLdsBytes, stream,
                       a, ntiles, int(chains));
    return hipGetLastError();
}

template <int G>
hipError_t launch_gates(const ChunkArgs& a, hipStream_t stream)
{
    return a.seg_len > 0 ? launch_mode<G, true>(a, stream) : launch_mode<G, false>(a, stream);
}

}  // namespace

hipError_t launch_chunk_fwd_mfma(const ChunkArgs& a, hipStream_t stream)
{
    // every valid gdn2_gate_flags combination
    switch (a.gates) {
        case 0: return launch_gates<0>(a, stream);
        case 1: return launch_gates<1>(a, stream);
        case 2: return launch_gates<2>(a, stream);
        case 3: return launch_gates<3>(a, stream);
        case 5: return launch_gates<5>(a, stream);
        case 8: return launch_gates<8>(a, stream);
        case 9: return launch_gates<9>(a, stream);
        case 10: return launch_gates<10>(a, stream);
        case 11: return launch_gates<11>(a, stream);
        case 13: return launch_gates<13>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace gdn2
