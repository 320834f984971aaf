// Chunkwise forward on gfx950 matrix cores (bf16 inputs, dk = 128).
//
// The chunkwise WY form (Gated DeltaNet-2 analysis, iplexlaw.co.kr, "Token
// processing and parallel training"): per 64-token chunk the cumulative
// channel-wise decay is absorbed into asymmetric erase factors, leaving a
// lower-triangular solve and dense products; FP32 is kept for the decay, the
// solve and the carried state.  With incoming state S, per key channel
// G_i = sum_{m<=i} log2 alpha_m and e = b k, z = w v:
//     A_ij = sum_c e_ic k_jc 2^(G_ic - G_jc)  (j < i)     P_ij = same with q, j <= i
//     U    = (I + A)^-1 (Z - Et S)                          Et_i = e_i 2^G_i
//     O    = Qt S + P U                                      Qt_i = q_i 2^G_i
//     S   <- Diag(2^G_last) S + Kb^T U                       Kb_j = k_j 2^(G_last - G_j)
//
// Decay factors.  The chunk is cut into four 16-token blocks.  For a row
// token i in block I and a column token j <= i, 2^(G_i - G_j) is split around
// the block's reference token m_I (its 8th token):
//     2^(G_i - G_j) = [2^(G_i - m_I)] * [2^(m_I - G_j)]
// Both factors are at most 2^(8 * 15) because log2 alpha >= -15 and i, j lie
// within 8 tokens of m_I on the side where a factor exceeds one; for j in an
// earlier block the column factor is <= 1.  All factors are FP32 products of
// alpha: forward and backward running products inside each 8-token half
// block, and per-half products combined across the chunk.  Underflow of a
// factor that is <= 1 only drops terms below 2^-126 of their neighbours.
//
// Matrix products (v_mfma_f32_16x16x32_bf16, FP32 accumulate):
//     A, P blocks (K = 128 channels), Et S, (Qt S)^T, the off-diagonal part of
//     the blocked solve, (P U)^T and Kb^T U (K = tokens);
// in FP32 (v_mfma_f32_16x16x4_f32) the diagonal-block solve U_I = T_II R_I,
// with T_II = (I + A_II)^-1 formed by FP32 forward substitution.
//
// Work split.  One workgroup of eight wavefronts (two per SIMD) per (sequence,
// head, value tile).  VW of them are value wavefronts: wavefront w < VW owns
// value columns 16w..16w+15 and keeps that 128 x 16 slice of the FP32 state in
// its accumulators for the whole sequence.  All eight share the key-side work
// of a chunk (decay factors, operand tiles, A, P, T) through LDS.  Workgroups
// of the same chain are placed on the same XCD so that every tile after the
// first re-reads the key-side inputs from L2.
//
// Operand layouts (16x16x32 bf16): lane l = 16 g + r provides row/column r and
// a group of eight K indices chosen by g; the accumulator holds rows 4g..4g+3
// of column r.  A and B only need to agree on the K order, so for a K-step over
// 32 channels or tokens group g takes {4g..4g+3} U {16+4g..16+4g+3}: exactly
// the rows a lane already holds in two adjacent accumulator blocks.  An
// accumulator tile therefore serves directly as a B operand, and also as an A
// operand of the transposed product (X Y)^T = Y^T X^T; transposed products
// give each lane four consecutive columns of one row, which makes the stores
// of A, P and O contiguous.
#include "gdn2_device.hpp"
#include "launch.hpp"

namespace gdn2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kDK = 128;         // key head size
constexpr int kC = 64;           // chunk
constexpr int kWaves = 8;        // wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kTWave = kWaves - 1;  // wavefront that forms T
constexpr float kAlphaMin = 3.0517578125e-05f;  // 2^-15

// ---- LDS map (bytes) -------------------------------------------------------
// Region 1, prep -> A/P:  Eh, Qh, Kh [64][128] bf16, Ko [6][16][128] bf16
// Region 1, A/P -> end:   Aneg, P [64][64] bf16, AdT, T [4][16][16] f32
// Region 2, prep -> end:  Et, Qt [64][128] bf16, KbT [128][64] bf16
// then Zs [DVT][68] f32 (z = w v, column major), per-half alpha products, gamma.
constexpr int kOffEh = 0, kOffQh = 16384, kOffKh = 32768, kOffKo = 49152;  // .. 73728
constexpr int kOffAneg = 0, kOffP = 8192, kOffAdT = 16384, kOffT = 20480;  // .. 24576
constexpr int kOffEt = 73728, kOffQt = 90112, kOffKbT = 106496, kOffZs = 122880;
constexpr int kZsStride = 68;  // floats per value column in Zs
template <int DVT>
struct Lds {
    static constexpr int kOffPh = kOffZs + DVT * kZsStride * 4;  // [8 halves][128] f32
    static constexpr int kOffGam = kOffPh + 8 * 128 * 4;         // [128] f32
    static constexpr int kBytes = kOffGam + 128 * 4;
    static_assert(kBytes <= 160 * 1024, "LDS budget");
};

// Byte offset of (row, ch) in a [rows][128] bf16 tile; 16-byte granules are
// XOR-swizzled by the row so that 16 rows read at one granule column hit
// different banks.
__device__ __forceinline__ int off_rc128(int row, int ch)
{
    return row * 256 + ((((ch >> 3) ^ row) & 15) << 4) + ((ch & 7) << 1);
}
// Byte offset of (row, col) in a [rows][64] bf16 tile (granule XOR by row/2;
// the row parity picks the bank half).
__device__ __forceinline__ int off_rc64(int row, int col)
{
    return row * 128 + ((((col >> 3) ^ (row >> 1)) & 7) << 4) + ((col & 7) << 1);
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

// Per-lane byte offsets of the operand reads, computed once.  For a tile row
// 16 k + r the swizzle term depends on r only, so every read below is one of
// these offsets plus a compile-time constant (the tile base and 16 k rows).
struct LaneOffs {
    int c128[4];     // [.][128] tile, channels 32 s + 8 g .. + 7 (16 bytes)
    int s128[4][2];  // [.][128] tile, channels 32 s + 4 g .. + 3 and 32 s + 16 + 4 g .. + 3
    int s64[2][2];   // [.][64] tile, columns 32 s + 4 g .. + 3 and 32 s + 16 + 4 g .. + 3
};

__device__ __forceinline__ LaneOffs lane_offsets(int r, int g)
{
    LaneOffs o;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        o.c128[s] = off_rc128(r, 32 * s + 8 * g);
        o.s128[s][0] = off_rc128(r, 32 * s + 4 * g);
        o.s128[s][1] = off_rc128(r, 32 * s + 16 + 4 * g);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        o.s64[s][0] = off_rc64(r, 32 * s + 4 * g);
        o.s64[s][1] = off_rc64(r, 32 * s + 16 + 4 * g);
    }
    return o;
}

// Operand of row 16 k + r of a [.][128] tile, contiguous K groups.
__device__ __forceinline__ bf16x8 ld_c128(const unsigned char* lds, const LaneOffs& o, int base, int k, int s)
{
    return as_bf16x8(lds_ld<uint4>(lds, base + 16 * k * 256 + o.c128[s]));
}
// Same tile with split K groups {32s+4g..+3} U {32s+16+4g..+3}.
__device__ __forceinline__ bf16x8 ld_s128(const unsigned char* lds, const LaneOffs& o, int base, int k, int s)
{
    const uint2 lo = lds_ld<uint2>(lds, base + 16 * k * 256 + o.s128[s][0]);
    const uint2 hi = lds_ld<uint2>(lds, base + 16 * k * 256 + o.s128[s][1]);
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}
// Split K groups, row 16 k + r of a [.][64] tile.
__device__ __forceinline__ bf16x8 ld_s64(const unsigned char* lds, const LaneOffs& o, int base, int k, int s)
{
    const uint2 lo = lds_ld<uint2>(lds, base + 16 * k * 128 + o.s64[s][0]);
    const uint2 hi = lds_ld<uint2>(lds, base + 16 * k * 128 + o.s64[s][1]);
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
__device__ __forceinline__ float clamp_alpha(float x) { return __builtin_amdgcn_fmed3f(x, kAlphaMin, 1.0f); }

// Raw buffer resources: one descriptor per tensor window, 32-bit per-lane
// offsets and per-token offsets in scalar registers.  Every access is guarded
// by an explicit token test, so the descriptor's own range check is not relied
// upon (its num_records is the window size).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;  // 32-bit raw buffer, gfx9 family

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), kRsrcFlags);
}

template <int DVT>
struct Raw {  // one thread's share of a chunk's global inputs
    static constexpr int kVW = DVT / 64;  // 16-byte value words per thread
    uint32_t q[8], k[8], b[8];            // 2 bf16 channels x 8 tokens
    float2 a[8];                          // alpha, 2 channels x 8 tokens
    uint4 v[kVW], w[kVW];                 // DVT / 8 value columns of one token
};

// Loads chunk [t0, t0 + L) of head h.  Key side: wavefront w reads tokens
// 8 w .. 8 w + 7, lane l the channel pair 2 l, 2 l + 1 (whole rows per
// instruction).  Value side: thread t reads DVT / 8 columns of token t / 8.
template <int DVT>
__device__ __forceinline__ void load_raw(Raw<DVT>& R, const ChunkArgs& a, int64_t brow, int64_t t0, int L,
                                         int h, int j0, int tid, int wave)
{
    const int lane = tid & 63;
    const int64_t row0 = (brow * a.T + t0) * a.H + h;  // (token t0, head h)
    const uint32_t kstride = uint32_t(a.H) * kDK * 2;  // bytes per token, bf16 key rows
    const uint32_t win = uint32_t(kC) * kstride;
    const rsrc_t rq = make_rsrc(static_cast<const bf16raw*>(a.q) + row0 * kDK, win);
    const rsrc_t rk = make_rsrc(static_cast<const bf16raw*>(a.k) + row0 * kDK, win);
    const rsrc_t rb = make_rsrc(static_cast<const bf16raw*>(a.b) + row0 * kDK, win);
    const rsrc_t ra = make_rsrc(a.alpha + row0 * kDK, 2 * win);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int tok = 8 * wave + i;
        if (tok < L) {
            const int so = tok * int(kstride);
            R.q[i] = __builtin_amdgcn_raw_buffer_load_b32(rq, 4 * lane, so, 0);
            R.k[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, 4 * lane, so, 0);
            R.b[i] = __builtin_amdgcn_raw_buffer_load_b32(rb, 4 * lane, so, 0);
            const u32x2 av = __builtin_amdgcn_raw_buffer_load_b64(ra, 8 * lane, 2 * so, 0);
            R.a[i] = make_float2(__uint_as_float(av[0]), __uint_as_float(av[1]));
        } else {
            R.q[i] = R.k[i] = R.b[i] = 0u;
            R.a[i] = make_float2(1.f, 1.f);
        }
    }
    constexpr int kVW = Raw<DVT>::kVW;
    const int vtok = tid >> 3, cz = tid & 7;
    const uint32_t vstride = uint32_t(a.H) * uint32_t(a.dv) * 2;
    const int64_t vrow0 = row0 * a.dv + j0;
    const rsrc_t rv = make_rsrc(static_cast<const bf16raw*>(a.v) + vrow0, uint32_t(kC) * vstride);
    const rsrc_t rw = make_rsrc(static_cast<const bf16raw*>(a.w) + vrow0, uint32_t(kC) * vstride);
    if (vtok < L) {
        const int vo = vtok * int(vstride) + 16 * kVW * cz;
#pragma unroll
        for (int u = 0; u < kVW; ++u) {
            const auto x = __builtin_amdgcn_raw_buffer_load_b128(rv, vo + 16 * u, 0, 0);
            const auto y = __builtin_amdgcn_raw_buffer_load_b128(rw, vo + 16 * u, 0, 0);
            R.v[u] = make_uint4(x[0], x[1], x[2], x[3]);
            R.w[u] = make_uint4(y[0], y[1], y[2], y[3]);
        }
    } else {
#pragma unroll
        for (int u = 0; u < kVW; ++u) R.v[u] = R.w[u] = make_uint4(0u, 0u, 0u, 0u);
    }
}

// Key-side elementwise work of one chunk (all threads): decay factors, the
// bf16 operand tiles Eh, Qh, Kh, Ko, Et, Qt, KbT, the value tile z = w v and
// the chunk decay gamma.  Ends with the tiles visible to every wavefront.
// Thread (wavefront hb, lane cp) handles tokens 8 hb .. 8 hb + 7 (half hb & 1
// of block hb >> 1) for channels 2 cp, 2 cp + 1.
template <int DVT>
__device__ __forceinline__ void prep_chunk(unsigned char* lds, const Raw<DVT>& R, int tid, int hb)
{
    const int cp = tid & 63;
    const int blk = hb >> 1, half = hb & 1;
    const float* ph = reinterpret_cast<const float*>(lds + Lds<DVT>::kOffPh);

    // pass 1: products of the clamped decay over this half block
    float al0[8], al1[8];
    float p0 = 1.f, p1 = 1.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        al0[i] = clamp_alpha(R.a[i].x);
        al1[i] = clamp_alpha(R.a[i].y);
        p0 *= al0[i];
        p1 *= al1[i];
    }
    lds_st<float2>(lds, Lds<DVT>::kOffPh + (hb * 128 + 2 * cp) * 4, make_float2(p0, p1));
    __syncthreads();

    // pass 2: factors between the block references, for this thread's channels
    float s1[2], s2[2], dsc[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int ch = 2 * cp + c;
        float lo[4], hi[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            lo[J] = ph[(2 * J) * 128 + ch];      // block start -> reference token
            hi[J] = ph[(2 * J + 1) * 128 + ch];  // reference token -> block end
        }
        float pre = 1.f;
#pragma unroll
        for (int J = 0; J < 4; ++J)
            if (J < blk) pre *= lo[J] * hi[J];
        s1[c] = pre * lo[blk];  // 2^(m_blk): chunk start -> reference of blk
        float post = hi[blk];
#pragma unroll
        for (int J = 0; J < 4; ++J)
            if (J > blk) post *= lo[J] * hi[J];
        s2[c] = post;  // 2^(G_last - m_blk)
        float run = hi[blk];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            if (I > blk) {
                dsc[c][I] = run * lo[I];  // 2^(m_I - m_blk)
                run *= lo[I] * hi[I];
            } else {
                dsc[c][I] = 0.f;
            }
        }
        if (hb == 0) {
            float gam = 1.f;
#pragma unroll
            for (int J = 0; J < 4; ++J) gam *= lo[J] * hi[J];
            reinterpret_cast<float*>(lds + Lds<DVT>::kOffGam)[ch] = gam;
        }
    }

    // per-token factors r = 2^(G_i - m), ri = 2^(m - G_i) around the block's
    // reference m (the last token of half 0):
    //   half 0: r_i = prod alpha[0..i] / p,   ri_i = prod alpha[i+1..7]
    //   half 1: r_i = prod alpha[0..i],       ri_i = prod alpha[i+1..7] / p
    // with p the product over the whole half.
    const float inv0 = __builtin_amdgcn_rcpf(p0), inv1 = __builtin_amdgcn_rcpf(p1);
    float suf0[8], suf1[8];
    suf0[7] = 1.f;
    suf1[7] = 1.f;
#pragma unroll
    for (int i = 6; i >= 0; --i) {
        suf0[i] = suf0[i + 1] * al0[i + 1];
        suf1[i] = suf1[i + 1] * al1[i + 1];
    }
    float cum0 = 1.f, cum1 = 1.f;
    uint32_t kb0[4], kb1[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        cum0 *= al0[i];
        cum1 *= al1[i];
        float r0, r1, ri0, ri1;
        if (half == 0) {
            r0 = i == 7 ? 1.f : cum0 * inv0;
            r1 = i == 7 ? 1.f : cum1 * inv1;
            ri0 = suf0[i];
            ri1 = suf1[i];
        } else {
            r0 = cum0;
            r1 = cum1;
            ri0 = suf0[i] * inv0;
            ri1 = suf1[i] * inv1;
        }
        const int row = 8 * hb + i;
        const float q0 = lo_f(R.q[i]), q1 = hi_f(R.q[i]);
        const float k0 = lo_f(R.k[i]), k1 = hi_f(R.k[i]);
        const float e0 = lo_f(R.b[i]) * k0, e1 = hi_f(R.b[i]) * k1;
        const float eh0 = e0 * r0, eh1 = e1 * r1;
        const float qh0 = q0 * r0, qh1 = q1 * r1;
        const float kh0 = k0 * ri0, kh1 = k1 * ri1;
        const int off = off_rc128(row, 2 * cp);
        lds_st<uint32_t>(lds, kOffEh + off, pack2(eh0, eh1));
        lds_st<uint32_t>(lds, kOffQh + off, pack2(qh0, qh1));
        lds_st<uint32_t>(lds, kOffKh + off, pack2(kh0, kh1));
        lds_st<uint32_t>(lds, kOffEt + off, pack2(eh0 * s1[0], eh1 * s1[1]));
        lds_st<uint32_t>(lds, kOffQt + off, pack2(qh0 * s1[0], qh1 * s1[1]));
#pragma unroll
        for (int I = 1; I < 4; ++I)
            if (I > blk) {
                const int pair = I * (I - 1) / 2 + blk;
                lds_st<uint32_t>(lds, kOffKo + pair * 4096 + off_rc128(8 * half + i, 2 * cp),
                                 pack2(kh0 * dsc[0][I], kh1 * dsc[1][I]));
            }
        const uint32_t kbp = pack2(kh0 * s2[0], kh1 * s2[1]);  // (channel 0, channel 1)
        if (i & 1) {
            kb0[i >> 1] |= kbp << 16;
            kb1[i >> 1] |= kbp & 0xffff0000u;
        } else {
            kb0[i >> 1] = kbp & 0xffffu;
            kb1[i >> 1] = kbp >> 16;
        }
    }
    lds_st<uint4>(lds, kOffKbT + off_rc64(2 * cp, 8 * hb), make_uint4(kb0[0], kb0[1], kb0[2], kb0[3]));
    lds_st<uint4>(lds, kOffKbT + off_rc64(2 * cp + 1, 8 * hb), make_uint4(kb1[0], kb1[1], kb1[2], kb1[3]));

    // z = w (.) v, column major for the accumulator-layout reads
    {
        constexpr int kVW = Raw<DVT>::kVW;
        const int tok = tid >> 3, cz = tid & 7;
        float* zs = reinterpret_cast<float*>(lds + kOffZs);
#pragma unroll
        for (int u = 0; u < kVW; ++u) {
            const uint32_t vv[4] = {R.v[u].x, R.v[u].y, R.v[u].z, R.v[u].w};
            const uint32_t ww[4] = {R.w[u].x, R.w[u].y, R.w[u].z, R.w[u].w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int col = 8 * kVW * cz + 8 * u + 2 * j;
                zs[col * kZsStride + tok] = lo_f(ww[j]) * lo_f(vv[j]);
                zs[(col + 1) * kZsStride + tok] = hi_f(ww[j]) * hi_f(vv[j]);
            }
        }
    }
    __syncthreads();
}

// One A or P block product.  Off-diagonal blocks and all P blocks are formed
// transposed (K rows as the A operand), which leaves row 16 I + r, columns
// 16 J + 4 g .. + 3 in each lane; the diagonal A block is formed directly and
// stored column major in FP32 for the forward substitution.
struct Item {
    int kind;  // 0: A block, 1: P block
    int I, J;
};

__device__ __forceinline__ void ap_block(const unsigned char* lds, const LaneOffs& o, const Item it, f32x4& acc)
{
    const int rowbase = it.kind == 0 ? kOffEh : kOffQh;
    const bool diag = it.J == it.I;
    const int kbase = diag ? kOffKh : kOffKo + (it.I * (it.I - 1) / 2 + it.J) * 4096;
    const int kblk = diag ? it.J : 0;
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
    if (it.kind == 0 && diag) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc = mfma_bf16(ld_c128(lds, o, rowbase, it.I, s), ld_c128(lds, o, kbase, kblk, s), acc);
    } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            acc = mfma_bf16(ld_c128(lds, o, kbase, kblk, s), ld_c128(lds, o, rowbase, it.I, s), acc);
    }
}

__device__ __forceinline__ void ap_store(unsigned char* lds, const Item it, int r, int g, const f32x4 acc)
{
    const int row = 16 * it.I + r;      // transposed blocks: this lane's row
    const int col = 16 * it.J + 4 * g;  // .. and its four columns
    if (it.kind == 0) {
        if (it.J < it.I) {
            lds_st<uint2>(lds, kOffAneg + off_rc64(row, col),
                          make_uint2(pack2(-acc[0], -acc[1]), pack2(-acc[2], -acc[3])));
        } else {
            // direct block: column r, rows 4g..4g+3; strictly lower part only
            float4 v;
            v.x = 4 * g + 0 > r ? acc[0] : 0.f;
            v.y = 4 * g + 1 > r ? acc[1] : 0.f;
            v.z = 4 * g + 2 > r ? acc[2] : 0.f;
            v.w = 4 * g + 3 > r ? acc[3] : 0.f;
            lds_st<float4>(lds, kOffAdT + ((it.I * 16 + r) * 16 + 4 * g) * 4, v);
            if (it.I == 1 || it.I == 3)  // diagonal blocks the blocked solve reads as zero
                lds_st<uint2>(lds, kOffAneg + off_rc64(row, col), make_uint2(0u, 0u));
        }
    } else {
        if (it.J < it.I) {
            lds_st<uint2>(lds, kOffP + off_rc64(row, col), make_uint2(pack2(acc[0], acc[1]), pack2(acc[2], acc[3])));
        } else {
            const float p0 = col + 0 <= row ? acc[0] : 0.f, p1 = col + 1 <= row ? acc[1] : 0.f;
            const float p2 = col + 2 <= row ? acc[2] : 0.f, p3 = col + 3 <= row ? acc[3] : 0.f;
            lds_st<uint2>(lds, kOffP + off_rc64(row, col), make_uint2(pack2(p0, p1), pack2(p2, p3)));
            if (it.I == 0 || it.I == 2)  // block right of the diagonal, read by P U as zero
                lds_st<uint2>(lds, kOffP + off_rc64(row, col + 16), make_uint2(0u, 0u));
        }
    }
}

// A/P work items of wavefront w (20 blocks over 8 wavefronts).
__device__ __forceinline__ int ap_items(int w, Item* out)
{
    switch (w) {
        case 0: out[0] = {0, 3, 0}; out[1] = {0, 3, 1}; return 2;
        case 1: out[0] = {0, 3, 2}; out[1] = {0, 3, 3}; return 2;
        case 2: out[0] = {1, 3, 0}; out[1] = {1, 3, 1}; return 2;
        case 3: out[0] = {1, 3, 2}; out[1] = {1, 3, 3}; return 2;
        case 4: out[0] = {0, 2, 0}; out[1] = {0, 2, 1}; out[2] = {0, 2, 2}; return 3;
        case 5: out[0] = {1, 2, 0}; out[1] = {1, 2, 1}; out[2] = {1, 2, 2}; return 3;
        case 6: out[0] = {0, 1, 0}; out[1] = {0, 1, 1}; out[2] = {0, 0, 0}; return 3;
        default: out[0] = {1, 1, 0}; out[1] = {1, 1, 1}; out[2] = {1, 0, 0}; return 3;
    }
}

template <int VW>
__global__ __launch_bounds__(kThreads) void chunk_fwd_mfma_kernel(ChunkArgs a, int ntiles, int nchains)
{
    constexpr int DVT = 16 * VW;
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int g = lane >> 4, r = lane & 15;
    const bool vwave = wave < VW;

    // XCD-aware mapping: all tiles of a chain share blockIdx.x % 8.
    const int bid = blockIdx.x;
    const int xcd = bid & 7, slot = bid >> 3;
    const int tile = slot % ntiles;
    const int chain = (slot / ntiles) * 8 + xcd;
    if (chain >= nchains) return;
    const int n = chain / a.H, h = chain % a.H;
    const int j0 = tile * DVT;
    const int64_t dv = a.dv;

    int64_t bos, eos, brow;
    sequence_bounds(a.cu_seqlens, n, a.T, bos, eos, brow);

    // state slice of a value wavefront: channels 16 cb + 4 g + i, column j0 + 16 wave + r
    f32x4 S[8];
    const int64_t sbase = (int64_t(n) * a.H + h) * kDK * dv + j0;
    const uint32_t sbytes = uint32_t(kDK * dv * 4);
    const int s_vo = ((4 * g) * int(dv) + 16 * wave + r) * 4;
#pragma unroll
    for (int cb = 0; cb < 8; ++cb) S[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (vwave && a.initial_state) {
        const rsrc_t rs = make_rsrc(a.initial_state + sbase, sbytes);
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[cb][i] = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(rs, s_vo, (16 * cb + i) * int(dv) * 4, 0));
    }

    Raw<DVT> R;
    if (bos < eos) load_raw(R, a, brow, bos, int(eos - bos < kC ? eos - bos : kC), h, j0, tid, wave);

    bf16raw* o = static_cast<bf16raw*>(a.o);
    const float* gam = reinterpret_cast<const float*>(lds + Lds<DVT>::kOffGam);
    const float* zcol = reinterpret_cast<const float*>(lds + kOffZs) + (16 * wave + r) * kZsStride;
    Item items[3];
    const int nitems = ap_items(wave, items);
    const LaneOffs lo_ = lane_offsets(r, g);

    for (int64_t t0 = bos; t0 < eos; t0 += kC) {
        const int L = int(eos - t0 < kC ? eos - t0 : kC);
        prep_chunk<DVT>(lds, R, tid, wave);
        if (t0 + kC < eos) {
            const int64_t tn = t0 + kC;
            load_raw(R, a, brow, tn, int(eos - tn < kC ? eos - tn : kC), h, j0, tid, wave);
        }

        // ---- A and P blocks
        f32x4 acc[3];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            if (k < nitems) ap_block(lds, lo_, items[k], acc[k]);
            __builtin_amdgcn_sched_barrier(0);
        }
        __syncthreads();  // region 1 operands consumed
#pragma unroll
        for (int k = 0; k < 3; ++k)
            if (k < nitems) ap_store(lds, items[k], r, g, acc[k]);
        __syncthreads();  // Aneg, P, AdT visible

        // ---- T_II = (I + A_II)^-1, FP32 right-looking substitution; lane group
        // g takes diagonal block g, lane r its column r
        if (wave == kTWave) {
            const float4* adt = reinterpret_cast<const float4*>(lds + kOffAdT) + g * 64;  // column j: adt[4 j ..]
            float t[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) t[i] = i == r ? 1.f : 0.f;
            float4 cur[4], nxt[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; ++q4) cur[q4] = adt[q4];
#pragma unroll
            for (int j = 0; j < 15; ++j) {
                if (j < 14)
#pragma unroll
                    for (int q4 = 0; q4 < 4; ++q4) nxt[q4] = adt[4 * (j + 1) + q4];
                const float col[16] = {cur[0].x, cur[0].y, cur[0].z, cur[0].w, cur[1].x, cur[1].y, cur[1].z, cur[1].w,
                                       cur[2].x, cur[2].y, cur[2].z, cur[2].w, cur[3].x, cur[3].y, cur[3].z, cur[3].w};
#pragma unroll
                for (int i = j + 1; i < 16; ++i) t[i] -= col[i] * t[j];
#pragma unroll
                for (int q4 = 0; q4 < 4; ++q4) cur[q4] = nxt[q4];
                __builtin_amdgcn_sched_barrier(0);
            }
            float* T = reinterpret_cast<float*>(lds + kOffT) + g * 256;
#pragma unroll
            for (int i = 0; i < 16; ++i) T[i * 16 + r] = t[i];
        }

        // ---- X = Z - Et S (direct) and (Qt S)^T
        f32x4 X[4], OT[4];
        bf16x8 sb[4];
        if (vwave) {
#pragma unroll
            for (int s = 0; s < 4; ++s) sb[s] = pack_acc_pair(S[2 * s], S[2 * s + 1]);
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                f32x4 xe = f32x4{0.f, 0.f, 0.f, 0.f}, xq = xe;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    xe = mfma_bf16(ld_s128(lds, lo_, kOffEt, I, s), sb[s], xe);
                    xq = mfma_bf16(sb[s], ld_s128(lds, lo_, kOffQt, I, s), xq);
                }
                const float4 z = *reinterpret_cast<const float4*>(zcol + 16 * I + 4 * g);
                X[I] = f32x4{z.x - xe[0], z.y - xe[1], z.z - xe[2], z.w - xe[3]};
                OT[I] = xq;
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        __syncthreads();  // T visible

        if (vwave) {
            // ---- blocked solve: R_I = X_I - sum_J A_IJ U_J ; U_I = T_II R_I
            f32x4 U[4];
            bf16x8 ub[2];
            const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                f32x4 R_ = X[I];
                if (I >= 1) R_ = mfma_bf16(ld_s64(lds, lo_, kOffAneg, I, 0), ub[0], R_);
                if (I >= 3) R_ = mfma_bf16(ld_s64(lds, lo_, kOffAneg, I, 1), ub[1], R_);
                const float4 tr = *reinterpret_cast<const float4*>(lds + kOffT + ((I * 16 + r) * 16 + 4 * g) * 4);
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
            const uint32_t ostride = uint32_t(a.H) * uint32_t(dv) * 2;
            const rsrc_t ro = make_rsrc(o + ((brow * a.T + t0) * a.H + h) * dv + j0, uint32_t(kC) * ostride);
            const int o_vo = r * int(ostride) + (16 * wave + 4 * g) * 2;
#pragma unroll
            for (int I = 0; I < 4; ++I) {
                f32x4 acc2 = OT[I];
                acc2 = mfma_bf16(ub[0], ld_s64(lds, lo_, kOffP, I, 0), acc2);
                if (I >= 2) acc2 = mfma_bf16(ub[1], ld_s64(lds, lo_, kOffP, I, 1), acc2);
                if (16 * I + r < L) {
                    u32x2 pk;
                    pk[0] = pack2(acc2[0], acc2[1]);
                    pk[1] = pack2(acc2[2], acc2[3]);
                    __builtin_amdgcn_raw_buffer_store_b64(pk, ro, o_vo, 16 * I * int(ostride), 0);
                }
            }

            // ---- S <- Diag(gamma) S + Kb^T U
#pragma unroll
            for (int cb = 0; cb < 8; ++cb) {
                const float4 gm = *reinterpret_cast<const float4*>(gam + 16 * cb + 4 * g);
                f32x4 acc3 = f32x4{S[cb][0] * gm.x, S[cb][1] * gm.y, S[cb][2] * gm.z, S[cb][3] * gm.w};
                acc3 = mfma_bf16(ld_s64(lds, lo_, kOffKbT, cb, 0), ub[0], acc3);
                acc3 = mfma_bf16(ld_s64(lds, lo_, kOffKbT, cb, 1), ub[1], acc3);
                S[cb] = acc3;
            }
        }
        __syncthreads();  // all reads of this chunk's tiles done
    }

    if (vwave && a.final_state) {
        const rsrc_t rs = make_rsrc(a.final_state + sbase, sbytes);
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(S[cb][i]), rs, s_vo,
                                                      (16 * cb + i) * int(dv) * 4, 0);
    }
}

template <int VW>
hipError_t launch_vw(const ChunkArgs& a, hipStream_t stream)
{
    constexpr int DVT = 16 * VW;
    constexpr int kBytes = Lds<DVT>::kBytes;
    // Allow the kernel its > 64 KiB of dynamic LDS (thread-safe one-time call).
    static const hipError_t attr = hipFuncSetAttribute(reinterpret_cast<const void*>(chunk_fwd_mfma_kernel<VW>),
                                                       hipFuncAttributeMaxDynamicSharedMemorySize, kBytes);
    if (attr != hipSuccess) return attr;
    const int ntiles = a.dv / DVT;
    const int64_t chains = int64_t(a.N) * a.H;
    const int64_t blocks = (chains + 7) / 8 * 8 * ntiles;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(chunk_fwd_mfma_kernel<VW>, dim3(unsigned(blocks)), dim3(kThreads), kBytes, stream, a, ntiles,
                       int(chains));
    return hipGetLastError();
}

}  // namespace

bool chunk_fwd_mfma_supported(const ChunkArgs& a, bool bf16)
{
    return bf16 && a.dk == kDK && a.dv % 64 == 0;
}

hipError_t launch_chunk_fwd_mfma(const ChunkArgs& a, hipStream_t stream)
{
    // 128-column tiles carry the key-side work once per chain; 64-column tiles
    // spread a chain over two workgroups when chains alone do not fill the chip.
    const int64_t chains = int64_t(a.N) * a.H;
    if (a.dv % 128 == 0 && chains >= a.cus) return launch_vw<8>(a, stream);
    return launch_vw<4>(a, stream);
}

}  // namespace gdn2
