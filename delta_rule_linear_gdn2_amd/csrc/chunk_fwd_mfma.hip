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
// earlier block the column factor is <= 1.  The factors are running products of
// alpha inside a block (FP32), plus one reciprocal per element; block-to-block
// factors are products of per-block alpha products.  Underflow of a factor
// that is <= 1 only drops terms below 2^-126 of their neighbours.
//
// Matrix products (v_mfma_f32_16x16x32_bf16, FP32 accumulate):
//     A, P blocks (Eh Kh^T, Qh Kh^T, 16x16 output, K = 128 channels)
//     Et S, Qt S          (64 x 16 per wavefront, K = 128)
//     off-diagonal solve  R_I = X_I - A_IJ U_J   (K = tokens of earlier blocks)
//     P U, Kb^T U         (K = 64 tokens)
// and in FP32 (v_mfma_f32_16x16x4_f32) the diagonal-block solve U_I = T_II R_I,
// with T_II = (I + A_II)^-1 formed by FP32 forward substitution.
//
// Work split.  One 256-thread workgroup (four wavefronts) per (sequence, head,
// 64-column value tile); wavefront w owns value columns 16w..16w+15 and keeps
// that 128 x 16 slice of the FP32 state in its MFMA accumulators for the whole
// sequence.  All four wavefronts share the key-side work of a chunk (decay
// factors, A, P, T) through LDS.  Workgroups of the same chain are placed on
// the same XCD so the second tile re-reads the key-side inputs from L2.
//
// Operand layouts (16x16x32 bf16): lane l = 16 g + r provides row/column r and
// a group of eight K indices chosen by g.  The contraction only needs A and B
// to agree on the K order, so K groups are chosen per product to match the
// accumulator layout of the other operand (lane l holds output rows 4g..4g+3
// of column r): for a K-step over 32 channels or tokens, group g takes indices
// {4g..4g+3} and {16+4g..16+4g+3}, which are exactly the rows that lane
// already holds in two adjacent accumulator blocks.
#include "gdn2_device.hpp"
#include "launch.hpp"

namespace gdn2 {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDK = 128;       // key head size
constexpr int kC = 64;         // chunk
constexpr int kWaves = 4;      // wavefronts per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kDVT = 16 * kWaves;  // value columns per workgroup
constexpr float kAlphaMin = 3.0517578125e-05f;  // 2^-15

// ---- LDS map (bytes) -------------------------------------------------------
// Region 1, prep -> A/P:  Eh, Qh, Kh [64][128] bf16, Ko [6][16][128] bf16
// Region 1, A/P -> end:   Aneg, P [64][64] bf16, Ad, T [4][16][16] f32
// Region 2, prep -> end:  Et, Qt [64][128] bf16, KbT [128][64] bf16, Zs [64][68] f32
constexpr int kOffEh = 0, kOffQh = 16384, kOffKh = 32768, kOffKo = 49152;  // .. 73728
constexpr int kOffAneg = 0, kOffP = 8192, kOffAd = 16384, kOffT = 20480;   // .. 24576
constexpr int kOffEt = 73728, kOffQt = 90112, kOffKbT = 106496, kOffZs = 122880;
constexpr int kZsStride = 68;  // floats per value column in Zs
constexpr int kOffPblk = 122880 + 64 * kZsStride * 4;  // [4 blocks][2][128] f32
constexpr int kOffGam = kOffPblk + 4 * 2 * 128 * 4;    // [128] f32
constexpr int kLdsBytes = kOffGam + 128 * 4;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");

// Byte offset of (row, ch) in a [rows][128] bf16 tile; 16-byte granules are
// XOR-swizzled by the row so that 16 rows read at one granule column hit
// different banks.
__device__ __forceinline__ int off_rc128(int row, int ch)
{
    return row * 256 + ((((ch >> 3) ^ row) & 15) << 4) + ((ch & 7) << 1);
}
// Byte offset of (row, col) in a [rows][64] bf16 tile (granule XOR by row/2,
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

// A-operand of a [rows][128] tile, contiguous K groups: lane (r, g) reads
// channels 32 s + 8 g .. +7 of row `row`.
__device__ __forceinline__ bf16x8 ld_rowk_contig(const unsigned char* lds, int base, int row, int s, int g)
{
    return as_bf16x8(lds_ld<uint4>(lds, base + off_rc128(row, 32 * s + 8 * g)));
}
// Same tile with split K groups {32s+4g..+3} U {32s+16+4g..+3}.
__device__ __forceinline__ bf16x8 ld_rowk_split128(const unsigned char* lds, int base, int row, int s, int g)
{
    const uint2 lo = lds_ld<uint2>(lds, base + off_rc128(row, 32 * s + 4 * g));
    const uint2 hi = lds_ld<uint2>(lds, base + off_rc128(row, 32 * s + 16 + 4 * g));
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}
// Split K groups on a [rows][64] tile.
__device__ __forceinline__ bf16x8 ld_rowk_split64(const unsigned char* lds, int base, int row, int s, int g)
{
    const uint2 lo = lds_ld<uint2>(lds, base + off_rc64(row, 32 * s + 4 * g));
    const uint2 hi = lds_ld<uint2>(lds, base + off_rc64(row, 32 * s + 16 + 4 * g));
    return as_bf16x8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}
// B-operand from two accumulator blocks held by this lane (rows 4g..4g+3 of
// blocks 2s and 2s+1), rounded to bf16.
__device__ __forceinline__ bf16x8 pack_acc_pair(f32x4 lo, f32x4 hi)
{
    return as_bf16x8(make_uint4(pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(hi[0], hi[1]),
                                pack2(hi[2], hi[3])));
}

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

struct Raw {  // one thread's share of a chunk's global inputs
    uint32_t q[16], k[16], b[16];  // 2 bf16 channels x 16 tokens
    float2 a[16];                  // alpha, 2 channels x 16 tokens
    uint4 v[2], w[2];              // 16 value columns of one token
};

// Loads chunk [t0, t0 + L) of head h.  Key side: wavefront w reads tokens
// 16 w .. 16 w + 15, lane l the channel pair 2 l, 2 l + 1 (whole rows per
// instruction).  Value side: thread t reads 16 columns of token t / 4.
__device__ __forceinline__ void load_raw(Raw& R, const ChunkArgs& a, int64_t brow, int64_t t0, int L, int h,
                                         int j0, int tid)
{
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int64_t row0 = (brow * a.T + t0) * a.H + h;  // (token t0, head h)
    const uint32_t kstride = uint32_t(a.H) * kDK * 2;  // bytes per token, bf16 key rows
    const uint32_t win = uint32_t(kC) * kstride;
    const rsrc_t rq = make_rsrc(static_cast<const bf16raw*>(a.q) + row0 * kDK, win);
    const rsrc_t rk = make_rsrc(static_cast<const bf16raw*>(a.k) + row0 * kDK, win);
    const rsrc_t rb = make_rsrc(static_cast<const bf16raw*>(a.b) + row0 * kDK, win);
    const rsrc_t ra = make_rsrc(a.alpha + row0 * kDK, 2 * win);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int tok = 16 * wave + i;
        if (tok < L) {
            const int so = tok * int(kstride);
            R.q[i] = __builtin_amdgcn_raw_buffer_load_b32(rq, 4 * lane, so, 0);
            R.k[i] = __builtin_amdgcn_raw_buffer_load_b32(rk, 4 * lane, so, 0);
            R.b[i] = __builtin_amdgcn_raw_buffer_load_b32(rb, 4 * lane, so, 0);
            const auto av = __builtin_amdgcn_raw_buffer_load_b64(ra, 8 * lane, 2 * so, 0);
            R.a[i] = make_float2(__uint_as_float(av[0]), __uint_as_float(av[1]));
        } else {
            R.q[i] = R.k[i] = R.b[i] = 0u;
            R.a[i] = make_float2(1.f, 1.f);
        }
    }
    const int vtok = tid >> 2, cq = tid & 3;
    const uint32_t vstride = uint32_t(a.H) * uint32_t(a.dv) * 2;
    const int64_t vrow0 = row0 * a.dv + j0;
    const rsrc_t rv = make_rsrc(static_cast<const bf16raw*>(a.v) + vrow0, uint32_t(kC) * vstride);
    const rsrc_t rw = make_rsrc(static_cast<const bf16raw*>(a.w) + vrow0, uint32_t(kC) * vstride);
    if (vtok < L) {
        const int vo = vtok * int(vstride) + 32 * cq;
        auto x0 = __builtin_amdgcn_raw_buffer_load_b128(rv, vo, 0, 0);
        auto x1 = __builtin_amdgcn_raw_buffer_load_b128(rv, vo + 16, 0, 0);
        auto y0 = __builtin_amdgcn_raw_buffer_load_b128(rw, vo, 0, 0);
        auto y1 = __builtin_amdgcn_raw_buffer_load_b128(rw, vo + 16, 0, 0);
        R.v[0] = make_uint4(x0[0], x0[1], x0[2], x0[3]);
        R.v[1] = make_uint4(x1[0], x1[1], x1[2], x1[3]);
        R.w[0] = make_uint4(y0[0], y0[1], y0[2], y0[3]);
        R.w[1] = make_uint4(y1[0], y1[1], y1[2], y1[3]);
    } else {
        R.v[0] = R.v[1] = R.w[0] = R.w[1] = make_uint4(0u, 0u, 0u, 0u);
    }
}

__device__ __forceinline__ float lo_f(uint32_t x) { return __uint_as_float(x << 16); }
__device__ __forceinline__ float hi_f(uint32_t x) { return __uint_as_float(x & 0xffff0000u); }

// Key-side elementwise work of one chunk (all threads): decay factors, the
// bf16 operand tiles Eh, Qh, Kh, Ko, Et, Qt, KbT, the value tile z = w v and
// the chunk decay gamma.  Ends with the tiles visible to every wavefront.
__device__ __forceinline__ void prep_chunk(unsigned char* lds, const Raw& R, int tid)
{
    const int blk = tid >> 6;        // this thread's 16-token block
    const int cp = tid & 63;         // channels 2 cp, 2 cp + 1
    float* pblk = reinterpret_cast<float*>(lds + kOffPblk);

    // pass 1: per-channel alpha products over the block's two halves
    float plo[2], phi[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        float p = 1.f, q = 1.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) p *= __builtin_amdgcn_fmed3f(c ? R.a[i].y : R.a[i].x, kAlphaMin, 1.0f);
#pragma unroll
        for (int i = 8; i < 16; ++i) q *= __builtin_amdgcn_fmed3f(c ? R.a[i].y : R.a[i].x, kAlphaMin, 1.0f);
        plo[c] = p;  // 2^(m - c_blk): block start -> reference token
        phi[c] = q;  // 2^(end_blk - m): reference token -> block end
        pblk[(blk * 2 + 0) * 128 + 2 * cp + c] = p;
        pblk[(blk * 2 + 1) * 128 + 2 * cp + c] = q;
    }
    __syncthreads();

    // block-to-block factors for this thread's two channels
    float s1[2], s2[2], dsc[2][4];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int ch = 2 * cp + c;
        float lo[4], hi[4];
#pragma unroll
        for (int J = 0; J < 4; ++J) {
            lo[J] = pblk[(J * 2 + 0) * 128 + ch];
            hi[J] = pblk[(J * 2 + 1) * 128 + ch];
        }
        float pre = 1.f;  // chunk start -> start of block blk
#pragma unroll
        for (int J = 0; J < 4; ++J)
            if (J < blk) pre *= lo[J] * hi[J];
        s1[c] = pre * lo[blk];  // 2^(m_blk)
        float post = hi[blk];   // m_blk -> chunk end
#pragma unroll
        for (int J = 0; J < 4; ++J)
            if (J > blk) post *= lo[J] * hi[J];
        s2[c] = post;
        // 2^(m_I - m_blk) for later blocks I
        float run = hi[blk];
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            if (I > blk) {
                dsc[c][I] = run * lo[I];
                run *= lo[I] * hi[I];
            } else {
                dsc[c][I] = 0.f;
            }
        }
        if (blk == 0) {
            float gam = 1.f;
#pragma unroll
            for (int J = 0; J < 4; ++J) gam *= lo[J] * hi[J];
            reinterpret_cast<float*>(lds + kOffGam)[ch] = gam;
        }
    }

    // pass 2: tokens in order.  With cum_i = prod alpha over [0, i] of the
    // block, the factors around the reference token m (local 7) are
    //   i <= 7: r_i = 2^(G_i - m) = cum_i / plo,   ri_i = 1 / r_i = plo / cum_i
    //   i >  7: r_i = prod alpha over [8, i],       ri_i = 1 / r_i
    const float ip0 = __builtin_amdgcn_rcpf(plo[0]), ip1 = __builtin_amdgcn_rcpf(plo[1]);
    float cum0 = 1.f, cum1 = 1.f;
    uint32_t kb_pk[2][8];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float a0 = __builtin_amdgcn_fmed3f(R.a[i].x, kAlphaMin, 1.0f);
        const float a1 = __builtin_amdgcn_fmed3f(R.a[i].y, kAlphaMin, 1.0f);
        if (i == 8) cum0 = cum1 = 1.f;
        cum0 *= a0;
        cum1 *= a1;
        float r0, r1, ri0, ri1;
        if (i < 7) {
            r0 = cum0 * ip0;
            r1 = cum1 * ip1;
            ri0 = plo[0] * __builtin_amdgcn_rcpf(cum0);
            ri1 = plo[1] * __builtin_amdgcn_rcpf(cum1);
        } else if (i == 7) {
            r0 = r1 = ri0 = ri1 = 1.f;
        } else {
            r0 = cum0;
            r1 = cum1;
            ri0 = __builtin_amdgcn_rcpf(cum0);
            ri1 = __builtin_amdgcn_rcpf(cum1);
        }
        const int row = 16 * blk + i;
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
        for (int I = 0; I < 4; ++I)
            if (I > blk) {
                const int pair = I * (I - 1) / 2 + blk;
                lds_st<uint32_t>(lds, kOffKo + pair * 4096 + off_rc128(i, 2 * cp),
                                 pack2(kh0 * dsc[0][I], kh1 * dsc[1][I]));
            }
        const float kb0 = kh0 * s2[0], kb1 = kh1 * s2[1];
        if (i & 1) {
            kb_pk[0][i >> 1] |= pack2(0.f, kb0) & 0xffff0000u;
            kb_pk[1][i >> 1] |= pack2(0.f, kb1) & 0xffff0000u;
        } else {
            kb_pk[0][i >> 1] = pack2(kb0, 0.f) & 0xffffu;
            kb_pk[1][i >> 1] = pack2(kb1, 0.f) & 0xffffu;
        }
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int ch = 2 * cp + c;
        lds_st<uint4>(lds, kOffKbT + off_rc64(ch, 16 * blk),
                      make_uint4(kb_pk[c][0], kb_pk[c][1], kb_pk[c][2], kb_pk[c][3]));
        lds_st<uint4>(lds, kOffKbT + off_rc64(ch, 16 * blk + 8),
                      make_uint4(kb_pk[c][4], kb_pk[c][5], kb_pk[c][6], kb_pk[c][7]));
    }
    // z = w (.) v, stored column-major for the accumulator-layout reads
    {
        const int tok = tid >> 2, cq = tid & 3;
        float* zs = reinterpret_cast<float*>(lds + kOffZs);
        const uint32_t vv[8] = {R.v[0].x, R.v[0].y, R.v[0].z, R.v[0].w, R.v[1].x, R.v[1].y, R.v[1].z, R.v[1].w};
        const uint32_t ww[8] = {R.w[0].x, R.w[0].y, R.w[0].z, R.w[0].w, R.w[1].x, R.w[1].y, R.w[1].z, R.w[1].w};
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            zs[(16 * cq + 2 * j) * kZsStride + tok] = lo_f(ww[j]) * lo_f(vv[j]);
            zs[(16 * cq + 2 * j + 1) * kZsStride + tok] = hi_f(ww[j]) * hi_f(vv[j]);
        }
    }
    __syncthreads();
}

__global__ __launch_bounds__(kThreads) void chunk_fwd_mfma_kernel(ChunkArgs a, int ntiles, int nchains)
{
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x;
    const int wave = tid >> 6, lane = tid & 63;
    const int g = lane >> 4, r = lane & 15;

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

    // state slice: channels 16 cb + 4 g + i, column j0 + 16 wave + r
    f32x4 S[8];
    const int64_t sbase = (int64_t(n) * a.H + h) * kDK * dv + j0;
    const uint32_t sbytes = uint32_t(kDK * dv * 4);
    const int s_vo = ((4 * g) * int(dv) + 16 * wave + r) * 4;  // per-lane byte offset
    if (a.initial_state) {
        const rsrc_t rs = make_rsrc(a.initial_state + sbase, sbytes);
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                S[cb][i] = __uint_as_float(
                    __builtin_amdgcn_raw_buffer_load_b32(rs, s_vo, (16 * cb + i) * int(dv) * 4, 0));
    } else {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) S[cb] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    Raw R;
    if (bos < eos) load_raw(R, a, brow, bos, int(eos - bos < kC ? eos - bos : kC), h, j0, tid);

    bf16raw* o = static_cast<bf16raw*>(a.o);
    const float* gam = reinterpret_cast<const float*>(lds + kOffGam);

    for (int64_t t0 = bos; t0 < eos; t0 += kC) {
        const int L = int(eos - t0 < kC ? eos - t0 : kC);
        // output window of this chunk: token t0 of head h, value column j0
        const uint32_t ostride = uint32_t(a.H) * uint32_t(dv) * 2;
        const rsrc_t ro = make_rsrc(o + ((brow * a.T + t0) * a.H + h) * dv + j0, uint32_t(kC) * ostride);
        const int o_vo = (4 * g) * int(ostride) + (16 * wave + r) * 2;
        prep_chunk(lds, R, tid);
        if (t0 + kC < eos) {
            const int64_t tn = t0 + kC;
            load_raw(R, a, brow, tn, int(eos - tn < kC ? eos - tn : kC), h, j0, tid);
        }

        // ---- A and P blocks: wave w takes A row-block w and P row-block 3 - w
        f32x4 accA[4], accP[4];
        {
            const int IA = wave, IP = 3 - wave;
            bf16x8 ea[4], qa[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                ea[s] = ld_rowk_contig(lds, kOffEh, 16 * IA + r, s, g);
                qa[s] = ld_rowk_contig(lds, kOffQh, 16 * IP + r, s, g);
            }
#pragma unroll
            for (int J = 0; J < 4; ++J) {
                accA[J] = f32x4{0.f, 0.f, 0.f, 0.f};
                accP[J] = f32x4{0.f, 0.f, 0.f, 0.f};
                if (J <= IA) {
                    const int base = J == IA ? kOffKh : kOffKo + (IA * (IA - 1) / 2 + J) * 4096;
                    const int row = J == IA ? r + 16 * J : r;
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const bf16x8 kb = as_bf16x8(lds_ld<uint4>(lds, base + off_rc128(row, 32 * s + 8 * g)));
                        accA[J] = mfma_bf16(ea[s], kb, accA[J]);
                    }
                }
                if (J <= IP) {
                    const int base = J == IP ? kOffKh : kOffKo + (IP * (IP - 1) / 2 + J) * 4096;
                    const int row = J == IP ? r + 16 * J : r;
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const bf16x8 kb = as_bf16x8(lds_ld<uint4>(lds, base + off_rc128(row, 32 * s + 8 * g)));
                        accP[J] = mfma_bf16(qa[s], kb, accP[J]);
                    }
                }
            }
        }
        __syncthreads();  // region 1 operands consumed
        {
            const int IA = wave, IP = 3 - wave;
#pragma unroll
            for (int J = 0; J < 4; ++J) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int lr = 4 * g + i;  // row inside the block
                    if (J < IA) {
                        lds_st<bf16raw>(lds, kOffAneg + off_rc64(16 * IA + lr, 16 * J + r),
                                        __builtin_bit_cast(bf16raw, static_cast<__bf16>(-accA[J][i])));
                    } else if (J == IA) {
                        reinterpret_cast<float*>(lds + kOffAd)[(IA * 16 + lr) * 16 + r] = r < lr ? accA[J][i] : 0.f;
                        if (IA == 1 || IA == 3)  // zero diagonal blocks read by the blocked solve
                            lds_st<bf16raw>(lds, kOffAneg + off_rc64(16 * IA + lr, 16 * J + r), bf16raw(0));
                    }
                    if (J < IP) {
                        lds_st<bf16raw>(lds, kOffP + off_rc64(16 * IP + lr, 16 * J + r),
                                        __builtin_bit_cast(bf16raw, static_cast<__bf16>(accP[J][i])));
                    } else if (J == IP) {
                        lds_st<bf16raw>(lds, kOffP + off_rc64(16 * IP + lr, 16 * J + r),
                                        __builtin_bit_cast(bf16raw, static_cast<__bf16>(r <= lr ? accP[J][i] : 0.f)));
                    } else if ((IP == 0 && J == 1) || (IP == 2 && J == 3)) {  // zero blocks read by P U
                        lds_st<bf16raw>(lds, kOffP + off_rc64(16 * IP + lr, 16 * J + r), bf16raw(0));
                    }
                }
            }
        }
        __syncthreads();  // A, P, Ad visible

        // ---- wavefront 0: T_II = (I + A_II)^-1 for the four diagonal blocks, FP32
        if (wave == 0) {
            const float* Ad = reinterpret_cast<const float*>(lds + kOffAd) + g * 256;  // block g
            float t[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float acc = i == r ? 1.f : 0.f;
#pragma unroll
                for (int j = 0; j < i; ++j) acc -= Ad[i * 16 + j] * t[j];
                t[i] = acc;
            }
            float* T = reinterpret_cast<float*>(lds + kOffT) + g * 256;
#pragma unroll
            for (int i = 0; i < 16; ++i) T[i * 16 + r] = t[i];
        }

        // ---- X = Z - Et S and Qt S (independent of T)
        bf16x8 sb[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) sb[s] = pack_acc_pair(S[2 * s], S[2 * s + 1]);
        f32x4 X[4], OQ[4];
        const float* zs = reinterpret_cast<const float*>(lds + kOffZs) + (16 * wave + r) * kZsStride;
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 xe = f32x4{0.f, 0.f, 0.f, 0.f}, xq = xe;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                xe = mfma_bf16(ld_rowk_split128(lds, kOffEt, 16 * I + r, s, g), sb[s], xe);
                xq = mfma_bf16(ld_rowk_split128(lds, kOffQt, 16 * I + r, s, g), sb[s], xq);
            }
            const float4 z = *reinterpret_cast<const float4*>(zs + 16 * I + 4 * g);
            X[I] = f32x4{z.x - xe[0], z.y - xe[1], z.z - xe[2], z.w - xe[3]};
            OQ[I] = xq;
        }
        __syncthreads();  // T visible

        // ---- blocked solve: R_I = X_I - sum_J A_IJ U_J ; U_I = T_II R_I
        f32x4 U[4];
        bf16x8 ub[2];
        ub[0] = ub[1] = as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 R_ = X[I];
            if (I >= 1) R_ = mfma_bf16(ld_rowk_split64(lds, kOffAneg, 16 * I + r, 0, g), ub[0], R_);
            if (I >= 3) R_ = mfma_bf16(ld_rowk_split64(lds, kOffAneg, 16 * I + r, 1, g), ub[1], R_);
            const float4 tr = *reinterpret_cast<const float4*>(lds + kOffT + ((I * 16 + r) * 16 + 4 * g) * 4);
            f32x4 u = f32x4{0.f, 0.f, 0.f, 0.f};
            u = mfma_f32(tr.x, R_[0], u);
            u = mfma_f32(tr.y, R_[1], u);
            u = mfma_f32(tr.z, R_[2], u);
            u = mfma_f32(tr.w, R_[3], u);
            U[I] = u;
            // B-operands over tokens 0..31 and 32..63; blocks not solved yet stay zero
            const f32x4 zero4 = f32x4{0.f, 0.f, 0.f, 0.f};
            if (I == 0) ub[0] = pack_acc_pair(U[0], zero4);
            if (I == 1) ub[0] = pack_acc_pair(U[0], U[1]);
            if (I == 2) ub[1] = pack_acc_pair(U[2], zero4);
            if (I == 3) ub[1] = pack_acc_pair(U[2], U[3]);
        }

        // ---- O = Qt S + P U, stored as bf16
#pragma unroll
        for (int I = 0; I < 4; ++I) {
            f32x4 acc = OQ[I];
            acc = mfma_bf16(ld_rowk_split64(lds, kOffP, 16 * I + r, 0, g), ub[0], acc);
            if (I >= 2) acc = mfma_bf16(ld_rowk_split64(lds, kOffP, 16 * I + r, 1, g), ub[1], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 16 * I + 4 * g + i;
                if (tok < L)
                    __builtin_amdgcn_raw_buffer_store_b16(
                        __builtin_bit_cast(unsigned short, static_cast<__bf16>(acc[i])), ro, o_vo,
                        (16 * I + i) * int(ostride), 0);
            }
        }

        // ---- S <- Diag(gamma) S + Kb^T U
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
            const float4 gm = *reinterpret_cast<const float4*>(gam + 16 * cb + 4 * g);
            f32x4 acc = f32x4{S[cb][0] * gm.x, S[cb][1] * gm.y, S[cb][2] * gm.z, S[cb][3] * gm.w};
            acc = mfma_bf16(ld_rowk_split64(lds, kOffKbT, 16 * cb + r, 0, g), ub[0], acc);
            acc = mfma_bf16(ld_rowk_split64(lds, kOffKbT, 16 * cb + r, 1, g), ub[1], acc);
            S[cb] = acc;
        }
        __syncthreads();  // all reads of this chunk's tiles done
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
    const int64_t groups = (chains + 7) / 8;
    const int64_t blocks = groups * 8 * ntiles;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(chunk_fwd_mfma_kernel, dim3(unsigned(blocks)), dim3(kThreads), kLdsBytes, stream, a,
                       ntiles, int(chains));
    return hipGetLastError();
}

}  // namespace gdn2
