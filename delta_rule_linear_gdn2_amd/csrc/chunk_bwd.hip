// Chunkwise backward pass of the GDN-2 recurrence for gfx950 (FP32
// arithmetic, any supported head size).
//
// The Gated DeltaNet-2 analysis (iplexlaw.co.kr, "Token processing and
// parallel training") asks for a backward pass that accumulates gradients
// through the gated keys and values: the channel-wise decay and erase gate
// stay inside the sums instead of being pulled out as one scalar.  Per chunk
// of L tokens with incoming state S, outgoing-state gradient dS', and per key
// channel G_i = sum_{m<=i} log2 alpha_m, F_ij = 2^(G_i - G_j):
//   forward   A = strict_lower(e k^T . F),  P = lower(q k^T . F)
//             Et = e 2^G,  Qt = q 2^G,  Kb = k 2^(G_L - G)
//             X = Z - Et S,  U = (I + A)^-1 X,  O = Qt S + P U,
//             S' = 2^G_L S + Kb^T U
//   backward  dU = Kb dS' + P^T dO,  dX = (I + A)^-T dU,  dZ = dX
//             dS = 2^G_L dS' + Qt^T dO - Et^T dX          (into the chunk before)
//             dA = -strict_lower(dX U^T),  dP = lower(dO U^T)
//             dEt = -dX S^T,  dQt = dO S^T,  dKb = U dS'^T
//   and through the pairwise factors and the cumulative decay, per channel:
//             de_i = sum_{j<i} dA_ij k_j F_ij + dEt_i 2^G_i
//             dq_i = sum_{j<=i} dP_ij k_j F_ij + dQt_i 2^G_i
//             dk_j = sum_{i>j} dA_ij e_i F_ij + sum_{i>=j} dP_ij q_i F_ij + dKb_j 2^(G_L - G_j)
//             dg_i = e_i de_i + q_i dq_i - k_i dk_i    (the pairwise parts only)
//                    + Et_i dEt_i + Qt_i dQt_i - Kb_i dKb_i
//             dg_L += sum_j Kb_j dKb_j + 2^G_L rowsum(dS' . S)
//             dlog(alpha_m) = sum_{i>=m} dg_i,  dalpha = dlog(alpha) / alpha
//             db = de k,  dk += de b,  dw = dZ v,  dv = dZ w
// (dg is the gradient with respect to the natural-log cumulative decay.)
// Every decay factor is a power of two with a non-positive exponent, so
// nothing overflows.  Where a channel's decay over a chunk stays above 2^-64,
// the pairwise sums use the factor split as 2^G_i 2^-G_j, which turns them
// into matrix products; a power-of-two scale is exact, so the sums are the
// same up to rounding, and below that bound the pairwise form is kept.  alpha
// is clamped to [2^-15, 1] as in the forward kernels; the gradient is zero
// where the clamp is active.
//
// Four kernels, 32-token chunks (the same mathematics as any chunk size):
//   bwd_prep    (chunk x head, all parallel)            A, P, Tm = (I + A)^-1,
//               Et, Qt, Kb and 2^G_L of every chunk, once, into the workspace;
//   bwd_states  (chain x value tile, chunks in order)   X, U = Tm X and the
//               state update; stores every chunk-start state and the U rows;
//   bwd_dstate  (chain x value tile, chunks in reverse) dU, dX = Tm^T dU and
//               the state-gradient recurrence; dv, dw and dS0; stores the dX
//               rows and each chunk-end state gradient;
//   bwd_keys    (chunk x head x channel block)          dA, dP, dEt, dQt, dKb
//               over all value columns, then dq, dk, db and dalpha.
// The two sequential kernels only multiply: all of a chunk's triangular
// algebra is done in parallel beforehand.  The products run on the FP32
// matrix cores (full FP32 arithmetic), one 16 x 16 output block per
// wavefront and instruction group.
#include "gdn2_device.hpp"
#include "launch.hpp"

namespace gdn2 {
namespace {

// Barrier for the sequential kernels, whose workgroups share data through LDS
// alone: a wave waits for its own LDS accesses (lgkmcnt = 0) and meets the
// others at s_barrier, while its global loads (the next chunk's) stay in
// flight; __syncthreads() would wait for them too.  The empty asm statements
// keep the compiler from moving memory accesses across.
__device__ __forceinline__ void lds_sync()
{
    __asm__ volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63, expcnt 7, lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
}

// 2^x with the hardware exponential (about one ulp; results below 2^-126 flush
// to zero, which only drops terms far below FP32 resolution: every factor here
// is at most 1 and multiplies values of order one).
__device__ __forceinline__ float pow2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr int kBwdThreads = 256;  // the parallel kernels
constexpr int CH = kBwdChunk;
constexpr int kTile = 32;          // value columns per workgroup of the sequential kernels
constexpr int kSeqThreads = 512;   // the sequential kernels: two wavefronts per SIMD
constexpr int NG = kSeqThreads / kTile;  // lane groups of the sequential kernels
constexpr int RR = CH / NG;              // chunk rows per thread
static_assert(kBwdThreads == 8 * kTile && CH == 32 && CH % NG == 0, "thread layouts below");

// XCD-aware block order: workgroups that read the same data (the channel
// blocks of one chunk, the value tiles of one chain) get the same blockIdx
// mod 8, so they run on one XCD and share its L2.  Group `group` member
// `member` of G is block ((group / 8) * G + member) * 8 + group % 8; the grid
// is padded to a multiple of 8 G and blocks past the last group exit.
__device__ __forceinline__ void xcd_group(int64_t bid, int G, int64_t& group, int& member)
{
    const int64_t q = bid >> 3;
    member = int(q % G);
    group = (q / G) * 8 + (bid & 7);
}
__host__ __device__ inline int64_t xcd_grid(int64_t groups, int G) { return (groups + 7) / 8 * 8 * G; }

__device__ __forceinline__ int64_t slot_of(const BwdArgs& a, int n, int64_t bos, int m)
{
    return a.cu_seqlens ? (bos + int64_t(m) * CH) / CH + n : int64_t(m);
}

// Offset of the (slot, head) state block of batch row `row` in ws_states / ws_dstates.
__device__ __forceinline__ int64_t slot_base(const BwdArgs& a, int64_t row, int64_t slot, int h)
{
    return ((row * a.slots + slot) * a.H + h) * int64_t(a.dk_) * a.dv_;
}

// Per-chunk prepared block (floats): Tm [CH][CH], Pm [CH][CH], Et, Qt, Kb [CH][dk], gamma [dk].
__host__ __device__ constexpr int64_t prep_floats(int dk) { return 2 * CH * CH + 3 * int64_t(CH) * dk + dk; }
constexpr int kPrepT = 0, kPrepP = CH * CH, kPrepE = 2 * CH * CH;
__device__ __forceinline__ int64_t prep_base(const BwdArgs& a, int64_t row, int64_t slot, int h)
{
    return ((row * a.slots + slot) * a.H + h) * prep_floats(a.dk_);
}

// The chunk that owns a slot (false for an unused slot).
__device__ bool chunk_of_slot(const BwdArgs& a, int64_t row, int64_t slot, int& n, int& m, int64_t& bos,
                              int64_t& eos, int64_t& brow)
{
    if (!a.cu_seqlens) {
        n = int(row);
        m = int(slot);
        sequence_bounds(nullptr, n, a.T, bos, eos, brow);
        return int64_t(m) * CH < eos;
    }
    // first slot of sequence s: bos_s / CH + s, strictly increasing in s; take
    // the last sequence whose first slot is <= slot
    int lo = 0, hi = a.N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        int64_t mb, me, mr;
        sequence_bounds(a.cu_seqlens, mid, a.T, mb, me, mr);
        if (mb / CH + mid <= slot) lo = mid; else hi = mid - 1;
    }
    n = lo;
    sequence_bounds(a.cu_seqlens, n, a.T, bos, eos, brow);
    const int64_t first = bos / CH + n;
    if (slot < first) return false;
    m = int(slot - first);
    return bos + int64_t(m) * CH < eos && slot_of(a, n, bos, m) == slot;
}

// Four consecutive values as FP32 (16-byte FP32 or 8-byte bf16 loads).
__device__ __forceinline__ float4 load4(const float* p, int64_t i) { return *reinterpret_cast<const float4*>(p + i); }
__device__ __forceinline__ float4 load4(const bf16raw* p, int64_t i)
{
    const uint2 u = *reinterpret_cast<const uint2*>(p + i);
    return make_float4(bf16_to_f32(bf16raw(u.x & 0xffffu)), bf16_to_f32(bf16raw(u.x >> 16)),
                       bf16_to_f32(bf16raw(u.y & 0xffffu)), bf16_to_f32(bf16raw(u.y >> 16)));
}
__device__ __forceinline__ void st4(float* row, int j, float4 v)
{
    row[j] = v.x;
    row[j + 1] = v.y;
    row[j + 2] = v.z;
    row[j + 3] = v.w;
}

// ---------------------------------------------------------------------------
// Products on the FP32 matrix cores
// (v_mfma_f32_16x16x4_f32, one 16 x 16 output block per instruction group).
// Lane l of a wavefront supplies A[row l % 16][k l / 16] and B[k l / 16][column
// l % 16] of a K = 4 step, and holds D[rows 4 (l / 16) .. + 3][column l % 16].
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ f32x4_t mfma4(float a, float b, f32x4_t c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
constexpr int kPad = 4;  // row padding of the LDS operands: the b32 operand reads stay free of bank conflicts
// Decay over a chunk (log2) above which a channel's pairwise factors
// 2^(G_i - G_j) may be split into 2^G_i 2^-G_j without overflow.
constexpr float kSplitMinPrep = -64.f;

// The forward quantities of one chunk.  Rows are padded by one float: lanes
// that walk different rows of the same column then fall in different banks.
template <int DK>
struct ChunkRows {
    float Q[CH][DK + 1];  // q, then Qt = q 2^G
    float K[CH][DK + 1];  // k, then Kb = k 2^(G_L - G)
    float E[CH][DK + 1];  // e = b k, then Et = e 2^G
    float G[CH][DK + 1];  // log2 alpha, then its running sum
    float A[CH][CH + 1];
    float P[CH][CH + 1];
};

// ---------------------------------------------------------------------------
// bwd_prep: everything of a chunk that does not involve the state.
template <typename T, int DK>
__global__ __launch_bounds__(kBwdThreads) void bwd_prep_kernel(BwdArgs a)
{
    if (a.gate && *a.gate == 0) return;  // the matrix-core path covers this call
    __shared__ ChunkRows<DK> c;
    __shared__ float Tm[CH][CH + 1];
    __shared__ float glv[DK];  // G at the chunk's last token
    __shared__ int split;      // every channel's decay over the chunk above 2^kSplitMinPrep

    const int tid = threadIdx.x;
    int64_t idx = blockIdx.x;
    const int h = int(idx % a.H);
    idx /= a.H;
    const int64_t slot = idx % a.slots, row = idx / a.slots;
    int n, m;
    int64_t bos, eos, brow;
    if (!chunk_of_slot(a, row, slot, n, m, bos, eos, brow)) return;
    const int64_t t0 = bos + int64_t(m) * CH;
    const int L = int(eos - t0 < CH ? eos - t0 : CH);
    const int64_t row0 = (brow * a.T + t0) * a.H + h;
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const T* b = static_cast<const T*>(a.b);

    for (int i2 = tid; i2 < CH * DK; i2 += kBwdThreads) {
        const int i = i2 / DK, ch = i2 % DK;
        if (i < L) {
            const int64_t off = (row0 + int64_t(i) * a.H) * DK + ch;
            const float kk = load_as_f32(k, off);
            c.Q[i][ch] = load_as_f32(q, off);
            c.K[i][ch] = kk;
            c.E[i][ch] = load_as_f32(b, off) * kk;
            c.G[i][ch] = log2_decay(a.alpha[off]);
        } else {
            c.Q[i][ch] = c.K[i][ch] = c.E[i][ch] = c.G[i][ch] = 0.f;
        }
    }
    __syncthreads();
    if (tid == 0) split = 1;
    for (int ch = tid; ch < DK; ch += kBwdThreads) {
        float g = 0.f;
        for (int i = 0; i < L; ++i) {
            g += c.G[i][ch];
            c.G[i][ch] = g;
        }
        glv[ch] = g;
    }
    __syncthreads();
    for (int ch = tid; ch < DK; ch += kBwdThreads)
        if (glv[ch] < kSplitMinPrep) split = 0;  // every writer stores the same value
    __syncthreads();
    const int lane = tid & 63, wave = tid >> 6, ln = lane & 15, lk = lane >> 4;
    if (split) {
        // A = strict_lower(Et Kd^T), P = lower(Qt Kd^T) with Et = E 2^G, Qt = Q 2^G
        // (the absorbed factors stored below) and Kd = K 2^-G: the pairwise
        // factor 2^(G_i - G_j) split into two.  Scaling by a power of two is
        // exact, and with every decay above 2^kSplitMinPrep nothing overflows.
        // Kd goes where G was; Kb = Kd 2^G_L below.
        for (int i2 = tid; i2 < CH * DK; i2 += kBwdThreads) {
            const int i = i2 / DK, ch = i2 % DK;
            const float g = c.G[i][ch], up = pow2(g);
            c.E[i][ch] *= up;
            c.Q[i][ch] *= up;
            c.G[i][ch] = c.K[i][ch] * pow2(-g);
        }
        __syncthreads();
        static_assert(kBwdThreads == 256 && CH == 32, "four wavefronts, one 16 x 16 block of A and of P each");
        const int r0 = 16 * (wave >> 1), cn = 16 * (wave & 1);
        f32x4_t aa = {0.f, 0.f, 0.f, 0.f}, pp = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int k0 = 0; k0 < DK; k0 += 4) {
            const float kd = c.G[cn + ln][k0 + lk];
            aa = mfma4(c.E[r0 + ln][k0 + lk], kd, aa);
            pp = mfma4(c.Q[r0 + ln][k0 + lk], kd, pp);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i = r0 + 4 * lk + e, j = cn + ln;
            c.A[i][j] = j < i ? aa[e] : 0.f;
            c.P[i][j] = j <= i ? pp[e] : 0.f;
        }
    } else {
        // A and P with every pairwise decay factor formed exactly (exponent <= 0):
        // zeros above the diagonal, then the CH (CH + 1) / 2 pairs j <= i spread
        // evenly over the threads (pair p: row i with i (i + 1) / 2 <= p, column
        // p - i (i + 1) / 2)
        for (int i2 = tid; i2 < CH * CH; i2 += kBwdThreads) {
            const int i = i2 / CH, j = i2 % CH;
            if (j > i) c.A[i][j] = c.P[i][j] = 0.f;
        }
        constexpr int kPairs = CH * (CH + 1) / 2;
        for (int p = tid; p < kPairs; p += kBwdThreads) {
            int i = int((sqrtf(8.f * float(p) + 1.f) - 1.f) * 0.5f);
            while ((i + 1) * (i + 2) / 2 <= p) ++i;
            while (i * (i + 1) / 2 > p) --i;
            const int j = p - i * (i + 1) / 2;
            float acc_a = 0.f, acc_p = 0.f;
            if (i < L) {
                for (int ch = 0; ch < DK; ++ch) {
                    const float kf = c.K[j][ch] * pow2(c.G[i][ch] - c.G[j][ch]);
                    acc_a += c.E[i][ch] * kf;
                    acc_p += c.Q[i][ch] * kf;
                }
            }
            c.A[i][j] = j < i ? acc_a : 0.f;
            c.P[i][j] = acc_p;
        }
    }
    __syncthreads();
    // Tm = (I + A)^-1 by columns: lane j keeps column j in registers
    // (substitution row by row, the same operations in the same order as a
    // column in memory)
    if (tid < CH) {
        const int j = tid;
        float t[CH];
#pragma unroll
        for (int i = 0; i < CH; ++i) t[i] = i == j ? 1.f : 0.f;
#pragma unroll
        for (int i = 1; i < CH; ++i) {
            if (i < L) {
                float acc = 0.f;
#pragma unroll
                for (int mm = 0; mm < i; ++mm) acc += c.A[i][mm] * t[mm];
                if (j < i) t[i] = -acc;
            }
        }
#pragma unroll
        for (int i = 0; i < CH; ++i) Tm[i][j] = t[i];
    }
    // absorb the decay into the row and column factors (already done for Et, Qt
    // on the split path)
    for (int i2 = tid; i2 < L * DK; i2 += kBwdThreads) {
        const int i = i2 / DK, ch = i2 % DK;
        if (split) {
            c.K[i][ch] = c.G[i][ch] * pow2(glv[ch]);
        } else {
            const float g = c.G[i][ch], up = pow2(g);
            c.E[i][ch] *= up;
            c.Q[i][ch] *= up;
            c.K[i][ch] *= pow2(glv[ch] - g);
        }
    }
    __syncthreads();
    float* dst = a.ws_prep + prep_base(a, row, slot, h);
    for (int i2 = tid; i2 < CH * CH; i2 += kBwdThreads) {
        const int i = i2 / CH, j = i2 % CH;
        dst[kPrepT + i2] = Tm[i][j];
        dst[kPrepP + i2] = c.P[i][j];
    }
    for (int i2 = tid; i2 < CH * DK; i2 += kBwdThreads) {
        const int i = i2 / DK, ch = i2 % DK;
        dst[kPrepE + i2] = c.E[i][ch];
        dst[kPrepE + CH * DK + i2] = c.Q[i][ch];
        dst[kPrepE + 2 * CH * DK + i2] = c.K[i][ch];
    }
    for (int ch = tid; ch < DK; ch += kBwdThreads) dst[kPrepE + 3 * CH * DK + ch] = pow2(glv[ch]);
}

// Thread layout of the sequential kernels: lane column jj = tid % 32 of the
// tile; chunk rows i0 + NG r (r < RR) and state rows c0 + NG r (r < DK / NG),
// with i0 = c0 = tid / 32.  The rows a wavefront reads at one time are two,
// so the row operand is a broadcast and the column operand is contiguous.

// A chunk's prepared rows (rows past the chunk are zero in the block), loaded
// with sixteen-byte loads into registers by issue() and written to LDS by
// store(): the sequential kernels issue the next chunk's loads while they
// compute the current one.
template <int DK, bool kQ, int NT>
struct PrepRegs {
    static constexpr int QR = CH * DK / 4;           // quads per row array
    static constexpr int NQ = (QR + NT - 1) / NT;    // quads per thread and array
    static constexpr int QT = CH * CH / 4;           // quads of Tm (and Pm)
    static_assert(QT <= NT && DK / 4 <= NT, "one quad of Tm, Pm and gamma per thread at most");
    float4 ve[NQ], vq[NQ], vk[NQ], vt, vp, vg;

    __device__ void issue(const float* src, int tid)
    {
        const float4* s4 = reinterpret_cast<const float4*>(src);
        const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int qd = 0; qd < NQ; ++qd) {
            const int i4 = tid + NT * qd;
            const bool in = i4 < QR;
            ve[qd] = in ? s4[kPrepE / 4 + i4] : z4;
            vq[qd] = in && kQ ? s4[kPrepE / 4 + QR + i4] : z4;
            vk[qd] = in ? s4[kPrepE / 4 + 2 * QR + i4] : z4;
        }
        vt = tid < QT ? s4[kPrepT / 4 + tid] : z4;
        vp = tid < QT && kQ ? s4[kPrepP / 4 + tid] : z4;
        vg = tid < DK / 4 ? s4[kPrepE / 4 + 3 * QR + tid] : z4;
    }
    template <int RSD, int RST>  // row strides of the [CH][DK] and [CH][CH] arrays
    __device__ void store(float (*Et)[RSD], float (*Qt)[RSD], float (*Kb)[RSD], float (*Tm)[RST],
                          float (*Pm)[RST], float* gam, int tid) const
    {
#pragma unroll
        for (int qd = 0; qd < NQ; ++qd) {
            const int i4 = tid + NT * qd;
            if (i4 >= QR) continue;
            const int i = i4 / (DK / 4), c = (i4 % (DK / 4)) * 4;
            st4(Et[i], c, ve[qd]);
            if (kQ) st4(Qt[i], c, vq[qd]);
            st4(Kb[i], c, vk[qd]);
        }
        if (tid < QT) {
            const int i = tid / (CH / 4), c = (tid % (CH / 4)) * 4;
            st4(Tm[i], c, vt);
            if (kQ) st4(Pm[i], c, vp);
        }
        if (tid < DK / 4) st4(gam, 4 * tid, vg);
    }
};

// ---------------------------------------------------------------------------
// bwd_states: the forward again, storing the state at every chunk start.
// Wavefront w owns the state blocks w, w + 8, ... (block t: rows 16 (t / 2),
// columns 16 (t % 2) of the 32-column tile) in accumulator registers;
// wavefronts 0..3 form the four blocks of X and U.
template <typename T, int DK>
__global__ __launch_bounds__(kSeqThreads) void bwd_states_kernel(BwdArgs a)
{
    if (a.gate && *a.gate == 0) return;  // the matrix-core path covers this call
    constexpr int NTS = (DK / 16) * (kTile / 16);  // 16 x 16 blocks of the state tile
    constexpr int TPW = (NTS + 7) / 8;             // per wavefront
    __shared__ float Et[CH][DK + kPad], Kb[CH][DK + kPad];
    __shared__ float Tm[CH][CH + kPad];
    __shared__ float gam[DK];
    __shared__ float Ss[DK][kTile];  // chunk-start state
    __shared__ float Zs[CH][kTile], Xs[CH][kTile], Us[CH][kTile];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 15, lk = lane >> 4;
    const int jj = tid % kTile, i0 = tid / kTile;
    const int ntiles = a.dv_ / kTile;
    int64_t chain64;
    int tile;
    xcd_group(blockIdx.x, ntiles, chain64, tile);
    if (chain64 >= int64_t(a.N) * a.H) return;
    const int chain = int(chain64);
    const int n = chain / a.H, h = chain % a.H;
    const int j0 = tile * kTile;
    const int64_t dv = a.dv_;
    int64_t bos, eos, brow;
    sequence_bounds(a.cu_seqlens, n, a.T, bos, eos, brow);
    const T* v = static_cast<const T*>(a.v);
    const T* w = static_cast<const T*>(a.w);

    f32x4_t st[TPW];
    const int64_t s_off = (int64_t(n) * a.H + h) * DK * dv + j0;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int t = wave + 8 * u;
        if (t >= NTS) continue;
        const int r0 = 16 * (t >> 1) + 4 * lk, c = 16 * (t & 1) + ln;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            st[u][i] = a.initial_state ? a.initial_state[s_off + int64_t(r0 + i) * dv + c] : 0.f;
            Ss[r0 + i][c] = st[u][i];
        }
    }

    // chunk m's prepared rows and v, w rows, loaded one chunk ahead
    const int M = int((eos - bos + CH - 1) / CH);
    PrepRegs<DK, false, kSeqThreads> pf;
    float pv[RR], pw[RR];
    auto issue = [&](int m) {
        const int64_t t0 = bos + int64_t(m) * CH;
        const int L = int(eos - t0 < CH ? eos - t0 : CH);
        const int64_t row0 = (brow * a.T + t0) * a.H + h;
        pf.issue(a.ws_prep + prep_base(a, brow, slot_of(a, n, bos, m), h), tid);
#pragma unroll
        for (int r = 0; r < RR; ++r) {
            const int i = i0 + NG * r;
            const int64_t off = (row0 + int64_t(i) * a.H) * dv + j0 + jj;
            pv[r] = i < L ? load_as_f32(v, off) : 0.f;
            pw[r] = i < L ? load_as_f32(w, off) : 0.f;
        }
    };
    if (M > 0) issue(0);
    for (int m = 0; m < M; ++m) {
        const int64_t t0 = bos + int64_t(m) * CH;
        const int L = int(eos - t0 < CH ? eos - t0 : CH);
        const int64_t row0 = (brow * a.T + t0) * a.H + h;
        const int64_t slot = slot_of(a, n, bos, m);
        float* dst = a.ws_states + slot_base(a, brow, slot, h) + j0;
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int t = wave + 8 * u;
            if (t >= NTS) continue;
            const int r0 = 16 * (t >> 1) + 4 * lk, c = 16 * (t & 1) + ln;
#pragma unroll
            for (int i = 0; i < 4; ++i) dst[int64_t(r0 + i) * dv + c] = st[u][i];
        }
        lds_sync();  // the previous chunk is done with Et, Kb, Tm, Zs, Xs and Us
        pf.template store<DK + kPad, CH + kPad>(Et, nullptr, Kb, Tm, nullptr, gam, tid);
#pragma unroll
        for (int r = 0; r < RR; ++r) Zs[i0 + NG * r][jj] = pw[r] * pv[r];
        if (m + 1 < M) issue(m + 1);  // in flight while this chunk is computed
        lds_sync();
        // X = Z - Et S  (rows past the chunk: zero rows of Et and Z give zero)
        if (wave < 4) {
            const int r0 = 16 * (wave >> 1), c = 16 * (wave & 1) + ln;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
            for (int k0 = 0; k0 < DK; k0 += 4) acc = mfma4(Et[r0 + ln][k0 + lk], Ss[k0 + lk][c], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) Xs[r0 + 4 * lk + i][c] = Zs[r0 + 4 * lk + i][c] - acc[i];
        }
        lds_sync();
        // U = Tm X (also to the workspace, for the key kernel)
        if (wave < 4) {
            const int r0 = 16 * (wave >> 1), c = 16 * (wave & 1) + ln;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < CH; k0 += 4) acc = mfma4(Tm[r0 + ln][k0 + lk], Xs[k0 + lk][c], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = r0 + 4 * lk + i;
                Us[r][c] = acc[i];
                if (r < L) a.ws_u[(row0 + int64_t(r) * a.H) * dv + j0 + c] = acc[i];
            }
        }
        lds_sync();
        // S <- 2^G_L S + Kb^T U  (Kb and U are zero past the chunk)
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int t = wave + 8 * u;
            if (t >= NTS) continue;
            const int r0 = 16 * (t >> 1), c = 16 * (t & 1) + ln;
            f32x4_t acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = gam[r0 + 4 * lk + i] * st[u][i];
#pragma unroll
            for (int k0 = 0; k0 < CH; k0 += 4) acc = mfma4(Kb[k0 + lk][r0 + ln], Us[k0 + lk][c], acc);
            st[u] = acc;
#pragma unroll
            for (int i = 0; i < 4; ++i) Ss[r0 + 4 * lk + i][c] = acc[i];
        }
    }
}

// ---------------------------------------------------------------------------
// bwd_dstate: chunks in reverse, carrying the state gradient (U comes from
// bwd_states through the workspace).  Wavefront w owns the gradient blocks
// w, w + 8, ... in accumulator registers; wavefronts 0..3 form the blocks of
// dU and dX.
template <typename T, int DK>
__global__ __launch_bounds__(kSeqThreads, 4) void bwd_dstate_kernel(BwdArgs a)
{
    if (a.gate && *a.gate == 0) return;  // the matrix-core path covers this call
    constexpr int NTS = (DK / 16) * (kTile / 16);
    constexpr int TPW = (NTS + 7) / 8;
    __shared__ float Et[CH][DK + kPad], Qt[CH][DK + kPad], Kb[CH][DK + kPad];
    __shared__ float Tm[CH][CH + 1], Pm[CH][CH + 1];  // read transposed: stride 33 keeps them conflict-free
    __shared__ float gam[DK];
    __shared__ float dSs[DK][kTile];  // gradient of the chunk-end state
    __shared__ float dOs[CH][kTile];
    // dU and dX live in Kb's space, which is free once dU is formed (about 80 KB
    // of LDS in all at dk = 128, so that two workgroups share a CU); with the
    // smallest heads Kb is too small and they get their own
    constexpr bool kInKb = 2 * CH * kTile <= CH * (DK + kPad);
    __shared__ float ux_own[kInKb ? 1 : 2 * CH * kTile];
    float* ux = kInKb ? &Kb[0][0] : ux_own;
    float (*dUs)[kTile] = reinterpret_cast<float (*)[kTile]>(ux);
    float (*dXs)[kTile] = reinterpret_cast<float (*)[kTile]>(ux + CH * kTile);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 15, lk = lane >> 4;
    const int jj = tid % kTile, i0 = tid / kTile;
    const int ntiles = a.dv_ / kTile;
    int64_t chain64;
    int tile;
    xcd_group(blockIdx.x, ntiles, chain64, tile);
    if (chain64 >= int64_t(a.N) * a.H) return;
    const int chain = int(chain64);
    const int n = chain / a.H, h = chain % a.H;
    const int j0 = tile * kTile;
    const int64_t dv = a.dv_;
    int64_t bos, eos, brow;
    sequence_bounds(a.cu_seqlens, n, a.T, bos, eos, brow);
    const T* dO = static_cast<const T*>(a.d_o);
    const T* v = static_cast<const T*>(a.v);
    const T* w = static_cast<const T*>(a.w);
    T* dv_out = static_cast<T*>(a.dv);
    T* dw_out = static_cast<T*>(a.dw);

    f32x4_t ds[TPW];
    const int64_t s_off = (int64_t(n) * a.H + h) * DK * dv + j0;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int t = wave + 8 * u;
        if (t >= NTS) continue;
        const int r0 = 16 * (t >> 1) + 4 * lk, c = 16 * (t & 1) + ln;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ds[u][i] = a.d_final_state ? a.d_final_state[s_off + int64_t(r0 + i) * dv + c] : 0.f;
            dSs[r0 + i][c] = ds[u][i];
        }
    }

    // chunk m's prepared rows, dO rows, and (wavefronts 0..3, in the layout of
    // their dX block) v and w; loaded at the chunk's start (the other
    // workgroup on the CU covers their latency)
    const int M = int((eos - bos + CH - 1) / CH);
    PrepRegs<DK, true, kSeqThreads> pf;
    float po[RR], pv[4], pw[4];
    auto issue = [&](int m) {
        const int64_t t0 = bos + int64_t(m) * CH;
        const int L = int(eos - t0 < CH ? eos - t0 : CH);
        const int64_t row0 = (brow * a.T + t0) * a.H + h;
        const int64_t slot = slot_of(a, n, bos, m);
        pf.issue(a.ws_prep + prep_base(a, brow, slot, h), tid);
#pragma unroll
        for (int r = 0; r < RR; ++r) {
            const int i = i0 + NG * r;
            const int64_t off = (row0 + int64_t(i) * a.H) * dv + j0 + jj;
            po[r] = i < L ? load_as_f32(dO, off) : 0.f;
        }
        if (wave < 4) {
            const int r0 = 16 * (wave >> 1) + 4 * lk, c = 16 * (wave & 1) + ln;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int i = r0 + e;
                const int64_t off = (row0 + int64_t(i) * a.H) * dv + j0 + c;
                pv[e] = i < L ? load_as_f32(v, off) : 0.f;
                pw[e] = i < L ? load_as_f32(w, off) : 0.f;
            }
        }
    };
    for (int m = M - 1; m >= 0; --m) {
        const int64_t t0 = bos + int64_t(m) * CH;
        const int L = int(eos - t0 < CH ? eos - t0 : CH);
        const int64_t row0 = (brow * a.T + t0) * a.H + h;
        const int64_t slot = slot_of(a, n, bos, m);
        float* dsd = a.ws_dstates + slot_base(a, brow, slot, h) + j0;
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int t = wave + 8 * u;
            if (t >= NTS) continue;
            const int r0 = 16 * (t >> 1) + 4 * lk, c = 16 * (t & 1) + ln;
#pragma unroll
            for (int i = 0; i < 4; ++i) dsd[int64_t(r0 + i) * dv + c] = ds[u][i];
        }
        issue(m);
        lds_sync();  // the previous chunk is done with the prepared rows and the row buffers
        pf.template store<DK + kPad, CH + 1>(Et, Qt, Kb, Tm, Pm, gam, tid);
#pragma unroll
        for (int r = 0; r < RR; ++r) dOs[i0 + NG * r][jj] = po[r];
        float vv[4], ww[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            vv[e] = pv[e];
            ww[e] = pw[e];
        }
        lds_sync();
        f32x4_t du = {0.f, 0.f, 0.f, 0.f};
        if (wave < 4) {  // dU = Kb dS' + Pm^T dO
            const int r0 = 16 * (wave >> 1), c = 16 * (wave & 1) + ln;
#pragma unroll 8
            for (int k0 = 0; k0 < DK; k0 += 4) du = mfma4(Kb[r0 + ln][k0 + lk], dSs[k0 + lk][c], du);
#pragma unroll
            for (int k0 = 0; k0 < CH; k0 += 4) du = mfma4(Pm[k0 + lk][r0 + ln], dOs[k0 + lk][c], du);
        }
        lds_sync();  // Kb is read: its space takes dU and dX
        if (wave < 4) {
            const int r0 = 16 * (wave >> 1), c = 16 * (wave & 1) + ln;
#pragma unroll
            for (int i = 0; i < 4; ++i) dUs[r0 + 4 * lk + i][c] = du[i];
        }
        lds_sync();
        if (wave < 4) {  // dX = Tm^T dU (zero past the chunk), dw = dX v, dv = dX w
            const int r0 = 16 * (wave >> 1), c = 16 * (wave & 1) + ln;
            f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int k0 = 0; k0 < CH; k0 += 4) acc = mfma4(Tm[k0 + lk][r0 + ln], dUs[k0 + lk][c], acc);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = r0 + 4 * lk + i;
                const float dx = row < L ? acc[i] : 0.f;
                dXs[row][c] = dx;
                if (row < L) {
                    const int64_t off = (row0 + int64_t(row) * a.H) * dv + j0 + c;
                    a.ws_dx[off] = dx;
                    store_from_f32(dw_out, off, dx * vv[i]);
                    store_from_f32(dv_out, off, dx * ww[i]);
                }
            }
        }
        lds_sync();
        // dS = 2^G_L dS' + Qt^T dO - Et^T dX  (the gradient of the chunk-start state)
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int t = wave + 8 * u;
            if (t >= NTS) continue;
            const int r0 = 16 * (t >> 1), c = 16 * (t & 1) + ln;
            f32x4_t acc, sub = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = gam[r0 + 4 * lk + i] * ds[u][i];
#pragma unroll
            for (int k0 = 0; k0 < CH; k0 += 4) {
                acc = mfma4(Qt[k0 + lk][r0 + ln], dOs[k0 + lk][c], acc);
                sub = mfma4(Et[k0 + lk][r0 + ln], dXs[k0 + lk][c], sub);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ds[u][i] = acc[i] - sub[i];
                dSs[r0 + 4 * lk + i][c] = ds[u][i];
            }
        }
    }
    if (a.d_initial_state) {
#pragma unroll
        for (int u = 0; u < TPW; ++u) {
            const int t = wave + 8 * u;
            if (t >= NTS) continue;
            const int r0 = 16 * (t >> 1) + 4 * lk, c = 16 * (t & 1) + ln;
#pragma unroll
            for (int i = 0; i < 4; ++i) a.d_initial_state[s_off + int64_t(r0 + i) * dv + c] = ds[u][i];
        }
    }
}

// ---------------------------------------------------------------------------
// bwd_keys: one chunk of one head, channels c0 .. c0 + CB - 1 (CB = 64 when
// both head sizes are at least 64, else 32), 8 CB threads.  Thread layout of the
// loads and elementwise steps: column (token j or channel cc) = tid % CB, rows
// i0 + 8 r with i0 = tid / CB.
template <int DK, int DV>
constexpr int keys_cb() { return DK >= 64 && DV >= 64 ? 64 : 32; }

template <typename T, int DK, int DV>
__global__ __launch_bounds__((8 * keys_cb<DK, DV>())) void bwd_keys_kernel(BwdArgs a)
{
    if (a.gate && *a.gate == 0) return;  // the matrix-core path covers this call
    constexpr int CB = keys_cb<DK, DV>(); // channels per block
    constexpr int NT = 8 * CB;            // threads: CB / 8 wavefronts
    constexpr int DH = 32;                // value columns per pass
    static_assert(DK % CB == 0 && DV % DH == 0 && CH == 32, "block shapes");
    // One region, used in turn for: each pass's U, dX, dO rows and the block's
    // S, dS' rows; the split factors K2, E2, Q2; dg and Kb dKb.  With alpha and
    // b read again where they are used, the kernel fits in about 74 KB of LDS
    // at CB = 64, so that two workgroups share a CU.
    constexpr int RP = DH + kPad, RC = CB + kPad;  // row strides: pass rows, channel-wide rows
    constexpr int kPassF = 3 * CH * RP + 2 * CB * RP, kSplitF = 3 * CH * RC, kGradF = 2 * CH * RC;
    constexpr int kFlat = kPassF > kSplitF ? (kPassF > kGradF ? kPassF : kGradF) : (kSplitF > kGradF ? kSplitF : kGradF);
    __shared__ __align__(16) float flat[kFlat];
    __shared__ float dA[CH][CH + 1], dP[CH][CH + 1];
    __shared__ float qb[CH][CB + 1], kb[CH][CB + 1], eb[CH][CB + 1], Gb[CH][CB + 1];
    __shared__ float rs[CB];
    float (*Us)[RP] = reinterpret_cast<float (*)[RP]>(flat);
    float (*dXs)[RP] = reinterpret_cast<float (*)[RP]>(flat + CH * RP);
    float (*dOs)[RP] = reinterpret_cast<float (*)[RP]>(flat + 2 * CH * RP);
    float (*Sb)[RP] = reinterpret_cast<float (*)[RP]>(flat + 3 * CH * RP);
    float (*dSb)[RP] = reinterpret_cast<float (*)[RP]>(flat + 3 * CH * RP + CB * RP);

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 15, lk = lane >> 4;
    const int col = tid % CB, i0 = tid / CB;
    constexpr int nblk = DK / CB;
    int64_t idx;
    int cblk;
    xcd_group(blockIdx.x, nblk, idx, cblk);
    if (idx >= int64_t(a.B) * a.slots * a.H) return;
    const int h = int(idx % a.H);
    idx /= a.H;
    const int64_t slot = idx % a.slots, row = idx / a.slots;
    int n, m;
    int64_t bos, eos, brow;
    if (!chunk_of_slot(a, row, slot, n, m, bos, eos, brow)) return;
    const int64_t t0 = bos + int64_t(m) * CH;
    const int L = int(eos - t0 < CH ? eos - t0 : CH);
    const int64_t row0 = (brow * a.T + t0) * a.H + h;
    const int c0 = cblk * CB;
    const int64_t sbase = slot_base(a, brow, slot, h);
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const T* b = static_cast<const T*>(a.b);
    const T* dO = static_cast<const T*>(a.d_o);

    // the passes' rows: four consecutive columns per thread, the next pass's
    // loads issued before this pass's products (the barriers wait on LDS only)
    constexpr int QR = CH * DH / 4, QS = CB * DH / 4;      // quads of the token rows and channel rows
    constexpr int NQR = (QR + NT - 1) / NT, NQS = (QS + NT - 1) / NT;  // per thread (the last partly idle)
    float4 vu[NQR], vx[NQR], vo[NQR], vs[NQS], vd[NQS];
    auto issue = [&](int jh) {
        const float4 z4 = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int qd = 0; qd < NQR; ++qd) {
            const int i4 = tid + NT * qd;
            const int i = i4 / (DH / 4), j = (i4 % (DH / 4)) * 4;
            const bool live = i4 < QR && i < L;
            const int64_t off = (row0 + int64_t(i) * a.H) * DV + jh + j;
            vu[qd] = live ? load4(a.ws_u, off) : z4;
            vx[qd] = live ? load4(a.ws_dx, off) : z4;
            vo[qd] = live ? load4(dO, off) : z4;
        }
#pragma unroll
        for (int qd = 0; qd < NQS; ++qd) {
            const int i4 = tid + NT * qd;
            const int c = i4 / (DH / 4), j = (i4 % (DH / 4)) * 4;
            const int64_t soff = sbase + int64_t(c0 + c) * DV + jh + j;
            vs[qd] = i4 < QS ? load4(a.ws_states, soff) : z4;
            vd[qd] = i4 < QS ? load4(a.ws_dstates, soff) : z4;
        }
    };
    issue(0);  // in flight with the token inputs below

#pragma unroll
    for (int r = 0; r < 4; ++r) {  // the block's token inputs, thread (i0 + 8 r, col)
        const int i = i0 + 8 * r;
        if (i < L) {
            const int64_t off = (row0 + int64_t(i) * a.H) * DK + c0 + col;
            const float kk = load_as_f32(k, off), bv = load_as_f32(b, off);
            qb[i][col] = load_as_f32(q, off);
            kb[i][col] = kk;
            eb[i][col] = bv * kk;
            Gb[i][col] = log2_decay(a.alpha[off]);
        } else {
            qb[i][col] = kb[i][col] = eb[i][col] = Gb[i][col] = 0.f;
        }
    }

    // Over all value columns, on the matrix cores: dX U^T, dO U^T (-> dA, dP),
    // dX S^T, dO S^T, U dS'^T (-> dEt, dQt, dKb).  Wavefront w forms the 16 x 16
    // blocks (tokens 16 tb, channels 16 cb) of the last three, and of dA, dP
    // (tokens 16 tb, tokens 16 jb) the ones given by:
    //   CB = 32 (4 wavefronts): tb = w / 2, cb = jb = w % 2, both dA and dP;
    //   CB = 64 (8 wavefronts): tb = w % 2, cb = w / 2, jb = (w / 2) % 2, dA for
    //   w < 4 and dP for w >= 4.
    // The row sums of dS' . S go with the first CB threads.
    const int tb = CB == 32 ? wave >> 1 : wave & 1;
    const int cb = CB == 32 ? wave & 1 : wave >> 1;
    const int jb = CB == 32 ? wave & 1 : (wave >> 1) & 1;
    const bool do_a = CB == 32 || wave < 4, do_p = CB == 32 || wave >= 4;
    const f32x4_t zero4 = {0.f, 0.f, 0.f, 0.f};
    f32x4_t ma = zero4, mp = zero4, me = zero4, mq = zero4, mk = zero4;
    float xr = 0.f;
    for (int jh = 0; jh < DV; jh += DH) {
#pragma unroll
        for (int qd = 0; qd < NQR; ++qd) {
            const int i4 = tid + NT * qd;
            const int i = i4 / (DH / 4), j = (i4 % (DH / 4)) * 4;
            if (i4 < QR) {
                st4(Us[i], j, vu[qd]);
                st4(dXs[i], j, vx[qd]);
                st4(dOs[i], j, vo[qd]);
            }
        }
#pragma unroll
        for (int qd = 0; qd < NQS; ++qd) {
            const int i4 = tid + NT * qd;
            const int c = i4 / (DH / 4), j = (i4 % (DH / 4)) * 4;
            if (i4 < QS) {
                st4(Sb[c], j, vs[qd]);
                st4(dSb[c], j, vd[qd]);
            }
        }
        if (jh + DH < DV) issue(jh + DH);
        lds_sync();
        {
            const int ra = 16 * tb + ln, rc = 16 * cb + ln, rj = 16 * jb + ln;
#pragma unroll 4
            for (int k0 = 0; k0 < DH; k0 += 4) {
                const int kk = k0 + lk;
                const float ax = dXs[ra][kk], ao = dOs[ra][kk], au = Us[ra][kk];
                const float bs = Sb[rc][kk], bd = dSb[rc][kk], bu = Us[rj][kk];
                if (do_a) ma = mfma4(ax, bu, ma);
                if (do_p) mp = mfma4(ao, bu, mp);
                me = mfma4(ax, bs, me);
                mq = mfma4(ao, bs, mq);
                mk = mfma4(au, bd, mk);
            }
            if (tid < CB)
                for (int j = 0; j < DH; ++j) xr += dSb[tid][j] * Sb[tid][j];
        }
        lds_sync();
    }
    // dA, dP blocks: token 16 tb + 4 lk + e, token 16 jb + ln
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = 16 * tb + 4 * lk + e, j = 16 * jb + ln;
        if (do_a) dA[i][j] = j < i ? -ma[e] : 0.f;
        if (do_p) dP[i][j] = j <= i ? mp[e] : 0.f;
    }
    if (tid < CB) rs[tid] = xr;
    for (int cc = tid; cc < CB; cc += NT) {  // running sums of the block's decay
        float g = 0.f;
        for (int i = 0; i < L; ++i) {
            g += Gb[i][cc];
            Gb[i][cc] = g;
        }
    }
    __syncthreads();

    // The pairwise sums as products.  With the decay split as
    // 2^(G_i - G_j) = 2^G_i 2^-G_j:
    //   de_a  = 2^G (.) (dA (K (.) 2^-G)),   dq_p = 2^G (.) (dP (K (.) 2^-G)),
    //   dk_ap = 2^-G (.) (dA^T (E (.) 2^G) + dP^T (Q (.) 2^G)).
    // Scaling by a power of two is exact, so this equals the pairwise form
    // wherever nothing overflows: for channels whose decay over the chunk stays
    // above 2^kSplitMin (then 2^-G <= 2^-kSplitMin).  Other channels take the
    // pairwise loops below.  Rows past the chunk are zero in every factor.
    constexpr float kSplitMin = -64.f;
    float (*K2)[RC] = reinterpret_cast<float (*)[RC]>(flat);
    float (*E2)[RC] = reinterpret_cast<float (*)[RC]>(flat + CH * RC);
    float (*Q2)[RC] = reinterpret_cast<float (*)[RC]>(flat + 2 * CH * RC);
#pragma unroll
    for (int r = 0; r < 4; ++r) {  // thread (i0 + 8 r, col)
        const int i = i0 + 8 * r;
        const float g = Gb[i][col], up = pow2(g);
        K2[i][col] = Gb[L - 1][col] >= kSplitMin ? kb[i][col] * pow2(-g) : 0.f;
        E2[i][col] = eb[i][col] * up;
        Q2[i][col] = qb[i][col] * up;
    }
    __syncthreads();
    f32x4_t y1 = zero4, y2 = zero4, y3 = zero4;
    {
        const int ra = 16 * tb + ln, cn = 16 * cb + ln;
#pragma unroll
        for (int k0 = 0; k0 < CH; k0 += 4) {
            const int kk = k0 + lk;
            const float bk = K2[kk][cn];
            y1 = mfma4(dA[ra][kk], bk, y1);
            y2 = mfma4(dP[ra][kk], bk, y2);
            y3 = mfma4(dA[kk][ra], E2[kk][cn], y3);
            y3 = mfma4(dP[kk][ra], Q2[kk][cn], y3);
        }
    }

    lds_sync();  // the split factors are read: their space takes dg and Kb dKb
    // pairwise and absorbed-factor gradients, in the block layout: token
    // 16 tb + 4 lk + e, channel cw
    float (*dg)[RC] = reinterpret_cast<float (*)[RC]>(flat);
    float (*kbd)[RC] = reinterpret_cast<float (*)[RC]>(flat + CH * RC);
    T* dq_out = static_cast<T*>(a.dq);
    T* dk_out = static_cast<T*>(a.dk);
    T* db_out = static_cast<T*>(a.db);
    const int cw = 16 * cb + ln;
    const float glw = Gb[L - 1][cw];
    const bool split = glw >= kSplitMin;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int i = 16 * tb + 4 * lk + e;
        if (i >= L) continue;
        const float gi = Gb[i][cw];
        const float up = pow2(gi), down = pow2(glw - gi);
        float de_a, dq_p, dk_ap;
        if (split) {
            de_a = up * y1[e];
            dq_p = up * y2[e];
            dk_ap = pow2(-gi) * y3[e];
        } else {
            de_a = dq_p = dk_ap = 0.f;
            for (int j = 0; j <= i; ++j) {
                const float kf = kb[j][cw] * pow2(gi - Gb[j][cw]);
                de_a += dA[i][j] * kf;  // dA is zero on the diagonal
                dq_p += dP[i][j] * kf;
            }
            for (int rr = i; rr < L; ++rr) {
                const float f = pow2(Gb[rr][cw] - gi);
                dk_ap += (dA[rr][i] * eb[rr][cw] + dP[rr][i] * qb[rr][cw]) * f;
            }
        }
        const float dEt = -me[e], dQt = mq[e], dKb = mk[e];
        const float de = de_a + dEt * up;
        const float dq = dq_p + dQt * up;
        const float dkk = dk_ap + dKb * down;
        dg[i][cw] = eb[i][cw] * de_a + qb[i][cw] * dq_p - kb[i][cw] * dk_ap + eb[i][cw] * up * dEt
                    + qb[i][cw] * up * dQt - kb[i][cw] * down * dKb;
        kbd[i][cw] = kb[i][cw] * down * dKb;
        const int64_t off = (row0 + int64_t(i) * a.H) * DK + c0 + cw;
        store_from_f32(dq_out, off, dq);
        store_from_f32(db_out, off, de * kb[i][cw]);
        store_from_f32(dk_out, off, dkk + de * load_as_f32(b, off));
    }
    __syncthreads();
    // the chunk-end terms, then the reverse running sum over the chunk's tokens
    if (tid < CB) {
        const int cc = tid;
        const float gl = Gb[L - 1][cc];
        float acc = pow2(gl) * rs[cc];
        for (int j = 0; j < L; ++j) acc += kbd[j][cc];
        for (int i = L - 1; i >= 0; --i) {
            acc += dg[i][cc];
            const float al = a.alpha[(row0 + int64_t(i) * a.H) * DK + c0 + cc];
            const float lg = __log2f(al);
            const bool clamped = !(lg >= kLog2AlphaFloor && lg <= 0.f);
            const int64_t off = (row0 + int64_t(i) * a.H) * DK + c0 + cc;
            a.dalpha[off] = clamped ? 0.f : acc / al;
        }
    }
}

template <typename T, int DK>
hipError_t launch_chain(const BwdArgs& a, hipStream_t stream)
{
    const int64_t chains = xcd_grid(int64_t(a.N) * a.H, a.dv_ / kTile);
    const int64_t chunks = int64_t(a.B) * a.slots * a.H;
    if (chains > 0x7fffffff || xcd_grid(chunks, DK / 32) > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (chunks > 0) {
        hipLaunchKernelGGL((bwd_prep_kernel<T, DK>), dim3(unsigned(chunks)), dim3(kBwdThreads), 0, stream, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        hipLaunchKernelGGL((bwd_states_kernel<T, DK>), dim3(unsigned(chains)), dim3(kSeqThreads), 0, stream, a);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    // runs for T = 0 as well: it passes the final-state gradient through
    hipLaunchKernelGGL((bwd_dstate_kernel<T, DK>), dim3(unsigned(chains)), dim3(kSeqThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int DK, int DV>
hipError_t launch_keys(const BwdArgs& a, hipStream_t stream)
{
    const int64_t groups = int64_t(a.B) * a.slots * a.H;
    if (groups == 0) return hipSuccess;
    constexpr int CB = keys_cb<DK, DV>();
    const int64_t blocks = xcd_grid(groups, DK / CB);
    hipLaunchKernelGGL((bwd_keys_kernel<T, DK, DV>), dim3(unsigned(blocks)), dim3(8 * CB), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int DK>
hipError_t launch_dk(const BwdArgs& a, hipStream_t stream)
{
    if (a.dv_ % kTile != 0) return hipErrorInvalidValue;
    hipError_t e = launch_chain<T, DK>(a, stream);
    if (e != hipSuccess) return e;
    switch (a.dv_) {
        case 32: return launch_keys<T, DK, 32>(a, stream);
        case 64: return launch_keys<T, DK, 64>(a, stream);
        case 128: return launch_keys<T, DK, 128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t launch_typed(const BwdArgs& a, hipStream_t stream)
{
    switch (a.dk_) {
        case 32: return launch_dk<T, 32>(a, stream);
        case 64: return launch_dk<T, 64>(a, stream);
        case 128: return launch_dk<T, 128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int64_t chunk_bwd_prep_floats(int dk) { return prep_floats(dk); }

hipError_t launch_chunk_bwd(const BwdArgs& a, bool bf16, hipStream_t stream)
{
    return bf16 ? launch_typed<bf16raw>(a, stream) : launch_typed<float>(a, stream);
}

}  // namespace gdn2
