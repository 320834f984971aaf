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
// nothing overflows.  alpha is clamped to [2^-15, 1] as in the forward
// kernels; the gradient is zero where the clamp is active.
//
// Three kernels, 32-token chunks (the same mathematics as any chunk size):
//   bwd_states  (chain x value tile, chunks in order)   recompute the forward,
//               store every chunk-start state;
//   bwd_dstate  (chain x value tile, chunks in reverse) U, dX and the state
//               gradient recurrence; dv, dw and dS0; store U and dX rows and
//               each chunk-end state gradient;
//   bwd_keys    (chunk x head x channel block)          dA, dP, dEt, dQt, dKb
//               over all value columns, then dq, dk, db and dalpha.
#include "gdn2_device.hpp"
#include "launch.hpp"

namespace gdn2 {
namespace {

constexpr int kBwdThreads = 256;
constexpr int CH = kBwdChunk;

__device__ __forceinline__ int64_t slot_of(const BwdArgs& a, int n, int64_t bos, int m)
{
    return a.cu_seqlens ? (bos + int64_t(m) * CH) / CH + n : int64_t(m);
}

// Offset of the (slot, head) state block of batch row `row` in ws_states / ws_dstates.
__device__ __forceinline__ int64_t slot_base(const BwdArgs& a, int64_t row, int64_t slot, int h)
{
    return ((row * a.slots + slot) * a.H + h) * int64_t(a.dk_) * a.dv_;
}

// The forward quantities of one chunk shared by the first two kernels.
template <int DK>
struct ChunkRows {
    float Q[CH][DK];  // q, then Qt = q 2^G
    float K[CH][DK];  // k, then Kb = k 2^(G_L - G)
    float E[CH][DK];  // e = b k, then Et = e 2^G
    float G[CH][DK];  // log2 alpha, then its running sum
    float A[CH][CH + 1];
    float P[CH][CH + 1];
};

// Stage rows row0 + H * i (i < L) and form A, P and the absorbed factors.
template <typename T, int DK>
__device__ void chunk_prologue(ChunkRows<DK>& c, const BwdArgs& a, int64_t row0, int L, int tid)
{
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const T* b = static_cast<const T*>(a.b);
    for (int idx = tid; idx < CH * DK; idx += kBwdThreads) {
        const int i = idx / DK, ch = idx % DK;
        if (i < L) {
            const int64_t off = (row0 + int64_t(i) * a.H) * DK + ch;
            const float kk = load_as_f32(k, off);
            c.Q[i][ch] = load_as_f32(q, off);
            c.K[i][ch] = kk;
            c.E[i][ch] = load_as_f32(b, off) * kk;
            c.G[i][ch] = log2_decay(a.alpha[off]);
        } else {
            c.Q[i][ch] = 0.f;
            c.K[i][ch] = 0.f;
            c.E[i][ch] = 0.f;
            c.G[i][ch] = 0.f;
        }
    }
    __syncthreads();
    for (int ch = tid; ch < DK; ch += kBwdThreads) {
        float g = 0.f;
        for (int i = 0; i < L; ++i) {
            g += c.G[i][ch];
            c.G[i][ch] = g;
        }
    }
    __syncthreads();
    for (int idx = tid; idx < CH * CH; idx += kBwdThreads) {
        const int i = idx / CH, j = idx % CH;
        float acc_a = 0.f, acc_p = 0.f;
        if (j <= i && i < L) {
            for (int ch = 0; ch < DK; ++ch) {
                const float kf = c.K[j][ch] * exp2f(c.G[i][ch] - c.G[j][ch]);
                acc_a += c.E[i][ch] * kf;
                acc_p += c.Q[i][ch] * kf;
            }
        }
        c.A[i][j] = j < i ? acc_a : 0.f;
        c.P[i][j] = acc_p;
    }
    __syncthreads();
    for (int idx = tid; idx < L * DK; idx += kBwdThreads) {
        const int i = idx / DK, ch = idx % DK;
        const float g = c.G[i][ch], up = exp2f(g);
        c.E[i][ch] *= up;
        c.Q[i][ch] *= up;
        c.K[i][ch] *= exp2f(c.G[L - 1][ch] - g);
    }
    __syncthreads();
}

// X = Z - Et S into U, then U = (I + A)^-1 X (column-oriented forward substitution).
template <typename T, int DK, int DVT>
__device__ void chunk_solve(const ChunkRows<DK>& c, const float (*S)[DVT], float (*U)[DVT], const BwdArgs& a,
                            int64_t row0, int L, int j0, int tid)
{
    const T* v = static_cast<const T*>(a.v);
    const T* w = static_cast<const T*>(a.w);
    for (int idx = tid; idx < L * DVT; idx += kBwdThreads) {
        const int i = idx / DVT, jj = idx % DVT;
        float acc = 0.f;
        for (int ch = 0; ch < DK; ++ch) acc += c.E[i][ch] * S[ch][jj];
        const int64_t off = (row0 + int64_t(i) * a.H) * a.dv_ + j0 + jj;
        U[i][jj] = load_as_f32(w, off) * load_as_f32(v, off) - acc;
    }
    __syncthreads();
    for (int i = 0; i + 1 < L; ++i) {
        for (int idx = tid; idx < (L - 1 - i) * DVT; idx += kBwdThreads) {
            const int m = i + 1 + idx / DVT, jj = idx % DVT;
            U[m][jj] -= c.A[m][i] * U[i][jj];
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// bwd_states: the forward again, storing the state at every chunk start.
template <typename T, int DK, int DVT>
__global__ __launch_bounds__(kBwdThreads) void bwd_states_kernel(BwdArgs a)
{
    __shared__ ChunkRows<DK> c;
    __shared__ float Ss[DK][DVT];
    __shared__ float Us[CH][DVT];

    const int tid = threadIdx.x;
    const int ntiles = a.dv_ / DVT;
    const int chain = blockIdx.x / ntiles, tile = blockIdx.x % ntiles;
    const int n = chain / a.H, h = chain % a.H;
    const int j0 = tile * DVT;
    const int64_t dv = a.dv_;
    int64_t bos, eos, brow;
    sequence_bounds(a.cu_seqlens, n, a.T, bos, eos, brow);
    const int64_t s_off = (int64_t(n) * a.H + h) * DK * dv + j0;

    for (int idx = tid; idx < DK * DVT; idx += kBwdThreads) {
        const int ch = idx / DVT, jj = idx % DVT;
        Ss[ch][jj] = a.initial_state ? a.initial_state[s_off + int64_t(ch) * dv + jj] : 0.f;
    }
    __syncthreads();
    int m = 0;
    for (int64_t t0 = bos; t0 < eos; t0 += CH, ++m) {
        const int L = int(eos - t0 < CH ? eos - t0 : CH);
        const int64_t row0 = (brow * a.T + t0) * a.H + h;
        float* dst = a.ws_states + slot_base(a, brow, slot_of(a, n, bos, m), h) + j0;
        for (int idx = tid; idx < DK * DVT; idx += kBwdThreads) {
            const int ch = idx / DVT, jj = idx % DVT;
            dst[int64_t(ch) * dv + jj] = Ss[ch][jj];
        }
        chunk_prologue<T, DK>(c, a, row0, L, tid);
        chunk_solve<T, DK, DVT>(c, Ss, Us, a, row0, L, j0, tid);
        for (int idx = tid; idx < DK * DVT; idx += kBwdThreads) {
            const int ch = idx / DVT, jj = idx % DVT;
            float acc = exp2f(c.G[L - 1][ch]) * Ss[ch][jj];
            for (int i = 0; i < L; ++i) acc += c.K[i][ch] * Us[i][jj];
            Ss[ch][jj] = acc;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// bwd_dstate: chunks in reverse, carrying the state gradient.
template <typename T, int DK, int DVT>
__global__ __launch_bounds__(kBwdThreads) void bwd_dstate_kernel(BwdArgs a)
{
    __shared__ ChunkRows<DK> c;
    __shared__ float Ss[DK][DVT];   // chunk-start state
    __shared__ float dSs[DK][DVT];  // gradient of the chunk-end state, then of its start
    __shared__ float Us[CH][DVT];
    __shared__ float dXs[CH][DVT];  // dU, then dX
    __shared__ float dOs[CH][DVT];

    const int tid = threadIdx.x;
    const int ntiles = a.dv_ / DVT;
    const int chain = blockIdx.x / ntiles, tile = blockIdx.x % ntiles;
    const int n = chain / a.H, h = chain % a.H;
    const int j0 = tile * DVT;
    const int64_t dv = a.dv_;
    int64_t bos, eos, brow;
    sequence_bounds(a.cu_seqlens, n, a.T, bos, eos, brow);
    const int64_t s_off = (int64_t(n) * a.H + h) * DK * dv + j0;
    const T* dO = static_cast<const T*>(a.d_o);
    const T* v = static_cast<const T*>(a.v);
    const T* w = static_cast<const T*>(a.w);
    T* dv_out = static_cast<T*>(a.dv);
    T* dw_out = static_cast<T*>(a.dw);

    for (int idx = tid; idx < DK * DVT; idx += kBwdThreads) {
        const int ch = idx / DVT, jj = idx % DVT;
        dSs[ch][jj] = a.d_final_state ? a.d_final_state[s_off + int64_t(ch) * dv + jj] : 0.f;
    }
    __syncthreads();
    const int M = int((eos - bos + CH - 1) / CH);
    for (int m = M - 1; m >= 0; --m) {
        const int64_t t0 = bos + int64_t(m) * CH;
        const int L = int(eos - t0 < CH ? eos - t0 : CH);
        const int64_t row0 = (brow * a.T + t0) * a.H + h;
        const int64_t sb = slot_base(a, brow, slot_of(a, n, bos, m), h) + j0;
        for (int idx = tid; idx < DK * DVT; idx += kBwdThreads) {
            const int ch = idx / DVT, jj = idx % DVT;
            a.ws_dstates[sb + int64_t(ch) * dv + jj] = dSs[ch][jj];
            Ss[ch][jj] = a.ws_states[sb + int64_t(ch) * dv + jj];
        }
        for (int idx = tid; idx < CH * DVT; idx += kBwdThreads) {
            const int i = idx / DVT, jj = idx % DVT;
            dOs[i][jj] = i < L ? load_as_f32(dO, (row0 + int64_t(i) * a.H) * dv + j0 + jj) : 0.f;
        }
        chunk_prologue<T, DK>(c, a, row0, L, tid);  // begins and ends with a barrier
        chunk_solve<T, DK, DVT>(c, Ss, Us, a, row0, L, j0, tid);
        // dU = Kb dS' + P^T dO
        for (int idx = tid; idx < L * DVT; idx += kBwdThreads) {
            const int i = idx / DVT, jj = idx % DVT;
            float acc = 0.f;
            for (int ch = 0; ch < DK; ++ch) acc += c.K[i][ch] * dSs[ch][jj];
            for (int r = i; r < L; ++r) acc += c.P[r][i] * dOs[r][jj];
            dXs[i][jj] = acc;
        }
        __syncthreads();
        // dX = (I + A)^-T dU: backward substitution, row i final once rows > i are done
        for (int i = L - 1; i >= 1; --i) {
            for (int idx = tid; idx < i * DVT; idx += kBwdThreads) {
                const int r = idx / DVT, jj = idx % DVT;
                dXs[r][jj] -= c.A[i][r] * dXs[i][jj];
            }
            __syncthreads();
        }
        for (int idx = tid; idx < L * DVT; idx += kBwdThreads) {
            const int i = idx / DVT, jj = idx % DVT;
            const int64_t off = (row0 + int64_t(i) * a.H) * dv + j0 + jj;
            const float dx = dXs[i][jj];
            a.ws_u[off] = Us[i][jj];
            a.ws_dx[off] = dx;
            store_from_f32(dw_out, off, dx * load_as_f32(v, off));
            store_from_f32(dv_out, off, dx * load_as_f32(w, off));
        }
        // dS = 2^G_L dS' + Qt^T dO - Et^T dX (each element read and written by one thread)
        for (int idx = tid; idx < DK * DVT; idx += kBwdThreads) {
            const int ch = idx / DVT, jj = idx % DVT;
            float acc = exp2f(c.G[L - 1][ch]) * dSs[ch][jj];
            for (int i = 0; i < L; ++i) acc += c.Q[i][ch] * dOs[i][jj] - c.E[i][ch] * dXs[i][jj];
            dSs[ch][jj] = acc;
        }
        __syncthreads();
    }
    if (a.d_initial_state)
        for (int idx = tid; idx < DK * DVT; idx += kBwdThreads) {
            const int ch = idx / DVT, jj = idx % DVT;
            a.d_initial_state[s_off + int64_t(ch) * dv + jj] = dSs[ch][jj];
        }
}

// ---------------------------------------------------------------------------
// bwd_keys: one chunk of one head, channels c0 .. c0 + CB - 1.
template <typename T, int DK, int DV, int CB>
__global__ __launch_bounds__(kBwdThreads) void bwd_keys_kernel(BwdArgs a)
{
    __shared__ float Us[CH][DV], dXs[CH][DV], dOs[CH][DV];
    __shared__ float Sb[CB][DV], dSb[CB][DV];   // rows c0.. of the chunk-start state and end gradient
    __shared__ float dA[CH][CH + 1], dP[CH][CH + 1];
    __shared__ float qb[CH][CB], kb[CH][CB], eb[CH][CB], bb[CH][CB], ab[CH][CB], Gb[CH][CB];
    __shared__ float dEt[CH][CB], dQt[CH][CB], dKb[CH][CB], dg[CH][CB];
    __shared__ float rs[CB];

    const int tid = threadIdx.x;
    constexpr int nblk = DK / CB;
    int64_t idx = blockIdx.x;
    const int cblk = int(idx % nblk);
    idx /= nblk;
    const int h = int(idx % a.H);
    idx /= a.H;
    const int64_t slot = idx % a.slots;
    const int64_t row = idx / a.slots;

    // which chunk of which sequence owns this slot
    int n, m;
    int64_t bos, eos, brow;
    if (!a.cu_seqlens) {
        n = int(row);
        m = int(slot);
        sequence_bounds(nullptr, n, a.T, bos, eos, brow);
        if (int64_t(m) * CH >= eos) return;
    } else {
        // first slot of sequence s: bos_s / CH + s, strictly increasing in s;
        // take the last sequence whose first slot is <= slot
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
        if (slot < first) return;
        m = int(slot - first);
        if (bos + int64_t(m) * CH >= eos || slot_of(a, n, bos, m) != slot) return;
    }
    const int64_t t0 = bos + int64_t(m) * CH;
    const int L = int(eos - t0 < CH ? eos - t0 : CH);
    const int64_t row0 = (brow * a.T + t0) * a.H + h;
    const int c0 = cblk * CB;
    const int64_t sbase = slot_base(a, brow, slot, h);
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const T* b = static_cast<const T*>(a.b);
    const T* dO = static_cast<const T*>(a.d_o);

    for (int i2 = tid; i2 < CH * DV; i2 += kBwdThreads) {
        const int i = i2 / DV, j = i2 % DV;
        const bool live = i < L;
        const int64_t off = (row0 + int64_t(i) * a.H) * DV + j;
        Us[i][j] = live ? a.ws_u[off] : 0.f;
        dXs[i][j] = live ? a.ws_dx[off] : 0.f;
        dOs[i][j] = live ? load_as_f32(dO, off) : 0.f;
    }
    for (int i2 = tid; i2 < CB * DV; i2 += kBwdThreads) {
        const int cc = i2 / DV, j = i2 % DV;
        const int64_t off = sbase + int64_t(c0 + cc) * DV + j;
        Sb[cc][j] = a.ws_states[off];
        dSb[cc][j] = a.ws_dstates[off];
    }
    for (int i2 = tid; i2 < CH * CB; i2 += kBwdThreads) {
        const int i = i2 / CB, cc = i2 % CB;
        if (i < L) {
            const int64_t off = (row0 + int64_t(i) * a.H) * DK + c0 + cc;
            const float kk = load_as_f32(k, off), bv = load_as_f32(b, off);
            qb[i][cc] = load_as_f32(q, off);
            kb[i][cc] = kk;
            bb[i][cc] = bv;
            eb[i][cc] = bv * kk;
            ab[i][cc] = a.alpha[off];
            Gb[i][cc] = log2_decay(a.alpha[off]);
        } else {
            qb[i][cc] = kb[i][cc] = bb[i][cc] = eb[i][cc] = Gb[i][cc] = 0.f;
            ab[i][cc] = 1.f;
        }
    }
    __syncthreads();
    for (int cc = tid; cc < CB; cc += kBwdThreads) {
        float g = 0.f;
        for (int i = 0; i < L; ++i) {
            g += Gb[i][cc];
            Gb[i][cc] = g;
        }
    }
    // dA = -strict_lower(dX U^T), dP = lower(dO U^T) over every value column
    for (int i2 = tid; i2 < CH * CH; i2 += kBwdThreads) {
        const int i = i2 / CH, j = i2 % CH;
        float xa = 0.f, xp = 0.f;
        if (j <= i && i < L)
            for (int jj = 0; jj < DV; ++jj) {
                xa += dXs[i][jj] * Us[j][jj];
                xp += dOs[i][jj] * Us[j][jj];
            }
        dA[i][j] = j < i ? -xa : 0.f;
        dP[i][j] = j <= i ? xp : 0.f;
    }
    // dEt = -dX S^T, dQt = dO S^T, dKb = U dS'^T (this block's channels)
    for (int i2 = tid; i2 < CH * CB; i2 += kBwdThreads) {
        const int i = i2 / CB, cc = i2 % CB;
        float xe = 0.f, xq = 0.f, xk = 0.f;
        if (i < L)
            for (int jj = 0; jj < DV; ++jj) {
                xe += dXs[i][jj] * Sb[cc][jj];
                xq += dOs[i][jj] * Sb[cc][jj];
                xk += Us[i][jj] * dSb[cc][jj];
            }
        dEt[i][cc] = -xe;
        dQt[i][cc] = xq;
        dKb[i][cc] = xk;
    }
    for (int cc = tid; cc < CB; cc += kBwdThreads) {
        float acc = 0.f;
        for (int jj = 0; jj < DV; ++jj) acc += dSb[cc][jj] * Sb[cc][jj];
        rs[cc] = acc;
    }
    __syncthreads();

    T* dq_out = static_cast<T*>(a.dq);
    T* dk_out = static_cast<T*>(a.dk);
    T* db_out = static_cast<T*>(a.db);
    for (int i2 = tid; i2 < L * CB; i2 += kBwdThreads) {
        const int i = i2 / CB, cc = i2 % CB;
        const float gi = Gb[i][cc];
        float de_a = 0.f, dq_p = 0.f, dk_ap = 0.f;
        for (int j = 0; j <= i; ++j) {
            const float kf = kb[j][cc] * exp2f(gi - Gb[j][cc]);
            if (j < i) de_a += dA[i][j] * kf;
            dq_p += dP[i][j] * kf;
        }
        for (int r = i; r < L; ++r) {
            const float f = exp2f(Gb[r][cc] - gi);
            if (r > i) dk_ap += dA[r][i] * eb[r][cc] * f;
            dk_ap += dP[r][i] * qb[r][cc] * f;
        }
        const float up = exp2f(gi), down = exp2f(Gb[L - 1][cc] - gi);
        const float de = de_a + dEt[i][cc] * up;
        const float dq = dq_p + dQt[i][cc] * up;
        const float dkk = dk_ap + dKb[i][cc] * down;
        dg[i][cc] = eb[i][cc] * de_a + qb[i][cc] * dq_p - kb[i][cc] * dk_ap
                    + eb[i][cc] * up * dEt[i][cc] + qb[i][cc] * up * dQt[i][cc] - kb[i][cc] * down * dKb[i][cc];
        const int64_t off = (row0 + int64_t(i) * a.H) * DK + c0 + cc;
        store_from_f32(dq_out, off, dq);
        store_from_f32(db_out, off, de * kb[i][cc]);
        store_from_f32(dk_out, off, dkk + de * bb[i][cc]);
    }
    __syncthreads();
    // the chunk-end terms, then the reverse running sum over the chunk's tokens
    for (int cc = tid; cc < CB; cc += kBwdThreads) {
        const float gl = Gb[L - 1][cc];
        float acc = exp2f(gl) * rs[cc];
        for (int j = 0; j < L; ++j) acc += kb[j][cc] * exp2f(gl - Gb[j][cc]) * dKb[j][cc];
        for (int i = L - 1; i >= 0; --i) {
            acc += dg[i][cc];
            const float al = ab[i][cc];
            const float lg = __log2f(al);
            const bool clamped = !(lg >= kLog2AlphaFloor && lg <= 0.f);
            const int64_t off = (row0 + int64_t(i) * a.H) * DK + c0 + cc;
            a.dalpha[off] = clamped ? 0.f : acc / al;
        }
    }
}

template <typename T, int DK, int DVT>
hipError_t launch_chain_kernels(const BwdArgs& a, hipStream_t stream)
{
    const int64_t blocks = int64_t(a.N) * a.H * (a.dv_ / DVT);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((bwd_states_kernel<T, DK, DVT>), dim3(unsigned(blocks)), dim3(kBwdThreads), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((bwd_dstate_kernel<T, DK, DVT>), dim3(unsigned(blocks)), dim3(kBwdThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int DK, int DV>
hipError_t launch_keys(const BwdArgs& a, hipStream_t stream)
{
    constexpr int CB = DK < 32 ? DK : 32;
    const int64_t blocks = int64_t(a.B) * a.slots * a.H * (DK / CB);
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL((bwd_keys_kernel<T, DK, DV, CB>), dim3(unsigned(blocks)), dim3(kBwdThreads), 0, stream, a);
    return hipGetLastError();
}

template <typename T, int DK>
hipError_t launch_dk(const BwdArgs& a, hipStream_t stream)
{
    if (a.dv_ % 32 != 0) return hipErrorInvalidValue;
    hipError_t e = launch_chain_kernels<T, DK, 32>(a, stream);
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

hipError_t launch_chunk_bwd(const BwdArgs& a, bool bf16, hipStream_t stream)
{
    return bf16 ? launch_typed<bf16raw>(a, stream) : launch_typed<float>(a, stream);
}

}  // namespace gdn2
