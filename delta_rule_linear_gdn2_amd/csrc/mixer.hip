// Token mixer around the recurrence, for gfx950: the prologue that turns
// projection outputs into q, k, v, b, w, and the epilogue after the
// recurrence.
//
// The Gated DeltaNet-2 analysis (iplexlaw.co.kr, "Token processing and
// parallel training") passes the query and key projections through a causal
// convolution of a few taps, SiLU and an L2 norm, the value projection
// through a convolution and SiLU, and follows the recurrence with an RMS norm
// and an output gate of its own.  The erase and write gates pass through a sigmoid ("Independent
// decisions on two axes").  Per channel c of head h and token t of a
// sequence that starts at bos:
//     y_t = sum_{i<K} W[h d + c][i] x_{t-K+1+i}     (x before bos: the carried state)
//     q = q_scale * L2norm(SiLU(y_q)),  k = L2norm(SiLU(y_k)),  v = SiLU(y_v)
//     b = sigmoid(b_logit),  w = sigmoid(w_logit)
//     out = o / sqrt(mean(o^2) + eps) * weight * act(gate)      (epilogue)
// with L2norm(x) = x / sqrt(sum x^2 + eps_l2).
//
// Each is one pass over HBM, with the norms as reductions inside lane groups.
//   * Prologue, filters of up to four taps (the usual short convolution): one
//     wavefront per (output, batch row, group of heads, run of 64 tokens),
//     where an output is one of q, k, v (convolution, SiLU, and the L2 norm
//     for q and k) or b, w (sigmoid).  A lane takes eight channels with
//     16-byte accesses and a head takes d / 8 lanes, so one load of the
//     wavefront covers 64 / (d / 8) adjacent heads of one token.  The three
//     inputs before the current token stay in registers; tokens go four at a
//     time with the next four's loads in flight.  At a sequence start the
//     window restarts from the carried state; the token that ends a sequence
//     writes the new state, and a small pass carries the state through empty
//     sequences.
//   * Prologue, longer filters (5 to 16 taps): a wavefront walks 16
//     consecutive tokens of one (sequence, head) with two channels per lane,
//     holding the taps and the window of the last K - 1 inputs in registers.
//   * Epilogue: a group of dv / 8 lanes per (token, head) row with 16-byte
//     accesses (four 128-wide rows per wavefront).
#include "gdn2_device.hpp"
#include "launch.hpp"

namespace gdn2 {
namespace {

constexpr int kMixThreads = 256;  // four rows per workgroup

__device__ __forceinline__ float wave_sum(float x)
{
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off, 64);
    return x;
}
// Sigmoid with the hardware reciprocal (about one ulp; the outputs are FP32 or bf16).
__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }

// Sequence of packed position t: the last n with cu[n] <= t (its sequence is
// non-empty and holds t).  Offsets are clamped like every other kernel's.
__device__ __forceinline__ int seq_of(const int32_t* cu, int N, int32_t T, int64_t t)
{
    int lo = 0, hi = N - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        int64_t c = cu[mid];
        c = c < 0 ? 0 : (c > T ? T : c);
        if (c <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Channels per lane: a pair for 128-wide heads (4-byte bf16 / 8-byte FP32
// accesses), one otherwise (32-wide heads use half the lanes).
template <int D>
constexpr int chans_per_lane() { return D >= 128 ? 2 : 1; }

__device__ __forceinline__ void load_ch(const bf16raw* p, int64_t i, float* v, int n)
{
    if (n == 2) {
        const uint32_t u = *reinterpret_cast<const uint32_t*>(p + i);
        v[0] = bf16_to_f32(bf16raw(u & 0xffffu));
        v[1] = bf16_to_f32(bf16raw(u >> 16));
    } else {
        v[0] = bf16_to_f32(p[i]);
    }
}
__device__ __forceinline__ void load_ch(const float* p, int64_t i, float* v, int n)
{
    if (n == 2) {
        const float2 u = *reinterpret_cast<const float2*>(p + i);
        v[0] = u.x;
        v[1] = u.y;
    } else {
        v[0] = p[i];
    }
}
__device__ __forceinline__ void store_ch(bf16raw* p, int64_t i, const float* v, int n)
{
    if (n == 2)
        *reinterpret_cast<uint32_t*>(p + i) = f32x2_to_bf16x2(v[0], v[1]);
    else
        p[i] = f32_to_bf16(v[0]);
}
__device__ __forceinline__ void store_ch(float* p, int64_t i, const float* v, int n)
{
    if (n == 2)
        *reinterpret_cast<float2*>(p + i) = make_float2(v[0], v[1]);
    else
        p[i] = v[0];
}

constexpr int kTokBlock = 16;  // tokens per wavefront

// One convolution path of one (sequence, head) for this lane's channels:
// filter taps and the window of the last K - 1 inputs in registers, for
// K <= KM taps.  Every array index is a compile-time constant (predicated on
// K), so the arrays stay in registers.
template <typename T, int D, int KM>
struct ConvLane {
    static constexpr int CPL = chans_per_lane<D>();
    float w[CPL][KM];        // taps; zero past K
    float win[CPL][KM - 1];  // win[c][j]: input j of the K - 1 before the current token, oldest first
    int c0;                 // first channel of this lane
    bool live;

    __device__ void init(const float* wgt, int h, int lane, int K)
    {
        c0 = lane * CPL;
        live = c0 < D;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
            for (int i = 0; i < KM; ++i) w[c][i] = live && i < K ? wgt[int64_t(h * D + c0 + c) * K + i] : 0.f;
    }
    // the K - 1 inputs before token t of a sequence starting at bos
    __device__ void fill(const T* x, const float* st_in, const MixerArgs& a, int64_t brow, int64_t t, int64_t bos,
                         int h, int n, int state_ch0)
    {
        const int K = a.K;
        const int64_t nch = int64_t(a.H) * (2 * a.dk + a.dv);
#pragma unroll
        for (int j = 0; j < KM - 1; ++j) {
            if (j >= K - 1 || !live) continue;
            const int64_t s = t - (K - 1) + j;
            float v[CPL];
            if (s >= bos) {
                load_ch(x, ((brow * a.T + s) * a.H + h) * D + c0, v, CPL);
            } else {
                const int64_t js = (K - 1) - (bos - s);
#pragma unroll
                for (int c = 0; c < CPL; ++c)
                    v[c] = (st_in && js >= 0) ? st_in[(int64_t(n) * nch + state_ch0 + h * D + c0 + c) * (K - 1) + js] : 0.f;
            }
#pragma unroll
            for (int c = 0; c < CPL; ++c) win[c][j] = v[c];
        }
    }
    // y for input x_t (then x_t joins the window)
    __device__ void step(const float* xt, float* y, int K)
    {
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            float acc = 0.f;
#pragma unroll
            for (int i = 0; i < KM; ++i) {
                const float val = i < K - 1 ? win[c][i < KM - 1 ? i : 0] : (i == K - 1 ? xt[c] : 0.f);
                acc += w[c][i] * val;
            }
            y[c] = acc;
#pragma unroll
            for (int j = 0; j < KM - 1; ++j)
                win[c][j] = j < K - 2 ? win[c][j + 1 < KM - 1 ? j + 1 : j] : (j == K - 2 ? xt[c] : win[c][j]);
        }
    }
    __device__ void write_state(float* st_out, const MixerArgs& a, int h, int n, int state_ch0) const
    {
        const int K = a.K;
        const int64_t nch = int64_t(a.H) * (2 * a.dk + a.dv);
        if (!live) return;
#pragma unroll
        for (int c = 0; c < CPL; ++c)
#pragma unroll
            for (int j = 0; j < KM - 1; ++j)
                if (j < K - 1) st_out[(int64_t(n) * nch + state_ch0 + h * D + c0 + c) * (K - 1) + j] = win[c][j];
    }
};

// One wavefront per (batch row, head, block of kTokBlock tokens of the packed
// axis); the block may cross sequence starts, where the window restarts.
template <typename T, int DK, int DV, int KM>
__global__ __launch_bounds__(kMixThreads) void mixer_prologue_kernel(MixerArgs a)
{
    const int lane = threadIdx.x % 64;
    const int64_t wid = int64_t(blockIdx.x) * (kMixThreads / 64) + threadIdx.x / 64;
    const int64_t nblk = (a.T + kTokBlock - 1) / kTokBlock;
    if (wid >= int64_t(a.B) * nblk * a.H) return;
    const int h = int(wid % a.H);
    const int64_t jb = (wid / a.H) % nblk, brow = wid / a.H / nblk;
    const int64_t t_begin = jb * kTokBlock;
    const int64_t t_end = t_begin + kTokBlock < a.T ? t_begin + kTokBlock : a.T;
    const int K = a.K;
    constexpr int CK = chans_per_lane<DK>(), CV = chans_per_lane<DV>();

    ConvLane<T, DK, KM> lq, lk;
    ConvLane<T, DV, KM> lv;
    lq.init(a.conv_q, h, lane, K);
    lk.init(a.conv_k, h, lane, K);
    lv.init(a.conv_v, h, lane, K);
    const T* xq = static_cast<const T*>(a.xq);
    const T* xk = static_cast<const T*>(a.xk);
    const T* xv = static_cast<const T*>(a.xv);
    const T* bl = static_cast<const T*>(a.b_logit);
    const T* wl = static_cast<const T*>(a.w_logit);
    T* q = static_cast<T*>(a.q);
    T* k = static_cast<T*>(a.k);
    T* v = static_cast<T*>(a.v);
    T* b = static_cast<T*>(a.b);
    T* w = static_cast<T*>(a.w);

    int n;
    int64_t bos, eos;
    if (a.cu_seqlens) {
        n = seq_of(a.cu_seqlens, a.N, a.T, t_begin);
        int64_t b2;
        sequence_bounds(a.cu_seqlens, n, a.T, bos, eos, b2);
    } else {
        n = int(brow);
        bos = 0;
        eos = a.T;
    }
    const int hk = a.H * DK;
    lq.fill(xq, a.conv_state_in, a, brow, t_begin, bos, h, n, 0);
    lk.fill(xk, a.conv_state_in, a, brow, t_begin, bos, h, n, hk);
    lv.fill(xv, a.conv_state_in, a, brow, t_begin, bos, h, n, 2 * hk);
    // this token's inputs, loaded one token ahead so that their latency overlaps the previous token's work
    float nq[CK] = {}, nk[CK] = {}, nb[CK] = {}, nv[CV] = {}, nw[CV] = {};
    auto load_token = [&](int64_t t) {
        const int64_t row = (brow * a.T + t) * a.H + h;
        if (lq.live) {
            load_ch(xq, row * DK + lq.c0, nq, CK);
            load_ch(xk, row * DK + lk.c0, nk, CK);
            load_ch(bl, row * DK + lq.c0, nb, CK);
        }
        if (lv.live) {
            load_ch(xv, row * DV + lv.c0, nv, CV);
            load_ch(wl, row * DV + lv.c0, nw, CV);
        }
    };
    if (t_begin < t_end) load_token(t_begin);
    for (int64_t t = t_begin; t < t_end; ++t) {
        if (t >= eos) {  // the next non-empty sequence starts here (packed input only)
            n = seq_of(a.cu_seqlens, a.N, a.T, t);
            int64_t b2;
            sequence_bounds(a.cu_seqlens, n, a.T, bos, eos, b2);
            lq.fill(xq, a.conv_state_in, a, brow, t, bos, h, n, 0);
            lk.fill(xk, a.conv_state_in, a, brow, t, bos, h, n, hk);
            lv.fill(xv, a.conv_state_in, a, brow, t, bos, h, n, 2 * hk);
        }
        const int64_t row = (brow * a.T + t) * a.H + h;
        float xq_t[CK], xk_t[CK], bl_t[CK], xv_t[CV], wl_t[CV], yq[CK] = {}, yk[CK] = {}, yv[CV] = {};
#pragma unroll
        for (int c = 0; c < CK; ++c) {
            xq_t[c] = nq[c];
            xk_t[c] = nk[c];
            bl_t[c] = nb[c];
        }
#pragma unroll
        for (int c = 0; c < CV; ++c) {
            xv_t[c] = nv[c];
            wl_t[c] = nw[c];
        }
        if (t + 1 < t_end) load_token(t + 1);
        lq.step(xq_t, yq, K);
        lk.step(xk_t, yk, K);
        lv.step(xv_t, yv, K);
        float sq = 0.f, sk = 0.f;
#pragma unroll
        for (int c = 0; c < CK; ++c) {
            yq[c] = lq.live ? silu_f(yq[c]) : 0.f;
            yk[c] = lk.live ? silu_f(yk[c]) : 0.f;
            sq += yq[c] * yq[c];
            sk += yk[c] * yk[c];
        }
        sq = wave_sum(sq);
        sk = wave_sum(sk);
        const float rq = a.q_scale * __builtin_amdgcn_rsqf(sq + a.eps_l2), rk = __builtin_amdgcn_rsqf(sk + a.eps_l2);
        if (lq.live) {
            float o[CK], g[CK];
#pragma unroll
            for (int c = 0; c < CK; ++c) o[c] = yq[c] * rq;
            store_ch(q, row * DK + lq.c0, o, CK);
#pragma unroll
            for (int c = 0; c < CK; ++c) o[c] = yk[c] * rk;
            store_ch(k, row * DK + lk.c0, o, CK);
#pragma unroll
            for (int c = 0; c < CK; ++c) g[c] = sigmoid_f(bl_t[c]);
            store_ch(b, row * DK + lq.c0, g, CK);
        }
        if (lv.live) {
            float o[CV], g[CV];
#pragma unroll
            for (int c = 0; c < CV; ++c) o[c] = silu_f(yv[c]);
            store_ch(v, row * DV + lv.c0, o, CV);
#pragma unroll
            for (int c = 0; c < CV; ++c) g[c] = sigmoid_f(wl_t[c]);
            store_ch(w, row * DV + lv.c0, g, CV);
        }
        if (a.conv_state_out && t == eos - 1 && K > 1) {  // the window now holds the sequence's last K - 1 inputs
            lq.write_state(a.conv_state_out, a, h, n, 0);
            lk.write_state(a.conv_state_out, a, h, n, hk);
            lv.write_state(a.conv_state_out, a, h, n, 2 * hk);
        }
    }
}

// Empty sequences carry their convolution state through unchanged.
__global__ __launch_bounds__(kMixThreads) void mixer_state_passthrough_kernel(MixerArgs a)
{
    const int64_t nch = int64_t(a.H) * (2 * a.dk + a.dv) * (a.K - 1);
    const int64_t i = int64_t(blockIdx.x) * kMixThreads + threadIdx.x;
    if (i >= int64_t(a.N) * nch) return;
    const int n = int(i / nch);
    int64_t bos, eos, brow;
    sequence_bounds(a.cu_seqlens, n, a.T, bos, eos, brow);
    if (eos > bos) return;
    a.conv_state_out[i] = a.conv_state_in ? a.conv_state_in[i] : 0.f;
}

// Eight channels of one row (16 bytes of bf16, 32 of FP32).
__device__ __forceinline__ void load8(const bf16raw* p, int64_t i, float* v)
{
    const uint4 u = *reinterpret_cast<const uint4*>(p + i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        v[2 * j] = bf16_to_f32(bf16raw(w[j] & 0xffffu));
        v[2 * j + 1] = bf16_to_f32(bf16raw(w[j] >> 16));
    }
}
__device__ __forceinline__ void load8(const float* p, int64_t i, float* v)
{
    const float4 a = *reinterpret_cast<const float4*>(p + i), b = *reinterpret_cast<const float4*>(p + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
// Outputs are written once and not read again by the writing kernel, so the
// stores are streaming (nontemporal): on MI355X this took the epilogue from 75
// to 60 us and the prologue from 318 to 311 us on B=8, T=4096, H=16, d=128.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void store8(bf16raw* p, int64_t i, const float* v)
{
    u32x4 w;
    w.x = f32x2_to_bf16x2(v[0], v[1]);
    w.y = f32x2_to_bf16x2(v[2], v[3]);
    w.z = f32x2_to_bf16x2(v[4], v[5]);
    w.w = f32x2_to_bf16x2(v[6], v[7]);
    __builtin_nontemporal_store(w, reinterpret_cast<u32x4*>(p + i));
}
__device__ __forceinline__ void store8(float* p, int64_t i, const float* v)
{
    const f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
    __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p + i));
    __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(p + i + 4));
}

// ---------------------------------------------------------------------------
// Prologue for filters of at most four taps (the usual short convolution): one
// wavefront per (output, batch row, group of heads, run of kRun tokens).  An
// output is one of q, k, v (convolution, SiLU; L2 norm for q and k) or b, w
// (sigmoid).  A lane takes eight channels (16-byte bf16 accesses) and a head
// D / 8 lanes, so one load of a wavefront is 64 / (D / 8) adjacent heads of one
// token, contiguous in memory; every lane walks the same tokens, so sequence
// starts of packed input are the same for the whole wavefront.  The three
// inputs before the current token stay in registers; tokens go kStep at a time
// with the next step's loads in flight.

constexpr int kRun = 64;  // tokens per wavefront
constexpr int kStep = 4;  // tokens per unrolled step
constexpr int kWin = 3;   // window rows: the inputs before the current token, for up to four taps

// Eight channels of one token row, as loaded (bf16 stays packed until used).
template <typename T>
struct Raw8;
template <>
struct Raw8<bf16raw> {
    uint4 u;
    __device__ void load(const bf16raw* p, int64_t i) { u = *reinterpret_cast<const uint4*>(p + i); }
    __device__ void get(float* v) const
    {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            v[2 * j] = __uint_as_float(w[j] << 16);
            v[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
        }
    }
};
template <>
struct Raw8<float> {
    float4 a, b;
    __device__ void load(const float* p, int64_t i)
    {
        a = *reinterpret_cast<const float4*>(p + i);
        b = *reinterpret_cast<const float4*>(p + i + 4);
    }
    __device__ void get(float* v) const
    {
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};

// Where wavefront wid of an output of head width D sits; false past the last.
template <int D>
struct PathPos {
    static constexpr int LPH = D / 8;      // lanes per head
    static constexpr int HPW = 64 / LPH;   // heads per wavefront
    int h, c0;
    int64_t brow, t_begin, t_end;
    __device__ bool init(const MixerArgs& a, int64_t wid, int lane)
    {
        const int ng = (a.H + HPW - 1) / HPW;
        const int64_t nruns = (int64_t(a.T) + kRun - 1) / kRun;
        if (wid >= int64_t(a.B) * nruns * ng) return false;
        const int g = int(wid % ng);
        const int64_t run = (wid / ng) % nruns;
        brow = wid / ng / nruns;
        h = g * HPW + lane / LPH;
        c0 = (lane % LPH) * 8;
        t_begin = run * kRun;
        t_end = t_begin + kRun < a.T ? t_begin + kRun : a.T;
        return h < a.H;  // lanes past the last head stop (they share no reduction with live lanes)
    }
};

template <typename T, int D>
__device__ void gate_path(const T* x, T* y, const MixerArgs& a, int64_t wid, int lane)
{
    PathPos<D> p;
    if (!p.init(a, wid, lane)) return;
    const int64_t stride = int64_t(a.H) * D;  // elements per token
    const int64_t base = ((p.brow * a.T + p.t_begin) * a.H + p.h) * D + p.c0;
    const int n = int(p.t_end - p.t_begin);
    for (int t0 = 0; t0 < n; t0 += 8) {
        Raw8<T> r[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j].load(x, base + int64_t(t0 + j < n ? t0 + j : n - 1) * stride);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            if (t0 + j < n) {
                float v[8];
                r[j].get(v);
#pragma unroll
                for (int c = 0; c < 8; ++c) v[c] = sigmoid_f(v[c]);
                store8(y, base + int64_t(t0 + j) * stride, v);
            }
        }
    }
}

// Convolution output KIND 0 (q: SiLU, L2 norm, q_scale), 1 (k: SiLU, L2 norm)
// or 2 (v: SiLU) of head width D; its convolution-state channels start at
// state_ch0.
template <typename T, int D, int KIND>
__device__ void conv_path(const T* x, const float* wgt, T* y, const MixerArgs& a, int state_ch0, int64_t wid,
                          int lane)
{
    PathPos<D> p;
    if (!p.init(a, wid, lane)) return;
    const int K = a.K;
    const int64_t stride = int64_t(a.H) * D;
    const int64_t nch = int64_t(a.H) * (2 * a.dk + a.dv);
    const int64_t row_base = (p.brow * a.T * a.H + p.h) * D + p.c0;  // token 0 of this row and head
    // wt[j]: the taps for the input kWin - j tokens before the current one (j = kWin: the current token);
    // zero for the j < 4 - K that a shorter filter does not reach
    float wt[kWin + 1][8];
#pragma unroll
    for (int j = 0; j <= kWin; ++j)
#pragma unroll
        for (int c = 0; c < 8; ++c)
            wt[j][c] = j >= kWin + 1 - K ? wgt[(int64_t(p.h) * D + p.c0 + c) * K + (j - (kWin + 1 - K))] : 0.f;

    int n;
    int64_t bos, eos;
    if (a.cu_seqlens) {
        n = seq_of(a.cu_seqlens, a.N, a.T, p.t_begin);
        int64_t b2;
        sequence_bounds(a.cu_seqlens, n, a.T, bos, eos, b2);
    } else {
        n = int(p.brow);
        bos = 0;
        eos = a.T;
    }
    // xr[j] for j < kWin: the input kWin - j tokens before the step's token 0;
    // xr[kWin + i]: the step's token i
    float xr[kWin + kStep][8];
    // the K - 1 inputs before token t (of sequence n from bos) into xr[j0 .. j0 + kWin - 1]
    auto window = [&](int64_t t, float (*w)[8]) {
#pragma unroll
        for (int j = 0; j < kWin; ++j) {
            const int64_t s = t - kWin + j;
#pragma unroll
            for (int c = 0; c < 8; ++c) w[j][c] = 0.f;
            if (j < kWin + 1 - K) continue;  // beyond the filter: stays zero
            if (s >= bos) {
                Raw8<T> r;
                r.load(x, row_base + s * stride);
                r.get(w[j]);
            } else if (a.conv_state_in) {
                const int64_t js = (K - 1) - (bos - s);  // position in the state, oldest first
                if (js >= 0) {
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                        w[j][c] = a.conv_state_in[(int64_t(n) * nch + state_ch0 + int64_t(p.h) * D + p.c0 + c) * (K - 1) + js];
                }
            }
        }
    };
    window(p.t_begin, xr);

    Raw8<T> nx[kStep];
    auto load_step = [&](int64_t t0) {
#pragma unroll
        for (int i = 0; i < kStep; ++i) nx[i].load(x, row_base + (t0 + i < p.t_end ? t0 + i : p.t_end - 1) * stride);
    };
    load_step(p.t_begin);
    for (int64_t t0 = p.t_begin; t0 < p.t_end; t0 += kStep) {
#pragma unroll
        for (int i = 0; i < kStep; ++i) nx[i].get(xr[kWin + i]);
        if (t0 + kStep < p.t_end) load_step(t0 + kStep);
#pragma unroll
        for (int j = 0; j < kStep; ++j) {
            const int64_t t = t0 + j;
            if (t >= p.t_end) continue;
            if (t >= eos) {  // the next non-empty sequence starts here (packed input only)
                n = seq_of(a.cu_seqlens, a.N, a.T, t);
                int64_t b2;
                sequence_bounds(a.cu_seqlens, n, a.T, bos, eos, b2);
                window(t, xr + j);  // rows j .. j + kWin - 1 hold tokens already used
            }
            float v[8];
            float ss = 0.f;
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                float acc = 0.f;
#pragma unroll
                for (int i = 0; i <= kWin; ++i)
                    if (i >= kWin + 1 - K) acc = fmaf(wt[i][c], xr[j + i][c], acc);
                v[c] = acc * sigmoid_f(acc);
                ss = fmaf(v[c], v[c], ss);
            }
            if (KIND < 2) {
#pragma unroll
                for (int off = PathPos<D>::LPH / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);
                const float r = (KIND == 0 ? a.q_scale : 1.0f) * __builtin_amdgcn_rsqf(ss + a.eps_l2);
#pragma unroll
                for (int c = 0; c < 8; ++c) v[c] *= r;
            }
            store8(y, row_base + t * stride, v);
            if (a.conv_state_out && t == eos - 1 && K > 1) {
                // the K - 1 inputs up to and including t, oldest first: rows j + 1 + m hold token t - 2 + m
#pragma unroll
                for (int m = 0; m < kWin; ++m) {
                    const int js = m + K - 1 - kWin;
                    if (js >= 0) {
#pragma unroll
                        for (int c = 0; c < 8; ++c)
                            a.conv_state_out[(int64_t(n) * nch + state_ch0 + int64_t(p.h) * D + p.c0 + c) * (K - 1) + js] =
                                xr[j + 1 + m][c];
                    }
                }
            }
        }
#pragma unroll
        for (int j = 0; j < kWin; ++j)
#pragma unroll
            for (int c = 0; c < 8; ++c) xr[j][c] = xr[kStep + j][c];
    }
}

// blockIdx.y selects the output: 0 q, 1 k, 2 v, 3 b, 4 w.
template <typename T, int DK, int DV>
__global__ __launch_bounds__(kMixThreads) void mixer_prologue_short_kernel(MixerArgs a)
{
    const int lane = threadIdx.x % 64;
    const int64_t wid = int64_t(blockIdx.x) * (kMixThreads / 64) + threadIdx.x / 64;
    const int hk = a.H * DK;
    switch (blockIdx.y) {
        case 0:
            conv_path<T, DK, 0>(static_cast<const T*>(a.xq), a.conv_q, static_cast<T*>(a.q), a, 0, wid, lane);
            break;
        case 1:
            conv_path<T, DK, 1>(static_cast<const T*>(a.xk), a.conv_k, static_cast<T*>(a.k), a, hk, wid, lane);
            break;
        case 2:
            conv_path<T, DV, 2>(static_cast<const T*>(a.xv), a.conv_v, static_cast<T*>(a.v), a, 2 * hk, wid, lane);
            break;
        case 3:
            gate_path<T, DK>(static_cast<const T*>(a.b_logit), static_cast<T*>(a.b), a, wid, lane);
            break;
        default:
            gate_path<T, DV>(static_cast<const T*>(a.w_logit), static_cast<T*>(a.w), a, wid, lane);
            break;
    }
}

// A group of DV / 8 lanes per row (eight channels each), 64 / (DV / 8) rows
// per wavefront; the mean square is a reduction inside the lane group.
template <typename T, int DV>
__global__ __launch_bounds__(kMixThreads) void mixer_epilogue_kernel(EpilogueArgs a)
{
    constexpr int G = DV / 8;            // lanes per row
    constexpr int RPW = 64 / G;          // rows per wavefront
    const int lane = threadIdx.x % 64;
    const int64_t r = (int64_t(blockIdx.x) * (kMixThreads / 64) + threadIdx.x / 64) * RPW + lane / G;
    const bool live = r < a.rows;
    const int c0 = (lane % G) * 8;
    const T* o = static_cast<const T*>(a.o);
    const T* g = static_cast<const T*>(a.gate);
    T* y = static_cast<T*>(a.y);
    float ov[8] = {}, gv[8] = {};
    if (live) {
        load8(o, r * DV + c0, ov);
        load8(g, r * DV + c0, gv);
    }
    float ss = 0.f;
#pragma unroll
    for (int c = 0; c < 8; ++c) ss += ov[c] * ov[c];
#pragma unroll
    for (int off = G / 2; off >= 1; off >>= 1) ss += __shfl_xor(ss, off, 64);  // within the row's lane group
    const float rr = __builtin_amdgcn_rsqf(ss * (1.0f / DV) + a.eps);
    if (!live) return;
    float out[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        const float act = a.act == 0 ? sigmoid_f(gv[c]) : silu_f(gv[c]);
        out[c] = ov[c] * rr * a.weight[c0 + c] * act;
    }
    store8(y, r * DV + c0, out);
}

template <typename T, int DK, int DV>
hipError_t launch_pro(const MixerArgs& a, hipStream_t stream)
{
    if (a.K <= 4) {
        // wavefronts of the output with the narrowest heads (the most head groups)
        const int64_t nruns = (int64_t(a.T) + kRun - 1) / kRun;
        const int hpw = 64 / ((DK < DV ? DK : DV) / 8);
        const int64_t waves = int64_t(a.B) * nruns * ((a.H + hpw - 1) / hpw);
        const int64_t blocks = (waves + 3) / 4;
        if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
        if (blocks > 0) {
            hipLaunchKernelGGL((mixer_prologue_short_kernel<T, DK, DV>), dim3(unsigned(blocks), 5), dim3(kMixThreads),
                               0, stream, a);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    const int64_t waves = int64_t(a.B) * ((a.T + kTokBlock - 1) / kTokBlock) * a.H;
    const int64_t blocks = (waves + 3) / 4;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (blocks > 0 && a.K > 4) {
        if (a.K <= 8)
            hipLaunchKernelGGL((mixer_prologue_kernel<T, DK, DV, 8>), dim3(unsigned(blocks)), dim3(kMixThreads), 0,
                               stream, a);
        else
            hipLaunchKernelGGL((mixer_prologue_kernel<T, DK, DV, 16>), dim3(unsigned(blocks)), dim3(kMixThreads), 0,
                               stream, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.conv_state_out && a.K > 1) {
        // sequences without tokens (every sequence when T = 0) carry the state through
        const int64_t n = int64_t(a.N) * a.H * (2 * a.dk + a.dv) * (a.K - 1);
        if (a.cu_seqlens || a.T == 0) {
            hipLaunchKernelGGL(mixer_state_passthrough_kernel, dim3(unsigned((n + kMixThreads - 1) / kMixThreads)),
                               dim3(kMixThreads), 0, stream, a);
            return hipGetLastError();
        }
    }
    return hipSuccess;
}

template <typename T, int DK>
hipError_t pro_dv(const MixerArgs& a, hipStream_t stream)
{
    switch (a.dv) {
        case 32: return launch_pro<T, DK, 32>(a, stream);
        case 64: return launch_pro<T, DK, 64>(a, stream);
        case 128: return launch_pro<T, DK, 128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t pro_typed(const MixerArgs& a, hipStream_t stream)
{
    switch (a.dk) {
        case 32: return pro_dv<T, 32>(a, stream);
        case 64: return pro_dv<T, 64>(a, stream);
        case 128: return pro_dv<T, 128>(a, stream);
        default: return hipErrorInvalidValue;
    }
}

template <typename T>
hipError_t epi_typed(const EpilogueArgs& a, hipStream_t stream)
{
    const int64_t rows_per_block = int64_t(kMixThreads / 64) * (64 / (a.dv / 8));
    const int64_t blocks = (a.rows + rows_per_block - 1) / rows_per_block;
    if (blocks > 0x7fffffff) return hipErrorInvalidConfiguration;
    if (blocks == 0) return hipSuccess;
    switch (a.dv) {
        case 32: hipLaunchKernelGGL((mixer_epilogue_kernel<T, 32>), dim3(unsigned(blocks)), dim3(kMixThreads), 0,
                                    stream, a); break;
        case 64: hipLaunchKernelGGL((mixer_epilogue_kernel<T, 64>), dim3(unsigned(blocks)), dim3(kMixThreads), 0,
                                    stream, a); break;
        case 128: hipLaunchKernelGGL((mixer_epilogue_kernel<T, 128>), dim3(unsigned(blocks)), dim3(kMixThreads), 0,
                                     stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_mixer_prologue(const MixerArgs& a, bool bf16, hipStream_t stream)
{
    return bf16 ? pro_typed<bf16raw>(a, stream) : pro_typed<float>(a, stream);
}

hipError_t launch_mixer_epilogue(const EpilogueArgs& a, bool bf16, hipStream_t stream)
{
    return bf16 ? epi_typed<bf16raw>(a, stream) : epi_typed<float>(a, stream);
}

}  // namespace gdn2
