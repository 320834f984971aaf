// C ABI of the GDN-2 library: argument validation and kernel dispatch.
//
// Every check runs on the host before anything is enqueued, so argument
// errors come back synchronously and never reach the device.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <atomic>
#include <cstdint>

#include "gdn2.h"
#include "launch.hpp"

namespace {

constexpr int32_t kVersion = 10000;  // 1.0.0

// Tokens per sequence from which gdn2_recurrent_fwd runs the chunkwise kernel
// (measured crossover on MI355X at N = 256, H = 16, d = 128: about 20).
constexpr int32_t kRecurrentChunkMinT = 24;

bool supported_head(int32_t d) { return d == 32 || d == 64 || d == 128; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Span {
    uintptr_t lo, hi;  // [lo, hi)
};

Span span(const void* p, int64_t bytes)
{
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return {lo, lo + uintptr_t(bytes)};
}

bool overlap(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }

int element_bytes(gdn2_dtype dt) { return dt == GDN2_DTYPE_BF16 ? 2 : 4; }

// Compute units of the current device, cached per device id.
int32_t device_cus()
{
    static std::atomic<int32_t> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
    if (dev < 64) {
        const int32_t c = cache[dev].load(std::memory_order_relaxed);
        if (c > 0) return c;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Sequence segments for chunkwise calls with few (sequence, head) chains: the
// plan and its workspace.  The matrix-core kernel runs one workgroup per
// (chain, 64-column value tile), one per CU, walking the sequence chunk by
// chunk, so B x H x dv / 64 workgroups leave most of the GPU idle when that
// is small.  Cutting each row into P segments gives P-fold parallelism for
// the cost of a second pass (see segments.hip):
//   pass 1: segments 0 .. P - 2 of every row, each with dv + dk columns (the
//           real ones from a zero state, segment 0 from the caller's; dk map
//           columns from the identity), final states into the workspace;
//           outputs of segment 0 only;
//   combine: the true incoming state of segments 1 .. P - 1;
//   pass 2: segments 1 .. P - 1 from those states, outputs and the final
//           state.
// P is chosen so that pass 1 fills the GPU once (at most one workgroup per
// CU); segments are whole chunks of at least 256 tokens, at least three are
// needed for a gain, and rows shorter than 1024 tokens keep the single pass.
struct SegPlan {
    int32_t P = 0, len = 0;
    size_t out_bytes = 0, in_bytes = 0, total = 0;
};

SegPlan seg_plan(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv, bool packed, bool bf16, int32_t cus)
{
    SegPlan sp;
    if (!bf16 || dk != 128 || dv % 64 != 0 || packed || B <= 0 || H <= 0 || T < 1024) return sp;
    const int64_t per_seg = int64_t(B) * H * ((dv + dk) / 64);  // pass-1 workgroups per segment
    const int64_t fit = cus / per_seg;                          // segments pass 1 can hold at once
    if (fit < 2) return sp;
    int64_t P = fit + 1;
    int64_t len = ((T + P - 1) / P + 63) / 64 * 64;
    if (len < 256) len = 256;
    P = (T + len - 1) / len;
    if (P < 3) return sp;
    sp.P = int32_t(P);
    sp.len = int32_t(len);
    sp.out_bytes = align256(size_t(B) * P * H * dk * (dv + dk) * 4);
    sp.in_bytes = align256(size_t(B) * P * H * dk * dv * 4);
    sp.total = sp.out_bytes + sp.in_bytes;
    return sp;
}

}  // namespace

extern "C" {

const char* gdn2_status_string(gdn2_status s)
{
    switch (s) {
        case GDN2_OK: return "GDN2_OK";
        case GDN2_ERR_NULL_POINTER: return "GDN2_ERR_NULL_POINTER: a required pointer is NULL";
        case GDN2_ERR_BAD_SHAPE: return "GDN2_ERR_BAD_SHAPE: invalid or inconsistent sizes";
        case GDN2_ERR_UNSUPPORTED: return "GDN2_ERR_UNSUPPORTED: head size not supported (dk, dv in {32, 64, 128})";
        case GDN2_ERR_BAD_DTYPE: return "GDN2_ERR_BAD_DTYPE: unknown dtype";
        case GDN2_ERR_MISALIGNED: return "GDN2_ERR_MISALIGNED: tensor pointer not 16-byte aligned";
        case GDN2_ERR_ALIAS: return "GDN2_ERR_ALIAS: an output overlaps an input";
        case GDN2_ERR_WORKSPACE: return "GDN2_ERR_WORKSPACE: workspace too small";
        case GDN2_ERR_HIP: return "GDN2_ERR_HIP: the HIP runtime reported an error";
        default: break;
    }
    return "GDN2: unknown status";
}

int32_t gdn2_version(void) { return kVersion; }

size_t gdn2_chunk_fwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv, int32_t num_seqs,
                                      gdn2_dtype dtype)
{
    return seg_plan(B, T, H, dk, dv, num_seqs > 0, dtype == GDN2_DTYPE_BF16, device_cus()).total;
}

}  // extern "C"

namespace {

// A gate layout: flags only, and the tie only between a scalar erase gate and
// the (then absent) write gate.
bool valid_gates(int32_t g)
{
    const int32_t all = GDN2_GATES_SCALAR_ERASE | GDN2_GATES_SCALAR_WRITE | GDN2_GATES_TIED | GDN2_GATES_SCALAR_DECAY;
    if (g & ~all) return false;
    if (g & GDN2_GATES_TIED) return (g & GDN2_GATES_SCALAR_ERASE) && !(g & GDN2_GATES_SCALAR_WRITE);
    return true;
}

gdn2_status chunk_fwd(const void* q, const void* k, const void* v, const float* alpha, const void* b, const void* w,
                      const float* initial_state, float* final_state, void* o, const int32_t* cu_seqlens, int32_t B,
                      int32_t T, int32_t H, int32_t dk, int32_t dv, int32_t num_seqs, gdn2_dtype dtype,
                      int32_t gates, void* workspace, size_t workspace_bytes, void* stream)
{
    if (dtype != GDN2_DTYPE_F32 && dtype != GDN2_DTYPE_BF16) return GDN2_ERR_BAD_DTYPE;
    if (!valid_gates(gates)) return GDN2_ERR_BAD_SHAPE;
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return GDN2_ERR_BAD_SHAPE;
    if (cu_seqlens && (B != 1 || num_seqs <= 0)) return GDN2_ERR_BAD_SHAPE;
    if (!supported_head(dk) || !supported_head(dv)) return GDN2_ERR_UNSUPPORTED;
    const bool tied = gates & GDN2_GATES_TIED;
    if (tied) w = nullptr;  // ignored
    const int32_t N = cu_seqlens ? num_seqs : B;
    if (T > 0 && (!q || !k || !v || !alpha || !b || (!tied && !w) || !o)) return GDN2_ERR_NULL_POINTER;
    const void* ptrs[] = {q, k, v, alpha, b, w, o, initial_state, final_state, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN2_ERR_MISALIGNED;
    if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) return GDN2_ERR_MISALIGNED;
    const bool bf16 = dtype == GDN2_DTYPE_BF16;
    // the segmented path runs when the caller passes the workspace it needs
    const SegPlan sp = workspace ? seg_plan(B, T, H, dk, dv, cu_seqlens != nullptr, bf16, device_cus()) : SegPlan{};
    if (sp.P > 0 && workspace_bytes < sp.total) return GDN2_ERR_WORKSPACE;

    const int64_t tokens = int64_t(B) * T * H;
    const int eb = element_bytes(dtype);
    const Span sq = span(q, tokens * dk * eb), sk = span(k, tokens * dk * eb);
    const Span sb = span(b, gates & GDN2_GATES_SCALAR_ERASE ? tokens * eb : tokens * dk * eb);
    const Span sv = span(v, tokens * dv * eb), so = span(o, tokens * dv * eb);
    const Span sw = span(w, tied ? 0 : gates & GDN2_GATES_SCALAR_WRITE ? tokens * eb : tokens * dv * eb);
    const Span sa = span(alpha, gates & GDN2_GATES_SCALAR_DECAY ? tokens * 4 : tokens * dk * 4);
    const int64_t state_bytes = int64_t(N) * H * dk * dv * 4;
    const Span si = span(initial_state, initial_state ? state_bytes : 0);
    const Span sf = span(final_state, final_state ? state_bytes : 0);
    const Span sc = span(cu_seqlens, cu_seqlens ? int64_t(N + 1) * 4 : 0);
    for (Span in : {sq, sk, sv, sa, sb, sw, si, sc})
        if (overlap(so, in)) return GDN2_ERR_ALIAS;
    for (Span in : {sq, sk, sv, sa, sb, sw, sc, so})
        if (overlap(sf, in)) return GDN2_ERR_ALIAS;
    if (overlap(sf, si) && final_state != initial_state) return GDN2_ERR_ALIAS;
    const Span sws = span(workspace, int64_t(sp.total));
    for (Span x : {sq, sk, sv, sa, sb, sw, si, sc, so, sf})
        if (overlap(sws, x)) return GDN2_ERR_ALIAS;

    gdn2::ChunkArgs a{q, k, v, alpha, b, w, initial_state, final_state, o, cu_seqlens,
                      B, T, H, dk, dv, N, device_cus(), gates};
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (sp.P > 0 && T > 0) {
        float* seg_out = static_cast<float*>(workspace);
        float* seg_in = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + sp.out_bytes);
        gdn2::ChunkArgs p1 = a;  // pass 1: segments 0 .. P - 2, real and map columns
        p1.dv = dv + dk;
        p1.dv_io = dv;
        p1.N = B * (sp.P - 1);
        p1.seg_len = sp.len;
        p1.seg_total = sp.P;
        p1.seg_first = 0;
        p1.seg_count = sp.P - 1;
        p1.seg_o_all = 0;
        p1.seg_states_out = seg_out;
        gdn2::ChunkArgs p2 = a;  // pass 2: segments 1 .. P - 1 from their true incoming states
        p2.dv_io = dv;
        p2.N = B * (sp.P - 1);
        p2.seg_len = sp.len;
        p2.seg_total = sp.P;
        p2.seg_first = 1;
        p2.seg_count = sp.P - 1;
        p2.seg_o_all = 1;
        p2.seg_states_in = seg_in;
        hipError_t e = gdn2::launch_chunk_fwd_mfma(p1, st);
        if (e == hipSuccess) e = gdn2::launch_segment_combine(seg_out, seg_in, B, H, dk, dv, sp.P, st);
        if (e == hipSuccess) e = gdn2::launch_chunk_fwd_mfma(p2, st);
        return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
    }
    const hipError_t e = gdn2::chunk_fwd_mfma_supported(a, bf16) ? gdn2::launch_chunk_fwd_mfma(a, st)
                                                                 : gdn2::launch_chunk_fwd_simple(a, bf16, st);
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

gdn2_status recurrent(const void* q, const void* k, const void* v, const float* alpha, const void* b, const void* w,
                      float* state, void* o, int32_t N, int32_t T, int32_t H, int32_t dk, int32_t dv,
                      gdn2_dtype dtype, int32_t gates, void* stream)
{
    if (dtype != GDN2_DTYPE_F32 && dtype != GDN2_DTYPE_BF16) return GDN2_ERR_BAD_DTYPE;
    if (!valid_gates(gates)) return GDN2_ERR_BAD_SHAPE;
    if (N <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return GDN2_ERR_BAD_SHAPE;
    if (!supported_head(dk) || !supported_head(dv)) return GDN2_ERR_UNSUPPORTED;
    const bool tied = gates & GDN2_GATES_TIED;
    if (tied) w = nullptr;  // ignored
    if (!state || (T > 0 && (!q || !k || !v || !alpha || !b || (!tied && !w) || !o))) return GDN2_ERR_NULL_POINTER;
    const void* ptrs[] = {q, k, v, alpha, b, w, state, o};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN2_ERR_MISALIGNED;
    const int64_t tokens = int64_t(N) * T * H;
    const int eb = element_bytes(dtype);
    const Span sq = span(q, tokens * dk * eb), sk = span(k, tokens * dk * eb);
    const Span sb = span(b, gates & GDN2_GATES_SCALAR_ERASE ? tokens * eb : tokens * dk * eb);
    const Span sv = span(v, tokens * dv * eb), so = span(o, tokens * dv * eb);
    const Span sw = span(w, tied ? 0 : gates & GDN2_GATES_SCALAR_WRITE ? tokens * eb : tokens * dv * eb);
    const Span sa = span(alpha, gates & GDN2_GATES_SCALAR_DECAY ? tokens * 4 : tokens * dk * 4);
    const Span ss = span(state, int64_t(N) * H * dk * dv * 4);
    for (Span in : {sq, sk, sv, sa, sb, sw, ss})
        if (overlap(so, in)) return GDN2_ERR_ALIAS;
    for (Span in : {sq, sk, sv, sa, sb, sw})
        if (overlap(ss, in)) return GDN2_ERR_ALIAS;
    if (T == 0) return GDN2_OK;  // nothing to do: the state is unchanged

    // From about 20 tokens per sequence the chunkwise matrix-core kernel is
    // faster (the same mathematics, the [N, T, H, .] inputs taken as a batch,
    // the state updated in place): hand the call to it where it applies.
    const bool bf16 = dtype == GDN2_DTYPE_BF16;
    if (T >= kRecurrentChunkMinT) {
        gdn2::ChunkArgs c{q, k, v, alpha, b, w, state, state, o, nullptr, N, T, H, dk, dv, N, device_cus(), gates};
        if (gdn2::chunk_fwd_mfma_supported(c, bf16)) {
            const hipError_t e = gdn2::launch_chunk_fwd_mfma(c, static_cast<hipStream_t>(stream));
            return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
        }
    }
    gdn2::StepArgs a{q, k, v, alpha, b, w, state, o, N, H, dk, dv, gates, T};
    const hipError_t e = gdn2::launch_recurrent(a, dtype == GDN2_DTYPE_BF16, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

gdn2_status mixer_prologue(const void* xq, const void* xk, const void* xv, const float* conv_q,
                           const float* conv_k, const float* conv_v, const void* b_logit, const void* w_logit,
                           const float* conv_state_in, float* conv_state_out, void* q, void* k, void* v, void* b,
                           void* w, const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H, int32_t dk,
                           int32_t dv, int32_t K, int32_t num_seqs, float q_scale, float eps_l2, gdn2_dtype dtype,
                           void* stream)
{
    if (dtype != GDN2_DTYPE_F32 && dtype != GDN2_DTYPE_BF16) return GDN2_ERR_BAD_DTYPE;
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0 || K < 1 || K > 16) return GDN2_ERR_BAD_SHAPE;
    if (cu_seqlens && (B != 1 || num_seqs <= 0)) return GDN2_ERR_BAD_SHAPE;
    if (!(eps_l2 >= 0.f)) return GDN2_ERR_BAD_SHAPE;
    if (!supported_head(dk) || !supported_head(dv)) return GDN2_ERR_UNSUPPORTED;
    const int32_t N = cu_seqlens ? num_seqs : B;
    if (T > 0 && (!xq || !xk || !xv || !conv_q || !conv_k || !conv_v || !b_logit || !w_logit || !q || !k || !v ||
                  !b || !w))
        return GDN2_ERR_NULL_POINTER;
    const void* ptrs[] = {xq, xk, xv, conv_q, conv_k, conv_v, b_logit, w_logit, conv_state_in, conv_state_out,
                          q, k, v, b, w};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN2_ERR_MISALIGNED;
    if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) return GDN2_ERR_MISALIGNED;
    const int64_t tokens = int64_t(B) * T * H;
    const int eb = element_bytes(dtype);
    const int64_t st_bytes = int64_t(N) * H * (2 * dk + dv) * (K - 1) * 4;
    const Span s_in = span(conv_state_in, conv_state_in ? st_bytes : 0);
    const Span in[] = {span(xq, tokens * dk * eb), span(xk, tokens * dk * eb), span(xv, tokens * dv * eb),
                       span(conv_q, int64_t(H) * dk * K * 4), span(conv_k, int64_t(H) * dk * K * 4),
                       span(conv_v, int64_t(H) * dv * K * 4), span(b_logit, tokens * dk * eb),
                       span(w_logit, tokens * dv * eb), s_in,
                       span(cu_seqlens, cu_seqlens ? int64_t(N + 1) * 4 : 0)};
    const Span out[] = {span(q, tokens * dk * eb), span(k, tokens * dk * eb), span(v, tokens * dv * eb),
                        span(b, tokens * dk * eb), span(w, tokens * dv * eb),
                        span(conv_state_out, conv_state_out ? st_bytes : 0)};
    // The state may be updated in place only when each sequence is one token
    // (a decode step): then one wavefront reads and writes each state row.
    const bool in_place_ok = !cu_seqlens && T == 1 && conv_state_out == conv_state_in;
    for (int i = 0; i < 6; ++i) {
        for (const Span& x : in) {
            if (i == 5 && in_place_ok && x.lo == s_in.lo) continue;
            if (overlap(out[i], x)) return GDN2_ERR_ALIAS;
        }
        for (int j = 0; j < i; ++j)
            if (overlap(out[i], out[j])) return GDN2_ERR_ALIAS;
    }
    gdn2::MixerArgs a{xq, xk, xv, conv_q, conv_k, conv_v, b_logit, w_logit, conv_state_in, conv_state_out,
                      q, k, v, b, w, cu_seqlens, B, T, H, dk, dv, K, N, q_scale, eps_l2};
    const hipError_t e = gdn2::launch_mixer_prologue(a, dtype == GDN2_DTYPE_BF16, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

gdn2_status mixer_epilogue(const void* o, const void* gate, const float* weight, void* y, int64_t rows, int32_t dv,
                           float eps, int32_t act, gdn2_dtype dtype, void* stream)
{
    if (dtype != GDN2_DTYPE_F32 && dtype != GDN2_DTYPE_BF16) return GDN2_ERR_BAD_DTYPE;
    if (rows < 0 || dv <= 0 || (act != 0 && act != 1) || !(eps > 0.f)) return GDN2_ERR_BAD_SHAPE;
    if (!supported_head(dv)) return GDN2_ERR_UNSUPPORTED;
    if (rows > 0 && (!o || !gate || !weight || !y)) return GDN2_ERR_NULL_POINTER;
    const void* ptrs[] = {o, gate, weight, y};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN2_ERR_MISALIGNED;
    const int eb = element_bytes(dtype);
    const Span sy = span(y, rows * dv * eb);
    for (Span x : {span(o, rows * dv * eb), span(gate, rows * dv * eb), span(weight, int64_t(dv) * 4)})
        if (overlap(sy, x)) return GDN2_ERR_ALIAS;
    gdn2::EpilogueArgs a{o, gate, weight, y, rows, dv, eps, act};
    const hipError_t e = gdn2::launch_mixer_epilogue(a, dtype == GDN2_DTYPE_BF16, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

// Workspace regions of the backward pass.  FP32 path: chunk-start states,
// chunk-end state gradients (slots x H x dk x dv FP32 each, per batch row), U
// and dX rows (B x T x H x dv FP32 each) and each chunk's prepared triangular
// algebra (slots x H per batch row), each region 256-byte aligned.  The
// matrix-core path (bf16, dk = dv = 128, T > 0) puts its range flag in the
// first 256 bytes; after it, its own regions (bf16 states and state gradients
// per 64-token slot, bf16 U and dX rows per slot) and the FP32 path's, which
// runs instead when the flag is raised, share the same memory.
struct BwdWorkspace {
    int64_t slots, slots64;
    size_t states, rows, prep, states16, rows16, total;
    bool mfma;
};

BwdWorkspace bwd_workspace(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv, bool varlen, int32_t N,
                           gdn2_dtype dtype)
{
    BwdWorkspace w;
    w.slots = T == 0 ? 0 : (int64_t(T) + gdn2::kBwdChunk - 1) / gdn2::kBwdChunk + (varlen ? N : 0);
    w.states = align256(size_t(B) * size_t(w.slots) * size_t(H) * size_t(dk) * size_t(dv) * 4);
    w.rows = align256(size_t(B) * size_t(T) * size_t(H) * size_t(dv) * 4);
    w.prep = align256(size_t(B) * size_t(w.slots) * size_t(H) * size_t(gdn2::chunk_bwd_prep_floats(dk)) * 4);
    w.total = 2 * w.states + 2 * w.rows + w.prep;
    w.mfma = T > 0 && gdn2::chunk_bwd_mfma_shape(dtype == GDN2_DTYPE_BF16, dk, dv);
    w.slots64 = T == 0 ? 0 : (int64_t(T) + 63) / 64 + (varlen ? N : 0);
    w.states16 = align256(size_t(B) * size_t(w.slots64) * size_t(H) * size_t(dk) * size_t(dv) * 2);
    w.rows16 = align256(size_t(B) * size_t(w.slots64) * size_t(H) * 64 * size_t(dv) * 2);
    if (w.mfma) w.total = 256 + std::max(w.total, 2 * w.states16 + 2 * w.rows16);
    return w;
}

// Host-side checks of a backward call (no HIP call): sizes, pointers,
// alignment, workspace size and overlaps.  ws receives the workspace layout.
// With own_workspace the library supplies the workspace itself: the caller's
// workspace arguments are ignored and no workspace check is made here.
gdn2_status chunk_bwd_check(const void* q, const void* k, const void* v, const float* alpha, const void* b,
                            const void* w, const float* initial_state, const void* d_o, const float* d_final_state,
                            void* dq, void* dk_, void* dv_, float* dalpha, void* db, void* dw,
                            float* d_initial_state, const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H,
                            int32_t dk, int32_t dv, int32_t num_seqs, gdn2_dtype dtype, const void* workspace,
                            size_t workspace_bytes, bool own_workspace, BwdWorkspace& ws)
{
    if (own_workspace) {
        workspace = nullptr;
        workspace_bytes = 0;
    }
    if (dtype != GDN2_DTYPE_F32 && dtype != GDN2_DTYPE_BF16) return GDN2_ERR_BAD_DTYPE;
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return GDN2_ERR_BAD_SHAPE;
    if (cu_seqlens && (B != 1 || num_seqs <= 0)) return GDN2_ERR_BAD_SHAPE;
    if (!supported_head(dk) || !supported_head(dv)) return GDN2_ERR_UNSUPPORTED;
    const int32_t N = cu_seqlens ? num_seqs : B;
    if (T > 0 && (!q || !k || !v || !alpha || !b || !w || !d_o || !dq || !dk_ || !dv_ || !dalpha || !db || !dw))
        return GDN2_ERR_NULL_POINTER;
    const void* ptrs[] = {q, k, v, alpha, b, w, initial_state, d_o, d_final_state,
                          dq, dk_, dv_, dalpha, db, dw, d_initial_state, workspace};
    for (const void* p : ptrs)
        if (p && !aligned16(p)) return GDN2_ERR_MISALIGNED;
    if (cu_seqlens && (reinterpret_cast<uintptr_t>(cu_seqlens) & 3u)) return GDN2_ERR_MISALIGNED;

    ws = bwd_workspace(B, T, H, dk, dv, cu_seqlens != nullptr, N, dtype);
    if (!own_workspace && ws.total > 0 && (!workspace || workspace_bytes < ws.total)) return GDN2_ERR_WORKSPACE;

    const int64_t tokens = int64_t(B) * T * H;
    const int eb = element_bytes(dtype);
    const int64_t state_bytes = int64_t(N) * H * dk * dv * 4;
    const Span in[] = {span(q, tokens * dk * eb), span(k, tokens * dk * eb), span(v, tokens * dv * eb),
                       span(alpha, tokens * dk * 4), span(b, tokens * dk * eb), span(w, tokens * dv * eb),
                       span(initial_state, initial_state ? state_bytes : 0), span(d_o, tokens * dv * eb),
                       span(d_final_state, d_final_state ? state_bytes : 0),
                       span(cu_seqlens, cu_seqlens ? int64_t(N + 1) * 4 : 0)};
    const Span out[] = {span(dq, tokens * dk * eb), span(dk_, tokens * dk * eb), span(dv_, tokens * dv * eb),
                        span(dalpha, tokens * dk * 4), span(db, tokens * dk * eb), span(dw, tokens * dv * eb),
                        span(d_initial_state, d_initial_state ? state_bytes : 0),
                        span(workspace, ws.total > 0 && !own_workspace ? int64_t(ws.total) : 0)};
    constexpr int kDInit = 6;
    for (int i = 0; i < 8; ++i) {
        for (const Span& x : in) {
            // the initial-state gradient may replace the final-state gradient in place
            if (i == kDInit && d_initial_state == d_final_state && x.lo == in[8].lo) continue;
            if (overlap(out[i], x)) return GDN2_ERR_ALIAS;
        }
        for (int j = 0; j < i; ++j)
            if (overlap(out[i], out[j])) return GDN2_ERR_ALIAS;
    }
    return GDN2_OK;
}

// Launches a checked backward call on the given workspace.
gdn2_status chunk_bwd_launch(const void* q, const void* k, const void* v, const float* alpha, const void* b,
                             const void* w, const float* initial_state, const void* d_o, const float* d_final_state,
                             void* dq, void* dk_, void* dv_, float* dalpha, void* db, void* dw,
                             float* d_initial_state, const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H,
                             int32_t dk, int32_t dv, int32_t num_seqs, gdn2_dtype dtype, void* workspace,
                             const BwdWorkspace& ws, void* stream)
{
    const int32_t N = cu_seqlens ? num_seqs : B;
    gdn2::BwdArgs a{};
    a.q = q; a.k = k; a.v = v; a.alpha = alpha; a.b = b; a.w = w;
    a.initial_state = initial_state; a.d_o = d_o; a.d_final_state = d_final_state;
    a.dq = dq; a.dk = dk_; a.dv = dv_; a.dalpha = dalpha; a.db = db; a.dw = dw;
    a.d_initial_state = d_initial_state; a.cu_seqlens = cu_seqlens;
    a.B = B; a.T = T; a.H = H; a.dk_ = dk; a.dv_ = dv; a.N = N;
    a.slots = ws.slots;
    unsigned char* base = static_cast<unsigned char*>(workspace);
    if (ws.mfma) {
        a.range_flag = reinterpret_cast<int32_t*>(base);
        base += 256;
        a.slots64 = ws.slots64;
        a.ws_s16 = reinterpret_cast<uint16_t*>(base);
        a.ws_ds16 = reinterpret_cast<uint16_t*>(base + ws.states16);
        a.ws_u16 = reinterpret_cast<uint16_t*>(base + 2 * ws.states16);
        a.ws_dx16 = reinterpret_cast<uint16_t*>(base + 2 * ws.states16 + ws.rows16);
    }
    a.ws_states = ws.total ? reinterpret_cast<float*>(base) : nullptr;
    a.ws_dstates = ws.total ? reinterpret_cast<float*>(base + ws.states) : nullptr;
    a.ws_u = ws.total ? reinterpret_cast<float*>(base + 2 * ws.states) : nullptr;
    a.ws_dx = ws.total ? reinterpret_cast<float*>(base + 2 * ws.states + ws.rows) : nullptr;
    a.ws_prep = ws.total ? reinterpret_cast<float*>(base + 2 * ws.states + 2 * ws.rows) : nullptr;
    const hipError_t e = ws.mfma ? gdn2::launch_chunk_bwd_mfma(a, static_cast<hipStream_t>(stream))
                                 : gdn2::launch_chunk_bwd(a, dtype == GDN2_DTYPE_BF16, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

gdn2_status chunk_bwd(const void* q, const void* k, const void* v, const float* alpha, const void* b, const void* w,
                      const float* initial_state, const void* d_o, const float* d_final_state, void* dq, void* dk_,
                      void* dv_, float* dalpha, void* db, void* dw, float* d_initial_state,
                      const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv,
                      int32_t num_seqs, gdn2_dtype dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    BwdWorkspace ws{};
    const gdn2_status st = chunk_bwd_check(q, k, v, alpha, b, w, initial_state, d_o, d_final_state, dq, dk_, dv_,
                                           dalpha, db, dw, d_initial_state, cu_seqlens, B, T, H, dk, dv, num_seqs,
                                           dtype, workspace, workspace_bytes, false, ws);
    if (st != GDN2_OK) return st;
    return chunk_bwd_launch(q, k, v, alpha, b, w, initial_state, d_o, d_final_state, dq, dk_, dv_, dalpha, db, dw,
                            d_initial_state, cu_seqlens, B, T, H, dk, dv, num_seqs, dtype, workspace, ws, stream);
}

// The same on the library's own scratch array: the host checks run first
// (the array cannot overlap caller memory), then the workspace size against
// the array's capacity (larger: GDN2_ERR_WORKSPACE); then the array's device
// address on the current device is looked up (once per device) and the
// kernels run on it.  Nothing is allocated.
gdn2_status chunk_bwd_noalloc(const void* q, const void* k, const void* v, const float* alpha, const void* b,
                              const void* w, const float* initial_state, const void* d_o,
                              const float* d_final_state, void* dq, void* dk_, void* dv_, float* dalpha, void* db,
                              void* dw, float* d_initial_state, const int32_t* cu_seqlens, int32_t B, int32_t T,
                              int32_t H, int32_t dk, int32_t dv, int32_t num_seqs, gdn2_dtype dtype, void* stream)
{
    BwdWorkspace ws{};
    const gdn2_status st = chunk_bwd_check(q, k, v, alpha, b, w, initial_state, d_o, d_final_state, dq, dk_, dv_,
                                           dalpha, db, dw, d_initial_state, cu_seqlens, B, T, H, dk, dv, num_seqs,
                                           dtype, nullptr, 0, true, ws);
    if (st != GDN2_OK) return st;
    if (ws.total > gdn2::kScratchBytes) return GDN2_ERR_WORKSPACE;
    void* scratch = nullptr;
    if (ws.total > 0 && gdn2::scratch_pointer(&scratch) != hipSuccess) return GDN2_ERR_HIP;
    return chunk_bwd_launch(q, k, v, alpha, b, w, initial_state, d_o, d_final_state, dq, dk_, dv_, dalpha, db, dw,
                            d_initial_state, cu_seqlens, B, T, H, dk, dv, num_seqs, dtype, scratch, ws, stream);
}

}  // namespace

extern "C" {

gdn2_status gdn2_chunk_fwd(const void* q, const void* k, const void* v, const float* alpha,
                           const void* b, const void* w, const float* initial_state,
                           float* final_state, void* o, const int32_t* cu_seqlens, int32_t B,
                           int32_t T, int32_t H, int32_t dk, int32_t dv, int32_t num_seqs,
                           gdn2_dtype dtype, void* workspace, size_t workspace_bytes, void* stream)
{
    return chunk_fwd(q, k, v, alpha, b, w, initial_state, final_state, o, cu_seqlens, B, T, H, dk, dv, num_seqs,
                     dtype, GDN2_GATES_FULL, workspace, workspace_bytes, stream);
}

gdn2_status gdn2_chunk_fwd_gates(const void* q, const void* k, const void* v, const float* alpha,
                                 const void* b, const void* w, const float* initial_state,
                                 float* final_state, void* o, const int32_t* cu_seqlens, int32_t B,
                                 int32_t T, int32_t H, int32_t dk, int32_t dv, int32_t num_seqs,
                                 gdn2_dtype dtype, int32_t gates, void* workspace,
                                 size_t workspace_bytes, void* stream)
{
    return chunk_fwd(q, k, v, alpha, b, w, initial_state, final_state, o, cu_seqlens, B, T, H, dk, dv, num_seqs,
                     dtype, gates, workspace, workspace_bytes, stream);
}

gdn2_status gdn2_recurrent_step(const void* q, const void* k, const void* v, const float* alpha,
                                const void* b, const void* w, float* state, void* o, int32_t N,
                                int32_t H, int32_t dk, int32_t dv, gdn2_dtype dtype, void* stream)
{
    return recurrent(q, k, v, alpha, b, w, state, o, N, 1, H, dk, dv, dtype, GDN2_GATES_FULL, stream);
}

gdn2_status gdn2_recurrent_step_gates(const void* q, const void* k, const void* v, const float* alpha,
                                      const void* b, const void* w, float* state, void* o, int32_t N,
                                      int32_t H, int32_t dk, int32_t dv, gdn2_dtype dtype,
                                      int32_t gates, void* stream)
{
    return recurrent(q, k, v, alpha, b, w, state, o, N, 1, H, dk, dv, dtype, gates, stream);
}

gdn2_status gdn2_recurrent_fwd(const void* q, const void* k, const void* v, const float* alpha, const void* b,
                               const void* w, float* state, void* o, int32_t N, int32_t T, int32_t H, int32_t dk,
                               int32_t dv, gdn2_dtype dtype, int32_t gates, void* stream)
{
    return recurrent(q, k, v, alpha, b, w, state, o, N, T, H, dk, dv, dtype, gates, stream);
}

gdn2_status gdn2_chunk_bwd(const void* q, const void* k, const void* v, const float* alpha, const void* b,
                           const void* w, const float* initial_state, const void* d_o, const float* d_final_state,
                           void* dq, void* dk, void* dv, float* dalpha, void* db, void* dw, float* d_initial_state,
                           const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H, int32_t dk_size,
                           int32_t dv_size, int32_t num_seqs, gdn2_dtype dtype, void* workspace,
                           size_t workspace_bytes, void* stream)
{
    return chunk_bwd(q, k, v, alpha, b, w, initial_state, d_o, d_final_state, dq, dk, dv, dalpha, db, dw,
                     d_initial_state, cu_seqlens, B, T, H, dk_size, dv_size, num_seqs, dtype, workspace,
                     workspace_bytes, stream);
}

gdn2_status gdn2_chunk_bwd_noalloc(const void* q, const void* k, const void* v, const float* alpha, const void* b,
                                   const void* w, const float* initial_state, const void* d_o,
                                   const float* d_final_state, void* dq, void* dk, void* dv, float* dalpha, void* db,
                                   void* dw, float* d_initial_state, const int32_t* cu_seqlens, int32_t B, int32_t T,
                                   int32_t H, int32_t dk_size, int32_t dv_size, int32_t num_seqs, gdn2_dtype dtype,
                                   void* stream)
{
    return chunk_bwd_noalloc(q, k, v, alpha, b, w, initial_state, d_o, d_final_state, dq, dk, dv, dalpha, db, dw,
                             d_initial_state, cu_seqlens, B, T, H, dk_size, dv_size, num_seqs, dtype, stream);
}

size_t gdn2_chunk_bwd_noalloc_max_workspace_bytes(void) { return gdn2::kScratchBytes; }

size_t gdn2_chunk_bwd_workspace_bytes(int32_t B, int32_t T, int32_t H, int32_t dk, int32_t dv, int32_t num_seqs,
                                      gdn2_dtype dtype)
{
    (void)dtype;
    if (B <= 0 || T < 0 || H <= 0 || dk <= 0 || dv <= 0) return 0;
    return bwd_workspace(B, T, H, dk, dv, num_seqs > 0, num_seqs, dtype).total;
}

gdn2_status gdn2_mixer_prologue(const void* xq, const void* xk, const void* xv, const float* conv_q,
                                const float* conv_k, const float* conv_v, const void* b_logit, const void* w_logit,
                                const float* conv_state_in, float* conv_state_out, void* q, void* k, void* v,
                                void* b, void* w, const int32_t* cu_seqlens, int32_t B, int32_t T, int32_t H,
                                int32_t dk, int32_t dv, int32_t kernel_size, int32_t num_seqs, float q_scale,
                                float eps_l2, gdn2_dtype dtype, void* stream)
{
    return mixer_prologue(xq, xk, xv, conv_q, conv_k, conv_v, b_logit, w_logit, conv_state_in, conv_state_out, q, k,
                          v, b, w, cu_seqlens, B, T, H, dk, dv, kernel_size, num_seqs, q_scale, eps_l2, dtype,
                          stream);
}

gdn2_status gdn2_mixer_epilogue(const void* o, const void* gate, const float* weight, void* y, int64_t rows,
                                int32_t dv, float eps, int32_t gate_act, gdn2_dtype dtype, void* stream)
{
    return mixer_epilogue(o, gate, weight, y, rows, dv, eps, gate_act, dtype, stream);
}

}  // extern "C"
