// Host-visible launch interface between the C ABI layer and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn2 {

// Gate layout flags (the values of gdn2_gate_flags).
constexpr int32_t kScalarErase = 1, kScalarWrite = 2, kTied = 4, kScalarDecay = 8;

struct ChunkArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const void* b;
    const void* w;
    const float* initial_state;
    float* final_state;
    void* o;
    const int32_t* cu_seqlens;
    int32_t B, T, H, dk, dv, N;
    int32_t cus;    // compute units of the device
    int32_t gates;  // gdn2_gate_flags, validated: 1 scalar erase, 2 scalar write, 4 write tied to erase, 8 scalar decay
    // Sequence segments (matrix-core kernel only; seg_len = 0: off).  Each
    // batch row (no cu_seqlens) is cut into seg_total segments of seg_len
    // tokens (the last may be shorter); launch sequence n is segment
    // seg_first + n % seg_count of row n / seg_count, and N = B * seg_count.
    // Value columns j >= dv_io are map columns: they start from the identity
    // (column j holds e_{j - dv_io}), take z = 0 and write no output, so they
    // carry the segment's state map.  Initial state of a segment: from
    // seg_states_in ([B][seg_total][H][dk][dv_io]) if given, else the
    // caller's initial_state for segment 0 and zero otherwise.  Final state:
    // into seg_states_out ([B][seg_total][H][dk][dv], every column) if given,
    // else the caller's final_state for the row's last segment.  o (dv_io
    // columns) is written for every segment when seg_o_all, else for segment
    // 0 only.
    int32_t seg_len, seg_total, seg_first, seg_count, seg_o_all;
    int32_t dv_io;  // columns of v, w, o and the caller's states (0: dv)
    const float* seg_states_in;
    float* seg_states_out;
};

struct StepArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const void* b;
    const void* w;
    float* state;
    void* o;
    int32_t N, H, dk, dv;
    int32_t gates;  // as in ChunkArgs
    int32_t T;      // tokens per sequence: inputs [N, T, H, .], o [N, T, H, dv]
};

// Chunkwise backward.  Chunk-start states and chunk-end state gradients sit
// in "slots": slot m of batch row n for packed-free input, and for packed
// sequences slot (bos + m * kBwdChunk) / kBwdChunk + n of row 0 (distinct
// for distinct chunks, fewer than ceil(T / kBwdChunk) + N).
constexpr int kBwdChunk = 32;

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const float* alpha;
    const void* b;
    const void* w;
    const float* initial_state;
    const void* d_o;
    const float* d_final_state;
    void* dq;
    void* dk;
    void* dv;
    float* dalpha;
    void* db;
    void* dw;
    float* d_initial_state;
    const int32_t* cu_seqlens;
    int32_t B, T, H, dk_, dv_, N;
    int64_t slots;       // chunk slots per batch row
    float* ws_states;    // [B][slots][H][dk][dv] state at each chunk start
    float* ws_dstates;   // [B][slots][H][dk][dv] gradient of the state at each chunk end
    float* ws_u;         // [B * T * H][dv] U rows
    float* ws_dx;        // [B * T * H][dv] dX rows
    float* ws_prep;      // [B][slots][H][chunk_bwd_prep_floats(dk)] per-chunk triangular algebra
    // The matrix-core path (bf16, dk = dv = 128, 64-token chunks), whose
    // workspace shares the memory above:
    int64_t slots64;     // 64-token chunk slots per batch row
    uint16_t* ws_s16;     // [B][slots64][H][dk][dv] state at each chunk start
    uint16_t* ws_ds16;    // [B][slots64][H][dk][dv] gradient of the state at each chunk end
    uint16_t* ws_u16;     // [B][slots64][H][64][dv] U rows of each chunk
    uint16_t* ws_dx16;    // [B][slots64][H][64][dv] dX rows of each chunk
    int32_t* range_flag; // set when some chunk decays below the split range: the FP32 path then runs
    const int32_t* gate; // FP32 path kernels do nothing when this is set and *gate == 0
};

// Whether a backward call takes the matrix-core path.
inline bool chunk_bwd_mfma_shape(bool bf16, int dk, int dv) { return bf16 && dk == 128 && dv == 128; }
hipError_t launch_chunk_bwd_mfma(const BwdArgs& a, hipStream_t stream);

// Floats of one chunk's prepared block in ws_prep.
int64_t chunk_bwd_prep_floats(int dk);

// Token-mixer prologue: q, k, v, b, w from projection outputs.
struct MixerArgs {
    const void* xq;
    const void* xk;
    const void* xv;
    const float* conv_q;  // [H * dk][K]
    const float* conv_k;  // [H * dk][K]
    const float* conv_v;  // [H * dv][K]
    const void* b_logit;
    const void* w_logit;
    const float* conv_state_in;  // [N][H * (2 dk + dv)][K - 1] or null (zeros)
    float* conv_state_out;       // same layout, or null
    void* q;
    void* k;
    void* v;
    void* b;
    void* w;
    const int32_t* cu_seqlens;
    int32_t B, T, H, dk, dv, K, N;
    float q_scale, eps_l2;
};

// Token-mixer epilogue: RMS norm times weight times act(gate), per row of dv.
struct EpilogueArgs {
    const void* o;
    const void* gate;
    const float* weight;  // [dv]
    void* y;
    int64_t rows;
    int32_t dv;
    float eps;
    int32_t act;  // 0 sigmoid, 1 SiLU
};

// Each returns hipSuccess or the launch error; bf16 selects the input dtype.
hipError_t launch_mixer_prologue(const MixerArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_mixer_epilogue(const EpilogueArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_chunk_bwd(const BwdArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_recurrent(const StepArgs& a, bool bf16, hipStream_t stream);
hipError_t launch_chunk_fwd_simple(const ChunkArgs& a, bool bf16, hipStream_t stream);

// Library-owned device scratch (scratch.hip): its capacity, and its device
// address on the current device (looked up once per device).
constexpr size_t kScratchBytes = size_t(256) << 20;
hipError_t scratch_pointer(void** out);

// Segment combine (segments.hip): S_in(1) = S_out(0), S_in(p + 1) = M_p
// S_in(p) + N_p for the layouts of ChunkArgs::seg_states_out (dv + dk
// columns) and ::seg_states_in (dv columns).
hipError_t launch_segment_combine(const float* seg_out, float* seg_in, int B, int H, int dk, int dv, int P,
                                  hipStream_t stream);

// Matrix-core chunk kernel: bf16 inputs, dk = 128, dv a multiple of 64.
bool chunk_fwd_mfma_supported(const ChunkArgs& a, bool bf16);
hipError_t launch_chunk_fwd_mfma(const ChunkArgs& a, hipStream_t stream);

}  // namespace gdn2
