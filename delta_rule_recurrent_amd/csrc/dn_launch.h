// dn_launch.h -- host-side launchers behind the C ABI (internal; not installed).
// Arguments are assumed validated by the ABI layer (abi.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace dn {

// KIND_SSM: the selective state-space recurrence S = alpha S + k v^T (Gated
// DeltaNet without the correction term: no beta, u = v).
enum Kind { KIND_DELTANET = 0, KIND_GATED = 1, KIND_KDA = 2, KIND_SSM = 3 };
enum DType { DT_F32 = 0, DT_BF16 = 1 };

constexpr int CHUNK = 64;

// Several value heads may share one key head (q and k repeated over the head
// axis, each key head serving g consecutive value heads). Head rows bh run over
// B x hv value heads; q and k are read at key-head row key(bh) of B x hv/g.
// The default (g == 1) is one key head per value head.
struct HeadMap {
    int hv = 1;   // value heads per sequence
    int g = 1;    // value heads per key head
    // (head rows are below 2^24: 32-bit arithmetic)
    __host__ __device__ long key(long bh) const {
        const int r = (int)bh;
        return g == 1 ? bh : (long)((r / hv) * (hv / g) + (r % hv) / g);
    }
};

// One fused decode step for BH (sequence, head) states.
hipError_t launch_decode(int kind, int dtype, const void* q, const void* k, const void* v,
                         const void* beta, const void* g, float* S, void* o, int BH, int dk,
                         int dv, hipStream_t stream, HeadMap hm = HeadMap());

// Token-by-token recurrence over T tokens; S_snap (or NULL): the state after
// every token, [BH][T][dk][dv] fp32.
hipError_t launch_recurrent(int kind, int dtype, const void* q, const void* k, const void* v,
                            const void* beta, const void* g, const float* S0, void* o,
                            float* S_final, int BH, int T, int dk, int dv, hipStream_t stream,
                            float* S_snap = nullptr);

// Chunkwise prefill, phase 1: every chunk in parallel, intermediates -> workspace.
hipError_t launch_chunk_prep(int kind, int dtype, const void* q, const void* k, const void* v,
                             const void* beta, const void* g, void* workspace, int BH, int T,
                             int dk, int dv, hipStream_t stream, HeadMap hm = HeadMap());

// Chunkwise prefill, phase 2: sequential scan over the chunks of every head.
hipError_t launch_chunk_scan(int kind, int dtype, const void* q, const float* S0, void* o,
                             float* S_final, const void* workspace, int BH, int T, int dk, int dv,
                             hipStream_t stream, HeadMap hm = HeadMap());

// Whole chunkwise prefill. FWD_TWO: the two phases above in order.
// FWD_FUSED: one launch (prep and scan workgroups together), or
// hipErrorNotSupported where that form does not exist. FWD_AUTO: the fused
// launch for long sequences where it exists, the two phases otherwise.
enum FwdMode { FWD_TWO = 0, FWD_FUSED = 1, FWD_AUTO = 2 };
hipError_t launch_chunk_fwd(int kind, int dtype, const void* q, const void* k, const void* v,
                            const void* beta, const void* g, const float* S0, void* o,
                            float* S_final, void* workspace, int BH, int T, int dk, int dv,
                            int mode, hipStream_t stream, HeadMap hm = HeadMap());

// Two-phase prefill that also writes the state after every chunk:
// S_bound [BH][ceil(T/64)][dk][dv] fp32.
hipError_t launch_chunk_fwd_states(int kind, int dtype, const void* q, const void* k,
                                   const void* v, const void* beta, const void* g,
                                   const float* S0, void* o, float* S_final, float* S_bound,
                                   void* ws, int BH, int T, int dk, int dv, hipStream_t stream,
                                   HeadMap hm = HeadMap());

// Chunkwise prefill over N packed sequences of different lengths: q, k, v, o
// [H][T] rows holding the sequences back to back (sequence n at tokens
// cu_seqlens[n] .. cu_seqlens[n+1], a device array of N + 1 ints), states
// [N][H]. Always the two phases; the workspace also holds the chunk table.
hipError_t launch_chunk_fwd_varlen(int kind, int dtype, const void* q, const void* k,
                                   const void* v, const void* beta, const void* g,
                                   const float* S0, void* o, float* S_final, const int* cu_seqlens,
                                   int N, int H, int T, int dk, int dv, void* workspace,
                                   hipStream_t stream);
size_t chunk_varlen_workspace_bytes(long long N, long long H, long long T, int dk, int dv,
                                    int dtype);

// Byte offset, in the prefill's workspace, of the one-launch form's error word
// and (next) the epoch of the latest one-launch call on that workspace.
size_t chunk_handoff_offset(long long BH, long long T, int dk, int dtype);

// Workspace bytes of the chunkwise prefill (per call).
size_t chunk_workspace_bytes(long long BH, long long T, int dk, int dv, int dtype);

// Two-phase DeltaNet / Gated DeltaNet prefill with chunks of `chunk` tokens
// (32, 64 or 128; bf16; 128 needs dk = 128); its workspace is BH x
// ceil(T/chunk) blocks. hipErrorNotSupported outside that.
bool chunk_len_supported(int chunk, int dk, int dtype);
size_t chunk_len_workspace_bytes(long long BH, long long T, int dk, int chunk);
hipError_t launch_chunk_fwd_len(int kind, int dtype, int chunk, const void* q, const void* k, const void* v,
                                const void* beta, const void* g, const float* S0, void* o, float* S_final,
                                void* ws, int BH, int T, int dk, hipStream_t st);

// KDA's chunk-parallel phase (chunk_kda.hip): nitems = head rows x nchunks
// (head, chunk) blocks of the workspace; with ctab (int2 per chunk: first token,
// length; length 0 = unused slot) the rows hold packed sequences.
// E is the element type (float or the device bf16), D = d_k = d_v.
template <typename E, int D>
hipError_t launch_kda_prep(const void* q, const void* k, const void* v, const void* beta, const void* g,
                           void* ws, long nitems, int T, int nchunks, HeadMap hm, const void* ctab,
                           hipStream_t st);

// The gated layer around the rule (d = d_k = d_v). Prologue: causal
// convolution + SiLU of the token-major q/k/v channel rows, head split,
// L2 norm of q and k (q also scaled by d^-1/2), gates beta = beta_scale *
// sigmoid(b) and g (g NULL: none);
// then, when conv_state_out != NULL, the new convolution state (may alias
// conv_state). Epilogue: gated RMSNorm of the head-major read-out into
// token-major rows.
hipError_t launch_layer_prologue(int dtype, const void* qkv, const void* conv_w,
                                 const void* conv_state, void* conv_state_out, const void* b,
                                 const void* a, const float* A_log, const float* dt_bias, void* q,
                                 void* k, void* v, void* beta, void* g, float beta_scale, int B,
                                 int T, int Hk, int Hv, int d, hipStream_t st);
hipError_t launch_layer_epilogue(int dtype, const void* o, const void* z, const void* norm_w,
                                 void* out, int B, int Hv, int T, int d, float eps,
                                 hipStream_t st);

// The whole layer for one token per sequence in one kernel (one workgroup per
// (sequence, value head)): the prologue's steps in the load stage, the decode
// step on S [B][Hv][d][d] in place, the gated RMSNorm in the store stage;
// a == NULL: no decay gate (DeltaNet). conv_state_out may alias conv_state
// only when Hk == Hv.
hipError_t launch_layer_decode(int dtype, const void* qkv, const void* conv_w, const void* conv_state,
                               void* conv_state_out, const void* b, const void* a, const float* A_log,
                               const float* dt_bias, const void* z, const void* norm_w, float eps, float* S,
                               void* out, float beta_scale, int B, int Hk, int Hv, int d, hipStream_t st);

// The gated layer's prefill between its projections in three launches (bf16,
// d = 128, T >= 1): the prefill's prep with the layer's prologue in its load
// stage, the scan, the gated RMSNorm. conv_state_out must not overlap
// conv_state; a == NULL: no decay gate. ws: layer_prefill_workspace_bytes.
size_t layer_prefill_workspace_bytes(long long B, long long T, int Hk, int Hv);
hipError_t launch_layer_prefill(const void* qkv, const void* conv_w, const void* conv_state, void* conv_state_out,
                                const void* b, const void* a, const float* A_log, const float* dt_bias,
                                const void* z, const void* norm_w, float eps, const float* S0, float* S_final,
                                void* out, float beta_scale, int B, int T, int Hk, int Hv, void* ws,
                                hipStream_t st);

// Generalized delta rule, token by token: S = (diag(exp g) - (a * kr) kr^T) S
// + kw v^T, o = S^T q; q, kw, kr, a, g [BH][T][d], v, o [BH][T][d]. S0 and
// S_final may be the same buffer (the decode step is T = 1 in place).
hipError_t launch_gdr_recurrent(int dtype, const void* q, const void* kw, const void* v,
                                const void* kr, const void* a, const void* g, const float* S0,
                                void* o, float* S_final, int BH, int T, int d, hipStream_t st);

// S_final = S0 (or zeros when S0 == NULL), n floats; used when T == 0.
hipError_t launch_state_copy(const float* S0, float* S_final, long long n, hipStream_t stream);

}  // namespace dn
