// abi.hip -- extern "C" entry points of the delta-rule library (see include/deltanet.h).
// Every argument check runs before the first HIP call, so every error return
// is synchronous and independent of device state.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/deltanet.h"
#include "dn_launch.h"

namespace dn {
// the chunked generalized delta rule (gdr_chunk.hip)
size_t gdr_chunk_workspace_bytes(long long BH, long long T, int d, int chunk);
hipError_t launch_gdr_chunk(int dtype, const void* q, const void* kw, const void* v,
                            const void* kr, const void* a, const void* g, const float* S0,
                            void* o, float* S_final, void* ws, int BH, int T, int d, int chunk,
                            hipStream_t st);
}  // namespace dn

namespace {

constexpr int kVersion = 3;

bool misaligned(const void* p, unsigned a = 16) {
    return (reinterpret_cast<uintptr_t>(p) & (uintptr_t)(a - 1)) != 0;
}

// Validation shared by all entry points. Vector-loaded tensors (q, k, v, o
// and the fp32 states) must be 16-byte aligned; beta and g are read element by
// element and need only the alignment of their element type. With T == 0 the
// per-token tensors are never read and may be NULL (empty tensors).
int check_common(const void* q, const void* k, const void* v, const void* beta, const void* g,
                 bool g_required, const void* S0, const void* o, const void* S_final, int B,
                 int H, int T, int dk, int dv, int dtype) {
    if (B < 1 || H < 1 || T < 0) return DN_EINVAL;
    if (dtype != DN_F32 && dtype != DN_BF16) return DN_EINVAL;
    if (T > 0) {
        if (!q || !k || !v || !beta || !o) return DN_EINVAL;
        if (g_required && !g) return DN_EINVAL;
    }
    const unsigned esz = dtype == DN_F32 ? 4u : 2u;
    if (misaligned(q) || misaligned(k) || misaligned(v) || misaligned(o) ||
        misaligned(beta, esz) || misaligned(g, esz) || misaligned(S0) || misaligned(S_final))
        return DN_EINVAL;
    if ((dk != 64 && dk != 128) || dk != dv) return DN_ENOTSUP;
    const long long BH = (long long)B * H;
    // grid sizes and 32-bit block indices: heads * chunks must fit the grid
    const long long nchunks = ((long long)T + 63) / 64;
    if (BH > (1LL << 24) || nchunks * BH > 0x7fffffffLL) return DN_EINVAL;
    return DN_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int hip_status(hipError_t e) { return e == hipSuccess ? DN_OK : DN_EHIP; }

int check_workspace(long long BH, int T, int dk, int dv, int dtype, const void* workspace,
                    size_t workspace_bytes) {
    const size_t need = dn::chunk_workspace_bytes(BH, T, dk, dv, dtype);
    if (!workspace || workspace_bytes < need) return DN_EWORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return DN_EWORKSPACE;
    return DN_OK;
}

int chunk_kind(bool kda, const void* g) {
    return kda ? dn::KIND_KDA : (g ? dn::KIND_GATED : dn::KIND_DELTANET);
}

int chunk_common(int kind, const void* q, const void* k, const void* v, const void* beta,
                 const void* g, const float* S0, void* o, float* S_final, int B, int H, int T,
                 int dk, int dv, int dtype, void* workspace, size_t workspace_bytes,
                 void* stream, int mode, dn::HeadMap hm = dn::HeadMap()) {
    int st = check_common(q, k, v, beta, g, kind == dn::KIND_KDA, S0, o, S_final, B, H, T, dk,
                          dv, dtype);
    if (st != DN_OK) return st;
    const long long BH = (long long)B * H;
    if (T == 0) {
        if (!S_final) return DN_OK;
        return hip_status(dn::launch_state_copy(S0, S_final, BH * dk * dv, as_stream(stream)));
    }
    st = check_workspace(BH, T, dk, dv, dtype, workspace, workspace_bytes);
    if (st != DN_OK) return st;
    const hipError_t e = dn::launch_chunk_fwd(kind, dtype, q, k, v, beta, g, S0, o, S_final,
                                              workspace, (int)BH, T, dk, dv, mode,
                                              as_stream(stream), hm);
    if (e == hipErrorNotSupported) return DN_ENOTSUP;
    return hip_status(e);
}

int recurrent_common(int kind, const void* q, const void* k, const void* v, const void* beta,
                     const void* g, const float* S0, void* o, float* S_final, int B, int H,
                     int T, int dk, int dv, int dtype, void* stream) {
    int st = check_common(q, k, v, beta, g, kind == dn::KIND_KDA, S0, o, S_final, B, H, T, dk,
                          dv, dtype);
    if (st != DN_OK) return st;
    const long long BH = (long long)B * H;
    if (T == 0) {
        if (!S_final) return DN_OK;
        return hip_status(dn::launch_state_copy(S0, S_final, BH * dk * dv, as_stream(stream)));
    }
    return hip_status(dn::launch_recurrent(kind, dtype, q, k, v, beta, g, S0, o, S_final,
                                           (int)BH, T, dk, dv, as_stream(stream)));
}

int decode_common(int kind, const void* q, const void* k, const void* v, const void* beta,
                  const void* g, float* S, void* o, int B, int H, int dk, int dv, int dtype,
                  void* stream, dn::HeadMap hm = dn::HeadMap()) {
    if (!S) return DN_EINVAL;
    int st = check_common(q, k, v, beta, g, kind == dn::KIND_KDA, S, o, S, B, H, 1, dk, dv, dtype);
    if (st != DN_OK) return st;
    const long long BH = (long long)B * H;
    return hip_status(dn::launch_decode(kind, dtype, q, k, v, beta, g, S, o, (int)BH, dk, dv,
                                        as_stream(stream), hm));
}

// Key heads shared by value heads: Hk >= 1 key heads, Hv a multiple of Hk.
bool head_map(int Hk, int Hv, dn::HeadMap* hm) {
    if (Hk < 1 || Hv < 1 || Hv % Hk != 0) return false;
    hm->hv = Hv;
    hm->g = Hv / Hk;
    return true;
}

// Scratch of dn_chunk_fwd_noalloc: a device array of the library itself, so
// that the call allocates nothing. Each GPU the library runs on holds its own
// copy until the process ends. In host code `scratch` is a host-side stand-in,
// not a device address: its address on a device comes from
// hipGetSymbolAddress, once per device, and only that address is ever passed
// to kernels.
constexpr size_t kScratchBytes = (size_t)128 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // address of `scratch` on each device

int scratch_address(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return DN_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DN_EHIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return DN_OK;
}

}  // namespace

extern "C" {

const char* dn_strerror(int status) {
    switch (status) {
        case DN_OK: return "success";
        case DN_EINVAL: return "invalid argument (NULL or misaligned pointer, bad size or dtype)";
        case DN_ENOTSUP: return "unsupported configuration (d_k, d_v must be equal and in {64, 128}; "
                                "dn_chunk_fwd_fused: no one-launch form)";
        case DN_EWORKSPACE: return "workspace missing, misaligned or smaller than dn_chunk_fwd_workspace()";
        case DN_EHIP: return "HIP runtime error at kernel launch";
        case DN_ESCRATCH: return "sizes need more scratch than dn_chunk_fwd_noalloc's built-in 128 MiB "
                                 "(use dn_chunk_fwd with a workspace)";
        case DN_EHANDOFF: return "the latest one-launch prefill on this workspace had a hand-off wait give up; "
                                 "its results were recomputed by the two phases (they are correct)";
        default: return "unknown status";
    }
}

int dn_version(void) { return kVersion; }

size_t dn_chunk_fwd_workspace(int B, int H, int T, int dk, int dv, int dtype) {
    if (B < 1 || H < 1 || T < 0) return 0;
    if ((dk != 64 && dk != 128) || dk != dv) return 0;
    if (dtype != DN_F32 && dtype != DN_BF16) return 0;
    if (T == 0) return 0;
    return dn::chunk_workspace_bytes((long long)B * H, T, dk, dv, dtype);
}

int dn_chunk_fwd(const void* q, const void* k, const void* v, const void* beta, const void* g,
                 const float* S0, void* o, float* S_final, int B, int H, int T, int dk, int dv,
                 int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    return chunk_common(g ? dn::KIND_GATED : dn::KIND_DELTANET, q, k, v, beta, g, S0, o, S_final,
                        B, H, T, dk, dv, dtype, workspace, workspace_bytes, stream, dn::FWD_AUTO);
}

int dn_chunk_fwd_noalloc(const void* q, const void* k, const void* v, const void* beta,
                         const void* g, const float* S0, void* o, float* S_final, int B, int H,
                         int T, int dk, int dv, int dtype, void* stream) {
    // every argument is checked before the first HIP call
    const int st = check_common(q, k, v, beta, g, false, S0, o, S_final, B, H, T, dk, dv, dtype);
    if (st != DN_OK) return st;
    const int kind = g ? dn::KIND_GATED : dn::KIND_DELTANET;
    if (T == 0)   // no workspace involved
        return chunk_common(kind, q, k, v, beta, g, S0, o, S_final, B, H, T, dk, dv, dtype, nullptr, 0,
                            stream, dn::FWD_AUTO);
    if (dn::chunk_workspace_bytes((long long)B * H, T, dk, dv, dtype) > kScratchBytes) return DN_ESCRATCH;
    void* ws = nullptr;
    const int sa = scratch_address(&ws);
    if (sa != DN_OK) return sa;
    return chunk_common(kind, q, k, v, beta, g, S0, o, S_final, B, H, T, dk, dv, dtype, ws, kScratchBytes,
                        stream, dn::FWD_AUTO);
}

int dn_chunk_fwd_handoff_status(const void* workspace, size_t workspace_bytes, int B, int H, int T,
                                int dk, int dv, int dtype, void* stream) {
    if (B < 1 || H < 1 || T < 0) return DN_EINVAL;
    if (dtype != DN_F32 && dtype != DN_BF16) return DN_EINVAL;
    if ((dk != 64 && dk != 128) || dk != dv) return DN_ENOTSUP;
    const long long BH = (long long)B * H;
    if (T == 0) return DN_OK;
    const int st = check_workspace(BH, T, dk, dv, dtype, workspace, workspace_bytes);
    if (st != DN_OK) return st;
    unsigned long long w[2] = {0, 0};
    const char* at = static_cast<const char*>(workspace) + dn::chunk_handoff_offset(BH, T, dk, dtype);
    if (hipMemcpyAsync(w, at, sizeof(w), hipMemcpyDeviceToHost, as_stream(stream)) != hipSuccess) return DN_EHIP;
    if (hipStreamSynchronize(as_stream(stream)) != hipSuccess) return DN_EHIP;
    // the error word holds the epoch of a failed launch; the word after it the
    // epoch of the latest one-launch call
    return (w[1] != 0 && w[0] == w[1]) ? DN_EHANDOFF : DN_OK;
}

int dn_chunk_fwd_fused(const void* q, const void* k, const void* v, const void* beta,
                       const void* g, const float* S0, void* o, float* S_final, int B, int H,
                       int T, int dk, int dv, int dtype, void* workspace, size_t workspace_bytes,
                       void* stream) {
    if (dtype != DN_BF16) {
        const int st = check_common(q, k, v, beta, g, false, S0, o, S_final, B, H, T, dk, dv, dtype);
        return st != DN_OK ? st : DN_ENOTSUP;
    }
    return chunk_common(g ? dn::KIND_GATED : dn::KIND_DELTANET, q, k, v, beta, g, S0, o, S_final,
                        B, H, T, dk, dv, dtype, workspace, workspace_bytes, stream, dn::FWD_FUSED);
}

size_t dn_chunk_fwd_len_workspace(int B, int H, int T, int dk, int dv, int dtype, int chunk) {
    if (B < 1 || H < 1 || T < 1 || dk != dv) return 0;
    if ((dk != 64 && dk != 128) || !dn::chunk_len_supported(chunk, dk, dtype)) return 0;
    return dn::chunk_len_workspace_bytes((long long)B * H, T, dk, chunk);
}

int dn_chunk_fwd_len(const void* q, const void* k, const void* v, const void* beta, const void* g,
                     const float* S0, void* o, float* S_final, int B, int H, int T, int dk, int dv,
                     int dtype, int chunk, void* workspace, size_t workspace_bytes, void* stream) {
    int st = check_common(q, k, v, beta, g, false, S0, o, S_final, B, H, T, dk, dv, dtype);
    if (st != DN_OK) return st;
    if (!dn::chunk_len_supported(chunk, dk, dtype)) return DN_ENOTSUP;
    const long long BH = (long long)B * H;
    if (T == 0) {
        if (!S_final) return DN_OK;
        return hip_status(dn::launch_state_copy(S0, S_final, BH * dk * dv, as_stream(stream)));
    }
    const size_t need = dn::chunk_len_workspace_bytes(BH, T, dk, chunk);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return DN_EWORKSPACE;
    const hipError_t e = dn::launch_chunk_fwd_len(g ? dn::KIND_GATED : dn::KIND_DELTANET, dtype, chunk, q, k, v,
                                                  beta, g, S0, o, S_final, workspace, (int)BH, T, dk,
                                                  as_stream(stream));
    if (e == hipErrorNotSupported) return DN_ENOTSUP;
    return hip_status(e);
}

int dn_kda_chunk_fwd(const void* q, const void* k, const void* v, const void* beta,
                     const void* g, const float* S0, void* o, float* S_final, int B, int H,
                     int T, int dk, int dv, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream) {
    return chunk_common(dn::KIND_KDA, q, k, v, beta, g, S0, o, S_final, B, H, T, dk, dv, dtype,
                        workspace, workspace_bytes, stream, dn::FWD_AUTO);
}

int dn_chunk_fwd_states(int kda, const void* q, const void* k, const void* v, const void* beta,
                        const void* g, const float* S0, void* o, float* S_final, float* S_chunks,
                        int B, int H, int T, int dk, int dv, int dtype, void* workspace,
                        size_t workspace_bytes, void* stream) {
    const int kind = chunk_kind(kda != 0, g);
    int st = check_common(q, k, v, beta, g, kda != 0, S0, o, S_final, B, H, T, dk, dv, dtype);
    if (st != DN_OK) return st;
    if (T > 0 && !S_chunks) return DN_EINVAL;
    if (misaligned(S_chunks)) return DN_EINVAL;
    const long long BH = (long long)B * H;
    if (T == 0) {
        if (!S_final) return DN_OK;
        return hip_status(dn::launch_state_copy(S0, S_final, BH * dk * dv, as_stream(stream)));
    }
    st = check_workspace(BH, T, dk, dv, dtype, workspace, workspace_bytes);
    if (st != DN_OK) return st;
    return hip_status(dn::launch_chunk_fwd_states(kind, dtype, q, k, v, beta, g, S0, o, S_final,
                                                  S_chunks, workspace, (int)BH, T, dk, dv,
                                                  as_stream(stream)));
}

int dn_chunk_fwd_gqa(int kda, const void* q, const void* k, const void* v, const void* beta,
                     const void* g, const float* S0, void* o, float* S_final, int B, int Hk,
                     int Hv, int T, int dk, int dv, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream) {
    dn::HeadMap hm;
    if (!head_map(Hk, Hv, &hm)) return DN_EINVAL;
    const int kind = chunk_kind(kda != 0, g);
    return chunk_common(kind, q, k, v, beta, g, S0, o, S_final, B, Hv, T, dk, dv, dtype,
                        workspace, workspace_bytes, stream, dn::FWD_AUTO, hm);
}

int dn_decode_step_gqa(int kda, const void* q, const void* k, const void* v, const void* beta,
                       const void* g, float* S, void* o, int B, int Hk, int Hv, int dk, int dv,
                       int dtype, void* stream) {
    dn::HeadMap hm;
    if (!head_map(Hk, Hv, &hm)) return DN_EINVAL;
    return decode_common(kda ? dn::KIND_KDA : (g ? dn::KIND_GATED : dn::KIND_DELTANET), q, k, v,
                         beta, g, S, o, B, Hv, dk, dv, dtype, stream, hm);
}

size_t dn_chunk_fwd_varlen_workspace(int N, int H, int T, int dk, int dv, int dtype) {
    if (N < 1 || H < 1 || T < 0) return 0;
    if ((dk != 64 && dk != 128) || dk != dv) return 0;
    if (dtype != DN_F32 && dtype != DN_BF16) return 0;
    if (T == 0) return 0;
    return dn::chunk_varlen_workspace_bytes(N, H, T, dk, dv, dtype);
}

int dn_chunk_fwd_varlen(int kda, const void* q, const void* k, const void* v, const void* beta,
                        const void* g, const float* S0, void* o, float* S_final,
                        const int* cu_seqlens, int N, int H, int T, int dk, int dv, int dtype,
                        void* workspace, size_t workspace_bytes, void* stream) {
    if (N < 1 || !cu_seqlens || misaligned(cu_seqlens, 4)) return DN_EINVAL;
    int st = check_common(q, k, v, beta, g, kda != 0, S0, o, S_final, 1, H, T, dk, dv, dtype);
    if (st != DN_OK) return st;
    const long long rows = (long long)N * H;
    const long long nc = ((long long)T + 63) / 64 + N;
    if (rows > (1LL << 24) || nc * H > 0x7fffffffLL) return DN_EINVAL;
    if (T == 0) {
        if (!S_final) return DN_OK;
        return hip_status(dn::launch_state_copy(S0, S_final, rows * dk * dv, as_stream(stream)));
    }
    const size_t need = dn::chunk_varlen_workspace_bytes(N, H, T, dk, dv, dtype);
    if (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0)
        return DN_EWORKSPACE;
    const hipError_t e = dn::launch_chunk_fwd_varlen(chunk_kind(kda != 0, g), dtype, q, k, v, beta,
                                                     g, S0, o, S_final, cu_seqlens, N, H, T, dk,
                                                     dv, workspace, as_stream(stream));
    if (e == hipErrorNotSupported) return DN_ENOTSUP;
    return hip_status(e);
}

int dn_decode_tokens(int kda, const void* q, const void* k, const void* v, const void* beta,
                     const void* g, float* S, void* o, float* S_snap, int B, int H, int K, int dk,
                     int dv, int dtype, void* stream) {
    if (!S || K < 1) return DN_EINVAL;
    const int kind = chunk_kind(kda != 0, g);
    int st = check_common(q, k, v, beta, g, kda != 0, S, o, S, B, H, K, dk, dv, dtype);
    if (st != DN_OK) return st;
    if (misaligned(S_snap)) return DN_EINVAL;
    const long long BH = (long long)B * H;
    return hip_status(dn::launch_recurrent(kind, dtype, q, k, v, beta, g, S, o, S, (int)BH, K, dk,
                                           dv, as_stream(stream), S_snap));
}

int dn_layer_prologue(const void* qkv, const void* conv_w, const void* conv_state,
                      void* conv_state_out, const void* b, const void* a, const float* A_log,
                      const float* dt_bias, void* q, void* k, void* v, void* beta, void* g,
                      int allow_neg_eigval, int B, int T, int Hk, int Hv, int dk, int dv,
                      int dtype, void* stream) {
    if (B < 1 || T < 0 || Hk < 1 || Hv < 1 || Hv % Hk != 0) return DN_EINVAL;
    if (dtype != DN_F32 && dtype != DN_BF16) return DN_EINVAL;
    if (B > 65535 || 2LL * Hk + Hv > 65535) return DN_EINVAL;
    if (!conv_w) return DN_EINVAL;
    if (T > 0 && (!qkv || !q || !k || !v || !b || !beta)) return DN_EINVAL;
    if (g && (!a || !A_log || !dt_bias)) return DN_EINVAL;
    const unsigned esz = dtype == DN_F32 ? 4u : 2u;
    if (misaligned(qkv) || misaligned(conv_w) || misaligned(conv_state) ||
        misaligned(conv_state_out) || misaligned(q) || misaligned(k) || misaligned(v) ||
        misaligned(b, esz) || misaligned(a, esz) || misaligned(beta, esz) || misaligned(g, esz) ||
        misaligned(A_log, 4) || misaligned(dt_bias, 4))
        return DN_EINVAL;
    if ((dk != 64 && dk != 128) || dk != dv) return DN_ENOTSUP;
    return hip_status(dn::launch_layer_prologue(dtype, qkv, conv_w, conv_state, conv_state_out, b,
                                                g ? a : nullptr, A_log, dt_bias, q, k, v, beta, g,
                                                allow_neg_eigval ? 2.0f : 1.0f, B, T, Hk, Hv, dk,
                                                as_stream(stream)));
}

int dn_layer_epilogue(const void* o, const void* z, const void* norm_w, void* out, int B, int Hv,
                      int T, int dv, float eps, int dtype, void* stream) {
    if (B < 1 || Hv < 1 || T < 0 || !(eps >= 0.0f && eps < 3.0e38f)) return DN_EINVAL;
    if (dtype != DN_F32 && dtype != DN_BF16) return DN_EINVAL;
    if (!norm_w) return DN_EINVAL;
    if (T > 0 && (!o || !z || !out)) return DN_EINVAL;
    if (misaligned(o) || misaligned(z) || misaligned(norm_w) || misaligned(out)) return DN_EINVAL;
    if ((long long)B * Hv * T > (1LL << 35)) return DN_EINVAL;
    if (dv != 64 && dv != 128) return DN_ENOTSUP;
    return hip_status(dn::launch_layer_epilogue(dtype, o, z, norm_w, out, B, Hv, T, dv, eps,
                                                as_stream(stream)));
}

int dn_layer_decode_step(const void* qkv, const void* conv_w, const void* conv_state,
                         void* conv_state_out, const void* b, const void* a, const float* A_log,
                         const float* dt_bias, const void* z, const void* norm_w, float eps, float* S,
                         void* out, int allow_neg_eigval, int B, int Hk, int Hv, int d, int dtype,
                         void* stream) {
    if (B < 1 || Hk < 1 || Hv < 1 || Hv % Hk != 0 || !(eps >= 0.0f && eps < 3.0e38f)) return DN_EINVAL;
    if (dtype != DN_F32 && dtype != DN_BF16) return DN_EINVAL;
    if ((long long)B * Hv > 0x7fffffffLL) return DN_EINVAL;
    if (!qkv || !conv_w || !b || !z || !norm_w || !S || !out) return DN_EINVAL;
    if (a && (!A_log || !dt_bias)) return DN_EINVAL;
    const unsigned esz = dtype == DN_F32 ? 4u : 2u;
    if (misaligned(qkv) || misaligned(conv_w) || misaligned(conv_state) || misaligned(conv_state_out) ||
        misaligned(z) || misaligned(norm_w) || misaligned(S) || misaligned(out) || misaligned(b, esz) ||
        misaligned(a, esz) || misaligned(A_log, 4) || misaligned(dt_bias, 4))
        return DN_EINVAL;
    if (d != 64 && d != 128) return DN_ENOTSUP;
    // the new convolution history in place only where no other workgroup
    // reads a channel's old entries (one value head per key head); otherwise
    // the two histories must not overlap at all
    if (conv_state && conv_state_out && conv_state != conv_state_out) {
        const long long bytes = (long long)B * (2LL * Hk + Hv) * d * 3 * esz;
        const char* x0 = static_cast<const char*>(conv_state);
        const char* y0 = static_cast<const char*>(conv_state_out);
        if (x0 < y0 + bytes && y0 < x0 + bytes) return DN_EINVAL;
    }
    if (conv_state && conv_state == conv_state_out && Hk != Hv) return DN_EINVAL;
    return hip_status(dn::launch_layer_decode(dtype, qkv, conv_w, conv_state, conv_state_out, b, a, A_log,
                                              dt_bias, z, norm_w, eps, S, out, allow_neg_eigval ? 2.0f : 1.0f,
                                              B, Hk, Hv, d, as_stream(stream)));
}

size_t dn_layer_prefill_workspace(int B, int T, int Hk, int Hv, int d, int dtype) {
    if (B < 1 || T < 0 || Hk < 1 || Hv < 1 || d != 128 || dtype != DN_BF16) return 0;
    return dn::layer_prefill_workspace_bytes(B, T, Hk, Hv);
}

int dn_layer_prefill(const void* qkv, const void* conv_w, const void* conv_state, void* conv_state_out,
                     const void* b, const void* a, const float* A_log, const float* dt_bias, const void* z,
                     const void* norm_w, float eps, const float* S0, float* S_final, void* out,
                     int allow_neg_eigval, int B, int T, int Hk, int Hv, int d, int dtype, void* workspace,
                     size_t workspace_bytes, void* stream) {
    if (B < 1 || T < 0 || Hk < 1 || Hv < 1 || Hv % Hk != 0 || !(eps >= 0.0f && eps < 3.0e38f)) return DN_EINVAL;
    if (dtype != DN_F32 && dtype != DN_BF16) return DN_EINVAL;
    if ((long long)B * Hv > (1 << 24) || (long long)B * Hv * ((T + 63) / 64) > 0x7fffffffLL) return DN_EINVAL;
    if (!conv_w || !norm_w || !S_final) return DN_EINVAL;
    if (T > 0 && (!qkv || !b || !z || !out)) return DN_EINVAL;
    if (a && (!A_log || !dt_bias)) return DN_EINVAL;
    const unsigned esz = dtype == DN_F32 ? 4u : 2u;
    if (misaligned(qkv) || misaligned(conv_w) || misaligned(conv_state) || misaligned(conv_state_out) ||
        misaligned(z) || misaligned(norm_w) || misaligned(out) || misaligned(S0) || misaligned(S_final) ||
        misaligned(b, esz) || misaligned(a, esz) || misaligned(A_log, 4) || misaligned(dt_bias, 4))
        return DN_EINVAL;
    if (d != 128 || dtype != DN_BF16) return DN_ENOTSUP;
    // the last chunk's items write the new history while the first chunk's read
    // the old one: the two must not overlap at all
    if (conv_state && conv_state_out) {
        const long long bytes = (long long)B * (2LL * Hk + Hv) * d * 3 * esz;
        const char* x0 = static_cast<const char*>(conv_state);
        const char* y0 = static_cast<const char*>(conv_state_out);
        if (x0 < y0 + bytes && y0 < x0 + bytes) return DN_EINVAL;
    }
    if (T == 0) {
        // no token: the history passes through, the state is copied
        const hipError_t e = dn::launch_layer_prologue(dtype, qkv, conv_w, conv_state, conv_state_out, b, nullptr,
                                                       nullptr, nullptr, nullptr, nullptr, nullptr, nullptr,
                                                       nullptr, 1.0f, B, 0, Hk, Hv, d, as_stream(stream));
        if (e != hipSuccess) return hip_status(e);
        return hip_status(dn::launch_state_copy(S0, S_final, (long long)B * Hv * d * d, as_stream(stream)));
    }
    if (!workspace || misaligned(workspace, 256) ||
        workspace_bytes < dn::layer_prefill_workspace_bytes(B, T, Hk, Hv))
        return DN_EWORKSPACE;
    return hip_status(dn::launch_layer_prefill(qkv, conv_w, conv_state, conv_state_out, b, a, A_log, dt_bias, z,
                                               norm_w, eps, S0, S_final, out, allow_neg_eigval ? 2.0f : 1.0f, B, T,
                                               Hk, Hv, workspace, as_stream(stream)));
}

int dn_ssm_chunk_fwd(const void* q, const void* k, const void* v, const void* g,
                     const float* S0, void* o, float* S_final, int B, int H, int T, int dk, int dv,
                     int dtype, void* workspace, size_t workspace_bytes, void* stream) {
    if (T > 0 && !g) return DN_EINVAL;
    // (g stands in for beta in the shared checks: the state-space kind has none)
    const int st = check_common(q, k, v, g, g, false, S0, o, S_final, B, H, T, dk, dv, dtype);
    if (st != DN_OK) return st;
    return chunk_common(dn::KIND_SSM, q, k, v, g, g, S0, o, S_final, B, H, T, dk, dv, dtype,
                        workspace, workspace_bytes, stream, dn::FWD_TWO);
}

int dn_ssm_recurrent_fwd(const void* q, const void* k, const void* v, const void* g,
                         const float* S0, void* o, float* S_final, int B, int H, int T, int dk,
                         int dv, int dtype, void* stream) {
    if (T > 0 && !g) return DN_EINVAL;
    return recurrent_common(dn::KIND_SSM, q, k, v, g, g, S0, o, S_final, B, H, T, dk, dv, dtype,
                            stream);
}

int dn_ssm_decode_step(const void* q, const void* k, const void* v, const void* g, float* S,
                       void* o, int B, int H, int dk, int dv, int dtype, void* stream) {
    if (!g) return DN_EINVAL;
    return decode_common(dn::KIND_SSM, q, k, v, g, g, S, o, B, H, dk, dv, dtype, stream);
}

// The generalized rule's single-token kernel reads the states, v and o as
// 16-byte vectors; the other per-token tensors are read element by element.
static int gdr_check(const void* q, const void* kw, const void* v, const void* kr, const void* a,
                     const void* g, const void* S0, const void* o, const void* S_final, int B,
                     int H, int T, int dk, int dv, int dtype) {
    if (B < 1 || H < 1 || T < 0) return DN_EINVAL;
    if (dtype != DN_F32 && dtype != DN_BF16) return DN_EINVAL;
    if (T > 0 && (!q || !kw || !v || !kr || !a || !g || !o)) return DN_EINVAL;
    const unsigned esz = dtype == DN_F32 ? 4u : 2u;
    if (misaligned(q, esz) || misaligned(kw, esz) || misaligned(v) || misaligned(kr, esz) ||
        misaligned(a, esz) || misaligned(g, esz) || misaligned(o) || misaligned(S0) ||
        misaligned(S_final))
        return DN_EINVAL;
    if ((dk != 64 && dk != 128) || dk != dv) return DN_ENOTSUP;
    if ((long long)B * H * (dk / 64) > 0x7fffffffLL) return DN_EINVAL;
    return DN_OK;
}

int dn_gdr_recurrent_fwd(const void* q, const void* kw, const void* v, const void* kr,
                         const void* a, const void* g, const float* S0, void* o, float* S_final,
                         int B, int H, int T, int dk, int dv, int dtype, void* stream) {
    const int st = gdr_check(q, kw, v, kr, a, g, S0, o, S_final, B, H, T, dk, dv, dtype);
    if (st != DN_OK) return st;
    const long long BH = (long long)B * H;
    if (T == 0) {
        if (!S_final) return DN_OK;
        return hip_status(dn::launch_state_copy(S0, S_final, BH * dk * dv, as_stream(stream)));
    }
    return hip_status(dn::launch_gdr_recurrent(dtype, q, kw, v, kr, a, g, S0, o, S_final, (int)BH,
                                               T, dk, as_stream(stream)));
}

static bool gdr_chunk_size_ok(int chunk) { return chunk == 16 || chunk == 32 || chunk == 64; }

size_t dn_gdr_chunk_workspace(int B, int H, int T, int dk, int dv, int dtype, int chunk) {
    if (B < 1 || H < 1 || T < 1 || !gdr_chunk_size_ok(chunk)) return 0;
    if ((dk != 64 && dk != 128) || dk != dv) return 0;
    if (dtype != DN_F32 && dtype != DN_BF16) return 0;
    return dn::gdr_chunk_workspace_bytes((long long)B * H, T, dk, chunk);
}

int dn_gdr_chunk_fwd(const void* q, const void* kw, const void* v, const void* kr, const void* a,
                     const void* g, const float* S0, void* o, float* S_final, int B, int H, int T,
                     int dk, int dv, int dtype, int chunk, void* workspace,
                     size_t workspace_bytes, void* stream) {
    const int st = gdr_check(q, kw, v, kr, a, g, S0, o, S_final, B, H, T, dk, dv, dtype);
    if (st != DN_OK) return st;
    // the chunked form's kernels read q, kw, kr, a and g as vectors of four
    // elements (8 bytes for bf16, 16 for fp32)
    const unsigned vsz = dtype == DN_F32 ? 16u : 8u;
    if (misaligned(q, vsz) || misaligned(kw, vsz) || misaligned(kr, vsz) || misaligned(a, vsz) ||
        misaligned(g, vsz))
        return DN_EINVAL;
    if (!gdr_chunk_size_ok(chunk)) return DN_ENOTSUP;
    const long long BH = (long long)B * H;
    if (T == 0) {
        if (!S_final) return DN_OK;
        return hip_status(dn::launch_state_copy(S0, S_final, BH * dk * dv, as_stream(stream)));
    }
    // every chunk is one workgroup of the map kernels, four of the products
    if (BH * ((T + chunk - 1) / chunk) > (1LL << 28)) return DN_EINVAL;
    const size_t need = dn::gdr_chunk_workspace_bytes(BH, T, dk, chunk);
    if (!workspace || workspace_bytes < need || misaligned(workspace, 256)) return DN_EWORKSPACE;
    return hip_status(dn::launch_gdr_chunk(dtype, q, kw, v, kr, a, g, S0, o, S_final, workspace,
                                           (int)BH, T, dk, chunk, as_stream(stream)));
}

int dn_gdr_decode_step(const void* q, const void* kw, const void* v, const void* kr,
                       const void* a, const void* g, float* S, void* o, int B, int H, int dk,
                       int dv, int dtype, void* stream) {
    if (!S) return DN_EINVAL;
    const int st = gdr_check(q, kw, v, kr, a, g, S, o, S, B, H, 1, dk, dv, dtype);
    if (st != DN_OK) return st;
    return hip_status(dn::launch_gdr_recurrent(dtype, q, kw, v, kr, a, g, S, o, S, B * H, 1, dk,
                                               as_stream(stream)));
}

int dn_chunk_prep(int kda, const void* q, const void* k, const void* v, const void* beta,
                  const void* g, int B, int H, int T, int dk, int dv, int dtype, void* workspace,
                  size_t workspace_bytes, void* stream) {
    // o is not touched by this phase: q stands in for it in the shared checks
    int st = check_common(q, k, v, beta, g, kda != 0, nullptr, q, nullptr, B, H, T, dk, dv, dtype);
    if (st != DN_OK) return st;
    if (T == 0) return DN_OK;
    const long long BH = (long long)B * H;
    st = check_workspace(BH, T, dk, dv, dtype, workspace, workspace_bytes);
    if (st != DN_OK) return st;
    return hip_status(dn::launch_chunk_prep(chunk_kind(kda != 0, g), dtype, q, k, v, beta, g,
                                            workspace, (int)BH, T, dk, dv, as_stream(stream)));
}

int dn_chunk_scan(int kda, const void* q, const float* S0, void* o, float* S_final, int B, int H,
                  int T, int dk, int dv, int dtype, const void* workspace, size_t workspace_bytes,
                  void* stream) {
    // k, v and beta are not read by this phase: q stands in for them
    int st = check_common(q, q, q, q, nullptr, false, S0, o, S_final, B, H, T, dk, dv, dtype);
    if (st != DN_OK) return st;
    const long long BH = (long long)B * H;
    if (T == 0) {
        if (!S_final) return DN_OK;
        return hip_status(dn::launch_state_copy(S0, S_final, BH * dk * dv, as_stream(stream)));
    }
    st = check_workspace(BH, T, dk, dv, dtype, workspace, workspace_bytes);
    if (st != DN_OK) return st;
    return hip_status(dn::launch_chunk_scan(kda ? dn::KIND_KDA : dn::KIND_GATED, dtype, q, S0, o,
                                            S_final, workspace, (int)BH, T, dk, dv,
                                            as_stream(stream)));
}

int dn_recurrent_fwd(const void* q, const void* k, const void* v, const void* beta,
                     const void* g, const float* S0, void* o, float* S_final, int B, int H,
                     int T, int dk, int dv, int dtype, void* stream) {
    return recurrent_common(g ? dn::KIND_GATED : dn::KIND_DELTANET, q, k, v, beta, g, S0, o,
                            S_final, B, H, T, dk, dv, dtype, stream);
}

int dn_kda_recurrent_fwd(const void* q, const void* k, const void* v, const void* beta,
                         const void* g, const float* S0, void* o, float* S_final, int B, int H,
                         int T, int dk, int dv, int dtype, void* stream) {
    return recurrent_common(dn::KIND_KDA, q, k, v, beta, g, S0, o, S_final, B, H, T, dk, dv,
                            dtype, stream);
}

int dn_decode_step(const void* q, const void* k, const void* v, const void* beta, const void* g,
                   float* S, void* o, int B, int H, int dk, int dv, int dtype, void* stream) {
    return decode_common(g ? dn::KIND_GATED : dn::KIND_DELTANET, q, k, v, beta, g, S, o, B, H,
                         dk, dv, dtype, stream);
}

int dn_kda_decode_step(const void* q, const void* k, const void* v, const void* beta,
                       const void* g, float* S, void* o, int B, int H, int dk, int dv, int dtype,
                       void* stream) {
    return decode_common(dn::KIND_KDA, q, k, v, beta, g, S, o, B, H, dk, dv, dtype, stream);
}

}  // extern "C"
