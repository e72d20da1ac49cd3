// chunk_kda.hip -- KDA's chunk-parallel phase (per-key-channel decay) on gfx950:
// the UT/WY quantities of every (head, 64-token chunk) written to the chunk
// workspace that the scan in chunk.hip reads (page "A walk through of the
// DeltaNet family of linear attention variants", KDA section; the chunked form
// of page "28. Linear attention and Gated DeltaNet", section "The chunked
// form: recurrence as matrix multiplication").
#include "dn_device.h"
#include "dn_launch.h"
#include "dn_chunk.h"
#include "dn_kda_prep.h"

namespace dn {

// bf16: two workgroups per CU (the LDS allows two) with two wavefronts per
// SIMD; fp32 fragments need more registers than that.
template <typename E, int DK, int DV, bool VARLEN>
__global__ __launch_bounds__(256, sizeof(E) == 2 ? 2 : 1) void chunk_prep_kda_kernel(const E* __restrict__ q,
                                                                                     const E* __restrict__ k,
                                                                                     const E* __restrict__ v,
                                                                                     const E* __restrict__ beta,
                                                                                     const E* __restrict__ g,
                                                                                     char* __restrict__ ws, int T,
                                                                                     int nchunks, HeadMap hm,
                                                                                     const int2* __restrict__ ctab) {
    __shared__ KdaPrepLds<E, DK, DV> lds;
    const long item = blockIdx.x;
    const long bh = item / nchunks;
    long tok0, tokk;
    int L;
    if constexpr (VARLEN) {
        // packed sequences: item = head * nchunks + global chunk, the chunk's
        // first token and length from the chunk table (length 0: unused slot)
        const int2 e = ctab[item % nchunks];
        if (e.y == 0) return;
        tok0 = tokk = bh * T + e.x;
        L = e.y;
    } else {
        const int t0 = (int)(item % nchunks) * CHUNK;
        tok0 = bh * T + t0;
        tokk = hm.key(bh) * T + t0;
        L = min(CHUNK, T - t0);
    }
    kda_prep4_item<E, DK, DV>(q, k, v, beta, g, ws + item * WsLayout<E, DK, DV>::BYTES, lds, tok0, tokk, L,
                              (int)(threadIdx.x >> 6), (int)(threadIdx.x & 63));
}

template <typename E, int D>
hipError_t launch_kda_prep(const void* q, const void* k, const void* v, const void* beta, const void* g,
                           void* ws, long nitems, int T, int nchunks, HeadMap hm, const void* ctab,
                           hipStream_t st) {
    if (ctab)
        hipLaunchKernelGGL((chunk_prep_kda_kernel<E, D, D, true>), dim3((unsigned)nitems), dim3(256), 0, st,
                           (const E*)q, (const E*)k, (const E*)v, (const E*)beta, (const E*)g, (char*)ws, T,
                           nchunks, hm, (const int2*)ctab);
    else
        hipLaunchKernelGGL((chunk_prep_kda_kernel<E, D, D, false>), dim3((unsigned)nitems), dim3(256), 0, st,
                           (const E*)q, (const E*)k, (const E*)v, (const E*)beta, (const E*)g, (char*)ws, T,
                           nchunks, hm, (const int2*)nullptr);
    return hipGetLastError();
}

template hipError_t launch_kda_prep<bf16, 64>(const void*, const void*, const void*, const void*, const void*,
                                              void*, long, int, int, HeadMap, const void*, hipStream_t);
template hipError_t launch_kda_prep<bf16, 128>(const void*, const void*, const void*, const void*, const void*,
                                               void*, long, int, int, HeadMap, const void*, hipStream_t);
template hipError_t launch_kda_prep<float, 64>(const void*, const void*, const void*, const void*, const void*,
                                               void*, long, int, int, HeadMap, const void*, hipStream_t);
template hipError_t launch_kda_prep<float, 128>(const void*, const void*, const void*, const void*, const void*,
                                                void*, long, int, int, HeadMap, const void*, hipStream_t);

}  // namespace dn
