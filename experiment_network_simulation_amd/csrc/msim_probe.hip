/* LDS read-bandwidth probe: the peak against which the LDS-resident
 * simulation kernels are priced.
 *
 * Each workgroup of 1,024 threads fills a 64 KiB LDS buffer, then every lane
 * reads 16-byte words in a lane-consecutive (bank-conflict-free) pattern,
 * eight reads per loop iteration from a start that moves every iteration so
 * no read can be hoisted.  Each word read is handed to an empty register-use
 * statement, which forces the read to complete without spending vector ALU
 * instructions on it, and one word per thread is written out at the end.
 * Bytes read per launch = blocks x 1,024 x iters x 8 x 16.  Two such
 * workgroups fit a CU's 160 KiB of LDS.
 */

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "msim.h"

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

#define PROBE_THREADS 1024u
#define PROBE_WORDS 4096u          /* 16-byte words: 64 KiB */

extern "C" __global__ void __launch_bounds__(1024) msim_lds_read_probe(uint32_t *out, uint32_t iters)
{
    __shared__ u32x4 buf[PROBE_WORDS];
    const uint32_t tid = threadIdx.x;
    for (uint32_t i = tid; i < PROBE_WORDS; i += PROBE_THREADS)
        buf[i] = u32x4{i, i * 3u + 1u, i * 5u + 2u, i * 7u + 3u};
    __syncthreads();
    /* the start stays below 2,048 words and the eight reads lie 256 words
     * apart, so every address is the start plus an immediate offset */
    uint32_t idx = tid & (PROBE_WORDS / 2 - 1);
    u32x4 v0 = {0, 0, 0, 0}, v1 = v0, v2 = v0, v3 = v0, v4 = v0, v5 = v0, v6 = v0, v7 = v0;
    for (uint32_t it = 0; it < iters; it++) {
        /* eight reads in flight together, one register group each */
        const u32x4 *b = buf + idx;
        v0 = b[0]; v1 = b[256]; v2 = b[512]; v3 = b[768];
        v4 = b[1024]; v5 = b[1280]; v6 = b[1536]; v7 = b[1792];
        asm volatile("" ::"v"(v0), "v"(v1), "v"(v2), "v"(v3), "v"(v4), "v"(v5), "v"(v6), "v"(v7));
        idx = (idx + 64u) & (PROBE_WORDS / 2 - 1);
    }
    const u32x4 last = v0 ^ v7;
    out[blockIdx.x * PROBE_THREADS + tid] = last.x ^ last.y ^ last.z ^ last.w;
}

extern "C" int msim_lds_probe(void *dev_out, uint64_t out_bytes, uint32_t blocks, uint32_t iters, void *hip_stream)
{
    if (!dev_out || blocks == 0 || blocks > (1u << 20) || iters == 0 ||
        out_bytes < (uint64_t)blocks * PROBE_THREADS * sizeof(uint32_t))
        return MSIM_E_ARG;
    hipLaunchKernelGGL(msim_lds_read_probe, dim3(blocks), dim3(PROBE_THREADS), 0, (hipStream_t)hip_stream,
                       (uint32_t *)dev_out, iters);
    return hipGetLastError() == hipSuccess ? MSIM_OK : MSIM_E_HIP;
}
