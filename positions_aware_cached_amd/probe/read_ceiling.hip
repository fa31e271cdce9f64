// read_ceiling.hip -- streaming-read ceiling of the device, for the roofline
// figures of bench.py (measurement code, not part of the decode library).
//
// A plain streaming read: every 16-byte chunk of a buffer is loaded once
// (non-temporal loads, the same kind the decode kernel uses for its key and
// value tiles), UNROLL loads in flight per lane on a grid-stride walk, and
// folded into one word per lane so nothing is optimized away.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

template <int UNROLL>
__global__ __launch_bounds__(256) void k_read(const u32x4 *__restrict__ src, uint64_t n16,
                                              uint32_t *__restrict__ sink)
{
    const uint64_t tid = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uint64_t nt = (uint64_t)gridDim.x * blockDim.x;
    uint32_t acc = 0;
    // a step covers UNROLL strides of the grid; the tail past the last full
    // step is read by the lanes it falls to, one chunk at a time
    uint64_t i = tid;
    for (; i + (UNROLL - 1) * nt < n16; i += UNROLL * nt) {
        u32x4 v[UNROLL];
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            v[u] = __builtin_nontemporal_load(src + i + u * nt);
#pragma unroll
        for (int u = 0; u < UNROLL; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n16; i += nt) {
        const u32x4 v = __builtin_nontemporal_load(src + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    sink[tid] = acc;
}

}  // namespace

// Read `bytes` (a multiple of 16, 16-byte aligned) at `src` once on `stream`
// with `blocks` work groups of 256 lanes and `unroll` (2, 4 or 8) loads in
// flight per lane; `sink` holds blocks * 256 words.  Returns a hipError_t.
extern "C" int mllm_probe_read(const void *src, uint64_t bytes, int blocks, int unroll,
                               uint32_t *sink, void *stream)
{
    if (!src || !sink || bytes % 16 != 0 || ((uintptr_t)src) % 16 != 0 || blocks < 1 ||
        blocks > 65536)
        return (int)hipErrorInvalidValue;
    const uint64_t n16 = bytes / 16;
    hipStream_t s = (hipStream_t)stream;
    if (unroll == 2)
        hipLaunchKernelGGL(k_read<2>, dim3(blocks), dim3(256), 0, s, (const u32x4 *)src, n16, sink);
    else if (unroll == 4)
        hipLaunchKernelGGL(k_read<4>, dim3(blocks), dim3(256), 0, s, (const u32x4 *)src, n16, sink);
    else if (unroll == 8)
        hipLaunchKernelGGL(k_read<8>, dim3(blocks), dim3(256), 0, s, (const u32x4 *)src, n16, sink);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}
