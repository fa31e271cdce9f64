// prefill.hip -- gfx950 kernels of the equal-length batched prefill.
//
// microLLM-rocm ARCHITECTURE.md, "Tensor ownership boundary": equal-length
// pending prompts run as one batch and each prefix lands in its target empty
// shared-cache row.  Here every token's rotated K and raw V go straight to
// (row, t) -- the same bytes the page's temporary-cache-then-copy produces --
// and attention of query t covers keys 0..t of the row.
//
//   k_prefill_store     one block per (token t, entry a): split-half RoPE of
//                       k_new -> BF16 store, v_new bit copy; blocks of entry 0
//                       also write the FP32 cos/sin table row of position t.
//   k_prefill_readable  one wave per (entry, token, query head), keys one at a
//                       time, FP32 throughout (reference-level kernel).
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mllm {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint32_t f2bf(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu))
        return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void rope_pair(float x, float y, float c, float s, float &lo, float &hi)
{
    lo = __fsub_rn(__fmul_rn(x, c), __fmul_rn(y, s));
    hi = __fadd_rn(__fmul_rn(y, c), __fmul_rn(x, s));
}

// workspace: cos/sin table [T][D/2] of float2 (cos, sin)
__global__ __launch_bounds__(256) void k_prefill_store(PrefillParams p, float2 *table)
{
    const int t = blockIdx.x, a = blockIdx.y, tid = threadIdx.x;
    const int D = p.D, H = D / 2;
    __shared__ float cs[kMaxHalfDim], sn[kMaxHalfDim];
    if (tid < H) {
        float theta = __fmul_rn((float)t, p.inv_freq[tid]);
        cs[tid] = (float)cos((double)theta);
        sn[tid] = (float)sin((double)theta);
        if (a == 0)
            table[(size_t)t * H + tid] = make_float2(cs[tid], sn[tid]);
    }
    __syncthreads();
    const int row = p.rows[a];
    if (row < 0 || row >= p.S)
        return;  // device rows disagree with the checked host copy: write nothing
    const size_t slot = (size_t)p.Hkv * D;
    const size_t dst = ((size_t)row * p.C + t) * slot;
    for (int idx = tid; idx < p.Hkv * H; idx += blockDim.x) {
        const int h = idx / H, i = idx - h * H;
        const uint16_t *k = p.k_new + a * p.kn_sa + t * p.kn_st + h * p.kn_sh;
        float lo, hi;
        rope_pair(bf2f(k[i]), bf2f(k[i + H]), cs[i], sn[i], lo, hi);
        uint16_t *kd = p.kc + dst + (size_t)h * D;
        kd[i] = (uint16_t)f2bf(lo);
        kd[i + H] = (uint16_t)f2bf(hi);
    }
    const int chunks = D / 8;
    for (int idx = tid; idx < p.Hkv * chunks; idx += blockDim.x) {
        const int h = idx / chunks, c = idx - h * chunks;
        const u32x4 v = *(const u32x4 *)(p.v_new + a * p.vn_sa + t * p.vn_st + h * p.vn_sh + c * 8);
        *(u32x4 *)(p.vc + dst + (size_t)h * D + c * 8) = v;
    }
}

__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

// One wave per (a, t, hq).  Lane l owns dims l and l + 64 (D = 128) or l
// (D = 64, the partner dim l +- 32 fetched by shuffle) of the query.
template <int D>
__global__ __launch_bounds__(64) void k_prefill_readable(PrefillParams p, const float2 *table)
{
    constexpr int H = D / 2;
    const int hq = blockIdx.x, t = blockIdx.y, a = blockIdx.z, lane = threadIdx.x;
    const int row = p.rows[a];
    uint16_t *out = p.out + a * p.o_sa + t * p.o_st + hq * p.o_sh;
    if (row < 0 || row >= p.S) {
#pragma unroll
        for (int e = 0; e < D / 64; ++e)
            out[lane + 64 * e] = 0x7fc0;
        return;
    }
    const int kv = hq / p.G;
    const uint16_t *qs = p.q + a * p.q_sa + t * p.q_st + hq * p.q_sh;
    float q[D / 64];
    if (D == 128) {
        const float2 cs = table[(size_t)t * H + lane];
        rope_pair(bf2f(qs[lane]), bf2f(qs[lane + 64]), cs.x, cs.y, q[0], q[D / 64 - 1]);
    } else {
        const int i = lane & (H - 1);
        const float2 cs = table[(size_t)t * H + i];
        float lo, hi;
        rope_pair(bf2f(qs[i]), bf2f(qs[i + H]), cs.x, cs.y, lo, hi);
        q[0] = lane < H ? lo : hi;
    }
    const size_t slot = (size_t)p.Hkv * D;
    const uint16_t *K = p.kc + (size_t)row * p.C * slot + (size_t)kv * D;
    const uint16_t *V = p.vc + (size_t)row * p.C * slot + (size_t)kv * D;
    float m = -INFINITY, l = 0.0f, o[D / 64];
#pragma unroll
    for (int e = 0; e < D / 64; ++e)
        o[e] = 0.0f;
    for (int j = 0; j <= t; ++j) {
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < D / 64; ++e)
            part += q[e] * bf2f(K[j * slot + lane + 64 * e]);
        const float s = wave_sum(part) * p.scale_log2;
        const float mn = fmaxf(m, s);
        const float corr = exp2f(m - mn);
        const float pj = exp2f(s - mn);
        l = l * corr + pj;
#pragma unroll
        for (int e = 0; e < D / 64; ++e)
            o[e] = o[e] * corr + pj * bf2f(V[j * slot + lane + 64 * e]);
        m = mn;
    }
#pragma unroll
    for (int e = 0; e < D / 64; ++e)
        out[lane + 64 * e] = (uint16_t)f2bf(o[e] / l);
}

}  // namespace

uint64_t prefill_workspace_bytes(int64_t A, int64_t T, int64_t Hq, int64_t D)
{
    (void)A;
    (void)Hq;
    return ((uint64_t)T * (D / 2) * 8u + 255u) & ~uint64_t(255);
}

hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream)
{
    float2 *table = (float2 *)p.qrot;
    hipLaunchKernelGGL(k_prefill_store, dim3(p.T, p.A), dim3(256), 0, stream, p, table);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const dim3 grid(p.Hq, p.T, p.A);
    if (p.D == 64)
        hipLaunchKernelGGL(k_prefill_readable<64>, grid, dim3(64), 0, stream, p, table);
    else
        hipLaunchKernelGGL(k_prefill_readable<128>, grid, dim3(64), 0, stream, p, table);
    return hipGetLastError();
}

}  // namespace mllm
