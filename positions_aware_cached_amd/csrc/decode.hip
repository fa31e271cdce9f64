// decode.hip -- gfx950 kernels of the positions-aware cached decode step.
//
// The step (microLLM-rocm ARCHITECTURE.md, "Tensor ownership boundary"):
// device positions[A] and cache_rows[A] parameterize decode RoPE, the K/V
// store and cached attention; rows not named in cache_rows stay untouched.
//
// Kernels, launched in this order on one stream:
//   k_rope_store      one block per entry: split-half RoPE of k_new stored as
//                     BF16 at (row, pos), v_new copied bit for bit, rotated
//                     queries kept in FP32 in the workspace.
//   k_decode_split    one wave per (entry, kv head, key split): scores on the
//                     matrix cores, online FP32 softmax, FP32 P.V, per-split
//                     partial (max, sum, unnormalized output).
//   k_decode_merge    one wave per (entry, query head): rescales and sums the
//                     split partials (the streaming-attention merge of the
//                     IPU refactor log, "Flash vs materialized attention"),
//                     divides, rounds to BF16.
//   k_decode_readable the plain reference-level kernel (one wave per
//                     (entry, query head), one key at a time), kept for
//                     diagnosis as the operator workflow asks
//                     (operator-development.md, "Acceptance rule").
//
// Numerics: the softmax runs in the log2 domain (scores pre-multiplied by
// log2(e)/sqrt(D), exp2), every sum is FP32, only the output is rounded.
// On the matrix cores the FP32 rotated query enters as the exact sum of three
// BF16 parts (hi + mid + lo == q exactly), so each product q_d * k_d is exact
// and accumulates in FP32: no rounding of the query is introduced.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace mllm {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// FP32 -> BF16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f2bf(float f)
{
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x7fffffu))
        return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Split-half rotation of one pair, every product and sum rounded separately.
__device__ __forceinline__ void rope_pair(float x, float y, float c, float s, float &lo, float &hi)
{
    lo = __fsub_rn(__fmul_rn(x, c), __fmul_rn(y, s));
    hi = __fadd_rn(__fmul_rn(y, c), __fmul_rn(x, s));
}

__device__ __forceinline__ bool entry_valid(const DecodeParams &p, int pos, int row)
{
    return pos >= 0 && pos < p.C && row >= 0 && row < p.S;
}

// ---------------------------------------------------------------- R1
__global__ __launch_bounds__(256) void k_rope_store(DecodeParams p)
{
    const int a = blockIdx.x;
    const int t = threadIdx.x;
    const int pos = p.positions[a];
    const int row = p.rows[a];
    if (!entry_valid(p, pos, row)) {
        if (t == 0 && p.status)
            p.status[0] = 1;
        return;
    }
    const int D = p.D, H = D / 2;
    __shared__ float cs[kMaxHalfDim], sn[kMaxHalfDim];
    if (t < H) {
        // angle = fl32(fl32(pos) * inv_freq[i]); cos/sin evaluated in double
        float theta = __fmul_rn((float)pos, p.inv_freq[t]);
        cs[t] = (float)cos((double)theta);
        sn[t] = (float)sin((double)theta);
    }
    __syncthreads();

    const size_t slot = (size_t)p.Hkv * D;
    const size_t dst = ((size_t)row * p.C + pos) * slot;
    for (int idx = t; idx < p.Hkv * H; idx += blockDim.x) {
        const int h = idx / H, i = idx - h * H;
        const uint16_t *k = p.k_new + a * p.kn_sa + h * p.kn_sh;
        float lo, hi;
        rope_pair(bf2f(k[i]), bf2f(k[i + H]), cs[i], sn[i], lo, hi);
        uint16_t *kd = p.kc + dst + (size_t)h * D;
        kd[i] = (uint16_t)f2bf(lo);
        kd[i + H] = (uint16_t)f2bf(hi);
    }
    const int chunks = D / 8;
    for (int idx = t; idx < p.Hkv * chunks; idx += blockDim.x) {
        const int h = idx / chunks, c = idx - h * chunks;
        const u32x4 v = *(const u32x4 *)(p.v_new + a * p.vn_sa + h * p.vn_sh + c * 8);
        *(u32x4 *)(p.vc + dst + (size_t)h * D + c * 8) = v;
    }
    for (int idx = t; idx < p.Hq * H; idx += blockDim.x) {
        const int hq = idx / H, i = idx - hq * H;
        const uint16_t *q = p.q + a * p.q_sa + hq * p.q_sh;
        float lo, hi;
        rope_pair(bf2f(q[i]), bf2f(q[i + H]), cs[i], sn[i], lo, hi);
        float *qr = p.qrot + ((size_t)a * p.Hq + hq) * D;
        qr[i] = lo;
        qr[i + H] = hi;
    }
}

// ---------------------------------------------------------------- R2
__device__ __forceinline__ float wave_sum(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v += __shfl_xor(v, o, 64);
    return v;
}

template <int D>
__global__ __launch_bounds__(64) void k_decode_readable(DecodeParams p)
{
    constexpr int PER = D / 64;
    const int hq = blockIdx.x, a = blockIdx.y, lane = threadIdx.x;
    const int pos = p.positions[a], row = p.rows[a];
    uint16_t *out = p.out + a * p.o_sa + hq * p.o_sh;
    if (!entry_valid(p, pos, row)) {
#pragma unroll
        for (int e = 0; e < PER; ++e)
            out[lane + 64 * e] = 0x7fc0;
        return;
    }
    const int kv = hq / p.G;
    const size_t slot = (size_t)p.Hkv * D;
    const uint16_t *K = p.kc + (size_t)row * p.C * slot + (size_t)kv * D;
    const uint16_t *V = p.vc + (size_t)row * p.C * slot + (size_t)kv * D;
    const float *qr = p.qrot + ((size_t)a * p.Hq + hq) * D;
    float q[PER], o[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        q[e] = qr[lane + 64 * e];
        o[e] = 0.0f;
    }
    float m = -INFINITY, l = 0.0f;
    for (int j = 0; j <= pos; ++j) {
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < PER; ++e)
            part += q[e] * bf2f(K[j * slot + lane + 64 * e]);
        const float s = wave_sum(part) * p.scale_log2;
        const float mn = fmaxf(m, s);
        const float corr = exp2f(m - mn);
        const float pj = exp2f(s - mn);
        l = l * corr + pj;
#pragma unroll
        for (int e = 0; e < PER; ++e)
            o[e] = o[e] * corr + pj * bf2f(V[j * slot + lane + 64 * e]);
        m = mn;
    }
#pragma unroll
    for (int e = 0; e < PER; ++e)
        out[lane + 64 * e] = (uint16_t)f2bf(o[e] / l);
}

// ---------------------------------------------------------------- R3
//
// One wave per (entry a, kv head h, split s).  The split's keys are visited in
// tiles of 32.  Per tile:
//   QK on the matrix cores: v_mfma_f32_16x16x32_bf16 with A = 16 keys x 32
//      dims of K (lane l: key l%16, dims 8*(l/16)..+7 of the k-step, loaded
//      straight from the cache row), B = 32 dims x 16 columns of the rotated
//      query, column n = query head n of the group; the three BF16 parts of
//      the FP32 query accumulate into one FP32 tile.  Lane l then holds the
//      scores of keys 4*(l/16)+i, i < 4, for head l%16.
//   softmax: tile max per head across the four row groups, running max,
//      exp2, running sum; the weights go through LDS as p[key][head].
//   PV on the vector ALUs in FP32: lane l owns 8 dims (l % (D/8)) of one key
//      slot (l / (D/8)); V rows are read coalesced along D (16 B per lane).
template <int D, int GP>
__global__ __launch_bounds__(64) void k_decode_split(DecodeParams p)
{
    constexpr int KS = D / 32;      // MFMA k-steps over the head dimension
    constexpr int LPK = D / 8;      // lanes per key in the P.V layout
    constexpr int KPS = 64 / LPK;   // keys per P.V step
    constexpr int TK = 32;          // keys per tile
    constexpr int NBLK = TK / 16;   // 16-key MFMA blocks per tile
    constexpr int NST = TK / KPS;   // P.V steps per tile

    const int s = blockIdx.x, h = blockIdx.y, a = blockIdx.z;
    const int lane = threadIdx.x;
    const int pos = p.positions[a], row = p.rows[a];
    if (!entry_valid(p, pos, row))
        return;
    const int nkeys = pos + 1;
    const int j0 = s * p.kps;
    if (j0 >= nkeys)
        return;
    const int j1 = min(nkeys, j0 + p.kps);
    const int G = p.G;

    __shared__ float p_lds[TK * GP];
    __shared__ float alpha_lds[GP];

    const int n = lane & 15, grp = lane >> 4;

    // B operands: three BF16 parts of the rotated query, column n = head n.
    bf16x8 bq[3][KS];
    {
        const float *qr = p.qrot + ((size_t)a * p.Hq + (size_t)h * G + n) * D;
        const bool live = n < G;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            u32x4 w[3];
#pragma unroll
            for (int j = 0; j < 8; j += 2) {
                uint32_t b0[3], b1[3];
#pragma unroll
                for (int half = 0; half < 2; ++half) {
                    const float x = live ? qr[ks * 32 + grp * 8 + j + half] : 0.0f;
                    const uint32_t hi = __float_as_uint(x) & 0xffff0000u;
                    const float r1 = x - __uint_as_float(hi);
                    const uint32_t mid = __float_as_uint(r1) & 0xffff0000u;
                    const float r2 = r1 - __uint_as_float(mid);
                    const uint32_t lo = __float_as_uint(r2) & 0xffff0000u;
                    uint32_t *dst = half ? b1 : b0;
                    dst[0] = hi >> 16;
                    dst[1] = mid >> 16;
                    dst[2] = lo >> 16;
                }
#pragma unroll
                for (int part = 0; part < 3; ++part)
                    w[part][j / 2] = b0[part] | (b1[part] << 16);
            }
#pragma unroll
            for (int part = 0; part < 3; ++part)
                bq[part][ks] = __builtin_bit_cast(bf16x8, w[part]);
        }
    }

    const size_t slot = (size_t)p.Hkv * D;
    const uint16_t *kbase = p.kc + (size_t)row * p.C * slot + (size_t)h * D;
    const uint16_t *vbase = p.vc + (size_t)row * p.C * slot + (size_t)h * D;
    const int kq = lane / LPK, dc = lane % LPK;

    float m_run = -INFINITY, l_run = 0.0f;
    float o[GP][8];
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e)
            o[g][e] = 0.0f;

    for (int jt = j0; jt < j1; jt += TK) {
        u32x4 kreg[NBLK][KS];
        u32x4 vreg[NST];
#pragma unroll
        for (int b = 0; b < NBLK; ++b) {
            const int key = min(jt + b * 16 + n, j1 - 1);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kreg[b][ks] = *(const u32x4 *)(kbase + (size_t)key * slot + ks * 32 + grp * 8);
        }
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            const int key = min(jt + st * KPS + kq, j1 - 1);
            vreg[st] = *(const u32x4 *)(vbase + (size_t)key * slot + dc * 8);
        }

        // scores
        float sc[NBLK][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int b = 0; b < NBLK; ++b) {
            f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int part = 0; part < 3; ++part)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks)
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, kreg[b][ks]), bq[part][ks], acc, 0, 0, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = jt + b * 16 + grp * 4 + i;
                const float v = key < j1 ? acc[i] * p.scale_log2 : -INFINITY;
                sc[b][i] = v;
                tmax = fmaxf(tmax, v);
            }
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m_run, tmax);
        const float alpha = exp2f(m_run - m_new);
        float psum = 0.0f;
#pragma unroll
        for (int b = 0; b < NBLK; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pv = exp2f(sc[b][i] - m_new);
                psum += pv;
                if (n < GP)
                    p_lds[(b * 16 + grp * 4 + i) * GP + n] = pv;
            }
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if (grp == 0 && n < GP)
            alpha_lds[n] = alpha;
        __syncthreads();

        float al[GP];
#pragma unroll
        for (int g = 0; g < GP; ++g)
            al[g] = alpha_lds[g];
#pragma unroll
        for (int g = 0; g < GP; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                o[g][e] *= al[g];
#pragma unroll
        for (int st = 0; st < NST; ++st) {
            const int kk = st * KPS + kq;
            float v[8];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                v[2 * w] = bf_lo(vreg[st][w]);
                v[2 * w + 1] = bf_hi(vreg[st][w]);
            }
#pragma unroll
            for (int g = 0; g < GP; ++g) {
                const float pg = p_lds[kk * GP + g];
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    o[g][e] += pg * v[e];
            }
        }
        __syncthreads();
    }

    // sum over the four row groups (l) and over the key slots (o)
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
#pragma unroll
    for (int g = 0; g < GP; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float v = o[g][e];
#pragma unroll
            for (int off = LPK; off < 64; off <<= 1)
                v += __shfl_xor(v, off, 64);
            o[g][e] = v;
        }

    const size_t base = ((size_t)a * p.Hq + (size_t)h * G) * p.NS + s;
    if (kq == 0) {
#pragma unroll
        for (int g = 0; g < GP; ++g) {
            if (g < G) {
                float *dst = p.part_o + (base + (size_t)g * p.NS) * D + dc * 8;
                *(f32x4 *)dst = f32x4{o[g][0], o[g][1], o[g][2], o[g][3]};
                *(f32x4 *)(dst + 4) = f32x4{o[g][4], o[g][5], o[g][6], o[g][7]};
            }
        }
    }
    if (grp == 0 && n < G) {
        float *dst = p.part_ml + (base + (size_t)n * p.NS) * 2;
        dst[0] = m_run;
        dst[1] = l_run;
    }
}

// ---------------------------------------------------------------- R4
template <int D>
__global__ __launch_bounds__(64) void k_decode_merge(DecodeParams p)
{
    constexpr int PER = D / 64;
    const int hq = blockIdx.x, a = blockIdx.y, lane = threadIdx.x;
    const int pos = p.positions[a], row = p.rows[a];
    uint16_t *out = p.out + a * p.o_sa + hq * p.o_sh;
    if (!entry_valid(p, pos, row)) {
#pragma unroll
        for (int e = 0; e < PER; ++e)
            out[lane + 64 * e] = 0x7fc0;
        return;
    }
    const int ns = (pos + p.kps) / p.kps;
    const size_t base = ((size_t)a * p.Hq + hq) * p.NS;
    const float *ml = p.part_ml + base * 2;
    const float *po = p.part_o + base * D;
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s)
        M = fmaxf(M, ml[2 * s]);
    float L = 0.0f, O[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e)
        O[e] = 0.0f;
    for (int s = 0; s < ns; ++s) {
        const float w = exp2f(ml[2 * s] - M);
        L += w * ml[2 * s + 1];
#pragma unroll
        for (int e = 0; e < PER; ++e)
            O[e] += w * po[(size_t)s * D + lane + 64 * e];
    }
#pragma unroll
    for (int e = 0; e < PER; ++e)
        out[lane + 64 * e] = (uint16_t)f2bf(O[e] / L);
}

}  // namespace

DecodeWorkspace decode_workspace_layout(int64_t A, int64_t Hq, int64_t D, int64_t NS)
{
    auto up = [](uint64_t x) { return (x + 255u) & ~uint64_t(255); };
    DecodeWorkspace w;
    w.qrot_off = 0;
    w.part_o_off = up(w.qrot_off + (uint64_t)A * Hq * D * 4);
    w.part_ml_off = up(w.part_o_off + (uint64_t)A * Hq * NS * D * 4);
    w.total = up(w.part_ml_off + (uint64_t)A * Hq * NS * 2 * 4);
    return w;
}

hipError_t launch_rope_store(const DecodeParams &p, hipStream_t stream)
{
    hipLaunchKernelGGL(k_rope_store, dim3(p.A), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_split_d(const DecodeParams &p, hipStream_t stream)
{
    const dim3 grid(p.NS, p.Hkv, p.A), block(64);
    if (p.G <= 1)
        hipLaunchKernelGGL((k_decode_split<D, 1>), grid, block, 0, stream, p);
    else if (p.G <= 2)
        hipLaunchKernelGGL((k_decode_split<D, 2>), grid, block, 0, stream, p);
    else if (p.G <= 4)
        hipLaunchKernelGGL((k_decode_split<D, 4>), grid, block, 0, stream, p);
    else if (p.G <= 8)
        hipLaunchKernelGGL((k_decode_split<D, 8>), grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL((k_decode_split<D, 16>), grid, block, 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_decode_split(const DecodeParams &p, hipStream_t stream)
{
    return p.D == 64 ? launch_split_d<64>(p, stream) : launch_split_d<128>(p, stream);
}

hipError_t launch_decode_merge(const DecodeParams &p, hipStream_t stream)
{
    const dim3 grid(p.Hq, p.A), block(64);
    if (p.D == 64)
        hipLaunchKernelGGL(k_decode_merge<64>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(k_decode_merge<128>, grid, block, 0, stream, p);
    return hipGetLastError();
}

hipError_t launch_decode_readable(const DecodeParams &p, hipStream_t stream)
{
    const dim3 grid(p.Hq, p.A), block(64);
    if (p.D == 64)
        hipLaunchKernelGGL(k_decode_readable<64>, grid, block, 0, stream, p);
    else
        hipLaunchKernelGGL(k_decode_readable<128>, grid, block, 0, stream, p);
    return hipGetLastError();
}

}  // namespace mllm
