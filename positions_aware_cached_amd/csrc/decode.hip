// decode.hip -- gfx950 kernels of the positions-aware cached decode step.
//
// The step (microLLM-rocm ARCHITECTURE.md, "Tensor ownership boundary"):
// device positions[A] and cache_rows[A] parameterize decode RoPE, the K/V
// store and cached attention; rows not named in cache_rows stay untouched.
//
// Tuned path, two launches on one stream:
//   k_decode_fused    one wave per (entry, kv head, key split): RoPE of the
//                     queries, RoPE(K) + K/V store by the split that holds the
//                     new position, scores and P.V on the matrix cores, online
//                     FP32 softmax, per-split partial (max, sum, unnormalized
//                     output) into the workspace;
//   k_decode_merge    one wave per (entry, query head): rescales and sums the
//                     split partials (the streaming-attention merge of the
//                     IPU refactor log, "Flash vs materialized attention"),
//                     divides, rounds to BF16.
// Readable path (reference level, kept for diagnosis as the operator workflow
// asks -- operator-development.md, "Acceptance rule"):
//   k_rope_store      one block per entry: RoPE(K) + K/V store, rotated
//                     queries in FP32 into the workspace;
//   k_decode_readable one wave per (entry, query head), one key at a time.
//
// Numerics: the softmax runs in the log2 domain (scores pre-multiplied by
// log2(e)/sqrt(D), exp2), every sum is FP32, only the output is rounded.
// On the matrix cores the FP32 rotated query and the FP32 softmax weights
// enter as sums of BF16 parts (see Cols below), so the products are those of
// the FP32 values (exactly for up to 4 query heads per kv head, to 2^-16
// relative beyond) and accumulate in FP32.
#include <hip/hip_ext.h>
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

// Split-half rotation of one pair, every product and sum rounded separately
// (contraction into fused multiply-adds is switched off: the BF16 rounding of
// the result must see the same FP32 value as a separately rounded evaluation).
__device__ __forceinline__ void rope_pair(float x, float y, float c, float s, float &lo, float &hi)
{
#pragma clang fp contract(off)
    const float xc = x * c, ys = y * s, yc = y * c, xs = x * s;
    lo = xc - ys;
    hi = yc + xs;
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

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1)
        v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// ---------------------------------------------------------------- R3
//
// k_decode_fused: one wave per (entry a, kv head h, key split s).
//
// Prologue: cos/sin of the entry's position (one pair index per lane, in
// double, rounded once); the wave rotates its G query heads itself.  The wave
// that owns the split holding position pos also rotates k_new, stores K' and
// V into (row, pos) and patches its own LDS copy of that key, so the key it
// attends to is exactly the stored one.
//
// Key tiles of 16: while tile t is computed from LDS, tile t+1 is in flight in
// registers (K in matrix-core operand order, V in row order, 16 B per lane).
//   QK  v_mfma_f32_16x16x32_bf16: A = 16 keys x 32 dims of K, B = 32 dims x
//       16 columns holding the BF16 parts of the FP32 rotated query heads;
//       lane l ends with the scores of keys 4*(l/16)+i for column l%16.
//   softmax per column in FP32 (exp2 on log2(e)/sqrt(D)-scaled scores),
//       running max / sum across tiles.
//   PV  v_mfma_f32_16x16x16bf16_1k: A = V^T (16 dims x 16 keys) read with
//       ds_read_b64_tr_b16 from the row-major LDS tile, B = the BF16 parts of
//       the FP32 weights in the same columns; FP32 accumulators O^T[d][col].
//
// Operand columns: part q (hi / mid / lo BF16 part) of head g sits in column
// q*GS + g (GCLS <= 8, one column group) or column g of group q (GCLS 16).
// Three parts reproduce an FP32 value exactly (GCLS <= 4); two parts carry
// it to 2^-16 relative (GCLS 8, 16).
template <int GCLS>
struct Cols {
    static constexpr int GS = GCLS;
    static constexpr int NPART = GCLS <= 4 ? 3 : 2;
    static constexpr int NGRP = GCLS == 16 ? 2 : 1;
};

typedef __attribute__((ext_vector_type(4))) short s16x4;

// 2^x for x <= HEADROOM or -inf (the softmax weights): the hardware exp2.
// Its result for arguments below -126 is flushed to zero, which only drops
// weights under 2^-126 of the running maximum.
__device__ __forceinline__ float exp2_nonpos(float x) { return __builtin_amdgcn_exp2f(x); }

// BF16 part `part` of x: with three parts hi + mid + lo == x exactly (each
// remainder is exact and the last has at most 8 significant bits); with two
// parts the remainder is rounded to nearest.
template <int NPART>
__device__ __forceinline__ uint32_t bf16_part(float x, int part)
{
    const uint32_t hi = __float_as_uint(x) & 0xffff0000u;
    if (part == 0)
        return hi >> 16;
    const float r1 = x - __uint_as_float(hi);
    if (NPART == 2)
        return f2bf(r1);
    const uint32_t mid = __float_as_uint(r1) & 0xffff0000u;
    if (part == 1)
        return mid >> 16;
    const float r2 = r1 - __uint_as_float(mid);
    return __float_as_uint(r2) >> 16;
}

#ifndef MLLM_DECODE_WAVES_PER_SIMD
#define MLLM_DECODE_WAVES_PER_SIMD 2
#endif
template <int D, int GCLS>
__global__ __launch_bounds__(64, GCLS == 16 ? 1 : MLLM_DECODE_WAVES_PER_SIMD) void k_decode_fused(DecodeParams p)
{
    using CL = Cols<GCLS>;
    constexpr int GS = CL::GS, NPART = CL::NPART, NGRP = CL::NGRP;
    constexpr int KS = D / 32;             // QK k-steps (32 dims each)
    constexpr int NDB = D / 16;            // PV dim blocks (16 dims each)
    constexpr int TK = 32;                 // keys per tile
    constexpr int NB = TK / 16;            // 16-key MFMA row blocks per tile
    constexpr int LPK = D / 8;             // lanes per key row (16 B each)
    constexpr int KPI = 64 / LPK;          // key rows per V load instruction
    constexpr int VLD = TK / KPI;          // V load instructions per tile
    constexpr int VROW = D * 2 + 16;       // padded LDS row of V, bytes
    constexpr float HEADROOM = 8.0f;       // log2 growth of a column max before O is rescaled

    const int s = blockIdx.x, h = blockIdx.y, a = blockIdx.z;
    const int lane = threadIdx.x, n = lane & 15, lg = lane >> 4;
    const int pos = p.positions[a], row = p.rows[a];
    const int G = p.G;
    if (!entry_valid(p, pos, row)) {
        if (s == 0 && h == 0 && lane == 0 && p.status)
            p.status[0] = 1;
        return;
    }
    const int nkeys = pos + 1;
    const int j0 = s * p.kps;
    if (j0 >= nkeys)
        return;
    const int j1 = min(nkeys, j0 + p.kps);

    __shared__ float cs[D / 2], sn[D / 2];
    __shared__ __attribute__((aligned(16))) unsigned char klds[TK * D * 2];
    __shared__ __attribute__((aligned(16))) unsigned char vlds[TK * VROW];
    __shared__ __attribute__((aligned(16))) uint16_t newk[D], newv[D];  // the new token

    const size_t slot = (size_t)p.Hkv * D;
    const size_t rbase = (size_t)row * p.C * slot + (size_t)h * D;
    const unsigned char *kb = (const unsigned char *)(p.kc + rbase);
    const unsigned char *vb = (const unsigned char *)(p.vc + rbase);
    const uint32_t slotb = (uint32_t)(slot * 2);  // bytes per position; a row fits in 2^31

    // ---- tile staging: registers (in flight) -> LDS (computed)
    u32x4 kn[NB][KS], vn[VLD];
    auto load_tile = [&](int jt) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint32_t off = (uint32_t)min(jt + b * 16 + n, j1 - 1) * slotb + lg * 16;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kn[b][ks] = *(const u32x4 *)(kb + off + ks * 64);
        }
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const uint32_t off = (uint32_t)min(jt + i * KPI + lane / LPK, j1 - 1) * slotb +
                                 (lane % LPK) * 16;
            vn[i] = *(const u32x4 *)(vb + off);
        }
    };
    load_tile(j0);  // first tile in flight during the prologue below

    if (lane < D / 2) {
        const float theta = __fmul_rn((float)pos, p.inv_freq[lane]);
        cs[lane] = (float)cos((double)theta);
        sn[lane] = (float)sin((double)theta);
    }
    __syncthreads();


    // ---- the new token: rotate k_new, store K' and V (split holding pos only)
    const bool owner = j1 == nkeys;
    if (owner) {
        if (lane < D / 2) {
            const uint16_t *k = p.k_new + a * p.kn_sa + h * p.kn_sh;
            float lo, hi;
            rope_pair(bf2f(k[lane]), bf2f(k[lane + D / 2]), cs[lane], sn[lane], lo, hi);
            const uint16_t klo = (uint16_t)f2bf(lo), khi = (uint16_t)f2bf(hi);
            uint16_t *kd = p.kc + rbase + (size_t)pos * slot;
            kd[lane] = klo;
            kd[lane + D / 2] = khi;
            newk[lane] = klo;
            newk[lane + D / 2] = khi;
        }
        if (lane < LPK) {
            const u32x4 v = *(const u32x4 *)(p.v_new + a * p.vn_sa + h * p.vn_sh + lane * 8);
            *(u32x4 *)(p.vc + rbase + (size_t)pos * slot + lane * 8) = v;
            *(u32x4 *)(newv + lane * 8) = v;
        }
    }

    // ---- B operands of QK: BF16 parts of the rotated query, by column
    bf16x8 bq[NGRP][KS];
    const int chead = NGRP == 1 ? n % GS : n;   // head of this lane's column
    const int cpart = NGRP == 1 ? n / GS : 0;   // part of this lane's column (one group)
    const bool ccol = chead < G && (NGRP == 2 || cpart < NPART);
    {
        float qv[KS][8];
        const uint16_t *qs = p.q + a * p.q_sa + (h * G + (ccol ? chead : 0)) * p.q_sh;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const u32x4 w = *(const u32x4 *)(qs + ks * 32 + lg * 8);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                qv[ks][2 * e] = bf_lo(w[e]);
                qv[ks][2 * e + 1] = bf_hi(w[e]);
            }
        }
#pragma unroll
        for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int i = ks * 32 + lg * 8 + j;
                float lo, hi;
                rope_pair(qv[ks][j], qv[ks + KS / 2][j], cs[i], sn[i], lo, hi);
                qv[ks][j] = lo;
                qv[ks + KS / 2][j] = hi;
            }
#pragma unroll
        for (int c = 0; c < NGRP; ++c) {
            const int part = NGRP == 1 ? min(cpart, NPART - 1) : c;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 w;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t b0 = ccol ? bf16_part<NPART>(qv[ks][2 * e], part) : 0u;
                    const uint32_t b1 = ccol ? bf16_part<NPART>(qv[ks][2 * e + 1], part) : 0u;
                    w[e] = b0 | (b1 << 16);
                }
                bq[c][ks] = __builtin_bit_cast(bf16x8, w);
            }
        }
    }

    auto store_tile = [&](int jt) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                *(u32x4 *)(klds + (b * KS + ks) * 1024 + lane * 16) = kn[b][ks];
#pragma unroll
        for (int i = 0; i < VLD; ++i)
            *(u32x4 *)(vlds + (i * KPI + lane / LPK) * VROW + (lane % LPK) * 16) = vn[i];
        if (owner && pos >= jt && pos < jt + TK) {
            // the key just stored: overwrite the stale copy that was loaded
            const int kk = pos - jt, b = kk >> 4, m = kk & 15;
            if (lane < LPK) {
                // 16-B chunk c = lane of the key: K operand slot (ks, lg) = (c / 4, c % 4)
                *(u32x4 *)(klds + (b * KS + (lane >> 2)) * 1024 + (m + 16 * (lane & 3)) * 16) =
                    *(const u32x4 *)(newk + lane * 8);
                *(u32x4 *)(vlds + kk * VROW + lane * 16) = *(const u32x4 *)(newv + lane * 8);
            }
            // keys past pos were clamped to pos and hold its stale bytes: they
            // carry zero weight, so give them zero values (0 * stale NaN = NaN)
            for (int idx = lane; idx < (TK - 1 - kk) * LPK; idx += 64)
                *(u32x4 *)(vlds + (kk + 1 + idx / LPK) * VROW + (idx % LPK) * 16) =
                    u32x4{0u, 0u, 0u, 0u};
        }
    };

    float m_run = -INFINITY, l_run = 0.0f;
    f32x4 O[NGRP][NDB];
#pragma unroll
    for (int c = 0; c < NGRP; ++c)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
            O[c][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    store_tile(j0);
    __syncthreads();
    for (int jt = j0; jt < j1; jt += TK) {
        const bool more = jt + TK < j1;
        if (more)
            load_tile(jt + TK);

        // QK: lane (n, lg) gets keys jt + 16 b + 4 lg + i of column n
        f32x4 acc[NB][NGRP];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int c = 0; c < NGRP; ++c)
                acc[b][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                const u32x4 kf = *(const u32x4 *)(klds + (b * KS + ks) * 1024 + lane * 16);
#pragma unroll
                for (int c = 0; c < NGRP; ++c)
                    acc[b][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        __builtin_bit_cast(bf16x8, kf), bq[c][ks], acc[b][c], 0, 0, 0);
            }
        float sc[NB][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v;
                if (NGRP == 1) {
                    v = 0.0f;
#pragma unroll
                    for (int q = 0; q < NPART; ++q)
                        v += __shfl(acc[b][0][i], lg * 16 + min(chead + q * GS, 15), 64);
                } else {
                    v = acc[b][0][i] + acc[b][1][i];
                }
                v = (jt + b * 16 + lg * 4 + i < j1) ? v * p.scale_log2 : -INFINITY;
                sc[b][i] = v;
                tmax = fmaxf(tmax, v);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        // the running max moves only when a column max grows past the headroom;
        // weights stay <= 2^HEADROOM and O is rescaled rarely
        const bool grow = tmax > m_run + HEADROOM;
        if (__any(grow)) {
            const float m_new = grow ? tmax : m_run;
            const float alpha = exp2_nonpos(m_run - m_new);
            l_run *= alpha;
#pragma unroll
            for (int c = 0; c < NGRP; ++c)
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    O[c][db] *= alpha;
            m_run = m_new;
        }
        float pv[NB][4];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                pv[b][i] = ccol ? exp2_nonpos(sc[b][i] - m_run) : 0.0f;
                l_run += pv[b][i];
            }

        // PV: k slot j < 4 is key 4 lg + j of block 0, slot 4 + j of block 1
        bf16x8 pb[NGRP];
#pragma unroll
        for (int c = 0; c < NGRP; ++c) {
            const int part = NGRP == 1 ? min(cpart, NPART - 1) : c;
            u32x4 w;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int b = e >> 1, i = (e & 1) * 2;
                w[e] = bf16_part<NPART>(pv[b][i], part) | (bf16_part<NPART>(pv[b][i + 1], part) << 16);
            }
            pb[c] = __builtin_bit_cast(bf16x8, w);
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int col = (db * 16 + 4 * (n & 3)) * 2;
            const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(vlds + (lg * 4 + (n >> 2)) * VROW + col));
            const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)(vlds + (16 + lg * 4 + (n >> 2)) * VROW +
                                                            col));
            const s16x4 vv[2] = {v0, v1};
            const bf16x8 vt = __builtin_bit_cast(bf16x8, vv);
#pragma unroll
            for (int c = 0; c < NGRP; ++c)
                O[c][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vt, pb[c], O[c][db], 0, 0, 0);
        }
        __syncthreads();
        if (more) {
            store_tile(jt + TK);
            __syncthreads();
        }
    }

    // ---- per-split partial: reference max, sum and unnormalized output per head
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    const size_t base = ((size_t)a * p.Hq + (size_t)h * G) * p.NS;
    const bool writer = n < G;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
        f32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float v;
            if (NGRP == 1) {
                v = 0.0f;
#pragma unroll
                for (int q = 0; q < NPART; ++q)
                    v += __shfl(O[0][db][i], lg * 16 + min(n + q * GS, 15), 64);
            } else {
                v = O[0][db][i] + O[1][db][i];
            }
            o[i] = v;
        }
        if (writer)
            *(f32x4 *)(p.part_o + (base + (size_t)n * p.NS + s) * D + db * 16 + lg * 4) = o;
    }
    if (writer && lg == 0) {
        float *dst = p.part_ml + (base + (size_t)n * p.NS + s) * 2;
        dst[0] = m_run;
        dst[1] = l_run;
    }
}


// ---------------------------------------------------------------- R4
// One wave per (entry, query head): lanes read the split statistics in
// parallel, the unnormalized split outputs are summed with weights
// 2^(m_s - M) (loads issued four splits at a time), divided by the weighted
// sum of l_s and rounded to BF16.
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
    for (int c = lane; c < ns; c += 64)
        M = fmaxf(M, ml[2 * c]);
    M = wave_max(M);
    float lw = 0.0f, O[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e)
        O[e] = 0.0f;
    for (int c = 0; c < ns; c += 64) {
        float w = 0.0f;
        if (c + lane < ns) {
            w = exp2f(ml[2 * (c + lane)] - M);
            lw += w * ml[2 * (c + lane) + 1];
        }
        const int cnt = min(64, ns - c);
        int k = 0;
        for (; k + 4 <= cnt; k += 4) {
            float wk[4], x[4][PER];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                wk[u] = __shfl(w, k + u, 64);
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    x[u][e] = po[(size_t)(c + k + u) * D + lane + 64 * e];
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    O[e] += wk[u] * x[u][e];
        }
        for (; k < cnt; ++k) {
            const float wk = __shfl(w, k, 64);
#pragma unroll
            for (int e = 0; e < PER; ++e)
                O[e] += wk * po[(size_t)(c + k) * D + lane + 64 * e];
        }
    }
    const float L = wave_sum(lw);
#pragma unroll
    for (int e = 0; e < PER; ++e)
        out[lane + 64 * e] = (uint16_t)f2bf(O[e] / L);
}

}  // namespace

DecodeWorkspace decode_workspace_layout(int64_t A, int64_t Hq, int64_t Hkv, int64_t D,
                                        int64_t NS)
{
    auto up = [](uint64_t x) { return (x + 255u) & ~uint64_t(255); };
    DecodeWorkspace w;
    w.qrot_off = 0;
    w.part_o_off = up(w.qrot_off + (uint64_t)A * Hq * D * 4);
    w.part_ml_off = up(w.part_o_off + (uint64_t)A * Hq * NS * D * 4);
    w.total = up(w.part_ml_off + (uint64_t)A * Hq * NS * 2 * 4);
    (void)Hkv;
    return w;
}

hipError_t launch_rope_store(const DecodeParams &p, hipStream_t stream)
{
    hipLaunchKernelGGL(k_rope_store, dim3(p.A), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_fused_d(const DecodeParams &p, hipStream_t stream, hipEvent_t e0,
                                 hipEvent_t e1)
{
    const dim3 grid(p.NS, p.Hkv, p.A), block(64);
    if (p.G <= 1)
        hipExtLaunchKernelGGL((k_decode_fused<D, 1>), grid, block, 0, stream, e0, e1, 0, p);
    else if (p.G <= 2)
        hipExtLaunchKernelGGL((k_decode_fused<D, 2>), grid, block, 0, stream, e0, e1, 0, p);
    else if (p.G <= 4)
        hipExtLaunchKernelGGL((k_decode_fused<D, 4>), grid, block, 0, stream, e0, e1, 0, p);
    else if (p.G <= 8)
        hipExtLaunchKernelGGL((k_decode_fused<D, 8>), grid, block, 0, stream, e0, e1, 0, p);
    else
        hipExtLaunchKernelGGL((k_decode_fused<D, 16>), grid, block, 0, stream, e0, e1, 0, p);
    return hipGetLastError();
}

hipError_t launch_decode_fused(const DecodeParams &p, hipStream_t stream, hipEvent_t e0,
                               hipEvent_t e1)
{
    return p.D == 64 ? launch_fused_d<64>(p, stream, e0, e1)
                     : launch_fused_d<128>(p, stream, e0, e1);
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

hipError_t launch_decode_readable(const DecodeParams &p, hipStream_t stream, hipEvent_t e0,
                                  hipEvent_t e1)
{
    const dim3 grid(p.Hq, p.A), block(64);
    if (p.D == 64)
        hipExtLaunchKernelGGL(k_decode_readable<64>, grid, block, 0, stream, e0, e1, 0, p);
    else
        hipExtLaunchKernelGGL(k_decode_readable<128>, grid, block, 0, stream, e0, e1, 0, p);
    return hipGetLastError();
}

}  // namespace mllm
