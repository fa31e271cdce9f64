// prefill.hip -- gfx950 kernels of the batched prefill, also as a chunk
// appended at per-entry start positions with per-entry lengths.
//
// microLLM-rocm ARCHITECTURE.md, "Tensor ownership boundary": equal-length
// pending prompts run as one batch and each prefix lands in its target empty
// shared-cache row.  Here every token's rotated K and raw V go straight to
// (row, s + t) -- the same bytes the page's temporary-cache-then-copy produces
// for s = 0 -- and attention of query t covers keys 0 .. s + t of the row: the
// prefix already cached and the chunk up to itself.  Entry a uses its first n
// tokens only (prompts of different lengths in one batch); s = 0, n = T is the
// page's equal-length prefill into empty rows.
//
//   k_prefill_store     one wave per (token t, entry a): split-half RoPE of
//                       k_new -> store in the storage type, v_new bit copy; the wave also
//                       writes the FP32 cos/sin table row of its position (one
//                       row per position in an equal-length prefill).
//   k_prefill_mfma      the tuned attention: one workgroup of four waves per
//                       (entry, four query heads of a kv head, 32-query tile;
//                       fewer heads and longer tiles when G is not a multiple
//                       of four), FlashAttention-
//                       style online softmax over 64-key tiles on the matrix
//                       cores (see below).
//   k_prefill_readable  one wave per (entry, token, query head), keys one at a
//                       time, FP32 throughout (reference-level kernel, kept for
//                       diagnosis).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <utility>
#include <vector>

#include "elem.h"
#include "kernels.h"

namespace mllm {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;
typedef __attribute__((ext_vector_type(4))) short s16x4;

// One 16-B global -> LDS load per active lane: lane l's bytes land at
// lds_base + 16 l (the LDS base is wave-uniform).
__device__ __forceinline__ void lds_dma16(const void *g, void *lds_base)
{
    __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)g,
                                     (__attribute__((address_space(3))) void *)lds_base, 16, 0, 0);
}

// Lanes l and l ^ 32 exchange a value: v_permlane32_swap on two copies
// leaves the low half's values in one register and the high half's in the
// other, in every lane.  Inline assembly, because the compiler builtin handed
// back one register for both results when its two inputs were the same value;
// the s_nop gives the two wait states the instruction needs after a vector
// write of its operands.
__device__ __forceinline__ void swap_halves(float &a, float &b)
{
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

// Split-half rotation of one pair, every product and sum rounded separately
// (contraction into fused multiply-adds is switched off: the rounding of the
// result to the storage type must see the same FP32 value as a separately
// rounded evaluation).
__device__ __forceinline__ void rope_pair(float x, float y, float c, float s, float &lo, float &hi)
{
#pragma clang fp contract(off)
    const float xc = x * c, ys = y * s, yc = y * c, xs = x * s;
    lo = xc - ys;
    hi = yc + xs;
}

// Entry a's chunk: cache row, first position s and token count n.  ok is false
// when the device values disagree with the host copy the library checked.
struct Chunk {
    int row, s, n;
    bool ok;
};
__device__ __forceinline__ Chunk chunk_of(const PrefillParams &p, int a)
{
    // the three loads go out together, each from a device array (an absent
    // one reads the row array instead and its value is dropped): one memory
    // round trip
    const int32_t *sp = p.starts ? p.starts : p.rows, *lp = p.lens ? p.lens : p.rows;
    int rv = __builtin_amdgcn_readfirstlane(p.rows[a]);
    int sv = __builtin_amdgcn_readfirstlane(sp[a]), lv = __builtin_amdgcn_readfirstlane(lp[a]);
    // opaque to the compiler, so it neither waits for the row before issuing
    // the other two nor folds the choice into one load's address
    asm volatile("" : "+s"(rv), "+s"(sv), "+s"(lv));
    Chunk c;
    c.row = rv;
    c.s = p.starts ? sv : 0;
    c.n = p.lens ? lv : p.T;
    c.ok = c.row >= 0 && c.row < p.S && c.s >= 0 && c.n >= 1 && c.n <= p.T && c.s <= p.C - c.n;
    return c;
}

// Row of the cos/sin table for token t of entry a: t in an equal-length
// prefill (all entries start at position 0), a T + t in a chunk.
__device__ __forceinline__ size_t table_row(const PrefillParams &p, int a, int t)
{
    return p.starts == nullptr ? (size_t)t : (size_t)a * p.T + t;
}

// workspace: cos/sin table of float2 (cos, sin) rows of D/2 pairs, at most
// [A][T] rows (see table_row).  One wave per token: cos/sin of its D/2 angles
// once (into LDS and the table), then each lane rotates 8 pairs of a kv head
// with 16-byte loads and stores, and V moves in 16-byte chunks.
template <class E>
__global__ __launch_bounds__(64) void k_prefill_store(PrefillParams p, float2 *table)
{
    // one-dimensional grid of A * T waves (the y and z grid sizes are limited)
    const int t = (int)(blockIdx.x % (unsigned)p.T), a = (int)(blockIdx.x / (unsigned)p.T);
    const int lane = threadIdx.x;
    const int D = p.D, H = D / 2;
    const Chunk ch = chunk_of(p, a);
    // equal-length prefill: every entry holds positions 0 .. T-1, so the table
    // has one row per position, written by entry 0's waves whatever that
    // entry's own state; a chunk has a row per (entry, token)
    const bool shared = p.starts == nullptr;
    const bool store = ch.ok && t < ch.n;
    if (!store && !(shared && a == 0))
        return;  // past the entry's length, or an invalid entry: write nothing
    const int pos = shared ? t : ch.s + t;
    __shared__ float cs[kMaxHalfDim], sn[kMaxHalfDim];
    if (lane < H) {
        float theta = __fmul_rn((float)pos, p.inv_freq[lane]);
        cs[lane] = (float)cos((double)theta);
        sn[lane] = (float)sin((double)theta);
        if (!shared || a == 0)
            table[table_row(p, a, t) * H + lane] = make_float2(cs[lane], sn[lane]);
    }
    if (!store)
        return;
    __syncthreads();
    const size_t slot = (size_t)p.Hkv * D;
    const size_t dst = ((size_t)ch.row * p.C + pos) * slot;
    const int CH = H / 8;  // 16-byte chunks per half head
    for (int idx = lane; idx < p.Hkv * CH; idx += 64) {
        const int h = idx / CH, c = idx - h * CH;
        const uint16_t *k = p.k_new + a * p.kn_sa + t * p.kn_st + h * p.kn_sh + c * 8;
        const u32x4 x4 = *(const u32x4 *)k, y4 = *(const u32x4 *)(k + H);
        u32x4 lo4, hi4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int i0 = c * 8 + 2 * e, i1 = i0 + 1;
            float l0, h0, l1, h1;
            rope_pair(E::lo(x4[e]), E::lo(y4[e]), cs[i0], sn[i0], l0, h0);
            rope_pair(E::hi(x4[e]), E::hi(y4[e]), cs[i1], sn[i1], l1, h1);
            // the packed conversion instruction: round to nearest even, two at a time
            lo4[e] = E::pack2(l0, l1);
            hi4[e] = E::pack2(h0, h1);
        }
        uint16_t *kd = p.kc + dst + (size_t)h * D + c * 8;
        *(u32x4 *)kd = lo4;
        *(u32x4 *)(kd + H) = hi4;
    }
    const int chunks = D / 8;
    for (int idx = lane; idx < p.Hkv * chunks; idx += 64) {
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
template <class E, int D>
__global__ __launch_bounds__(64) void k_prefill_readable(PrefillParams p, const float2 *table)
{
    constexpr int H = D / 2;
    // one-dimensional grid of A * T * Hq waves
    const unsigned at = blockIdx.x / (unsigned)p.Hq;
    const int hq = (int)(blockIdx.x % (unsigned)p.Hq), t = (int)(at % (unsigned)p.T),
              a = (int)(at / (unsigned)p.T), lane = threadIdx.x;
    const Chunk ch = chunk_of(p, a);
    uint16_t *out = p.out + a * p.o_sa + t * p.o_st + hq * p.o_sh;
    if (!ch.ok) {  // device values disagree with the checked host copy: NaN output
#pragma unroll
        for (int e = 0; e < D / 64; ++e)
            out[lane + 64 * e] = E::qnan;
        return;
    }
    if (t >= ch.n)
        return;
    const int row = ch.row, last = ch.s + t;
    const int kv = hq / p.G;
    const uint16_t *qs = p.q + a * p.q_sa + t * p.q_st + hq * p.q_sh;
    const float2 *tab = table + table_row(p, a, t) * H;
    float q[D / 64];
    if (D == 128) {
        const float2 cs = tab[lane];
        rope_pair(E::to_f(qs[lane]), E::to_f(qs[lane + 64]), cs.x, cs.y, q[0], q[D / 64 - 1]);
    } else {
        const int i = lane & (H - 1);
        const float2 cs = tab[i];
        float lo, hi;
        rope_pair(E::to_f(qs[i]), E::to_f(qs[i + H]), cs.x, cs.y, lo, hi);
        q[0] = lane < H ? lo : hi;
    }
    const size_t slot = (size_t)p.Hkv * D;
    const uint16_t *K = p.kc + (size_t)row * p.C * slot + (size_t)kv * D;
    const uint16_t *V = p.vc + (size_t)row * p.C * slot + (size_t)kv * D;
    float m = -INFINITY, l = 0.0f, o[D / 64];
#pragma unroll
    for (int e = 0; e < D / 64; ++e)
        o[e] = 0.0f;
    for (int j = 0; j <= last; ++j) {
        float part = 0.0f;
#pragma unroll
        for (int e = 0; e < D / 64; ++e)
            part += q[e] * E::to_f(K[j * slot + lane + 64 * e]);
        const float s = wave_sum(part) * p.scale_log2;
        const float mn = fmaxf(m, s);
        const float corr = exp2f(m - mn);
        const float pj = exp2f(s - mn);
        l = l * corr + pj;
#pragma unroll
        for (int e = 0; e < D / 64; ++e)
            o[e] = o[e] * corr + pj * E::to_f(V[j * slot + lane + 64 * e]);
        m = mn;
    }
#pragma unroll
    for (int e = 0; e < D / 64; ++e)
        out[lane + 64 * e] = (uint16_t)E::from_f(o[e] / l);
}


// ---------------------------------------------------------------- tuned

// LDS slot of the 16-B chunks of key row r: chunk c sits at slot c ^ swz(r).
// Only r % 16 matters.  Within each aligned group of four rows the slot bits
// 1-2 and the bits 2-3 each take all four values, and the group constant sets
// bits 0 and 3, which keeps the 16 rows' patterns distinct (also modulo 8): so
// the K operand reads (16 consecutive rows at one chunk) and the transposing V
// reads (4 rows x 4 chunks per 32 lanes) both hit every bank once per pass,
// for 32 as for 64 four-byte banks.
__device__ __forceinline__ int swz(int r)
{
    const int b0 = r & 1, b1 = (r >> 1) & 1, g = (r >> 2) & 3;
    return ((b0 << 1) | (b1 << 2) | ((b0 ^ b1) << 3)) ^ ((g & 1) | ((g >> 1) << 3));
}

template <int B>
struct Buf {
    static constexpr int value = B;
};
//
// Query heads of one kv head that share a matrix-core work group: four when G
// allows, else two or one; the four waves cover HB heads times 4 / HB
// sub-tiles of 32 query positions.
__host__ __device__ __forceinline__ int heads_per_block(int G)
{
    return (G & 3) == 0 ? 4 : ((G & 1) == 0 ? 2 : 1);
}

// One workgroup of 4 waves per (entry a, kv head, group of HB query heads,
// query tile q0 .. q0 + 128 / HB - 1): wave w owns query head HB g + w % HB of
// the kv head's G and queries q0 + 32 (w / HB) .. + 31.  Key tiles
// of 64 move from memory straight into two LDS buffers by LDS-DMA (the next
// tile while the current one is computed), each key row's 16-byte chunks
// permuted by swz.  Per tile and wave:
//   S^T = K Q^T on v_mfma_f32_32x32x16_{bf16,f16} (A = 32 keys x 16 dims of K, B =
//       16 dims x 32 queries of the rotated query): lane l owns query l % 32
//       and keys 8 (i / 4) + 4 (l / 32) + i % 4 (i < 16) of each 32-key block,
//       so the softmax over keys is in-lane plus one exchange with lane l ^ 32;
//   online softmax in FP32 (log2 domain, causal mask on the diagonal);
//   O^T += V^T P^T on the same instruction: the score registers are already
//       the B operand (16 keys per k-step, in the key order above) and V^T is
//       read from the row-major LDS tile with ds_read_b64_tr_b16 in that order.
// The FP32 rotated query enters the matrix cores as two parts in the storage
// type (the high part and the rounded remainder: 2^-16 relative for BF16,
// 2^-22 for FP16), so the scores keep their accuracy at any magnitude; the
// weights (in [0, 1]) are rounded once to nearest even; products accumulate
// in FP32; the output is rounded once.
template <class E, int D>
__global__ __launch_bounds__(256, 2) void k_prefill_mfma(PrefillParams p, const float2 *table)
{
    typedef typename E::vec8 vec8;
    typedef typename E::vec2 vec2;
    constexpr int BM = 128, BN = 64;
    constexpr int KS = D / 16;              // QK k-steps
    constexpr int NDB = D / 32;             // PV dim blocks
    constexpr int ROW = D * 2;              // LDS row of a key, bytes (chunk-swizzled)
    constexpr int CPR = D / 8;              // 16-B chunks per key row
    constexpr int RPI = 64 / CPR;           // key rows per 1-KiB LDS-DMA instruction
    constexpr int NI = BN / RPI;            // DMA instructions per tile and tensor
    constexpr float HEADROOM = 8.0f;

    // The four waves hold HB query heads of one kv head times 4 / HB sub-tiles of
    // 32 query positions (HB = 4 whenever G allows): with four heads at the same
    // positions every wave has the same causal extent, so no wave idles through
    // the block's last key tiles while the others finish the diagonal.
    const int HB = heads_per_block(p.G), BQ = BM / HB, nhb = p.G / HB;
    const int nqt = (p.T + BQ - 1) / BQ;
    // Work groups are handed to the eight XCDs in turn (group b to XCD b % 8),
    // and each XCD has its own L2.  The G query heads and all query tiles of a kv
    // head read the same K/V tiles, so all blocks of one (entry, kv head) pair go
    // to one XCD: pair i lives on XCD i % 8.  An XCD takes its pairs in chunks of
    // PG, so that the K/V rows in use at once fit its L2 (all of an XCD's pairs
    // at once did not: every tile was fetched several times), and runs a chunk's
    // blocks longest query tile first (the tile rank is the slowest index within
    // the chunk), its pairs and head groups within a rank.  Inside an XCD the
    // dispatcher deals consecutive groups to its shader engines in turn, so the
    // order of the pairs within a rank rotates by one per rank: one pair's blocks
    // spread over the engines, and a pair with a long cached prefix (a chunk at a
    // late start) does not load one engine with all its long blocks.
    int qt, hg, a, kv;
    {
        const int b = blockIdx.x, npairs = p.A * p.Hkv;
        int pair, rank, rem;
        if ((npairs & 7) == 0) {
            constexpr int PG = 4;
            const int ppx = npairs >> 3;  // pairs per XCD
            const int x = b & 7, j = b >> 3;
            const int cb = PG * nhb * nqt;  // blocks of a full chunk of PG pairs
            const int c = j / cb, jj = j - c * cb;
            const int per = min(PG, ppx - c * PG) * nhb;  // blocks of one tile rank in the chunk
            rank = jj / per;
            rem = (jj - rank * per + rank) % per;
            pair = (c * PG + rem / nhb) * 8 + x;
        } else {
            const int per = npairs * nhb;
            rank = b / per;
            rem = (b - rank * per + rank) % per;
            pair = rem / nhb;
        }
        a = pair / p.Hkv;
        kv = pair - a * p.Hkv;
        if (a < p.n_order)
            a = p.order[a];
        hg = rem % nhb;
        qt = nqt - 1 - rank;
    }
    const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
    const int qi = lane & 31, hh = lane >> 5;
    const int hq = kv * p.G + hg * HB + w % HB;  // this wave's query head
    const int q0 = qt * BQ, qw = q0 + 32 * (w / HB), qrow = qw + qi;
    const Chunk ch = chunk_of(p, a);
    if (!ch.ok) {  // device values disagree with the checked host copy: NaN output
        if (qrow < p.T && hh == 0)
            for (int d = 0; d < D; ++d)
                p.out[a * p.o_sa + qrow * p.o_st + hq * p.o_sh + d] = E::qnan;
        return;
    }
    if (q0 >= ch.n)
        return;  // the whole query tile lies past this entry's length
    const int row = ch.row, s0 = ch.s, n = ch.n;
    // keys 0 .. s0 + n - 1 exist (the cached prefix and the chunk); the tile's
    // last query sees up to key s0 + min(q0 + BQ, n) - 1
    const int nkeys = s0 + min(q0 + BQ, n);
    const int ntiles = (nkeys + BN - 1) / BN;

    // K and V tiles, double-buffered, filled straight from memory by LDS-DMA.
    // Chunk c of key row r sits at chunk slot c ^ swz(r) of its LDS row, so the
    // operand reads below spread over all banks without padding.
    // Separate arrays per buffer, not one indexed by the buffer: accesses to
    // distinct LDS variables are known not to alias, so the reads of one buffer
    // need not wait for the memory-to-LDS loads into the other.  The second
    // buffer's K and V tiles share one array (K, then V), which also stages the
    // four waves' query rows before the first tile is in use.
    __shared__ __attribute__((aligned(16))) unsigned char klds0[BN * ROW], vlds0[BN * ROW];
    __shared__ __attribute__((aligned(16))) unsigned char kvlds1[2 * BN * ROW];
    // cos/sin rows of the block's 32 positions when its four waves share them
    __shared__ __attribute__((aligned(16))) unsigned char tlds[32 * D * 4];

    const size_t slot = (size_t)p.Hkv * D;
    const size_t rb = (size_t)row * p.C * slot + (size_t)kv * D;
    const unsigned char *kb = (const unsigned char *)(p.kc + rb);
    const unsigned char *vb = (const unsigned char *)(p.vc + rb);
    const uint32_t slotb = (uint32_t)(slot * 2);

    // tile t into buffer buf: wave w issues DMA instructions w, w + 4, ...; lane
    // l of instruction i fetches chunk (l % CPR) ^ swz(r) of key row
    // r = RPI i + l / CPR (clamped into the prompt) into slot l % CPR
    auto load_tile = [&](int t, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        unsigned char *kd = buf ? kvlds1 : klds0, *vd = buf ? kvlds1 + BN * ROW : vlds0;
#pragma unroll
        for (int i = w; i < NI; i += 4) {
            const int r = i * RPI + lane / CPR;
            const uint32_t off = (uint32_t)min(t * BN + r, nkeys - 1) * slotb +
                                 ((((lane % CPR) ^ swz(r)) & (CPR - 1)) << 4);
            lds_dma16(kb + off, kd + i * 1024);
            lds_dma16(vb + off, vd + i * 1024);
        }
    };
    load_tile(0, Buf<0>{});

    // Per-lane byte offsets of the operand reads inside a tile; the key block,
    // the PV k-step and the buffer only add constants.
    //   K: key row qi (+ 32 for the second block), chunk 2 ks + hh (dims
    //      16 ks + 8 hh .. + 7);
    //   V: key row 4 hh + j16 / 4 (+ 8 for the second read, + 16 / 32 for the
    //      k-step), dims 32 db + 16 (g % 2) + 4 (j16 % 4) .. + 3.
    const int j16 = lane & 15, g = lane >> 4;
    uint32_t koff[KS], voff[2][NDB];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
        koff[ks] = qi * ROW + ((((2 * ks + hh) ^ swz(qi)) & (CPR - 1)) << 4);
#pragma unroll
    for (int s8 = 0; s8 < 2; ++s8) {
        const int r = 4 * hh + (j16 >> 2) + 8 * s8;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int col = (32 * db + 16 * (g & 1) + 4 * (j16 & 3)) * 2;  // bytes
            voff[s8][db] = r * ROW + ((((col >> 4) ^ swz(r)) & (CPR - 1)) << 4) + (col & 15);
        }
    }

    // B operands of QK: the rotated query of this lane's row, dims 16 ks + 8 hh + j,
    // as two parts in the storage type (high part and rounded remainder)
    vec8 bq[2][KS];
    {
        u32x4 qv[KS];
        float4 cv[KS / 2][4];
        if (HB == 4) {
            // The four waves hold the same 32 positions: their query rows and the
            // positions' cos/sin rows move by LDS-DMA, every instruction 1 KiB of
            // whole rows (per-lane 16-B loads of 32 rows each touched 32 cache
            // lines per instruction).  Wave w's query rows go to the second tile
            // buffer (free until the first tile is in use) in the K tile layout,
            // so the K operand offsets read them; the block's cos/sin rows go to
            // tlds, chunk c of row r at slot c ^ swz(r).
            const uint16_t *qb = p.q + a * p.q_sa + hq * p.q_sh;
            unsigned char *qs = kvlds1 + w * 32 * ROW;
#pragma unroll
            for (int i = 0; i < 32 / RPI; ++i) {
                const int r = i * RPI + lane / CPR;
                const int c = ((lane % CPR) ^ swz(r)) & (CPR - 1);
                lds_dma16(qb + (size_t)min(qw + r, n - 1) * p.q_st + c * 8, qs + i * 1024);
            }
            constexpr int CPT = D / 4;     // 16-B chunks of a cos/sin row
            constexpr int RPT = 64 / CPT;  // cos/sin rows per DMA instruction
#pragma unroll
            for (int k = 0; k < 32 / RPT / 4; ++k) {  // a fixed count: no loop
                const int i = w + 4 * k;
                const int r = i * RPT + lane / CPT;
                const int c = ((lane % CPT) ^ swz(r)) & (CPT - 1);
                lds_dma16(table + table_row(p, a, min(q0 + r, n - 1)) * (D / 2) + c * 2,
                          tlds + i * 1024);
            }
            __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA; the barrier covers the others
            __syncthreads();
            const unsigned char *qd = kvlds1 + w * 32 * ROW;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qv[ks] = *(const u32x4 *)(qd + koff[ks]);
#pragma unroll
            for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    cv[ks][j] = *(const float4 *)(tlds + qi * (CPT * 16) +
                                                  (((8 * ks + 4 * hh + j) ^ swz(qi)) << 4));
        } else {
            // waves at different positions: per-lane loads, both in flight before
            // either is used (one memory round trip)
            const int tq = min(qrow, n - 1);
            const uint16_t *qs = p.q + a * p.q_sa + tq * p.q_st + hq * p.q_sh;
            const float4 *cs = (const float4 *)(table + table_row(p, a, tq) * (D / 2));
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                qv[ks] = *(const u32x4 *)(qs + ks * 16 + hh * 8);
#pragma unroll
            for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    cv[ks][j] = cs[ks * 8 + hh * 4 + j];
            // everything is needed next anyway; waiting here also leaves no load
            // pending where the two paths join
            __builtin_amdgcn_s_waitcnt(0);
        }
        float x[KS][8];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                x[ks][2 * e] = E::lo(qv[ks][e]);
                x[ks][2 * e + 1] = E::hi(qv[ks][e]);
            }
#pragma unroll
        for (int ks = 0; ks < KS / 2; ++ks)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float4 c4 = cv[ks][j >> 1];
                const float c = (j & 1) ? c4.z : c4.x, sn = (j & 1) ? c4.w : c4.y;
                float lo, hi;
                rope_pair(x[ks][j], x[ks + KS / 2][j], c, sn, lo, hi);
                x[ks][j] = lo;
                x[ks + KS / 2][j] = hi;
            }
        if constexpr (E::code == Bf16::code) {
            // the same two parts as E::part<2>, two values per instruction: the
            // high part is x with its low 16 bits cleared, the remainder x - hi
            // (exact in FP32) goes through the hardware conversion, which rounds
            // to nearest even like the storage type's own rounding
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 vh, vl;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const uint32_t h0 = __float_as_uint(x[ks][2 * e]) & 0xffff0000u;
                    const uint32_t h1 = __float_as_uint(x[ks][2 * e + 1]) & 0xffff0000u;
                    vh[e] = (h0 >> 16) | h1;
                    vl[e] = E::pack2(x[ks][2 * e] - __uint_as_float(h0),
                                     x[ks][2 * e + 1] - __uint_as_float(h1));
                }
                bq[0][ks] = __builtin_bit_cast(vec8, vh);
                bq[1][ks] = __builtin_bit_cast(vec8, vl);
            }
        } else {
#pragma unroll
            for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                for (int ks = 0; ks < KS; ++ks) {
                    u32x4 v;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        v[e] = E::template part<2>(x[ks][2 * e], pp) |
                               (E::template part<2>(x[ks][2 * e + 1], pp) << 16);
                    bq[pp][ks] = __builtin_bit_cast(vec8, v);
                }
        }
    }

    f32x16 O[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i)
            O[db][i] = 0.0f;
    float m_run = -INFINITY, l_run = 0.0f;
    bool fresh = true;  // no tile seen yet (wave-uniform)

    __builtin_amdgcn_s_waitcnt(0);  // this wave's DMA; the barrier covers the others
    __syncthreads();
    // one key tile from LDS buffer B (a compile-time constant, so every operand
    // read is a per-lane offset plus an immediate)
    auto tile = [&](const int t, auto bufc) {
        constexpr int buf = decltype(bufc)::value;
        if (t + 1 < ntiles)
            load_tile(t + 1, Buf<buf ^ 1>{});
        const int k0 = t * BN;
        // some key of the tile is visible to one of this wave's queries, and the
        // wave holds at least one query of the entry
        // NBLK live 32-key blocks of the tile: 2, or 1 on the causal diagonal
        // when the tile's second block lies past every query of the wave
        auto body = [&](auto nblk) {
            constexpr int NBLK = decltype(nblk)::value;
            const unsigned char *kt = buf ? kvlds1 : klds0, *vt = buf ? kvlds1 + BN * ROW : vlds0;
            // independent 32-key blocks per k-step, so each fragment read
            // overlaps the other block's product
            f32x16 st[NBLK];
#pragma unroll
            for (int b = 0; b < NBLK; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    st[b][i] = 0.0f;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
                u32x4 kf[NBLK];
#pragma unroll
                for (int b = 0; b < NBLK; ++b)
                    kf[b] = *(const u32x4 *)(kt + koff[ks] + b * 32 * ROW);
#pragma unroll
                for (int pp = 0; pp < 2; ++pp)
#pragma unroll
                    for (int b = 0; b < NBLK; ++b)
                        st[b] = E::mma32(__builtin_bit_cast(vec8, kf[b]), bq[pp][ks], st[b]);
            }
            // raw scores; the scale (> 0) is applied inside exp2 below, so the max
            // is taken on the raw values.  Only tiles that reach past the first
            // query of the wave need the causal mask.
            float tmax = -INFINITY;
            if (k0 + BN - 1 > s0 + qw) {
                // key k0 + 4 hh + rel is visible to query qrow iff rel <= lim
                const int lim = s0 + qrow - k0 - 4 * hh;
#pragma unroll
                for (int b = 0; b < NBLK; ++b)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int rel = b * 32 + 8 * (i >> 2) + (i & 3);
                        st[b][i] = rel <= lim ? st[b][i] : -INFINITY;
                    }
            }
#pragma unroll
            for (int b = 0; b < NBLK; ++b)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    tmax = fmaxf(tmax, st[b][i]);
            {
                float hi = tmax;
                swap_halves(tmax, hi);
                tmax = fmaxf(tmax, hi) * p.scale_log2;
            }
            const bool grow = tmax > m_run + HEADROOM;
            if (fresh) {
                // the wave's first visible tile: key 0 is visible to every query,
                // so every column's max is finite; O and l are still zero
                m_run = tmax;
                fresh = false;
            } else if (__any(grow)) {
                const float m_new = grow ? tmax : m_run;
                const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
                l_run *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    O[db] *= alpha;
                m_run = m_new;
            }
            vec8 pb[2 * NBLK];
#pragma unroll
            for (int k2 = 0; k2 < 2 * NBLK; ++k2) {
                u32x4 v;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const float p0 = __builtin_amdgcn_exp2f(
                        __builtin_fmaf(st[k2 >> 1][8 * (k2 & 1) + 2 * e], p.scale_log2, -m_run));
                    const float p1 = __builtin_amdgcn_exp2f(
                        __builtin_fmaf(st[k2 >> 1][8 * (k2 & 1) + 2 * e + 1], p.scale_log2, -m_run));
                    const vec2 pk = E::cvt2(p0, p1);
                    v[e] = __builtin_bit_cast(uint32_t, pk);
                    // the row sum takes the same rounded weights the PV product uses
                    // (fed from the converted pair itself: reading the pair back
                    // out of v[] compiled to the same register for every e)
                    l_run = E::sum2(pk, l_run);
                }
                pb[k2] = __builtin_bit_cast(vec8, v);
            }
            // PV: slot j of k-step k2 is key 32 (k2 / 2) + 16 (k2 % 2) + 8 (j / 4) + 4 hh + j % 4
#pragma unroll
            for (int k2 = 0; k2 < 2 * NBLK; ++k2) {
                const int rows_k2 = (32 * (k2 >> 1) + 16 * (k2 & 1)) * ROW;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4 *)(vt + voff[0][db] + rows_k2));
                    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) s16x4 *)(vt + voff[1][db] + rows_k2));
                    const s16x4 vv[2] = {v0, v1};
                    O[db] = E::mma32(__builtin_bit_cast(vec8, vv), pb[k2], O[db]);
                }
            }
        };
        if (k0 <= s0 + qw + 31 && qw < n) {
            if (k0 + 32 > s0 + qw + 31)
                body(Buf<1>{});
            else
                body(Buf<2>{});
        }
        __builtin_amdgcn_s_waitcnt(0);  // the next tile's DMA (this wave's share)
        __syncthreads();                // ... and every wave's; buffer buf is free again
    };
    for (int t = 0; t < ntiles; t += 2) {
        tile(t, Buf<0>{});
        if (t + 1 < ntiles)
            tile(t + 1, Buf<1>{});
    }

    {
        float hi = l_run;
        swap_halves(l_run, hi);
        l_run += hi;
    }
    if (qrow < n) {
        const float inv = 1.0f / l_run;
        uint16_t *out = p.out + a * p.o_sa + qrow * p.o_st + hq * p.o_sh;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                u32x2 v;  // finite values: the conversion instruction rounds to nearest even
                v[0] = E::pack2(O[db][4 * r] * inv, O[db][4 * r + 1] * inv);
                v[1] = E::pack2(O[db][4 * r + 2] * inv, O[db][4 * r + 3] * inv);
                *(u32x2 *)(out + 32 * db + 8 * r + 4 * hh) = v;
            }
    }
}

}  // namespace

void prefill_order(PrefillParams &p, const int32_t *starts_host, const int32_t *lens_host)
{
    p.n_order = 0;
    if (!starts_host || p.A > kMaxPrefillOrder)
        return;
    // key tiles of one (entry, kv head, head group): the kernel's blocks of BQ
    // queries, block j seeing keys up to s + min((j + 1) BQ, n) - 1
    const int BQ = 128 / heads_per_block(p.G);
    std::vector<std::pair<long long, int>> w(p.A);
    for (int a = 0; a < p.A; ++a) {
        const long long s = starts_host[a], n = lens_host[a];
        long long tiles = 0;
        for (long long q0 = 0; q0 < n; q0 += BQ)
            tiles += (s + std::min(q0 + BQ, n) + 63) / 64;
        w[a] = {-tiles, a};
    }
    std::stable_sort(w.begin(), w.end());
    for (int a = 0; a < p.A; ++a)
        p.order[a] = (uint16_t)w[a].second;
    p.n_order = p.A;
}

uint64_t prefill_workspace_bytes(int64_t A, int64_t T, int64_t Hq, int64_t D)
{
    (void)Hq;
    return ((uint64_t)A * T * (D / 2) * 8u + 255u) & ~uint64_t(255);
}

template <class E>
static void launch_prefill_e(const PrefillParams &p, hipStream_t stream, int kernel, hipEvent_t e0,
                             hipEvent_t e1)
{
    const float2 *table = p.table;
    if (kernel == 1) {
        const dim3 grid(p.Hq * p.T * p.A);
        if (p.D == 64)
            hipExtLaunchKernelGGL((k_prefill_readable<E, 64>), grid, dim3(64), 0, stream, e0, e1, 0,
                                  p, table);
        else
            hipExtLaunchKernelGGL((k_prefill_readable<E, 128>), grid, dim3(64), 0, stream, e0, e1, 0,
                                  p, table);
    } else {
        const int hb = heads_per_block(p.G);
        const dim3 grid(p.Hq / hb * p.A * ((p.T + 128 / hb - 1) / (128 / hb)));
        if (p.D == 64)
            hipExtLaunchKernelGGL((k_prefill_mfma<E, 64>), grid, dim3(256), 0, stream, e0, e1, 0, p,
                                  table);
        else
            hipExtLaunchKernelGGL((k_prefill_mfma<E, 128>), grid, dim3(256), 0, stream, e0, e1, 0, p,
                                  table);
    }
}

hipError_t launch_prefill(const PrefillParams &p, hipStream_t stream, int kernel, hipEvent_t e0,
                          hipEvent_t e1)
{
    if (p.dtype == F16::code)
        hipLaunchKernelGGL(k_prefill_store<F16>, dim3(p.T * p.A), dim3(64), 0, stream, p, p.table);
    else
        hipLaunchKernelGGL(k_prefill_store<Bf16>, dim3(p.T * p.A), dim3(64), 0, stream, p, p.table);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (p.dtype == F16::code)
        launch_prefill_e<F16>(p, stream, kernel, e0, e1);
    else
        launch_prefill_e<Bf16>(p, stream, kernel, e0, e1);
    return hipGetLastError();
}

}  // namespace mllm
