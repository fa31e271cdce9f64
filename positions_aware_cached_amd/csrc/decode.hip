// decode.hip -- gfx950 kernels of the positions-aware cached decode step.
//
// The step (microLLM-rocm ARCHITECTURE.md, "Tensor ownership boundary"):
// device positions[A] and cache_rows[A] parameterize decode RoPE, the K/V
// store and cached attention; rows not named in cache_rows stay untouched.
//
// Tuned path, two launches on one stream:
//   k_decode_stream   NW resident work groups (one wave per kv head of a head
//                     group) split the keys of all (entry, head group)
//                     segments evenly: RoPE of the queries, RoPE(K) + K/V store
//                     by the group that holds a segment's last tile, scores and
//                     P.V on the matrix cores, online FP32 softmax, one partial
//                     (max, sum, unnormalized output) per segment, group and
//                     query head;
//   k_decode_merge    one wave per (entry, query head): rescales and sums the
//                     partials of its segment (the streaming-attention merge
//                     of the IPU refactor log, "Flash vs materialized
//                     attention"), divides, rounds to the storage type.
// Readable path (reference level, kept for diagnosis as the operator workflow
// asks -- operator-development.md, "Acceptance rule"):
//   k_rope_store      one block per entry: RoPE(K) + K/V store, rotated
//                     queries in FP32 into the workspace;
//   k_decode_readable one wave per (entry, query head), one key at a time.
//
// Every kernel is written once over the storage type E of the cache and the
// tensors (BF16 or FP16, elem.h).  Numerics: the softmax runs in the log2
// domain (scores pre-multiplied by log2(e)/sqrt(D), exp2), every sum is FP32,
// only the output is rounded.  On the matrix cores the FP32 rotated query and
// the FP32 softmax weights enter as sums of parts in the storage type (see
// Cols below), so the products are those of the FP32 values (BF16: exactly
// for up to 4 query heads per kv head, to 2^-16 relative beyond; FP16: to
// 2^-22) and accumulate in FP32.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <mutex>

#include "elem.h"
#include "kernels.h"

namespace mllm {
namespace {

typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;

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

__device__ __forceinline__ bool entry_valid(const DecodeParams &p, int pos, int row)
{
    return pos >= 0 && pos < p.C && row >= 0 && row < p.S;
}

// ---------------------------------------------------------------- R1
template <class E>
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
        rope_pair(E::to_f(k[i]), E::to_f(k[i + H]), cs[i], sn[i], lo, hi);
        uint16_t *kd = p.kc + dst + (size_t)h * D;
        kd[i] = (uint16_t)E::from_f(lo);
        kd[i + H] = (uint16_t)E::from_f(hi);
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
        rope_pair(E::to_f(q[i]), E::to_f(q[i + H]), cs[i], sn[i], lo, hi);
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

template <class E, int D>
__global__ __launch_bounds__(64) void k_decode_readable(DecodeParams p)
{
    constexpr int PER = D / 64;
    // one-dimensional grid of A * Hq waves (the y and z grid sizes are limited)
    const int hq = (int)(blockIdx.x % (unsigned)p.Hq), a = (int)(blockIdx.x / (unsigned)p.Hq);
    const int lane = threadIdx.x;
    const int pos = p.positions[a], row = p.rows[a];
    uint16_t *out = p.out + a * p.o_sa + hq * p.o_sh;
    if (!entry_valid(p, pos, row)) {
#pragma unroll
        for (int e = 0; e < PER; ++e)
            out[lane + 64 * e] = E::qnan;
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
            part += q[e] * E::to_f(K[j * slot + lane + 64 * e]);
        const float s = wave_sum(part) * p.scale_log2;
        const float mn = fmaxf(m, s);
        const float corr = exp2f(m - mn);
        const float pj = exp2f(s - mn);
        l = l * corr + pj;
#pragma unroll
        for (int e = 0; e < PER; ++e)
            o[e] = o[e] * corr + pj * E::to_f(V[j * slot + lane + 64 * e]);
        m = mn;
    }
#pragma unroll
    for (int e = 0; e < PER; ++e)
        out[lane + 64 * e] = (uint16_t)E::from_f(o[e] / l);
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
// k_decode_stream: the tuned decode step, one launch of NW resident waves.
//
// Work plan.  The keys of every (entry a, kv head h) segment are cut into
// tiles of kTile keys; segments follow in entry-major order (seg = a * Hkv +
// h), so segment (a, h) covers the global tiles [Hkv E(a) + h n(a), + n(a)),
// where n(a) is entry a's tile count (0 for an entry whose position or row is
// out of range) and E(a) = n(0) + ... + n(a - 1).  The plan splits the tiles,
// and with short segments their starts too, into NW ranges of equal work
// whatever the row lengths (with two groups per compute unit the
// first-dispatched half gets a larger share, see make_plan); group w owns the
// global tiles [t0(w), t0(w + 1)) that start in its range.  A wave
// walks its range across segment boundaries, keeps the next tile in flight
// across them, and writes one partial (reference max, sum, unnormalized
// output of each of the G query heads) per segment it touches into slot
// seg + w -- distinct for distinct (seg, w) because waves visit segments in
// order -- so at most A Hkv + NW slots.
//
// Per segment, on entry: cos/sin of the entry's position (one pair index per
// lane, in double, rounded once), the G rotated queries as matrix-core B
// operands, and -- in the wave that holds the segment's last tile -- RoPE of
// k_new and the store of K' and V at (row, pos), staged in LDS so that the
// wave attends to exactly the stored bytes.  The queries, key and value come
// into registers with the segment's first tile and move to LDS at its start.
//
// Per 32-key tile: the next tile is in flight in registers (K in operand
// order, V in row order, 16 B per lane, non-temporal loads: every cached byte
// is read once per step) while this one is computed from LDS; as soon as it
// has landed the tile after it is issued, so the end of one segment and the
// start of the next run with loads in flight:
//   QK  v_mfma_f32_16x16x32_{bf16,f16}: A = 16 keys x 32 dims of K, B = 32 dims
//       x 16 columns holding the parts of the FP32 rotated query heads; lane l
//       ends with the scores of keys 4 (l / 16) + i of column l % 16.
//   softmax per column in FP32 (exp2 of log2(e)/sqrt(D)-scaled scores); the
//       reference max moves only when a column max grows past a headroom, so
//       the accumulators are rescaled rarely.
//   PV  the same instruction with A = V^T read by ds_read_b64_tr_b16 from the
//       row-major padded LDS tile and B = the parts of the FP32 weights.
//
// Operand columns: part q (hi / mid / lo part, in the storage type) of head g
// sits in column q GS + g (GCLS <= 8, one column group) or column g of group q
// (GCLS 16).  BF16: three parts reproduce an FP32 value exactly (GCLS <= 4),
// two carry it to 2^-16 relative (GCLS 8, 16); FP16: two parts, 2^-22.
constexpr int kTile = 32;
#ifdef MLLM_STAMPS
__device__ unsigned long long mllm_stamps[4096 * 8];
#define STAMP(k, v) do { if (threadIdx.x == 0) mllm_stamps[blockIdx.x * 8 + (k)] = (v); } while (0)
#else
#define STAMP(k, v) do { } while (0)
#endif

template <int GCLS, class E>
struct Cols {
    static constexpr int GS = GCLS;
    static constexpr int NPART = GCLS <= 4 ? E::max_parts : 2;
    static constexpr int NGRP = GCLS == 16 ? 2 : 1;
};

typedef __attribute__((ext_vector_type(4))) short s16x4;

// v rotated by K lanes within each row of 16 lanes (DPP row_ror: VALU only)
template <int K>
__device__ __forceinline__ float row_ror(float v)
{
    return __builtin_bit_cast(
        float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x120 + K, 0xf, 0xf, false));
}

// Sum of v over the lanes of this lane's 16-lane row that share lane % GS
// (one operand column class: the parts of one head).  A rotation tree, so
// every lane of a class ends with the same bits.
template <int GS>
__device__ __forceinline__ float class_sum(float v)
{
    if constexpr (GS <= 8)
        v += row_ror<8>(v);
    if constexpr (GS <= 4)
        v += row_ror<4>(v);
    if constexpr (GS <= 2)
        v += row_ror<2>(v);
    if constexpr (GS <= 1)
        v += row_ror<1>(v);
    return v;
}

// 2^x for x <= HEADROOM or -inf (the softmax weights): the hardware exp2.
// Its result for arguments below -126 is flushed to zero, which only drops
// weights under 2^-126 of the running maximum.
__device__ __forceinline__ float exp2_nonpos(float x) { return __builtin_amdgcn_exp2f(x); }

// v shifted up by K lanes within each row of 16 lanes, 0 in the row's first K
// lanes (DPP row_shr)
template <int K>
__device__ __forceinline__ int row_shr_zero(int v)
{
    return __builtin_amdgcn_update_dpp(0, v, 0x110 + K, 0xf, 0xf, false);
}

// Inclusive prefix sum over the 64 lanes: a shift-and-add tree within each
// 16-lane row, then the totals of the rows below (lanes 15, 31, 47).
__device__ __forceinline__ int wave_incl_scan(int v, int lane)
{
    v += row_shr_zero<1>(v);
    v += row_shr_zero<2>(v);
    v += row_shr_zero<4>(v);
    v += row_shr_zero<8>(v);
    const int r0 = __builtin_amdgcn_readlane(v, 15), r1 = __builtin_amdgcn_readlane(v, 31),
              r2 = __builtin_amdgcn_readlane(v, 47);
    const int row = lane >> 4;
    return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// Keeps a wave-uniform value in scalar registers from here on: the compiler
// would otherwise reload a kernel argument before each use, every reload a
// scalar memory round trip the wave waits for.
template <class T>
__device__ __forceinline__ void pin(T &v)
{
    asm volatile("" : "+s"(v));
}

// The kernel arguments the plan reads, loaded once and pinned.
struct Entries {
    const int32_t *positions, *rows;
    int A, S, C, NHG;
};
__device__ __forceinline__ Entries entries_of(const DecodeParams &p)
{
    Entries e = {p.positions, p.rows, p.A, p.S, p.C, p.NHG};
    pin(e.positions);
    pin(e.rows);
    pin(e.A);
    pin(e.S);
    pin(e.C);
    pin(e.NHG);
    return e;
}

// Tile count of entry x from its position and row: 0 when x >= A or the entry
// is invalid.  Branch-free, so every lane consumes its loads at this point.
__device__ __forceinline__ int tiles_of(const Entries &p, int x, int pos, int row)
{
    const bool ok = (x < p.A) & (pos >= 0) & (pos < p.C) & (row >= 0) & (row < p.S);
    return ok ? (pos + kTile) / kTile : 0;
}

// Entries are read 4 x 64 at a time: lane l of block c0 holds entries
// c0 + 64 k + l (indices clamped into [0, A), so every load is in bounds and
// all of them are issued before the first is used).
struct EntryBlock {
    int pos[4], row[4], na[4];
};
__device__ __forceinline__ void load_block(const Entries &p, int c0, int lane, EntryBlock &b)
{
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int x = min(c0 + 64 * k + lane, p.A - 1);
        b.pos[k] = p.positions[x];
        b.row[k] = p.rows[x];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
        b.na[k] = tiles_of(p, c0 + 64 * k + lane, b.pos[k], b.row[k]);
}

// A block of entries with the inclusive scans of its tile counts and of its
// valid entries: incl[k] on lane l sums n(c0 + 64 k + i) for i <= l, cnt[k]
// counts the i <= l with n(c0 + 64 k + i) > 0.
struct ScanBlock {
    EntryBlock b;
    int incl[4], cnt[4];
};
__device__ __forceinline__ void scan_block(const Entries &p, int c0, int lane, ScanBlock &s)
{
    load_block(p, c0, lane, s.b);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        s.incl[k] = wave_incl_scan(s.b.na[k], lane);
        // the ballot's bits below this lane, plus its own
        const unsigned long long v = __ballot(s.b.na[k] > 0);
        s.cnt[k] = __builtin_amdgcn_mbcnt_hi((unsigned)(v >> 32),
                                             __builtin_amdgcn_mbcnt_lo((unsigned)v, 0u)) +
                   (s.b.na[k] > 0);
    }
}

// Totals on every lane: NT = NHG * sum_a n(a) tiles in NSEG = NHG * #{a :
// n(a) > 0} segments; the first block (entries 0..255) is left in first, so
// that the plan's later passes need not read it again.
struct Totals {
    long long NT, NSEG;
};
__device__ Totals plan_total(const Entries &p, int lane, ScanBlock &first)
{
    scan_block(p, 0, lane, first);
    long long s = 0, c = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        s += __builtin_amdgcn_readlane(first.incl[k], 63);
        c += __builtin_amdgcn_readlane(first.cnt[k], 63);
    }
    for (int c0 = 256; c0 < p.A; c0 += 256) {
        ScanBlock sb;
        scan_block(p, c0, lane, sb);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            s += __builtin_amdgcn_readlane(sb.incl[k], 63);
            c += __builtin_amdgcn_readlane(sb.cnt[k], 63);
        }
    }
    return Totals{s * p.NHG, c * p.NHG};
}

// Groups of the plan: min(launched, NT); group w owns the units
// [v0(w), v0(w + 1)) (below), never an empty range, and with them the tiles
// that start there (possibly none: a range of segment starts only).
__device__ __forceinline__ int plan_waves(int launched, long long NT)
{
    return (int)min((long long)launched, NT);
}

// Plan units.  A tile is one unit of work.  When the segments are short (on
// average under 32 tiles each) a segment's start -- its queries, cos/sin, the
// store of the new token, the partial it writes -- costs about as much as a
// tile and is one more unit (su = 1), laid out before the segment's tiles, so
// a group that starts many segments gets fewer tiles; with long segments the
// starts are a small share and the plan counts tiles only (su = 0, measured
// as fast on MI355X).  Segment (a, h) of n(a) > 0 tiles is then u(a) = n(a) +
// su units, and the NU = NT + su NSEG units are split as follows.
//
// First unit of group w.  With two resident groups per compute unit the
// groups of the first half are each unit's first-dispatched group, whose waves
// win the instruction-issue ties of their SIMDs and run ahead, and the first
// half gets weight plan_wa, the second plan_wb: v0(w) = floor(W(w) NU /
// W(NW)), W the running weight.  The host picks the ratio by the work per
// tile (measured on MI355X with the K/V tiles read non-temporally: 46 : 30
// with up to 4 query heads per kv head, the best of the ratios 1.37, 1.46,
// 1.53 and 1.60 on the Llama-like batch, and with the waves' progress-based
// priorities also of 42 : 30 - 48 : 30; 45 : 28 with 5-16, against 37 : 28 and
// 41 : 28 on the long-context batch; with su = 1 the 4-head ratio measured
// faster than a uniform split on a ragged batch).  The split stays uniform (weight 1 each) when NW is odd or
// there are fewer than four tiles per group (no range is empty).
// The plan of a launch, computed once and pinned in scalar registers.
struct Plan {
    long long NU, WNW, wa, wb;
    int NW, half, su;
};
__device__ __forceinline__ Plan make_plan(const DecodeParams &p, long long NT, long long NSEG,
                                          int NW)
{
    Plan P;
    P.su = NT < 32ll * p.A * p.NHG ? 1 : 0;
    P.NU = P.su ? NT + NSEG : NT;
    P.NW = NW;
    P.half = NW >> 1;
    const bool weighted = p.plan_weighted && !(NW & 1) && NT >= 4ll * NW;
    P.wa = weighted ? p.plan_wa : 1;
    P.wb = weighted ? p.plan_wb : 1;
    P.WNW = P.wa * P.half + P.wb * (NW - P.half);
    pin(P.NU);
    pin(P.WNW);
    pin(P.wa);
    pin(P.wb);
    pin(P.NW);
    pin(P.half);
    return P;
}
__device__ __forceinline__ long long plan_weight(const Plan &P, int w)
{
    return w <= P.half ? P.wa * w : P.wa * P.half + P.wb * (w - P.half);
}
__device__ __forceinline__ long long plan_v0(const Plan &P, int w)
{
    return plan_weight(P, w) * P.NU / P.WNW;
}

// Group that owns unit v: the largest w with v0(w) <= v, i.e. with
// W(w) <= X = floor(((v + 1) W(NW) - 1) / NU).
__device__ __forceinline__ int plan_wave_of(const Plan &P, long long v)
{
    const long long X = ((v + 1) * P.WNW - 1) / P.NU;
    const long long C = P.half;
    const long long w = X <= P.wa * C ? X / P.wa : C + (X - P.wa * C) / P.wb;
    return (int)min(w, (long long)P.NW - 1);
}

// Units of an entry of na tiles, and of the scanned entries up to this lane.
__device__ __forceinline__ int units_of(const Plan &P, int na) { return na + (na > 0 ? P.su : 0); }
__device__ __forceinline__ int units_incl(const Plan &P, const ScanBlock &s, int k)
{
    return s.incl[k] + P.su * s.cnt[k];
}

// Where plan unit v < NU falls: its entry a and tile count na, the entry's
// first tile (NHG * E(a)) and first unit, and the 64-entry chunk around it
// (lane l: entry ec + l), on every lane.
struct Located {
    int a, na, ec, e_pos, e_row, e_na;
    long long tbase, ubase;
};
__device__ Located plan_locate(const Entries &p, const Plan &P, long long v, int lane,
                               const ScanBlock &first)
{
    long long run = 0, urun = 0;
    for (int c0 = 0; c0 < p.A; c0 += 256) {
        ScanBlock sb;
        if (c0 == 0)
            sb = first;
        else
            scan_block(p, c0, lane, sb);
        const EntryBlock &b = sb.b;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int ui = units_incl(P, sb, k);
            const long long uend = urun + (long long)p.NHG * ui;
            const unsigned long long hit = __ballot(v < uend && b.na[k] > 0);
            if (hit) {
                const int l = __ffsll((long long)hit) - 1;
                Located r;
                r.a = c0 + 64 * k + l;
                r.na = __builtin_amdgcn_readlane(b.na[k], l);
                r.tbase = run + (long long)p.NHG * __builtin_amdgcn_readlane(sb.incl[k] - r.na, l);
                r.ubase = urun + (long long)p.NHG *
                                     __builtin_amdgcn_readlane(ui - units_of(P, r.na), l);
                r.ec = c0 + 64 * k;
                r.e_pos = b.pos[k];
                r.e_row = b.row[k];
                r.e_na = b.na[k];
                return r;
            }
            run += (long long)p.NHG * __builtin_amdgcn_readlane(sb.incl[k], 63);
            urun += (long long)p.NHG * __builtin_amdgcn_readlane(ui, 63);
        }
    }
    Located r;  // not reached for v < NU
    r.a = p.A;
    r.na = 0;
    r.tbase = run;
    r.ubase = urun;
    r.ec = 0;
    r.e_pos = r.e_row = r.e_na = 0;
    return r;
}

// The first tile that starts at unit v or later, where v falls in L: in head
// group h of the entry at offset o < na + su, tile max(o - su, 0) of that head
// group (a segment's start unit comes before its tiles, so it maps to its
// first tile).
__device__ __forceinline__ long long plan_tile_at(const Plan &P, const Located &L, long long v)
{
    const int un = L.na + P.su;
    const long long loc = v - L.ubase;
    const int h = (int)(loc / un), o = (int)(loc - (long long)h * un);
    return L.tbase + (long long)h * L.na + max(o - P.su, 0);
}

// Issue priority of this wave for quarter q (0..3) of its group's range: 3
// down to 0.  The two groups that share a compute unit hold unequal ranges
// and drift apart; with the priority falling as a group advances, on each
// SIMD the wave of the group that is further behind wins the issue ties, so
// the pair finishes closer together (measured on MI355X: about 1 % off the
// Llama-like, ragged and long-context launches against no priorities).
__device__ __forceinline__ void set_range_priority(int q)
{
    if (q == 0)
        __builtin_amdgcn_s_setprio(3);
    else if (q == 1)
        __builtin_amdgcn_s_setprio(2);
    else if (q == 2)
        __builtin_amdgcn_s_setprio(1);
    else
        __builtin_amdgcn_s_setprio(0);
}

// LDS of one wave: K tile, padded V tile, new key / value (rotated and raw),
// the segment's query heads; and, shared by the group, cos/sin.
template <int D, int GCLS>
struct WaveLds {
    static constexpr int K = kTile * D * 2, V = kTile * (D * 2 + 16), NEW = D * 2,
                         Q = GCLS * D * 2;
    static constexpr int bytes = K + V + 3 * NEW + Q;
    static constexpr int shared = D * 4;  // cos[D/2], sin[D/2]
};
template <int D, int GCLS>
constexpr int decode_lds_bytes(int hg)
{
    return hg * WaveLds<D, GCLS>::bytes + WaveLds<D, GCLS>::shared;
}

// Up to 8 waves per group (2 per SIMD); 4 with 16-column operands (1 per SIMD).
template <class E, int D, int GCLS>
__global__ __launch_bounds__(GCLS == 16 ? 256 : 512, 1) void k_decode_stream(DecodeParams p)
{
    using CL = Cols<GCLS, E>;
    typedef typename E::vec8 vec8;
    constexpr int GS = CL::GS, NPART = CL::NPART, NGRP = CL::NGRP;
    constexpr int KS = D / 32;             // QK k-steps (32 dims each)
    constexpr int NDB = D / 16;            // PV dim blocks (16 dims each)
    constexpr int TK = kTile;              // keys per tile
    constexpr int NB = TK / 16;            // 16-key MFMA row blocks per tile
    constexpr int LPK = D / 8;             // lanes per key row (16 B each)
    constexpr int KPI = 64 / LPK;          // key rows per V load instruction
    constexpr int VLD = TK / KPI;          // V load instructions per tile
    constexpr int VROW = D * 2 + 16;       // padded LDS row of V, bytes
    constexpr float HEADROOM = 8.0f;       // log2 growth of a column max before O is rescaled

    const int w = blockIdx.x;  // work group: one wave per kv head of a head group
    STAMP(0, wall_clock64());
    STAMP(4, ((unsigned long long)__builtin_amdgcn_s_getreg((20) | (0 << 6) | (15 << 11)) << 32) |
                 __builtin_amdgcn_s_getreg((4) | (0 << 6) | (31 << 11)));
    const int wi = threadIdx.x >> 6, HG = p.HG, NHG = p.NHG;
    const int lane = threadIdx.x & 63, n = lane & 15, lg = lane >> 4;
    const int G = p.G, Hkv = p.Hkv;
    // this lane's RoPE frequency (lanes < D / 2), read once
    const float my_freq = p.inv_freq[lane & (D / 2 - 1)];

    // the plan uses min(launched groups, NT) groups, so each owns at least one tile
    const Entries ent = entries_of(p);
    // the tensors the segment and tile loads address, pinned like the plan's
    // arguments (each is needed before the first tile can be requested)
    const uint16_t *qp = p.q, *knp = p.k_new, *vnp = p.v_new;
    uint16_t *kcp = p.kc, *vcp = p.vc;
    long long q_sa = p.q_sa, q_sh = p.q_sh, kn_sa = p.kn_sa, kn_sh = p.kn_sh, vn_sa = p.vn_sa,
              vn_sh = p.vn_sh;
    pin(qp);
    pin(knp);
    pin(vnp);
    pin(kcp);
    pin(vcp);
    pin(q_sa);
    pin(q_sh);
    pin(kn_sa);
    pin(kn_sh);
    pin(vn_sa);
    pin(vn_sh);
    ScanBlock first;
    const Totals tot = plan_total(ent, lane, first);
    const long long NT = tot.NT;
    const int NW = plan_waves(p.NS, NT);
    const Plan P = make_plan(p, NT, tot.NSEG, NW);
    if (w == 0 && wi == 0) {
        // the plan's prefix for the merge kernel: units before each entry,
        // then the totals of tiles and segments
        long long run = 0;
        for (int c0 = 0; c0 < p.A; c0 += 256) {
            ScanBlock sb;
            if (c0 == 0)
                sb = first;
            else
                scan_block(ent, c0, lane, sb);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int x = c0 + 64 * k + lane;
                const int ui = units_incl(P, sb, k);
                if (x < p.A)
                    p.plan[x] = run + (long long)NHG * (ui - units_of(P, sb.b.na[k]));
                run += (long long)NHG * __builtin_amdgcn_readlane(ui, 63);
            }
        }
        if (lane == 0) {
            p.plan[p.A] = NT;
            p.plan[p.A + 1] = tot.NSEG;
        }
    }
    STAMP(1, wall_clock64());
    if (w >= NW)
        return;
    // this group's tiles [t0, t1): those that start in its units (the units
    // themselves when they are tiles only)
    const long long v0 = plan_v0(P, w), v1 = plan_v0(P, w + 1);
    const Located L0 = plan_locate(ent, P, v0, lane, first);
    long long t0 = v0, t1 = v1;
    if (P.su) {
        t0 = plan_tile_at(P, L0, v0);
        t1 = w + 1 < NW ? plan_tile_at(P, plan_locate(ent, P, v1, lane, first), v1) : NT;
    }
    if (t0 >= t1)
        return;  // only segment starts in its units

    extern __shared__ __attribute__((aligned(16))) unsigned char lds[];
    using L = WaveLds<D, GCLS>;
    float *cs = (float *)lds, *sn = cs + D / 2;
    unsigned char *klds = lds + L::shared + wi * L::bytes;
    unsigned char *vlds = klds + L::K;
    uint16_t *newk = (uint16_t *)(vlds + L::V);  // the new token, rotated key
    uint16_t *newv = newk + D;                   // its value
    uint16_t *kraw = newv + D;                   // its key, unrotated
    uint16_t *qlds = kraw + D;                   // the segment's query heads

    const size_t slot = (size_t)Hkv * D;
    const uint32_t slotb = (uint32_t)(slot * 2);  // bytes per position; a row fits in 2^31
    const int chead = NGRP == 1 ? n % GS : n;     // head of this lane's column
    const int cpart = NGRP == 1 ? n / GS : 0;     // part of this lane's column (one group)
    const bool ccol = chead < G && (NGRP == 2 || cpart < NPART);

    // ---- entry table: lane l holds position, row and tile count of entry ec + l
    int ec = L0.ec, e_pos = L0.e_pos, e_row = L0.e_row, e_na = L0.e_na;
    int a = L0.a, h, j, na, row, pos;
    long long ebase = L0.tbase;
    auto entry = [&](int e, int &pos_o, int &row_o, int &na_o) {
        if (e < ec || e >= ec + 64) {  // wave-uniform; once per 64 entries
            ec = e & ~63;
            const int x = ec + lane, xc = min(x, ent.A - 1);
            e_pos = ent.positions[xc];
            e_row = ent.rows[xc];
            e_na = tiles_of(ent, x, e_pos, e_row);
        }
        pos_o = __shfl(e_pos, e - ec, 64);
        row_o = __shfl(e_row, e - ec, 64);
        na_o = __shfl(e_na, e - ec, 64);
    };
    entry(a, pos, row, na);

    // ---- tiles ahead of the current one (a, h, j), h the head group (this
    // wave's kv head is h HG + wi): nxt has its loads in flight while the
    // current tile is computed, nx2 is issued once nxt has landed
    struct TilePos {
        int a, h, j, na, row, pos;
        long long base;
    };
    auto advance = [&](TilePos &x) {  // x := the tile after x
        if (++x.j < x.na)
            return;
        x.j = 0;
        if (++x.h < NHG)
            return;
        x.h = 0;
        x.base += (long long)NHG * x.na;
        do {
            ++x.a;
            entry(x.a, x.pos, x.row, x.na);
        } while (x.na == 0 && x.a < ent.A);
    };
    {
        const long long loc = t0 - ebase;  // t0 is a tile of entry a
        h = (int)(loc / na);
        j = (int)(loc - (long long)h * na);
    }
    TilePos nxt = {a, h, j, na, row, pos, ebase}, nx2 = nxt;

    auto seg_base = [&](int srow, int hg, const uint16_t *blk) {
        return (const unsigned char *)(blk + (size_t)srow * p.C * slot + (size_t)(hg * HG + wi) * D);
    };

    u32x4 kn[NB][KS], vn[VLD];
    auto load_tile = [&](const unsigned char *kb, const unsigned char *vb, int jt, int jend) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const uint32_t off = (uint32_t)min(jt + b * 16 + n, jend - 1) * slotb + lg * 16;
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kn[b][ks] = __builtin_nontemporal_load((const u32x4 *)(kb + off + ks * 64));
        }
#pragma unroll
        for (int i = 0; i < VLD; ++i) {
            const uint32_t off = (uint32_t)min(jt + i * KPI + lane / LPK, jend - 1) * slotb +
                                 (lane % LPK) * 16;
            vn[i] = __builtin_nontemporal_load((const u32x4 *)(vb + off));
        }
    };
    auto store_tile = [&]() {
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                *(u32x4 *)(klds + (b * KS + ks) * 1024 + lane * 16) = kn[b][ks];
#pragma unroll
        for (int i = 0; i < VLD; ++i)
            *(u32x4 *)(vlds + (i * KPI + lane / LPK) * VROW + (lane % LPK) * 16) = vn[i];
    };
    // The segment's last tile, held by its owner: the key just stored replaces
    // the stale copy that was loaded, and keys past pos (clamped to pos, with
    // its stale bytes) get zero values, as they carry zero weight and a stale
    // NaN times zero would be NaN.
    auto patch_tile = [&](int kk) {
        const int b = kk >> 4, m = kk & 15;
        if (lane < LPK) {
            // 16-B chunk c = lane of the key: K operand slot (ks, lg) = (c / 4, c % 4)
            *(u32x4 *)(klds + (b * KS + (lane >> 2)) * 1024 + (m + 16 * (lane & 3)) * 16) =
                *(const u32x4 *)(newk + lane * 8);
            *(u32x4 *)(vlds + kk * VROW + lane * 16) = *(const u32x4 *)(newv + lane * 8);
        }
        for (int idx = lane; idx < (TK - 1 - kk) * LPK; idx += 64)
            *(u32x4 *)(vlds + (kk + 1 + idx / LPK) * VROW + (idx % LPK) * 16) =
                u32x4{0u, 0u, 0u, 0u};
    };

    // ---- segment inputs: the G query heads (16 B per lane per load), and for
    // the group that holds the segment's last tile the new key and value,
    // loaded into registers with the segment's first tile and moved to LDS
    // when the segment starts
    constexpr int QCH = D / 8;                          // 16-B chunks per head
    constexpr int NQL = (GCLS * QCH + 63) / 64;         // query loads per lane
    bool own_pre = false;
    int cs_entry = -1;  // entry whose cos/sin sit in cs/sn
    u32x4 qreg[NQL], kvreg = {0u, 0u, 0u, 0u};  // kvreg: lanes < LPK the key, next LPK the value
#pragma unroll
    for (int i = 0; i < NQL; ++i)
        qreg[i] = u32x4{0u, 0u, 0u, 0u};
    auto load_segment = [&](int ea, int hg, long long eb, int ena) {
        const int eh = hg * HG + wi;
        const uint16_t *qs = qp + ea * q_sa + eh * G * q_sh;
#pragma unroll
        for (int i = 0; i < NQL; ++i) {
            const int c = i * 64 + lane;
            if (c < G * QCH)
                qreg[i] = *(const u32x4 *)(qs + (c / QCH) * q_sh + (c % QCH) * 8);
        }
        own_pre = eb + (long long)hg * ena + ena - 1 < t1;  // holds the last tile
        if (own_pre && lane < 2 * LPK)
            kvreg = lane < LPK
                        ? *(const u32x4 *)(knp + ea * kn_sa + eh * kn_sh + lane * 8)
                        : *(const u32x4 *)(vnp + ea * vn_sa + eh * vn_sh + (lane - LPK) * 8);
    };
    // cos/sin of entry ea's angles, written by wave 0 for the whole group (ALU
    // only; the heads of an entry share them)
    auto angles = [&](int ea, int epos) {
        if (ea != cs_entry) {
            cs_entry = ea;
            if (wi == 0 && lane < D / 2) {
                const float theta = __fmul_rn((float)epos, my_freq);
                cs[lane] = (float)cos((double)theta);
                sn[lane] = (float)sin((double)theta);
            }
        }
    };

    // ---- per-segment state
    int nkeys = 0;
    bool owner = false;
    vec8 bq[NGRP][KS];
    float m_run, l_run;
    f32x4 O[NGRP][NDB];
    auto start_segment = [&](int hg, int erow, int epos) {
        const int eh = hg * HG + wi;
        pos = epos;
        nkeys = epos + 1;
        owner = own_pre;
#pragma unroll
        for (int i = 0; i < NQL; ++i) {
            const int c = i * 64 + lane;
            if (c < G * QCH)
                *(u32x4 *)(qlds + c * 8) = qreg[i];
        }
        if (owner && lane < 2 * LPK)
            *(u32x4 *)(lane < LPK ? kraw + lane * 8 : newv + (lane - LPK) * 8) = kvreg;
        __syncthreads();  // cs/sn from wave 0, the segment inputs from other lanes
        if (owner) {
            const size_t at = ((size_t)erow * p.C + epos) * slot + (size_t)eh * D;
            if (lane < D / 2) {
                float lo, hi;
                rope_pair(E::to_f(kraw[lane]), E::to_f(kraw[lane + D / 2]), cs[lane], sn[lane], lo,
                          hi);
                const uint16_t klo = (uint16_t)E::from_f(lo), khi = (uint16_t)E::from_f(hi);
                kcp[at + lane] = klo;
                kcp[at + lane + D / 2] = khi;
                newk[lane] = klo;
                newk[lane + D / 2] = khi;
            }
            if (lane >= LPK && lane < 2 * LPK)
                *(u32x4 *)(vcp + at + (lane - LPK) * 8) = kvreg;
        }
        // B operands of QK: the parts of the rotated query, by column; one
        // rotation pair of 32-dim blocks (ks, ks + KS/2) at a time
        const unsigned char *qrow = (const unsigned char *)qlds + (ccol ? chead : 0) * D * 2;
#pragma unroll
        for (int ks = 0; ks < KS / 2; ++ks) {
            const u32x4 vx = *(const u32x4 *)(qrow + (ks * 32 + lg * 8) * 2);
            const u32x4 vy = *(const u32x4 *)(qrow + ((ks + KS / 2) * 32 + lg * 8) * 2);
            float lo[8], hi[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
                const int i = ks * 32 + lg * 8 + jj;
                const float x = (jj & 1) ? E::hi(vx[jj >> 1]) : E::lo(vx[jj >> 1]);
                const float y = (jj & 1) ? E::hi(vy[jj >> 1]) : E::lo(vy[jj >> 1]);
                rope_pair(x, y, cs[i], sn[i], lo[jj], hi[jj]);
            }
#pragma unroll
            for (int c = 0; c < NGRP; ++c) {
                const int part = NGRP == 1 ? min(cpart, NPART - 1) : c;
                u32x4 wl, wh;
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    wl[e] = ccol ? E::template part<NPART>(lo[2 * e], part) |
                                       (E::template part<NPART>(lo[2 * e + 1], part) << 16)
                                 : 0u;
                    wh[e] = ccol ? E::template part<NPART>(hi[2 * e], part) |
                                       (E::template part<NPART>(hi[2 * e + 1], part) << 16)
                                 : 0u;
                }
                bq[c][ks] = __builtin_bit_cast(vec8, wl);
                bq[c][ks + KS / 2] = __builtin_bit_cast(vec8, wh);
            }
        }
        m_run = -INFINITY;
        l_run = 0.0f;
#pragma unroll
        for (int c = 0; c < NGRP; ++c)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
                O[c][db] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    };
    auto end_segment = [&](int ea, int hg) {
        float l = l_run;
        l += __shfl_xor(l, 16, 64);
        l += __shfl_xor(l, 32, 64);
        const size_t sl = ((size_t)(ea * NHG + hg + w) * HG + wi) * G;  // slot (seg + w, head)
        const bool writer = n < G;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            f32x4 o;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v;
                if (NGRP == 1) {
                    v = class_sum<GS>(ccol ? O[0][db][i] : 0.0f);
                } else {
                    v = O[0][db][i] + O[1][db][i];
                }
                o[i] = v;
            }
            if (writer)
                *(f32x4 *)(p.part_o + (sl + n) * D + db * 16 + lg * 4) = o;
        }
        if (writer && lg == 0) {
            float *dst = p.part_ml + (sl + n) * 2;
            dst[0] = m_run;
            dst[1] = l;
        }
    };

    // ---- first tile, then the next one in flight before the segment's start work
    load_segment(a, h, ebase, na);
    load_tile(seg_base(row, h, kcp), seg_base(row, h, vcp), j * TK, pos + 1);
    STAMP(6, wall_clock64());
    angles(a, pos);
    store_tile();
    STAMP(7, wall_clock64());
    if (t0 + 1 < t1) {
        advance(nxt);
        load_tile(seg_base(nxt.row, nxt.h, kcp), seg_base(nxt.row, nxt.h, vcp), nxt.j * TK,
                  nxt.pos + 1);
    }
    start_segment(h, row, pos);
    if (owner && j == na - 1)
        patch_tile(pos - j * TK);
    if (t0 + 1 < t1 && nxt.j == 0)
        load_segment(nxt.a, nxt.h, nxt.base, nxt.na);
    __syncthreads();
    STAMP(2, wall_clock64());
    STAMP(5, (unsigned long long)(t1 - t0));

    // Per tile t: tile t is in LDS, t + 1 (nxt) in flight.  After t is
    // computed, t + 1 moves to LDS and t + 2 (nx2) is issued at once, so the
    // segment end / start work that follows runs with loads in flight.
    // quarter of the range reached and the tile where the next one starts:
    // quarter q from tile t0 + ceil(q (t1 - t0) / 4)
    int prio_q = 0;
    long long prio_at = t0;
    for (long long t = t0; t < t1; ++t) {
        const bool more = t + 1 < t1, more2 = t + 2 < t1;
        while (prio_q < 4 && t >= prio_at) {  // at most four steps in all
            set_range_priority(prio_q);
            ++prio_q;
            prio_at = t0 + (prio_q * (t1 - t0) + 3) / 4;
        }
        // cos/sin of a segment that starts at t + 1, used at the end of this
        // iteration (the last reads of cs/sn were fenced by the barrier that
        // ended the previous iteration; the barrier below publishes these)
        if (more && nxt.j == 0)
            angles(nxt.a, nxt.pos);
        const bool seg_ends = !more || nxt.j == 0;
        const int jt = j * TK;
        // QK: lane (n, lg) gets keys jt + 16 b + 4 lg + i of column n
        f32x4 acc[NB][NGRP];
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int c = 0; c < NGRP; ++c)
                acc[b][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            u32x4 kf[KS];
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
                kf[ks] = *(const u32x4 *)(klds + (b * KS + ks) * 1024 + lane * 16);
#pragma unroll
            for (int ks = 0; ks < KS; ++ks)
#pragma unroll
                for (int c = 0; c < NGRP; ++c)
                    acc[b][c] = E::mma16(__builtin_bit_cast(vec8, kf[ks]), bq[c][ks], acc[b][c]);
        }
        // the scheduler keeps each block's fragment reads together, ahead of its products
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);
            __builtin_amdgcn_sched_group_barrier(0x008, KS * NGRP, 0);
        }
        float sc[NB][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float v;
                if (NGRP == 1) {
                    v = class_sum<GS>(ccol ? acc[b][0][i] : 0.0f);
                } else {
                    v = acc[b][0][i] + acc[b][1][i];
                }
                v = (jt + b * 16 + lg * 4 + i < nkeys) ? v * p.scale_log2 : -INFINITY;
                sc[b][i] = v;
                tmax = fmaxf(tmax, v);
            }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
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

        // PV: k slot jj < 4 is key 4 lg + jj of block 0, slot 4 + jj of block 1
        vec8 pb[NGRP];
#pragma unroll
        for (int c = 0; c < NGRP; ++c) {
            const int part = NGRP == 1 ? min(cpart, NPART - 1) : c;
            u32x4 v;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int b = e >> 1, i = (e & 1) * 2;
                v[e] = E::template part<NPART>(pv[b][i], part) |
                       (E::template part<NPART>(pv[b][i + 1], part) << 16);
            }
            pb[c] = __builtin_bit_cast(vec8, v);
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
            const vec8 vt = __builtin_bit_cast(vec8, vv);
#pragma unroll
            for (int c = 0; c < NGRP; ++c)
                O[c][db] = E::mma16(vt, pb[c], O[c][db]);
        }
        __syncthreads();  // LDS of tile t fully read

        // the one wait per tile: t + 1 into LDS; then t + 2 goes out before
        // this segment's partial and the next segment's start
        if (more) {
            store_tile();
            if (more2) {
                nx2 = nxt;
                advance(nx2);
                load_tile(seg_base(nx2.row, nx2.h, kcp), seg_base(nx2.row, nx2.h, vcp),
                          nx2.j * TK, nx2.pos + 1);
            }
        }
        if (seg_ends)
            end_segment(a, h);
        if (more) {
            if (seg_ends)
                start_segment(nxt.h, nxt.row, nxt.pos);
            a = nxt.a;
            h = nxt.h;
            j = nxt.j;
            na = nxt.na;
            row = nxt.row;
            ebase = nxt.base;
            nxt = nx2;
            if (owner && j == na - 1)
                patch_tile(pos - j * TK);
            // the segment inputs of t + 2, once this segment's start has read the registers
            if (more2 && nxt.j == 0)
                load_segment(nxt.a, nxt.h, nxt.base, nxt.na);
            __syncthreads();
        }
    }

    STAMP(3, wall_clock64());
}

// ---------------------------------------------------------------- R4
// One wave per (entry, query head): the partials of segment (a, h = hq / G)
// sit in slots seg + w for the groups w that touched it (the plan of the
// decode kernel, whose prefix it left in the workspace); they are summed with
// weights 2^(m_w - M), divided by the weighted sum of l_w and rounded to the
// storage type.  An entry with an out-of-range position or row gets a NaN
// output and sets the status word.  The loads are issued in as few round trips
// as the data allows: the entry's indices together with its plan prefix, then
// every (max, sum) pair together with up to kMergeBatch partial outputs per
// lane.
constexpr int kMergeBatch = 16;

// The merge waves: one per (entry, query head), WPG to a work group in a
// one-dimensional grid (the y and z grid sizes are limited).  The waves of a
// group share nothing.  Four to a group for the merge of many rows, where
// thousands of one-wave groups had to be started; one for the wide merge of
// a few long rows, whose few waves each wait on many loads and ran slower
// when four shared a compute unit.
constexpr int kMergeWaves = 4, kMergeWideWaves = 1;
template <int WPG>
__device__ __forceinline__ bool merge_wave(const DecodeParams &p, int &a, int &hq)
{
    const unsigned id = blockIdx.x * WPG + (threadIdx.x >> 6);
    if (id >= (unsigned)p.A * (unsigned)p.Hq)
        return false;  // the last group's spare waves
    hq = (int)(id % (unsigned)p.Hq);
    a = (int)(id / (unsigned)p.Hq);
    return true;
}

template <class E, int D>
__global__ __launch_bounds__(64 * kMergeWaves) void k_decode_merge(DecodeParams p)
{
    constexpr int PER = D / 64;
    int a, hq;
    if (!merge_wave<kMergeWaves>(p, a, hq))
        return;
    const int lane = threadIdx.x & 63;
    const int pos = p.positions[a], row = p.rows[a];
    const long long before = p.plan[a], NT = p.plan[p.A], NSEG = p.plan[p.A + 1];
    uint16_t *out = p.out + a * p.o_sa + hq * p.o_sh;
    if (!entry_valid(p, pos, row)) {
#pragma unroll
        for (int e = 0; e < PER; ++e)
            out[lane + 64 * e] = E::qnan;
        if (hq == 0 && lane == 0 && p.status)
            p.status[0] = 1;
        return;
    }
    const int G = p.G, h = hq / G, g = hq - h * G, HG = p.HG, NHG = p.NHG;
    const int hg = h / HG, wi = h - hg * HG;  // head group, wave of the group
    const int NW = plan_waves(p.NS, NT);      // NT >= 1: this entry is valid
    const Plan P = make_plan(p, NT, NSEG, NW);
    const int na = (pos + kTile) / kTile;
    // the groups that own the segment's first and last tiles, by their units
    const long long us = before + (long long)hg * units_of(P, na) + P.su;
    const int wf = plan_wave_of(P, us), wl = plan_wave_of(P, us + na - 1);
    const int ns = wl - wf + 1;
    // partial of group wf + x for this head: (max, sum) and D outputs
    auto slot_of = [&](int x) { return ((size_t)(a * NHG + hg + wf + x) * HG + wi) * G + g; };
    float lw = 0.0f, O[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e)
        O[e] = 0.0f;
    float M = -INFINITY;
    for (int c = 0; c < ns; c += 64) {
        // lane u holds the (max, sum) of slot c + u; every lane loads its
        // elements of the first batch of outputs in the same round trip
        float m_u = -INFINITY, l_u = 0.0f;
        if (c + lane < ns) {
            const float2 ml = *(const float2 *)(p.part_ml + slot_of(c + lane) * 2);
            m_u = ml.x;
            l_u = ml.y;
        }
        const int cnt = min(64, ns - c);
        float x[kMergeBatch][PER];
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u)
#pragma unroll
            for (int e = 0; e < PER; ++e)
                x[u][e] = u < cnt ? p.part_o[slot_of(c + u) * D + lane + 64 * e] : 0.0f;
        // rescale what earlier batches of 64 slots summed to the new maximum
        const float m_new = fmaxf(M, wave_max(m_u));
        const float alpha = exp2f(M - m_new);  // 0 on the first batch (M = -inf)
        lw *= alpha;
#pragma unroll
        for (int e = 0; e < PER; ++e)
            O[e] *= alpha;
        M = m_new;
        const float wgt = c + lane < ns ? exp2f(m_u - M) : 0.0f;
        lw += wgt * l_u;
#pragma unroll
        for (int u = 0; u < kMergeBatch; ++u) {
            const float wk = __shfl(wgt, u, 64);
#pragma unroll
            for (int e = 0; e < PER; ++e)
                O[e] += wk * x[u][e];
        }
        for (int k = kMergeBatch; k < cnt; k += kMergeBatch) {
            const int left = min(kMergeBatch, cnt - k);
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u)
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    x[u][e] = u < left ? p.part_o[slot_of(c + k + u) * D + lane + 64 * e] : 0.0f;
#pragma unroll
            for (int u = 0; u < kMergeBatch; ++u) {
                const float wk = __shfl(wgt, k + u, 64);
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    O[e] += wk * x[u][e];
            }
        }
    }
    const float L = wave_sum(lw);
#pragma unroll
    for (int e = 0; e < PER; ++e)
        out[lane + 64 * e] = (uint16_t)E::from_f(O[e] / L);
}

// ---------------------------------------------------------------- R4 (wide)
// The same merge for rows split over many groups (small batches, fan-in of
// tens to hundreds): per batch of up to 64 groups their (max, sum) pairs and
// every lane's PER consecutive output dims (one vector load per group, at a
// constant stride from one base), so a fan-in of 100 takes two trips where
// the kernel above takes seven.
template <class E, int D>
__global__ __launch_bounds__(64 * kMergeWideWaves) void k_decode_merge_wide(DecodeParams p)
{
    constexpr int B = 64, CH = 8;  // groups per round trip, per load chunk
    constexpr int PER = D / 64;  // lane l owns the output dims PER l .. PER l + PER - 1
    int a, hq;
    if (!merge_wave<kMergeWideWaves>(p, a, hq))
        return;
    const int lane = threadIdx.x & 63;
    const int pos = p.positions[a], row = p.rows[a];
    const long long before = p.plan[a], NT = p.plan[p.A], NSEG = p.plan[p.A + 1];
    uint16_t *out = p.out + a * p.o_sa + hq * p.o_sh + lane * PER;
    if (!entry_valid(p, pos, row)) {
#pragma unroll
        for (int e = 0; e < PER; ++e)
            out[e] = E::qnan;
        if (hq == 0 && lane == 0 && p.status)
            p.status[0] = 1;
        return;
    }
    const int G = p.G, h = hq / G, g = hq - h * G, HG = p.HG, NHG = p.NHG;
    const int hg = h / HG, wi = h - hg * HG;  // head group, wave of the group
    const int NW = plan_waves(p.NS, NT);      // NT >= 1: this entry is valid
    const Plan P = make_plan(p, NT, NSEG, NW);
    const int na = (pos + kTile) / kTile;
    // the groups that own the segment's first and last tiles, by their units
    const long long us = before + (long long)hg * units_of(P, na) + P.su;
    const int wf = plan_wave_of(P, us), wl = plan_wave_of(P, us + na - 1);
    const int ns = wl - wf + 1;
    // the partial of group wf + x for this head sits in slot slot0 + x * step:
    // (max, sum) pairs step apart, outputs step * D floats apart (at most
    // 8 * 16 * 128 * 4 B, so 64 of them span less than 2^32 bytes)
    const size_t slot0 = ((size_t)(a * NHG + hg + wf) * HG + wi) * G + g;
    const size_t step = (size_t)HG * G;
    const float2 *ml_base = (const float2 *)p.part_ml + slot0;
    const unsigned char *o_base = (const unsigned char *)(p.part_o + slot0 * D);
    const uint32_t o_step = (uint32_t)(step * D * 4), o_lane = (uint32_t)(lane * PER * 4);
    float lw = 0.0f, O[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e)
        O[e] = 0.0f;
    float M = -INFINITY;
    // batches of up to B groups, each in one round trip: lane u loads the
    // (max, sum) of group c + u, and every lane its dims of every output
    for (int c = 0; c < ns; c += B) {
        float m_u = -INFINITY, l_u = 0.0f;
        if (c + lane < ns) {
            const float2 ml = ml_base[(size_t)(c + lane) * step];
            m_u = ml.x;
            l_u = ml.y;
        }
        const int cnt = min(B, ns - c);
        const unsigned char *ob = o_base + (size_t)c * o_step;
        // outputs in chunks of CH groups; within a started chunk, groups past
        // cnt re-read group cnt - 1 (in bounds, finite) and get weight 0
        float x[B][PER];
#pragma unroll
        for (int k = 0; k < B; k += CH) {
            if (k < cnt) {
#pragma unroll
                for (int u = k; u < k + CH; ++u) {
                    const unsigned char *src = ob + (uint32_t)min(u, cnt - 1) * o_step + o_lane;
                    if constexpr (PER == 2) {
                        const float2 v = *(const float2 *)src;
                        x[u][0] = v.x;
                        x[u][1] = v.y;
                    } else {
                        x[u][0] = *(const float *)src;
                    }
                }
            } else {
#pragma unroll
                for (int u = k; u < k + CH; ++u)
#pragma unroll
                    for (int e = 0; e < PER; ++e)
                        x[u][e] = 0.0f;
            }
        }
        // rescale what earlier batches summed to the new maximum
        const float m_new = fmaxf(M, wave_max(m_u));
        const float alpha = exp2f(M - m_new);  // 0 on the first batch (M = -inf)
        lw *= alpha;
#pragma unroll
        for (int e = 0; e < PER; ++e)
            O[e] *= alpha;
        M = m_new;
        const float wgt = c + lane < ns ? exp2f(m_u - M) : 0.0f;
        lw += wgt * l_u;
#pragma unroll
        for (int u = 0; u < B; ++u) {
            const float wk = __shfl(wgt, u, 64);
#pragma unroll
            for (int e = 0; e < PER; ++e)
                O[e] += wk * x[u][e];
        }
    }
    const float L = wave_sum(lw);
    if constexpr (PER == 2)  // both values in one 4-byte store (rows are 16-byte aligned)
        *(uint32_t *)out = (uint32_t)(uint16_t)E::from_f(O[0] / L) |
                           ((uint32_t)(uint16_t)E::from_f(O[1] / L) << 16);
    else
        out[0] = (uint16_t)E::from_f(O[0] / L);
}

}  // namespace

DecodeWorkspace decode_workspace_layout(int64_t A, int64_t Hq, int64_t Hkv, int64_t D,
                                        int64_t NS)
{
    auto up = [](uint64_t x) { return (x + 255u) & ~uint64_t(255); };
    DecodeWorkspace w;
    w.qrot_off = 0;
    // partial slots: at most A * Hkv + NS (waves of the launch), G heads each
    const uint64_t slots = ((uint64_t)A * Hkv + NS) * (Hq / Hkv);
    w.part_o_off = up(w.qrot_off + (uint64_t)A * Hq * D * 4);
    w.part_ml_off = up(w.part_o_off + slots * D * 4);
    w.plan_off = up(w.part_ml_off + slots * 2 * 4);
    w.total = up(w.plan_off + ((uint64_t)A + 2) * 8);
    return w;
}

hipError_t launch_rope_store(const DecodeParams &p, hipStream_t stream)
{
    if (p.dtype == F16::code)
        hipLaunchKernelGGL(k_rope_store<F16>, dim3(p.A), dim3(256), 0, stream, p);
    else
        hipLaunchKernelGGL(k_rope_store<Bf16>, dim3(p.A), dim3(256), 0, stream, p);
    return hipGetLastError();
}

template <class E, int D, int GCLS>
static hipError_t launch_stream_v(const DecodeParams &p, hipStream_t stream, hipEvent_t e0,
                                  hipEvent_t e1)
{
    const int lds = decode_lds_bytes<D, GCLS>(p.HG);
    static std::once_flag once;
    static hipError_t attr = hipSuccess;
    std::call_once(once, [] {
        attr = hipFuncSetAttribute((const void *)k_decode_stream<E, D, GCLS>,
                                   hipFuncAttributeMaxDynamicSharedMemorySize,
                                   decode_lds_bytes<D, GCLS>(GCLS == 16 ? 4 : 8));
    });
    if (attr != hipSuccess)
        return attr;
    hipExtLaunchKernelGGL((k_decode_stream<E, D, GCLS>), dim3(p.NS), dim3(64 * p.HG), lds, stream,
                          e0, e1, 0, p);
    return hipGetLastError();
}

template <class E, int D>
static hipError_t launch_stream_d(const DecodeParams &p, hipStream_t stream, hipEvent_t e0,
                                  hipEvent_t e1)
{
    if (p.G <= 1)
        return launch_stream_v<E, D, 1>(p, stream, e0, e1);
    if (p.G <= 2)
        return launch_stream_v<E, D, 2>(p, stream, e0, e1);
    if (p.G <= 4)
        return launch_stream_v<E, D, 4>(p, stream, e0, e1);
    if (p.G <= 8)
        return launch_stream_v<E, D, 8>(p, stream, e0, e1);
    return launch_stream_v<E, D, 16>(p, stream, e0, e1);
}

template <class E>
static hipError_t launch_stream_e(const DecodeParams &p, hipStream_t stream, hipEvent_t e0,
                                  hipEvent_t e1)
{
    return p.D == 64 ? launch_stream_d<E, 64>(p, stream, e0, e1)
                     : launch_stream_d<E, 128>(p, stream, e0, e1);
}

hipError_t launch_decode_fused(const DecodeParams &p, hipStream_t stream, hipEvent_t e0,
                               hipEvent_t e1)
{
    return p.dtype == F16::code ? launch_stream_e<F16>(p, stream, e0, e1)
                                : launch_stream_e<Bf16>(p, stream, e0, e1);
}

// A segment's fan-in is about NS / (A * NHG) + 1 groups when every launched
// group holds tiles.  Above 12 the wide merge runs (measured on MI355X: A = 1
// 9.7 -> 6.6 us, A = 8 6.5 -> 4.9 us), below it the narrow one (fan-in 2-9:
// 5-6 us, where the wide one measured 0.2-0.9 us slower).
template <class E, int D>
static void launch_merge_d(const DecodeParams &p, hipStream_t stream)
{
    const int waves = p.Hq * p.A;
    if ((long long)p.NS > 12ll * p.A * p.NHG)
        hipLaunchKernelGGL((k_decode_merge_wide<E, D>),
                           dim3((waves + kMergeWideWaves - 1) / kMergeWideWaves),
                           dim3(64 * kMergeWideWaves), 0, stream, p);
    else
        hipLaunchKernelGGL((k_decode_merge<E, D>), dim3((waves + kMergeWaves - 1) / kMergeWaves),
                           dim3(64 * kMergeWaves), 0, stream, p);
}

template <class E>
static void launch_merge_e(const DecodeParams &p, hipStream_t stream)
{
    if (p.D == 64)
        launch_merge_d<E, 64>(p, stream);
    else
        launch_merge_d<E, 128>(p, stream);
}

hipError_t launch_decode_merge(const DecodeParams &p, hipStream_t stream)
{
    if (p.dtype == F16::code)
        launch_merge_e<F16>(p, stream);
    else
        launch_merge_e<Bf16>(p, stream);
    return hipGetLastError();
}

// Four kv heads per group: two groups share a compute unit, so one streams
// while the other waits at a barrier (measured on MI355X: 4 beats 8 by 2-5 %,
// and beats 2 and 1 on the ragged batch).
#ifndef MLLM_HEAD_GROUP_CAP
#define MLLM_HEAD_GROUP_CAP 4
#endif
int decode_head_group(int Hkv, int G)
{
    const int cap = G > 8 ? 4 : MLLM_HEAD_GROUP_CAP;
    int hg = 1;
    while (hg * 2 <= cap && Hkv % (hg * 2) == 0)
        hg *= 2;
    return hg;
}

template <class E, int D, int GCLS>
static int resident_groups_v(int cus, int HG)
{
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k_decode_stream<E, D, GCLS>, 64 * HG,
                                                     decode_lds_bytes<D, GCLS>(HG)) != hipSuccess)
        return 0;
    return cus * per_cu;
}

template <class E, int D>
static int resident_groups_d(int cus, int G, int HG)
{
    return G <= 1 ? resident_groups_v<E, D, 1>(cus, HG)
         : G <= 2 ? resident_groups_v<E, D, 2>(cus, HG)
         : G <= 4 ? resident_groups_v<E, D, 4>(cus, HG)
         : G <= 8 ? resident_groups_v<E, D, 8>(cus, HG)
                  : resident_groups_v<E, D, 16>(cus, HG);
}

int decode_resident_groups(int device, int D, int G, int HG, int dtype)
{
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess)
        return 0;
    if (dtype == F16::code)
        return D == 64 ? resident_groups_d<F16, 64>(cus, G, HG) : resident_groups_d<F16, 128>(cus, G, HG);
    return D == 64 ? resident_groups_d<Bf16, 64>(cus, G, HG) : resident_groups_d<Bf16, 128>(cus, G, HG);
}

template <class E>
static void launch_readable_e(const DecodeParams &p, hipStream_t stream, hipEvent_t e0, hipEvent_t e1)
{
    const dim3 grid(p.Hq * p.A), block(64);
    if (p.D == 64)
        hipExtLaunchKernelGGL((k_decode_readable<E, 64>), grid, block, 0, stream, e0, e1, 0, p);
    else
        hipExtLaunchKernelGGL((k_decode_readable<E, 128>), grid, block, 0, stream, e0, e1, 0, p);
}

hipError_t launch_decode_readable(const DecodeParams &p, hipStream_t stream, hipEvent_t e0,
                                  hipEvent_t e1)
{
    if (p.dtype == F16::code)
        launch_readable_e<F16>(p, stream, e0, e1);
    else
        launch_readable_e<Bf16>(p, stream, e0, e1);
    return hipGetLastError();
}

#ifdef MLLM_STAMPS
extern "C" int mllm_debug_stamps(void *dst, size_t bytes)
{
    return (int)hipMemcpyFromSymbol(dst, HIP_SYMBOL(mllm_stamps), bytes);
}
#endif
}  // namespace mllm
