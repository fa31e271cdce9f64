/*
 * oracle.c -- plain, slow, single-threaded CPU oracle for the positions-aware
 * cached decode step and the equal-length batched prefill (also as a chunk
 * appended at per-row start positions).
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU
 * baseline leg of the benchmark may load this library.  The product path
 * (the HIP library under positions_aware_cached_amd/) never calls it, and the
 * two share no code, header, table or helper.
 *
 * What is computed (microLLM-rocm ARCHITECTURE.md, "Tensor ownership boundary"):
 * for A active entries, each with its own position p and shared-cache row r,
 *   1. rotate K (and Q) of the new token by split-half RoPE at position p
 *      (same page, "Attention layout boundary": split-half RoPE, even D,
 *      non-negative position, positive base);
 *   2. store the rotated K and the raw V of the token into row r, slot p, of a
 *      persistent [slots, capacity, H_kv, D] BF16 cache; nothing else written;
 *   3. causal GQA attention of each query head against keys 0..p of row r, the
 *      softmax reduced in FP32 and only the BF16 output rounded
 *      (operator-development.md, "Public interfaces": typed FP16/BF16 softmax
 *      reduces in FP32 registers and rounds only the caller output).
 * The serial per-row loop mirrors the pages' serial B=1 oracle
 * (forward_cached_rows / forward_prefill_cached_row, "Tensor ownership
 * boundary"): no blocking, no splitting, no fusion.
 *
 * Readings of points the pages leave open (each listed in the design notes):
 *  - RoPE frequencies: inv_freq[i] = base^(-2i/D), i < D/2 (RoFormer form),
 *    evaluated in double and rounded once to FP32; angle = fl32(fl32(p) *
 *    inv_freq[i]); cos/sin of that FP32 angle evaluated in double, rounded
 *    once to FP32.  Pairing is (i, i + D/2) ("split-half").
 *  - Rotation: lo = x*c - y*s, hi = y*c + x*s, each product and the sum
 *    rounded to FP32 separately (no fused multiply-add).
 *  - GQA: query head hq reads kv head hq / (H_q / H_kv) (heads repeated, not
 *    cycled: "GQA repeats/reduces Q/K heads on dimension 1").
 *  - Scores: s_j = fl32( (sum over d ascending of q'_d * k_jd) * fl32(1/sqrt(D)) );
 *    softmax m = max s_j, e_j = expf(s_j - m), l = sum e_j (ascending j);
 *    o_d = (sum_j e_j v_jd) / l, then BF16 round-to-nearest-even.
 *  - The new token's key (j = p) is read back from the cache after the store,
 *    i.e. it is the BF16-rounded rotated key.
 *  - Position p is the slot the token is stored in; attention covers the
 *    p + 1 keys 0..p inclusive.
 *  - A prefill chunk of T tokens appended at a nonzero start s (rows that
 *    already hold s tokens) is T decode steps at positions s..s+T-1 taken
 *    together; the pages only define the start-0 case (empty rows).
 *  - A batch whose entries have different lengths is the separate
 *    equal-length groups the pages form, run one after another.
 *  - FP16 storage (the pages' typed softmax covers FP16 and BF16) follows the
 *    same steps with IEEE binary16 conversions: exact widening, and
 *    round-to-nearest-even narrowing with subnormals and overflow to infinity.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (see oracle/build.py).  -ffp-contract=off keeps every product rounded.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------- BF16 <-> FP32 ------------------------------------------------ */

/* BF16 is the top half of an IEEE binary32. */
float orc_bf16_to_f32(uint16_t h)
{
    uint32_t u = ((uint32_t)h) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* FP32 -> BF16, round to nearest, ties to even.  NaN stays a quiet NaN. */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0u)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t keep = u >> 16;
    uint32_t rest = u & 0xffffu;
    if (rest > 0x8000u || (rest == 0x8000u && (keep & 1u)))
        keep += 1u; /* carries into the exponent correctly, up to infinity */
    return (uint16_t)keep;
}

/* ---------- FP16 <-> FP32 (IEEE 754 binary16) ----------------------------- */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits; exponent 0
 * holds the subnormals frac * 2^-24, exponent 31 infinity and NaN. */
float orc_f16_to_f32(uint16_t h)
{
    const int neg = h >> 15, ex = (h >> 10) & 31, fr = h & 1023;
    if (ex == 31) {
        uint32_t u = ((uint32_t)neg << 31) | 0x7f800000u | ((uint32_t)fr << 13);
        float f;
        memcpy(&f, &u, sizeof f);
        return f;
    }
    double v = ex == 0 ? ldexp((double)fr, -24) : ldexp((double)(1024 + fr), ex - 25);
    return (float)(neg ? -v : v);
}

/* FP32 -> FP16, round to nearest, ties to even, through the subnormal range;
 * magnitudes from 65520 (the midpoint above the largest finite 65504, which
 * ties to the even neighbour 2^16) become infinity; NaN stays a quiet NaN. */
uint16_t orc_f32_to_f16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)(sign | 0x7e00u | ((u >> 13) & 0x3ffu));
    const double x = fabs((double)f);
    if (x >= 65520.0)
        return (uint16_t)(sign | 0x7c00u);
    if (x == 0.0)
        return sign;
    int e;
    frexp(x, &e);           /* x = m 2^e, 0.5 <= m < 1: binade of x is e - 1 */
    int ex = e - 1;
    if (ex < -14)
        ex = -14;           /* subnormals share the quantum of the lowest binade */
    const double n = x / ldexp(1.0, ex - 10);  /* x in quanta of its binade: exact */
    double r = floor(n);
    const double fr = n - r;
    if (fr > 0.5 || (fr == 0.5 && fmod(r, 2.0) == 1.0))
        r += 1.0;
    if (r < 1024.0)         /* only in the lowest binade: a subnormal (or zero) */
        return (uint16_t)(sign | (uint16_t)r);
    if (r == 2048.0) {      /* rounded up into the next binade */
        r = 1024.0;
        ex += 1;
    }
    return (uint16_t)(sign | (uint16_t)((ex + 15) << 10) | (uint16_t)(r - 1024.0));
}

/* Storage types of the cache and the call's tensors. */
#define ORC_BF16 1
#define ORC_F16 2

static float to_f32(int dt, uint16_t h)
{
    return dt == ORC_F16 ? orc_f16_to_f32(h) : orc_bf16_to_f32(h);
}

static uint16_t from_f32(int dt, float f)
{
    return dt == ORC_F16 ? orc_f32_to_f16(f) : orc_f32_to_bf16(f);
}

/* ---------- RoPE ---------------------------------------------------------- */

/* inv_freq[i] = fl32(base^(-2i/D)) for i = 0 .. D/2-1. */
void orc_rope_inv_freq(double base, int D, float *inv_freq)
{
    for (int i = 0; i < D / 2; ++i)
        inv_freq[i] = (float)pow(base, -2.0 * (double)i / (double)D);
}

/* cos/sin of the FP32 angle fl32(fl32(pos) * inv_freq[i]). */
void orc_rope_cos_sin(int pos, int D, const float *inv_freq, float *c, float *s)
{
    for (int i = 0; i < D / 2; ++i) {
        float p = (float)pos;
        float theta = p * inv_freq[i];
        c[i] = (float)cos((double)theta);
        s[i] = (float)sin((double)theta);
    }
}

/* Rotate one head vector x[D] (FP32) by the tables c/s; pairs (i, i+D/2). */
void orc_rope_apply(const float *x, int D, const float *c, const float *s, float *y)
{
    int h = D / 2;
    for (int i = 0; i < h; ++i) {
        float a = x[i];
        float b = x[i + h];
        float ac = a * c[i];
        float bs = b * s[i];
        float bc = b * c[i];
        float as = a * s[i];
        y[i] = ac - bs;
        y[i + h] = bc + as;
    }
}

/* ---------- argument checks (the pages: unsupported input fails explicitly) */

#define ORC_OK 0
#define ORC_ERR_SHAPE 1
#define ORC_ERR_INDEX 2
#define ORC_ERR_DUP_ROW 3
#define ORC_ERR_NOMEM 4

static int check_shapes(int A, int S, int C, int Hq, int Hkv, int D)
{
    if (A < 0 || S <= 0 || C <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0)
        return ORC_ERR_SHAPE;
    if (D % 2 != 0 || Hq % Hkv != 0)
        return ORC_ERR_SHAPE;
    return ORC_OK;
}

static int check_rows_unique(int A, int S, const int32_t *rows)
{
    for (int a = 0; a < A; ++a) {
        if (rows[a] < 0 || rows[a] >= S)
            return ORC_ERR_INDEX;
        for (int b = 0; b < a; ++b)
            if (rows[b] == rows[a])
                return ORC_ERR_DUP_ROW;
    }
    return ORC_OK;
}

/* ---------- attention of one query vector over keys 0..last of one row ---- */

/*
 * q_rot: rotated query (FP32, unrounded), D values.
 * Kr, Vr: the cache row base for kv head kv: element (j, d) at [j*row_stride + d].
 * out_bits: D values of storage type dt.  e: scratch of last+1 floats.
 */
static void attend_one(int dt, const float *q_rot, int D, const uint16_t *Kr,
                       const uint16_t *Vr, long row_stride, int last, float scale, float *e,
                       uint16_t *out_bits, float *out_f32)
{
    float m = -INFINITY;
    for (int j = 0; j <= last; ++j) {
        const uint16_t *k = Kr + (long)j * row_stride;
        float dot = 0.0f;
        for (int d = 0; d < D; ++d)
            dot = dot + q_rot[d] * to_f32(dt, k[d]);
        float sj = dot * scale;
        e[j] = sj;
        if (sj > m)
            m = sj;
    }
    float l = 0.0f;
    for (int j = 0; j <= last; ++j) {
        e[j] = expf(e[j] - m);
        l = l + e[j];
    }
    for (int d = 0; d < D; ++d) {
        float acc = 0.0f;
        for (int j = 0; j <= last; ++j)
            acc = acc + e[j] * to_f32(dt, Vr[(long)j * row_stride + d]);
        float o = acc / l;
        if (out_f32)
            out_f32[d] = o;
        out_bits[d] = from_f32(dt, o);
    }
}

/* ---------- the decode step ------------------------------------------------ */

/*
 * One layer of the positions-aware cached decode step.
 *
 *  dt     storage type of every 16-bit tensor: ORC_BF16 or ORC_F16
 *         (operator-development.md, "Public interfaces": typed FP16/BF16
 *         softmax with FP32 reduction)
 *  q      [A, Hq, D]  bits           k_new, v_new [A, Hkv, D] bits
 *  pos    [A] int32 in [0, C)        rows [A] int32 in [0, S), distinct
 *  Kc, Vc [S, C, Hkv, D] bits, updated in place (only (rows[a], pos[a]))
 *  out    [A, Hq, D] bits            out_f32: optional [A, Hq, D] FP32 before rounding
 *
 * Returns 0, or a nonzero code with nothing written when an argument is invalid.
 */
int orc_decode_step_dt(int dt, int A, int S, int C, int Hq, int Hkv, int D, double base,
                       const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                       const int32_t *pos, const int32_t *rows, uint16_t *Kc, uint16_t *Vc,
                       uint16_t *out, float *out_f32)
{
    if (dt != ORC_BF16 && dt != ORC_F16)
        return ORC_ERR_SHAPE;
    int rc = check_shapes(A, S, C, Hq, Hkv, D);
    if (rc)
        return rc;
    rc = check_rows_unique(A, S, rows);
    if (rc)
        return rc;
    for (int a = 0; a < A; ++a)
        if (pos[a] < 0 || pos[a] >= C)
            return ORC_ERR_INDEX;

    const int G = Hq / Hkv;
    const long slot = (long)Hkv * D;        /* elements per (row, position) */
    const long row = (long)C * slot;         /* elements per cache row */
    const float scale = (float)(1.0 / sqrt((double)D));

    float *inv_freq = malloc(sizeof(float) * (size_t)(D / 2));
    float *cs = malloc(sizeof(float) * (size_t)(D / 2));
    float *sn = malloc(sizeof(float) * (size_t)(D / 2));
    float *x = malloc(sizeof(float) * (size_t)D);
    float *y = malloc(sizeof(float) * (size_t)D);
    int maxpos = 0;
    for (int a = 0; a < A; ++a)
        if (pos[a] > maxpos)
            maxpos = pos[a];
    float *e = malloc(sizeof(float) * (size_t)(maxpos + 1));
    if (!inv_freq || !cs || !sn || !x || !y || !e) {
        free(inv_freq); free(cs); free(sn); free(x); free(y); free(e);
        return ORC_ERR_NOMEM;
    }
    orc_rope_inv_freq(base, D, inv_freq);

    /* steps 1-2: rotate K, store K and V of every active entry */
    for (int a = 0; a < A; ++a) {
        orc_rope_cos_sin(pos[a], D, inv_freq, cs, sn);
        for (int h = 0; h < Hkv; ++h) {
            const uint16_t *k = k_new + ((long)a * Hkv + h) * D;
            const uint16_t *v = v_new + ((long)a * Hkv + h) * D;
            uint16_t *kd = Kc + rows[a] * row + (long)pos[a] * slot + (long)h * D;
            uint16_t *vd = Vc + rows[a] * row + (long)pos[a] * slot + (long)h * D;
            for (int d = 0; d < D; ++d)
                x[d] = to_f32(dt, k[d]);
            orc_rope_apply(x, D, cs, sn, y);
            for (int d = 0; d < D; ++d) {
                kd[d] = from_f32(dt, y[d]);
                vd[d] = v[d];
            }
        }
    }

    /* step 3: causal GQA attention of each rotated query over keys 0..pos */
    for (int a = 0; a < A; ++a) {
        orc_rope_cos_sin(pos[a], D, inv_freq, cs, sn);
        for (int hq = 0; hq < Hq; ++hq) {
            int kv = hq / G;
            const uint16_t *qa = q + ((long)a * Hq + hq) * D;
            for (int d = 0; d < D; ++d)
                x[d] = to_f32(dt, qa[d]);
            orc_rope_apply(x, D, cs, sn, y);
            const uint16_t *Kr = Kc + rows[a] * row + (long)kv * D;
            const uint16_t *Vr = Vc + rows[a] * row + (long)kv * D;
            long o = ((long)a * Hq + hq) * D;
            attend_one(dt, y, D, Kr, Vr, slot, pos[a], scale, e, out + o,
                       out_f32 ? out_f32 + o : NULL);
        }
    }
    free(inv_freq); free(cs); free(sn); free(x); free(y); free(e);
    return ORC_OK;
}

/* ---------- equal-length batched prefill --------------------------------- */

/*
 * Prefill of A equal-length prompts of T tokens into empty rows, positions
 * 0..T-1 ("Tensor ownership boundary": equal-length pending prompts run as one
 * batch whose prefixes land in their target empty shared rows).  The result is
 * that of storing every token's rotated K and V at its position, then causal
 * attention of query t over keys 0..t of the same row.
 *
 *  q [A, T, Hq, D], k_new / v_new [A, T, Hkv, D], rows [A], Kc/Vc [S, C, Hkv, D]
 *  out [A, T, Hq, D].
 *  t_list / n_t: optional subset of query positions to compute (NULL = all T);
 *  the cache is always stored for all T tokens.  Outputs for positions not in
 *  the list are left as they were.
 */
/*
 * Chunk of T tokens appended to each entry's row at its own start position
 * s = starts[a] (starts == NULL: every s = 0, the equal-length prefill into
 * empty rows of "Tensor ownership boundary").  The pages define the decode
 * step (one token at a per-row position, attention over the row's cached
 * prefix) and the equal-length prefill; a chunk at a nonzero start is read
 * here as T decode steps at positions s .. s+T-1 taken together: every token
 * t is rotated at s + t and stored at slot s + t of its row, then query t
 * attends keys 0 .. s + t of the row -- the prefix already in the cache and
 * the chunk up to itself.  With T = 1 this is exactly orc_decode_step.
 * lens (optional, NULL = every entry T tokens) gives entry a only its first
 * lens[a] tokens (1 <= lens[a] <= T): the page keeps prompts of different
 * lengths as separate groups, and a batch of several lengths here is read as
 * those groups run one after another -- tokens t >= lens[a] are neither
 * stored nor attended, and their output rows are not written.
 * t_list (optional) restricts which query positions t are computed.
 */
int orc_prefill_chunk_dt(int dt, int A, int T, int S, int C, int Hq, int Hkv, int D,
                         double base, const uint16_t *q, const uint16_t *k_new,
                         const uint16_t *v_new, const int32_t *starts, const int32_t *lens,
                         const int32_t *rows, uint16_t *Kc, uint16_t *Vc, uint16_t *out,
                         const int32_t *t_list, int n_t)
{
    if (dt != ORC_BF16 && dt != ORC_F16)
        return ORC_ERR_SHAPE;
    int rc = check_shapes(A, S, C, Hq, Hkv, D);
    if (rc)
        return rc;
    if (T < 1 || T > C)
        return ORC_ERR_SHAPE;
    rc = check_rows_unique(A, S, rows);
    if (rc)
        return rc;
    for (int a = 0; a < A; ++a) {
        const int s0 = starts ? starts[a] : 0, n = lens ? lens[a] : T;
        if (n < 1 || n > T || s0 < 0 || s0 > C - n)
            return ORC_ERR_INDEX;
    }
    if (t_list)
        for (int i = 0; i < n_t; ++i)
            if (t_list[i] < 0 || t_list[i] >= T)
                return ORC_ERR_INDEX;

    const int G = Hq / Hkv;
    const long slot = (long)Hkv * D;
    const long row = (long)C * slot;
    const float scale = (float)(1.0 / sqrt((double)D));

    float *inv_freq = malloc(sizeof(float) * (size_t)(D / 2));
    float *cs = malloc(sizeof(float) * (size_t)(D / 2));
    float *sn = malloc(sizeof(float) * (size_t)(D / 2));
    float *x = malloc(sizeof(float) * (size_t)D);
    float *y = malloc(sizeof(float) * (size_t)D);
    float *e = malloc(sizeof(float) * (size_t)C);
    if (!inv_freq || !cs || !sn || !x || !y || !e) {
        free(inv_freq); free(cs); free(sn); free(x); free(y); free(e);
        return ORC_ERR_NOMEM;
    }
    orc_rope_inv_freq(base, D, inv_freq);

    /* 1. every token of every entry: rotated K and raw V into its slot */
    for (int a = 0; a < A; ++a) {
        const int s0 = starts ? starts[a] : 0, n = lens ? lens[a] : T;
        for (int t = 0; t < n; ++t) {
            orc_rope_cos_sin(s0 + t, D, inv_freq, cs, sn);
            for (int h = 0; h < Hkv; ++h) {
                const uint16_t *k = k_new + (((long)a * T + t) * Hkv + h) * D;
                const uint16_t *v = v_new + (((long)a * T + t) * Hkv + h) * D;
                uint16_t *kd = Kc + rows[a] * row + (long)(s0 + t) * slot + (long)h * D;
                uint16_t *vd = Vc + rows[a] * row + (long)(s0 + t) * slot + (long)h * D;
                for (int d = 0; d < D; ++d)
                    x[d] = to_f32(dt, k[d]);
                orc_rope_apply(x, D, cs, sn, y);
                for (int d = 0; d < D; ++d) {
                    kd[d] = from_f32(dt, y[d]);
                    vd[d] = v[d];
                }
            }
        }
    }

    /* 2. query t of entry a: rotated at s + t, attends keys 0 .. s + t */
    int count = t_list ? n_t : T;
    for (int a = 0; a < A; ++a) {
        const int s0 = starts ? starts[a] : 0, n = lens ? lens[a] : T;
        for (int i = 0; i < count; ++i) {
            int t = t_list ? t_list[i] : i;
            if (t >= n)
                continue;
            orc_rope_cos_sin(s0 + t, D, inv_freq, cs, sn);
            for (int hq = 0; hq < Hq; ++hq) {
                int kv = hq / G;
                const uint16_t *qa = q + (((long)a * T + t) * Hq + hq) * D;
                for (int d = 0; d < D; ++d)
                    x[d] = to_f32(dt, qa[d]);
                orc_rope_apply(x, D, cs, sn, y);
                const uint16_t *Kr = Kc + rows[a] * row + (long)kv * D;
                const uint16_t *Vr = Vc + rows[a] * row + (long)kv * D;
                long o = (((long)a * T + t) * Hq + hq) * D;
                attend_one(dt, y, D, Kr, Vr, slot, s0 + t, scale, e, out + o, NULL);
            }
        }
    }
    free(inv_freq); free(cs); free(sn); free(x); free(y); free(e);
    return ORC_OK;
}

/* The BF16 entry points. */
int orc_decode_step(int A, int S, int C, int Hq, int Hkv, int D, double base,
                    const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                    const int32_t *pos, const int32_t *rows, uint16_t *Kc, uint16_t *Vc,
                    uint16_t *out, float *out_f32)
{
    return orc_decode_step_dt(ORC_BF16, A, S, C, Hq, Hkv, D, base, q, k_new, v_new, pos, rows,
                              Kc, Vc, out, out_f32);
}

int orc_prefill_chunk(int A, int T, int S, int C, int Hq, int Hkv, int D, double base,
                      const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                      const int32_t *starts, const int32_t *lens, const int32_t *rows,
                      uint16_t *Kc, uint16_t *Vc, uint16_t *out, const int32_t *t_list, int n_t)
{
    return orc_prefill_chunk_dt(ORC_BF16, A, T, S, C, Hq, Hkv, D, base, q, k_new, v_new, starts,
                                lens, rows, Kc, Vc, out, t_list, n_t);
}

/* Equal-length prefill into empty rows: the chunk at start 0 of every row. */
int orc_prefill(int A, int T, int S, int C, int Hq, int Hkv, int D, double base,
                const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                const int32_t *rows, uint16_t *Kc, uint16_t *Vc, uint16_t *out,
                const int32_t *t_list, int n_t)
{
    return orc_prefill_chunk(A, T, S, C, Hq, Hkv, D, base, q, k_new, v_new, NULL, NULL, rows,
                             Kc, Vc, out, t_list, n_t);
}
