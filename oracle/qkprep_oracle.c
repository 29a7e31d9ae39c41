/*
 * qkprep_oracle.c -- CPU oracle for the pre-attention "prepare" pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load this library.  It shares no code,
 * header, table or helper with the HIP library; it is plain, single-threaded
 * C99, computes in fp64 from the exact input values and rounds once at the
 * end, exactly as the definitions below state.  Nothing here is blocked,
 * fused or reordered beyond what the definitions say.
 *
 * Sources (the pages):
 *  - FlashInfer PR "fused QK RMSNorm + NeoX RoPE + FP8 E4M3 quantize + NHD
 *    paged-KV append" (Cake route), sections "What changes" (the fp32
 *    reference of the 51 tests: per-head RMSNorm eps 1e-6, NeoX RoPE,
 *    max(|q|,1e-6)/upper_max or static scale, x/scale K/V payloads) and
 *    "Contract" (packed qkv, NHD caches, q_scale layouts, seq_lens after the
 *    append, tail clear of each request's last page, all-or-nothing device
 *    validation writing -1 flags).  Its security review (negative derived
 *    positions are suppressed by the BF16 sibling) and review threads
 *    (seq_len < q_len, page count > max_pages_per_request, positions past
 *    the cos/sin table) give the extra validation adopted here.
 *  - TensorRT-LLM PR "Fuse Qwen3.5 gated QKV preprocessing", Phase 2 (Gemma
 *    Q/K RMSNorm with scale (1 + w), NeoX RoPE, strided QKV rows) and the
 *    review of its RMS reduction (sum of squares over one head of one token,
 *    rsqrt(sum/headSize + eps)).
 *  - SGLang PR "fused Q/K RMSNorm + RoPE with cos_sin_cache", Modifications
 *    (fp32 cos_sin_cache indexed by 1-D int64 positions, strided views into
 *    packed QKV).
 *  - vLLM issue "ROPE + KV-Cache-Write + pre-attn prepare-ops fusion"
 *    (reshape_and_cache slot scatter, concat_and_cache_mla latent + rope
 *    concat, interleaved RoPE for DeepSeek MLA; model table).
 *
 * Readings where the pages are silent:
 *  - cos_sin_cache row p is [cos(p f_0) .. cos(p f_{R/2-1}) | sin(...)].
 *    NeoX pairs (i, i + R/2) use angle i; interleaved pairs (2i, 2i+1) use
 *    angle i.  With R < D the first R dims of a head rotate and the rest
 *    pass through; with R = 0 no dim rotates and positions are not read.
 *  - norm 0 = none, 1 = x * inv * w, 2 = x * inv * (1 + w).
 *  - The fused pass keeps full precision until the final store; the oracle
 *    keeps fp64, rounds the rotated value once to fp32 ("v32"), and encodes
 *    v32 (bf16 RNE, or E4M3 RN-satfinite of v32 / scale in fp64).
 *  - A token whose position lies outside [0, cos_sin_rows) writes nothing.
 *  - In slot addressing a negative or out-of-capacity slot skips the K/V
 *    write of that token only.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_OK 0
#define ORC_BAD_ARGS 1

/* ------------------------------------------------------------------ */
/* Number formats                                                      */
/* ------------------------------------------------------------------ */

/* bf16 bits -> exact value.  A bf16 number is the upper half of an IEEE
 * binary32 pattern. */
double oracle_bf16_to_f64(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static uint32_t f32_bits(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return u;
}

static float f32_from_bits(uint32_t u)
{
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* fp32 -> bf16, round to nearest, ties to even, by comparing the two
 * neighbouring bf16 numbers (the one obtained by truncation and the next one
 * away from zero).  The distance of each neighbour is computed exactly in
 * fp64.  Overflow past the largest finite bf16 yields infinity (IEEE RNE).
 * NaN keeps its sign and becomes a quiet NaN. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u = f32_bits(f);
    if ((u & 0x7f800000u) == 0x7f800000u) {                 /* inf or NaN */
        if (u & 0x007fffffu) return (uint16_t)((u >> 16) | 0x0040u);
        return (uint16_t)(u >> 16);
    }
    uint32_t lo_bits = u & 0xffff0000u;                     /* toward zero */
    uint32_t hi_bits = lo_bits + 0x00010000u;               /* away from zero */
    double x = fabs((double)f);
    double lo = fabs((double)f32_from_bits(lo_bits));
    /* past the largest finite bf16 the next value of the format's grid is
     * 2^128; rounding up to it means overflow to infinity */
    double hi = ((hi_bits & 0x7fffffffu) == 0x7f800000u) ? ldexp(1.0, 128)
                                                         : fabs((double)f32_from_bits(hi_bits));
    double dlo = x - lo, dhi = hi - x;
    uint32_t pick;
    if (dlo < dhi) pick = lo_bits;
    else if (dhi < dlo) pick = hi_bits;
    else pick = ((lo_bits >> 16) & 1u) ? hi_bits : lo_bits; /* tie: even */
    return (uint16_t)(pick >> 16);
}

/* OCP FP8 E4M3 ("E4M3FN"): 1 sign bit, 4 exponent bits (bias 7), 3
 * mantissa bits, no infinities, one NaN pattern per sign (S.1111.111).
 * Value of a non-negative code c in 0x00..0x7E:
 *   e = c >> 3, m = c & 7;  e == 0 ? (m / 8) * 2^-6 : (1 + m / 8) * 2^(e-7).
 * The largest finite value is 0x7E = 448. */
double oracle_e4m3_to_f64(uint8_t c)
{
    int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
    if (e == 15 && m == 7) return NAN;
    double v = (e == 0) ? ldexp((double)m / 8.0, -6) : ldexp(1.0 + (double)m / 8.0, e - 7);
    return s ? -v : v;
}

static double e4m3_table[127];
static int e4m3_ready = 0;

static void e4m3_init(void)
{
    if (e4m3_ready) return;
    for (int c = 0; c < 127; ++c) e4m3_table[c] = oracle_e4m3_to_f64((uint8_t)c);
    e4m3_ready = 1;
}

/* Round-to-nearest-even, saturating to the largest finite value
 * ("RN satfinite" in the FlashInfer contract): |x| is compared against the
 * monotone table of the 127 finite non-negative codes; the nearest code
 * wins, a tie picks the code whose mantissa LSB is 0; |x| > 448 clamps to
 * 448.  The sign bit is kept (a negative value that rounds to zero gives
 * 0x80).  NaN inputs are outside the contract and map to 0x7F. */
uint8_t oracle_f64_to_e4m3(double x)
{
    e4m3_init();
    if (isnan(x)) return 0x7f;
    uint8_t sign = signbit(x) ? 0x80 : 0x00;
    double a = fabs(x);
    if (a >= e4m3_table[126]) return (uint8_t)(sign | 126);
    /* largest code with value <= a (binary search over the table) */
    int lo = 0, hi = 126;
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (e4m3_table[mid] <= a) lo = mid; else hi = mid;
    }
    /* now table[lo] <= a < table[lo + 1] */
    double dlo = a - e4m3_table[lo], dhi = e4m3_table[lo + 1] - a;
    int pick;
    if (dlo < dhi) pick = lo;
    else if (dhi < dlo) pick = lo + 1;
    else pick = (lo & 1) ? lo + 1 : lo;
    return (uint8_t)(sign | pick);
}

/* ------------------------------------------------------------------ */
/* Step functions (each exported so the CPU tests can pin it alone)    */
/* ------------------------------------------------------------------ */

/* Per-head RMSNorm of one head row (TensorRT-LLM review of the fused
 * preprocessing kernel; FlashInfer "What changes": eps 1e-6):
 *   inv = 1 / sqrt(sum(x^2) / D + eps),  y = x * inv * w   (norm 1)
 *                                        y = x * inv * (1 + w) (norm 2)
 *   norm 0 copies x. */
void oracle_rmsnorm(const double *x, int D, const float *w, int norm, double eps, double *y)
{
    if (norm == 0) {
        for (int d = 0; d < D; ++d) y[d] = x[d];
        return;
    }
    double ss = 0.0;
    for (int d = 0; d < D; ++d) ss += x[d] * x[d];
    double inv = 1.0 / sqrt(ss / (double)D + eps);
    for (int d = 0; d < D; ++d) {
        double wd = (double)w[d];
        double scale = (norm == 2) ? (1.0 + wd) : wd;
        y[d] = x[d] * inv * scale;
    }
}

/* Rotary embedding of one head row of length D whose first R dims rotate
 * (R even, 0 <= R <= D); dims [R, D) pass through unchanged (the partial
 * rotary of the vLLM issue's model table: RoPE on part of the head, NoPE on
 * the rest; R = 0 is a NoPE layer).  c[i], s[i] (i < R/2) are the cosine and
 * sine of angle i.
 *   NeoX (rope 0):        pair (i, i + R/2)
 *   interleaved (rope 1): pair (2i, 2i + 1)
 * For a pair (a, b):  a' = a c - b s,  b' = b c + a s. */
void oracle_rope_partial(const double *y, int D, int R, int rope, const double *c, const double *s,
                         double *o)
{
    int half = R / 2;
    for (int d = R; d < D; ++d) o[d] = y[d];
    for (int i = 0; i < half; ++i) {
        int ia = (rope == 0) ? i : 2 * i;
        int ib = (rope == 0) ? i + half : 2 * i + 1;
        double a = y[ia], b = y[ib];
        o[ia] = a * c[i] - b * s[i];
        o[ib] = b * c[i] + a * s[i];
    }
}

/* The whole head rotates (R = D). */
void oracle_rope(const double *y, int D, int rope, const double *c, const double *s, double *o)
{
    oracle_rope_partial(y, D, D, rope, c, s, o);
}

/* Dynamic per-(token, head) FP8 scale (FlashInfer "What changes"):
 *   s = max(amax(|v|), 1e-6) / upper_max, stored as fp32. */
float oracle_q_scale(const float *v, int D, double upper_max)
{
    double amax = 0.0;
    for (int d = 0; d < D; ++d) {
        double a = fabs((double)v[d]);
        if (a > amax) amax = a;
    }
    double m = amax > 1e-6 ? amax : 1e-6;
    return (float)(m / upper_max);
}

/* ------------------------------------------------------------------ */
/* Fused prepare pass over packed / strided QKV                        */
/* ------------------------------------------------------------------ */

typedef struct {
    /* shapes; rot = rotated dims per head (even, 0..D) */
    int32_t T, Hq, Hkv, D, rot;
    /* qkv: bf16 bits, row t at qkv + t * qkv_row_stride, Q | K | V heads */
    const uint16_t *qkv;
    int64_t qkv_row_stride;
    /* norm */
    int32_t norm;
    float eps;
    const float *q_w, *k_w;
    /* rope */
    int32_t rope;
    const float *cos_sin;
    int64_t cs_rows;
    const int64_t *positions;
    /* placement */
    int32_t addressing;              /* 0 page table, 1 slot mapping */
    int32_t B;
    const int32_t *q_indptr, *seq_lens, *page_table;
    int32_t maxp;
    const int64_t *slot_mapping;
    /* caches: NHD [num_pages, page_size, Hkv, D] */
    void *k_cache, *v_cache;
    int32_t kv_fp8;                  /* 0 bf16, 1 E4M3 */
    int32_t num_pages, page_size;
    int64_t k_page_stride, v_page_stride;   /* elements */
    float k_scale, v_scale;
    int32_t zero_tail;
    /* q */
    void *q_out;
    int64_t q_out_row_stride;        /* elements */
    int32_t q_mode;                  /* 0 bf16, 1 FP8 dynamic, 2 FP8 static */
    float *q_scale;
    int32_t q_scale_padded;          /* 0 [T, Hq], 1 [B, Hq, round_up(max_seqlen, 128)] */
    int32_t max_seqlen;
    float q_scale_inv;
    float upper_max;
    /* optional bf16 write-back of the normed + roped K */
    uint16_t *k_out;
    int64_t k_out_row_stride;
    /* [B, Hkv] */
    int32_t *flags;
    /* K/V redirect: when out_k != NULL the K / V rows of token t go to row t
     * of out_k / out_v (row stride in elements) instead of the caches */
    void *out_k, *out_v;
    int64_t out_kv_row_stride;
    /* FP8 K/V scales: 0 the static scalars k_scale / v_scale; 1 one dynamic
     * scale per (token, kv head); 2 one per kv_group_size consecutive dims.
     * Dynamic scales go to k_scale_out / v_scale_out, [cache row][Hkv][D/g]
     * (cache row = page * page_size + row, or t when redirected). */
    int32_t kv_scale_mode, kv_group_size;
    float *k_scale_out, *v_scale_out;
} oracle_nra_args;

/* The contract's metadata validation (FlashInfer "Contract": malformed
 * q_indptr or a request above max_seqlen; review threads: seq_len < q_len,
 * more pages than max_pages_per_request) plus touched page ids inside the
 * pool.  Returns 1 if the call is invalid. */
static int nra_invalid(const oracle_nra_args *a)
{
    if (a->addressing != 0) return 0;
    if (a->B <= 0) return a->T > 0;
    if (a->q_indptr[0] != 0) return 1;
    if (a->q_indptr[a->B] != a->T) return 1;
    for (int b = 0; b < a->B; ++b) {
        int32_t qlen = a->q_indptr[b + 1] - a->q_indptr[b];
        if (qlen < 0) return 1;
    }
    int64_t P = ((int64_t)a->max_seqlen + 127) / 128 * 128;
    (void)P;
    for (int b = 0; b < a->B; ++b) {
        int64_t qlen = a->q_indptr[b + 1] - a->q_indptr[b];
        int64_t sl = a->seq_lens[b];
        if (sl < qlen) return 1;
        if (sl > (int64_t)a->maxp * a->page_size) return 1;
        if (a->q_mode == 1 && a->q_scale_padded && qlen > a->max_seqlen) return 1;
        /* page ids are checked for the pages this call writes: the
         * appended rows' pages, and the last page if its tail is cleared.
         * With K/V redirected to out_k / out_v the call writes no page, so
         * no page id is checked (and none is read). */
        if (a->out_k) continue;
        int64_t first_row = sl - qlen;
        if (a->zero_tail && qlen == 0 && sl > 0) first_row = sl - 1;
        for (int64_t L = first_row; L < sl; ++L) {
            int32_t p = a->page_table[(int64_t)b * a->maxp + L / a->page_size];
            if (p < 0 || p >= a->num_pages) return 1;
        }
    }
    return 0;
}

static void store_q(const oracle_nra_args *a, int64_t t, int h, int64_t b, int64_t j,
                    const float *v32)
{
    int D = a->D;
    if (a->q_mode == 0) {
        uint16_t *q = (uint16_t *)a->q_out + t * a->q_out_row_stride + (int64_t)h * D;
        for (int d = 0; d < D; ++d) q[d] = oracle_f32_to_bf16(v32[d]);
        return;
    }
    uint8_t *q = (uint8_t *)a->q_out + t * a->q_out_row_stride + (int64_t)h * D;
    if (a->q_mode == 1) {
        float s = oracle_q_scale(v32, D, (double)a->upper_max);
        for (int d = 0; d < D; ++d) q[d] = oracle_f64_to_e4m3((double)v32[d] / (double)s);
        int64_t idx;
        if (a->q_scale_padded) {
            int64_t P = ((int64_t)a->max_seqlen + 127) / 128 * 128;
            idx = (b * a->Hq + h) * P + j;
        } else {
            idx = t * a->Hq + h;
        }
        a->q_scale[idx] = s;
    } else {
        for (int d = 0; d < D; ++d)
            q[d] = oracle_f64_to_e4m3((double)v32[d] * (double)a->q_scale_inv);
    }
}

/* Dims per K/V scale: the whole head row (static scalars, per-token mode)
 * or kv_group_size. */
static int kv_group(const oracle_nra_args *a)
{
    return a->kv_scale_mode == 2 ? a->kv_group_size : a->D;
}

/* Store one K or V head row.  v32 holds the encoded values as fp32 (K:
 * normalised and rotated; V: the raw bf16 values, exact).  The row goes to
 * the cache cell (page, row), or to row t of out_k / out_v when the call
 * redirects K/V (FlashInfer "Contract": caller-owned out_k / out_v).
 *   bf16 cache: RNE of v32 (for V a bit copy of raw)
 *   FP8, static scale: E4M3(v32 / scale)
 *   FP8, dynamic scales (the vLLM issue's dynamic per-token and per-group
 *   question): for each group of g dims s = fp32(max(amax, 1e-6) / 448),
 *   E4M3(v32 / s), s stored in the scale array at the row's entry. */
static void store_kv(const oracle_nra_args *a, int is_v, int64_t t, int64_t page, int64_t row, int kh,
                     const float *v32, const uint16_t *raw)
{
    int D = a->D;
    int64_t esz = a->kv_fp8 ? 1 : 2;
    char *dst;
    int64_t srow;
    if (a->out_k) {
        dst = (char *)(is_v ? a->out_v : a->out_k) + (t * a->out_kv_row_stride + (int64_t)kh * D) * esz;
        srow = t;
    } else {
        int64_t ps = is_v ? a->v_page_stride : a->k_page_stride;
        dst = (char *)(is_v ? a->v_cache : a->k_cache) + (page * ps + (row * a->Hkv + kh) * (int64_t)D) * esz;
        srow = page * a->page_size + row;
    }
    if (!a->kv_fp8) {
        uint16_t *d16 = (uint16_t *)dst;
        for (int d = 0; d < D; ++d) d16[d] = raw ? raw[d] : oracle_f32_to_bf16(v32[d]);
        return;
    }
    uint8_t *d8 = (uint8_t *)dst;
    if (a->kv_scale_mode == 0) {
        double scale = (double)(is_v ? a->v_scale : a->k_scale);
        for (int d = 0; d < D; ++d) d8[d] = oracle_f64_to_e4m3((double)v32[d] / scale);
        return;
    }
    int g = kv_group(a), ng = D / g;
    float *sc = (is_v ? a->v_scale_out : a->k_scale_out) + (srow * a->Hkv + kh) * ng;
    for (int k = 0; k < ng; ++k) {
        float s = oracle_q_scale(v32 + k * g, g, 448.0);
        sc[k] = s;
        for (int d = k * g; d < (k + 1) * g; ++d) d8[d] = oracle_f64_to_e4m3((double)v32[d] / (double)s);
    }
}

/* One token: norm + rope of each Q and K head, encode and store; V copied
 * or quantised.  (b, j) locate the token inside its request (for the
 * padded q_scale layout); page < 0 means "no K/V write". */
static void nra_token(const oracle_nra_args *a, int64_t t, int64_t b, int64_t j, int64_t pos,
                      int64_t page, int64_t row)
{
    int D = a->D, Hq = a->Hq, Hkv = a->Hkv, Rr = a->rot;
    double *x = malloc(sizeof(double) * (size_t)D);
    double *y = malloc(sizeof(double) * (size_t)D);
    double *o = malloc(sizeof(double) * (size_t)D);
    double *c = malloc(sizeof(double) * (size_t)(D / 2 + 1));
    double *s = malloc(sizeof(double) * (size_t)(D / 2 + 1));
    float *v32 = malloc(sizeof(float) * (size_t)D);
    uint16_t *raw = malloc(sizeof(uint16_t) * (size_t)D);
    /* the fp32 table values, not recomputed angles; table rows hold R floats */
    for (int i = 0; i < Rr / 2; ++i) {
        c[i] = (double)a->cos_sin[pos * Rr + i];
        s[i] = (double)a->cos_sin[pos * Rr + Rr / 2 + i];
    }
    const uint16_t *rowp = a->qkv + t * a->qkv_row_stride;
    /* read every head of the token before any write: q_out / k_out may
     * alias the Q / K columns of qkv */
    int R = Hq + 2 * Hkv;
    uint16_t *tok = malloc(sizeof(uint16_t) * (size_t)R * (size_t)D);
    memcpy(tok, rowp, sizeof(uint16_t) * (size_t)R * (size_t)D);
    for (int h = 0; h < Hq + Hkv; ++h) {
        int is_q = h < Hq;
        const uint16_t *src = tok + (int64_t)h * D;
        for (int d = 0; d < D; ++d) x[d] = oracle_bf16_to_f64(src[d]);
        oracle_rmsnorm(x, D, is_q ? a->q_w : a->k_w, a->norm, (double)a->eps, y);
        oracle_rope_partial(y, D, Rr, a->rope, c, s, o);
        for (int d = 0; d < D; ++d) v32[d] = (float)o[d];
        if (is_q) {
            store_q(a, t, h, b, j, v32);
        } else {
            int kh = h - Hq;
            if (page >= 0 || a->out_k) store_kv(a, 0, t, page, row, kh, v32, NULL);
            if (a->k_out) {
                uint16_t *ko = a->k_out + t * a->k_out_row_stride + (int64_t)kh * D;
                for (int d = 0; d < D; ++d) ko[d] = oracle_f32_to_bf16(v32[d]);
            }
        }
    }
    if (page >= 0 || a->out_k) {
        for (int vh = 0; vh < Hkv; ++vh) {
            memcpy(raw, tok + (int64_t)(Hq + Hkv + vh) * D, sizeof(uint16_t) * (size_t)D);
            for (int d = 0; d < D; ++d) v32[d] = (float)oracle_bf16_to_f64(raw[d]);
            store_kv(a, 1, t, page, row, vh, v32, raw);
        }
    }
    free(tok); free(x); free(y); free(o); free(c); free(s); free(v32); free(raw);
}

/* Whether token t is suppressed: its position lies outside the cos/sin
 * table.  Without rotated dims (R = 0) positions are not used at all. */
static int position_out_of_table(const oracle_nra_args *a, int64_t t)
{
    if (a->rot == 0) return 0;
    int64_t pos = a->positions[t];
    return pos < 0 || pos >= a->cs_rows;
}

int oracle_norm_rope_append(const oracle_nra_args *a)
{
    if (a->D % 2 || a->rot % 2 || a->rot < 0 || a->rot > a->D) return ORC_BAD_ARGS;
    if (a->kv_scale_mode < 0 || a->kv_scale_mode > 2) return ORC_BAD_ARGS;
    if (a->kv_scale_mode && (!a->kv_fp8 || !a->k_scale_out || !a->v_scale_out)) return ORC_BAD_ARGS;
    if (a->kv_scale_mode == 2 && (a->kv_group_size <= 0 || a->D % a->kv_group_size)) return ORC_BAD_ARGS;
    if ((a->out_k == NULL) != (a->out_v == NULL)) return ORC_BAD_ARGS;
    if (a->addressing == 0) {
        int bad = nra_invalid(a);
        if (a->flags)
            for (int64_t i = 0; i < (int64_t)a->B * a->Hkv; ++i) a->flags[i] = bad ? -1 : 0;
        if (bad) return ORC_OK;
        for (int b = 0; b < a->B; ++b) {
            int64_t beg = a->q_indptr[b], end = a->q_indptr[b + 1];
            int64_t qlen = end - beg, sl = a->seq_lens[b];
            for (int64_t j = 0; j < qlen; ++j) {
                int64_t t = beg + j;
                if (position_out_of_table(a, t)) continue;
                int64_t pos = a->rot ? a->positions[t] : 0;
                int64_t L = sl - qlen + j;            /* logical row in the request */
                /* (redirected K/V rows are addressed by token: no page is read) */
                int64_t page = a->out_k ? -1 : a->page_table[(int64_t)b * a->maxp + L / a->page_size];
                nra_token(a, t, b, j, pos, page, L % a->page_size);
            }
        }
        /* no tail clear when K/V are redirected (FlashInfer review: the
         * caches are not touched then) */
        if (a->zero_tail && !a->out_k) {
            for (int b = 0; b < a->B; ++b) {
                int64_t sl = a->seq_lens[b];
                if (sl <= 0) continue;
                int64_t last = (sl - 1) % a->page_size;
                int64_t page = a->page_table[(int64_t)b * a->maxp + (sl - 1) / a->page_size];
                int64_t row_elems = (int64_t)a->Hkv * a->D;
                int64_t n = (a->page_size - 1 - last) * row_elems;
                int64_t esz = a->kv_fp8 ? 1 : 2;
                memset((char *)a->k_cache + (page * a->k_page_stride + (last + 1) * row_elems) * esz, 0,
                       (size_t)(n * esz));
                memset((char *)a->v_cache + (page * a->v_page_stride + (last + 1) * row_elems) * esz, 0,
                       (size_t)(n * esz));
                if (a->kv_scale_mode) {
                    /* the cleared rows' dynamic scales are zeroed too */
                    int64_t ns = (int64_t)a->Hkv * (a->D / kv_group(a));
                    int64_t first = (page * a->page_size + last + 1) * ns;
                    for (int64_t i = 0; i < (a->page_size - 1 - last) * ns; ++i) {
                        a->k_scale_out[first + i] = 0.0f;
                        a->v_scale_out[first + i] = 0.0f;
                    }
                }
            }
        }
        return ORC_OK;
    }
    /* slot addressing (vLLM reshape_and_cache): slot s -> page s / ps, row s % ps */
    int64_t capacity = (int64_t)a->num_pages * a->page_size;
    for (int64_t t = 0; t < a->T; ++t) {
        if (position_out_of_table(a, t)) continue;
        int64_t pos = a->rot ? a->positions[t] : 0;
        int64_t slot = a->slot_mapping ? a->slot_mapping[t] : -1;
        int64_t page = -1, row = 0;
        if (slot >= 0 && slot < capacity) {
            page = slot / a->page_size;
            row = slot % a->page_size;
        }
        nra_token(a, t, 0, 0, pos, page, row);
    }
    return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* MLA: RoPE on q's rope slice in place, latent + rope concat to cache */
/* ------------------------------------------------------------------ */

typedef struct {
    int32_t T, H, nope_dim, rope_dim, kv_lora_rank;
    uint16_t *q;                      /* bf16, [T, H, nope + rope] via strides */
    int64_t q_token_stride, q_head_stride;
    const uint16_t *kv_c;             /* bf16 [T, kv_lora_rank] */
    int64_t kv_c_stride;
    const uint16_t *k_pe;             /* bf16 [T, rope_dim], read-only */
    int64_t k_pe_stride;
    int32_t rope;
    const float *cos_sin;             /* [rows, rope_dim] */
    int64_t cs_rows;
    const int64_t *positions;
    const int64_t *slot_mapping;
    void *kv_cache;                   /* [num_blocks, block_size, kv_lora_rank + rope_dim] */
    int32_t kv_fp8;
    int64_t num_blocks;
    int32_t block_size;
    int64_t block_stride;             /* elements */
    float kv_scale;
    /* Q output: 0 = RoPE in place in q (bf16); 1 = E4M3 with one dynamic
     * scale per token over all its heads; 2 = E4M3 with a static scale */
    int32_t q_mode;
    uint8_t *q_out;                   /* E4M3 codes, [T, H, nope + rope] via strides */
    int64_t q_out_token_stride, q_out_head_stride;
    float *q_scale;                   /* [T], q_mode 1 */
    float q_scale_inv;                /* q_mode 2 */
    float upper_max;                  /* q_mode 1 */
} oracle_mla_args;

/* Q of one token in the FP8 modes (vLLM issue: the FlashInfer MLA RoPE +
 * quantize kernel, and the question of static per-tensor and dynamic
 * per-token scales).  Every head's [q_nope | RoPE(q_rope)] is rounded once
 * to fp32 (v32; q_nope is exact), then encoded E4M3(v32 * q_scale_inv)
 * (static) or E4M3(v32 / s) with s = max(amax, 1e-6) / upper_max over all
 * heads and dims of the token (dynamic), s stored at q_scale[t].  q itself
 * is not modified. */
static void mla_q_fp8(const oracle_mla_args *a, int64_t t, const double *c, const double *s)
{
    int N = a->nope_dim, R = a->rope_dim, W = N + R;
    float *v32 = malloc(sizeof(float) * (size_t)a->H * (size_t)W);
    double *x = malloc(sizeof(double) * (size_t)R);
    double *o = malloc(sizeof(double) * (size_t)R);
    for (int h = 0; h < a->H; ++h) {
        const uint16_t *qh = a->q + t * a->q_token_stride + (int64_t)h * a->q_head_stride;
        float *vh = v32 + (int64_t)h * W;
        for (int d = 0; d < N; ++d) vh[d] = (float)oracle_bf16_to_f64(qh[d]);
        for (int d = 0; d < R; ++d) x[d] = oracle_bf16_to_f64(qh[N + d]);
        oracle_rope(x, R, a->rope, c, s, o);
        for (int d = 0; d < R; ++d) vh[N + d] = (float)o[d];
    }
    double sc = 0.0;
    if (a->q_mode == 1) {
        float st = oracle_q_scale(v32, a->H * W, (double)a->upper_max);
        a->q_scale[t] = st;
        sc = (double)st;
    }
    for (int h = 0; h < a->H; ++h) {
        uint8_t *dst = a->q_out + t * a->q_out_token_stride + (int64_t)h * a->q_out_head_stride;
        const float *vh = v32 + (int64_t)h * W;
        for (int d = 0; d < W; ++d)
            dst[d] = (a->q_mode == 1) ? oracle_f64_to_e4m3((double)vh[d] / sc)
                                      : oracle_f64_to_e4m3((double)vh[d] * (double)a->q_scale_inv);
    }
    free(v32); free(x); free(o);
}

/* vLLM issue: DeepSeek R1 keeps q_rope / q_nope and k_rope / k_nope apart,
 * RoPE interleaved; concat_and_cache_mla stores [kv_c | rope(k_pe)] into
 * the latent cache.  FP8 entries are x / kv_scale, RN-satfinite. */
int oracle_mla_concat_rope_append(const oracle_mla_args *a)
{
    int R = a->rope_dim, K = a->kv_lora_rank;
    if (R % 2) return ORC_BAD_ARGS;
    if (a->q_mode < 0 || a->q_mode > 2) return ORC_BAD_ARGS;
    double *x = malloc(sizeof(double) * (size_t)R);
    double *o = malloc(sizeof(double) * (size_t)R);
    double *c = malloc(sizeof(double) * (size_t)R / 2);
    double *s = malloc(sizeof(double) * (size_t)R / 2);
    float *v32 = malloc(sizeof(float) * (size_t)R);
    int64_t capacity = a->num_blocks * a->block_size;
    for (int64_t t = 0; t < a->T; ++t) {
        int64_t pos = a->positions[t];
        if (pos < 0 || pos >= a->cs_rows) continue;
        for (int i = 0; i < R / 2; ++i) {
            c[i] = (double)a->cos_sin[pos * R + i];
            s[i] = (double)a->cos_sin[pos * R + R / 2 + i];
        }
        if (a->q_mode == 0) {
            for (int h = 0; h < a->H; ++h) {
                uint16_t *qr = a->q + t * a->q_token_stride + (int64_t)h * a->q_head_stride + a->nope_dim;
                for (int d = 0; d < R; ++d) x[d] = oracle_bf16_to_f64(qr[d]);
                oracle_rope(x, R, a->rope, c, s, o);
                for (int d = 0; d < R; ++d) qr[d] = oracle_f32_to_bf16((float)o[d]);
            }
        } else {
            mla_q_fp8(a, t, c, s);
        }
        const uint16_t *kp = a->k_pe + t * a->k_pe_stride;
        for (int d = 0; d < R; ++d) x[d] = oracle_bf16_to_f64(kp[d]);
        oracle_rope(x, R, a->rope, c, s, o);
        for (int d = 0; d < R; ++d) v32[d] = (float)o[d];
        int64_t slot = a->slot_mapping[t];
        if (slot < 0 || slot >= capacity) continue;
        int64_t off = (slot / a->block_size) * a->block_stride + (slot % a->block_size) * (int64_t)(K + R);
        const uint16_t *kc = a->kv_c + t * a->kv_c_stride;
        if (a->kv_fp8) {
            uint8_t *dst = (uint8_t *)a->kv_cache + off;
            for (int d = 0; d < K; ++d)
                dst[d] = oracle_f64_to_e4m3(oracle_bf16_to_f64(kc[d]) / (double)a->kv_scale);
            for (int d = 0; d < R; ++d)
                dst[K + d] = oracle_f64_to_e4m3((double)v32[d] / (double)a->kv_scale);
        } else {
            uint16_t *dst = (uint16_t *)a->kv_cache + off;
            for (int d = 0; d < K; ++d) dst[d] = kc[d];
            for (int d = 0; d < R; ++d) dst[K + d] = oracle_f32_to_bf16(v32[d]);
        }
    }
    free(x); free(o); free(c); free(s); free(v32);
    return ORC_OK;
}

/* Bulk converters for the CPU pin tests. */
void oracle_f32_to_bf16_n(const float *in, uint16_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f32_to_bf16(in[i]);
}

void oracle_f64_to_e4m3_n(const double *in, uint8_t *out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = oracle_f64_to_e4m3(in[i]);
}
