/*
 * rope_oracle.c -- scalar CPU oracle for rotary position embedding apply.
 *
 * TEST INFRASTRUCTURE ONLY (see rope_oracle.h): the plain definition, one
 * element at a time, products and sums in binary64, one rounding to the
 * storage type at the end. No blocking, no vectors, no fusion. Built with
 * -ffp-contract=off so that no multiply-add is fused behind our back.
 *
 * Page citations are by page title and section; the page list is in
 * rope_oracle.h.
 */
#include "rope_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* binary16 <-> binary64, written from the IEEE-754 binary16 encoding:
 * 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */

double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);             /* zero or subnormal: m * 2^-24 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    return sign ? -v : v;
}

uint16_t oracle_f64_to_f16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7e00);
    if (a == 0.0)
        return sign;
    if (a >= 65520.0) /* halfway between 65504 and 2^16 or above: overflows */
        return (uint16_t)(sign | 0x7c00);

    /* binade exponent E: 2^E <= a < 2^(E+1); below 2^-14 every binary16 value
     * is a multiple of 2^-24, so the quantum stops shrinking there. */
    int ex;
    frexp(a, &ex);
    int E = ex - 1;
    if (E < -14)
        E = -14;
    double quantum = ldexp(1.0, E - 10);
    double n = nearbyint(a / quantum); /* a/quantum is exact; ties to even */
    double r = n * quantum;            /* the rounded magnitude */

    if (r < ldexp(1.0, -14))
        return (uint16_t)(sign | (uint16_t)n); /* subnormal: fraction = r/2^-24 */
    frexp(r, &ex); /* r may have moved up one binade */
    E = ex - 1;
    uint16_t frac = (uint16_t)(ldexp(r, 10 - E) - 1024.0);
    return (uint16_t)(sign | (uint16_t)((E + 15) << 10) | frac);
}

/* bfloat16: the upper 16 bits of a binary32 -- 8 exponent bits (bias 127),
 * 7 fraction bits. Same rounding rule as above with the binary32 exponent
 * range: binades from 2^-126, quantum 2^(E-7), below 2^-126 a fixed 2^-133. */

double oracle_bf16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int m = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)m, -133);            /* zero or subnormal: m * 2^-133 */
    else if (e == 255)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + m), e - 134); /* (1 + m/128) * 2^(e-127) */
    return sign ? -v : v;
}

uint16_t oracle_f64_to_bf16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7fc0);
    if (a == 0.0)
        return sign;
    /* halfway between the largest finite value (2 - 2^-7) * 2^127 and 2^128 */
    if (a >= ldexp(2.0 - ldexp(1.0, -8), 127))
        return (uint16_t)(sign | 0x7f80);
    int ex;
    frexp(a, &ex);
    int E = ex - 1;
    if (E < -126)
        E = -126;
    double quantum = ldexp(1.0, E - 7);
    double n = nearbyint(a / quantum);
    double r = n * quantum;
    if (r < ldexp(1.0, -126))
        return (uint16_t)(sign | (uint16_t)n); /* subnormal: fraction = r/2^-133 */
    frexp(r, &ex);
    E = ex - 1;
    uint16_t frac = (uint16_t)(ldexp(r, 7 - E) - 128.0);
    return (uint16_t)(sign | (uint16_t)((E + 127) << 7) | frac);
}

/* ------------------------------------------------------------------------ */
/* element access in the storage type */

static double load_elem(int dtype, const void* p, int64_t idx)
{
    if (dtype == ORACLE_F32)
        return (double)((const float*)p)[idx];
    if (dtype == ORACLE_BF16)
        return oracle_bf16_to_f64(((const uint16_t*)p)[idx]);
    return oracle_f16_to_f64(((const uint16_t*)p)[idx]);
}

static void store_elem(int dtype, void* p, int64_t idx, double v)
{
    if (dtype == ORACLE_F32)
        ((float*)p)[idx] = (float)v; /* one rounding, nearest-even */
    else if (dtype == ORACLE_BF16)
        ((uint16_t*)p)[idx] = oracle_f64_to_bf16(v);
    else
        ((uint16_t*)p)[idx] = oracle_f64_to_f16(v);
}

/* bit copy of element sidx of src to element didx of dst */
static void copy_elem_to(int dtype, const void* src, int64_t sidx, void* dst,
                         int64_t didx)
{
    size_t w = dtype == ORACLE_F32 ? 4 : 2;
    memcpy((char*)dst + w * (size_t)didx, (const char*)src + w * (size_t)sidx, w);
}

/* rnd_T(v) as a double */
static double round_to_storage(int dtype, double v)
{
    if (dtype == ORACLE_F32)
        return (double)(float)v;
    if (dtype == ORACLE_BF16)
        return oracle_bf16_to_f64(oracle_f64_to_bf16(v));
    return oracle_f16_to_f64(oracle_f64_to_f16(v));
}

/* Offset of x(b,h,s,0): [RE] `inputs` X -- rank 3 is (B, S, H*D) with head h
 * occupying elements h*D..h*D+D-1 of the hidden axis, rank 4 is (B, H, S, D). */
static int64_t row_offset(int rank, int64_t S, int64_t H, int64_t D,
                          int64_t b, int64_t h, int64_t s)
{
    if (rank == 4)
        return ((b * H + h) * S + s) * D;
    return ((b * S + s) * H + h) * D;
}

/* One head row of one token. For pair i < R/2 the two elements are
 * (i, i + R/2) for the half-split pairing and (2i, 2i+1) for the interleaved
 * one ([RE] `interleaved`; [SA] `rotary_interleaved`). The rotation is
 * q*cos + rotate_half(q)*sin with rotate_half(q) = cat(-q2, q1) ([PR] review,
 * rotate_half and apply_rotary_pos_emb), i.e. per pair
 *     y1 = x1*c - x2*s,   y2 = x2*c + x1*s.
 * Both products are exact in binary64 for binary16/binary32 operands; the
 * sum is rounded to binary64 and then once to the storage type.
 * A pair flagged `copy` and every element at or beyond R are bit copies
 * ([RE] `rotary_embedding_dim`: only the leading R elements rotate, the
 * others are kept; [MRE] Description: a pair whose id is out of range is
 * kept as it was). */
static void rotate_row_to(int dtype, const void* x, int64_t xoff, void* y,
                          int64_t yoff, int64_t D, int64_t R,
                          int64_t interleaved, const double* c,
                          const double* s, const unsigned char* copy)
{
    int64_t half = R / 2;
    for (int64_t i = 0; i < half; ++i) {
        int64_t j1 = interleaved ? 2 * i : i;
        int64_t j2 = interleaved ? 2 * i + 1 : i + half;
        if (copy[i]) {
            copy_elem_to(dtype, x, xoff + j1, y, yoff + j1);
            copy_elem_to(dtype, x, xoff + j2, y, yoff + j2);
            continue;
        }
        double x1 = load_elem(dtype, x, xoff + j1);
        double x2 = load_elem(dtype, x, xoff + j2);
        store_elem(dtype, y, yoff + j1, x1 * c[i] - x2 * s[i]);
        store_elem(dtype, y, yoff + j2, x2 * c[i] + x1 * s[i]);
    }
    for (int64_t j = R; j < D; ++j)
        copy_elem_to(dtype, x, xoff + j, y, yoff + j);
}

/* The same row of x and y (y may be x). */
static void rotate_row(int dtype, const void* x, void* y, int64_t off,
                       int64_t D, int64_t R, int64_t interleaved,
                       const double* c, const double* s,
                       const unsigned char* copy)
{
    rotate_row_to(dtype, x, off, y, off, D, R, interleaved, c, s, copy);
}

typedef struct {
    double* c;
    double* s;
    unsigned char* copy;
} coef_row;

static int coef_alloc(coef_row* r, int64_t half)
{
    size_t n = (size_t)(half > 0 ? half : 1);
    r->c = (double*)calloc(n, sizeof(double));
    r->s = (double*)calloc(n, sizeof(double));
    r->copy = (unsigned char*)calloc(n, 1);
    return r->c && r->s && r->copy;
}

static void coef_free(coef_row* r)
{
    free(r->c);
    free(r->s);
    free(r->copy);
}

/* ------------------------------------------------------------------------ */

void oracle_inv_freq(double base, int64_t rotary_dim, float* inv_freq)
{
    for (int64_t i = 0; i < rotary_dim / 2; ++i)
        inv_freq[i] = (float)pow(base, -2.0 * (double)i / (double)rotary_dim);
}

/* [PR] Motivation and review item 4: freqs[p][i] = p * inv_freq[i] formed in
 * binary32 (position cast to float, then a float multiply), cos/sin of it,
 * multiplied by the attention scaling, cast to the model dtype. */
static void coefficient(int dtype, int64_t p, float inv_freq_i, float scaling,
                        double* c, double* s)
{
    float pf = (float)p;
    float theta = (float)((double)pf * (double)inv_freq_i);
    float cf = (float)cos((double)theta);
    float sf = (float)sin((double)theta);
    float cs = (float)((double)cf * (double)scaling);
    float ss = (float)((double)sf * (double)scaling);
    *c = round_to_storage(dtype, (double)cs);
    *s = round_to_storage(dtype, (double)ss);
}

void oracle_cos_sin_cache(int dtype, int64_t rows, int64_t half,
                          const float* inv_freq, float scaling,
                          void* cos_out, void* sin_out)
{
    for (int64_t p = 0; p < rows; ++p)
        for (int64_t i = 0; i < half; ++i) {
            double c, s;
            coefficient(dtype, p, inv_freq[i], scaling, &c, &s);
            store_elem(dtype, cos_out, p * half + i, c);
            store_elem(dtype, sin_out, p * half + i, s);
        }
}

void oracle_onthefly_row(int dtype, int64_t p, const float* inv_freq,
                         int64_t half, float scaling, void* cos_row,
                         void* sin_row)
{
    for (int64_t i = 0; i < half; ++i) {
        double c, s;
        coefficient(dtype, p, inv_freq[i], scaling, &c, &s);
        store_elem(dtype, cos_row, i, c);
        store_elem(dtype, sin_row, i, s);
    }
}

/* ------------------------------------------------------------------------ */
/* RotaryEmbedding: [RE] `inputs` (cos_cache shapes with and without
 * position_ids), `attributes`, `attributeDescriptions`. */

void oracle_rope_apply(int dtype, int rank, int64_t B, int64_t S, int64_t H,
                       int64_t D, int64_t R, int64_t interleaved,
                       const void* x, void* y, const void* cos_cache,
                       const void* sin_cache, const int64_t* ids, int64_t M)
{
    int64_t half = R / 2;
    coef_row cr;
    if (!coef_alloc(&cr, half))
        abort();
    for (int64_t b = 0; b < B; ++b)
        for (int64_t s = 0; s < S; ++s) {
            int64_t row;
            int in_range = 1;
            if (ids) {
                row = ids[b * S + s];
                in_range = row >= 0 && row < M;
            } else {
                row = b * S + s;
            }
            for (int64_t i = 0; i < half; ++i) {
                cr.copy[i] = (unsigned char)!in_range;
                if (in_range) {
                    cr.c[i] = load_elem(dtype, cos_cache, row * half + i);
                    cr.s[i] = load_elem(dtype, sin_cache, row * half + i);
                }
            }
            for (int64_t h = 0; h < H; ++h)
                rotate_row(dtype, x, y, row_offset(rank, S, H, D, b, h, s), D,
                           R, interleaved, cr.c, cr.s, cr.copy);
        }
    coef_free(&cr);
}

/* ------------------------------------------------------------------------ */
/* MRotaryEmbedding: [MRE] Description, Inputs, Attributes. */

int oracle_mrope_slot_streams(int64_t half, const int64_t section[3],
                              int64_t layout, int8_t* stream_of_slot)
{
    if (section[0] < 0 || section[1] < 0 || section[2] < 0 ||
        section[0] + section[1] + section[2] != half)
        return -1;
    if (layout == 0) {
        /* sectioned: t owns the first section[0] slots, then h, then w */
        for (int64_t i = 0; i < half; ++i)
            stream_of_slot[i] = (int8_t)(i < section[0] ? 0
                                         : i < section[0] + section[1] ? 1
                                                                       : 2);
        return 0;
    }
    /* interleaved: deal slots to t, h, w in turn; a stream that already holds
     * its section count is passed over */
    int64_t used[3] = {0, 0, 0};
    int k = 0;
    for (int64_t i = 0; i < half; ++i) {
        while (used[k] == section[k])
            k = (k + 1) % 3;
        stream_of_slot[i] = (int8_t)k;
        used[k] += 1;
        k = (k + 1) % 3;
    }
    return 0;
}

void oracle_mrope_apply(int dtype, int rank, int64_t B, int64_t S, int64_t H,
                        int64_t D, int64_t R, int64_t interleaved,
                        const void* x, void* y, const void* cos_cache,
                        const void* sin_cache, const int64_t* ids, int64_t M,
                        const int64_t section[3], int64_t layout, float scale)
{
    int64_t half = R / 2;
    int8_t* stream = (int8_t*)calloc((size_t)(half > 0 ? half : 1), 1);
    coef_row cr;
    if (!stream || !coef_alloc(&cr, half))
        abort();
    if (oracle_mrope_slot_streams(half, section, layout, stream) != 0)
        abort();
    for (int64_t b = 0; b < B; ++b)
        for (int64_t s = 0; s < S; ++s) {
            for (int64_t i = 0; i < half; ++i) {
                int64_t p = ids[(int64_t)stream[i] * B * S + b * S + s];
                cr.copy[i] = (unsigned char)!(p >= 0 && p < M);
                if (cr.copy[i])
                    continue;
                double c = load_elem(dtype, cos_cache, p * half + i);
                double sn = load_elem(dtype, sin_cache, p * half + i);
                /* scale in binary32, then back to the storage type */
                cr.c[i] = round_to_storage(dtype, (double)(float)(c * (double)scale));
                cr.s[i] = round_to_storage(dtype, (double)(float)(sn * (double)scale));
            }
            for (int64_t h = 0; h < H; ++h)
                rotate_row(dtype, x, y, row_offset(rank, S, H, D, b, h, s), D,
                           R, interleaved, cr.c, cr.s, cr.copy);
        }
    coef_free(&cr);
    free(stream);
}

/* ------------------------------------------------------------------------ */
/* Q and K with shared coefficients: [PR] apply_rotary_pos_emb (q_embed and
 * k_embed from one cos/sin), [SA] Attributes (`kv_num_heads`, rotary on Q and
 * on K). */

void oracle_rope_apply_qk(int dtype, int rank, int64_t B, int64_t S, int64_t H,
                          int64_t Hk, int64_t D, int64_t R,
                          int64_t interleaved, const void* q, const void* k,
                          void* yq, void* yk, const void* cos_cache,
                          const void* sin_cache, const int64_t* ids, int64_t M,
                          const float* inv_freq, float scaling)
{
    if (cos_cache) {
        oracle_rope_apply(dtype, rank, B, S, H, D, R, interleaved, q, yq,
                          cos_cache, sin_cache, ids, M);
        oracle_rope_apply(dtype, rank, B, S, Hk, D, R, interleaved, k, yk,
                          cos_cache, sin_cache, ids, M);
        return;
    }
    int64_t half = R / 2;
    coef_row cr;
    if (!coef_alloc(&cr, half))
        abort();
    for (int64_t b = 0; b < B; ++b)
        for (int64_t s = 0; s < S; ++s) {
            int64_t p = ids[b * S + s];
            for (int64_t i = 0; i < half; ++i)
                coefficient(dtype, p, inv_freq[i], scaling, &cr.c[i], &cr.s[i]);
            for (int64_t h = 0; h < H; ++h)
                rotate_row(dtype, q, yq, row_offset(rank, S, H, D, b, h, s), D,
                           R, interleaved, cr.c, cr.s, cr.copy);
            for (int64_t h = 0; h < Hk; ++h)
                rotate_row(dtype, k, yk, row_offset(rank, S, Hk, D, b, h, s),
                           D, R, interleaved, cr.c, cr.s, cr.copy);
        }
    coef_free(&cr);
}

/* ------------------------------------------------------------------------ */
/* RoPE on Q and K and the key/value cache append: [SA] Description (the
 * past/present caches share storage and are updated in place), Inputs
 * (`query` plain or packed [Q|K|V], `past_key`/`past_value` of shape
 * (B, Hk, Smax, D), `total_sequence_length`, `key_total_sequence_lengths`,
 * `cos_cache`/`sin_cache` of width R/2), Attributes (`do_rotary`: Q and K are
 * rotated before K enters the cache; `rotary_interleaved`; `kv_num_heads`).
 *
 * The page decides the past length from total_sequence_length alone: equal
 * to S is the prompt, where every sequence starts at 0. Otherwise the
 * per-batch total key length L[b] counts the past plus the S new tokens, so
 * the past is L[b] - S (reading taken: new tokens follow the past directly).
 * Token s of sequence b has position p = past + s: its pairs use table row p
 * (an id outside [0, M) keeps the pair, as elsewhere in this file), its
 * rotated Q row goes to q_out, its rotated K row and its V row go to row p of
 * the caches (a row outside [0, Smax) is not written -- outside the contract,
 * which bounds L[b] by total_sequence_length and that by the cache).
 * key == NULL: query is packed, per token H query heads, then Hk key heads,
 * then Hk value heads. */
static void norm_row(int dtype, const void* x, int64_t off, const void* w,
                     int64_t D, double eps, double* z);
static void rotate_values(int dtype, const double* z, void* y, int64_t off,
                          int64_t D, int64_t R, int64_t interleaved,
                          const double* c, const double* s,
                          const unsigned char* copy);

void oracle_rope_kv_append(int dtype, int64_t B, int64_t S, int64_t H,
                           int64_t Hk, int64_t D, int64_t R,
                           int64_t interleaved, const void* query,
                           const void* key, const void* value,
                           const int32_t* key_total_sequence_lengths,
                           int64_t total_sequence_length,
                           const void* cos_cache, const void* sin_cache,
                           int64_t M, void* past_key, void* past_value,
                           int64_t Smax, void* q_out, const void* q_weight,
                           const void* k_weight, float epsilon)
{
    int64_t half = R / 2;
    int packed = key == NULL;
    int64_t qw = packed ? (H + 2 * Hk) * D : H * D; /* query row width */
    int64_t kw = packed ? qw : Hk * D;
    const void* ksrc = packed ? query : key;
    const void* vsrc = packed ? query : value;
    int64_t k0 = packed ? H * D : 0;            /* first key element of a token */
    int64_t v0 = packed ? (H + Hk) * D : 0;
    int prompt = total_sequence_length == S;
    coef_row cr;
    double* z = (double*)calloc((size_t)(D > 0 ? D : 1), sizeof(double));
    if (!z || !coef_alloc(&cr, half))
        abort();
    for (int64_t b = 0; b < B; ++b) {
        int64_t past = prompt ? 0 : (int64_t)key_total_sequence_lengths[b] - S;
        for (int64_t s = 0; s < S; ++s) {
            int64_t p = past + s;
            int in_range = p >= 0 && p < M;
            for (int64_t i = 0; i < half; ++i) {
                cr.copy[i] = (unsigned char)!in_range;
                if (in_range) {
                    cr.c[i] = load_elem(dtype, cos_cache, p * half + i);
                    cr.s[i] = load_elem(dtype, sin_cache, p * half + i);
                }
            }
            int64_t tok = b * S + s;
            for (int64_t h = 0; h < H; ++h) {
                if (q_weight) { /* QK-norm first (oracle_rope_apply_qk_norm) */
                    norm_row(dtype, query, tok * qw + h * D, q_weight, D,
                             (double)epsilon, z);
                    rotate_values(dtype, z, q_out, (tok * H + h) * D, D, R,
                                  interleaved, cr.c, cr.s, cr.copy);
                } else {
                    rotate_row_to(dtype, query, tok * qw + h * D, q_out,
                                  (tok * H + h) * D, D, R, interleaved, cr.c,
                                  cr.s, cr.copy);
                }
            }
            if (p < 0 || p >= Smax)
                continue;
            for (int64_t h = 0; h < Hk; ++h) {
                int64_t dst = ((b * Hk + h) * Smax + p) * D;
                if (k_weight) {
                    norm_row(dtype, ksrc, tok * kw + k0 + h * D, k_weight, D,
                             (double)epsilon, z);
                    rotate_values(dtype, z, past_key, dst, D, R, interleaved,
                                  cr.c, cr.s, cr.copy);
                } else {
                    rotate_row_to(dtype, ksrc, tok * kw + k0 + h * D, past_key,
                                  dst, D, R, interleaved, cr.c, cr.s, cr.copy);
                }
                for (int64_t j = 0; j < D; ++j)
                    copy_elem_to(dtype, vsrc, tok * kw + v0 + h * D + j,
                                 past_value, dst + j);
            }
        }
    }
    coef_free(&cr);
    free(z);
}

/* ------------------------------------------------------------------------ */
/* QK-norm then RoPE: [PR] review, Qwen3 architecture (RMSNorm is applied to Q
 * and K after the projection and reshape, before RoPE; the fused graph holds
 * SimplifiedLayerNormalization nodes for it). RMSNorm of a head row x of D
 * elements with weight g (D values) and epsilon e:
 *     z_j = x_j * g_j / sqrt(mean_k(x_k^2) + e)
 * (reading taken: the standard RMSNorm over the head dimension; the pages
 * name it without writing it out). The rotation then acts on z exactly as
 * oracle_rope_apply_qk acts on x; a kept pair and the tail hold z. All in
 * binary64, one rounding to the storage type (the fused op never stores z).
 * q_weight and k_weight are (D,) arrays of the storage type. */
static void norm_row(int dtype, const void* x, int64_t off, const void* w,
                     int64_t D, double eps, double* z)
{
    double ss = 0.0;
    for (int64_t j = 0; j < D; ++j) {
        double v = load_elem(dtype, x, off + j);
        ss += v * v;
    }
    double inv_rms = 1.0 / sqrt(ss / (double)D + eps);
    for (int64_t j = 0; j < D; ++j)
        z[j] = load_elem(dtype, x, off + j) * inv_rms * load_elem(dtype, w, j);
}

static void rotate_values(int dtype, const double* z, void* y, int64_t off,
                          int64_t D, int64_t R, int64_t interleaved,
                          const double* c, const double* s,
                          const unsigned char* copy)
{
    int64_t half = R / 2;
    for (int64_t i = 0; i < half; ++i) {
        int64_t j1 = interleaved ? 2 * i : i;
        int64_t j2 = interleaved ? 2 * i + 1 : i + half;
        if (copy[i]) {
            store_elem(dtype, y, off + j1, z[j1]);
            store_elem(dtype, y, off + j2, z[j2]);
            continue;
        }
        store_elem(dtype, y, off + j1, z[j1] * c[i] - z[j2] * s[i]);
        store_elem(dtype, y, off + j2, z[j2] * c[i] + z[j1] * s[i]);
    }
    for (int64_t j = R; j < D; ++j)
        store_elem(dtype, y, off + j, z[j]);
}

void oracle_rope_apply_qk_norm(int dtype, int rank, int64_t B, int64_t S,
                               int64_t H, int64_t Hk, int64_t D, int64_t R,
                               int64_t interleaved, const void* q,
                               const void* k, const void* q_weight,
                               const void* k_weight, float epsilon, void* yq,
                               void* yk, const void* cos_cache,
                               const void* sin_cache, const int64_t* ids,
                               int64_t M, const float* inv_freq,
                               float scaling)
{
    int64_t half = R / 2;
    coef_row cr;
    double* z = (double*)calloc((size_t)(D > 0 ? D : 1), sizeof(double));
    if (!z || !coef_alloc(&cr, half))
        abort();
    for (int64_t b = 0; b < B; ++b)
        for (int64_t s = 0; s < S; ++s) {
            /* the coefficient row of the token: table row (gathered or per
             * token), or on the fly from inv_freq */
            int64_t row = ids ? ids[b * S + s] : b * S + s;
            int in_range = cos_cache == NULL || !ids || (row >= 0 && row < M);
            for (int64_t i = 0; i < half; ++i) {
                cr.copy[i] = (unsigned char)!in_range;
                if (!in_range)
                    continue;
                if (cos_cache) {
                    cr.c[i] = load_elem(dtype, cos_cache, row * half + i);
                    cr.s[i] = load_elem(dtype, sin_cache, row * half + i);
                } else {
                    coefficient(dtype, row, inv_freq[i], scaling, &cr.c[i],
                                &cr.s[i]);
                }
            }
            for (int64_t h = 0; h < H; ++h) {
                int64_t off = row_offset(rank, S, H, D, b, h, s);
                norm_row(dtype, q, off, q_weight, D, (double)epsilon, z);
                rotate_values(dtype, z, yq, off, D, R, interleaved, cr.c, cr.s,
                              cr.copy);
            }
            for (int64_t h = 0; h < Hk; ++h) {
                int64_t off = row_offset(rank, S, Hk, D, b, h, s);
                norm_row(dtype, k, off, k_weight, D, (double)epsilon, z);
                rotate_values(dtype, z, yk, off, D, R, interleaved, cr.c, cr.s,
                              cr.copy);
            }
        }
    coef_free(&cr);
    free(z);
}
