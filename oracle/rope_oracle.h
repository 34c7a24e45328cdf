/*
 * rope_oracle.h -- scalar CPU oracle for rotary position embedding apply.
 *
 * TEST INFRASTRUCTURE ONLY. This is the plain, slow definition of what the
 * GPU library computes, evaluated one element at a time in binary64 and
 * rounded once to the storage type. Only the test suite, the smoke check and
 * the benchmark's CPU-baseline leg may load it. The product library never
 * links it and shares no code, header, table or helper with it.
 *
 * Sources (web pages, cited by title and section):
 *  [RE]  "ai.onnx.RotaryEmbedding" WebGPU kernel manifest: `inputs`,
 *        `attributes`, `attributeDescriptions`, `derive` contracts.
 *  [MRE] "com.microsoft.MRotaryEmbedding" README: Description, Inputs,
 *        Attributes, Implementation variants (`pairs4`).
 *  [PR]  onnxruntime PR #27590 "Add RotaryEmbedding fusion for Qwen3
 *        on-the-fly RoPE patterns": Motivation (on-the-fly cos/sin), review
 *        "Modeling Code Alignment Check" (forward, rotate_half,
 *        apply_rotary_pos_emb), review item 4 (cache = cos(freqs)*scaling).
 *  [SA]  "com.microsoft.SparseAttention" README: Attributes (`do_rotary`,
 *        `rotary_interleaved`, `kv_num_heads`).
 *
 * Storage types use ONNX TensorProto codes: 1 = float32, 10 = float16,
 * 16 = bfloat16. float16 and bfloat16 tensors are passed as arrays of
 * uint16_t bit patterns.
 * All pointers are host pointers; all arrays are dense row-major.
 *
 * Parity status of each function is listed in its comment; "parity unpinned"
 * marks a reading that nothing on the pages fixes.
 */
#ifndef ROPE_ORACLE_H
#define ROPE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_F32 1
#define ORACLE_F16 10
#define ORACLE_BF16 16

/* IEEE-754 binary16 <-> binary64, round-to-nearest-even, subnormals kept. */
double   oracle_f16_to_f64(uint16_t h);
uint16_t oracle_f64_to_f16(double v);

/* bfloat16 (1 sign, 8 exponent bits with bias 127, 7 fraction bits: the
 * upper half of a binary32) <-> binary64, nearest-even, subnormals kept. */
double   oracle_bf16_to_f64(uint16_t h);
uint16_t oracle_f64_to_bf16(double v);

/* Frequency schedule inv_freq[i] = rnd_f32(base^(-2i/R)), i < R/2.
 * The pages never print the formula ([PR] takes inv_freq from the model's
 * initializer); this is the standard schedule the workloads name. */
void oracle_inv_freq(double base, int64_t rotary_dim, float* inv_freq);

/* cos/sin table of [PR] review item 4: for row p and slot i,
 *   theta = rnd_f32(rnd_f32(p) * inv_freq[i])
 *   cos[p][i] = rnd_T(rnd_f32(rnd_f32(cos(theta)) * scaling)), sin likewise,
 * with cos/sin of the exact binary32 theta evaluated in binary64.
 * Outputs are (rows, half) arrays of storage type `dtype`. */
void oracle_cos_sin_cache(int dtype, int64_t rows, int64_t half,
                          const float* inv_freq, float scaling,
                          void* cos_out, void* sin_out);

/* RotaryEmbedding [RE]. X viewed as x(b,h,s,d):
 *   rank 4: X[b][h][s][d]; rank 3: X[b][s][h*D + d].
 * ids == NULL: cos/sin are (B,S,R/2) and token (b,s) uses row b*S+s.
 * ids != NULL: cos/sin are (M,R/2), token (b,s) uses row ids[b*S+s];
 *   an id outside [0,M) copies every rotation pair of that token through
 *   unchanged (reading taken where [RE] leaves such ids outside the contract).
 * Pairing: interleaved==0 -> (i, i+R/2); interleaved!=0 -> (2i, 2i+1).
 * Elements R..D-1 are bit-copied. */
void oracle_rope_apply(int dtype, int rank, int64_t B, int64_t S, int64_t H,
                       int64_t D, int64_t R, int64_t interleaved,
                       const void* x, void* y, const void* cos_cache,
                       const void* sin_cache, const int64_t* ids, int64_t M);

/* M-RoPE slot -> stream map (0 = temporal, 1 = height, 2 = width) for the
 * half-rotary axis of `half` slots [MRE] Attributes `mrope_section`,
 * `mrope_layout`. Layout 0: consecutive sections. Layout 1: slots visited in
 * order, streams taken in turn t, h, w, a stream skipped once it holds its
 * section count (reading taken where [MRE] names the layout without defining
 * it; parity unpinned where section_h != section_w or section_t < section_h).
 * Returns 0, or -1 if the sections are negative or do not sum to `half`. */
int oracle_mrope_slot_streams(int64_t half, const int64_t section[3],
                              int64_t layout, int8_t* stream_of_slot);

/* MRotaryEmbedding [MRE]. ids is (3,B,S); cos/sin are (M, R/2). Slot i of
 * token (b,s) reads row p = ids[k][b][s] with k its stream. If p is outside
 * [0,M) the pair is bit-copied; otherwise the coefficients are
 * rnd_T(rnd_f32(c * scale)) ([MRE] `pairs4`: scaled coefficients rounded to
 * the storage type). Tail bit-copied. */
void oracle_mrope_apply(int dtype, int rank, int64_t B, int64_t S, int64_t H,
                        int64_t D, int64_t R, int64_t interleaved,
                        const void* x, void* y, const void* cos_cache,
                        const void* sin_cache, const int64_t* ids, int64_t M,
                        const int64_t section[3], int64_t layout, float scale);

/* Coefficient row of the on-the-fly variant [PR] Motivation: the same
 * arithmetic as oracle_cos_sin_cache for one position p (any int64). */
void oracle_onthefly_row(int dtype, int64_t p, const float* inv_freq,
                         int64_t half, float scaling, void* cos_row,
                         void* sin_row);

/* Q and K of one attention layer rotated with the same ids and coefficients
 * ([PR] apply_rotary_pos_emb; [SA] "RoPE on Q and on K"). Q has H heads, K has
 * Hk heads, same B, S, D, rank. If cos_cache == NULL the coefficients come
 * from oracle_onthefly_row(ids[b*S+s], inv_freq, R/2, scaling); ids required.
 * Otherwise exactly oracle_rope_apply on Q and on K. */
void oracle_rope_apply_qk(int dtype, int rank, int64_t B, int64_t S, int64_t H,
                          int64_t Hk, int64_t D, int64_t R,
                          int64_t interleaved, const void* q, const void* k,
                          void* yq, void* yk, const void* cos_cache,
                          const void* sin_cache, const int64_t* ids, int64_t M,
                          const float* inv_freq, float scaling);

/* RoPE on Q and K plus the in-place key/value cache append of [SA]
 * (Description, Inputs, Attributes). query is (B, S, H*D), or packed
 * (B, S, (H + 2*Hk)*D) when key == value == NULL; key/value (B, S, Hk*D);
 * past_key/past_value (B, Hk, Smax, D), updated in place; cos/sin (M, R/2);
 * key_total_sequence_lengths (B,) int32; q_out (B, S, H*D).
 * Prompt (total_sequence_length == S): past = 0; otherwise past =
 * key_total_sequence_lengths[b] - S (reading taken). Token s has position
 * p = past + s: Q and K rows rotated with table row p (p outside [0, M)
 * keeps the pairs), Q to q_out, K and V (bit copy) to cache row p when
 * 0 <= p < Smax (rows outside are not written).
 * q_weight/k_weight non-NULL: the Q, resp. K, rows are first RMS-normalised
 * exactly as in oracle_rope_apply_qk_norm (epsilon; V is never normalised):
 * the decode step of a model with QK-norm, in one call. */
void oracle_rope_kv_append(int dtype, int64_t B, int64_t S, int64_t H,
                           int64_t Hk, int64_t D, int64_t R,
                           int64_t interleaved, const void* query,
                           const void* key, const void* value,
                           const int32_t* key_total_sequence_lengths,
                           int64_t total_sequence_length,
                           const void* cos_cache, const void* sin_cache,
                           int64_t M, void* past_key, void* past_value,
                           int64_t Smax, void* q_out, const void* q_weight,
                           const void* k_weight, float epsilon);

/* QK-norm then RoPE ([PR] review, Qwen3 architecture: RMSNorm on Q and K
 * before RoPE). Each head row x of Q (K) becomes
 *     z_j = x_j * w_j / sqrt(mean_k(x_k^2) + epsilon)
 * with w = q_weight (k_weight), (D,) of the storage type (reading taken: the
 * standard RMSNorm over the head dimension). z is then rotated as
 * oracle_rope_apply_qk rotates x (same tables, ids, on-the-fly rule); kept
 * pairs and the tail hold z. Binary64 throughout, one rounding to the storage
 * type. Parity pinned by closed forms and invariants (mean of squares,
 * epsilon, weights, scale invariance). */
void oracle_rope_apply_qk_norm(int dtype, int rank, int64_t B, int64_t S,
                               int64_t H, int64_t Hk, int64_t D, int64_t R,
                               int64_t interleaved, const void* q,
                               const void* k, const void* q_weight,
                               const void* k_weight, float epsilon, void* yq,
                               void* yk, const void* cos_cache,
                               const void* sin_cache, const int64_t* ids,
                               int64_t M, const float* inv_freq,
                               float scaling);

#ifdef __cplusplus
}
#endif

#endif /* ROPE_ORACLE_H */
