/*
 * rope_mi355x.h -- C ABI of the rotary position embedding library for
 * AMD Instinct MI355X (gfx950).
 *
 * Operations (the pages are cited by title and section):
 *   rope_apply         ONNX RotaryEmbedding -- "ai.onnx.RotaryEmbedding"
 *                      WebGPU kernel manifest: inputs, attributes,
 *                      attributeDescriptions, derive contracts, variants.
 *   mrope_apply        com.microsoft.MRotaryEmbedding -- its README:
 *                      Description, Inputs, Attributes.
 *   rope_apply_qk      Q and K of one attention layer rotated with the same
 *                      coefficients, from a table or computed on the fly --
 *                      onnxruntime PR #27590 (Motivation; review "Modeling
 *                      Code Alignment Check": Qwen3RotaryEmbedding.forward,
 *                      apply_rotary_pos_emb, GQA) and the
 *                      "com.microsoft.SparseAttention" README (Attributes:
 *                      kv_num_heads, rotary on Q and on K).
 *   rope_apply_qkv_packed  the same on a packed [Q|K|V] activation --
 *                      "com.microsoft.SparseAttention" README (Inputs).
 *   rope_apply_qk_norm RMSNorm of every Q and K head row, then the rotation of
 *                      rope_apply_qk, in one pass -- PR #27590 review, Qwen3
 *                      architecture (QK-Norm before RoPE).
 *   rope_kv_append     RoPE on Q and K with K and V appended to the key and
 *                      value caches in place, one launch --
 *                      "com.microsoft.SparseAttention" README (Description,
 *                      Inputs, Outputs, Attributes).
 *   rope_kv_append_qk_norm  the same with Q and K RMS-normalised first
 *                      (QK-norm before RoPE, as rope_apply_qk_norm).
 *   rope_inv_freq,     the frequency vector and the cos/sin table the
 *   rope_cos_sin_cache gathered ops read -- PR #27590 review item 4
 *                      (cos_cache = cos(pos * inv_freq) * scaling).
 *
 * Conventions for every entry point
 *   - Tensors are described by rope_tensor: a DEVICE pointer to dense
 *     row-major data, an ONNX TensorProto element type and a shape.
 *     Storage types: ROPE_FLOAT (binary32), ROPE_FLOAT16 (binary16) and
 *     ROPE_BFLOAT16 (bfloat16: the upper half of a binary32). The
 *     MRotaryEmbedding README (Description) lists bfloat16 as not implemented
 *     in its package; here it is the same arithmetic with another storage
 *     type. Positions are ROPE_INT64.
 *   - The caller owns every buffer. The library never allocates, frees,
 *     copies to the host or synchronises: it validates on the host, then
 *     enqueues its kernels on `stream` (a hipStream_t; NULL = the null
 *     stream) and returns. Results are ready when the stream reaches them.
 *   - Validation is complete before anything is enqueued: a non-zero return
 *     means nothing was launched. ROPE_ERR_LAUNCH means a launch was
 *     attempted and the HIP runtime refused it. Problems of 2^31 tokens or
 *     more (or whose vector kernel would need 2^31 waves) run on the
 *     grid-stride scalar kernel, whose grid is bounded. A head size or a
 *     head count above 2^31 - 1 is ROPE_ERR_UNSUPPORTED.
 *   - A tensor with a zero dimension is valid; an op whose output is empty
 *     launches nothing and returns ROPE_OK. Data pointers of non-empty
 *     tensors must not be NULL.
 *   - Outputs may be the same buffer as their input (y == x, in place);
 *     any other overlap between an output and an input or another output is
 *     ROPE_ERR_ALIAS.
 *   - Arithmetic: products and sums in binary32 with fused multiply-add,
 *     one rounding to the storage type at the end; subnormals kept. For
 *     binary32 storage the rotation's two products and their sum are formed
 *     in binary64 (both products exact there) and rounded to binary32 once,
 *     so a pair whose products nearly cancel keeps full relative accuracy.
 *     Pass-through elements (the tail beyond the rotary dimension, pairs
 *     with an out-of-range position) are bit copies.
 *   - Stateless and thread-safe; rope_last_error() is per thread.
 */
#ifndef ROPE_MI355X_H
#define ROPE_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ONNX TensorProto element types. */
#define ROPE_FLOAT 1
#define ROPE_INT32 6
#define ROPE_INT64 7
#define ROPE_FLOAT16 10
#define ROPE_BFLOAT16 16

typedef struct rope_tensor {
    void* data;       /* device pointer, dense row-major */
    int32_t dtype;    /* ROPE_FLOAT, ROPE_FLOAT16, ROPE_BFLOAT16, ROPE_INT32, ROPE_INT64 */
    int32_t rank;     /* 1..4 */
    int64_t shape[4]; /* entries beyond `rank` are ignored */
} rope_tensor;

enum rope_status {
    ROPE_OK = 0,
    ROPE_ERR_NULL = -1,        /* missing tensor or NULL data of a non-empty tensor */
    ROPE_ERR_DTYPE = -2,       /* storage type not allowed or inputs disagree */
    ROPE_ERR_RANK = -3,        /* tensor rank not allowed */
    ROPE_ERR_SHAPE = -4,       /* a shape clause of the op's contract fails */
    ROPE_ERR_ATTRIBUTE = -5,   /* attribute value outside its allowed set */
    ROPE_ERR_UNSUPPORTED = -6, /* defined by the op but not implemented here */
    ROPE_ERR_ALIAS = -7,       /* an output overlaps an input or another output */
    ROPE_ERR_LAUNCH = -8       /* the HIP runtime rejected a kernel launch */
};

/* Name of a status code ("ROPE_OK", ...). Never NULL. */
const char* rope_status_string(int status);

/* Human-readable reason of the last non-zero status returned on this thread
 * (which contract clause failed). Empty string if none. */
const char* rope_last_error(void);

/*
 * rope_apply -- ONNX RotaryEmbedding ("ai.onnx.RotaryEmbedding" manifest).
 *
 * x:            rank 3 (B, S, H*D) with num_heads = H, or rank 4 (B, H, S, D).
 *               D must be even. Storage type T in {ROPE_FLOAT, ROPE_FLOAT16, ROPE_BFLOAT16}.
 * cos_cache,
 * sin_cache:    type T, same shape. With position_ids: (M, R/2), row p
 *               serves position p. Without: (B, S, R/2), row (b, s) serves
 *               token (b, s). (manifest `inputs`, `derive`.)
 * position_ids: NULL (absent) or int64 (B, S). An id outside [0, M) passes
 *               the token's rotary pairs through unchanged and never reads
 *               the table (the manifest keeps such ids outside its contract;
 *               this is the behaviour taken).
 * y:            same shape and type as x; may be x itself.
 * interleaved:  0 = pairs (i, i + R/2) (split halves), 1 = pairs (2i, 2i+1).
 * num_heads:    required (>= 1) for rank 3; for rank 4, 0 or dim 1 of x.
 * rotary_embedding_dim: 0 = R = D, else the even R <= D of leading elements
 *               rotated; elements R..D-1 are copied.
 * Per pair with coefficients (c, s) of its slot i:
 *   y1 = x1*c - x2*s,  y2 = x2*c + x1*s.
 */
int rope_apply(const rope_tensor* x, const rope_tensor* cos_cache,
               const rope_tensor* sin_cache, const rope_tensor* position_ids,
               const rope_tensor* y, int64_t interleaved, int64_t num_heads,
               int64_t rotary_embedding_dim, void* stream);

/*
 * mrope_apply -- com.microsoft.MRotaryEmbedding (its README).
 *
 * x:            rank 3 (B, S, H*D) or rank 4 (B, H, S, D), type T.
 * position_ids: int64 (3, B, S): temporal, height, width streams. Required.
 * cos_cache,
 * sin_cache:    type T, (M, R/2), shared by the three streams.
 * y:            same shape and type as x; may be x itself.
 * interleaved:  pairing as for rope_apply; independent of mrope_layout.
 * is_packed_batching: must be 0 (1 is ROPE_ERR_UNSUPPORTED, as on the page).
 * mrope_layout: 0 = sectioned (slots [0,t) temporal, then h height, then w
 *               width); 1 = interleaved: slots dealt to t, h, w in turn, a
 *               stream passed over once it holds its section count (the page
 *               names this layout without spelling out the slot order; this
 *               is the reading taken, and it equals the stride-3 rule of the
 *               models the page names whenever section_h == section_w <=
 *               section_t).
 * mrope_section: 3 non-negative int64 summing to R/2.
 * num_heads:    required (> 0) for rank 3 and whenever rotary_embedding_dim
 *               != 0; for rank 4 it must then equal dim 1 of x.
 * rotary_embedding_dim: 0 = R = D (D must be even), else an even R <= D
 *               (D may then be odd); elements R..D-1 are copied.
 * scale:        applied to gathered coefficients: c' = rnd_T(rnd_f32(c*scale)).
 * Slot i of token (b, s) reads row p = position_ids[k][b][s] of its stream
 * k; p outside [0, M) copies that pair unchanged. Limit: R/2 <= 512.
 */
int mrope_apply(const rope_tensor* x, const rope_tensor* position_ids,
                const rope_tensor* cos_cache, const rope_tensor* sin_cache,
                const rope_tensor* y, int64_t interleaved,
                int64_t is_packed_batching, int64_t mrope_layout,
                const int64_t mrope_section[3], int64_t num_heads,
                int64_t rotary_embedding_dim, float scale, void* stream);

/*
 * rope_apply_qk -- Q (num_heads heads) and K (kv_num_heads heads) of one
 * layer rotated with the same position ids and coefficients, in one launch.
 *
 * q, k:         both rank 3 ((B, S, H*D) and (B, S, Hk*D)) or both rank 4
 *               ((B, H, S, D) and (B, Hk, S, D)); same B, S, D and type T.
 *               kv_num_heads must divide num_heads.
 * yq, yk:       outputs shaped like q and k; may be q and k themselves.
 * Table path:   cos_cache and sin_cache given: exactly rope_apply on q and
 *               on k (gathered with position_ids, or per-token tables).
 * On-the-fly:   cos_cache == sin_cache == NULL: inv_freq (float32, (R/2,))
 *               and position_ids are required, and slot i of a token at
 *               position p uses theta = rnd_f32(rnd_f32(p) * inv_freq[i]),
 *               c = rnd_T(rnd_f32(rnd_f32(cos theta) * attention_scaling)),
 *               s likewise -- the same values rope_cos_sin_cache stores, so
 *               both paths give bit-identical results. Any int64 p is valid.
 * num_heads, kv_num_heads: required for rank 3; for rank 4, 0 or dim 1.
 */
int rope_apply_qk(const rope_tensor* q, const rope_tensor* k,
                  const rope_tensor* cos_cache, const rope_tensor* sin_cache,
                  const rope_tensor* position_ids, const rope_tensor* yq,
                  const rope_tensor* yk, int64_t interleaved,
                  int64_t num_heads, int64_t kv_num_heads,
                  int64_t rotary_embedding_dim, const rope_tensor* inv_freq,
                  float attention_scaling, void* stream);

/*
 * rope_apply_qkv_packed -- the Q and K parts of a packed [Q|K|V] activation
 * ("com.microsoft.SparseAttention" README, Inputs: a packed query holds the
 * query, key and value heads of each token when key and value are omitted)
 * rotated with shared coefficients, in one launch.
 *
 * qkv:          rank 3 (B, S, (H + 2*Hk)*D): per token H query heads, then
 *               Hk key heads, then Hk value heads; or rank 4
 *               (B, H + 2*Hk, S, D) with the head groups in that order.
 * y:            same shape and type. Query and key heads rotated exactly as
 *               rope_apply_qk would; value heads copied bit for bit. y may be
 *               qkv itself (in place); then the value heads are not touched.
 * num_heads, kv_num_heads: required (>= 1, num_heads <= 2^31 - 1); kv_num_heads divides num_heads.
 * Tables, position_ids, inv_freq (on the fly when both tables are NULL),
 * interleaved, rotary_embedding_dim, attention_scaling: as rope_apply_qk.
 */
int rope_apply_qkv_packed(const rope_tensor* qkv, const rope_tensor* cos_cache,
                          const rope_tensor* sin_cache,
                          const rope_tensor* position_ids, const rope_tensor* y,
                          int64_t interleaved, int64_t num_heads,
                          int64_t kv_num_heads, int64_t rotary_embedding_dim,
                          const rope_tensor* inv_freq, float attention_scaling,
                          void* stream);

/*
 * rope_apply_qk_norm -- QK-norm then RoPE in one pass (PR #27590 review,
 * Qwen3 architecture: RMSNorm is applied to Q and K after the projection and
 * reshape, before RoPE). Each head row x (D elements) of Q, resp. K, becomes
 *     z_j = x_j * w_j / sqrt(mean_k(x_k^2) + epsilon)
 * with w = q_weight, resp. k_weight (type T, shape (D,)), and z is rotated
 * exactly as rope_apply_qk rotates x: same tables or on-the-fly rule, ids,
 * interleaved, rotary_embedding_dim, attention_scaling. Pairs kept by an
 * out-of-range id and the tail beyond the rotary dimension hold z. z is not
 * stored: the sum of squares, the scale and the rotation are binary32, with
 * one rounding to T at the end.
 * epsilon: finite, >= 0 (the model's RMSNorm epsilon).
 * Other arguments, shapes, aliasing rules: as rope_apply_qk; the outputs may
 * not overlap the weights.
 */
int rope_apply_qk_norm(const rope_tensor* q, const rope_tensor* k,
                       const rope_tensor* q_weight, const rope_tensor* k_weight,
                       float epsilon, const rope_tensor* cos_cache,
                       const rope_tensor* sin_cache,
                       const rope_tensor* position_ids, const rope_tensor* yq,
                       const rope_tensor* yk, int64_t interleaved,
                       int64_t num_heads, int64_t kv_num_heads,
                       int64_t rotary_embedding_dim,
                       const rope_tensor* inv_freq, float attention_scaling,
                       void* stream);

/*
 * rope_kv_append -- the rotary part of "com.microsoft.SparseAttention"
 * (README Description: past and present key/value caches share storage and
 * are updated in place; Attributes: do_rotary rotates Q and K before K enters
 * the cache, rotary_interleaved, kv_num_heads): Q rotated to q_out, K rotated
 * and V copied into the caches at each token's row, in one launch.
 *
 * query:        (B, S, H*D) of type T (float32, float16, bfloat16); or the
 *               packed (B, S, (H + 2*Hk)*D) -- per token H query, Hk key,
 *               Hk value heads -- when key and value are both NULL.
 * key, value:   (B, S, Hk*D), type T, or both NULL (packed query).
 * past_key, past_value: (B, Hk, Smax, D), type T; rows are written in place
 *               (Outputs: present_key/present_value are these tensors).
 * key_total_sequence_lengths: int32 (B,): per sequence, the total key length
 *               after this call (past + new tokens, padding excluded).
 * total_sequence_length: host value; S <= it <= Smax and <= M required.
 *               Equal to S: the prompt, every sequence starts at position 0.
 *               Otherwise token s of sequence b has position
 *               key_total_sequence_lengths[b] - S + s (the README decides the
 *               past length this way; new tokens follow the past directly).
 * cos_cache, sin_cache: (M, R/2) of type T, R/2 >= 1, R <= D. Rotation as
 *               rope_apply with these tables and those positions (R from the
 *               table width, as the README's cos_cache shape states).
 * q_out:        (B, S, H*D), type T; may be `query` itself when it is not
 *               packed (in place). The caches may not overlap any input,
 *               q_out or each other.
 * rotary_interleaved: 1 adjacent pairs; any other value the half-split
 *               (NeoX) pairs, as the README's Attributes table says.
 * num_heads, kv_num_heads: >= 1, num_heads <= 2^31 - 1, kv_num_heads divides num_heads.
 * Device data outside the README's bounds (a per-sequence length above
 * total_sequence_length or below S): a row outside [0, Smax) is not written
 * and a position outside [0, M) keeps its pairs; nothing is read or written
 * out of bounds.
 */
int rope_kv_append(const rope_tensor* query, const rope_tensor* key,
                   const rope_tensor* value, const rope_tensor* past_key,
                   const rope_tensor* past_value,
                   const rope_tensor* key_total_sequence_lengths,
                   int64_t total_sequence_length, const rope_tensor* cos_cache,
                   const rope_tensor* sin_cache, const rope_tensor* q_out,
                   int64_t rotary_interleaved, int64_t num_heads,
                   int64_t kv_num_heads, void* stream);

/*
 * rope_kv_append_qk_norm -- rope_kv_append with each Q and K head row first
 * RMS-normalised exactly as rope_apply_qk_norm does (weights q_weight and
 * k_weight, type T, shape (D,); epsilon finite and >= 0): the decode step of
 * a model with QK-norm (PR #27590 review, Qwen3 architecture) before
 * attention, in one launch. V is copied into the value cache unnormalised.
 * Arguments, layouts and bounds otherwise as rope_kv_append; the outputs and
 * caches may not overlap the weights.
 */
int rope_kv_append_qk_norm(const rope_tensor* query, const rope_tensor* key,
                           const rope_tensor* value, const rope_tensor* past_key,
                           const rope_tensor* past_value,
                           const rope_tensor* key_total_sequence_lengths,
                           int64_t total_sequence_length,
                           const rope_tensor* cos_cache,
                           const rope_tensor* sin_cache,
                           const rope_tensor* q_out, const rope_tensor* q_weight,
                           const rope_tensor* k_weight, float epsilon,
                           int64_t rotary_interleaved, int64_t num_heads,
                           int64_t kv_num_heads, void* stream);

/*
 * rope_inv_freq -- inv_freq[i] = rnd_f32(base^(-2i/R)) for i < R/2 with
 * R = 2 * dim 0 of inv_freq (float32, rank 1). The pages take inv_freq from
 * the model; this is the standard schedule. base must be > 0.
 */
int rope_inv_freq(const rope_tensor* inv_freq, double base, void* stream);

/*
 * rope_cos_sin_cache -- the (M, R/2) tables of type T for positions 0..M-1:
 *   cos_out[p][i] = rnd_T(rnd_f32(rnd_f32(cos theta) * scaling)),
 *   theta = rnd_f32(rnd_f32(p) * inv_freq[i]), sin likewise
 * (PR #27590 review item 4: the table equals the on-the-fly values).
 * inv_freq: float32 (R/2,). cos_out, sin_out: type T, (M, R/2).
 */
int rope_cos_sin_cache(const rope_tensor* inv_freq, float scaling,
                       const rope_tensor* cos_out, const rope_tensor* sin_out,
                       void* stream);

/*
 * Validation without launching: the same checks as the op, and the kernel
 * variant it would run (static string: the kernel, "vec16", "row16" or
 * "scalar", then "/norm" for the QK-norm ops, then the coefficient source,
 * "gather", "per_token", "mrope", "on_the_fly" or "append"; e.g.
 * "vec16/gather"), written to
 * *variant when variant != NULL and the status is ROPE_OK. Never touches
 * the GPU, so it can be called on a machine without one.
 */
int rope_apply_check(const rope_tensor* x, const rope_tensor* cos_cache,
                     const rope_tensor* sin_cache,
                     const rope_tensor* position_ids, const rope_tensor* y,
                     int64_t interleaved, int64_t num_heads,
                     int64_t rotary_embedding_dim, const char** variant);

int mrope_apply_check(const rope_tensor* x, const rope_tensor* position_ids,
                      const rope_tensor* cos_cache,
                      const rope_tensor* sin_cache, const rope_tensor* y,
                      int64_t interleaved, int64_t is_packed_batching,
                      int64_t mrope_layout, const int64_t mrope_section[3],
                      int64_t num_heads, int64_t rotary_embedding_dim,
                      float scale, const char** variant);

int rope_apply_qk_check(const rope_tensor* q, const rope_tensor* k,
                        const rope_tensor* cos_cache,
                        const rope_tensor* sin_cache,
                        const rope_tensor* position_ids, const rope_tensor* yq,
                        const rope_tensor* yk, int64_t interleaved,
                        int64_t num_heads, int64_t kv_num_heads,
                        int64_t rotary_embedding_dim,
                        const rope_tensor* inv_freq, float attention_scaling,
                        const char** variant);

int rope_apply_qkv_packed_check(const rope_tensor* qkv,
                                const rope_tensor* cos_cache,
                                const rope_tensor* sin_cache,
                                const rope_tensor* position_ids,
                                const rope_tensor* y, int64_t interleaved,
                                int64_t num_heads, int64_t kv_num_heads,
                                int64_t rotary_embedding_dim,
                                const rope_tensor* inv_freq,
                                float attention_scaling, const char** variant);

int rope_apply_qk_norm_check(const rope_tensor* q, const rope_tensor* k,
                             const rope_tensor* q_weight,
                             const rope_tensor* k_weight, float epsilon,
                             const rope_tensor* cos_cache,
                             const rope_tensor* sin_cache,
                             const rope_tensor* position_ids,
                             const rope_tensor* yq, const rope_tensor* yk,
                             int64_t interleaved, int64_t num_heads,
                             int64_t kv_num_heads,
                             int64_t rotary_embedding_dim,
                             const rope_tensor* inv_freq,
                             float attention_scaling, const char** variant);

int rope_kv_append_check(const rope_tensor* query, const rope_tensor* key,
                         const rope_tensor* value, const rope_tensor* past_key,
                         const rope_tensor* past_value,
                         const rope_tensor* key_total_sequence_lengths,
                         int64_t total_sequence_length,
                         const rope_tensor* cos_cache,
                         const rope_tensor* sin_cache,
                         const rope_tensor* q_out, int64_t rotary_interleaved,
                         int64_t num_heads, int64_t kv_num_heads,
                         const char** variant);

int rope_kv_append_qk_norm_check(const rope_tensor* query,
                                 const rope_tensor* key,
                                 const rope_tensor* value,
                                 const rope_tensor* past_key,
                                 const rope_tensor* past_value,
                                 const rope_tensor* key_total_sequence_lengths,
                                 int64_t total_sequence_length,
                                 const rope_tensor* cos_cache,
                                 const rope_tensor* sin_cache,
                                 const rope_tensor* q_out,
                                 const rope_tensor* q_weight,
                                 const rope_tensor* k_weight, float epsilon,
                                 int64_t rotary_interleaved, int64_t num_heads,
                                 int64_t kv_num_heads, const char** variant);

/*
 * Kernel choice for all ops: 0 = automatic (the row kernel for decode-sized
 * launches and for larger ones whose head rows the vector kernel's 16-byte
 * items fit poorly, the vector kernel for the other larger ones, where shapes
 * and alignment allow; the scalar kernel otherwise), 1 = always the scalar
 * kernel, 2 = the
 * vector kernel wherever it applies (never the row kernel), 3 = the row
 * kernel wherever its shape rules allow, at any size. Any other value is
 * taken as 0. Process-wide; returns the previous value. Used to test every
 * path.
 */
int rope_set_kernel_policy(int policy);

#ifdef __cplusplus
}
#endif

#endif /* ROPE_MI355X_H */
