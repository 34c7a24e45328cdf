// rope_abi.cpp -- the extern "C" entry points declared in rope_mi355x.h:
// validate (rope_plan.cpp), then enqueue (rope_kernels.hip).
#include "rope_launch.hpp"
#include "rope_mi355x.h"
#include "rope_plan.hpp"

using rope::Plan;

extern "C" {

const char* rope_status_string(int status) {
    switch (status) {
        case ROPE_OK: return "ROPE_OK";
        case ROPE_ERR_NULL: return "ROPE_ERR_NULL";
        case ROPE_ERR_DTYPE: return "ROPE_ERR_DTYPE";
        case ROPE_ERR_RANK: return "ROPE_ERR_RANK";
        case ROPE_ERR_SHAPE: return "ROPE_ERR_SHAPE";
        case ROPE_ERR_ATTRIBUTE: return "ROPE_ERR_ATTRIBUTE";
        case ROPE_ERR_UNSUPPORTED: return "ROPE_ERR_UNSUPPORTED";
        case ROPE_ERR_ALIAS: return "ROPE_ERR_ALIAS";
        case ROPE_ERR_LAUNCH: return "ROPE_ERR_LAUNCH";
        default: return "ROPE_ERR_UNKNOWN";
    }
}

const char* rope_last_error(void) { return rope::last_error(); }

int rope_set_kernel_policy(int policy) {
    return rope::set_kernel_policy(policy >= 1 && policy <= 3 ? policy : 0);
}

int rope_apply_check(const rope_tensor* x, const rope_tensor* cos_cache,
                     const rope_tensor* sin_cache, const rope_tensor* position_ids,
                     const rope_tensor* y, int64_t interleaved, int64_t num_heads,
                     int64_t rotary_embedding_dim, const char** variant) {
    Plan pl;
    int rc = rope::plan_rope(x, cos_cache, sin_cache, position_ids, y, interleaved, num_heads,
                             rotary_embedding_dim, &pl);
    if (rc == ROPE_OK && variant) *variant = pl.g.variant;
    return rc;
}

int rope_apply(const rope_tensor* x, const rope_tensor* cos_cache, const rope_tensor* sin_cache,
               const rope_tensor* position_ids, const rope_tensor* y, int64_t interleaved,
               int64_t num_heads, int64_t rotary_embedding_dim, void* stream) {
    Plan pl;
    int rc = rope::plan_rope(x, cos_cache, sin_cache, position_ids, y, interleaved, num_heads,
                             rotary_embedding_dim, &pl);
    if (rc != ROPE_OK) return rc;
    return rope::launch_plan(pl, stream);
}

int mrope_apply_check(const rope_tensor* x, const rope_tensor* position_ids,
                      const rope_tensor* cos_cache, const rope_tensor* sin_cache,
                      const rope_tensor* y, int64_t interleaved, int64_t is_packed_batching,
                      int64_t mrope_layout, const int64_t mrope_section[3], int64_t num_heads,
                      int64_t rotary_embedding_dim, float scale, const char** variant) {
    Plan pl;
    int rc = rope::plan_mrope(x, position_ids, cos_cache, sin_cache, y, interleaved,
                              is_packed_batching, mrope_layout, mrope_section, num_heads,
                              rotary_embedding_dim, scale, &pl);
    if (rc == ROPE_OK && variant) *variant = pl.g.variant;
    return rc;
}

int mrope_apply(const rope_tensor* x, const rope_tensor* position_ids, const rope_tensor* cos_cache,
                const rope_tensor* sin_cache, const rope_tensor* y, int64_t interleaved,
                int64_t is_packed_batching, int64_t mrope_layout, const int64_t mrope_section[3],
                int64_t num_heads, int64_t rotary_embedding_dim, float scale, void* stream) {
    Plan pl;
    int rc = rope::plan_mrope(x, position_ids, cos_cache, sin_cache, y, interleaved,
                              is_packed_batching, mrope_layout, mrope_section, num_heads,
                              rotary_embedding_dim, scale, &pl);
    if (rc != ROPE_OK) return rc;
    return rope::launch_plan(pl, stream);
}

int rope_apply_qk_check(const rope_tensor* q, const rope_tensor* k, const rope_tensor* cos_cache,
                        const rope_tensor* sin_cache, const rope_tensor* position_ids,
                        const rope_tensor* yq, const rope_tensor* yk, int64_t interleaved,
                        int64_t num_heads, int64_t kv_num_heads, int64_t rotary_embedding_dim,
                        const rope_tensor* inv_freq, float attention_scaling,
                        const char** variant) {
    Plan pl;
    int rc = rope::plan_rope_qk(q, k, cos_cache, sin_cache, position_ids, yq, yk, interleaved,
                                num_heads, kv_num_heads, rotary_embedding_dim, inv_freq,
                                attention_scaling, &pl);
    if (rc == ROPE_OK && variant) *variant = pl.g.variant;
    return rc;
}

int rope_apply_qk(const rope_tensor* q, const rope_tensor* k, const rope_tensor* cos_cache,
                  const rope_tensor* sin_cache, const rope_tensor* position_ids,
                  const rope_tensor* yq, const rope_tensor* yk, int64_t interleaved,
                  int64_t num_heads, int64_t kv_num_heads, int64_t rotary_embedding_dim,
                  const rope_tensor* inv_freq, float attention_scaling, void* stream) {
    Plan pl;
    int rc = rope::plan_rope_qk(q, k, cos_cache, sin_cache, position_ids, yq, yk, interleaved,
                                num_heads, kv_num_heads, rotary_embedding_dim, inv_freq,
                                attention_scaling, &pl);
    if (rc != ROPE_OK) return rc;
    return rope::launch_plan(pl, stream);
}

int rope_apply_qkv_packed_check(const rope_tensor* qkv, const rope_tensor* cos_cache,
                                const rope_tensor* sin_cache, const rope_tensor* position_ids,
                                const rope_tensor* y, int64_t interleaved, int64_t num_heads,
                                int64_t kv_num_heads, int64_t rotary_embedding_dim,
                                const rope_tensor* inv_freq, float attention_scaling,
                                const char** variant) {
    Plan pl;
    int rc = rope::plan_rope_qkv_packed(qkv, cos_cache, sin_cache, position_ids, y, interleaved,
                                        num_heads, kv_num_heads, rotary_embedding_dim, inv_freq,
                                        attention_scaling, &pl);
    if (rc == ROPE_OK && variant) *variant = pl.g.variant;
    return rc;
}

int rope_apply_qkv_packed(const rope_tensor* qkv, const rope_tensor* cos_cache,
                          const rope_tensor* sin_cache, const rope_tensor* position_ids,
                          const rope_tensor* y, int64_t interleaved, int64_t num_heads,
                          int64_t kv_num_heads, int64_t rotary_embedding_dim,
                          const rope_tensor* inv_freq, float attention_scaling, void* stream) {
    Plan pl;
    int rc = rope::plan_rope_qkv_packed(qkv, cos_cache, sin_cache, position_ids, y, interleaved,
                                        num_heads, kv_num_heads, rotary_embedding_dim, inv_freq,
                                        attention_scaling, &pl);
    if (rc != ROPE_OK) return rc;
    return rope::launch_plan(pl, stream);
}

int rope_apply_qk_norm_check(const rope_tensor* q, const rope_tensor* k, const rope_tensor* q_weight,
                             const rope_tensor* k_weight, float epsilon, const rope_tensor* cos_cache,
                             const rope_tensor* sin_cache, const rope_tensor* position_ids,
                             const rope_tensor* yq, const rope_tensor* yk, int64_t interleaved,
                             int64_t num_heads, int64_t kv_num_heads, int64_t rotary_embedding_dim,
                             const rope_tensor* inv_freq, float attention_scaling, const char** variant) {
    Plan pl;
    int rc = rope::plan_rope_qk_norm(q, k, q_weight, k_weight, epsilon, cos_cache, sin_cache,
                                     position_ids, yq, yk, interleaved, num_heads, kv_num_heads,
                                     rotary_embedding_dim, inv_freq, attention_scaling, &pl);
    if (rc == ROPE_OK && variant) *variant = pl.g.variant;
    return rc;
}

int rope_apply_qk_norm(const rope_tensor* q, const rope_tensor* k, const rope_tensor* q_weight,
                       const rope_tensor* k_weight, float epsilon, const rope_tensor* cos_cache,
                       const rope_tensor* sin_cache, const rope_tensor* position_ids,
                       const rope_tensor* yq, const rope_tensor* yk, int64_t interleaved,
                       int64_t num_heads, int64_t kv_num_heads, int64_t rotary_embedding_dim,
                       const rope_tensor* inv_freq, float attention_scaling, void* stream) {
    Plan pl;
    int rc = rope::plan_rope_qk_norm(q, k, q_weight, k_weight, epsilon, cos_cache, sin_cache,
                                     position_ids, yq, yk, interleaved, num_heads, kv_num_heads,
                                     rotary_embedding_dim, inv_freq, attention_scaling, &pl);
    if (rc != ROPE_OK) return rc;
    return rope::launch_plan(pl, stream);
}

int rope_kv_append_check(const rope_tensor* query, const rope_tensor* key, const rope_tensor* value,
                         const rope_tensor* past_key, const rope_tensor* past_value,
                         const rope_tensor* key_total_sequence_lengths, int64_t total_sequence_length,
                         const rope_tensor* cos_cache, const rope_tensor* sin_cache,
                         const rope_tensor* q_out, int64_t rotary_interleaved, int64_t num_heads,
                         int64_t kv_num_heads, const char** variant) {
    Plan pl;
    int rc = rope::plan_rope_kv_append(query, key, value, past_key, past_value,
                                       key_total_sequence_lengths, total_sequence_length, cos_cache,
                                       sin_cache, q_out, rotary_interleaved, num_heads, kv_num_heads,
                                       &pl);
    if (rc == ROPE_OK && variant) *variant = pl.g.variant;
    return rc;
}

int rope_kv_append(const rope_tensor* query, const rope_tensor* key, const rope_tensor* value,
                   const rope_tensor* past_key, const rope_tensor* past_value,
                   const rope_tensor* key_total_sequence_lengths, int64_t total_sequence_length,
                   const rope_tensor* cos_cache, const rope_tensor* sin_cache,
                   const rope_tensor* q_out, int64_t rotary_interleaved, int64_t num_heads,
                   int64_t kv_num_heads, void* stream) {
    Plan pl;
    int rc = rope::plan_rope_kv_append(query, key, value, past_key, past_value,
                                       key_total_sequence_lengths, total_sequence_length, cos_cache,
                                       sin_cache, q_out, rotary_interleaved, num_heads, kv_num_heads,
                                       &pl);
    if (rc != ROPE_OK) return rc;
    return rope::launch_plan(pl, stream);
}

int rope_kv_append_qk_norm_check(const rope_tensor* query, const rope_tensor* key,
                                 const rope_tensor* value, const rope_tensor* past_key,
                                 const rope_tensor* past_value,
                                 const rope_tensor* key_total_sequence_lengths,
                                 int64_t total_sequence_length, const rope_tensor* cos_cache,
                                 const rope_tensor* sin_cache, const rope_tensor* q_out,
                                 const rope_tensor* q_weight, const rope_tensor* k_weight,
                                 float epsilon, int64_t rotary_interleaved, int64_t num_heads,
                                 int64_t kv_num_heads, const char** variant) {
    Plan pl;
    int rc = rope::plan_rope_kv_append_qk_norm(query, key, value, past_key, past_value,
                                               key_total_sequence_lengths, total_sequence_length,
                                               cos_cache, sin_cache, q_out, q_weight, k_weight,
                                               epsilon, rotary_interleaved, num_heads, kv_num_heads,
                                               &pl);
    if (rc == ROPE_OK && variant) *variant = pl.g.variant;
    return rc;
}

int rope_kv_append_qk_norm(const rope_tensor* query, const rope_tensor* key,
                           const rope_tensor* value, const rope_tensor* past_key,
                           const rope_tensor* past_value,
                           const rope_tensor* key_total_sequence_lengths,
                           int64_t total_sequence_length, const rope_tensor* cos_cache,
                           const rope_tensor* sin_cache, const rope_tensor* q_out,
                           const rope_tensor* q_weight, const rope_tensor* k_weight, float epsilon,
                           int64_t rotary_interleaved, int64_t num_heads, int64_t kv_num_heads,
                           void* stream) {
    Plan pl;
    int rc = rope::plan_rope_kv_append_qk_norm(query, key, value, past_key, past_value,
                                               key_total_sequence_lengths, total_sequence_length,
                                               cos_cache, sin_cache, q_out, q_weight, k_weight,
                                               epsilon, rotary_interleaved, num_heads, kv_num_heads,
                                               &pl);
    if (rc != ROPE_OK) return rc;
    return rope::launch_plan(pl, stream);
}

int rope_inv_freq(const rope_tensor* inv_freq, double base, void* stream) {
    float* out;
    int64_t half;
    int rc = rope::plan_inv_freq(inv_freq, base, &out, &half);
    if (rc != ROPE_OK) return rc;
    return rope::launch_inv_freq(out, half, base, stream);
}

int rope_cos_sin_cache(const rope_tensor* inv_freq, float scaling, const rope_tensor* cos_out,
                       const rope_tensor* sin_out, void* stream) {
    rope::TablePlan t;
    int rc = rope::plan_cos_sin_cache(inv_freq, scaling, cos_out, sin_out, &t);
    if (rc != ROPE_OK) return rc;
    return rope::launch_cos_sin_cache(t, stream);
}

}  // extern "C"
