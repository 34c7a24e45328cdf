// rope_plan.hpp -- host-side description of one rotary-embedding launch.
//
// Validation (the ops' contracts) and kernel choice are plain C++ with no HIP
// dependency (rope_plan.cpp); rope_kernels.hip turns a Plan into launches of
// the kernels in rope_device.hpp.
#pragma once

#include <cstdint>

#include "rope_mi355x.h"

namespace rope {

// How a token's coefficient row is obtained.
enum CoefKind : int32_t {
    kCoefGather = 0,   // row ids[b,s] of an (M, R/2) table, id outside [0,M) -> copy
    kCoefPerToken = 1, // row b*S+s of a (B, S, R/2) table
    kCoefMrope = 2,    // slot i from row ids[stream(i), b, s], scaled, per-pair copy
    kCoefOnTheFly = 3, // computed from inv_freq and the position
    kCoefAppend = 4    // row past(b) + s of an (M, R/2) table; outputs may go to
                       // cache row past(b) + s (key/value cache append)
};

constexpr int kMaxMropeHalf = 512;             // slots the stream table can hold
constexpr int kSelWords = kMaxMropeHalf / 16;  // 2 bits per slot

// One input/output pair rotated with the shared coefficients (or, with
// copy set, copied to the output as it is).
struct Task {
    const void* x;
    void* y;
    int64_t heads;
    int64_t stride_b, stride_h, stride_s;  // element strides of x(b, h, s, 0)
    // element strides of y(b, h, row, 0); row = s, or with yrow set (append
    // kind only) the token's position. Equal to the x strides unless set.
    int64_t ystride_b, ystride_h, ystride_s;
    int32_t copy;
    int32_t yrow;
    const void* weight;   // QK-norm: (D,) RMSNorm weight of this projection
};

constexpr int kMaxPlanTasks = 3;

// Waves per workgroup of the vector kernel (the planner's grouping rules
// depend on it).
constexpr int kWavesPerBlock = 4;
// vector kernel, interleaved binary32 data: at most this many heads per wave
// (the head loop of those instances is unrolled)
constexpr int kVecMaxHeads = 16;
// row kernel: 16-byte load instructions per wave (each covering 64 / row_lanes head rows)
constexpr int kRowLoads = 8;
// row kernel, on the fly: slots per token computed once per wave (LDS rows)
constexpr int kRowMaxSlots = 256;
// row kernel, element-wise pairs: at most this many instructions per wave
#ifndef ROPE_ROW_ELEM_LOADS
#define ROPE_ROW_ELEM_LOADS 4
#endif
constexpr int kRowElemLoads = ROPE_ROW_ELEM_LOADS;

struct Problem {
    int32_t dtype;        // ROPE_FLOAT, ROPE_FLOAT16 or ROPE_BFLOAT16
    int32_t interleaved;  // 0 or 1
    int64_t B, S, D, R;   // batch, sequence, head size, rotary dim
    Task task[kMaxPlanTasks];
    int32_t ntask;
    CoefKind coef;
    const void* cos;
    const void* sin;
    const int64_t* ids;
    int64_t M;            // table rows (gathered kinds)
    const float* inv_freq;
    float scaling;        // on-the-fly attention scaling
    float scale;          // M-RoPE coefficient scale
    uint32_t sel[kSelWords];  // M-RoPE stream of slot i in bits 2*(i%16) of word i/16
    int32_t mrope_single;     // M-RoPE: every 16-byte chunk's slots take one stream
    // cache append: per-sequence total lengths, prompt flag, cache rows
    const int32_t* seqlens;
    int32_t prompt;
    int64_t rows_out;
    // QK-norm: every head row RMS-normalised (weights per task) before rotation
    int32_t norm;
    float eps;
};

// Launch geometry of the vector kernel (see rope_device.hpp for the mapping).
struct Geometry {
    bool vector;          // false: scalar kernel
    int32_t rank;         // of the activations
    int32_t items_per_lane;
    int32_t head_batch;   // heads whose loads are issued together (kernel template)
    int32_t W;            // 16-byte work items per head row
    int32_t NP;           // of which rotation items
    int32_t TG;           // tokens per wave
    int32_t tile;         // token groups per head chunk in a tile of waves
    int32_t share_coef;   // on the fly: the 4 waves of a workgroup share one token group
    int32_t group_major;  // three tasks: waves in token-group order (see KArgs)
    int32_t row_kernel;   // 1: the row kernel (lanes along head rows of one token)
    int32_t row_lanes;    // row kernel: lanes per head row
    int32_t row_general;  // row kernel: rows of a size other than a power of two, or partners
                          // a number of lanes apart other than a power of two
    int32_t half_lanes;   // row kernel, split halves: lanes between partner chunks
    int32_t heads_per_wave[kMaxPlanTasks];
    int32_t chunks[kMaxPlanTasks];  // head chunks per token group
    int64_t waves[kMaxPlanTasks];
    const char* variant;
};

struct Plan {
    Problem p;
    Geometry g;
    bool empty;           // nothing to launch
};

int plan_rope(const rope_tensor* x, const rope_tensor* cos_cache,
              const rope_tensor* sin_cache, const rope_tensor* position_ids,
              const rope_tensor* y, int64_t interleaved, int64_t num_heads,
              int64_t rotary_embedding_dim, Plan* out);

int plan_mrope(const rope_tensor* x, const rope_tensor* position_ids,
               const rope_tensor* cos_cache, const rope_tensor* sin_cache,
               const rope_tensor* y, int64_t interleaved,
               int64_t is_packed_batching, int64_t mrope_layout,
               const int64_t mrope_section[3], int64_t num_heads,
               int64_t rotary_embedding_dim, float scale, Plan* out);

int plan_rope_qk(const rope_tensor* q, const rope_tensor* k,
                 const rope_tensor* cos_cache, const rope_tensor* sin_cache,
                 const rope_tensor* position_ids, const rope_tensor* yq,
                 const rope_tensor* yk, int64_t interleaved, int64_t num_heads,
                 int64_t kv_num_heads, int64_t rotary_embedding_dim,
                 const rope_tensor* inv_freq, float attention_scaling,
                 Plan* out);

int plan_rope_qkv_packed(const rope_tensor* qkv, const rope_tensor* cos_cache,
                         const rope_tensor* sin_cache, const rope_tensor* position_ids,
                         const rope_tensor* y, int64_t interleaved, int64_t num_heads,
                         int64_t kv_num_heads, int64_t rotary_embedding_dim,
                         const rope_tensor* inv_freq, float attention_scaling, Plan* out);

int plan_rope_qk_norm(const rope_tensor* q, const rope_tensor* k,
                      const rope_tensor* q_weight, const rope_tensor* k_weight,
                      float epsilon, const rope_tensor* cos_cache,
                      const rope_tensor* sin_cache, const rope_tensor* position_ids,
                      const rope_tensor* yq, const rope_tensor* yk, int64_t interleaved,
                      int64_t num_heads, int64_t kv_num_heads,
                      int64_t rotary_embedding_dim, const rope_tensor* inv_freq,
                      float attention_scaling, Plan* out);

int plan_rope_kv_append(const rope_tensor* query, const rope_tensor* key,
                        const rope_tensor* value, const rope_tensor* past_key,
                        const rope_tensor* past_value,
                        const rope_tensor* key_total_sequence_lengths,
                        int64_t total_sequence_length, const rope_tensor* cos_cache,
                        const rope_tensor* sin_cache, const rope_tensor* q_out,
                        int64_t interleaved, int64_t num_heads, int64_t kv_num_heads,
                        Plan* out);

int plan_rope_kv_append_qk_norm(const rope_tensor* query, const rope_tensor* key,
                                const rope_tensor* value, const rope_tensor* past_key,
                                const rope_tensor* past_value,
                                const rope_tensor* key_total_sequence_lengths,
                                int64_t total_sequence_length, const rope_tensor* cos_cache,
                                const rope_tensor* sin_cache, const rope_tensor* q_out,
                                const rope_tensor* q_weight, const rope_tensor* k_weight,
                                float epsilon, int64_t interleaved, int64_t num_heads,
                                int64_t kv_num_heads, Plan* out);

struct TablePlan {
    const float* inv_freq;
    void* cos;
    void* sin;
    int32_t dtype;
    int64_t rows, half;
    float scaling;
};

int plan_inv_freq(const rope_tensor* inv_freq, double base, float** out,
                  int64_t* half);
int plan_cos_sin_cache(const rope_tensor* inv_freq, float scaling,
                       const rope_tensor* cos_out, const rope_tensor* sin_out,
                       TablePlan* out);

// Stream of each M-RoPE slot (0 t, 1 h, 2 w) for layout 0 or 1; the caller
// has checked that the sections are non-negative and sum to `half`.
void mrope_streams(int64_t half, const int64_t section[3], int64_t layout,
                   uint8_t* stream_of_slot);

// Error reporting: sets the thread's message and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();
const char* last_error();

int kernel_policy();
int set_kernel_policy(int policy);

}  // namespace rope
