// rope_plan.cpp -- contracts of the ops and the choice of kernel, host only.
//
// Contract clauses follow the pages:
//   RotaryEmbedding: "ai.onnx.RotaryEmbedding" manifest, `derive`
//     (rank3Contract, rank4Contract, rank3PosContract, rank4PosContract),
//     `attributeConstraints`, `typeConstraints`.
//   MRotaryEmbedding: its README, Inputs and Attributes tables.
//   Q+K: onnxruntime PR #27590 (GQA, shared cos/sin) and the SparseAttention
//     README Attributes (kv_num_heads divides num_heads).
// Every failing clause returns its status and records a message.
#include "rope_plan.hpp"

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

namespace rope {

// ---------------------------------------------------------------------------
// errors

static thread_local char g_error[512];

int fail(int code, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_error, sizeof(g_error), fmt, ap);
    va_end(ap);
    return code;
}

void clear_error() { g_error[0] = '\0'; }
const char* last_error() { return g_error; }

// process-wide; atomic so that concurrent calls see one value or the other
static std::atomic<int> g_policy{0};
int kernel_policy() { return g_policy.load(std::memory_order_relaxed); }
int set_kernel_policy(int policy) { return g_policy.exchange(policy, std::memory_order_relaxed); }

// ---------------------------------------------------------------------------
// tensor descriptors

static int elem_size(int32_t dtype) {
    switch (dtype) {
        case ROPE_FLOAT: return 4;
        case ROPE_FLOAT16: return 2;
        case ROPE_BFLOAT16: return 2;
        case ROPE_INT32: return 4;
        case ROPE_INT64: return 8;
        default: return 0;
    }
}

static bool is_float(int32_t dtype) {
    return dtype == ROPE_FLOAT || dtype == ROPE_FLOAT16 || dtype == ROPE_BFLOAT16;
}

static int64_t numel(const rope_tensor* t) {
    int64_t n = 1;
    for (int i = 0; i < t->rank; ++i) n *= t->shape[i];
    return n;
}

static int64_t nbytes(const rope_tensor* t) { return numel(t) * elem_size(t->dtype); }

// Rank in [1,4], dims >= 0, element and byte counts fit in int64, known
// element type, data present when there is data.
static int check_desc(const rope_tensor* t, const char* name) {
    if (t->rank < 1 || t->rank > 4)
        return fail(ROPE_ERR_RANK, "%s: rank %d outside 1..4", name, (int)t->rank);
    if (elem_size(t->dtype) == 0)
        return fail(ROPE_ERR_DTYPE, "%s: unknown element type %d", name, (int)t->dtype);
    int64_t n = 1;
    for (int i = 0; i < t->rank; ++i) {
        if (t->shape[i] < 0)
            return fail(ROPE_ERR_SHAPE, "%s: dimension %d is negative", name, i);
        if (__builtin_mul_overflow(n, t->shape[i], &n))
            return fail(ROPE_ERR_SHAPE, "%s: element count overflows", name);
    }
    int64_t b;
    if (__builtin_mul_overflow(n, (int64_t)elem_size(t->dtype), &b))
        return fail(ROPE_ERR_SHAPE, "%s: byte count overflows", name);
    if (n > 0 && t->data == nullptr)
        return fail(ROPE_ERR_NULL, "%s: data is NULL", name);
    return ROPE_OK;
}

static bool same_shape(const rope_tensor* a, const rope_tensor* b) {
    if (a->rank != b->rank) return false;
    for (int i = 0; i < a->rank; ++i)
        if (a->shape[i] != b->shape[i]) return false;
    return true;
}

static bool overlaps(const rope_tensor* a, const rope_tensor* b) {
    if (!a || !b) return false;
    int64_t na = nbytes(a), nb = nbytes(b);
    if (na == 0 || nb == 0) return false;
    uintptr_t a0 = (uintptr_t)a->data, b0 = (uintptr_t)b->data;
    return a0 < b0 + (uintptr_t)nb && b0 < a0 + (uintptr_t)na;
}

// Output `out` may be exactly `in` (same address, same size); no other overlap.
static bool in_place(const rope_tensor* out, const rope_tensor* in) {
    return in && out->data == in->data && nbytes(out) == nbytes(in);
}

static int check_output(const rope_tensor* out, const char* oname,
                        const rope_tensor* same_ok, const rope_tensor* const* others,
                        const char* const* onames, int nothers) {
    if (overlaps(out, same_ok) && !in_place(out, same_ok))
        return fail(ROPE_ERR_ALIAS, "%s partially overlaps its input", oname);
    for (int i = 0; i < nothers; ++i)
        if (overlaps(out, others[i]))
            return fail(ROPE_ERR_ALIAS, "%s overlaps %s", oname, onames[i]);
    return ROPE_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// ---------------------------------------------------------------------------
// M-RoPE slot streams ([MRE] Attributes: mrope_section, mrope_layout)

void mrope_streams(int64_t half, const int64_t section[3], int64_t layout,
                   uint8_t* stream_of_slot) {
    if (layout == 0) {
        for (int64_t i = 0; i < half; ++i)
            stream_of_slot[i] = i < section[0] ? 0 : (i < section[0] + section[1] ? 1 : 2);
        return;
    }
    // Rounds: in round r every stream whose section exceeds r takes one slot,
    // in the order temporal, height, width.
    int64_t i = 0;
    for (int64_t r = 0; i < half; ++r)
        for (int k = 0; k < 3 && i < half; ++k)
            if (section[k] > r) stream_of_slot[i++] = (uint8_t)k;
}

// ---------------------------------------------------------------------------
// kernel choice

static const char* variant_name(bool vec, CoefKind c, bool norm) {
    static const char* names[2][5] = {
        {"scalar/gather", "scalar/per_token", "scalar/mrope", "scalar/on_the_fly", "scalar/append"},
        {"vec16/gather", "vec16/per_token", "vec16/mrope", "vec16/on_the_fly", "vec16/append"}};
    static const char* norm_names[2][5] = {
        {"scalar/norm/gather", "scalar/norm/per_token", "", "scalar/norm/on_the_fly", "scalar/norm/append"},
        {"vec16/norm/gather", "vec16/norm/per_token", "", "vec16/norm/on_the_fly", "vec16/norm/append"}};
    return (norm ? norm_names : names)[vec ? 1 : 0][(int)c];
}

static const char* row_variant_name(CoefKind c, bool norm) {
    static const char* names[5] = {"row16/gather", "row16/per_token", "row16/mrope", "row16/on_the_fly", "row16/append"};
    static const char* norm_names[5] = {"row16/norm/gather", "row16/norm/per_token", "", "row16/norm/on_the_fly",
                                        "row16/norm/append"};
    return (norm ? norm_names : names)[(int)c];
}

static int env_int(const char* name) {
    const char* e = getenv(name);
    return e ? atoi(e) : 0;
}

// Tuning overrides for measurement sweeps, read once per process (getenv
// scans the environment: too slow for every call).
struct TuningOverrides {
    int heads_per_wave, items_per_lane, head_batch, wave_tile, no_share, row_loads, task_order;
};
static const TuningOverrides& overrides() {
    static const TuningOverrides o = {env_int("ROPE_HEADS_PER_WAVE"), env_int("ROPE_ITEMS_PER_LANE"),
                                      env_int("ROPE_HEAD_BATCH"),     env_int("ROPE_WAVE_TILE"),
                                      env_int("ROPE_NO_SHARE"),
                                      env_int("ROPE_ROW_LOADS"),      env_int("ROPE_TASK_ORDER")};
    return o;
}

static bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// Row kernel (rope_device.hpp): lanes along the head rows of one token, for
// head rows of 32 bytes to 1 KiB (rows of other than a power-of-two size, or
// split-half partners other than a power of two of lanes apart, in its
// general instances: not QK-norm, not M-RoPE), coefficients gathered, per
// token, M-RoPE-assembled, on the fly or at the cache-append position. Used
// for launches that read at
// most kRowMaxBytes of activations (decode steps): there its short per-wave
// dependence chain (one wave-uniform position, at most kRowLoads loads per
// lane) makes the launch 0.5-0.7 us shorter than the vector kernel's
// (fp16, 32 heads of 128: 2.7 vs 3.4 us at 64 tokens, 3.2 vs 3.7 at 256);
// for large launches of heads of 128 with full split-half rotations the
// vector kernel streams faster (22.8 vs 23.9 us at 8192 tokens), both
// measured on MI355X.
// A wave takes up to kRowLoads instructions of one token; smaller launches
// take fewer per wave so that they spread over the chip.
// Between 4 and 8 MiB (fp16, heads of 128, µs row / vector kernel): Q+K of
// 512 tokens (5 MiB) 3.64 / 3.99 with a table and 3.99 / 5.16 on the fly,
// QK-norm on the fly 4.63 / 5.65; 1536 tokens of 4 heads (6 MiB) 3.72 /
// 3.95; 4 x 192 tokens of 32 heads (6 MiB) 3.70 / 3.93; Q+K of 768 tokens
// (7.5 MiB) 4.32 / 4.37; at 8 MiB 4.78 / 4.32 (4 heads) and 4.39 / 4.27 (32
// heads). M-RoPE (rank 4, 28 heads) turns earlier: 4.37 / 4.53 at 3.5 MiB,
// 5.04 / 4.67 at 5.25 MiB.
// Larger launches take the row kernel too where the vector kernel's items
// fit the rows poorly, for head rows making at least 1 KiB a token, not
// M-RoPE: 2-byte types with a token's head rows adjacent (rank 3) and rows
// not a power of two in size (or partners not a power of two of lanes
// apart), interleaved pairs, split halves shorter than 128 bytes, two tasks
// (Q+K) or the cache append; with head rows apart (rank 4), rows of a
// power-of-two size with interleaved pairs or split halves shorter than 128
// bytes; float32 rank 3 with rows of other sizes, a partial rotation of
// split halves or coefficients on the fly; QK-norm rank 3 in float32 or with
// 2-byte split halves of other than 128 bytes.
// Measured on MI355X (fp16, 8192 tokens, µs row / vector kernel, the vector
// kernel in its best geometry of 2, 4 or 8 heads per wave): heads of 64, 64
// heads 23.9 / 27.4; rotary_embedding_dim 64 of 128 24.0 / 27.2, 32 of 128
// 23.8 / 31.7; interleaved pairs 22.5 / 23.4, heads of 64 22.5 / 25.3, of
// 256 22.5 / 27.4; Q+K with a table 29.4 / 29.9, on the fly 29.7 / 32.0; a 4
// x 2048-token prompt with the cache append 34.2 / 35.4; at 2048 tokens
// heads of 64 6.66 / 7.19, rotary_embedding_dim 64 6.65 / 8.91, interleaved
// 6.48 / 7.04; rows of 160 bytes (rotary_embedding_dim 32) 16.5 / 31.4,
// of 192 bytes 19.1 / 24.7, interleaved 19.0 / 20.1, of 384 bytes 18.5 /
// 20.1 (16 heads), of 224, 320, 640 and 768 bytes (heads of 112, 160,
// 320 and 384; the one of 640 bytes leaves 24 lanes idle) 21.2 / 33.0,
// 16.6 / 23.0, 16.5 / 17.3, 18.6 / 21.7; rank 4 (8 x 32 heads x 1024 tokens): heads of 128
// interleaved 22.8 / 24.3, heads of 64 13.8 / 17.1 (interleaved 11.5 /
// 14.1), rotary_embedding_dim 64 of 128 24.6 / 31.2, but rows of 192 bytes
// (rotary_embedding_dim 64, interleaved) 21.2 / 18.3; float32: heads of 96
// 35.3 / 36.4 (rotary_embedding_dim 64 interleaved 34.7 / 36.8), of 80 with
// rotary_embedding_dim 32 31.2 / 34.9, rotary_embedding_dim 64 of 128 46.1 /
// 52.6 (at 2048 tokens 12.5 / 15.9), 32 of 64 46.4 / 48.8, Q+K on the fly
// 54.5 / 58.6 (with the table 54.3 / 54.9: kept); QK-norm with
// heads of 256 58.0 / 63.2 (bf16 58.2 / 63.8), with heads of 64 17.8 / 18.5
// (8 or 2 heads per batch; 4: 21.2), in float32 57.1 / 58.2 (heads of 64:
// 29.3 / 30.0). The vector kernel stays faster for split halves of 128 bytes
// or more in one task (32 heads of 128: 22.8 / 23.9; 16 heads 11.6 / 13.3;
// 32 heads of 256: 44.8 / 46.5), float32 heads of 128 (44.2 / 46.5), M-RoPE (20.7 /
// 24.5), packed [Q|K|V] (38.6 / 40.0), 2-byte QK-norm with heads of 128
// (30.1 / 30.6), float32 rows of 256 or 512 bytes with full or interleaved
// rotations (heads of 64 45.2 / 46.0, of 256 46.1 / 46.5, rotary_embedding_dim 64 of
// 128 interleaved 46.5 / 47.5), float32 packed [Q|K|V] (69.2 / 67.5) and
// the float32 prompt with the cache append (66.3 / 65.2).
static constexpr int64_t kRowMaxBytes = 6 << 20;
static constexpr int64_t kRowMaxBytesMrope = 4 << 20;

static bool row_kernel_fits_better(const Problem& p, int es, bool general) {
    if (p.coef == kCoefMrope) return false;
    bool adjacent = true;
    for (int t = 0; t < p.ntask; ++t) {
        if (p.task[t].heads > 1 && p.task[t].stride_h != p.D) adjacent = false;  // rank 4
        // a token's rows fill at least one 1 KiB instruction of a wave
        if (p.task[t].heads > 0 && p.task[t].heads * p.D * es < 1024) return false;
    }
    const int64_t half_bytes = (p.R / 2) * es;
    // QK-norm (rows of a power-of-two size): float32 data, or 2-byte split
    // halves other than 128 bytes long
    if (p.norm) return adjacent && (es == 4 || (!p.interleaved && half_bytes != 128));
    // float32: rows of other sizes, a partial rotation of split halves, or
    // coefficients on the fly
    if (es == 4) return adjacent && (general || (!p.interleaved && p.R < p.D) || p.coef == kCoefOnTheFly);
    // head rows apart (rank 4): rows of a power-of-two size only
    if (!adjacent) return !general && (p.interleaved || half_bytes < 128);
    return general || p.interleaved || half_bytes < 128 || p.ntask == 2 || p.coef == kCoefAppend;
}

// vec_can: the vector kernel could take the launch (else the row kernel takes
// it at any size when its rules allow, before the scalar kernel); elementwise:
// pairs that do not fall on 16-byte chunks (the element-wise instances)
static bool choose_row_geometry(Plan* pl, bool vec_can, bool elementwise = false) {
    Problem& p = pl->p;
    Geometry& g = pl->g;
    const int policy = kernel_policy();
    if (policy == 2) return false;
    if ((p.coef == kCoefOnTheFly || elementwise) && p.R / 2 > kRowMaxSlots) return false;
    if (elementwise && (p.norm || p.coef == kCoefMrope)) return false;
    const int es = elem_size(p.dtype);
    const int64_t row_bytes = p.D * es;
    if (row_bytes % 16 != 0 || row_bytes < 32 || row_bytes > 1024) return false;
    const int64_t dl = p.interleaved || elementwise ? 0 : (p.R / 2) * es / 16;
    // rows of other sizes, or partners a number of lanes apart other than a
    // power of two: the kernel's general instances (no M-RoPE)
    const bool general = elementwise || !pow2(row_bytes) || (!p.interleaved && !pow2(dl));
    if (general && p.coef == kCoefMrope) return false;
    int64_t xbytes = 0;
    for (int t = 0; t < p.ntask; ++t) xbytes += p.B * p.S * p.task[t].heads * row_bytes;
    const int64_t max_bytes = p.coef == kCoefMrope ? kRowMaxBytesMrope : kRowMaxBytes;
    if (xbytes > max_bytes && policy != 3 && vec_can && !row_kernel_fits_better(p, es, general)) return false;
    const int RL = (int)(row_bytes / 16);
    const int rpi = 64 / RL;
    const int64_t ntok = p.B * p.S;
    // Fewer loads per wave (more waves) while a launch has fewer than ~4096
    // waves: measured on MI355X in HIP-graph replay (fp16 decode steps, 256
    // tokens, 32 + 8 heads of 128), one instruction per wave against the
    // earlier rule of ~1024 waves: packed [Q|K|V] 3.33 vs 3.75 us, cache
    // append 3.61 vs 4.05, QK-norm on the fly 4.19 vs 4.45, QK-norm + cache
    // append 4.10 vs 4.93; Q+K with a table 3.31 vs 3.29; Q+K on the fly
    // (each wave computes its token's slots) 3.35 vs 3.47 with two
    // instructions per wave.
    const int64_t target_waves = 4096;
    // Q+K past the decode sizes: 4 instructions per wave (fp16, heads of
    // 128, µs with 8 / 4: 2048 tokens 7.96 / 7.51, 8192 tokens 29.4 / 28.5,
    // on the fly 29.7 / 28.6, 16384 tokens 55.4 / 53.7; heads of 64 15.6 /
    // 15.6); one-task launches keep 8 (interleaved heads of 128 22.5 / 24.2)
    // and so does the prompt with the cache append (at 4 x 512 tokens 9.23 /
    // 10.12)
    int loads = p.ntask == 2 && !p.norm && xbytes > max_bytes ? 4 : kRowLoads;
    for (;;) {
        int64_t waves = 0;
        for (int t = 0; t < p.ntask; ++t) {
            const int64_t H = p.task[t].heads;
            const int64_t hpw = std::min<int64_t>(H, (int64_t)loads * rpi);
            waves += H > 0 ? ntok * ((H + hpw - 1) / hpw) : 0;
        }
        if (waves >= target_waves || loads == 1) break;
        loads /= 2;
    }
    const int over_loads = overrides().row_loads;  // tuning override (sweeps)
    if (over_loads == 1 || over_loads == 2 || over_loads == 4 || over_loads == 8) loads = over_loads;
    if (elementwise && loads > kRowElemLoads) loads = kRowElemLoads;
    int64_t total_waves = 0;
    for (int t = 0; t < p.ntask; ++t) {
        const int64_t H = p.task[t].heads;
        const int64_t hpw = H > 0 ? std::min<int64_t>(H, (int64_t)loads * rpi) : 1;
        const int64_t chunks = H > 0 ? (H + hpw - 1) / hpw : 1;
        g.heads_per_wave[t] = (int32_t)hpw;
        g.chunks[t] = (int32_t)chunks;
        g.waves[t] = H > 0 ? ntok * chunks : 0;
        total_waves += g.waves[t];
    }
    // the kernel's index arithmetic is 32-bit
    if (total_waves > INT32_MAX || ntok > INT32_MAX) return false;
    g.row_kernel = 1;
    g.row_general = elementwise ? 2 : (general ? 1 : 0);
    g.row_lanes = RL;
    g.half_lanes = (int32_t)dl;
    g.NP = (int32_t)(p.R * es / 16);  // chunks of the rotated prefix (unused element-wise)
    g.W = RL;
    g.TG = 1;
    g.tile = 1;
    g.items_per_lane = 1;
    g.head_batch = loads;
    g.share_coef = 0;
    return true;
}

// Vector kernel: a head row of D elements is cut into 16-byte items; a
// rotation item holds E = 16/sizeof(T) pairs' first elements (split halves,
// with its partner item R/2 elements later) or E/2 whole pairs
// (interleaved); tail items are copied. A wave owns TG consecutive tokens
// times W items (items_per_lane items per lane) and loops over a chunk of
// heads, keeping each lane's coefficients in registers.
// Vector-kernel launches: heads per wave are halved while the launch then
// stays within this many waves (about one round of resident waves of the
// 16-bit instances).
static constexpr int64_t kVecTargetWaves = 4096;
// M-RoPE keeps 4 heads per wave while that still gives this many waves.
static constexpr int64_t kVecMropeMinWaves = 1536;

static void choose_geometry(Plan* pl) {
    Problem& p = pl->p;
    Geometry& g = pl->g;
    const int es = elem_size(p.dtype);
    const int E = 16 / es;
    const int64_t half = p.R / 2;
    bool ok = kernel_policy() != 1;
    // rows in 16-byte chunks; pairs within chunk boundaries (else only the
    // row kernel's element-wise instances, or the scalar kernel)
    ok = ok && p.D % E == 0;
    const bool pairs_ok = p.R % E == 0 && (p.interleaved || half % E == 0);
    for (int t = 0; t < p.ntask; ++t)
        ok = ok && aligned16(p.task[t].x) && aligned16(p.task[t].y);
    if (p.norm)
        for (int t = 0; t < p.ntask; ++t) ok = ok && aligned16(p.task[t].weight);
    if (p.coef != kCoefOnTheFly)
        ok = ok && aligned16(p.cos) && aligned16(p.sin);
    if (ok && !pairs_ok) {
        g.row_kernel = 0;
        g.row_general = 0;
        g.group_major = 0;
        g.vector = true;
        if (choose_row_geometry(pl, false, true)) {
            g.variant = row_variant_name(p.coef, p.norm != 0);
            return;
        }
        g.vector = false;
        g.variant = variant_name(false, p.coef, p.norm != 0);
        return;
    }
    const int64_t NP = p.interleaved ? p.R / E : half / E;
    const int64_t NT = (p.D - p.R) / E;
    const int64_t W = NP + NT;
    ok = ok && pairs_ok && W >= 1 && W <= 256;
    // QK-norm in the vector kernel: a row's items must sit in one aligned
    // group of W lanes (W a power of two dividing the wave) for the in-wave
    // sum of squares; the row kernel sums any row of up to 64 lanes
    const bool vec_can = !p.norm || (W <= 64 && (W & (W - 1)) == 0);
    g.vector = ok;
    g.variant = variant_name(ok, p.coef, p.norm != 0);
    g.row_kernel = 0;
    g.row_general = 0;
    g.group_major = 0;
    if (!ok) return;
    if (choose_row_geometry(pl, vec_can)) {
        g.variant = row_variant_name(p.coef, p.norm != 0);
        return;
    }
    if (!vec_can) {
        g.vector = false;
        g.variant = variant_name(false, p.coef, p.norm != 0);
        return;
    }

    // Items per lane (ipl) and head batch (hb: heads whose X loads a lane
    // issues together), among the instantiated pairs. Chosen from sweeps on
    // MI355X over all pairs:
    //  * 2-byte types: lanes all busy if some ipl allows it, then the most
    //    16-byte loads in flight per lane up to 16, then the fewer items per
    //    lane (split fp16 rows of 128: (1, 8); interleaved: (2, 8), 24.2 vs
    //    27.1 us for (1, 8); 12 items per row: (3, 4), 19.3 vs 20.8 us);
    //  * 4-byte types: the smallest ipl keeping 3/4 of the lanes busy and at
    //    most 4 heads per batch (fp32 prefill 44.2 vs 51.1 us with 8 heads;
    //    the partial interleaved fp32 case, 24 items per row, 35.9 us with
    //    one item per lane and 4 heads per batch, 36.9 with three items and
    //    2 heads, 38.2 with two and 4, 39.4 with four and 4);
    //  * QK-norm: one item per lane (its only instantiation).
    static const int kPairs[][2] = {{1, 2}, {1, 4}, {1, 8}, {2, 2}, {2, 4}, {2, 8},
                                    {3, 2}, {3, 4}, {4, 2}, {4, 4}};
    const int per_item = p.interleaved ? 1 : 2;
    const double loads_per_item = (double)(NP * per_item + NT) / (double)W;
    const int over_ipl = overrides().items_per_lane;
    const int over_batch = overrides().head_batch;
    int best = 0, hb = 2;
    if (es == 2 && !p.norm) {
        double best_key[4] = {-1, -1, -1, -1};
        for (const auto& pr : kPairs) {
            const int ipl = pr[0], h = pr[1];
            const int64_t tg = 64 * ipl / W;
            if (tg < 1) continue;
            const double util = (double)(tg * W) / (64.0 * ipl);
            const double loads = ipl * h * loads_per_item;
            if (loads > 16.0 + 1e-9) continue;
            const bool full = util >= 0.99;
            const double key[4] = {full ? 1.0 : 0.0, full ? 0.0 : util, loads, -(double)ipl};
            bool better = false;
            for (int k = 0; k < 4; ++k) {
                if (key[k] > best_key[k] + 1e-9) { better = true; break; }
                if (key[k] < best_key[k] - 1e-9) break;
            }
            if (better) {
                for (int k = 0; k < 4; ++k) best_key[k] = key[k];
                best = ipl;
                hb = h;
            }
        }
    } else {
        double best_util = 0.0;
        for (int ipl = 1; ipl <= (p.norm ? 1 : 4); ++ipl) {
            int64_t tg = 64 * ipl / W;
            if (tg < 1) continue;
            double util = (double)(tg * W) / (64.0 * ipl);
            if (util > best_util + 1e-9) {
                best_util = util;
                best = ipl;
            }
            if (util >= 0.75) break;
        }
        const int max_batch = es == 4 ? 4 : 8;
        hb = 2;
        while (hb * 2 <= max_batch && best * hb * 2 * per_item <= 16) hb *= 2;
    }
    // tuning overrides (sweeps): items per lane, then head batch
    if (over_ipl > 0 && over_ipl <= 4 && !p.norm && 64 * over_ipl / W >= 1) best = over_ipl;
    for (int ipl = 1; best == 0 && ipl <= 4; ++ipl)  // nothing chosen: the first that fits
        if (64 * ipl / W >= 1) { best = ipl; hb = 2; }
    const int max_batch = best <= 2 ? 8 : 4;
    if (hb > max_batch) hb = max_batch;
    if (over_batch == 2 || over_batch == 4 || over_batch == 8)
        hb = over_batch <= max_batch ? over_batch : max_batch;
    g.items_per_lane = best;
    g.W = (int32_t)W;
    g.NP = (int32_t)NP;
    g.TG = (int32_t)(64 * best / W);
    const int64_t ntok = p.B * p.S;
    const int64_t groups = (ntok + g.TG - 1) / g.TG;
    const int over = overrides().heads_per_wave;
    g.head_batch = hb;
    // Heads per wave: one batch, split evenly over the head count (28 heads
    // with batch 8 -> 4 waves of 7); halved while the launch then keeps
    // within kVecTargetWaves waves, so that smaller launches still fill the
    // chip, down to 2 heads per wave (4 for M-RoPE, whose per-wave
    // coefficient assembly would otherwise serve too few heads, unless that
    // leaves fewer than kVecMropeMinWaves waves: 2 x 28 heads x 768 tokens
    // 5.85 us with 2688 waves of 2, 6.05 with 1344 of 4; x 384 tokens 4.46
    // with 1344 of 2, 4.69 with 672 of 4; x 1024 tokens 7.78 with 3584 of 2,
    // 6.50 with 1792 of 4); the batch
    // then no wider than a wave's heads. Measured on MI355X (fp16, heads of
    // 128): 8192 tokens of 16 heads 12.1 us with 2048 waves of 8 heads, 11.7
    // with 4096 of 4, 13.1 with 8192 of 2; 8192 tokens of 4 heads (one GPU's
    // share of an 8-way head split) 4.75 us with 1024 waves of 4 heads, 4.32
    // with 2048 of 2; M-RoPE with 28 heads and 4096 tokens 12.2 us with 2048
    // waves of 7 heads, 11.2 with 3584 of 4, 13.8 with 7168 of 2; c2 and c4
    // (4096 waves) lose 14-16% with 4 heads per wave.
    // Interleaved binary32 data runs two batches per wave, the second one's
    // loads in flight while the first stores (fp32 partial interleaved
    // prefill 36.2 -> 35.7 us); its head loop is unrolled over at most
    // kVecMaxHeads heads.
    const bool pipelined = es == 4 && p.interleaved && !p.norm;
    int64_t hpw_cap = pipelined ? 2 * hb : hb;
    auto waves_at = [&](int64_t cap) {
        int64_t w = 0;
        for (int t = 0; t < p.ntask; ++t) w += groups * ((p.task[t].heads + cap - 1) / cap);
        return w;
    };
    // Launches whose full-batch waves need more than one round (one or two
    // items per lane, not the pipelined binary32 instances): many small
    // waves, batches of 2, which measured faster (fp16, µs, batch 8 / 2):
    // 8192 tokens of 40 heads 33.2 / 29.7,
    // of 36 heads 30.7 / 26.8, of 64 heads 50.8 / 45.7; 16384 tokens of 32
    // heads 49.9 / 45.5; Q+K of 8192 tokens 33.4 / 30.0, of 16384 62.9 /
    // 56.5; a 4 x 2048-token prompt with cache append 40.2 / 35.2; M-RoPE of
    // 2 x 28 heads x 8192 tokens 43.3 / 41.5; packed [Q|K|V] of 8192 tokens
    // 41.9 / 40.4; interleaved pairs (two items per lane), 16384 tokens of 32
    // heads 53.0 / 48.0; fp32 (batch 4 / 2) 8192 tokens of 32 heads 45.0 /
    // 44.0, 16384 tokens 86.4 / 83.9. Launches of one round keep their batch
    // (c2 23.0 / 24.5, c4 20.6 / 23.4, interleaved c2 23.5 / 25.8); QK-norm
    // (29.7 / 33.8) and coefficients on the fly (32.1 / 32.4) keep it too.
    // 2-byte split halves longer than 128 bytes take batches of 2 at any
    // size (heads of 256, 16 heads, 8192 tokens: 27.4 us in one round of 8
    // heads per wave, 25.5 with 4, 24.2 with 2).
    const bool wide_halves = es == 2 && !p.interleaved && p.coef != kCoefMrope && half * es > 128;
    const bool many_small = !p.norm && p.coef != kCoefOnTheFly && best <= 2 && !pipelined &&
                            over <= 0 && over_batch == 0 && hb > 2 &&
                            (waves_at(hpw_cap) > kVecTargetWaves || wide_halves);
    if (many_small) g.head_batch = hb = hpw_cap = 2;
    const int64_t min_hpw = p.coef == kCoefMrope && waves_at(4) >= kVecMropeMinWaves ? 4 : 2;
    while (hpw_cap / 2 >= min_hpw && waves_at(hpw_cap / 2) <= kVecTargetWaves) hpw_cap /= 2;
    if (!pipelined && over <= 0 && over_batch == 0 && hb > hpw_cap) g.head_batch = hb = (int)hpw_cap;
    if (over > 0) hpw_cap = over;  // tuning override (a wave loops over its batches)
    if (pipelined && hpw_cap > kVecMaxHeads) hpw_cap = kVecMaxHeads;
    // Wave order: rank 4 keeps a head's tokens contiguous, so a tile of
    // token groups per head chunk gives each workgroup longer runs per head:
    // 2 groups for 2-byte types, 4 for 4-byte ones (measured on MI355X: the
    // fp16 M-RoPE prefill 21.7 us with 2, 22.1 with 4, 22.6 with 3; the fp32
    // partial interleaved case 35.9 us with 4, 36.3 with 8).
    const int over_tile = overrides().wave_tile;
    g.tile = over_tile > 0 ? over_tile : (g.rank == 4 ? (es == 2 ? 2 : 4) : 1);
    const int64_t tiles = (groups + g.tile - 1) / g.tile;
    for (int t = 0; t < p.ntask; ++t) {
        const int64_t H = p.task[t].heads;
        int64_t chunks = H > 0 ? (H + hpw_cap - 1) / hpw_cap : 1;
        int64_t hpw = H > 0 ? (H + chunks - 1) / chunks : 1;
        g.heads_per_wave[t] = (int32_t)hpw;
        g.chunks[t] = (int32_t)chunks;
        g.waves[t] = H > 0 ? tiles * g.tile * chunks : 0;
    }
    // On the fly, every head chunk of a token group computes the same
    // coefficients. When each workgroup's waves are chunks of one token group
    // of one task (a tile of one group, chunk counts divisible by the waves
    // per workgroup), they split that work and exchange it through LDS.
    // the kernel's index arithmetic is 32-bit: larger launches take the
    // scalar kernel
    int64_t total_waves = 0;
    for (int t = 0; t < p.ntask; ++t) total_waves += g.waves[t];
    if (total_waves > INT32_MAX || ntok > INT32_MAX) {
        g.vector = false;
        g.variant = variant_name(false, p.coef, p.norm != 0);
        return;
    }
    g.share_coef = 0;
    if (p.coef == kCoefOnTheFly && g.tile == 1 && overrides().no_share == 0) {
        bool ok_share = true;
        for (int t = 0; t < p.ntask; ++t)
            if (p.task[t].heads > 0 && g.chunks[t] % kWavesPerBlock != 0) ok_share = false;
        g.share_coef = ok_share ? 1 : 0;
    }
    // Three tasks read from one packed rank-3 tensor ([Q|K|V] in each token's
    // row: the packed op, or the cache append's packed query), in a launch of
    // more than one round of waves: waves in token-group order, so that the
    // three tasks' chunks of one token group run together and a token's row
    // is read in one visit instead of its Q part in the first waves and its
    // K and V parts in the last. Measured on MI355X (fp16, µs, token-group /
    // task order): packed [Q|K|V] of 8192 tokens 38.3 / 40.8 (on the fly
    // 38.4 / 40.8), of 2048 tokens (one round) 9.63 / 9.36; with separate Q,
    // K and V tensors the task order is faster (the cache append of a 4 x
    // 2048-token prompt 36.3 / 35.3, its QK-norm form 40.3 / 38.3). With
    // coefficients shared through LDS every chunk count is a multiple of the
    // waves per workgroup, so a workgroup still holds chunks of one task and
    // one token group.
    g.group_major = 0;
    const int order = overrides().task_order;  // 1: token-group order, 2: task order (sweeps)
    if (p.ntask == 3 && g.tile == 1 && order != 2) {
        const uintptr_t x0 = (uintptr_t)p.task[0].x;
        const uintptr_t row = (uintptr_t)(p.task[0].stride_s * es);  // bytes of a token's row
        bool packed = true, ok_order = true;
        for (int t = 0; t < p.ntask; ++t) {
            const uintptr_t xt = (uintptr_t)p.task[t].x;
            packed = packed && p.task[t].stride_s == p.task[0].stride_s &&
                     p.task[t].stride_b == p.task[0].stride_b && xt >= x0 && xt - x0 < row;
            if (p.task[t].heads <= 0 || g.waves[t] != groups * g.chunks[t]) ok_order = false;
        }
        g.group_major = ok_order && (order == 1 || (packed && total_waves > kVecTargetWaves)) ? 1 : 0;
    }
}

// The kernels take the head size and head counts as 32-bit values (every
// other size is 64-bit): larger ones are refused before anything launches.
// Then the kernel choice.
static int finish_plan(Plan* pl) {
    const Problem& p = pl->p;
    if (p.D > INT32_MAX)
        return fail(ROPE_ERR_UNSUPPORTED, "head_size %lld exceeds 2^31 - 1", (long long)p.D);
    for (int t = 0; t < p.ntask; ++t)
        if (p.task[t].heads > INT32_MAX)
            return fail(ROPE_ERR_UNSUPPORTED, "head count %lld exceeds 2^31 - 1", (long long)p.task[t].heads);
    choose_geometry(pl);
    return ROPE_OK;
}

static void fill_strides(Task* t, int rank, int64_t S, int64_t H, int64_t D) {
    t->heads = H;
    if (rank == 4) {
        t->stride_b = H * S * D;
        t->stride_h = S * D;
        t->stride_s = D;
    } else {
        t->stride_b = S * H * D;
        t->stride_s = H * D;
        t->stride_h = D;
    }
    t->ystride_b = t->stride_b;
    t->ystride_h = t->stride_h;
    t->ystride_s = t->stride_s;
}

// (B, S, H, D) of a rank-3 or rank-4 activation.
static int activation_dims(const rope_tensor* x, const char* name, int64_t heads_attr,
                           bool heads_required, int64_t* B, int64_t* S, int64_t* H,
                           int64_t* D) {
    if (x->rank == 3) {
        if (heads_attr < 1)
            return fail(ROPE_ERR_ATTRIBUTE, "%s: the head count attribute is required (>= 1) for rank 3",
                        name);
        if (x->shape[2] % heads_attr != 0)
            return fail(ROPE_ERR_SHAPE, "%s: hidden size %lld is not divisible by %lld heads", name,
                        (long long)x->shape[2], (long long)heads_attr);
        *B = x->shape[0];
        *S = x->shape[1];
        *H = heads_attr;
        *D = x->shape[2] / heads_attr;
        return ROPE_OK;
    }
    if (x->rank == 4) {
        if (heads_required && heads_attr < 1)
            return fail(ROPE_ERR_ATTRIBUTE, "%s: num_heads must be positive here", name);
        if (heads_attr != 0 && heads_attr != x->shape[1])
            return fail(ROPE_ERR_SHAPE, "%s: head count attribute %lld disagrees with dim 1 = %lld",
                        name, (long long)heads_attr, (long long)x->shape[1]);
        *B = x->shape[0];
        *H = x->shape[1];
        *S = x->shape[2];
        *D = x->shape[3];
        return ROPE_OK;
    }
    return fail(ROPE_ERR_RANK, "%s must be rank 3 or 4, got %d", name, (int)x->rank);
}

// Head counts of the packed layouts (num_heads + 2 * kv_num_heads heads per
// token, kv_num_heads dividing num_heads): bounded so that the sum fits.
static int check_head_count(int64_t num_heads) {
    if (num_heads > INT32_MAX)
        return fail(ROPE_ERR_ATTRIBUTE, "num_heads %lld exceeds 2^31 - 1", (long long)num_heads);
    return ROPE_OK;
}

#define TRY(expr)                          \
    do {                                   \
        int rc_ = (expr);                  \
        if (rc_ != ROPE_OK) return rc_;    \
    } while (0)

// cos/sin tables of a gathered (ids) or per-token (no ids) RotaryEmbedding:
// manifest derive rank*PosContract / rank*Contract.
static int check_tables(const rope_tensor* cos, const rope_tensor* sin, const rope_tensor* ids,
                        int64_t B, int64_t S, int64_t R, int64_t* M) {
    if (!same_shape(cos, sin))
        return fail(ROPE_ERR_SHAPE, "sin_cache must have the shape of cos_cache");
    if (ids) {
        if (cos->rank != 2)
            return fail(ROPE_ERR_RANK, "cos_cache must be rank 2 (max_sequence_length, rotary_dim/2) with position_ids");
        if (cos->shape[1] != R / 2)
            return fail(ROPE_ERR_SHAPE, "cos_cache width %lld * 2 != rotary dim %lld",
                        (long long)cos->shape[1], (long long)R);
        if (ids->rank != 2)
            return fail(ROPE_ERR_RANK, "position_ids must be rank 2 (batch, sequence)");
        if (ids->shape[0] != B || ids->shape[1] != S)
            return fail(ROPE_ERR_SHAPE, "position_ids shape (%lld, %lld) != (batch %lld, sequence %lld)",
                        (long long)ids->shape[0], (long long)ids->shape[1], (long long)B, (long long)S);
        *M = cos->shape[0];
        return ROPE_OK;
    }
    if (cos->rank != 3)
        return fail(ROPE_ERR_RANK, "cos_cache must be rank 3 (batch, sequence, rotary_dim/2) without position_ids");
    if (cos->shape[0] != B || cos->shape[1] != S)
        return fail(ROPE_ERR_SHAPE, "cos_cache leading dims (%lld, %lld) != (batch %lld, sequence %lld)",
                    (long long)cos->shape[0], (long long)cos->shape[1], (long long)B, (long long)S);
    if (cos->shape[2] != R / 2)
        return fail(ROPE_ERR_SHAPE, "cos_cache width %lld * 2 != rotary dim %lld",
                    (long long)cos->shape[2], (long long)R);
    *M = 0;
    return ROPE_OK;
}

static int check_rotary_dim(int64_t D, int64_t rotary_embedding_dim, int64_t* R) {
    if (rotary_embedding_dim < 0)
        return fail(ROPE_ERR_ATTRIBUTE, "rotary_embedding_dim must be >= 0");
    if (rotary_embedding_dim % 2 != 0)
        return fail(ROPE_ERR_ATTRIBUTE, "rotary_embedding_dim must be even");
    if (rotary_embedding_dim > D)
        return fail(ROPE_ERR_SHAPE, "rotary_embedding_dim %lld exceeds head_size %lld",
                    (long long)rotary_embedding_dim, (long long)D);
    *R = rotary_embedding_dim ? rotary_embedding_dim : D;
    return ROPE_OK;
}

// ---------------------------------------------------------------------------

int plan_rope(const rope_tensor* x, const rope_tensor* cos_cache, const rope_tensor* sin_cache,
              const rope_tensor* position_ids, const rope_tensor* y, int64_t interleaved,
              int64_t num_heads, int64_t rotary_embedding_dim, Plan* out) {
    clear_error();
    memset(out, 0, sizeof(*out));
    if (!x) return fail(ROPE_ERR_NULL, "x is missing");
    if (!cos_cache) return fail(ROPE_ERR_NULL, "cos_cache is missing");
    if (!sin_cache) return fail(ROPE_ERR_NULL, "sin_cache is missing");
    if (!y) return fail(ROPE_ERR_NULL, "y is missing");
    TRY(check_desc(x, "x"));
    TRY(check_desc(cos_cache, "cos_cache"));
    TRY(check_desc(sin_cache, "sin_cache"));
    TRY(check_desc(y, "y"));
    if (position_ids) TRY(check_desc(position_ids, "position_ids"));

    if (!is_float(x->dtype))
        return fail(ROPE_ERR_DTYPE, "x must be float32, float16 or bfloat16");
    if (cos_cache->dtype != x->dtype || sin_cache->dtype != x->dtype || y->dtype != x->dtype)
        return fail(ROPE_ERR_DTYPE, "cos_cache, sin_cache and y must have the type of x");
    if (position_ids && position_ids->dtype != ROPE_INT64)
        return fail(ROPE_ERR_DTYPE, "position_ids must be int64");
    if (interleaved != 0 && interleaved != 1)
        return fail(ROPE_ERR_ATTRIBUTE, "interleaved must be 0 or 1");
    if (num_heads < 0) return fail(ROPE_ERR_ATTRIBUTE, "num_heads must be >= 0");

    if (x->rank != 3 && x->rank != 4)
        return fail(ROPE_ERR_RANK, "x must be rank 3 or 4, got %d", (int)x->rank);
    if (!same_shape(x, y)) return fail(ROPE_ERR_SHAPE, "y must have the shape of x");
    int64_t B, S, H, D, R, M;
    TRY(activation_dims(x, "x", num_heads, false, &B, &S, &H, &D));
    if (D % 2 != 0) return fail(ROPE_ERR_SHAPE, "head_size %lld must be even", (long long)D);
    TRY(check_rotary_dim(D, rotary_embedding_dim, &R));
    TRY(check_tables(cos_cache, sin_cache, position_ids, B, S, R, &M));

    const rope_tensor* others[3] = {cos_cache, sin_cache, position_ids};
    const char* names[3] = {"cos_cache", "sin_cache", "position_ids"};
    TRY(check_output(y, "y", x, others, names, 3));

    Problem& p = out->p;
    p.dtype = x->dtype;
    p.interleaved = (int32_t)interleaved;
    p.B = B; p.S = S; p.D = D; p.R = R;
    p.ntask = 1;
    p.task[0].x = x->data;
    p.task[0].y = y->data;
    fill_strides(&p.task[0], x->rank, S, H, D);
    p.coef = position_ids ? kCoefGather : kCoefPerToken;
    p.cos = cos_cache->data;
    p.sin = sin_cache->data;
    p.ids = position_ids ? (const int64_t*)position_ids->data : nullptr;
    p.M = M;
    p.scale = 1.0f;
    p.scaling = 1.0f;
    out->empty = numel(x) == 0;
    out->g.rank = x->rank;
    return finish_plan(out);
}

int plan_mrope(const rope_tensor* x, const rope_tensor* position_ids, const rope_tensor* cos_cache,
               const rope_tensor* sin_cache, const rope_tensor* y, int64_t interleaved,
               int64_t is_packed_batching, int64_t mrope_layout, const int64_t mrope_section[3],
               int64_t num_heads, int64_t rotary_embedding_dim, float scale, Plan* out) {
    clear_error();
    memset(out, 0, sizeof(*out));
    if (!x) return fail(ROPE_ERR_NULL, "x is missing");
    if (!position_ids) return fail(ROPE_ERR_NULL, "position_ids is required");
    if (!cos_cache) return fail(ROPE_ERR_NULL, "cos_cache is missing");
    if (!sin_cache) return fail(ROPE_ERR_NULL, "sin_cache is missing");
    if (!y) return fail(ROPE_ERR_NULL, "y is missing");
    if (!mrope_section) return fail(ROPE_ERR_NULL, "mrope_section is required");
    TRY(check_desc(x, "x"));
    TRY(check_desc(position_ids, "position_ids"));
    TRY(check_desc(cos_cache, "cos_cache"));
    TRY(check_desc(sin_cache, "sin_cache"));
    TRY(check_desc(y, "y"));

    if (!is_float(x->dtype))
        return fail(ROPE_ERR_DTYPE, "x must be float32, float16 or bfloat16");
    if (cos_cache->dtype != x->dtype || sin_cache->dtype != x->dtype || y->dtype != x->dtype)
        return fail(ROPE_ERR_DTYPE, "cos_cache, sin_cache and y must have the type of x");
    if (position_ids->dtype != ROPE_INT64)
        return fail(ROPE_ERR_DTYPE, "position_ids must be int64");
    if (is_packed_batching != 0 && is_packed_batching != 1)
        return fail(ROPE_ERR_ATTRIBUTE, "is_packed_batching must be 0 or 1");
    if (is_packed_batching == 1)
        return fail(ROPE_ERR_UNSUPPORTED, "packed batching (is_packed_batching=1) is not implemented");
    if (mrope_layout != 0 && mrope_layout != 1)
        return fail(ROPE_ERR_ATTRIBUTE, "mrope_layout must be 0 or 1");
    if (interleaved != 0 && interleaved != 1)
        return fail(ROPE_ERR_ATTRIBUTE, "interleaved must be 0 or 1");
    for (int k = 0; k < 3; ++k)
        if (mrope_section[k] < 0)
            return fail(ROPE_ERR_ATTRIBUTE, "mrope_section entries must be non-negative");
    if (num_heads < 0) return fail(ROPE_ERR_ATTRIBUTE, "num_heads must be >= 0");
    if (rotary_embedding_dim < 0 || rotary_embedding_dim % 2 != 0)
        return fail(ROPE_ERR_ATTRIBUTE, "rotary_embedding_dim must be 0 or a positive even number");

    if (x->rank != 3 && x->rank != 4)
        return fail(ROPE_ERR_RANK, "x must be rank 3 or 4, got %d", (int)x->rank);
    if (!same_shape(x, y)) return fail(ROPE_ERR_SHAPE, "y must have the shape of x");
    int64_t B, S, H, D, R;
    TRY(activation_dims(x, "x", num_heads, rotary_embedding_dim != 0, &B, &S, &H, &D));
    if (rotary_embedding_dim == 0) {
        if (D % 2 != 0)
            return fail(ROPE_ERR_SHAPE, "head_size %lld must be even when rotary_embedding_dim is 0",
                        (long long)D);
        R = D;
    } else {
        if (rotary_embedding_dim > D)
            return fail(ROPE_ERR_SHAPE, "rotary_embedding_dim %lld exceeds head_size %lld",
                        (long long)rotary_embedding_dim, (long long)D);
        R = rotary_embedding_dim;
    }
    const int64_t half = R / 2;
    if (half > kMaxMropeHalf)
        return fail(ROPE_ERR_UNSUPPORTED, "rotary dim / 2 = %lld exceeds %d", (long long)half,
                    kMaxMropeHalf);
    if (mrope_section[0] > half || mrope_section[1] > half || mrope_section[2] > half ||
        mrope_section[0] + mrope_section[1] + mrope_section[2] != half)  // no overflow: each <= half
        return fail(ROPE_ERR_ATTRIBUTE, "mrope_section (%lld, %lld, %lld) must sum to rotary dim / 2 = %lld",
                    (long long)mrope_section[0], (long long)mrope_section[1], (long long)mrope_section[2],
                    (long long)half);
    if (cos_cache->rank != 2)
        return fail(ROPE_ERR_RANK, "cos_cache must be rank 2 (max_sequence_length, rotary_dim/2)");
    if (!same_shape(cos_cache, sin_cache))
        return fail(ROPE_ERR_SHAPE, "sin_cache must have the shape of cos_cache");
    if (cos_cache->shape[1] != half)
        return fail(ROPE_ERR_SHAPE, "cos_cache width %lld != rotary dim / 2 = %lld",
                    (long long)cos_cache->shape[1], (long long)half);
    if (position_ids->rank != 3)
        return fail(ROPE_ERR_RANK, "position_ids must be rank 3 (3, batch, sequence)");
    if (position_ids->shape[0] != 3 || position_ids->shape[1] != B || position_ids->shape[2] != S)
        return fail(ROPE_ERR_SHAPE, "position_ids must be (3, %lld, %lld)", (long long)B, (long long)S);

    const rope_tensor* others[3] = {cos_cache, sin_cache, position_ids};
    const char* names[3] = {"cos_cache", "sin_cache", "position_ids"};
    TRY(check_output(y, "y", x, others, names, 3));

    Problem& p = out->p;
    p.dtype = x->dtype;
    p.interleaved = (int32_t)interleaved;
    p.B = B; p.S = S; p.D = D; p.R = R;
    p.ntask = 1;
    p.task[0].x = x->data;
    p.task[0].y = y->data;
    fill_strides(&p.task[0], x->rank, S, H, D);
    p.coef = kCoefMrope;
    p.cos = cos_cache->data;
    p.sin = sin_cache->data;
    p.ids = (const int64_t*)position_ids->data;
    p.M = cos_cache->shape[0];
    p.scale = scale;
    p.scaling = 1.0f;
    uint8_t streams[kMaxMropeHalf];
    mrope_streams(half, mrope_section, mrope_layout, streams);
    for (int64_t i = 0; i < half; ++i)
        p.sel[i / 16] |= (uint32_t)streams[i] << (2 * (i % 16));
    // the slots a 16-byte chunk of X rotates with (8 / 4 of them for 2- /
    // 4-byte split halves, half that interleaved) all from one stream, as
    // sectioned layouts with sections in multiples of that give
    const int64_t chunk_slots = (16 / elem_size(p.dtype)) / (p.interleaved ? 2 : 1);
    p.mrope_single = 1;
    for (int64_t i = 0; i < half; ++i)
        if (streams[i] != streams[i - i % chunk_slots]) p.mrope_single = 0;
    out->empty = numel(x) == 0;
    out->g.rank = x->rank;
    return finish_plan(out);
}

int plan_rope_qk(const rope_tensor* q, const rope_tensor* k, const rope_tensor* cos_cache,
                 const rope_tensor* sin_cache, const rope_tensor* position_ids,
                 const rope_tensor* yq, const rope_tensor* yk, int64_t interleaved,
                 int64_t num_heads, int64_t kv_num_heads, int64_t rotary_embedding_dim,
                 const rope_tensor* inv_freq, float attention_scaling, Plan* out) {
    clear_error();
    memset(out, 0, sizeof(*out));
    if (!q) return fail(ROPE_ERR_NULL, "q is missing");
    if (!k) return fail(ROPE_ERR_NULL, "k is missing");
    if (!yq) return fail(ROPE_ERR_NULL, "yq is missing");
    if (!yk) return fail(ROPE_ERR_NULL, "yk is missing");
    if ((cos_cache == nullptr) != (sin_cache == nullptr))
        return fail(ROPE_ERR_NULL, "cos_cache and sin_cache must both be given or both be NULL");
    const bool onthefly = cos_cache == nullptr;
    if (onthefly && !inv_freq)
        return fail(ROPE_ERR_NULL, "inv_freq is required when cos/sin tables are absent");
    if (onthefly && !position_ids)
        return fail(ROPE_ERR_NULL, "position_ids are required when cos/sin tables are absent");
    TRY(check_desc(q, "q"));
    TRY(check_desc(k, "k"));
    TRY(check_desc(yq, "yq"));
    TRY(check_desc(yk, "yk"));
    if (cos_cache) TRY(check_desc(cos_cache, "cos_cache"));
    if (sin_cache) TRY(check_desc(sin_cache, "sin_cache"));
    if (position_ids) TRY(check_desc(position_ids, "position_ids"));
    if (onthefly) TRY(check_desc(inv_freq, "inv_freq"));

    if (!is_float(q->dtype)) return fail(ROPE_ERR_DTYPE, "q must be float32, float16 or bfloat16");
    if (k->dtype != q->dtype || yq->dtype != q->dtype || yk->dtype != q->dtype)
        return fail(ROPE_ERR_DTYPE, "k, yq and yk must have the type of q");
    if (cos_cache && (cos_cache->dtype != q->dtype || sin_cache->dtype != q->dtype))
        return fail(ROPE_ERR_DTYPE, "cos_cache and sin_cache must have the type of q");
    if (position_ids && position_ids->dtype != ROPE_INT64)
        return fail(ROPE_ERR_DTYPE, "position_ids must be int64");
    if (onthefly && inv_freq->dtype != ROPE_FLOAT)
        return fail(ROPE_ERR_DTYPE, "inv_freq must be float32");
    if (interleaved != 0 && interleaved != 1)
        return fail(ROPE_ERR_ATTRIBUTE, "interleaved must be 0 or 1");
    if (num_heads < 0 || kv_num_heads < 0)
        return fail(ROPE_ERR_ATTRIBUTE, "num_heads and kv_num_heads must be >= 0");

    if (q->rank != 3 && q->rank != 4)
        return fail(ROPE_ERR_RANK, "q must be rank 3 or 4, got %d", (int)q->rank);
    if (k->rank != q->rank) return fail(ROPE_ERR_RANK, "k must have the rank of q");
    if (!same_shape(q, yq)) return fail(ROPE_ERR_SHAPE, "yq must have the shape of q");
    if (!same_shape(k, yk)) return fail(ROPE_ERR_SHAPE, "yk must have the shape of k");
    int64_t B, S, H, D, Bk, Sk, Hk, Dk, R, M = 0;
    TRY(activation_dims(q, "q", num_heads, false, &B, &S, &H, &D));
    TRY(activation_dims(k, "k", kv_num_heads, false, &Bk, &Sk, &Hk, &Dk));
    if (Bk != B || Sk != S)
        return fail(ROPE_ERR_SHAPE, "q and k disagree on batch or sequence length");
    if (Dk != D) return fail(ROPE_ERR_SHAPE, "q and k disagree on head_size");
    if (Hk > 0 && H % Hk != 0)
        return fail(ROPE_ERR_SHAPE, "kv_num_heads %lld must divide num_heads %lld", (long long)Hk,
                    (long long)H);
    if (D % 2 != 0) return fail(ROPE_ERR_SHAPE, "head_size %lld must be even", (long long)D);
    TRY(check_rotary_dim(D, rotary_embedding_dim, &R));
    if (!onthefly) {
        TRY(check_tables(cos_cache, sin_cache, position_ids, B, S, R, &M));
    } else {
        if (inv_freq->rank != 1 || inv_freq->shape[0] != R / 2)
            return fail(ROPE_ERR_SHAPE, "inv_freq must be (rotary_dim/2,) = (%lld,)", (long long)(R / 2));
        if (position_ids->rank != 2)
            return fail(ROPE_ERR_RANK, "position_ids must be rank 2 (batch, sequence)");
        if (position_ids->shape[0] != B || position_ids->shape[1] != S)
            return fail(ROPE_ERR_SHAPE, "position_ids must be (%lld, %lld)", (long long)B, (long long)S);
    }

    const rope_tensor* in_q[5] = {k, cos_cache, sin_cache, position_ids, onthefly ? inv_freq : nullptr};
    const char* nm_q[5] = {"k", "cos_cache", "sin_cache", "position_ids", "inv_freq"};
    TRY(check_output(yq, "yq", q, in_q, nm_q, 5));
    const rope_tensor* in_k[6] = {q, cos_cache, sin_cache, position_ids,
                                  onthefly ? inv_freq : nullptr, yq};
    const char* nm_k[6] = {"q", "cos_cache", "sin_cache", "position_ids", "inv_freq", "yq"};
    TRY(check_output(yk, "yk", k, in_k, nm_k, 6));

    Problem& p = out->p;
    p.dtype = q->dtype;
    p.interleaved = (int32_t)interleaved;
    p.B = B; p.S = S; p.D = D; p.R = R;
    p.ntask = 2;
    p.task[0].x = q->data;
    p.task[0].y = yq->data;
    fill_strides(&p.task[0], q->rank, S, H, D);
    p.task[1].x = k->data;
    p.task[1].y = yk->data;
    fill_strides(&p.task[1], k->rank, S, Hk, D);
    p.ids = position_ids ? (const int64_t*)position_ids->data : nullptr;
    p.M = M;
    p.scale = 1.0f;
    p.scaling = attention_scaling;
    if (onthefly) {
        p.coef = kCoefOnTheFly;
        p.inv_freq = (const float*)inv_freq->data;
    } else {
        p.coef = position_ids ? kCoefGather : kCoefPerToken;
        p.cos = cos_cache->data;
        p.sin = sin_cache->data;
    }
    out->empty = numel(q) == 0 && numel(k) == 0;
    out->g.rank = q->rank;
    return finish_plan(out);
}

// QK-norm then RoPE: onnxruntime PR #27590 review, Qwen3 architecture (RMSNorm
// on Q and K after the projection, before RoPE). The Q+K contract plus the
// two (D,) weights of the storage type and a finite epsilon >= 0.
int plan_rope_qk_norm(const rope_tensor* q, const rope_tensor* k, const rope_tensor* q_weight,
                      const rope_tensor* k_weight, float epsilon, const rope_tensor* cos_cache,
                      const rope_tensor* sin_cache, const rope_tensor* position_ids,
                      const rope_tensor* yq, const rope_tensor* yk, int64_t interleaved,
                      int64_t num_heads, int64_t kv_num_heads, int64_t rotary_embedding_dim,
                      const rope_tensor* inv_freq, float attention_scaling, Plan* out) {
    TRY(plan_rope_qk(q, k, cos_cache, sin_cache, position_ids, yq, yk, interleaved, num_heads,
                     kv_num_heads, rotary_embedding_dim, inv_freq, attention_scaling, out));
    if (!q_weight) return fail(ROPE_ERR_NULL, "q_weight is missing");
    if (!k_weight) return fail(ROPE_ERR_NULL, "k_weight is missing");
    TRY(check_desc(q_weight, "q_weight"));
    TRY(check_desc(k_weight, "k_weight"));
    Problem& p = out->p;
    if (q_weight->dtype != p.dtype || k_weight->dtype != p.dtype)
        return fail(ROPE_ERR_DTYPE, "q_weight and k_weight must have the type of q");
    if (q_weight->rank != 1 || k_weight->rank != 1)
        return fail(ROPE_ERR_RANK, "q_weight and k_weight must be rank 1 (head_size,)");
    if (q_weight->shape[0] != p.D || k_weight->shape[0] != p.D)
        return fail(ROPE_ERR_SHAPE, "q_weight and k_weight must be (%lld,)", (long long)p.D);
    if (!(epsilon >= 0.0f) || !std::isfinite(epsilon))
        return fail(ROPE_ERR_ATTRIBUTE, "epsilon must be finite and >= 0");
    const rope_tensor* w[2] = {q_weight, k_weight};
    const char* wn[2] = {"q_weight", "k_weight"};
    TRY(check_output(yq, "yq", nullptr, w, wn, 2));
    TRY(check_output(yk, "yk", nullptr, w, wn, 2));
    p.norm = 1;
    p.eps = epsilon;
    p.task[0].weight = q_weight->data;
    p.task[1].weight = k_weight->data;
    return finish_plan(out);
}

// Packed [Q|K|V]: the SparseAttention README's packed query input holds,
// per token, num_heads query heads, then kv_num_heads key heads, then
// kv_num_heads value heads. Q and K are rotated; V is copied to y unless y is
// the input itself (in place), where it is left alone.
int plan_rope_qkv_packed(const rope_tensor* qkv, const rope_tensor* cos_cache,
                         const rope_tensor* sin_cache, const rope_tensor* position_ids,
                         const rope_tensor* y, int64_t interleaved, int64_t num_heads,
                         int64_t kv_num_heads, int64_t rotary_embedding_dim,
                         const rope_tensor* inv_freq, float attention_scaling, Plan* out) {
    clear_error();
    memset(out, 0, sizeof(*out));
    if (!qkv) return fail(ROPE_ERR_NULL, "qkv is missing");
    if (!y) return fail(ROPE_ERR_NULL, "y is missing");
    if ((cos_cache == nullptr) != (sin_cache == nullptr))
        return fail(ROPE_ERR_NULL, "cos_cache and sin_cache must both be given or both be NULL");
    const bool onthefly = cos_cache == nullptr;
    if (onthefly && !inv_freq)
        return fail(ROPE_ERR_NULL, "inv_freq is required when cos/sin tables are absent");
    if (onthefly && !position_ids)
        return fail(ROPE_ERR_NULL, "position_ids are required when cos/sin tables are absent");
    TRY(check_desc(qkv, "qkv"));
    TRY(check_desc(y, "y"));
    if (cos_cache) TRY(check_desc(cos_cache, "cos_cache"));
    if (sin_cache) TRY(check_desc(sin_cache, "sin_cache"));
    if (position_ids) TRY(check_desc(position_ids, "position_ids"));
    if (onthefly) TRY(check_desc(inv_freq, "inv_freq"));
    if (!is_float(qkv->dtype)) return fail(ROPE_ERR_DTYPE, "qkv must be float32, float16 or bfloat16");
    if (y->dtype != qkv->dtype) return fail(ROPE_ERR_DTYPE, "y must have the type of qkv");
    if (cos_cache && (cos_cache->dtype != qkv->dtype || sin_cache->dtype != qkv->dtype))
        return fail(ROPE_ERR_DTYPE, "cos_cache and sin_cache must have the type of qkv");
    if (position_ids && position_ids->dtype != ROPE_INT64)
        return fail(ROPE_ERR_DTYPE, "position_ids must be int64");
    if (onthefly && inv_freq->dtype != ROPE_FLOAT)
        return fail(ROPE_ERR_DTYPE, "inv_freq must be float32");
    if (interleaved != 0 && interleaved != 1)
        return fail(ROPE_ERR_ATTRIBUTE, "interleaved must be 0 or 1");
    if (num_heads < 1 || kv_num_heads < 1)
        return fail(ROPE_ERR_ATTRIBUTE, "num_heads and kv_num_heads are required (>= 1) for packed QKV");
    TRY(check_head_count(num_heads));
    if (num_heads % kv_num_heads != 0)
        return fail(ROPE_ERR_SHAPE, "kv_num_heads %lld must divide num_heads %lld",
                    (long long)kv_num_heads, (long long)num_heads);
    if (qkv->rank != 3 && qkv->rank != 4)
        return fail(ROPE_ERR_RANK, "qkv must be rank 3 or 4, got %d", (int)qkv->rank);
    if (!same_shape(qkv, y)) return fail(ROPE_ERR_SHAPE, "y must have the shape of qkv");
    const int64_t Hall = num_heads + 2 * kv_num_heads;
    int64_t B, S, D, R, M = 0;
    if (qkv->rank == 3) {
        if (qkv->shape[2] % Hall != 0)
            return fail(ROPE_ERR_SHAPE, "packed width %lld is not (num_heads + 2*kv_num_heads) * head_size",
                        (long long)qkv->shape[2]);
        B = qkv->shape[0];
        S = qkv->shape[1];
        D = qkv->shape[2] / Hall;
    } else {
        if (qkv->shape[1] != Hall)
            return fail(ROPE_ERR_SHAPE, "packed dim 1 = %lld != num_heads + 2*kv_num_heads = %lld",
                        (long long)qkv->shape[1], (long long)Hall);
        B = qkv->shape[0];
        S = qkv->shape[2];
        D = qkv->shape[3];
    }
    if (D % 2 != 0) return fail(ROPE_ERR_SHAPE, "head_size %lld must be even", (long long)D);
    TRY(check_rotary_dim(D, rotary_embedding_dim, &R));
    if (!onthefly) {
        TRY(check_tables(cos_cache, sin_cache, position_ids, B, S, R, &M));
    } else {
        if (inv_freq->rank != 1 || inv_freq->shape[0] != R / 2)
            return fail(ROPE_ERR_SHAPE, "inv_freq must be (rotary_dim/2,) = (%lld,)", (long long)(R / 2));
        if (position_ids->rank != 2)
            return fail(ROPE_ERR_RANK, "position_ids must be rank 2 (batch, sequence)");
        if (position_ids->shape[0] != B || position_ids->shape[1] != S)
            return fail(ROPE_ERR_SHAPE, "position_ids must be (%lld, %lld)", (long long)B, (long long)S);
    }
    const rope_tensor* others[4] = {cos_cache, sin_cache, position_ids, onthefly ? inv_freq : nullptr};
    const char* names[4] = {"cos_cache", "sin_cache", "position_ids", "inv_freq"};
    TRY(check_output(y, "y", qkv, others, names, 4));

    Problem& p = out->p;
    p.dtype = qkv->dtype;
    p.interleaved = (int32_t)interleaved;
    p.B = B; p.S = S; p.D = D; p.R = R;
    const int es = elem_size(qkv->dtype);
    // the three head groups share the packed strides; they start H*D (rank 3)
    // or H*S*D (rank 4) elements apart
    Task base = {};
    fill_strides(&base, qkv->rank, S, Hall, D);
    const int64_t group_step = qkv->rank == 3 ? D : S * D;  // elements per head step
    const int64_t first[3] = {0, num_heads, num_heads + kv_num_heads};
    const int64_t heads[3] = {num_heads, kv_num_heads, kv_num_heads};
    const bool inplace = y->data == qkv->data;
    p.ntask = inplace ? 2 : 3;
    for (int t = 0; t < p.ntask; ++t) {
        p.task[t] = base;
        p.task[t].heads = heads[t];
        p.task[t].x = (const char*)qkv->data + first[t] * group_step * es;
        p.task[t].y = (char*)y->data + first[t] * group_step * es;
        p.task[t].copy = t == 2;
    }
    p.ids = position_ids ? (const int64_t*)position_ids->data : nullptr;
    p.M = M;
    p.scale = 1.0f;
    p.scaling = attention_scaling;
    if (onthefly) {
        p.coef = kCoefOnTheFly;
        p.inv_freq = (const float*)inv_freq->data;
    } else {
        p.coef = position_ids ? kCoefGather : kCoefPerToken;
        p.cos = cos_cache->data;
        p.sin = sin_cache->data;
    }
    out->empty = numel(qkv) == 0;
    out->g.rank = qkv->rank;
    return finish_plan(out);
}

// RoPE on Q and K with the key/value cache append: the SparseAttention
// README's inputs (query plain or packed, past_key/past_value updated in
// place, total_sequence_length, key_total_sequence_lengths, cos/sin caches)
// and attributes (rotary_interleaved, num_heads, kv_num_heads).
int plan_rope_kv_append(const rope_tensor* query, const rope_tensor* key,
                        const rope_tensor* value, const rope_tensor* past_key,
                        const rope_tensor* past_value,
                        const rope_tensor* key_total_sequence_lengths,
                        int64_t total_sequence_length, const rope_tensor* cos_cache,
                        const rope_tensor* sin_cache, const rope_tensor* q_out,
                        int64_t interleaved, int64_t num_heads, int64_t kv_num_heads,
                        Plan* out) {
    clear_error();
    memset(out, 0, sizeof(*out));
    if (!query) return fail(ROPE_ERR_NULL, "query is missing");
    if ((key == nullptr) != (value == nullptr))
        return fail(ROPE_ERR_NULL, "key and value must both be given or both be NULL (packed query)");
    if (!past_key) return fail(ROPE_ERR_NULL, "past_key is missing");
    if (!past_value) return fail(ROPE_ERR_NULL, "past_value is missing");
    if (!key_total_sequence_lengths) return fail(ROPE_ERR_NULL, "key_total_sequence_lengths is missing");
    if (!cos_cache) return fail(ROPE_ERR_NULL, "cos_cache is missing");
    if (!sin_cache) return fail(ROPE_ERR_NULL, "sin_cache is missing");
    if (!q_out) return fail(ROPE_ERR_NULL, "q_out is missing");
    const bool packed = key == nullptr;
    TRY(check_desc(query, "query"));
    if (!packed) {
        TRY(check_desc(key, "key"));
        TRY(check_desc(value, "value"));
    }
    TRY(check_desc(past_key, "past_key"));
    TRY(check_desc(past_value, "past_value"));
    TRY(check_desc(key_total_sequence_lengths, "key_total_sequence_lengths"));
    TRY(check_desc(cos_cache, "cos_cache"));
    TRY(check_desc(sin_cache, "sin_cache"));
    TRY(check_desc(q_out, "q_out"));

    const int32_t T = query->dtype;
    if (!is_float(T)) return fail(ROPE_ERR_DTYPE, "query must be float32, float16 or bfloat16");
    if ((!packed && (key->dtype != T || value->dtype != T)) || past_key->dtype != T ||
        past_value->dtype != T || cos_cache->dtype != T || sin_cache->dtype != T || q_out->dtype != T)
        return fail(ROPE_ERR_DTYPE, "key, value, caches, tables and q_out must have the type of query");
    if (key_total_sequence_lengths->dtype != ROPE_INT32)
        return fail(ROPE_ERR_DTYPE, "key_total_sequence_lengths must be int32");
    // SparseAttention README, Attributes: 1 rotates adjacent pairs and every
    // other value selects the NeoX half-split
    interleaved = interleaved == 1 ? 1 : 0;
    if (num_heads < 1 || kv_num_heads < 1)
        return fail(ROPE_ERR_ATTRIBUTE, "num_heads and kv_num_heads are required (>= 1)");
    TRY(check_head_count(num_heads));
    if (num_heads % kv_num_heads != 0)
        return fail(ROPE_ERR_SHAPE, "kv_num_heads %lld must divide num_heads %lld",
                    (long long)kv_num_heads, (long long)num_heads);

    if (query->rank != 3) return fail(ROPE_ERR_RANK, "query must be rank 3 (batch, sequence, hidden)");
    const int64_t B = query->shape[0], S = query->shape[1];
    const int64_t groups = packed ? num_heads + 2 * kv_num_heads : num_heads;
    if (query->shape[2] % groups != 0)
        return fail(ROPE_ERR_SHAPE, "query width %lld is not %s * head_size", (long long)query->shape[2],
                    packed ? "(num_heads + 2*kv_num_heads)" : "num_heads");
    const int64_t D = query->shape[2] / groups;
    if (D % 2 != 0) return fail(ROPE_ERR_SHAPE, "head_size %lld must be even", (long long)D);
    if (!packed) {
        if (key->rank != 3 || value->rank != 3) return fail(ROPE_ERR_RANK, "key and value must be rank 3");
        if (key->shape[0] != B || key->shape[1] != S || key->shape[2] != kv_num_heads * D)
            return fail(ROPE_ERR_SHAPE, "key must be (%lld, %lld, %lld)", (long long)B, (long long)S,
                        (long long)(kv_num_heads * D));
        if (!same_shape(key, value)) return fail(ROPE_ERR_SHAPE, "value must have the shape of key");
    }
    if (past_key->rank != 4) return fail(ROPE_ERR_RANK, "past_key must be rank 4 (batch, kv_num_heads, max_sequence, head_size)");
    if (past_key->shape[0] != B || past_key->shape[1] != kv_num_heads || past_key->shape[3] != D)
        return fail(ROPE_ERR_SHAPE, "past_key must be (%lld, %lld, max_sequence, %lld)", (long long)B,
                    (long long)kv_num_heads, (long long)D);
    if (!same_shape(past_key, past_value)) return fail(ROPE_ERR_SHAPE, "past_value must have the shape of past_key");
    const int64_t Smax = past_key->shape[2];
    if (key_total_sequence_lengths->rank != 1 || key_total_sequence_lengths->shape[0] != B)
        return fail(ROPE_ERR_SHAPE, "key_total_sequence_lengths must be (batch,) = (%lld,)", (long long)B);
    if (cos_cache->rank != 2) return fail(ROPE_ERR_RANK, "cos_cache must be rank 2 (rows, rotary_dim/2)");
    if (!same_shape(cos_cache, sin_cache)) return fail(ROPE_ERR_SHAPE, "sin_cache must have the shape of cos_cache");
    if (cos_cache->shape[1] < 1 || cos_cache->shape[1] > D / 2)
        return fail(ROPE_ERR_SHAPE, "cos_cache width %lld must be in [1, head_size/2 = %lld]",
                    (long long)cos_cache->shape[1], (long long)(D / 2));
    const int64_t R = 2 * cos_cache->shape[1];
    const int64_t M = cos_cache->shape[0];
    if (q_out->rank != 3 || q_out->shape[0] != B || q_out->shape[1] != S || q_out->shape[2] != num_heads * D)
        return fail(ROPE_ERR_SHAPE, "q_out must be (%lld, %lld, %lld)", (long long)B, (long long)S,
                    (long long)(num_heads * D));
    if (total_sequence_length < S || total_sequence_length > Smax || total_sequence_length > M)
        return fail(ROPE_ERR_SHAPE,
                    "total_sequence_length %lld must lie in [sequence %lld, min(cache rows %lld, table rows %lld)]",
                    (long long)total_sequence_length, (long long)S, (long long)Smax, (long long)M);

    // aliasing: q_out may be the (unpacked) query itself; the caches are
    // written in place and overlap nothing else
    const rope_tensor* ins[6] = {key, value, cos_cache, sin_cache, key_total_sequence_lengths,
                                 packed ? query : nullptr};
    const char* in_names[6] = {"key", "value", "cos_cache", "sin_cache", "key_total_sequence_lengths", "query"};
    TRY(check_output(q_out, "q_out", packed ? nullptr : query, ins, in_names, 6));
    const rope_tensor* all[8] = {query, key, value, cos_cache, sin_cache, key_total_sequence_lengths, q_out,
                                 past_value};
    const char* all_names[8] = {"query", "key", "value", "cos_cache", "sin_cache",
                                "key_total_sequence_lengths", "q_out", "past_value"};
    TRY(check_output(past_key, "past_key", nullptr, all, all_names, 8));
    TRY(check_output(past_value, "past_value", nullptr, all, all_names, 7));

    Problem& p = out->p;
    p.dtype = T;
    p.interleaved = (int32_t)interleaved;
    p.B = B; p.S = S; p.D = D; p.R = R;
    const int es = elem_size(T);
    const int64_t Hall = packed ? num_heads + 2 * kv_num_heads : num_heads;
    p.ntask = 3;
    // Q: rows of the query (packed or not) to the dense q_out
    fill_strides(&p.task[0], 3, S, Hall, D);
    p.task[0].heads = num_heads;
    p.task[0].x = query->data;
    p.task[0].y = q_out->data;
    p.task[0].ystride_b = S * num_heads * D;
    p.task[0].ystride_s = num_heads * D;
    p.task[0].ystride_h = D;
    // K (rotated) and V (copied) to row `position` of the caches
    for (int t = 1; t < 3; ++t) {
        Task& k = p.task[t];
        if (packed) {
            fill_strides(&k, 3, S, Hall, D);
            k.x = (const char*)query->data + (t == 1 ? num_heads : num_heads + kv_num_heads) * D * es;
        } else {
            fill_strides(&k, 3, S, kv_num_heads, D);
            k.x = t == 1 ? key->data : value->data;
        }
        k.heads = kv_num_heads;
        k.y = t == 1 ? past_key->data : past_value->data;
        k.ystride_b = kv_num_heads * Smax * D;
        k.ystride_h = Smax * D;
        k.ystride_s = D;
        k.yrow = 1;
        k.copy = t == 2;
    }
    p.coef = kCoefAppend;
    p.cos = cos_cache->data;
    p.sin = sin_cache->data;
    p.M = M;
    p.seqlens = (const int32_t*)key_total_sequence_lengths->data;
    p.prompt = total_sequence_length == S;
    p.rows_out = Smax;
    p.scale = 1.0f;
    p.scaling = 1.0f;
    out->empty = B * S == 0;
    out->g.rank = 3;
    return finish_plan(out);
}

// The cache append with QK-norm: Q and K RMS-normalised before the rotation
// (PR #27590 review, Qwen3 architecture), V copied as it is: a QK-norm
// model's decode step before attention, in one launch.
int plan_rope_kv_append_qk_norm(const rope_tensor* query, const rope_tensor* key,
                                const rope_tensor* value, const rope_tensor* past_key,
                                const rope_tensor* past_value,
                                const rope_tensor* key_total_sequence_lengths,
                                int64_t total_sequence_length, const rope_tensor* cos_cache,
                                const rope_tensor* sin_cache, const rope_tensor* q_out,
                                const rope_tensor* q_weight, const rope_tensor* k_weight,
                                float epsilon, int64_t interleaved, int64_t num_heads,
                                int64_t kv_num_heads, Plan* out) {
    TRY(plan_rope_kv_append(query, key, value, past_key, past_value, key_total_sequence_lengths,
                            total_sequence_length, cos_cache, sin_cache, q_out, interleaved, num_heads,
                            kv_num_heads, out));
    if (!q_weight) return fail(ROPE_ERR_NULL, "q_weight is missing");
    if (!k_weight) return fail(ROPE_ERR_NULL, "k_weight is missing");
    TRY(check_desc(q_weight, "q_weight"));
    TRY(check_desc(k_weight, "k_weight"));
    Problem& p = out->p;
    if (q_weight->dtype != p.dtype || k_weight->dtype != p.dtype)
        return fail(ROPE_ERR_DTYPE, "q_weight and k_weight must have the type of query");
    if (q_weight->rank != 1 || k_weight->rank != 1)
        return fail(ROPE_ERR_RANK, "q_weight and k_weight must be rank 1 (head_size,)");
    if (q_weight->shape[0] != p.D || k_weight->shape[0] != p.D)
        return fail(ROPE_ERR_SHAPE, "q_weight and k_weight must be (%lld,)", (long long)p.D);
    if (!(epsilon >= 0.0f) || !std::isfinite(epsilon))
        return fail(ROPE_ERR_ATTRIBUTE, "epsilon must be finite and >= 0");
    const rope_tensor* w[2] = {q_weight, k_weight};
    const char* wn[2] = {"q_weight", "k_weight"};
    TRY(check_output(q_out, "q_out", nullptr, w, wn, 2));
    TRY(check_output(past_key, "past_key", nullptr, w, wn, 2));
    TRY(check_output(past_value, "past_value", nullptr, w, wn, 2));
    p.norm = 1;
    p.eps = epsilon;
    p.task[0].weight = q_weight->data;
    p.task[1].weight = k_weight->data;
    p.task[2].weight = nullptr;  // V: copied, never normalised
    return finish_plan(out);
}

int plan_inv_freq(const rope_tensor* inv_freq, double base, float** out, int64_t* half) {
    clear_error();
    if (!inv_freq) return fail(ROPE_ERR_NULL, "inv_freq is missing");
    TRY(check_desc(inv_freq, "inv_freq"));
    if (inv_freq->dtype != ROPE_FLOAT) return fail(ROPE_ERR_DTYPE, "inv_freq must be float32");
    if (inv_freq->rank != 1) return fail(ROPE_ERR_RANK, "inv_freq must be rank 1");
    if (!(base > 0.0) || !std::isfinite(base))
        return fail(ROPE_ERR_ATTRIBUTE, "base must be positive and finite");
    *out = (float*)inv_freq->data;
    *half = inv_freq->shape[0];
    return ROPE_OK;
}

int plan_cos_sin_cache(const rope_tensor* inv_freq, float scaling, const rope_tensor* cos_out,
                       const rope_tensor* sin_out, TablePlan* out) {
    clear_error();
    memset(out, 0, sizeof(*out));
    if (!inv_freq) return fail(ROPE_ERR_NULL, "inv_freq is missing");
    if (!cos_out) return fail(ROPE_ERR_NULL, "cos_out is missing");
    if (!sin_out) return fail(ROPE_ERR_NULL, "sin_out is missing");
    TRY(check_desc(inv_freq, "inv_freq"));
    TRY(check_desc(cos_out, "cos_out"));
    TRY(check_desc(sin_out, "sin_out"));
    if (inv_freq->dtype != ROPE_FLOAT) return fail(ROPE_ERR_DTYPE, "inv_freq must be float32");
    if (!is_float(cos_out->dtype) || sin_out->dtype != cos_out->dtype)
        return fail(ROPE_ERR_DTYPE, "cos_out and sin_out must both be float32 or both float16");
    if (inv_freq->rank != 1) return fail(ROPE_ERR_RANK, "inv_freq must be rank 1");
    if (cos_out->rank != 2) return fail(ROPE_ERR_RANK, "cos_out must be rank 2 (rows, rotary_dim/2)");
    if (!same_shape(cos_out, sin_out)) return fail(ROPE_ERR_SHAPE, "sin_out must have the shape of cos_out");
    if (cos_out->shape[1] != inv_freq->shape[0])
        return fail(ROPE_ERR_SHAPE, "table width %lld != inv_freq length %lld",
                    (long long)cos_out->shape[1], (long long)inv_freq->shape[0]);
    if (overlaps(cos_out, inv_freq) || overlaps(sin_out, inv_freq) || overlaps(cos_out, sin_out))
        return fail(ROPE_ERR_ALIAS, "outputs overlap each other or inv_freq");
    out->inv_freq = (const float*)inv_freq->data;
    out->cos = cos_out->data;
    out->sin = sin_out->data;
    out->dtype = cos_out->dtype;
    out->rows = cos_out->shape[0];
    out->half = cos_out->shape[1];
    out->scaling = scaling;
    return ROPE_OK;
}

}  // namespace rope
