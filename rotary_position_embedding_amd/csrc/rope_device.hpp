// rope_device.hpp -- the kernels and their launch templates (device side),
// included by rope_kernels.hip and by two translation units per storage
// type (rope_kernels_<type>.hip: the vector kernel; rope_kernels_<type>_row.hip:
// the row, scalar and table kernels), which instantiate them in parallel
// builds.
//
//
// What is computed (pages cited by title and section):
//   per pair (x1, x2) of a head row with coefficients (c, s) of its slot,
//   y1 = x1*c - x2*s, y2 = x2*c + x1*s  -- onnxruntime PR #27590 review,
//   rotate_half / apply_rotary_pos_emb; pairs (i, i+R/2) or (2i, 2i+1) --
//   "ai.onnx.RotaryEmbedding" manifest, attributeDescriptions.interleaved;
//   elements R..D-1 copied -- same, rotary_embedding_dim.
// Coefficient rows: gathered by position id, per-token, M-RoPE (slot i from
// its stream's row, scaled and rounded to the storage type, out-of-range id
// copies the pair -- "com.microsoft.MRotaryEmbedding" README), computed
// on the fly from inv_freq (PR #27590 Motivation), or gathered at the
// position past + s of a key/value cache append, whose K and V rows are
// written to that cache row ("com.microsoft.SparseAttention" README).
// With the QK-norm, each head row is first RMS-normalised and weighted (PR
// #27590 review, Qwen3 architecture) and the rotation acts on the result.
// A launch holds up to three tasks (Q, K, V or a packed [Q|K|V]); storage is
// float32, float16 or bfloat16.
//
// Per fp16 pair the op moves 8 bytes (read 4, write 4) and does 6 flops:
// it is HBM-bound and has no contraction, so no MFMA. Design:
//   * a head row is cut into 16-byte items (global_load/store_dwordx4);
//   * a wave owns TG consecutive tokens x W items of one row shape, so each
//     lane's coefficients (one 16-byte slice of cos and of sin) are fetched
//     once into registers and reused for every head of a head chunk;
//   * loads for several heads are issued before the first use, so each lane
//     keeps several 16-byte loads in flight;
//   * math in fp32 with fma and one rounding to the storage type; copies are
//     bit moves (no arithmetic on pass-through elements).
// A scalar kernel (one thread per pair or tail element) covers every shape
// and alignment the vector kernel does not.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "rope_plan.hpp"


namespace rope {

using half_t = _Float16;
using bf16_t = __bf16;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 64 * kWavesPerBlock;

constexpr int kMaxTasks = 3;

struct KTask {
    const char* x;
    char* y;
    int64_t sb, sh, ss;    // element strides of (b, h, s)
    int64_t wave_begin;    // first wave of this task (vector kernel)
    int64_t item_begin;    // first thread item of this task (scalar kernel)
    int32_t heads, hpw, chunks, tile;  // tile: token groups per head chunk in a wave tile
    int32_t copy;          // copy: pass every element through (no rotation)
    int32_t yrow;          // append kind: y row is the token's position
    int64_t ysb, ysh, yss; // append kind: element strides of y (b, h, row)
    const char* wgt;       // QK-norm: (D,) weight of this projection
    // division by chunks, tile and tile * chunks (multiply-high and shift)
    uint32_t chunks_m, chunks_s, tile_m, tile_s, per_tile_m, per_tile_s;
};

struct KArgs {
    KTask t[kMaxTasks];
    int64_t ntok, S, M;
    const char* cos;
    const char* sin;
    const int64_t* ids;
    const float* inv_freq;
    int32_t ntask, W, NP, TG, P, R, D, interleaved;
    int32_t group_major;        // three-task vector launch: waves in token-group order
    int32_t prompt;             // prompt: append kind, every sequence starts at 0
    float scaling, scale;
    float eps;                  // QK-norm epsilon
    float inv_d;                // QK-norm: 1/D rounded to binary32
    int32_t share_coef;         // on the fly: the waves of a workgroup split the slots
    int32_t row_lanes;          // row kernel: lanes per head row
    int32_t row_shift;          // log2(row_lanes) (rows of a power-of-two size)
    int32_t half_lanes;         // row kernel, split halves: lanes between partner chunks
    int32_t row_rpi;            // row kernel, other row sizes: head rows per instruction
    uint32_t row_m;             // ... and ceil(2^16 / row_lanes): lane / row_lanes as a multiply-shift
    uint32_t w_m, w_s, s_m, s_s;  // division by W and by S (multiply-high and shift)
    // group_major: per token group the chunks of task 0, then 1, then 2
    // (c0, c0 + c1 and c0 + c1 + c2 chunks), and the division by the last
    int32_t gm_c0, gm_c01, gm_c;
    uint32_t gm_m, gm_s;
    int32_t mrope_single;       // M-RoPE: every rotation item's slots take one stream
    const int32_t* seqlens;     // append kind: total key length per sequence
    int64_t rows_out;           // append kind: cache rows
    uint32_t sel[kSelWords];
};

template <typename T> struct Elem;
template <> struct Elem<float> { using bits = uint32_t; static constexpr int E = 4; };
template <> struct Elem<half_t> { using bits = uint16_t; static constexpr int E = 8; };
template <> struct Elem<bf16_t> { using bits = uint16_t; static constexpr int E = 8; };

// Materialise a binary32 value in a register. Without it the compiler may
// merge a binary32 multiply or fma with the following conversion to binary16
// into one v_fma_mixlo_f16, which rounds the exact result once to binary16
// and so skips the binary32 rounding the arithmetic here specifies.
__device__ inline float keep_f32(float v) {
    asm volatile("" : "+v"(v));
    return v;
}

__device__ inline float to_f(float v) { return v; }
__device__ inline float to_f(half_t v) { return (float)v; }
__device__ inline float to_f(bf16_t v) { return (float)v; }  // exact: the upper half of a binary32
template <typename T> __device__ inline T from_f(float v);
template <> __device__ inline float from_f<float>(float v) { return v; }
template <> __device__ inline half_t from_f<half_t>(float v) {
    return (half_t)keep_f32(v);  // nearest-even from the binary32 value
}
template <> __device__ inline bf16_t from_f<bf16_t>(float v) {
    return (bf16_t)keep_f32(v);  // nearest-even from the binary32 value
}
template <typename T> __device__ inline float round_to(float v) { return to_f(from_f<T>(v)); }

// One output of a pair's rotation, a*b + c*d (the caller folds the sign into
// d), as the binary32 value that is then converted to T.
//   binary16 / bfloat16 storage: c*d is exact in binary32 (11 + 11 or 8 + 8
//   significant bits), so one fma rounds the exact sum once to binary32.
//   binary32 storage: c*d is not exact in binary32, and rounding it before
//   the fma would make the error relative to the products rather than to the
//   result when they cancel. Both products are exact in binary64 (24 + 24
//   bits, exponents far inside its range), so the sum is formed there with
//   one rounding and then rounded to binary32: the value the definition
//   gives when evaluated in binary64, overflow included.
template <typename T>
__device__ inline float rot_out(float a, float b, float c, float d) {
    if (sizeof(T) == 4) return (float)fma((double)a, (double)b, (double)c * (double)d);
    return fmaf(a, b, c * d);
}

// Element e of a 16-byte chunk, as float. The whole chunk is reinterpreted
// as a vector of T and then indexed (a bit_cast applied to a single vector
// element is miscompiled to element 0 by this toolchain, so it is avoided).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef half_t f16x8 __attribute__((ext_vector_type(8)));
typedef bf16_t bf16x8 __attribute__((ext_vector_type(8)));
template <typename T> struct ChunkVec;
template <> struct ChunkVec<float> { typedef f32x4 type; };
template <> struct ChunkVec<half_t> { typedef f16x8 type; };
template <> struct ChunkVec<bf16_t> { typedef bf16x8 type; };

template <typename T>
__device__ inline typename ChunkVec<T>::type chunk_values(const u32x4& v) {
    return __builtin_bit_cast(typename ChunkVec<T>::type, v);
}

template <typename T>
__device__ inline u32x4 chunk_pack(const float* f) {
    typename ChunkVec<T>::type r;
#pragma unroll
    for (int i = 0; i < Elem<T>::E; ++i) r[i] = from_f<T>(f[i]);
    return __builtin_bit_cast(u32x4, r);
}

// set the bits of element e of a chunk in a mask
template <typename T> __device__ inline void mask_elem(u32x4& m, int e) {
    if (sizeof(T) == 4) m[e] = 0xffffffffu;
    else m[e >> 1] |= 0xffffu << (16 * (e & 1));
}

// Activations are reached through pointers the compiler cannot trace back to
// kernel arguments (the task selection hides them), so without a cast it
// emits flat instructions; these go through global (address space 1) ones.
#define ROPE_GLOBAL __attribute__((address_space(1)))
__device__ inline u32x4 load16_global(const char* p) { return *(const ROPE_GLOBAL u32x4*)p; }
__device__ inline u32x4 load_nt(const char* p) { return __builtin_nontemporal_load((const ROPE_GLOBAL u32x4*)p); }
__device__ inline void store_nt(char* p, const u32x4& v) { __builtin_nontemporal_store(v, (ROPE_GLOBAL u32x4*)p); }

__device__ inline u32x4 select_bits(const u32x4& keep_mask, const u32x4& keep, const u32x4& other) {
    return (keep & keep_mask) | (other & ~keep_mask);
}

// v from another lane of the same row of 16 lanes (DPP control word CTRL).
template <int CTRL>
__device__ inline float dpp_move(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xf, 0xf, false));
}

// Sum of v over aligned groups of W lanes (W a power of two <= 64, uniform);
// every lane of a group receives the same total (pairs are combined
// symmetrically, and a + b == b + a). Lanes 1 and 2 apart: quad permutes
// [1,0,3,2] and [2,3,0,1]; the other quad of an 8-lane half: half-row mirror
// (lane i <-> 7 - i); the other half of a 16-lane row: row mirror
// (i <-> 15 - i); rows 16 and 32 apart: xor shuffles.
__device__ inline float group_sum(float v, int W) {
    if (W >= 2) v += dpp_move<0xb1>(v);
    if (W >= 4) v += dpp_move<0x4e>(v);
    if (W >= 8) v += dpp_move<0x141>(v);
    if (W >= 16) v += dpp_move<0x140>(v);
    if (W >= 32) v += __shfl_xor(v, 16);
    if (W >= 64) v += __shfl_xor(v, 32);
    return v;
}

// The sum of v over a row of W consecutive lanes starting at lane `first`
// (any W up to 64; c = lane - first): at step d each lane adds the partial
// sum of the lane d above it when that lane is in the same row, so that
// after the steps 1, 2, ..., 32 the row's first lane holds the sum of the
// whole row (only values of the row are ever added), which every lane of the
// row then reads. Every lane of the wave takes part.
__device__ inline float row_sum(float v, int c, int W, int first) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const float t = __shfl_down(v, d);
        if (c + d < W) v += t;
    }
    return __shfl(v, first);
}

// Coefficient of slot i at position p computed on the fly (PR #27590
// Motivation): theta = rnd_f32(rnd_f32(p) * inv_freq[i]); cos and sin of the
// exact binary32 theta in binary64, rounded to binary32, times the scaling in
// binary32, rounded to the storage type. Shared by the table builder so the
// table and on-the-fly paths agree bit for bit.
template <typename T>
__device__ inline void onthefly_coef(float inv, int64_t p, float scaling, float& c, float& s) {
    const float pf = (float)p;
    const float theta = keep_f32(pf * inv);
    double sd, cd;
    sincos((double)theta, &sd, &cd);
    const float cf = keep_f32((float)cd);
    const float sf = keep_f32((float)sd);
    c = round_to<T>(keep_f32(cf * scaling));
    s = round_to<T>(keep_f32(sf * scaling));
}

__device__ inline int mrope_stream(const KArgs& a, int i) {
    return (a.sel[i >> 4] >> (2 * (i & 15))) & 3;
}

// Cache append: token n = b*S + s has position past(b) + s, past = 0 in the
// prompt and the sequence's total key length minus S otherwise.
__device__ inline int64_t append_position(const KArgs& a, int64_t n) {
    const int64_t b = n / a.S;
    const int64_t s = n - b * a.S;
    const int64_t past = a.prompt ? 0 : (int64_t)a.seqlens[b] - a.S;
    return past + s;
}

// Coefficient (c, s) of slot i for token n, or copy = true.
template <typename T, int COEF>
__device__ inline void coef_slot(const KArgs& a, int64_t n, int i, float& c, float& s, bool& copy) {
    const T* cos_t = reinterpret_cast<const T*>(a.cos);
    const T* sin_t = reinterpret_cast<const T*>(a.sin);
    copy = false;
    c = 1.0f;
    s = 0.0f;
    if (COEF == kCoefGather) {
        const int64_t p = a.ids[n];
        if (p < 0 || p >= a.M) { copy = true; return; }
        c = to_f(cos_t[p * a.P + i]);
        s = to_f(sin_t[p * a.P + i]);
    } else if (COEF == kCoefPerToken) {
        c = to_f(cos_t[n * a.P + i]);
        s = to_f(sin_t[n * a.P + i]);
    } else if (COEF == kCoefAppend) {
        const int64_t p = append_position(a, n);
        if (p < 0 || p >= a.M) { copy = true; return; }
        c = to_f(cos_t[p * a.P + i]);
        s = to_f(sin_t[p * a.P + i]);
    } else if (COEF == kCoefMrope) {
        const int64_t p = a.ids[(int64_t)mrope_stream(a, i) * a.ntok + n];
        if (p < 0 || p >= a.M) { copy = true; return; }
        c = round_to<T>(keep_f32(to_f(cos_t[p * a.P + i]) * a.scale));
        s = round_to<T>(keep_f32(to_f(sin_t[p * a.P + i]) * a.scale));
    } else {
        onthefly_coef<T>(a.inv_freq[i], a.ids[n], a.scaling, c, s);
    }
}

struct TaskView {
    const char* x;
    char* y;
    int64_t sb, sh, ss, wave_begin, item_begin;
    int32_t heads, hpw, chunks, tile, copy, yrow;
    int64_t ysb, ysh, yss;
    const char* wgt;
    uint32_t chunks_m, chunks_s, tile_m, tile_s, per_tile_m, per_tile_s;
};

// n / d for n < 2^31 from the divisor's multiplier m and shift l, computed
// on the host (ceil(log2 d) = l, m = floor(2^32 (2^l - d) / d) + 1): with
// t = mulhi(m, n), n / d = (t + n) >> l (the round-up method of Granlund
// and Montgomery, "Division by invariant integers using multiplication",
// 1994; the sum stays below 2^32 because t <= n < 2^31).
__device__ inline uint32_t fast_div(uint32_t n, uint32_t m, uint32_t l) {
    return (__umulhi(m, n) + n) >> l;
}

// An SGPR value the compiler must treat as opaque: keeps a select of two
// kernel-argument loads from being folded into one load from a selected
// address (that costs the wave a second, dependent round of scalar loads).
template <typename V>
__device__ inline V opaque_s(V v) {
    asm("" : "+s"(v));  // not volatile: dropped when the value is unused
    return v;
}

// Task i (0..2) of the launch: every task's fields are read in the first
// batch of scalar loads and the values are selected. The output geometry is
// the input's except for the append kind.
template <int COEF, bool NORM = false, int NT = kMaxTasks>
__device__ inline TaskView task_of(const KArgs& a, int i) {
#define ROPE_PICK(f)                                                                      \
    do {                                                                                  \
        const auto f0 = opaque_s(a.t[0].f), f1 = opaque_s(a.t[1].f);                      \
        if (NT == 2) {                                                                    \
            v.f = i == 1 ? f1 : f0;                                                       \
        } else {                                                                          \
            const auto f2 = opaque_s(a.t[2].f);                                           \
            v.f = i == 2 ? f2 : (i == 1 ? f1 : f0);                                       \
        }                                                                                 \
    } while (0)
    TaskView v;
    ROPE_PICK(x);
    ROPE_PICK(y);
    ROPE_PICK(sb);
    ROPE_PICK(sh);
    ROPE_PICK(ss);
    ROPE_PICK(wave_begin);
    ROPE_PICK(item_begin);
    ROPE_PICK(heads);
    ROPE_PICK(hpw);
    ROPE_PICK(chunks);
    ROPE_PICK(tile);
    ROPE_PICK(chunks_m);
    ROPE_PICK(chunks_s);
    ROPE_PICK(tile_m);
    ROPE_PICK(tile_s);
    ROPE_PICK(per_tile_m);
    ROPE_PICK(per_tile_s);
    ROPE_PICK(copy);
    if (COEF == kCoefAppend) {
        ROPE_PICK(yrow);
        ROPE_PICK(ysb);
        ROPE_PICK(ysh);
        ROPE_PICK(yss);
    } else {
        v.yrow = 0;
        v.ysb = v.sb;
        v.ysh = v.sh;
        v.yss = v.ss;
    }
    if (NORM) ROPE_PICK(wgt);
    else v.wgt = nullptr;
#undef ROPE_PICK
    return v;
}

// Task 0 of a single-task launch: its own fields only, no selection (the
// selection costs measurable time in launches of many waves: fp16 prefill
// 23.5 -> 23.2 us, fp32 partial interleaved 36.8 -> 36.2, M-RoPE decode
// 3.86 -> 3.62).
template <int COEF, bool NORM = false>
__device__ inline TaskView task0_of(const KArgs& a) {
    const KTask& t = a.t[0];
    TaskView v;
    v.x = t.x;
    v.y = t.y;
    v.sb = t.sb;
    v.sh = t.sh;
    v.ss = t.ss;
    v.wave_begin = t.wave_begin;
    v.item_begin = t.item_begin;
    v.heads = t.heads;
    v.hpw = t.hpw;
    v.chunks = t.chunks;
    v.tile = t.tile;
    v.chunks_m = t.chunks_m;
    v.chunks_s = t.chunks_s;
    v.tile_m = t.tile_m;
    v.tile_s = t.tile_s;
    v.per_tile_m = t.per_tile_m;
    v.per_tile_s = t.per_tile_s;
    v.copy = t.copy;
    v.yrow = COEF == kCoefAppend ? t.yrow : 0;
    v.ysb = COEF == kCoefAppend ? t.ysb : t.sb;
    v.ysh = COEF == kCoefAppend ? t.ysh : t.sh;
    v.yss = COEF == kCoefAppend ? t.yss : t.ss;
    v.wgt = NORM ? t.wgt : nullptr;
    return v;
}

// Tasks occupy consecutive ranges; unused ones start at INT64_MAX.
__device__ inline int task_index(const KArgs& a, int64_t wave) {
    return wave >= a.t[2].wave_begin ? 2 : (wave >= a.t[1].wave_begin ? 1 : 0);
}

// The task of wave gw in a launch of NT tasks (compile time: a runtime
// branch on the count would put one more dependent scalar load before the
// fields): one task reads task 0's fields only, two select between two.
template <int COEF, bool NORM, int NT>
__device__ inline TaskView task_pick(const KArgs& a, int64_t gw) {
    if (NT == 1) return task0_of<COEF, NORM>(a);
    if (NT == 2) return task_of<COEF, NORM, 2>(a, gw >= a.t[1].wave_begin ? 1 : 0);
    return task_of<COEF, NORM>(a, task_index(a, gw));
}

__device__ inline int task_index_items(const KArgs& a, int64_t item) {
    return item >= a.t[2].item_begin ? 2 : (item >= a.t[1].item_begin ? 1 : 0);
}

// ---------------------------------------------------------------------------
// Vector kernel.
//   wave -> (task, token group g, head chunk hc) in tiles of `tile` token
//   groups x all chunks: g varies fastest inside a tile. tile = 1 (rank 3:
//   a token's heads are contiguous) puts the chunks of one token group in one
//   workgroup; tile = 2 or 4 (rank 4: a head's tokens are contiguous) gives
//   each head chunk a run of consecutive token groups (with 2, a workgroup
//   holds two chunks of two groups).
//   lane item q = lane + 64*m (m < IPL) -> token t = q / W, item w = q % W.
//   item w < NP rotates: split halves -> elements [w*E, w*E+E) with partners
//   R/2 later; interleaved -> elements [w*E, w*E+E) = E/2 pairs.
//   item w >= NP copies elements [R + (w-NP)*E, +E).
// Memory order per wave: the position ids, the X chunks of the head batch
// (predicated per item and head), then the table gather, then per head the
// rotation and its stores. The compiler places a full wait before each head's
// stores, so a lane has at most two 16-byte stores in flight; measured on
// MI355X this metering is faster than letting a wave's stores pile up (a
// batch of 16 unmetered stores per lane doubled the kernel time), and so are
// the predicated loads (versus clamped unconditional ones), except for
// interleaved binary32 data, whose head batches are pipelined (in the
// kernel). X and Y are touched once: nontemporal loads and stores.

// Workgroups are dispatched to the 8 XCDs in turn (workgroup i to XCD i % 8).
// A remapping that keeps consecutive logical workgroups on one XCD (so that
// the waves sharing a token group's coefficient rows fill one L2) measured
// slower on MI355X and is not used; the workgroup order is the dispatch
// order, which also keeps the kernel-argument loads in one batch.

// X chunks of one head batch (one or two 16-byte chunks per item and head).
template <typename T, int IL, int IPL, int HU>
__device__ inline void load_batch(const char* x, const int64_t* off, const bool* act, const bool* rot,
                                  int h, int h_end, int64_t sh_bytes, int64_t half_bytes,
                                  u32x4 (*in1)[IPL], u32x4 (*in2)[IPL]) {
#pragma unroll
    for (int u = 0; u < HU; ++u) {
#pragma unroll
        for (int m = 0; m < IPL; ++m) {
            if (act[m] && h + u < h_end) {
                const char* px = x + off[m] + (int64_t)(h + u) * sh_bytes;
                in1[u][m] = load_nt(px);
                if (!IL && rot[m])
                    in2[u][m] = load_nt(px + half_bytes);
            }
        }
    }
}

// The same with every load issued, so that the compiler can count them: it
// then waits for one head batch while the next is in flight. Inactive items
// read their task's first row (offset 0) and heads past the chunk's end
// repeat its last head; the values of such loads are never used.
template <typename T, int IL, int IPL, int HU>
__device__ inline void load_batch_all(const char* x, const int64_t* off, const bool* rot,
                                      int h, int h_end, int64_t sh_bytes, int64_t half_bytes,
                                      u32x4 (*in1)[IPL], u32x4 (*in2)[IPL]) {
#pragma unroll
    for (int u = 0; u < HU; ++u) {
        const int hh = min(h + u, h_end - 1);
#pragma unroll
        for (int m = 0; m < IPL; ++m) {
            const char* px = x + off[m] + (int64_t)hh * sh_bytes;
            in1[u][m] = load_nt(px);
            if (!IL) in2[u][m] = load_nt(px + (rot[m] ? half_bytes : 0));
        }
    }
}

template <typename T, int IL, int COEF, int IPL, int HU, bool NORM = false, int NT = kMaxTasks>
__global__ __launch_bounds__(kBlock) void rope_vec_kernel(const KArgs a) {
    constexpr int E = Elem<T>::E;
    constexpr int CE = IL ? E / 2 : E;  // coefficient slots per rotation item
    constexpr int ES = (int)sizeof(T);
    typedef T cvec __attribute__((ext_vector_type(CE)));

    const int lane = threadIdx.x & 63;
    // wave-uniform by construction; readfirstlane lets the compiler keep the
    // task selection and its fields in scalar registers
    const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block;
    TaskView tk;
    if (NT == 3 && a.group_major) {
        // token-group order: the chunks of all three tasks of one token group
        // are consecutive waves (a packed [Q|K|V] row is read in one visit);
        // gw becomes the wave's index in its task's own order
        const uint32_t g = fast_div((uint32_t)gw, a.gm_m, a.gm_s);
        const int r = (int)((uint32_t)gw - g * (uint32_t)a.gm_c);
        const int ti = r < a.gm_c0 ? 0 : (r < a.gm_c01 ? 1 : 2);
        const int first = ti == 0 ? 0 : (ti == 1 ? a.gm_c0 : a.gm_c01);
        const int next = ti == 0 ? a.gm_c0 : (ti == 1 ? a.gm_c01 : a.gm_c);
        tk = task_of<COEF, NORM>(a, ti);
        gw = tk.wave_begin + (int64_t)g * (next - first) + (r - first);
    } else {
        tk = task_pick<COEF, NORM, NT>(a, gw);
    }
    // 32-bit index arithmetic (the planner keeps a vector-kernel launch's
    // waves and tokens below 2^31): a short scalar prologue before the loads
    const uint32_t local = (uint32_t)(gw - tk.wave_begin);
    // The QK-norm instances keep the hardware-sequence divisions: measured on
    // MI355X, a shorter prologue made their prefill slower (31.8 vs 30.9 us;
    // at 160 VGPRs they run 3 waves per SIMD, so the launch comes in two
    // rounds of waves, and earlier loads arrive in a sharper burst).
    const uint32_t per_tile = (uint32_t)tk.tile * (uint32_t)tk.chunks;
    const uint32_t tile = NORM ? local / per_tile : fast_div(local, tk.per_tile_m, tk.per_tile_s);
    const int r = (int)(local - tile * per_tile);
    const int hc = NORM ? r / tk.tile : (int)fast_div((uint32_t)r, tk.tile_m, tk.tile_s);
    const uint32_t g = tile * (uint32_t)tk.tile + (uint32_t)(r - hc * tk.tile);
    const uint32_t n0 = g * (uint32_t)a.TG;
    // No early exit for waves past the last token (the rest of a partial
    // tile): their items are inactive, so they load and store nothing. An exit
    // branch here made the compiler defer kernel-argument loads behind it, one
    // more dependent round of scalar loads for every wave.
    const int h_begin = hc * tk.hpw;
    const int h_end = min(tk.heads, h_begin + tk.hpw);
    const int64_t sh_bytes = tk.sh * ES;
    const int64_t ysh_bytes = tk.ysh * ES;
    const int64_t half_bytes = (int64_t)a.P * ES;

    // -- items of this lane (no memory traffic but the append kind's lengths)
    bool act[IPL], rot[IPL];
    int64_t off[IPL];    // byte offset of the item's first chunk for head 0
    int64_t yoff[IPL];   // the same in y
    bool wr[IPL];        // the item's output row exists
    int64_t tok[IPL];
    int64_t apos[IPL];   // append kind: the token's position
    int slot0[IPL];
    int64_t elem0[IPL];  // first element of the item in its head row
#pragma unroll
    for (int m = 0; m < IPL; ++m) {
        const int q = lane + 64 * m;
        const int t = NORM ? q / a.W : (int)fast_div((uint32_t)q, a.w_m, a.w_s);
        const int w = q - t * a.W;
        const uint32_t n = n0 + (uint32_t)t;
        act[m] = t < a.TG && n < (uint64_t)a.ntok;
        rot[m] = act[m] && w < a.NP;
        const uint32_t n32 = act[m] ? n : 0u;
        const uint32_t b32 = NORM ? n32 / (uint32_t)a.S : fast_div(n32, a.s_m, a.s_s);
        tok[m] = n32;
        const int64_t b = b32;
        const int64_t s = (int64_t)(n32 - b32 * (uint32_t)a.S);
        const int64_t e0 = w < a.NP ? (int64_t)w * E : (int64_t)a.R + (int64_t)(w - a.NP) * E;
        off[m] = act[m] ? (b * tk.sb + s * tk.ss + e0) * ES : 0;
        slot0[m] = rot[m] ? w * CE : 0;  // non-rotation items read slot 0 (unused)
        elem0[m] = e0;
        if (COEF == kCoefAppend) {
            // the lengths are read for every item (sequence 0 for inactive ones)
            const int64_t past = a.prompt ? 0 : (int64_t)a.seqlens[b] - a.S;
            apos[m] = past + s;
            const int64_t row = tk.yrow ? apos[m] : s;
            wr[m] = act[m] && (!tk.yrow || (row >= 0 && row < a.rows_out));
            yoff[m] = wr[m] ? (b * tk.ysb + row * tk.yss + e0) * ES : 0;
        } else {
            apos[m] = 0;
            wr[m] = act[m];
            yoff[m] = off[m];
        }
    }

    // -- position ids, then X, then the dependent table reads --------------
    int64_t pos[IPL][COEF == kCoefMrope ? 3 : 1];
    const bool need = !tk.copy;
    // ids are read for every item (index 0 for inactive ones): unconditional
    if (COEF == kCoefGather || COEF == kCoefOnTheFly) {
#pragma unroll
        for (int m = 0; m < IPL; ++m) pos[m][0] = a.ids[tok[m]];
    } else if (COEF == kCoefAppend) {
#pragma unroll
        for (int m = 0; m < IPL; ++m) pos[m][0] = apos[m];
    } else if (COEF == kCoefMrope) {
#pragma unroll
        for (int m = 0; m < IPL; ++m)
#pragma unroll
            for (int k = 0; k < 3; ++k) pos[m][k] = a.ids[k * a.ntok + tok[m]];
    }

    uint32_t codes[IPL];  // M-RoPE: 2-bit stream of each slot of the item
    if (COEF == kCoefMrope) {
#pragma unroll
        for (int m = 0; m < IPL; ++m) codes[m] = a.sel[slot0[m] >> 4] >> (2 * (slot0[m] & 15));
    }

    // Interleaved binary32 data (rotation in binary64, longer per-pair
    // latency): every load issued and two or more head batches per wave
    // pipelined, the next batch's loads before this batch's stores (measured
    // on MI355X: fp32 partial interleaved prefill 36.2 -> 35.7 us). Other
    // instances: predicated loads, one batch at a time, the compiler waiting
    // for all of a batch's loads and placing a full wait before each head's
    // stores, which measured faster for them (with the pipelining: fp16
    // prefill 23.0 -> 24.3 us, M-RoPE 20.6 -> 24.4, split-half fp32 44.9 ->
    // 50.5).
    constexpr bool kPipe = sizeof(T) == 4 && IL && !NORM;
    u32x4 in1[HU][IPL], in2[HU][IPL];
    if (kPipe)
        load_batch_all<T, IL, IPL, HU>(tk.x, off, rot, h_begin, h_end, sh_bytes, half_bytes, in1, in2);
    else
        load_batch<T, IL, IPL, HU>(tk.x, off, act, rot, h_begin, h_end, sh_bytes, half_bytes, in1, in2);

    T cf[IPL][CE], sf[IPL][CE];
    u32x4 keep[IPL];  // input bits copied to the output as they are
#pragma unroll
    for (int m = 0; m < IPL; ++m) {
        keep[m] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < CE; ++j) { cf[m][j] = (T)1.0f; sf[m][j] = (T)0.0f; }
        if (!need) {  // a pass-through task: every element copied
            keep[m] = u32x4{0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
            continue;
        }
        if (COEF == kCoefGather || COEF == kCoefPerToken || COEF == kCoefAppend) {
            // the row is read unconditionally: an out-of-range id reads row 0
            // (with an empty table the host points the table at valid memory)
            // and the pair is then copied
            const int64_t row = COEF == kCoefPerToken ? tok[m] : pos[m][0];
            const bool valid = COEF == kCoefPerToken || (row >= 0 && row < a.M);
            const int64_t e = ((valid ? row : 0) * a.P + slot0[m]) * ES;
            const cvec cv = *reinterpret_cast<const cvec*>(a.cos + e);
            const cvec sv = *reinterpret_cast<const cvec*>(a.sin + e);
#pragma unroll
            for (int j = 0; j < CE; ++j) { cf[m][j] = cv[j]; sf[m][j] = sv[j]; }
            if (!valid) keep[m] = u32x4{0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
        } else if (COEF == kCoefMrope && a.mrope_single) {
            // every slot of the item takes the stream of its first slot: that
            // stream's row alone, the whole item copied when its id is out of
            // range
            const uint32_t k0 = codes[m] & 3u;
            const int64_t p = k0 == 0 ? pos[m][0] : (k0 == 1 ? pos[m][1] : pos[m][2]);
            const bool ok = p >= 0 && p < a.M;
            const int64_t e = ((ok ? p : 0) * a.P + slot0[m]) * ES;  // row 0 if out of range
            const cvec cv = *reinterpret_cast<const cvec*>(a.cos + e);
            const cvec sv = *reinterpret_cast<const cvec*>(a.sin + e);
            if (a.scale == 1.0f) {
#pragma unroll
                for (int j = 0; j < CE; ++j) { cf[m][j] = cv[j]; sf[m][j] = sv[j]; }
            } else {
                // scaled coefficient: binary32 product rounded to T
#pragma unroll
                for (int j = 0; j < CE; ++j) {
                    cf[m][j] = from_f<T>(keep_f32(to_f(cv[j]) * a.scale));
                    sf[m][j] = from_f<T>(keep_f32(to_f(sv[j]) * a.scale));
                }
            }
            if (!ok) keep[m] = u32x4{0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
        } else if (COEF == kCoefMrope) {
            // Slots [slot0, slot0 + CE) of the three stream rows; slot i takes
            // its stream's value. Per-stream element masks over the slice are
            // built once, then the slice is assembled with bitwise and/or on
            // whole dwords; a stream whose id is out of range contributes its
            // slots to the copy mask instead.
            constexpr int CW = CE * ES / 4;  // dwords in a coefficient slice
            typedef uint32_t cbits __attribute__((ext_vector_type(CW)));
            cbits msk0 = {}, msk1 = {}, msk2 = {};
#pragma unroll
            for (int j = 0; j < CE; ++j) {
                const uint32_t k = (codes[m] >> (2 * j)) & 3u;
                const int dw = (j * ES) / 4;
                const uint32_t bitsj = ES == 4 ? 0xffffffffu : 0xffffu << (16 * (j & 1));
                msk0[dw] |= k == 0 ? bitsj : 0u;
                msk1[dw] |= k == 1 ? bitsj : 0u;
                msk2[dw] |= k == 2 ? bitsj : 0u;
            }
            cbits cs = {}, ss = {}, copy = {};
#pragma unroll
            for (int k = 0; k < 3; ++k) {
                const int64_t p = pos[m][k];
                const cbits mk = k == 0 ? msk0 : (k == 1 ? msk1 : msk2);
                const bool ok = p >= 0 && p < a.M;
                const int64_t e = ((ok ? p : 0) * a.P + slot0[m]) * ES;  // row 0 if out of range
                const cbits cl = *reinterpret_cast<const cbits*>(a.cos + e);
                const cbits sl = *reinterpret_cast<const cbits*>(a.sin + e);
                const cbits use = ok ? mk : cbits{};
                cs |= cl & use;
                ss |= sl & use;
                copy |= ok ? cbits{} : mk;
            }
            const cvec cv = __builtin_bit_cast(cvec, cs);
            const cvec sv = __builtin_bit_cast(cvec, ss);
            if (a.scale == 1.0f) {
#pragma unroll
                for (int j = 0; j < CE; ++j) { cf[m][j] = cv[j]; sf[m][j] = sv[j]; }
            } else {
                // scaled coefficient: binary32 product rounded to T
#pragma unroll
                for (int j = 0; j < CE; ++j) {
                    cf[m][j] = from_f<T>(keep_f32(to_f(cv[j]) * a.scale));
                    sf[m][j] = from_f<T>(keep_f32(to_f(sv[j]) * a.scale));
                }
            }
            // copy mask over the X chunk: split halves share the slice layout;
            // interleaved slot j covers chunk elements 2j and 2j+1
            if (!IL) {
#pragma unroll
                for (int d = 0; d < 4; ++d) keep[m][d] = copy[d % CW];
            } else {
#pragma unroll
                for (int j = 0; j < CE; ++j) {
                    const uint32_t cj = ES == 4 ? copy[j] : (copy[j >> 1] >> (16 * (j & 1))) & 0xffffu;
                    if (cj) { mask_elem<T>(keep[m], 2 * j); mask_elem<T>(keep[m], 2 * j + 1); }
                }
            }
        } else if (a.share_coef) {
            // The four waves of this workgroup hold the same token group and
            // lane mapping (the host guarantees it): each computes every
            // fourth slot, and the values are exchanged through LDS.
            __shared__ float lds_c[CE * 64], lds_s[CE * 64];
#pragma unroll
            for (int j = 0; j < CE; ++j) {
                if (j % kWavesPerBlock != wave_in_block) continue;
                float c, s;
                onthefly_coef<T>(a.inv_freq[slot0[m] + j], pos[m][0], a.scaling, c, s);
                lds_c[j * 64 + lane] = c;
                lds_s[j * 64 + lane] = s;
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < CE; ++j) {
                cf[m][j] = from_f<T>(lds_c[j * 64 + lane]);
                sf[m][j] = from_f<T>(lds_s[j * 64 + lane]);
            }
            __syncthreads();  // the next item reuses the buffers
        } else {
#pragma unroll
            for (int j = 0; j < CE; ++j) {
                float c, s;
                onthefly_coef<T>(a.inv_freq[slot0[m] + j], pos[m][0], a.scaling, c, s);
                cf[m][j] = from_f<T>(c);
                sf[m][j] = from_f<T>(s);
            }
        }
    }

    // QK-norm (one item per lane): the weights of the item's elements, and
    // per slot the weights folded into the coefficients, so that per head
    // y1 = (1/rms) * (x1*(w1*c) - x2*(w2*s)), y2 = (1/rms) * (x2*(w2*c) + x1*(w1*s))
    float gw1[NORM ? E : 1], gw2[NORM ? E : 1];
    float fa1[NORM ? E : 1], fb1[NORM ? E : 1], fa2[NORM ? E : 1], fb2[NORM ? E : 1];
    bool kany = false;  // some lane of the wave keeps input bits (pairs or a copied task)
    // a copied task (V of the cache append, the only norm launch that has
    // one) is never normalised; elsewhere the decision is compile-time
    const bool norm = NORM && (COEF != kCoefAppend || !tk.copy);
    if (norm) {
        const auto w1 = chunk_values<T>(load16_global(tk.wgt + elem0[0] * ES));
        const auto w2 = chunk_values<T>(load16_global(tk.wgt + (elem0[0] + (rot[0] && !IL ? a.P : 0)) * ES));
#pragma unroll
        for (int e = 0; e < E; ++e) { gw1[e] = to_f(w1[e]); gw2[e] = to_f(w2[e]); }
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const int j = IL ? e / 2 : e;
            const float c = to_f(cf[0][j]), s = to_f(sf[0][j]);
            // split halves: element e pairs with its partner chunk's element e;
            // interleaved: elements 2j and 2j+1 of this chunk
            const float wa = IL ? gw1[2 * j] : gw1[e];
            const float wb = IL ? gw1[2 * j + 1] : gw2[e];
            fa1[e] = wa * c;
            fb1[e] = wb * s;
            fa2[e] = wb * c;
            fb2[e] = wa * s;
        }
        if (COEF == kCoefGather || COEF == kCoefAppend) kany = __ballot(keep[0][0] != 0u) != 0;
    } else if (COEF == kCoefGather || COEF == kCoefMrope || COEF == kCoefAppend) {
        // some lane of the wave keeps an element: only then merge input bits
        bool k = tk.copy != 0;
#pragma unroll
        for (int m = 0; m < IPL; ++m) k = k || (keep[m][0] | keep[m][1] | keep[m][2] | keep[m][3]) != 0u;
        kany = __ballot(k) != 0;
    }

    // -- rotate and store, one head batch at a time --------------------------
    if (kPipe) {
        // interleaved pairs only: whole pairs inside each item, no partner chunk
        auto store_batch = [&](int h, u32x4 (&b1)[HU][IPL]) {
#pragma unroll
            for (int u = 0; u < HU; ++u) {
#pragma unroll
                for (int m = 0; m < IPL; ++m) {
                    if (!(wr[m] && h + u < h_end)) continue;
                    char* py = tk.y + yoff[m] + (int64_t)(h + u) * ysh_bytes;
                    if (!rot[m]) {
                        store_nt(py, b1[u][m]);
                        continue;
                    }
                    const auto xv = chunk_values<T>(b1[u][m]);
                    float r[E];
#pragma unroll
                    for (int j = 0; j < CE; ++j) {
                        const float x1 = to_f(xv[2 * j]);
                        const float x2 = to_f(xv[2 * j + 1]);
                        const float c = to_f(cf[m][j]), s = to_f(sf[m][j]);
                        r[2 * j] = rot_out<T>(x1, c, x2, -s);
                        r[2 * j + 1] = rot_out<T>(x2, c, x1, s);
                    }
                    u32x4 o = chunk_pack<T>(r);
                    if ((COEF == kCoefGather || COEF == kCoefMrope || COEF == kCoefAppend || tk.copy) && kany)
                        o = select_bits(keep[m], b1[u][m], o);
                    store_nt(py, o);
                }
            }
        };
        // At most kVecMaxHeads / HU batches per wave (the planner keeps these
        // instances' head chunks within kVecMaxHeads heads), written out step
        // by step: buffers in1 and nx1 hold batches in turn (a copy between
        // them would wait for the loads), and each step's stores appear on
        // both sides of the test for a next batch, so that no branch merges
        // between a prefetch and the stores it overlaps.
        constexpr int kMaxBatches = kVecMaxHeads / HU;
        static_assert(kMaxBatches >= 1 && kMaxBatches <= 8, "head batches per wave");
        u32x4 nx1[HU][IPL], nx2[HU][IPL];
        int h = h_begin;
#define ROPE_PIPE_STEP(K, C1, N1, N2)                                                                   \
        if ((K) < kMaxBatches) {                                                                        \
            if ((K) + 1 < kMaxBatches && h + HU < h_end) {                                              \
                load_batch_all<T, IL, IPL, HU>(tk.x, off, rot, h + HU, h_end, sh_bytes, half_bytes, N1, N2); \
                store_batch(h, C1);                                                                     \
                h += HU;                                                                                \
            } else {                                                                                    \
                store_batch(h, C1);                                                                     \
                return;                                                                                 \
            }                                                                                           \
        }
        ROPE_PIPE_STEP(0, in1, nx1, nx2)
        ROPE_PIPE_STEP(1, nx1, in1, in2)
        ROPE_PIPE_STEP(2, in1, nx1, nx2)
        ROPE_PIPE_STEP(3, nx1, in1, in2)
        ROPE_PIPE_STEP(4, in1, nx1, nx2)
        ROPE_PIPE_STEP(5, nx1, in1, in2)
        ROPE_PIPE_STEP(6, in1, nx1, nx2)
        ROPE_PIPE_STEP(7, nx1, in1, in2)
#undef ROPE_PIPE_STEP
        return;
    }
    for (int h = h_begin; h < h_end; h += HU) {
        if (norm) {
            // RMSNorm of each head row first: the lane's sum of squares, summed
            // over the row's W lanes (an aligned group: W divides 64), then
            // z = (x / rms) * weight, rotated like x; kept pairs and tail
            // items store z
            float rn[HU];
#pragma unroll
            for (int u = 0; u < HU; ++u) {
                float ss = 0.0f;
                if (act[0] && h + u < h_end) {
                    const auto v1 = chunk_values<T>(in1[u][0]);
#pragma unroll
                    for (int e = 0; e < E; ++e) ss = fmaf(to_f(v1[e]), to_f(v1[e]), ss);
                    if (!IL && rot[0]) {
                        const auto v2 = chunk_values<T>(in2[u][0]);
#pragma unroll
                        for (int e = 0; e < E; ++e) ss = fmaf(to_f(v2[e]), to_f(v2[e]), ss);
                    }
                }
                ss = group_sum(ss, a.W);
                rn[u] = rsqrtf(ss * a.inv_d + a.eps);  // v_rsq_f32: about 1 ulp
            }
#pragma unroll
            for (int u = 0; u < HU; ++u) {
                if (!(wr[0] && h + u < h_end)) continue;
                char* py = tk.y + yoff[0] + (int64_t)(h + u) * ysh_bytes;
                const float r = rn[u];
                const auto xv1 = chunk_values<T>(in1[u][0]);
                if (!rot[0]) {
                    float z[E];
#pragma unroll
                    for (int e = 0; e < E; ++e) z[e] = (to_f(xv1[e]) * r) * gw1[e];
                    store_nt(py, chunk_pack<T>(z));
                    continue;
                }
                if (IL) {
                    float o[E];
#pragma unroll
                    for (int j = 0; j < CE; ++j) {
                        const float x1 = to_f(xv1[2 * j]), x2 = to_f(xv1[2 * j + 1]);
                        o[2 * j] = r * fmaf(x1, fa1[2 * j], -(x2 * fb1[2 * j]));
                        o[2 * j + 1] = r * fmaf(x2, fa2[2 * j], x1 * fb2[2 * j]);
                    }
                    u32x4 ov = chunk_pack<T>(o);
                    if ((COEF == kCoefGather || COEF == kCoefAppend) && kany) {
                        float z[E];
#pragma unroll
                        for (int e = 0; e < E; ++e) z[e] = (to_f(xv1[e]) * r) * gw1[e];
                        ov = select_bits(keep[0], chunk_pack<T>(z), ov);
                    }
                    store_nt(py, ov);
                } else {
                    const auto xv2 = chunk_values<T>(in2[u][0]);
                    float o1[E], o2[E];
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const float x1 = to_f(xv1[e]), x2 = to_f(xv2[e]);
                        o1[e] = r * fmaf(x1, fa1[e], -(x2 * fb1[e]));
                        o2[e] = r * fmaf(x2, fa2[e], x1 * fb2[e]);
                    }
                    u32x4 ov1 = chunk_pack<T>(o1);
                    u32x4 ov2 = chunk_pack<T>(o2);
                    if ((COEF == kCoefGather || COEF == kCoefAppend) && kany) {
                        float z1[E], z2[E];
#pragma unroll
                        for (int e = 0; e < E; ++e) {
                            z1[e] = (to_f(xv1[e]) * r) * gw1[e];
                            z2[e] = (to_f(xv2[e]) * r) * gw2[e];
                        }
                        ov1 = select_bits(keep[0], chunk_pack<T>(z1), ov1);
                        ov2 = select_bits(keep[0], chunk_pack<T>(z2), ov2);
                    }
                    store_nt(py, ov1);
                    store_nt(py + half_bytes, ov2);
                }
            }
            if (h + HU < h_end)
                load_batch<T, IL, IPL, HU>(tk.x, off, act, rot, h + HU, h_end, sh_bytes, half_bytes, in1, in2);
            continue;
        }
#pragma unroll
        for (int u = 0; u < HU; ++u) {
#pragma unroll
            for (int m = 0; m < IPL; ++m) {
                if (!(wr[m] && h + u < h_end)) continue;
                char* py = tk.y + yoff[m] + (int64_t)(h + u) * ysh_bytes;
                if (!rot[m]) {
                    store_nt(py, in1[u][m]);
                    continue;
                }
                if (NT == 3 && tk.copy) {  // a pass-through task (V): its chunks as loaded
                    store_nt(py, in1[u][m]);
                    if (!IL) store_nt(py + half_bytes, in2[u][m]);
                    continue;
                }
                if (IL) {
                    const auto xv = chunk_values<T>(in1[u][m]);
                    float r[E];
#pragma unroll
                    for (int j = 0; j < CE; ++j) {
                        const float x1 = to_f(xv[2 * j]);
                        const float x2 = to_f(xv[2 * j + 1]);
                        const float c = to_f(cf[m][j]), s = to_f(sf[m][j]);
                        r[2 * j] = rot_out<T>(x1, c, x2, -s);
                        r[2 * j + 1] = rot_out<T>(x2, c, x1, s);
                    }
                    u32x4 o = chunk_pack<T>(r);
                    if ((COEF == kCoefGather || COEF == kCoefMrope || COEF == kCoefAppend || tk.copy) && kany)
                        o = select_bits(keep[m], in1[u][m], o);
                    store_nt(py, o);
                } else {
                    const auto xv1 = chunk_values<T>(in1[u][m]);
                    const auto xv2 = chunk_values<T>(in2[u][m]);
                    float r1[E], r2[E];
#pragma unroll
                    for (int j = 0; j < E; ++j) {
                        const float x1 = to_f(xv1[j]);
                        const float x2 = to_f(xv2[j]);
                        const float c = to_f(cf[m][j]), s = to_f(sf[m][j]);
                        r1[j] = rot_out<T>(x1, c, x2, -s);
                        r2[j] = rot_out<T>(x2, c, x1, s);
                    }
                    u32x4 o1 = chunk_pack<T>(r1);
                    u32x4 o2 = chunk_pack<T>(r2);
                    if ((COEF == kCoefGather || COEF == kCoefMrope || COEF == kCoefAppend || tk.copy) && kany) {
                        o1 = select_bits(keep[m], in1[u][m], o1);
                        o2 = select_bits(keep[m], in2[u][m], o2);
                    }
                    store_nt(py, o1);
                    store_nt(py + half_bytes, o2);
                }
            }
        }
        if (h + HU < h_end)
            load_batch<T, IL, IPL, HU>(tk.x, off, act, rot, h + HU, h_end, sh_bytes, half_bytes, in1, in2);
    }
}

// ---------------------------------------------------------------------------
// Row kernel, for head rows of 32 bytes to 1 KiB, coefficients gathered by
// id, per token, M-RoPE-assembled, on the fly or at the cache-append
// position; the planner uses it for decode-sized launches and for larger ones
// whose rows the vector kernel's items fit poorly. The lanes of a
// wave hold consecutive 16-byte chunks of consecutive head rows of one
// token: lane l has chunk l % row_lanes of head l / row_lanes, and load u of
// the wave covers the next 64 / row_lanes heads (with a token's heads
// adjacent, 1 KiB of contiguous memory per instruction). A wave covers up to
// kRowLoads instructions (hpw heads) of one token, so the position, its bound
// check and each lane's coefficient slice are the same for all of them: the
// dependence chain of a wave is one scalar position load and one slice
// gather, which is what makes small launches shorter than with the vector
// kernel (whose lanes each hold another token). For large launches it reads
// each token's rows whole, where the vector kernel's items would load
// half-used lines or sparse partner instructions (short, interleaved or
// odd-sized rows); for full split halves of 128 bytes or more the vector
// kernel streams faster.
//   split halves: chunk c < half_lanes holds first elements, its partner
//   (R/2 elements later) is chunk c + half_lanes of the same row, i.e. the
//   lane half_lanes away, fetched by a cross-lane move;
//   interleaved: whole pairs inside the chunk; chunks from the rotated
//   prefix on are copied (or, with the QK-norm, store z).
// Rows of a power-of-two size (GEN = 0) take lane l as chunk l % row_lanes
// of row l / row_lanes by shift and mask, and partners a power of two of
// lanes apart by DPP or an XOR permute. Other rows (GEN = 1: 16-byte chunks,
// row_lanes up to 64; not M-RoPE) take 64 / row_lanes rows per instruction,
// the remaining lanes idle, the row and chunk by a multiply-shift, each
// lane's partner by a permute from lane l +- half_lanes, and the QK-norm's
// sum of squares by a segmented reduction over the row's lanes.
// The chunk of lane (lane ^ d), d a power of two < 64 (uniform): DPP row
// permutes for d = 1, 2, 4, 8 (4: a quad reverse, i -> i ^ 3, then the
// half-row mirror, i -> i ^ 7), a permute through the LDS crossbar for 16 and
// 32. Every lane of the wave takes part.
template <int CTRL>
__device__ inline uint32_t dpp_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, false);
}

__device__ inline u32x4 chunk_xor(const u32x4& v, int d) {
    u32x4 r;
    switch (d) {
        case 1:
#pragma unroll
            for (int k = 0; k < 4; ++k) r[k] = dpp_u32<0xb1>(v[k]);
            break;
        case 2:
#pragma unroll
            for (int k = 0; k < 4; ++k) r[k] = dpp_u32<0x4e>(v[k]);
            break;
        case 4:
#pragma unroll
            for (int k = 0; k < 4; ++k) r[k] = dpp_u32<0x141>(dpp_u32<0x1b>(v[k]));
            break;
        case 8:
#pragma unroll
            for (int k = 0; k < 4; ++k) r[k] = dpp_u32<0x128>(v[k]);  // row rotate by 8
            break;
        default:
#pragma unroll
            for (int k = 0; k < 4; ++k) r[k] = (uint32_t)__shfl_xor((int)v[k], d);
            break;
    }
    return r;
}

// The chunk of lane src (any lane of the wave; every lane takes part).
__device__ inline u32x4 chunk_from(const u32x4& v, int src) {
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = (uint32_t)__shfl((int)v[k], src);
    return r;
}

// A wave-uniform 64-bit value placed in scalar registers.
__device__ inline int64_t uniform64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

template <typename T, int IL, int COEF, bool NORM, int NT = kMaxTasks, int GEN = 0>
__global__ __launch_bounds__(kBlock) void rope_row_kernel(const KArgs a) {
    static_assert(!GEN || COEF != kCoefMrope, "rows of other sizes: no M-RoPE");
    constexpr int E = Elem<T>::E;
    constexpr int CE = IL ? E / 2 : E;  // coefficient slots per rotation chunk
    constexpr int ES = (int)sizeof(T);
    typedef T cvec __attribute__((ext_vector_type(CE)));

    const int lane = threadIdx.x & 63;
    const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block;
    const TaskView tk = task_pick<COEF, NORM, NT>(a, gw);
    // 32-bit index arithmetic: the planner keeps the waves and tokens of a
    // row-kernel launch below 2^31
    const uint32_t local = (uint32_t)(gw - tk.wave_begin);
    const uint32_t nw = fast_div(local, tk.chunks_m, tk.chunks_s);  // the token
    const int part = (int)(local - nw * (uint32_t)tk.chunks);
    // Waves past the last token (in the last workgroup) run on a valid token
    // and store nothing: an early exit makes the compiler defer
    // kernel-argument loads behind the branch (measured slower, except for
    // the cache-append kind, which exits)
    const bool live = nw < (uint64_t)a.ntok;
    if (COEF == kCoefAppend && !live) return;
    const uint32_t n32 = live ? nw : (uint32_t)(a.ntok - 1);
    // head rows per instruction; the lane's row and chunk (GEN: lanes past
    // the last whole row idle)
    const int rpi = GEN ? a.row_rpi : 64 >> a.row_shift;
    const int hi = GEN ? (int)(((uint32_t)lane * a.row_m) >> 16) : lane >> a.row_shift;
    const int c = GEN ? lane - hi * a.row_lanes : lane & (a.row_lanes - 1);
    const bool lane_ok = !GEN || hi < rpi;
    const int h0 = part * tk.hpw;
    const int nh = min(tk.heads - h0, tk.hpw);
    const uint32_t b32 = fast_div(n32, a.s_m, a.s_s);
    const int64_t n = n32;
    const int64_t b = b32;
    const int64_t s = (int64_t)(n32 - b32 * (uint32_t)a.S);

    // the position (wave-uniform: scalar loads through the scalar data cache,
    // read-only), then X, then the coefficient slice
    typedef const __attribute__((address_space(4))) int64_t* const_i64;
    typedef const __attribute__((address_space(4))) int32_t* const_i32;
    bool valid = true;   // the coefficient row exists (else the pairs are copied)
    int64_t row = 0;     // coefficient row
    int64_t pos = 0;     // on the fly: the position
    int64_t yrow = s;    // output row: the cache row of the append kind's K and V
    if (COEF == kCoefGather || COEF == kCoefOnTheFly) {
        pos = ((const_i64)a.ids)[n];
        valid = COEF == kCoefOnTheFly || (pos >= 0 && pos < a.M);
        row = valid ? pos : 0;
    } else if (COEF == kCoefPerToken) {
        row = n;
    } else if (COEF == kCoefMrope) {
        // the three streams' positions; bound checks per slot below
    } else if (COEF == kCoefAppend) {
        const int64_t past = a.prompt ? 0 : (int64_t)((const_i32)a.seqlens)[b] - a.S;
        pos = past + s;
        valid = pos >= 0 && pos < a.M;
        row = valid ? pos : 0;
        if (tk.yrow) {
            if (pos < 0 || pos >= a.rows_out) return;  // no such cache row
            yrow = pos;
        }
    }
    int64_t mpos[COEF == kCoefMrope ? 3 : 1];
    if (COEF == kCoefMrope) {
#pragma unroll
        for (int k = 0; k < 3; ++k) mpos[k] = ((const_i64)a.ids)[k * a.ntok + n];
    }
    const char* px = tk.x + (b * tk.sb + s * tk.ss + (int64_t)(h0 + hi) * tk.sh) * ES + c * 16;
    char* py = tk.y + (b * tk.ysb + yrow * tk.yss + (int64_t)(h0 + hi) * tk.ysh) * ES + c * 16;
    const int64_t xstep = (int64_t)rpi * tk.sh * ES;
    const int64_t ystep = (int64_t)rpi * tk.ysh * ES;

    // on the fly: this lane's inv_freq values (slots lane, lane + 64, ...)
    // are requested before X, so that the slot computation can start while
    // the X loads are in flight (loads complete in issue order)
    constexpr int kOtf = COEF == kCoefOnTheFly ? kRowMaxSlots / 64 : 1;
    float invf[kOtf];
#pragma unroll
    for (int k = 0; k < kOtf; ++k) {
        invf[k] = 0.0f;
        if (COEF == kCoefOnTheFly && lane + 64 * k < a.P) invf[k] = a.inv_freq[lane + 64 * k];
    }

    u32x4 in[kRowLoads];
#pragma unroll
    for (int u = 0; u < kRowLoads; ++u) {
        in[u] = u32x4{0u, 0u, 0u, 0u};
        if (lane_ok && u * rpi + hi < nh) in[u] = load_nt(px + u * xstep);
    }

    const bool rotate = valid && !tk.copy;  // wave-uniform
    const bool rotc = c < a.NP;            // a chunk of the rotated prefix
    const int dl = a.half_lanes;
    const bool lower = !IL && c < dl;      // split halves: the first element of its pairs
    const int slot0 = !rotc ? 0 : (IL ? c * CE : (GEN ? (lower ? c : c - dl) : (c & (dl - 1))) * E);
    float cf[CE], sf[CE];  // split halves: sf carries the sign of the lane's half
#pragma unroll
    for (int j = 0; j < CE; ++j) { cf[j] = 1.0f; sf[j] = 0.0f; }
    u32x4 keep = u32x4{0u, 0u, 0u, 0u};  // M-RoPE: chunk bits passed through
    if (COEF == kCoefMrope && rotate) {
        // slot i takes its stream's row (2-bit code per slot); the lane's
        // slice of each of the three rows, then a per-slot select; a stream
        // whose position is out of range passes its slots' pairs through
        const uint32_t codes = a.sel[slot0 >> 4] >> (2 * (slot0 & 15));
        cvec cs[3], sn[3];
        bool ok[3];
        // the three positions are wave-uniform; a text token has them equal,
        // and then one row serves every slot: one gather instead of three
        // (M-RoPE decode 3.45 -> 3.32 us in a graph replay; in the vector
        // kernel, whose lanes hold several tokens, the same test measured no
        // gain for the prefill)
        const bool same = mpos[0] == mpos[1] && mpos[0] == mpos[2];
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            if (k > 0 && same) {
                cs[k] = cs[0];
                sn[k] = sn[0];
                ok[k] = ok[0];
                continue;
            }
            ok[k] = mpos[k] >= 0 && mpos[k] < a.M;
            const int64_t e = ((ok[k] ? mpos[k] : 0) * a.P + slot0) * ES;  // row 0 if out of range
            cs[k] = *reinterpret_cast<const cvec*>(a.cos + e);
            sn[k] = *reinterpret_cast<const cvec*>(a.sin + e);
        }
#pragma unroll
        for (int j = 0; j < CE; ++j) {
            const uint32_t k = (codes >> (2 * j)) & 3u;
            const T cv = k == 0 ? cs[0][j] : (k == 1 ? cs[1][j] : cs[2][j]);
            const T sv = k == 0 ? sn[0][j] : (k == 1 ? sn[1][j] : sn[2][j]);
            const bool okj = k == 0 ? ok[0] : (k == 1 ? ok[1] : ok[2]);
            float c1 = to_f(cv), s1 = to_f(sv);
            if (a.scale != 1.0f) {  // scaled coefficient: binary32 product rounded to T
                c1 = round_to<T>(keep_f32(c1 * a.scale));
                s1 = round_to<T>(keep_f32(s1 * a.scale));
            }
            cf[j] = c1;
            sf[j] = lower ? -s1 : s1;  // y1 = x1*c + x2*(-s)
            if (rotc && !okj) {
                if (IL) {
                    mask_elem<T>(keep, 2 * j);
                    mask_elem<T>(keep, 2 * j + 1);
                } else {
                    mask_elem<T>(keep, j);
                }
            }
        }
    } else if (COEF == kCoefOnTheFly && rotate) {
        // every slot of the token once per wave (lane l computes slots l,
        // l + 64, ...), exchanged through the wave's own LDS rows
        __shared__ float lds_cs[kWavesPerBlock][2][kRowMaxSlots];
        float* wc = lds_cs[wave_in_block][0];
        float* ws = lds_cs[wave_in_block][1];
#pragma unroll
        for (int k = 0; k < kOtf; ++k) {
            const int i = lane + 64 * k;
            if (i >= a.P) break;
            float cv, sv;
            onthefly_coef<T>(invf[k], pos, a.scaling, cv, sv);
            wc[i] = cv;
            ws[i] = sv;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int j = 0; j < CE; ++j) {
            cf[j] = wc[slot0 + j];
            sf[j] = lower ? -ws[slot0 + j] : ws[slot0 + j];  // y1 = x1*c + x2*(-s)
        }
    } else if (rotate) {
        const int64_t e = (row * a.P + slot0) * ES;
        const cvec cv = *reinterpret_cast<const cvec*>(a.cos + e);
        const cvec sv = *reinterpret_cast<const cvec*>(a.sin + e);
#pragma unroll
        for (int j = 0; j < CE; ++j) {
            cf[j] = to_f(cv[j]);
            sf[j] = lower ? -to_f(sv[j]) : to_f(sv[j]);  // y1 = x1*c + x2*(-s)
        }
    }

    // QK-norm: the weights of the lane's chunk and of its partner chunk,
    // folded into the coefficients once: y = (1/rms) * (x*(w*c) +- p*(w'*s))
    float wo[NORM ? E : 1], fa[NORM ? E : 1], fb[NORM ? E : 1];
    const bool norm = NORM && !tk.copy;
    if (norm) {
        const auto w1 = chunk_values<T>(load16_global(tk.wgt + c * 16));
#pragma unroll
        for (int e = 0; e < E; ++e) wo[e] = to_f(w1[e]);
        if (IL) {
#pragma unroll
            for (int j = 0; j < CE; ++j) {
                fa[2 * j] = wo[2 * j] * cf[j];          // w1 c
                fb[2 * j] = wo[2 * j + 1] * sf[j];      // w2 s
                fa[2 * j + 1] = wo[2 * j + 1] * cf[j];  // w2 c
                fb[2 * j + 1] = wo[2 * j] * sf[j];      // w1 s
            }
        } else {
            const int cp = rotc ? (GEN ? (lower ? c + dl : c - dl) : (c ^ dl)) : c;
            const auto w2 = chunk_values<T>(load16_global(tk.wgt + cp * 16));
#pragma unroll
            for (int e = 0; e < E; ++e) {
                fa[e] = wo[e] * cf[e];
                fb[e] = to_f(w2[e]) * sf[e];  // the sign of the lane's half is in sf
            }
        }
    }

#pragma unroll
    for (int u = 0; u < kRowLoads; ++u) {
        if (u * rpi >= nh) break;
        const bool act = lane_ok && u * rpi + hi < nh;
        // split halves: the partner chunk
        u32x4 pv = in[u];
        if (!IL && rotate)
            pv = GEN ? chunk_from(in[u], rotc && lane_ok ? (lower ? lane + dl : lane - dl) : lane) : chunk_xor(in[u], dl);
        u32x4 o = in[u];
        const auto xv = chunk_values<T>(in[u]);
        const auto pvv = chunk_values<T>(pv);
        if (norm) {
            float ss = 0.0f;
#pragma unroll
            for (int e = 0; e < E; ++e) ss = fmaf(to_f(xv[e]), to_f(xv[e]), ss);
            ss = GEN ? row_sum(ss, c, a.row_lanes, hi * a.row_lanes) : group_sum(ss, a.row_lanes);
            const float r = rsqrtf(ss * a.inv_d + a.eps);  // v_rsq_f32: about 1 ulp
            float z[E];
            if (rotate && rotc) {
                if (IL) {
#pragma unroll
                    for (int j = 0; j < CE; ++j) {
                        const float x1 = to_f(xv[2 * j]), x2 = to_f(xv[2 * j + 1]);
                        z[2 * j] = r * fmaf(x1, fa[2 * j], -(x2 * fb[2 * j]));
                        z[2 * j + 1] = r * fmaf(x2, fa[2 * j + 1], x1 * fb[2 * j + 1]);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) z[e] = r * fmaf(to_f(xv[e]), fa[e], to_f(pvv[e]) * fb[e]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) z[e] = (to_f(xv[e]) * r) * wo[e];
            }
            o = chunk_pack<T>(z);
        } else if (rotate && rotc) {
            float y[E];
            if (IL) {
#pragma unroll
                for (int j = 0; j < CE; ++j) {
                    const float x1 = to_f(xv[2 * j]), x2 = to_f(xv[2 * j + 1]);
                    y[2 * j] = rot_out<T>(x1, cf[j], x2, -sf[j]);
                    y[2 * j + 1] = rot_out<T>(x2, cf[j], x1, sf[j]);
                }
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) y[e] = rot_out<T>(to_f(xv[e]), cf[e], to_f(pvv[e]), sf[e]);
            }
            o = chunk_pack<T>(y);
            if (COEF == kCoefMrope) o = select_bits(keep, in[u], o);
        }
        if (act && live) store_nt(py + u * ystep, o);
    }
}

// ---------------------------------------------------------------------------
// Row kernel, element-wise pairs: rows of 16-byte chunks (32 bytes to 1 KiB)
// whose pairs do not fall on chunk boundaries, i.e. a rotary_embedding_dim
// whose half (split halves) or whole (interleaved pairs) is not a multiple of
// the elements of a chunk (GPT-NeoX-style partial rotations such as 24 of 96
// or 20 of 80 dimensions). Lanes, waves and memory order as in the row
// kernel's general rows (lane l: chunk l % row_lanes of row l / row_lanes,
// 64 / row_lanes rows per instruction, whole chunks loaded and stored); each
// wave puts its token's coefficient slots and, per instruction, its chunks in
// its own LDS, and every element reads its partner element and its slot's
// coefficients there. Binary32 (binary64 for float32 data) arithmetic as in
// the other kernels; copied elements keep their bits. No QK-norm, no M-RoPE.
template <typename T, int IL, int COEF, int NT>
__global__ __launch_bounds__(kBlock) void rope_row_elem_kernel(const KArgs a) {
    constexpr int kElemLoads = kRowElemLoads;  // instructions per wave (their chunks all in LDS)
    static_assert(COEF != kCoefMrope, "element-wise pairs: no M-RoPE");
    constexpr int E = Elem<T>::E;
    constexpr int ES = (int)sizeof(T);

    const int lane = threadIdx.x & 63;
    const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t gw = (int64_t)blockIdx.x * kWavesPerBlock + wave_in_block;
    const TaskView tk = task_pick<COEF, false, NT>(a, gw);
    const uint32_t local = (uint32_t)(gw - tk.wave_begin);
    const uint32_t nw = fast_div(local, tk.chunks_m, tk.chunks_s);  // the token
    const int part = (int)(local - nw * (uint32_t)tk.chunks);
    const bool live = nw < (uint64_t)a.ntok;
    if (COEF == kCoefAppend && !live) return;
    const uint32_t n32 = live ? nw : (uint32_t)(a.ntok - 1);
    const int RL = a.row_lanes;
    const int rpi = a.row_rpi;
    const int hi = (int)(((uint32_t)lane * a.row_m) >> 16);
    const int c = lane - hi * RL;
    const bool lane_ok = hi < rpi;  // lanes past the last whole row idle
    const int h0 = part * tk.hpw;
    const int nh = min(tk.heads - h0, tk.hpw);
    const uint32_t b32 = fast_div(n32, a.s_m, a.s_s);
    const int64_t n = n32;
    const int64_t b = b32;
    const int64_t s = (int64_t)(n32 - b32 * (uint32_t)a.S);

    typedef const __attribute__((address_space(4))) int64_t* const_i64;
    typedef const __attribute__((address_space(4))) int32_t* const_i32;
    bool valid = true;   // the coefficient row exists (else the pairs are copied)
    int64_t row = 0;     // coefficient row
    int64_t pos = 0;     // on the fly: the position
    int64_t yrow = s;    // output row: the cache row of the append kind's K and V
    if (COEF == kCoefGather || COEF == kCoefOnTheFly) {
        pos = ((const_i64)a.ids)[n];
        valid = COEF == kCoefOnTheFly || (pos >= 0 && pos < a.M);
        row = valid ? pos : 0;
    } else if (COEF == kCoefPerToken) {
        row = n;
    } else if (COEF == kCoefAppend) {
        const int64_t past = a.prompt ? 0 : (int64_t)((const_i32)a.seqlens)[b] - a.S;
        pos = past + s;
        valid = pos >= 0 && pos < a.M;
        row = valid ? pos : 0;
        if (tk.yrow) {
            if (pos < 0 || pos >= a.rows_out) return;  // no such cache row
            yrow = pos;
        }
    }
    const char* px = tk.x + (b * tk.sb + s * tk.ss + (int64_t)(h0 + hi) * tk.sh) * ES + c * 16;
    char* py = tk.y + (b * tk.ysb + yrow * tk.yss + (int64_t)(h0 + hi) * tk.ysh) * ES + c * 16;
    const int64_t xstep = (int64_t)rpi * tk.sh * ES;
    const int64_t ystep = (int64_t)rpi * tk.ysh * ES;

    u32x4 in[kElemLoads];
#pragma unroll
    for (int u = 0; u < kElemLoads; ++u) {
        in[u] = u32x4{0u, 0u, 0u, 0u};
        if (lane_ok && u * rpi + hi < nh) in[u] = load_nt(px + u * xstep);
    }

    // the token's coefficient slots (binary32 values of T), slot i in lane
    // i % 64, and the wave's chunks, all in the wave's own LDS rows; one wave
    // barrier (no workgroup barrier) before any element reads them
    __shared__ float lds_cs[kWavesPerBlock][2][kRowMaxSlots];
    __shared__ u32x4 lds_x[kWavesPerBlock][kElemLoads][64];
    float* wc = lds_cs[wave_in_block][0];
    float* ws = lds_cs[wave_in_block][1];
    const int P = a.P;
    const bool rotate = valid && !tk.copy;  // wave-uniform
    if (rotate) {
        for (int i = lane; i < P; i += 64) {
            float cv, sv;
            if (COEF == kCoefOnTheFly) {
                onthefly_coef<T>(a.inv_freq[i], pos, a.scaling, cv, sv);
            } else {
                const int64_t e = row * P + i;
                cv = to_f(reinterpret_cast<const T*>(a.cos)[e]);
                sv = to_f(reinterpret_cast<const T*>(a.sin)[e]);
            }
            wc[i] = cv;
            ws[i] = sv;
        }
#pragma unroll
        for (int u = 0; u < kElemLoads; ++u)
            if (u * rpi < nh) lds_x[wave_in_block][u][lane] = in[u];
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // lanes holding rotated elements (the rest copy their chunks); a lane's
    // coefficients, signs and partner offsets are the same for every row of
    // the token, so they are read once
    const bool rot_lane = rotate && lane_ok && c * E < a.R;
    float cf[E], sf[E];
    int pd[E];
    u32x4 keep = u32x4{0u, 0u, 0u, 0u};  // elements copied as they are
#pragma unroll
    for (int j = 0; j < E; ++j) {
        const int d = c * E + j;  // element of the head row
        cf[j] = 1.0f;
        sf[j] = 0.0f;
        pd[j] = 0;
        if (d >= a.R) {
            mask_elem<T>(keep, j);
            continue;
        }
        if (!rot_lane) continue;
        // interleaved: (2i, 2i+1) take slot i; split halves: (i, i+P)
        const bool first = IL ? (d & 1) == 0 : d < P;
        const int slot = IL ? (d >> 1) : (first ? d : d - P);
        pd[j] = IL ? (d ^ 1) : (first ? d + P : d - P);
        cf[j] = wc[slot];
        sf[j] = first ? -ws[slot] : ws[slot];
    }
#pragma unroll
    for (int u = 0; u < kElemLoads; ++u) {
        if (u * rpi >= nh) break;
        const bool act = lane_ok && u * rpi + hi < nh;
        u32x4 o = in[u];
        if (rot_lane) {
            const T* xrow = reinterpret_cast<const T*>(&lds_x[wave_in_block][u][hi * RL]);
            const auto xv = chunk_values<T>(in[u]);
            float y[E];
#pragma unroll
            for (int j = 0; j < E; ++j) y[j] = rot_out<T>(to_f(xv[j]), cf[j], to_f(xrow[pd[j]]), sf[j]);
            o = select_bits(keep, in[u], chunk_pack<T>(y));
        }
        if (act && live) store_nt(py + u * ystep, o);
    }
}

// ---------------------------------------------------------------------------
// Scalar kernel: one thread per (token, head, k), k < R/2 a pair, k >= R/2 a
// tail element R + k - R/2. Any head size, rotary dim and alignment.
template <typename T, int COEF>
__global__ __launch_bounds__(kBlock) void rope_scalar_kernel(const KArgs a, int64_t total) {
    using B = typename Elem<T>::bits;
    const int64_t K = a.P + (a.D - a.R);
    for (int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * kBlock) {
        const TaskView tk = task_of<COEF>(a, task_index_items(a, idx));
        const int64_t local = idx - tk.item_begin;
        const int64_t k = local % K;
        const int64_t rest = local / K;
        const int64_t h = rest % tk.heads;
        const int64_t n = rest / tk.heads;
        const int64_t b = n / a.S;
        const int64_t s = n - b * a.S;
        const int64_t base = b * tk.sb + h * tk.sh + s * tk.ss;
        int64_t ybase = base;
        if (COEF == kCoefAppend) {
            const int64_t row = tk.yrow ? append_position(a, n) : s;
            if (tk.yrow && (row < 0 || row >= a.rows_out)) continue;  // no such cache row
            ybase = b * tk.ysb + h * tk.ysh + row * tk.yss;
        }
        const B* xb = reinterpret_cast<const B*>(tk.x) + base;
        B* yb = reinterpret_cast<B*>(tk.y) + ybase;
        if (k >= a.P) {
            const int64_t j = a.R + (k - a.P);
            yb[j] = xb[j];
            continue;
        }
        const int i = (int)k;
        const int64_t j1 = a.interleaved ? 2 * (int64_t)i : i;
        const int64_t j2 = a.interleaved ? 2 * (int64_t)i + 1 : (int64_t)i + a.P;
        float c = 1.0f, sn = 0.0f;
        bool copy = tk.copy != 0;
        if (!copy) coef_slot<T, COEF>(a, n, i, c, sn, copy);
        if (copy) {
            yb[j1] = xb[j1];
            yb[j2] = xb[j2];
            continue;
        }
        const float x1 = to_f(__builtin_bit_cast(T, xb[j1]));
        const float x2 = to_f(__builtin_bit_cast(T, xb[j2]));
        yb[j1] = __builtin_bit_cast(B, from_f<T>(rot_out<T>(x1, c, x2, -sn)));
        yb[j2] = __builtin_bit_cast(B, from_f<T>(rot_out<T>(x2, c, x1, sn)));
    }
}

// Scalar QK-norm kernel: one thread per (task, token, head) row -- the sum
// of squares over the row, then every pair rotated from z = (x / rms) * w
// and every tail element stored as z. Any head size and alignment.
template <typename T, int COEF>
__global__ __launch_bounds__(kBlock) void rope_norm_row_kernel(const KArgs a, int64_t total) {
    using B = typename Elem<T>::bits;
    for (int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * kBlock) {
        const TaskView tk = task_of<COEF, true>(a, task_index_items(a, idx));
        const int64_t local = idx - tk.item_begin;
        const int64_t h = local % tk.heads;
        const int64_t n = local / tk.heads;
        const int64_t b = n / a.S;
        const int64_t s = n - b * a.S;
        const int64_t base = b * tk.sb + h * tk.sh + s * tk.ss;
        int64_t ybase = base;
        if (COEF == kCoefAppend) {
            const int64_t row = tk.yrow ? append_position(a, n) : s;
            if (tk.yrow && (row < 0 || row >= a.rows_out)) continue;  // no such cache row
            ybase = b * tk.ysb + h * tk.ysh + row * tk.yss;
        }
        const B* xb = reinterpret_cast<const B*>(tk.x) + base;
        B* yb = reinterpret_cast<B*>(tk.y) + ybase;
        if (tk.copy) {  // a copied task (V of the cache append): bits as they are
            for (int j = 0; j < a.D; ++j) yb[j] = xb[j];
            continue;
        }
        const B* wb = reinterpret_cast<const B*>(tk.wgt);
        // the sum of squares in binary64 (one long sequential sum here)
        double ss = 0.0;
        for (int j = 0; j < a.D; ++j) {
            const double v = to_f(__builtin_bit_cast(T, xb[j]));
            ss = fma(v, v, ss);
        }
        const float rn = 1.0f / sqrtf((float)(ss / (double)a.D) + a.eps);
        for (int i = 0; i < a.P; ++i) {
            const int j1 = a.interleaved ? 2 * i : i;
            const int j2 = a.interleaved ? 2 * i + 1 : i + a.P;
            const float z1 = (to_f(__builtin_bit_cast(T, xb[j1])) * rn) * to_f(__builtin_bit_cast(T, wb[j1]));
            const float z2 = (to_f(__builtin_bit_cast(T, xb[j2])) * rn) * to_f(__builtin_bit_cast(T, wb[j2]));
            float c = 1.0f, sn = 0.0f;
            bool copy = false;
            coef_slot<T, COEF>(a, n, i, c, sn, copy);
            if (copy) {
                yb[j1] = __builtin_bit_cast(B, from_f<T>(z1));
                yb[j2] = __builtin_bit_cast(B, from_f<T>(z2));
                continue;
            }
            yb[j1] = __builtin_bit_cast(B, from_f<T>(fmaf(z1, c, -(z2 * sn))));
            yb[j2] = __builtin_bit_cast(B, from_f<T>(fmaf(z2, c, z1 * sn)));
        }
        for (int j = a.R; j < a.D; ++j) {
            const float z = (to_f(__builtin_bit_cast(T, xb[j])) * rn) * to_f(__builtin_bit_cast(T, wb[j]));
            yb[j] = __builtin_bit_cast(B, from_f<T>(z));
        }
    }
}

// ---------------------------------------------------------------------------
// Table builders.


template <typename T>
__global__ __launch_bounds__(kBlock) void table_kernel(const float* inv_freq, T* cos_out, T* sin_out,
                                                       int64_t rows, int64_t half, float scaling) {
    const int64_t total = rows * half;
    for (int64_t idx = (int64_t)blockIdx.x * kBlock + threadIdx.x; idx < total;
         idx += (int64_t)gridDim.x * kBlock) {
        const int64_t p = idx / half;
        const int64_t i = idx - p * half;
        float c, s;
        onthefly_coef<T>(inv_freq[i], p, scaling, c, s);
        cos_out[idx] = from_f<T>(c);
        sin_out[idx] = from_f<T>(s);
    }
}

// ---------------------------------------------------------------------------
// Launch.

inline int launched(hipError_t e) {
    if (e != hipSuccess)
        return fail(ROPE_ERR_LAUNCH, "kernel launch failed: %s", hipGetErrorString(e));
    return ROPE_OK;
}

// Instantiated (items per lane, head batch) pairs; the planner picks one.
template <typename T, int IL, int COEF, int NT>
inline hipError_t launch_vec_ipl(const KArgs& a, int ipl, int hu, dim3 grid, hipStream_t st) {
    void* args[] = {const_cast<KArgs*>(&a)};
    const void* fn;
#define ROPE_VEC(I, H) (const void*)rope_vec_kernel<T, IL, COEF, I, H, false, NT>
    switch (ipl * 16 + hu) {
        case 1 * 16 + 2: fn = ROPE_VEC(1, 2); break;
        case 1 * 16 + 4: fn = ROPE_VEC(1, 4); break;
        case 1 * 16 + 8: fn = ROPE_VEC(1, 8); break;
        case 2 * 16 + 2: fn = ROPE_VEC(2, 2); break;
        case 2 * 16 + 4: fn = ROPE_VEC(2, 4); break;
        case 2 * 16 + 8: fn = ROPE_VEC(2, 8); break;
        case 3 * 16 + 2: fn = ROPE_VEC(3, 2); break;
        case 3 * 16 + 4: fn = ROPE_VEC(3, 4); break;
        case 4 * 16 + 2: fn = ROPE_VEC(4, 2); break;
        case 4 * 16 + 4: fn = ROPE_VEC(4, 4); break;
        default: return hipErrorInvalidValue;
    }
#undef ROPE_VEC
    return hipLaunchKernel(fn, grid, dim3(kBlock), args, 0, st);
}

template <typename T, int IL, int COEF>
inline hipError_t launch_vec_nt(const KArgs& a, int ipl, int hu, dim3 grid, hipStream_t st) {
    switch (a.ntask) {
        case 1: return launch_vec_ipl<T, IL, COEF, 1>(a, ipl, hu, grid, st);
        case 2: return launch_vec_ipl<T, IL, COEF, 2>(a, ipl, hu, grid, st);
        case 3: return launch_vec_ipl<T, IL, COEF, 3>(a, ipl, hu, grid, st);
        default: return hipErrorInvalidValue;
    }
}

// QK-norm: one item per lane, any instantiated head batch.
template <typename T, int IL, int COEF>
inline hipError_t launch_vec_norm(const KArgs& a, int hu, dim3 grid, hipStream_t st) {
    // QK-norm launches hold Q and K, the cache append Q, K and V
    constexpr int NT = COEF == kCoefAppend ? 3 : 2;
    if (a.ntask != NT) return hipErrorInvalidValue;
    void* args[] = {const_cast<KArgs*>(&a)};
    const void* fn;
    switch (hu) {
        case 2: fn = (const void*)rope_vec_kernel<T, IL, COEF, 1, 2, true, NT>; break;
        case 4: fn = (const void*)rope_vec_kernel<T, IL, COEF, 1, 4, true, NT>; break;
        case 8: fn = (const void*)rope_vec_kernel<T, IL, COEF, 1, 8, true, NT>; break;
        default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, grid, dim3(kBlock), args, 0, st);
}

template <typename T, int IL>
inline hipError_t launch_vec_coef(const KArgs& a, CoefKind c, int ipl, int hu, dim3 grid,
                                  hipStream_t st, bool norm) {
    if (norm) {
        if (ipl != 1) return hipErrorInvalidValue;
        switch (c) {
            case kCoefGather: return launch_vec_norm<T, IL, kCoefGather>(a, hu, grid, st);
            case kCoefPerToken: return launch_vec_norm<T, IL, kCoefPerToken>(a, hu, grid, st);
            case kCoefOnTheFly: return launch_vec_norm<T, IL, kCoefOnTheFly>(a, hu, grid, st);
            case kCoefAppend: return launch_vec_norm<T, IL, kCoefAppend>(a, hu, grid, st);
            default: return hipErrorInvalidValue;
        }
    }
    switch (c) {
        // M-RoPE launches hold one task, the cache append three (Q, K, V);
        // the others one (RotaryEmbedding), two (Q+K) or three (packed)
        case kCoefGather: return launch_vec_nt<T, IL, kCoefGather>(a, ipl, hu, grid, st);
        case kCoefPerToken: return launch_vec_nt<T, IL, kCoefPerToken>(a, ipl, hu, grid, st);
        case kCoefMrope:
            if (a.ntask != 1) return hipErrorInvalidValue;
            return launch_vec_ipl<T, IL, kCoefMrope, 1>(a, ipl, hu, grid, st);
        case kCoefAppend:
            if (a.ntask != 3) return hipErrorInvalidValue;
            return launch_vec_ipl<T, IL, kCoefAppend, 3>(a, ipl, hu, grid, st);
        default: return launch_vec_nt<T, IL, kCoefOnTheFly>(a, ipl, hu, grid, st);
    }
}

template <typename T, int IL>
inline hipError_t launch_row_il(const KArgs& a, CoefKind c, dim3 grid, hipStream_t st, bool norm, int gen) {
    void* args[] = {const_cast<KArgs*>(&a)};
    const void* fn;
    // QK-norm launches hold Q and K; the cache append Q, K and V; M-RoPE one
    // task; the others one (RotaryEmbedding), two (Q+K) or three (packed).
    // Rows of other sizes (gen): no M-RoPE.
#define ROPE_ROW_NT(K, G)                                                          \
    (a.ntask == 1   ? (const void*)rope_row_kernel<T, IL, K, false, 1, G>          \
     : a.ntask == 2 ? (const void*)rope_row_kernel<T, IL, K, false, 2, G>          \
     : a.ntask == 3 ? (const void*)rope_row_kernel<T, IL, K, false, 3, G>          \
                    : nullptr)
#define ROPE_ROW(K)                                                                         \
    (norm ? (a.ntask != 2 ? nullptr                                                         \
             : gen        ? (const void*)rope_row_kernel<T, IL, K, true, 2, 1>              \
                          : (const void*)rope_row_kernel<T, IL, K, true, 2>)                 \
          : (gen ? ROPE_ROW_NT(K, 1) : ROPE_ROW_NT(K, 0)))
    if (gen == 2) {  // element-wise pairs: no QK-norm, no M-RoPE
        if (norm) return hipErrorInvalidValue;
#define ROPE_ELEM(K)                                                                \
    (a.ntask == 1   ? (const void*)rope_row_elem_kernel<T, IL, K, 1>                \
     : a.ntask == 2 ? (const void*)rope_row_elem_kernel<T, IL, K, 2>                \
     : a.ntask == 3 ? (const void*)rope_row_elem_kernel<T, IL, K, 3>                \
                    : nullptr)
        switch (c) {
            case kCoefGather: fn = ROPE_ELEM(kCoefGather); break;
            case kCoefPerToken: fn = ROPE_ELEM(kCoefPerToken); break;
            case kCoefOnTheFly: fn = ROPE_ELEM(kCoefOnTheFly); break;
            case kCoefAppend:
                if (a.ntask != 3) return hipErrorInvalidValue;
                fn = (const void*)rope_row_elem_kernel<T, IL, kCoefAppend, 3>;
                break;
            default: return hipErrorInvalidValue;
        }
#undef ROPE_ELEM
        if (!fn) return hipErrorInvalidValue;
        return hipLaunchKernel(fn, grid, dim3(kBlock), args, 0, st);
    }
    switch (c) {
        case kCoefGather: fn = ROPE_ROW(kCoefGather); break;
        case kCoefPerToken: fn = ROPE_ROW(kCoefPerToken); break;
        case kCoefOnTheFly: fn = ROPE_ROW(kCoefOnTheFly); break;
        case kCoefAppend:
            if (a.ntask != 3) return hipErrorInvalidValue;
            fn = norm ? (gen ? (const void*)rope_row_kernel<T, IL, kCoefAppend, true, 3, 1>
                             : (const void*)rope_row_kernel<T, IL, kCoefAppend, true, 3>)
                      : (gen ? (const void*)rope_row_kernel<T, IL, kCoefAppend, false, 3, 1>
                             : (const void*)rope_row_kernel<T, IL, kCoefAppend, false, 3>);
            break;
        case kCoefMrope:
            if (norm || gen || a.ntask != 1) return hipErrorInvalidValue;
            fn = (const void*)rope_row_kernel<T, IL, kCoefMrope, false, 1>;
            break;
        default: return hipErrorInvalidValue;
    }
    if (!fn) return hipErrorInvalidValue;
#undef ROPE_ROW
#undef ROPE_ROW_NT
    return hipLaunchKernel(fn, grid, dim3(kBlock), args, 0, st);
}

template <typename T>
inline hipError_t launch_scalar(const KArgs& a, CoefKind c, int64_t total, hipStream_t st, bool norm) {
    int64_t blocks = (total + kBlock - 1) / kBlock;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    void* args[] = {const_cast<KArgs*>(&a), &total};
    const void* fn;
    if (norm) {
        switch (c) {
            case kCoefGather: fn = (const void*)rope_norm_row_kernel<T, kCoefGather>; break;
            case kCoefPerToken: fn = (const void*)rope_norm_row_kernel<T, kCoefPerToken>; break;
            case kCoefOnTheFly: fn = (const void*)rope_norm_row_kernel<T, kCoefOnTheFly>; break;
            case kCoefAppend: fn = (const void*)rope_norm_row_kernel<T, kCoefAppend>; break;
            default: return hipErrorInvalidValue;
        }
        return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kBlock), args, 0, st);
    }
    switch (c) {
        case kCoefGather: fn = (const void*)rope_scalar_kernel<T, kCoefGather>; break;
        case kCoefPerToken: fn = (const void*)rope_scalar_kernel<T, kCoefPerToken>; break;
        case kCoefMrope: fn = (const void*)rope_scalar_kernel<T, kCoefMrope>; break;
        case kCoefAppend: fn = (const void*)rope_scalar_kernel<T, kCoefAppend>; break;
        default: fn = (const void*)rope_scalar_kernel<T, kCoefOnTheFly>; break;
    }
    return hipLaunchKernel(fn, dim3((unsigned)blocks), dim3(kBlock), args, 0, st);
}

// Per storage type entry points of the launch code, instantiated in
// rope_kernels_<type>.hip (one translation unit each, built in parallel).
template <typename T>
hipError_t launch_vector_for(const KArgs& a, CoefKind c, int interleaved, int ipl, int hu, dim3 grid,
                             hipStream_t st, bool norm) {
    return interleaved ? launch_vec_coef<T, 1>(a, c, ipl, hu, grid, st, norm)
                       : launch_vec_coef<T, 0>(a, c, ipl, hu, grid, st, norm);
}

template <typename T>
hipError_t launch_row_for(const KArgs& a, CoefKind c, int interleaved, dim3 grid, hipStream_t st, bool norm,
                          int gen) {
    return interleaved ? launch_row_il<T, 1>(a, c, grid, st, norm, gen)
                       : launch_row_il<T, 0>(a, c, grid, st, norm, gen);
}

template <typename T>
hipError_t launch_scalar_for(const KArgs& a, CoefKind c, int64_t total, hipStream_t st, bool norm) {
    return launch_scalar<T>(a, c, total, st, norm);
}

template <typename T>
hipError_t launch_table_for(const float* inv, void* cos, void* sin, int64_t rows, int64_t half,
                            float scaling, dim3 grid, hipStream_t st) {
    T* c = static_cast<T*>(cos);
    T* s = static_cast<T*>(sin);
    void* args[] = {&inv, &c, &s, &rows, &half, &scaling};
    return hipLaunchKernel((const void*)table_kernel<T>, grid, dim3(kBlock), args, 0, st);
}

#define ROPE_VEC_ENTRY_POINTS(EXT, T)                                                              \
    EXT template hipError_t launch_vector_for<T>(const KArgs&, CoefKind, int, int, int, dim3,      \
                                                 hipStream_t, bool);
#define ROPE_ROW_ENTRY_POINTS(EXT, T)                                                              \
    EXT template hipError_t launch_row_for<T>(const KArgs&, CoefKind, int, dim3, hipStream_t, bool, int); \
    EXT template hipError_t launch_scalar_for<T>(const KArgs&, CoefKind, int64_t, hipStream_t, bool); \
    EXT template hipError_t launch_table_for<T>(const float*, void*, void*, int64_t, int64_t, float, \
                                                dim3, hipStream_t);
#define ROPE_TYPE_ENTRY_POINTS(EXT, T) ROPE_VEC_ENTRY_POINTS(EXT, T) ROPE_ROW_ENTRY_POINTS(EXT, T)
// instantiated elsewhere: every translation unit but its own refers to them
ROPE_TYPE_ENTRY_POINTS(extern, float)
ROPE_TYPE_ENTRY_POINTS(extern, half_t)
ROPE_TYPE_ENTRY_POINTS(extern, bf16_t)

}  // namespace rope
