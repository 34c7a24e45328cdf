// rope_kernels.hip -- launch of a validated plan (the kernels themselves are
// in rope_device.hpp, instantiated per storage type in rope_kernels_<type>.hip).
#include "rope_device.hpp"
#include "rope_launch.hpp"

namespace rope {

// ---------------------------------------------------------------------------
// Table builders.

__global__ __launch_bounds__(kBlock) void inv_freq_kernel(float* out, int64_t half, double base) {
    const int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (i >= half) return;
    out[i] = (float)pow(base, -2.0 * (double)i / (double)(2 * half));
}

// Multiplier and shift for division by d (1 <= d < 2^31) of dividends below
// 2^31, as fast_div in rope_device.hpp uses them.
static void fast_div_magic(int64_t d, uint32_t* m, uint32_t* l) {
    if (d < 1) d = 1;
    uint32_t s = 0;
    while (((int64_t)1 << s) < d) ++s;
    const unsigned __int128 num = ((unsigned __int128)1 << 32) * (unsigned __int128)(((int64_t)1 << s) - d);
    *m = (uint32_t)(num / (unsigned __int128)d + 1);
    *l = s;
}

int launch_plan(const Plan& pl, void* stream) {
    if (pl.empty) return ROPE_OK;
    const Problem& p = pl.p;
    const Geometry& g = pl.g;
    hipStream_t st = (hipStream_t)stream;
    KArgs a = {};
    // scalar work items per (token, head): pairs plus tail elements, or the
    // whole row for the QK-norm kernel
    const int64_t K = p.norm ? 1 : p.R / 2 + (p.D - p.R);
    int64_t wave_begin = 0, item_begin = 0;
    for (int t = 0; t < kMaxTasks; ++t) {
        a.t[t].wave_begin = INT64_MAX;
        a.t[t].item_begin = INT64_MAX;
        a.t[t].chunks = 1;
        a.t[t].tile = 1;
        a.t[t].hpw = 1;
    }
    for (int t = 0; t < p.ntask; ++t) {
        a.t[t].x = (const char*)p.task[t].x;
        a.t[t].y = (char*)p.task[t].y;
        a.t[t].sb = p.task[t].stride_b;
        a.t[t].sh = p.task[t].stride_h;
        a.t[t].ss = p.task[t].stride_s;
        a.t[t].heads = (int32_t)p.task[t].heads;
        a.t[t].copy = p.task[t].copy;
        a.t[t].yrow = p.task[t].yrow;
        a.t[t].ysb = p.task[t].ystride_b;
        a.t[t].ysh = p.task[t].ystride_h;
        a.t[t].yss = p.task[t].ystride_s;
        a.t[t].wgt = (const char*)p.task[t].weight;
        const int64_t items = p.B * p.S * p.task[t].heads * K;
        if (items > 0) {  // an empty task keeps INT64_MAX and is never selected
            a.t[t].item_begin = item_begin;
            item_begin += items;
        }
        if (g.vector) {
            a.t[t].hpw = g.heads_per_wave[t];
            a.t[t].chunks = g.chunks[t] > 0 ? g.chunks[t] : 1;
            a.t[t].tile = g.tile > 0 ? g.tile : 1;
            fast_div_magic(a.t[t].chunks, &a.t[t].chunks_m, &a.t[t].chunks_s);
            fast_div_magic(a.t[t].tile, &a.t[t].tile_m, &a.t[t].tile_s);
            fast_div_magic((int64_t)a.t[t].tile * a.t[t].chunks, &a.t[t].per_tile_m, &a.t[t].per_tile_s);
            if (g.waves[t] > 0) {
                a.t[t].wave_begin = wave_begin;
                wave_begin += g.waves[t];
            }
        }
    }
    a.group_major = 0;
    if (g.vector && !g.row_kernel && g.group_major && p.ntask == 3) {
        a.group_major = 1;
        a.gm_c0 = a.t[0].chunks;
        a.gm_c01 = a.t[0].chunks + a.t[1].chunks;
        a.gm_c = a.gm_c01 + a.t[2].chunks;
        fast_div_magic(a.gm_c, &a.gm_m, &a.gm_s);
    }
    a.ntok = p.B * p.S;
    a.S = p.S;
    a.M = p.M;
    a.cos = (const char*)p.cos;
    a.sin = (const char*)p.sin;
    if (g.vector && p.M == 0 && (p.coef == kCoefGather || p.coef == kCoefMrope)) {
        // empty table: every id is out of range and every pair is copied, but
        // the vector kernel reads a row unconditionally; point it at the
        // first non-empty input (16-byte aligned, at least one row long)
        for (int t = p.ntask - 1; t >= 0; --t)
            if (p.task[t].heads > 0) a.cos = a.sin = (const char*)p.task[t].x;
    }
    a.ids = p.ids;
    a.inv_freq = p.inv_freq;
    a.ntask = p.ntask;
    a.W = g.W;
    a.NP = g.NP;
    a.TG = g.TG;
    a.P = (int32_t)(p.R / 2);
    a.R = (int32_t)p.R;
    a.D = (int32_t)p.D;
    a.interleaved = p.interleaved;
    a.scaling = p.scaling;
    a.scale = p.scale;
    a.eps = p.eps;
    a.share_coef = g.vector && g.share_coef;
    a.row_lanes = g.row_kernel ? g.row_lanes : 1;
    a.row_shift = 0;
    while ((1 << a.row_shift) < a.row_lanes) ++a.row_shift;
    a.half_lanes = g.row_kernel ? g.half_lanes : 0;
    a.row_rpi = 64 / a.row_lanes;
    a.row_m = (uint32_t)((65536 + a.row_lanes - 1) / a.row_lanes);
    fast_div_magic(a.W > 0 ? a.W : 1, &a.w_m, &a.w_s);
    fast_div_magic(a.S > 0 ? a.S : 1, &a.s_m, &a.s_s);
    a.inv_d = 1.0f / (float)p.D;
    a.seqlens = p.seqlens;
    a.prompt = p.prompt;
    a.rows_out = p.rows_out;
    for (int i = 0; i < kSelWords; ++i) a.sel[i] = p.sel[i];
    a.mrope_single = p.mrope_single;

    hipError_t e;
    if (g.vector) {
        const int64_t waves = wave_begin;
        if (waves == 0) return ROPE_OK;
        const int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
        if (blocks > INT32_MAX)  // beyond the grid limit (about 2^39 elements): refuse, never wrap
            return fail(ROPE_ERR_UNSUPPORTED, "launch of %lld workgroups exceeds the grid limit", (long long)blocks);
        const dim3 grid((unsigned)blocks);
        const int ipl = g.items_per_lane;
        const int hu = g.head_batch;
        if (g.row_kernel) {
            const int gen = g.row_general;  // 0, 1 general rows, 2 element-wise pairs
            e = p.dtype == ROPE_FLOAT16    ? launch_row_for<half_t>(a, p.coef, p.interleaved, grid, st, p.norm, gen)
                : p.dtype == ROPE_BFLOAT16 ? launch_row_for<bf16_t>(a, p.coef, p.interleaved, grid, st, p.norm, gen)
                                           : launch_row_for<float>(a, p.coef, p.interleaved, grid, st, p.norm, gen);
        }
        else if (p.dtype == ROPE_FLOAT16)
            e = launch_vector_for<half_t>(a, p.coef, p.interleaved, ipl, hu, grid, st, p.norm);
        else if (p.dtype == ROPE_BFLOAT16)
            e = launch_vector_for<bf16_t>(a, p.coef, p.interleaved, ipl, hu, grid, st, p.norm);
        else
            e = launch_vector_for<float>(a, p.coef, p.interleaved, ipl, hu, grid, st, p.norm);
    } else {
        if (item_begin == 0) return ROPE_OK;
        e = p.dtype == ROPE_FLOAT16    ? launch_scalar_for<half_t>(a, p.coef, item_begin, st, p.norm)
            : p.dtype == ROPE_BFLOAT16 ? launch_scalar_for<bf16_t>(a, p.coef, item_begin, st, p.norm)
                                       : launch_scalar_for<float>(a, p.coef, item_begin, st, p.norm);
    }
    return launched(e);
}

int launch_inv_freq(float* inv_freq, int64_t half, double base, void* stream) {
    if (half == 0) return ROPE_OK;
    void* args[] = {&inv_freq, &half, &base};
    const dim3 grid((unsigned)((half + kBlock - 1) / kBlock));
    return launched(hipLaunchKernel((const void*)inv_freq_kernel, grid, dim3(kBlock), args, 0,
                                    (hipStream_t)stream));
}

int launch_cos_sin_cache(const TablePlan& t, void* stream) {
    const int64_t total = t.rows * t.half;
    if (total == 0) return ROPE_OK;
    int64_t blocks = (total + kBlock - 1) / kBlock;
    if (blocks > 65536) blocks = 65536;
    const dim3 grid((unsigned)blocks);
    hipStream_t st = (hipStream_t)stream;
    const hipError_t e =
        t.dtype == ROPE_FLOAT16    ? launch_table_for<half_t>(t.inv_freq, t.cos, t.sin, t.rows, t.half, t.scaling, grid, st)
        : t.dtype == ROPE_BFLOAT16 ? launch_table_for<bf16_t>(t.inv_freq, t.cos, t.sin, t.rows, t.half, t.scaling, grid, st)
                                   : launch_table_for<float>(t.inv_freq, t.cos, t.sin, t.rows, t.half, t.scaling, grid, st);
    return launched(e);
}

}  // namespace rope
