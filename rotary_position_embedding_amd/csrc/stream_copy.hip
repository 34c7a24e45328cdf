// stream_copy.hip -- plain streaming copies of device memory, no rotation:
// the measuring stick for the rotary kernels' HBM rate. bench.py times them
// on the same number of bytes as a workload's X (read) and Y (written), so
// that a step's rate can be set beside the rate the GPU reaches for a copy of
// that size in the same run. Built into libstream_copy.so, separate from the
// rotary library and its C ABI.
//
// Access patterns (every 16-byte item of the buffer read once and written
// once; loads and stores nontemporal, as in the rotary kernels):
//   1  one 1 KiB run per wave (64 lanes x 16 bytes);
//   2  one 16 KiB run per wave (16 loads per lane, then 16 stores);
//   3  persistent: `blocks` workgroups of 4 waves step through 4 KiB chunks
//      with a stride of the whole grid, the next chunk loaded before the
//      current one is stored;
//   4  the same with 8 KiB chunks.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline u32x4 ld(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ inline void st(u32x4* p, const u32x4& v) { __builtin_nontemporal_store(v, p); }

// One run of NL KiB per wave: every load, then every store.
template <int NL>
__global__ __launch_bounds__(256) void copy_runs(const u32x4* __restrict__ x, u32x4* __restrict__ y, int64_t n16) {
    const int64_t wave = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t base = wave * NL * 64 + (threadIdx.x & 63);
    u32x4 v[NL];
#pragma unroll
    for (int u = 0; u < NL; ++u) {
        const int64_t i = base + (int64_t)u * 64;
        v[u] = i < n16 ? ld(x + i) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < NL; ++u) {
        const int64_t i = base + (int64_t)u * 64;
        if (i < n16) st(y + i, v[u]);
    }
}

// Chunks of NL KiB: wave w takes chunks w, w + G, w + 2G, ... (G waves in the
// grid); the next chunk's loads are issued before the current chunk's stores.
template <int NL>
__global__ __launch_bounds__(256) void copy_persistent(const u32x4* __restrict__ x, u32x4* __restrict__ y,
                                                       int64_t n16) {
    const int64_t G = (int64_t)gridDim.x * 4;
    const int64_t lane = threadIdx.x & 63;
    const int64_t nchunks = (n16 + NL * 64 - 1) / (NL * 64);
    int64_t c = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (c >= nchunks) return;
    u32x4 a[NL], b[NL];
#pragma unroll
    for (int u = 0; u < NL; ++u) {
        const int64_t i = c * NL * 64 + u * 64 + lane;
        a[u] = i < n16 ? ld(x + i) : u32x4{0u, 0u, 0u, 0u};
    }
    while (true) {
        const int64_t cn = c + G;
        const bool more = cn < nchunks;
        if (more) {
#pragma unroll
            for (int u = 0; u < NL; ++u) {
                const int64_t i = cn * NL * 64 + u * 64 + lane;
                b[u] = i < n16 ? ld(x + i) : u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int u = 0; u < NL; ++u) {
            const int64_t i = c * NL * 64 + u * 64 + lane;
            if (i < n16) st(y + i, a[u]);
        }
        if (!more) break;
#pragma unroll
        for (int u = 0; u < NL; ++u) a[u] = b[u];
        c = cn;
    }
}

}  // namespace

extern "C" {

// Copies nbytes from x to y (device pointers, 16-byte aligned, nbytes a
// multiple of 16, no overlap) on `stream` with access pattern 1-4 above;
// `blocks` is the workgroup count of the persistent patterns (1 to 65536).
// Returns 0, -1 for an argument outside those rules (nothing enqueued), or -2
// if the runtime rejects the launch. Enqueues and returns; allocates nothing.
int stream_copy(const void* x, void* y, int64_t nbytes, int pattern, int blocks, void* stream) {
    if (!x || !y || nbytes < 0 || nbytes % 16 != 0) return -1;
    if (((uintptr_t)x | (uintptr_t)y) % 16 != 0) return -1;
    const uintptr_t xa = (uintptr_t)x, ya = (uintptr_t)y;
    if (xa < ya + (uintptr_t)nbytes && ya < xa + (uintptr_t)nbytes && nbytes > 0) return -1;
    if (nbytes == 0) return 0;
    const int64_t n16 = nbytes / 16;
    const u32x4* xs = static_cast<const u32x4*>(x);
    u32x4* ys = static_cast<u32x4*>(y);
    hipStream_t st = static_cast<hipStream_t>(stream);
    auto grid_of = [n16](int64_t per_wave) {
        const int64_t waves = (n16 + per_wave - 1) / per_wave;
        return (waves + 3) / 4;
    };
    int64_t grid;
    switch (pattern) {
        case 1:
            grid = grid_of(64);
            if (grid > INT32_MAX) return -1;
            copy_runs<1><<<dim3((unsigned)grid), dim3(256), 0, st>>>(xs, ys, n16);
            break;
        case 2:
            grid = grid_of(16 * 64);
            if (grid > INT32_MAX) return -1;
            copy_runs<16><<<dim3((unsigned)grid), dim3(256), 0, st>>>(xs, ys, n16);
            break;
        case 3:
            if (blocks < 1 || blocks > 65536) return -1;
            copy_persistent<4><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(xs, ys, n16);
            break;
        case 4:
            if (blocks < 1 || blocks > 65536) return -1;
            copy_persistent<8><<<dim3((unsigned)blocks), dim3(256), 0, st>>>(xs, ys, n16);
            break;
        default:
            return -1;
    }
    return hipGetLastError() == hipSuccess ? 0 : -2;
}

}  // extern "C"
