// Measured ceilings of the resources the walks lean on besides HBM, on gfx950:
// gathers of 64-byte rows (a width-16 float row) from LDS and from L2, global
// and LDS float atomics, and the fixed cost of a launch. Built into
// libvspmm_probe.so, which only the benchmark's ceilings mode loads; the
// product library does not contain or call any of this.
//
// Every gather kernel has the shape of the aligned walk's inner loop: a wave
// loads a window of 64 consecutive row numbers (one per lane, coalesced) and
// then takes 4 steps; in step t the 4 lanes of quad q take the row number held
// by lane 4q + t (a DPP quad broadcast) and each reads one 16-byte piece of
// that row, which it adds into an accumulator.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr int kThreads = 1024;

__device__ __forceinline__ int quad_bcast(int x, int t) {
    switch (t) {
        case 0: return __builtin_amdgcn_mov_dpp(x, 0x00, 0xf, 0xf, false);
        case 1: return __builtin_amdgcn_mov_dpp(x, 0x55, 0xf, 0xf, false);
        case 2: return __builtin_amdgcn_mov_dpp(x, 0xaa, 0xf, 0xf, false);
        default: return __builtin_amdgcn_mov_dpp(x, 0xff, 0xf, 0xf, false);
    }
}

// The window a wave reads in iteration it (windows cycle through idx).
__device__ __forceinline__ const int *window(const int *idx, int n_win, int it) {
    const int wave = (blockIdx.x * (blockDim.x >> 6)) + (threadIdx.x >> 6);
    const int k = (int)(((long long)wave * 7919 + (long long)it * 104729) % n_win);
    return idx + (size_t)k * 64;
}

// LDS gathers. MODE 0: the drawn rows; MODE 1: conflict-free (step t, quad q
// reads row 16t + q + 64 (it mod 16), so a wave reads 16 whole consecutive
// rows; needs n_rows >= 1024); MODE 2: the drawn rows, each 16-byte piece read
// as two 8-byte reads.
template <int MODE>
__global__ void __launch_bounds__(kThreads)
k_lds_gather(const float *table, int n_rows, const int *idx, int n_win, int iters, float *sink) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int lane = threadIdx.x & 63;
    for (int k = threadIdx.x; k < n_rows * 16; k += blockDim.x) lds[k] = table[k];
    __syncthreads();
    const uint32_t coff = (uint32_t)(lane & 3) * 16u;
    float a0 = 0, a1 = 0, a2 = 0, a3 = 0;
    for (int it = 0; it < iters; ++it) {
        const int ix = window(idx, n_win, it)[lane];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = MODE == 1 ? (lane >> 2) + 16 * t + 64 * (it & 15) : quad_bcast(ix, t);
            const char *p = reinterpret_cast<const char *>(lds) + (uint32_t)r * 64u + coff;
            if constexpr (MODE == 2) {
                const float2 x = *reinterpret_cast<const float2 *>(p);
                const float2 y = *reinterpret_cast<const float2 *>(p + 8);
                a0 += x.x; a1 += x.y; a2 += y.x; a3 += y.y;
            } else {
                const float4 x = *reinterpret_cast<const float4 *>(p);
                a0 += x.x; a1 += x.y; a2 += x.z; a3 += x.w;
            }
        }
    }
    sink[blockIdx.x * blockDim.x + threadIdx.x] = a0 + a1 + a2 + a3;
}

// The same gathers from global memory (a table of n_rows rows; L2 or the
// Infinity Cache serve it after the first touches).
__global__ void __launch_bounds__(kThreads)
k_l2_gather(const float *table, const int *idx, int n_win, int iters, float *sink) {
    const int lane = threadIdx.x & 63;
    const uint32_t coff = (uint32_t)(lane & 3) * 16u;
    float a0 = 0, a1 = 0, a2 = 0, a3 = 0;
    const char *base = reinterpret_cast<const char *>(table);
    for (int it = 0; it < iters; ++it) {
        const int ix = window(idx, n_win, it)[lane];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int r = quad_bcast(ix, t);
            const float4 x = *reinterpret_cast<const float4 *>(base + (size_t)r * 64u + coff);
            a0 += x.x; a1 += x.y; a2 += x.z; a3 += x.w;
        }
    }
    sink[blockIdx.x * blockDim.x + threadIdx.x] = a0 + a1 + a2 + a3;
}

// Global float atomics the way a width-16 scatter adds: 16 lanes per row,
// one column each, so one instruction adds into four whole 64-byte rows; in
// step t lane group g takes the row held by lane 16g + t.
__global__ void __launch_bounds__(kThreads)
k_atomic(float *out, const int *idx, int n_win, int iters) {
    const int lane = threadIdx.x & 63;
    for (int it = 0; it < iters; ++it) {
        const int ix = window(idx, n_win, it)[lane];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int r = __builtin_amdgcn_ds_bpermute(((lane >> 4) * 16 + t) * 4, ix);
            unsafeAtomicAdd(out + (size_t)r * 16 + (lane & 15), 1.0f);
        }
    }
}

// LDS float atomics the same way, into a per-block LDS copy of an n_rows x 16
// float output (the scatter walk's private copy of out): in step t lane group
// g takes the row held by lane 16g + t and adds into its 16 columns.
__global__ void __launch_bounds__(kThreads)
k_lds_atomic(int n_rows, const int *idx, int n_win, int iters, float *sink) {
    extern __shared__ __attribute__((aligned(16))) float lds[];
    const int lane = threadIdx.x & 63;
    for (int k = threadIdx.x; k < n_rows * 16; k += blockDim.x) lds[k] = 0.0f;
    __syncthreads();
    for (int it = 0; it < iters; ++it) {
        const int ix = window(idx, n_win, it)[lane];
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const int r = __builtin_amdgcn_ds_bpermute(((lane >> 4) * 16 + t) * 4, ix);
            atomicAdd(lds + r * 16 + (lane & 15), 1.0f);
        }
    }
    __syncthreads();
    sink[blockIdx.x * blockDim.x + threadIdx.x] = lds[threadIdx.x % (n_rows * 16)];
}

__global__ void k_empty(float *sink) {
    if (sink && threadIdx.x == 0 && blockIdx.x == 0x7fffffff) sink[0] = 0;
}

}  // namespace

extern "C" {

// kind 0: LDS gathers (mode 0, 1, 2 as k_lds_gather), table of n_rows <= 2560
// rows; 1: global gathers; 2: global float atomics into out (n_rows x 16
// floats); 3: empty launches; 4: LDS float atomics into a per-block n_rows x
// 16 copy (n_rows <= 2560). idx: n_win * 64 row numbers in [0, n_rows).
// sink: grid * 1024 floats. Runs `reps` launches between two events on
// `stream` and returns their total milliseconds in *ms. Returns 0, or -1 on
// bad arguments, or the HIP error code.
int vspmm_probe(int kind, int mode, const float *table, int n_rows, const int *idx, int n_win,
                int iters, int grid, float *sink, float *out, int reps, hipStream_t stream,
                float *ms) {
    if (!ms || reps < 1 || grid < 1 || n_win < 1 || iters < 0) return -1;
    if (kind != 3 && (!idx || n_rows < 1)) return -1;
    if (kind == 0 && (n_rows > 2560 || (mode == 1 && n_rows < 1024) || mode < 0 || mode > 2 ||
                      !table || !sink))
        return -1;
    if (kind == 1 && (!table || !sink)) return -1;
    if (kind == 2 && !out) return -1;
    if (kind == 4 && (n_rows > 2560 || !sink)) return -1;
    if (kind < 0 || kind > 4) return -1;
    const size_t lds = kind == 0 || kind == 4 ? (size_t)n_rows * 64 : 0;
    if (kind == 4)
        (void)hipFuncSetAttribute((const void *)&k_lds_atomic,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (kind == 0) {
        const void *fns[3] = {(const void *)&k_lds_gather<0>, (const void *)&k_lds_gather<1>,
                              (const void *)&k_lds_gather<2>};
        (void)hipFuncSetAttribute(fns[mode], hipFuncAttributeMaxDynamicSharedMemorySize,
                                  160 * 1024);
    }
    hipEvent_t a, b;
    if (hipEventCreate(&a) != hipSuccess || hipEventCreate(&b) != hipSuccess) return -2;
    auto launch = [&]() {
        const dim3 g(grid), t(kThreads);
        switch (kind) {
            case 0:
                if (mode == 0) hipLaunchKernelGGL(k_lds_gather<0>, g, t, lds, stream, table, n_rows, idx, n_win, iters, sink);
                else if (mode == 1) hipLaunchKernelGGL(k_lds_gather<1>, g, t, lds, stream, table, n_rows, idx, n_win, iters, sink);
                else hipLaunchKernelGGL(k_lds_gather<2>, g, t, lds, stream, table, n_rows, idx, n_win, iters, sink);
                break;
            case 1: hipLaunchKernelGGL(k_l2_gather, g, t, 0, stream, table, idx, n_win, iters, sink); break;
            case 2: hipLaunchKernelGGL(k_atomic, g, t, 0, stream, out, idx, n_win, iters); break;
            case 4: hipLaunchKernelGGL(k_lds_atomic, g, t, lds, stream, n_rows, idx, n_win, iters, sink); break;
            default: hipLaunchKernelGGL(k_empty, g, dim3(256), 0, stream, sink); break;
        }
    };
    launch();  // warm-up (and the first fetch of the table)
    hipError_t e = hipEventRecord(a, stream);
    for (int r = 0; r < reps; ++r) launch();
    if (e == hipSuccess) e = hipEventRecord(b, stream);
    if (e == hipSuccess) e = hipEventSynchronize(b);
    if (e == hipSuccess) e = hipEventElapsedTime(ms, a, b);
    if (e == hipSuccess) e = hipGetLastError();
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
    return e == hipSuccess ? 0 : (int)e;
}

}  // extern "C"
