// Slice walks for gfx950 (wave64): the aligned walk (output rows are the
// layout's major slices) and the scatter walk (output rows are the minor
// indices). Both follow the lane split of the vsparse page, section "The
// kernels", widened to a 64-lane wave: a slice is walked by G "entry lanes"
// that take its entries in stride, and each entry lane is WW "width lanes"
// wide, each covering VEC consecutive elements of the dense width. With
// G * WW < 64, a wave walks R = 64 / (G * WW) slices side by side (the
// regridding page's row groups, section "How it is built").
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vspmm {

template <typename T, int N>
struct vec_of {
    typedef T type __attribute__((ext_vector_type(N)));
};
template <typename T>
struct vec_of<T, 1> {
    typedef T type;
};

template <typename T, int N>
__device__ __forceinline__ void load_vec(const T *p, T (&r)[N]) {
    if constexpr (N == 1) {
        r[0] = *p;
    } else {
        const auto x = *reinterpret_cast<const typename vec_of<T, N>::type *>(p);
#pragma unroll
        for (int e = 0; e < N; ++e) r[e] = x[e];
    }
}

template <typename T, int N>
__device__ __forceinline__ void store_vec(T *p, const T (&r)[N]) {
    if constexpr (N == 1) {
        *p = r[0];
    } else {
        typename vec_of<T, N>::type x;
#pragma unroll
        for (int e = 0; e < N; ++e) x[e] = r[e];
        *reinterpret_cast<typename vec_of<T, N>::type *>(p) = x;
    }
}

__device__ __forceinline__ float fma_t(float a, float b, float c) { return __builtin_fmaf(a, b, c); }
__device__ __forceinline__ double fma_t(double a, double b, double c) { return __builtin_fma(a, b, c); }

__device__ __forceinline__ int readlane(int x, int l) { return __builtin_amdgcn_readlane(x, l); }
__device__ __forceinline__ float readlane(float x, int l) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), l));
}

__device__ __forceinline__ void atomic_add_t(float *p, float v) { unsafeAtomicAdd(p, v); }
__device__ __forceinline__ void atomic_add_t(double *p, double v) { unsafeAtomicAdd(p, v); }

// Lane geometry of one product.
struct Split {
    int log_ww;  // width lanes per entry lane (log2)
    int log_g;   // entry lanes per slice (log2)
};

// Walks the entries [e0, e1) of one slice in steps of G. For a VCS slice the
// value of each entry is its group's: with UNIFORM (one slice per wave) the
// wave keeps up to 64 group starts and values in lanes and advances a
// wave-uniform group cursor with readlane; otherwise each lane keeps its own
// cursor. Calls body(p, index, value) for the lane's entry p of each step
// (p >= e1 marks an idle lane).
template <bool VCS, bool UNIFORM, typename T, typename Body>
__device__ __forceinline__ void walk_slice(int lane, int slot, int G, int ka, int kb, int e0,
                                           int e1, const int *__restrict__ vptr,
                                           const T *__restrict__ vals,
                                           const int *__restrict__ idx, Body &&body) {
    if constexpr (!VCS) {
        for (int q = e0; q < e1; q += G) {
            const int p = q + slot;
            const bool valid = p < e1;
            const int i = valid ? idx[p] : 0;
            const T v = valid ? vals[p] : T(0);
            body(valid, i, v);
        }
    } else if constexpr (UNIFORM) {
        if (kb <= ka) return;
        int gb = ka;  // group held by lane 0
        int u = 0;    // current group, as a lane of the window (wave-uniform)
        int gs = vptr[min(gb + lane, kb)];        // start of group gb + lane
        T gv = vals[min(gb + lane, kb - 1)];      // value of group gb + lane
        for (int q = e0; q < e1; q += G) {
            const int p = q + slot;
            const bool valid = p < e1;
            const int i = valid ? idx[p] : 0;
            const int qend = min(q + G, e1);
            T v = readlane(gv, u);
            for (;;) {
                if (u == 63) {  // slide the window of group starts
                    gb += 63;
                    u = 0;
                    gs = vptr[min(gb + lane, kb)];
                    gv = vals[min(gb + lane, kb - 1)];
                }
                const int ns = readlane(gs, u + 1);
                if (ns >= qend) break;
                ++u;
                const T nv = readlane(gv, u);
                v = (p >= ns) ? nv : v;
            }
            body(valid, i, v);
        }
    } else {
        int kc = ka;
        int kend = (kb > ka) ? vptr[ka + 1] : 0;
        for (int q = e0; q < e1; q += G) {
            const int p = q + slot;
            const bool valid = p < e1;
            const int i = valid ? idx[p] : 0;
            T v = T(0);
            if (valid) {
                while (p >= kend) {
                    ++kc;
                    kend = vptr[kc + 1];
                }
                v = vals[kc];
            }
            body(valid, i, v);
        }
    }
}

// Aligned walk: out[s][:] = sum over the entries (s, i, v) of slice s of
// v * B[i][:]. Each lane accumulates its own entries in order with fused
// multiply-adds, then the G entry lanes are summed by a fixed xor tree, so the
// result depends only on the matrix and G, never on timing.
//   sptr: CSR row pointers or VCS major_ptr; vptr: VCS value_ptr (unused for
//   CSR); vals: CSR values or VCS group values; idx: minor indices;
//   B: n_minor x w; out: n_slices x w.
template <bool VCS, typename T, int VEC, bool UNIFORM>
__global__ void __launch_bounds__(256)
k_aligned(int n_slices, const int *__restrict__ sptr, const int *__restrict__ vptr,
          const T *__restrict__ vals, const int *__restrict__ idx,
          const T *__restrict__ B, T *__restrict__ out, int w, Split sp) {
    const int lane = threadIdx.x & 63;
    const int waves = blockDim.x >> 6;
    const int log_sub = sp.log_ww + sp.log_g;
    const int G = 1 << sp.log_g;
    const int sub = lane >> log_sub;
    const int slot = (lane >> sp.log_ww) & (G - 1);
    const int cl = lane & ((1 << sp.log_ww) - 1);
    const int R = 64 >> log_sub;
    const int chunk = VEC << sp.log_ww;
    const int stride = gridDim.x * waves * R;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int s = (blockIdx.x * waves + wave) * R + (UNIFORM ? 0 : sub); s < n_slices;
         s += stride) {
        int e0, e1, ka = 0, kb = 0;
        if constexpr (VCS) {
            ka = sptr[s];
            kb = sptr[s + 1];
            e0 = vptr[ka];
            e1 = vptr[kb];
        } else {
            e0 = sptr[s];
            e1 = sptr[s + 1];
        }
        for (int c0 = 0; c0 < w; c0 += chunk) {
            const int col = c0 + cl * VEC;
            const bool act = col < w;
            T acc[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[e] = T(0);
            walk_slice<VCS, UNIFORM, T>(lane, slot, G, ka, kb, e0, e1, vptr, vals, idx,
                                        [&](bool valid, int i, T v) {
                                            if (valid && act) {
                                                T b[VEC];
                                                load_vec<T, VEC>(B + (size_t)i * w + col, b);
#pragma unroll
                                                for (int e = 0; e < VEC; ++e)
                                                    acc[e] = fma_t(v, b[e], acc[e]);
                                            }
                                        });
            for (int off = 1 << sp.log_ww; off < (1 << log_sub); off <<= 1) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[e] += __shfl_xor(acc[e], off);
            }
            if (slot == 0 && act) store_vec<T, VEC>(out + (size_t)s * w + col, acc);
        }
    }
}

// Scatter walk: for every entry (s, i, v) of slice s, out[i][:] += v * B[s][:]
// with hardware float atomics (out must be zeroed first). B: n_slices x w,
// out: n_minor x w. One element per width lane, so the lanes of an entry hit
// one contiguous run of out.
template <bool VCS, typename T, bool UNIFORM>
__global__ void __launch_bounds__(256)
k_scatter(int n_slices, const int *__restrict__ sptr, const int *__restrict__ vptr,
          const T *__restrict__ vals, const int *__restrict__ idx,
          const T *__restrict__ B, T *__restrict__ out, int w, Split sp) {
    const int lane = threadIdx.x & 63;
    const int waves = blockDim.x >> 6;
    const int log_sub = sp.log_ww + sp.log_g;
    const int G = 1 << sp.log_g;
    const int sub = lane >> log_sub;
    const int slot = (lane >> sp.log_ww) & (G - 1);
    const int cl = lane & ((1 << sp.log_ww) - 1);
    const int R = 64 >> log_sub;
    const int chunk = 1 << sp.log_ww;
    const int stride = gridDim.x * waves * R;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    for (int s = (blockIdx.x * waves + wave) * R + (UNIFORM ? 0 : sub); s < n_slices;
         s += stride) {
        int e0, e1, ka = 0, kb = 0;
        if constexpr (VCS) {
            ka = sptr[s];
            kb = sptr[s + 1];
            e0 = vptr[ka];
            e1 = vptr[kb];
        } else {
            e0 = sptr[s];
            e1 = sptr[s + 1];
        }
        for (int c0 = 0; c0 < w; c0 += chunk) {
            const int col = c0 + cl;
            const bool act = col < w;
            const T b = act ? B[(size_t)s * w + col] : T(0);
            walk_slice<VCS, UNIFORM, T>(lane, slot, G, ka, kb, e0, e1, vptr, vals, idx,
                                        [&](bool valid, int i, T v) {
                                            if (valid && act)
                                                atomic_add_t(out + (size_t)i * w + col, v * b);
                                        });
        }
    }
}

// Fill n bytes (a multiple of 4) at p with zeros; p is 4-byte aligned.
__global__ void __launch_bounds__(256) k_zero(uint32_t *__restrict__ p, size_t n_words) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    size_t t = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const uintptr_t mis = ((uintptr_t)p >> 2) & 3;  // words before 16-byte alignment
    const size_t head = mis ? (4 - mis) : 0;
    if (head >= n_words) {
        if (t < n_words) p[t] = 0;
        return;
    }
    if (t < head) p[t] = 0;
    uint4 *q = reinterpret_cast<uint4 *>(p + head);
    const size_t n4 = (n_words - head) >> 2;
    for (size_t k = t; k < n4; k += stride) q[k] = make_uint4(0, 0, 0, 0);
    const size_t tail0 = head + (n4 << 2);
    if (t < n_words - tail0) p[tail0 + t] = 0;
}

// Structure checks: flag bit 1 = pointer array does not start at 0, bit 2 =
// decreasing, bit 4 = last pointer differs from count, bit 8 = index out of
// range.
__global__ void __launch_bounds__(256)
k_validate_ptr(const int *__restrict__ ptr, int n, int count, int *__restrict__ flag) {
    const int stride = gridDim.x * blockDim.x;
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i <= n; i += stride) {
        const int a = ptr[i];
        int f = 0;
        if (i == 0 && a != 0) f |= 1;
        if (i < n && ptr[i + 1] < a) f |= 2;
        if (i == n && a != count) f |= 4;
        if (f) atomicOr(flag, f);
    }
}

__global__ void __launch_bounds__(256)
k_validate_idx(const int *__restrict__ idx, int nnz, int n_minor, int *__restrict__ flag) {
    const int stride = gridDim.x * blockDim.x;
    int f = 0;
    for (int p = blockIdx.x * blockDim.x + threadIdx.x; p < nnz; p += stride) {
        const int i = idx[p];
        if (i < 0 || i >= n_minor) f = 8;
    }
    if (f) atomicOr(flag, f);
}

}  // namespace vspmm
