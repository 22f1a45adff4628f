// FFN activation kernels for MI355X (gfx950): ffn_swiglu_backward,
// ffn_gelu_backward and gelu_inplace, as defined on the page
// "ffn_gelu_backward ve ffn_swiglu_backward — FFN Activation Backward"
// (https://llm.istanbul/learn/tr/09_backward_ffn), sections "Türevler" and
// "Satır Satır".
//
// Element-wise and HBM-bound (ffn_swiglu_backward moves 20 bytes per element,
// the others 12 and 8): each thread takes four consecutive elements per
// 16-byte access, in a grid-stride loop over a grid of a few workgroups per
// CU, so every access is coalesced and the launch stays small.  Arrays that
// are not 16-byte aligned take a 4-byte path.  The sigmoid branches on the
// sign so that exp only sees a non-positive argument, as the page's helper
// does; sigmoid, silu and silu' share one exp.
//
// The two backward kernels use non-temporal loads and stores when their
// arrays together exceed the 256 MB Infinity Cache: on 25M-element arrays
// that took ffn_swiglu_backward from 5.2 to 5.7 TB/s and ffn_gelu_backward
// from 5.7 to 5.9.  On data the cache holds the same hints cost up to a
// quarter of the rate, so smaller launches keep the ordinary accesses; and
// gelu_inplace (one read, two writes) measured 8% slower with them, so it
// never takes them.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <cmath>

#include "activation.h"
#include "gemm_fwd.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kSqrt2OverPi = 0.7978845608028654f;
constexpr float kGeluCoeff = 0.044715f;

__device__ __forceinline__ float nan_guard(float x) { return __builtin_isfinite(x) ? x : 0.0f; }

template <bool NT>
__device__ __forceinline__ f32x4 ld4(const float *p, int64_t q) {
    const f32x4 *a = reinterpret_cast<const f32x4 *>(p) + q;
    if constexpr (NT) return __builtin_nontemporal_load(a);
    else return *a;
}
template <bool NT>
__device__ __forceinline__ void st4(float *p, int64_t q, f32x4 v) {
    f32x4 *a = reinterpret_cast<f32x4 *>(p) + q;
    if constexpr (NT) __builtin_nontemporal_store(v, a);
    else *a = v;
}

__device__ __forceinline__ float sigmoid(float x) {
    const float e = __expf(-__builtin_fabsf(x));
    const float r = 1.0f / (1.0f + e);
    return x >= 0.0f ? r : e * r;
}

struct SwigluGrad {
    __device__ __forceinline__ void operator()(float g, float x, float u, float &dg, float &du) const {
        const float s = sigmoid(x);
        dg = nan_guard(g * u * (s * (1.0f + x * (1.0f - s))));
        du = nan_guard(g * (x * s));
    }
};

__device__ __forceinline__ float gelu_derivative(float x_in) {
    const float x = fminf(fmaxf(x_in, -100.0f), 100.0f);
    const float x2 = x * x;
    const float inner = kSqrt2OverPi * (x + kGeluCoeff * x2 * x);
    const float t = tanhf(inner);
    const float sech2 = 1.0f - t * t;
    const float d_inner = kSqrt2OverPi * (1.0f + 3.0f * kGeluCoeff * x2);
    return 0.5f * (1.0f + t) + 0.5f * x * sech2 * d_inner;
}

__device__ __forceinline__ float gelu(float x) {
    const float xc = fminf(fmaxf(x, -100.0f), 100.0f);
    const float inner = kSqrt2OverPi * (xc + kGeluCoeff * xc * xc * xc);
    return 0.5f * x * (1.0f + tanhf(inner));
}

// Grid-stride loops: VEC processes float4 groups (n4 of them) then the
// scalar tail; the scalar form processes every element one by one.
template <bool VEC, bool NT>
__global__ __launch_bounds__(256) void swiglu_backward_kernel(const float *gh, const float *gate, const float *up,
                                                              float *dgate, float *dup, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    SwigluGrad f;
    if (VEC) {
        const int64_t n4 = n / 4;
        for (int64_t q = i; q < n4; q += stride) {
            const f32x4 g = ld4<NT>(gh, q);
            const f32x4 x = ld4<NT>(gate, q);
            const f32x4 u = ld4<NT>(up, q);
            float a[4], b[4];
#pragma unroll
            for (int c = 0; c < 4; ++c) f(g[c], x[c], u[c], a[c], b[c]);
            st4<NT>(dgate, q, f32x4{a[0], a[1], a[2], a[3]});
            st4<NT>(dup, q, f32x4{b[0], b[1], b[2], b[3]});
        }
        i += n4 * 4;   // the tail: at most 3 elements, taken by the first threads
        if (i < n && (int64_t)blockIdx.x * 256 + threadIdx.x < 4) {
            float a, b;
            f(gh[i], gate[i], up[i], a, b);
            dgate[i] = a;
            dup[i] = b;
        }
        return;
    }
    for (; i < n; i += stride) {
        float a, b;
        f(gh[i], gate[i], up[i], a, b);
        dgate[i] = a;
        dup[i] = b;
    }
}

template <bool VEC, bool NT>
__global__ __launch_bounds__(256) void gelu_backward_kernel(const float *gh, const float *pre, float *dpre, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (VEC) {
        const int64_t n4 = n / 4;
        for (int64_t q = i; q < n4; q += stride) {
            const f32x4 g = ld4<NT>(gh, q);
            const f32x4 x = ld4<NT>(pre, q);
            st4<NT>(dpre, q,
                    f32x4{nan_guard(g.x * gelu_derivative(x.x)), nan_guard(g.y * gelu_derivative(x.y)),
                          nan_guard(g.z * gelu_derivative(x.z)), nan_guard(g.w * gelu_derivative(x.w))});
        }
        i += n4 * 4;
        if (i < n && (int64_t)blockIdx.x * 256 + threadIdx.x < 4) dpre[i] = nan_guard(gh[i] * gelu_derivative(pre[i]));
        return;
    }
    for (; i < n; i += stride) dpre[i] = nan_guard(gh[i] * gelu_derivative(pre[i]));
}

template <bool VEC>
__global__ __launch_bounds__(256) void gelu_inplace_kernel(float *x, float *pre, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * 256;
    int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (VEC) {
        const int64_t n4 = n / 4;
        for (int64_t q = i; q < n4; q += stride) {
            const f32x4 v = ld4<false>(x, q);
            if (pre) st4<false>(pre, q, v);
            st4<false>(x, q, f32x4{gelu(v.x), gelu(v.y), gelu(v.z), gelu(v.w)});
        }
        i += n4 * 4;
        if (i < n && (int64_t)blockIdx.x * 256 + threadIdx.x < 4) {
            const float v = x[i];
            if (pre) pre[i] = v;
            x[i] = gelu(v);
        }
        return;
    }
    for (; i < n; i += stride) {
        const float v = x[i];
        if (pre) pre[i] = v;
        x[i] = gelu(v);
    }
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Partial overlap is an error; the very same array is allowed.
bool bad_overlap(const void *a, const void *b, int64_t n) {
    if (a == nullptr || b == nullptr || a == b) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    const uintptr_t len = (uintptr_t)n * 4;
    return a0 < b0 + len && b0 < a0 + len;
}

// 8 workgroups per CU at most; larger grids measured no faster.
constexpr int64_t kMaxGrid = 2048;

// Combined size of a launch's arrays from which the accesses stream past the
// Infinity Cache (non-temporal).
constexpr int64_t kStreamBytes = (int64_t)256 << 20;

unsigned grid_for(int64_t n, bool vec) {
    const int64_t items = vec ? (n + 3) / 4 : n;
    const int64_t want = (items + 255) / 256;
    return (unsigned)(want < kMaxGrid ? (want > 0 ? want : 1) : kMaxGrid);
}

}  // namespace

extern "C" {

int act_ffn_swiglu_backward(const float *grad_hidden, const float *gate, const float *up, float *grad_gate,
                            float *grad_up, int64_t n, void *stream) {
    if (n < 0 || n >= ((int64_t)1 << 40)) return GEMM_ERR_SHAPE;
    if (n == 0) return GEMM_OK;
    if (!grad_hidden || !gate || !up || !grad_gate || !grad_up) return GEMM_ERR_NULL;
    const void *ins[3] = {grad_hidden, gate, up};
    const void *outs[2] = {grad_gate, grad_up};
    for (const void *p : ins)
        if (!aligned(p, 4)) return GEMM_ERR_ALIGN;
    for (const void *p : outs)
        if (!aligned(p, 4)) return GEMM_ERR_ALIGN;
    if (grad_gate == grad_up) return GEMM_ERR_ALIAS;
    for (const void *o : outs)
        for (const void *p : ins)
            if (bad_overlap(o, p, n)) return GEMM_ERR_ALIAS;
    if (bad_overlap(grad_gate, grad_up, n)) return GEMM_ERR_ALIAS;
    bool vec = true;
    for (const void *p : ins) vec = vec && aligned(p, 16);
    for (const void *p : outs) vec = vec && aligned(p, 16);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (vec && n * 20 >= kStreamBytes)
        hipLaunchKernelGGL((swiglu_backward_kernel<true, true>), dim3(grid_for(n, true)), dim3(256), 0, st, grad_hidden,
                           gate, up, grad_gate, grad_up, n);
    else if (vec)
        hipLaunchKernelGGL((swiglu_backward_kernel<true, false>), dim3(grid_for(n, true)), dim3(256), 0, st,
                           grad_hidden, gate, up, grad_gate, grad_up, n);
    else
        hipLaunchKernelGGL((swiglu_backward_kernel<false, false>), dim3(grid_for(n, false)), dim3(256), 0, st,
                           grad_hidden, gate, up, grad_gate, grad_up, n);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

int act_ffn_gelu_backward(const float *grad_hidden, const float *pre_gelu, float *grad_pre, int64_t n, void *stream) {
    if (n < 0 || n >= ((int64_t)1 << 40)) return GEMM_ERR_SHAPE;
    if (n == 0) return GEMM_OK;
    if (!grad_hidden || !pre_gelu || !grad_pre) return GEMM_ERR_NULL;
    if (!aligned(grad_hidden, 4) || !aligned(pre_gelu, 4) || !aligned(grad_pre, 4)) return GEMM_ERR_ALIGN;
    if (bad_overlap(grad_pre, grad_hidden, n) || bad_overlap(grad_pre, pre_gelu, n)) return GEMM_ERR_ALIAS;
    const bool vec = aligned(grad_hidden, 16) && aligned(pre_gelu, 16) && aligned(grad_pre, 16);
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (vec && n * 12 >= kStreamBytes)
        hipLaunchKernelGGL((gelu_backward_kernel<true, true>), dim3(grid_for(n, true)), dim3(256), 0, st, grad_hidden,
                           pre_gelu, grad_pre, n);
    else if (vec)
        hipLaunchKernelGGL((gelu_backward_kernel<true, false>), dim3(grid_for(n, true)), dim3(256), 0, st, grad_hidden,
                           pre_gelu, grad_pre, n);
    else
        hipLaunchKernelGGL((gelu_backward_kernel<false, false>), dim3(grid_for(n, false)), dim3(256), 0, st,
                           grad_hidden, pre_gelu, grad_pre, n);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

int act_gelu_inplace(float *x, float *pre_gelu, int64_t n, void *stream) {
    if (n < 0 || n >= ((int64_t)1 << 40)) return GEMM_ERR_SHAPE;
    if (n == 0) return GEMM_OK;
    if (!x) return GEMM_ERR_NULL;
    if (!aligned(x, 4) || (pre_gelu && !aligned(pre_gelu, 4))) return GEMM_ERR_ALIGN;
    if (pre_gelu == x || bad_overlap(x, pre_gelu, n)) return GEMM_ERR_ALIAS;
    const bool vec = aligned(x, 16) && (!pre_gelu || aligned(pre_gelu, 16));
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (vec)
        hipLaunchKernelGGL((gelu_inplace_kernel<true>), dim3(grid_for(n, true)), dim3(256), 0, st, x, pre_gelu,
                           n);
    else
        hipLaunchKernelGGL((gelu_inplace_kernel<false>), dim3(grid_for(n, false)), dim3(256), 0, st, x,
                           pre_gelu, n);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

}  // extern "C"
