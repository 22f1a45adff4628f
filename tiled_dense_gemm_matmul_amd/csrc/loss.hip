// Fused loss kernels for MI355X (gfx950): cross_entropy (loss + in-place
// dLogits, label smoothing and z-loss) and sum_losses, as defined on the page
// "cross_entropy ve sum_losses — Fused Loss + dLogits"
// (https://llm.istanbul/learn/tr/07_loss), sections "Ne Yapar?" and "Satır
// Satır".
//
// The work is HBM-bound: every logit is read and its gradient written, so
// the ideal is one read and one write of the [S x V] array.  The page reads
// each row three times (max, sum, gradient); here a workgroup of 256 to 1024
// threads keeps its whole row in registers (16 to 64 values per thread: rows
// of up to 65536 logits with 16-byte accesses, 16384 with 4-byte ones), so
// the row is read from memory once.  With 16-byte accesses the workgroup is
// sized to the row: 256 x 16 up to 4096 logits, 512 x 16 up to 8192,
// 512 x 32 up to 16384, 1024 x 32 up to 32768, 1024 x 64 beyond (the fewer
// idle register slots, the more rows in flight per CU: 512 x 16384 logits in
// 10.1 against 12.2 us on 256 x 64, 2048 x 4096 in 10.1 against 21.0).
// Longer rows fall back to the page's streaming order.
//  * Loads are 16-byte buffer loads when V % 4 == 0 and the array is 16-byte
//    aligned, else 4-byte loads; both coalesced along the row.  Elements past
//    V come back as zeros from the buffer's range check and are masked out of
//    the reductions by their index.
//  * Reductions: a butterfly over the 64 lanes of a wave, then the waves'
//    partials in a fixed order from LDS.  Each reduction has its own LDS
//    slots, so consecutive reductions need no trailing barrier.
//  * exp(l - max) is computed once per element and kept for the gradient.
//  * Logit arrays of 256 MiB or more (past the Infinity Cache) are read and
//    written with the non-temporal cache policy; smaller ones, which the cache
//    can hold, keep the default.

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <cmath>

#include "gemm_fwd.h"
#include "loss.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4v __attribute__((vector_size(16)));
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr int kOOB = (int)0x80000000u;
constexpr int kNonTemporal = 2;                       // buffer-access cache policy: nt
constexpr int64_t kStreamBytes = (int64_t)256 << 20;  // arrays past the Infinity Cache

__device__ __forceinline__ Rsrc row_rsrc(const void *base, int bytes) {
    const uint64_t b = reinterpret_cast<uint64_t>(base);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32));
    void *ub = reinterpret_cast<void *>((static_cast<uint64_t>(hi) << 32) | lo);
    return __builtin_amdgcn_make_buffer_rsrc(ub, (short)0, __builtin_amdgcn_readfirstlane(bytes), 0x00020000);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Workgroup reduction into every thread: wave butterflies, then the NW wave
// partials added (or maxed) in wave order from `slots`.
template <int NW, bool MAX>
__device__ __forceinline__ float block_reduce(float v, float *slots) {
    v = MAX ? wave_max(v) : wave_sum(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) slots[wave] = v;
    __syncthreads();
    float r = slots[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = MAX ? fmaxf(r, slots[w]) : r + slots[w];
    return r;
}

// The loss of one row from its reductions (the page's phase 3).
__device__ __forceinline__ float row_loss(float lse, float l_t, float mean_l, float alpha, float beta) {
    return (lse - (1.0f - alpha) * l_t - alpha * mean_l) + beta * lse * lse;
}

// One workgroup per row, the row held in registers: CAP values per thread,
// in groups of W consecutive elements (W = 4 with 16-byte accesses).  Group
// j of thread t covers elements [(j NT + t) W, +W); a group past the row end
// is fetched and stored at an offset past the buffer's range, so its loads
// return zeros and its stores are dropped, and it is left out of the
// reductions by comparing j with the thread's count of valid groups.
template <int NT, int CAP, bool VEC, bool STREAM>
__global__ __launch_bounds__(NT) void cross_entropy_resident(float *logits, const uint32_t *tgts, float *losses,
                                                             int V, float alpha, float beta, float inv_norm) {
    constexpr int NW = NT / 64;
    constexpr int W = VEC ? 4 : 1;
    constexpr int G = CAP / W;
    constexpr int POL = STREAM ? kNonTemporal : 0;  // cache policy of the row's loads and stores
    __shared__ float red[3][NW];
    const int tid = threadIdx.x;
    const int s = blockIdx.x;
    float *row = logits + (size_t)s * V;
    const Rsrc rr = row_rsrc(row, V * 4);
    const uint32_t tgt = tgts[s];
    auto off = [&](int j) { return (j * NT + tid) * (W * 4); };
    if (tgt >= (uint32_t)V) {
        // ignored row: zero loss, zero gradient (nothing to read)
        if (tid == 0) losses[s] = 0.0f;
#pragma unroll
        for (int j = 0; j < G; ++j) {
            if (VEC) __builtin_amdgcn_raw_buffer_store_b128(u32x4v{0u, 0u, 0u, 0u}, rr, off(j), 0, POL);
            else __builtin_amdgcn_raw_buffer_store_b32(0u, rr, off(j), 0, POL);
        }
        return;
    }
    const int ng = V / W;                                   // groups in the row
    const int nv = ng > tid ? min(G, (ng - tid + NT - 1) / NT) : 0;  // this thread's valid groups
    float x[CAP];
#pragma unroll
    for (int j = 0; j < G; ++j) {
        if (VEC) {
            const f32x4 q = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rr, off(j), 0, POL));
            x[4 * j] = q.x; x[4 * j + 1] = q.y; x[4 * j + 2] = q.z; x[4 * j + 3] = q.w;
        } else {
            x[j] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rr, off(j), 0, POL));
        }
    }
    // phase 1: row max (and the plain sum for label smoothing)
    float m = -INFINITY, sl = 0.0f;
#pragma unroll
    for (int j = 0; j < G; ++j) {
        if (j < nv) {
#pragma unroll
            for (int c = 0; c < W; ++c) {
                m = fmaxf(m, x[W * j + c]);
                sl += x[W * j + c];
            }
        }
    }
    const float row_max = block_reduce<NW, true>(m, red[0]);
    // phase 2: denominator; keep exp(l - max) for the gradient
    float se = 0.0f;
#pragma unroll
    for (int j = 0; j < G; ++j) {
#pragma unroll
        for (int c = 0; c < W; ++c) {
            const float e = j < nv ? __expf(x[W * j + c] - row_max) : 0.0f;
            se += e;
            x[W * j + c] = e;
        }
    }
    const float denom = fmaxf(block_reduce<NW, false>(se, red[1]), 1e-30f);
    const float sum_l = alpha > 0.0f ? block_reduce<NW, false>(sl, red[2]) : 0.0f;
    const float inv_denom = 1.0f / denom;
    const float lse = row_max + __logf(denom);
    if (tid == 0) {
        const float l_t = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rr, (int)tgt * 4, 0, 0));
        losses[s] = row_loss(lse, l_t, sum_l / (float)V, alpha, beta);
    }
    // Thread 0 has read the target's logit (its value is used above); the
    // thread that owns that element overwrites it only after this barrier.
    __syncthreads();
    // phase 4: the gradient, in place.  The target's register slot in the
    // thread that holds it (-1 elsewhere).
    const int tg = (int)tgt / W;
    const int tslot = (tg % NT == tid) ? (tg / NT) * W + (int)tgt % W : -1;
    const float zf = 2.0f * beta * lse;
    const float smooth = alpha / (float)V;
    const float hit = 1.0f - alpha;
#pragma unroll
    for (int j = 0; j < G; ++j) {
        float g[W];
#pragma unroll
        for (int c = 0; c < W; ++c) {
            const int i = W * j + c;
            const float p = x[i] * inv_denom;
            const float t = (i == tslot ? hit : 0.0f) + smooth;
            g[c] = ((p - t) + zf * p) * inv_norm;
        }
        if (VEC) {
            const f32x4 q = f32x4{g[0], g[W > 1 ? 1 : 0], g[W > 2 ? 2 : 0], g[W > 3 ? 3 : 0]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4v, q), rr, off(j), 0, POL);
        } else {
            __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, g[0]), rr, off(j), 0, POL);
        }
    }
}

// Rows too long for the registers: the page's order, reading the row three
// times (max and plain sum, exp sum, gradient).
template <int NT>
__global__ __launch_bounds__(NT) void cross_entropy_stream(float *logits, const uint32_t *tgts, float *losses, int V,
                                                           float alpha, float beta, float inv_norm) {
    constexpr int NW = NT / 64;
    __shared__ float red[3][NW];
    const int tid = threadIdx.x;
    const int s = blockIdx.x;
    float *row = logits + (size_t)s * V;
    const uint32_t tgt = tgts[s];
    if (tgt >= (uint32_t)V) {
        if (tid == 0) losses[s] = 0.0f;
        for (int v = tid; v < V; v += NT) row[v] = 0.0f;
        return;
    }
    float m = -INFINITY, sl = 0.0f;
    for (int v = tid; v < V; v += NT) {
        const float l = row[v];
        m = fmaxf(m, l);
        sl += l;
    }
    const float row_max = block_reduce<NW, true>(m, red[0]);
    float se = 0.0f;
    for (int v = tid; v < V; v += NT) se += __expf(row[v] - row_max);
    const float denom = fmaxf(block_reduce<NW, false>(se, red[1]), 1e-30f);
    const float sum_l = alpha > 0.0f ? block_reduce<NW, false>(sl, red[2]) : 0.0f;
    const float inv_denom = 1.0f / denom;
    const float lse = row_max + __logf(denom);
    if (tid == 0) losses[s] = row_loss(lse, row[tgt], sum_l / (float)V, alpha, beta);
    __syncthreads();
    const float zf = 2.0f * beta * lse;
    const float smooth = alpha / (float)V;
    for (int v = tid; v < V; v += NT) {
        const float p = __expf(row[v] - row_max) * inv_denom;
        const float t = (v == (int)tgt ? 1.0f - alpha : 0.0f) + smooth;
        row[v] = ((p - t) + zf * p) * inv_norm;
    }
}

// sum_losses: one workgroup; thread t adds t, t + NT, ... in order, then the
// fixed-order workgroup reduction.
template <int NT>
__global__ __launch_bounds__(NT) void sum_losses_kernel(const float *losses, float *out, int S) {
    __shared__ float red[NT / 64];
    float acc = 0.0f;
    for (int i = threadIdx.x; i < S; i += NT) acc += losses[i];
    const float total = block_reduce<NT / 64, false>(acc, red);
    if (threadIdx.x == 0) out[0] = total;
}

bool overlaps(const void *a, size_t abytes, const void *b, size_t bbytes) {
    if (a == nullptr || b == nullptr || abytes == 0 || bbytes == 0) return false;
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
    return a0 < b0 + bbytes && b0 < a0 + abytes;
}

bool aligned(const void *p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

extern "C" {

int loss_cross_entropy(float *logits, const uint32_t *targets, float *losses, int64_t S, int64_t V, float alpha,
                       float beta, float inv_norm, void *stream) {
    if (S < 0 || V < 0 || S >= ((int64_t)1 << 31) || V >= ((int64_t)1 << 29)) return GEMM_ERR_SHAPE;
    if (S > 0 && (targets == nullptr || losses == nullptr || (V > 0 && logits == nullptr))) return GEMM_ERR_NULL;
    if (!aligned(logits, 4) || !aligned(targets, 4) || !aligned(losses, 4)) return GEMM_ERR_ALIGN;
    if (!(alpha >= 0.0f && alpha <= 1.0f) || !(beta >= 0.0f) || !std::isfinite(beta) || !std::isfinite(inv_norm))
        return GEMM_ERR_DTYPE;
    if (overlaps(losses, (size_t)S * 4, logits, (size_t)S * V * 4) || overlaps(losses, (size_t)S * 4, targets, (size_t)S * 4))
        return GEMM_ERR_ALIAS;
    if (S == 0) return GEMM_OK;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const int s = (int)S, v = (int)V;
    const bool vec = V % 4 == 0 && aligned(logits, 16);
    const bool stream_hint = S * V * 4 >= kStreamBytes;
    // a resident launch of NT threads holding CAP logits each
#define LOSS_RESIDENT(NT, CAP)                                                                                   \
    do {                                                                                                          \
        if (stream_hint)                                                                                          \
            hipLaunchKernelGGL((cross_entropy_resident<NT, CAP, true, true>), dim3(s), dim3(NT), 0, st, logits,  \
                               targets, losses, v, alpha, beta, inv_norm);                                        \
        else                                                                                                      \
            hipLaunchKernelGGL((cross_entropy_resident<NT, CAP, true, false>), dim3(s), dim3(NT), 0, st, logits, \
                               targets, losses, v, alpha, beta, inv_norm);                                        \
    } while (0)
    if (vec && V <= 256 * 16) {
        LOSS_RESIDENT(256, 16);
    } else if (vec && V <= 512 * 16) {
        LOSS_RESIDENT(512, 16);
    } else if (vec && V <= 512 * 32) {
        LOSS_RESIDENT(512, 32);
    } else if (vec && V <= 1024 * 32) {
        LOSS_RESIDENT(1024, 32);
    } else if (V <= 256 * 64 && !vec) {
        hipLaunchKernelGGL((cross_entropy_resident<256, 64, false, false>), dim3(s), dim3(256), 0, st, logits, targets, losses, v, alpha, beta, inv_norm);
    } else if (V <= 1024 * 64 && vec) {
        if (stream_hint) hipLaunchKernelGGL((cross_entropy_resident<1024, 64, true, true>), dim3(s), dim3(1024), 0, st, logits, targets, losses, v, alpha, beta, inv_norm);
        else hipLaunchKernelGGL((cross_entropy_resident<1024, 64, true, false>), dim3(s), dim3(1024), 0, st, logits, targets, losses, v, alpha, beta, inv_norm);
    } else {
        hipLaunchKernelGGL((cross_entropy_stream<1024>), dim3(s), dim3(1024), 0, st, logits, targets, losses, v, alpha, beta, inv_norm);
    }
#undef LOSS_RESIDENT
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

int loss_sum_losses(const float *losses, float *out, int64_t S, void *stream) {
    if (S < 0 || S >= ((int64_t)1 << 31)) return GEMM_ERR_SHAPE;
    if (out == nullptr || (S > 0 && losses == nullptr)) return GEMM_ERR_NULL;
    if (!aligned(losses, 4) || !aligned(out, 4)) return GEMM_ERR_ALIGN;
    if (overlaps(out, 4, losses, (size_t)S * 4)) return GEMM_ERR_ALIAS;
    hipLaunchKernelGGL((sum_losses_kernel<1024>), dim3(1), dim3(1024), 0, static_cast<hipStream_t>(stream), losses, out,
                       (int)S);
    return hipGetLastError() == hipSuccess ? GEMM_OK : GEMM_ERR_LAUNCH;
}

}  // extern "C"
