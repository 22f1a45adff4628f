/*
 * activation.h — C ABI of the FFN activation kernels for MI355X (gfx950).
 *
 * The element-wise kernels of the page "ffn_gelu_backward ve
 * ffn_swiglu_backward — FFN Activation Backward"
 * (https://llm.istanbul/learn/tr/09_backward_ffn), sections "Ne Yapar?",
 * "Türevler" and "Satır Satır", for n elements:
 *
 *   ffn_swiglu_backward: grad_gate = nan_guard(g * up * silu'(gate))
 *                        grad_up   = nan_guard(g * silu(gate))
 *       silu(x) = x s(x), silu'(x) = s(x) (1 + x (1 - s(x))), s the sigmoid
 *   ffn_gelu_backward:   grad_pre  = nan_guard(g * gelu'(pre_gelu)),
 *       gelu' the derivative of the tanh approximation with x clamped to
 *       [-100, 100]
 *   gelu_inplace:        x = gelu(x) = 0.5 x (1 + tanh(sqrt(2/pi)(x + 0.044715 x^3)))
 *       (the GeLU FFN's forward activation, read from its name; it may keep a
 *       copy of x for the backward, which needs it)
 *
 * where g is the gradient of the hidden activation and nan_guard turns a
 * NaN or an infinity into 0 (the shared preamble's helper).
 *
 * All arrays are fp32 device arrays of n elements owned by the caller, 4-byte
 * aligned (16-byte alignment enables 16-byte accesses).  An output may be the
 * very same array as one of the inputs (every element is read before it is
 * written, by the same thread) but may not overlap any other array partially,
 * and the two outputs of ffn_swiglu_backward may not overlap.  A call only
 * enqueues work on `stream` (a hipStream_t, NULL for the null stream); n == 0
 * enqueues nothing.  Status values are those of gemm_fwd.h: GEMM_ERR_NULL,
 * GEMM_ERR_SHAPE (n < 0 or n >= 2^40), GEMM_ERR_ALIGN, GEMM_ERR_ALIAS,
 * GEMM_ERR_LAUNCH; validation happens before anything is enqueued.
 */
#ifndef ACTIVATION_H
#define ACTIVATION_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int act_ffn_swiglu_backward(const float *grad_hidden, const float *gate, const float *up, float *grad_gate,
                            float *grad_up, int64_t n, void *stream);

int act_ffn_gelu_backward(const float *grad_hidden, const float *pre_gelu, float *grad_pre, int64_t n, void *stream);

/* x = gelu(x) in place; when pre_gelu is not NULL it receives the input values. */
int act_gelu_inplace(float *x, float *pre_gelu, int64_t n, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* ACTIVATION_H */
