// Test program for the library's host code built with AddressSanitizer and
// UndefinedBehaviorSanitizer (hipcc, instrumentation on the host side only):
// every entry point's argument validation (each status code, extreme and
// overflowing shapes, aliasing, workspace errors), and the tile-choice and
// workspace-size queries over a sweep of shapes.  Only paths that return
// before a launch are taken, so no GPU is needed.  Exits non-zero on a wrong
// status; the sanitizers abort on a memory or undefined-behaviour error.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "activation.h"
#include "gemm_fwd.h"
#include "loss.h"

static int failures = 0;
#define EXPECT(expr, want)                                                                      \
    do {                                                                                        \
        const long long got_ = (long long)(expr);                                               \
        if (got_ != (long long)(want)) {                                                        \
            std::fprintf(stderr, "line %d: %s = %lld, want %lld\n", __LINE__, #expr, got_,     \
                         (long long)(want));                                                    \
            ++failures;                                                                         \
        }                                                                                       \
    } while (0)

int main() {
    // fake, aligned, non-overlapping addresses: validation never dereferences
    float *X = reinterpret_cast<float *>(0x10000000), *W = reinterpret_cast<float *>(0x20000000);
    float *R = reinterpret_cast<float *>(0x30000000), *Y = reinterpret_cast<float *>(0x40000000);
    float *U = reinterpret_cast<float *>(0x50000000);
    void *WS = reinterpret_cast<void *>(0x60000000);
    const int64_t big = (int64_t)1 << 62;
    gemm_opts o;
    std::memset(&o, 0, sizeof o);
    o.config = -1;

    // forward: every status code
    EXPECT(gemm_fwd(nullptr, W, nullptr, Y, 4, 4, 4, 0, nullptr), GEMM_ERR_NULL);
    EXPECT(gemm_fwd(X, W, nullptr, Y, 4, 6, 4, 0, nullptr), GEMM_ERR_SHAPE);
    EXPECT(gemm_fwd(X, W, nullptr, Y, -1, 4, 4, 0, nullptr), GEMM_ERR_SHAPE);
    EXPECT(gemm_fwd(X, W, nullptr, Y, big, big, big, 0, nullptr), GEMM_ERR_SHAPE);
    EXPECT(gemm_fwd(X, W, nullptr, Y, INT64_MAX, 4, 4, 0, nullptr), GEMM_ERR_SHAPE);
    EXPECT(gemm_fwd(X, W, nullptr, Y, 4, (int64_t)1 << 21, 4, 0, nullptr), GEMM_ERR_SHAPE);
    EXPECT(gemm_fwd(X + 1, W, nullptr, Y, 4, 4, 4, 0, nullptr), GEMM_ERR_ALIGN);
    EXPECT(gemm_fwd(X, W, nullptr, Y, 4, 4, 4, 0x4, nullptr), GEMM_ERR_DTYPE);
    EXPECT(gemm_fwd(X, W, Y, Y, 4, 4, 4, 0, nullptr), GEMM_ERR_ALIAS);
    EXPECT(gemm_fwd(X, W, nullptr, Y, 0, 4, 4, 0, nullptr), GEMM_OK);
    EXPECT(gemm_fwd_swiglu(X, U, W, nullptr, Y, 4, 4, 4, 0, nullptr), GEMM_ERR_NULL);
    EXPECT(gemm_fwd_swiglu(X, U, W, R, Y, 4, 4, 4, 7, nullptr), GEMM_ERR_DTYPE);
    EXPECT(gemm_fwd_swiglu_noalloc(X, U, W, R, Y, 4, 4, 4, 7, nullptr), GEMM_ERR_DTYPE);
    EXPECT(gemm_fwd_swiglu_noalloc(X, U, W, R, Y, 4, 6, 4, 0, nullptr), GEMM_ERR_SHAPE);
    EXPECT(gemm_fwd_swiglu_noalloc(X, U, W, R, R, 4, 4, 4, 0, nullptr), GEMM_ERR_ALIAS);
    o.config = gemm_num_configs();
    EXPECT(gemm_fwd_ex(X, W, nullptr, Y, 4, 4, 4, 0, &o, nullptr), GEMM_ERR_CONFIG);
    o.config = -1;
    o.workspace = nullptr;
    o.workspace_bytes = 64;
    EXPECT(gemm_fwd_ex(X, W, nullptr, Y, 4, 4, 4, 0, &o, nullptr), GEMM_ERR_WORKSPACE);
    o.workspace = static_cast<char *>(WS) + 64;
    o.workspace_bytes = 1 << 20;
    EXPECT(gemm_fwd_ex(X, W, nullptr, Y, 4, 4, 4, 0, &o, nullptr), GEMM_ERR_ALIGN);
    o.workspace = Y;
    EXPECT(gemm_fwd_ex(X, W, nullptr, Y, 4, 4, 4, 0, &o, nullptr), GEMM_ERR_ALIAS);
    // an explicit split-K configuration without a workspace
    int ks = -1;
    for (int c = 0; c < gemm_num_configs(); ++c)
        if (std::strstr(gemm_config_name(c), "_ks")) ks = c;
    EXPECT(ks >= 0, 1);
    o.config = ks;
    o.workspace = nullptr;
    o.workspace_bytes = 0;
    EXPECT(gemm_fwd_swiglu_ex(X, U, W, R, Y, 64, 256, 64, 0, &o, nullptr), GEMM_ERR_WORKSPACE);
    o.config = -1;

    // backward
    EXPECT(gemm_matmul_t(nullptr, W, Y, 4, 4, 4, 0, nullptr), GEMM_ERR_NULL);
    EXPECT(gemm_matmul_at(X, W, Y, 4, 6, 4, 0, nullptr), GEMM_ERR_SHAPE);
    EXPECT(gemm_matmul_at_swiglu_a(X, U, W, Y, big, 4, 4, 0, nullptr), GEMM_ERR_SHAPE);
    EXPECT(gemm_matmul_t(X, W, Y, 4, 4, 4, 0x1, nullptr), GEMM_ERR_DTYPE);
    EXPECT(gemm_matmul_at(X, W, X, 4, 4, 4, 0, nullptr), GEMM_ERR_ALIAS);
    EXPECT(gemm_matmul_t_swiglu_bwd(X, W, R, U, Y, Y, 4, 4, 4, nullptr), GEMM_ERR_ALIAS);
    o.config = gemm_bwd_num_configs();
    EXPECT(gemm_matmul_t_ex(X, W, Y, 4, 4, 4, 0, &o, nullptr), GEMM_ERR_CONFIG);
    o.config = -1;

    // loss and activation kernels
    EXPECT(loss_cross_entropy(nullptr, reinterpret_cast<uint32_t *>(W), R, 4, 4, 0.f, 0.f, 1.f, nullptr),
           GEMM_ERR_NULL);
    EXPECT(loss_cross_entropy(X, reinterpret_cast<uint32_t *>(W), R, -1, 4, 0.f, 0.f, 1.f, nullptr), GEMM_ERR_SHAPE);
    EXPECT(loss_cross_entropy(X, reinterpret_cast<uint32_t *>(W), R, 4, 4, 2.f, 0.f, 1.f, nullptr), GEMM_ERR_DTYPE);
    EXPECT(loss_sum_losses(X, X, 4, nullptr), GEMM_ERR_ALIAS);
    EXPECT(act_ffn_swiglu_backward(X, W, U, R, R, 64, nullptr), GEMM_ERR_ALIAS);
    EXPECT(act_ffn_gelu_backward(X, W, Y, -1, nullptr), GEMM_ERR_SHAPE);
    EXPECT(act_gelu_inplace(X, X, 64, nullptr), GEMM_ERR_ALIAS);

    // queries over a sweep of shapes, including ones near the limits
    const int64_t dims[] = {0, 1, 4, 16, 100, 128, 512, 768, 3072, 8191, 8192, 50304, (int64_t)1 << 20,
                            ((int64_t)1 << 21) - 4, (int64_t)1 << 30, ((int64_t)1 << 31) - 1};
    long long acc = 0;
    for (int64_t M : dims)
        for (int64_t K : dims)
            for (int64_t N : dims)
                for (int sw = 0; sw < 2; ++sw) {
                    for (int ws = 0; ws < 2; ++ws) {
                        acc += gemm_select_config(M, K, N, sw, sw, ws);
                        acc += gemm_bwd_select_config(1 + sw, M, K, N, sw, ws);
                    }
                    acc += gemm_fwd_workspace_bytes(M, K, N, sw, 0, -1) >= -1;
                    acc += gemm_bwd_workspace_bytes(1 + sw, M, K, N, sw, -1) >= -1;
                }
    for (int c = -2; c <= gemm_num_configs(); ++c) acc += gemm_config_name(c) != nullptr;
    for (int c = -2; c <= gemm_bwd_num_configs(); ++c) acc += gemm_bwd_config_name(c) != nullptr;
    for (int s = -20; s <= 2; ++s) acc += (long long)std::strlen(gemm_status_string(s));
    EXPECT(gemm_fwd_workspace_bytes(-1, 4, 4, 0, 0, -1), -1);
    EXPECT(gemm_bwd_workspace_bytes(3, 4, 4, 4, 0, -1), -1);
    if (failures == 0) std::printf("host checks ok (%lld)\n", acc);
    return failures == 0 ? 0 : 1;
}
