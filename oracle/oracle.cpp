// Reference oracle for the forward linear-layer GEMM family.
//
// TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
// this file; only the test suite, the smoke check and the benchmark's CPU
// baseline leg do.  It shares no source with the HIP library and is compiled
// by g++ (not hipcc) as a plain host library.
//
// It is deliberately slow and literal: every value is formed in IEEE double,
// every dot product runs k = 0, 1, ..., K-1 from 0.0, with no blocking,
// reassociation or fused multiply-add (built with -ffp-contract=off).
//
// Sources (web pages of the "llm.istanbul/learn" series):
//   [LF] "matmul ve matmul_residual — Tiled Matrix Multiply (Forward)",
//        https://llm.istanbul/learn/tr/03_linear_forward
//   [FB] "ffn_gelu_backward ve ffn_swiglu_backward — FFN Activation Backward",
//        https://llm.istanbul/learn/tr/09_backward_ffn
//   IEEE Std 754-2008, binary16 interchange format (for the f16 weights).
//
// Parity status of every exported function is pinned by tests/test_oracle.py
// (brute force, closed forms, library cross-checks); none is "parity unpinned".

#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <vector>
#include <omp.h>

extern "C" {

// IEEE 754 binary16 -> double, from the format definition: 1 sign bit,
// 5 exponent bits with bias 15, 10 fraction bits.  Exponent 0 encodes zero and
// the subnormals f * 2^-24; exponent 31 encodes infinities and NaNs.
// [LF] "Önemli Optimizasyonlar" §1 binds W as vec4<f16> in the mixed-precision
// variants; the tiles it is staged into are f32, so each weight enters the
// product as the exact value of its f16 encoding.
double oracle_half_to_double(uint16_t h) {
    const int sign = (h >> 15) & 1;
    const int expo = (h >> 10) & 0x1f;
    const int frac = h & 0x3ff;
    double mag;
    if (expo == 0) {
        mag = std::ldexp(static_cast<double>(frac), -24);
    } else if (expo == 31) {
        mag = frac ? std::nan("") : HUGE_VAL;
    } else {
        // (1 + frac/1024) * 2^(expo-15) == (1024 + frac) * 2^(expo-25)
        mag = std::ldexp(static_cast<double>(1024 + frac), expo - 25);
    }
    return sign ? -mag : mag;
}

// Logistic sigmoid, branched on the sign so that exp() only ever receives a
// non-positive argument and no input is clamped: [FB] "Türevler / SiLU'" gives
// the two branches, and "WGSL-Spesifik Notlar" §2 states that the old ±50
// clamp was removed in favour of this branch.
double oracle_sigmoid(double x) {
    if (x >= 0.0) {
        return 1.0 / (1.0 + std::exp(-x));
    }
    const double e = std::exp(x);
    return e / (1.0 + e);
}

// silu(x) = x * sigmoid(x)   ([FB] "Türevler / SiLU'", forward definition).
double oracle_silu(double x) { return x * oracle_sigmoid(x); }

// One A-operand element, the value that enters the contraction.
//   plain   : a_ik = X_ik                                  ([LF] "Ne Yapar?")
//   swiglu  : a_ik = silu(GATE_ik) * UP_ik                 ([LF] "Ne Yapar?",
//             matmul_residual_swiglu_a; "Önemli Optimizasyonlar" §3: the
//             SwiGLU combine is applied to A as it is loaded)
static inline double a_value(const float *A, const float *U, int64_t idx) {
    if (U == nullptr) return static_cast<double>(A[idx]);
    return oracle_silu(static_cast<double>(A[idx])) * static_cast<double>(U[idx]);
}

// The forward GEMM family on a set of output rows.
//
//   Y[M,N] = A[M,K] @ W[K,N]  (+ R[M,N])            [LF] "Ne Yapar?"
//
// A is X (U == NULL) or the SwiGLU combine of GATE=A and UP=U.  W is fp32
// (w_is_f16 == 0) or IEEE binary16 bits (w_is_f16 == 1).  R may be NULL
// (matmul) or the residual added after the sum (matmul_residual, the
// "epilogue" of [LF] "Ne Yapar?").  All arrays are dense row-major, as bound
// in [LF] "Bind Group ABI".
//
// rows/nrows select which output rows to produce (rows == NULL: all M rows in
// order, nrows ignored).  Output row r of Yref (and of Bscale if non-NULL) is
// output row rows[r] of the product, in double:
//   Yref[r, j]   = (sum_{k=0}^{K-1} a_{i,k} * w_{k,j})  + R[i, j]
//   Bscale[r, j] =  sum_{k=0}^{K-1} |a_{i,k}| * |w_{k,j}|
// Bscale is the scale of the element-wise parity tolerance, not part of the
// method.  Returns 0, or -1 on a bad argument.  nthreads <= 0 uses OpenMP's
// default.
int oracle_gemm_rows(const float *A, const float *U, const void *W, int w_is_f16,
                     const float *R, int64_t M, int64_t K, int64_t N,
                     const int64_t *rows, int64_t nrows,
                     double *Yref, double *Bscale, int nthreads) {
    if (A == nullptr || W == nullptr || Yref == nullptr) return -1;
    if (M < 0 || K < 0 || N < 0) return -1;
    if (rows == nullptr) nrows = M;
    if (nrows < 0) return -1;
    for (int64_t r = 0; rows != nullptr && r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;
    if (nthreads <= 0) nthreads = omp_get_max_threads();

    // w_{k,j} as double: exact for fp32, and for binary16 via the decoder above.
    std::vector<double> w(static_cast<size_t>(K) * static_cast<size_t>(N));
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t j = 0; j < N; ++j) {
            const size_t idx = static_cast<size_t>(k) * N + j;
            w[idx] = w_is_f16
                ? oracle_half_to_double(static_cast<const uint16_t *>(W)[idx])
                : static_cast<double>(static_cast<const float *>(W)[idx]);
        }
    }

    // One output row per iteration.  The loop order i, k, j keeps every
    // element's own sum in the order k = 0..K-1, exactly as the i, j, k
    // textbook loop, while reading W one contiguous row at a time.
#pragma omp parallel num_threads(nthreads)
    {
        std::vector<double> a(static_cast<size_t>(K));
        std::vector<double> acc(static_cast<size_t>(N));
        std::vector<double> mag(Bscale ? static_cast<size_t>(N) : 0);
#pragma omp for schedule(dynamic, 1)
        for (int64_t r = 0; r < nrows; ++r) {
            const int64_t i = rows ? rows[r] : r;
            for (int64_t k = 0; k < K; ++k) a[k] = a_value(A, U, i * K + k);
            for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double aik = a[k];
                const double *wk = &w[static_cast<size_t>(k) * N];
                for (int64_t j = 0; j < N; ++j) acc[j] += aik * wk[j];
            }
            double *yrow = Yref + static_cast<size_t>(r) * N;
            for (int64_t j = 0; j < N; ++j)
                yrow[j] = R ? acc[j] + static_cast<double>(R[i * N + j]) : acc[j];
            if (Bscale) {
                for (int64_t j = 0; j < N; ++j) mag[j] = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    const double aik = std::fabs(a[k]);
                    const double *wk = &w[static_cast<size_t>(k) * N];
                    for (int64_t j = 0; j < N; ++j) mag[j] += aik * std::fabs(wk[j]);
                }
                double *brow = Bscale + static_cast<size_t>(r) * N;
                for (int64_t j = 0; j < N; ++j) brow[j] = mag[j];
            }
        }
    }
    return 0;
}

// Row and column sums of the product, from linearity of the definition above:
//   sum_j Y[i,j] = sum_k a_{i,k} * (sum_j w_{k,j})  + sum_j R[i,j]
//   sum_i Y[i,j] = sum_k (sum_i a_{i,k}) * w_{k,j}  + sum_i R[i,j]
// with the matching magnitudes (the tolerance scale summed over the same
// index):
//   row_mag[i] = sum_k |a_{i,k}| * sum_j |w_{k,j}|
//   col_mag[j] = sum_k (sum_i |a_{i,k}|) * |w_{k,j}|
// They cost O(MK + KN) instead of O(MKN), so every row and every column of a
// full-size result can be checked.  Any output pointer may be NULL.
int oracle_row_col_sums(const float *A, const float *U, const void *W, int w_is_f16,
                        const float *R, int64_t M, int64_t K, int64_t N,
                        double *row_sum, double *row_mag, double *col_sum, double *col_mag,
                        int nthreads) {
    if (A == nullptr || W == nullptr || M < 0 || K < 0 || N < 0) return -1;
    if (nthreads <= 0) nthreads = omp_get_max_threads();
    std::vector<double> wsum(static_cast<size_t>(K)), wabs(static_cast<size_t>(K));
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t k = 0; k < K; ++k) {
        double s = 0.0, a = 0.0;
        for (int64_t j = 0; j < N; ++j) {
            const size_t idx = static_cast<size_t>(k) * N + j;
            const double w = w_is_f16
                ? oracle_half_to_double(static_cast<const uint16_t *>(W)[idx])
                : static_cast<double>(static_cast<const float *>(W)[idx]);
            s += w;
            a += std::fabs(w);
        }
        wsum[k] = s;
        wabs[k] = a;
    }
    // per-row pass: row sums, and per-thread column sums of a and |a|
    std::vector<double> asum(static_cast<size_t>(K), 0.0), aabs(static_cast<size_t>(K), 0.0);
#pragma omp parallel num_threads(nthreads)
    {
        std::vector<double> ls(static_cast<size_t>(K), 0.0), la(static_cast<size_t>(K), 0.0);
#pragma omp for schedule(static)
        for (int64_t i = 0; i < M; ++i) {
            double s = 0.0, m = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double a = a_value(A, U, i * K + k);
                s += a * wsum[k];
                m += std::fabs(a) * wabs[k];
                ls[k] += a;
                la[k] += std::fabs(a);
            }
            double rs = 0.0;
            for (int64_t j = 0; R != nullptr && j < N; ++j) rs += static_cast<double>(R[i * N + j]);
            if (row_sum) row_sum[i] = s + rs;
            if (row_mag) row_mag[i] = m;
        }
#pragma omp critical
        for (int64_t k = 0; k < K; ++k) {
            asum[k] += ls[k];
            aabs[k] += la[k];
        }
    }
    if (col_sum == nullptr && col_mag == nullptr) return 0;
#pragma omp parallel for num_threads(nthreads) schedule(static)
    for (int64_t j = 0; j < N; ++j) {
        double s = 0.0, m = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const size_t idx = static_cast<size_t>(k) * N + j;
            const double w = w_is_f16
                ? oracle_half_to_double(static_cast<const uint16_t *>(W)[idx])
                : static_cast<double>(static_cast<const float *>(W)[idx]);
            s += asum[k] * w;
            m += aabs[k] * std::fabs(w);
        }
        double rs = 0.0;
        for (int64_t i = 0; R != nullptr && i < M; ++i) rs += static_cast<double>(R[i * N + j]);
        if (col_sum) col_sum[j] = s + rs;
        if (col_mag) col_mag[j] = m;
    }
    return 0;
}

// The A operand as the contraction sees it, materialised: H[i,k] = a_{i,k}
// for the rows selected (rows == NULL: all).  Used by the pins that check
// swiglu_a(G, U, W, R) == matmul_residual(silu(G)*U, W, R).
int oracle_a_rows(const float *A, const float *U, int64_t M, int64_t K,
                  const int64_t *rows, int64_t nrows, double *H) {
    if (A == nullptr || H == nullptr || M < 0 || K < 0) return -1;
    if (rows == nullptr) nrows = M;
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows ? rows[r] : r;
        if (i < 0 || i >= M) return -1;
        for (int64_t k = 0; k < K; ++k) H[r * K + k] = a_value(A, U, i * K + k);
    }
    return 0;
}

// Same contraction as oracle_gemm_rows with a double-precision A operand
// (used by the swiglu identity pin: feed the materialised H back in).
int oracle_gemm_rows_f64a(const double *A, const void *W, int w_is_f16, const float *R,
                          int64_t M, int64_t K, int64_t N, double *Yref, int nthreads) {
    if (A == nullptr || W == nullptr || Yref == nullptr) return -1;
    if (M < 0 || K < 0 || N < 0) return -1;
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
    {
        std::vector<double> acc(static_cast<size_t>(N));
#pragma omp for schedule(dynamic, 1)
        for (int64_t i = 0; i < M; ++i) {
            for (int64_t j = 0; j < N; ++j) acc[j] = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double aik = A[i * K + k];
                for (int64_t j = 0; j < N; ++j) {
                    const size_t idx = static_cast<size_t>(k) * N + j;
                    const double wkj = w_is_f16
                        ? oracle_half_to_double(static_cast<const uint16_t *>(W)[idx])
                        : static_cast<double>(static_cast<const float *>(W)[idx]);
                    acc[j] += aik * wkj;
                }
            }
            for (int64_t j = 0; j < N; ++j)
                Yref[i * N + j] = R ? acc[j] + static_cast<double>(R[i * N + j]) : acc[j];
        }
    }
    return 0;
}

}  // extern "C"
