// Test program for the oracle built with AddressSanitizer and UndefinedBehavior-
// Sanitizer (host code, g++): brute-force integer products (all variants,
// row subsets, binary16 weights), the binary16 decoder over every pattern,
// row/column sums, and the argument checks.  Exits non-zero on a mismatch;
// the sanitizers abort on a memory or undefined-behaviour error.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

extern "C" {
double oracle_half_to_double(uint16_t h);
double oracle_sigmoid(double x);
double oracle_silu(double x);
int oracle_gemm_rows(const float *A, const float *U, const void *W, int w_is_f16, const float *R, int64_t M,
                     int64_t K, int64_t N, const int64_t *rows, int64_t nrows, double *Yref, double *Bscale,
                     int nthreads);
int oracle_row_col_sums(const float *A, const float *U, const void *W, int w_is_f16, const float *R, int64_t M,
                        int64_t K, int64_t N, double *row_sum, double *row_mag, double *col_sum, double *col_mag,
                        int nthreads);
int oracle_a_rows(const float *A, const float *U, int64_t M, int64_t K, const int64_t *rows, int64_t nrows,
                  double *H);
int oracle_gemm_rows_f64a(const double *A, const void *W, int w_is_f16, const float *R, int64_t M, int64_t K,
                          int64_t N, double *Yref, int nthreads);
}

static int failures = 0;
#define CHECK(c)                                                         \
    do {                                                                 \
        if (!(c)) {                                                      \
            std::fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
            ++failures;                                                  \
        }                                                                \
    } while (0)

static uint32_t lcg(uint32_t &s) { return s = s * 1664525u + 1013904223u; }

int main() {
    uint32_t seed = 12345;
    // every binary16 pattern decodes without fault; spot values
    for (uint32_t h = 0; h < 65536; ++h) (void)oracle_half_to_double(static_cast<uint16_t>(h));
    CHECK(oracle_half_to_double(0x3C00) == 1.0 && oracle_half_to_double(0x0001) == std::ldexp(1.0, -24));
    CHECK(oracle_sigmoid(0.0) == 0.5 && oracle_silu(0.0) == 0.0);
    const int shapes[][3] = {{1, 1, 1}, {3, 5, 7}, {8, 4, 2}, {7, 8, 5}, {16, 12, 9}};
    for (const auto &sh : shapes) {
        const int M = sh[0], K = sh[1], N = sh[2];
        std::vector<float> X(M * K), W(K * N), R(M * N);
        std::vector<uint16_t> W16(K * N);
        for (auto &v : X) v = static_cast<float>(static_cast<int>(lcg(seed) % 17) - 8);
        for (int i = 0; i < K * N; ++i) {
            const int w = static_cast<int>(lcg(seed) % 17) - 8;
            W[i] = static_cast<float>(w);
            // integers up to 8 in binary16: sign, exponent, fraction by hand
            uint16_t bits = 0;
            if (w != 0) {
                const int a = w < 0 ? -w : w;
                int e = 0;
                while ((a >> (e + 1)) != 0) ++e;
                const int frac = (a << (10 - e)) & 0x3ff;
                bits = static_cast<uint16_t>((w < 0 ? 0x8000 : 0) | ((e + 15) << 10) | frac);
            }
            W16[i] = bits;
        }
        for (auto &v : R) v = static_cast<float>(static_cast<int>(lcg(seed) % 17) - 8);
        std::vector<double> Y(M * N), B(M * N), Y16(M * N);
        CHECK(oracle_gemm_rows(X.data(), nullptr, W.data(), 0, R.data(), M, K, N, nullptr, 0, Y.data(), B.data(),
                               2) == 0);
        CHECK(oracle_gemm_rows(X.data(), nullptr, W16.data(), 1, R.data(), M, K, N, nullptr, 0, Y16.data(),
                               nullptr, 2) == 0);
        for (int i = 0; i < M; ++i)
            for (int j = 0; j < N; ++j) {
                long long y = 0, b = 0;
                for (int k = 0; k < K; ++k) {
                    y += static_cast<long long>(X[i * K + k]) * static_cast<long long>(W[k * N + j]);
                    b += std::llabs(static_cast<long long>(X[i * K + k]) * static_cast<long long>(W[k * N + j]));
                }
                y += static_cast<long long>(R[i * N + j]);
                CHECK(Y[i * N + j] == static_cast<double>(y) && Y16[i * N + j] == static_cast<double>(y));
                CHECK(B[i * N + j] == static_cast<double>(b));
            }
        // a row subset, in reverse order
        std::vector<int64_t> rows(M);
        for (int i = 0; i < M; ++i) rows[i] = M - 1 - i;
        std::vector<double> Ys(M * N);
        CHECK(oracle_gemm_rows(X.data(), nullptr, W.data(), 0, R.data(), M, K, N, rows.data(), M, Ys.data(),
                               nullptr, 2) == 0);
        for (int r = 0; r < M; ++r)
            for (int j = 0; j < N; ++j) CHECK(Ys[r * N + j] == Y[rows[r] * N + j]);
        // the SwiGLU variant through the materialised activation
        std::vector<float> U(M * K);
        for (auto &v : U) v = static_cast<float>(static_cast<int>(lcg(seed) % 9) - 4);
        std::vector<double> H(M * K), Ysw(M * N), Yh(M * N);
        CHECK(oracle_a_rows(X.data(), U.data(), M, K, nullptr, 0, H.data()) == 0);
        CHECK(oracle_gemm_rows(X.data(), U.data(), W.data(), 0, R.data(), M, K, N, nullptr, 0, Ysw.data(), nullptr,
                               2) == 0);
        CHECK(oracle_gemm_rows_f64a(H.data(), W.data(), 0, R.data(), M, K, N, Yh.data(), 2) == 0);
        for (int i = 0; i < M * N; ++i) CHECK(Ysw[i] == Yh[i]);
        // row and column sums against the full product
        std::vector<double> rs(M), rm(M), cs(N), cm(N);
        CHECK(oracle_row_col_sums(X.data(), nullptr, W.data(), 0, R.data(), M, K, N, rs.data(), rm.data(), cs.data(),
                                  cm.data(), 2) == 0);
        for (int i = 0; i < M; ++i) {
            double s = 0;
            for (int j = 0; j < N; ++j) s += Y[i * N + j];
            CHECK(std::fabs(s - rs[i]) <= 1e-9 * (1 + std::fabs(s)));
        }
    }
    // argument checks return -1 without touching memory
    double out[4];
    const float one = 1.0f;
    CHECK(oracle_gemm_rows(nullptr, nullptr, &one, 0, nullptr, 1, 1, 1, nullptr, 0, out, nullptr, 1) == -1);
    CHECK(oracle_gemm_rows(&one, nullptr, &one, 0, nullptr, -1, 1, 1, nullptr, 0, out, nullptr, 1) == -1);
    const int64_t bad_row = 5;
    CHECK(oracle_gemm_rows(&one, nullptr, &one, 0, nullptr, 1, 1, 1, &bad_row, 1, out, nullptr, 1) == -1);
    CHECK(oracle_a_rows(&one, nullptr, 1, 1, &bad_row, 1, out) == -1);
    CHECK(oracle_row_col_sums(nullptr, nullptr, &one, 0, nullptr, 1, 1, 1, nullptr, nullptr, nullptr, nullptr, 1) == -1);
    if (failures == 0) std::printf("oracle checks ok\n");
    return failures == 0 ? 0 : 1;
}
