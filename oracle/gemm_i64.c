/* Oracle integer GEMM: a plain triple loop with 64-bit accumulation.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product library links or calls this.
 *
 * acc[m][n] = sum_k q[m][k] * w[n][k]
 *
 * q holds the activation codes (int8 for W4A8, int4 values for W4A4) and w the
 * weight codes with the zero point already taken off (c - z, in [-15, 15]).
 * This is the "INT8 GEMM" step of the ConvRot forward pass (ComfyUI-INT-Crush
 * README, "Inference / INT4" and "Forward Pass" step 5) written out as its
 * definition, with no blocking and no reordering: one multiply-add per (m, n, k),
 * k running upward. Rows m are split over OpenMP threads; each output element is
 * still summed by one thread in k order.
 */
#include <stdint.h>

int oracle_gemm_i64(const int8_t *q, const int8_t *w, int64_t M, int64_t N, int64_t K,
                    int64_t *acc)
{
    if (M < 0 || N < 0 || K < 0) return 1;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)q[m * K + k] * (int64_t)w[n * K + k];
            acc[m * N + n] = s;
        }
    }
    return 0;
}

int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            extern int omp_get_num_threads(void);
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}
