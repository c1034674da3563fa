/*
 * Brute-force checker for the fused GEMM + tile-reduce result.
 * TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).
 *
 * out[i][j] = sum_k a[i][k] * b[k][j] + sum_p peers[p][i][j], all in double,
 * with a and b given as bfloat16 bit patterns.  This is the plain definition
 * of one rank's GEMM+AllReduce output (abstract of "mKernel: Fast Multi-GPU,
 * Multi-Node Fused Kernels"; GEMM + AllReduce row of the five-kernel tables
 * on the MarkTechPost and chathome pages), written as three nested loops so
 * that it shares nothing with the numpy path or the GPU path.
 */
#include <stdint.h>
#include <string.h>

static double bf16_value(uint16_t h)
{
    /* a bfloat16 pattern is the high half of a binary32 pattern */
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

void mk_brute_gemm_reduce(const uint16_t *a, const uint16_t *b, const float *peers,
                          int num_peers, int64_t m, int64_t n, int64_t k, double *out)
{
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int64_t kk = 0; kk < k; ++kk)
                acc += bf16_value(a[i * k + kk]) * bf16_value(b[kk * n + j]);
            for (int p = 0; p < num_peers; ++p)
                acc += (double)peers[((int64_t)p * m + i) * n + j];
            out[i * n + j] = acc;
        }
    }
}
