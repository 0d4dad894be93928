/*
 * A C client of the rd library: no Python, no torch.  It allocates device
 * memory with the HIP runtime, creates a stream, calls the entry points of
 * include/rd.h on integer-valued data and compares every output with the
 * CPU oracle (oracle/liboracle.so) -- bit for bit, since integer sums below
 * 2^24 are exact in any order.  It also checks a few error codes.  Built
 * and run by tests/test_gpu_c_client.py; prints "c client ok" and exits 0
 * on success, prints the first mismatch and exits 1 otherwise.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "rd.h"

/* the oracle's entry points (oracle/oracle.c), linked from liboracle.so */
void oracle_sum_1d(const float* x, int64_t n, double* sum, double* abs_sum);
void oracle_reduce_dim(const float* x, int64_t outer, int64_t R, int64_t inner, int op,
                       double* out, double* abs_out, int nthreads);
void oracle_sum_dim(const float* x, int64_t outer, int64_t R, int64_t inner, double* out,
                    double* abs_out, int nthreads);
void oracle_cumsum_dim(const float* x, int64_t outer, int64_t R, int64_t inner, int reverse,
                       double* out, double* abs_out, int nthreads);
void oracle_softmax_denom_dim(const float* x, int64_t outer, int64_t R, int64_t inner,
                              double* m_out, double* s_out, int nthreads);

#define HIP_OK(call)                                                        \
    do {                                                                    \
        hipError_t e_ = (call);                                             \
        if (e_ != hipSuccess) {                                             \
            fprintf(stderr, "%s failed: %d\n", #call, (int)e_);             \
            exit(1);                                                        \
        }                                                                   \
    } while (0)

#define RD_OK_(call)                                                        \
    do {                                                                    \
        rd_status s_ = (call);                                              \
        if (s_ != RD_OK) {                                                  \
            fprintf(stderr, "%s: %s (hip %d)\n", #call, rd_status_string(s_), \
                    rd_last_hip_error());                                   \
            exit(1);                                                        \
        }                                                                   \
    } while (0)

static int same_bits(const float* got, const double* want, int64_t n, const char* what) {
    for (int64_t k = 0; k < n; ++k) {
        float w = (float)want[k];
        if (memcmp(&got[k], &w, sizeof(float)) != 0) {
            fprintf(stderr, "%s: output %lld is %.9g, the oracle says %.9g\n", what, (long long)k,
                    got[k], w);
            return 0;
        }
    }
    return 1;
}

int main(void) {
    const int64_t outer = 37, R = 5003, inner = 129, n = outer * R * inner;
    float* h = (float*)malloc((size_t)n * sizeof(float));
    uint64_t st = 12345;
    for (int64_t k = 0; k < n; ++k) {  /* integers in [-8, 8] from a 64-bit LCG */
        st = st * 6364136223846793005ull + 1442695040888963407ull;
        h[k] = (float)((int)((st >> 33) % 17) - 8);
    }
    float *x, *out, *out2;
    hipStream_t s;
    HIP_OK(hipStreamCreate(&s));
    HIP_OK(hipMalloc((void**)&x, (size_t)n * sizeof(float)));
    HIP_OK(hipMalloc((void**)&out, (size_t)n * sizeof(float)));
    HIP_OK(hipMalloc((void**)&out2, (size_t)outer * inner * sizeof(float)));
    HIP_OK(hipMemcpy(x, h, (size_t)n * sizeof(float), hipMemcpyHostToDevice));

    float* g = (float*)malloc((size_t)n * sizeof(float));
    float* g2 = (float*)malloc((size_t)outer * inner * sizeof(float));
    double* w = (double*)malloc((size_t)n * sizeof(double));
    double* a = (double*)malloc((size_t)n * sizeof(double));
    int ok = 1;

    /* full reduce */
    RD_OK_(rd_sum_1d(x, n, out, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(g, out, sizeof(float), hipMemcpyDeviceToHost));
    oracle_sum_1d(h, n, w, a);
    ok &= same_bits(g, w, 1, "rd_sum_1d");

    /* axis reduces: the sum and the maximum over the middle axis */
    RD_OK_(rd_sum_dim(x, outer, R, inner, out, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(g, out, (size_t)outer * inner * sizeof(float), hipMemcpyDeviceToHost));
    oracle_sum_dim(h, outer, R, inner, w, a, 0);
    ok &= same_bits(g, w, outer * inner, "rd_sum_dim");
    RD_OK_(rd_reduce_dim(x, outer, R, inner, RD_OP_MAX, out, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(g, out, (size_t)outer * inner * sizeof(float), hipMemcpyDeviceToHost));
    oracle_reduce_dim(h, outer, R, inner, 2, w, a, 0);
    ok &= same_bits(g, w, outer * inner, "rd_reduce_dim max");

    /* a strided view: the first axis transposed away -- sums over the outer
       axis of [outer, R*inner] read as [1, outer, R*inner] with stride R*inner */
    RD_OK_(rd_reduce_strided(x, 1, outer, R * inner, 0, R * inner, 1, RD_OP_SUM, out, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(g, out, (size_t)R * inner * sizeof(float), hipMemcpyDeviceToHost));
    oracle_sum_dim(h, 1, outer, R * inner, w, a, 0);
    ok &= same_bits(g, w, R * inner, "rd_reduce_strided");

    /* the reverse cumulative sum along the middle axis */
    RD_OK_(rd_cumsum_dim(x, outer, R, inner, 1, out, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(g, out, (size_t)n * sizeof(float), hipMemcpyDeviceToHost));
    oracle_cumsum_dim(h, outer, R, inner, 1, w, a, 0);
    ok &= same_bits(g, w, n, "rd_cumsum_dim");

    /* the forward cumulative sum over the transposed view [R*inner, outer]
       (stride 1 between outputs, R*inner along the scan), contiguous out */
    {
        const int64_t P = R * inner;
        float* ht = (float*)malloc((size_t)n * sizeof(float));
        for (int64_t o = 0; o < outer; ++o)
            for (int64_t p = 0; p < P; ++p) ht[p * outer + o] = h[o * P + p];
        RD_OK_(rd_cumsum_strided(x, P, outer, 1, 1, P, 1, 0, out, s));
        HIP_OK(hipStreamSynchronize(s));
        HIP_OK(hipMemcpy(g, out, (size_t)n * sizeof(float), hipMemcpyDeviceToHost));
        oracle_cumsum_dim(ht, P, outer, 1, 0, w, a, 0);
        ok &= same_bits(g, w, n, "rd_cumsum_strided");
        free(ht);
    }

    /* the softmax denominator on terms 0 / -Inf: s counts the zeros exactly */
    for (int64_t k = 0; k < n; ++k) h[k] = h[k] > 0 ? 0.f : -__builtin_inff();
    HIP_OK(hipMemcpy(x, h, (size_t)n * sizeof(float), hipMemcpyHostToDevice));
    RD_OK_(rd_softmax_denom_dim(x, outer, R, inner, out, out2, s));
    HIP_OK(hipStreamSynchronize(s));
    HIP_OK(hipMemcpy(g, out, (size_t)outer * inner * sizeof(float), hipMemcpyDeviceToHost));
    HIP_OK(hipMemcpy(g2, out2, (size_t)outer * inner * sizeof(float), hipMemcpyDeviceToHost));
    oracle_softmax_denom_dim(h, outer, R, inner, w, a, 0);
    ok &= same_bits(g, w, outer * inner, "rd_softmax_denom_dim max");
    ok &= same_bits(g2, a, outer * inner, "rd_softmax_denom_dim sum");

    /* error codes: nothing enqueued, outputs untouched */
    ok &= rd_sum_1d(x, -1, out, s) == RD_ERR_INVALID_ARG;
    ok &= rd_sum_dim(x, outer, R, inner, (float*)((char*)out + 2), s) == RD_ERR_INVALID_ARG;
    ok &= rd_reduce_dim(x, outer, R, inner, 9, out, s) == RD_ERR_INVALID_ARG;
    ok &= rd_sum_dim(x, outer, R, inner, x + 5, s) == RD_ERR_INVALID_ARG;  /* overlap */
    if (!ok) {
        fprintf(stderr, "c client: mismatch or unexpected status\n");
        return 1;
    }
    HIP_OK(hipFree(x));
    HIP_OK(hipFree(out));
    HIP_OK(hipFree(out2));
    HIP_OK(hipStreamDestroy(s));
    free(h), free(g), free(g2), free(w), free(a);
    printf("c client ok (version %d)\n", rd_version());
    return 0;
}
