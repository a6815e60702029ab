/*
 * Oracle (test infrastructure only): router logits of the MoE layer in the one
 * canonical float32 order the whole project uses.
 *
 * The router is the small linear layer that scores every token against every
 * expert (Perplexity, "Enabling trillion-parameter models on AWS EFA", 2025,
 * introduction: a linear routing layer decides which expert multiplies a token).
 * The article fixes neither the precision nor the summation order. Because the
 * logits decide integers (which experts a token goes to), the oracle and the GPU
 * library take that decision in the same precision and the same order:
 *
 *     acc_0 = +0.0f,   acc_{i+1} = fmaf(x[t,i], w[e,i], acc_i)   for i = 0 .. d-1,
 *     logit[t,e] = acc_d
 *
 * i.e. one fused multiply-add per input element, in index order, rounded to
 * float32 after every step. No bias. With bf16 inputs every product is exact in
 * float32, so this is also the sequentially rounded float32 sum of the products.
 *
 * Built by oracle/build.py with gcc; never linked into the GPU library.
 */
#include <math.h>
#include <stdint.h>

void oracle_router_logits_f32(const float *x, const float *w, int64_t T, int64_t d,
                              int64_t E, float *out)
{
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        const float *xt = x + t * d;
        for (int64_t e = 0; e < E; ++e) {
            const float *we = w + e * d;
            float acc = 0.0f;
            for (int64_t i = 0; i < d; ++i)
                acc = fmaf(xt[i], we[i], acc);
            out[t * E + e] = acc;
        }
    }
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
