/*
 * Rotary cos/sin tables for the QSA oracle -- TEST INFRASTRUCTURE ONLY.
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg use
 * the oracle; the product path never links or loads this file.
 *
 * Each entry is the host libm cos/sin of the fp64 angle pos * inv_freq[j],
 * rounded once to fp32 (the rotary phases of the QSA core and indexer; the
 * frequencies come from the rope_parameters block of the PyTorchKR post
 * "Qwen3.8-Flash-Next, 1/9의 학습 비용으로 Qwen3.7-Plus(397B-A17B) 수준에 도달한
 * 125B-A6B 모델", section "100만 토큰까지 늘리기").
 *
 * Built with -fno-builtin so that the compiler calls cos() and sin() as written
 * and never substitutes its own expansion or a fused sincos.
 */
#include <math.h>
#include <stdint.h>

void oracle_rope_table(const double *inv_freq, int32_t n_freq,
                       const int64_t *pos, int64_t n_pos,
                       float *cos_out, float *sin_out)
{
    for (int64_t i = 0; i < n_pos; ++i) {
        for (int32_t j = 0; j < n_freq; ++j) {
            double angle = (double)pos[i] * inv_freq[j];
            cos_out[i * n_freq + j] = (float)cos(angle);
            sin_out[i * n_freq + j] = (float)sin(angle);
        }
    }
}
