// Host-side rotary tables of the QSA library.
//
// Frequencies: omega_j = theta^(-2j/64), j = 0..31, theta = 1e7 and 64 rotary
// dims (PyTorchKR post "Qwen3.8-Flash-Next, 1/9의 학습 비용으로 …", section
// "100만 토큰까지 늘리기": rope_theta, partial_rotary_factor 0.25; the M-RoPE
// sections [11, 11, 10] share one position for text, leaving plain 1-D RoPE).
// With a YaRN factor s > 1 each pair follows the NTK-by-parts ramp of Peng et
// al. 2023: r_j = L_orig * omega_j / (2 pi), gamma_j = clamp((r_j - 1) / 31, 0, 1),
// omega'_j = (1 - gamma_j) * omega_j / s + gamma_j * omega_j.
//
// Each table entry is libm cos/sin of the fp64 angle position * omega'_j,
// rounded once to fp32.  This file is compiled with -fno-builtin and
// -ffp-contract=off so the expressions are evaluated exactly as written.
#include <math.h>
#include <stdint.h>

namespace qsa {

void host_inv_freq(double theta, double yarn_factor, int64_t yarn_orig_ctx, double *out /*[32]*/)
{
    for (int j = 0; j < 32; ++j) {
        double w = pow(theta, -(2.0 * j) / 64.0);
        if (yarn_factor > 1.0) {
            double wavelength = 2.0 * M_PI / w;
            double r = (double)yarn_orig_ctx / wavelength;
            double g = (r - 1.0) / (32.0 - 1.0);
            g = g < 0.0 ? 0.0 : (g > 1.0 ? 1.0 : g);
            w = (1.0 - g) * w / yarn_factor + g * w;
        }
        out[j] = w;
    }
}

void host_rope_tables(const double *inv_freq, int64_t n_pos, float *cos_out, float *sin_out)
{
    for (int64_t p = 0; p < n_pos; ++p) {
        for (int j = 0; j < 32; ++j) {
            double angle = (double)p * inv_freq[j];
            cos_out[p * 32 + j] = (float)cos(angle);
            sin_out[p * 32 + j] = (float)sin(angle);
        }
    }
}

}  // namespace qsa
