// Host-side tables of the DiT step: RoPE rows and the FlowMatch Euler sigma
// schedule.  Built with -ffp-contract=off so each float operation is one
// IEEE-rounded operation, as the host contract's fp32 arithmetic requires.
#include <cmath>
#include <cstdint>
#include <vector>

#include "../../include/qi.h"

namespace {
constexpr int kPosMin = -1024, kPosMax = 8191, kRows = kPosMax - kPosMin + 1;  // 9216 rows

// One axis of the RoPE tables (Host contract -- RGBA-Image-2.1, s.4): entry
// (p, k) is the unit complex number at angle p * w_k, with the inverse
// frequency w_k = 1 / 10000^(2k/d), for positions p = -1024..8191.  The
// contract requires these tables bit-exact, so each arithmetic step is one
// fp32 operation: the exponent 2k/d, the power (evaluated in double and
// rounded once), its reciprocal, and the product with the position; cos and
// sin of the fp32 angle are evaluated in double and rounded once.
void axis_table(int d, float *c, float *s) {
  const int P = d / 2;
  for (int k = 0; k < P; ++k) {
    const float ex = (float)(2 * k) / (float)d;
    const float pw = (float)std::pow(10000.0, (double)ex);
    const float fr = 1.0f / pw;
    for (int p = kPosMin; p <= kPosMax; ++p) {
      const float ang = (float)p * fr;
      const size_t i = (size_t)(p - kPosMin) * P + k;
      c[i] = (float)std::cos((double)ang);
      s[i] = (float)std::sin((double)ang);
    }
  }
}
}  // namespace

extern "C" {

qi_status qi_rope_axis_table(int32_t d, float *cos_out, float *sin_out) {
  if (!cos_out || !sin_out) return QI_ERR_NULL;
  if (d < 2 || d > 128 || (d & 1)) return QI_ERR_RANGE;
  axis_table(d, cos_out, sin_out);
  return QI_OK;
}

// Host contract s.4: text token i -> (i, i, i); image token (y, x) ->
// (L, y - (h - h/2), x - (w - w/2)); rows = axis-0 (d 16) ++ axis-1 (d 56) ++
// axis-2 (d 56) table rows of those positions.
qi_status qi_rope_tables(int32_t L, int32_t h, int32_t w, float *txt_cos, float *txt_sin, float *img_cos,
                         float *img_sin) {
  if (L < 0 || h < 1 || w < 1) return QI_ERR_RANGE;
  if ((L > 0 && (!txt_cos || !txt_sin)) || !img_cos || !img_sin) return QI_ERR_NULL;
  const int ylo = -(h - h / 2), yhi = h - 1 - (h - h / 2);
  const int xlo = -(w - w / 2), xhi = w - 1 - (w - w / 2);
  if (L - 1 > kPosMax || L > kPosMax || ylo < kPosMin || xlo < kPosMin || yhi > kPosMax || xhi > kPosMax)
    return QI_ERR_RANGE;
  std::vector<float> c0((size_t)kRows * 8), s0((size_t)kRows * 8), c1((size_t)kRows * 28),
      s1((size_t)kRows * 28);
  axis_table(16, c0.data(), s0.data());
  axis_table(56, c1.data(), s1.data());  // axes 1 and 2 share width 56, hence one table
  auto put = [&](float *co, float *so, int f, int hy, int wx) {
    const size_t r0 = (size_t)(f - kPosMin), r1 = (size_t)(hy - kPosMin), r2 = (size_t)(wx - kPosMin);
    for (int k = 0; k < 8; ++k) {
      co[k] = c0[r0 * 8 + k];
      so[k] = s0[r0 * 8 + k];
    }
    for (int k = 0; k < 28; ++k) {
      co[8 + k] = c1[r1 * 28 + k];
      so[8 + k] = s1[r1 * 28 + k];
      co[36 + k] = c1[r2 * 28 + k];
      so[36 + k] = s1[r2 * 28 + k];
    }
  };
  for (int i = 0; i < L; ++i) put(txt_cos + (size_t)i * 64, txt_sin + (size_t)i * 64, i, i, i);
  for (int y = 0; y < h; ++y)
    for (int x = 0; x < w; ++x) {
      const size_t t = (size_t)y * w + x;
      put(img_cos + t * 64, img_sin + t * 64, L, y - (h - h / 2), x - (w - w / 2));
    }
  return QI_OK;
}

// The FlowMatch Euler schedule (Host contract -- RGBA-Image-2.1, s.6).  The
// schedule is a uniform grid from 1 down to 1/steps, bent by the exponential
// time shift s -> e^mu / (e^mu + 1/s - 1) whose strength mu grows linearly
// with the image token count (0.5 at 256 tokens, 0.9 at 8192: the constants
// that give the contract's printed mu values), then stretched affinely in
// 1 - s so that the last value lands on 0.02; timesteps are the sigmas times
// 1000, and a final sigma 0 is appended.  The contract gates sigmas bit for
// bit, so the fp32 operation order is fixed: the grid points are computed in
// double as start + i * step (the last one set to the end value) and rounded
// once, mu and e^mu in double rounded once, and every later array operation
// is one fp32 operation.
qi_status qi_flow_sigmas(int32_t steps, int32_t n_img_tokens, float *sigmas, float *timesteps) {
  if (!sigmas || !timesteps) return QI_ERR_NULL;
  if (steps < 2 || steps > 100000 || n_img_tokens < 1) return QI_ERR_RANGE;
  const double base_shift = 0.5, max_shift = 0.9, base_seq = 256.0, max_seq = 8192.0;
  const double m = (max_shift - base_shift) / (max_seq - base_seq);
  const double b = base_shift - m * base_seq;
  const double mu = (double)n_img_tokens * m + b;
  const float em = (float)std::exp(mu);
  const double start = 1.0, stop = 1.0 / steps, step = (stop - start) / (double)(steps - 1);
  std::vector<float> s(steps);
  for (int i = 0; i < steps; ++i) {
    const double v = (i == steps - 1) ? stop : (double)i * step + start;
    s[i] = (float)v;
  }
  const float one = 1.0f;
  for (int i = 0; i < steps; ++i) s[i] = em / (em + (one / s[i] - one));
  const float denom = (one - s[steps - 1]) / (one - 0.02f);
  for (int i = 0; i < steps; ++i) s[i] = one - (one - s[i]) / denom;
  for (int i = 0; i < steps; ++i) {
    sigmas[i] = s[i];
    timesteps[i] = s[i] * 1000.0f;
  }
  sigmas[steps] = 0.0f;
  return QI_OK;
}

// Encoder RoPE rows (the encoder declaration's rule): steps rounded to fp32,
// pow / cos / sin evaluated in double and rounded once.
qi_status qi_enc_rope_table(int32_t L, float theta, float *cos_out, float *sin_out) {
  if (!cos_out || !sin_out) return QI_ERR_NULL;
  if (L < 1 || L > 1000000 || !(theta > 1.0f)) return QI_ERR_RANGE;
  float inv[64];
  for (int i = 0; i < 64; ++i) {
    const float e = (float)(2 * i) / 128.0f;
    const float pw = (float)std::pow((double)theta, (double)e);
    inv[i] = 1.0f / pw;
  }
  for (int p = 0; p < L; ++p)
    for (int i = 0; i < 64; ++i) {
      const float a = (float)p * inv[i];
      cos_out[(size_t)p * 64 + i] = (float)std::cos((double)a);
      sin_out[(size_t)p * 64 + i] = (float)std::sin((double)a);
    }
  return QI_OK;
}

// DPM++ 2M coefficients (DPM-Solver++(2M), Lu et al. 2022, written for the
// flow x = (1 - sigma) x0 + sigma eps): alpha = 1 - sigma, lambda =
// log(alpha / sigma), x_next = a x - b D with a = sigma_next / sigma_cur,
// b = alpha_next (e^-h - 1), h = lambda_next - lambda_cur, and
// D = c1 x0 - c2 x0_prev, c2 = 1 / (2 r), r = h_prev / h, c1 = 1 + c2.  First
// order (c1 = 1, c2 = 0) without a previous prediction, after sigma = 1 (r
// infinite) and at the final step (sigma_next = 0: a = 0, b = -1, x_next = x0).
// Returns the order (1 or 2).  Double precision throughout.
static double flow_lambda(double s) { return s >= 1.0 ? -INFINITY : std::log1p(-s) - std::log(s); }

qi_status qi_dpmpp_2m_coeffs(int32_t has_prev, float sigma_prev, float sigma_cur, float sigma_next, double *coef) {
  if (!coef) return QI_ERR_NULL;
  const double sp = sigma_prev, sc = sigma_cur, sn = sigma_next;
  if (!(sc > 0.0 && sc <= 1.0) || !(sn >= 0.0 && sn < sc) || (has_prev && !(sp > sc && sp <= 1.0)))
    return QI_ERR_RANGE;
  if (sn <= 0.0) {
    coef[0] = 0.0; coef[1] = -1.0; coef[2] = 1.0; coef[3] = 0.0;
    return 1;
  }
  const double h = flow_lambda(sn) - flow_lambda(sc);
  coef[0] = sn / sc;
  coef[1] = (1.0 - sn) * std::expm1(-h);
  coef[2] = 1.0;
  coef[3] = 0.0;
  if (!has_prev) return 1;
  const double r = (flow_lambda(sc) - flow_lambda(sp)) / h;
  if (std::isinf(r)) return 1;
  coef[3] = 1.0 / (2.0 * r);
  coef[2] = 1.0 + coef[3];
  return 2;
}

}  // extern "C"
