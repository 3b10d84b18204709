// NF4 blockwise codec on the host (the load-time quantizer of the frozen base).
//
// The pages name the format only: the streamed base is optionally quantized
// to NF4, about four times smaller than fp16 ("Soup: Fine-Tune an 8B Model on a
// 4 GB GPU", "The Core Idea: Layer Streaming").  Construction used here:
//   levels: 8 positive standard-normal quantiles at the first 8 of 9 evenly
//   spaced probabilities from 1-delta down to 1/2, 7 negative ones from the
//   first 7 of 8 such points (mirrored), and an exact 0; divided by the
//   largest; delta = (1/32 + 1/30)/2.  Quantiles come from inverting the
//   normal CDF 0.5*erfc(-x/sqrt 2) by bisection in double precision; each
//   level and each midpoint (c_j + c_{j+1})/2 is then rounded once to fp32.
//   code(w) = number of fp32 midpoints strictly below fl32(w / absmax) with
//   absmax = max |w| over 64 consecutive elements; an all-zero block stores
//   absmax 0 and code 7 everywhere.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <thread>
#include <vector>

#include "host_codec.h"

namespace lsn {

static double normal_cdf(double x) { return 0.5 * erfc(-x / sqrt(2.0)); }

static double normal_quantile(double p) {
  double lo = -12.0, hi = 12.0;
  for (int i = 0; i < 200; ++i) {
    const double mid = 0.5 * (lo + hi);
    if (normal_cdf(mid) < p)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

struct Nf4Tables {
  double lv64[16];
  float lv[16];
  float mid[15];
  Nf4Tables() {
    const double delta = 0.5 * (1.0 / 32.0 + 1.0 / 30.0);
    const double top = 1.0 - delta;
    double v[16];
    int n = 0;
    for (int i = 0; i < 8; ++i) {  // 9 points top .. 0.5, drop the last
      const double p = top + (0.5 - top) * i / 8.0;
      v[n++] = normal_quantile(p);
    }
    for (int i = 0; i < 7; ++i) {  // 8 points top .. 0.5, drop the last
      const double p = top + (0.5 - top) * i / 7.0;
      v[n++] = -normal_quantile(p);
    }
    v[n++] = 0.0;
    std::sort(v, v + 16);
    const double mx = v[15];
    for (int i = 0; i < 16; ++i) {
      lv64[i] = v[i] / mx;
      lv[i] = (float)lv64[i];
    }
    lv64[15] = 1.0;
    lv[15] = 1.0f;
    for (int i = 0; i < 15; ++i) mid[i] = (float)((lv64[i] + lv64[i + 1]) / 2.0);
  }
};

static const Nf4Tables& tables() {
  static const Nf4Tables t;
  return t;
}

void nf4_levels(float out[16]) { memcpy(out, tables().lv, sizeof(float) * 16); }

static inline uint8_t code_of(float x, const float* mid) {
  uint8_t c = 0;
  for (int j = 0; j < 15; ++j) c += (x > mid[j]) ? 1 : 0;
  return c;
}

static void quantize_blocks(const float* w, uint64_t n, uint64_t b0, uint64_t b1, uint8_t* codes,
                            float* absmax) {
  const float* mid = tables().mid;
  uint8_t cb[64];
  for (uint64_t b = b0; b < b1; ++b) {
    const uint64_t e0 = b * 64, e1 = std::min<uint64_t>(e0 + 64, n);
    float a = 0.f;
    for (uint64_t e = e0; e < e1; ++e) a = std::max(a, fabsf(w[e]));
    absmax[b] = a;
    const int len = (int)(e1 - e0);
    for (int i = 0; i < len; ++i) {
      if (a == 0.f) {
        cb[i] = 7;
      } else {
        volatile float x = w[e0 + i] / a;  // one IEEE fp32 division
        cb[i] = code_of(x, mid);
      }
    }
    for (int i = len; i < 64; ++i) cb[i] = 0;
    const uint64_t nbytes = (uint64_t)(len + 1) / 2;
    for (uint64_t i = 0; i < nbytes; ++i)
      codes[e0 / 2 + i] = (uint8_t)(cb[2 * i] | (cb[2 * i + 1] << 4));
  }
}

bool nf4_quantize(const float* w, uint64_t n, uint8_t* codes, float* absmax) {
  // reject non-finite input
  std::atomic<bool> bad{false};
  const uint64_t nblocks = (n + 63) / 64;
  unsigned nt = std::max(1u, std::min(16u, std::thread::hardware_concurrency()));
  if (nblocks < 4096) nt = 1;
  auto check = [&](uint64_t lo, uint64_t hi) {
    for (uint64_t e = lo; e < hi; ++e)
      if (!std::isfinite(w[e])) {
        bad = true;
        return;
      }
  };
  {
    std::vector<std::thread> th;
    for (unsigned t = 0; t < nt; ++t)
      th.emplace_back(check, n * t / nt, n * (t + 1) / nt);
    for (auto& x : th) x.join();
  }
  if (bad) return false;
  std::vector<std::thread> th;
  for (unsigned t = 0; t < nt; ++t)
    th.emplace_back(quantize_blocks, w, n, nblocks * t / nt, nblocks * (t + 1) / nt, codes,
                    absmax);
  for (auto& x : th) x.join();
  return true;
}

void nf4_dequantize_host(const uint8_t* codes, const float* absmax, uint64_t n, float* w) {
  const float* lv = tables().lv;
  for (uint64_t e = 0; e < n; ++e) {
    const uint8_t byte = codes[e >> 1];
    const uint8_t c = (e & 1) ? (byte >> 4) : (byte & 15);
    w[e] = lv[c] * absmax[e >> 6];
  }
}

}  // namespace lsn
