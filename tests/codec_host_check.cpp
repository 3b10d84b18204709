// Host NF4 codec under the sanitizers (built by tests/test_host_sanitizers.py
// with g++ -fsanitize=address,undefined, and separately with
// -fsanitize=thread for the multithreaded quantizer).  For several lengths,
// including odd ones, partial last blocks, all-zero blocks and lengths that
// take the multithreaded path, it quantizes seeded normal weights, checks
// every absmax against the block's largest magnitude, checks that every
// code lies in 0..15 and that an odd length leaves the last byte's high
// nibble zero, dequantizes, and requantizes the dequantized weights: the
// codes and absmax must come back unchanged (the round trip is exact).
// Prints "ok <cases>" and exits 0, or the first failure and exits 1.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <random>
#include <vector>

#include "../layer_streamed_nf4_double_amd/csrc/host_codec.h"

static int fail(const char* what, uint64_t n, uint64_t i) {
  printf("FAIL %s n=%llu at %llu\n", what, (unsigned long long)n, (unsigned long long)i);
  return 1;
}

int main() {
  const uint64_t lengths[] = {1, 2, 3, 63, 64, 65, 127, 688 * 3, 4096 * 64 + 37, 4096 * 64 * 5};
  std::mt19937_64 rng(12345);
  std::normal_distribution<float> nd(0.f, 0.02f);
  int cases = 0;
  for (uint64_t n : lengths) {
    for (int zero_blocks = 0; zero_blocks < 2; ++zero_blocks) {
      std::vector<float> w(n);
      for (auto& x : w) x = nd(rng);
      if (zero_blocks)
        for (uint64_t e = 0; e < n; ++e)
          if ((e / 64) % 3 == 1) w[e] = 0.f;
      const uint64_t nb = (n + 63) / 64, nc = (n + 1) / 2;
      std::vector<uint8_t> codes(nc, 0xAB), codes2(nc, 0xCD);
      std::vector<float> amax(nb, -1.f), amax2(nb, -2.f), deq(n);
      if (!lsn::nf4_quantize(w.data(), n, codes.data(), amax.data())) return fail("quantize", n, 0);
      for (uint64_t b = 0; b < nb; ++b) {
        float m = 0.f;
        for (uint64_t e = b * 64; e < std::min<uint64_t>(n, b * 64 + 64); ++e) m = fmaxf(m, fabsf(w[e]));
        if (m != amax[b]) return fail("absmax", n, b);
      }
      if ((n & 1) && (codes[nc - 1] >> 4) != 0) return fail("odd tail nibble", n, nc - 1);
      lsn::nf4_dequantize_host(codes.data(), amax.data(), n, deq.data());
      if (!lsn::nf4_quantize(deq.data(), n, codes2.data(), amax2.data())) return fail("requantize", n, 0);
      if (memcmp(codes.data(), codes2.data(), nc) != 0) return fail("round-trip codes", n, 0);
      if (memcmp(amax.data(), amax2.data(), nb * sizeof(float)) != 0) return fail("round-trip absmax", n, 0);
      ++cases;
    }
  }
  // non-finite input is refused
  std::vector<float> w(300, 0.01f);
  std::vector<uint8_t> c(150);
  std::vector<float> a(5);
  w[77] = NAN;
  if (lsn::nf4_quantize(w.data(), w.size(), c.data(), a.data())) return fail("NaN accepted", 300, 77);
  w[77] = INFINITY;
  if (lsn::nf4_quantize(w.data(), w.size(), c.data(), a.data())) return fail("Inf accepted", 300, 77);
  printf("ok %d\n", cases + 2);
  return 0;
}
