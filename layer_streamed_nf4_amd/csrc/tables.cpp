// The two code tables of the NF4 double-quant format, derived at load time
// from their published definitions, in double precision, then rounded once to
// fp32. The gate walkthrough ("Soup layer-streamed NF4 training measured",
// section 2.4) fixes only that there are 16 NF4 levels and 256 nested levels,
// fp32, identical for every weight and shared.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "common.h"

namespace nf4s {
namespace {

// Standard normal quantile by bisection on the complementary error function.
double normal_quantile(double p) {
  double lo = -10.0, hi = 10.0;
  for (int i = 0; i < 200; ++i) {
    double mid = 0.5 * (lo + hi);
    if (0.5 * std::erfc(-mid / std::sqrt(2.0)) < p)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

// NormalFloat-4 (QLoRA section 3): 8 equal-probability normal quantiles on the
// positive side, 7 on the negative side, one shared exact zero, normalised by
// the largest so the range is [-1, 1]. The outermost probability is the mean
// of the top-bin centres for 15 and 16 equal bins.
void build_nf4(float* out) {
  const double delta = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0));
  const double zmax = normal_quantile(delta);
  std::vector<double> v;
  for (int i = 0; i < 8; ++i) v.push_back(normal_quantile(delta - (delta - 0.5) * i / 8.0) / zmax);
  for (int i = 0; i < 7; ++i) v.push_back(-normal_quantile(delta - (delta - 0.5) * i / 7.0) / zmax);
  v.push_back(0.0);
  std::sort(v.begin(), v.end());
  v.front() = -1.0;
  v.back() = 1.0;
  for (int i = 0; i < 16; ++i) out[i] = (float)v[i];
}

// Signed dynamic-tree map (8-bit Optimizers via Block-wise Quantization,
// section 2): sign bit, a run of e zero bits giving the factor 10^-e, an
// indicator bit, then 6-e bits indexing linear bins of [0.1, 1] whose centres
// are the levels. The all-zero magnitude pattern encodes 0 (sign 0) and 1.0
// (sign 1). Enumerated here from the bit patterns.
void build_dynamic(float* out) {
  static const double pow10n[7] = {1.0, 0.1, 0.01, 0.001, 0.0001, 0.00001, 0.000001};
  std::vector<double> v;
  for (int code = 0; code < 256; ++code) {
    const bool neg = code & 0x80;
    const int bits = code & 0x7F;
    if (bits == 0) {
      v.push_back(neg ? 1.0 : 0.0);
      continue;
    }
    int e = 0;
    while (!((bits >> (6 - e)) & 1)) ++e;
    const int frac_bits = 6 - e;
    const int j = bits & ((1 << frac_bits) - 1);
    const int nbins = 1 << frac_bits;
    const double centre = 0.1 + 0.9 * (2.0 * j + 1.0) / (2.0 * nbins);
    const double mag = centre * pow10n[e];
    v.push_back(neg ? -mag : mag);
  }
  std::sort(v.begin(), v.end());
  for (int i = 0; i < 256; ++i) out[i] = (float)v[i];
}

struct State {
  Tables t;
  Mids4 m4;
  Mids8 m8;
  Buckets4 b4;
  uint64_t hash;
};

const State& state() {
  static State s;
  static std::once_flag once;
  std::call_once(once, [] {
    build_nf4(s.t.c4);
    build_dynamic(s.t.c8);
    // decision thresholds between consecutive levels, in fp32
    for (int i = 0; i < 15; ++i) s.m4.m[i] = (s.t.c4[i] + s.t.c4[i + 1]) * 0.5f;
    for (int i = 0; i < 255; ++i) s.m8.m[i] = (s.t.c8[i] + s.t.c8[i + 1]) * 0.5f;
    // the quantiser's bucket table (exact: t and the next fp32 sum in fp64)
    s.b4.ok = 1;
    for (int i = 0; i < 15; ++i) {
      const float t = s.m4.m[i];
      s.b4.b_mid[i] = ((double)t + (double)std::nextafter(t, INFINITY)) * 0.5;
      const double pos = ((double)t + 1.0) * 128.0;
      const double f = pos - std::floor(pos);
      if (f < 1.0 / 64 || f > 1.0 - 1.0 / 64) s.b4.ok = 0;
    }
    s.b4.b_mid[15] = INFINITY;
    for (int b = 0; b < 260; ++b) {
      const double lo = b / 128.0 - 1.0;
      int c = 0;
      for (int i = 0; i < 15; ++i) c += (double)s.m4.m[i] < lo;
      s.b4.code[b] = (uint8_t)c;
    }
    // FNV-1a 64 over the little-endian fp32 bytes, NF4 table then nested table
    uint64_t h = 0xCBF29CE484222325ull;
    auto eat = [&h](const float* p, int n) {
      const unsigned char* b = reinterpret_cast<const unsigned char*>(p);
      for (int i = 0; i < 4 * n; ++i) {
        h ^= b[i];
        h *= 0x100000001B3ull;
      }
    };
    eat(s.t.c4, 16);
    eat(s.t.c8, 256);
    s.hash = h;
  });
  return s;
}

}  // namespace

const Tables& host_tables() { return state().t; }
const Mids4& host_mids4() { return state().m4; }
const Mids8& host_mids8() { return state().m8; }
const Buckets4& host_buckets4() { return state().b4; }
uint64_t host_table_hash() { return state().hash; }

}  // namespace nf4s
