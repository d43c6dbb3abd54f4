// Host-side checks of the 12-bit block floating-point records that carry the selection partials
// (rec12_* in fast_common.hpp, the same functions the kernels call).  Prints one line per failed
// check and "rec12 ok" when every check passes; the exit status is the number of failures.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <random>

#include "../sparse_attention_long_fwd_amd/csrc/fast_common.hpp"

static int g_fail = 0;
#define CHECK(c, ...)                 \
  do {                                \
    if (!(c)) {                       \
      ++g_fail;                       \
      if (g_fail < 20) {              \
        std::printf("FAIL %s: ", #c); \
        std::printf(__VA_ARGS__);     \
        std::printf("\n");            \
      }                               \
    }                                 \
  } while (0)

// Encodes 128 values as the kernels do (both halves with the record's exponent), decodes them,
// and checks the step bound: |x - X 2^(e - 11)| <= 2^(e - 12), |X| <= 2047.
static void roundtrip(const float* x, float mul, const char* what) {
  float amax = 0.f;
  for (int i = 0; i < 128; ++i) amax = std::fmax(amax, std::fabs(x[i]));
  amax *= mul;
  const int e = rec12_exp(amax);
  CHECK(e >= -20 && e <= 128, "%s: e = %d", what, e);
  const float scale = ldexpf(mul, 11 - e);
  for (int p = 0; p < 16; ++p) {
    uint32_t w[3];
    rec12_pack8(x + 8 * p, scale, w);
    float y[8];
    rec12_unpack8(w[0], w[1], w[2], y);
    for (int i = 0; i < 8; ++i) {
      const double xv = (double)x[8 * p + i] * mul;
      CHECK(std::fabs(y[i]) <= 2047.f, "%s: |X| = %g", what, y[i]);
      const double err = std::fabs(xv - std::ldexp((double)y[i], e - 11));
      CHECK(err <= std::ldexp(1.0, e - 12) * (1 + 1e-6), "%s: value %.9g decoded %.9g (e %d)", what, xv,
            std::ldexp((double)y[i], e - 11), e);
    }
  }
}

int main() {
  // Bit layout: value i of a pack at bits [12 i, 12 i + 12) of the 96-bit little-endian string.
  {
    const float v[8] = {1, -1, 2047, -2047, 0, 1365, -1366, 7};
    uint32_t w[3];
    rec12_pack8(v, 1.f, w);
    const unsigned __int128 str = (unsigned __int128)w[0] | ((unsigned __int128)w[1] << 32) |
                                  ((unsigned __int128)w[2] << 64);
    for (int i = 0; i < 8; ++i) {
      const int u = (int)((str >> (12 * i)) & 0xFFF);
      const int s = u >= 2048 ? u - 4096 : u;
      CHECK(s == (int)v[i], "layout: value %d reads %d at bit %d", (int)v[i], s, 12 * i);
    }
    float y[8];
    rec12_unpack8(w[0], w[1], w[2], y);
    for (int i = 0; i < 8; ++i) CHECK(y[i] == v[i], "unpack %d: %g", i, y[i]);
  }
  // Rounding: to the nearest integer, ties to even (the FMA against 1.5 * 2^23).
  {
    const float v[8] = {0.5f, 1.5f, -0.5f, -1.5f, 2.49f, 2.51f, -2047.4f, 1000.5f};
    const float want[8] = {0, 2, 0, -2, 2, 3, -2047, 1000};
    uint32_t w[3];
    rec12_pack8(v, 1.f, w);
    float y[8];
    rec12_unpack8(w[0], w[1], w[2], y);
    for (int i = 0; i < 8; ++i) CHECK(y[i] == want[i], "round %g: %g, want %g", v[i], y[i], want[i]);
  }
  // Exponent: the largest magnitude times 2^(11 - e) stays at or below 2047 after rounding, also
  // just below a power of two; tiny records clamp to e = -20 (an all-zero record keeps frexp's 0).
  {
    CHECK(rec12_exp(0.f) == 0, "rec12_exp(0) = %d", rec12_exp(0.f));
    CHECK(rec12_exp(1e-30f) == -20, "rec12_exp(1e-30) = %d", rec12_exp(1e-30f));
    CHECK(rec12_exp(1.f) == 1, "rec12_exp(1) = %d", rec12_exp(1.f));
    CHECK(rec12_exp(0.99999994f) == 1, "rec12_exp(1 - 2^-24) = %d", rec12_exp(0.99999994f));
    CHECK(rec12_exp(0.999f) == 0, "rec12_exp(0.999) = %d", rec12_exp(0.999f));
    CHECK(rec12_exp(3.0e38f) == 128, "rec12_exp(3e38) = %d", rec12_exp(3.0e38f));
  }
  // Round trips over magnitudes, signs, exact powers of two and near-power maxima.
  std::mt19937 rng(12345);
  std::normal_distribution<float> nd(0.f, 1.f);
  float x[128];
  const float scales[] = {1e-12f, 3e-7f, 1e-3f, 0.37f, 1.f, 5.f, 1234.f, 6.5e4f, 1e20f};
  for (float sc : scales)
    for (int rep = 0; rep < 50; ++rep) {
      for (int i = 0; i < 128; ++i) x[i] = nd(rng) * sc;
      if (rep % 5 == 1) x[rep % 128] = sc;                          // maximum at a power of ten
      if (rep % 5 == 2) x[rep % 128] = -ldexpf(1.f, (int)std::log2(sc));  // exact power of two
      if (rep % 5 == 3) x[rep % 128] = ldexpf(0.99999994f, 1 + (int)std::log2(sc));  // just below
      if (rep % 5 == 4) for (int i = 0; i < 64; ++i) x[i] = 0.f;   // one half all zero
      roundtrip(x, 1.f, "plain");
      roundtrip(x, 0.0123f, "scaled");  // the window pass stores values times 1 / sum
    }
  for (int i = 0; i < 128; ++i) x[i] = 0.f;
  roundtrip(x, 1.f, "zeros");
  // The step folded into (max, sum): merging records through (m + e - 11, l 2^(11 - e)) with the
  // merge's weights 2^(m' - M') / L' applied to the integers equals the merge of the exact
  // partials, 2^(m - M) o / L, within the records' step bound.
  {
    const int S = 5;
    float m[S], l[S], o[S][128];
    for (int s = 0; s < S; ++s) {
      m[s] = 3.f * nd(rng);
      l[s] = 1.f + 40.f * std::fabs(nd(rng));
      const float mag = ldexpf(1.f, (int)(8 * nd(rng)));
      for (int i = 0; i < 128; ++i) o[s][i] = nd(rng) * mag * l[s];
    }
    double M = -1e30, Mq = -1e30;
    float mq[S], lq[S], X[S][128];
    int es[S];
    for (int s = 0; s < S; ++s) {
      float amax = 0.f;
      for (int i = 0; i < 128; ++i) amax = std::fmax(amax, std::fabs(o[s][i]));
      es[s] = rec12_exp(amax);
      const float2 ml = rec12_ml(m[s], l[s], es[s]);
      mq[s] = ml.x;
      lq[s] = ml.y;
      for (int p = 0; p < 16; ++p) {
        uint32_t w[3];
        rec12_pack8(o[s] + 8 * p, ldexpf(1.f, 11 - es[s]), w);
        rec12_unpack8(w[0], w[1], w[2], X[s] + 8 * p);
      }
      M = std::fmax(M, (double)m[s]);
      Mq = std::fmax(Mq, (double)mq[s]);
    }
    double L = 0, Lq = 0;
    for (int s = 0; s < S; ++s) {
      L += std::exp2(m[s] - M) * l[s];
      Lq += std::exp2(mq[s] - Mq) * lq[s];
    }
    CHECK(std::fabs(L * std::exp2(M - Mq) - Lq) <= 1e-5 * Lq, "normaliser %.9g vs %.9g", L * std::exp2(M - Mq), Lq);
    for (int i = 0; i < 128; ++i) {
      double ex = 0, got = 0, bound = 0;
      for (int s = 0; s < S; ++s) {
        ex += std::exp2(m[s] - M) * o[s][i] / L;
        got += std::exp2(mq[s] - Mq) * X[s][i] / Lq;
        bound += std::exp2(m[s] - M) / L * std::ldexp(1.0, es[s] - 12);
      }
      CHECK(std::fabs(ex - got) <= bound * 1.0001 + 1e-6 * std::fabs(ex), "merge dim %d: %.9g vs %.9g (bound %g)", i,
            got, ex, bound);
    }
  }
  if (g_fail == 0) std::printf("rec12 ok\n");
  return g_fail;
}
