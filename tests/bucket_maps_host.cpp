// Host checks of the select's bucket maps and order-preserving keys
// (score_top_token_amd/csrc/li_bucket.h, the same header the kernels use).
// Prints one line per failed check and "ok <checks>" at the end; exit status 1
// on any failure.
#include <stdio.h>

#include <algorithm>
#include <cmath>
#include <random>
#include <vector>

#include "li_bucket.h"

static long g_checks = 0, g_fail = 0;
#define CHECK(cond, ...)                        \
  do {                                          \
    ++g_checks;                                 \
    if (!(cond)) {                              \
      ++g_fail;                                 \
      if (g_fail < 40) {                        \
        printf("FAIL %s:%d ", __FILE__, __LINE__); \
        printf(__VA_ARGS__);                    \
        printf("\n");                           \
      }                                         \
    }                                           \
  } while (0)

static const float kInf = INFINITY;

// Sorted probe values: both infinities, extremes, denormals, signed zeros and
// values around and inside [lo, hi].
static std::vector<float> probes(float lo, float hi, std::mt19937& rng) {
  std::vector<float> v = {-kInf, -3.4e38f, -1e30f, -1.0f, -1e-40f, -0.0f, 0.0f, 1e-40f,
                          1e-30f, 1.0f, 1e30f, 3.4e38f, kInf};
  for (float x : {lo, hi}) {
    if (std::isfinite(x)) {
      v.push_back(x);
      v.push_back(std::nextafter(x, -kInf));
      v.push_back(std::nextafter(x, kInf));
    }
  }
  if (std::isfinite(lo) && std::isfinite(hi) && lo < hi) {
    std::uniform_real_distribution<double> u(lo, hi);
    for (int i = 0; i < 4000; ++i) v.push_back((float)u(rng));
  }
  std::uniform_real_distribution<float> any(-1e6f, 1e6f);
  for (int i = 0; i < 500; ++i) v.push_back(any(rng));
  std::sort(v.begin(), v.end());
  return v;
}

template <int NB>
static void check_lin(float lo, float hi, std::mt19937& rng) {
  const li::LinBucket<NB> b(lo, hi);
  const std::vector<float> v = probes(lo, hi, rng);
  uint32_t prev = 0;
  bool first = true;
  std::vector<char> seen(NB, 0);
  for (float f : v) {
    const uint32_t k = b(f);
    CHECK(k < (uint32_t)NB, "LinBucket<%d>(%g, %g)(%g) = %u out of range", NB, lo, hi, f, k);
    if (!first) CHECK(k >= prev, "LinBucket<%d>(%g, %g) not monotone at %g", NB, lo, hi, f);
    prev = k;
    first = false;
    if (std::isfinite(lo) && std::isfinite(hi) && f >= lo && f <= hi && k < (uint32_t)NB) seen[k] = 1;
  }
  // finite lo < hi with a normal span: the range [lo, hi] starts in bucket 0,
  // ends in one of the top buckets and spreads over most buckets
  if (std::isfinite(lo) && std::isfinite(hi) && lo < hi && (hi - lo) > 1e-30f * std::max(1.0f, std::fabs(lo))) {
    CHECK(b(lo) == 0u, "LinBucket<%d>(%g, %g)(lo) = %u", NB, lo, hi, b(lo));
    CHECK(b(hi) >= (uint32_t)(NB - 2), "LinBucket<%d>(%g, %g)(hi) = %u", NB, lo, hi, b(hi));
    int used = 0;
    for (int i = 0; i < NB; ++i) used += seen[i];
    if ((hi - lo) / std::max(std::fabs(lo), std::fabs(hi)) > 1e-3f)
      CHECK(used >= NB / 2, "LinBucket<%d>(%g, %g) uses %d buckets", NB, lo, hi, used);
  }
}

template <int NB>
static void check_key(uint32_t ulo, uint32_t uhi, std::mt19937& rng) {
  const li::KeyBucket<NB> b(ulo, uhi);
  std::vector<uint32_t> v = {ulo, uhi};
  std::uniform_int_distribution<uint64_t> u(ulo, uhi);
  for (int i = 0; i < 3000; ++i) v.push_back((uint32_t)u(rng));
  std::sort(v.begin(), v.end());
  uint32_t prev = 0;
  for (size_t i = 0; i < v.size(); ++i) {
    const uint32_t k = b(v[i]);
    CHECK(k < (uint32_t)NB, "KeyBucket<%d>(%u, %u)(%u) = %u", NB, ulo, uhi, v[i], k);
    if (i) CHECK(k >= prev, "KeyBucket<%d>(%u, %u) not monotone at %u", NB, ulo, uhi, v[i]);
    prev = k;
  }
  CHECK(b(ulo) == 0u, "KeyBucket<%d>(%u, %u)(ulo) = %u", NB, ulo, uhi, b(ulo));
  // the shift rounds the span up to a power of two: the top key reaches at
  // least the upper half of the buckets, and a span below NB maps one to one
  if (uhi - ulo >= (uint32_t)NB)
    CHECK(b(uhi) >= (uint32_t)(NB / 2 - 1), "KeyBucket<%d>(%u, %u)(uhi) = %u", NB, ulo, uhi, b(uhi));
  else
    CHECK(b(uhi) == uhi - ulo, "KeyBucket<%d>(%u, %u)(uhi) = %u", NB, ulo, uhi, b(uhi));
  // a key above the range (filtered by the callers) still lands in range
  if (uhi < 0xFFFFFFFFu) CHECK(b(uhi + 1) < (uint32_t)NB, "KeyBucket<%d> above range", NB);
}

int main() {
  std::mt19937 rng(12345);
  // bounds: ordinary, tiny and huge magnitudes, equal, inverted, infinite
  const float pairs[][2] = {{-1.0f, 1.0f},   {0.0f, 1e-30f},   {-3.4e38f, 3.4e38f}, {1e25f, 1e26f},
                            {-1e-30f, 0.0f}, {5.0f, 5.0f},     {3.0f, 1.0f},        {-kInf, 5.0f},
                            {-5.0f, kInf},   {-kInf, kInf},    {-kInf, -kInf},      {kInf, kInf},
                            {0.0f, 0.0f},    {1.0f, 1.0000001f}, {-2e-38f, 2e-38f}, {100.0f, 1e9f}};
  for (const auto& p : pairs) {
    check_lin<256>(p[0], p[1], rng);
    check_lin<512>(p[0], p[1], rng);
    check_lin<2048>(p[0], p[1], rng);
  }
  const uint32_t kp[][2] = {{0u, 0u},         {5u, 5u},         {0u, 255u},          {0u, 256u},
                            {100u, 100000u},  {0u, 0xFFFFFFFFu}, {0x80000000u, 0xBF800000u},
                            {0xFFFFFF00u, 0xFFFFFFFFu}, {0x7F800000u, 0x807FFFFFu}};
  for (const auto& p : kp) {
    check_key<256>(p[0], p[1], rng);
    check_key<2048>(p[0], p[1], rng);
  }
  // order-preserving keys: strictly increasing over distinct sorted floats, -0
  // equal to +0, and key2f inverts f2key (with -0 read back as +0)
  std::vector<float> fs = probes(-1.0f, 1.0f, rng);
  fs.erase(std::unique(fs.begin(), fs.end()), fs.end());
  for (size_t i = 0; i < fs.size(); ++i) {
    const float f = fs[i];
    const float back = li::key2f(li::f2key(f));
    CHECK(back == f && !(f == 0.0f && std::signbit(back)), "key2f(f2key(%g)) = %g", f, back);
    CHECK(li::f2key(f) > 0x007FFFFFu || f == -kInf, "f2key(%g) = %08x in the reserved range", f, li::f2key(f));
    if (i) {
      const bool zeros = fs[i - 1] == 0.0f && f == 0.0f;
      if (zeros) CHECK(li::f2key(fs[i - 1]) == li::f2key(f), "-0 and +0 differ");
      else CHECK(li::f2key(fs[i - 1]) < li::f2key(f), "f2key not increasing at %g", f);
    }
  }
  printf("%s %ld checks, %ld failed\n", g_fail ? "FAILED" : "ok", g_checks, g_fail);
  return g_fail ? 1 : 0;
}
