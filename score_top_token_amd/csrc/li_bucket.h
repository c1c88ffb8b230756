// Bucket maps of the exact top-k select and the order-preserving float key.
//
// Plain C++ with no HIP dependency, so that a host program can compile the
// very same maps (tests/bucket_maps_host.cpp checks their range and
// monotonicity, including infinite and inverted bounds).  Under HIP every
// function is __host__ __device__.
#pragma once

#include <math.h>
#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#define LI_HD __host__ __device__
#else
#define LI_HD
#endif

namespace li {

LI_HD inline uint32_t float_bits(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return u;
}
LI_HD inline float bits_float(uint32_t u) {
  float f;
  memcpy(&f, &u, 4);
  return f;
}

// fp32 <-> order-preserving u32: a > b as floats  <=>  key(a) > key(b) as u32.
// -0 is folded to +0 first.  Every finite value maps above 0x007FFFFF, so the
// key 0 never belongs to a real score.
LI_HD inline uint32_t f2key(float f) {
  if (f == 0.0f) f = 0.0f;
  const uint32_t u = float_bits(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
LI_HD inline float key2f(uint32_t u) {
  const uint32_t v = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return bits_float(v);
}

// x clamped to [lo, hi] (lo <= hi).  A NaN x (only from an infinite bound,
// where the scale is 0) gives lo on the host; on the device the conversion to
// u32 that follows turns a NaN median into 0 as well.
LI_HD inline float clamp_med3(float x, float lo, float hi) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __builtin_amdgcn_fmed3f(x, lo, hi);
#else
  return fminf(fmaxf(x, lo), hi);
#endif
}

// Linear value bucket in [0, NB): one fused multiply-add, a median-of-three
// clamp and a conversion, each monotone in f, so a key of a higher bucket is
// never below a key of a lower one.  Halving first keeps (hi - lo) finite; for f
// in [lo, hi] the product f * a stays within a few units of NB * 2^24.  With an
// infinite or inverted bound the scale is 0 and every value shares one bucket
// (the select then refines on the u32 keys); values outside [lo, hi] clamp to
// the end buckets.
template <int NB>
struct LinBucket {
  float a, c;
  LI_HD LinBucket(float lo, float hi) {
    const float lo2 = lo * 0.5f;
    // an inverted range (hi < lo) gets the scale 0 too: one bucket, not a
    // decreasing map
    const float scale = fmaxf(fminf((float)NB / (hi * 0.5f - lo2), 3.0e38f), 0.0f);
    a = 0.5f * scale;
    c = -lo2 * scale;
  }
  LI_HD uint32_t operator()(float f) const {
    return (uint32_t)clamp_med3(fmaf(f, a, c), 0.0f, (float)(NB - 1));
  }
};

// Bucket of u32 keys in [ulo, uhi]: (u - ulo) >> shift, at most NB - 1
// (NB a power of two).  Keys outside the range are filtered by the callers;
// one above uhi clamps to NB - 1.
template <int NB>
struct KeyBucket {
  uint32_t ulo;
  int shift;
  LI_HD KeyBucket(uint32_t lo, uint32_t hi) : ulo(lo) {
    static_assert((NB & (NB - 1)) == 0, "NB is a power of two");
    constexpr int kBits = __builtin_ctz(NB);
    const uint32_t span = hi - lo;
    const int bits = span ? 32 - __builtin_clz(span) : 0;
    shift = bits > kBits ? bits - kBits : 0;
  }
  LI_HD uint32_t operator()(uint32_t u) const {
    const uint32_t b = (u - ulo) >> shift;
    return b > (uint32_t)(NB - 1) ? (uint32_t)(NB - 1) : b;
  }
};

}  // namespace li
