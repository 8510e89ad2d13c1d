// Per-coordinate and per-group arithmetic of the lossy encoder, compiled for the host
// encoder (g++) and the GPU encoder (hipcc) from this one source, so both take the same
// decisions bit for bit (float64 with no contraction on both sides).
//
// [ABS]: weights are row-normalised, quantised onto the E8 lattice and coded with a
// conditional model.  E8 = D8 u (D8 + 1/2): the nearest point is the nearer of the
// nearest D8 point and the nearest point of the shifted coset (Conway & Sloane's
// decoder); D8's nearest point rounds every coordinate and, if the sum is odd, moves
// the worst-rounded coordinate the other way.  Coordinates are kept doubled (u = 2p).
#pragma once
#include <cmath>
#include <cstdint>

#include "../../include/entropack.h"

#ifdef __HIPCC__
#define EP_HD __host__ __device__
#else
#define EP_HD
#endif

namespace ep {
namespace cm {

// ---------------------------------------------------------------- containers -> float64
EP_HD inline double fp8_e4m3fn_value(uint8_t b) {
  int e = (b >> 3) & 15, m = b & 7;
  double v;
  if (e == 0) v = ldexp(m / 8.0, -6);
  else v = ldexp(1.0 + m / 8.0, e - 7);
  if (e == 15 && m == 7) v = NAN;
  return (b & 0x80) ? -v : v;
}

EP_HD inline double fp16_value(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp(1.0 + m / 1024.0, e - 15);
  return s ? -v : v;
}

EP_HD inline double bf16_value(uint16_t b) {
  union {
    uint32_t u;
    float f;
  } x;
  x.u = uint32_t(b) << 16;
  return (double)x.f;
}

// element i of a container array
EP_HD inline double widen_one(const void* src, int dtype, int64_t i) {
  switch (dtype) {
    case EP_BF16: return bf16_value(((const uint16_t*)src)[i]);
    case EP_FP16: return fp16_value(((const uint16_t*)src)[i]);
    case EP_FP32: return (double)((const float*)src)[i];
    case EP_FP8_E4M3FN: return fp8_e4m3fn_value(((const uint8_t*)src)[i]);
    default: return (double)((const int8_t*)src)[i];
  }
}

// ---------------------------------------------------------------- E8
EP_HD inline void d8_nearest(const double* v, double* f) {
  double s = 0.0;
  for (int i = 0; i < 8; ++i) {
    f[i] = nearbyint(v[i]);
    s += f[i];
  }
  if (fmod(s, 2.0) != 0.0) {
    int best = 0;
    double be = fabs(v[0] - f[0]);
    for (int i = 1; i < 8; ++i) {
      double e = fabs(v[i] - f[i]);
      if (e > be) {
        be = e;
        best = i;
      }
    }
    f[best] += (v[best] - f[best] >= 0.0) ? 1.0 : -1.0;
  }
}

EP_HD inline void e8_doubled(const double* y, int32_t* u) {
  double p0[8], p1[8], ym[8];
  d8_nearest(y, p0);
  for (int i = 0; i < 8; ++i) ym[i] = y[i] - 0.5;
  d8_nearest(ym, p1);
  for (int i = 0; i < 8; ++i) p1[i] += 0.5;
  double t = y[0] - p0[0];
  double d0 = t * t;
  for (int i = 1; i < 8; ++i) {
    t = y[i] - p0[i];
    d0 = d0 + t * t;
  }
  t = y[0] - p1[0];
  double d1 = t * t;
  for (int i = 1; i < 8; ++i) {
    t = y[i] - p1[i];
    d1 = d1 + t * t;
  }
  const double* p = (d1 < d0) ? p1 : p0;
  for (int i = 0; i < 8; ++i) u[i] = (int32_t)(2.0 * p[i]);
}

// ---------------------------------------------------------------- symbols
struct Sym {
  int ctx, id, rawbits;
  uint32_t rawval;
};

EP_HD inline int ilog2(uint32_t v) { return 31 - __builtin_clz(v); }

// u -> 8 coded symbols in decoding order (FIRST: coordinate 0 joint with the coset,
// FREE[c]: 1..6, LAST[c][pi]: 7); magnitudes below K = 2^k direct, larger ones as a
// log bucket (4 per octave) + raw bits.  Returns the coset; msym[] for counting.
EP_HD inline int symbolize(const int32_t* u, int k, Sym* s, int* msym) {
  const int K = 1 << k;
  int c = u[0] & 1;
  int q_sum = 0;
  int neg[8], raw_rb[8];
  uint32_t raw[8];
  for (int i = 0; i < 8; ++i) {
    int a = u[i] < 0 ? -u[i] : u[i];
    uint32_t m = (uint32_t)((a - c) >> 1);
    neg[i] = u[i] < 0;
    if ((int64_t)m < K) {
      msym[i] = (int)m;
      raw[i] = 0;
      raw_rb[i] = 0;
    } else {
      int e = ilog2(m);
      int top2 = (m >> (e - 2)) & 3;
      msym[i] = K + 4 * (e - k) + top2;
      raw[i] = m & ((1u << (e - 2)) - 1u);
      raw_rb[i] = e - 2;
    }
    if (i < 7) q_sum += (u[i] >> 1);
  }
  int pi = q_sum & 1;
  for (int i = 0; i < 8; ++i) {
    int sid = 2 * msym[i] + neg[i];
    s[i].ctx = i == 0 ? 0 : (i < 7 ? 1 + c : 3 + 2 * c + pi);
    s[i].id = i == 0 ? 512 * c + sid : sid;
    s[i].rawval = raw[i];
    s[i].rawbits = raw_rb[i];
  }
  if (msym[7] >= K) {   // the low raw bit of the last coordinate is implied
    s[7].rawval >>= 1;
    s[7].rawbits -= 1;
  }
  return c;
}

}  // namespace cm
}  // namespace ep
