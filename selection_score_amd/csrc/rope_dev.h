// RoPE and 16-byte vector helpers shared by the gather kernels (device code).
#pragma once

#include "common.h"

#include <math.h>

namespace kvsel {
namespace rope {

constexpr double kTwoPiHi = 6.28318530717958623200e+00;
constexpr double kTwoPiLo = 2.44929359829470635445e-16;
constexpr double kInvTwoPi = 1.59154943091895345608e-01;

// cos/sin of p * f, with the product reduced modulo 2*pi in float64.
__device__ __forceinline__ void angle_sincos(double p, double f, float* c, float* s) {
  const double phi = p * f;
  const double n = rint(phi * kInvTwoPi);
  double r = fma(-n, kTwoPiHi, phi);
  r = fma(-n, kTwoPiLo, r);
  sincosf(static_cast<float>(r), s, c);
}

template <int DT>
struct Vec16 {
  static constexpr int kElems = (DT == KVSEL_F32) ? 4 : 8;
};

template <int DT>
__device__ __forceinline__ void unpack16(const uint4& v, float* x) {
  if constexpr (DT == KVSEL_F32) {
    x[0] = __uint_as_float(v.x);
    x[1] = __uint_as_float(v.y);
    x[2] = __uint_as_float(v.z);
    x[3] = __uint_as_float(v.w);
  } else {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    for (int i = 0; i < 4; ++i) {
      const uint16_t lo = static_cast<uint16_t>(w[i] & 0xFFFFu);
      const uint16_t hi = static_cast<uint16_t>(w[i] >> 16);
      if constexpr (DT == KVSEL_BF16) {
        x[2 * i] = bf16_to_f32(lo);
        x[2 * i + 1] = bf16_to_f32(hi);
      } else {
        x[2 * i] = f16_to_f32(lo);
        x[2 * i + 1] = f16_to_f32(hi);
      }
    }
  }
}

template <int DT>
__device__ __forceinline__ uint4 pack16(const float* x) {
  uint4 v;
  if constexpr (DT == KVSEL_F32) {
    v.x = __float_as_uint(x[0]);
    v.y = __float_as_uint(x[1]);
    v.z = __float_as_uint(x[2]);
    v.w = __float_as_uint(x[3]);
  } else {
    // round-to-nearest-even conversions, two elements per instruction
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    uint32_t w[4];
    for (int i = 0; i < 4; ++i) {
      const f32x2 pr = {x[2 * i], x[2 * i + 1]};
      if constexpr (DT == KVSEL_BF16) {
        w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, bf16x2));
      } else {
        w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(pr, f16x2));
      }
    }
    v.x = w[0];
    v.y = w[1];
    v.z = w[2];
    v.w = w[3];
  }
  return v;
}

__device__ __forceinline__ uint4 shfl16(const uint4& v, int src) {
  uint4 r;
  r.x = __shfl(v.x, src, 64);
  r.y = __shfl(v.y, src, 64);
  r.z = __shfl(v.z, src, 64);
  r.w = __shfl(v.w, src, 64);
  return r;
}

// Rotate this lane's 16-byte chunk given per-element cos/sin.  `own` holds
// dims [d0, d0+E); for rotate-half the partner chunk (other half of the
// pair) is `other`; `first` says whether own dims are the pair's first half.
template <int DT>
__device__ __forceinline__ uint4 rotate_chunk(const uint4& own, const uint4& other, bool first,
                                              bool interleaved, const float* cs, const float* sn) {
  constexpr int E = Vec16<DT>::kElems;
  float a[E], b[E], y[E];
  unpack16<DT>(own, a);
  if (interleaved) {
    for (int i = 0; i < E; i += 2) {
      y[i] = a[i] * cs[i / 2] - a[i + 1] * sn[i / 2];
      y[i + 1] = a[i] * sn[i / 2] + a[i + 1] * cs[i / 2];
    }
  } else {
    unpack16<DT>(other, b);
    for (int i = 0; i < E; ++i) {
      y[i] = first ? (a[i] * cs[i] - b[i] * sn[i]) : (b[i] * sn[i] + a[i] * cs[i]);
    }
  }
  return pack16<DT>(y);
}

// One lane's 16-byte chunk rotated by (c, s) per pair.  Rotate-half: `own`
// holds dims [d0, d0+E) of one half, `other` the matching dims of the other
// half, and `sgn` is -1 for the first half (x_m c - x_{m+D/2} s) and +1 for
// the second (x_{m+D/2} c + x_m s).  Interleaved: pairs are adjacent in `own`.
// cos and sin of a + b from those of a and b (angle addition), each with
// one rounded product and one fused multiply-add in a fixed order, so the
// bits do not depend on how the compiler contracts the expression.
__device__ __forceinline__ void add_angles(float ca, float sa, float cb, float sb, float* c, float* s) {
  *c = fmaf(ca, cb, -(sa * sb));
  *s = fmaf(sa, cb, ca * sb);
}

template <int DT, bool kInter>
__device__ __forceinline__ uint4 rotate16(const uint4& own, const uint4& other, float sgn, const float* c,
                                          const float* s) {
  constexpr int E = Vec16<DT>::kElems;
  float a[E], y[E];
  unpack16<DT>(own, a);
  if constexpr (kInter) {
    for (int i = 0; i < E; i += 2) {
      y[i] = fmaf(a[i], c[i / 2], -(a[i + 1] * s[i / 2]));
      y[i + 1] = fmaf(a[i], s[i / 2], a[i + 1] * c[i / 2]);
    }
  } else {
    float b[E];
    unpack16<DT>(other, b);
    for (int i = 0; i < E; ++i) y[i] = fmaf(b[i], sgn * s[i], a[i] * c[i]);
  }
  return pack16<DT>(y);
}

}  // namespace rope
}  // namespace kvsel
