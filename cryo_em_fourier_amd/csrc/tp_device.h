// Device-side building blocks shared by the projector kernels (gfx950).
//
// The method is the one summarised in "torch-projectors: A High-Performance
// Differentiable Projection Library for PyTorch" (gist.science, it/de/ja/ko/ar
// pages, technical sections 1-2): rotate each output frequency into the
// reference's rfft half-spectrum, read negative-x taps through Friedel
// symmetry, interpolate (linear or Catmull-Rom a = -0.5), apply a shift phase.
//
// Friedel handling used by every kernel.  Per tap, x < 0 reads conj(V[-t]) and
// x >= 0 reads V[t].  For a sample point p split the stencil sum as
//   S(p) = D0(p) + conj(D1(-p)),
//   D0(q) = sum over taps of q with x >= 0, D1(q) = sum over taps with x >= 1,
// (the stencil of -p is the negated stencil of p, up to taps of weight 0 when
// a coordinate is an integer).  With c = (p_x < 0) and m = c ? -p : p (so
// m_x >= 0), the kernels evaluate a "main" sum at m and, only for lanes whose
// stencil reaches the x = 0 plane, a "secondary" sum at -m:
//   c = 0:  S = D0(m) + conj(D1(-m))      c = 1:  S = conj(D1(m)) + D0(-m).
// Both sums read taps with x >= 0 only, so every load is a plain lookup.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {

constexpr int kBlock = 256;
constexpr double kCoordLimit = 1073741824.0;  // 2^30
// Byte offset that is past every reference entry (entries are limited to
// 2^31 - 4096 bytes): raw buffer loads at or beyond num_records return 0.
// Two of them plus a small immediate still fit in 32 bits.
constexpr uint32_t kBig = 0x7FFFF000u;
constexpr int kNumXcd = 8;

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  // raw buffer (stride 0), range-checked against nbytes; gfx9 data format word
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes,
                                           0x00020000);
}

// 8-byte complex load.  The whole 2 x i32 result is bit-cast at once: taking
// its elements one by one lets this compiler narrow the load to one dword and
// return the real part twice.
__device__ __forceinline__ float2 load_c64(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, 0));
}

// Round-robin dispatch sends workgroup g to XCD g % 8.  Remap so that each
// XCD walks a contiguous range of logical tiles (hence the same pose and the
// same reference neighbourhood stay in one XCD's L2).
__device__ __forceinline__ uint32_t xcd_remap(uint32_t g, uint32_t G) {
  const uint32_t xcd = g % kNumXcd, local = g / kNumXcd;
  const uint32_t per = G / kNumXcd, rem = G % kNumXcd;
  return xcd < rem ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// ------------------------------------------------------------ kernels

// Interpolation weights of the taps floor(q) + OFF + d for fraction f in [0,1).
template <int INTERP> struct Kern;

template <> struct Kern<0> {  // linear: taps floor(q), floor(q)+1
  static constexpr int T = 2, OFF = 0;
  __device__ static __forceinline__ void w(float f, float* w) { w[0] = 1.f - f; w[1] = f; }
  __device__ static __forceinline__ void dw(float, float* d) { d[0] = -1.f; d[1] = 1.f; }
};

template <> struct Kern<1> {  // Catmull-Rom (Keys, a = -0.5): taps floor(q)-1 .. floor(q)+2
  static constexpr int T = 4, OFF = -1;
  __device__ static __forceinline__ void w(float f, float* w) {
    const float g = 1.f - f;
    w[0] = -0.5f * f * g * g;                  // K(1 + f)
    w[1] = (1.5f * f - 2.5f) * f * f + 1.f;    // K(f)
    w[2] = (1.5f * g - 2.5f) * g * g + 1.f;    // K(1 - f)
    w[3] = -0.5f * g * f * f;                  // K(2 - f)
  }
  __device__ static __forceinline__ void dw(float f, float* d) {  // d/df of the above
    const float g = 1.f - f;
    d[0] = (-1.5f * f + 2.f) * f - 0.5f;
    d[1] = (4.5f * f - 5.f) * f;
    d[2] = (-4.5f * g + 5.f) * g;
    d[3] = (1.5f * f - 1.f) * f;
  }
};

// One axis of a stencil: integer start, fraction, validity window.
struct AxisPos {
  int x0;     // first tap index (floor + OFF)
  float f;    // fraction in [0, 1)
};

// LEFT takes the stencil from ceil(q) - 1 instead of floor(q).  At a
// non-integer q the two agree; at an integer q the taps move one down and the
// fraction is 1 instead of 0, with the same weights.  The gradient gathers
// use it where they evaluate a stencil at the negated sample point -p: the
// tap set, weights and derivative weights are then exactly the mirror of
// floor(p)'s, so the linear kernel's one-sided derivative at an integer
// coordinate is the right derivative in p there as well.
__device__ __forceinline__ AxisPos axis_pos(double q, int off, bool left = false) {
  const double fl = left ? ceil(q) - 1.0 : floor(q);
  AxisPos a;
  a.x0 = (int)fl + off;
  a.f = (float)(q - fl);
  return a;
}

// Shift an x-weight array left by sh (0..T-1) positions, filling with zero,
// so that the first loaded tap is at x >= 0 (masked taps have weight 0).
template <int T>
__device__ __forceinline__ void shift_left(float* w, int sh) {
  if (T == 4) {
    const bool s1 = sh & 1, s2 = sh & 2;
    float a0 = s1 ? w[1] : w[0], a1 = s1 ? w[2] : w[1], a2 = s1 ? w[3] : w[2], a3 = s1 ? 0.f : w[3];
    w[0] = s2 ? a2 : a0; w[1] = s2 ? a3 : a1; w[2] = s2 ? 0.f : a2; w[3] = s2 ? 0.f : a3;
  } else {
    const bool s1 = sh & 1;
    w[0] = s1 ? w[1] : w[0];
    w[1] = s1 ? 0.f : w[1];
  }
}

// Geometry of one reference entry.
struct RefGeom {
  int N;            // full-axis length
  int xmax;         // N / 2 (last stored x)
  int lo, hi;       // stored signed range of the full axes
  uint32_t row;     // bytes per x-row: (N/2+1) * 8
  uint32_t plane;   // bytes per z-plane: N * row (3D)
};

// Byte offset of index t along an axis of byte stride `stride` (kBig outside
// the stored range).  A 24-bit multiply (full rate) is exact here: the index
// is below 2^16, and an entry of at most 2^31 bytes keeps the row and plane
// strides below 2^24 (a plane exceeds 2^24 bytes only for N >= 128 with
// N * plane > 2^31) and every offset below 2^31.
__device__ __forceinline__ uint32_t axis_off(int t, const RefGeom& g, uint32_t stride) {
  const bool ok = t >= g.lo && t <= g.hi;
  const int w = t < 0 ? t + g.N : t;
  return ok ? __umul24((uint32_t)w, stride) : kBig;
}

// exp(-2 pi i t) for t in turns.  t is reduced in fp64 (so that large k*s
// products keep full fp32 accuracy) to a quarter-turn count q in [-2, 2] and
// a rest r = t - q/4 in [-1/8, 1/8]; sin and cos of 2 pi r come from
// polynomials in r^2 fitted by least squares on that interval at Chebyshev
// nodes (largest error 9e-8 evaluated in fp32), then turn by q quarter turns.
__device__ __forceinline__ float2 phase_of_turns(double t) {
  t -= rint(t);
  const double q = rint(4.0 * t);
  const float r = (float)(t - 0.25 * q), u = r * r;
  const float sn = r * fmaf(fmaf(fmaf(-75.40180791f, u, 81.59254745f), u, -41.34166260f), u, 6.28318529f);
  const float cs = fmaf(fmaf(fmaf(fmaf(59.22026777f, u, -85.44284776f), u, 64.93931617f), u, -19.73920865f), u, 1.f);
  // theta = 2 pi r + q pi / 2: cos theta = cs, -sn, -cs, sn and sin theta =
  // sn, cs, -sn, -cs for q mod 4 = 0, 1, 2, 3; the phase is (cos, -sin)
  const int k = (int)q & 3;
  const float ca = (k & 1) ? sn : cs, sa = (k & 1) ? cs : sn;
  return make_float2(((k + 1) & 2) ? -ca : ca, (k & 2) ? sa : -sa);
}

// exp(-2 pi i (kx sx + ky sy) / n_out)
__device__ __forceinline__ float2 shift_phase(int kx, int ky, float sx, float sy, double inv_n) {
  return phase_of_turns(((double)kx * (double)sx + (double)ky * (double)sy) * inv_n);
}

__device__ __forceinline__ float2 cmul(float2 a, float2 b) {
  return make_float2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
__device__ __forceinline__ float2 conjf2(float2 a) { return make_float2(a.x, -a.y); }

// Wave sum of eight doubles by halving: each exchange step sends half of the
// values still held, so 10 shuffles replace 8 x 6.  On return lane l holds the
// total of value 4*bit5(l) + 2*bit4(l) + bit3(l).
__device__ __forceinline__ double wave_sum8(const double* a) {
  const int lane = threadIdx.x & 63;
  const bool b5 = lane & 32, b4 = lane & 16, b3 = lane & 8;
  double b[4], c[2];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const double send = b5 ? a[k] : a[k + 4], keep = b5 ? a[k + 4] : a[k];
    b[k] = keep + __shfl_xor(send, 32, 64);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const double send = b4 ? b[k] : b[k + 2], keep = b4 ? b[k + 2] : b[k];
    c[k] = keep + __shfl_xor(send, 16, 64);
  }
  const double send = b3 ? c[0] : c[1], keep = b3 ? c[1] : c[0];
  double d = keep + __shfl_xor(send, 8, 64);
  d += __shfl_xor(d, 4, 64);
  d += __shfl_xor(d, 2, 64);
  d += __shfl_xor(d, 1, 64);
  return d;
}

// Signed frequency of row index iy of an n-row rfft image.
__device__ __forceinline__ int signed_row(int iy, int n) { return iy <= (n - 1) / 2 ? iy : iy - n; }

}  // namespace tp
