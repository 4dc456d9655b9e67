// Separable stencils of the projector: gather (forward) and gather with the
// kernel derivative (pose gradients), for 2D and 3D references, linear or
// Catmull-Rom.  See tp_device.h for the main/secondary
// split that keeps every tap at x >= 0.
#pragma once

#include "tp_device.h"
#include "tp_internal.h"

namespace tp {

__device__ __forceinline__ RefGeom ref_geom(const OpParams& p) {
  RefGeom g;
  g.N = p.N;
  g.xmax = p.N / 2;
  g.lo = -(p.N / 2);
  g.hi = (p.N + 1) / 2 - 1;
  g.row = (uint32_t)(p.N / 2 + 1) * 8u;
  g.plane = (uint32_t)p.N * g.row;
  return g;
}

// x axis: weights (zeroed outside [xmin, xmax]) and the byte offset of the
// first loaded tap, which is moved to x >= 0 by shifting the weights.
// (left: see axis_pos; only the linear kernel's derivative depends on it)
template <int INTERP, bool GRAD>
__device__ __forceinline__ uint32_t setup_x(const RefGeom& g, double q, int xmin, float* w, float* dw,
                                            bool left = false) {
  using K = Kern<INTERP>;
  constexpr int T = K::T;
  const AxisPos a = axis_pos(q, K::OFF, INTERP == 0 && left);
  K::w(a.f, w);
  if (GRAD) K::dw(a.f, dw);
#pragma unroll
  for (int d = 0; d < T; ++d) {
    const int t = a.x0 + d;
    if (t < xmin || t > g.xmax) {
      w[d] = 0.f;
      if (GRAD) dw[d] = 0.f;
    }
  }
  int start = a.x0;
  if (start < 0) {
    const int sh = -start;
    if (sh >= T) {
#pragma unroll
      for (int d = 0; d < T; ++d) { w[d] = 0.f; if (GRAD) dw[d] = 0.f; }
    } else {
      shift_left<T>(w, sh);
      if (GRAD) shift_left<T>(dw, sh);
    }
    start = 0;
  }
  return (uint32_t)start * 8u;
}

// y or z axis: weights and byte offsets (kBig for taps outside the stored
// range); returns the first tap's coordinate.
template <int INTERP, bool GRAD>
__device__ __forceinline__ int setup_yz(const RefGeom& g, double q, uint32_t stride, float* w,
                                        float* dw, uint32_t* off, bool left = false) {
  using K = Kern<INTERP>;
  const AxisPos a = axis_pos(q, K::OFF, INTERP == 0 && left);
  K::w(a.f, w);
  if (GRAD) K::dw(a.f, dw);
#pragma unroll
  for (int d = 0; d < K::T; ++d) off[d] = axis_off(a.x0 + d, g, stride);
  return a.x0;
}

// Reorder the T taps of an axis (consecutive coordinates from `first`) so
// that entry t holds the tap whose coordinate is congruent to t modulo T.
// When every lane of a wave walks its rows in this order, the lanes of
// neighbouring outputs, whose stencils overlap, load the same row of the
// reference in the same instruction: one load touches fewer distinct cache
// sectors, and the L1's sector rate is what bounds the 3D gathers.  The sum
// over the taps is the same up to rounding order.
template <int T, typename V>
__device__ __forceinline__ void by_residue(V* a, int first) {
  const int s = (-first) & (T - 1);  // entry t <- a[(t + s) mod T]
#pragma unroll
  for (int b = 1; b < T; b <<= 1) {
    const bool on = (s & b) != 0;
    V r[T];
#pragma unroll
    for (int t = 0; t < T; ++t) r[t] = a[(t + b) & (T - 1)];
#pragma unroll
    for (int t = 0; t < T; ++t) a[t] = on ? r[t] : a[t];
  }
}

// ---------------------------------------------------------------- gather

// Sum over taps with x >= xmin of w * V[t] at q (2D; the 3D forwards use
// the lane-pair form below).
template <int INTERP>
__device__ __forceinline__ float2 gather2(rsrc_t rs, const RefGeom& g, double qx, double qy,
                                          int xmin) {
  constexpr int T = Kern<INTERP>::T;
  float wx[T], wy[T];
  uint32_t yb[T];
  const uint32_t xo = setup_x<INTERP, false>(g, qx, xmin, wx, nullptr);
  setup_yz<INTERP, false>(g, qy, g.row, wy, nullptr, yb);
  float2 acc = make_float2(0.f, 0.f);
#pragma unroll
  for (int dy = 0; dy < T; ++dy) {
    const uint32_t ro = yb[dy] == kBig ? kBig : yb[dy] + xo;
    float2 r = make_float2(0.f, 0.f);
#pragma unroll
    for (int dx = 0; dx < T; ++dx) {
      const float2 v = load_c64(rs, ro + 8u * dx);
      r.x = fmaf(wx[dx], v.x, r.x);
      r.y = fmaf(wx[dx], v.y, r.y);
    }
    acc.x = fmaf(wy[dy], r.x, acc.x);
    acc.y = fmaf(wy[dy], r.y, acc.y);
  }
  return acc;
}

// Value and gradient w.r.t. the sample point (2D): out[0] = S, out[1 + j] =
// dS/dq_j.  left: q is the negated sample point (see axis_pos).
template <int INTERP>
__device__ __forceinline__ void gather2_grad(rsrc_t rs, const RefGeom& g, double qx, double qy,
                                             int xmin, float2* out, bool left) {
  constexpr int T = Kern<INTERP>::T;
  float wx[T], wy[T], dwx[T], dwy[T];
  uint32_t yb[T];
  const uint32_t xo = setup_x<INTERP, true>(g, qx, xmin, wx, dwx, left);
  setup_yz<INTERP, true>(g, qy, g.row, wy, dwy, yb, left);
  float2 s = make_float2(0.f, 0.f), sx = s, sy = s;
#pragma unroll
  for (int dy = 0; dy < T; ++dy) {
    const uint32_t ro = yb[dy] == kBig ? kBig : yb[dy] + xo;
    float2 r = make_float2(0.f, 0.f), rd = r;
#pragma unroll
    for (int dx = 0; dx < T; ++dx) {
      const float2 v = load_c64(rs, ro + 8u * dx);
      r.x = fmaf(wx[dx], v.x, r.x);
      r.y = fmaf(wx[dx], v.y, r.y);
      rd.x = fmaf(dwx[dx], v.x, rd.x);
      rd.y = fmaf(dwx[dx], v.y, rd.y);
    }
    s.x = fmaf(wy[dy], r.x, s.x);
    s.y = fmaf(wy[dy], r.y, s.y);
    sx.x = fmaf(wy[dy], rd.x, sx.x);
    sx.y = fmaf(wy[dy], rd.y, sx.y);
    sy.x = fmaf(dwy[dy], r.x, sy.x);
    sy.y = fmaf(dwy[dy], r.y, sy.y);
  }
  out[0] = s;
  out[1] = sx;
  out[2] = sy;
}

// ------------------------------------------------ half stencils (lane pairs)
//
// Two lanes share one output: lane half h reads x-taps [h*T/2, (h+1)*T/2) of
// every row with one load, so a load instruction covers the whole row of 32
// outputs in adjacent lanes (one cache line each) instead of half-rows of 64.
// In the value gather the y and z axis setups are split over the pair: the
// even lane sets up y, the odd lane z, and every lane then reads y from the
// even lane of its pair and z from the odd one (DPP quad permutes 0,0,2,2 and
// 1,1,3,3).  Both lanes of a pair take the same branches, so the lanes read
// are always active.  (The gradient gathers keep a full setup per lane: with
// the derivative weights the exchange spills at 128 registers.)

// (quad permutes read within the lane pair, whose two lanes are always
// active together, so no lane reads a disabled one and no old value is
// needed: a single v_mov_b32_dpp each)
__device__ __forceinline__ int from_even_lane(int v) { return __builtin_amdgcn_mov_dpp(v, 0xA0, 0xF, 0xF, true); }
__device__ __forceinline__ int from_odd_lane(int v) { return __builtin_amdgcn_mov_dpp(v, 0xF5, 0xF, 0xF, true); }

// The pair's y and z weights and row offsets (in residue order, see
// by_residue): each lane sets up one axis.
template <int INTERP>
__device__ __forceinline__ void setup_yz_pair(const RefGeom& g, double qy, double qz, int h, float* wy,
                                              uint32_t* yb, float* wz, uint32_t* zb) {
  constexpr int T = Kern<INTERP>::T;
  float w[T];
  uint32_t off[T];
  const int first = setup_yz<INTERP, false>(g, h ? qz : qy, h ? g.plane : g.row, w, nullptr, off);
  by_residue<T>(w, first);
  by_residue<T>(off, first);
#pragma unroll
  for (int d = 0; d < T; ++d) {
    wy[d] = __int_as_float(from_even_lane(__float_as_int(w[d])));
    wz[d] = __int_as_float(from_odd_lane(__float_as_int(w[d])));
    yb[d] = (uint32_t)from_even_lane((int)off[d]);
    zb[d] = (uint32_t)from_odd_lane((int)off[d]);
  }
}

template <int INTERP>
__device__ __forceinline__ float2 gather3_half(rsrc_t rs, const RefGeom& g, double qx, double qy,
                                               double qz, int xmin, int h) {
  constexpr int T = Kern<INTERP>::T, H = T / 2;
  float wx[T], wy[T], wz[T];
  uint32_t yb[T], zb[T];
  const uint32_t xo = setup_x<INTERP, false>(g, qx, xmin, wx, nullptr) + 8u * H * h;
  setup_yz_pair<INTERP>(g, qy, qz, h, wy, yb, wz, zb);
  // the lane's x weights folded into the y weights: two multiply-adds per
  // component and row
  float cy[T][H];
#pragma unroll
  for (int dy = 0; dy < T; ++dy)
#pragma unroll
    for (int d = 0; d < H; ++d) cy[dy][d] = wy[dy] * (h ? wx[H + d] : wx[d]);
#pragma unroll
  for (int d = 0; d < T; ++d) yb[d] = yb[d] == kBig ? kBig : yb[d] + xo;
  float2 acc = make_float2(0.f, 0.f);
#pragma unroll
  for (int dz = 0; dz < T; ++dz) {
    float2 pl = make_float2(0.f, 0.f);
#pragma unroll
    for (int dy = 0; dy < T; ++dy) {
      const uint32_t ro = zb[dz] + yb[dy];
      if (H == 2) {
        const float4 v = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)ro, 0, 0));
        pl.x = fmaf(cy[dy][0], v.x, pl.x);
        pl.y = fmaf(cy[dy][0], v.y, pl.y);
        pl.x = fmaf(cy[dy][H - 1], v.z, pl.x);
        pl.y = fmaf(cy[dy][H - 1], v.w, pl.y);
      } else {
        const float2 v = load_c64(rs, ro);
        pl.x = fmaf(cy[dy][0], v.x, pl.x);
        pl.y = fmaf(cy[dy][0], v.y, pl.y);
      }
    }
    acc.x = fmaf(wz[dz], pl.x, acc.x);
    acc.y = fmaf(wz[dz], pl.y, acc.y);
  }
  return acc;
}

// (left: q is the negated sample point, see axis_pos)
template <int INTERP>
__device__ __forceinline__ void gather3_grad_half(rsrc_t rs, const RefGeom& g, double qx, double qy,
                                                  double qz, int xmin, int h, float2* out, bool left) {
  constexpr int T = Kern<INTERP>::T, H = T / 2;
  float wx[T], wy[T], wz[T], dwx[T], dwy[T], dwz[T];
  uint32_t yb[T], zb[T];
  const uint32_t xo = setup_x<INTERP, true>(g, qx, xmin, wx, dwx, left) + 8u * H * h;
  const int y0 = setup_yz<INTERP, true>(g, qy, g.row, wy, dwy, yb, left);
  const int z0 = setup_yz<INTERP, true>(g, qz, g.plane, wz, dwz, zb, left);
  by_residue<T>(wy, y0);
  by_residue<T>(dwy, y0);
  by_residue<T>(yb, y0);
  by_residue<T>(wz, z0);
  by_residue<T>(dwz, z0);
  by_residue<T>(zb, z0);
  float wh[H], dh[H];
#pragma unroll
  for (int d = 0; d < H; ++d) {
    wh[d] = h ? wx[H + d] : wx[d];
    dh[d] = h ? dwx[H + d] : dwx[d];
  }
#pragma unroll
  for (int d = 0; d < T; ++d) yb[d] = yb[d] == kBig ? kBig : yb[d] + xo;
  float2 s = make_float2(0.f, 0.f), sx = s, sy = s, sz = s;
#pragma unroll
  for (int dz = 0; dz < T; ++dz) {
    float2 p0 = make_float2(0.f, 0.f), px = p0, py = p0;
#pragma unroll
    for (int dy = 0; dy < T; ++dy) {
      const uint32_t ro = zb[dz] + yb[dy];
      float2 r, rd;
      if (H == 2) {
        const float4 v = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)ro, 0, 0));
        r.x = fmaf(wh[0], v.x, wh[H - 1] * v.z);
        r.y = fmaf(wh[0], v.y, wh[H - 1] * v.w);
        rd.x = fmaf(dh[0], v.x, dh[H - 1] * v.z);
        rd.y = fmaf(dh[0], v.y, dh[H - 1] * v.w);
      } else {
        const float2 v = load_c64(rs, ro);
        r.x = wh[0] * v.x;
        r.y = wh[0] * v.y;
        rd.x = dh[0] * v.x;
        rd.y = dh[0] * v.y;
      }
      p0.x = fmaf(wy[dy], r.x, p0.x);
      p0.y = fmaf(wy[dy], r.y, p0.y);
      px.x = fmaf(wy[dy], rd.x, px.x);
      px.y = fmaf(wy[dy], rd.y, px.y);
      py.x = fmaf(dwy[dy], r.x, py.x);
      py.y = fmaf(dwy[dy], r.y, py.y);
    }
    s.x = fmaf(wz[dz], p0.x, s.x);
    s.y = fmaf(wz[dz], p0.y, s.y);
    sx.x = fmaf(wz[dz], px.x, sx.x);
    sx.y = fmaf(wz[dz], px.y, sx.y);
    sy.x = fmaf(wz[dz], py.x, sy.x);
    sy.y = fmaf(wz[dz], py.y, sy.y);
    sz.x = fmaf(dwz[dz], p0.x, sz.x);
    sz.y = fmaf(dwz[dz], p0.y, sz.y);
  }
  out[0] = s;
  out[1] = sx;
  out[2] = sy;
  out[3] = sz;
}

// Sum of a value over the two lanes of a pair: a DPP quad permutation (lanes
// 1, 0, 3, 2) feeds the add, with no LDS round trip.  Every lane of the wave
// must be active.
__device__ __forceinline__ float pair_sum1(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float2 pair_sum(float2 v) { return make_float2(pair_sum1(v.x), pair_sum1(v.y)); }

// Does the secondary sum at -m (x-taps >= xmin2) have a tap of nonzero
// weight?  For the cubic kernel a tap of zero weight still has a nonzero
// derivative (K'(+-1) = -+0.5), so any tap in range counts.  For the linear
// kernel the only candidate tap, floor(-m_x) + 1, has weight frac(-m_x); at an
// integer -m_x it carries no value and is skipped, which keeps the gradient a
// one-sided derivative at the kink.
template <int INTERP>
__device__ __forceinline__ bool needs_secondary(double mx, int xmin2) {
  using K = Kern<INTERP>;
  const double q = -mx, fl = floor(q);
  if (INTERP == 0) return (int)fl + 1 >= xmin2 && q > fl;
  return (int)fl + K::OFF + K::T - 1 >= xmin2;
}

// The same test for the gradient gathers, whose main sum at m = -p (folded
// samples, xmin2 = 0) uses the mirrored stencil of axis_pos's LEFT form, and
// whose secondary sum is then taken at p itself with floor(p).  A linear tap
// of weight 0 still carries derivative +1, so the secondary sum is needed
// whenever its first tap floor(p_x) + 1 >= 0 (p_x >= -1), integer or not.
// Unfolded linear samples (xmin2 = 1) have every tap at x >= 0.  Cubic
// stencils are C1, and the tests of needs_secondary already count every tap.
template <int INTERP>
__device__ __forceinline__ bool needs_secondary_grad(double mx, int xmin2) {
  if (INTERP == 0) return xmin2 == 0 && floor(-mx) >= -1.0;
  return needs_secondary<INTERP>(mx, xmin2);
}

}  // namespace tp
