// Building blocks of the brick-owned adjoint kernels of tp_adjoint.hip (the
// adjoint and its modes): brick decomposition, the LDS accumulator layout and
// its int32 fixed point, lattice points and their values, the spread of one
// lattice point over its taps.
//
// The adjoint spreads every kept output c = conj(phase) G over the taps the
// forward read it from; a tap with x < 0 sends conj(w c) to -t (the forward's
// Friedel fold).  Equivalently, extend each projection to the full frequency
// plane: a real output k (kx >= 0) lands at p(k) with value c(k) on taps with
// x >= 0, its mirror -k lands at p(-k) = -p(k) with value conj(c(k)) on taps
// with x >= 1.  The kx = 0 column carries both.
#pragma once

#include "tp_bricks.h"
#include "tp_internal.h"
#include "tp_stencil.h"

namespace tp {
namespace adj {
constexpr int kVox = 4096;          // voxels per brick
constexpr int kGroupMax = 16;       // poses per fixed-point group

// Fixed point.  A pose adds to a voxel at most 2 m (a lattice point carries
// a real and a mirror value, m the largest |re| + |im| of G) times W, the sum
// of |w| over its lattice points.  Searched over orientations, voxel offsets
// and oversampling 0.25 to 2 (a CPU test), W / dens stays below 1.62 (cubic
// slices), 1.27 (linear slices), 2.05 (cubic volume lattices) and 1.44
// (linear volume lattices); nearly degenerate rows cap dens at 0.4 times
// their rectangle's lattice count + 1, which bounds W by itself (every |w| <=
// 1).  The quantum assumes W <= kDensBound dens:
//   q = 2 kDensBound sum_poses(dens) m_assume / 2^kQuantumBits,
// not rounded to a power of two, with m_assume >= the group's m (checked;
// else the group is redone).  Every int32 sum then stays below
// 2.05 / 2.5 * 2^30, under 2^31 / 2.4.
constexpr float kDensBound = 2.5f;
constexpr int kQuantumBits = 30;

// Brick of the stored half-volume owned by one workgroup: 16 x 16 x BZ
// voxels in 3D, 64 x 64 pixels in 2D.
template <int NDIM, int BZ = 16>
struct Brick {
  static constexpr int X = NDIM == 3 ? 16 : 64, Y = NDIM == 3 ? 16 : 64, Z = NDIM == 3 ? BZ : 1;
};

// LDS accumulator of a brick: W slots (packed (re, im) pairs, or int32 real
// parts for the weight volume) holding the brick's (y, z) rows of X voxels
// at a stride of S = X + kGuard slots, starting kGuard slots in, so the
// kGuard slots before each row are shared guard slots: a tap up to kGuard
// voxels beyond the brick in x, on either side, lands in them and they are
// never read.  A tap's slot is then its row's base plus a compile-time
// offset, and no x test is needed.  Bank pairs are slot mod 16: the odd row
// stride and a z-plane stride of 5 mod 16 (padded) keep taps that differ in
// y or z only off each other's banks.
constexpr int kGuard = 3;  // the cubic stencil reaches 3 voxels past its first tap
// G guard rows and planes follow the brick's last row and plane (exclusive
// y and z ownership).
template <int NDIM, int G = 0, int BZ = 16>
struct AccLayout {
  static constexpr int S = Brick<NDIM, BZ>::X + kGuard;
  static constexpr int ROWS = Brick<NDIM, BZ>::Y + G;
  static constexpr int PZ = NDIM == 3 ? ROWS * S + ((5 - ROWS * S % 16) + 16) % 16 : 0;
  static constexpr int W = (NDIM == 3 ? (Brick<NDIM, BZ>::Z + G) * PZ : Brick<NDIM, BZ>::Y * S) + kGuard;
};
template <int NDIM, int G = 0, int BZ = 16>
__device__ __forceinline__ int acc_word(int x, int y, int z) {
  return kGuard + z * AccLayout<NDIM, G, BZ>::PZ + y * AccLayout<NDIM, G, BZ>::S + x;
}

// (re, im) int32 pair as one int64, re * 2^32 + im: sums of such values
// decode uniquely while both component sums stay inside int32.
__device__ __forceinline__ unsigned long long pack_pair(int re, int im) {
  const unsigned hi = (unsigned)(re + (im >> 31));
  return ((unsigned long long)hi << 32) | (unsigned)im;
}
__device__ __forceinline__ void unpack_pair(unsigned long long v, int& re, int& im) {
  im = (int)(unsigned)(v & 0xFFFFFFFFull);
  re = (int)(long long)((long long)v >> 32) + (im < 0 ? 1 : 0);
}

// float -> int32, rounding to nearest (ties up): one VALU instruction.
__device__ __forceinline__ int cvt_rpi(float x) {
  int r;
  asm("v_cvt_rpi_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}

struct BrickPos {
  int b;            // batch entry
  int x0, y0, z0;   // first voxel (x from 0, y and z signed)
  int x1, y1, z1;   // last voxel (inclusive, clipped to the stored range)
  int xlim, ylim, zlim;  // last x column, y row and z plane that taps are
                         // spread to (x1, y1 and z1, or with exclusive
                         // ownership the guards in range)
  bool xbottom, ybottom, zbottom;  // the lowest brick of the stored x / y / z range
  int n0, n1;       // pose range of this workgroup
  bool chunked;     // merged with atomics
  bool valid;
};

// Pose chunks of a brick.  A random plane through the origin meets a ball of
// radius rho centred at distance r with probability about rho / r, so bricks
// near the origin see every pose and outer ones a fraction; each chunk gets
// about pmax of the poses expected to reach the brick.
template <int NDIM, int BZ = 16>
__device__ __forceinline__ int brick_chunks(const OpParams& p, const BrickParams& bp, int x0, int y0,
                                            int z0) {
  using BR = Brick<NDIM, BZ>;
  double frac = 1.0;
  if (NDIM == 3) {
    const double cx = x0 + 0.5 * (BR::X - 1), cy = y0 + 0.5 * (BR::Y - 1), cz = z0 + 0.5 * (BR::Z - 1);
    const double r = sqrt(cx * cx + cy * cy + cz * cz);
    const double rho = 0.5 * sqrt((double)((BR::X + 4) * (BR::X + 4) + (BR::Y + 4) * (BR::Y + 4) +
                                           (BR::Z + 4) * (BR::Z + 4)));
    frac = r > rho ? rho / r : 1.0;
  }
  const double c = ceil((double)p.P * frac / (double)bp.pmax);
  return (int)fmin(fmax(c, 1.0), (double)bp.cmax);
}

template <int NDIM, bool VOL, int BZ = 16>
__device__ __forceinline__ BrickPos decode(const OpParams& p, const BrickParams& bp, uint32_t lin) {
  using BR = Brick<NDIM, BZ>;
  BrickPos r;
  // plain round-robin over the XCDs: consecutive bricks (and the mostly empty
  // high chunk slots) spread evenly; bricks share little data across XCDs.
  // High chunk slots go first: only the busiest bricks near the origin have
  // them, so the long workgroups start early and the short ones fill the end.
  const int brick = (int)(lin % (uint32_t)bp.nbricks);
  const int ch = bp.cmax - 1 - (int)((lin / (uint32_t)bp.nbricks) % (uint32_t)bp.cmax);
  r.b = (int)(lin / ((uint32_t)bp.nbricks * (uint32_t)bp.cmax));
  const int bi = brick % bp.nb[0], bj = (brick / bp.nb[0]) % bp.nb[1], bk = brick / (bp.nb[0] * bp.nb[1]);
  const int lo = -(p.N / 2), hi = (p.N + 1) / 2 - 1;
  r.x0 = bi * BR::X;
  r.x1 = min(r.x0 + BR::X - 1, p.N / 2);
  r.y0 = lo + bj * BR::Y;
  r.y1 = min(r.y0 + BR::Y - 1, hi);
  if (NDIM == 3) {
    r.z0 = lo + bk * BR::Z;
    r.z1 = min(r.z0 + BR::Z - 1, hi);
  } else {
    r.z0 = r.z1 = 0;
  }
  r.xlim = r.x1;
  r.ylim = r.y1;
  r.zlim = r.z1;
  r.xbottom = r.x0 == 0;
  r.ybottom = r.y0 == lo;
  r.zbottom = r.z0 == (NDIM == 3 ? lo : 0);
  // every pose of a volume lattice reaches every brick inside its sphere
  const int nch = VOL ? bp.cmax : brick_chunks<NDIM, BZ>(p, bp, r.x0, r.y0, r.z0);
  r.valid = ch < nch && r.b < p.B;
  r.chunked = nch > 1;
  r.n0 = (int)((long long)p.P * ch / nch);
  r.n1 = (int)((long long)p.P * (ch + 1) / nch);
  return r;
}

// Sample points whose stencil can reach the brick lie in the brick widened
// by the stencil reach: [x0 - r, x1 + r) per axis (r = 2 cubic, 1 linear);
// any point outside has all its taps outside the brick.  With exclusive z
// ownership the brick takes in z only the points whose first tap lies in
// [z0, z1], q_z in [z0 - OFF, z1 + r), except the lowest brick, which also
// takes those whose first tap lies below the stored range.
template <int NDIM, int INTERP, bool EXCLZ = false>
__device__ __forceinline__ Box reach_box(const BrickPos& br) {
  constexpr double reach = INTERP ? 2.0 : 1.0;
  Box bx = {{br.x0 - reach, br.y0 - reach, br.z0 - reach}, {br.x1 + reach, br.y1 + reach, br.z1 + reach}};
  if (EXCLZ && !br.zbottom) bx.lo[2] = (double)(br.z0 - Kern<INTERP>::OFF);
  if (EXCLZ && !br.ybottom) bx.lo[1] = (double)(br.y0 - Kern<INTERP>::OFF);
  if (EXCLZ && !br.xbottom) bx.lo[0] = (double)(br.x0 - Kern<INTERP>::OFF);
  if (NDIM == 2) bx.lo[2] = bx.hi[2] = 0.0;
  return bx;
}

// A lattice point (kx, ky) of the full plane carries the real output (kx, ky)
// when kx >= 0 and the mirror of the real output (-kx, -ky) when kx <= 0.
__device__ __forceinline__ void lattice_parts(const OpParams& p, int kx, int ky, bool& real, bool& mirr) {
  const int rlo = -(p.No / 2), rhi = (p.No - 1) / 2;
  real = kx >= 0 && kx <= p.No / 2 && ky >= rlo && ky <= rhi;
  mirr = kx <= 0 && -kx <= p.No / 2 && -ky >= rlo && -ky <= rhi;
}

// G entries of a lattice point: the real output (kx, ky) and the real output
// (-kx, -ky) whose mirror it carries (zero where absent, or where valid is
// false).  (WEIGHTS: real weights, as (w, 0).)  Both loads are issued
// unconditionally, an absent entry reading the image's first entry instead,
// so that a caller can keep the loads in flight across other work (no
// branch between the loads and their use).
// (the image's offset is taken once; the in-image offsets are 32-bit, below
// No * Wo < 2^32)
template <bool WEIGHTS>
__device__ __forceinline__ void lattice_load(const OpParams& p, size_t img, int kx, int ky, bool valid, float2& gr,
                                             float2& gm) {
  bool real, mirr;
  lattice_parts(p, kx, ky, real, mirr);
  real = real && valid;
  mirr = mirr && valid;
  const size_t base = img * ((size_t)p.No * p.Wo);
  const uint32_t wo = (uint32_t)p.Wo;
  const uint32_t or_ = real ? (uint32_t)(ky < 0 ? ky + p.No : ky) * wo + (uint32_t)kx : 0u;
  const uint32_t om = mirr ? (uint32_t)(-ky < 0 ? -ky + p.No : -ky) * wo + (uint32_t)(-kx) : 0u;
  if (WEIGHTS) {
    const float* w = p.wimg + base;
    const float a = w[or_], b = w[om];
    gr = make_float2(real ? a : 0.f, 0.f);
    gm = make_float2(mirr ? b : 0.f, 0.f);
  } else {
    const float2* g = p.img + base;
    const float2 a = g[or_], b = g[om];
    gr = real ? a : make_float2(0.f, 0.f);
    gm = mirr ? b : make_float2(0.f, 0.f);
  }
}

// Phase B: sample point and the values spread by a lattice point that hit.
struct Cand {
  double q[3];
  float2 v0;   // value for taps at x = 0 (real part only)
  float2 v1;   // value for taps at x >= 1 (real + conj(mirror))
};

template <int NDIM>
__device__ __forceinline__ void lattice_values(const OpParams& p, const PoseView& pv, int kx, int ky,
                                               float2 gr, float2 gm, Cand& cd) {
#pragma unroll
  for (int j = 0; j < NDIM; ++j) cd.q[j] = (double)kx * pv.u[j] + (double)ky * pv.v[j];
  float2 cr = gr, cm = gm;
  if (p.shift) {
    // conj(phase(k)) G(k), and for the mirror conj(phase(-k)) G(-k) =
    // phase(k) G(-k): one phase per lattice point
    const float2 ph = shift_phase(kx, ky, pv.sx, pv.sy, p.inv_no);
    cr = cmul(conjf2(ph), gr);
    cm = cmul(ph, gm);
  }
  cd.v0 = cr;
  cd.v1 = make_float2(cr.x + cm.x, cr.y - cm.y);
}

// Hit of thread tid within a block of workgroup-size consecutive hits: each
// pair of waves takes alternate hits of its own 128.
// Consecutive hits are neighbouring lattice points whose sample points can
// share a voxel, and lanes adding to one LDS address in the same instruction
// serialise; two lattice steps apart (two voxels at oversampling 1) they
// cannot.  Measured against strides 1, 4 and 8, which were slower.
__device__ __forceinline__ int hit_slot(int tid) { return (tid & 63) * 2 + ((tid >> 6) & 1) + (tid >> 7) * 64 * 2; }

// Spread one lattice point over its taps inside the brick (int32 fixed point).
// The point lies in the brick's reach box, so its first x tap is at most
// kGuard voxels before the brick and its last at most kGuard after it: taps
// outside the brick in x fall into guard words.  Rows outside in y or z are
// skipped.  REAL: int32 real parts only (the weight volume), else packed
// pairs.
template <int NDIM, int INTERP, bool REAL, int G = 0>
__device__ __forceinline__ void spread(const BrickPos& br, const Cand& cd, float inv_q, unsigned long long* acc) {
  using L = AccLayout<NDIM, G>;
  using K = Kern<INTERP>;
  constexpr int T = K::T;
  static_assert(T - 1 <= kGuard, "guard words must cover the stencil");
  const AxisPos ax = axis_pos(cd.q[0], K::OFF), ay = axis_pos(cd.q[1], K::OFF);
  float wx[T], wy[T], wz[T];
  K::w(ax.f, wx);
  K::w(ay.f, wy);
  int z0 = 0;
  if (NDIM == 3) {
    const AxisPos az = axis_pos(cd.q[2], K::OFF);
    K::w(az.f, wz);
    z0 = az.x0;
  } else {
#pragma unroll
    for (int d = 0; d < T; ++d) wz[d] = d == 0 ? 1.f : 0.f;
  }
  // x weights folded with the per-x value (x = 0 takes the real part only)
  float are[T], aim[T];
#pragma unroll
  for (int d = 0; d < T; ++d) {
    const float2 v = ax.x0 + d >= 1 ? cd.v1 : cd.v0;
    are[d] = wx[d] * v.x * inv_q;
    aim[d] = wx[d] * v.y * inv_q;
    // with guard columns read back, a tap before x = 0 (whose slot is the
    // previous row's guard column) must add nothing
    if (G > 0 && ax.x0 + d < 0) are[d] = aim[d] = 0.f;
  }
  const int x0w = acc_word<NDIM, G>(ax.x0 - br.x0, 0, 0);
#pragma unroll
  for (int dz = 0; dz < (NDIM == 3 ? T : 1); ++dz) {
    const int tz = z0 + dz;
    if (NDIM == 3 && (tz < br.z0 || tz > br.zlim)) continue;
#pragma unroll
    for (int dy = 0; dy < T; ++dy) {
      const int ty = ay.x0 + dy;
      if (ty < br.y0 || ty > br.ylim) continue;
      const float wyz = wy[dy] * wz[dz];
      const int w = x0w + (NDIM == 3 ? tz - br.z0 : 0) * L::PZ + (ty - br.y0) * L::S;
#pragma unroll
      for (int dx = 0; dx < T; ++dx) {
        if (REAL) atomicAdd(reinterpret_cast<int*>(acc) + w + dx, cvt_rpi(are[dx] * wyz));
        else atomicAdd(acc + w + dx, pack_pair(cvt_rpi(are[dx] * wyz), cvt_rpi(aim[dx] * wyz)));
      }
    }
  }
}

// Which spread a 3D brick with guard columns, rows and planes (G = kGuard)
// takes: 0 the general one (spread()); 1 or 2 spread_interior(), for bricks
// that are not the lowest in y or z and whose guard rows and planes lie
// inside the stored range, so that every tap of a lattice point in the reach
// box lands in the accumulator (its first tap lies in the brick on every
// axis).  2: not the lowest brick in x either, so every x tap is at x >= 1;
// 1: the lowest, whose taps at x = 0 take the real part only and whose taps
// at x < 0 add nothing.
template <int NDIM, int G, int BZ = 16>
__device__ __forceinline__ int brick_kind(const BrickPos& br) {
  using BR = Brick<NDIM, BZ>;
  if (NDIM != 3 || G < kGuard) return 0;
  const bool yz = !br.ybottom && !br.zbottom && br.ylim == br.y0 + BR::Y + G - 1 && br.zlim == br.z0 + BR::Z + G - 1;
  return yz ? (br.xbottom ? 1 : 2) : 0;
}

// Spread of an interior brick (brick_kind 1 or 2), with the lanes of a wave
// reassigned so that the lanes of each LDS pass add to distinct banks.
//
// A wave's 64-bit LDS add is served 16 lanes at a time (lanes 16j .. 16j +
// 15), and lanes of one pass whose slots share a bank pair (slot mod 16)
// are served one after the other.  Every tap of a lattice point sits at a
// compile-time offset from its first tap's slot, so the bank pairs of all 64
// tap adds of a lane follow from that base slot.  The wave ranks its lattice
// points by base mod 16 (a counting sort, wave_rank) and deals them out
// round-robin over the four passes: with four points per bank pair every
// pass gets one of each.  The lattice points themselves (their G loads, the
// phase, the sample point) stay in the lanes that read them, which keeps the
// loads coalesced; only the spread's inputs move, through ds_permute.

// Inclusive prefix sum over the wave's 64 lanes (DPP row shifts within each
// row of 16 lanes, then the row broadcasts of lanes 15 and 31).  Every lane
// of the wave must be active.
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// The rank of each lane's key in the wave's stable ascending order of keys,
// for keys 0..15, with the lanes of key 16 (no point) after all others.  A
// counting sort: 16 counters of 8 bits in four words, one-hot per lane,
// prefix-summed over the lanes (counts stay below 65, so bytes never carry);
// the totals of the last lane, prefix-summed over the keys bytewise (a
// multiply by 0x01010101), give each key's first rank.  Every lane of the
// wave must be active.
__device__ __forceinline__ int wave_rank(int key) {
  const bool act = key < 16;
  const int wsel = key >> 2, sh = (key & 3) * 8;
  const uint32_t bit = act ? (1u << sh) : 0u;
  uint32_t c[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) c[w] = wave_prefix_sum(wsel == w ? bit : 0u);
  uint32_t first[4];  // byte b of word w: the first rank of key 4 w + b
  uint32_t below = 0;  // points with keys of the earlier words
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t inc = (uint32_t)__builtin_amdgcn_readlane((int)c[w], 63) * 0x01010101u;
    first[w] = (inc << 8) + below * 0x01010101u;
    below += inc >> 24;
  }
  const uint32_t fw = wsel == 0 ? first[0] : wsel == 1 ? first[1] : wsel == 2 ? first[2] : first[3];
  const uint32_t cw = wsel == 0 ? c[0] : wsel == 1 ? c[1] : wsel == 2 ? c[2] : c[3];
  const unsigned long long none = __ballot(!act);
  const int before = (int)__builtin_amdgcn_mbcnt_hi((unsigned)(none >> 32), __builtin_amdgcn_mbcnt_lo((unsigned)none, 0u));
  return act ? (int)(((fw >> sh) & 0xFFu) + ((cw >> sh) & 0xFFu) - 1u) : (int)below + before;
}

// Sends v to lane dest (a permutation of the wave's lanes).
__device__ __forceinline__ float permute_f(int dest, float v) {
  return __int_as_float(__builtin_amdgcn_ds_permute(dest << 2, __float_as_int(v)));
}

// Every lane of the wave calls it; act: the lane holds a lattice point in the
// reach box (cd valid).  XB: the lowest brick in x (brick_kind 1).  Packed
// (re, im) adds only: the weight volume keeps the general spread.
template <int INTERP, int G, bool XB, int BZ = 16>
__device__ __forceinline__ void spread_interior(const BrickPos& br, const Cand& cd, bool act, float inv_q,
                                                unsigned long long* acc) {
  using L = AccLayout<3, G, BZ>;
  using K = Kern<INTERP>;
  constexpr int T = K::T;
  uint32_t base = ~0u;  // XB: the first x tap + 8 in bits 16 and up
  float fx = 0.f, fy = 0.f, fz = 0.f, vr = 0.f, vi = 0.f, vr0 = 0.f, vi0 = 0.f;
  if (act) {
    const AxisPos ax = axis_pos(cd.q[0], K::OFF), ay = axis_pos(cd.q[1], K::OFF), az = axis_pos(cd.q[2], K::OFF);
    base = (uint32_t)acc_word<3, G, BZ>(ax.x0 - br.x0, ay.x0 - br.y0, az.x0 - br.z0);
    fx = ax.f;
    fy = ay.f;
    fz = az.f;
    vr = cd.v1.x * inv_q;
    vi = cd.v1.y * inv_q;
    if (XB) {
      vr0 = cd.v0.x * inv_q;
      vi0 = cd.v0.y * inv_q;
    }
  }
  const int rank = wave_rank(act ? (int)(base & 15u) : 16);
  const int dest = ((rank & 3) << 4) | (rank >> 2);
  if (XB && act) base |= (uint32_t)(axis_pos(cd.q[0], K::OFF).x0 + 8) << 16;
  base = (uint32_t)__builtin_amdgcn_ds_permute(dest << 2, (int)base);
  fx = permute_f(dest, fx);
  fy = permute_f(dest, fy);
  fz = permute_f(dest, fz);
  vr = permute_f(dest, vr);
  vi = permute_f(dest, vi);
  if (XB) {
    vr0 = permute_f(dest, vr0);
    vi0 = permute_f(dest, vi0);
  }
  if (base == ~0u) return;
  float wx[T], wy[T], wz[T];
  K::w(fx, wx);
  K::w(fy, wy);
  K::w(fz, wz);
  float are[T], aim[T];
  const int x0 = XB ? (int)(base >> 16) - 8 : 1;
  if (XB) base &= 0xFFFFu;
#pragma unroll
  for (int d = 0; d < T; ++d) {
    // (XB: a tap at x < 0, whose slot is the previous row's guard column,
    // adds nothing; a tap at x = 0 takes the real output's value only)
    const int xt = x0 + d;
    are[d] = wx[d] * (!XB || xt >= 1 ? vr : (xt == 0 ? vr0 : 0.f));
    aim[d] = wx[d] * (!XB || xt >= 1 ? vi : (xt == 0 ? vi0 : 0.f));
  }
  unsigned long long* a = acc + base;
#pragma unroll
  for (int dz = 0; dz < T; ++dz) {
#pragma unroll
    for (int dy = 0; dy < T; ++dy) {
      const float wyz = wy[dy] * wz[dz];
#pragma unroll
      for (int dx = 0; dx < T; ++dx) {
        const int o = dz * L::PZ + dy * L::S + dx;
        atomicAdd(a + o, pack_pair(cvt_rpi(are[dx] * wyz), cvt_rpi(aim[dx] * wyz)));
      }
    }
  }
}

// Mark the accumulator slots (set them to 1) that a lattice point's taps
// reach inside the brick, where its spread values are not finite: the x = 0
// taps when v0 is not, the x >= 1 taps when v1 is not (the same taps and row
// tests as spread(), whatever their weight: the product of a weight of 0 and a
// non-finite value is not finite either).
template <int NDIM, int INTERP, bool REAL, int G = 0, int BZ = 16>
__device__ __forceinline__ void mark_taps(const BrickPos& br, const double* q, bool bad0, bool bad1,
                                          unsigned long long* acc) {
  using L = AccLayout<NDIM, G, BZ>;
  using K = Kern<INTERP>;
  constexpr int T = K::T;
  const AxisPos ax = axis_pos(q[0], K::OFF), ay = axis_pos(q[1], K::OFF);
  const int z0 = NDIM == 3 ? axis_pos(q[2], K::OFF).x0 : 0;
  const int x0w = acc_word<NDIM, G, BZ>(ax.x0 - br.x0, 0, 0);
  for (int dz = 0; dz < (NDIM == 3 ? T : 1); ++dz) {
    const int tz = z0 + dz;
    if (NDIM == 3 && (tz < br.z0 || tz > br.zlim)) continue;
    for (int dy = 0; dy < T; ++dy) {
      const int ty = ay.x0 + dy;
      if (ty < br.y0 || ty > br.ylim) continue;
      const int w = x0w + (NDIM == 3 ? tz - br.z0 : 0) * L::PZ + (ty - br.y0) * L::S;
      for (int dx = 0; dx < T; ++dx) {
        const int tx = ax.x0 + dx;
        if (tx < 0 || !(tx == 0 ? bad0 : bad1)) continue;
        if (REAL) reinterpret_cast<int*>(acc)[w + dx] = 1;
        else acc[w + dx] = 1ull;
      }
    }
  }
}

__device__ __forceinline__ bool finite2(float2 v) { return isfinite(v.x) && isfinite(v.y); }

}  // namespace adj
}  // namespace tp
