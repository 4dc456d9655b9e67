// Projector kernels for gfx950: forward gather and pose gradients (the
// adjoint lives in tp_adjoint.hip); 2D and 3D references; linear and Catmull-Rom
// interpolation; the forward that saves each output's Jacobian and the pose
// gradients taken from it.
//
// 2D: one thread per output frequency, a 256-thread workgroup covers a 16x16
// tile (kx, ky-row) of one projection.  3D: two lanes per output, each
// gathering half of every x-row, so a workgroup covers 8x16 outputs (a wave
// 8x4).  The
// grid enumerates (batch, pose, tile) pose-major and is remapped so each XCD
// walks contiguous tiles of the same pose.  The rotation and shift of a pose
// are wave-uniform (kernel-argument derived addresses -> scalar loads).
#include "tp_gradjac.h"
#include "tp_internal.h"
#include "tp_stencil.h"

namespace tp {

namespace {

struct Out {
  int b, n, kx, iy, ky;
  bool in;    // inside the output array
  bool keep;  // inside the cutoff
};

// PAIRS: two lanes per output (lane pair = output threadIdx.x / 2).
template <bool PAIRS = false>
__device__ __forceinline__ Out locate(const OpParams& p) {
  Out o;
  const uint32_t g = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t tile = g % (uint32_t)p.tiles_per_pose;
  const uint32_t bn = g / (uint32_t)p.tiles_per_pose;
  o.n = (int)(bn % (uint32_t)p.P);
  o.b = (int)(bn / (uint32_t)p.P);
  const int oi = PAIRS ? (int)(threadIdx.x >> 1) : (int)threadIdx.x;
  constexpr int TX = PAIRS ? kTileXPairs : kTileX;
  o.kx = (int)(tile % (uint32_t)p.tiles_x) * TX + oi % TX;
  o.iy = (int)(tile / (uint32_t)p.tiles_x) * p.tile_y + oi / TX;
  o.in = o.kx < p.Wo && o.iy < p.No;
  o.ky = signed_row(o.iy, p.No);
  const long long k2 = (long long)o.kx * o.kx + (long long)o.ky * o.ky;
  o.keep = o.in && (p.cut2 < 0 || k2 <= p.cut2);
  return o;
}

// The two-tile 3D kernel (k_grad3p): a workgroup takes two vertically adjacent tiles
// of one pose (tile rows 2r and 2r + 1), batch t the tile row 2r + t, two
// lanes per output in both.
__device__ __forceinline__ void locate2(const OpParams& p, Out* o) {
  const uint32_t per = (uint32_t)p.tiles_x * (((uint32_t)p.tiles_y + 1u) >> 1);
  const uint32_t g = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t tile = g % per, bn = g / per;
  const int oi = (int)(threadIdx.x >> 1);
  const int kx = (int)(tile % (uint32_t)p.tiles_x) * kTileXPairs + oi % kTileXPairs;
  const int row0 = (int)(tile / (uint32_t)p.tiles_x) * 2 * p.tile_y + oi / kTileXPairs;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    o[t].n = (int)(bn % (uint32_t)p.P);
    o[t].b = (int)(bn / (uint32_t)p.P);
    o[t].kx = kx;
    o[t].iy = row0 + t * p.tile_y;
    o[t].in = o[t].kx < p.Wo && o[t].iy < p.No;
    o[t].ky = signed_row(o[t].iy, p.No);
    const long long k2 = (long long)o[t].kx * o[t].kx + (long long)o[t].ky * o[t].ky;
    o[t].keep = o[t].in && (p.cut2 < 0 || k2 <= p.cut2);
  }
}

// p = os * (kx R[0,:] + ky R[1,:]) in fp64; false if a component is not finite
// or beyond +-2^30 (such samples read 0).
template <int NDIM>
__device__ __forceinline__ bool sample_point(const OpParams& p, const Out& o, double* q) {
  const float* R = p.rot + ((size_t)(p.B_rot == 1 ? 0 : o.b) * p.P + o.n) * (NDIM * NDIM);
  const double os = (double)p.os;
  bool ok = true;
#pragma unroll
  for (int j = 0; j < NDIM; ++j) {
    q[j] = os * ((double)o.kx * (double)R[j] + (double)o.ky * (double)R[NDIM + j]);
    ok = ok && (fabs(q[j]) <= kCoordLimit);
  }
  return ok;
}

__device__ __forceinline__ float2 pose_shift(const OpParams& p, const Out& o) {
  if (!p.shift) return make_float2(0.f, 0.f);
  const float* s = p.shift + ((size_t)(p.B_shift == 1 ? 0 : o.b) * p.P + o.n) * 2;
  return make_float2(s[0], s[1]);
}

// (the pose's offset is uniform over the workgroup; the in-image offset is
// below No * Wo < 2^32 for boxes up to 65535)
__device__ __forceinline__ size_t img_index(const OpParams& p, const Out& o) {
  const size_t pose = (size_t)o.b * p.P + o.n;
  return pose * ((size_t)p.No * p.Wo) + ((uint32_t)o.iy * (uint32_t)p.Wo + (uint32_t)o.kx);
}

// The one-lane-per-output kernels below run the 2D path only (the 3D
// forwards and gradients use lane pairs).
template <int NDIM, int INTERP>
__device__ __forceinline__ float2 gather(rsrc_t rs, const RefGeom& g, const double* q, int xmin) {
  static_assert(NDIM == 2, "3D gathers use the lane-pair kernels");
  return gather2<INTERP>(rs, g, q[0], q[1], xmin);
}

template <int NDIM, int INTERP>
__device__ __forceinline__ void gather_grad(rsrc_t rs, const RefGeom& g, const double* q, int xmin,
                                            float2* out, bool left) {
  static_assert(NDIM == 2, "3D gathers use the lane-pair kernels");
  gather2_grad<INTERP>(rs, g, q[0], q[1], xmin, out, left);
}

// ------------------------------------------------------------------ forward

template <int NDIM, int INTERP>
__global__ __launch_bounds__(kBlock) void k_project(OpParams p) {
  const Out o = locate(p);
  if (!o.in) return;
  float2 res = make_float2(0.f, 0.f);
  double q[NDIM];
  if (o.keep && sample_point<NDIM>(p, o, q)) {
    const RefGeom g = ref_geom(p);
    const rsrc_t rs = make_rsrc(p.ref + (size_t)o.b * p.ref_elems, p.ref_bytes);
    const bool c = q[0] < 0.0;
    double m[NDIM], mneg[NDIM];
#pragma unroll
    for (int j = 0; j < NDIM; ++j) {
      m[j] = c ? -q[j] : q[j];
      mneg[j] = -m[j];
    }
    const int xmin1 = c ? 1 : 0, xmin2 = c ? 0 : 1;
    float2 mv = gather<NDIM, INTERP>(rs, g, m, xmin1);
    asm volatile("" : "+v"(mv.x), "+v"(mv.y));  // main sum first (see k_project3p)
    float2 sv = make_float2(0.f, 0.f);
    if (needs_secondary<INTERP>(m[0], xmin2)) sv = gather<NDIM, INTERP>(rs, g, mneg, xmin2);
    res = c ? make_float2(mv.x + sv.x, sv.y - mv.y) : make_float2(mv.x + sv.x, mv.y - sv.y);
    if (p.shift) {
      const float2 s = pose_shift(p, o);
      res = cmul(shift_phase(o.kx, o.ky, s.x, s.y, p.inv_no), res);
    }
  }
  p.img_out[img_index(p, o)] = res;
}

// ----------------------------------------------------------- pose gradients

template <int NDIM, int INTERP>
__global__ __launch_bounds__(kBlock) void k_grad_pose(OpParams p) {
  constexpr int NV = 2 * NDIM + 2;  // dR rows 0 and 1, then ds_x, ds_y
  const Out o = locate(p);
  double acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.0;
  double q[NDIM];
  if (o.keep && sample_point<NDIM>(p, o, q)) {
    const RefGeom g = ref_geom(p);
    const rsrc_t rs = make_rsrc(p.ref + (size_t)o.b * p.ref_elems, p.ref_bytes);
    const bool c = q[0] < 0.0;
    double m[NDIM], mneg[NDIM];
#pragma unroll
    for (int j = 0; j < NDIM; ++j) {
      m[j] = c ? -q[j] : q[j];
      mneg[j] = -m[j];
    }
    const int xmin1 = c ? 1 : 0, xmin2 = c ? 0 : 1;
    float2 mv[NDIM + 1], sv[NDIM + 1];
    // the stencil at the negated sample point is the mirror of p's (left)
    gather_grad<NDIM, INTERP>(rs, g, m, xmin1, mv, c);
#pragma unroll
    for (int j = 0; j <= NDIM; ++j) asm volatile("" : "+v"(mv[j].x), "+v"(mv[j].y));  // main sums first
#pragma unroll
    for (int j = 0; j <= NDIM; ++j) sv[j] = make_float2(0.f, 0.f);
    if (needs_secondary_grad<INTERP>(m[0], xmin2)) gather_grad<NDIM, INTERP>(rs, g, mneg, xmin2, sv, !c);
    // S and dS/dp (chain rule through m = +-p, see tp_device.h)
    float2 S, dS[NDIM];
    if (c) {
      S = make_float2(mv[0].x + sv[0].x, sv[0].y - mv[0].y);
#pragma unroll
      for (int j = 0; j < NDIM; ++j) dS[j] = make_float2(sv[j + 1].x - mv[j + 1].x, sv[j + 1].y + mv[j + 1].y);
    } else {
      S = make_float2(mv[0].x + sv[0].x, mv[0].y - sv[0].y);
#pragma unroll
      for (int j = 0; j < NDIM; ++j) dS[j] = make_float2(mv[j + 1].x - sv[j + 1].x, mv[j + 1].y + sv[j + 1].y);
    }
    const float2 G = p.img[img_index(p, o)];
    float2 gph = conjf2(G);  // conj(G) * phase
    if (p.shift) {
      const float2 s = pose_shift(p, o);
      gph = cmul(gph, shift_phase(o.kx, o.ky, s.x, s.y, p.inv_no));
    }
    const double os = (double)p.os;
#pragma unroll
    for (int j = 0; j < NDIM; ++j) {
      const double dldp = (double)gph.x * dS[j].x - (double)gph.y * dS[j].y;  // Re(g dS_j)
      acc[j] = os * o.kx * dldp;
      acc[NDIM + j] = os * o.ky * dldp;
    }
    const double im_gs = (double)gph.x * S.y + (double)gph.y * S.x;  // Im(g S)
    const double two_pi_over_n = 6.283185307179586476925 * p.inv_no;
    acc[2 * NDIM] = two_pi_over_n * o.kx * im_gs;
    acc[2 * NDIM + 1] = two_pi_over_n * o.ky * im_gs;
  }
  // workgroup reduction in fp64: wave shuffles, then LDS across the 4 waves
  __shared__ double red[kBlock / 64][8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (__ballot(o.keep) != 0ull) {
    double a8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a8[i] = i < NV ? acc[i] : 0.0;
    const double d = wave_sum8(a8);
    if ((lane & 7) == 0) red[wave][lane >> 3] = d;
  } else if (lane < 8) {
    red[wave][lane] = 0.0;
  }
  __syncthreads();
  if (threadIdx.x < NV) {
    const int i = threadIdx.x;
    double v = 0.0;
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) v += red[w][i];
    const uint32_t g = xcd_remap(blockIdx.x, gridDim.x);
    const uint32_t bn = g / (uint32_t)p.tiles_per_pose;
    const int n = (int)(bn % (uint32_t)p.P), b = (int)(bn / (uint32_t)p.P);
    if (i < 2 * NDIM) {
      if (p.grad_rot) {
        const int row = i / NDIM, col = i % NDIM;
        const size_t br = p.B_rot == 1 ? 0 : (size_t)b;
        unsafeAtomicAdd(p.grad_rot + ((br * p.P + n) * NDIM + row) * NDIM + col, (float)v);
      }
    } else if (p.grad_shift) {
      const size_t bs = p.B_shift == 1 ? 0 : (size_t)b;
      unsafeAtomicAdd(p.grad_shift + (bs * p.P + n) * 2 + (i - 2 * NDIM), (float)v);
    }
  }
}

// ------------------------------------------------- 3D with two lanes per output

// MAIN_FIRST: finish the main sum before the secondary gather (the reference
// is in the Infinity Cache; see ref_cached)
template <int INTERP, bool MAIN_FIRST>
__global__ __launch_bounds__(kBlock) void k_project3p(OpParams p) {
  const Out o = locate<true>(p);
  const int h = threadIdx.x & 1;
  const float2 sh = pose_shift(p, o);  // read before any store: a scalar load
  double q[3] = {0.0, 0.0, 0.0};
  const bool active = o.keep && sample_point<3>(p, o, q);
  float2 res = make_float2(0.f, 0.f);
  if (active) {
    const RefGeom g = ref_geom(p);
    const rsrc_t rs = make_rsrc(p.ref + (size_t)o.b * p.ref_elems, p.ref_bytes);
    const bool c = q[0] < 0.0;
    double m[3], mneg[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      m[j] = c ? -q[j] : q[j];
      mneg[j] = -m[j];
    }
    const int xmin1 = c ? 1 : 0, xmin2 = c ? 0 : 1;
    float2 mv = gather3_half<INTERP>(rs, g, m[0], m[1], m[2], xmin1, h);
    // finish the main sum before the secondary gather: its loads then find
    // the main gather's registers free and go out together
    if (MAIN_FIRST) asm volatile("" : "+v"(mv.x), "+v"(mv.y));
    float2 sv = make_float2(0.f, 0.f);
    if (needs_secondary<INTERP>(m[0], xmin2)) sv = gather3_half<INTERP>(rs, g, mneg[0], mneg[1], mneg[2], xmin2, h);
    res = c ? make_float2(mv.x + sv.x, sv.y - mv.y) : make_float2(mv.x + sv.x, mv.y - sv.y);
  }
  res = pair_sum(res);  // both lanes of a pair share `active`
  if (!o.in || h) return;
  if (active && p.shift) res = cmul(shift_phase(o.kx, o.ky, sh.x, sh.y, p.inv_no), res);
  p.img_out[img_index(p, o)] = res;
}

// S and dS/dp at an output's sample point from the value and derivative
// gathers, summed over the lane pair (both lanes hold the totals; zero where
// the output is not active).
// MAIN_FIRST: finish the main sums before the secondary gather (faster for
// k_grad3p; the Jacobian forward measured slower with it).
template <int INTERP, bool MAIN_FIRST>
__device__ __forceinline__ void pair_grad_values(const OpParams& p, const Out& o, int h, bool active,
                                                 const double* q, float2& S, float2* dS) {
  S = make_float2(0.f, 0.f);
#pragma unroll
  for (int j = 0; j < 3; ++j) dS[j] = S;
  if (active) {
    const bool c = q[0] < 0.0;
    const RefGeom g = ref_geom(p);
    const rsrc_t rs = make_rsrc(p.ref + (size_t)o.b * p.ref_elems, p.ref_bytes);
    double m[3], mneg[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      m[j] = c ? -q[j] : q[j];
      mneg[j] = -m[j];
    }
    const int xmin1 = c ? 1 : 0, xmin2 = c ? 0 : 1;
    float2 mv[4], sv[4];
    // the stencil at the negated sample point is the mirror of p's (left)
    gather3_grad_half<INTERP>(rs, g, m[0], m[1], m[2], xmin1, h, mv, c);
    if (MAIN_FIRST) {
#pragma unroll
      for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(mv[j].x), "+v"(mv[j].y));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) sv[j] = make_float2(0.f, 0.f);
    if (needs_secondary_grad<INTERP>(m[0], xmin2))
      gather3_grad_half<INTERP>(rs, g, mneg[0], mneg[1], mneg[2], xmin2, h, sv, !c);
    // S and dS/dp (chain rule through m = +-p, see tp_device.h); linear in the halves
    if (c) {
      S = make_float2(mv[0].x + sv[0].x, sv[0].y - mv[0].y);
#pragma unroll
      for (int j = 0; j < 3; ++j) dS[j] = make_float2(sv[j + 1].x - mv[j + 1].x, sv[j + 1].y + mv[j + 1].y);
    } else {
      S = make_float2(mv[0].x + sv[0].x, mv[0].y - sv[0].y);
#pragma unroll
      for (int j = 0; j < 3; ++j) dS[j] = make_float2(mv[j + 1].x - sv[j + 1].x, mv[j + 1].y + sv[j + 1].y);
    }
  }
  S = pair_sum(S);  // both lanes of a pair share `active`
#pragma unroll
  for (int j = 0; j < 3; ++j) dS[j] = pair_sum(dS[j]);
}

// Two tiles per workgroup (locate2): the lane pairs gather S and dS for
// one output of each tile, then every lane forms the gradient terms of
// its own output and the wave reduces 64 outputs at once, so the G read, the
// phase and the fp64 terms run on every lane (3.70 against 4.22 ms for one
// tile at box 256, 4096 poses, 5 waves per SIMD in 91 registers).  With the
// reference streamed from HBM one tile per workgroup (k_grad3p_1) measured
// faster (6.29 against 6.78 ms at box 256, oversampling 2).  The forward
// keeps one tile:
// its two-tile form needs 93 registers, and the lost occupancy cost more
// than the shared tail saved.
template <int INTERP>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(5))) void k_grad3p(OpParams p) {
  constexpr int NV = 8;  // dR rows 0 and 1, then ds_x, ds_y
  constexpr int NT = 2;
  __shared__ double red[kBlock / 64][NV];
  Out ob[NT];
  locate2(p, ob);
  const int h = threadIdx.x & 1;
  const float2 sh = pose_shift(p, ob[0]);  // one pose, read before any store: a scalar load
  float2 S[NT], dS[NT][3];
  bool act[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    double q[3] = {0.0, 0.0, 0.0};
    act[t] = ob[t].keep && sample_point<3>(p, ob[t], q);
    pair_grad_values<INTERP, true>(p, ob[t], h, act[t], q, S[t], dS[t]);
    // the first tile's sums are finished before the second tile's gathers
    asm volatile("" : "+v"(S[t].x), "+v"(S[t].y));
#pragma unroll
    for (int j = 0; j < 3; ++j) asm volatile("" : "+v"(dS[t][j].x), "+v"(dS[t][j].y));
  }
  // lane h takes the pair's output in tile h
  const Out& o = h ? ob[1] : ob[0];
  const bool active = h ? act[1] : act[0];
  const float2 Sh = h ? S[1] : S[0];
  double acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.0;
  if (active) {
    // (G read here: reading it before the gathers raised the registers and
    // measured slower)
    float2 gph = conjf2(p.img[img_index(p, o)]);
    if (p.shift) gph = cmul(gph, shift_phase(o.kx, o.ky, sh.x, sh.y, p.inv_no));
    const double os = (double)p.os;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const float2 d = h ? dS[1][j] : dS[0][j];
      const double dldp = (double)gph.x * d.x - (double)gph.y * d.y;
      acc[j] = os * o.kx * dldp;
      acc[3 + j] = os * o.ky * dldp;
    }
    const double im_gs = (double)gph.x * Sh.y + (double)gph.y * Sh.x;
    const double two_pi_over_n = 6.283185307179586476925 * p.inv_no;
    acc[6] = two_pi_over_n * o.kx * im_gs;
    acc[7] = two_pi_over_n * o.ky * im_gs;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (__ballot(active) != 0ull) {
    const double d = wave_sum8(acc);
    if ((lane & 7) == 0) red[wave][lane >> 3] = d;
  } else if (lane < NV) {
    red[wave][lane] = 0.0;
  }
  __syncthreads();
  if (threadIdx.x < NV) {
    const int i = threadIdx.x;
    double v = 0.0;
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) v += red[w][i];
    if (v == 0.0) return;
    const int b = ob[0].b, n = ob[0].n;
    if (i < 6) {
      if (p.grad_rot) {
        const size_t br = p.B_rot == 1 ? 0 : (size_t)b;
        unsafeAtomicAdd(p.grad_rot + ((br * p.P + n) * 3 + i / 3) * 3 + i % 3, (float)v);
      }
    } else if (p.grad_shift) {
      const size_t bs = p.B_shift == 1 ? 0 : (size_t)b;
      unsafeAtomicAdd(p.grad_shift + (bs * p.P + n) * 2 + (i - 6), (float)v);
    }
  }
}

// One tile per workgroup: lane 0 of each pair forms its output's gradient
// terms.  Taken when the reference streams from HBM (see ref_cached).
// (4 waves per SIMD: capping registers at 128 measured 12 % faster at box
// 256 than the 155 the compiler picks on its own, with no spills)
template <int INTERP>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_grad3p_1(OpParams p) {
  constexpr int NV = 8;  // dR rows 0 and 1, then ds_x, ds_y
  __shared__ double red[kBlock / 64][NV];
  const Out o = locate<true>(p);
  const int h = threadIdx.x & 1;
  const float2 sh = pose_shift(p, o);  // read before any store: a scalar load
  double q[3] = {0.0, 0.0, 0.0};
  const bool active = o.keep && sample_point<3>(p, o, q);
  float2 S, dS[3];
  pair_grad_values<INTERP, true>(p, o, h, active, q, S, dS);
  double acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.0;
  if (active && h == 0) {
    // (G read here: reading it before the gathers raised the registers to
    // 117 and measured slower)
    float2 gph = conjf2(p.img[img_index(p, o)]);
    if (p.shift) gph = cmul(gph, shift_phase(o.kx, o.ky, sh.x, sh.y, p.inv_no));
    const double os = (double)p.os;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const double dldp = (double)gph.x * dS[j].x - (double)gph.y * dS[j].y;
      acc[j] = os * o.kx * dldp;
      acc[3 + j] = os * o.ky * dldp;
    }
    const double im_gs = (double)gph.x * S.y + (double)gph.y * S.x;
    const double two_pi_over_n = 6.283185307179586476925 * p.inv_no;
    acc[6] = two_pi_over_n * o.kx * im_gs;
    acc[7] = two_pi_over_n * o.ky * im_gs;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (__ballot(active) != 0ull) {
    const double d = wave_sum8(acc);
    if ((lane & 7) == 0) red[wave][lane >> 3] = d;
  } else if (lane < NV) {
    red[wave][lane] = 0.0;
  }
  __syncthreads();
  if (threadIdx.x < NV) {
    const int i = threadIdx.x;
    double v = 0.0;
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) v += red[w][i];
    if (v == 0.0) return;
    if (i < 6) {
      if (p.grad_rot) {
        const size_t br = p.B_rot == 1 ? 0 : (size_t)o.b;
        unsafeAtomicAdd(p.grad_rot + ((br * p.P + o.n) * 3 + i / 3) * 3 + i % 3, (float)v);
      }
    } else if (p.grad_shift) {
      const size_t bs = p.B_shift == 1 ? 0 : (size_t)o.b;
      unsafeAtomicAdd(p.grad_shift + (bs * p.P + o.n) * 2 + (i - 6), (float)v);
    }
  }
}

// Forward that also saves the Jacobian of every output with respect to its
// sample point, jac_j = phase * dS/dp_j, so that the pose gradients need no
// second pass over the reference (k_grad_jac).  The gathers are
// k_grad3p's; lane 0 of a pair writes the output and jac_x, lane 1 jac_y and
// jac_z ([B, P, 3, No, Wo], one plane per component).
// (4 waves per SIMD: capping registers at 128 measured faster than the 148
// the compiler picks on its own)
template <int INTERP>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_project3p_jac(OpParams p) {
  const Out o = locate<true>(p);
  const int h = threadIdx.x & 1;
  double q[3] = {0.0, 0.0, 0.0};
  const bool active = o.keep && sample_point<3>(p, o, q);
  float2 S, dS[3];
  pair_grad_values<INTERP, false>(p, o, h, active, q, S, dS);
  // lane 0 of a pair stores the output and jac_x, lane 1 jac_y and jac_z
  float2 a = h ? dS[1] : S, c = h ? dS[2] : dS[0];
  if (active && p.shift) {
    const float2 s = pose_shift(p, o);
    const float2 ph = shift_phase(o.kx, o.ky, s.x, s.y, p.inv_no);
    a = cmul(ph, a);
    c = cmul(ph, c);
  }
  if (!o.in) return;
  const size_t plane = (size_t)p.No * p.Wo;
  const size_t pose = (size_t)o.b * p.P + o.n;
  const size_t e = (size_t)o.iy * p.Wo + o.kx;
  float2* jac = p.jac_out + pose * 3 * plane + e;
  *(h ? jac + plane : p.img_out + pose * plane + e) = a;
  *(h ? jac + 2 * plane : jac) = c;
}

// Pose gradients from a saved Jacobian and projection: one workgroup per
// (batch, pose) streams the pose's outputs inside the cutoff (coalesced).
__global__ __launch_bounds__(kBlock) void k_grad_jac(OpParams p) {
  __shared__ double red[kBlock / 64][8];
  grad_jac_pose<kBlock>(p, blockIdx.x, red);
}

// Hermitian symmetry of the x = 0 plane: V(0, y, z) <- (V(0, y, z) +
// conj V(0, -y, -z)) / 2, indices mod N (self-mirrored entries keep their
// real part).  One thread per mirror pair, so the update is in place.
template <int NDIM>
__global__ __launch_bounds__(kBlock) void k_symmetrize_x0(float2* ref, int B, int N) {
  const long long per = NDIM == 3 ? (long long)N * N : (long long)N;
  const long long i = (long long)blockIdx.x * kBlock + threadIdx.x;
  if (i >= per * B) return;
  const int b = (int)(i / per);
  const int r = (int)(i % per);
  const int iy = r % N, iz = NDIM == 3 ? r / N : 0;
  const int my = (N - iy) % N, mz = NDIM == 3 ? (N - iz) % N : 0;
  const int mr = mz * N + my;
  if (mr < r) return;  // the pair's other thread does it
  const size_t wh = (size_t)(N / 2 + 1);
  float2* base = ref + (size_t)b * (size_t)per * wh;
  float2* a = base + (size_t)r * wh;
  float2* c = base + (size_t)mr * wh;
  const float2 va = *a, vc = *c;
  const float2 h = make_float2(0.5f * (va.x + vc.x), 0.5f * (va.y - vc.y));
  *a = h;
  *c = make_float2(h.x, -h.y);
}

__global__ __launch_bounds__(kBlock) void k_zero(uint32_t* ptr, size_t words) {
  const size_t stride = (size_t)gridDim.x * kBlock;
  for (size_t i = (size_t)blockIdx.x * kBlock + threadIdx.x; i < words; i += stride) ptr[i] = 0u;
}

}  // namespace

// One batch entry's reference fits the 256 MB Infinity Cache (box 256 at
// oversampling 1: 67.6 MB; box 320: 132 MB; box 256 at oversampling 2:
// 539 MB streams from HBM).  The gathers' scheduling choices (main sum
// first, two-tile pose gradients) were measured faster there and slower
// when the taps come from HBM, where more loads in flight per wave pay.
static bool ref_cached(const OpParams& p) { return (uint64_t)p.ref_elems * 8u <= (256ull << 20); }

hipError_t launch_project(const OpParams& p, int interp, hipStream_t s) {
  const dim3 grid(p.nblocks), block(kBlock);
  if (p.ndim == 3) {
    const bool c = ref_cached(p);
    if (interp) {
      if (c) hipLaunchKernelGGL((k_project3p<1, true>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((k_project3p<1, false>), grid, block, 0, s, p);
    } else {
      if (c) hipLaunchKernelGGL((k_project3p<0, true>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((k_project3p<0, false>), grid, block, 0, s, p);
    }
  } else {
    if (interp) hipLaunchKernelGGL((k_project<2, 1>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_project<2, 0>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_grad_pose(const OpParams& p, int interp, hipStream_t s) {
  const dim3 grid(p.nblocks), block(kBlock);
  if (p.ndim == 3) {
    if (ref_cached(p)) {
      if (interp) hipLaunchKernelGGL((k_grad3p<1>), dim3(p.nblocks2), block, 0, s, p);
      else hipLaunchKernelGGL((k_grad3p<0>), dim3(p.nblocks2), block, 0, s, p);
    } else {
      if (interp) hipLaunchKernelGGL((k_grad3p_1<1>), grid, block, 0, s, p);
      else hipLaunchKernelGGL((k_grad3p_1<0>), grid, block, 0, s, p);
    }
  } else {
    if (interp) hipLaunchKernelGGL((k_grad_pose<2, 1>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_grad_pose<2, 0>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

hipError_t launch_project_jac(const OpParams& p, int interp, hipStream_t s) {
  const dim3 grid(p.nblocks), block(kBlock);
  if (interp) hipLaunchKernelGGL((k_project3p_jac<1>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((k_project3p_jac<0>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_grad_jac(const OpParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_grad_jac, dim3((unsigned)((size_t)p.B * p.P)), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_symmetrize_x0(float2* ref, int ndim, int B, int N, hipStream_t s) {
  const long long n = (long long)B * N * (ndim == 3 ? N : 1);
  const dim3 grid((unsigned)((n + kBlock - 1) / kBlock)), block(kBlock);
  if (ndim == 3) hipLaunchKernelGGL((k_symmetrize_x0<3>), grid, block, 0, s, ref, B, N);
  else hipLaunchKernelGGL((k_symmetrize_x0<2>), grid, block, 0, s, ref, B, N);
  return hipGetLastError();
}

hipError_t launch_zero(void* ptr, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  size_t blocks = (words + kBlock - 1) / kBlock;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(k_zero, dim3((unsigned)blocks), dim3(kBlock), 0, s, (uint32_t*)ptr, words);
  return hipGetLastError();
}

}  // namespace tp
