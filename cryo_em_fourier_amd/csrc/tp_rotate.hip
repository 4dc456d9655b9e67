// 3D -> 3D rotation of a reference half-spectrum (subtomogram averaging):
// forward gather, its adjoint and the pose gradients, for gfx950.
//
// Every output frequency k = (kx, ky, kz) of an [N_out, N_out, N_out/2+1]
// half-spectrum samples the reference at p = os R^T k = os (kx R[0,:] +
// ky R[1,:] + kz R[2,:]) with the same per-tap Friedel fold and kernels as
// the central slice (which is the kz = 0 plane of this op), times the shift
// phase exp(-2 pi i k.s / N_out) of a 3-vector shift, inside the sphere
// |k| <= cutoff.  Two lanes per output, each gathering half of every x-row
// (as the central-slice kernels); a 256-lane workgroup covers 8 kx columns
// of 16 (kz, ky) rows of one pose.  The adjoint is the brick adjoint of
// tp_adjoint.hip run over volume lattices.
#include "tp_gradjac.h"
#include "tp_internal.h"
#include "tp_stencil.h"

namespace tp {

namespace {

struct ROut {
  int b, n, kx, ky, kz;
  size_t idx;   // output element
  bool in, keep;
};

__device__ __forceinline__ ROut rlocate(const OpParams& p) {
  ROut o;
  const uint32_t g = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t tile = g % (uint32_t)p.tiles_per_pose;
  const uint32_t bn = g / (uint32_t)p.tiles_per_pose;
  o.n = (int)(bn % (uint32_t)p.P);
  o.b = (int)(bn / (uint32_t)p.P);
  const int oi = (int)(threadIdx.x >> 1);  // lane pair
  o.kx = (int)(tile % (uint32_t)p.tiles_x) * kTileXPairs + oi % kTileXPairs;
  const long long row = (long long)(tile / (uint32_t)p.tiles_x) * kTileYPairs + oi / kTileXPairs;
  const long long rows = (long long)p.No * p.No;
  o.in = o.kx < p.Wo && row < rows;
  const int iz = (int)(row / p.No), iy = (int)(row % p.No);
  o.ky = signed_row(iy, p.No);
  o.kz = signed_row(iz, p.No);
  const long long k2 = (long long)o.kx * o.kx + (long long)o.ky * o.ky + (long long)o.kz * o.kz;
  o.keep = o.in && (p.cut2 < 0 || k2 <= p.cut2);
  o.idx = (((size_t)o.b * p.P + o.n) * (size_t)rows + (size_t)row) * p.Wo + o.kx;
  return o;
}

__device__ __forceinline__ const float* rrow(const OpParams& p, const ROut& o) {
  return p.rot + ((size_t)(p.B_rot == 1 ? 0 : o.b) * p.P + o.n) * 9;
}

// p = os R^T k in fp64; false if a component is not finite or beyond 2^30.
__device__ __forceinline__ bool rsample(const OpParams& p, const ROut& o, double* q) {
  const float* R = rrow(p, o);
  const double os = (double)p.os;
  bool ok = true;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    q[j] = os * ((double)o.kx * (double)R[j] + (double)o.ky * (double)R[3 + j] + (double)o.kz * (double)R[6 + j]);
    ok = ok && (fabs(q[j]) <= kCoordLimit);
  }
  return ok;
}

// exp(-2 pi i (kx sx + ky sy + kz sz) / N_out), turns reduced in fp64.
__device__ __forceinline__ float2 rphase(const OpParams& p, const ROut& o) {
  if (!p.shift) return make_float2(1.f, 0.f);
  const float* s = p.shift + ((size_t)(p.B_shift == 1 ? 0 : o.b) * p.P + o.n) * 3;
  return phase_of_turns(((double)o.kx * s[0] + (double)o.ky * s[1] + (double)o.kz * s[2]) * p.inv_no);
}

template <int INTERP>
__global__ __launch_bounds__(kBlock) void k_rotate(OpParams p) {
  const ROut o = rlocate(p);
  const int h = threadIdx.x & 1;
  float2 res = make_float2(0.f, 0.f);
  double q[3] = {0.0, 0.0, 0.0};
  const bool active = o.keep && rsample(p, o, q);
  if (active) {
    const RefGeom g = ref_geom(p);
    const rsrc_t rs = make_rsrc(p.ref + (size_t)o.b * p.ref_elems, p.ref_bytes);
    // main stencil around m = |p_x|-side sample, secondary across x = 0
    const bool c = q[0] < 0.0;
    double m[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) m[j] = c ? -q[j] : q[j];
    float2 mv = gather3_half<INTERP>(rs, g, m[0], m[1], m[2], c ? 1 : 0, h);
    // finish the main sum before the secondary gather, whose loads then go
    // out together instead of one round trip each
    asm volatile("" : "+v"(mv.x), "+v"(mv.y));
    float2 sv = make_float2(0.f, 0.f);
    if (needs_secondary<INTERP>(m[0], c ? 0 : 1)) sv = gather3_half<INTERP>(rs, g, -m[0], -m[1], -m[2], c ? 0 : 1, h);
    res = c ? make_float2(mv.x + sv.x, sv.y - mv.y) : make_float2(mv.x + sv.x, mv.y - sv.y);
  }
  res = pair_sum(res);  // both lanes of a pair share `active`
  if (!o.in || h) return;
  if (active) res = cmul(rphase(p, o), res);
  p.img_out[o.idx] = res;
}

// S and dS/dp at an output's sample point from the value and derivative
// gathers, summed over the lane pair (both lanes hold the totals; zero where
// the output is not active).
template <int INTERP>
__device__ __forceinline__ void rpair_grad_values(const OpParams& p, const ROut& o, int h, bool active,
                                                  const double* q, float2& S, float2* dS) {
  S = make_float2(0.f, 0.f);
#pragma unroll
  for (int j = 0; j < 3; ++j) dS[j] = S;
  if (active) {
    const RefGeom g = ref_geom(p);
    const rsrc_t rs = make_rsrc(p.ref + (size_t)o.b * p.ref_elems, p.ref_bytes);
    const bool c = q[0] < 0.0;
    double m[3];
#pragma unroll
    for (int j = 0; j < 3; ++j) m[j] = c ? -q[j] : q[j];
    float2 mv[4], sv[4];
    // the stencil at the negated sample point is the mirror of p's (left)
    gather3_grad_half<INTERP>(rs, g, m[0], m[1], m[2], c ? 1 : 0, h, mv, c);
#pragma unroll
    for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(mv[j].x), "+v"(mv[j].y));  // main sums first
#pragma unroll
    for (int j = 0; j < 4; ++j) sv[j] = make_float2(0.f, 0.f);
    if (needs_secondary_grad<INTERP>(m[0], c ? 0 : 1))
      gather3_grad_half<INTERP>(rs, g, -m[0], -m[1], -m[2], c ? 0 : 1, h, sv, !c);
    // S and dS/dp through m = +-p (as the central-slice gradient kernels)
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

// Pose gradients of L = Re sum conj(G) rotate(V): dL/dR[i][j] =
// os sum k_i Re(conj(G) phase dS/dp_j) (all three rows), dL/ds_j =
// sum (2 pi k_j / N_out) Im(conj(G) phase S).
// (4 waves per SIMD: measured 7 % faster at box 64 than the 161 registers
// the compiler picks on its own)
template <int INTERP>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_rotate_grad(OpParams p) {
  constexpr int NV = 12;
  __shared__ double red[kBlock / 64][16];
  const ROut o = rlocate(p);
  const int h = threadIdx.x & 1;
  double acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0;
  double q[3] = {0.0, 0.0, 0.0};
  const bool active = o.keep && rsample(p, o, q);
  float2 S, dS[3];
  rpair_grad_values<INTERP>(p, o, h, active, q, S, dS);
  if (active && h == 0) {
    const float2 gph = cmul(conjf2(p.img[o.idx]), rphase(p, o));
    const double os = (double)p.os;
    const double k[3] = {(double)o.kx, (double)o.ky, (double)o.kz};
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const double dldp = (double)gph.x * dS[j].x - (double)gph.y * dS[j].y;
#pragma unroll
      for (int i = 0; i < 3; ++i) acc[3 * i + j] = os * k[i] * dldp;
    }
    const double im_gs = (double)gph.x * S.y + (double)gph.y * S.x;
    const double two_pi_over_n = 6.283185307179586476925 * p.inv_no;
#pragma unroll
    for (int i = 0; i < 3; ++i) acc[9 + i] = two_pi_over_n * k[i] * im_gs;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const double d0 = wave_sum8(acc), d1 = wave_sum8(acc + 8);
  if ((lane & 7) == 0) {
    red[wave][lane >> 3] = d0;
    red[wave][8 + (lane >> 3)] = d1;
  }
  __syncthreads();
  if (threadIdx.x < NV) {
    const int i = threadIdx.x;
    double v = 0.0;
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) v += red[w][i];
    if (v == 0.0) return;
    const uint32_t gi = xcd_remap(blockIdx.x, gridDim.x);
    const uint32_t bn = gi / (uint32_t)p.tiles_per_pose;
    const int n = (int)(bn % (uint32_t)p.P), b = (int)(bn / (uint32_t)p.P);
    if (i < 9) {
      if (p.grad_rot) {
        const size_t br = p.B_rot == 1 ? 0 : (size_t)b;
        unsafeAtomicAdd(p.grad_rot + (br * p.P + n) * 9 + i, (float)v);
      }
    } else if (p.grad_shift) {
      const size_t bs = p.B_shift == 1 ? 0 : (size_t)b;
      unsafeAtomicAdd(p.grad_shift + (bs * p.P + n) * 3 + (i - 9), (float)v);
    }
  }
}

// Rotation that also saves the Jacobian of every output with respect to its
// sample point, jac_j = phase * dS/dp_j ([B, P, 3, No, No, Wo], one volume
// per component), for k_rotate_grad_jac: the gathers of k_rotate_grad,
// stored instead of reduced (lane 0 of a pair writes the output and jac_x,
// lane 1 jac_y and jac_z).
template <int INTERP>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(4))) void k_rotate_jac(OpParams p) {
  const ROut o = rlocate(p);
  const int h = threadIdx.x & 1;
  double q[3] = {0.0, 0.0, 0.0};
  const bool active = o.keep && rsample(p, o, q);
  float2 S, dS[3];
  rpair_grad_values<INTERP>(p, o, h, active, q, S, dS);
  if (!o.in) return;
  // lane 0 of a pair stores the output and jac_x, lane 1 jac_y and jac_z
  float2 a = h ? dS[1] : S, c = h ? dS[2] : dS[0];
  if (active && p.shift) {
    const float2 ph = rphase(p, o);
    a = cmul(ph, a);
    c = cmul(ph, c);
  }
  const size_t vol = (size_t)p.No * p.No * p.Wo;
  const size_t pose = (size_t)o.b * p.P + o.n;
  float2* jac = p.jac_out + pose * 3 * vol + (o.idx - pose * vol);
  *(h ? jac + vol : p.img_out + o.idx) = a;
  *(h ? jac + 2 * vol : jac) = c;
}

// Pose gradients from a saved Jacobian and rotation output: one workgroup
// per (batch, pose) streams the pose's outputs inside the sphere.
__global__ __launch_bounds__(kBlock) void k_rotate_grad_jac(OpParams p) {
  __shared__ double red[kBlock / 64][16];
  grad_jac_vol<kBlock>(p, blockIdx.x, red);
}

}  // namespace

hipError_t launch_rotate_jac(const OpParams& p, int interp, hipStream_t s) {
  const dim3 grid(p.nblocks), block(kBlock);
  if (interp) hipLaunchKernelGGL((k_rotate_jac<1>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((k_rotate_jac<0>), grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_rotate_grad_jac(const OpParams& p, hipStream_t s) {
  hipLaunchKernelGGL(k_rotate_grad_jac, dim3((unsigned)((size_t)p.B * p.P)), dim3(kBlock), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_rotate(const OpParams& p, int interp, int what, hipStream_t s) {
  const dim3 grid(p.nblocks), block(kBlock);
  if (what == 0) {
    if (interp) hipLaunchKernelGGL((k_rotate<1>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_rotate<0>), grid, block, 0, s, p);
  } else {
    if (interp) hipLaunchKernelGGL((k_rotate_grad<1>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((k_rotate_grad<0>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace tp
