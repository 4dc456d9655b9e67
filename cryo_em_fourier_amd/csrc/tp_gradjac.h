// Pose gradients of one (batch, pose) from a saved Jacobian and projection
// (the streaming reduction of tp_grad_pose_jac), for a workgroup of BS
// threads; shared by the standalone kernel and the fused backward.
//   dL/dR[i][j] = os sum_k k_i Re(conj(G) jac_j),
//   dL/ds_j     = (2 pi / No) sum_k k_j Im(conj(G) proj),
// over the outputs inside the cutoff, in fp64; the eight totals are added to
// the zeroed gradients with float atomics.
#pragma once

#include "tp_device.h"
#include "tp_internal.h"

namespace tp {

// red: BS / 64 x 8 doubles of LDS.  Every thread of the workgroup must call.
template <int BS>
__device__ __forceinline__ void grad_jac_pose(const OpParams& p, uint32_t bn, double (*red)[8]) {
  constexpr int NV = 8;
  const int n = (int)(bn % (uint32_t)p.P), b = (int)(bn / (uint32_t)p.P);
  const uint32_t plane = (uint32_t)p.No * (uint32_t)p.Wo;
  const float2* G = p.img + (size_t)bn * plane;
  const float2* Y = p.proj + (size_t)bn * plane;
  const float2* J = p.jac + (size_t)bn * 3 * plane;
  double acc[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) acc[i] = 0.0;
#pragma unroll 2
  for (uint32_t e = threadIdx.x; e < plane; e += BS) {
    const int iy = (int)(e / (uint32_t)p.Wo), kx = (int)(e - (uint32_t)iy * (uint32_t)p.Wo);
    const int ky = signed_row(iy, p.No);
    if (p.cut2 >= 0 && (long long)kx * kx + (long long)ky * ky > p.cut2) continue;
    const float2 g = G[e], y = Y[e], j0 = J[e], j1 = J[e + plane], j2 = J[e + 2 * plane];
    const double a0 = (double)g.x * j0.x + (double)g.y * j0.y;
    const double a1 = (double)g.x * j1.x + (double)g.y * j1.y;
    const double a2 = (double)g.x * j2.x + (double)g.y * j2.y;
    const double im = (double)g.x * y.y - (double)g.y * y.x;
    const double dx = (double)kx, dy = (double)ky;
    acc[0] = fma(dx, a0, acc[0]);
    acc[1] = fma(dx, a1, acc[1]);
    acc[2] = fma(dx, a2, acc[2]);
    acc[3] = fma(dy, a0, acc[3]);
    acc[4] = fma(dy, a1, acc[4]);
    acc[5] = fma(dy, a2, acc[5]);
    acc[6] = fma(dx, im, acc[6]);
    acc[7] = fma(dy, im, acc[7]);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const double d = wave_sum8(acc);
  if ((lane & 7) == 0) red[wave][lane >> 3] = d;
  __syncthreads();
  if (threadIdx.x < NV) {
    const int i = threadIdx.x;
    double v = 0.0;
#pragma unroll
    for (int w = 0; w < BS / 64; ++w) v += red[w][i];
    if (v == 0.0) return;
    if (i < 6) {
      if (p.grad_rot) {
        const size_t br = p.B_rot == 1 ? 0 : (size_t)b;
        unsafeAtomicAdd(p.grad_rot + ((br * p.P + n) * 3 + i / 3) * 3 + i % 3, (float)((double)p.os * v));
      }
    } else if (p.grad_shift) {
      const size_t bs = p.B_shift == 1 ? 0 : (size_t)b;
      unsafeAtomicAdd(p.grad_shift + (bs * p.P + n) * 2 + (i - 6), (float)(6.283185307179586476925 * p.inv_no * v));
    }
  }
}

// The 3D -> 3D rotation's counterpart over an [No, No, Wo] output volume
// (tp_rotate_grad_pose_jac): all three rows of dL/dR and a 3-vector shift,
// twelve sums.  red: BS / 64 x 16 doubles of LDS.
//   dL/dR[i][j] = os sum_k k_i Re(conj(G) jac_j),
//   dL/ds_j     = (2 pi / No) sum_k k_j Im(conj(G) out),
// over the outputs inside the sphere.
template <int BS>
__device__ __forceinline__ void grad_jac_vol(const OpParams& p, uint32_t bn, double (*red)[16]) {
  constexpr int NV = 12;
  const int n = (int)(bn % (uint32_t)p.P), b = (int)(bn / (uint32_t)p.P);
  const uint32_t vol = (uint32_t)p.No * (uint32_t)p.No * (uint32_t)p.Wo;
  const float2* G = p.img + (size_t)bn * vol;
  const float2* Y = p.proj + (size_t)bn * vol;
  const float2* J = p.jac + (size_t)bn * 3 * vol;
  double acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.0;
  for (uint32_t e = threadIdx.x; e < vol; e += BS) {
    const uint32_t row = e / (uint32_t)p.Wo;
    const int kx = (int)(e - row * (uint32_t)p.Wo);
    const int ky = signed_row((int)(row % (uint32_t)p.No), p.No);
    const int kz = signed_row((int)(row / (uint32_t)p.No), p.No);
    if (p.cut2 >= 0 && (long long)kx * kx + (long long)ky * ky + (long long)kz * kz > p.cut2) continue;
    const float2 g = G[e], y = Y[e], j0 = J[e], j1 = J[e + vol], j2 = J[e + 2 * vol];
    const double a[3] = {(double)g.x * j0.x + (double)g.y * j0.y, (double)g.x * j1.x + (double)g.y * j1.y,
                         (double)g.x * j2.x + (double)g.y * j2.y};
    const double im = (double)g.x * y.y - (double)g.y * y.x;
    const double k[3] = {(double)kx, (double)ky, (double)kz};
#pragma unroll
    for (int i = 0; i < 3; ++i) {
#pragma unroll
      for (int j = 0; j < 3; ++j) acc[3 * i + j] = fma(k[i], a[j], acc[3 * i + j]);
      acc[9 + i] = fma(k[i], im, acc[9 + i]);
    }
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
    for (int w = 0; w < BS / 64; ++w) v += red[w][i];
    if (v == 0.0) return;
    if (i < 9) {
      if (p.grad_rot) {
        const size_t br = p.B_rot == 1 ? 0 : (size_t)b;
        unsafeAtomicAdd(p.grad_rot + (br * p.P + n) * 9 + i, (float)((double)p.os * v));
      }
    } else if (p.grad_shift) {
      const size_t bs = p.B_shift == 1 ? 0 : (size_t)b;
      unsafeAtomicAdd(p.grad_shift + (bs * p.P + n) * 3 + (i - 9),
                      (float)(6.283185307179586476925 * p.inv_no * v));
    }
  }
}

}  // namespace tp
