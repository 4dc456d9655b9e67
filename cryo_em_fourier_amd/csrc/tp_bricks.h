// Brick-owned kernels (the adjoints): which poses' sample
// planes meet a box of sample positions, and which lattice points of a pose
// fall in it, enumerated row by row.
//
// A pose maps output frequency (kx, ky) to the sample point
// p = kx u + ky v, u = os R[0, :], v = os R[1, :].  A workgroup owns a box of
// sample positions [lo, hi) and, for the poses of its chunk, lists the lattice
// points whose sample point lies in the box.
#pragma once

#include "tp_device.h"
#include "tp_internal.h"

namespace tp {

// Sample positions [lo, hi) per axis (2D: the third axis is lo = hi = 0).
struct Box {
  double lo[3], hi[3];
};

// Everything about one pose that the brick loop needs (uniform values).
struct PoseView {
  double u[3], v[3];      // p = kx u + ky v (+ kz w for a volume lattice)
  double iu[3];           // 1 / u (0 where u = 0)
  double w[3];            // volume lattice only
  float sx, sy, sz;
  float dens;             // max(1, 1 / |u x v|) (volume: 1 / |det|): lattice points per unit area (volume)
  int kx0, kx1, ky0, ky1; // candidate rectangle, clipped to the output range
  int kz0, kz1;           // volume lattice only
  int hit;
};

__device__ __forceinline__ void pose_rows(const OpParams& p, int b, int n, int ndim, double* u, double* v) {
  const float* R = p.rot + ((size_t)(p.B_rot == 1 ? 0 : b) * p.P + n) * (ndim * ndim);
  const double os = (double)p.os;
  for (int j = 0; j < 3; ++j) {
    u[j] = j < ndim ? os * (double)R[j] : 0.0;
    v[j] = j < ndim ? os * (double)R[ndim + j] : 0.0;
  }
}

__device__ __forceinline__ bool finite3(const double* a) {
  return isfinite(a[0]) && isfinite(a[1]) && isfinite(a[2]);
}

// The pose's view of a box.  half: real outputs only (kx in [0, No/2], ky in
// [-(No/2), (No-1)/2]); otherwise the full plane, kx and ky in [-No/2, No/2].
template <int NDIM>
__device__ __forceinline__ PoseView pose_view(const OpParams& p, int b, const Box& bx, int n, bool half) {
  PoseView pv;
  pose_rows(p, b, n, NDIM, pv.u, pv.v);
  for (int j = 0; j < 3; ++j) pv.iu[j] = pv.u[j] != 0.0 ? 1.0 / pv.u[j] : 0.0;
  if (p.shift) {
    const float* s = p.shift + ((size_t)(p.B_shift == 1 ? 0 : b) * p.P + n) * 2;
    pv.sx = s[0];
    pv.sy = s[1];
  } else {
    pv.sx = pv.sy = 0.f;
  }
  const double uu = pv.u[0] * pv.u[0] + pv.u[1] * pv.u[1] + pv.u[2] * pv.u[2];
  const double vv = pv.v[0] * pv.v[0] + pv.v[1] * pv.v[1] + pv.v[2] * pv.v[2];
  const double uv = pv.u[0] * pv.v[0] + pv.u[1] * pv.v[1] + pv.u[2] * pv.v[2];
  const double D = uu * vv - uv * uv;
  const int lim = p.No / 2;
  pv.kx0 = half ? 0 : -lim;
  pv.kx1 = lim;
  pv.ky0 = -lim;
  pv.ky1 = half ? (p.No - 1) / 2 : lim;
  if (p.cut2 >= 0) {
    const int c = (int)floor(sqrt((double)p.cut2));
    pv.kx0 = max(pv.kx0, -c); pv.kx1 = min(pv.kx1, c);
    pv.ky0 = max(pv.ky0, -c); pv.ky1 = min(pv.ky1, c);
  }
  pv.hit = 1;
  pv.dens = 1e30f;
  if (D > 0.0 && isfinite(D)) {
    const double iD = 1.0 / D;  // one division; the rectangle below has a margin of 1
    pv.dens = (float)fmax(1.0, sqrt(iD));
    double ud[3], vd[3];  // dual basis: kx = p . ud, ky = p . vd for points on the plane
    for (int j = 0; j < 3; ++j) {
      ud[j] = (vv * pv.u[j] - uv * pv.v[j]) * iD;
      vd[j] = (uu * pv.v[j] - uv * pv.u[j]) * iD;
    }
    // the plane through the origin with normal u x v must cross the box
    double nrm[3] = {pv.u[1] * pv.v[2] - pv.u[2] * pv.v[1], pv.u[2] * pv.v[0] - pv.u[0] * pv.v[2],
                     pv.u[0] * pv.v[1] - pv.u[1] * pv.v[0]};
    double mn = 0.0, mx = 0.0, kmin[2] = {0.0, 0.0}, kmax[2] = {0.0, 0.0};
    for (int j = 0; j < 3; ++j) {
      const double a = bx.lo[j] * nrm[j], c = bx.hi[j] * nrm[j];
      mn += fmin(a, c);
      mx += fmax(a, c);
      const double xa = bx.lo[j] * ud[j], xb = bx.hi[j] * ud[j];
      kmin[0] += fmin(xa, xb);
      kmax[0] += fmax(xa, xb);
      const double ya = bx.lo[j] * vd[j], yb = bx.hi[j] * vd[j];
      kmin[1] += fmin(ya, yb);
      kmax[1] += fmax(ya, yb);
    }
    const double slack = 1e-9 * (fabs(mn) + fabs(mx) + 1.0);
    if (NDIM == 3 && (mn > slack || mx < -slack)) pv.hit = 0;
    if (fabs(kmin[0]) < 1e9 && fabs(kmax[0]) < 1e9 && fabs(kmin[1]) < 1e9 && fabs(kmax[1]) < 1e9) {
      pv.kx0 = max(pv.kx0, (int)floor(kmin[0]) - 1);
      pv.kx1 = min(pv.kx1, (int)ceil(kmax[0]) + 1);
      pv.ky0 = max(pv.ky0, (int)floor(kmin[1]) - 1);
      pv.ky1 = min(pv.ky1, (int)ceil(kmax[1]) + 1);
    }
  }  // degenerate rows: no dual basis; visit the whole clipped plane
  if (!finite3(pv.u) || !finite3(pv.v)) pv.hit = 0;
  if (pv.kx0 > pv.kx1 || pv.ky0 > pv.ky1) pv.hit = 0;
  // every weight is at most 1 in magnitude, so a pose adds at most its
  // rectangle's lattice count of them to a voxel: this caps the density
  // bound of nearly degenerate rows (the adjoint assumes 2.5 dens per pose,
  // and 2.5 (0.4 count + 1) exceeds the count)
  if (pv.hit) pv.dens = fminf(pv.dens, 0.4f * (float)(pv.kx1 - pv.kx0 + 1) * (float)(pv.ky1 - pv.ky0 + 1) + 1.f);
  return pv;
}

// Scan test: can pose n's sample plane bring a kept lattice point into the
// box?  The plane (through the origin, normal u x v) must cross the box, and
// the box must come within the largest |p| of a kept output (cutoff or the
// output box, times the largest stretch of the rows).
template <int NDIM>
__device__ __forceinline__ bool plane_meets(const OpParams& p, int b, const Box& bx, int n) {
  double u[3], v[3];
  pose_rows(p, b, n, NDIM, u, v);
  if (!finite3(u) || !finite3(v)) return false;
  if (NDIM == 3) {
    const double nrm[3] = {u[1] * v[2] - u[2] * v[1], u[2] * v[0] - u[0] * v[2], u[0] * v[1] - u[1] * v[0]};
    double mn = 0.0, mx = 0.0;
    for (int j = 0; j < 3; ++j) {
      const double a = bx.lo[j] * nrm[j], c = bx.hi[j] * nrm[j];
      mn += fmin(a, c);
      mx += fmax(a, c);
    }
    const double slack = 1e-9 * (fabs(mn) + fabs(mx) + 1.0);
    if (mn > slack || mx < -slack) return false;
  }
  // |p|^2 <= |k|^2 * largest eigenvalue of the rows' Gram matrix
  const double uu = u[0] * u[0] + u[1] * u[1] + u[2] * u[2];
  const double vv = v[0] * v[0] + v[1] * v[1] + v[2] * v[2];
  const double uv = u[0] * v[0] + u[1] * v[1] + u[2] * v[2];
  const double lmax = 0.5 * (uu + vv) + sqrt(0.25 * (uu - vv) * (uu - vv) + uv * uv);
  const double h = 0.5 * p.No;
  const double k2 = p.cut2 >= 0 ? fmin((double)p.cut2, 2.0 * h * h) : 2.0 * h * h;
  double d2 = 0.0;  // squared distance from the origin to the box
  for (int j = 0; j < NDIM; ++j) {
    const double d = bx.lo[j] > 0.0 ? bx.lo[j] : (bx.hi[j] < 0.0 ? -bx.hi[j] : 0.0);
    d2 += d * d;
  }
  return d2 <= k2 * lmax * (1.0 + 1e-9) + 1e-9;
}

template <int NDIM>
__device__ __forceinline__ bool in_box(const Box& bx, const double* q) {
  bool in = true;
#pragma unroll
  for (int j = 0; j < NDIM; ++j) in = in && q[j] >= bx.lo[j] && q[j] < bx.hi[j];
  return in;
}

// Clip [ta, tb] to |kx| <= floor(sqrt(rem)), rem = cut2 - (the other
// squared frequencies); empty when rem < 0.  Remainders of 2^30 or more clip
// nothing (|kx| <= 2^15).  Below that the fp32 root is within 0.01 of the
// true one, so one integer correction each way gives the floor (squares stay
// below 2^32).
__device__ __forceinline__ void clip_kx_to_disk(long long rem, double& ta, double& tb, bool& empty) {
  if (rem < 0) {
    empty = true;
  } else if (rem < (1ll << 30)) {
    const uint32_t r = (uint32_t)rem;
    uint32_t m = (uint32_t)sqrtf((float)r);
    if ((m + 1u) * (m + 1u) <= r) ++m;
    if (m * m > r) --m;
    ta = fmax(ta, -(double)m);
    tb = fmin(tb, (double)m);
  }
}

// The kx range [a, b] of row ky whose sample points fall in the box widened
// by 1e-6 (the margin covers the rounding of this fp64 arithmetic; callers
// decide membership exactly from the sample point itself), clipped to the
// pose's rectangle and to the cutoff disk.  Empty when b < a.
template <int NDIM>
__device__ __forceinline__ void row_range(const OpParams& p, const PoseView& pv, const Box& bx, int ky, int& a,
                                          int& b) {
  double ta = (double)pv.kx0, tb = (double)pv.kx1;
  bool empty = false;
#pragma unroll
  for (int j = 0; j < NDIM; ++j) {
    const double lo = bx.lo[j] - 1e-6, hi = bx.hi[j] + 1e-6;
    const double c = (double)ky * pv.v[j];
    if (pv.iu[j] == 0.0) {
      empty = empty || !(c >= lo && c < hi);
    } else {
      const double t0 = (lo - c) * pv.iu[j], t1 = (hi - c) * pv.iu[j];
      ta = fmax(ta, fmin(t0, t1));
      tb = fmin(tb, fmax(t0, t1));
    }
  }
  if (p.cut2 >= 0) clip_kx_to_disk(p.cut2 - (long long)ky * ky, ta, tb, empty);
  a = (int)ceil(ta);
  b = empty ? a - 1 : (int)floor(tb);
}

__device__ __forceinline__ size_t out_index(const OpParams& p, size_t img, int kx, int ky) {
  return (img * p.No + (ky < 0 ? ky + p.No : ky)) * p.Wo + kx;
}

// Hit-list entry: pose slot in the group (4 bits), row and column offsets in
// the pose's rectangle (14 bits each: outputs up to 16383 wide).
constexpr int kHitPoses = 16;
constexpr int kHitSpan = 1 << 14;
__device__ __forceinline__ uint32_t hit_tag(int g, int dky, int dkx) {
  return ((uint32_t)g << 28) | ((uint32_t)dky << 14) | (uint32_t)dkx;
}
__device__ __forceinline__ int hit_pose(uint32_t h) { return (int)(h >> 28); }
__device__ __forceinline__ int hit_kx(uint32_t h, const PoseView& pv) { return pv.kx0 + (int)(h & 0x3FFFu); }
__device__ __forceinline__ int hit_ky(uint32_t h, const PoseView& pv) { return pv.ky0 + (int)((h >> 14) & 0x3FFFu); }

// Workgroup scan of poses [w0, min(w0 + BS, n1)): the poses n with
// meets(n), in order, into s_poses; returns their count.  Every thread of
// the (BS-thread) workgroup calls it.
template <int BS = kBlock, typename Meets>
__device__ __forceinline__ int scan_poses_if(Meets meets, int w0, int n1, int* s_poses, int* s_wcnt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = w0 + tid;
  const bool hit = n < n1 && meets(n);
  const unsigned long long m = __ballot(hit);
  __syncthreads();
  if (lane == 0) s_wcnt[wave] = __popcll(m);
  __syncthreads();
  const int wc = lane < BS / 64 ? s_wcnt[lane] : 0;  // one read per lane, then readlane
  int off = 0, total = 0;
#pragma unroll
  for (int w = 0; w < BS / 64; ++w) {
    const int c = __builtin_amdgcn_readlane(wc, w);
    off += w < wave ? c : 0;
    total += c;
  }
  if (hit) s_poses[off + __popcll(m & ((1ull << lane) - 1ull))] = n;
  __syncthreads();
  return total;
}

// The poses whose plane meets the box.
template <int NDIM, int BS = kBlock>
__device__ __forceinline__ int scan_poses(const OpParams& p, int b, const Box& bx, int w0, int n1, int* s_poses,
                                          int* s_wcnt) {
  return scan_poses_if<BS>([&](int n) { return plane_meets<NDIM>(p, b, bx, n); }, w0, n1, s_poses, s_wcnt);
}

// Uniform sums over a group's pose views s_view[0, cnt) (cnt <= MAXG): the
// lattice density summed over the poses that hit, and cum[g], the candidate
// rows of poses 0..g.  Each lane below cnt reads one view, and the values go
// to every lane through readlane (scalar registers), so the group costs one
// LDS read per lane instead of a loop of reads of every view by every
// thread.  The density sum is taken in pose order.
template <int MAXG>
__device__ __forceinline__ void group_sums(const PoseView* s_view, int cnt, float& dens_sum, int* cum) {
  const int lane = threadIdx.x & 63;
  int H = 0;
  float d = 0.f;
  if (lane < cnt && s_view[lane].hit) {
    H = s_view[lane].ky1 - s_view[lane].ky0 + 1;
    d = s_view[lane].dens;
  }
  int run = 0;
  float ds = 0.f;
#pragma unroll
  for (int g = 0; g < MAXG; ++g) {
    run += __builtin_amdgcn_readlane(H, g);
    cum[g] = run;
    ds += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(d), g));
  }
  dens_sum = ds;
}

// List the lattice points of the poses s_view[0, cnt) (cnt <= MAXG) whose
// sample points fall in the (widened) box, row by row.  The flat index runs
// over the rows of pose 0, then pose 1, ...; entries with flat index in
// [h0, h0 + cap) go to s_hits[flat - h0].  cum: group_sums' row counts.
// Returns the total count (the same for every h0).
// Every thread of the workgroup calls it.
template <int NDIM, int MAXG, int BS = kBlock>
__device__ __forceinline__ int list_hits(const OpParams& p, const Box& bx, const PoseView* s_view, const int* cum,
                                         int h0, int cap, uint32_t* s_hits, int* s_wcnt) {
  static_assert(MAXG <= kHitPoses, "pose slot does not fit the hit tag");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rows_total = cum[MAXG - 1];
  const int h1 = h0 + cap;
  int carry = 0;
  for (int rw = 0; rw < rows_total; rw += BS) {
    const int r = rw + tid;
    int g = 0, rb = 0, cr = 0, a = 0;
#pragma unroll
    for (int i = 0; i < MAXG; ++i) {
      if (r >= cum[i]) {
        g = i + 1;
        rb = cum[i];
      }
    }
    if (r < rows_total) {
      const PoseView& pv = s_view[g];
      int b;
      row_range<NDIM>(p, pv, bx, pv.ky0 + (r - rb), a, b);
      cr = max(0, b - a + 1);
      a -= pv.kx0;
    }
    // exclusive block scan of the row counts
    int incl = cr;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (lane == 63) s_wcnt[wave] = incl;
    __syncthreads();
    const int wc = lane < BS / 64 ? s_wcnt[lane] : 0;  // one read per lane, then readlane
    int off = carry + incl - cr, tot = 0;
#pragma unroll
    for (int w = 0; w < BS / 64; ++w) {
      const int c = __builtin_amdgcn_readlane(wc, w);
      off += w < wave ? c : 0;
      tot += c;
    }
    for (int j = max(0, h0 - off); j < cr && off + j < h1; ++j) s_hits[off + j - h0] = hit_tag(g, r - rb, a + j);
    carry += tot;
    __syncthreads();
  }
  return carry;
}

}  // namespace tp
