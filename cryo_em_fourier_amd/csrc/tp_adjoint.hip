// Adjoint (backprojection) of the projector, brick-owned, for gfx950.
//
// The adjoint spreads every kept output c = conj(phase) G over the taps the
// forward read it from; a tap with x < 0 sends conj(w c) to -t (the forward's
// Friedel fold).  Equivalently, extend each projection to the full frequency
// plane: a real output k (kx >= 0) lands at p(k) with value c(k) on taps with
// x >= 0, its mirror -k lands at p(-k) = -p(k) with value conj(c(k)) on taps
// with x >= 1.  The kx = 0 column carries both.
//
// A workgroup owns one brick of the stored half-volume (16^3 voxels in 3D,
// 64^2 pixels in 2D) and loops over the poses whose sample plane passes
// through the brick (plus the stencil reach).  For each such pose it visits
// the plane lattice points whose stencil can touch the brick and adds their
// tap contributions to the brick in LDS.  LDS float atomics are slow on this
// part, integer ones are not: contributions are accumulated as int32 fixed
// point (exact, order independent), with a power-of-two quantum chosen per
// group of poses from a pre-scan of |G| so the sums cannot overflow, and the
// group is flushed into fp32 registers.  Bricks near the origin, which every
// pose crosses, are split over pose chunks and merged with coalesced float
// atomics; all other bricks are written with plain stores.
#include "tp_internal.h"
#include "tp_stencil.h"

namespace tp {

namespace {

constexpr int kVox = 4096;          // voxels per brick
constexpr int kPerThread = kVox / kBlock;
constexpr int kGroup = 8;           // poses per fixed-point group

template <int NDIM> struct Brick;
template <> struct Brick<3> { static constexpr int X = 16, Y = 16, Z = 16; };
template <> struct Brick<2> { static constexpr int X = 64, Y = 64, Z = 1; };

struct BrickPos {
  int b;            // batch entry
  int x0, y0, z0;   // first voxel (x from 0, y and z signed)
  int x1, y1, z1;   // last voxel (inclusive, clipped to the stored range)
  int n0, n1;       // pose range of this workgroup
  bool chunked;     // merged with atomics
  bool valid;
};

template <int NDIM>
__device__ __forceinline__ BrickPos decode(const OpParams& p, const BrickParams& bp) {
  using BR = Brick<NDIM>;
  BrickPos r;
  uint32_t g = xcd_remap(blockIdx.x, gridDim.x);
  const uint32_t per_b = bp.near_count * bp.chunks + bp.nbricks;
  r.b = (int)(g / per_b);
  g %= per_b;
  int bi, bj, bk;
  if (g < (uint32_t)(bp.near_count * bp.chunks)) {
    const int nb = (int)(g / bp.chunks), ch = (int)(g % bp.chunks);
    bi = bp.near_lo[0] + nb % bp.near_ext[0];
    bj = bp.near_lo[1] + (nb / bp.near_ext[0]) % bp.near_ext[1];
    bk = bp.near_lo[2] + nb / (bp.near_ext[0] * bp.near_ext[1]);
    r.n0 = (int)((long long)p.P * ch / bp.chunks);
    r.n1 = (int)((long long)p.P * (ch + 1) / bp.chunks);
    r.chunked = true;
    r.valid = true;
  } else {
    const int f = (int)(g - bp.near_count * bp.chunks);
    bi = f % bp.nb[0];
    bj = (f / bp.nb[0]) % bp.nb[1];
    bk = f / (bp.nb[0] * bp.nb[1]);
    const bool near = bi >= bp.near_lo[0] && bi < bp.near_lo[0] + bp.near_ext[0] &&
                      bj >= bp.near_lo[1] && bj < bp.near_lo[1] + bp.near_ext[1] &&
                      bk >= bp.near_lo[2] && bk < bp.near_lo[2] + bp.near_ext[2];
    r.valid = !near;
    r.n0 = 0;
    r.n1 = p.P;
    r.chunked = false;
  }
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
  return r;
}

// Everything about one pose that the brick loop needs (uniform values).
struct PoseView {
  double u[3], v[3];      // p = kx u + ky v
  double ud[3], vd[3];    // dual basis: kx = p . ud, ky = p . vd (points on the plane)
  float sx, sy;
  double cell;            // |u x v| (area of the lattice cell), 0 if degenerate
  int kx0, kx1, ky0, ky1; // candidate rectangle (full plane, clipped)
  bool hit;
};

template <int NDIM, int INTERP>
__device__ __forceinline__ PoseView pose_view(const OpParams& p, const BrickPos& br, int n) {
  PoseView pv;
  const float* R = p.rot + ((size_t)(p.B_rot == 1 ? 0 : br.b) * p.P + n) * (NDIM * NDIM);
  const double os = (double)p.os;
  for (int j = 0; j < 3; ++j) {
    pv.u[j] = j < NDIM ? os * (double)R[j] : 0.0;
    pv.v[j] = j < NDIM ? os * (double)R[NDIM + j] : 0.0;
  }
  if (p.shift) {
    const float* s = p.shift + ((size_t)(p.B_shift == 1 ? 0 : br.b) * p.P + n) * 2;
    pv.sx = s[0];
    pv.sy = s[1];
  } else {
    pv.sx = pv.sy = 0.f;
  }
  // box of sample positions whose stencil reaches the brick: p_j in [t0-R, t1+R)
  constexpr double reach = INTERP ? 2.0 : 1.0;
  double lo[3] = {br.x0 - reach, br.y0 - reach, br.z0 - reach};
  double hi[3] = {br.x1 + reach, br.y1 + reach, br.z1 + reach};
  if (NDIM == 2) { lo[2] = 0.0; hi[2] = 0.0; }
  const double uu = pv.u[0] * pv.u[0] + pv.u[1] * pv.u[1] + pv.u[2] * pv.u[2];
  const double vv = pv.v[0] * pv.v[0] + pv.v[1] * pv.v[1] + pv.v[2] * pv.v[2];
  const double uv = pv.u[0] * pv.v[0] + pv.u[1] * pv.v[1] + pv.u[2] * pv.v[2];
  const double D = uu * vv - uv * uv;
  const int kxlim = p.No / 2, kylim = p.No / 2;
  pv.kx0 = -kxlim; pv.kx1 = kxlim; pv.ky0 = -kylim; pv.ky1 = kylim;
  if (p.cut2 >= 0) {
    const int c = (int)floor(sqrt((double)p.cut2));
    pv.kx0 = max(pv.kx0, -c); pv.kx1 = min(pv.kx1, c);
    pv.ky0 = max(pv.ky0, -c); pv.ky1 = min(pv.ky1, c);
  }
  pv.hit = true;
  pv.cell = 0.0;
  if (D > 0.0 && isfinite(D)) {
    pv.cell = sqrt(D);
    for (int j = 0; j < 3; ++j) {
      pv.ud[j] = (vv * pv.u[j] - uv * pv.v[j]) / D;
      pv.vd[j] = (uu * pv.v[j] - uv * pv.u[j]) / D;
    }
    // plane through the origin with normal u x v must cross the box
    double nrm[3] = {pv.u[1] * pv.v[2] - pv.u[2] * pv.v[1], pv.u[2] * pv.v[0] - pv.u[0] * pv.v[2],
                     pv.u[0] * pv.v[1] - pv.u[1] * pv.v[0]};
    double mn = 0.0, mx = 0.0, kmin[2] = {0.0, 0.0}, kmax[2] = {0.0, 0.0};
    for (int j = 0; j < 3; ++j) {
      const double a = lo[j] * nrm[j], b = hi[j] * nrm[j];
      mn += fmin(a, b);
      mx += fmax(a, b);
      const double xa = lo[j] * pv.ud[j], xb = hi[j] * pv.ud[j];
      kmin[0] += fmin(xa, xb);
      kmax[0] += fmax(xa, xb);
      const double ya = lo[j] * pv.vd[j], yb = hi[j] * pv.vd[j];
      kmin[1] += fmin(ya, yb);
      kmax[1] += fmax(ya, yb);
    }
    const double slack = 1e-9 * (fabs(mn) + fabs(mx) + 1.0);
    if (NDIM == 3 && (mn > slack || mx < -slack)) pv.hit = false;
    if (fabs(kmin[0]) < 1e9 && fabs(kmax[0]) < 1e9 && fabs(kmin[1]) < 1e9 && fabs(kmax[1]) < 1e9) {
      pv.kx0 = max(pv.kx0, (int)floor(kmin[0]) - 1);
      pv.kx1 = min(pv.kx1, (int)ceil(kmax[0]) + 1);
      pv.ky0 = max(pv.ky0, (int)floor(kmin[1]) - 1);
      pv.ky1 = min(pv.ky1, (int)ceil(kmax[1]) + 1);
    }
  } else {
    // degenerate rows: no dual basis; visit the whole clipped plane
    for (int j = 0; j < 3; ++j) pv.ud[j] = pv.vd[j] = 0.0;
  }
  if (!(isfinite(pv.u[0]) && isfinite(pv.u[1]) && isfinite(pv.u[2]) && isfinite(pv.v[0]) &&
        isfinite(pv.v[1]) && isfinite(pv.v[2])))
    pv.hit = false;
  if (pv.kx0 > pv.kx1 || pv.ky0 > pv.ky1) pv.hit = false;
  return pv;
}

// One lattice point of the full plane: its sample point and the values it
// spreads (real part on x >= 0, real + mirror on x >= 1).  false if it
// carries nothing or its stencil misses the brick.
struct Cand {
  double q[3];
  float2 v0;   // value for taps at x = 0
  float2 v1;   // value for taps at x >= 1
};

template <int NDIM, int INTERP>
__device__ __forceinline__ bool candidate(const OpParams& p, const BrickPos& br, const PoseView& pv,
                                          int n, int kx, int ky, bool want_values, Cand& cd,
                                          float& amax) {
  if (p.cut2 >= 0 && (long long)kx * kx + (long long)ky * ky > p.cut2) return false;
  const int rlo = -(p.No / 2), rhi = (p.No - 1) / 2;
  const bool real = kx >= 0 && kx <= p.No / 2 && ky >= rlo && ky <= rhi;
  const bool mirr = kx <= 0 && -kx <= p.No / 2 && -ky >= rlo && -ky <= rhi;
  if (!real && !mirr) return false;
  constexpr double reach = INTERP ? 2.0 : 1.0;
  const double lo[3] = {br.x0 - reach, br.y0 - reach, br.z0 - reach};
  const double hi[3] = {br.x1 + reach, br.y1 + reach, br.z1 + reach};
  bool in = true;
#pragma unroll
  for (int j = 0; j < NDIM; ++j) {
    cd.q[j] = (double)kx * pv.u[j] + (double)ky * pv.v[j];
    in = in && cd.q[j] >= lo[j] && cd.q[j] < hi[j];
  }
  if (!in) return false;
  const size_t img = (size_t)br.b * p.P + n;
  float2 gr = make_float2(0.f, 0.f), gm = gr;
  if (real) gr = p.img[(img * p.No + (ky < 0 ? ky + p.No : ky)) * p.Wo + kx];
  if (mirr) gm = p.img[(img * p.No + (-ky < 0 ? -ky + p.No : -ky)) * p.Wo + (-kx)];
  amax = fmaxf(amax, fmaxf(fabsf(gr.x) + fabsf(gr.y), fabsf(gm.x) + fabsf(gm.y)));
  if (!want_values) return true;
  float2 cr = gr, cm = gm;
  if (p.shift) {
    if (real) cr = cmul(conjf2(shift_phase(kx, ky, pv.sx, pv.sy, p.inv_no)), gr);
    if (mirr) cm = cmul(conjf2(shift_phase(-kx, -ky, pv.sx, pv.sy, p.inv_no)), gm);
  }
  cd.v0 = cr;                                                      // real only
  cd.v1 = make_float2(cr.x + cm.x, cr.y - cm.y);                   // real + conj(mirror)
  return true;
}

template <int NDIM, int INTERP>
__global__ __launch_bounds__(kBlock) void k_adjoint_bricks(OpParams p, BrickParams bp) {
  using BR = Brick<NDIM>;
  using K = Kern<INTERP>;
  constexpr int T = K::T;
  __shared__ int acc[2][kVox];
  __shared__ int s_poses[kBlock];
  __shared__ PoseView s_view[kGroup];
  __shared__ int s_wcnt[kBlock / 64];
  __shared__ float s_red[kBlock / 64];

  const BrickPos br = decode<NDIM>(p, bp);
  if (!br.valid) return;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float fre[kPerThread], fim[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    fre[i] = fim[i] = 0.f;
    acc[0][tid + i * kBlock] = 0;
    acc[1][tid + i * kBlock] = 0;
  }
  const int lx = tid % 16, ly = tid / 16;  // 16x16 thread grid over candidate rectangles

  for (int w0 = br.n0; w0 < br.n1; w0 += kBlock) {
    // one pose per thread: does its plane reach this brick?  ordered compaction
    const int n = w0 + tid;
    const bool hit = n < br.n1 && pose_view<NDIM, INTERP>(p, br, n).hit;
    const unsigned long long m = __ballot(hit);
    __syncthreads();
    if (lane == 0) s_wcnt[wave] = __popcll(m);
    __syncthreads();
    int off = 0, total = 0;
#pragma unroll
    for (int w = 0; w < kBlock / 64; ++w) {
      off += w < wave ? s_wcnt[w] : 0;
      total += s_wcnt[w];
    }
    if (hit) s_poses[off + __popcll(m & ((1ull << lane) - 1ull))] = n;
    __syncthreads();

    for (int g0 = 0; g0 < total; g0 += kGroup) {
      const int cnt = min(kGroup, total - g0);
      if (tid < cnt) s_view[tid] = pose_view<NDIM, INTERP>(p, br, s_poses[g0 + tid]);
      __syncthreads();

      // pre-scan: bound on the group's contributions -> fixed-point quantum.
      // Per pose and voxel, sum |w| over the lattice <= 4 / cell and every
      // value is <= 2 max|G|.
      float amax = 0.f;
      double dens_sum = 0.0;
      for (int g = 0; g < cnt; ++g) {
        const PoseView& pv = s_view[g];
        const int pn = s_poses[g0 + g];
        dens_sum += 8.0 * (pv.cell > 0.0 ? fmax(1.0, 1.0 / pv.cell) : 1e30);
        for (int ky = pv.ky0 + ly; ky <= pv.ky1; ky += 16)
          for (int kx = pv.kx0 + lx; kx <= pv.kx1; kx += 16) {
            Cand cd;
            candidate<NDIM, INTERP>(p, br, pv, pn, kx, ky, false, cd, amax);
          }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
      if (lane == 0) s_red[wave] = amax;
      __syncthreads();
      float gmax = s_red[0];
#pragma unroll
      for (int w = 1; w < kBlock / 64; ++w) gmax = fmaxf(gmax, s_red[w]);
      const float gb = (float)fmin(dens_sum * (double)gmax, 1e30);
      if (gb > 0.f) {
        // quantum q = 2^e with |sum| <= gb / q < 2^29
        int e;
        frexpf(gb, &e);  // gb < 2^e
        const float inv_q = ldexpf(1.f, 29 - e);
        const float q = ldexpf(1.f, e - 29);

        for (int g = 0; g < cnt; ++g) {
          const PoseView& pv = s_view[g];
          const int pn = s_poses[g0 + g];
          for (int ky = pv.ky0 + ly; ky <= pv.ky1; ky += 16)
            for (int kx = pv.kx0 + lx; kx <= pv.kx1; kx += 16) {
              Cand cd;
              float dummy = 0.f;
              if (!candidate<NDIM, INTERP>(p, br, pv, pn, kx, ky, true, cd, dummy)) continue;
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
                const int tx = ax.x0 + d;
                const float2 v = tx >= 1 ? cd.v1 : cd.v0;
                const bool inx = tx >= br.x0 && tx <= br.x1;
                are[d] = inx ? wx[d] * v.x * inv_q : 0.f;
                aim[d] = inx ? wx[d] * v.y * inv_q : 0.f;
              }
#pragma unroll
              for (int dz = 0; dz < (NDIM == 3 ? T : 1); ++dz) {
                const int tz = z0 + dz;
                if (NDIM == 3 && (tz < br.z0 || tz > br.z1)) continue;
#pragma unroll
                for (int dy = 0; dy < T; ++dy) {
                  const int ty = ay.x0 + dy;
                  if (ty < br.y0 || ty > br.y1) continue;
                  const float wyz = wy[dy] * wz[dz];
                  const int base = (((NDIM == 3 ? tz - br.z0 : 0) * BR::Y) + (ty - br.y0)) * BR::X +
                                   (ax.x0 - br.x0);
#pragma unroll
                  for (int dx = 0; dx < T; ++dx) {
                    const int ir = (int)rintf(are[dx] * wyz), ii = (int)rintf(aim[dx] * wyz);
                    if ((ir | ii) != 0) {
                      atomicAdd(&acc[0][base + dx], ir);
                      atomicAdd(&acc[1][base + dx], ii);
                    }
                  }
                }
              }
            }
        }
        // flush the group into fp32 registers
        __syncthreads();
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
          const int v = tid + i * kBlock;
          fre[i] = fmaf((float)acc[0][v], q, fre[i]);
          fim[i] = fmaf((float)acc[1][v], q, fim[i]);
          acc[0][v] = 0;
          acc[1][v] = 0;
        }
      }
      __syncthreads();
    }
  }

  // write the brick: plain stores, or float atomics for pose-chunked bricks
  float2* out = p.ref_out + (size_t)br.b * p.ref_elems;
  const int wh = p.N / 2 + 1;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int v = tid + i * kBlock;
    const int x = br.x0 + v % BR::X;
    const int y = br.y0 + (v / BR::X) % BR::Y;
    const int z = br.z0 + v / (BR::X * BR::Y);
    if (x > br.x1 || y > br.y1 || (NDIM == 3 && z > br.z1)) continue;
    const size_t row = NDIM == 3 ? (size_t)(z < 0 ? z + p.N : z) * p.N + (y < 0 ? y + p.N : y)
                                 : (size_t)(y < 0 ? y + p.N : y);
    float2* dst = out + row * wh + x;
    if (br.chunked) {
      if (fre[i] != 0.f) unsafeAtomicAdd(&dst->x, fre[i]);
      if (fim[i] != 0.f) unsafeAtomicAdd(&dst->y, fim[i]);
    } else {
      *dst = make_float2(fre[i], fim[i]);
    }
  }
}

}  // namespace

template <int NDIM>
static BrickParams brick_params(const OpParams& p) {
  using BR = Brick<NDIM>;
  BrickParams bp{};
  const int lo = -(p.N / 2);
  bp.nb[0] = (p.N / 2 + 1 + BR::X - 1) / BR::X;
  bp.nb[1] = (p.N + BR::Y - 1) / BR::Y;
  bp.nb[2] = NDIM == 3 ? (p.N + BR::Z - 1) / BR::Z : 1;
  bp.nbricks = bp.nb[0] * bp.nb[1] * bp.nb[2];
  // bricks next to the origin are crossed by every pose: split their poses
  const int jo = (0 - lo) / BR::Y;  // brick holding y = 0
  int nlo[3] = {0, jo - 2, NDIM == 3 ? jo - 2 : 0};
  int nhi[3] = {2, jo + 2, NDIM == 3 ? jo + 2 : 1};
  if (NDIM == 2) { nhi[0] = 1; nlo[1] = jo - 1; nhi[1] = jo + 1; }
  bp.near_count = 1;
  for (int j = 0; j < 3; ++j) {
    nlo[j] = nlo[j] < 0 ? 0 : nlo[j];
    nhi[j] = nhi[j] > bp.nb[j] ? bp.nb[j] : nhi[j];
    bp.near_lo[j] = nlo[j];
    bp.near_ext[j] = nhi[j] > nlo[j] ? nhi[j] - nlo[j] : 0;
    bp.near_count *= bp.near_ext[j];
  }
  int chunks = (p.P + 255) / 256;  // about 256 poses per chunk
  bp.chunks = chunks < 1 ? 1 : (chunks > 32 ? 32 : chunks);
  if (bp.chunks == 1 || bp.near_count == 0) {  // nothing to split
    bp.chunks = 1;
    bp.near_count = 0;
    for (int j = 0; j < 3; ++j) bp.near_ext[j] = 0;
  }
  return bp;
}

uint64_t adjoint_blocks(const OpParams& p) {
  const BrickParams bp = p.ndim == 3 ? brick_params<3>(p) : brick_params<2>(p);
  return (uint64_t)p.B * ((uint64_t)bp.near_count * bp.chunks + bp.nbricks);
}

hipError_t launch_backproject(const OpParams& p, int interp, hipStream_t s) {
  const BrickParams bp = p.ndim == 3 ? brick_params<3>(p) : brick_params<2>(p);
  const dim3 grid((unsigned)adjoint_blocks(p)), block(kBlock);
  if (p.ndim == 3) {
    if (interp) hipLaunchKernelGGL((k_adjoint_bricks<3, 1>), grid, block, 0, s, p, bp);
    else hipLaunchKernelGGL((k_adjoint_bricks<3, 0>), grid, block, 0, s, p, bp);
  } else {
    if (interp) hipLaunchKernelGGL((k_adjoint_bricks<2, 1>), grid, block, 0, s, p, bp);
    else hipLaunchKernelGGL((k_adjoint_bricks<2, 0>), grid, block, 0, s, p, bp);
  }
  return hipGetLastError();
}

}  // namespace tp
