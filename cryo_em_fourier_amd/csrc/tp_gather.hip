// Brick gather for gfx950: the 3D pose gradients with the reference staged
// in LDS.
//
// A workgroup owns the sample points whose floor lies in a 16^3 core of
// sample space (x of both signs) and loads into LDS every reference value a
// stencil of those points can read: the core plus the stencil's halo, with
// the Friedel fold applied while loading (a tap with x < 0 holds conj V[-t],
// a tap outside the stored range holds 0).  For the poses of its chunk it
// lists the real outputs whose sample point lies in the core (the lattice
// enumeration shared with the adjoint) and evaluates value and gradient
// stencils from LDS.  Each output is owned by exactly one workgroup, the one
// whose core holds floor(p), and p is computed by the same code everywhere,
// so every output is counted once.
//
// Gathering from LDS avoids the vector L1's per-cache-line cost of scattered
// 64-tap stencils, but pays for the tile loads and the enumeration per (pose,
// brick).  It wins where many poses cross a brick and the lattice is dense
// (measured: box 320 cubic at oversampling 1; the per-output kernel wins at
// box 256 and 128 and at oversampling 2), and the host picks it only there.
#include "tp_bricks.h"
#include "tp_internal.h"

namespace tp {

namespace {


// owned floor values per axis (x, y, z)
constexpr int kCX = 16, kCY = 16, kCZ = 16;
constexpr int kWaveHits = 512; // hit-list entries per wave

template <int INTERP>
struct GTile {
  static constexpr int T = Kern<INTERP>::T;
  static constexpr int OFF = Kern<INTERP>::OFF;  // first tap = floor + OFF
  static constexpr int SX = kCX + T - 1, SY = kCY + T - 1, SZ = kCZ + T - 1;  // tile sides
  static constexpr int VOX = SX * SY * SZ;
};

// floor(p) values that can read a stored tap, per axis: taps reach
// [-(N/2), N/2] (x < 0 through the fold), so floor lies in
// [-(N/2) - OFF - T + 1, N/2 - OFF].
template <int INTERP>
__host__ __device__ inline int floor_lo(int N) {
  return -(N / 2) - GTile<INTERP>::OFF - GTile<INTERP>::T + 1;
}
template <int INTERP>
__host__ __device__ inline int bricks_per_axis(int N, int core) {
  return (2 * (N / 2) + GTile<INTERP>::T + core - 1) / core;
}

struct GBrick {
  int b;
  int c0[3];     // first owned floor value per axis (x, y, z)
  int n0, n1;    // pose range of this workgroup
  bool valid;
};

template <int INTERP>
__device__ __forceinline__ GBrick gdecode(const OpParams& p, const BrickParams& bp) {
  GBrick r;
  // busiest chunk slots first (see the adjoint's decode)
  const uint32_t lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const int brick = (int)(lin % (uint32_t)bp.nbricks);
  const int ch = bp.cmax - 1 - (int)((lin / (uint32_t)bp.nbricks) % (uint32_t)bp.cmax);
  r.b = (int)(lin / ((uint32_t)bp.nbricks * (uint32_t)bp.cmax));
  const int lo = floor_lo<INTERP>(p.N);
  r.c0[0] = lo + kCX * (brick % bp.nb[0]);
  r.c0[1] = lo + kCY * ((brick / bp.nb[0]) % bp.nb[1]);
  r.c0[2] = lo + kCZ * (brick / (bp.nb[0] * bp.nb[1]));
  // pose chunks as in the adjoint: a random plane through the origin meets a
  // ball of radius rho at distance r with probability about rho / r
  const double cx = r.c0[0] + 0.5 * kCX, cy = r.c0[1] + 0.5 * kCY, cz = r.c0[2] + 0.5 * kCZ;
  const double rho = 0.5 * sqrt((double)(kCX * kCX + kCY * kCY + kCZ * kCZ)), rr = sqrt(cx * cx + cy * cy + cz * cz);
  const double frac = rr > rho ? rho / rr : 1.0;
  const int nch = (int)fmin(fmax(ceil((double)p.P * frac / (double)bp.pmax), 1.0), (double)bp.cmax);
  r.valid = ch < nch;
  r.n0 = (int)((long long)p.P * ch / nch);
  r.n1 = (int)((long long)p.P * (ch + 1) / nch);
  return r;
}

// Reference values of the tile, Friedel fold applied.  Loads are issued in
// batches of kTileBatch per thread before their LDS stores, so their latency
// overlaps.
constexpr int kTileBatch = 8;

template <int INTERP>
__device__ __forceinline__ void load_tile(const OpParams& p, const GBrick& br, float2* tile) {
  using TL = GTile<INTERP>;
  constexpr int SX = TL::SX, SY = TL::SY;
  const int N = p.N, hx = N / 2, ylo = -(N / 2), yhi = (N + 1) / 2 - 1, wh = N / 2 + 1;
  const float2* V = p.ref + (size_t)br.b * p.ref_elems;
  for (int i0 = threadIdx.x; i0 < TL::VOX; i0 += kTileBatch * kBlock) {
    float2 v[kTileBatch];
#pragma unroll
    for (int k = 0; k < kTileBatch; ++k) {
      const int i = i0 + k * kBlock;
      const int tx = br.c0[0] + TL::OFF + i % SX;
      const int ty = br.c0[1] + TL::OFF + (i / SX) % SY;
      const int tz = br.c0[2] + TL::OFF + i / (SX * SY);
      const bool fold = tx < 0;
      const int mx = fold ? -tx : tx, my = fold ? -ty : ty, mz = fold ? -tz : tz;
      v[k] = make_float2(0.f, 0.f);
      if (i < TL::VOX && mx <= hx && my >= ylo && my <= yhi && mz >= ylo && mz <= yhi) {
        v[k] = V[((size_t)(mz < 0 ? mz + N : mz) * N + (my < 0 ? my + N : my)) * wh + mx];
        if (fold) v[k].y = -v[k].y;
      }
    }
#pragma unroll
    for (int k = 0; k < kTileBatch; ++k)
      if (i0 + k * kBlock < TL::VOX) tile[i0 + k * kBlock] = v[k];
  }
}

// Owned sample point of a listed lattice point: floor(p) in the core.
struct GPoint {
  int l[3];     // floor(p) - core origin, in [0, core size)
  float f[3];   // fractions
  bool owned;
};

// p = kx u + ky v with u = os R[0, :], v = os R[1, :] in fp64: the same
// arithmetic in every workgroup, so exactly one owns each output.
__device__ __forceinline__ GPoint own_point(const GBrick& br, const float* r0, const float* r1, double os, int kx,
                                            int ky) {
  GPoint g;
  g.owned = true;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const double q = (double)kx * (os * (double)r0[j]) + (double)ky * (os * (double)r1[j]);
    const double fl = floor(q);
    const double l = fl - (double)br.c0[j];
    const int ext = j == 0 ? kCX : (j == 1 ? kCY : kCZ);
    g.owned = g.owned && l >= 0.0 && l < (double)ext;
    g.l[j] = g.owned ? (int)l : 0;
    g.f[j] = (float)(q - fl);
  }
  return g;
}

// `after` only orders the reads after the value's computation (keeping the
// phase's temporaries and the 64 reads from being live together).
template <int INTERP>
__device__ __forceinline__ void gather_grad(const float2* tile, const GPoint& g, float after, float2& S, float2* dS) {
  using K = Kern<INTERP>;
  using TL = GTile<INTERP>;
  constexpr int T = K::T, SX = TL::SX, SY = TL::SY;
  float wx[T], wy[T], wz[T], dx[T], dy[T], dz[T];
  K::w(g.f[0], wx);
  K::w(g.f[1], wy);
  K::w(g.f[2], wz);
  K::dw(g.f[0], dx);
  K::dw(g.f[1], dy);
  K::dw(g.f[2], dz);
  S = make_float2(0.f, 0.f);
  float2 sx = S, sy = S, sz = S;
  int base = (g.l[2] * SY + g.l[1]) * SX + g.l[0];
  asm volatile("" : "+v"(base) : "v"(after));
#pragma unroll
  for (int iz = 0; iz < T; ++iz) {
    float2 py = make_float2(0.f, 0.f), pdx = py, pdy = py;
    if (iz > 0) {
      // the next plane's address formally depends on this point's sums so
      // far: its 16 reads cannot be hoisted above the previous plane's
      // arithmetic (all 64 in flight would take 128 VGPRs)
      asm volatile("" : "+v"(base) : "v"(S.x));
    }
#pragma unroll
    for (int iy = 0; iy < T; ++iy) {
      const float2* r = tile + base + (iz * SY + iy) * SX;
      float2 rx = make_float2(0.f, 0.f), rdx = rx;
#pragma unroll
      for (int ix = 0; ix < T; ++ix) {
        const float2 v = r[ix];
        rx.x = fmaf(wx[ix], v.x, rx.x);
        rx.y = fmaf(wx[ix], v.y, rx.y);
        rdx.x = fmaf(dx[ix], v.x, rdx.x);
        rdx.y = fmaf(dx[ix], v.y, rdx.y);
      }
      py.x = fmaf(wy[iy], rx.x, py.x);
      py.y = fmaf(wy[iy], rx.y, py.y);
      pdx.x = fmaf(wy[iy], rdx.x, pdx.x);
      pdx.y = fmaf(wy[iy], rdx.y, pdx.y);
      pdy.x = fmaf(dy[iy], rx.x, pdy.x);
      pdy.y = fmaf(dy[iy], rx.y, pdy.y);
    }
    S.x = fmaf(wz[iz], py.x, S.x);
    S.y = fmaf(wz[iz], py.y, S.y);
    sx.x = fmaf(wz[iz], pdx.x, sx.x);
    sx.y = fmaf(wz[iz], pdx.y, sx.y);
    sy.x = fmaf(wz[iz], pdy.x, sy.x);
    sy.y = fmaf(wz[iz], pdy.y, sy.y);
    sz.x = fmaf(dz[iz], py.x, sz.x);
    sz.y = fmaf(dz[iz], py.y, sz.y);
  }
  dS[0] = sx;
  dS[1] = sy;
  dS[2] = sz;
}

// A listed pose as the waves see it (LDS): rotation rows, the candidate
// rectangle packed as 16-bit pairs (empty: the pose misses), the shift.
struct CView {
  float r0[3], r1[3];
  int kx01, ky01;
  float sx, sy;
};

__device__ __forceinline__ CView compact_view(const OpParams& p, int b, const Box& bx, int n) {
  const PoseView pv = pose_view<3>(p, b, bx, n, true);
  CView c;
  const float* R = p.rot + ((size_t)(p.B_rot == 1 ? 0 : b) * p.P + n) * 9;
  for (int j = 0; j < 3; ++j) {
    c.r0[j] = R[j];
    c.r1[j] = R[3 + j];
  }
  const bool hit = pv.hit != 0;
  c.kx01 = (int)((uint32_t)(pv.kx0 & 0xFFFF) | ((uint32_t)(hit ? pv.kx1 : pv.kx0 - 1) << 16));
  c.ky01 = (int)((uint32_t)(pv.ky0 & 0xFFFF) | ((uint32_t)(hit ? pv.ky1 : pv.ky0 - 1) << 16));
  c.sx = pv.sx;
  c.sy = pv.sy;
  return c;
}

__device__ __forceinline__ int lo16(int v) { return (int)(short)(v & 0xFFFF); }
__device__ __forceinline__ int hi16(int v) { return v >> 16; }

// Row ky's kx range [a, b] whose sample points fall in the box, in fp32 with
// margins that cover its rounding (a superset: ownership is decided exactly
// by own_point), clipped to [kx0, kx1] and to the cutoff disk.
__device__ __forceinline__ void row_range_f(const OpParams& p, const float* u, const float* v, const Box& bx,
                                            int kx0, int kx1, int ky, int& a, int& b) {
  float ta = (float)kx0, tb = (float)kx1;
  bool empty = false;
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const float c = (float)ky * v[j];
    const float lo0 = (float)bx.lo[j], hi0 = (float)bx.hi[j];
    const float m = 0.05f + 3e-7f * (fabsf(c) + fabsf(lo0) + fabsf(hi0));
    const float lo = lo0 - m, hi = hi0 + m;
    if (u[j] == 0.f) {
      empty = empty || !(c >= lo && c < hi);
    } else {
      const float iu = 1.f / u[j];
      const float t0 = (lo - c) * iu, t1 = (hi - c) * iu;
      ta = fmaxf(ta, fminf(t0, t1));
      tb = fminf(tb, fmaxf(t0, t1));
    }
  }
  // relative rounding of the kx bounds themselves
  ta -= 1e-3f + 1e-6f * fabsf(ta);
  tb += 1e-3f + 1e-6f * fabsf(tb);
  if (p.cut2 >= 0) {
    const long long rem = p.cut2 - (long long)ky * ky;
    if (rem < 0) {
      empty = true;
    } else {
      long long mm = (long long)sqrtf((float)rem);
      while ((mm + 1) * (mm + 1) <= rem) ++mm;
      while (mm * mm > rem) --mm;
      ta = fmaxf(ta, (float)-mm);
      tb = fminf(tb, (float)mm);
    }
  }
  a = (int)ceilf(ta);
  b = empty ? a - 1 : (int)floorf(tb);
}

// Wave-private hit list entry: output column kx (13 bits) and row ky + 8192
// (14 bits); outputs up to 16383 wide.
__device__ __forceinline__ uint32_t whit(int kx, int ky) { return ((uint32_t)(ky + 8192) << 13) | (uint32_t)kx; }
__device__ __forceinline__ int whit_kx(uint32_t h) { return (int)(h & 0x1FFFu); }
__device__ __forceinline__ int whit_ky(uint32_t h) { return (int)(h >> 13) - 8192; }

// Per pose, dL/dR rows 0-1 and dL/ds summed over the owned outputs, merged
// with float atomics.
//
// After the workgroup's pose scan every listed pose gets a compact view in
// LDS; waves then take poses one at a time from a shared counter.  A pose's
// rows go one per lane, their kx ranges are expanded into the wave's own
// slice of the hit list, and the hits are evaluated 64 at a time.
template <int INTERP>
__global__ __launch_bounds__(kBlock) __attribute__((amdgpu_waves_per_eu(2))) void k_grad_bricks(OpParams p,
                                                                                          BrickParams bp) {
  using TL = GTile<INTERP>;
  constexpr int NW = kBlock / 64;
  __shared__ float2 tile[TL::VOX];
  __shared__ uint32_t s_hit[NW][kWaveHits];
  __shared__ int s_poses[kBlock];
  __shared__ CView s_cv[kBlock];
  __shared__ int s_wcnt[NW];
  __shared__ int s_next;

  const GBrick br = gdecode<INTERP>(p, bp);
  if (!br.valid) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t* hits = s_hit[wave];
  const double os = (double)p.os;
  const Box bx = {{(double)br.c0[0], (double)br.c0[1], (double)br.c0[2]},
                  {(double)(br.c0[0] + kCX), (double)(br.c0[1] + kCY), (double)(br.c0[2] + kCZ)}};
  bool loaded = false;
  for (int w0 = br.n0; w0 < br.n1; w0 += kBlock) {
    const int total = scan_poses<3>(p, br.b, bx, w0, br.n1, s_poses, s_wcnt);
    if (total == 0) continue;
    if (!loaded) {
      load_tile<INTERP>(p, br, tile);
      loaded = true;
    }
    if (tid < total) s_cv[tid] = compact_view(p, br.b, bx, s_poses[tid]);
    if (tid == 0) s_next = 0;
    __syncthreads();
    while (true) {
      int slot = 0;
      if (lane == 0) slot = atomicAdd(&s_next, 1);
      slot = __builtin_amdgcn_readfirstlane(__shfl(slot, 0, 64));
      if (slot >= total) break;
      const CView& cv = s_cv[slot];
      float r0[3], r1[3], u[3], v[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        r0[j] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, cv.r0[j])));
        r1[j] = __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, cv.r1[j])));
        u[j] = p.os * r0[j];
        v[j] = p.os * r1[j];
      }
      const int kx01 = __builtin_amdgcn_readfirstlane(cv.kx01), ky01 = __builtin_amdgcn_readfirstlane(cv.ky01);
      const float sx = cv.sx, sy = cv.sy;
      const int kx0 = lo16(kx01), kx1 = hi16(kx01), ky0 = lo16(ky01), ky1 = hi16(ky01);
      if (ky1 < ky0 || kx1 < kx0) continue;
      const int n = s_poses[slot];
      const size_t img = (size_t)br.b * p.P + n;
      float acc[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = 0.f;
      const int rows = ky1 - ky0 + 1;
      for (int rr = 0; rr < rows; rr += 64) {
        // one row per lane: its kx range, then the wave's exclusive prefix
        const int ky = ky0 + rr + lane;
        int a = 0, c = 0;
        if (rr + lane < rows) {
          int b;
          row_range_f(p, u, v, bx, kx0, kx1, ky, a, b);
          c = max(0, b - a + 1);
        }
        int incl = c;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int t = __shfl_up(incl, o, 64);
          if (lane >= o) incl += t;
        }
        const int excl = incl - c;
        const int wtot = __builtin_amdgcn_readlane(incl, 63);
        for (int h0 = 0; h0 < wtot; h0 += kWaveHits) {
#pragma unroll 1
          for (int j = max(0, h0 - excl); j < c && excl + j < h0 + kWaveHits; ++j)
            hits[excl + j - h0] = whit(a + j, ky);
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          const int nh = min(kWaveHits, wtot - h0);
#pragma unroll 1
          for (int i0 = 0; i0 < nh; i0 += 64) {
            const int i = i0 + lane;
            if (i >= nh) continue;
            const uint32_t h = hits[i];
            const int kx = whit_kx(h), kyh = whit_ky(h);
            const GPoint gp = own_point(br, r0, r1, os, kx, kyh);
            if (!gp.owned) continue;
            float2 ph = make_float2(1.f, 0.f);
            if (p.shift) ph = shift_phase(kx, kyh, sx, sy, p.inv_no);
            float2 S, dS[3];
            gather_grad<INTERP>(tile, gp, ph.x, S, dS);
            {
              const float2 G = p.img[out_index(p, img, kx, kyh)];
              const float2 gph = cmul(conjf2(G), ph);  // conj(G) * phase
#pragma unroll
              for (int j = 0; j < 3; ++j) {
                const double dldp = (double)gph.x * dS[j].x - (double)gph.y * dS[j].y;  // Re(g dS_j)
                acc[j] += (float)(os * kx * dldp);
                acc[3 + j] += (float)(os * kyh * dldp);
              }
              const double im_gs = (double)gph.x * S.y + (double)gph.y * S.x;  // Im(g S)
              const double two_pi_over_n = 6.283185307179586476925 * p.inv_no;
              acc[6] += (float)(two_pi_over_n * kx * im_gs);
              acc[7] += (float)(two_pi_over_n * kyh * im_gs);
            }
          }
          __builtin_amdgcn_wave_barrier();
        }
      }
      {
        double a8[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) a8[k] = (double)acc[k];
        const double d = wave_sum8(a8);
        const int k = lane >> 3;
        if ((lane & 7) == 0 && d != 0.0) {
          if (k < 6) {
            if (p.grad_rot) {
              const size_t brot = p.B_rot == 1 ? 0 : (size_t)br.b;
              unsafeAtomicAdd(p.grad_rot + ((brot * p.P + n) * 3 + k / 3) * 3 + k % 3, (float)d);
            }
          } else if (p.grad_shift) {
            const size_t bs = p.B_shift == 1 ? 0 : (size_t)br.b;
            unsafeAtomicAdd(p.grad_shift + (bs * p.P + n) * 2 + (k - 6), (float)d);
          }
        }
      }
    }
    __syncthreads();  // s_poses, s_cv and s_next are rewritten by the next window
  }
}

template <int INTERP>
BrickParams gather_params(const OpParams& p) {
  BrickParams bp{};
  bp.nb[0] = bricks_per_axis<INTERP>(p.N, kCX);
  bp.nb[1] = bricks_per_axis<INTERP>(p.N, kCY);
  bp.nb[2] = bricks_per_axis<INTERP>(p.N, kCZ);
  bp.nbricks = bp.nb[0] * bp.nb[1] * bp.nb[2];
  bp.pmax = 256;
  const int c = (p.P + bp.pmax - 1) / bp.pmax;
  bp.cmax = c < 1 ? 1 : (c > 64 ? 64 : c);
  return bp;
}

template <int INTERP>
hipError_t launch_grad(const OpParams& p, hipStream_t s) {
  const BrickParams bp = gather_params<INTERP>(p);
  const dim3 grid((unsigned)bp.nbricks, (unsigned)bp.cmax, (unsigned)p.B), block(kBlock);
  hipLaunchKernelGGL((k_grad_bricks<INTERP>), grid, block, 0, s, p, bp);
  return hipGetLastError();
}

}  // namespace

bool use_grad_bricks(const OpParams& p, int interp) {
  if (!(p.ndim == 3 && p.os <= 1.25f && p.N >= 288 && p.P >= 256)) return false;
  if (p.No > kMaxBrickOut || p.B > 65535) return false;
  const BrickParams bp = interp ? gather_params<1>(p) : gather_params<0>(p);
  return (uint64_t)p.B * (uint64_t)bp.nbricks * (uint64_t)bp.cmax <= 0x7FFFFFFFull;
}

hipError_t launch_grad_bricks(const OpParams& p, int interp, hipStream_t s) {
  return interp ? launch_grad<1>(p, s) : launch_grad<0>(p, s);
}

}  // namespace tp
