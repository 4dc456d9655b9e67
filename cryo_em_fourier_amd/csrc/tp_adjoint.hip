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
// point (exact, order independent; a (re, im) pair packed in one 64-bit
// word, or one int32 for the real weight volume), with a quantum chosen per
// group of poses from a bound on |G| that is checked
// against the values read (a group that exceeds it is redone), so the sums
// cannot overflow; each group is flushed into fp32 registers.  Bricks are split over pose chunks in
// proportion to the poses expected to cross them (near the origin: all of
// them); chunks of one brick merge with coalesced float atomics, unsplit
// bricks are written with plain stores.
//
// The same kernel runs the weight volume (real weights, int32 slots), the
// adjoint of the 3D -> 3D rotation (volume lattices), and the fused
// backwards: the adjoint followed, in the same launch, by workgroups that
// stream the pose gradients from a saved Jacobian (tp_gradjac.h).
#include "tp_adjoint.h"
#include "tp_gradjac.h"

namespace tp {

namespace {

using namespace adj;

// Workgroup shapes.  512 threads (8 waves, two workgroups per CU, 4 waves
// per SIMD) with a hit list that holds a whole pose group, for dense
// lattices; 256 threads (three workgroups per CU, 3 waves per SIMD) for
// sparse ones (oversampling above 1.25), whose bricks hold few hits.  The hit
// lists are sized so that the workgroups fit a CU's LDS beside the
// accumulator.
// EXCLZ (3D, 512 threads): z ownership is exclusive.  A lattice point is
// spread by the brick that holds its first z tap only, and the taps past the
// brick's last plane go to kGuard guard planes that are added to the next
// brick's first planes in global memory.  A stencil then crosses brick faces
// in x and y only, so each brick spreads about 16 % fewer lattice points.
template <int NDIM, int BS>
struct AdjShape {
  static constexpr bool EXCLZ = NDIM == 3 && BS == 512;
  static constexpr int HIT_CAP = BS == 512 ? (EXCLZ ? 5120 : 8192) : 2560;  // lattice points per group slice
  static constexpr int NVOX = EXCLZ ? 19 * 19 * 19 : kVox;  // brick voxels, guard columns, rows and planes included
  static constexpr int PER_THREAD = (NVOX + BS - 1) / BS;     // brick voxels per thread
  static constexpr int WAVES_PER_EU = BS == 512 ? 4 : 3;
};
// kSliceGrad / kVolumeGrad: kSlice / kVolume followed by B * P workgroups
// (1D grid) that each reduce one pose's gradients from a saved Jacobian (the
// fused backwards of the projection and of the rotation)
constexpr int kSlice = 0, kWeights = 1, kVolume = 2, kSliceGrad = 3, kVolumeGrad = 4;

// ---- volume lattice (the adjoint of the 3D -> 3D rotation) ----
// Lattice point k = (kx, ky, kz) of the full output volume carries the real
// output k when kx >= 0 and the mirror of the real output -k when kx <= 0;
// p = kx u + ky v + kz w with u, v, w = os R[0, :], os R[1, :], os R[2, :].

__device__ __forceinline__ void lattice_parts3(const OpParams& p, int kx, int ky, int kz, bool& real, bool& mirr) {
  const int rlo = -(p.No / 2), rhi = (p.No - 1) / 2;
  real = kx >= 0 && kx <= p.No / 2 && ky >= rlo && ky <= rhi && kz >= rlo && kz <= rhi;
  mirr = kx <= 0 && -kx <= p.No / 2 && -ky >= rlo && -ky <= rhi && -kz >= rlo && -kz <= rhi;
}

__device__ __forceinline__ size_t out_index3(const OpParams& p, size_t img, int kx, int ky, int kz) {
  return ((img * p.No + (kz < 0 ? kz + p.No : kz)) * p.No + (ky < 0 ? ky + p.No : ky)) * p.Wo + kx;
}

// Scan test of a volume lattice: finite rows, and the box within the largest
// |p| of a kept output (|k| <= cutoff, or the output cube's corner, times
// the Frobenius norm of os R, which bounds its largest singular value).
__device__ __forceinline__ bool vol_meets(const OpParams& p, int b, const Box& bx, int n) {
  const float* R = p.rot + ((size_t)(p.B_rot == 1 ? 0 : b) * p.P + n) * 9;
  double f2 = 0.0;
  for (int i = 0; i < 9; ++i) {
    const double r = (double)p.os * (double)R[i];
    if (!isfinite(r)) return false;
    f2 += r * r;
  }
  const double h = 0.5 * p.No;
  const double k2 = p.cut2 >= 0 ? fmin((double)p.cut2, 3.0 * h * h) : 3.0 * h * h;
  double d2 = 0.0;
  for (int j = 0; j < 3; ++j) {
    const double d = bx.lo[j] > 0.0 ? bx.lo[j] : (bx.hi[j] < 0.0 ? -bx.hi[j] : 0.0);
    d2 += d * d;
  }
  return d2 <= k2 * f2 * (1.0 + 1e-9) + 1e-9;
}

// Pose view of a volume lattice: the box's preimage k = A^-1 p (A = [u v w])
// bounds the (kx, ky, kz) ranges; a singular A keeps the whole clipped range.
__device__ __forceinline__ PoseView vol_view(const OpParams& p, int b, const Box& bx, int n) {
  PoseView pv;
  const float* R = p.rot + ((size_t)(p.B_rot == 1 ? 0 : b) * p.P + n) * 9;
  const double os = (double)p.os;
  for (int j = 0; j < 3; ++j) {
    pv.u[j] = os * (double)R[j];
    pv.v[j] = os * (double)R[3 + j];
    pv.w[j] = os * (double)R[6 + j];
    pv.iu[j] = pv.u[j] != 0.0 ? 1.0 / pv.u[j] : 0.0;
  }
  pv.sx = pv.sy = pv.sz = 0.f;
  if (p.shift) {
    const float* s = p.shift + ((size_t)(p.B_shift == 1 ? 0 : b) * p.P + n) * 3;
    pv.sx = s[0];
    pv.sy = s[1];
    pv.sz = s[2];
  }
  int lim = p.No / 2;
  if (p.cut2 >= 0) lim = min(lim, (int)floor(sqrt((double)p.cut2)));
  pv.kx0 = pv.ky0 = pv.kz0 = -lim;
  pv.kx1 = pv.ky1 = pv.kz1 = lim;
  // A[j][i]: component j of the column of k_i
  const double A[3][3] = {{pv.u[0], pv.v[0], pv.w[0]}, {pv.u[1], pv.v[1], pv.w[1]}, {pv.u[2], pv.v[2], pv.w[2]}};
  const double det = A[0][0] * (A[1][1] * A[2][2] - A[1][2] * A[2][1]) -
                     A[0][1] * (A[1][0] * A[2][2] - A[1][2] * A[2][0]) +
                     A[0][2] * (A[1][0] * A[2][1] - A[1][1] * A[2][0]);
  pv.dens = 1e30f;
  if (det != 0.0 && isfinite(det)) {
    pv.dens = (float)fmax(1.0, 1.0 / fabs(det));
    double inv[3][3];  // inverse by cofactors
    inv[0][0] = (A[1][1] * A[2][2] - A[1][2] * A[2][1]) / det;
    inv[0][1] = (A[0][2] * A[2][1] - A[0][1] * A[2][2]) / det;
    inv[0][2] = (A[0][1] * A[1][2] - A[0][2] * A[1][1]) / det;
    inv[1][0] = (A[1][2] * A[2][0] - A[1][0] * A[2][2]) / det;
    inv[1][1] = (A[0][0] * A[2][2] - A[0][2] * A[2][0]) / det;
    inv[1][2] = (A[0][2] * A[1][0] - A[0][0] * A[1][2]) / det;
    inv[2][0] = (A[1][0] * A[2][1] - A[1][1] * A[2][0]) / det;
    inv[2][1] = (A[0][1] * A[2][0] - A[0][0] * A[2][1]) / det;
    inv[2][2] = (A[0][0] * A[1][1] - A[0][1] * A[1][0]) / det;
    int* lo[3] = {&pv.kx0, &pv.ky0, &pv.kz0};
    int* hi[3] = {&pv.kx1, &pv.ky1, &pv.kz1};
    for (int i = 0; i < 3; ++i) {
      double kmin = 0.0, kmax = 0.0;
      for (int j = 0; j < 3; ++j) {
        const double a = bx.lo[j] * inv[i][j], c = bx.hi[j] * inv[i][j];
        kmin += fmin(a, c);
        kmax += fmax(a, c);
      }
      if (fabs(kmin) < 1e9 && fabs(kmax) < 1e9) {
        *lo[i] = max(*lo[i], (int)floor(kmin) - 1);
        *hi[i] = min(*hi[i], (int)ceil(kmax) + 1);
      }
    }
  }
  pv.hit = finite3(pv.u) && finite3(pv.v) && finite3(pv.w) && pv.kx0 <= pv.kx1 && pv.ky0 <= pv.ky1 &&
           pv.kz0 <= pv.kz1;
  if (pv.hit)
    pv.dens = fminf(pv.dens, 0.4f * (float)(pv.kx1 - pv.kx0 + 1) * (float)(pv.ky1 - pv.ky0 + 1) *
                                 (float)(pv.kz1 - pv.kz0 + 1) + 1.f);
  return pv;
}

// Volume hit tags: 10-bit offsets of kz, ky, kx in the pose's box.
__device__ __forceinline__ uint32_t vhit(int dkz, int dky, int dkx) {
  return ((uint32_t)dkz << 20) | ((uint32_t)dky << 10) | (uint32_t)dkx;
}

// List a volume lattice's points in the (widened) box, row by row over
// (ky, kz); flat indices [h0, h0 + cap) go to s_hits.  Returns the total.
template <int BS>
__device__ __forceinline__ int list_hits_vol(const OpParams& p, const Box& bx, const PoseView& pv, int h0, int cap,
                                             uint32_t* s_hits, int* s_wcnt) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nky = pv.ky1 - pv.ky0 + 1, nkz = pv.kz1 - pv.kz0 + 1;
  const int rows_total = pv.hit ? nky * nkz : 0;
  const int h1 = h0 + cap;
  int carry = 0;
  for (int rw = 0; rw < rows_total; rw += BS) {
    const int r = rw + tid;
    int cr = 0, a = 0, dky = 0, dkz = 0;
    if (r < rows_total) {
      dky = r % nky;
      dkz = r / nky;
      const int ky = pv.ky0 + dky, kz = pv.kz0 + dkz;
      double ta = (double)pv.kx0, tb = (double)pv.kx1;
      bool empty = false;
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const double lo = bx.lo[j] - 1e-6, hi = bx.hi[j] + 1e-6;
        const double c = (double)ky * pv.v[j] + (double)kz * pv.w[j];
        if (pv.iu[j] == 0.0) {
          empty = empty || !(c >= lo && c < hi);
        } else {
          const double t0 = (lo - c) * pv.iu[j], t1 = (hi - c) * pv.iu[j];
          ta = fmax(ta, fmin(t0, t1));
          tb = fmin(tb, fmax(t0, t1));
        }
      }
      if (p.cut2 >= 0) clip_kx_to_disk(p.cut2 - (long long)ky * ky - (long long)kz * kz, ta, tb, empty);
      a = (int)ceil(ta);
      const int b = empty ? a - 1 : (int)floor(tb);
      cr = max(0, b - a + 1);
      a -= pv.kx0;
    }
    int incl = cr;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(incl, o, 64);
      if (lane >= o) incl += t;
    }
    if (lane == 63) s_wcnt[wave] = incl;
    __syncthreads();
    int off = carry + incl - cr, tot = 0;
#pragma unroll
    for (int w = 0; w < BS / 64; ++w) {
      off += w < wave ? s_wcnt[w] : 0;
      tot += s_wcnt[w];
    }
    for (int j = max(0, h0 - off); j < cr && off + j < h1; ++j) s_hits[off + j - h0] = vhit(dkz, dky, a + j);
    carry += tot;
    __syncthreads();
  }
  return carry;
}

__device__ __forceinline__ void lattice_values3(const OpParams& p, const PoseView& pv, int kx, int ky, int kz,
                                                float2 gr, float2 gm, Cand& cd) {
#pragma unroll
  for (int j = 0; j < 3; ++j) cd.q[j] = (double)kx * pv.u[j] + (double)ky * pv.v[j] + (double)kz * pv.w[j];
  float2 cr = gr, cm = gm;
  if (p.shift) {
    const float2 ph = phase_of_turns(((double)kx * pv.sx + (double)ky * pv.sy + (double)kz * pv.sz) * p.inv_no);
    cr = cmul(conjf2(ph), gr);
    cm = cmul(ph, gm);
  }
  cd.v0 = cr;
  cd.v1 = make_float2(cr.x + cm.x, cr.y - cm.y);
}

// MODE: kSlice (the projector's adjoint), kWeights (real weight volume),
// kVolume (the adjoint of the 3D -> 3D rotation: volume lattices, one pose
// per group), kSliceGrad / kVolumeGrad (kSlice / kVolume and the pose
// gradients from a Jacobian).
template <int NDIM, int INTERP, int MODE, int BS>
__global__ __launch_bounds__(BS) __attribute__((amdgpu_waves_per_eu(AdjShape<NDIM, BS>::WAVES_PER_EU))) void k_adjoint_bricks(OpParams p,
                                                                                           BrickParams bp) {
  constexpr bool WEIGHTS = MODE == kWeights;
  constexpr bool VOL = MODE == kVolume || MODE == kVolumeGrad;
  constexpr int GMAX = VOL ? 1 : kGroupMax;
  using BR = Brick<NDIM>;
  using SH = AdjShape<NDIM, BS>;
  constexpr bool EXCLZ = SH::EXCLZ;
  using AL = AccLayout<NDIM, EXCLZ ? kGuard : 0>;
  __shared__ unsigned long long acc[AL::W];
  int* acc_r = reinterpret_cast<int*>(acc);  // the weight volume's int32 slots
  constexpr int kHitCap = SH::HIT_CAP;
  constexpr int kPerThread = SH::PER_THREAD;
  constexpr int kNVox = SH::NVOX;
  // RAW (exclusive ownership): thread tid keeps the accumulator slots tid +
  // i BS (one base address, immediate offsets in the flushes); the write-out
  // maps a slot back to its voxel.  Otherwise it keeps voxels tid + i BS.
  constexpr bool RAW = SH::EXCLZ;
  constexpr int G = EXCLZ ? kGuard : 0;
  constexpr int XR = BR::X + G, YR = BR::Y + G;  // x columns and y rows of the accumulator
  static_assert(!RAW || ((AL::W + BS - 1) / BS <= kPerThread && AL::S == XR && AL::ROWS == YR),
                "raw accumulator slots must fit the per-thread registers");
  // accumulator slot of entry i of this thread (-1: none)
  auto slot_of = [&](int i) -> int {
    const int v = threadIdx.x + i * BS;
    if (RAW) return v < AL::W ? v : -1;
    return v < kNVox ? acc_word<NDIM, G>(v % XR, (v / XR) % YR, v / (XR * YR)) : -1;
  };
  __shared__ uint32_t s_hits[kHitCap];
  __shared__ int s_poses[BS];
  __shared__ PoseView s_view[kGroupMax];
  __shared__ int s_wcnt[BS / 64];
  __shared__ float s_red[BS / 64];
  __shared__ int s_bad[BS / 64];

  const uint32_t lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  if constexpr (MODE == kSliceGrad || MODE == kVolumeGrad) {
    // fused backward: the workgroups after the bricks stream one pose's
    // gradient reduction each (HBM-bound), filling the CUs that the
    // LDS-bound bricks leave idle at the end of the launch
    const uint32_t adj = (uint32_t)bp.nbricks * (uint32_t)bp.cmax * (uint32_t)p.B;
    if (lin >= adj) {
      if constexpr (MODE == kSliceGrad) grad_jac_pose<BS>(p, lin - adj, reinterpret_cast<double(*)[8]>(acc));
      else grad_jac_vol<BS>(p, lin - adj, reinterpret_cast<double(*)[16]>(acc));
      return;
    }
  }
  BrickPos br = decode<NDIM, VOL>(p, bp, lin);
  if (!br.valid) return;
  if (EXCLZ) {
    br.xlim = min(br.x0 + BR::X + kGuard - 1, p.N / 2);
    br.ylim = min(br.y0 + BR::Y + kGuard - 1, (p.N + 1) / 2 - 1);
    br.zlim = min(br.z0 + BR::Z + kGuard - 1, (p.N + 1) / 2 - 1);
  }

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float m_prev = 0.f;  // max |G| of the previous group (0: none yet)
  float fre[kPerThread], fim[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) fre[i] = fim[i] = 0.f;
  for (int i = tid; i < AL::W; i += BS) acc[i] = 0ull;
  __syncthreads();

  const Box bx = reach_box<NDIM, INTERP, EXCLZ>(br);
  // (the linear kernel's 8 taps per point do not pay for the wave's ranking:
  // 2.39 against 2.10 ms at box 256, 4096 poses, so it keeps the general
  // spread; so does the weight volume, whose 32-bit adds are served 32 lanes
  // at a time over 32 banks: 3.11 against 3.08 ms)
  const int kind = INTERP && !WEIGHTS ? brick_kind<NDIM, G>(br) : 0;
  int g0 = 0;  // first pose of the current group in s_poses

  // G entries of hit h of the current group
  auto load_hit = [&](uint32_t h, float2& gr, float2& gm, bool valid = true) {
    if (VOL) {
      const PoseView& pv = s_view[0];
      const int kx = pv.kx0 + (int)(h & 0x3FFu), ky = pv.ky0 + (int)((h >> 10) & 0x3FFu), kz = pv.kz0 + (int)(h >> 20);
      const size_t img = (size_t)br.b * p.P + s_poses[g0];
      bool real, mirr;
      lattice_parts3(p, kx, ky, kz, real, mirr);
      gr = real && valid ? p.img[out_index3(p, img, kx, ky, kz)] : make_float2(0.f, 0.f);
      gm = mirr && valid ? p.img[out_index3(p, img, -kx, -ky, -kz)] : make_float2(0.f, 0.f);
    } else {
      const PoseView& pv = s_view[hit_pose(h)];
      lattice_load<WEIGHTS>(p, (size_t)br.b * p.P + s_poses[g0 + hit_pose(h)], hit_kx(h, pv), hit_ky(h, pv), valid, gr,
                            gm);
    }
  };

  // Every slice of lattice points that can reach the brick: pose windows of
  // the chunk, groups of up to GMAX poses, and slices of kHitCap hits when a
  // group overflows the hit list.  on_slice(nh, dens_sum) runs with the
  // slice's hits in s_hits[0, nh); a barrier follows it.
  auto traverse = [&](auto&& on_slice) {
    for (int w0 = br.n0; w0 < br.n1; w0 += BS) {
      // the poses whose plane (volume) can reach this brick, in order
      const int total = VOL ? scan_poses_if<BS>([&](int n) { return vol_meets(p, br.b, bx, n); }, w0, br.n1,
                                                s_poses, s_wcnt)
                            : scan_poses<NDIM, BS>(p, br.b, bx, w0, br.n1, s_poses, s_wcnt);
      for (g0 = 0; g0 < total; g0 += GMAX) {
        const int cnt = min(GMAX, total - g0);
        if (tid < cnt)
          s_view[tid] = VOL ? vol_view(p, br.b, bx, s_poses[g0 + tid])
                            : pose_view<NDIM>(p, br.b, bx, s_poses[g0 + tid], false);
        __syncthreads();
        float dens_sum;
        int cum[kGroupMax];
        group_sums<kGroupMax>(s_view, cnt, dens_sum, cum);
        for (int h0 = 0, hits_total = 1; h0 < hits_total; h0 += kHitCap) {
          // phase A: list the lattice points that can reach the brick (this
          // slice keeps the flat indices [h0, h0 + kHitCap))
          hits_total = VOL ? list_hits_vol<BS>(p, bx, s_view[0], h0, kHitCap, s_hits, s_wcnt)
                           : list_hits<NDIM, kGroupMax, BS>(p, bx, s_view, cum, h0, kHitCap, s_hits, s_wcnt);
          on_slice(max(0, min(hits_total, h0 + kHitCap) - h0), dens_sum);
          __syncthreads();
        }
      }
    }
  };

  bool brick_bad = false;  // some slice read a non-finite value (uniform)
  traverse([&](int nh, float dens_sum) {
    // phase B: spread the hits.  The fixed-point quantum assumes the
    // group's max |G| is at most twice the previous group's; the values
    // actually read are checked, and a group that exceeds its assumption
    // is cleared and redone with the measured bound (the first group of a
    // workgroup only measures).  See the bound at kQuantumBits.  Values
    // that are not finite are left out of the sums and of the bound.
    bool measure_only = m_prev <= 0.f;
    float m_assume = 2.f * m_prev, q = 0.f;
    while (nh > 0) {
      float inv_q = 0.f;
      if (!measure_only) {
        // (|G| below ~1e-19 gets a coarser quantum than needed)
        const float x = fminf(fmaxf(2.f * kDensBound * dens_sum * m_assume, 0x1p-60f), 3e38f);
        q = ldexpf(x, -kQuantumBits);
        inv_q = 1.f / q;
      }
      float amax = 0.f;
      bool bad = false;
      // software pipeline: the G values of a thread's next hit are loaded
      // while its current hit is spread
      float2 ngr, ngm;
      uint32_t nh_tag = s_hits[min(hit_slot(tid), nh - 1)];
      load_hit(nh_tag, ngr, ngm, hit_slot(tid) < nh);
      for (int i0 = 0; i0 < nh; i0 += BS) {
        const int i = i0 + hit_slot(tid);
        const uint32_t h = nh_tag;
        float2 gr = ngr, gm = ngm;
        nh_tag = s_hits[min(i + BS, nh - 1)];
        load_hit(nh_tag, ngr, ngm, i + BS < nh);
        if (!finite2(gr)) { gr = make_float2(0.f, 0.f); bad = true; }
        if (!finite2(gm)) { gm = make_float2(0.f, 0.f); bad = true; }
        amax = fmaxf(amax, fmaxf(fabsf(gr.x) + fabsf(gr.y), fabsf(gm.x) + fabsf(gm.y)));
        if (measure_only) continue;
        // (interior bricks: every lane of the wave takes part in the spread)
        if (i >= nh && kind == 0) continue;
        Cand cd;
        bool act = i < nh;
        if (act) {
          if (VOL) {
            const PoseView& pv = s_view[0];
            lattice_values3(p, pv, pv.kx0 + (int)(h & 0x3FFu), pv.ky0 + (int)((h >> 10) & 0x3FFu),
                            pv.kz0 + (int)(h >> 20), gr, gm, cd);
          } else {
            const PoseView& pv = s_view[hit_pose(h)];
            lattice_values<NDIM>(p, pv, hit_kx(h, pv), hit_ky(h, pv), gr, gm, cd);
          }
          act = in_box<NDIM>(bx, cd.q);
        }
        if (NDIM == 3 && G > 0 && kind == 2) {
          if constexpr (NDIM == 3 && G > 0 && !WEIGHTS) spread_interior<INTERP, G, false>(br, cd, act, inv_q, acc);
        } else if (NDIM == 3 && G > 0 && kind == 1) {
          if constexpr (NDIM == 3 && G > 0 && !WEIGHTS) spread_interior<INTERP, G, true>(br, cd, act, inv_q, acc);
        } else if (act) {
          spread<NDIM, INTERP, WEIGHTS, G>(br, cd, inv_q, acc);
        }
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
      const bool wbad = __ballot(bad) != 0ull;
      __syncthreads();
      if (lane == 0) {
        s_red[wave] = amax;
        s_bad[wave] = wbad;
      }
      __syncthreads();
      // one read per lane, then readlane: the workgroup's max and flag
      const float rv = lane < BS / 64 ? s_red[lane] : 0.f;
      const int bv = lane < BS / 64 ? s_bad[lane] : 0;
      float gmax = 0.f;
#pragma unroll
      for (int w = 0; w < BS / 64; ++w) {
        gmax = fmaxf(gmax, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rv), w)));
        brick_bad = brick_bad || __builtin_amdgcn_readlane(bv, w) != 0;
      }
      if (!(gmax > 0.f)) break;  // an all-zero slice adds nothing
      if (!measure_only && gmax <= m_assume) {
        // flush the slice into fp32 registers
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
          const int sl = slot_of(i);
          if (sl < 0) continue;
          if (WEIGHTS) {
            fre[i] = fmaf((float)acc_r[sl], q, fre[i]);
            acc_r[sl] = 0;
          } else {
            int ir, ii;
            unpack_pair(acc[sl], ir, ii);
            fre[i] = fmaf((float)ir, q, fre[i]);
            fim[i] = fmaf((float)ii, q, fim[i]);
            acc[sl] = 0ull;
          }
        }
        m_prev = gmax;
        break;
      }
      if (!measure_only) {
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
          const int sl = slot_of(i);
          if (sl < 0) continue;
          if (WEIGHTS) acc_r[sl] = 0;
          else acc[sl] = 0ull;
        }
        __syncthreads();
      }
      m_assume = gmax;
      measure_only = false;
    }
  });

  if (brick_bad) {
    // Some upstream values were not finite.  Walk the slices again and mark
    // the slots that their taps reach in the accumulator (clear after the
    // last flush); those voxels become NaN, as a non-finite term makes the
    // adjoint's sum there.
    traverse([&](int nh, float) {
      for (int i = tid; i < nh; i += BS) {
        const uint32_t h = s_hits[i];
        float2 gr, gm;
        load_hit(h, gr, gm);
        const bool b0 = !finite2(gr), b1 = b0 || !finite2(gm);
        if (!b1) continue;
        double qp[3] = {0.0, 0.0, 0.0};
        if (VOL) {
          const PoseView& pv = s_view[0];
          const int kx = pv.kx0 + (int)(h & 0x3FFu), ky = pv.ky0 + (int)((h >> 10) & 0x3FFu), kz = pv.kz0 + (int)(h >> 20);
          for (int j = 0; j < 3; ++j) qp[j] = (double)kx * pv.u[j] + (double)ky * pv.v[j] + (double)kz * pv.w[j];
        } else {
          const PoseView& pv = s_view[hit_pose(h)];
          const int kx = hit_kx(h, pv), ky = hit_ky(h, pv);
          for (int j = 0; j < NDIM; ++j) qp[j] = (double)kx * pv.u[j] + (double)ky * pv.v[j];
        }
        if (in_box<NDIM>(bx, qp)) mark_taps<NDIM, INTERP, WEIGHTS, G>(br, qp, b0, b1, acc);
      }
    });
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int sl = slot_of(i);
      if (sl < 0) continue;
      if (WEIGHTS ? acc_r[sl] != 0 : acc[sl] != 0ull) fre[i] = fim[i] = __builtin_nanf("");
    }
  }

  // write the brick: plain stores, or float atomics for pose-chunked bricks
  // and, with exclusive z ownership, for the guard planes and the first
  // kGuard planes (which the brick below adds its guard planes to)
  float2* out = p.ref_out + (size_t)br.b * p.ref_elems;
  float* wout = p.wref_out + (size_t)br.b * p.ref_elems;
  const int wh = p.N / 2 + 1;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    int xr, yr, zr;
    if (RAW) {
      const int t = tid + i * BS - kGuard;  // (the leading guard slots hold no voxel)
      if (t < 0 || t >= AL::W - kGuard) continue;
      zr = t / AL::PZ;
      const int r = t - zr * AL::PZ;
      if (r >= AL::ROWS * AL::S) continue;  // plane padding
      yr = r / AL::S;
      xr = r - yr * AL::S;
    } else {
      const int v = tid + i * BS;
      if (v >= kNVox) continue;
      xr = v % XR;
      yr = (v / XR) % YR;
      zr = v / (XR * YR);
    }
    const int x = br.x0 + xr;
    const int y = br.y0 + yr;
    const int z = br.z0 + zr;
    if (x > br.xlim || y > br.ylim || (NDIM == 3 && z > br.zlim)) continue;
    const bool merge = br.chunked || (EXCLZ && (xr >= BR::X || yr >= BR::Y || zr >= BR::Z ||
                                                (xr < kGuard && !br.xbottom) || (yr < kGuard && !br.ybottom) ||
                                                (zr < kGuard && !br.zbottom)));
    const size_t row = NDIM == 3 ? (size_t)(z < 0 ? z + p.N : z) * p.N + (y < 0 ? y + p.N : y)
                                 : (size_t)(y < 0 ? y + p.N : y);
    if (WEIGHTS) {
      float* wdst = wout + row * wh + x;
      if (merge) {
        if (fre[i] != 0.f) unsafeAtomicAdd(wdst, fre[i]);
      } else {
        *wdst = fre[i];
      }
      continue;
    }
    float2* dst = out + row * wh + x;
    if (merge) {
      if (fre[i] != 0.f) unsafeAtomicAdd(&dst->x, fre[i]);
      if (fim[i] != 0.f) unsafeAtomicAdd(&dst->y, fim[i]);
    } else {
      *dst = make_float2(fre[i], fim[i]);
    }
  }
}

}  // namespace

template <int NDIM>
static BrickParams brick_params(const OpParams& p, bool vol = false, int pmax = 256) {
  using BR = Brick<NDIM>;
  BrickParams bp{};
  bp.nb[0] = (p.N / 2 + 1 + BR::X - 1) / BR::X;
  bp.nb[1] = (p.N + BR::Y - 1) / BR::Y;
  bp.nb[2] = NDIM == 3 ? (p.N + BR::Z - 1) / BR::Z : 1;
  bp.nbricks = bp.nb[0] * bp.nb[1] * bp.nb[2];
  // a volume lattice sends every pose to every brick: small chunks (box 64,
  // 512 poses: 2.42 ms with 8 poses per chunk, 2.54 with 16, 2.72 with 32)
  bp.pmax = vol ? 8 : pmax;
  const int c = (p.P + bp.pmax - 1) / bp.pmax;
  bp.cmax = c < 1 ? 1 : (c > 64 ? 64 : c);
  return bp;
}

uint64_t adjoint_blocks(const OpParams& p) {
  const BrickParams bp = p.ndim == 3 ? brick_params<3>(p) : brick_params<2>(p);
  return (uint64_t)p.B * (uint64_t)bp.nbricks * (uint64_t)bp.cmax;
}

// Dense lattices fill a brick with hits and run faster on 512-thread
// workgroups (in 3D with exclusive ownership); sparse ones on 256.  Measured
// at box 256 with 4096 poses: 5.9 against 6.4 ms at oversampling 1 (up to
// 1.25 for every kernel); with the bank-ranked spread and raw flush slots,
// the 3D cubic adjoint at oversampling 2 takes 7.84 against 8.16 ms on 512
// threads (cubic 3D: up to 2), the linear one 6.33 against 4.62 ms.
static bool wide_adjoint(const OpParams& p, int interp) {
  return p.os <= (p.ndim == 3 && interp == 1 ? 2.f : 1.25f);  // 1: cubic
}

template <int MODE, int BS>
static void launch_modes(const OpParams& p, const BrickParams& bp, int ndim, int interp, hipStream_t s) {
  dim3 grid((unsigned)bp.nbricks, (unsigned)bp.cmax, (unsigned)p.B), block(BS);
  if (MODE == kSliceGrad || MODE == kVolumeGrad) grid = dim3((unsigned)((uint64_t)bp.nbricks * bp.cmax * p.B + (uint64_t)p.B * p.P));
  if (ndim == 3) {
    if (interp) hipLaunchKernelGGL((k_adjoint_bricks<3, 1, MODE, BS>), grid, block, 0, s, p, bp);
    else hipLaunchKernelGGL((k_adjoint_bricks<3, 0, MODE, BS>), grid, block, 0, s, p, bp);
  } else {
    if constexpr (MODE == kSlice || MODE == kWeights) {  // volume lattices and the fused backward are 3D only
      if (interp) hipLaunchKernelGGL((k_adjoint_bricks<2, 1, MODE, BS>), grid, block, 0, s, p, bp);
      else hipLaunchKernelGGL((k_adjoint_bricks<2, 0, MODE, BS>), grid, block, 0, s, p, bp);
    }
  }
}

template <int MODE>
static hipError_t launch_adjoint(const OpParams& p, const BrickParams& bp, int ndim, int interp, hipStream_t s) {
  if (wide_adjoint(p, interp)) launch_modes<MODE, 512>(p, bp, ndim, interp, s);
  else launch_modes<MODE, 256>(p, bp, ndim, interp, s);
  return hipGetLastError();
}

hipError_t launch_backproject(const OpParams& p, int interp, hipStream_t s) {
  const BrickParams bp = p.ndim == 3 ? brick_params<3>(p) : brick_params<2>(p);
  return launch_adjoint<kSlice>(p, bp, p.ndim, interp, s);
}

// The adjoint and the pose gradients from a saved Jacobian in one launch:
// measured at box 256 with 4096 poses, 6.0 ms against 6.65 ms for the two launches (the gradient
// workgroups fill the adjoint's tail).  Spreading them among the bricks
// instead was slower (7.2 to 8.8 ms): they take the LDS-bound bricks' slots.
hipError_t launch_backward_jac(const OpParams& p, int interp, hipStream_t s) {
  // with many bricks (boxes from 256), larger pose chunks than the plain
  // adjoint's: fewer, longer brick workgroups, whose uneven end the gradient
  // workgroups fill (box 256, 4096 poses: 6.01 ms with 512 poses per chunk,
  // 6.10 with 256, 6.2 with 768; box 320, 8192 poses: 16.35 against 16.66;
  // a box of 128 has 320 bricks and
  // needs the smaller chunks to fill the GPU: 1.23 against 0.80 ms)
  const BrickParams bp = brick_params<3>(p);
  return launch_adjoint<kSliceGrad>(p, bp.nbricks >= 2048 ? brick_params<3>(p, false, 512) : bp, 3, interp, s);
}

uint64_t backward_jac_blocks(const OpParams& p) {
  return adjoint_blocks(p) + (uint64_t)p.B * (uint64_t)p.P;
}

hipError_t launch_backproject_weights(const OpParams& p, int interp, hipStream_t s) {
  const BrickParams bp = p.ndim == 3 ? brick_params<3>(p) : brick_params<2>(p);
  return launch_adjoint<kWeights>(p, bp, p.ndim, interp, s);
}

uint64_t rotate_adjoint_blocks(const OpParams& p) {
  const BrickParams bp = brick_params<3>(p, true);
  return (uint64_t)p.B * (uint64_t)bp.nbricks * (uint64_t)bp.cmax;
}

// the rotation's adjoint and its pose gradients from a saved Jacobian in one
// launch (as launch_backward_jac)
hipError_t launch_rotate_backward_jac(const OpParams& p, int interp, hipStream_t s) {
  return launch_adjoint<kVolumeGrad>(p, brick_params<3>(p, true), 3, interp, s);
}

uint64_t rotate_backward_jac_blocks(const OpParams& p) {
  return rotate_adjoint_blocks(p) + (uint64_t)p.B * (uint64_t)p.P;
}

hipError_t launch_rotate_adjoint(const OpParams& p, int interp, hipStream_t s) {
  return launch_adjoint<kVolume>(p, brick_params<3>(p, true), 3, interp, s);
}

}  // namespace tp
