// Single-pass backward of the 3D -> 2D projection for gfx950 (cubic): the
// adjoint (the reference's gradient) and the rotation and shift gradients
// from one walk over the lattice points, reading the reference itself and
// nothing the forward saved (it page tech. section 3: one pass, no
// intermediate tensors; ar page tech. section 2: pose gradients by the chain
// rule through the kernel's derivative; ko page tech. section 2: the
// backward is the adjoint).
//
// It is the brick adjoint of tp_adjoint.hip (exclusive ownership: a lattice
// point belongs to the brick that holds its first x, y and z taps, whose
// accumulator has guard columns, rows and planes for the other taps) with
// the brick's part of the reference staged in LDS beside the accumulator, in
// the same slot layout.  For every tap of a lattice point the kernel adds
// its weighted value to the accumulator and reads the reference at the same
// slot, so the weights, derivative weights and row addresses serve both
// directions.
//
// Pose gradients in the lattice form of the adjoint.  A lattice point k of
// the full frequency plane, at sample point q = kx u + ky v, spreads v0 =
// c(k) to its taps at x = 0 and v1 = c(k) + conj(c(-k)) to its taps at
// x >= 1 (c = conj(phase) G; the parts of outputs that do not exist are 0).
// Splitting each output's stencil sum at x = 0 and mirroring the x < 0 taps
// (see tp_device.h) gives, summed over the lattice points of a pose,
//   dL/dR[0][j] = os sum kx A_j,   dL/dR[1][j] = os sum ky A_j,
//   dL/ds_x = 2 pi / N_out sum kx B,   dL/ds_y = 2 pi / N_out sum ky B,
//   A_j = sum_taps dw/dq_j Re(conj(v) V[t]),  B = sum_taps w Im(conj(v) V[t]),
// with v = v0 or v1 by the tap's x: the chain rule of tp_grad_pose, with the
// mirrored taps' derivative and conjugation signs cancelling against -k.
// The stencil is floor(q)'s at every lattice point, which for the C1 cubic
// kernel is the derivative in p itself (the extra tap of a mirrored integer
// coordinate has weight and derivative 0).
//
// A wave's lanes hold consecutive hits of the pose-ordered hit list, so the
// eight terms of each hit are summed per pose with a segmented wave
// reduction into LDS (fp64), and each slice's per-pose sums go to the
// outputs with float atomics once its fixed-point pass is accepted (a redone
// pass discards them).
#include "tp_adjoint.h"

namespace tp {

namespace {

using namespace adj;

// Shapes.  BZ: brick depth (16 x 16 x BZ voxels).  The accumulator and the
// reference tile share the guarded slot layout; the hit list takes what is
// left of the LDS.
template <int BZ, int BS>
struct BwdShape {
  using AL = AccLayout<3, kGuard, BZ>;
  static constexpr int XR = 16 + kGuard, YR = 16 + kGuard, ZR = BZ + kGuard;
  static constexpr int NVOX = XR * YR * ZR;                    // voxels with guards
  static constexpr int PER_THREAD = (NVOX + BS - 1) / BS;
  static constexpr int WGS_PER_CU = BZ <= 8 ? 2 : 1;
  static constexpr int LDS_BYTES = 163840 / WGS_PER_CU;
  static constexpr int FIXED = 2 * AL::W * 8 + BS * 4 + kGroupMax * (int)sizeof(PoseView) + kGroupMax * 64 +
                               3 * (BS / 64) * 4 + 64;
  static constexpr int HIT_CAP = ((LDS_BYTES - FIXED) / 4) & ~255;
  static constexpr int WAVES_PER_EU = BS / 64 * WGS_PER_CU / 4;
  static_assert(HIT_CAP >= 1024, "hit list too small");
};

// The eight pose-gradient terms of the lanes' hits, summed per pose slot
// into s_grad (fp64).  Lanes hold non-decreasing slots (slot < 0: no hit);
// every lane of the wave calls it.
__device__ __forceinline__ void add_pose_terms(int slot, const float* g, double (*s_grad)[8]) {
  const int lane = threadIdx.x & 63;
  unsigned long long pending = __ballot(slot >= 0);
  while (pending) {
    const int first = __ffsll((long long)pending) - 1;
    const int s = __shfl(slot, first, 64);
    const bool in = slot == s;
    double a[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) a[k] = in ? (double)g[k] : 0.0;
    const double d = wave_sum8(a);
    if ((lane & 7) == 0) atomicAdd(&s_grad[s][lane >> 3], d);
    pending &= ~__ballot(in);
  }
}

template <int BZ, int BS>
__global__ __launch_bounds__(BS) __attribute__((amdgpu_waves_per_eu(BwdShape<BZ, BS>::WAVES_PER_EU))) void
k_backward_bricks(OpParams p, BrickParams bp) {
  using SH = BwdShape<BZ, BS>;
  using AL = typename SH::AL;
  using K = Kern<1>;
  constexpr int G = kGuard;
  constexpr int XR = SH::XR, YR = SH::YR;
  constexpr int kPerThread = SH::PER_THREAD;
  constexpr int kHitCap = SH::HIT_CAP;
  // the reference tile first, then the accumulator, in one buffer: a row's
  // tile reads (8-bit offsets) and atomic adds (16-bit offsets) then share
  // one base address
  static_assert(AL::W * 8 + 64 <= 65535, "accumulator beyond the LDS instructions' offset range");
  __shared__ float2 lds_ta[2 * AL::W];
  float2* tile = lds_ta;
  unsigned long long* acc = reinterpret_cast<unsigned long long*>(lds_ta + AL::W);
  __shared__ uint32_t s_hits[kHitCap];
  __shared__ int s_poses[BS];
  __shared__ PoseView s_view[kGroupMax];
  __shared__ double s_grad[kGroupMax][8];
  __shared__ int s_wcnt[BS / 64];
  __shared__ float s_red[BS / 64];
  __shared__ int s_bad[BS / 64];

  const uint32_t lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  BrickPos br = decode<3, false, BZ>(p, bp, lin);
  if (!br.valid) return;
  const int hi = (p.N + 1) / 2 - 1;
  br.xlim = min(br.x0 + 16 + kGuard - 1, p.N / 2);
  br.ylim = min(br.y0 + 16 + kGuard - 1, hi);
  br.zlim = min(br.z0 + BZ + kGuard - 1, hi);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float fre[kPerThread], fim[kPerThread];
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) fre[i] = fim[i] = 0.f;
  for (int i = tid; i < AL::W; i += BS) {
    acc[i] = 0ull;
    tile[i] = make_float2(0.f, 0.f);
  }
  if (tid < kGroupMax * 8) s_grad[tid >> 3][tid & 7] = 0.0;
  __syncthreads();
  {
    // the reference over the brick and its guards (0 outside the stored range)
    const float2* V = p.ref + (size_t)br.b * p.ref_elems;
    const int N = p.N, wh = N / 2 + 1;
    for (int v = tid; v < SH::NVOX; v += BS) {
      const int xr = v % XR, yr = (v / XR) % YR, zr = v / (XR * YR);
      const int x = br.x0 + xr, y = br.y0 + yr, z = br.z0 + zr;
      if (x <= br.xlim && y <= br.ylim && z <= br.zlim)
        tile[acc_word<3, G, BZ>(xr, yr, zr)] =
            V[((size_t)(z < 0 ? z + N : z) * N + (y < 0 ? y + N : y)) * wh + x];
    }
  }
  __syncthreads();

  const Box bx = reach_box<3, 1, true>(br);
  const double os = (double)p.os;
  const float two_pi_over_n = (float)(6.283185307179586476925 * p.inv_no);
  const size_t brot = p.B_rot == 1 ? 0 : (size_t)br.b;
  const size_t bsh = p.B_shift == 1 ? 0 : (size_t)br.b;
  float m_prev = 0.f;
  int g0 = 0;

  auto load_hit = [&](uint32_t h, float2& gr, float2& gm) {
    const PoseView& pv = s_view[hit_pose(h)];
    lattice_load<false>(p, (size_t)br.b * p.P + s_poses[g0 + hit_pose(h)], hit_kx(h, pv), hit_ky(h, pv), gr, gm);
  };

  // Every slice of lattice points that can reach the brick (as the adjoint's
  // walk); on_slice(nh, dens_sum, cnt) runs with the slice's hits in
  // s_hits[0, nh) and the group's cnt poses in s_view; a barrier follows.
  auto traverse = [&](auto&& on_slice) {
    for (int w0 = br.n0; w0 < br.n1; w0 += BS) {
      const int total = scan_poses<3, BS>(p, br.b, bx, w0, br.n1, s_poses, s_wcnt);
      for (g0 = 0; g0 < total; g0 += kGroupMax) {
        const int cnt = min(kGroupMax, total - g0);
        if (tid < cnt) s_view[tid] = pose_view<3>(p, br.b, bx, s_poses[g0 + tid], false);
        __syncthreads();
        float dens_sum;
        int cum[kGroupMax];
        group_sums<kGroupMax>(s_view, cnt, dens_sum, cum);
        for (int h0 = 0, hits_total = 1; h0 < hits_total; h0 += kHitCap) {
          hits_total = list_hits<3, kGroupMax, BS>(p, bx, s_view, cum, h0, kHitCap, s_hits, s_wcnt);
          on_slice(max(0, min(hits_total, h0 + kHitCap) - h0), dens_sum, cnt);
          __syncthreads();
        }
      }
    }
  };

  bool brick_bad = false;
  traverse([&](int nh, float dens_sum, int cnt) {
    bool measure_only = m_prev <= 0.f;
    float m_assume = 2.f * m_prev, q = 0.f;
    while (nh > 0) {
      float inv_q = 0.f;
      if (!measure_only) {
        const float x = fminf(fmaxf(2.f * kDensBound * dens_sum * m_assume, 0x1p-60f), 3e38f);
        q = ldexpf(x, -kQuantumBits);
        inv_q = 1.f / q;
      }
      float amax = 0.f;
      bool bad = false;
      for (int i0 = 0; i0 < nh; i0 += kPrefetch * BS) {
        float2 gr[kPrefetch], gm[kPrefetch];
        bool hbad[kPrefetch];
#pragma unroll
        for (int k = 0; k < kPrefetch; ++k) {
          const int i = i0 + hit_slot(tid) + k * BS;
          gr[k] = gm[k] = make_float2(0.f, 0.f);
          if (i < nh) load_hit(s_hits[i], gr[k], gm[k]);
        }
#pragma unroll
        for (int k = 0; k < kPrefetch; ++k) {
          hbad[k] = !finite2(gr[k]) || !finite2(gm[k]);
          if (!finite2(gr[k])) gr[k] = make_float2(0.f, 0.f);
          if (!finite2(gm[k])) gm[k] = make_float2(0.f, 0.f);
          bad = bad || hbad[k];
          amax = fmaxf(amax, fmaxf(fabsf(gr[k].x) + fabsf(gr[k].y), fabsf(gm[k].x) + fabsf(gm[k].y)));
        }
        if (measure_only) continue;
#pragma unroll
        for (int k = 0; k < kPrefetch; ++k) {
          const int i = i0 + hit_slot(tid) + k * BS;
          int slot = -1;
          float gt[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) gt[j] = 0.f;
          if (i < nh) {
            const uint32_t h = s_hits[i];
            const PoseView& pv = s_view[hit_pose(h)];
            const int kx = hit_kx(h, pv), ky = hit_ky(h, pv);
            Cand cd;
            lattice_values<3>(p, pv, kx, ky, gr[k], gm[k], cd);
            if (in_box<3>(bx, cd.q)) {
              slot = hit_pose(h);
              const AxisPos ax = axis_pos(cd.q[0], K::OFF), ay = axis_pos(cd.q[1], K::OFF),
                            az = axis_pos(cd.q[2], K::OFF);
              float wy[4], wz[4], dwy[4], dwz[4];
              K::w(ay.f, wy);
              K::w(az.f, wz);
              K::dw(ay.f, dwy);
              K::dw(az.f, dwz);
              // x factors: e = w_x v, f = w_x' v with v = v0 at x = 0, v1
              // at x >= 1 and 0 before x = 0 (those taps are the mirror
              // lattice point's)
              float2 e[4], f[4];
              {
                float wx[4], dwx[4];
                K::w(ax.f, wx);
                K::dw(ax.f, dwx);
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                  const int tx = ax.x0 + d;
                  const float2 v = tx >= 1 ? cd.v1 : (tx == 0 ? cd.v0 : make_float2(0.f, 0.f));
                  e[d] = make_float2(wx[d] * v.x, wx[d] * v.y);
                  f[d] = make_float2(dwx[d] * v.x, dwx[d] * v.y);
                }
              }
              // Rows and planes outside the brick's range (only in the lowest
              // and highest bricks of an axis) get weight 0 and a clamped
              // slot, so the 64 taps run without branches; the row and plane
              // offsets are set up once per lattice point.
              int oy[4], oz[4];
#pragma unroll
              for (int d = 0; d < 4; ++d) {
                const int ty = ay.x0 + d, tz = az.x0 + d;
                const bool yok = ty >= br.y0 && ty <= br.ylim, zok = tz >= br.z0 && tz <= br.zlim;
                oy[d] = (min(max(ty, br.y0), br.ylim) - br.y0) * AL::S;
                oz[d] = (min(max(tz, br.z0), br.zlim) - br.z0) * AL::PZ;
                if (!yok) wy[d] = dwy[d] = 0.f;
                if (!zok) wz[d] = dwz[d] = 0.f;
              }
              float wzq[4];  // the z weights times the quantum's inverse (the spread's scale)
#pragma unroll
              for (int d = 0; d < 4; ++d) wzq[d] = wz[d] * inv_q;
              const int x0w = acc_word<3, G, BZ>(ax.x0 - br.x0, 0, 0);
              float sa_x = 0.f, sa_y = 0.f, sa_z = 0.f, sb = 0.f;
#pragma unroll
              for (int dz = 0; dz < 4; ++dz) {
                float px = 0.f, py = 0.f, pz = 0.f, pb = 0.f;
#pragma unroll
                for (int dy = 0; dy < 4; ++dy) {
                  const int w = x0w + oz[dz] + oy[dy];
                  float2 V[4];
#pragma unroll
                  for (int dx = 0; dx < 4; ++dx) V[dx] = tile[w + dx];
                  const float sq = wy[dy] * wzq[dz];
#pragma unroll
                  for (int dx = 0; dx < 4; ++dx)
                    atomicAdd(acc + w + dx, pack_pair(cvt_rpi(e[dx].x * sq), cvt_rpi(e[dx].y * sq)));
                  float rr = 0.f, ri = 0.f, rd = 0.f;
#pragma unroll
                  for (int dx = 0; dx < 4; ++dx) {
                    rr = fmaf(e[dx].x, V[dx].x, fmaf(e[dx].y, V[dx].y, rr));
                    ri = fmaf(e[dx].x, V[dx].y, fmaf(-e[dx].y, V[dx].x, ri));
                    rd = fmaf(f[dx].x, V[dx].x, fmaf(f[dx].y, V[dx].y, rd));
                  }
                  px = fmaf(wy[dy], rd, px);
                  py = fmaf(dwy[dy], rr, py);
                  pz = fmaf(wy[dy], rr, pz);
                  pb = fmaf(wy[dy], ri, pb);
                }
                sa_x = fmaf(wz[dz], px, sa_x);
                sa_y = fmaf(wz[dz], py, sa_y);
                sa_z = fmaf(dwz[dz], pz, sa_z);
                sb = fmaf(wz[dz], pb, sb);
              }
              const float okx = (float)(os * kx), oky = (float)(os * ky);
              gt[0] = okx * sa_x;
              gt[1] = okx * sa_y;
              gt[2] = okx * sa_z;
              gt[3] = oky * sa_x;
              gt[4] = oky * sa_y;
              gt[5] = oky * sa_z;
              gt[6] = two_pi_over_n * (float)kx * sb;
              gt[7] = two_pi_over_n * (float)ky * sb;
              if (hbad[k]) {  // a non-finite upstream value: its pose's gradient is not finite either
#pragma unroll
                for (int j = 0; j < 8; ++j) gt[j] = __builtin_nanf("");
              }
            }
          }
          add_pose_terms(slot, gt, s_grad);
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
      bool any_bad = false;
#pragma unroll
      for (int w = 0; w < BS / 64; ++w) {
        gmax = fmaxf(gmax, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rv), w)));
        any_bad = any_bad || __builtin_amdgcn_readlane(bv, w) != 0;
      }
      brick_bad = brick_bad || any_bad;
      // (a pass whose finite values are all 0 is accepted too: its
      // non-finite hits still make their poses' gradients NaN)
      if (!measure_only && gmax <= m_assume) {
        // flush the slice into fp32 registers and its pose terms to the outputs
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
          const int v = tid + i * BS;
          if (v >= SH::NVOX) continue;
          const int sl = acc_word<3, G, BZ>(v % XR, (v / XR) % YR, v / (XR * YR));
          int ir, ii;
          unpack_pair(acc[sl], ir, ii);
          fre[i] = fmaf((float)ir, q, fre[i]);
          fim[i] = fmaf((float)ii, q, fim[i]);
          acc[sl] = 0ull;
        }
        if (tid < cnt * 8) {
          const int s = tid >> 3, j = tid & 7;
          const double v = s_grad[s][j];
          const int n = s_poses[g0 + s];
          if (v != 0.0) {
            if (j < 6) {
              if (p.grad_rot) unsafeAtomicAdd(p.grad_rot + ((brot * p.P + n) * 3 + j / 3) * 3 + j % 3, (float)v);
            } else if (p.grad_shift) {
              unsafeAtomicAdd(p.grad_shift + (bsh * p.P + n) * 2 + (j - 6), (float)v);
            }
          }
          s_grad[s][j] = 0.0;
        }
        if (gmax > 0.f) m_prev = gmax;
        break;
      }
      if (!(gmax > 0.f) && !any_bad) break;  // an all-zero slice adds nothing
      if (!measure_only) {
        // redo: clear the slice's sums and pose terms
#pragma unroll
        for (int i = 0; i < kPerThread; ++i) {
          const int v = tid + i * BS;
          if (v < SH::NVOX) acc[acc_word<3, G, BZ>(v % XR, (v / XR) % YR, v / (XR * YR))] = 0ull;
        }
        if (tid < kGroupMax * 8) s_grad[tid >> 3][tid & 7] = 0.0;
        __syncthreads();
      }
      m_assume = gmax > 0.f ? gmax : 1.f;
      measure_only = false;
    }
  });

  if (brick_bad) {
    // non-finite upstream values: the voxels their taps reach become NaN
    traverse([&](int nh, float, int) {
      for (int i = tid; i < nh; i += BS) {
        const uint32_t h = s_hits[i];
        float2 gr, gm;
        load_hit(h, gr, gm);
        const bool b0 = !finite2(gr), b1 = b0 || !finite2(gm);
        if (!b1) continue;
        const PoseView& pv = s_view[hit_pose(h)];
        const int kx = hit_kx(h, pv), ky = hit_ky(h, pv);
        double qp[3];
        for (int j = 0; j < 3; ++j) qp[j] = (double)kx * pv.u[j] + (double)ky * pv.v[j];
        if (in_box<3>(bx, qp)) mark_taps<3, 1, false, G, BZ>(br, qp, b0, b1, acc);
      }
    });
#pragma unroll
    for (int i = 0; i < kPerThread; ++i) {
      const int v = tid + i * BS;
      if (v >= SH::NVOX) continue;
      if (acc[acc_word<3, G, BZ>(v % XR, (v / XR) % YR, v / (XR * YR))] != 0ull) fre[i] = fim[i] = __builtin_nanf("");
    }
  }

  // write the brick: plain stores; float atomics for pose-chunked bricks,
  // the guards and the first kGuard columns, rows and planes (which the
  // bricks below add their guards to)
  float2* out = p.ref_out + (size_t)br.b * p.ref_elems;
  const int wh = p.N / 2 + 1;
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int v = tid + i * BS;
    if (v >= SH::NVOX) continue;
    const int xr = v % XR, yr = (v / XR) % YR, zr = v / (XR * YR);
    const int x = br.x0 + xr, y = br.y0 + yr, z = br.z0 + zr;
    if (x > br.xlim || y > br.ylim || z > br.zlim) continue;
    const bool merge = br.chunked || xr >= 16 || yr >= 16 || zr >= BZ || (xr < kGuard && !br.xbottom) ||
                       (yr < kGuard && !br.ybottom) || (zr < kGuard && !br.zbottom);
    float2* dst = out + ((size_t)(z < 0 ? z + p.N : z) * p.N + (y < 0 ? y + p.N : y)) * wh + x;
    if (merge) {
      if (fre[i] != 0.f) unsafeAtomicAdd(&dst->x, fre[i]);
      if (fim[i] != 0.f) unsafeAtomicAdd(&dst->y, fim[i]);
    } else {
      *dst = make_float2(fre[i], fim[i]);
    }
  }
}

template <int BZ>
BrickParams backward_params(const OpParams& p) {
  BrickParams bp{};
  bp.nb[0] = (p.N / 2 + 1 + 15) / 16;
  bp.nb[1] = (p.N + 15) / 16;
  bp.nb[2] = (p.N + BZ - 1) / BZ;
  bp.nbricks = bp.nb[0] * bp.nb[1] * bp.nb[2];
  bp.pmax = 256;
  const int c = (p.P + bp.pmax - 1) / bp.pmax;
  bp.cmax = c < 1 ? 1 : (c > 64 ? 64 : c);
  return bp;
}

template <int BZ, int BS>
hipError_t launch_bz(const OpParams& p, hipStream_t s) {
  const BrickParams bp = backward_params<BZ>(p);
  const dim3 grid((unsigned)bp.nbricks, (unsigned)bp.cmax, (unsigned)p.B), block(BS);
  hipLaunchKernelGGL((k_backward_bricks<BZ, BS>), grid, block, 0, s, p, bp);
  return hipGetLastError();
}

// brick depth and workgroup size (a build-time choice; see the launch)
constexpr int kBwdBZ = 8;
constexpr int kBwdBS = 512;

}  // namespace

uint64_t backward_blocks(const OpParams& p) {
  const BrickParams bp = backward_params<kBwdBZ>(p);
  return (uint64_t)p.B * (uint64_t)bp.nbricks * (uint64_t)bp.cmax;
}

// The single-pass backward for the cubic kernel; the linear kernel takes the
// adjoint and the per-output gradient kernel (two launches on the stream).
hipError_t launch_backward(const OpParams& p, int interp, hipStream_t s) {
  if (interp == 1) return launch_bz<kBwdBZ, kBwdBS>(p, s);
  hipError_t e = hipSuccess;
  if (p.ref_out) e = launch_backproject(p, interp, s);
  if (e == hipSuccess && (p.grad_rot || p.grad_shift)) e = launch_grad_pose(p, interp, s);
  return e;
}

}  // namespace tp
