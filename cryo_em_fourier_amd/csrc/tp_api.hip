// C ABI of the projector (declared in include/tp.h): argument checks, launch
// geometry, kernel dispatch.  Every check runs before the first HIP call, so
// invalid calls return without touching the device.
#include <cmath>
#include <cstdint>

#include "../../include/tp.h"
#include "tp_internal.h"

namespace {

constexpr int64_t kMaxBox = 65535;
constexpr uint64_t kMaxRefBytes = (1ull << 31) - 4096;  // see kBig in tp_device.h
constexpr uint64_t kMaxBlocks = 0x7FFFFFFFull;

bool aligned8(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 7u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

struct Common {
  int64_t B, N, P, N_out, B_rot, B_shift;
  int interp, ndim;
  float os, cutoff;
  const float* rot;
  const float* shift;
};

// Shared checks; returns TP_OK and fills the kernel parameters.
tp_status check_and_fill(const Common& c, tp::OpParams& p) {
  if (c.ndim != 2 && c.ndim != 3) return TP_EINVAL;
  if (c.B <= 0 || c.N <= 0 || c.P <= 0 || c.N_out <= 0) return TP_EINVAL;
  if (c.interp != TP_LINEAR && c.interp != TP_CUBIC) return TP_EINVAL;
  if (!std::isfinite(c.os) || !(c.os > 0.f)) return TP_EINVAL;
  if (std::isnan(c.cutoff)) return TP_EINVAL;
  if (!c.rot || !aligned4(c.rot)) return TP_EINVAL;
  if (c.B_rot != 1 && c.B_rot != c.B) return TP_EINVAL;
  if (c.shift) {
    if (!aligned4(c.shift)) return TP_EINVAL;
    if (c.B_shift != 1 && c.B_shift != c.B) return TP_EINVAL;
  }
  if (c.N > kMaxBox || c.N_out > kMaxBox) return TP_EUNSUPPORTED;
  const uint64_t wh = (uint64_t)(c.N / 2 + 1);
  const uint64_t elems = (c.ndim == 3 ? (uint64_t)c.N * (uint64_t)c.N : (uint64_t)c.N) * wh;
  if (elems * 8ull > kMaxRefBytes) return TP_EUNSUPPORTED;
  const int64_t wo = c.N_out / 2 + 1;
  const int64_t tile_x = c.ndim == 3 ? tp::kTileXPairs : tp::kTileX;
  const int64_t tile_y = c.ndim == 3 ? tp::kTileYPairs : tp::kTileY;
  const int64_t tx = (wo + tile_x - 1) / tile_x;
  const int64_t ty = (c.N_out + tile_y - 1) / tile_y;
  const uint64_t blocks = (uint64_t)c.B * (uint64_t)c.P * (uint64_t)(tx * ty);
  if (blocks > kMaxBlocks) return TP_EUNSUPPORTED;

  p = tp::OpParams{};
  p.rot = c.rot;
  p.shift = c.shift;
  p.B = (int)c.B;
  p.P = (int)c.P;
  p.N = (int)c.N;
  p.No = (int)c.N_out;
  p.Wo = (int)wo;
  p.B_rot = (int)c.B_rot;
  p.B_shift = c.shift ? (int)c.B_shift : 1;
  p.ndim = c.ndim;
  p.os = c.os;
  if (c.cutoff < 0.f) {
    p.cut2 = -1;
  } else {
    const double c2 = (double)c.cutoff * (double)c.cutoff;
    p.cut2 = c2 > 9.0e18 ? (long long)9.0e18 : (long long)std::floor(c2);
  }
  p.ref_bytes = (uint32_t)(elems * 8ull);
  p.ref_elems = (long long)elems;
  p.inv_no = 1.0 / (double)c.N_out;
  p.tiles_x = (int)tx;
  p.tiles_y = (int)ty;
  p.tiles_per_pose = (int)(tx * ty);
  p.tile_y = (int)tile_y;
  p.nblocks = (uint32_t)blocks;
  p.nblocks2 = (uint32_t)((uint64_t)c.B * (uint64_t)c.P * (uint64_t)(tx * ((ty + 1) / 2)));
  return TP_OK;
}

tp_status hip_status(hipError_t e) { return e == hipSuccess ? TP_OK : TP_EHIP; }

size_t ref_bytes_total(const tp::OpParams& p) { return (size_t)p.B * (size_t)p.ref_elems * 8u; }

tp_status project(int ndim, const tp_c64* ref, int64_t B, int64_t N, const float* rot,
                  int64_t B_rot, int64_t P, const float* shift, int64_t B_shift, int64_t N_out,
                  int interp, float os, float cutoff, tp_c64* out, void* stream) {
  if (!ref || !out || !aligned8(ref) || !aligned8(out)) return TP_EINVAL;
  tp::OpParams p;
  const Common c{B, N, P, N_out, B_rot, B_shift, interp, ndim, os, cutoff, rot, shift};
  const tp_status st = check_and_fill(c, p);
  if (st != TP_OK) return st;
  p.ref = reinterpret_cast<const float2*>(ref);
  p.img_out = reinterpret_cast<float2*>(out);
  return hip_status(tp::launch_project(p, interp, (hipStream_t)stream));
}

tp_status backproject(int ndim, const tp_c64* proj, int64_t B, int64_t P, int64_t N_out,
                      const float* rot, int64_t B_rot, const float* shift, int64_t B_shift,
                      int64_t N, int interp, float os, float cutoff, tp_c64* ref_out,
                      void* stream) {
  if (!proj || !ref_out || !aligned8(proj) || !aligned8(ref_out)) return TP_EINVAL;
  tp::OpParams p;
  const Common c{B, N, P, N_out, B_rot, B_shift, interp, ndim, os, cutoff, rot, shift};
  const tp_status st = check_and_fill(c, p);
  if (st != TP_OK) return st;
  // the brick kernels' lattice lists hold 14-bit offsets within an output image
  if (N_out > tp::kMaxBrickOut || B > 65535 || tp::adjoint_blocks(p) > kMaxBlocks) return TP_EUNSUPPORTED;
  p.img = reinterpret_cast<const float2*>(proj);
  p.ref_out = reinterpret_cast<float2*>(ref_out);
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e = tp::launch_zero(p.ref_out, ref_bytes_total(p), s);
  if (e != hipSuccess) return TP_EHIP;
  return hip_status(tp::launch_backproject(p, interp, s));
}

tp_status backproject_weights(int ndim, const float* w, int64_t B, int64_t P, int64_t N_out,
                              const float* rot, int64_t B_rot, int64_t N, int interp, float os,
                              float cutoff, float* wref_out, void* stream) {
  if (!w || !wref_out || !aligned4(w) || !aligned4(wref_out)) return TP_EINVAL;
  tp::OpParams p;
  const Common c{B, N, P, N_out, B_rot, 1, interp, ndim, os, cutoff, rot, nullptr};
  const tp_status st = check_and_fill(c, p);
  if (st != TP_OK) return st;
  if (N_out > tp::kMaxBrickOut || B > 65535 || tp::adjoint_blocks(p) > kMaxBlocks) return TP_EUNSUPPORTED;
  p.wimg = w;
  p.wref_out = wref_out;
  const hipStream_t s = (hipStream_t)stream;
  if (tp::launch_zero(wref_out, (size_t)p.B * (size_t)p.ref_elems * sizeof(float), s) != hipSuccess)
    return TP_EHIP;
  return hip_status(tp::launch_backproject_weights(p, interp, s));
}

// The 3D -> 3D rotation: the reference's checks, then a tiling of the
// [N_out, N_out, N_out/2+1] output (8 kx columns x 16 (kz, ky) rows, two
// lanes per output).
tp_status rotate_fill(const Common& c, tp::OpParams& p) {
  const tp_status st = check_and_fill(c, p);
  if (st != TP_OK) return st;
  const uint64_t rows = (uint64_t)c.N_out * (uint64_t)c.N_out;
  const uint64_t tx = (uint64_t)(p.Wo + tp::kTileXPairs - 1) / tp::kTileXPairs;
  const uint64_t ty = (rows + tp::kTileYPairs - 1) / tp::kTileYPairs;
  const uint64_t blocks = (uint64_t)c.B * (uint64_t)c.P * tx * ty;
  if (blocks > kMaxBlocks || tx * ty > 0x7FFFFFFFull) return TP_EUNSUPPORTED;
  p.tiles_x = (int)tx;
  p.tiles_y = (int)ty;
  p.tiles_per_pose = (int)(tx * ty);
  p.tile_y = tp::kTileYPairs;
  p.nblocks = (uint32_t)blocks;
  return TP_OK;
}

}  // namespace

extern "C" {

int tp_abi_version(void) { return TP_ABI_VERSION; }

const char* tp_status_str(tp_status status) {
  switch ((int)status) {
    case TP_OK: return "TP_OK";
    case TP_EINVAL: return "TP_EINVAL: invalid argument";
    case TP_EUNSUPPORTED: return "TP_EUNSUPPORTED: size or shape not supported";
    case TP_EHIP: return "TP_EHIP: HIP runtime error";
    default: return "TP_UNKNOWN";
  }
}

tp_status tp_project_3d(const tp_c64* vol, int64_t B, int64_t N, const float* rot, int64_t B_rot,
                        int64_t P, const float* shift, int64_t B_shift, int64_t N_out, tp_interp interp,
                        float oversampling, float cutoff, tp_c64* out, void* stream) {
  return project(3, vol, B, N, rot, B_rot, P, shift, B_shift, N_out, interp, oversampling, cutoff,
                 out, stream);
}

tp_status tp_project_2d(const tp_c64* img, int64_t B, int64_t N, const float* rot, int64_t B_rot,
                        int64_t P, const float* shift, int64_t B_shift, int64_t N_out, tp_interp interp,
                        float oversampling, float cutoff, tp_c64* out, void* stream) {
  return project(2, img, B, N, rot, B_rot, P, shift, B_shift, N_out, interp, oversampling, cutoff,
                 out, stream);
}

tp_status tp_backproject_3d(const tp_c64* proj, int64_t B, int64_t P, int64_t N_out,
                            const float* rot, int64_t B_rot, const float* shift, int64_t B_shift,
                            int64_t N, tp_interp interp, float oversampling, float cutoff,
                            tp_c64* vol_out, void* stream) {
  return backproject(3, proj, B, P, N_out, rot, B_rot, shift, B_shift, N, interp, oversampling,
                     cutoff, vol_out, stream);
}

tp_status tp_backproject_2d(const tp_c64* proj, int64_t B, int64_t P, int64_t N_out,
                            const float* rot, int64_t B_rot, const float* shift, int64_t B_shift,
                            int64_t N, tp_interp interp, float oversampling, float cutoff,
                            tp_c64* img_out, void* stream) {
  return backproject(2, proj, B, P, N_out, rot, B_rot, shift, B_shift, N, interp, oversampling,
                     cutoff, img_out, stream);
}

tp_status tp_backproject_weights_3d(const float* weights, int64_t B, int64_t P, int64_t N_out,
                                    const float* rot, int64_t B_rot, int64_t N, tp_interp interp,
                                    float oversampling, float cutoff, float* wvol_out, void* stream) {
  return backproject_weights(3, weights, B, P, N_out, rot, B_rot, N, interp, oversampling, cutoff, wvol_out,
                             stream);
}

tp_status tp_backproject_weights_2d(const float* weights, int64_t B, int64_t P, int64_t N_out,
                                    const float* rot, int64_t B_rot, int64_t N, tp_interp interp,
                                    float oversampling, float cutoff, float* wimg_out, void* stream) {
  return backproject_weights(2, weights, B, P, N_out, rot, B_rot, N, interp, oversampling, cutoff, wimg_out,
                             stream);
}

tp_status tp_rotate_3d(const tp_c64* vol, int64_t B, int64_t N, const float* rot, int64_t B_rot, int64_t P,
                       const float* shift, int64_t B_shift, int64_t N_out, tp_interp interp, float oversampling,
                       float cutoff, tp_c64* out, void* stream) {
  if (!vol || !out || !aligned8(vol) || !aligned8(out)) return TP_EINVAL;
  tp::OpParams p;
  const Common c{B, N, P, N_out, B_rot, B_shift, interp, 3, oversampling, cutoff, rot, shift};
  const tp_status st = rotate_fill(c, p);
  if (st != TP_OK) return st;
  p.ref = reinterpret_cast<const float2*>(vol);
  p.img_out = reinterpret_cast<float2*>(out);
  return hip_status(tp::launch_rotate(p, interp, 0, (hipStream_t)stream));
}

tp_status tp_rotate_backproject_3d(const tp_c64* grad_out, int64_t B, int64_t P, int64_t N_out, const float* rot,
                                   int64_t B_rot, const float* shift, int64_t B_shift, int64_t N, tp_interp interp,
                                   float oversampling, float cutoff, tp_c64* vol_out, void* stream) {
  if (!grad_out || !vol_out || !aligned8(grad_out) || !aligned8(vol_out)) return TP_EINVAL;
  tp::OpParams p;
  const Common c{B, N, P, N_out, B_rot, B_shift, interp, 3, oversampling, cutoff, rot, shift};
  const tp_status st = rotate_fill(c, p);
  if (st != TP_OK) return st;
  if (N_out > tp::kMaxRotateAdjointOut || B > 65535 || tp::rotate_adjoint_blocks(p) > kMaxBlocks)
    return TP_EUNSUPPORTED;
  p.img = reinterpret_cast<const float2*>(grad_out);
  p.ref_out = reinterpret_cast<float2*>(vol_out);
  const hipStream_t s = (hipStream_t)stream;
  if (tp::launch_zero(p.ref_out, ref_bytes_total(p), s) != hipSuccess) return TP_EHIP;
  return hip_status(tp::launch_rotate_adjoint(p, interp, s));
}

tp_status tp_rotate_grad_pose(const tp_c64* vol, int64_t B, int64_t N, const tp_c64* grad_out, const float* rot,
                              int64_t B_rot, int64_t P, const float* shift, int64_t B_shift, int64_t N_out,
                              tp_interp interp, float oversampling, float cutoff, float* grad_rot, float* grad_shift,
                              void* stream) {
  if (!vol || !grad_out || !aligned8(vol) || !aligned8(grad_out)) return TP_EINVAL;
  if ((grad_rot && !aligned4(grad_rot)) || (grad_shift && !aligned4(grad_shift))) return TP_EINVAL;
  if (grad_shift && B_shift != 1 && B_shift != B) return TP_EINVAL;
  tp::OpParams p;
  const Common c{B, N, P, N_out, B_rot, B_shift, interp, 3, oversampling, cutoff, rot, shift};
  const tp_status st = rotate_fill(c, p);
  if (st != TP_OK) return st;
  if (!grad_rot && !grad_shift) return TP_OK;
  p.ref = reinterpret_cast<const float2*>(vol);
  p.img = reinterpret_cast<const float2*>(grad_out);
  p.grad_rot = grad_rot;
  p.grad_shift = grad_shift;
  if (!shift) p.B_shift = (int)B_shift;
  const hipStream_t s = (hipStream_t)stream;
  if (grad_rot && tp::launch_zero(grad_rot, (size_t)p.B_rot * p.P * 9 * sizeof(float), s) != hipSuccess)
    return TP_EHIP;
  if (grad_shift && tp::launch_zero(grad_shift, (size_t)p.B_shift * p.P * 3 * sizeof(float), s) != hipSuccess)
    return TP_EHIP;
  return hip_status(tp::launch_rotate(p, interp, 2, s));
}

tp_status tp_symmetrize_x0(int ndim, tp_c64* ref, int64_t B, int64_t N, void* stream) {
  if (ndim != 2 && ndim != 3) return TP_EINVAL;
  if (!ref || !aligned8(ref) || B <= 0 || N <= 0) return TP_EINVAL;
  if (N > kMaxBox || B > 0x7FFFFFFF) return TP_EUNSUPPORTED;
  const uint64_t rows = (uint64_t)B * (uint64_t)N * (uint64_t)(ndim == 3 ? N : 1);
  if ((rows + 255) / 256 > kMaxBlocks) return TP_EUNSUPPORTED;
  return hip_status(tp::launch_symmetrize_x0(reinterpret_cast<float2*>(ref), ndim, (int)B, (int)N,
                                             (hipStream_t)stream));
}

tp_status tp_grad_pose(int ndim, const tp_c64* ref, int64_t B, int64_t N, const tp_c64* grad_out,
                       const float* rot, int64_t B_rot, int64_t P, const float* shift,
                       int64_t B_shift, int64_t N_out, tp_interp interp, float oversampling,
                       float cutoff, float* grad_rot, float* grad_shift, void* stream) {
  if (!ref || !grad_out || !aligned8(ref) || !aligned8(grad_out)) return TP_EINVAL;
  if ((grad_rot && !aligned4(grad_rot)) || (grad_shift && !aligned4(grad_shift))) return TP_EINVAL;
  if (grad_shift && B_shift != 1 && B_shift != B) return TP_EINVAL;
  tp::OpParams p;
  const Common c{B, N, P, N_out, B_rot, B_shift, interp, ndim, oversampling, cutoff, rot, shift};
  const tp_status st = check_and_fill(c, p);
  if (st != TP_OK) return st;
  if (!grad_rot && !grad_shift) return TP_OK;
  p.ref = reinterpret_cast<const float2*>(ref);
  p.img = reinterpret_cast<const float2*>(grad_out);
  p.grad_rot = grad_rot;
  p.grad_shift = grad_shift;
  // with no shift tensor the shift is 0, but grad_shift keeps its B_shift rows
  if (!shift) p.B_shift = (int)B_shift;
  const hipStream_t s = (hipStream_t)stream;
  if (grad_rot) {
    const size_t n = (size_t)p.B_rot * p.P * ndim * ndim * sizeof(float);
    if (tp::launch_zero(grad_rot, n, s) != hipSuccess) return TP_EHIP;
  }
  if (grad_shift) {
    const size_t n = (size_t)p.B_shift * p.P * 2 * sizeof(float);
    if (tp::launch_zero(grad_shift, n, s) != hipSuccess) return TP_EHIP;
  }
  return hip_status(tp::launch_grad_pose(p, interp, s));
}

tp_status tp_backward_3d(const tp_c64* vol, int64_t B, int64_t N, const tp_c64* grad_out, const float* rot,
                         int64_t B_rot, int64_t P, const float* shift, int64_t B_shift, int64_t N_out,
                         tp_interp interp, float oversampling, float cutoff, tp_c64* vol_grad, float* grad_rot,
                         float* grad_shift, void* stream) {
  if (!vol || !grad_out || !aligned8(vol) || !aligned8(grad_out)) return TP_EINVAL;
  if (vol_grad && !aligned8(vol_grad)) return TP_EINVAL;
  if ((grad_rot && !aligned4(grad_rot)) || (grad_shift && !aligned4(grad_shift))) return TP_EINVAL;
  if (grad_shift && B_shift != 1 && B_shift != B) return TP_EINVAL;
  tp::OpParams p;
  const Common c{B, N, P, N_out, B_rot, B_shift, interp, 3, oversampling, cutoff, rot, shift};
  const tp_status st = check_and_fill(c, p);
  if (st != TP_OK) return st;
  if (vol_grad && (N_out > tp::kMaxBrickOut || B > 65535 || tp::adjoint_blocks(p) > kMaxBlocks))
    return TP_EUNSUPPORTED;
  if (!vol_grad && !grad_rot && !grad_shift) return TP_OK;
  p.ref = reinterpret_cast<const float2*>(vol);
  p.img = reinterpret_cast<const float2*>(grad_out);
  p.ref_out = reinterpret_cast<float2*>(vol_grad);
  p.grad_rot = grad_rot;
  p.grad_shift = grad_shift;
  if (!shift) p.B_shift = (int)B_shift;
  const hipStream_t s = (hipStream_t)stream;
  if (grad_rot && tp::launch_zero(grad_rot, (size_t)p.B_rot * p.P * 9 * sizeof(float), s) != hipSuccess)
    return TP_EHIP;
  if (grad_shift && tp::launch_zero(grad_shift, (size_t)p.B_shift * p.P * 2 * sizeof(float), s) != hipSuccess)
    return TP_EHIP;
  if (!vol_grad) return hip_status(tp::launch_grad_pose(p, interp, s));
  if (tp::launch_zero(p.ref_out, ref_bytes_total(p), s) != hipSuccess) return TP_EHIP;
  const hipError_t e = tp::launch_backproject(p, interp, s);
  if (e != hipSuccess || (!grad_rot && !grad_shift)) return hip_status(e);
  return hip_status(tp::launch_grad_pose(p, interp, s));
}

tp_status tp_project_3d_jac(const tp_c64* vol, int64_t B, int64_t N, const float* rot, int64_t B_rot,
                            int64_t P, const float* shift, int64_t B_shift, int64_t N_out, tp_interp interp,
                            float oversampling, float cutoff, tp_c64* out, tp_c64* jac, void* stream) {
  if (!vol || !out || !jac || !aligned8(vol) || !aligned8(out) || !aligned8(jac)) return TP_EINVAL;
  tp::OpParams p;
  const Common c{B, N, P, N_out, B_rot, B_shift, interp, 3, oversampling, cutoff, rot, shift};
  const tp_status st = check_and_fill(c, p);
  if (st != TP_OK) return st;
  p.ref = reinterpret_cast<const float2*>(vol);
  p.img_out = reinterpret_cast<float2*>(out);
  p.jac_out = reinterpret_cast<float2*>(jac);
  return hip_status(tp::launch_project_jac(p, interp, (hipStream_t)stream));
}

tp_status tp_grad_pose_jac(const tp_c64* grad_out, const tp_c64* proj, const tp_c64* jac, int64_t B, int64_t P,
                           int64_t N_out, int64_t B_rot, int64_t B_shift, float oversampling, float cutoff,
                           float* grad_rot, float* grad_shift, void* stream) {
  if (!grad_out || !proj || !jac || !aligned8(grad_out) || !aligned8(proj) || !aligned8(jac)) return TP_EINVAL;
  if ((grad_rot && !aligned4(grad_rot)) || (grad_shift && !aligned4(grad_shift))) return TP_EINVAL;
  if (B <= 0 || P <= 0 || N_out <= 0) return TP_EINVAL;
  if (B_rot != 1 && B_rot != B) return TP_EINVAL;
  if (grad_shift && B_shift != 1 && B_shift != B) return TP_EINVAL;
  if (!std::isfinite(oversampling) || !(oversampling > 0.f) || std::isnan(cutoff)) return TP_EINVAL;
  if (N_out > kMaxBox || (uint64_t)B * (uint64_t)P > kMaxBlocks) return TP_EUNSUPPORTED;
  if (!grad_rot && !grad_shift) return TP_OK;
  tp::OpParams p{};
  p.B = (int)B;
  p.P = (int)P;
  p.No = (int)N_out;
  p.Wo = (int)(N_out / 2 + 1);
  p.B_rot = (int)B_rot;
  p.B_shift = grad_shift ? (int)B_shift : 1;
  p.ndim = 3;
  p.os = oversampling;
  if (cutoff < 0.f) {
    p.cut2 = -1;
  } else {
    const double c2 = (double)cutoff * (double)cutoff;
    p.cut2 = c2 > 9.0e18 ? (long long)9.0e18 : (long long)std::floor(c2);
  }
  p.inv_no = 1.0 / (double)N_out;
  p.img = reinterpret_cast<const float2*>(grad_out);
  p.proj = reinterpret_cast<const float2*>(proj);
  p.jac = reinterpret_cast<const float2*>(jac);
  p.grad_rot = grad_rot;
  p.grad_shift = grad_shift;
  const hipStream_t s = (hipStream_t)stream;
  if (grad_rot && tp::launch_zero(grad_rot, (size_t)p.B_rot * p.P * 9 * sizeof(float), s) != hipSuccess)
    return TP_EHIP;
  if (grad_shift && tp::launch_zero(grad_shift, (size_t)p.B_shift * p.P * 2 * sizeof(float), s) != hipSuccess)
    return TP_EHIP;
  return hip_status(tp::launch_grad_jac(p, s));
}

tp_status tp_backward_3d_jac(const tp_c64* grad_out, const tp_c64* proj, const tp_c64* jac, int64_t B, int64_t P,
                            int64_t N_out, const float* rot, int64_t B_rot, const float* shift, int64_t B_shift,
                            int64_t N, tp_interp interp, float oversampling, float cutoff, tp_c64* vol_out,
                            float* grad_rot, float* grad_shift, void* stream) {
  if (!grad_out || !proj || !jac || !vol_out) return TP_EINVAL;
  if (!aligned8(grad_out) || !aligned8(proj) || !aligned8(jac) || !aligned8(vol_out)) return TP_EINVAL;
  if ((grad_rot && !aligned4(grad_rot)) || (grad_shift && !aligned4(grad_shift))) return TP_EINVAL;
  if (grad_shift && B_shift != 1 && B_shift != B) return TP_EINVAL;
  tp::OpParams p;
  const Common c{B, N, P, N_out, B_rot, B_shift, interp, 3, oversampling, cutoff, rot, shift};
  const tp_status st = check_and_fill(c, p);
  if (st != TP_OK) return st;
  if (N_out > tp::kMaxBrickOut || B > 65535 || tp::backward_jac_blocks(p) > kMaxBlocks) return TP_EUNSUPPORTED;
  p.img = reinterpret_cast<const float2*>(grad_out);
  p.ref_out = reinterpret_cast<float2*>(vol_out);
  p.proj = reinterpret_cast<const float2*>(proj);
  p.jac = reinterpret_cast<const float2*>(jac);
  p.grad_rot = grad_rot;
  p.grad_shift = grad_shift;
  // with no shift tensor the shift is 0, but grad_shift keeps its B_shift rows
  if (!shift && grad_shift) p.B_shift = (int)B_shift;
  const hipStream_t s = (hipStream_t)stream;
  if (tp::launch_zero(p.ref_out, ref_bytes_total(p), s) != hipSuccess) return TP_EHIP;
  if (!grad_rot && !grad_shift) return hip_status(tp::launch_backproject(p, interp, s));
  if (grad_rot && tp::launch_zero(grad_rot, (size_t)p.B_rot * p.P * 9 * sizeof(float), s) != hipSuccess)
    return TP_EHIP;
  if (grad_shift && tp::launch_zero(grad_shift, (size_t)p.B_shift * p.P * 2 * sizeof(float), s) != hipSuccess)
    return TP_EHIP;
  return hip_status(tp::launch_backward_jac(p, interp, s));
}

tp_status tp_rotate_backward_3d_jac(const tp_c64* grad_out, const tp_c64* out, const tp_c64* jac, int64_t B,
                                   int64_t P, int64_t N_out, const float* rot, int64_t B_rot, const float* shift,
                                   int64_t B_shift, int64_t N, tp_interp interp, float oversampling, float cutoff,
                                   tp_c64* vol_out, float* grad_rot, float* grad_shift, void* stream) {
  if (!grad_out || !out || !jac || !vol_out) return TP_EINVAL;
  if (!aligned8(grad_out) || !aligned8(out) || !aligned8(jac) || !aligned8(vol_out)) return TP_EINVAL;
  if ((grad_rot && !aligned4(grad_rot)) || (grad_shift && !aligned4(grad_shift))) return TP_EINVAL;
  if (grad_shift && B_shift != 1 && B_shift != B) return TP_EINVAL;
  tp::OpParams p;
  const Common c{B, N, P, N_out, B_rot, B_shift, interp, 3, oversampling, cutoff, rot, shift};
  const tp_status st = rotate_fill(c, p);
  if (st != TP_OK) return st;
  if (N_out > tp::kMaxRotateAdjointOut || B > 65535 || tp::rotate_backward_jac_blocks(p) > kMaxBlocks)
    return TP_EUNSUPPORTED;
  p.img = reinterpret_cast<const float2*>(grad_out);
  p.ref_out = reinterpret_cast<float2*>(vol_out);
  p.proj = reinterpret_cast<const float2*>(out);
  p.jac = reinterpret_cast<const float2*>(jac);
  p.grad_rot = grad_rot;
  p.grad_shift = grad_shift;
  // with no shift tensor the shift is 0, but grad_shift keeps its B_shift rows
  if (!shift && grad_shift) p.B_shift = (int)B_shift;
  const hipStream_t s = (hipStream_t)stream;
  if (tp::launch_zero(p.ref_out, ref_bytes_total(p), s) != hipSuccess) return TP_EHIP;
  if (!grad_rot && !grad_shift) return hip_status(tp::launch_rotate_adjoint(p, interp, s));
  if (grad_rot && tp::launch_zero(grad_rot, (size_t)p.B_rot * p.P * 9 * sizeof(float), s) != hipSuccess)
    return TP_EHIP;
  if (grad_shift && tp::launch_zero(grad_shift, (size_t)p.B_shift * p.P * 3 * sizeof(float), s) != hipSuccess)
    return TP_EHIP;
  return hip_status(tp::launch_rotate_backward_jac(p, interp, s));
}

tp_status tp_rotate_3d_jac(const tp_c64* vol, int64_t B, int64_t N, const float* rot, int64_t B_rot, int64_t P,
                           const float* shift, int64_t B_shift, int64_t N_out, tp_interp interp, float oversampling,
                           float cutoff, tp_c64* out, tp_c64* jac, void* stream) {
  if (!vol || !out || !jac || !aligned8(vol) || !aligned8(out) || !aligned8(jac)) return TP_EINVAL;
  tp::OpParams p;
  const Common c{B, N, P, N_out, B_rot, B_shift, interp, 3, oversampling, cutoff, rot, shift};
  const tp_status st = rotate_fill(c, p);
  if (st != TP_OK) return st;
  if (N_out > tp::kMaxRotateAdjointOut) return TP_EUNSUPPORTED;
  p.ref = reinterpret_cast<const float2*>(vol);
  p.img_out = reinterpret_cast<float2*>(out);
  p.jac_out = reinterpret_cast<float2*>(jac);
  return hip_status(tp::launch_rotate_jac(p, interp, (hipStream_t)stream));
}

tp_status tp_rotate_grad_pose_jac(const tp_c64* grad_out, const tp_c64* out, const tp_c64* jac, int64_t B,
                                  int64_t P, int64_t N_out, int64_t B_rot, int64_t B_shift, float oversampling,
                                  float cutoff, float* grad_rot, float* grad_shift, void* stream) {
  if (!grad_out || !out || !jac || !aligned8(grad_out) || !aligned8(out) || !aligned8(jac)) return TP_EINVAL;
  if ((grad_rot && !aligned4(grad_rot)) || (grad_shift && !aligned4(grad_shift))) return TP_EINVAL;
  if (B <= 0 || P <= 0 || N_out <= 0) return TP_EINVAL;
  if (B_rot != 1 && B_rot != B) return TP_EINVAL;
  if (grad_shift && B_shift != 1 && B_shift != B) return TP_EINVAL;
  if (!std::isfinite(oversampling) || !(oversampling > 0.f) || std::isnan(cutoff)) return TP_EINVAL;
  if (N_out > tp::kMaxRotateAdjointOut || (uint64_t)B * (uint64_t)P > kMaxBlocks) return TP_EUNSUPPORTED;
  if (!grad_rot && !grad_shift) return TP_OK;
  tp::OpParams p{};
  p.B = (int)B;
  p.P = (int)P;
  p.No = (int)N_out;
  p.Wo = (int)(N_out / 2 + 1);
  p.B_rot = (int)B_rot;
  p.B_shift = grad_shift ? (int)B_shift : 1;
  p.ndim = 3;
  p.os = oversampling;
  if (cutoff < 0.f) {
    p.cut2 = -1;
  } else {
    const double c2 = (double)cutoff * (double)cutoff;
    p.cut2 = c2 > 9.0e18 ? (long long)9.0e18 : (long long)std::floor(c2);
  }
  p.inv_no = 1.0 / (double)N_out;
  p.img = reinterpret_cast<const float2*>(grad_out);
  p.proj = reinterpret_cast<const float2*>(out);
  p.jac = reinterpret_cast<const float2*>(jac);
  p.grad_rot = grad_rot;
  p.grad_shift = grad_shift;
  const hipStream_t s = (hipStream_t)stream;
  if (grad_rot && tp::launch_zero(grad_rot, (size_t)p.B_rot * p.P * 9 * sizeof(float), s) != hipSuccess)
    return TP_EHIP;
  if (grad_shift && tp::launch_zero(grad_shift, (size_t)p.B_shift * p.P * 3 * sizeof(float), s) != hipSuccess)
    return TP_EHIP;
  return hip_status(tp::launch_rotate_grad_jac(p, s));
}

}  // extern "C"
