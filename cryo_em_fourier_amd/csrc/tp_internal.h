// Host-side interface between the C ABI (tp_api.hip) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tp {

// Everything a kernel needs for one call; passed by value.
struct OpParams {
  const float2* ref;      // reference [B, N, N, N/2+1] or [B, N, N/2+1] (forward, gradient)
  float2* ref_out;        // adjoint output, same shape
  const float2* img;      // projections [B, P, No, No/2+1] (adjoint input, gradient's G)
  float2* img_out;        // forward output
  const float* rot;       // [B_rot, P, d, d]
  const float* shift;     // [B_shift, P, 2] or nullptr
  float* grad_rot;        // [B_rot, P, d, d] or nullptr
  float* grad_shift;      // [B_shift, P, 2] or nullptr
  const float* wimg;      // real weights [B, P, No, No/2+1] (weight backprojection)
  float* wref_out;        // real weight volume, the reference's shape
  const float2* proj;     // saved forward output (pose gradients from a Jacobian)
  const float2* jac;      // saved Jacobian [B, P, 3, No, Wo]
  float2* jac_out;        // Jacobian output of the saving forward
  int B, P, N, No, Wo, B_rot, B_shift, ndim;
  float os;
  long long cut2;         // keep kx^2+ky^2 <= cut2; -1: keep everything
  uint32_t ref_bytes;     // bytes of one reference entry
  long long ref_elems;    // complex elements of one reference entry
  double inv_no;          // 1 / No
  int tiles_x, tiles_y, tiles_per_pose;
  int tile_y;             // ky-rows per tile (kTileY, or kTileYPairs for the paired 3D kernels)
  uint32_t nblocks;
  uint32_t nblocks2;      // workgroups of the two-tile pose-gradient kernel (tile rows taken in pairs)
};

// Brick decomposition of the adjoint (tp_adjoint.hip).
struct BrickParams {
  int nb[3];          // bricks along x, y, z
  int nbricks;
  int cmax;           // pose-chunk slots per brick (grid y)
  int pmax;           // target poses per chunk
};

// Output tile of one workgroup: kTileX kx-columns x kTileY ky-rows with one
// lane per output (2D kernels), or kTileXPairs x kTileYPairs with two lanes
// per output (3D kernels: a wave covers 8 kx x 4 rows, whose sample points
// share more cache lines than a 16 x 2 strip; measured 5 % faster).
constexpr int kTileX = 16;
constexpr int kTileY = 16;
constexpr int kTileXPairs = 8;
constexpr int kTileYPairs = 16;

hipError_t launch_project(const OpParams& p, int interp, hipStream_t s);
hipError_t launch_backproject(const OpParams& p, int interp, hipStream_t s);
hipError_t launch_backproject_weights(const OpParams& p, int interp, hipStream_t s);
hipError_t launch_symmetrize_x0(float2* ref, int ndim, int B, int N, hipStream_t s);
// 3D -> 3D rotation (tp_rotate.hip): what = 0 forward, 2 pose gradients;
// its adjoint is the brick adjoint over volume lattices (tp_adjoint.hip)
hipError_t launch_rotate(const OpParams& p, int interp, int what, hipStream_t s);
hipError_t launch_rotate_adjoint(const OpParams& p, int interp, hipStream_t s);
// the rotation that saves its Jacobian, and the pose gradients from it
hipError_t launch_rotate_jac(const OpParams& p, int interp, hipStream_t s);
hipError_t launch_rotate_grad_jac(const OpParams& p, hipStream_t s);
uint64_t rotate_adjoint_blocks(const OpParams& p);
// the rotation's adjoint and its pose gradients from a saved Jacobian in one launch
hipError_t launch_rotate_backward_jac(const OpParams& p, int interp, hipStream_t s);
uint64_t rotate_backward_jac_blocks(const OpParams& p);
constexpr int64_t kMaxRotateAdjointOut = 1023;  // 10-bit lattice offsets
hipError_t launch_grad_pose(const OpParams& p, int interp, hipStream_t s);
// 3D forward that saves the Jacobian of each output w.r.t. its sample point,
// and the pose gradients from it (one workgroup per (batch, pose))
hipError_t launch_project_jac(const OpParams& p, int interp, hipStream_t s);
hipError_t launch_grad_jac(const OpParams& p, hipStream_t s);
// the adjoint with the pose gradients from a saved Jacobian in the same launch
hipError_t launch_backward_jac(const OpParams& p, int interp, hipStream_t s);
uint64_t backward_jac_blocks(const OpParams& p);
hipError_t launch_zero(void* ptr, size_t bytes, hipStream_t s);
uint64_t adjoint_blocks(const OpParams& p);

// Largest output box of the brick kernels (14-bit lattice offsets).
constexpr int64_t kMaxBrickOut = (1 << 14) - 1;

}  // namespace tp
