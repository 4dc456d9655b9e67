/*
 * tp.h -- C ABI of the MI355X differentiable Fourier-space slice projector.
 *
 * The operations follow the technical summaries of "torch-projectors: A
 * High-Performance Differentiable Projection Library for PyTorch"
 * (gist.science pages in it/de/ja/ko/ar):
 *   - forward projection 3D->2D and 2D->2D: every output frequency of a 2D
 *     rfft image is rotated into the reference's rfft half-spectrum,
 *     interpolated there and multiplied by a shift phase (tech. section 2 of
 *     every page; Fourier slice theorem, tech. section 1);
 *   - backprojection: the exact adjoint of the forward (ko page tech. section
 *     2), which is also the gradient w.r.t. the reference;
 *   - analytic gradients w.r.t. the rotation matrices and shift vectors (ar
 *     page tech. section 2, de page tech. section 3).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Layout.  Complex tensors are interleaved float pairs (re, im), i.e. the
 *   memory of a contiguous torch.complex64 tensor, in PyTorch/FFTW rfft layout
 *   (pages, tech. section 2: the RFFT format is kept through every op):
 *     3D reference  [B, N, N, N/2+1]  (z, y, x), x = halved last axis
 *     2D reference  [B, N, N/2+1]     (y, x)
 *     projections   [B, P, N_out, N_out/2+1]
 *   Index i of a full axis of length n holds the signed frequency
 *   i if i <= (n-1)/2 else i-n; the halved axis holds 0..n/2.
 * Poses.  rot is float32 [B_rot, P, d, d] (d = 3 or 2), row-major, with
 *   B_rot in {1, B} (1 = the same P poses for every batch entry).  An output
 *   frequency (kx, ky) samples the reference at
 *     p = oversampling * (kx * rot[0,:] + ky * rot[1,:])   (x, y[, z] order),
 *   i.e. p = os * R^T (kx, ky[, 0]): the reference rotated by R is projected
 *   along z (ko page tech. section 2: coordinates through the inverse of the
 *   rotation).  Rows beyond the first two are not read.
 *   shift is float32 [B_shift, P, 2] = (s_x, s_y) in output pixels, or NULL
 *   for no shift; B_shift in {1, B}.  The output is multiplied by
 *   exp(-2 pi i (kx s_x + ky s_y) / N_out) (de/ar pages tech. section 2).
 * Friedel.  A tap with x < 0 reads conj(ref[-t]) (F(-k) = conj F(k), every
 *   page tech. section 2).  Taps with x = 0 read the stored entry as it is.
 *   Taps outside the stored range read 0.  Sample points with a component
 *   beyond +-2^30 or not finite read 0.
 * Interpolation.  interp = TP_LINEAR (2 taps per axis: 4 in 2D, 8 in 3D) or
 *   TP_CUBIC (Catmull-Rom / Keys a = -0.5, 4 taps per axis: 16 in 2D, 64 in
 *   3D) (every page tech. section 2).
 * Oversampling.  oversampling > 0 scales p; the reference spectrum is that of
 *   a box zero-padded by the caller to os*N_out (centred, then ifftshift,
 *   then rfftn).  The library does no padding and no FFT.
 * Cutoff.  Outputs with kx^2 + ky^2 > cutoff^2 are 0 and take no part in the
 *   adjoint or the gradients; cutoff < 0 disables it.
 * Ownership.  Every pointer is a device pointer owned by the caller; inputs
 *   must be 8-byte aligned, contiguous and must not alias outputs.  The
 *   library allocates nothing and keeps no state between calls.
 * Writes.  Outputs are overwritten (the adjoint and the gradients clear their
 *   outputs on the stream before accumulating into them).
 * Streams.  stream is a hipStream_t (NULL = default stream); every call is
 *   asynchronous on it and may be issued from several host threads.
 * Errors.  Arguments are checked before anything is launched:
 *   TP_EINVAL        null pointer, non-positive size, misaligned pointer,
 *                    bad interp, oversampling <= 0 or not finite, cutoff NaN,
 *                    B_rot or B_shift not in {1, B}, ndim not in {2, 3};
 *   TP_EUNSUPPORTED  a reference entry larger than 2^31 - 4096 bytes, a box
 *                    above 65535, a launch grid above 2^31 - 1 blocks, or,
 *                    for the adjoints, N_out above 16383 or B above 65535;
 *   TP_EHIP          the HIP runtime reported an error at launch.
 *   Nothing is thrown across the ABI.
 * Results.  Forward and pose gradients are deterministic up to the order of
 *   float atomics that merge per-workgroup partial sums of the pose
 *   gradients.  The adjoint sums each brick's contributions exactly in
 *   int32 fixed point, one quantum per group of up to 16 poses (for
 *   oversampling >= 1 at most 2^-22 of the largest |re| + |im| of proj read
 *   by that group or the previous one), and merges the pose chunks of bricks
 *   near the origin with float atomics, so its last bits there may differ
 *   between runs.  A non-finite proj value makes the voxels its stencil
 *   reaches NaN (the rest of the adjoint is unaffected).
 */
#ifndef TP_H
#define TP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct { float re, im; } tp_c64; /* == torch.complex64 */

typedef enum { TP_LINEAR = 0, TP_CUBIC = 1 } tp_interp;

typedef enum {
  TP_OK = 0,
  TP_EINVAL = -1,
  TP_EUNSUPPORTED = -2,
  TP_EHIP = -3
} tp_status;

/* ABI version of this header (major * 100 + minor). */
#define TP_ABI_VERSION 101
int tp_abi_version(void);

/* Human-readable name of a status code (static string, never NULL). */
const char* tp_status_str(tp_status status);

/*
 * Forward 3D -> 2D (central slice): the projection of the rotated, shifted
 * reference is its central slice in Fourier space (Fourier slice theorem,
 * it/de pages tech. section 1; rotation, Friedel fold, interpolation and
 * shift phase as in tech. section 2 of every page).
 *   vol    [B, N, N, N/2+1] complex64, input
 *   rot    [B_rot, P, 3, 3] float32, input
 *   shift  [B_shift, P, 2] float32 or NULL, input
 *   out    [B, P, N_out, N_out/2+1] complex64, overwritten
 */
tp_status tp_project_3d(const tp_c64* vol, int64_t B, int64_t N,
                        const float* rot, int64_t B_rot, int64_t P,
                        const float* shift, int64_t B_shift,
                        int64_t N_out, tp_interp interp, float oversampling, float cutoff,
                        tp_c64* out, void* stream);

/*
 * Adjoint of tp_project_3d for the real inner product Re sum conj(a) b
 * (2D -> 3D backprojection; ko page tech. section 2: the backward pass is the
 * adjoint, accumulated with the conjugate phase; it page results: scatter
 * with atomic adds, the slow direction): every kept output c = conj(phase) * proj is
 * spread with the forward's interpolation weights onto the taps it was read
 * from; a folded tap (x < 0) receives conj(w c) at -t.
 *   proj     [B, P, N_out, N_out/2+1] complex64, input
 *   vol_out  [B, N, N, N/2+1] complex64, overwritten
 */
tp_status tp_backproject_3d(const tp_c64* proj, int64_t B, int64_t P, int64_t N_out,
                            const float* rot, int64_t B_rot,
                            const float* shift, int64_t B_shift,
                            int64_t N, tp_interp interp, float oversampling, float cutoff,
                            tp_c64* vol_out, void* stream);

/*
 * Forward 2D -> 2D (rotated, shifted copy of a 2D reference; the 2D variant
 * of the operations list, it/ko pages tech. section 2).
 *   img    [B, N, N/2+1] complex64, input
 *   rot    [B_rot, P, 2, 2] float32, input
 *   out    [B, P, N_out, N_out/2+1] complex64, overwritten
 */
tp_status tp_project_2d(const tp_c64* img, int64_t B, int64_t N,
                        const float* rot, int64_t B_rot, int64_t P,
                        const float* shift, int64_t B_shift,
                        int64_t N_out, tp_interp interp, float oversampling, float cutoff,
                        tp_c64* out, void* stream);

/* Adjoint of tp_project_2d (ko page tech. section 2, as tp_backproject_3d);
 * img_out [B, N, N/2+1] is overwritten. */
tp_status tp_backproject_2d(const tp_c64* proj, int64_t B, int64_t P, int64_t N_out,
                            const float* rot, int64_t B_rot,
                            const float* shift, int64_t B_shift,
                            int64_t N, tp_interp interp, float oversampling, float cutoff,
                            tp_c64* img_out, void* stream);

/*
 * Weight backprojection (the second, real volume of a dual-volume
 * reconstruction: per-frequency weights such as CTF^2 spread with the same
 * interpolation weights as the adjoint, for normalisation or Wiener-style
 * deconvolution; it/de/ar pages tech. section 2).  Real weights carry no
 * phase, so there is no shift; a folded tap (x < 0) adds w * weight at -t.
 * It is the adjoint of the real-valued forward (interpolation of a real
 * volume at the sample points, folded taps unconjugated).
 *   weights  [B, P, N_out, N_out/2+1] float32, input
 *   rot      [B_rot, P, 3, 3] (3D) or [B_rot, P, 2, 2] (2D) float32
 *   wvol_out [B, N, N, N/2+1] (3D) or wimg_out [B, N, N/2+1] (2D) float32,
 *            overwritten
 * Limits and errors as tp_backproject_3d; pointers need 4-byte alignment.
 */
tp_status tp_backproject_weights_3d(const float* weights, int64_t B, int64_t P, int64_t N_out,
                                    const float* rot, int64_t B_rot, int64_t N, tp_interp interp,
                                    float oversampling, float cutoff, float* wvol_out, void* stream);
tp_status tp_backproject_weights_2d(const float* weights, int64_t B, int64_t P, int64_t N_out,
                                    const float* rot, int64_t B_rot, int64_t N, tp_interp interp,
                                    float oversampling, float cutoff, float* wimg_out, void* stream);

/*
 * Hermitian symmetrisation of the x = 0 plane of an rfft half-spectrum, in
 * place: V(0, y, z) <- (V(0, y, z) + conj V(0, -y, -z)) / 2 with indices mod
 * N (entries that are their own mirror keep their real part); other planes
 * are untouched.  The alternative treatment of the zero-frequency axis in
 * the backward pass (de page tech. section 2: no double counting on that
 * axis; ar page tech. section 2: symmetric accumulation there), offered as a
 * step after tp_backproject_*.  It is R-linear and self-adjoint.
 *   ref  [B, N, N, N/2+1] (ndim 3) or [B, N, N/2+1] (ndim 2) complex64
 * Errors: TP_EINVAL for ndim not in {2, 3}, a null or misaligned pointer or
 * a non-positive size; TP_EUNSUPPORTED for N above 65535.
 */
tp_status tp_symmetrize_x0(int ndim, tp_c64* ref, int64_t B, int64_t N, void* stream);

/*
 * 3D -> 3D rotation of a reference half-spectrum (subtomogram averaging; it
 * page tech. section 2, list of operations: 3D -> 3D for general
 * rotations).  Every output frequency k = (kx, ky, kz) of an
 * [N_out, N_out, N_out/2+1] half-spectrum samples the reference at
 *   p = oversampling * (kx rot[0,:] + ky rot[1,:] + kz rot[2,:])
 * with the central slice's fold, kernels and out-of-range rules (the kz = 0
 * plane of the output is tp_project_3d's slice), times
 * exp(-2 pi i (kx s_x + ky s_y + kz s_z) / N_out), and is 0 outside the
 * sphere kx^2 + ky^2 + kz^2 <= cutoff^2 (cutoff < 0: none).
 *   vol    [B, N, N, N/2+1] complex64, input
 *   rot    [B_rot, P, 3, 3] float32
 *   shift  [B_shift, P, 3] float32 (s_x, s_y, s_z in output voxels) or NULL
 *   out    [B, P, N_out, N_out, N_out/2+1] complex64, overwritten
 * Errors as tp_project_3d (the grid counts 8 x 16 output tiles of the
 * N_out^2 (kz, ky) rows).
 */
tp_status tp_rotate_3d(const tp_c64* vol, int64_t B, int64_t N, const float* rot, int64_t B_rot, int64_t P,
                       const float* shift, int64_t B_shift, int64_t N_out, tp_interp interp, float oversampling,
                       float cutoff, tp_c64* out, void* stream);

/*
 * Adjoint of tp_rotate_3d for Re sum conj(a) b: every kept output
 * c = conj(phase) * grad_out is spread with the forward's weights onto its
 * taps (a folded tap receives conj(w c) at -t), accumulated per brick of the
 * reference like tp_backproject_3d.
 *   grad_out [B, P, N_out, N_out, N_out/2+1] complex64, input
 *   vol_out  [B, N, N, N/2+1] complex64, overwritten
 * Errors as tp_backproject_3d, with N_out limited to 1023.
 */
tp_status tp_rotate_backproject_3d(const tp_c64* grad_out, int64_t B, int64_t P, int64_t N_out, const float* rot,
                                   int64_t B_rot, const float* shift, int64_t B_shift, int64_t N, tp_interp interp,
                                   float oversampling, float cutoff, tp_c64* vol_out, void* stream);

/*
 * Gradients of L = Re sum conj(grad_out) * rotate(vol, rot, shift):
 *   dL/dR[i][j] = os sum_k k_i Re(conj(G) phase dS/dp_j)  (all three rows)
 *   dL/ds_j     = sum_k (2 pi k_j / N_out) Im(conj(G) phase S)
 *   grad_rot [B_rot, P, 3, 3] float32, overwritten, or NULL
 *   grad_shift [B_shift, P, 3] float32, overwritten, or NULL (with
 *              shift == NULL the shift is 0 and B_shift rows are kept)
 */
tp_status tp_rotate_grad_pose(const tp_c64* vol, int64_t B, int64_t N, const tp_c64* grad_out, const float* rot,
                              int64_t B_rot, int64_t P, const float* shift, int64_t B_shift, int64_t N_out,
                              tp_interp interp, float oversampling, float cutoff, float* grad_rot, float* grad_shift,
                              void* stream);

/*
 * Gradients of L = Re sum conj(grad_out) * project(ref, rot, shift) w.r.t.
 * the rotations and the shifts (ndim = 3: tp_project_3d, ndim = 2:
 * tp_project_2d), by the chain rule through the interpolation kernel's
 * derivative (ar page tech. section 2):
 *   dL/dR[i][j] = os * sum_k k_i Re(conj(G) phase dS/dp_j)   (i = 0: kx, 1: ky)
 *   dL/ds_j     = sum_k Re(conj(G) (-2 pi i k_j / N_out) phase S)
 * The last row of dL/dR is 0 in 3D.  With B_rot = 1 (or B_shift = 1) and
 * B > 1 the gradient is summed over the batch.
 *   ref       [B, N, N, N/2+1] (3D) or [B, N, N/2+1] (2D) complex64, input
 *   grad_out  [B, P, N_out, N_out/2+1] complex64, input
 *   grad_rot  [B_rot, P, ndim, ndim] float32, overwritten, or NULL to skip
 *   grad_shift[B_shift, P, 2] float32, overwritten, or NULL to skip
 *             (with shift == NULL the shift is 0 and grad_shift still has
 *             B_shift rows, B_shift in {1, B})
 */
tp_status tp_grad_pose(int ndim, const tp_c64* ref, int64_t B, int64_t N,
                       const tp_c64* grad_out, const float* rot, int64_t B_rot, int64_t P,
                       const float* shift, int64_t B_shift,
                       int64_t N_out, tp_interp interp, float oversampling, float cutoff,
                       float* grad_rot, float* grad_shift, void* stream);

/*
 * The backward of tp_project_3d in one call, storing nothing between the
 * forward and the backward (it page tech. section 3: no intermediate
 * tensors): for L = Re sum conj(grad_out) * project_3d(vol, rot, shift),
 *   vol_grad   = dL/dvol, the adjoint of tp_backproject_3d applied to
 *                grad_out (ko page tech. section 2: the backward is the
 *                adjoint; conjugate phase)
 *   grad_rot, grad_shift = the rotation and shift gradients of tp_grad_pose
 *                (ar page tech. section 2: chain rule through the
 *                interpolation kernel's derivative)
 * It runs tp_backproject_3d's and tp_grad_pose's kernels on the stream,
 * one after the other, and its results are those of the two calls (the
 * adjoint's fixed point as tp_backproject_3d; gradient sums merged with
 * float atomics).
 *   vol        [B, N, N, N/2+1] complex64, input (the forward's reference)
 *   grad_out   [B, P, N_out, N_out/2+1] complex64, input
 *   rot, shift as tp_project_3d
 *   vol_grad   [B, N, N, N/2+1] complex64, overwritten, or NULL to skip
 *   grad_rot   [B_rot, P, 3, 3] float32, overwritten (last row 0), or NULL
 *   grad_shift [B_shift, P, 2] float32, overwritten, or NULL (with shift ==
 *              NULL the shift is 0 and grad_shift still has B_shift rows)
 * With vol_grad NULL this is tp_grad_pose (ndim 3), with both gradients
 * NULL tp_backproject_3d.  Errors as tp_backproject_3d and tp_grad_pose.
 */
tp_status tp_backward_3d(const tp_c64* vol, int64_t B, int64_t N, const tp_c64* grad_out,
                         const float* rot, int64_t B_rot, int64_t P,
                         const float* shift, int64_t B_shift, int64_t N_out,
                         tp_interp interp, float oversampling, float cutoff,
                         tp_c64* vol_grad, float* grad_rot, float* grad_shift, void* stream);

/*
 * Forward 3D -> 2D that also saves what the pose gradients need, so that
 * they take one streaming pass instead of a second pass of gathers over the
 * reference (the analytic gradients of the ar page tech. section 2, by the
 * same chain rule as tp_grad_pose):
 *   out  [B, P, N_out, N_out/2+1] complex64, overwritten: the values of
 *        tp_project_3d for the same arguments (same arithmetic up to the
 *        order of float additions)
 *   jac  [B, P, 3, N_out, N_out/2+1] complex64, overwritten: for each
 *        output, phase * dS/dp_j (j = x, y, z), the derivative of the output
 *        with respect to its sample point p in reference index units; 0
 *        outside the cutoff and where the output reads 0
 * Other arguments and errors as tp_project_3d.
 */
tp_status tp_project_3d_jac(const tp_c64* vol, int64_t B, int64_t N,
                            const float* rot, int64_t B_rot, int64_t P,
                            const float* shift, int64_t B_shift,
                            int64_t N_out, tp_interp interp, float oversampling, float cutoff,
                            tp_c64* out, tp_c64* jac, void* stream);

/*
 * Pose gradients of L = Re sum conj(grad_out) * project_3d(...) from the
 * saved out and jac of tp_project_3d_jac (same B, P, N_out, oversampling and
 * cutoff; B_rot and B_shift as that call's):
 *   dL/dR[i][j] = os * sum_k k_i Re(conj(G) jac_j)       (i = 0: kx, 1: ky)
 *   dL/ds_j     = (2 pi / N_out) sum_k k_j Im(conj(G) out)
 * the values of tp_grad_pose (ndim = 3) for that call, without reading the
 * reference.  Only outputs inside the cutoff are read.
 *   grad_out   [B, P, N_out, N_out/2+1] complex64, input
 *   proj, jac  the outputs of tp_project_3d_jac, input
 *   grad_rot   [B_rot, P, 3, 3] float32, overwritten (last row 0), or NULL
 *   grad_shift [B_shift, P, 2] float32, overwritten, or NULL
 * Errors: TP_EINVAL for null or misaligned buffers, sizes <= 0, B_rot or
 * B_shift not in {1, B}, a bad oversampling or a NaN cutoff;
 * TP_EUNSUPPORTED for N_out above 65535 or B * P above 2^31 - 1.
 */
tp_status tp_grad_pose_jac(const tp_c64* grad_out, const tp_c64* proj, const tp_c64* jac,
                           int64_t B, int64_t P, int64_t N_out, int64_t B_rot, int64_t B_shift,
                           float oversampling, float cutoff,
                           float* grad_rot, float* grad_shift, void* stream);

/*
 * The backward of tp_project_3d_jac in one launch: the adjoint of
 * tp_backproject_3d and the pose gradients of tp_grad_pose_jac, whose
 * streaming reduction runs on workgroups placed after the adjoint's bricks,
 * so that they fill the CUs the bricks leave idle at the end.  The adjoint
 * is the exact adjoint of the forward (ko page tech. section 2), the
 * gradients the analytic ones of the ar page tech. section 2.
 *   grad_out   [B, P, N_out, N_out/2+1] complex64, input
 *   proj, jac  the outputs of tp_project_3d_jac for the same arguments, input
 *   vol_out    [B, N, N, N/2+1] complex64, overwritten: tp_backproject_3d's
 *   grad_rot   [B_rot, P, 3, 3] float32, overwritten (last row 0), or NULL
 *   grad_shift [B_shift, P, 2] float32, overwritten, or NULL (with shift ==
 *              NULL the shift is 0 and grad_shift still has B_shift rows)
 * With both gradients NULL this is tp_backproject_3d.  Other arguments and
 * errors as tp_backproject_3d and tp_grad_pose_jac.
 */
tp_status tp_backward_3d_jac(const tp_c64* grad_out, const tp_c64* proj, const tp_c64* jac,
                             int64_t B, int64_t P, int64_t N_out,
                             const float* rot, int64_t B_rot, const float* shift, int64_t B_shift,
                             int64_t N, tp_interp interp, float oversampling, float cutoff,
                             tp_c64* vol_out, float* grad_rot, float* grad_shift, void* stream);

/*
 * 3D -> 3D rotation that also saves, for its pose gradients, the Jacobian of
 * every output with respect to its sample point (the rotation's counterpart
 * of tp_project_3d_jac; same chain rule as tp_rotate_grad_pose):
 *   out  [B, P, N_out, N_out, N_out/2+1] complex64, overwritten: the values
 *        of tp_rotate_3d for the same arguments
 *   jac  [B, P, 3, N_out, N_out, N_out/2+1] complex64, overwritten:
 *        phase * dS/dp_j (j = x, y, z) per output; 0 outside the sphere and
 *        where the output reads 0
 * Other arguments and errors as tp_rotate_3d; N_out above 1023 is
 * TP_EUNSUPPORTED.
 */
tp_status tp_rotate_3d_jac(const tp_c64* vol, int64_t B, int64_t N, const float* rot, int64_t B_rot, int64_t P,
                           const float* shift, int64_t B_shift, int64_t N_out, tp_interp interp, float oversampling,
                           float cutoff, tp_c64* out, tp_c64* jac, void* stream);

/*
 * Pose gradients of L = Re sum conj(grad_out) * rotate_3d(...) from the
 * saved out and jac of tp_rotate_3d_jac (same B, P, N_out, oversampling and
 * cutoff; B_rot and B_shift as that call's):
 *   dL/dR[i][j] = os * sum_k k_i Re(conj(G) jac_j)     (i, j = x, y, z)
 *   dL/ds_j     = (2 pi / N_out) sum_k k_j Im(conj(G) out)
 * the values of tp_rotate_grad_pose for that call, without reading the
 * reference.  Only outputs inside the sphere are read.
 *   grad_rot   [B_rot, P, 3, 3] float32, overwritten, or NULL
 *   grad_shift [B_shift, P, 3] float32, overwritten, or NULL
 * Errors as tp_grad_pose_jac; N_out above 1023 is TP_EUNSUPPORTED.
 */
tp_status tp_rotate_grad_pose_jac(const tp_c64* grad_out, const tp_c64* out, const tp_c64* jac, int64_t B,
                                  int64_t P, int64_t N_out, int64_t B_rot, int64_t B_shift, float oversampling,
                                  float cutoff, float* grad_rot, float* grad_shift, void* stream);

/*
 * The backward of tp_rotate_3d_jac in one launch (the rotation's counterpart
 * of tp_backward_3d_jac): the adjoint of tp_rotate_backproject_3d and the
 * pose gradients of tp_rotate_grad_pose_jac, whose streaming reduction runs
 * on workgroups after the adjoint's bricks.
 *   grad_out   [B, P, N_out, N_out, N_out/2+1] complex64, input
 *   out, jac   the outputs of tp_rotate_3d_jac for the same arguments, input
 *   vol_out    [B, N, N, N/2+1] complex64, overwritten
 *   grad_rot   [B_rot, P, 3, 3] float32, overwritten, or NULL
 *   grad_shift [B_shift, P, 3] float32, overwritten, or NULL (with shift ==
 *              NULL the shift is 0 and grad_shift still has B_shift rows)
 * With both gradients NULL this is tp_rotate_backproject_3d.  Other
 * arguments and errors as tp_rotate_backproject_3d and
 * tp_rotate_grad_pose_jac.
 */
tp_status tp_rotate_backward_3d_jac(const tp_c64* grad_out, const tp_c64* out, const tp_c64* jac,
                                    int64_t B, int64_t P, int64_t N_out,
                                    const float* rot, int64_t B_rot, const float* shift, int64_t B_shift,
                                    int64_t N, tp_interp interp, float oversampling, float cutoff,
                                    tp_c64* vol_out, float* grad_rot, float* grad_shift, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* TP_H */
