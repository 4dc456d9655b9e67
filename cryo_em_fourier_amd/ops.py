"""PyTorch-facing binding of the projector.

``tp_project_3d``, ``tp_backproject_3d``, ``tp_project_2d``,
``tp_backproject_2d``, ``tp_grad_pose``, ``tp_backproject_weights_3d``,
``tp_backproject_weights_2d`` and ``tp_symmetrize_x0`` mirror the C ABI of
the same names (include/tp.h) on device tensors: they check shapes, allocate
outputs with torch and pass raw pointers and the current HIP stream.

Differentiable forms (torch.autograd.Function; pages, tech. section 2:
autograd functions wrapping the native ops):

* ``project_3d`` / ``project_2d``: the backward computes the reference
  gradient (the adjoint) and the rotation and shift gradients, each only
  when needed; in 3D both together come from one ``tp_backward_3d`` call.
  Nothing is kept from the forward but its inputs (it page tech. section 3:
  no intermediate tensors).  ``project_3d(save_jacobian=True)`` opts into a forward
  (``tp_project_3d_jac``) that also saves each output's Jacobian with
  respect to its sample point (3 complex values per output, 24 bytes), which
  the backward then streams instead of gathering from the reference again.
* ``backproject_3d`` / ``backproject_2d``: backprojection as an op of its
  own (2D -> 3D; it page tech. section 2, list of operations), optionally
  with the x = 0 plane symmetrised.  Its backward is the forward projection
  (gradient to the projections) and ``tp_grad_pose`` with the reference and
  upstream roles swapped (Re<Y, P^T G> = Re<P Y, G>).
* ``rotate_3d``: the 3D -> 3D rotation of a half-spectrum (it page tech.
  section 2: 3D -> 3D for general rotations), with gradients to the
  reference (its adjoint), the rotations and the 3-vector shifts (from a
  Jacobian saved by the forward, as ``project_3d``).
* ``backproject_weights_3d`` / ``backproject_weights_2d``: the real weight
  volume of a dual-volume reconstruction, with gradients to the weights
  (the real forward projection) and to the rotations (ar page tech. section
  2: optional gradients through the weight components).
"""
from __future__ import annotations

import torch

from . import _lib

_INTERP = {"linear": _lib.TP_LINEAR, "cubic": _lib.TP_CUBIC,
           _lib.TP_LINEAR: _lib.TP_LINEAR, _lib.TP_CUBIC: _lib.TP_CUBIC}


def _interp(x) -> int:
    try:
        return _INTERP[x]
    except KeyError:
        raise ValueError(f"interp must be 'linear' or 'cubic', got {x!r}") from None


def _stream(dev: torch.device) -> int:
    return torch.cuda.current_stream(dev).cuda_stream


def _need(t: torch.Tensor, name: str, dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor (no CPU path)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _ref_dims(ref: torch.Tensor, ndim: int, name: str):
    _need(ref, name, torch.complex64, ndim + 1)
    B, N = ref.shape[0], ref.shape[1]
    want = (B,) + (N,) * (ndim - 1) + (N // 2 + 1,)
    if tuple(ref.shape) != want:
        raise ValueError(f"{name} must be a square/cubic rfft half-spectrum {want}, got {tuple(ref.shape)}")
    return B, N


def _pose_dims(rot, shift, ndim, B, dev):
    _need(rot, "rot", torch.float32, 4)
    B_rot, P = rot.shape[0], rot.shape[1]
    if tuple(rot.shape[2:]) != (ndim, ndim):
        raise ValueError(f"rot must be [B_rot, P, {ndim}, {ndim}], got {tuple(rot.shape)}")
    if B_rot not in (1, B):
        raise ValueError(f"rot batch {B_rot} must be 1 or {B}")
    if rot.device != dev:
        raise ValueError("rot is on another device")
    B_shift = 1
    if shift is not None:
        _need(shift, "shift", torch.float32, 3)
        B_shift = shift.shape[0]
        if tuple(shift.shape[1:]) != (P, 2) or B_shift not in (1, B):
            raise ValueError(f"shift must be [1 or {B}, {P}, 2], got {tuple(shift.shape)}")
        if shift.device != dev:
            raise ValueError("shift is on another device")
    return B_rot, P, B_shift


def _ptr(t):
    return None if t is None else t.data_ptr()


def _project(ndim, ref, rot, shift, n_out, interp, oversampling, cutoff):
    B, N = _ref_dims(ref, ndim, "reference")
    B_rot, P, B_shift = _pose_dims(rot, shift, ndim, B, ref.device)
    if n_out is None:
        n_out = int(round(N / float(oversampling)))
    out = torch.empty((B, P, n_out, n_out // 2 + 1), dtype=torch.complex64, device=ref.device)
    fn = _lib.lib().tp_project_3d if ndim == 3 else _lib.lib().tp_project_2d
    st = fn(ref.data_ptr(), B, N, rot.data_ptr(), B_rot, P, _ptr(shift), B_shift, n_out,
            _interp(interp), float(oversampling), float(cutoff), out.data_ptr(), _stream(ref.device))
    _lib.check(st, f"tp_project_{ndim}d")
    return out


def _backproject(ndim, proj, rot, shift, N, interp, oversampling, cutoff):
    _need(proj, "proj", torch.complex64, 4)
    B, P, n_out = proj.shape[0], proj.shape[1], proj.shape[2]
    if proj.shape[3] != n_out // 2 + 1:
        raise ValueError(f"proj must be [B, P, n, n//2+1], got {tuple(proj.shape)}")
    B_rot, P2, B_shift = _pose_dims(rot, shift, ndim, B, proj.device)
    if P2 != P:
        raise ValueError(f"rot has {P2} poses, proj has {P}")
    shape = (B,) + (N,) * (ndim - 1) + (N // 2 + 1,)
    out = torch.empty(shape, dtype=torch.complex64, device=proj.device)
    fn = _lib.lib().tp_backproject_3d if ndim == 3 else _lib.lib().tp_backproject_2d
    st = fn(proj.data_ptr(), B, P, n_out, rot.data_ptr(), B_rot, _ptr(shift), B_shift, N,
            _interp(interp), float(oversampling), float(cutoff), out.data_ptr(), _stream(proj.device))
    _lib.check(st, f"tp_backproject_{ndim}d")
    return out


def tp_project_3d(vol, rot, shift=None, n_out=None, interp="cubic", oversampling=1.0, cutoff=-1.0):
    """vol [B,N,N,N//2+1] c64, rot [B_rot,P,3,3] f32, shift [B_shift,P,2] f32 or None
    -> [B,P,n_out,n_out//2+1] c64 (n_out defaults to round(N / oversampling))."""
    return _project(3, vol, rot, shift, n_out, interp, oversampling, cutoff)


def tp_project_2d(img, rot, shift=None, n_out=None, interp="cubic", oversampling=1.0, cutoff=-1.0):
    """img [B,N,N//2+1] c64, rot [B_rot,P,2,2] f32 -> [B,P,n_out,n_out//2+1] c64."""
    return _project(2, img, rot, shift, n_out, interp, oversampling, cutoff)


def tp_backproject_3d(proj, rot, shift=None, N=None, interp="cubic", oversampling=1.0, cutoff=-1.0):
    """Adjoint of tp_project_3d: proj [B,P,n,n//2+1] -> [B,N,N,N//2+1]."""
    if N is None:
        N = int(round(proj.shape[2] * float(oversampling)))
    return _backproject(3, proj, rot, shift, N, interp, oversampling, cutoff)


def tp_backproject_2d(proj, rot, shift=None, N=None, interp="cubic", oversampling=1.0, cutoff=-1.0):
    """Adjoint of tp_project_2d: proj [B,P,n,n//2+1] -> [B,N,N//2+1]."""
    if N is None:
        N = int(round(proj.shape[2] * float(oversampling)))
    return _backproject(2, proj, rot, shift, N, interp, oversampling, cutoff)


def tp_grad_pose(ref, grad_out, rot, shift=None, interp="cubic", oversampling=1.0, cutoff=-1.0,
                 want_rot=True, want_shift=True, B_shift=None):
    """Rotation and shift gradients of Re sum conj(grad_out) * project(ref, rot, shift).

    Returns (grad_rot or None, grad_shift or None); grad_rot has rot's shape,
    grad_shift has shift's shape (or [B_shift, P, 2] when shift is None)."""
    ndim = rot.shape[-1] if isinstance(rot, torch.Tensor) else 0
    if ndim not in (2, 3):
        raise ValueError("rot must be [B_rot, P, d, d] with d = 2 or 3")
    B, N = _ref_dims(ref, ndim, "reference")
    B_rot, P, Bs = _pose_dims(rot, shift, ndim, B, ref.device)
    _need(grad_out, "grad_out", torch.complex64, 4)
    if grad_out.shape[0] != B or grad_out.shape[1] != P or grad_out.shape[3] != grad_out.shape[2] // 2 + 1:
        raise ValueError(f"grad_out must be [{B}, {P}, n, n//2+1], got {tuple(grad_out.shape)}")
    n_out = grad_out.shape[2]
    if shift is None:
        Bs = 1 if B_shift is None else int(B_shift)
    gr = torch.empty_like(rot) if want_rot else None
    gs = torch.empty((Bs, P, 2), dtype=torch.float32, device=ref.device) if want_shift else None
    st = _lib.lib().tp_grad_pose(ndim, ref.data_ptr(), B, N, grad_out.data_ptr(), rot.data_ptr(),
                                 B_rot, P, _ptr(shift), Bs, n_out, _interp(interp),
                                 float(oversampling), float(cutoff), _ptr(gr), _ptr(gs),
                                 _stream(ref.device))
    _lib.check(st, "tp_grad_pose")
    return gr, gs


def tp_backward_3d(vol, grad_out, rot, shift=None, interp="cubic", oversampling=1.0, cutoff=-1.0,
                   want_vol=True, want_rot=True, want_shift=True, B_shift=None):
    """The backward of tp_project_3d in one call, storing nothing from the
    forward: (d_vol [B,N,N,N//2+1] or None, grad_rot [B_rot,P,3,3] or None,
    grad_shift or None), the values of tp_backproject_3d and tp_grad_pose."""
    B, N = _ref_dims(vol, 3, "reference")
    B_rot, P, Bs = _pose_dims(rot, shift, 3, B, vol.device)
    _need(grad_out, "grad_out", torch.complex64, 4)
    if grad_out.shape[0] != B or grad_out.shape[1] != P or grad_out.shape[3] != grad_out.shape[2] // 2 + 1:
        raise ValueError(f"grad_out must be [{B}, {P}, n, n//2+1], got {tuple(grad_out.shape)}")
    if grad_out.device != vol.device:
        raise ValueError("grad_out is on another device")
    n_out = grad_out.shape[2]
    if shift is None:
        Bs = 1 if B_shift is None else int(B_shift)
    dev = vol.device
    dv = torch.empty_like(vol) if want_vol else None
    gr = torch.empty_like(rot) if want_rot else None
    gs = torch.empty((Bs, P, 2), dtype=torch.float32, device=dev) if want_shift else None
    st = _lib.lib().tp_backward_3d(vol.data_ptr(), B, N, grad_out.data_ptr(), rot.data_ptr(), B_rot, P,
                                   _ptr(shift), Bs, n_out, _interp(interp), float(oversampling), float(cutoff),
                                   _ptr(dv), _ptr(gr), _ptr(gs), _stream(dev))
    _lib.check(st, "tp_backward_3d")
    return dv, gr, gs


def tp_project_3d_jac(vol, rot, shift=None, n_out=None, interp="cubic", oversampling=1.0, cutoff=-1.0):
    """tp_project_3d that also returns the Jacobian of each output w.r.t. its
    sample point: (out [B,P,n,n//2+1], jac [B,P,3,n,n//2+1]) c64."""
    B, N = _ref_dims(vol, 3, "reference")
    B_rot, P, B_shift = _pose_dims(rot, shift, 3, B, vol.device)
    if n_out is None:
        n_out = int(round(N / float(oversampling)))
    out = torch.empty((B, P, n_out, n_out // 2 + 1), dtype=torch.complex64, device=vol.device)
    jac = torch.empty((B, P, 3, n_out, n_out // 2 + 1), dtype=torch.complex64, device=vol.device)
    st = _lib.lib().tp_project_3d_jac(vol.data_ptr(), B, N, rot.data_ptr(), B_rot, P, _ptr(shift), B_shift,
                                      n_out, _interp(interp), float(oversampling), float(cutoff), out.data_ptr(),
                                      jac.data_ptr(), _stream(vol.device))
    _lib.check(st, "tp_project_3d_jac")
    return out, jac


def tp_grad_pose_jac(grad_out, proj, jac, B_rot=1, B_shift=1, oversampling=1.0, cutoff=-1.0,
                     want_rot=True, want_shift=True):
    """Pose gradients from tp_project_3d_jac's (proj, jac):
    (grad_rot [B_rot,P,3,3] or None, grad_shift [B_shift,P,2] or None)."""
    _need(grad_out, "grad_out", torch.complex64, 4)
    _need(proj, "proj", torch.complex64, 4)
    _need(jac, "jac", torch.complex64, 5)
    B, P, n_out = proj.shape[0], proj.shape[1], proj.shape[2]
    if tuple(proj.shape) != (B, P, n_out, n_out // 2 + 1) or grad_out.shape != proj.shape:
        raise ValueError(f"grad_out and proj must be [B, P, n, n//2+1], got {tuple(grad_out.shape)}, "
                         f"{tuple(proj.shape)}")
    if tuple(jac.shape) != (B, P, 3, n_out, n_out // 2 + 1):
        raise ValueError(f"jac must be [{B}, {P}, 3, {n_out}, {n_out // 2 + 1}], got {tuple(jac.shape)}")
    if grad_out.device != proj.device or jac.device != proj.device:
        raise ValueError("grad_out, proj and jac must be on one device")
    gr = torch.empty((B_rot, P, 3, 3), dtype=torch.float32, device=proj.device) if want_rot else None
    gs = torch.empty((B_shift, P, 2), dtype=torch.float32, device=proj.device) if want_shift else None
    st = _lib.lib().tp_grad_pose_jac(grad_out.data_ptr(), proj.data_ptr(), jac.data_ptr(), B, P, n_out,
                                     int(B_rot), int(B_shift), float(oversampling), float(cutoff), _ptr(gr),
                                     _ptr(gs), _stream(proj.device))
    _lib.check(st, "tp_grad_pose_jac")
    return gr, gs


def tp_backward_3d_jac(grad_out, proj, jac, rot, shift=None, N=None, interp="cubic", oversampling=1.0,
                       cutoff=-1.0, want_rot=True, want_shift=True, B_shift=None):
    """The backward of tp_project_3d_jac in one launch: (d_vol [B,N,N,N//2+1],
    grad_rot [B_rot,P,3,3] or None, grad_shift [B_shift,P,2] or None), the
    values of tp_backproject_3d and tp_grad_pose_jac."""
    _need(grad_out, "grad_out", torch.complex64, 4)
    _need(proj, "proj", torch.complex64, 4)
    _need(jac, "jac", torch.complex64, 5)
    B, P, n_out = proj.shape[0], proj.shape[1], proj.shape[2]
    if tuple(proj.shape) != (B, P, n_out, n_out // 2 + 1) or grad_out.shape != proj.shape:
        raise ValueError(f"grad_out and proj must be [B, P, n, n//2+1], got {tuple(grad_out.shape)}, "
                         f"{tuple(proj.shape)}")
    if tuple(jac.shape) != (B, P, 3, n_out, n_out // 2 + 1):
        raise ValueError(f"jac must be [{B}, {P}, 3, {n_out}, {n_out // 2 + 1}], got {tuple(jac.shape)}")
    if grad_out.device != proj.device or jac.device != proj.device:
        raise ValueError("grad_out, proj and jac must be on one device")
    B_rot, P2, Bs = _pose_dims(rot, shift, 3, B, proj.device)
    if P2 != P:
        raise ValueError(f"rot has {P2} poses, proj has {P}")
    if shift is None:
        Bs = 1 if B_shift is None else int(B_shift)
    if N is None:
        N = int(round(n_out * float(oversampling)))
    dev = proj.device
    vol = torch.empty((B, N, N, N // 2 + 1), dtype=torch.complex64, device=dev)
    gr = torch.empty((B_rot, P, 3, 3), dtype=torch.float32, device=dev) if want_rot else None
    gs = torch.empty((Bs, P, 2), dtype=torch.float32, device=dev) if want_shift else None
    st = _lib.lib().tp_backward_3d_jac(grad_out.data_ptr(), proj.data_ptr(), jac.data_ptr(), B, P, n_out,
                                       rot.data_ptr(), B_rot, _ptr(shift), Bs, int(N), _interp(interp),
                                       float(oversampling), float(cutoff), vol.data_ptr(), _ptr(gr), _ptr(gs),
                                       _stream(dev))
    _lib.check(st, "tp_backward_3d_jac")
    return vol, gr, gs


class _Project(torch.autograd.Function):
    @staticmethod
    def forward(ctx, ref, rot, shift, ndim, n_out, interp, oversampling, cutoff, save_jacobian):
        pose_grads = ctx.needs_input_grad[1] or (shift is not None and ctx.needs_input_grad[2])
        jac = None
        if ndim == 3 and save_jacobian and pose_grads:
            out, jac = tp_project_3d_jac(ref, rot, shift, n_out, interp, oversampling, cutoff)
            ctx.save_for_backward(ref, rot, shift, out, jac)
        else:
            out = _project(ndim, ref, rot, shift, n_out, interp, oversampling, cutoff)
            ctx.save_for_backward(ref, rot, shift)
        ctx.has_jac = jac is not None
        ctx.cfg = (ndim, interp, oversampling, cutoff)
        return out

    @staticmethod
    def backward(ctx, g):
        if ctx.has_jac:
            ref, rot, shift, out, jac = ctx.saved_tensors
        else:
            ref, rot, shift = ctx.saved_tensors
        ndim, interp, oversampling, cutoff = ctx.cfg
        g = g.contiguous()
        if g.dtype != torch.complex64:
            g = g.to(torch.complex64)
        d_ref = d_rot = d_shift = None
        want_rot = ctx.needs_input_grad[1]
        want_shift = shift is not None and ctx.needs_input_grad[2]
        if ctx.needs_input_grad[0] and (want_rot or want_shift) and ctx.has_jac:
            # both gradients from one launch
            d_ref, d_rot, d_shift = tp_backward_3d_jac(g, out, jac, rot, shift, ref.shape[1], interp,
                                                       oversampling, cutoff, want_rot, want_shift)
            return d_ref, d_rot, d_shift, None, None, None, None, None, None
        if ndim == 3 and ctx.needs_input_grad[0] and (want_rot or want_shift):
            # both gradients in one call (the adjoint, then the pose-gradient gather)
            d_ref, d_rot, d_shift = tp_backward_3d(ref, g, rot, shift, interp, oversampling, cutoff, True,
                                                   want_rot, want_shift)
            return d_ref, d_rot, d_shift, None, None, None, None, None, None
        if ctx.needs_input_grad[0]:
            d_ref = _backproject(ndim, g, rot, shift, ref.shape[1], interp, oversampling, cutoff)
        if (want_rot or want_shift) and ctx.has_jac:
            B_shift = shift.shape[0] if shift is not None else 1
            d_rot, d_shift = tp_grad_pose_jac(g, out, jac, rot.shape[0], B_shift, oversampling, cutoff,
                                              want_rot=want_rot, want_shift=want_shift)
        elif want_rot or want_shift:
            d_rot, d_shift = tp_grad_pose(ref, g, rot, shift, interp, oversampling, cutoff,
                                          want_rot=want_rot, want_shift=want_shift)
        return d_ref, d_rot, d_shift, None, None, None, None, None, None


def project_3d(vol, rot, shift=None, n_out=None, interp="cubic", oversampling=1.0, cutoff=-1.0,
               save_jacobian=False):
    """Differentiable 3D->2D projection (gradients to vol, rot and shift).

    By default the forward stores nothing beyond its inputs.  With pose
    gradients needed and save_jacobian=True, it keeps 24 bytes per output
    for a backward without a second gather pass."""
    return _Project.apply(vol, rot, shift, 3, n_out, interp, oversampling, cutoff, save_jacobian)


def project_2d(img, rot, shift=None, n_out=None, interp="cubic", oversampling=1.0, cutoff=-1.0):
    """Differentiable 2D->2D projection (gradients to img, rot and shift)."""
    return _Project.apply(img, rot, shift, 2, n_out, interp, oversampling, cutoff, False)


# --------------------------------------------------- weights and x = 0 plane

def _backproject_weights(ndim, weights, rot, N, interp, oversampling, cutoff):
    _need(weights, "weights", torch.float32, 4)
    B, P, n_out = weights.shape[0], weights.shape[1], weights.shape[2]
    if weights.shape[3] != n_out // 2 + 1:
        raise ValueError(f"weights must be [B, P, n, n//2+1], got {tuple(weights.shape)}")
    B_rot, P2, _ = _pose_dims(rot, None, ndim, B, weights.device)
    if P2 != P:
        raise ValueError(f"rot has {P2} poses, weights has {P}")
    shape = (B,) + (N,) * (ndim - 1) + (N // 2 + 1,)
    out = torch.empty(shape, dtype=torch.float32, device=weights.device)
    fn = _lib.lib().tp_backproject_weights_3d if ndim == 3 else _lib.lib().tp_backproject_weights_2d
    st = fn(weights.data_ptr(), B, P, n_out, rot.data_ptr(), B_rot, N, _interp(interp), float(oversampling),
            float(cutoff), out.data_ptr(), _stream(weights.device))
    _lib.check(st, f"tp_backproject_weights_{ndim}d")
    return out


def tp_backproject_weights_3d(weights, rot, N=None, interp="cubic", oversampling=1.0, cutoff=-1.0):
    """Real weights [B,P,n,n//2+1] f32 spread like the adjoint (no phase)
    -> real weight volume [B,N,N,N//2+1] f32."""
    if N is None:
        N = int(round(weights.shape[2] * float(oversampling)))
    return _backproject_weights(3, weights, rot, N, interp, oversampling, cutoff)


def tp_backproject_weights_2d(weights, rot, N=None, interp="cubic", oversampling=1.0, cutoff=-1.0):
    """2D form of tp_backproject_weights_3d -> [B,N,N//2+1] f32."""
    if N is None:
        N = int(round(weights.shape[2] * float(oversampling)))
    return _backproject_weights(2, weights, rot, N, interp, oversampling, cutoff)


def tp_symmetrize_x0(ref):
    """Hermitian symmetrisation of the x = 0 plane of a complex64 rfft
    half-spectrum [B,N,N,N//2+1] or [B,N,N//2+1], in place; returns ref."""
    if not isinstance(ref, torch.Tensor) or ref.dim() not in (3, 4):
        raise ValueError("ref must be [B,N,N//2+1] or [B,N,N,N//2+1]")
    ndim = ref.dim() - 1
    B, N = _ref_dims(ref, ndim, "ref")
    _lib.check(_lib.lib().tp_symmetrize_x0(ndim, ref.data_ptr(), B, N, _stream(ref.device)), "tp_symmetrize_x0")
    return ref


def _as_c64(x):
    return torch.complex(x, torch.zeros_like(x))


class _Backproject(torch.autograd.Function):
    @staticmethod
    def forward(ctx, proj, rot, shift, ndim, N, interp, oversampling, cutoff, symmetrize):
        out = _backproject(ndim, proj, rot, shift, N, interp, oversampling, cutoff)
        if symmetrize:
            tp_symmetrize_x0(out)
        ctx.save_for_backward(proj, rot, shift)
        ctx.cfg = (ndim, interp, oversampling, cutoff, symmetrize)
        return out

    @staticmethod
    def backward(ctx, g):
        proj, rot, shift = ctx.saved_tensors
        ndim, interp, oversampling, cutoff, symmetrize = ctx.cfg
        g = g.contiguous()
        if g.dtype != torch.complex64:
            g = g.to(torch.complex64)
        if symmetrize:  # the symmetrisation is self-adjoint
            g = tp_symmetrize_x0(g.clone())
        d_proj = d_rot = d_shift = None
        if ctx.needs_input_grad[0]:
            d_proj = _project(ndim, g, rot, shift, proj.shape[2], interp, oversampling, cutoff)
        want_rot = ctx.needs_input_grad[1]
        want_shift = shift is not None and ctx.needs_input_grad[2]
        if want_rot or want_shift:
            d_rot, d_shift = tp_grad_pose(g, proj, rot, shift, interp, oversampling, cutoff,
                                          want_rot=want_rot, want_shift=want_shift)
        return d_proj, d_rot, d_shift, None, None, None, None, None, None


def backproject_3d(proj, rot, shift=None, N=None, interp="cubic", oversampling=1.0, cutoff=-1.0,
                   symmetrize=False):
    """Differentiable 2D->3D backprojection (gradients to proj, rot and shift)."""
    if N is None:
        N = int(round(proj.shape[2] * float(oversampling)))
    return _Backproject.apply(proj, rot, shift, 3, N, interp, oversampling, cutoff, symmetrize)


def backproject_2d(proj, rot, shift=None, N=None, interp="cubic", oversampling=1.0, cutoff=-1.0,
                   symmetrize=False):
    """Differentiable 2D->2D backprojection (gradients to proj, rot and shift)."""
    if N is None:
        N = int(round(proj.shape[2] * float(oversampling)))
    return _Backproject.apply(proj, rot, shift, 2, N, interp, oversampling, cutoff, symmetrize)


class _BackprojectWeights(torch.autograd.Function):
    @staticmethod
    def forward(ctx, weights, rot, ndim, N, interp, oversampling, cutoff):
        out = _backproject_weights(ndim, weights, rot, N, interp, oversampling, cutoff)
        ctx.save_for_backward(weights, rot)
        ctx.cfg = (ndim, interp, oversampling, cutoff)
        return out

    @staticmethod
    def backward(ctx, g):
        weights, rot = ctx.saved_tensors
        ndim, interp, oversampling, cutoff = ctx.cfg
        gc = _as_c64(g.contiguous().to(torch.float32))
        d_w = d_rot = None
        if ctx.needs_input_grad[0]:
            # the real forward: a real reference's projection has no imaginary part
            d_w = _project(ndim, gc, rot, None, weights.shape[2], interp, oversampling, cutoff).real.contiguous()
        if ctx.needs_input_grad[1]:
            d_rot, _ = tp_grad_pose(gc, _as_c64(weights.contiguous()), rot, None, interp, oversampling, cutoff,
                                    want_rot=True, want_shift=False)
        return d_w, d_rot, None, None, None, None, None


def backproject_weights_3d(weights, rot, N=None, interp="cubic", oversampling=1.0, cutoff=-1.0):
    """Differentiable weight backprojection (gradients to weights and rot)."""
    if N is None:
        N = int(round(weights.shape[2] * float(oversampling)))
    return _BackprojectWeights.apply(weights, rot, 3, N, interp, oversampling, cutoff)


def backproject_weights_2d(weights, rot, N=None, interp="cubic", oversampling=1.0, cutoff=-1.0):
    """Differentiable 2D weight backprojection (gradients to weights and rot)."""
    if N is None:
        N = int(round(weights.shape[2] * float(oversampling)))
    return _BackprojectWeights.apply(weights, rot, 2, N, interp, oversampling, cutoff)


# -------------------------------------------------------- 3D -> 3D rotation

def _rot_poses(rot, shift, B, dev):
    _need(rot, "rot", torch.float32, 4)
    B_rot, P = rot.shape[0], rot.shape[1]
    if tuple(rot.shape[2:]) != (3, 3) or B_rot not in (1, B) or rot.device != dev:
        raise ValueError(f"rot must be [1 or {B}, P, 3, 3] on the reference's device, got {tuple(rot.shape)}")
    B_shift = 1
    if shift is not None:
        _need(shift, "shift", torch.float32, 3)
        B_shift = shift.shape[0]
        if tuple(shift.shape[1:]) != (P, 3) or B_shift not in (1, B) or shift.device != dev:
            raise ValueError(f"shift must be [1 or {B}, {P}, 3], got {tuple(shift.shape)}")
    return B_rot, P, B_shift


def tp_rotate_3d(vol, rot, shift=None, n_out=None, interp="cubic", oversampling=1.0, cutoff=-1.0):
    """vol [B,N,N,N//2+1] c64, rot [B_rot,P,3,3], shift [B_shift,P,3] or None
    -> [B,P,n_out,n_out,n_out//2+1] c64."""
    B, N = _ref_dims(vol, 3, "reference")
    B_rot, P, B_shift = _rot_poses(rot, shift, B, vol.device)
    if n_out is None:
        n_out = int(round(N / float(oversampling)))
    out = torch.empty((B, P, n_out, n_out, n_out // 2 + 1), dtype=torch.complex64, device=vol.device)
    st = _lib.lib().tp_rotate_3d(vol.data_ptr(), B, N, rot.data_ptr(), B_rot, P, _ptr(shift), B_shift, n_out,
                                 _interp(interp), float(oversampling), float(cutoff), out.data_ptr(),
                                 _stream(vol.device))
    _lib.check(st, "tp_rotate_3d")
    return out


def tp_rotate_backproject_3d(grad_out, rot, shift=None, N=None, interp="cubic", oversampling=1.0, cutoff=-1.0):
    """Adjoint of tp_rotate_3d: [B,P,n,n,n//2+1] -> [B,N,N,N//2+1]."""
    _need(grad_out, "grad_out", torch.complex64, 5)
    B, P, n_out = grad_out.shape[0], grad_out.shape[1], grad_out.shape[2]
    if tuple(grad_out.shape[3:]) != (n_out, n_out // 2 + 1):
        raise ValueError(f"grad_out must be [B, P, n, n, n//2+1], got {tuple(grad_out.shape)}")
    B_rot, P2, B_shift = _rot_poses(rot, shift, B, grad_out.device)
    if P2 != P:
        raise ValueError(f"rot has {P2} poses, grad_out has {P}")
    if N is None:
        N = int(round(n_out * float(oversampling)))
    out = torch.empty((B, N, N, N // 2 + 1), dtype=torch.complex64, device=grad_out.device)
    st = _lib.lib().tp_rotate_backproject_3d(grad_out.data_ptr(), B, P, n_out, rot.data_ptr(), B_rot, _ptr(shift),
                                             B_shift, N, _interp(interp), float(oversampling), float(cutoff),
                                             out.data_ptr(), _stream(grad_out.device))
    _lib.check(st, "tp_rotate_backproject_3d")
    return out


def tp_rotate_grad_pose(vol, grad_out, rot, shift=None, interp="cubic", oversampling=1.0, cutoff=-1.0,
                        want_rot=True, want_shift=True, B_shift=None):
    """Rotation and shift gradients of Re sum conj(grad_out) * rotate_3d(vol, rot, shift):
    (grad_rot [B_rot,P,3,3] or None, grad_shift [B_shift,P,3] or None)."""
    B, N = _ref_dims(vol, 3, "reference")
    B_rot, P, Bs = _rot_poses(rot, shift, B, vol.device)
    _need(grad_out, "grad_out", torch.complex64, 5)
    n_out = grad_out.shape[2]
    if tuple(grad_out.shape) != (B, P, n_out, n_out, n_out // 2 + 1):
        raise ValueError(f"grad_out must be [{B}, {P}, n, n, n//2+1], got {tuple(grad_out.shape)}")
    if shift is None:
        Bs = 1 if B_shift is None else int(B_shift)
    gr = torch.empty_like(rot) if want_rot else None
    gs = torch.empty((Bs, P, 3), dtype=torch.float32, device=vol.device) if want_shift else None
    st = _lib.lib().tp_rotate_grad_pose(vol.data_ptr(), B, N, grad_out.data_ptr(), rot.data_ptr(), B_rot, P,
                                        _ptr(shift), Bs, n_out, _interp(interp), float(oversampling), float(cutoff),
                                        _ptr(gr), _ptr(gs), _stream(vol.device))
    _lib.check(st, "tp_rotate_grad_pose")
    return gr, gs


def tp_rotate_3d_jac(vol, rot, shift=None, n_out=None, interp="cubic", oversampling=1.0, cutoff=-1.0):
    """tp_rotate_3d that also returns the Jacobian of each output w.r.t. its
    sample point: (out [B,P,n,n,n//2+1], jac [B,P,3,n,n,n//2+1]) c64."""
    B, N = _ref_dims(vol, 3, "reference")
    B_rot, P, B_shift = _rot_poses(rot, shift, B, vol.device)
    if n_out is None:
        n_out = int(round(N / float(oversampling)))
    out = torch.empty((B, P, n_out, n_out, n_out // 2 + 1), dtype=torch.complex64, device=vol.device)
    jac = torch.empty((B, P, 3, n_out, n_out, n_out // 2 + 1), dtype=torch.complex64, device=vol.device)
    st = _lib.lib().tp_rotate_3d_jac(vol.data_ptr(), B, N, rot.data_ptr(), B_rot, P, _ptr(shift), B_shift, n_out,
                                     _interp(interp), float(oversampling), float(cutoff), out.data_ptr(),
                                     jac.data_ptr(), _stream(vol.device))
    _lib.check(st, "tp_rotate_3d_jac")
    return out, jac


def tp_rotate_grad_pose_jac(grad_out, out, jac, B_rot=1, B_shift=1, oversampling=1.0, cutoff=-1.0,
                            want_rot=True, want_shift=True):
    """Pose gradients from tp_rotate_3d_jac's (out, jac):
    (grad_rot [B_rot,P,3,3] or None, grad_shift [B_shift,P,3] or None)."""
    _need(grad_out, "grad_out", torch.complex64, 5)
    _need(out, "out", torch.complex64, 5)
    _need(jac, "jac", torch.complex64, 6)
    B, P, n_out = out.shape[0], out.shape[1], out.shape[2]
    if tuple(out.shape) != (B, P, n_out, n_out, n_out // 2 + 1) or grad_out.shape != out.shape:
        raise ValueError(f"grad_out and out must be [B, P, n, n, n//2+1], got {tuple(grad_out.shape)}, "
                         f"{tuple(out.shape)}")
    if tuple(jac.shape) != (B, P, 3) + tuple(out.shape[2:]):
        raise ValueError(f"jac must be [{B}, {P}, 3, {n_out}, {n_out}, {n_out // 2 + 1}], got {tuple(jac.shape)}")
    if grad_out.device != out.device or jac.device != out.device:
        raise ValueError("grad_out, out and jac must be on one device")
    gr = torch.empty((B_rot, P, 3, 3), dtype=torch.float32, device=out.device) if want_rot else None
    gs = torch.empty((B_shift, P, 3), dtype=torch.float32, device=out.device) if want_shift else None
    st = _lib.lib().tp_rotate_grad_pose_jac(grad_out.data_ptr(), out.data_ptr(), jac.data_ptr(), B, P, n_out,
                                            int(B_rot), int(B_shift), float(oversampling), float(cutoff), _ptr(gr),
                                            _ptr(gs), _stream(out.device))
    _lib.check(st, "tp_rotate_grad_pose_jac")
    return gr, gs


def tp_rotate_backward_3d_jac(grad_out, out, jac, rot, shift=None, N=None, interp="cubic", oversampling=1.0,
                              cutoff=-1.0, want_rot=True, want_shift=True, B_shift=None):
    """The backward of tp_rotate_3d_jac in one launch: (d_vol [B,N,N,N//2+1],
    grad_rot [B_rot,P,3,3] or None, grad_shift [B_shift,P,3] or None), the
    values of tp_rotate_backproject_3d and tp_rotate_grad_pose_jac."""
    _need(grad_out, "grad_out", torch.complex64, 5)
    _need(out, "out", torch.complex64, 5)
    _need(jac, "jac", torch.complex64, 6)
    B, P, n_out = out.shape[0], out.shape[1], out.shape[2]
    if tuple(out.shape) != (B, P, n_out, n_out, n_out // 2 + 1) or grad_out.shape != out.shape:
        raise ValueError(f"grad_out and out must be [B, P, n, n, n//2+1], got {tuple(grad_out.shape)}, "
                         f"{tuple(out.shape)}")
    if tuple(jac.shape) != (B, P, 3) + tuple(out.shape[2:]):
        raise ValueError(f"jac must be [{B}, {P}, 3, {n_out}, {n_out}, {n_out // 2 + 1}], got {tuple(jac.shape)}")
    if grad_out.device != out.device or jac.device != out.device:
        raise ValueError("grad_out, out and jac must be on one device")
    B_rot, P2, Bs = _rot_poses(rot, shift, B, out.device)
    if P2 != P:
        raise ValueError(f"rot has {P2} poses, out has {P}")
    if shift is None:
        Bs = 1 if B_shift is None else int(B_shift)
    if N is None:
        N = int(round(n_out * float(oversampling)))
    dev = out.device
    vol = torch.empty((B, N, N, N // 2 + 1), dtype=torch.complex64, device=dev)
    gr = torch.empty((B_rot, P, 3, 3), dtype=torch.float32, device=dev) if want_rot else None
    gs = torch.empty((Bs, P, 3), dtype=torch.float32, device=dev) if want_shift else None
    st = _lib.lib().tp_rotate_backward_3d_jac(grad_out.data_ptr(), out.data_ptr(), jac.data_ptr(), B, P, n_out,
                                              rot.data_ptr(), B_rot, _ptr(shift), Bs, int(N), _interp(interp),
                                              float(oversampling), float(cutoff), vol.data_ptr(), _ptr(gr),
                                              _ptr(gs), _stream(dev))
    _lib.check(st, "tp_rotate_backward_3d_jac")
    return vol, gr, gs


class _Rotate(torch.autograd.Function):
    @staticmethod
    def forward(ctx, vol, rot, shift, n_out, interp, oversampling, cutoff, save_jacobian):
        pose_grads = ctx.needs_input_grad[1] or (shift is not None and ctx.needs_input_grad[2])
        jac = None
        if save_jacobian and pose_grads:
            out, jac = tp_rotate_3d_jac(vol, rot, shift, n_out, interp, oversampling, cutoff)
            ctx.save_for_backward(vol, rot, shift, out, jac)
        else:
            out = tp_rotate_3d(vol, rot, shift, n_out, interp, oversampling, cutoff)
            ctx.save_for_backward(vol, rot, shift)
        ctx.has_jac = jac is not None
        ctx.cfg = (interp, oversampling, cutoff)
        return out

    @staticmethod
    def backward(ctx, g):
        if ctx.has_jac:
            vol, rot, shift, out, jac = ctx.saved_tensors
        else:
            vol, rot, shift = ctx.saved_tensors
        interp, oversampling, cutoff = ctx.cfg
        g = g.contiguous()
        if g.dtype != torch.complex64:
            g = g.to(torch.complex64)
        d_vol = d_rot = d_shift = None
        want_rot = ctx.needs_input_grad[1]
        want_shift = shift is not None and ctx.needs_input_grad[2]
        if ctx.needs_input_grad[0] and (want_rot or want_shift) and ctx.has_jac:
            # both gradients from one launch
            d_vol, d_rot, d_shift = tp_rotate_backward_3d_jac(g, out, jac, rot, shift, vol.shape[1], interp,
                                                              oversampling, cutoff, want_rot, want_shift)
            return d_vol, d_rot, d_shift, None, None, None, None, None
        if ctx.needs_input_grad[0]:
            d_vol = tp_rotate_backproject_3d(g, rot, shift, vol.shape[1], interp, oversampling, cutoff)
        if (want_rot or want_shift) and ctx.has_jac:
            B_shift = shift.shape[0] if shift is not None else 1
            d_rot, d_shift = tp_rotate_grad_pose_jac(g, out, jac, rot.shape[0], B_shift, oversampling, cutoff,
                                                     want_rot=want_rot, want_shift=want_shift)
        elif want_rot or want_shift:
            d_rot, d_shift = tp_rotate_grad_pose(vol, g, rot, shift, interp, oversampling, cutoff,
                                                 want_rot=want_rot, want_shift=want_shift)
        return d_vol, d_rot, d_shift, None, None, None, None, None


def rotate_3d(vol, rot, shift=None, n_out=None, interp="cubic", oversampling=1.0, cutoff=-1.0, save_jacobian=False):
    """Differentiable 3D->3D rotation (gradients to vol, rot and shift).

    With pose gradients needed and save_jacobian (output boxes up to 1023),
    the forward keeps 24 bytes per output for a backward without a second
    gather pass."""
    if n_out is None:
        n_out = int(round(vol.shape[1] / float(oversampling)))
    save_jacobian = save_jacobian and n_out <= 1023
    return _Rotate.apply(vol, rot, shift, n_out, interp, oversampling, cutoff, save_jacobian)
