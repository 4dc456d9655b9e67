"""ctypes binding of the projector's C ABI (include/tp.h).

Argument marshalling only: every computation runs in libtp.so's HIP kernels.
Loading fails loudly when the library has not been built; there is no CPU
fallback.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("TP_LIBRARY", os.path.join(HERE, "libtp.so"))

TP_OK, TP_EINVAL, TP_EUNSUPPORTED, TP_EHIP = 0, -1, -2, -3
TP_LINEAR, TP_CUBIC = 0, 1

EXPORTS = (
    "tp_abi_version",
    "tp_status_str",
    "tp_project_3d",
    "tp_backproject_3d",
    "tp_project_2d",
    "tp_backproject_2d",
    "tp_grad_pose",
    "tp_backproject_weights_3d",
    "tp_backproject_weights_2d",
    "tp_symmetrize_x0",
    "tp_rotate_3d",
    "tp_rotate_backproject_3d",
    "tp_rotate_grad_pose",
    "tp_backward_3d",
    "tp_project_3d_jac",
    "tp_grad_pose_jac",
    "tp_backward_3d_jac",
    "tp_rotate_3d_jac",
    "tp_rotate_grad_pose_jac",
    "tp_rotate_backward_3d_jac",
)

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int
_f32 = ctypes.c_float

_SIGS = {
    "tp_abi_version": ([], _int),
    "tp_status_str": ([_int], ctypes.c_char_p),
    # vol, B, N, rot, B_rot, P, shift, B_shift, N_out, interp, os, cutoff, out, stream
    "tp_project_3d": ([_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _int, _f32, _f32, _vp, _vp], _int),
    "tp_project_2d": ([_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _int, _f32, _f32, _vp, _vp], _int),
    # proj, B, P, N_out, rot, B_rot, shift, B_shift, N, interp, os, cutoff, ref_out, stream
    "tp_backproject_3d": ([_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _int, _f32, _f32, _vp, _vp], _int),
    "tp_backproject_2d": ([_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _int, _f32, _f32, _vp, _vp], _int),
    # ndim, ref, B, N, grad_out, rot, B_rot, P, shift, B_shift, N_out, interp, os, cutoff,
    # grad_rot, grad_shift, stream
    "tp_grad_pose": ([_int, _vp, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _int, _f32, _f32,
                      _vp, _vp, _vp], _int),
    # weights, B, P, N_out, rot, B_rot, N, interp, os, cutoff, wref_out, stream
    "tp_backproject_weights_3d": ([_vp, _i64, _i64, _i64, _vp, _i64, _i64, _int, _f32, _f32, _vp, _vp], _int),
    "tp_backproject_weights_2d": ([_vp, _i64, _i64, _i64, _vp, _i64, _i64, _int, _f32, _f32, _vp, _vp], _int),
    # ndim, ref, B, N, stream
    "tp_symmetrize_x0": ([_int, _vp, _i64, _i64, _vp], _int),
    # vol, B, N, rot, B_rot, P, shift, B_shift, N_out, interp, os, cutoff, out, stream
    "tp_rotate_3d": ([_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _int, _f32, _f32, _vp, _vp], _int),
    # grad_out, B, P, N_out, rot, B_rot, shift, B_shift, N, interp, os, cutoff, vol_out, stream
    "tp_rotate_backproject_3d": ([_vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _int, _f32, _f32, _vp, _vp],
                                 _int),
    # vol, B, N, grad_out, rot, B_rot, P, shift, B_shift, N_out, interp, os, cutoff, grad_rot, grad_shift, stream
    "tp_rotate_grad_pose": ([_vp, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _int, _f32, _f32, _vp, _vp,
                             _vp], _int),
    # vol, B, N, grad_out, rot, B_rot, P, shift, B_shift, N_out, interp, os, cutoff, vol_grad,
    # grad_rot, grad_shift, stream
    "tp_backward_3d": ([_vp, _i64, _i64, _vp, _vp, _i64, _i64, _vp, _i64, _i64, _int, _f32, _f32, _vp, _vp, _vp,
                        _vp], _int),
    # vol, B, N, rot, B_rot, P, shift, B_shift, N_out, interp, os, cutoff, out, jac, stream
    "tp_project_3d_jac": ([_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _int, _f32, _f32, _vp, _vp, _vp],
                          _int),
    # grad_out, proj, jac, B, P, N_out, B_rot, B_shift, os, cutoff, grad_rot, grad_shift, stream
    "tp_grad_pose_jac": ([_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f32, _f32, _vp, _vp, _vp], _int),
    # grad_out, proj, jac, B, P, N_out, rot, B_rot, shift, B_shift, N, interp, os, cutoff, vol_out,
    # grad_rot, grad_shift, stream
    "tp_backward_3d_jac": ([_vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _int, _f32, _f32, _vp,
                            _vp, _vp, _vp], _int),
    # as tp_project_3d_jac / tp_grad_pose_jac, for the 3D -> 3D rotation
    "tp_rotate_3d_jac": ([_vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _int, _f32, _f32, _vp, _vp, _vp],
                         _int),
    "tp_rotate_grad_pose_jac": ([_vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _f32, _f32, _vp, _vp, _vp], _int),
    # as tp_backward_3d_jac, for the 3D -> 3D rotation
    "tp_rotate_backward_3d_jac": ([_vp, _vp, _vp, _i64, _i64, _i64, _vp, _i64, _vp, _i64, _i64, _int, _f32, _f32,
                                   _vp, _vp, _vp, _vp], _int),
}

_lib = None


class TPError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().tp_status_str(status).decode()
        super().__init__(f"{where}: {msg} ({status})")


def lib() -> ctypes.CDLL:
    """The loaded libtp.so (raises if it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m cryo_em_fourier_amd.build` "
                "(the projector has no CPU fallback)")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = res
        _lib = L
    return _lib


def check(status: int, where: str) -> None:
    if status != TP_OK:
        raise TPError(status, where)
