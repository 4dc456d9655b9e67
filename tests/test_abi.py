"""C-ABI library checks that need no GPU: it loads, exports every symbol the
header declares, and rejects invalid arguments before launching anything."""
import ctypes
import math
import os
import re

import pytest

from cryo_em_fourier_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tp.h")

FAKE = 0x10000          # 64 KiB-aligned fake device address: never dereferenced
FAKE_ODD = 0x10004      # 4- but not 8-byte aligned


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z0-9_]+)\s*\(", src)))


def test_header_declares_the_five_entry_points():
    names = declared_functions()
    for n in ("tp_project_3d", "tp_backproject_3d", "tp_project_2d", "tp_backproject_2d", "tp_grad_pose"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert set(declared_functions()) == set(_lib.EXPORTS)
    assert L.tp_abi_version() == 101


def test_status_strings():
    L = _lib.lib()
    for code in (0, -1, -2, -3, 7):
        assert L.tp_status_str(code)


def proj3(**kw):
    a = dict(vol=FAKE, B=1, N=32, rot=FAKE, B_rot=1, P=4, shift=None, B_shift=1, N_out=32,
             interp=1, os=1.0, cutoff=16.0, out=FAKE, stream=None)
    a.update(kw)
    return _lib.lib().tp_project_3d(*a.values())


def back3(**kw):
    a = dict(proj=FAKE, B=1, P=4, N_out=32, rot=FAKE, B_rot=1, shift=None, B_shift=1, N=32,
             interp=1, os=1.0, cutoff=16.0, out=FAKE, stream=None)
    a.update(kw)
    return _lib.lib().tp_backproject_3d(*a.values())


def grad(**kw):
    a = dict(ndim=3, ref=FAKE, B=1, N=32, g=FAKE, rot=FAKE, B_rot=1, P=4, shift=None, B_shift=1,
             N_out=32, interp=1, os=1.0, cutoff=16.0, gr=FAKE, gs=None, stream=None)
    a.update(kw)
    return _lib.lib().tp_grad_pose(*a.values())


def bwd3(**kw):
    a = dict(vol=FAKE, B=1, N=32, g=FAKE, rot=FAKE, B_rot=1, P=4, shift=None, B_shift=1, N_out=32,
             interp=1, os=1.0, cutoff=16.0, vg=FAKE, gr=FAKE, gs=None, stream=None)
    a.update(kw)
    return _lib.lib().tp_backward_3d(*a.values())


EINVAL, EUNSUP = _lib.TP_EINVAL, _lib.TP_EUNSUPPORTED


@pytest.mark.parametrize("kw,code", [
    (dict(vol=None), EINVAL), (dict(out=None), EINVAL), (dict(rot=None), EINVAL),
    (dict(vol=FAKE_ODD), EINVAL), (dict(out=FAKE_ODD), EINVAL),
    (dict(B=0), EINVAL), (dict(N=0), EINVAL), (dict(P=0), EINVAL), (dict(N_out=-3), EINVAL),
    (dict(interp=2), EINVAL), (dict(interp=-1), EINVAL),
    (dict(os=0.0), EINVAL), (dict(os=-1.0), EINVAL), (dict(os=math.inf), EINVAL), (dict(os=math.nan), EINVAL),
    (dict(cutoff=math.nan), EINVAL),
    (dict(B=2, B_rot=3), EINVAL), (dict(B=2, shift=FAKE, B_shift=3), EINVAL),
    (dict(N=70000), EUNSUP), (dict(N_out=70000), EUNSUP),
    (dict(N=1024), EUNSUP),                 # 1024^2 * 513 * 8 bytes > 2 GiB
    (dict(B=1 << 20, B_rot=1 << 20, P=1 << 20), EUNSUP),  # grid too large
])
def test_project_3d_argument_checks(kw, code):
    assert proj3(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(proj=None), EINVAL), (dict(out=None), EINVAL), (dict(interp=5), EINVAL),
    (dict(os=0.0), EINVAL), (dict(B=3, B_rot=2), EINVAL), (dict(N=2000), EUNSUP),
    (dict(N_out=16384), EUNSUP),            # 14-bit lattice offsets in the hit lists
    (dict(B=70000, B_rot=1), EUNSUP),       # the batch is a grid dimension
])
def test_backproject_3d_argument_checks(kw, code):
    assert back3(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(ndim=4), EINVAL), (dict(ndim=1), EINVAL), (dict(ref=None), EINVAL), (dict(g=None), EINVAL),
    (dict(gr=FAKE + 2), EINVAL), (dict(gs=FAKE, B=2, B_rot=2, B_shift=3), EINVAL),
    (dict(cutoff=math.nan), EINVAL),
])
def test_grad_pose_argument_checks(kw, code):
    assert grad(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(vol=None), EINVAL), (dict(g=None), EINVAL), (dict(rot=None), EINVAL),
    (dict(vol=FAKE_ODD), EINVAL), (dict(vg=FAKE_ODD), EINVAL), (dict(gr=FAKE + 2), EINVAL),
    (dict(gs=FAKE, B=2, B_rot=2, B_shift=3), EINVAL), (dict(interp=2), EINVAL), (dict(os=0.0), EINVAL),
    (dict(cutoff=math.nan), EINVAL), (dict(B=3, B_rot=2), EINVAL),
    (dict(N=2000), EUNSUP), (dict(N_out=16384), EUNSUP), (dict(B=70000, B_rot=1), EUNSUP),
])
def test_backward_3d_argument_checks(kw, code):
    assert bwd3(**kw) == code


def test_backward_3d_with_nothing_to_compute_launches_nothing():
    # no volume gradient and no pose gradients: valid, and no device access
    assert bwd3(vg=None, gr=None, gs=None) == _lib.TP_OK


def test_2d_entry_points_check_arguments():
    L = _lib.lib()
    assert L.tp_project_2d(None, 1, 32, FAKE, 1, 4, None, 1, 32, 1, 1.0, -1.0, FAKE, None) == EINVAL
    assert L.tp_project_2d(FAKE, 1, 32, FAKE, 1, 4, None, 1, 32, 3, 1.0, -1.0, FAKE, None) == EINVAL
    assert L.tp_backproject_2d(FAKE, 1, 4, 32, FAKE, 1, None, 1, 32, 1, -2.0, -1.0, FAKE, None) == EINVAL
    # 2D references are limited by the same 2 GiB per entry
    assert L.tp_project_2d(FAKE, 1, 60000, FAKE, 1, 4, None, 1, 32, 1, 1.0, -1.0, FAKE, None) == EUNSUP


def test_python_binding_rejects_cpu_tensors():
    import torch

    from cryo_em_fourier_amd import tp_project_3d

    vol = torch.zeros((1, 8, 8, 5), dtype=torch.complex64)
    rot = torch.eye(3).reshape(1, 1, 3, 3)
    with pytest.raises(ValueError, match="GPU"):
        tp_project_3d(vol, rot)


def test_weights_and_symmetrize_check_arguments():
    L = _lib.lib()
    # weights, B, P, N_out, rot, B_rot, N, interp, os, cutoff, out, stream
    assert L.tp_backproject_weights_3d(None, 1, 4, 32, FAKE, 1, 32, 1, 1.0, -1.0, FAKE, None) == EINVAL
    assert L.tp_backproject_weights_3d(FAKE, 1, 4, 32, FAKE, 1, 32, 1, 1.0, -1.0, None, None) == EINVAL
    assert L.tp_backproject_weights_3d(FAKE, 1, 4, 32, FAKE, 1, 32, 7, 1.0, -1.0, FAKE, None) == EINVAL
    assert L.tp_backproject_weights_3d(FAKE, 2, 4, 32, FAKE, 3, 32, 1, 1.0, -1.0, FAKE, None) == EINVAL
    assert L.tp_backproject_weights_3d(FAKE, 1, 4, 16384, FAKE, 1, 32, 1, 1.0, -1.0, FAKE, None) == EUNSUP
    assert L.tp_backproject_weights_2d(FAKE, 1, 4, 32, FAKE, 1, 32, 1, 0.0, -1.0, FAKE, None) == EINVAL
    assert L.tp_backproject_weights_2d(FAKE + 2, 1, 4, 32, FAKE, 1, 32, 1, 1.0, -1.0, FAKE, None) == EINVAL
    # ndim, ref, B, N, stream
    assert L.tp_symmetrize_x0(4, FAKE, 1, 8, None) == EINVAL
    assert L.tp_symmetrize_x0(3, None, 1, 8, None) == EINVAL
    assert L.tp_symmetrize_x0(3, FAKE_ODD, 1, 8, None) == EINVAL
    assert L.tp_symmetrize_x0(2, FAKE, 0, 8, None) == EINVAL
    assert L.tp_symmetrize_x0(2, FAKE, 1, 70000, None) == EUNSUP


def test_rotate_entry_points_check_arguments():
    L = _lib.lib()
    # vol, B, N, rot, B_rot, P, shift, B_shift, N_out, interp, os, cutoff, out, stream
    assert L.tp_rotate_3d(None, 1, 16, FAKE, 1, 2, None, 1, 16, 1, 1.0, -1.0, FAKE, None) == EINVAL
    assert L.tp_rotate_3d(FAKE, 1, 16, FAKE, 1, 2, None, 1, 16, 3, 1.0, -1.0, FAKE, None) == EINVAL
    assert L.tp_rotate_3d(FAKE, 2, 16, FAKE, 3, 2, None, 1, 16, 1, 1.0, -1.0, FAKE, None) == EINVAL
    assert L.tp_rotate_3d(FAKE, 1, 1024, FAKE, 1, 2, None, 1, 16, 1, 1.0, -1.0, FAKE, None) == EUNSUP
    assert L.tp_rotate_3d(FAKE, 1, 16, FAKE, 1, 1 << 30, None, 1, 4096, 1, 1.0, -1.0, FAKE, None) == EUNSUP
    # grad_out, B, P, N_out, rot, B_rot, shift, B_shift, N, interp, os, cutoff, vol_out, stream
    assert L.tp_rotate_backproject_3d(FAKE, 1, 2, 16, FAKE, 1, None, 1, 16, 1, 0.0, -1.0, FAKE, None) == EINVAL
    assert L.tp_rotate_backproject_3d(FAKE_ODD, 1, 2, 16, FAKE, 1, None, 1, 16, 1, 1.0, -1.0, FAKE, None) == EINVAL
    # 10-bit lattice offsets in the adjoint's hit lists
    assert L.tp_rotate_backproject_3d(FAKE, 1, 2, 1024, FAKE, 1, None, 1, 16, 1, 1.0, -1.0, FAKE, None) == EUNSUP
    # vol, B, N, grad_out, rot, B_rot, P, shift, B_shift, N_out, interp, os, cutoff, gr, gs, stream
    assert L.tp_rotate_grad_pose(FAKE, 1, 16, None, FAKE, 1, 2, None, 1, 16, 1, 1.0, -1.0, FAKE, None, None) == EINVAL
    assert L.tp_rotate_grad_pose(FAKE, 1, 16, FAKE, FAKE, 1, 2, None, 1, 16, 1, 1.0, math.nan, FAKE, None,
                                 None) == EINVAL


def test_jacobian_entry_points_check_arguments():
    L = _lib.lib()
    # vol, B, N, rot, B_rot, P, shift, B_shift, N_out, interp, os, cutoff, out, jac, stream
    assert L.tp_project_3d_jac(FAKE, 1, 32, FAKE, 1, 4, None, 1, 32, 1, 1.0, -1.0, FAKE, None, None) == EINVAL
    assert L.tp_project_3d_jac(FAKE, 1, 32, FAKE, 1, 4, None, 1, 32, 1, 1.0, -1.0, FAKE, FAKE_ODD, None) == EINVAL
    assert L.tp_project_3d_jac(FAKE, 1, 32, FAKE, 1, 4, None, 1, 32, 2, 1.0, -1.0, FAKE, FAKE, None) == EINVAL
    assert L.tp_project_3d_jac(FAKE, 1, 70000, FAKE, 1, 4, None, 1, 32, 1, 1.0, -1.0, FAKE, FAKE, None) == EUNSUP
    # grad_out, proj, jac, B, P, N_out, B_rot, B_shift, os, cutoff, grad_rot, grad_shift, stream
    assert L.tp_grad_pose_jac(FAKE, None, FAKE, 1, 4, 32, 1, 1, 1.0, -1.0, FAKE, None, None) == EINVAL
    assert L.tp_grad_pose_jac(FAKE, FAKE, FAKE_ODD, 1, 4, 32, 1, 1, 1.0, -1.0, FAKE, None, None) == EINVAL
    assert L.tp_grad_pose_jac(FAKE, FAKE, FAKE, 0, 4, 32, 1, 1, 1.0, -1.0, FAKE, None, None) == EINVAL
    assert L.tp_grad_pose_jac(FAKE, FAKE, FAKE, 2, 4, 32, 3, 1, 1.0, -1.0, FAKE, None, None) == EINVAL
    assert L.tp_grad_pose_jac(FAKE, FAKE, FAKE, 2, 4, 32, 1, 3, 1.0, -1.0, None, FAKE, None) == EINVAL
    assert L.tp_grad_pose_jac(FAKE, FAKE, FAKE, 1, 4, 32, 1, 1, 0.0, -1.0, FAKE, None, None) == EINVAL
    assert L.tp_grad_pose_jac(FAKE, FAKE, FAKE, 1, 4, 32, 1, 1, 1.0, math.nan, FAKE, None, None) == EINVAL
    assert L.tp_grad_pose_jac(FAKE, FAKE, FAKE, 1, 4, 32, 1, 1, 1.0, -1.0, FAKE + 2, None, None) == EINVAL
    assert L.tp_grad_pose_jac(FAKE, FAKE, FAKE, 1, 4, 70000, 1, 1, 1.0, -1.0, FAKE, None, None) == EUNSUP
    assert L.tp_grad_pose_jac(FAKE, FAKE, FAKE, 1 << 20, 1 << 12, 32, 1, 1, 1.0, -1.0, FAKE, None, None) == EUNSUP
    # nothing requested: a no-op that touches no pointer
    assert L.tp_grad_pose_jac(FAKE, FAKE, FAKE, 1, 4, 32, 1, 1, 1.0, -1.0, None, None, None) == _lib.TP_OK


def test_fused_backward_checks_arguments():
    L = _lib.lib()
    f = L.tp_backward_3d_jac
    # grad_out, proj, jac, B, P, N_out, rot, B_rot, shift, B_shift, N, interp, os, cutoff, vol_out,
    # grad_rot, grad_shift, stream
    ok = [FAKE, FAKE, FAKE, 1, 4, 32, FAKE, 1, None, 1, 32, 1, 1.0, -1.0, FAKE, FAKE, None, None]

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a2=None) == EINVAL                 # no jac
    assert call(a14=None) == EINVAL                # no volume
    assert call(a1=FAKE_ODD) == EINVAL             # misaligned proj
    assert call(a15=FAKE + 2) == EINVAL            # misaligned grad_rot
    assert call(a3=0) == EINVAL                    # B = 0
    assert call(a7=3) == EINVAL                    # B_rot not in {1, B}
    assert call(a16=FAKE, a9=3) == EINVAL          # B_shift not in {1, B} with grad_shift
    assert call(a11=2) == EINVAL                   # interpolation
    assert call(a12=0.0) == EINVAL                 # oversampling
    assert call(a13=math.nan) == EINVAL            # cutoff
    assert call(a5=(1 << 14)) == EUNSUP            # lattice offsets are 14-bit
    assert call(a10=70000) == EUNSUP               # box


def test_rotation_fused_backward_checks_arguments():
    L = _lib.lib()
    f = L.tp_rotate_backward_3d_jac
    # grad_out, out, jac, B, P, N_out, rot, B_rot, shift, B_shift, N, interp, os, cutoff, vol_out,
    # grad_rot, grad_shift, stream
    ok = [FAKE, FAKE, FAKE, 1, 2, 16, FAKE, 1, None, 1, 16, 1, 1.0, -1.0, FAKE, FAKE, None, None]

    def call(**kw):
        a = list(ok)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return f(*a)

    assert call(a0=None) == EINVAL                 # no upstream gradient
    assert call(a14=None) == EINVAL                # no volume
    assert call(a2=FAKE_ODD) == EINVAL             # misaligned jac
    assert call(a16=FAKE + 2) == EINVAL            # misaligned grad_shift
    assert call(a7=3, a3=2) == EINVAL              # B_rot not in {1, B}
    assert call(a16=FAKE, a9=3) == EINVAL          # B_shift not in {1, B} with grad_shift
    assert call(a12=-1.0) == EINVAL                # oversampling
    assert call(a13=math.nan) == EINVAL            # cutoff
    assert call(a5=1024) == EUNSUP                 # 10-bit lattice offsets


def test_rotation_jacobian_entry_points_check_arguments():
    L = _lib.lib()
    # vol, B, N, rot, B_rot, P, shift, B_shift, N_out, interp, os, cutoff, out, jac, stream
    assert L.tp_rotate_3d_jac(FAKE, 1, 16, FAKE, 1, 2, None, 1, 16, 1, 1.0, -1.0, FAKE, None, None) == EINVAL
    assert L.tp_rotate_3d_jac(FAKE, 1, 16, FAKE, 1, 2, None, 1, 16, 1, 1.0, -1.0, FAKE, FAKE_ODD, None) == EINVAL
    assert L.tp_rotate_3d_jac(FAKE, 2, 16, FAKE, 3, 2, None, 1, 16, 1, 1.0, -1.0, FAKE, FAKE, None) == EINVAL
    assert L.tp_rotate_3d_jac(FAKE, 1, 16, FAKE, 1, 2, None, 1, 1024, 1, 1.0, -1.0, FAKE, FAKE, None) == EUNSUP
    # grad_out, out, jac, B, P, N_out, B_rot, B_shift, os, cutoff, grad_rot, grad_shift, stream
    assert L.tp_rotate_grad_pose_jac(None, FAKE, FAKE, 1, 2, 16, 1, 1, 1.0, -1.0, FAKE, None, None) == EINVAL
    assert L.tp_rotate_grad_pose_jac(FAKE, FAKE, FAKE, 2, 2, 16, 3, 1, 1.0, -1.0, FAKE, None, None) == EINVAL
    assert L.tp_rotate_grad_pose_jac(FAKE, FAKE, FAKE, 1, 2, 16, 1, 1, -1.0, -1.0, FAKE, None, None) == EINVAL
    assert L.tp_rotate_grad_pose_jac(FAKE, FAKE, FAKE, 1, 2, 1024, 1, 1, 1.0, -1.0, FAKE, None, None) == EUNSUP
    assert L.tp_rotate_grad_pose_jac(FAKE, FAKE, FAKE, 1, 2, 16, 1, 1, 1.0, -1.0, None, None, None) == _lib.TP_OK


def test_peak_probe_library_loads_and_checks_arguments():
    """The roofline probes (libtp_peaks.so) export what include/tp_peaks.h
    declares and reject invalid arguments before launching anything."""
    from cryo_em_fourier_amd import build as _build

    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "tp_peaks.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(tpk_[a-z0-9_]+)\s*\(", src)))
    assert names == ["tpk_fma", "tpk_lds_add", "tpk_read", "tpk_threads_per_block"]
    L = ctypes.CDLL(_build.PEAKS_LIB)
    for n in names:
        assert hasattr(L, n), n
    vp, u64, i64, ci = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int
    L.tpk_read.argtypes = [vp, u64, i64, u64, ci, ci, vp, vp]
    L.tpk_fma.argtypes = [i64, ci, vp, vp]
    L.tpk_lds_add.argtypes = [i64, ci, vp, vp]
    assert L.tpk_threads_per_block() == 256
    assert L.tpk_read(None, 1024, 1, 0, 1, 8, FAKE, None) == -1        # no buffer
    assert L.tpk_read(FAKE + 8, 1024, 1, 0, 1, 8, FAKE, None) == -1    # misaligned
    assert L.tpk_read(FAKE, 1024, 1, 0, 3, 9, FAKE, None) == -1        # regions not 1 or 8
    assert L.tpk_read(FAKE, 1020, 1, 0, 8, 8, FAKE, None) == -1        # n16 not a multiple of regions
    assert L.tpk_read(FAKE, 1024, 0, 0, 1, 8, FAKE, None) == -1        # no pass
    assert L.tpk_fma(0, 8, FAKE, None) == -1
    assert L.tpk_lds_add(10, 0, FAKE, None) == -1
