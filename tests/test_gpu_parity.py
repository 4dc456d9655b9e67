"""GPU parity: the HIP library (through its C ABI) against the fp64 oracle.

Small cases that span several 16x16 output tiles with ragged edges, odd and
even boxes, oversampling 1 / 1.5 / 2 / 2.5, batches with per-entry and broadcast
poses, no cutoff (taps reach the Nyquist planes), and adversarial poses: the
identity, cube rotations (on-grid samples), the slice plane on the x = 0 plane
(every stencil straddles the Friedel fold), near it, and +-60 degree tilts.
Bar: relative L2 <= 1e-5 and max-abs <= 1e-4 * max|oracle|.
"""
import functools
import math
import zlib

import numpy as np
import pytest

from cryo_em_fourier_amd import synth
from oracle import CUBIC, LINEAR
import oracle

from _gpu import assert_parity, complex_normal, log, rel_errors, to_dev

pytestmark = pytest.mark.gpu


def adversarial_rotations(rng):
    I = np.eye(3)
    cyc = np.array([[0.0, 1, 0], [0, 0, 1], [1, 0, 0]])       # slice plane = the x = 0 plane
    Rz90 = np.array([[0.0, -1, 0], [1, 0, 0], [0, 0, 1]])
    Rx90 = np.array([[1.0, 0, 0], [0, 0, -1], [0, 1, 0]])
    near = cyc @ synth.axis_angle(np.array([0.36, 0.48, 0.8]), 1e-3)   # slightly off the x = 0 plane
    tilt_p = synth.axis_angle(np.array([0.0, 1.0, 0.0]), math.radians(60))
    tilt_m = synth.axis_angle(np.array([0.6, 0.8, 0.0]), math.radians(-60))
    mats = [I, cyc, Rz90, Rx90, near, tilt_p, tilt_m, -np.diag([1.0, 1.0, -1.0])]
    return np.stack(mats).astype(np.float32)


@functools.lru_cache(maxsize=None)
def case3d(name):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    # name: N, N_out, B, P, B_rot, B_shift(0 = no shift), interp, os, cutoff, vol, poses
    spec = {
        "c1":            (32, 32, 1, 16, 1, 0, LINEAR, 1.0, 16.0, "c1", "c1"),
        "c1-cubic":      (32, 32, 1, 16, 1, 1, CUBIC, 1.0, 16.0, "c1", "c1"),
        "odd-nocut":     (33, 33, 1, 6, 1, 1, CUBIC, 1.0, -1.0, "cplx", "so3"),
        "os2":           (40, 20, 1, 6, 1, 1, CUBIC, 2.0, 9.0, "pad2", "so3"),
        "os1.5-linear":  (36, 24, 1, 5, 1, 1, LINEAR, 1.5, 11.0, "cplx", "so3"),
        # above oversampling 2 the cubic 3D adjoint takes the 256-thread
        # bricks (os2 runs the 512-thread ones)
        "os2.5":         (40, 16, 1, 6, 1, 1, CUBIC, 2.5, 7.0, "cplx", "so3"),
        "batch":         (24, 24, 2, 4, 2, 2, CUBIC, 1.0, 11.0, "cplx", "so3"),
        "batch-bcast":   (20, 22, 3, 3, 1, 1, LINEAR, 1.0, 10.5, "cplx", "so3"),
        "adv-cubic":     (32, 32, 1, 8, 1, 1, CUBIC, 1.0, -1.0, "real", "adv"),
        "adv-linear":    (32, 32, 1, 8, 1, 0, LINEAR, 1.0, -1.0, "cplx", "adv"),
        "ragged":        (40, 37, 1, 4, 1, 1, CUBIC, 40 / 37, 18.0, "cplx", "so3"),
        "mixed-rot":     (24, 24, 2, 4, 2, 1, CUBIC, 1.0, 11.0, "cplx", "so3"),
        "mixed-shift":   (22, 20, 2, 3, 1, 2, LINEAR, 1.1, 9.0, "cplx", "so3"),
        "bcast-cubic":   (20, 22, 3, 3, 1, 1, CUBIC, 1.0, 10.5, "cplx", "so3"),
        "adv-cubic-cplx": (32, 32, 1, 8, 1, 1, CUBIC, 1.0, 15.0, "cplx", "adv"),
        # the shift phase's fp64 turn reduction: shifts of thousands of pixels,
        # and shifts in multiples of N_out / 8 that put the rest r exactly on
        # the ends of its [-1/8, 1/8] interval
        "big-shift":     (32, 32, 1, 6, 1, 1, CUBIC, 1.0, 15.0, "cplx", "so3"),
        "eighth-shift":  (32, 32, 1, 6, 1, 1, LINEAR, 1.0, 15.0, "cplx", "so3"),
    }[name]
    N, n_out, B, P, B_rot, B_shift, interp, os_, cutoff, vk, pk = spec
    if vk == "c1":
        V = synth.make_reference(synth.WORKLOADS["c1"])
    elif vk == "cplx":
        V = complex_normal(rng, (B, N, N, N // 2 + 1))
    elif vk == "real":
        V = np.stack([synth.rfft_spectrum(rng.standard_normal((N, N, N)).astype(np.float32), 3) for _ in range(B)])
    elif vk == "pad2":
        V = np.stack([synth.rfft_spectrum(synth.blob_volume(rng, N // 2, 12), 3, pad_to=N) for _ in range(B)])
    if pk == "c1":
        R = synth.make_rotations(synth.WORKLOADS["c1"])
    elif pk == "adv":
        R = adversarial_rotations(rng)[None]
    else:
        R = np.stack([synth.uniform_rotations(rng, P) for _ in range(B_rot)])
    s = None if B_shift == 0 else rng.uniform(-4, 4, (B_shift, P, 2)).astype(np.float32)
    if name == "big-shift":
        s = rng.uniform(-3000, 3000, (B_shift, P, 2)).astype(np.float32)
    elif name == "eighth-shift":
        s = (rng.integers(-40, 41, (B_shift, P, 2)) * (n_out / 8)).astype(np.float32)
    G = complex_normal(rng, (B, P, n_out, n_out // 2 + 1))
    return dict(V=V.astype(np.complex64), R=R.astype(np.float32), s=s, G=G, N=N, n_out=n_out,
                interp=interp, os=np.float32(os_), cutoff=np.float32(cutoff))


CASES3 = ["c1", "c1-cubic", "odd-nocut", "os2", "os1.5-linear", "os2.5", "batch", "batch-bcast",
          "adv-cubic", "adv-linear", "ragged", "mixed-rot", "mixed-shift", "bcast-cubic", "adv-cubic-cplx",
          "big-shift", "eighth-shift"]


def _dev(c):
    from cryo_em_fourier_amd import _lib  # noqa: F401  (loads the library)

    s = None if c["s"] is None else to_dev(c["s"])
    return to_dev(c["V"]), to_dev(c["R"]), s, to_dev(c["G"])


@pytest.mark.parametrize("name", CASES3)
def test_project_3d_matches_oracle(name):
    from cryo_em_fourier_amd import tp_project_3d

    c = case3d(name)
    log(f"[project_3d] {name} V{c['V'].shape} R{c['R'].shape}")
    V, R, s, _ = _dev(c)
    out = tp_project_3d(V, R, s, c["n_out"], c["interp"], float(c["os"]), float(c["cutoff"])).cpu().numpy()
    ref = oracle.project(c["V"], c["R"], c["s"], c["n_out"], c["interp"], c["os"], c["cutoff"])
    assert_parity(out, ref, f"project_3d {name}")


@pytest.mark.parametrize("name", CASES3)
def test_backproject_3d_matches_oracle(name):
    from cryo_em_fourier_amd import tp_backproject_3d

    c = case3d(name)
    log(f"[backproject_3d] {name}")
    _, R, s, G = _dev(c)
    got = tp_backproject_3d(G, R, s, c["N"], c["interp"], float(c["os"]), float(c["cutoff"])).cpu().numpy()
    ref = oracle.backproject(c["G"], c["R"], c["s"], c["N"], c["interp"], c["os"], c["cutoff"])
    assert_parity(got, ref, f"backproject_3d {name}")


@pytest.mark.parametrize("name", CASES3)
def test_grad_pose_3d_matches_oracle(name):
    from cryo_em_fourier_amd import tp_grad_pose

    c = case3d(name)
    log(f"[grad_pose_3d] {name}")
    V, R, s, G = _dev(c)
    gr, gs = tp_grad_pose(V, G, R, s, c["interp"], float(c["os"]), float(c["cutoff"]))
    dR, ds = oracle.grad_pose(c["V"], c["G"], c["R"], c["s"], c["n_out"], c["interp"], c["os"], c["cutoff"])
    # adv-linear: every pose, including those whose samples sit on the linear
    # kernel's kinks (integer coordinates, folded or not), where both sides
    # take the right derivative in p
    assert_parity(gr.cpu().numpy(), dR, f"grad_rot {name}")
    assert_parity(gs.cpu().numpy(), ds, f"grad_shift {name}")


@pytest.mark.parametrize("name", CASES3)
def test_project_3d_jac_and_grad_pose_jac_match_oracle(name):
    """The Jacobian-saving forward gives the forward's values, and the pose
    gradients taken from its Jacobian give the oracle's gradients."""
    from cryo_em_fourier_amd import tp_grad_pose_jac, tp_project_3d_jac

    c = case3d(name)
    log(f"[project_3d_jac + grad_pose_jac] {name}")
    V, R, s, G = _dev(c)
    out, jac = tp_project_3d_jac(V, R, s, c["n_out"], c["interp"], float(c["os"]), float(c["cutoff"]))
    ref = oracle.project(c["V"], c["R"], c["s"], c["n_out"], c["interp"], c["os"], c["cutoff"])
    assert_parity(out.cpu().numpy(), ref, f"project_3d_jac {name}")
    B_shift = 1 if c["s"] is None else c["s"].shape[0]
    gr, gs = tp_grad_pose_jac(G, out, jac, c["R"].shape[0], B_shift, float(c["os"]), float(c["cutoff"]))
    dR, ds = oracle.grad_pose(c["V"], c["G"], c["R"], c["s"], c["n_out"], c["interp"], c["os"], c["cutoff"])
    gr, gs = gr.cpu().numpy(), gs.cpu().numpy()
    assert_parity(gr, dR, f"grad_rot (jac) {name}")
    assert_parity(gs, ds, f"grad_shift (jac) {name}")
    assert not gr[:, :, 2].any(), "the last row of dL/dR is 0"


@pytest.mark.parametrize("name", CASES3)
def test_backward_3d_jac_matches_oracle(name):
    """The fused backward gives the oracle's adjoint and pose gradients (the
    values of tp_backproject_3d and tp_grad_pose_jac)."""
    from cryo_em_fourier_amd import tp_backward_3d_jac, tp_project_3d_jac

    c = case3d(name)
    log(f"[backward_3d_jac] {name}")
    V, R, s, G = _dev(c)
    out, jac = tp_project_3d_jac(V, R, s, c["n_out"], c["interp"], float(c["os"]), float(c["cutoff"]))
    d_vol, gr, gs = tp_backward_3d_jac(G, out, jac, R, s, c["N"], c["interp"], float(c["os"]), float(c["cutoff"]))
    ref = oracle.backproject(c["G"], c["R"], c["s"], c["N"], c["interp"], c["os"], c["cutoff"])
    assert_parity(d_vol.cpu().numpy(), ref, f"backward_3d_jac volume {name}")
    dR, ds = oracle.grad_pose(c["V"], c["G"], c["R"], c["s"], c["n_out"], c["interp"], c["os"], c["cutoff"])
    gr, gs = gr.cpu().numpy(), gs.cpu().numpy()
    assert_parity(gr, dR, f"grad_rot (backward_3d_jac) {name}")
    assert_parity(gs, ds, f"grad_shift (backward_3d_jac) {name}")


# ------------------------------------------------------------------- 2D

@functools.lru_cache(maxsize=None)
def case2d(name):
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    spec = {
        # N, n_out, B, P, per-image poses?, shift?, interp, os, cutoff, vol
        "c2-small":   (32, 32, 8, 1, True, True, CUBIC, 1.0, 16.0, "images"),
        "multipose":  (24, 24, 2, 5, False, True, LINEAR, 1.0, -1.0, "cplx"),
        "os2":        (48, 24, 3, 2, True, True, CUBIC, 2.0, 11.0, "pad2"),
        "odd":        (31, 31, 2, 3, True, True, CUBIC, 1.0, 15.0, "cplx"),
        "adv":        (32, 32, 1, 6, False, False, CUBIC, 1.0, -1.0, "cplx"),
        "adv-linear": (32, 32, 1, 6, False, True, LINEAR, 1.0, 15.0, "cplx"),
    }[name]
    N, n_out, B, P, per_img, shifted, interp, os_, cutoff, vk = spec
    if vk == "images":
        V = synth.rfft_spectrum(synth.blob_images(rng, B, N, 20), 2)
    elif vk == "pad2":
        V = synth.rfft_spectrum(synth.blob_images(rng, B, N // 2, 10), 2, pad_to=N)
    else:
        V = complex_normal(rng, (B, N, N // 2 + 1))
    Br = B if per_img else 1
    if name.startswith("adv"):
        ang = np.array([0.0, math.pi / 2, math.pi, 1.5 * math.pi, math.pi / 2 + 1e-3, 0.3])
    else:
        ang = rng.uniform(0, 2 * math.pi, Br * P)
    R = synth.inplane_rotations(ang).reshape(Br, P, 2, 2)
    s = rng.uniform(-5, 5, (Br, P, 2)).astype(np.float32) if shifted else None
    G = complex_normal(rng, (B, P, n_out, n_out // 2 + 1))
    return dict(V=V.astype(np.complex64), R=R, s=s, G=G, N=N, n_out=n_out, interp=interp,
                os=np.float32(os_), cutoff=np.float32(cutoff))


CASES2 = ["c2-small", "multipose", "os2", "odd", "adv", "adv-linear"]


@pytest.mark.parametrize("name", CASES2)
def test_project_2d_matches_oracle(name):
    from cryo_em_fourier_amd import tp_project_2d

    c = case2d(name)
    log(f"[project_2d] {name}")
    V, R, s, _ = _dev(c)
    out = tp_project_2d(V, R, s, c["n_out"], c["interp"], float(c["os"]), float(c["cutoff"])).cpu().numpy()
    ref = oracle.project(c["V"], c["R"], c["s"], c["n_out"], c["interp"], c["os"], c["cutoff"])
    assert_parity(out, ref, f"project_2d {name}")


@pytest.mark.parametrize("name", CASES2)
def test_backproject_2d_matches_oracle(name):
    from cryo_em_fourier_amd import tp_backproject_2d

    c = case2d(name)
    log(f"[backproject_2d] {name}")
    _, R, s, G = _dev(c)
    got = tp_backproject_2d(G, R, s, c["N"], c["interp"], float(c["os"]), float(c["cutoff"])).cpu().numpy()
    ref = oracle.backproject(c["G"], c["R"], c["s"], c["N"], c["interp"], c["os"], c["cutoff"])
    assert_parity(got, ref, f"backproject_2d {name}")


@pytest.mark.parametrize("name", CASES2)
def test_grad_pose_2d_matches_oracle(name):
    from cryo_em_fourier_amd import tp_grad_pose

    c = case2d(name)
    log(f"[grad_pose_2d] {name}")
    V, R, s, G = _dev(c)
    gr, gs = tp_grad_pose(V, G, R, s, c["interp"], float(c["os"]), float(c["cutoff"]))
    dR, ds = oracle.grad_pose(c["V"], c["G"], c["R"], c["s"], c["n_out"], c["interp"], c["os"], c["cutoff"])
    assert_parity(gr.cpu().numpy(), dR, f"grad_rot2d {name}")
    assert_parity(gs.cpu().numpy(), ds, f"grad_shift2d {name}")


# ------------------------------------------------------- properties on the GPU

def test_forward_is_deterministic_and_adjoint_repeatable():
    from cryo_em_fourier_amd import tp_backproject_3d, tp_project_3d

    c = case3d("odd-nocut")
    V, R, s, G = _dev(c)
    a = tp_project_3d(V, R, s, c["n_out"], c["interp"], 1.0, -1.0)
    b = tp_project_3d(V, R, s, c["n_out"], c["interp"], 1.0, -1.0)
    assert bool((a == b).all())
    x = tp_backproject_3d(G, R, s, c["N"], c["interp"], 1.0, -1.0).cpu().numpy()
    y = tp_backproject_3d(G, R, s, c["N"], c["interp"], 1.0, -1.0).cpu().numpy()
    rel, mabs = rel_errors(x, y)
    assert rel <= 1e-6 and mabs <= 1e-6


@pytest.mark.parametrize("ndim", [2, 3])
def test_adjoint_identity_on_gpu(ndim):
    """Re<P x, y> = Re<x, P^T y> with the GPU's forward and adjoint."""
    from cryo_em_fourier_amd import tp_backproject_2d, tp_backproject_3d, tp_project_2d, tp_project_3d

    c = case3d("batch") if ndim == 3 else case2d("os2")
    V, R, s, G = _dev(c)
    fwd, adj = (tp_project_3d, tp_backproject_3d) if ndim == 3 else (tp_project_2d, tp_backproject_2d)
    Px = fwd(V, R, s, c["n_out"], c["interp"], float(c["os"]), float(c["cutoff"])).cpu().numpy()
    PtG = adj(G, R, s, c["N"], c["interp"], float(c["os"]), float(c["cutoff"])).cpu().numpy()
    lhs = np.real(np.vdot(Px.astype(np.complex128).ravel(), c["G"].astype(np.complex128).ravel()))
    rhs = np.real(np.vdot(c["V"].astype(np.complex128).ravel(), PtG.astype(np.complex128).ravel()))
    scale = np.linalg.norm(Px.ravel()) * np.linalg.norm(c["G"].ravel())
    log(f"  adjoint identity {ndim}D: {lhs:.6e} vs {rhs:.6e} (scale {scale:.3e})")
    assert abs(lhs - rhs) <= 1e-6 * scale


@pytest.mark.parametrize("save_jacobian", [True, False])
def test_autograd_matches_direct_calls(save_jacobian):
    import torch

    from cryo_em_fourier_amd import project_3d, tp_backproject_3d, tp_grad_pose

    c = case3d("batch")
    V, R, s, G = _dev(c)
    Vg, Rg, sg = V.clone().requires_grad_(), R.clone().requires_grad_(), s.clone().requires_grad_()
    out = project_3d(Vg, Rg, sg, c["n_out"], c["interp"], float(c["os"]), float(c["cutoff"]),
                     save_jacobian=save_jacobian)
    loss = torch.sum((torch.conj(G) * out).real)
    loss.backward()
    dV = tp_backproject_3d(G, R, s, c["N"], c["interp"], float(c["os"]), float(c["cutoff"]))
    dR, ds = tp_grad_pose(V, G, R, s, c["interp"], float(c["os"]), float(c["cutoff"]))
    assert_parity(Vg.grad.cpu().numpy(), dV.cpu().numpy(), "autograd dV")
    assert_parity(Rg.grad.cpu().numpy(), dR.cpu().numpy(), "autograd dR")
    assert_parity(sg.grad.cpu().numpy(), ds.cpu().numpy(), "autograd ds")


def test_empty_cutoff_and_edge_sizes():
    """cutoff 0 keeps only the DC term; N = 1 and N_out = 1 boxes work."""
    from cryo_em_fourier_amd import tp_backproject_3d, tp_grad_pose, tp_project_3d

    c = case3d("odd-nocut")
    V, R, s, G = _dev(c)
    out = tp_project_3d(V, R, s, c["n_out"], c["interp"], 1.0, 0.0).cpu().numpy()
    ref = oracle.project(c["V"], c["R"], c["s"], c["n_out"], c["interp"], 1.0, 0.0)
    assert_parity(out, ref, "cutoff 0")
    assert np.count_nonzero(out) <= out.shape[1]
    # N_out = 1: only the DC output
    out1 = tp_project_3d(V, R, s, 1, c["interp"], 1.0, -1.0).cpu().numpy()
    ref1 = oracle.project(c["V"], c["R"], c["s"], 1, c["interp"], 1.0, -1.0)
    assert_parity(out1, ref1, "N_out 1")
    G1 = to_dev(c["G"][:, :, :1, :1].copy())
    a1 = tp_backproject_3d(G1, R, s, c["N"], c["interp"], 1.0, -1.0).cpu().numpy()
    r1 = oracle.backproject(c["G"][:, :, :1, :1], c["R"], c["s"], c["N"], c["interp"], 1.0, -1.0)
    assert_parity(a1, r1, "backproject N_out 1")
    # a 1-voxel reference
    V1 = to_dev(c["V"][:, :1, :1, :1].copy())
    o = tp_project_3d(V1, R, s, 6, c["interp"], 1.0, -1.0).cpu().numpy()
    r = oracle.project(c["V"][:, :1, :1, :1], c["R"], c["s"], 6, c["interp"], 1.0, -1.0)
    assert_parity(o, r, "N 1")
    gr, gs = tp_grad_pose(V, G, R, s, c["interp"], 1.0, 0.0)
    assert np.all(gr.cpu().numpy() == 0) and np.all(gs.cpu().numpy() == 0)


def test_jacobian_path_edge_cases():
    """The saved-Jacobian pair at cutoff 0 (DC only: zero pose gradients),
    N_out = 1, no shift with a pose broadcast over the batch, and one
    gradient requested at a time."""
    from cryo_em_fourier_amd import tp_grad_pose_jac, tp_project_3d_jac

    c = case3d("odd-nocut")
    V, R, s, G = _dev(c)
    log("[jacobian edge] cutoff 0")
    out, jac = tp_project_3d_jac(V, R, s, c["n_out"], c["interp"], 1.0, 0.0)
    assert_parity(out.cpu().numpy(), oracle.project(c["V"], c["R"], c["s"], c["n_out"], c["interp"], 1.0, 0.0),
                  "jac forward cutoff 0")
    gr, gs = tp_grad_pose_jac(G, out, jac, 1, 1, 1.0, 0.0)
    assert not gr.cpu().numpy().any() and not gs.cpu().numpy().any()
    log("[jacobian edge] N_out 1")
    out1, jac1 = tp_project_3d_jac(V, R, s, 1, c["interp"], 1.0, -1.0)
    assert_parity(out1.cpu().numpy(), oracle.project(c["V"], c["R"], c["s"], 1, c["interp"], 1.0, -1.0),
                  "jac forward N_out 1")
    G1 = to_dev(c["G"][:, :, :1, :1].copy())
    gr, gs = tp_grad_pose_jac(G1, out1, jac1, 1, 1, 1.0, -1.0)
    dR, ds = oracle.grad_pose(c["V"], c["G"][:, :, :1, :1], c["R"], c["s"], 1, c["interp"], 1.0, -1.0)
    # the DC output has k = 0: every pose gradient is 0
    assert not gr.cpu().numpy().any() and not np.asarray(dR).any()
    log("[jacobian edge] batch 2, broadcast pose, no shift, one gradient at a time")
    b = case3d("batch-bcast")
    Vb, Rb, _, Gb = _dev(b)
    outb, jacb = tp_project_3d_jac(Vb, Rb, None, b["n_out"], b["interp"], float(b["os"]), float(b["cutoff"]))
    dR, ds = oracle.grad_pose(b["V"], b["G"], b["R"], None, b["n_out"], b["interp"], b["os"], b["cutoff"])
    gr, none_s = tp_grad_pose_jac(Gb, outb, jacb, 1, 1, float(b["os"]), float(b["cutoff"]), want_shift=False)
    assert none_s is None
    assert_parity(gr.cpu().numpy(), dR, "jac grad_rot broadcast")
    none_r, gs = tp_grad_pose_jac(Gb, outb, jacb, 1, b["V"].shape[0], float(b["os"]), float(b["cutoff"]),
                                  want_rot=False)
    assert none_r is None
    dR2, ds2 = oracle.grad_pose(b["V"], b["G"], b["R"], np.zeros((b["V"].shape[0], b["R"].shape[1], 2), np.float32),
                                b["n_out"], b["interp"], b["os"], b["cutoff"])
    assert_parity(gs.cpu().numpy(), ds2, "jac grad_shift per batch entry")


def test_fused_backward_edge_cases():
    """tp_backward_3d_jac at cutoff 0, N_out = 1, a pose broadcast over the
    batch without a shift (grad_shift per batch entry), one gradient at a
    time, and none (the plain adjoint)."""
    from cryo_em_fourier_amd import tp_backward_3d_jac, tp_project_3d_jac

    c = case3d("odd-nocut")
    V, R, s, G = _dev(c)
    for n_out, cut in ((c["n_out"], 0.0), (1, -1.0)):
        log(f"[fused edge] N_out {n_out} cutoff {cut}")
        out, jac = tp_project_3d_jac(V, R, s, n_out, c["interp"], 1.0, cut)
        Gc = to_dev(c["G"][:, :, :n_out, :n_out // 2 + 1].copy())
        vol, gr, gs = tp_backward_3d_jac(Gc, out, jac, R, s, c["N"], c["interp"], 1.0, cut)
        ref = oracle.backproject(c["G"][:, :, :n_out, :n_out // 2 + 1], c["R"], c["s"], c["N"], c["interp"], 1.0, cut)
        assert_parity(vol.cpu().numpy(), ref, f"fused volume N_out {n_out} cutoff {cut}")
        # only the DC output is kept: k = 0 gives zero pose gradients
        assert not gr.cpu().numpy().any() and not gs.cpu().numpy().any()
    log("[fused edge] batch 2, broadcast pose, no shift, one gradient at a time, none")
    b = case3d("batch-bcast")
    Vb, Rb, _, Gb = _dev(b)
    args = (b["N"], b["interp"], float(b["os"]), float(b["cutoff"]))
    outb, jacb = tp_project_3d_jac(Vb, Rb, None, b["n_out"], b["interp"], float(b["os"]), float(b["cutoff"]))
    ref = oracle.backproject(b["G"], b["R"], None, *args)
    dR, _ = oracle.grad_pose(b["V"], b["G"], b["R"], None, b["n_out"], b["interp"], b["os"], b["cutoff"])
    nb = b["V"].shape[0]
    _, ds = oracle.grad_pose(b["V"], b["G"], b["R"], np.zeros((nb, b["R"].shape[1], 2), np.float32), b["n_out"],
                             b["interp"], b["os"], b["cutoff"])
    vol, gr, none_s = tp_backward_3d_jac(Gb, outb, jacb, Rb, None, *args, want_shift=False)
    assert none_s is None
    assert_parity(vol.cpu().numpy(), ref, "fused volume broadcast")
    assert_parity(gr.cpu().numpy(), dR, "fused grad_rot broadcast")
    vol, none_r, gs = tp_backward_3d_jac(Gb, outb, jacb, Rb, None, *args, want_rot=False, B_shift=nb)
    assert none_r is None
    assert_parity(gs.cpu().numpy(), ds, "fused grad_shift per batch entry")
    vol, none_r, none_s = tp_backward_3d_jac(Gb, outb, jacb, Rb, None, *args, want_rot=False, want_shift=False)
    assert none_r is None and none_s is None
    assert_parity(vol.cpu().numpy(), ref, "fused volume without gradients")


def test_nonfinite_rotation_reads_zero():
    """Poses whose sample points are beyond 2^30 or not finite read 0 and add
    nothing: forward, adjoint and pose gradients of every path, fused
    included, against the oracle (whose gradients for them are 0)."""
    from cryo_em_fourier_amd import (tp_backproject_3d, tp_backward_3d_jac, tp_grad_pose, tp_grad_pose_jac,
                                     tp_project_3d, tp_project_3d_jac)

    c = case3d("odd-nocut")
    R = np.stack([np.eye(3) * 1e12, np.full((3, 3), np.nan), np.eye(3)]).astype(np.float32)[None]
    V, Rd = to_dev(c["V"]), to_dev(R)
    out = tp_project_3d(V, Rd, None, 12, CUBIC, 1.0, -1.0).cpu().numpy()
    ref = oracle.project(c["V"], R, None, 12, CUBIC, 1.0, -1.0)
    assert np.all(np.isfinite(out))
    assert_parity(out, ref, "non-finite rotations")
    G = complex_normal(np.random.default_rng(5), (1, 3, 12, 7))
    Gd = to_dev(G)
    A = oracle.backproject(G, R, None, c["N"], CUBIC, 1.0, -1.0)
    dR, _ = oracle.grad_pose(c["V"], G, R, None, 12, CUBIC, 1.0, -1.0)
    assert_parity(tp_backproject_3d(Gd, Rd, None, c["N"], CUBIC, 1.0, -1.0).cpu().numpy(), A, "adjoint, non-finite")
    gr, _ = tp_grad_pose(V, Gd, Rd, None, CUBIC, 1.0, -1.0)
    assert_parity(gr.cpu().numpy(), dR, "grad_rot, non-finite")
    out_j, jac = tp_project_3d_jac(V, Rd, None, 12, CUBIC, 1.0, -1.0)
    assert np.all(np.isfinite(jac.cpu().numpy()))
    assert_parity(out_j.cpu().numpy(), ref, "jac forward, non-finite")
    gr, _ = tp_grad_pose_jac(Gd, out_j, jac, 1, 1, 1.0, -1.0)
    assert_parity(gr.cpu().numpy(), dR, "grad_rot (jac), non-finite")
    vol, gr, gs = tp_backward_3d_jac(Gd, out_j, jac, Rd, None, c["N"], CUBIC, 1.0, -1.0)
    assert_parity(vol.cpu().numpy(), A, "fused volume, non-finite")
    assert_parity(gr.cpu().numpy(), dR, "fused grad_rot, non-finite")
    assert not gr.cpu().numpy()[0, :2].any() and np.all(np.isfinite(gs.cpu().numpy()))


@pytest.mark.parametrize("N", [8, 9, 16])
@pytest.mark.parametrize("interp", [LINEAR, CUBIC])
def test_taps_at_the_end_of_the_reference(N, interp):
    """Sample points on the last stored row (y = z = -1) next to x = N/2,
    whose tap windows reach past the end of the reference buffer."""
    from cryo_em_fourier_amd import tp_project_2d, tp_project_3d

    rng = np.random.default_rng(N * 10 + interp)
    xm = N // 2
    pts = [(xm - 0.5, -1.0, -1.0), (xm + 0.0, -1.0, -1.0), (xm - 0.25, -1.0, -1.0), (xm - 1.0, -1.0, -1.0),
           (-(xm - 0.5), 1.0, 1.0), (xm - 0.5, -1.5, -1.0)]
    R = np.zeros((1, len(pts), 3, 3), np.float32)
    for i, p in enumerate(pts):
        R[0, i, 0] = p                       # output (kx=1, ky=0) samples p
        R[0, i, 1] = (p[0] * 0.5, p[1], p[2])  # output (kx=0, ky=1) samples this
    V = complex_normal(rng, (1, N, N, N // 2 + 1))
    out = tp_project_3d(to_dev(V), to_dev(R), None, 4, interp, 1.0, -1.0).cpu().numpy()
    ref = oracle.project(V, R, None, 4, interp, 1.0, -1.0)
    assert_parity(out, ref, f"end-of-buffer 3D N={N}")
    R2 = np.ascontiguousarray(R[:, :, :2, :2])
    V2 = complex_normal(rng, (1, N, N // 2 + 1))
    out = tp_project_2d(to_dev(V2), to_dev(R2), None, 4, interp, 1.0, -1.0).cpu().numpy()
    ref = oracle.project(V2, R2, None, 4, interp, 1.0, -1.0)
    assert_parity(out, ref, f"end-of-buffer 2D N={N}")


# ------------------------------------------- the adjoint's fixed-point groups

def _ramp_upstream(rng, B, P, n_out, period=60):
    """Dense complex upstream gradient whose per-pose amplitude climbs from
    1e-3 to 1 over `period` consecutive poses, then starts again: a brick's
    group of 16 crossing poses then usually holds more than twice the
    previous group's largest value (its fixed-point quantum is redone), and
    after each restart a group is far below its predecessor."""
    G = complex_normal(rng, (B, P, n_out, n_out // 2 + 1))
    amp = 10.0 ** (-3.0 + 3.0 * ((np.arange(P) % period) / (period - 1)))
    return (G * amp[None, :, None, None]).astype(np.complex64)


@functools.lru_cache(maxsize=None)
def dense_case(P):
    rng = np.random.default_rng(4800 + P)
    N = 48
    V = synth.rfft_spectrum(synth.blob_volume(rng, N, 30), 3)[None].astype(np.complex64)
    R = synth.uniform_rotations(rng, P)[None]
    s = rng.uniform(-4, 4, (1, P, 2)).astype(np.float32)
    G = _ramp_upstream(rng, 1, P, N)
    return dict(V=V, R=R, s=s, G=G, N=N, n_out=N, interp=CUBIC, os=1.0, cutoff=23.0)


@pytest.mark.parametrize("P", [240, 600])
def test_adjoint_many_poses_per_brick_dense(P):
    """Box 48 with 240 or 600 poses and a dense upstream gradient: every brick
    near the origin takes 15 to 38 groups of 16 poses (600 poses also split
    them into pose chunks merged with atomics), carrying the quantum from
    group to group and redoing groups that exceed it.  Element by element
    against the oracle, for the adjoint and the fused backward's volume."""
    from cryo_em_fourier_amd import tp_backproject_3d, tp_backward_3d_jac, tp_project_3d_jac

    c = dense_case(P)
    log(f"[adjoint dense] N={c['N']} P={P}")
    V, R, s, G = to_dev(c["V"]), to_dev(c["R"]), to_dev(c["s"]), to_dev(c["G"])
    got = tp_backproject_3d(G, R, s, c["N"], c["interp"], c["os"], c["cutoff"]).cpu().numpy()
    ref = oracle.backproject(c["G"], c["R"], c["s"], c["N"], c["interp"], c["os"], c["cutoff"])
    assert_parity(got, ref, f"backproject_3d dense P={P}")
    out, jac = tp_project_3d_jac(V, R, s, c["n_out"], c["interp"], c["os"], c["cutoff"])
    d_vol, gr, gs = tp_backward_3d_jac(G, out, jac, R, s, c["N"], c["interp"], c["os"], c["cutoff"])
    assert_parity(d_vol.cpu().numpy(), ref, f"backward_3d_jac volume dense P={P}")
    dR, ds = oracle.grad_pose(c["V"], c["G"], c["R"], c["s"], c["n_out"], c["interp"], c["os"], c["cutoff"])
    assert_parity(gr.cpu().numpy(), dR, f"grad_rot (backward_3d_jac) dense P={P}")
    assert_parity(gs.cpu().numpy(), ds, f"grad_shift (backward_3d_jac) dense P={P}")


# ------------------------------------------------- non-finite upstream values

def _nonfinite_parity(got, ref, what):
    """Non-finite entries where and only where the oracle has them; the
    finite rest within the parity bar."""
    with np.errstate(invalid="ignore"):
        bad_ref = ~np.isfinite(ref)
        bad_got = ~np.isfinite(got)
    log(f"  {what}: {int(bad_ref.sum())} non-finite entries in the oracle, {int(bad_got.sum())} on the GPU")
    assert bad_ref.any(), "the case must reach the output"
    assert np.array_equal(bad_ref, bad_got), f"{what}: non-finite entries differ"
    assert_parity(np.where(bad_got, 0, got), np.where(bad_ref, 0, ref), f"{what} (finite entries)")


@pytest.mark.parametrize("ndim,N", [(3, 24), (3, 48), (2, 24)])
def test_adjoint_propagates_nonfinite_upstream(ndim, N):
    """A NaN and an Inf in the upstream gradient make the voxels their
    stencils reach non-finite (the oracle's sums there are NaN or +-Inf; the
    adjoint writes NaN), in the adjoint and the fused backward; everything
    else is unaffected.  At N = 48 the central 16^3 bricks are interior
    (guards inside the stored range), so the non-finite values meet the
    bank-ranked spread of the lowest and of the other x bricks."""
    import warnings

    from cryo_em_fourier_amd import (tp_backproject_2d, tp_backproject_3d, tp_backward_3d_jac,
                                     tp_project_3d_jac)

    rng = np.random.default_rng(77 + ndim + N)
    P = 6
    if ndim == 3:
        V = complex_normal(rng, (1, N, N, N // 2 + 1))
        R = synth.uniform_rotations(rng, P)[None]
    else:
        V = complex_normal(rng, (1, N, N // 2 + 1))
        R = synth.inplane_rotations(rng.uniform(0, 2 * math.pi, P)).reshape(1, P, 2, 2)
    s = rng.uniform(-3, 3, (1, P, 2)).astype(np.float32)
    G = complex_normal(rng, (1, P, N, N // 2 + 1))
    G[0, 1, 3, 5] = np.nan                       # kx = 5, ky = 3
    G[0, 4, N - 7, 0] = np.complex64(np.inf)     # kx = 0 column, ky = -7: real output and its mirror
    G[0, 5, 10, 2] = np.complex64(complex(1.0, -np.inf))
    with warnings.catch_warnings():
        warnings.simplefilter("ignore", RuntimeWarning)
        ref = oracle.backproject(G, R, s, N, CUBIC, 1.0, 11.0)
    Gd, Rd, sd = to_dev(G), to_dev(R), to_dev(s)
    if ndim == 3:
        got = tp_backproject_3d(Gd, Rd, sd, N, CUBIC, 1.0, 11.0).cpu().numpy()
        _nonfinite_parity(got, ref, "backproject_3d")
        out, jac = tp_project_3d_jac(to_dev(V), Rd, sd, N, CUBIC, 1.0, 11.0)
        d_vol, gr, gs = tp_backward_3d_jac(Gd, out, jac, Rd, sd, N, CUBIC, 1.0, 11.0)
        _nonfinite_parity(d_vol.cpu().numpy(), ref, "backward_3d_jac volume")
        gr, gs = gr.cpu().numpy(), gs.cpu().numpy()
        assert not np.isfinite(gr[0, [1, 4, 5]]).all() and np.isfinite(gr[0, [0, 2, 3]]).all()
        assert not np.isfinite(gs[0, [1, 4, 5]]).all() and np.isfinite(gs[0, [0, 2, 3]]).all()
    else:
        got = tp_backproject_2d(Gd, Rd, sd, N, CUBIC, 1.0, 11.0).cpu().numpy()
        _nonfinite_parity(got, ref, "backproject_2d")
