"""GPU parity of tp_backward_3d, the backward of the 3D projection in one
call with nothing saved by the forward (it runs the adjoint and the
per-output pose-gradient kernels): its volume gradient against the oracle's
adjoint and its rotation and shift gradients against the oracle's pose
gradients, element by element.

Cases: every small parity case of the forward (odd and even boxes,
oversampling 1 / 1.5 / 2, batches with per-entry and broadcast poses and
shifts, adversarial poses on the grid and across x = 0, no cutoff), the
edge cases (cutoff 0, N_out = 1, each output requested alone), a dense
upstream gradient over many poses per brick (fixed-point groups carried,
redone and chunked), non-finite upstream values, and the full workloads in
the benchmark's launch shape.
Bar: relative L2 <= 1e-5 and max-abs <= 1e-4 * max|oracle|.
"""
import warnings

import numpy as np
import pytest

from cryo_em_fourier_amd import synth
from oracle import CUBIC
import oracle

from _gpu import assert_parity, complex_normal, log, to_dev
from test_gpu_parity import CASES3, _dev, _nonfinite_parity, case3d, dense_case

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", CASES3)
def test_backward_3d_matches_oracle(name):
    from cryo_em_fourier_amd import tp_backward_3d

    c = case3d(name)
    log(f"[backward_3d] {name} V{c['V'].shape} R{c['R'].shape}")
    V, R, s, G = _dev(c)
    dv, gr, gs = tp_backward_3d(V, G, R, s, c["interp"], float(c["os"]), float(c["cutoff"]))
    ref = oracle.backproject(c["G"], c["R"], c["s"], c["N"], c["interp"], c["os"], c["cutoff"])
    assert_parity(dv.cpu().numpy(), ref, f"backward_3d volume {name}")
    dR, ds = oracle.grad_pose(c["V"], c["G"], c["R"], c["s"], c["n_out"], c["interp"], c["os"], c["cutoff"])
    gr = gr.cpu().numpy()
    assert_parity(gr, dR, f"backward_3d grad_rot {name}")
    assert_parity(gs.cpu().numpy(), ds, f"backward_3d grad_shift {name}")
    assert not gr[:, :, 2].any(), "the last row of dL/dR is 0"


def test_backward_3d_edge_cases():
    """Cubic: cutoff 0 and N_out = 1 (DC only: zero pose gradients), a pose
    broadcast over the batch without a shift (grad_shift per batch entry),
    and each output requested alone."""
    from cryo_em_fourier_amd import tp_backward_3d

    c = case3d("odd-nocut")
    V, R, s, G = _dev(c)
    for n_out, cut in ((c["n_out"], 0.0), (1, -1.0)):
        log(f"[backward_3d edge] N_out {n_out} cutoff {cut}")
        Gc = c["G"][:, :, :n_out, :n_out // 2 + 1].copy()
        dv, gr, gs = tp_backward_3d(V, to_dev(Gc), R, s, CUBIC, 1.0, cut)
        ref = oracle.backproject(Gc, c["R"], c["s"], c["N"], CUBIC, 1.0, cut)
        assert_parity(dv.cpu().numpy(), ref, f"backward_3d volume N_out {n_out} cutoff {cut}")
        assert not gr.cpu().numpy().any() and not gs.cpu().numpy().any()
    log("[backward_3d edge] batch 3, broadcast pose, no shift, one output at a time")
    b = case3d("bcast-cubic")
    Vb, Rb, _, Gb = _dev(b)
    args = (CUBIC, float(b["os"]), float(b["cutoff"]))
    nb = b["V"].shape[0]
    ref = oracle.backproject(b["G"], b["R"], None, b["N"], *args)
    dR, _ = oracle.grad_pose(b["V"], b["G"], b["R"], None, b["n_out"], *args)
    _, ds = oracle.grad_pose(b["V"], b["G"], b["R"], np.zeros((nb, b["R"].shape[1], 2), np.float32), b["n_out"],
                             *args)
    dv, gr, gs = tp_backward_3d(Vb, Gb, Rb, None, *args, B_shift=nb)
    assert_parity(dv.cpu().numpy(), ref, "backward_3d volume broadcast")
    assert_parity(gr.cpu().numpy(), dR, "backward_3d grad_rot broadcast")
    assert_parity(gs.cpu().numpy(), ds, "backward_3d grad_shift per batch entry")
    dv, none_r, none_s = tp_backward_3d(Vb, Gb, Rb, None, *args, want_rot=False, want_shift=False)
    assert none_r is None and none_s is None
    assert_parity(dv.cpu().numpy(), ref, "backward_3d volume alone")
    none_v, gr, none_s = tp_backward_3d(Vb, Gb, Rb, None, *args, want_vol=False, want_shift=False)
    assert none_v is None and none_s is None
    assert_parity(gr.cpu().numpy(), dR, "backward_3d grad_rot alone")
    none_v, none_r, gs = tp_backward_3d(Vb, Gb, Rb, None, *args, want_vol=False, want_rot=False, B_shift=nb)
    assert none_v is None and none_r is None
    assert_parity(gs.cpu().numpy(), ds, "backward_3d grad_shift alone")


@pytest.mark.parametrize("P", [240, 600])
def test_backward_3d_many_poses_per_brick_dense(P):
    """Dense upstream gradient with ramped per-pose amplitudes at box 48:
    every brick near the origin carries its fixed-point quantum over 15 to 38
    groups, redoes groups that exceed it (their pose terms are discarded with
    them), and 600 poses also split bricks into chunks."""
    from cryo_em_fourier_amd import tp_backward_3d

    c = dense_case(P)
    log(f"[backward_3d dense] N={c['N']} P={P}")
    V, R, s, G = to_dev(c["V"]), to_dev(c["R"]), to_dev(c["s"]), to_dev(c["G"])
    dv, gr, gs = tp_backward_3d(V, G, R, s, c["interp"], c["os"], c["cutoff"])
    ref = oracle.backproject(c["G"], c["R"], c["s"], c["N"], c["interp"], c["os"], c["cutoff"])
    assert_parity(dv.cpu().numpy(), ref, f"backward_3d volume dense P={P}")
    dR, ds = oracle.grad_pose(c["V"], c["G"], c["R"], c["s"], c["n_out"], c["interp"], c["os"], c["cutoff"])
    assert_parity(gr.cpu().numpy(), dR, f"backward_3d grad_rot dense P={P}")
    assert_parity(gs.cpu().numpy(), ds, f"backward_3d grad_shift dense P={P}")


@pytest.mark.parametrize("N", [24, 48])
def test_backward_3d_propagates_nonfinite_upstream(N):
    """A NaN and an Inf upstream: the voxels their stencils reach and the
    gradients of their poses are not finite; everything else matches.  (At
    N = 48 the central bricks take the bank-ranked spread.)"""
    import math

    from cryo_em_fourier_amd import tp_backward_3d

    rng = np.random.default_rng(91 + N)
    P = 6
    V = complex_normal(rng, (1, N, N, N // 2 + 1))
    R = synth.uniform_rotations(rng, P)[None]
    s = rng.uniform(-3, 3, (1, P, 2)).astype(np.float32)
    G = complex_normal(rng, (1, P, N, N // 2 + 1))
    G[0, 1, 3, 5] = np.nan
    G[0, 4, N - 7, 0] = np.complex64(np.inf)
    G[0, 5, 10, 2] = np.complex64(complex(1.0, -math.inf))
    with warnings.catch_warnings():
        warnings.simplefilter("ignore", RuntimeWarning)
        ref = oracle.backproject(G, R, s, N, CUBIC, 1.0, 11.0)
        dR, ds = oracle.grad_pose(V, G, R, s, N, CUBIC, 1.0, 11.0)
    dv, gr, gs = tp_backward_3d(to_dev(V), to_dev(G), to_dev(R), to_dev(s), CUBIC, 1.0, 11.0)
    _nonfinite_parity(dv.cpu().numpy(), ref, "backward_3d volume")
    gr, gs = gr.cpu().numpy(), gs.cpu().numpy()
    bad = [1, 4, 5]
    good = [0, 2, 3]
    # (inf or NaN, by the order in which the infinite terms meet; the
    # oracle's are not finite either)
    assert not np.isfinite(gr[0, bad, :2]).any() and not np.isfinite(gs[0, bad]).any()
    assert not np.isfinite(dR[0, bad, :2]).any() and not np.isfinite(ds[0, bad]).any()
    assert_parity(gr[0, good], dR[0, good], "backward_3d grad_rot (finite poses)")
    assert_parity(gs[0, good], ds[0, good], "backward_3d grad_shift (finite poses)")
