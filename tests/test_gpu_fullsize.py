"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (all poses of the workload in one call).

The oracle cannot run a whole box-256 call, so each workload is checked on
what it can compute one by one, plus properties that hold at any size:

* forward: every output of a few seeded poses against the oracle;
* adjoint and pose gradients: the upstream gradient is zero except on those
  poses, the call still covers all poses; the result must equal the oracle's
  adjoint / gradients of the sampled poses, and every other pose's gradient
  must be exactly zero;
* adjoint identity with a dense upstream gradient (the forward's own output):
  Re<P V, P V> = Re<V, P^T P V>, summed in fp64 on the device.

Also the largest sizes the ABI accepts: a reference entry just under 2 GiB
and an adjoint at N_out = 4095.
"""
import functools

import numpy as np
import pytest

from cryo_em_fourier_amd import synth
import oracle

from _gpu import assert_parity, log, to_dev

pytestmark = pytest.mark.gpu

N_SAMPLE = 4


@functools.lru_cache(maxsize=1)
def workload(key):
    """Inputs of one workload: key = 'c3', 'c4', 'c4-os2', 'c5'."""
    name, _, os_tag = key.partition("-")
    w = synth.WORKLOADS[name]
    os_ = 2 if os_tag == "os2" else 1
    N = w.N * os_
    V = synth.make_reference(w, pad_to=N if os_ != 1 else None)
    R = synth.make_rotations(w)
    s = synth.make_shifts(w)
    rng = np.random.default_rng(9000 + w.cfg_id)
    idx = np.sort(rng.choice(w.P, size=N_SAMPLE, replace=False))
    if name == "c5":
        idx = np.unique(np.concatenate([idx, [0, 63]]))  # both tilt extremes of series 0
    G_sub = synth.make_upstream(w, poses=idx)
    return dict(w=w, N=N, os=float(os_), V=V, R=R, s=s, idx=idx, G_sub=G_sub)


KEYS = ["c3", "c4", "c4-os2", "c5"]


def _sparse_upstream(c):
    """Device upstream gradient over all poses, zero except the sampled ones."""
    import torch

    w = c["w"]
    G = torch.zeros((w.B, w.P, w.N_out, w.N_out // 2 + 1), dtype=torch.complex64, device="cuda")
    G[:, torch.from_numpy(c["idx"]).cuda()] = to_dev(c["G_sub"])
    return G


@pytest.mark.parametrize("key", KEYS)
def test_fullsize_forward_sampled_poses(key):
    from cryo_em_fourier_amd import tp_project_3d

    c = workload(key)
    w = c["w"]
    log(f"[fullsize forward] {key}: ref {c['V'].shape}, {w.P} poses, sampled {c['idx'].tolist()}")
    out = tp_project_3d(to_dev(c["V"]), to_dev(c["R"]), to_dev(c["s"]), w.N_out, w.interp, c["os"], w.cutoff)
    got = out[:, c["idx"]].cpu().numpy()
    ref = oracle.project(c["V"], c["R"][:, c["idx"]], c["s"][:, c["idx"]], w.N_out, w.interp, c["os"], w.cutoff)
    assert_parity(got, ref, f"forward {key}")


@pytest.mark.parametrize("key", KEYS)
def test_fullsize_adjoint_sampled_poses(key):
    from cryo_em_fourier_amd import tp_backproject_3d

    c = workload(key)
    w = c["w"]
    log(f"[fullsize adjoint] {key}: {w.P} poses, upstream nonzero on {c['idx'].tolist()}")
    got = tp_backproject_3d(_sparse_upstream(c), to_dev(c["R"]), to_dev(c["s"]), c["N"], w.interp, c["os"],
                            w.cutoff).cpu().numpy()
    ref = oracle.backproject(c["G_sub"], c["R"][:, c["idx"]], c["s"][:, c["idx"]], c["N"], w.interp, c["os"],
                             w.cutoff)
    assert_parity(got, ref, f"adjoint {key}")


@pytest.mark.parametrize("key", KEYS)
def test_fullsize_grad_pose_sampled_poses(key):
    from cryo_em_fourier_amd import tp_grad_pose

    c = workload(key)
    w = c["w"]
    log(f"[fullsize grad_pose] {key}: {w.P} poses, upstream nonzero on {c['idx'].tolist()}")
    gr, gs = tp_grad_pose(to_dev(c["V"]), _sparse_upstream(c), to_dev(c["R"]), to_dev(c["s"]), w.interp,
                          c["os"], w.cutoff)
    gr, gs = gr.cpu().numpy(), gs.cpu().numpy()
    dR, ds = oracle.grad_pose(c["V"], c["G_sub"], c["R"][:, c["idx"]], c["s"][:, c["idx"]], w.N_out, w.interp,
                              c["os"], w.cutoff)
    assert_parity(gr[:, c["idx"]], dR, f"grad_rot {key}")
    assert_parity(gs[:, c["idx"]], ds, f"grad_shift {key}")
    rest = np.setdiff1d(np.arange(w.P), c["idx"])
    assert not gr[:, rest].any() and not gs[:, rest].any(), "poses with zero upstream must get zero gradients"


def test_streamed_reference_linear_sampled_poses():
    """A reference above the Infinity Cache's 256 MB (box 256 padded to 512:
    539 MB) takes the gathers' other scheduling (the forward without the
    main-first order, the one-tile pose-gradient kernel); the cubic cases
    above cover it for the cubic kernel, this one for the linear kernel:
    forward and pose gradients of the sampled poses against the oracle."""
    from cryo_em_fourier_amd import tp_grad_pose, tp_project_3d

    c = workload("c4-os2")
    w = c["w"]
    assert c["V"][0].nbytes > 256 << 20
    log(f"[streamed reference, linear] c4-os2: ref {c['V'].shape}, sampled {c['idx'].tolist()}")
    lin = oracle.LINEAR
    out = tp_project_3d(to_dev(c["V"]), to_dev(c["R"]), to_dev(c["s"]), w.N_out, lin, c["os"], w.cutoff)
    ref = oracle.project(c["V"], c["R"][:, c["idx"]], c["s"][:, c["idx"]], w.N_out, lin, c["os"], w.cutoff)
    assert_parity(out[:, c["idx"]].cpu().numpy(), ref, "forward c4-os2 linear")
    del out
    gr, gs = tp_grad_pose(to_dev(c["V"]), _sparse_upstream(c), to_dev(c["R"]), to_dev(c["s"]), lin, c["os"],
                          w.cutoff)
    dR, ds = oracle.grad_pose(c["V"], c["G_sub"], c["R"][:, c["idx"]], c["s"][:, c["idx"]], w.N_out, lin, c["os"],
                              w.cutoff)
    assert_parity(gr.cpu().numpy()[:, c["idx"]], dR, "grad_rot c4-os2 linear")
    assert_parity(gs.cpu().numpy()[:, c["idx"]], ds, "grad_shift c4-os2 linear")


@pytest.mark.parametrize("key", KEYS)
def test_fullsize_grad_pose_jac_sampled_poses(key):
    """The Jacobian-saving forward over all poses, then the pose gradients
    from it with the sparse upstream gradient, alone and in the fused backward
    (the benchmark's step) with the adjoint."""
    import torch

    from cryo_em_fourier_amd import tp_backward_3d_jac, tp_grad_pose_jac, tp_project_3d_jac

    c = workload(key)
    w = c["w"]
    log(f"[fullsize grad_pose_jac + backward_3d_jac] {key}: {w.P} poses, upstream nonzero on {c['idx'].tolist()}")
    R, s = to_dev(c["R"]), to_dev(c["s"])
    out, jac = tp_project_3d_jac(to_dev(c["V"]), R, s, w.N_out, w.interp, c["os"], w.cutoff)
    G = _sparse_upstream(c)
    gr, gs = tp_grad_pose_jac(G, out, jac, c["R"].shape[0], c["s"].shape[0], c["os"], w.cutoff)
    vol_f, gr_f, gs_f = tp_backward_3d_jac(G, out, jac, R, s, c["N"], w.interp, c["os"], w.cutoff)
    got = out[:, c["idx"]].cpu().numpy()
    del out, jac, G
    torch.cuda.empty_cache()
    ref = oracle.project(c["V"], c["R"][:, c["idx"]], c["s"][:, c["idx"]], w.N_out, w.interp, c["os"], w.cutoff)
    assert_parity(got, ref, f"forward (jac) {key}")
    dR, ds = oracle.grad_pose(c["V"], c["G_sub"], c["R"][:, c["idx"]], c["s"][:, c["idx"]], w.N_out, w.interp,
                              c["os"], w.cutoff)
    rest = np.setdiff1d(np.arange(w.P), c["idx"])
    for tag, a, b in (("jac", gr, gs), ("fused", gr_f, gs_f)):
        a, b = a.cpu().numpy(), b.cpu().numpy()
        assert_parity(a[:, c["idx"]], dR, f"grad_rot ({tag}) {key}")
        assert_parity(b[:, c["idx"]], ds, f"grad_shift ({tag}) {key}")
        assert not a[:, rest].any() and not b[:, rest].any(), "poses with zero upstream must get zero gradients"
    ref = oracle.backproject(c["G_sub"], c["R"][:, c["idx"]], c["s"][:, c["idx"]], c["N"], w.interp, c["os"],
                             w.cutoff)
    assert_parity(vol_f.cpu().numpy(), ref, f"adjoint (fused) {key}")


@pytest.mark.parametrize("key", KEYS)
def test_fullsize_adjoint_identity_dense(key):
    import torch

    from cryo_em_fourier_amd import tp_backproject_3d, tp_project_3d

    c = workload(key)
    w = c["w"]
    log(f"[fullsize adjoint identity] {key}: {w.P} poses, dense upstream = forward output")
    V, R, s = to_dev(c["V"]), to_dev(c["R"]), to_dev(c["s"])
    out = tp_project_3d(V, R, s, w.N_out, w.interp, c["os"], w.cutoff)
    back = tp_backproject_3d(out, R, s, c["N"], w.interp, c["os"], w.cutoff)
    lhs = torch.view_as_real(out).double().square().sum().item()
    rhs = (torch.view_as_real(V).double() * torch.view_as_real(back).double()).sum().item()
    rel = abs(lhs - rhs) / abs(lhs)
    log(f"  <PV,PV> = {lhs:.10e}  <V,P^T PV> = {rhs:.10e}  rel {rel:.2e}")
    assert rel <= 1e-5


# ------------------------------------------------------------------ 2D (c2)

@functools.lru_cache(maxsize=1)
def workload2d():
    w = synth.WORKLOADS["c2"]
    V = synth.make_reference(w)
    R = synth.make_rotations(w)
    s = synth.make_shifts(w)
    rng = np.random.default_rng(9002)
    idx = np.sort(rng.choice(w.B, size=N_SAMPLE, replace=False))
    G = synth.make_upstream(w)  # [256, 1, 128, 65]: small enough to build whole
    return dict(w=w, V=V, R=R, s=s, idx=idx, G=G)


def test_fullsize_2d_all_entries():
    """c2 in one call: 256 images, one pose each; forward and gradients on
    sampled images, adjoint of sampled images with the rest zero."""
    import torch

    from cryo_em_fourier_amd import tp_backproject_2d, tp_grad_pose, tp_project_2d

    c = workload2d()
    w, idx = c["w"], c["idx"]
    log(f"[fullsize 2D] c2: {w.B} images, sampled {idx.tolist()}")
    V, R, s = to_dev(c["V"]), to_dev(c["R"]), to_dev(c["s"])
    out = tp_project_2d(V, R, s, w.N_out, w.interp, 1.0, w.cutoff).cpu().numpy()
    ref = oracle.project(c["V"][idx], c["R"][idx], c["s"][idx], w.N_out, w.interp, 1.0, w.cutoff)
    assert_parity(out[idx], ref, "forward c2")

    G = torch.zeros((w.B, 1, w.N_out, w.N_out // 2 + 1), dtype=torch.complex64, device="cuda")
    G[torch.from_numpy(idx).cuda()] = to_dev(c["G"][idx])
    got = tp_backproject_2d(G, R, s, w.N, w.interp, 1.0, w.cutoff).cpu().numpy()
    ref = oracle.backproject(c["G"][idx], c["R"][idx], c["s"][idx], w.N, w.interp, 1.0, w.cutoff)
    assert_parity(got[idx], ref, "adjoint c2")
    rest = np.setdiff1d(np.arange(w.B), idx)
    assert not got[rest].any(), "images with zero upstream must get a zero adjoint"

    gr, gs = tp_grad_pose(V, to_dev(c["G"]), R, s, w.interp, 1.0, w.cutoff)
    dR, ds = oracle.grad_pose(c["V"][idx], c["G"][idx], c["R"][idx], c["s"][idx], w.N_out, w.interp, 1.0,
                              w.cutoff)
    assert_parity(gr.cpu().numpy()[idx], dR, "grad_rot c2")
    assert_parity(gs.cpu().numpy()[idx], ds, "grad_shift c2")


# ------------------------------------------------------------ largest sizes

def test_largest_reference_entry():
    """A reference entry just under the 2^31 - 4096 byte limit (N = 812,
    2.147e9 bytes), sampled across its whole extent (os = N / N_out)."""
    from cryo_em_fourier_amd import tp_backproject_3d, tp_grad_pose, tp_project_3d

    N, n_out, P = 812, 96, 3
    assert N * N * (N // 2 + 1) * 8 <= 2**31 - 4096
    rng = np.random.default_rng(812)
    V = ((rng.standard_normal((1, N, N, N // 2 + 1), dtype=np.float32)
          + 1j * rng.standard_normal((1, N, N, N // 2 + 1), dtype=np.float32)) * np.float32(0.7071)).astype(np.complex64)
    R = synth.uniform_rotations(rng, P)[None]
    s = rng.uniform(-4, 4, (1, P, 2)).astype(np.float32)
    G = ((rng.standard_normal((1, P, n_out, n_out // 2 + 1)) + 1j * rng.standard_normal(
        (1, P, n_out, n_out // 2 + 1))) * np.sqrt(0.5)).astype(np.complex64)
    os_ = np.float32(N / n_out)
    log(f"[largest reference] N={N} ({V.nbytes / 2**30:.3f} GiB) N_out={n_out} os={os_}")
    Vd, Rd, sd, Gd = to_dev(V), to_dev(R), to_dev(s), to_dev(G)
    out = tp_project_3d(Vd, Rd, sd, n_out, 1, float(os_), -1.0).cpu().numpy()
    assert_parity(out, oracle.project(V, R, s, n_out, 1, os_, -1.0), "forward N=812")
    gr, gs = tp_grad_pose(Vd, Gd, Rd, sd, 1, float(os_), -1.0)
    dR, ds = oracle.grad_pose(V, G, R, s, n_out, 1, os_, -1.0)
    assert_parity(gr.cpu().numpy(), dR, "grad_rot N=812")
    assert_parity(gs.cpu().numpy(), ds, "grad_shift N=812")
    del Vd
    got = tp_backproject_3d(Gd, Rd, sd, N, 1, float(os_), -1.0).cpu().numpy()
    assert_parity(got, oracle.backproject(G, R, s, N, 1, os_, -1.0), "adjoint N=812")


def test_largest_adjoint_output_box():
    """The adjoint's largest output box, N_out = 4095 (odd): 67 MB per
    projection, ky rows wrapping far from the origin; os = 0.5 and the
    cutoff keep the samples inside a 400^3 reference; linear taps keep the
    oracle quick."""
    from cryo_em_fourier_amd import tp_backproject_3d, tp_project_3d

    N, n_out, P = 400, 4095, 2
    rng = np.random.default_rng(4095)
    V = ((rng.standard_normal((1, N, N, N // 2 + 1), dtype=np.float32)
          + 1j * rng.standard_normal((1, N, N, N // 2 + 1), dtype=np.float32)) * np.float32(0.7071)).astype(np.complex64)
    R = synth.uniform_rotations(rng, P)[None]
    s = rng.uniform(-40, 40, (1, P, 2)).astype(np.float32)
    os_, cutoff = np.float32(0.5), np.float32(390.0)
    G = ((rng.standard_normal((1, P, n_out, n_out // 2 + 1), dtype=np.float32) + 1j * rng.standard_normal(
        (1, P, n_out, n_out // 2 + 1), dtype=np.float32)) * np.float32(0.7071)).astype(np.complex64)
    log(f"[largest adjoint box] N={N} N_out={n_out} os={os_}")
    Rd, sd = to_dev(R), to_dev(s)
    out = tp_project_3d(to_dev(V), Rd, sd, n_out, 0, float(os_), float(cutoff)).cpu().numpy()
    assert_parity(out, oracle.project(V, R, s, n_out, 0, os_, cutoff), "forward N_out=4095")
    got = tp_backproject_3d(to_dev(G), Rd, sd, N, 0, float(os_), float(cutoff)).cpu().numpy()
    assert_parity(got, oracle.backproject(G, R, s, N, 0, os_, cutoff), "adjoint N_out=4095")


# ------------------------------------------------- pose gradients at box 288

@pytest.mark.parametrize("interp,os_,batch", [(1, 1.0, 1), (0, 1.0, 1), (1, 1.2, 2), (0, 1.25, 1)])
def test_grad_pose_box288_against_oracle(interp, os_, batch):
    """Box 288, 260 poses, oversampling 1 to 1.25, one or two batch entries:
    the two-tile pose-gradient kernel on a dense lattice with a ragged last
    tile row.  Every pose is processed; the upstream gradient is nonzero on a
    sample that includes on-grid and x = 0-plane poses (linear kinks at
    integer coordinates: both sides take the right derivative in p)."""
    import torch

    from cryo_em_fourier_amd import tp_grad_pose
    from test_gpu_parity import adversarial_rotations

    N, P = 288, 260
    n_out = int(round(N / os_))
    rng = np.random.default_rng(200 + interp + 10 * batch)
    V = np.stack([synth.rfft_spectrum(synth.blob_volume(rng, int(N / os_) if os_ != 1.0 else N, 60), 3,
                                      pad_to=N if os_ != 1.0 else None) for _ in range(batch)]).astype(np.complex64)
    R = np.stack([synth.uniform_rotations(rng, P) for _ in range(batch)])
    R[:, :8] = adversarial_rotations(rng)
    s = rng.uniform(-6, 6, (batch, P, 2)).astype(np.float32)
    cutoff = np.float32(n_out // 2 - 1)
    idx = np.array([0, 1, 2, 3, 4, 7, 100, 259])
    G_sub = ((rng.standard_normal((batch, len(idx), n_out, n_out // 2 + 1))
              + 1j * rng.standard_normal((batch, len(idx), n_out, n_out // 2 + 1))) * np.sqrt(0.5)).astype(np.complex64)
    log(f"[grad box 288] N={N} P={P} B={batch} interp={interp} os={os_} n_out={n_out}")
    G = torch.zeros((batch, P, n_out, n_out // 2 + 1), dtype=torch.complex64, device="cuda")
    G[:, torch.from_numpy(idx).cuda()] = to_dev(G_sub)
    gr, gs = tp_grad_pose(to_dev(V), G, to_dev(R), to_dev(s), interp, os_, float(cutoff))
    gr, gs = gr.cpu().numpy(), gs.cpu().numpy()
    dR, ds = oracle.grad_pose(V, G_sub, R[:, idx], s[:, idx], n_out, interp, np.float32(os_), cutoff)
    assert_parity(gr[:, idx], dR, f"grad_rot box 288 interp={interp} os={os_}")
    assert_parity(gs[:, idx], ds, f"grad_shift box 288 interp={interp} os={os_}")
    rest = np.setdiff1d(np.arange(P), idx)
    assert not gr[:, rest].any() and not gs[:, rest].any()


@pytest.mark.parametrize("key", KEYS)
def test_fullsize_backward_sampled_poses(key):
    """tp_backward_3d (the backward of the benchmark's step in one call) over all
    poses with the sparse upstream gradient: its volume gradient is the
    oracle's adjoint of the sampled poses, their pose gradients the oracle's,
    every other pose's gradients exactly 0."""
    import torch

    from cryo_em_fourier_amd import tp_backward_3d

    c = workload(key)
    w = c["w"]
    log(f"[fullsize backward_3d] {key}: {w.P} poses, upstream nonzero on {c['idx'].tolist()}")
    dv, gr, gs = tp_backward_3d(to_dev(c["V"]), _sparse_upstream(c), to_dev(c["R"]), to_dev(c["s"]), w.interp,
                                c["os"], w.cutoff)
    dv, gr, gs = dv.cpu().numpy(), gr.cpu().numpy(), gs.cpu().numpy()
    torch.cuda.empty_cache()
    ref = oracle.backproject(c["G_sub"], c["R"][:, c["idx"]], c["s"][:, c["idx"]], c["N"], w.interp, c["os"],
                             w.cutoff)
    assert_parity(dv, ref, f"backward_3d volume {key}")
    dR, ds = oracle.grad_pose(c["V"], c["G_sub"], c["R"][:, c["idx"]], c["s"][:, c["idx"]], w.N_out, w.interp,
                              c["os"], w.cutoff)
    assert_parity(gr[:, c["idx"]], dR, f"backward_3d grad_rot {key}")
    assert_parity(gs[:, c["idx"]], ds, f"backward_3d grad_shift {key}")
    rest = np.setdiff1d(np.arange(w.P), c["idx"])
    assert not gr[:, rest].any() and not gs[:, rest].any(), "poses with zero upstream must get zero gradients"


def test_fullsize_c3_adjoint_dense_all_poses():
    """c3 (box 128, 1024 poses) with a dense upstream gradient on every pose:
    the adjoint and tp_backward_3d in the benchmark's launch shape.
    Volumes element by element against the oracle's adjoint (summed over pose
    chunks in CPU worker processes); tp_backward_3d's pose gradients
    of sampled poses against the oracle's (a pose's gradient depends on its
    own upstream values only).  Every brick near the origin runs dozens of
    fixed-point groups and pose chunks."""
    from _gpu import oracle_backproject_pooled

    from cryo_em_fourier_amd import tp_backproject_3d, tp_backward_3d

    w = synth.WORKLOADS["c3"]
    V, R, s = synth.make_reference(w), synth.make_rotations(w), synth.make_shifts(w)
    G = synth.make_upstream(w, poses=np.arange(w.P))
    log(f"[fullsize adjoint dense] c3: {w.P} poses, dense upstream")
    Gd, Rd, sd = to_dev(G), to_dev(R), to_dev(s)
    got = tp_backproject_3d(Gd, Rd, sd, w.N, w.interp, 1.0, w.cutoff).cpu().numpy()
    dv, gr, gs = tp_backward_3d(to_dev(V), Gd, Rd, sd, w.interp, 1.0, w.cutoff)
    dv, gr, gs = dv.cpu().numpy(), gr.cpu().numpy(), gs.cpu().numpy()
    ref = oracle_backproject_pooled(G, R, s, w.N, w.interp, 1.0, w.cutoff)
    assert_parity(got, ref, "adjoint c3 dense")
    assert_parity(dv, ref, "backward_3d volume c3 dense")
    idx = np.sort(np.random.default_rng(31).choice(w.P, size=6, replace=False))
    dR, ds = oracle.grad_pose(V, G[:, idx], R[:, idx], s[:, idx], w.N_out, w.interp, 1.0, w.cutoff)
    assert_parity(gr[:, idx], dR, "backward_3d grad_rot c3 dense (sampled poses)")
    assert_parity(gs[:, idx], ds, "backward_3d grad_shift c3 dense (sampled poses)")
