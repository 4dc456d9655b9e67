"""Throughput of the Fourier-slice projector's hot path on one MI355X.

One step = the whole path on one batch: forward projection, then the
backward of a loss on its output: the adjoint for the reference gradient
and the rotation + shift gradients, with nothing stored between the two
beyond the forward's output.  By default (``--pose-grads separate``) the
step is tp_project_3d + tp_backproject_3d + tp_grad_pose (the kernels that
tp_backward_3d runs); ``--pose-grads jacobian`` times the path that stores
each output's Jacobian in the forward (tp_project_3d_jac +
tp_backward_3d_jac, 24 extra bytes per output).  The kernels of the other modes ride along in
``extras``.  Default workload
(``c4``): a 256^3 blob phantom (rfft half-spectrum 256x256x129 complex64),
4096 uniform SO(3) poses, shifts U[-10,10] px, Catmull-Rom cubic,
oversampling 1, cutoff 128.

Prints one JSON line:  value = projections/s forward+backward; the forward
rate, per-kernel times, the roofline of the dominant kernel (tap bytes
against the L2 bandwidth from unit counts and clock, with the compulsory
HBM bytes beside it) and the CPU baseline (the fp64 oracle on a bounded
pose sample, timed on the host before the GPU is touched) ride along.
"""
from __future__ import annotations

import argparse
import json
import math
import multiprocessing as mp
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from cryo_em_fourier_amd import synth  # noqa: E402

METRIC = "projections/sec fwd and fwd+bwd, box 256 cubic; % of HBM/L2 roofline"

# MI355X published peaks
HBM_PEAK_GBS = 8000.0
FP32_VECTOR_PEAK_TFLOPS = 157.3
# L2 read bandwidth derived from unit counts and clock:
# 8 XCDs x 16 channels x 128 B/clk x 2.4 GHz
L2_PEAK_GBS = 8 * 16 * 128 * 2.4


def kernel_source_digest() -> str:
    """sha256 over the projector's HIP sources (not the peak probes) with
    comments and blank lines removed: counter data is valid only for this
    code (a comment edit keeps it)."""
    import hashlib
    import re

    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "cryo_em_fourier_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        if f.endswith((".hip", ".h")) and f != "peaks.hip":
            with open(os.path.join(csrc, f), encoding="utf-8") as fh:
                text = re.sub(r"/\*.*?\*/", "", fh.read(), flags=re.S)
            lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
            code = "\n".join(ln for ln in lines if ln.strip())
            h.update(f.encode() + b"\0" + code.encode())
    return h.hexdigest()


def measured_traffic(workload: str, copy_bytes: int) -> dict:
    """Per-launch HBM bytes from the committed counter summary of this
    workload (FETCH_SIZE and WRITE_SIZE, each scaled by what the counter
    read for the calibration copy), or {} when there is none or the kernel
    sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"hbm_traffic_{workload}.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return {}
    if d.get("kernel_source_sha256") != kernel_source_digest() or d.get("copy_bytes") != copy_bytes:
        return {}
    out = {}
    for k, v in d.get("kernels", {}).items():
        out[k] = int(round(v["fetch_kib"] * 1024 * d["fetch_scale"] + v["write_kib"] * 1024 * d["write_scale"]))
    return out


def in_cutoff_count(n_out: int, cutoff: float) -> int:
    kx = np.arange(n_out // 2 + 1)[None, :]
    iy = np.arange(n_out)[:, None]
    ky = np.where(iy <= (n_out - 1) // 2, iy, iy - n_out)
    if cutoff < 0:
        return n_out * (n_out // 2 + 1)
    return int(np.count_nonzero(kx * kx + ky * ky <= cutoff * cutoff))


# ------------------------------------------------------------- CPU baseline

_CPU = {}


def _oracle_worker(idx):
    import oracle

    c = _CPU
    R = c["R"][:, idx]
    s = c["s"][:, idx]
    G = c["G"][:, idx]
    t0 = time.perf_counter()
    oracle.project(c["V"], R, s, c["n_out"], c["interp"], c["os"], c["cutoff"])
    t1 = time.perf_counter()
    oracle.backproject(G, R, s, c["N"], c["interp"], c["os"], c["cutoff"])
    oracle.grad_pose(c["V"], G, R, s, c["n_out"], c["interp"], c["os"], c["cutoff"])
    t2 = time.perf_counter()
    return len(idx), t1 - t0, t2 - t1


def _oracle_worker_2d(idx):
    import oracle

    c = _CPU
    V, R, s, G = c["V"][idx], c["R"][idx], c["s"][idx], c["G"][idx]
    t0 = time.perf_counter()
    oracle.project(V, R, s, c["n_out"], c["interp"], c["os"], c["cutoff"])
    t1 = time.perf_counter()
    oracle.backproject(G, R, s, c["N"], c["interp"], c["os"], c["cutoff"])
    oracle.grad_pose(V, G, R, s, c["n_out"], c["interp"], c["os"], c["cutoff"])
    t2 = time.perf_counter()
    return len(idx), t1 - t0, t2 - t1


def cpu_baseline_2d(V, R, s, G, w: synth.Workload, images_per_worker: int):
    """The oracle's 2D path on a seeded sample of images, in forked workers."""
    ncpu = host_cores()
    workers = max(1, min(CPU_SHARE, ncpu))
    rng = np.random.default_rng(12345)
    n_img = min(w.B, max(images_per_worker, 1) * 32)  # all 256 images at the default: a few seconds
    sample = np.sort(rng.choice(w.B, size=n_img, replace=False))
    _CPU.update(V=V[sample], R=R[sample], s=s[sample], G=G[sample], n_out=w.N_out, N=w.N,
                interp=w.interp, os=1.0, cutoff=w.cutoff)
    chunks = [list(range(i, n_img, workers)) for i in range(workers)]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        res = pool.map(_oracle_worker_2d, [c for c in chunks if c])
    wall = time.perf_counter() - t0
    n = sum(r[0] for r in res)
    fwd = sum(r[1] for r in res)
    bwd = sum(r[2] for r in res)
    return {
        "value": n / wall,
        "unit": "images/s fwd+bwd",
        "cores": workers,
        "host_cores": ncpu,
        "kind": "oracle",
        "sample": f"{n} of {w.B} images (seeded), {workers} single-threaded workers, fork pool "
                  f"({ncpu} host cores visible)",
        "value_1core": n / (fwd + bwd) if fwd + bwd > 0 else None,
        "wall_s": wall,
    }


def bench_2d(args, w: synth.Workload):
    """The 2D -> 2D path on the c2 workload (one in-plane pose per image):
    tp_project_2d + tp_backproject_2d + tp_grad_pose(ndim = 2) per step."""
    V = synth.make_reference(w)
    R = synth.make_rotations(w)
    s = synth.make_shifts(w)
    G = synth.make_upstream(w)
    cpu = None if args.no_cpu_baseline else cpu_baseline_2d(V, R, s, G, w, args.cpu_poses_per_worker)

    import torch

    from cryo_em_fourier_amd import _lib

    L = _lib.lib()
    dev = torch.device("cuda:0")
    Wo = w.N_out // 2 + 1
    Vd, Rd, sd, Gd = (torch.from_numpy(x).to(dev) for x in (V, R, s, G))
    out = torch.empty((w.B, w.P, w.N_out, Wo), dtype=torch.complex64, device=dev)
    dV = torch.empty_like(Vd)
    dR = torch.empty_like(Rd)
    ds = torch.empty_like(sd)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    B, P, N = w.B, w.P, w.N

    def fwd():
        _lib.check(L.tp_project_2d(Vd.data_ptr(), B, N, Rd.data_ptr(), R.shape[0], P, sd.data_ptr(), s.shape[0],
                                   w.N_out, w.interp, 1.0, w.cutoff, out.data_ptr(), sh), "tp_project_2d")

    def adj():
        _lib.check(L.tp_backproject_2d(Gd.data_ptr(), B, P, w.N_out, Rd.data_ptr(), R.shape[0], sd.data_ptr(),
                                       s.shape[0], N, w.interp, 1.0, w.cutoff, dV.data_ptr(), sh),
                   "tp_backproject_2d")

    def grad():
        _lib.check(L.tp_grad_pose(2, Vd.data_ptr(), B, N, Gd.data_ptr(), Rd.data_ptr(), R.shape[0], P,
                                  sd.data_ptr(), s.shape[0], w.N_out, w.interp, 1.0, w.cutoff, dR.data_ptr(),
                                  ds.data_ptr(), sh), "tp_grad_pose")

    kernels = [("project_2d", fwd), ("backproject_2d", adj), ("grad_pose_2d", grad)]
    for _ in range(args.warmup):
        for _, f in kernels:
            f()
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)] for _ in range(args.steps)]
    for k in range(args.steps):
        ev[k][0].record(stream)
        for j, (_, f) in enumerate(kernels):
            f()
            ev[k][j + 1].record(stream)
    torch.cuda.synchronize()
    per = {n: [ev[k][j].elapsed_time(ev[k][j + 1]) for k in range(args.steps)] for j, (n, _) in enumerate(kernels)}
    avg = {n: float(np.mean(v)) for n, v in per.items()}
    ms_step = float(np.mean([ev[k][0].elapsed_time(ev[k][-1]) for k in range(args.steps)]))
    n_c = in_cutoff_count(w.N_out, w.cutoff)
    units = B * P * n_c
    taps = 16 if w.interp == synth.CUBIC else 4
    img_bytes = B * P * w.N_out * Wo * 8
    hbm = {"project_2d": V.nbytes + img_bytes + R.nbytes + s.nbytes,
           "backproject_2d": units * 8 + 2 * V.nbytes + R.nbytes + s.nbytes,
           "grad_pose_2d": V.nbytes + units * 8 + R.nbytes + s.nbytes}
    dom = max(avg, key=avg.get)
    achieved = hbm[dom] / (avg[dom] * 1e-3) / 1e9
    res = {
        "metric": "images/sec fwd+bwd, 2D 128^2 cubic (2D -> 2D path)",
        "value": round(B * P / (ms_step * 1e-3), 1),
        "unit": "images/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"c2: 2D->2D forward+backward, {B} images {w.N}^2, one in-plane pose each, cubic, "
                               f"cutoff {w.cutoff:g}, shifts U[-{w.shift_max:g},{w.shift_max:g}]",
                   "images": B, "box": w.N, "in_cutoff_outputs_per_image": n_c},
        "kernel_ms_mean": {k: round(v, 4) for k, v in avg.items()},
        "roofline": {"kernel": dom, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": hbm[dom]},
        "roofline_tap": {"bound": "l2", "peak": L2_PEAK_GBS, "unit": "GB/s",
                         "kernels": {k: {"achieved": round(units * taps * 8 / (avg[k] * 1e-3) / 1e9, 1)} for k in avg}},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


def host_cores() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


# A GPU machine gives one GPU's process a CPU share of 16 cores, whatever the
# host shows: the oracle's pool takes at most that many workers.
CPU_SHARE = 16


def cpu_baseline(V, R, s, w: synth.Workload, N: int, os_: float, poses_per_worker: int):
    """Time the oracle on a bounded pose sample with a fork pool (no GPU yet)."""
    ncpu = host_cores()
    workers = max(1, min(CPU_SHARE, ncpu))
    rng = np.random.default_rng(12345)
    sample = rng.choice(w.P, size=workers * poses_per_worker, replace=False)
    G = synth.make_upstream(w, poses=sample)
    _CPU.update(V=V, R=R[:, sample], s=s[:, sample], G=G, n_out=w.N_out, N=N,
                interp=w.interp, os=os_, cutoff=w.cutoff)
    chunks = [list(range(i * poses_per_worker, (i + 1) * poses_per_worker)) for i in range(workers)]
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        res = pool.map(_oracle_worker, chunks)
    wall = time.perf_counter() - t0
    n = sum(r[0] for r in res)
    fwd = sum(r[1] for r in res)
    bwd = sum(r[2] for r in res)
    # throughput of the pool: poses per wall second, split by the measured work
    rate_total = n / wall
    return {
        "value": rate_total,
        "unit": "projections/s fwd+bwd",
        "cores": workers,
        "host_cores": ncpu,
        "kind": "oracle",
        "sample": f"{n} of {w.P} poses (seeded), {workers} single-threaded workers, fork pool "
                  f"({ncpu} host cores visible)",
        "fwd_proj_per_s": n / (fwd / workers) if fwd > 0 else None,
        # one core: poses per second of a single-threaded worker's own time
        "value_1core": n / (fwd + bwd) if fwd + bwd > 0 else None,
        "wall_s": wall,
    }


# -------------------------------------------------------------------- GPU

def time_extras(L, _lib, torch, stream, Gd, Rd, R, dV, w, N, os_, B, P, reps=5):
    """Per-launch times of the dual-volume weight backprojection (weights
    |G|^2 on the same poses) and of the x = 0 symmetrisation of the adjoint's
    output, HIP events on the launch stream."""
    sh = stream.cuda_stream
    Wd = Gd.abs().square().contiguous()
    wV = torch.empty(dV.shape, dtype=torch.float32, device=dV.device)

    def weights():
        _lib.check(L.tp_backproject_weights_3d(Wd.data_ptr(), B, P, w.N_out, Rd.data_ptr(), R.shape[0], N,
                                               w.interp, os_, w.cutoff, wV.data_ptr(), sh),
                   "tp_backproject_weights_3d")

    def sym():
        _lib.check(L.tp_symmetrize_x0(3, dV.data_ptr(), B, N, sh), "tp_symmetrize_x0")

    # 3D -> 3D rotation on a subtomogram-sized workload: box 64 blob phantom,
    # 512 poses, cubic, cutoff 32, shifts U[-3, 3] voxels
    rng = np.random.default_rng([7, 0])
    n3, p3 = 64, 512
    sub = torch.from_numpy(synth.rfft_spectrum(synth.blob_volume(rng, n3, 40), 3)[None]).to(dV.device)
    r3 = torch.from_numpy(synth.uniform_rotations(rng, p3)[None].astype(np.float32)).to(dV.device)
    s3 = torch.from_numpy(rng.uniform(-3, 3, (1, p3, 3)).astype(np.float32)).to(dV.device)
    o3 = torch.empty((1, p3, n3, n3, n3 // 2 + 1), dtype=torch.complex64, device=dV.device)
    g3 = torch.randn_like(o3)
    v3 = torch.empty_like(sub)
    gr3 = torch.empty_like(r3)
    gs3 = torch.empty_like(s3)
    j3 = torch.empty((1, p3, 3, n3, n3, n3 // 2 + 1), dtype=torch.complex64, device=dV.device)

    def rot_fwd():
        _lib.check(L.tp_rotate_3d(sub.data_ptr(), 1, n3, r3.data_ptr(), 1, p3, s3.data_ptr(), 1, n3, 1, 1.0, 32.0,
                                  o3.data_ptr(), sh), "tp_rotate_3d")

    def rot_adj():
        _lib.check(L.tp_rotate_backproject_3d(g3.data_ptr(), 1, p3, n3, r3.data_ptr(), 1, s3.data_ptr(), 1, n3, 1,
                                              1.0, 32.0, v3.data_ptr(), sh), "tp_rotate_backproject_3d")

    def rot_grad():
        _lib.check(L.tp_rotate_grad_pose(sub.data_ptr(), 1, n3, g3.data_ptr(), r3.data_ptr(), 1, p3, s3.data_ptr(), 1,
                                         n3, 1, 1.0, 32.0, gr3.data_ptr(), gs3.data_ptr(), sh), "tp_rotate_grad_pose")

    def rot_fwd_jac():
        _lib.check(L.tp_rotate_3d_jac(sub.data_ptr(), 1, n3, r3.data_ptr(), 1, p3, s3.data_ptr(), 1, n3, 1, 1.0,
                                      32.0, o3.data_ptr(), j3.data_ptr(), sh), "tp_rotate_3d_jac")

    def rot_grad_jac():
        _lib.check(L.tp_rotate_grad_pose_jac(g3.data_ptr(), o3.data_ptr(), j3.data_ptr(), 1, p3, n3, 1, 1, 1.0, 32.0,
                                             gr3.data_ptr(), gs3.data_ptr(), sh), "tp_rotate_grad_pose_jac")

    def rot_bwd_jac():
        _lib.check(L.tp_rotate_backward_3d_jac(g3.data_ptr(), o3.data_ptr(), j3.data_ptr(), 1, p3, n3, r3.data_ptr(),
                                               1, s3.data_ptr(), 1, n3, 1, 1.0, 32.0, v3.data_ptr(), gr3.data_ptr(),
                                               gs3.data_ptr(), sh), "tp_rotate_backward_3d_jac")

    out = {"rotate_workload": "box 64 blob phantom, 512 poses, cubic, cutoff 32, shifts U[-3,3]"}
    for name, f in (("backproject_weights", weights), ("symmetrize_x0", sym), ("rotate_3d", rot_fwd),
                    ("rotate_backproject_3d", rot_adj), ("rotate_grad_pose", rot_grad),
                    ("rotate_3d_jac", rot_fwd_jac), ("rotate_grad_pose_jac", rot_grad_jac),
                    ("rotate_backward_3d_jac", rot_bwd_jac)):
        out[name + "_ms"] = time_launches(torch, stream, f, reps)
    del Wd, wV, o3, g3, j3
    return out


def measure_peaks(torch, dev, stream, reps=5):
    """Sustained peaks of this GPU from the probes of libtp_peaks.so (built
    beside libtp.so): read GB/s from HBM (4 GiB buffer, beyond the Infinity
    Cache), from the Infinity Cache (128 MiB, beyond L2) and from L2 (each
    XCD re-reading its own 2 MiB), fp32 FMA TFLOP/s without packed math, and
    LDS 64-bit atomic lane operations per second.  Best of `reps` launches
    after one warmup, HIP events on the launch stream."""
    import ctypes

    from cryo_em_fourier_amd import build as _build

    if not os.path.exists(_build.PEAKS_LIB):
        raise RuntimeError(f"{_build.PEAKS_LIB} is missing: run python -m cryo_em_fourier_amd.build")
    Lp = ctypes.CDLL(_build.PEAKS_LIB)
    vp, u64, i64, ci = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int
    Lp.tpk_read.argtypes = [vp, u64, i64, u64, ci, ci, vp, vp]
    Lp.tpk_fma.argtypes = [i64, ci, vp, vp]
    Lp.tpk_lds_add.argtypes = [i64, ci, vp, vp]
    for f in (Lp.tpk_read, Lp.tpk_fma, Lp.tpk_lds_add, Lp.tpk_threads_per_block):
        f.restype = ci
    sh = stream.cuda_stream
    threads = Lp.tpk_threads_per_block()
    blocks = 256 * 8  # 8 workgroups per CU
    sink = torch.zeros(4096, dtype=torch.int64, device=dev)

    def best_ms(f):
        f()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for k in range(reps):
            f()
            ev[k + 1].record(stream)
        torch.cuda.synchronize()
        return min(ev[k].elapsed_time(ev[k + 1]) for k in range(reps))

    def check(st, name):
        if st != 0:
            raise RuntimeError(f"{name} failed ({st})")

    # the best of a few buffer sizes and workgroup counts per level: the
    # probes are sensitive to their shape, so the L2 figure is a measured
    # lower bound of what 16-byte coalesced loads can pull from L2
    out = {}
    for name, sizes, passes_per_mib, regions in (("hbm_read_GBs", (4 << 30,), 0, 1),
                                                 ("mall_read_GBs", (64 << 20, 128 << 20), 1024, 1),
                                                 ("l2_read_GBs", (8 * (2 << 20), 8 * (3 << 20)), 1024, 8)):
        best = 0.0
        for nbytes in sizes:
            buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            n16 = nbytes // 16
            passes = max(1, passes_per_mib * (1 << 20) // nbytes)
            rot = (n16 // regions) * 5 // 11 + 1
            for nb in (1024, 2048, 4096):
                ms = best_ms(lambda: check(Lp.tpk_read(buf.data_ptr(), n16, passes, rot, regions, nb,
                                                       sink.data_ptr(), sh), "tpk_read"))
                best = max(best, nbytes * passes / (ms * 1e-3) / 1e9)
            del buf
        out[name] = round(best, 1)
    iters = 20000
    ms = best_ms(lambda: check(Lp.tpk_fma(iters, blocks, sink.data_ptr(), sh), "tpk_fma"))
    out["fp32_fma_TFLOPs"] = round(16.0 * iters * blocks * threads / (ms * 1e-3) / 1e12, 2)
    iters = 5000
    ms = best_ms(lambda: check(Lp.tpk_lds_add(iters, blocks, sink.data_ptr(), sh), "tpk_lds_add"))
    out["lds_add64_Glanes_per_s"] = round(8.0 * iters * blocks * threads / (ms * 1e-3) / 1e9, 1)
    torch.cuda.synchronize()
    return out


def time_launches(torch, stream, f, reps=5):
    """Mean per-launch time (ms) of f over reps launches after one warmup,
    HIP events on the launch stream."""
    f()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for i in range(reps):
        f()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    return round(float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)])), 4)


# --------------------------------------------------------- oversampling study

def blob_slice_truth(params, R, n_out: int, N: int, cutoff: float):
    """Analytic central slices of the blob phantom: the continuous Fourier
    transform of sum a exp(-|x - c|^2 / 2 s^2), box centre at the origin,
    at the sample points p = R^T (kx, ky, 0) (frequency p / N cycles/voxel):
    a (2 pi s^2)^(3/2) exp(-2 pi^2 s^2 |p|^2 / N^2) exp(-2 pi i p.(c - N/2) / N).
    Returns [P, n_out, n_out//2+1] complex128 and the kept mask."""
    c, sg, a = params
    c = c - N // 2                                   # (z, y, x) relative to the centre
    kx = np.arange(n_out // 2 + 1)[None, :].astype(np.float64)
    iy = np.arange(n_out)[:, None]
    ky = np.where(iy <= (n_out - 1) // 2, iy, iy - n_out).astype(np.float64)
    keep = (kx * kx + ky * ky <= cutoff * cutoff) if cutoff >= 0 else np.ones((n_out, n_out // 2 + 1), bool)
    kxk, kyk = np.broadcast_to(kx, keep.shape)[keep], np.broadcast_to(ky, keep.shape)[keep]
    out = np.zeros((R.shape[0], n_out, n_out // 2 + 1), np.complex128)
    for n in range(R.shape[0]):
        p = kxk[:, None] * R[n, 0][None, :] + kyk[:, None] * R[n, 1][None, :]   # (x, y, z)
        p2 = np.sum(p * p, axis=1)
        pc = p[:, 0:1] * c[None, :, 2] + p[:, 1:2] * c[None, :, 1] + p[:, 2:3] * c[None, :, 0]
        amp = a * (2 * np.pi * sg * sg) ** 1.5
        val = (amp[None, :] * np.exp(-2 * np.pi ** 2 * sg[None, :] ** 2 * p2[:, None] / N ** 2)
               * np.exp(-2j * np.pi * pc / N)).sum(axis=1)
        out[n][keep] = val
    return out, keep


def shell_stats(got, truth, keep, n_out: int, fracs=(0.1, 0.2, 0.3, 0.4, 0.45, 0.5)):
    """Fourier ring correlation, relative error and amplitude ratio of
    got vs truth per ring |k| / n_out in (f - 0.05, f]."""
    kx = np.arange(n_out // 2 + 1)[None, :]
    iy = np.arange(n_out)[:, None]
    ky = np.where(iy <= (n_out - 1) // 2, iy, iy - n_out)
    r = np.sqrt(kx * kx + ky * ky) / n_out
    res = {}
    for f in fracs:
        m = keep & (r > f - 0.05) & (r <= f)
        g, t = got[:, m], truth[:, m]
        frc = float(np.real(np.sum(g * np.conj(t))) / np.sqrt(np.sum(np.abs(g) ** 2) * np.sum(np.abs(t) ** 2)))
        err = float(np.linalg.norm(g - t) / np.linalg.norm(t))
        ratio = float(np.sum(np.abs(g)) / np.sum(np.abs(t)))
        res[f"{f:g}"] = {"frc": round(frc, 6), "rel_err": round(err, 6), "amp_ratio": round(ratio, 5)}
    return res


def kernel_ft(interp: int, nu: np.ndarray) -> np.ndarray:
    """Continuous Fourier transform of the interpolation kernel (tent or
    Keys' a = -0.5 cubic; both even) at nu cycles per voxel, by quadrature."""
    t = np.linspace(-2.0, 2.0, 40001)
    a = np.abs(t)
    if interp == synth.LINEAR:
        w = np.maximum(0.0, 1.0 - a)
    else:
        w = np.where(a <= 1, 1.5 * a ** 3 - 2.5 * a ** 2 + 1, np.where(a < 2, -0.5 * a ** 3 + 2.5 * a ** 2 - 4 * a + 2, 0.0))
    nu = np.asarray(nu, np.float64)
    return np.trapezoid(w[None, :] * np.cos(2 * np.pi * nu.reshape(-1, 1) * t[None, :]), t, axis=1).reshape(nu.shape)


def attenuation_study(pipelines, N: int, n_out: int, cutoff: float, poses_per_dir: int = 16, n_dirs: int = 3,
                      fracs=(0.0, 0.05, 0.1, 0.15, 0.2, 0.25, 0.3, 0.35, 0.4, 0.45), sigma: float = 1.5):
    """Real-space intensity against radius.  Phantoms of small blobs
    (sigma 1.5 voxels, amplitude 1) at r = f N from the box centre along a
    seeded direction, projected by each pipeline along poses that see the
    direction nearly in plane (in-plane length >= 0.95, so the blobs'
    images stay apart); each projection goes back to real space (irfft2)
    and each blob's intensity (the sum over a disc of radius 4 sigma about
    its projected centre) is divided by the same sum in the analytic
    projection.  ``predicted``: the product over axes of the kernel's
    Fourier transform at the blob's position in cycles per voxel of the
    (padded) reference, the factor by which interpolation in Fourier space
    scales a point's real-space signal."""
    import torch

    rng = np.random.default_rng(777)
    pool = synth.uniform_rotations(rng, 4000).astype(np.float64)
    fr = np.asarray(fracs)
    rad = 4.0 * sigma
    yy, xx = np.mgrid[0:n_out, 0:n_out]
    acc = {name: [] for name in pipelines}
    pred = {name: [] for name in pipelines}
    for _ in range(n_dirs):
        d = rng.standard_normal(3)
        d /= np.linalg.norm(d)                              # (z, y, x)
        c = N // 2 + np.outer(fr * N, d)
        params = (c, np.full(len(fr), sigma), np.ones(len(fr)))
        real = synth.render_blobs(params, N)
        dxyz = d[::-1]
        inplane = np.hypot(pool[:, 0] @ dxyz, pool[:, 1] @ dxyz)
        R = pool[inplane >= 0.95][:poses_per_dir]
        truth, _ = blob_slice_truth(params, R, n_out, N, cutoff)
        timg = np.fft.fftshift(np.fft.irfft2(truth, s=(n_out, n_out)), axes=(-2, -1))
        rel = (c - N // 2)[:, ::-1]                         # (x, y, z) from the centre
        ix = n_out // 2 + rel @ R[:, 0].T                   # [blob, pose]
        iy = n_out // 2 + rel @ R[:, 1].T
        masks = [[(yy - iy[j, n]) ** 2 + (xx - ix[j, n]) ** 2 <= rad * rad for n in range(len(R))]
                 for j in range(len(fr))]
        t_int = np.array([[timg[n][masks[j][n]].sum() for n in range(len(R))] for j in range(len(fr))])
        Rd = torch.from_numpy(R.astype(np.float32))[None].cuda()
        for name, (project, interp, os_) in pipelines.items():
            out = project(torch.from_numpy(real).cuda(), Rd, interp, os_)
            img = torch.fft.fftshift(torch.fft.irfft2(out[0], s=(n_out, n_out)), dim=(-2, -1)).double().cpu().numpy()
            g_int = np.array([[img[n][masks[j][n]].sum() for n in range(len(R))] for j in range(len(fr))])
            acc[name].append((g_int / t_int).mean(axis=1))
            nu = np.outer(fr * N, np.abs(d)) / (os_ * N)
            pred[name].append(np.prod(kernel_ft(interp, nu), axis=1))
    res = {}
    for name in pipelines:
        m = np.mean(acc[name], axis=0)
        p_ = np.mean(pred[name], axis=0)
        keep90 = [f for f, v in zip(fr, m) if v >= 0.9]
        res[name] = {"radius_frac": [round(float(f), 3) for f in fr],
                     "intensity_ratio": [round(float(v), 4) for v in m],
                     "predicted": [round(float(v), 4) for v in p_],
                     "max_radius_frac_ratio_ge_0.9": round(float(max(keep90)), 3) if keep90 else 0.0}
    return res


def oversampling_study(args):
    """Cubic at oversampling 1 against linear at oversampling 2 with the
    padding and FFT done on the fly, on the c4 phantom: wall time of the
    forward pipeline (the spectrum step of the real volume + projection)
    and of the training step (+ the adjoint, the pose gradients and the
    volume gradient back to real space), accuracy of the projections
    against the analytic slices of the blobs per Fourier ring, and the
    real-space intensity against radius (``attenuation_study``).  One JSON
    line."""
    import torch

    from cryo_em_fourier_amd import _lib
    from cryo_em_fourier_amd.spectrum import real_from_spectrum, rfft_spectrum

    w = synth.WORKLOADS["c4"]
    rng = synth.rng_for(w.cfg_id, synth.STREAM_VOLUME)
    params = synth.blob_params(rng, w.N, w.n_blobs)
    real = synth.make_real(w)[0]
    R = synth.make_rotations(w)
    L = _lib.lib()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    realt = torch.from_numpy(real).to(dev)
    Rd = torch.from_numpy(R).to(dev)
    P, n_out, Wo = w.P, w.N_out, w.N_out // 2 + 1
    G = torch.randn((1, P, n_out, Wo), dtype=torch.complex64, device=dev,
                    generator=torch.Generator(device=dev).manual_seed(4))
    out = torch.empty((1, P, n_out, Wo), dtype=torch.complex64, device=dev)
    dR = torch.empty_like(Rd)

    def pipeline(interp, os_, backward):
        # forward: the spectrum step + tp_project_3d; training step: + the
        # adjoint and the pose gradients (nothing stored between forward and
        # backward), then the volume gradient back to real space
        V = rfft_spectrum(realt[None], 3, w.N * os_)
        M = V.shape[1]
        _lib.check(L.tp_project_3d(V.data_ptr(), 1, M, Rd.data_ptr(), 1, P, None, 1, n_out, interp,
                                   float(os_), w.cutoff, out.data_ptr(), sh), "project")
        if not backward:
            return
        dV = torch.empty_like(V)
        _lib.check(L.tp_backproject_3d(G.data_ptr(), 1, P, n_out, Rd.data_ptr(), 1, None, 1, M, interp, float(os_),
                                       w.cutoff, dV.data_ptr(), sh), "backproject")
        _lib.check(L.tp_grad_pose(3, V.data_ptr(), 1, M, G.data_ptr(), Rd.data_ptr(), 1, P, None, 1, n_out, interp,
                                  float(os_), w.cutoff, dR.data_ptr(), None, sh), "grad_pose")
        real_from_spectrum(dV, w.N, 3)

    def timed(f, reps=5):
        f()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
        ev[0].record(stream)
        for i in range(reps):
            f()
            ev[i + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(reps)]))

    cases = {"cubic_os1": (synth.CUBIC, 1), "linear_os2": (synth.LINEAR, 2),
             "linear_os1": (synth.LINEAR, 1), "cubic_os2": (synth.CUBIC, 2)}
    Ps = min(args.study_poses, P)
    truth, keep = blob_slice_truth(params, R[0, :Ps].astype(np.float64), n_out, w.N, w.cutoff)
    res = {}
    for name, (interp, os_) in cases.items():
        t_fwd = timed(lambda: pipeline(interp, os_, False))
        t_step = timed(lambda: pipeline(interp, os_, True), reps=3)
        pipeline(interp, os_, False)
        got = out[0, :Ps].cpu().numpy().astype(np.complex128)
        res[name] = {"fwd_pipeline_ms": round(t_fwd, 3), "step_pipeline_ms": round(t_step, 3),
                     "fwd_proj_per_s": round(P / (t_fwd * 1e-3), 1),
                     "rings": shell_stats(got, truth, keep, n_out)}
        print(f"# {name}: fwd {t_fwd:.2f} ms, step {t_step:.2f} ms", file=sys.stderr, flush=True)
    res["speedup_cubic_os1_over_linear_os2"] = {
        "fwd": round(res["linear_os2"]["fwd_pipeline_ms"] / res["cubic_os1"]["fwd_pipeline_ms"], 3),
        "step": round(res["linear_os2"]["step_pipeline_ms"] / res["cubic_os1"]["step_pipeline_ms"], 3)}

    def project(real_t, Rt, interp, os_):
        V = rfft_spectrum(real_t[None], 3, w.N * os_)
        o = torch.empty((1, Rt.shape[1], n_out, Wo), dtype=torch.complex64, device=dev)
        _lib.check(L.tp_project_3d(V.data_ptr(), 1, V.shape[1], Rt.data_ptr(), 1, Rt.shape[1], None, 1, n_out,
                                   interp, float(os_), w.cutoff, o.data_ptr(), sh), "project")
        return o

    att = attenuation_study({k: (project, i, o) for k, (i, o) in cases.items()}, w.N, n_out, w.cutoff)
    print(json.dumps({"study": "oversampling", "workload": "c4 blob phantom, box 256, 4096 poses, cutoff 128, "
                      "no shifts; accuracy on the first %d poses against analytic blob slices" % Ps,
                      "results": res, "attenuation": att}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--config", default="c4", choices=["c2", "c3", "c4", "c5"],
                    help="c2 runs the 2D -> 2D path (images/s); the others the 3D -> 2D path")
    ap.add_argument("--oversampling", type=int, default=1, choices=[1, 2])
    ap.add_argument("--poses", type=int, default=0, help="override the pose count")
    ap.add_argument("--pose-grads", choices=["separate", "jacobian"], default="separate",
                    help="separate: the adjoint and a second gather pass for the pose gradients, nothing stored "
                         "(tp_backward_3d's kernels); jacobian: the forward saves each output's Jacobian for the "
                         "backward")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="time the step only: no other kernels, no peak probes (for counter runs)")
    ap.add_argument("--cpu-poses-per-worker", type=int, default=40,
                    help="oracle poses per CPU worker (about 13 s of host time with 16 workers at c4)")
    ap.add_argument("--study", choices=["oversampling"], default=None,
                    help="run a study instead of the step benchmark")
    ap.add_argument("--study-poses", type=int, default=64, help="poses scored against the analytic slice")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU; --gpus {args.gpus} is not supported "
              "(the projector is single-GPU; sharding is a design note only)", file=sys.stderr)
        sys.exit(2)

    if args.study == "oversampling":
        oversampling_study(args)
        return

    w = synth.WORKLOADS[args.config]
    if w.ndim == 2:
        bench_2d(args, w)
        return
    if args.poses:
        w = synth.Workload(**{**w.__dict__, "P": args.poses})
    os_ = float(args.oversampling)
    N = w.N * args.oversampling
    t0 = time.perf_counter()
    V = synth.make_reference(w, pad_to=N if args.oversampling != 1 else None)
    R = synth.make_rotations(w)
    s = synth.make_shifts(w)
    print(f"# inputs: reference {V.shape} rot {R.shape} ({time.perf_counter() - t0:.1f}s)",
          file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(V, R, s, w, N, os_, args.cpu_poses_per_worker)
        print(f"# cpu baseline: {cpu['value']:.3f} proj/s on {cpu['cores']} cores "
              f"({cpu['wall_s']:.1f}s)", file=sys.stderr, flush=True)

    import torch

    from cryo_em_fourier_amd import _lib

    L = _lib.lib()
    dev = torch.device("cuda:0")
    Wo = w.N_out // 2 + 1
    Vd = torch.from_numpy(V).to(dev)
    Rd = torch.from_numpy(R).to(dev)
    sd = torch.from_numpy(s).to(dev)
    G = synth.make_upstream(w)
    Gd = torch.from_numpy(G).to(dev)
    del G
    out = torch.empty((w.B, w.P, w.N_out, Wo), dtype=torch.complex64, device=dev)
    jac = torch.empty((w.B, w.P, 3, w.N_out, Wo), dtype=torch.complex64, device=dev)
    dV = torch.empty_like(Vd)
    dR = torch.empty_like(Rd)
    ds = torch.empty_like(sd)
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    B, P = w.B, w.P

    def fwd():
        _lib.check(L.tp_project_3d(Vd.data_ptr(), B, N, Rd.data_ptr(), R.shape[0], P, sd.data_ptr(),
                                   s.shape[0], w.N_out, w.interp, os_, w.cutoff, out.data_ptr(), sh),
                   "tp_project_3d")

    def fwd_jac():
        _lib.check(L.tp_project_3d_jac(Vd.data_ptr(), B, N, Rd.data_ptr(), R.shape[0], P, sd.data_ptr(),
                                       s.shape[0], w.N_out, w.interp, os_, w.cutoff, out.data_ptr(), jac.data_ptr(),
                                       sh), "tp_project_3d_jac")

    def adj():
        _lib.check(L.tp_backproject_3d(Gd.data_ptr(), B, P, w.N_out, Rd.data_ptr(), R.shape[0],
                                       sd.data_ptr(), s.shape[0], N, w.interp, os_, w.cutoff,
                                       dV.data_ptr(), sh), "tp_backproject_3d")

    def grad():
        _lib.check(L.tp_grad_pose(3, Vd.data_ptr(), B, N, Gd.data_ptr(), Rd.data_ptr(), R.shape[0], P,
                                  sd.data_ptr(), s.shape[0], w.N_out, w.interp, os_, w.cutoff,
                                  dR.data_ptr(), ds.data_ptr(), sh), "tp_grad_pose")

    def grad_jac():
        _lib.check(L.tp_grad_pose_jac(Gd.data_ptr(), out.data_ptr(), jac.data_ptr(), B, P, w.N_out, R.shape[0],
                                      s.shape[0], os_, w.cutoff, dR.data_ptr(), ds.data_ptr(), sh),
                   "tp_grad_pose_jac")

    def bwd_jac():
        _lib.check(L.tp_backward_3d_jac(Gd.data_ptr(), out.data_ptr(), jac.data_ptr(), B, P, w.N_out, Rd.data_ptr(),
                                        R.shape[0], sd.data_ptr(), s.shape[0], N, w.interp, os_, w.cutoff,
                                        dV.data_ptr(), dR.data_ptr(), ds.data_ptr(), sh), "tp_backward_3d_jac")

    modes = {
        "separate": [("project", fwd), ("backproject", adj), ("grad_pose", grad)],
        "jacobian": [("project_jac", fwd_jac), ("backward_jac", bwd_jac)],
    }
    kernels = modes[args.pose_grads]
    named = dict(kernels)
    other = [(n, f) for m in modes.values() for n, f in m if n not in named]
    other.append(("grad_pose_jac", grad_jac))

    # calibration for HBM byte counters: one plain streaming copy (y = x * 1)
    # of known size, outside the timed region.  A counter run of this same
    # command reads FETCH_SIZE / WRITE_SIZE for it and for the kernels.
    cal_src, cal_dst = Gd.view(torch.float32), out.view(torch.float32)
    torch.mul(cal_src, 1.0, out=cal_dst)
    torch.cuda.synchronize()
    copy_bytes = cal_src.numel() * 4

    for i in range(args.warmup):
        for _, f in kernels:
            f()
    torch.cuda.synchronize()
    print(f"# warmup done ({args.warmup} steps)", file=sys.stderr, flush=True)

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(kernels) + 1)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(args.steps):
        ev[k][0].record(stream)
        for j, (_, f) in enumerate(kernels):
            f()
            ev[k][j + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    avg_names = {name for name, _ in kernels}
    # the widened ops, timed after the step on the same inputs (not part of it)
    extras = {}
    if not args.no_extras:
        extras = time_extras(L, _lib, torch, stream, Gd, Rd, R, dV, w, N, os_, B, P)
        for name, f in other:  # the other pose-gradient paths, same inputs
            extras[name + "_ms"] = time_launches(torch, stream, f)
    elif "project" not in avg_names:
        extras["project_ms"] = time_launches(torch, stream, fwd)

    per_kernel = {name: [] for name, _ in kernels}
    step_ms = []
    for k in range(args.steps):
        for j, (name, _) in enumerate(kernels):
            per_kernel[name].append(ev[k][j].elapsed_time(ev[k][j + 1]))
        step_ms.append(ev[k][0].elapsed_time(ev[k][-1]))
    avg = {n: float(np.mean(v)) for n, v in per_kernel.items()}
    med = {n: float(np.median(v)) for n, v in per_kernel.items()}
    ms_step = float(np.mean(step_ms))
    fwd_bwd_rate = B * P / (ms_step * 1e-3)
    fwd_ms = avg["project"] if "project" in avg else extras["project_ms"]
    # the step's tap bytes against the unit-count L2 figure (3 B_tap per
    # forward + backward: the forward's gather, the adjoint's scatter and the
    # pose gradients' gather)
    fwd_rate = B * P / (fwd_ms * 1e-3)  # the plain forward (no Jacobian saved)

    # algorithmic traffic / work per launch
    n_c = in_cutoff_count(w.N_out, w.cutoff)
    taps = 64 if w.interp == synth.CUBIC else 8
    units = B * P * n_c                        # in-cutoff output frequencies per launch
    ref_bytes = V.nbytes
    img_bytes = B * P * w.N_out * Wo * 8
    pose_bytes = R.nbytes + s.nbytes
    grad_bytes = dR.numel() * 4 + ds.numel() * 4
    hbm = {  # compulsory HBM bytes per launch
        "project": ref_bytes + img_bytes + pose_bytes,
        "project_jac": ref_bytes + 4 * img_bytes + pose_bytes,   # out + 3 Jacobian planes
        "backproject": units * 8 + 2 * ref_bytes + pose_bytes,
        "grad_pose": ref_bytes + units * 8 + pose_bytes + grad_bytes,
        "grad_pose_jac": units * 40 + grad_bytes,                # G, out and jac inside the cutoff
        # both: G, out and jac inside the cutoff, the volume (fill + write)
        "backward_jac": units * 40 + 2 * ref_bytes + pose_bytes + grad_bytes,
    }
    # tap bytes per launch: 8 B x taps x in-cutoff outputs per pass over the taps
    tap_bytes = {"project": units * taps * 8, "project_jac": units * taps * 8, "backproject": units * taps * 8,
                 "grad_pose": units * taps * 8, "grad_pose_jac": 0, "backward_jac": units * taps * 8}
    dom = max(avg, key=avg.get)
    wl_key = f"{w.name}_os{args.oversampling}" + (f"_p{P}" if args.poses else "")
    traffic = measured_traffic(wl_key, copy_bytes)
    # The dominant kernel on the bound that applies to a gather or scatter:
    # its tap bytes (8 B x taps x in-cutoff outputs per pass over the taps)
    # against the L2 bandwidth derived from unit counts and clock (8 XCDs x
    # 16 channels x 128 B/clk x 2.4 GHz); the compulsory HBM bytes against
    # HBM's 8 TB/s beside it.
    achieved = tap_bytes[dom] / (avg[dom] * 1e-3) / 1e9
    achieved_hbm = hbm[dom] / (avg[dom] * 1e-3) / 1e9
    roof = {
        "kernel": dom,
        "bound": "l2",
        "achieved": round(achieved, 1),
        "peak": L2_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / L2_PEAK_GBS, 4),
        "traffic": traffic.get(dom),
        "algorithmic_bytes_per_launch": tap_bytes[dom],
        "hbm_compulsory": {"bytes_per_launch": hbm[dom], "achieved": round(achieved_hbm, 1),
                           "peak": HBM_PEAK_GBS, "frac": round(achieved_hbm / HBM_PEAK_GBS, 4)},
    }
    # every kernel's tap bytes against the same L2 figure
    tap_roof = {
        k: {"achieved": round(tap_bytes[k] / (avg[k] * 1e-3) / 1e9, 1),
            "frac": round(tap_bytes[k] / (avg[k] * 1e-3) / 1e9 / L2_PEAK_GBS, 4)}
        for k in avg if tap_bytes[k]
    }
    roof_tap = {"bound": "l2", "peak": L2_PEAK_GBS, "unit": "GB/s", "kernels": tap_roof}
    # the same fractions against this GPU's measured peaks (probes run after
    # the timed steps); the adjoint's LDS adds against the measured LDS rate
    peaks = {} if args.no_extras else measure_peaks(torch, dev, stream)
    frac_measured = {}
    for k in (avg if peaks else ()):
        f = {"hbm_compulsory": round(hbm[k] / (avg[k] * 1e-3) / 1e9 / peaks["hbm_read_GBs"], 4)}
        if tap_bytes[k]:
            f["l2_tap"] = round(tap_bytes[k] / (avg[k] * 1e-3) / 1e9 / peaks["l2_read_GBs"], 4)
        if k in ("backproject", "backward_jac"):
            f["lds_tap_adds"] = round(units * taps / (avg[k] * 1e-3) / 1e9 / peaks["lds_add64_Glanes_per_s"], 4)
        frac_measured[k] = f
    if peaks:
        peaks["fractions"] = frac_measured
    # the tap-gather roofline of the whole step at the measured L2 peak, with
    # the scope table's accounting: B_tap = 8 B x taps x in-cutoff outputs
    # per call; a forward touches B_tap, a forward + backward 3 B_tap (a
    # gather for the pose gradients and a scatter for the volume)
    b_tap = units * taps * 8
    if peaks:
        # (the L2 probe is a measured lower bound of the L2 read rate, about
        # half the unit-count figure: fractions against it are upper bounds)
        roof_fwd = B * P / (b_tap / (peaks["l2_read_GBs"] * 1e9))
        peaks["l2_tap_roofline_at_probe"] = {
            "fwd_proj_per_s": round(roof_fwd, 1), "fwd_frac": round(fwd_rate / roof_fwd, 4),
            "fwd_bwd_proj_per_s": round(roof_fwd / 3, 1), "fwd_bwd_frac": round(fwd_bwd_rate / (roof_fwd / 3), 4),
            "b_tap_per_call": b_tap,
        }
    res = {
        "metric": METRIC,
        "value": round(fwd_bwd_rate, 1),
        "unit": "projections/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"{w.name}: 3D->2D forward+backward, box {w.N}, {P} poses, cubic, "
                        f"oversampling {args.oversampling}, cutoff {w.cutoff:g}, shifts U[-{w.shift_max:g},{w.shift_max:g}]",
            "pose_grads": args.pose_grads,
            "box": w.N, "spectrum_box": N, "poses": P, "batch": B, "interp": "cubic" if w.interp else "linear",
            "oversampling": args.oversampling, "cutoff": w.cutoff, "in_cutoff_outputs_per_pose": n_c,
        },
        "fwd_proj_per_s": round(fwd_rate, 1),
        "step_l2_tap_frac": round(3 * units * taps * 8 / (ms_step * 1e-3) / 1e9 / L2_PEAK_GBS, 4),
        "fwd_l2_tap_frac": round(units * taps * 8 / (fwd_ms * 1e-3) / 1e9 / L2_PEAK_GBS, 4),
        "kernel_ms_mean": {k: round(v, 4) for k, v in avg.items()},
        "kernel_ms_median": {k: round(v, 4) for k, v in med.items()},
        "wall_s_timed": round(wall, 3),
        "roofline": roof,
        "roofline_tap": roof_tap,
        "peaks_measured": peaks,
        "traffic_all": traffic or None,
        "counter_calibration_copy_bytes": copy_bytes,
        "extras": extras,
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
