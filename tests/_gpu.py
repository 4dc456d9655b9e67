"""Shared helpers of the GPU parity tests (not collected by pytest)."""
import sys

import numpy as np

# Tolerances of the parity bar: relative L2 error and max-abs error relative
# to the reference's largest magnitude (fp32 kernels vs the fp64 oracle).
REL_L2 = 1e-5
MAX_ABS = 1e-4


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype=None):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def rel_errors(got, ref):
    got = np.asarray(got, np.complex128 if np.iscomplexobj(got) or np.iscomplexobj(ref) else np.float64)
    ref = np.asarray(ref)
    diff = got - ref
    nref = np.linalg.norm(ref.ravel())
    rel = np.linalg.norm(diff.ravel()) / nref if nref > 0 else np.linalg.norm(diff.ravel())
    mref = np.abs(ref).max() if ref.size else 0.0
    mabs = np.abs(diff).max() / mref if mref > 0 else np.abs(diff).max()
    return float(rel), float(mabs)


def assert_parity(got, ref, what: str, rel_tol: float = REL_L2, abs_tol: float = MAX_ABS):
    rel, mabs = rel_errors(got, ref)
    log(f"  parity {what}: rel-L2 {rel:.2e}  max-abs/max {mabs:.2e}")
    assert rel <= rel_tol and mabs <= abs_tol, (
        f"{what}: rel-L2 {rel:.3e} (tol {rel_tol:.0e}), max-abs/max {mabs:.3e} (tol {abs_tol:.0e})")


def complex_normal(rng, shape):
    return (rng.standard_normal(shape) + 1j * rng.standard_normal(shape)).astype(np.complex64) * np.float32(np.sqrt(0.5))


def _oracle_backproject_part(args):
    import oracle

    G, R, s, N, interp, os_, cutoff = args
    return oracle.backproject(G, R, s, N, interp, os_, cutoff)


def oracle_backproject_pooled(G, R, s, N, interp, os_, cutoff, workers=16):
    """oracle.backproject summed over pose chunks computed by CPU worker
    processes (spawned: they import numpy and the oracle only, never the
    GPU).  The adjoint is linear in the poses, so the sum is the oracle's
    adjoint of all of them, up to the order of fp64 additions."""
    import multiprocessing as mp
    import os

    P = G.shape[1]
    nw = max(1, min(workers, len(os.sched_getaffinity(0)), P))
    chunks = [c for c in np.array_split(np.arange(P), 2 * nw) if c.size]
    jobs = [(G[:, c], R[:, c], None if s is None else s[:, c], N, interp, os_, cutoff) for c in chunks]
    with mp.get_context("spawn").Pool(nw) as pool:
        parts = pool.map(_oracle_backproject_part, jobs)
    return np.sum(parts, axis=0)
