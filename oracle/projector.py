"""fp64 CPU oracle of the differentiable Fourier-space central-slice projector.

TEST INFRASTRUCTURE.  Only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The GPU library
shares no code with it; it is plain, slow and meant to be checked by eye
against the pages (torch-projectors: A High-Performance Differentiable
Projection Library for PyTorch, gist.science summaries in it/de/ja/ko/ar).

What it computes (NumPy, complex128; inputs are upcast from complex64/fp32):

* Layout: PyTorch/FFTW rfft half-spectra kept as they are, with no format
  conversion anywhere [tech. §2 of every page].
  3D reference ``V[b, z, y, x]`` with x = the halved last axis, 2D reference
  ``V[b, y, x]``.  Index -> signed frequency is ``f_N(i) = i if i <= (N-1)//2
  else i - N``.  Stored: x in [0, N//2], y and z in [-(N//2), (N+1)//2 - 1].
* Rotation: an output frequency k = (kx, ky) is mapped into the reference as
  p = os * (kx * R[0, :] + ky * R[1, :]) = os * R^T (kx, ky[, 0]), components
  in (x, y[, z]) order [ko page tech. §2: coordinates through the inverse of
  the rotation; ar page tech. §2: rotation by matrix multiplication].
* Friedel: a tap with negative x reads the conjugate of the entry at -t,
  F(-k) = conj F(k) [it/de/ar tech. §2, ko tech. §2].  Taps with x = 0 read
  the stored entry as it is.  Taps outside the stored range read 0.
* Interpolation: trilinear/bilinear (2 taps per axis) or Catmull-Rom cubic,
  Keys' kernel with a = -0.5 (4 taps per axis) [it/de/ja/ko/ar tech. §2].
* Shift: multiplication by exp(-2 pi i k.s / N_out), k in integer frequency
  units, s in output pixels, s[..., 0] = x [de tech. §2, ar tech. §2].
* Cutoff: outputs with kx^2 + ky^2 > cutoff^2 are 0 (cutoff < 0: none).
* Backprojection is the exact adjoint of the forward for the real inner
  product Re sum conj(a) b [ko tech. §2: backward projection is the adjoint;
  gradient accumulation uses the conjugate phase].
* Pose gradients by the chain rule through the interpolation-kernel
  derivatives [ar tech. §2; de tech. §3 item 4].

Where the pages are silent this module takes the plainest reading and says
so in the function that applies it: per-tap fold, zero outside the stored
range, right derivative of the linear kernel at integers, sample points with
a non-finite or |p| > 2**30 component read 0.  Every function here is pinned by tests in ``tests/test_oracle_*.py``.
"""
from __future__ import annotations

import itertools

import numpy as np

LINEAR = 0
CUBIC = 1
COORD_LIMIT = 2.0 ** 30


# ------------------------------------------------------------ index helpers

def signed_freq(i, n: int):
    """Array index -> signed frequency (numpy's fftfreq times n)."""
    i = np.asarray(i)
    return np.where(i <= (n - 1) // 2, i, i - n)


def output_grid(n_out: int, cutoff: float):
    """Signed (kx, ky) of every output entry of an [n_out, n_out//2+1] rfft
    image and the mask of entries kept by the cutoff (inclusive)."""
    iy, ix = np.meshgrid(np.arange(n_out), np.arange(n_out // 2 + 1), indexing="ij")
    kx = ix.astype(np.int64)
    ky = signed_freq(iy, n_out).astype(np.int64)
    if cutoff < 0:
        keep = np.ones(kx.shape, bool)
    else:
        keep = (kx * kx + ky * ky).astype(np.float64) <= float(cutoff) ** 2
    return kx, ky, keep


# ------------------------------------------------------ interpolation kernels

def kernel(interp: int, t):
    """Interpolation kernel K(t).

    Linear: the tent max(0, 1 - |t|).
    Cubic: Keys' cubic convolution kernel with a = -0.5 (Catmull-Rom),
      (a+2)|t|^3 - (a+3)|t|^2 + 1          for |t| <= 1,
      a|t|^3 - 5a|t|^2 + 8a|t| - 4a        for 1 < |t| < 2,
      0                                    otherwise.
    """
    t = np.abs(np.asarray(t, np.float64))
    if interp == LINEAR:
        return np.maximum(0.0, 1.0 - t)
    a = -0.5
    inner = (a + 2) * t ** 3 - (a + 3) * t ** 2 + 1
    outer = a * t ** 3 - 5 * a * t ** 2 + 8 * a * t - 4 * a
    return np.where(t <= 1, inner, np.where(t < 2, outer, 0.0))


def kernel_deriv(interp: int, u):
    """dK(u)/du.  The cubic kernel is C^1, so its derivative is unique; the
    linear tent takes the right derivative at its kinks (u = -1, 0, 1)."""
    u = np.asarray(u, np.float64)
    if interp == LINEAR:
        return np.where((u >= -1) & (u < 0), 1.0, np.where((u >= 0) & (u < 1), -1.0, 0.0))
    a = -0.5
    t = np.abs(u)
    sg = np.sign(u)
    inner = 3 * (a + 2) * t ** 2 - 2 * (a + 3) * t
    outer = 3 * a * t ** 2 - 10 * a * t + 8 * a
    return sg * np.where(t <= 1, inner, np.where(t < 2, outer, 0.0))


def tap_offsets(interp: int):
    """Tap positions relative to floor(p) along one axis."""
    return (0, 1) if interp == LINEAR else (-1, 0, 1, 2)


# ------------------------------------------------------------- tap lookup

def resolve_taps(t: np.ndarray, N: int):
    """Integer taps t[..., ndim] in (x, y[, z]) order -> (valid, flat index into
    one reference of shape [N, (N,) N//2+1], conjugate flag).

    A tap with x < 0 is replaced by -t and flagged for conjugation (Friedel);
    it is valid when the (possibly negated) tap lies in the stored range.
    """
    ndim = t.shape[-1]
    conj = t[..., 0] < 0
    tt = np.where(conj[..., None], -t, t)
    x = tt[..., 0]
    lo, hi = -(N // 2), (N + 1) // 2 - 1
    valid = (x >= 0) & (x <= N // 2)
    for j in range(1, ndim):
        valid &= (tt[..., j] >= lo) & (tt[..., j] <= hi)
    wh = N // 2 + 1
    idx = np.zeros(x.shape, np.int64)
    for j in range(ndim - 1, 0, -1):           # slowest axis first: z, then y
        idx = idx * N + np.mod(tt[..., j], N)
    idx = idx * wh + np.clip(x, 0, N // 2)
    idx = np.where(valid, idx, 0)
    return valid, idx, conj


def lookup(Vflat: np.ndarray, t: np.ndarray, N: int):
    """E(t): the stored value, conjugated for folded taps, 0 out of range."""
    valid, idx, conj = resolve_taps(t, N)
    v = Vflat[idx]
    v = np.where(conj, np.conj(v), v)
    return np.where(valid, v, 0.0)


# ------------------------------------------------------------ per-pose core

def _sample_points(kx, ky, Rm: np.ndarray, os: float):
    """p = os * (kx R[0,:] + ky R[1,:]) for the kept outputs, (n, ndim)."""
    Rm = np.asarray(Rm, np.float64)
    p = float(os) * (kx[:, None] * Rm[0][None, :] + ky[:, None] * Rm[1][None, :])
    ok = np.all(np.isfinite(p) & (np.abs(p) <= COORD_LIMIT), axis=1)
    return np.where(ok[:, None], p, 0.0), ok


def _phase(kx, ky, sv, n_out: int):
    """exp(-2 pi i (kx s_x + ky s_y) / n_out)."""
    sv = np.asarray(sv, np.float64)
    return np.exp(-2j * np.pi * (kx * sv[0] + ky * sv[1]) / n_out)


def _interpolate(Vflat, N: int, p: np.ndarray, interp: int, want_grad: bool):
    """S(p) = sum over the separable stencil of prod_j K(p_j - t_j) E(t), and
    optionally dS/dp_j (the j-th factor replaced by K')."""
    n, ndim = p.shape
    base = np.floor(p).astype(np.int64)
    S = np.zeros(n, np.complex128)
    dS = np.zeros((n, ndim), np.complex128) if want_grad else None
    for d in itertools.product(tap_offsets(interp), repeat=ndim):
        t = base + np.asarray(d, np.int64)[None, :]
        u = p - t
        k = kernel(interp, u)
        val = lookup(Vflat, t, N)
        S += np.prod(k, axis=1) * val
        if want_grad:
            dk = kernel_deriv(interp, u)
            for j in range(ndim):
                w = dk[:, j].copy()
                for i in range(ndim):
                    if i != j:
                        w *= k[:, i]
                dS[:, j] += w * val
    return S, dS


def _scatter(Aflat, N: int, p: np.ndarray, c: np.ndarray, interp: int):
    """Adjoint of _interpolate: each tap t with weight w receives w*c, or
    w*conj(c) at -t when the tap was folded."""
    ndim = p.shape[1]
    base = np.floor(p).astype(np.int64)
    for d in itertools.product(tap_offsets(interp), repeat=ndim):
        t = base + np.asarray(d, np.int64)[None, :]
        w = np.prod(kernel(interp, p - t), axis=1)
        valid, idx, conj = resolve_taps(t, N)
        val = w * np.where(conj, np.conj(c), c)
        np.add.at(Aflat, idx[valid], val[valid])


# ---------------------------------------------------------------- public ops

def _dims(V, R):
    ndim = R.shape[-1]
    assert ndim in (2, 3) and R.shape[-2] == ndim
    N = V.shape[-2]
    assert V.shape[-1] == N // 2 + 1 and V.ndim == ndim + 1
    assert all(s == N for s in V.shape[1:-1])
    return ndim, N


def _bidx(Bx: int, b: int) -> int:
    return 0 if Bx == 1 else b


def project(V, R, s, n_out: int, interp: int, os: float = 1.0, cutoff: float = -1.0):
    """Forward projection.  V [B, N, N, N//2+1] (3D) or [B, N, N//2+1] (2D),
    R [B_rot, P, d, d], s [B_shift, P, 2] or None -> [B, P, n_out, n_out//2+1].
    """
    V = np.asarray(V, np.complex128)
    R = np.asarray(R, np.float64)
    ndim, N = _dims(V, R)
    B, P = V.shape[0], R.shape[1]
    kx, ky, keep = output_grid(n_out, cutoff)
    kxk, kyk = kx[keep], ky[keep]
    out = np.zeros((B, P, n_out, n_out // 2 + 1), np.complex128)
    for b in range(B):
        Vflat = V[b].reshape(-1)
        for n in range(P):
            Rm = R[_bidx(R.shape[0], b), n]
            sv = (0.0, 0.0) if s is None else s[_bidx(s.shape[0], b), n]
            p, ok = _sample_points(kxk, kyk, Rm, os)
            S, _ = _interpolate(Vflat, N, p, interp, False)
            S = np.where(ok, S, 0.0)
            out[b, n][keep] = _phase(kxk, kyk, sv, n_out) * S
    return out


def backproject(G, R, s, N: int, interp: int, os: float = 1.0, cutoff: float = -1.0):
    """Adjoint of ``project`` w.r.t. Re<a, b>: G [B, P, n_out, n_out//2+1]
    -> A [B, N, N, N//2+1] (3D) or [B, N, N//2+1] (2D)."""
    G = np.asarray(G, np.complex128)
    R = np.asarray(R, np.float64)
    ndim = R.shape[-1]
    B, P, n_out = G.shape[0], G.shape[1], G.shape[2]
    kx, ky, keep = output_grid(n_out, cutoff)
    kxk, kyk = kx[keep], ky[keep]
    A = np.zeros((B,) + (N,) * (ndim - 1) + (N // 2 + 1,), np.complex128)
    for b in range(B):
        Aflat = np.zeros(A[b].size, np.complex128)
        for n in range(P):
            Rm = R[_bidx(R.shape[0], b), n]
            sv = (0.0, 0.0) if s is None else s[_bidx(s.shape[0], b), n]
            p, ok = _sample_points(kxk, kyk, Rm, os)
            c = np.conj(_phase(kxk, kyk, sv, n_out)) * G[b, n][keep]
            c = np.where(ok, c, 0.0)
            _scatter(Aflat, N, p, c, interp)
        A[b] = Aflat.reshape(A[b].shape)
    return A


def grad_pose(V, G, R, s, n_out: int, interp: int, os: float = 1.0, cutoff: float = -1.0):
    """Gradients of L = Re sum conj(G) * project(V, R, s) w.r.t. R and s.

    dL/dR [B_rot, P, d, d] (the last row is 0 in 3D: the output plane has
    kz = 0), dL/ds [B_shift, P, 2].  Broadcast poses (B_rot = 1 or
    B_shift = 1 with B > 1) receive the sum over the batch.
    """
    V = np.asarray(V, np.complex128)
    G = np.asarray(G, np.complex128)
    R = np.asarray(R, np.float64)
    ndim, N = _dims(V, R)
    B, P = V.shape[0], R.shape[1]
    kx, ky, keep = output_grid(n_out, cutoff)
    kxk, kyk = kx[keep], ky[keep]
    dR = np.zeros(R.shape, np.float64)
    Bs = 1 if s is None else s.shape[0]
    ds = np.zeros((Bs, P, 2), np.float64)
    for b in range(B):
        Vflat = V[b].reshape(-1)
        for n in range(P):
            br = _bidx(R.shape[0], b)
            bs = _bidx(Bs, b)
            sv = (0.0, 0.0) if s is None else s[bs, n]
            p, ok = _sample_points(kxk, kyk, R[br, n], os)
            S, dS = _interpolate(Vflat, N, p, interp, True)
            S = np.where(ok, S, 0.0)
            dS = np.where(ok[:, None], dS, 0.0)
            phi = _phase(kxk, kyk, sv, n_out)
            g = np.conj(G[b, n][keep]) * phi
            dLdp = np.real(g[:, None] * dS)                       # (n, ndim)
            dR[br, n, 0, :] += float(os) * np.sum(kxk[:, None] * dLdp, axis=0)
            dR[br, n, 1, :] += float(os) * np.sum(kyk[:, None] * dLdp, axis=0)
            for j, kj in enumerate((kxk, kyk)):
                ds[bs, n, j] += np.sum(np.real(g * (-2j * np.pi * kj / n_out) * S))
    return dR, ds


# --------------------------------------------- dual-volume weights, x = 0 plane

def backproject_weights(W, R, N: int, interp: int, os: float = 1.0, cutoff: float = -1.0):
    """Second (real) volume of a dual-volume reconstruction: every in-cutoff
    output's real weight W (e.g. CTF^2) is spread with the same
    interpolation weights as the adjoint; no phase; a folded tap (x < 0)
    adds to -t (real, so nothing to conjugate) [it tech. §2: optional
    weight accumulation for CTF correction; de tech. §2: dual-volume
    approach, second tensor for weights; ar tech. §2: dual-volume weighting].

    W [B, P, n_out, n_out//2+1] real -> [B, N, N, N//2+1] (3D) or
    [B, N, N//2+1] (2D) real.
    """
    W = np.asarray(W, np.float64)
    R = np.asarray(R, np.float64)
    ndim = R.shape[-1]
    B, P, n_out = W.shape[0], W.shape[1], W.shape[2]
    kx, ky, keep = output_grid(n_out, cutoff)
    kxk, kyk = kx[keep], ky[keep]
    A = np.zeros((B,) + (N,) * (ndim - 1) + (N // 2 + 1,), np.float64)
    for b in range(B):
        Aflat = np.zeros(A[b].size, np.float64)
        for n in range(P):
            p, ok = _sample_points(kxk, kyk, R[_bidx(R.shape[0], b), n], os)
            c = np.where(ok, W[b, n][keep], 0.0)
            base = np.floor(p).astype(np.int64)
            for d in itertools.product(tap_offsets(interp), repeat=ndim):
                t = base + np.asarray(d, np.int64)[None, :]
                w = np.prod(kernel(interp, p - t), axis=1)
                valid, idx, _ = resolve_taps(t, N)
                np.add.at(Aflat, idx[valid], (w * c)[valid])
        A[b] = Aflat.reshape(A[b].shape)
    return A


def symmetrize_x0(V):
    """Hermitian symmetrisation of the x = 0 plane of an rfft half-spectrum:
    V(0, y, z) <- (V(0, y, z) + conj V(0, -y, -z)) / 2, indices taken mod N
    (the periodic mirror of the DFT); every other plane is unchanged [de
    tech. §2: the zero-frequency axis is treated so that nothing is counted
    twice; ar tech. §2: symmetric accumulation on that axis].

    V [B, N, N, N//2+1] (3D) or [B, N, N//2+1] (2D), complex -> same shape.
    Plain loops over the plane.
    """
    V = np.array(V, np.complex128)
    N = V.shape[1]
    out = V.copy()
    if V.ndim == 4:
        for b in range(V.shape[0]):
            for iz in range(N):
                for iy in range(N):
                    mz, my = (-iz) % N, (-iy) % N
                    out[b, iz, iy, 0] = 0.5 * (V[b, iz, iy, 0] + np.conj(V[b, mz, my, 0]))
    else:
        for b in range(V.shape[0]):
            for iy in range(N):
                my = (-iy) % N
                out[b, iy, 0] = 0.5 * (V[b, iy, 0] + np.conj(V[b, my, 0]))
    return out


# ------------------------------------------------------------ 3D -> 3D rotation

def output_grid_3d(n_out: int, cutoff: float):
    """Signed (kx, ky, kz) of every entry of an [n_out, n_out, n_out//2+1]
    rfft half-spectrum (z, y, x) and the mask of entries inside the sphere
    kx^2 + ky^2 + kz^2 <= cutoff^2 (all of them when cutoff < 0)."""
    iz, iy, ix = np.meshgrid(np.arange(n_out), np.arange(n_out), np.arange(n_out // 2 + 1), indexing="ij")
    kx = ix.astype(np.int64)
    ky = signed_freq(iy, n_out).astype(np.int64)
    kz = signed_freq(iz, n_out).astype(np.int64)
    if cutoff < 0:
        keep = np.ones(kx.shape, bool)
    else:
        keep = (kx * kx + ky * ky + kz * kz).astype(np.float64) <= float(cutoff) ** 2
    return kx, ky, kz, keep


def _rot_points(kx, ky, kz, Rm, os: float):
    """p = os * R^T k = os * (kx R[0,:] + ky R[1,:] + kz R[2,:]), (n, 3)."""
    Rm = np.asarray(Rm, np.float64)
    p = float(os) * (kx[:, None] * Rm[0][None, :] + ky[:, None] * Rm[1][None, :] + kz[:, None] * Rm[2][None, :])
    ok = np.all(np.isfinite(p) & (np.abs(p) <= COORD_LIMIT), axis=1)
    return np.where(ok[:, None], p, 0.0), ok


def _phase3(kx, ky, kz, sv, n_out: int):
    """exp(-2 pi i (kx s_x + ky s_y + kz s_z) / n_out)."""
    sv = np.asarray(sv, np.float64)
    return np.exp(-2j * np.pi * (kx * sv[0] + ky * sv[1] + kz * sv[2]) / n_out)


def rotate_3d(V, R, s, n_out: int, interp: int, os: float = 1.0, cutoff: float = -1.0):
    """3D -> 3D rotation [it tech. §2: 3D -> 3D projection for general
    rotations]: every frequency k of the output half-spectrum samples the
    reference at p = os R^T k with the central slice's fold and kernels (so
    its kz = 0 plane is ``project``'s slice), times the phase of a 3-vector
    shift in output voxels; 0 outside the cutoff sphere.

    V [B, N, N, N//2+1], R [B_rot, P, 3, 3], s [B_shift, P, 3] or None
    -> [B, P, n_out, n_out, n_out//2+1].
    """
    V = np.asarray(V, np.complex128)
    R = np.asarray(R, np.float64)
    _, N = _dims(V, R)
    B, P = V.shape[0], R.shape[1]
    kx, ky, kz, keep = output_grid_3d(n_out, cutoff)
    kxk, kyk, kzk = kx[keep], ky[keep], kz[keep]
    out = np.zeros((B, P, n_out, n_out, n_out // 2 + 1), np.complex128)
    for b in range(B):
        Vflat = V[b].reshape(-1)
        for n in range(P):
            sv = (0.0, 0.0, 0.0) if s is None else s[_bidx(s.shape[0], b), n]
            p, ok = _rot_points(kxk, kyk, kzk, R[_bidx(R.shape[0], b), n], os)
            S, _ = _interpolate(Vflat, N, p, interp, False)
            out[b, n][keep] = _phase3(kxk, kyk, kzk, sv, n_out) * np.where(ok, S, 0.0)
    return out


def rotate_backproject_3d(G, R, s, N: int, interp: int, os: float = 1.0, cutoff: float = -1.0):
    """Adjoint of ``rotate_3d`` w.r.t. Re<a, b>: G [B, P, n, n, n//2+1] ->
    [B, N, N, N//2+1]."""
    G = np.asarray(G, np.complex128)
    R = np.asarray(R, np.float64)
    B, P, n_out = G.shape[0], G.shape[1], G.shape[2]
    kx, ky, kz, keep = output_grid_3d(n_out, cutoff)
    kxk, kyk, kzk = kx[keep], ky[keep], kz[keep]
    A = np.zeros((B, N, N, N // 2 + 1), np.complex128)
    for b in range(B):
        Aflat = np.zeros(A[b].size, np.complex128)
        for n in range(P):
            sv = (0.0, 0.0, 0.0) if s is None else s[_bidx(s.shape[0], b), n]
            p, ok = _rot_points(kxk, kyk, kzk, R[_bidx(R.shape[0], b), n], os)
            c = np.conj(_phase3(kxk, kyk, kzk, sv, n_out)) * G[b, n][keep]
            _scatter(Aflat, N, p, np.where(ok, c, 0.0), interp)
        A[b] = Aflat.reshape(A[b].shape)
    return A


def rotate_grad_pose(V, G, R, s, n_out: int, interp: int, os: float = 1.0, cutoff: float = -1.0):
    """Gradients of L = Re sum conj(G) rotate_3d(V, R, s) w.r.t. R (all
    three rows: dL/dR_ij = os sum k_i dL/dp_j) and s (3 components)."""
    V = np.asarray(V, np.complex128)
    G = np.asarray(G, np.complex128)
    R = np.asarray(R, np.float64)
    _, N = _dims(V, R)
    B, P = V.shape[0], R.shape[1]
    kx, ky, kz, keep = output_grid_3d(n_out, cutoff)
    ks = (kx[keep], ky[keep], kz[keep])
    dR = np.zeros(R.shape, np.float64)
    Bs = 1 if s is None else s.shape[0]
    ds = np.zeros((Bs, P, 3), np.float64)
    for b in range(B):
        Vflat = V[b].reshape(-1)
        for n in range(P):
            br, bs = _bidx(R.shape[0], b), _bidx(Bs, b)
            sv = (0.0, 0.0, 0.0) if s is None else s[bs, n]
            p, ok = _rot_points(*ks, R[br, n], os)
            S, dS = _interpolate(Vflat, N, p, interp, True)
            S = np.where(ok, S, 0.0)
            dS = np.where(ok[:, None], dS, 0.0)
            g = np.conj(G[b, n][keep]) * _phase3(*ks, sv, n_out)
            dLdp = np.real(g[:, None] * dS)
            for i in range(3):
                dR[br, n, i, :] += float(os) * np.sum(ks[i][:, None] * dLdp, axis=0)
                ds[bs, n, i] += np.sum(np.real(g * (-2j * np.pi * ks[i] / n_out) * S))
    return dR, ds



# ------------------------------------------------- the caller's spectrum step

def spectrum(real, ndim: int, pad_to: int | None = None):
    """The reference the projector samples, made from a centred real box
    (the last ``ndim`` axes; leading axes are a batch): zero-padded to
    ``pad_to`` (default: no padding) with the box centre N // 2 placed at
    the padded box's centre M // 2, the centre moved to index 0
    (ifftshift), then rfftn, complex128.  With pad_to = os * N the
    projector samples it at oversampling os: the pages' on-the-fly
    oversampling pays this padding and FFT on every pass (it/de/ja pages,
    results section on interpolation), and their reference layout is
    PyTorch's rfftn half-spectrum (tech. section 2 of every page)."""
    x = np.asarray(real, np.float64)
    N = x.shape[-1]
    M = N if pad_to is None else int(pad_to)
    if M < N or any(d != N for d in x.shape[-ndim:]):
        raise ValueError("a cube (square) of side N, padded to M >= N")
    big = np.zeros(x.shape[:-ndim] + (M,) * ndim)
    off = M // 2 - N // 2
    big[(Ellipsis,) + (slice(off, off + N),) * ndim] = x
    axes = tuple(range(-ndim, 0))
    return np.fft.rfftn(np.fft.ifftshift(big, axes=axes), axes=axes)
