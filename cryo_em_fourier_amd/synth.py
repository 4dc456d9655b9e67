"""Seeded synthetic workloads for the Fourier-slice projector.

This module only *builds inputs*: real-space phantoms, their rfft spectra
(the caller's own FFT step, done before any projector call), rotation and
shift batches, and upstream gradients.  It holds none of the projector's
arithmetic (no slice extraction, interpolation, phase ramp or adjoint), so
both the fp64 oracle and the GPU path can be fed from it without sharing any
of the method.

The pages summarising torch-projectors describe single-particle analysis and
electron tomography workloads in general terms (torch-projectors summary,
every language, technical section 1) but name no dataset.  The shapes below
stand in for them:

* ``c1``  32^3 i.i.d. N(0,1) voxels, 16 uniform SO(3) poses, no shift,
          linear, cutoff 16.
* ``c2``  256 images 128^2 (20 Gaussians each, sigma 2..8 px, plus noise of
          std 0.1), one in-plane pose per image, shifts U[-5,5] px, cubic,
          cutoff 64.
* ``c3``  128^3 blob phantom (200 blobs, sigma 1.5..4 voxels, amplitude
          U[0.5,1]), 1024 poses, shifts U[-8,8], cubic, cutoff 64.
* ``c4``  256^3 blob phantom (200 blobs), 4096 poses, shifts U[-10,10],
          cubic, oversampling 1 or 2 (zero-padded to 512^3), cutoff 128.
* ``c5``  320^3 blob phantom (1000 blobs), 128 tilt series x 64 tilts in
          -60..+60 degrees about a random in-plane axis, shifts U[-15,15],
          cubic, cutoff 160.

Random streams: ``np.random.default_rng([cfg_id, stream])`` with stream
0 = volume, 1 = rotations, 2 = shifts, 3 = upstream gradient (the gradient
uses one sub-stream per pose, ``[cfg_id, 3, pose]``, so any subset of poses
can be regenerated on its own).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

STREAM_VOLUME = 0
STREAM_ROT = 1
STREAM_SHIFT = 2
STREAM_GRAD = 3

LINEAR = 0
CUBIC = 1


def rng_for(cfg_id: int, stream: int, *sub: int) -> np.random.Generator:
    return np.random.default_rng([int(cfg_id), int(stream), *[int(s) for s in sub]])


# ---------------------------------------------------------------- rotations

def uniform_rotations(rng: np.random.Generator, n: int) -> np.ndarray:
    """Uniform SO(3) samples: normalised Gaussian unit quaternions -> 3x3."""
    q = rng.standard_normal((n, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    w, x, y, z = q.T
    R = np.empty((n, 3, 3))
    R[:, 0, 0] = 1 - 2 * (y * y + z * z)
    R[:, 0, 1] = 2 * (x * y - w * z)
    R[:, 0, 2] = 2 * (x * z + w * y)
    R[:, 1, 0] = 2 * (x * y + w * z)
    R[:, 1, 1] = 1 - 2 * (x * x + z * z)
    R[:, 1, 2] = 2 * (y * z - w * x)
    R[:, 2, 0] = 2 * (x * z - w * y)
    R[:, 2, 1] = 2 * (y * z + w * x)
    R[:, 2, 2] = 1 - 2 * (x * x + y * y)
    return R.astype(np.float32)


def inplane_rotations(angles: np.ndarray) -> np.ndarray:
    c, s = np.cos(angles), np.sin(angles)
    R = np.empty((len(angles), 2, 2))
    R[:, 0, 0] = c
    R[:, 0, 1] = -s
    R[:, 1, 0] = s
    R[:, 1, 1] = c
    return R.astype(np.float32)


def axis_angle(axis: np.ndarray, theta: float) -> np.ndarray:
    """Rodrigues' formula for a unit axis (3,) and an angle in radians."""
    u = np.asarray(axis, dtype=np.float64)
    K = np.array([[0, -u[2], u[1]], [u[2], 0, -u[0]], [-u[1], u[0], 0]])
    return np.eye(3) * math.cos(theta) + math.sin(theta) * K + (1 - math.cos(theta)) * np.outer(u, u)


def tilt_series_rotations(rng: np.random.Generator, n_series: int, n_tilts: int,
                          max_deg: float = 60.0) -> np.ndarray:
    psi = rng.uniform(0.0, 2 * math.pi, n_series)
    out = np.empty((n_series * n_tilts, 3, 3))
    for i in range(n_series):
        axis = np.array([math.cos(psi[i]), math.sin(psi[i]), 0.0])
        for t in range(n_tilts):
            theta = math.radians(-max_deg + t * (2 * max_deg) / (n_tilts - 1))
            out[i * n_tilts + t] = axis_angle(axis, theta)
    return out.astype(np.float32)


# ----------------------------------------------------------------- phantoms

def _ball_points(rng: np.random.Generator, n: int, dim: int, radius: float) -> np.ndarray:
    d = rng.standard_normal((n, dim))
    d /= np.linalg.norm(d, axis=1, keepdims=True)
    r = radius * rng.uniform(0.0, 1.0, n) ** (1.0 / dim)
    return d * r[:, None]


def blob_params(rng: np.random.Generator, N: int, n_blobs: int, sigma=(1.5, 4.0), amp=(0.5, 1.0)):
    """Centres (z, y, x voxel coordinates, uniform in a ball of radius N/4
    about the box centre N//2), widths and amplitudes of the blob phantom."""
    c = _ball_points(rng, n_blobs, 3, N / 4.0) + N // 2
    s = rng.uniform(sigma[0], sigma[1], n_blobs)
    a = rng.uniform(amp[0], amp[1], n_blobs)
    return c, s, a


def blob_volume(rng: np.random.Generator, N: int, n_blobs: int,
                sigma=(1.5, 4.0), amp=(0.5, 1.0)) -> np.ndarray:
    """Sum of isotropic Gaussian blobs on an N^3 grid (z, y, x), centred box
    (parameters from ``blob_params``).

    Each blob is evaluated on a +-4 sigma window (separable), which is exact
    to ~3e-4 of its peak and keeps generation cheap at N = 256..512.
    """
    return render_blobs(blob_params(rng, N, n_blobs, sigma, amp), N)


def render_blobs(params, N: int) -> np.ndarray:
    """The N^3 volume (z, y, x) of blobs with the given (centres, widths,
    amplitudes), each evaluated on a +-4 sigma window."""
    c, s, a = params
    vol = np.zeros((N, N, N), np.float64)
    for i in range(len(s)):
        h = int(math.ceil(4 * s[i]))
        lo = np.maximum(np.floor(c[i]).astype(int) - h, 0)
        hi = np.minimum(np.floor(c[i]).astype(int) + h + 2, N)
        g = [np.exp(-((np.arange(lo[d], hi[d]) - c[i][d]) ** 2) / (2 * s[i] ** 2)) for d in range(3)]
        vol[lo[0]:hi[0], lo[1]:hi[1], lo[2]:hi[2]] += a[i] * g[0][:, None, None] * g[1][None, :, None] * g[2][None, None, :]
    return vol.astype(np.float32)


def blob_images(rng: np.random.Generator, B: int, N: int, n_blobs: int = 20,
                sigma=(2.0, 8.0), amp=(0.5, 1.0), noise: float = 0.1) -> np.ndarray:
    """B images N^2 (y, x): sums of Gaussians (centres in a radius-N/4 disc
    about N//2) plus white noise of standard deviation ``noise``."""
    out = np.empty((B, N, N), np.float32)
    yy = np.arange(N)[:, None]
    xx = np.arange(N)[None, :]
    for b in range(B):
        c = _ball_points(rng, n_blobs, 2, N / 4.0) + N // 2
        s = rng.uniform(sigma[0], sigma[1], n_blobs)
        a = rng.uniform(amp[0], amp[1], n_blobs)
        img = np.zeros((N, N))
        for i in range(n_blobs):
            img += a[i] * np.exp(-((yy - c[i, 0]) ** 2 + (xx - c[i, 1]) ** 2) / (2 * s[i] ** 2))
        img += noise * rng.standard_normal((N, N))
        out[b] = img
    return out


# ---------------------------------------------------------- caller's FFT step

def rfft_spectrum(real: np.ndarray, ndim: int, pad_to: int | None = None,
                  workers: int | None = None) -> np.ndarray:
    """Centred real box(es) -> zero-pad to ``pad_to`` (centred) -> ifftshift
    (box centre to index 0) -> rfftn over the last ``ndim`` axes, complex64.

    This is the caller's preparation step: the projector consumes the
    half-spectrum it returns.  The centre index N//2 maps to M//2 of the padded
    box, so the spectrum of the padded box at even indices equals that of the
    unpadded one when M = 2N.
    """
    import scipy.fft as sfft

    N = real.shape[-1]
    M = N if pad_to is None else int(pad_to)
    axes = tuple(range(-ndim, 0))
    x = np.asarray(real, np.float32)
    if M != N:
        off = M // 2 - N // 2
        shape = x.shape[:-ndim] + (M,) * ndim
        big = np.zeros(shape, np.float32)
        sl = (Ellipsis,) + (slice(off, off + N),) * ndim
        big[sl] = x
        x = big
    x = np.fft.ifftshift(x, axes=axes)
    if workers is None:
        workers = max(1, min(16, len(_affinity())))
    return sfft.rfftn(x, axes=axes, workers=workers).astype(np.complex64)


def _affinity():
    import os
    try:
        return os.sched_getaffinity(0)
    except AttributeError:  # pragma: no cover
        return range(os.cpu_count() or 1)


def complex_normal(rng: np.random.Generator, shape) -> np.ndarray:
    """Complex N(0,1): real and imaginary parts each N(0, 1/2)."""
    z = np.empty(shape, np.complex64)
    z.real = rng.standard_normal(shape, dtype=np.float32) * np.float32(math.sqrt(0.5))
    z.imag = rng.standard_normal(shape, dtype=np.float32) * np.float32(math.sqrt(0.5))
    return z


# ------------------------------------------------------------------ configs

@dataclass
class Workload:
    name: str
    cfg_id: int
    ndim: int          # 3: volume -> images, 2: image -> images
    N: int             # real-space box of the reference
    N_out: int         # output box
    B: int             # batch of references
    P: int             # poses per reference
    interp: int
    cutoff: float
    shift_max: float
    n_blobs: int = 0
    rot_kind: str = "so3"   # so3 | inplane | tilt
    vol_kind: str = "blobs"  # blobs | iid | images
    tilt: tuple = field(default=(0, 0))

    def wh(self, n: int) -> int:
        return n // 2 + 1


WORKLOADS = {
    "c1": Workload("c1", 1, 3, 32, 32, 1, 16, LINEAR, 16.0, 0.0, vol_kind="iid"),
    "c2": Workload("c2", 2, 2, 128, 128, 256, 1, CUBIC, 64.0, 5.0, n_blobs=20,
                   rot_kind="inplane", vol_kind="images"),
    "c3": Workload("c3", 3, 3, 128, 128, 1, 1024, CUBIC, 64.0, 8.0, n_blobs=200),
    "c4": Workload("c4", 4, 3, 256, 256, 1, 4096, CUBIC, 128.0, 10.0, n_blobs=200),
    "c5": Workload("c5", 5, 3, 320, 320, 1, 8192, CUBIC, 160.0, 15.0, n_blobs=1000,
                   rot_kind="tilt", tilt=(128, 64)),
}


def make_real(w: Workload) -> np.ndarray:
    """The real-space reference, centred: [B, N, N, N] (3D) or [B, N, N] (2D), float32."""
    rng = rng_for(w.cfg_id, STREAM_VOLUME)
    if w.vol_kind == "iid":
        return rng.standard_normal((w.N,) * 3).astype(np.float32)[None]
    if w.vol_kind == "blobs":
        return blob_volume(rng, w.N, w.n_blobs)[None]
    if w.vol_kind == "images":
        return blob_images(rng, w.B, w.N, w.n_blobs)
    raise ValueError(w.vol_kind)


def make_reference(w: Workload, pad_to: int | None = None) -> np.ndarray:
    """The reference half-spectrum [B, M, M, M//2+1] (3D) or [B, M, M//2+1] (2D)."""
    return rfft_spectrum(make_real(w), w.ndim, pad_to)


def make_rotations(w: Workload) -> np.ndarray:
    """[B_rot, P, d, d] float32."""
    rng = rng_for(w.cfg_id, STREAM_ROT)
    if w.rot_kind == "so3":
        return uniform_rotations(rng, w.P)[None]
    if w.rot_kind == "inplane":
        ang = rng.uniform(0.0, 2 * math.pi, w.B * w.P)
        return inplane_rotations(ang).reshape(w.B, w.P, 2, 2)
    if w.rot_kind == "tilt":
        return tilt_series_rotations(rng, w.tilt[0], w.tilt[1])[None]
    raise ValueError(w.rot_kind)


def make_shifts(w: Workload) -> np.ndarray:
    """[B_shift, P, 2] float32, (s_x, s_y) in output pixels."""
    rng = rng_for(w.cfg_id, STREAM_SHIFT)
    bs = w.B if w.rot_kind == "inplane" else 1
    if w.shift_max == 0.0:
        return np.zeros((bs, w.P, 2), np.float32)
    return rng.uniform(-w.shift_max, w.shift_max, (bs, w.P, 2)).astype(np.float32)


def make_upstream(w: Workload, poses=None, b: int | None = None) -> np.ndarray:
    """Upstream gradient for the given poses: [B, len(poses), N_out, N_out//2+1]
    complex64 (complex N(0,1)); ``b`` restricts to one batch entry."""
    poses = range(w.P) if poses is None else poses
    bs = range(w.B) if b is None else [b]
    Wo = w.N_out // 2 + 1
    out = np.empty((len(bs), len(poses), w.N_out, Wo), np.complex64)
    for i, bi in enumerate(bs):
        for j, n in enumerate(poses):
            out[i, j] = complex_normal(rng_for(w.cfg_id, STREAM_GRAD, bi, n), (w.N_out, Wo))
    return out
