"""Pins of the oracle's dual-volume weight backprojection and x = 0
symmetrisation (test infrastructure, CPU only).

The weight volume is pinned by closed forms (on-grid identity and half-turn
poses put each weight on one voxel), by conservation of the total weight
(interpolation weights sum to one; folded taps stay inside the volume) and by
the adjoint identity against the forward projection of a real volume (a
different code path of the oracle, pinned in test_oracle_projector.py).
The symmetrisation is pinned by real data (the rfft of a real volume is
already Hermitian), by brute force on a tiny hand-checked case, and by its
algebra (Hermitian result, idempotent, self-adjoint, other planes untouched).
"""
import numpy as np
import pytest

import oracle
from oracle import CUBIC, LINEAR


def rot3(mats):
    return np.asarray(mats, np.float64)[None]


def random_rotations(rng, n):
    q = rng.standard_normal((n, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    w, x, y, z = q.T
    return np.stack([
        np.stack([1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)], -1),
        np.stack([2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)], -1),
        np.stack([2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)], -1)], 1)


# ------------------------------------------------------------ weight volume

@pytest.mark.parametrize("interp", [LINEAR, CUBIC])
def test_weights_identity_pose_lands_on_the_central_plane(interp):
    N, n_out, cutoff = 12, 12, 5.0
    rng = np.random.default_rng(1)
    W = rng.uniform(0.5, 2.0, (1, 1, n_out, n_out // 2 + 1))
    A = oracle.backproject_weights(W, rot3([np.eye(3)]), N, interp, 1.0, cutoff)
    kx, ky, keep = oracle.output_grid(n_out, cutoff)
    want = np.zeros((N, N, N // 2 + 1))
    for iy in range(n_out):
        for ix in range(n_out // 2 + 1):
            if keep[iy, ix]:
                want[0, ky[iy, ix] % N, kx[iy, ix]] += W[0, 0, iy, ix]
    np.testing.assert_allclose(A[0], want, atol=1e-12)


def test_weights_half_turn_folds_onto_the_same_voxels():
    # R = diag(-1, -1, 1): p = (-kx, -ky, 0); taps with x < 0 fold to (kx, ky, 0),
    # taps with x = 0 stay at (0, -ky, 0)
    N, n_out, cutoff = 10, 10, 4.0
    rng = np.random.default_rng(2)
    W = rng.uniform(0.5, 2.0, (1, 1, n_out, n_out // 2 + 1))
    A = oracle.backproject_weights(W, rot3([np.diag([-1.0, -1.0, 1.0])]), N, LINEAR, 1.0, cutoff)
    kx, ky, keep = oracle.output_grid(n_out, cutoff)
    want = np.zeros((N, N, N // 2 + 1))
    for iy in range(n_out):
        for ix in range(n_out // 2 + 1):
            if keep[iy, ix]:
                x, y = kx[iy, ix], ky[iy, ix]
                if x == 0:
                    want[0, (-y) % N, 0] += W[0, 0, iy, ix]
                else:
                    want[0, y % N, x] += W[0, 0, iy, ix]
    np.testing.assert_allclose(A[0], want, atol=1e-12)


@pytest.mark.parametrize("interp,os_", [(LINEAR, 1.0), (CUBIC, 1.0), (CUBIC, 1.5)])
def test_weights_total_is_conserved(interp, os_):
    # every tap of every kept output lies inside the stored range (cutoff well
    # inside the box), and the interpolation weights sum to one
    N, n_out, cutoff = 24, 16, 5.0
    rng = np.random.default_rng(3)
    W = rng.uniform(0.0, 1.0, (2, 5, n_out, n_out // 2 + 1))
    R = random_rotations(rng, 10).reshape(2, 5, 3, 3)
    A = oracle.backproject_weights(W, R, N, interp, os_, cutoff)
    _, _, keep = oracle.output_grid(n_out, cutoff)
    for b in range(2):
        np.testing.assert_allclose(A[b].sum(), W[b][:, keep].sum(), rtol=1e-12)


@pytest.mark.parametrize("interp,ndim", [(LINEAR, 3), (CUBIC, 3), (CUBIC, 2), (LINEAR, 2)])
def test_weights_are_the_adjoint_of_the_real_forward(interp, ndim):
    # sum_k W(k) * S_x(p_k) = sum_t x(t) * A(t) for a real reference x, where
    # S_x is the forward projection (no shift); no cutoff, taps reach the edges
    N, n_out, P = 9, 8, 4
    rng = np.random.default_rng(4 + ndim)
    x = rng.standard_normal((1,) + (N,) * (ndim - 1) + (N // 2 + 1,))
    if ndim == 3:
        R = random_rotations(rng, P)[None]
    else:
        a = rng.uniform(0, 2 * np.pi, P)
        R = np.stack([np.stack([np.cos(a), -np.sin(a)], -1), np.stack([np.sin(a), np.cos(a)], -1)], 1)[None]
    W = rng.standard_normal((1, P, n_out, n_out // 2 + 1))
    fwd = oracle.project(x.astype(np.complex128), R, None, n_out, interp, 1.3, -1.0)
    assert np.abs(fwd.imag).max() < 1e-12  # folded taps of a real reference stay real
    lhs = float(np.sum(W * fwd.real))
    rhs = float(np.sum(x * oracle.backproject_weights(W, R, N, interp, 1.3, -1.0)))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


# -------------------------------------------------------- x = 0 symmetrisation

@pytest.mark.parametrize("N", [8, 9])
def test_symmetrize_keeps_the_spectrum_of_real_data(N):
    rng = np.random.default_rng(N)
    v = rng.standard_normal((2, N, N, N))
    V = np.fft.rfftn(v, axes=(1, 2, 3))
    np.testing.assert_allclose(oracle.symmetrize_x0(V), V, atol=1e-10)
    img = rng.standard_normal((3, N, N))
    I = np.fft.rfftn(img, axes=(1, 2))
    np.testing.assert_allclose(oracle.symmetrize_x0(I), I, atol=1e-10)


def test_symmetrize_tiny_case_by_hand():
    # 2D, N = 4: the x = 0 column pairs rows 1 <-> 3, rows 0 and 2 are their
    # own mirrors (mod 4); values worked out by hand
    V = np.zeros((1, 4, 3), np.complex128)
    V[0, :, 0] = [1 + 2j, 3 - 1j, -2 + 0.5j, 5 + 4j]
    V[0, :, 1] = [7j, 1, 2, 3]
    V[0, :, 2] = [-1, -2j, 0.25, 9]
    out = oracle.symmetrize_x0(V)[0]
    np.testing.assert_allclose(out[:, 0], [1, 4 - 2.5j, -2, 4 + 2.5j], atol=1e-15)
    np.testing.assert_array_equal(out[:, 1:], V[0, :, 1:])


@pytest.mark.parametrize("shape", [(2, 6, 6, 4), (1, 7, 7, 4), (3, 10, 6)])
def test_symmetrize_algebra(shape):
    rng = np.random.default_rng(len(shape) * 10 + shape[1])
    a = rng.standard_normal(shape) + 1j * rng.standard_normal(shape)
    b = rng.standard_normal(shape) + 1j * rng.standard_normal(shape)
    Sa = oracle.symmetrize_x0(a)
    N = shape[1]
    # x = 0 plane Hermitian (mod N), other planes untouched
    if len(shape) == 4:
        for iz in range(N):
            for iy in range(N):
                assert abs(Sa[0, iz, iy, 0] - np.conj(Sa[0, (-iz) % N, (-iy) % N, 0])) < 1e-14
        np.testing.assert_array_equal(Sa[..., 1:], a[..., 1:])
    else:
        for iy in range(N):
            assert abs(Sa[0, iy, 0] - np.conj(Sa[0, (-iy) % N, 0])) < 1e-14
        np.testing.assert_array_equal(Sa[..., 1:], a[..., 1:])
    # idempotent and self-adjoint for Re<u, v>
    np.testing.assert_allclose(oracle.symmetrize_x0(Sa), Sa, atol=1e-14)
    lhs = np.real(np.vdot(Sa, b))
    rhs = np.real(np.vdot(a, oracle.symmetrize_x0(b)))
    assert abs(lhs - rhs) < 1e-10


# ------------------------------------------------- the caller's spectrum step
# A centred delta transforms to 1, an offset delta to a pure phase ramp, and
# zero-padding to 2N samples the same transform twice as finely (the even
# indices are the unpadded spectrum): the definition of the DFT with its
# origin at the box centre, which is what on-the-fly oversampling relies on.

SPECTRUM_CASES = [(3, 8, None), (3, 8, 16), (3, 7, 14), (3, 6, 9), (2, 10, 20), (2, 9, None), (2, 9, 18)]


def _spectrum_shape(ndim, M):
    return (M,) * (ndim - 1) + (M // 2 + 1,)


@pytest.mark.parametrize("ndim,N,M", SPECTRUM_CASES)
def test_spectrum_of_the_centred_delta_is_one(ndim, N, M):
    x = np.zeros((N,) * ndim)
    x[(N // 2,) * ndim] = 1.0
    S = oracle.spectrum(x, ndim, M)
    assert S.shape == _spectrum_shape(ndim, N if M is None else M)
    np.testing.assert_allclose(S, 1.0, rtol=0, atol=1e-12)


@pytest.mark.parametrize("ndim,N,M", SPECTRUM_CASES)
def test_spectrum_of_an_offset_delta_is_a_phase_ramp(ndim, N, M):
    rng = np.random.default_rng(ndim * 100 + N)
    d = rng.integers(-(N // 2), (N + 1) // 2, ndim)      # offset from the centre, array order
    x = np.zeros((N,) * ndim)
    x[tuple(N // 2 + d)] = 1.0
    Mm = N if M is None else M
    S = oracle.spectrum(x, ndim, M)
    grids = np.meshgrid(*[np.arange(n) for n in _spectrum_shape(ndim, Mm)], indexing="ij")
    expect = np.exp(-2j * np.pi * sum(g * di for g, di in zip(grids, d)) / Mm)
    np.testing.assert_allclose(S, expect, rtol=0, atol=1e-11)


@pytest.mark.parametrize("ndim,N", [(3, 8), (3, 7), (2, 12), (2, 11)])
def test_twice_padded_spectrum_at_even_indices_is_the_unpadded_one(ndim, N):
    x = np.random.default_rng(N).standard_normal((2,) + (N,) * ndim)   # a batch of two boxes
    S1 = oracle.spectrum(x, ndim)
    S2 = oracle.spectrum(x, ndim, 2 * N)
    assert S2.shape == (2,) + _spectrum_shape(ndim, 2 * N)
    np.testing.assert_allclose(S2[(Ellipsis,) + (slice(None, None, 2),) * ndim], S1, rtol=0,
                               atol=1e-10 * np.abs(S1).max())


@pytest.mark.parametrize("ndim,N,M", SPECTRUM_CASES)
def test_spectrum_dc_and_parseval(ndim, N, M):
    x = np.random.default_rng(7 + N).standard_normal((N,) * ndim)
    Mm = N if M is None else M
    S = oracle.spectrum(x, ndim, M)
    assert abs(S[(0,) * ndim] - x.sum()) < 1e-10
    # the full spectrum's energy: half-spectrum columns with a mirror that is
    # not stored count twice
    w = np.full(S.shape[-1], 2.0)
    w[0] = 1.0
    if Mm % 2 == 0:
        w[-1] = 1.0
    assert np.isclose(float((np.abs(S) ** 2 * w).sum()), Mm ** ndim * float((x * x).sum()), rtol=1e-12)
