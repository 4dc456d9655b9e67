"""Pins of the oracle's 3D -> 3D rotation (test infrastructure, CPU only).

* identity pose: the output is the reference itself (both kernels pass
  through the grid values);
* cube rotations: the output is the rfftn of the real volume rotated on the
  grid, v_R(x) = v(R^T x) (the central slice's convention, one dimension up);
* integer shifts: the output is the rfftn of np.roll of the real volume;
* its kz = 0 plane is the central-slice projection at any pose;
* the adjoint identity and finite differences of the pose gradients.
"""
import itertools

import numpy as np
import pytest

import oracle
from oracle import CUBIC, LINEAR


def cube_rotations():
    mats = []
    for perm in itertools.permutations(range(3)):
        for signs in itertools.product((1, -1), repeat=3):
            M = np.zeros((3, 3))
            for i, j in enumerate(perm):
                M[i, j] = signs[i]
            if np.isclose(np.linalg.det(M), 1.0):
                mats.append(M)
    return mats


def rotate_real(v, R):
    """v_R[x] = v[R^T x] on the periodic grid, coordinates (x, y, z) = last,
    middle, first array axis, origin at index 0."""
    N = v.shape[0]
    out = np.empty_like(v)
    idx = np.arange(N)
    Z, Y, X = np.meshgrid(idx, idx, idx, indexing="ij")
    coords = np.stack([X, Y, Z], -1).reshape(-1, 3)                  # (x, y, z)
    src = (coords @ np.rint(R).astype(np.int64)) % N                  # R^T x, row-vector form
    out.reshape(-1)[:] = v[src[:, 2], src[:, 1], src[:, 0]]
    return out


@pytest.mark.parametrize("interp", [LINEAR, CUBIC])
def test_identity_returns_the_reference(interp):
    rng = np.random.default_rng(1)
    N = 8
    V = rng.standard_normal((1, N, N, N // 2 + 1)) + 1j * rng.standard_normal((1, N, N, N // 2 + 1))
    out = oracle.rotate_3d(V, np.eye(3)[None, None], None, N, interp)
    np.testing.assert_allclose(out[0, 0], V[0], atol=1e-12)


@pytest.mark.parametrize("N", [8, 9])
def test_cube_rotations_rotate_the_real_volume(N):
    rng = np.random.default_rng(N)
    v = rng.standard_normal((N, N, N))
    V = np.fft.rfftn(v)[None]
    mats = cube_rotations()
    assert len(mats) == 24
    R = np.stack(mats)[None]
    # inside the sphere |k| <= N/2 - 1 no rotated frequency reaches the
    # Nyquist planes, which exist on one side only of the stored range
    cutoff = N // 2 - 1
    out = oracle.rotate_3d(V, R, None, N, CUBIC, 1.0, cutoff)
    keep = oracle.output_grid_3d(N, cutoff)[3]
    for n, M in enumerate(mats):
        want = np.where(keep, np.fft.rfftn(rotate_real(v, M)), 0.0)
        np.testing.assert_allclose(out[0, n], want, atol=1e-9, err_msg=str(M))


def test_integer_shift_is_a_roll():
    rng = np.random.default_rng(5)
    N = 10
    v = rng.standard_normal((N, N, N))
    s = np.array([[[2.0, -3.0, 1.0]]])
    out = oracle.rotate_3d(np.fft.rfftn(v)[None], np.eye(3)[None, None], s, N, LINEAR)
    want = np.fft.rfftn(np.roll(v, (1, -3, 2), axis=(0, 1, 2)))
    np.testing.assert_allclose(out[0, 0], want, atol=1e-9)


@pytest.mark.parametrize("interp,os_", [(LINEAR, 1.0), (CUBIC, 1.3)])
def test_kz0_plane_is_the_central_slice(interp, os_):
    rng = np.random.default_rng(6)
    N, n_out, P = 12, 10, 3
    V = rng.standard_normal((1, N, N, N // 2 + 1)) + 1j * rng.standard_normal((1, N, N, N // 2 + 1))
    q = rng.standard_normal((P, 4))
    q /= np.linalg.norm(q, axis=1, keepdims=True)
    w, x, y, z = q.T
    R = np.stack([np.stack([1 - 2 * (y * y + z * z), 2 * (x * y - w * z), 2 * (x * z + w * y)], -1),
                  np.stack([2 * (x * y + w * z), 1 - 2 * (x * x + z * z), 2 * (y * z - w * x)], -1),
                  np.stack([2 * (x * z - w * y), 2 * (y * z + w * x), 1 - 2 * (x * x + y * y)], -1)], 1)[None]
    s2 = rng.uniform(-2, 2, (1, P, 2))
    s3 = np.concatenate([s2, rng.uniform(-2, 2, (1, P, 1))], -1)
    vol = oracle.rotate_3d(V, R, s3, n_out, interp, os_, 4.5)
    sl = oracle.project(V, R, s2, n_out, interp, os_, 4.5)
    np.testing.assert_allclose(vol[:, :, 0], sl, atol=1e-12)


@pytest.mark.parametrize("interp", [LINEAR, CUBIC])
def test_rotate_adjoint_identity(interp):
    rng = np.random.default_rng(7 + interp)
    N, n_out, P = 7, 6, 2
    x = rng.standard_normal((1, N, N, N // 2 + 1)) + 1j * rng.standard_normal((1, N, N, N // 2 + 1))
    y = (rng.standard_normal((1, P, n_out, n_out, n_out // 2 + 1))
         + 1j * rng.standard_normal((1, P, n_out, n_out, n_out // 2 + 1)))
    R = np.stack([np.linalg.qr(rng.standard_normal((3, 3)))[0] for _ in range(P)])[None]
    s = rng.uniform(-2, 2, (1, P, 3))
    lhs = np.real(np.vdot(oracle.rotate_3d(x, R, s, n_out, interp, 1.2, -1.0), y))
    rhs = np.real(np.vdot(x, oracle.rotate_backproject_3d(y, R, s, N, interp, 1.2, -1.0)))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


def test_rotate_gradients_match_finite_differences():
    rng = np.random.default_rng(11)
    N, n_out, P = 8, 6, 2
    V = np.fft.rfftn(rng.standard_normal((N, N, N)))[None]
    G = (rng.standard_normal((1, P, n_out, n_out, n_out // 2 + 1))
         + 1j * rng.standard_normal((1, P, n_out, n_out, n_out // 2 + 1)))
    R = np.stack([np.linalg.qr(rng.standard_normal((3, 3)))[0] for _ in range(P)])[None]
    s = rng.uniform(-2, 2, (1, P, 3))

    def loss(Rv, sv):
        return np.real(np.vdot(G, oracle.rotate_3d(V, Rv, sv, n_out, CUBIC, 1.0, 3.5)))

    dR, ds = oracle.rotate_grad_pose(V, G, R, s, n_out, CUBIC, 1.0, 3.5)
    h = 1e-6
    for n in range(P):
        for i in range(3):
            for j in range(3):
                Rp, Rm = R.copy(), R.copy()
                Rp[0, n, i, j] += h
                Rm[0, n, i, j] -= h
                fd = (loss(Rp, s) - loss(Rm, s)) / (2 * h)
                assert abs(fd - dR[0, n, i, j]) <= 1e-5 * max(1.0, abs(fd)), (n, i, j, fd, dR[0, n, i, j])
        for j in range(3):
            sp, sm = s.copy(), s.copy()
            sp[0, n, j] += h
            sm[0, n, j] -= h
            fd = (loss(R, sp) - loss(R, sm)) / (2 * h)
            assert abs(fd - ds[0, n, j]) <= 1e-5 * max(1.0, abs(fd)), (n, j, fd, ds[0, n, j])

# Lattice points on the sphere of radius 5 (Pythagorean triples and the axes),
# written out by hand: the cutoff keeps |k| <= c, boundary included.
ON_SPHERE_5 = [(5, 0, 0), (0, 5, 0), (0, 0, 5), (0, -5, 0), (0, 0, -5), (3, 4, 0), (4, 3, 0), (4, 0, 3),
               (3, 0, 4), (0, 3, 4), (0, 4, 3), (3, -4, 0), (4, 0, -3), (0, -3, 4), (0, 4, -3), (0, -4, -3)]
JUST_OUTSIDE_5 = [(5, 1, 0), (1, 0, 5), (4, 3, 1), (0, 5, 1), (3, 4, 1), (1, 5, 0)]


def test_sphere_cutoff_keeps_its_boundary():
    """At the identity pose the output is the reference inside the sphere:
    points with |k| = 5 exactly keep their value at cutoff 5, points with
    |k|^2 = 26 are zero."""
    rng = np.random.default_rng(21)
    N = 12
    V = rng.standard_normal((1, N, N, N // 2 + 1)) + 1j * rng.standard_normal((1, N, N, N // 2 + 1))
    out = oracle.rotate_3d(V, np.eye(3)[None, None], None, N, CUBIC, 1.0, 5.0)[0, 0]
    for kx, ky, kz in ON_SPHERE_5:
        assert out[kz % N, ky % N, kx] == pytest.approx(V[0, kz % N, ky % N, kx], abs=1e-12), (kx, ky, kz)
    for kx, ky, kz in JUST_OUTSIDE_5:
        assert out[kz % N, ky % N, kx] == 0, (kx, ky, kz)
    # and the count of kept entries is the number of lattice points in the
    # ball of radius 5 with kx >= 0 (brute force over the box)
    kept = sum(1 for kx in range(0, 6) for ky in range(-5, 6) for kz in range(-5, 6)
               if kx * kx + ky * ky + kz * kz <= 25)
    assert int(np.count_nonzero(out)) == kept


def test_sphere_cutoff_zero_keeps_only_dc():
    rng = np.random.default_rng(22)
    N = 8
    V = rng.standard_normal((1, N, N, N // 2 + 1)) + 1j * rng.standard_normal((1, N, N, N // 2 + 1))
    out = oracle.rotate_3d(V, np.eye(3)[None, None], None, N, LINEAR, 1.0, 0.0)[0, 0]
    assert out[0, 0, 0] == pytest.approx(V[0, 0, 0, 0], abs=1e-12)
    out[0, 0, 0] = 0
    assert not out.any()


@pytest.mark.parametrize("interp", [LINEAR, CUBIC])
def test_kz0_plane_is_the_slice_at_an_integer_cutoff(interp):
    """Cutoff 5 puts (3, 4), (4, 3), (5, 0) and (0, 5) on the circle: the
    sphere's kz = 0 plane and the slice's disk must keep the same entries."""
    rng = np.random.default_rng(23)
    N = 12
    V = rng.standard_normal((1, N, N, N // 2 + 1)) + 1j * rng.standard_normal((1, N, N, N // 2 + 1))
    R = np.stack([np.linalg.qr(rng.standard_normal((3, 3)))[0] for _ in range(2)])[None]
    vol = oracle.rotate_3d(V, R, None, N, interp, 1.0, 5.0)
    sl = oracle.project(V, R, None, N, interp, 1.0, 5.0)
    np.testing.assert_allclose(vol[:, :, 0], sl, atol=1e-12)
    assert np.all(sl[0, :, 4, 3] != 0) and np.all(sl[0, :, 3, 4] != 0)
