"""GPU parity of the caller's spectrum step (centred pad -> ifftshift ->
rfftn, ``cryo_em_fourier_amd.spectrum``) against the oracle, alone and
feeding the projector at oversampling 2, plus the full-size c4 case at
oversampling 2 through properties that hold at any size."""
import numpy as np
import pytest

from cryo_em_fourier_amd import synth
import oracle

from _gpu import assert_parity, log, to_dev

pytestmark = pytest.mark.gpu

# (ndim, N, pad_to): even and odd boxes, no padding, padding to 2N and to a
# size that is not a multiple of N
CASES = [(3, 32, None), (3, 32, 64), (3, 31, 62), (3, 24, 40), (2, 64, 128), (2, 63, None), (2, 63, 126)]


def _real(ndim, N, seed):
    rng = np.random.default_rng(seed)
    if ndim == 3:
        return synth.blob_volume(rng, N, 12)[None]
    return synth.blob_images(rng, 2, N, 6)


@pytest.mark.parametrize("ndim,N,M", CASES, ids=[f"{d}d-N{n}-M{m}" for d, n, m in CASES])
def test_spectrum_matches_oracle(ndim, N, M):
    from cryo_em_fourier_amd.spectrum import rfft_spectrum

    log(f"spectrum ndim={ndim} N={N} pad_to={M}")
    x = _real(ndim, N, 100 + N)
    got = rfft_spectrum(to_dev(x), ndim, M).cpu().numpy()
    assert_parity(got, oracle.spectrum(x, ndim, M), f"spectrum {ndim}D N={N} M={M}")


@pytest.mark.parametrize("ndim,N,M", [(3, 32, 64), (3, 31, None), (2, 63, 126)])
def test_real_from_spectrum_inverts_it(ndim, N, M):
    from cryo_em_fourier_amd.spectrum import real_from_spectrum, rfft_spectrum

    x = _real(ndim, N, 200 + N)
    back = real_from_spectrum(rfft_spectrum(to_dev(x), ndim, M), N, ndim).cpu().numpy()
    assert back.shape == x.shape
    assert_parity(back, x, f"round trip {ndim}D N={N} M={M}")


@pytest.mark.parametrize("interp", ["linear", "cubic"])
def test_oversampled_projection_3d_matches_oracle(interp):
    """real volume -> GPU spectrum padded to 2N -> tp_project_3d at
    oversampling 2, against the oracle's spectrum and projection."""
    from cryo_em_fourier_amd import ops
    from cryo_em_fourier_amd.spectrum import rfft_spectrum

    N, n_out, P = 32, 32, 12
    rng = np.random.default_rng(301)
    x = synth.blob_volume(rng, N, 15)[None]
    R = synth.uniform_rotations(rng, P)[None]
    s = rng.uniform(-3.0, 3.0, (1, P, 2)).astype(np.float32)
    log(f"os2 projection 3D interp={interp}")
    V = rfft_spectrum(to_dev(x), 3, 2 * N)
    got = ops.tp_project_3d(V, to_dev(R), to_dev(s), n_out, interp, 2.0, 16.0).cpu().numpy()
    ki = oracle.LINEAR if interp == "linear" else oracle.CUBIC
    ref = oracle.project(oracle.spectrum(x, 3, 2 * N), R, s, n_out, ki, 2.0, 16.0)
    assert_parity(got, ref, f"os2 projection 3D {interp}")


def test_oversampled_projection_2d_matches_oracle():
    from cryo_em_fourier_amd import ops
    from cryo_em_fourier_amd.spectrum import rfft_spectrum

    N, P = 48, 5
    rng = np.random.default_rng(302)
    x = synth.blob_images(rng, 2, N, 6)
    R = synth.inplane_rotations(rng.uniform(0, 2 * np.pi, 2 * P)).reshape(2, P, 2, 2).astype(np.float32)
    s = rng.uniform(-2.0, 2.0, (2, P, 2)).astype(np.float32)
    log("os2 projection 2D cubic")
    V = rfft_spectrum(to_dev(x), 2, 2 * N)
    got = ops.tp_project_2d(V, to_dev(R), to_dev(s), N, "cubic", 2.0, 24.0).cpu().numpy()
    ref = oracle.project(oracle.spectrum(x, 2, 2 * N), R, s, N, oracle.CUBIC, 2.0, 24.0)
    assert_parity(got, ref, "os2 projection 2D cubic")


def test_fullsize_c4_os2_spectrum():
    """The c4 phantom at box 256 padded to 512 on the GPU: the even indices
    of the padded spectrum are the unpadded spectrum (a property of the
    padding at any size), and the padded spectrum equals the reference that
    the oversampling-2 parity tests feed the projector (scipy, on the
    host)."""
    import torch

    from cryo_em_fourier_amd.spectrum import rfft_spectrum

    w = synth.WORKLOADS["c4"]
    x = synth.make_real(w)
    log("c4 spectrum at 256 and padded to 512")
    xd = to_dev(x)
    S1 = rfft_spectrum(xd, 3)
    S2 = rfft_spectrum(xd, 3, 2 * w.N)
    assert S2.shape == (1, 512, 512, 257)
    even = S2[:, ::2, ::2, ::2]
    d = (even - S1).abs().pow(2).sum().sqrt() / S1.abs().pow(2).sum().sqrt()
    m = (even - S1).abs().max() / S1.abs().max()
    log(f"  even indices vs unpadded: rel-L2 {float(d):.2e}  max-abs/max {float(m):.2e}")
    assert float(d) <= 1e-5 and float(m) <= 1e-4
    del S1, even
    ref = torch.from_numpy(synth.make_reference(w, pad_to=2 * w.N)).cuda()
    d = (S2 - ref).abs().pow(2).sum().sqrt() / ref.abs().pow(2).sum().sqrt()
    m = (S2 - ref).abs().max() / ref.abs().max()
    log(f"  padded vs host reference: rel-L2 {float(d):.2e}  max-abs/max {float(m):.2e}")
    assert float(d) <= 1e-5 and float(m) <= 1e-4


def test_spectrum_rejects_bad_input():
    import torch

    from cryo_em_fourier_amd.spectrum import real_from_spectrum, rfft_spectrum

    x = torch.zeros((8, 8, 8), device="cuda")
    with pytest.raises(ValueError):
        rfft_spectrum(x, 3, 4)                       # pad below the box
    with pytest.raises(ValueError):
        rfft_spectrum(torch.zeros((8, 8, 7), device="cuda"), 3)
    with pytest.raises(TypeError):
        rfft_spectrum(x.double(), 3)
    with pytest.raises(ValueError):
        rfft_spectrum(x.cpu(), 3)                    # GPU tensors only
    with pytest.raises(ValueError):
        real_from_spectrum(rfft_spectrum(x, 3), 9)   # crop larger than the box
