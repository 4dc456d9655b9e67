"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake in a temporary copy of ``oracle/projector.py``
(on the CPU, never touching the real oracle) and runs the oracle pin tests
against it in a subprocess; the run must fail.  The mistakes are the kind a
reader of the pages could make: a flipped phase sign, a missing conjugate on
a folded tap, a fold at the wrong x, a shifted stencil, R used instead of
R^T, a stored range one entry too wide, a non-conjugated adjoint phase, a
dropped gradient row, a wrong kernel-derivative term, a sign error in the
folded index.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = [
    ("phase sign", "np.exp(-2j * np.pi", "np.exp(2j * np.pi"),
    ("fold at x < -1", "conj = t[..., 0] < 0", "conj = t[..., 0] < -1"),
    ("no conjugate on folded taps", "v = np.where(conj, np.conj(v), v)", "v = v"),
    ("cubic stencil shifted", "else (-1, 0, 1, 2)", "else (-2, -1, 0, 1)"),
    ("R instead of R^T",
     "kx[:, None] * Rm[0][None, :] + ky[:, None] * Rm[1][None, :]",
     "kx[:, None] * Rm[:, 0][None, :] + ky[:, None] * Rm[:, 1][None, :]"),
    ("stored range one too wide",
     "lo, hi = -(N // 2), (N + 1) // 2 - 1", "lo, hi = -(N // 2) - 1, (N + 1) // 2"),
    ("adjoint ignores the fold", "val = w * np.where(conj, np.conj(c), c)", "val = w * c"),
    ("gradient row dropped", "dR[br, n, 1, :] += float(os)", "dR[br, n, 1, :] += 0 * float(os)"),
    ("kernel derivative term", "- 2 * (a + 3) * t\n", "- 2 * (a + 2) * t\n"),
    ("adjoint phase not conjugated",
     "c = np.conj(_phase(kxk, kyk, sv, n_out)) * G[b, n][keep]",
     "c = _phase(kxk, kyk, sv, n_out) * G[b, n][keep]"),
    ("folded index sign", "idx = idx * N + np.mod(tt[..., j], N)", "idx = idx * N + np.mod(-tt[..., j], N)"),
    ("2D cutoff exclusive", "keep = (kx * kx + ky * ky).astype(np.float64) <= float(cutoff) ** 2",
     "keep = (kx * kx + ky * ky).astype(np.float64) < float(cutoff) ** 2"),
    ("3D cutoff exclusive", "keep = (kx * kx + ky * ky + kz * kz).astype(np.float64) <= float(cutoff) ** 2",
     "keep = (kx * kx + ky * ky + kz * kz).astype(np.float64) < float(cutoff) ** 2"),
    ("weights without interpolation weight", "np.add.at(Aflat, idx[valid], (w * c)[valid])",
     "np.add.at(Aflat, idx[valid], c[valid])"),
    ("weights stencil from round", "            base = np.floor(p).astype(np.int64)\n            for d",
     "            base = np.round(p).astype(np.int64)\n            for d"),
    ("symmetrize mirror off by one", "mz, my = (-iz) % N, (-iy) % N", "mz, my = (N - 1 - iz) % N, (N - 1 - iy) % N"),
    ("symmetrize without conjugate", "0.5 * (V[b, iz, iy, 0] + np.conj(V[b, mz, my, 0]))",
     "0.5 * (V[b, iz, iy, 0] + V[b, mz, my, 0])"),
    ("symmetrize not halved 2D", "0.5 * (V[b, iy, 0] + np.conj(V[b, my, 0]))", "(V[b, iy, 0] + np.conj(V[b, my, 0]))"),
    ("rotation uses R, not R^T",
     "kx[:, None] * Rm[0][None, :] + ky[:, None] * Rm[1][None, :] + kz[:, None] * Rm[2][None, :]",
     "kx[:, None] * Rm[:, 0][None, :] + ky[:, None] * Rm[:, 1][None, :] + kz[:, None] * Rm[:, 2][None, :]"),
    ("rotation drops kz", "+ kz[:, None] * Rm[2][None, :])", ")"),
    ("3D phase drops s_z", "(kx * sv[0] + ky * sv[1] + kz * sv[2]) / n_out", "(kx * sv[0] + ky * sv[1]) / n_out"),
    ("spectrum pad off centre", "off = M // 2 - N // 2", "off = M // 2 - (N - 1) // 2"),
    ("spectrum without ifftshift", "np.fft.rfftn(np.fft.ifftshift(big, axes=axes), axes=axes)",
     "np.fft.rfftn(big, axes=axes)"),
    ("rotation gradient row 2 dropped", "for i in range(3):\n                dR[br, n, i, :]", "for i in range(2):\n                dR[br, n, i, :]"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path):
    for d in ("oracle", "tests"):
        shutil.copytree(os.path.join(ROOT, d), tmp_path / d,
                        ignore=shutil.ignore_patterns("__pycache__"))
    pkg = tmp_path / "cryo_em_fourier_amd"
    pkg.mkdir()
    (pkg / "__init__.py").write_text("")
    shutil.copy(os.path.join(ROOT, "cryo_em_fourier_amd", "synth.py"), pkg / "synth.py")
    src = (tmp_path / "oracle" / "projector.py").read_text()
    assert src.count(old) >= 1, f"mutation anchor not found: {old!r}"
    (tmp_path / "oracle" / "projector.py").write_text(src.replace(old, new))
    env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
         "tests/test_oracle_kernels.py", "tests/test_oracle_projector.py", "tests/test_oracle_extras.py",
         "tests/test_oracle_rotate.py"],
        cwd=tmp_path, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch: {name}\n{r.stdout[-2000:]}"
