"""The caller's spectrum step on the GPU, before the projector and after its
adjoint.

The projector samples a reference given as the rfft half-spectrum of a
real box whose centre sits at index 0.  Oversampling by os on the fly
means zero-padding the centred box to os * N in real space and taking that
FFT on every pass (torch-projectors pages, results section on
interpolation: cubic at oversampling 1 avoids exactly this padding and
FFT; tech. section 2: the reference layout is PyTorch's rfftn).

``rfft_spectrum`` does centred zero-pad -> ifftshift -> rfftn with
torch.fft (rocFFT) on the tensor's device; ``real_from_spectrum`` inverts
it (irfftn -> fftshift -> crop of the centred box), which is how a volume
gradient from the adjoint returns to real space.  Both run on a GPU
tensor only: there is no CPU path.
"""
from __future__ import annotations

import torch


def _check(x: torch.Tensor, ndim: int) -> None:
    if ndim not in (2, 3):
        raise ValueError("ndim must be 2 or 3")
    if not x.is_cuda:
        raise ValueError("the spectrum step runs on a GPU tensor")
    if x.dim() < ndim:
        raise ValueError(f"need at least {ndim} dimensions")


def rfft_spectrum(real: torch.Tensor, ndim: int = 3, pad_to: int | None = None) -> torch.Tensor:
    """Centred real box(es) ``real[..., N, N(, N)]`` (float32; leading axes
    are a batch) -> zero-pad to ``pad_to`` = M >= N with the centre N // 2
    placed at M // 2 -> ifftshift (centre to index 0) -> rfftn over the last
    ``ndim`` axes.  Returns complex64 ``[..., M(, M), M // 2 + 1]``,
    contiguous: the reference layout of tp_project_3d / tp_project_2d at
    oversampling M / N."""
    _check(real, ndim)
    if real.dtype != torch.float32:
        raise TypeError("real must be float32")
    N = real.shape[-1]
    if any(d != N for d in real.shape[-ndim:]):
        raise ValueError("the box must be a cube (square)")
    M = N if pad_to is None else int(pad_to)
    if M < N:
        raise ValueError("pad_to must be at least the box size")
    x = real
    if M != N:
        off = M // 2 - N // 2
        x = real.new_zeros(real.shape[:-ndim] + (M,) * ndim)
        x[(Ellipsis,) + (slice(off, off + N),) * ndim] = real
    dims = tuple(range(-ndim, 0))
    return torch.fft.rfftn(torch.fft.ifftshift(x, dim=dims), dim=dims).contiguous()


def real_from_spectrum(spec: torch.Tensor, n: int, ndim: int = 3) -> torch.Tensor:
    """Inverse of ``rfft_spectrum``: the half-spectrum ``spec[..., M(, M),
    M // 2 + 1]`` -> irfftn to the M box -> fftshift (index 0 back to the
    centre) -> the centred n box, float32 ``[..., n, n(, n)]``."""
    _check(spec, ndim)
    if not spec.is_complex():
        raise TypeError("spec must be complex")
    M = spec.shape[-2]
    if spec.shape[-1] != M // 2 + 1 or (ndim == 3 and spec.shape[-3] != M):
        raise ValueError("not an rfft half-spectrum of a cube (square)")
    if not 1 <= n <= M:
        raise ValueError("n must be in [1, M]")
    dims = tuple(range(-ndim, 0))
    x = torch.fft.fftshift(torch.fft.irfftn(spec, s=(M,) * ndim, dim=dims), dim=dims)
    off = M // 2 - n // 2
    return x[(Ellipsis,) + (slice(off, off + n),) * ndim].contiguous()
