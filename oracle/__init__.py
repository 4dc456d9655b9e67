"""fp64 CPU oracle (test infrastructure; see ``oracle.projector``)."""
from .projector import (  # noqa: F401
    CUBIC,
    LINEAR,
    backproject,
    grad_pose,
    kernel,
    kernel_deriv,
    lookup,
    output_grid,
    project,
    resolve_taps,
    signed_freq,
    tap_offsets,
)
