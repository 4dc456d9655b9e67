"""fp64 CPU oracle (test infrastructure; see ``oracle.projector``)."""
from .projector import (  # noqa: F401
    CUBIC,
    LINEAR,
    backproject,
    backproject_weights,
    grad_pose,
    kernel,
    kernel_deriv,
    lookup,
    output_grid,
    project,
    resolve_taps,
    signed_freq,
    symmetrize_x0,
    tap_offsets,
)
