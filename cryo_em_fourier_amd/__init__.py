"""MI355X-native differentiable Fourier-space central-slice projector.

The HIP library (libtp.so, C ABI in include/tp.h) is loaded on first use;
importing the package does not touch the GPU.
"""
from .ops import (  # noqa: F401
    project_2d,
    project_3d,
    tp_backproject_2d,
    tp_backproject_3d,
    tp_grad_pose,
    tp_project_2d,
    tp_project_3d,
)

__all__ = [
    "project_2d",
    "project_3d",
    "tp_backproject_2d",
    "tp_backproject_3d",
    "tp_grad_pose",
    "tp_project_2d",
    "tp_project_3d",
]
