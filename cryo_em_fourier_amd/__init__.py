"""MI355X-native differentiable Fourier-space central-slice projector.

The HIP library (libtp.so, C ABI in include/tp.h) is loaded on first use;
importing the package does not touch the GPU.
"""
from .ops import (  # noqa: F401
    backproject_2d,
    backproject_3d,
    backproject_weights_2d,
    backproject_weights_3d,
    project_2d,
    project_3d,
    rotate_3d,
    tp_backproject_2d,
    tp_backproject_3d,
    tp_backproject_weights_2d,
    tp_backproject_weights_3d,
    tp_grad_pose,
    tp_grad_pose_jac,
    tp_project_2d,
    tp_project_3d,
    tp_project_3d_jac,
    tp_rotate_3d,
    tp_rotate_3d_jac,
    tp_rotate_backproject_3d,
    tp_rotate_grad_pose,
    tp_rotate_grad_pose_jac,
    tp_symmetrize_x0,
)

__all__ = [
    "backproject_2d",
    "backproject_3d",
    "backproject_weights_2d",
    "backproject_weights_3d",
    "project_2d",
    "project_3d",
    "rotate_3d",
    "tp_backproject_2d",
    "tp_backproject_3d",
    "tp_backproject_weights_2d",
    "tp_backproject_weights_3d",
    "tp_grad_pose",
    "tp_grad_pose_jac",
    "tp_project_2d",
    "tp_project_3d",
    "tp_project_3d_jac",
    "tp_rotate_3d",
    "tp_rotate_3d_jac",
    "tp_rotate_backproject_3d",
    "tp_rotate_grad_pose",
    "tp_rotate_grad_pose_jac",
    "tp_symmetrize_x0",
]
