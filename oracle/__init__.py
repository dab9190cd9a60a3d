"""float64 CPU oracle for the causal long convolution (1D: forward, short filters, frequency-sparse
filters, state-space filters, gradients, learned Butterfly factors) and the cropped 2D and 3D linear convolutions.

TEST INFRASTRUCTURE ONLY: tests, the smoke check and the bench's CPU-baseline leg may import it;
the product path (the HIP library and its Python binding) never does, and the two share no code.
"""
from .oracle import (  # noqa: F401
    DT_F32, DT_F16, DT_BF16,
    build, conv1d_rows, conv1d_points, conv2d_points, conv2d_dft, conv2d_bwd, conv3d_points, widen,
    ssm_kernel, ssm_rows,
    conv1d_bwd_rows, conv1d_bwd_dk, conv1d_bwd_points, conv1d_bwd_dk_points,
    conv1d_short_points, conv1d_circ_rows, sparse_filter,
    conv1d_short_bwd_rows, conv1d_short_bwd_points, conv1d_short_bwd_dk, conv1d_short_bwd_dk_points,
    transform_length,
    conv1d_toeplitz, conv1d_python_int,
)
from . import butterfly  # noqa: F401,E402
