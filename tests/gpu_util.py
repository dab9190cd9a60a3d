"""Helpers shared by the GPU tests: host <-> device transfer of storage-dtype arrays and the
error metric.  No convolution arithmetic lives here."""
import sys

import numpy as np

import oracle
from fft_long_convolution_amd import workloads as wl

TOL = {"f32": 1e-4, "f16": 2e-2, "bf16": 2e-2}
DT_ORACLE = {"f32": oracle.DT_F32, "f16": oracle.DT_F16, "bf16": oracle.DT_BF16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def to_dev(a, dtype):
    import torch
    if a is None:
        return None
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def from_dev(t, dtype):
    import torch
    if dtype == "bf16":
        return wl.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.float().cpu().numpy().astype(np.float64)


def rel_l2_rows(got, ref):
    """Relative L2 error per row (last axis)."""
    num = np.linalg.norm(got - ref, axis=-1)
    den = np.linalg.norm(ref, axis=-1)
    return num / np.maximum(den, 1e-300)


def rel_l2(got, ref):
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
