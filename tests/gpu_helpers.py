"""Helpers shared by the GPU parity tests: device transfer, error metrics,
tolerances.  Tolerances (stated with the workloads): fp32 inputs, relative L2
<= 1e-5; bf16 inputs, relative L2 <= 5e-3 and max |err| <= 2e-2 * max |ref|,
applied to every output tensor (o and the final states)."""
import sys

import numpy as np

TOL_FP32_REL_L2 = 1e-5
TOL_BF16_REL_L2 = 5e-3
TOL_BF16_MAX_ABS = 2e-2


def log(msg: str):
    sys.stderr.write(msg + "\n")
    sys.stderr.flush()


def to_dev(a: np.ndarray):
    import torch

    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_host(t) -> np.ndarray:
    import torch

    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


class ErrAcc:
    """Accumulates ||gpu - ref||^2, ||ref||^2 and the max errors over chunks."""

    def __init__(self):
        self.d2 = 0.0
        self.r2 = 0.0
        self.max_err = 0.0
        self.max_ref = 0.0
        self.n = 0

    def add(self, gpu, ref):
        g = as_f64(gpu) if gpu.dtype != np.float64 else gpu
        r = np.asarray(ref, dtype=np.float64)
        assert g.shape == r.shape, (g.shape, r.shape)
        if not np.all(np.isfinite(g)):
            self.d2 = float("inf")
        diff = g - r
        self.d2 += float(np.sum(diff * diff))
        self.r2 += float(np.sum(r * r))
        if diff.size:
            self.max_err = max(self.max_err, float(np.max(np.abs(diff))))
            self.max_ref = max(self.max_ref, float(np.max(np.abs(r))))
        self.n += r.size
        return self

    @property
    def rel_l2(self):
        if self.r2 == 0.0:
            return 0.0 if self.d2 == 0.0 else float("inf")
        return float(np.sqrt(self.d2 / self.r2))

    @property
    def max_rel(self):
        if self.max_ref == 0.0:
            return 0.0 if self.max_err == 0.0 else float("inf")
        return self.max_err / self.max_ref

    def check(self, fp32: bool, what: str):
        log(f"    {what}: rel_l2={self.rel_l2:.3e} max_err/max_ref={self.max_rel:.3e} n={self.n}")
        if fp32:
            assert self.rel_l2 <= TOL_FP32_REL_L2, f"{what}: rel L2 {self.rel_l2:.3e} > {TOL_FP32_REL_L2}"
        else:
            assert self.rel_l2 <= TOL_BF16_REL_L2, f"{what}: rel L2 {self.rel_l2:.3e} > {TOL_BF16_REL_L2}"
            assert self.max_rel <= TOL_BF16_MAX_ABS, f"{what}: max err {self.max_rel:.3e} > {TOL_BF16_MAX_ABS}"


def bf16_rne_from_f64(x: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits (via fp32, both round-to-nearest-even); exact-integer tests only."""
    f = np.asarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lower = u >> 16
    rem = u & 0xFFFF
    up = (rem > 0x8000) | ((rem == 0x8000) & ((lower & 1) == 1))
    return (lower + up).astype(np.uint16)
