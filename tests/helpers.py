"""Shared helpers of the GPU parity tests."""
import numpy as np
import torch

# Tolerances of the parity bar: max abs error of out and lse against the
# fp64 oracle, by input dtype.
TOL = {torch.bfloat16: 2e-3, torch.float32: 1e-5}


def f64(t: torch.Tensor) -> np.ndarray:
    """Exact float64 copy of a device tensor (bf16/fp32 -> fp64 is exact)."""
    return t.detach().to("cpu", torch.float64).numpy()


def f32(t: torch.Tensor) -> np.ndarray:
    """Exact float32 copy of a bf16/fp32 device tensor (half the host memory
    of f64 for large pools)."""
    return t.detach().to("cpu", torch.float32).numpy()


def max_err(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    d = np.where(both_inf, 0.0, np.abs(a - b))
    return float(np.nan_to_num(d, nan=np.inf).max()) if d.size else 0.0


def packed_to_device(p, dev):
    return dict(codes=torch.from_numpy(np.ascontiguousarray(p["codes"]).view(np.int32)).to(dev),
                zs=torch.from_numpy(np.ascontiguousarray(p["zs"]).view(np.int16)).to(dev),
                res=torch.from_numpy(np.ascontiguousarray(p["res"])).to(dev),
                rs=torch.from_numpy(np.ascontiguousarray(p["rs"]).view(np.int16)).to(dev))


def packed_to_host(p):
    return dict(codes=p["codes"].cpu().numpy().view(np.uint32),
                zs=p["zs"].cpu().numpy().view(np.float16),
                res=p["res"].cpu().numpy(),
                rs=p["rs"].cpu().numpy().view(np.float16))


def banner(msg: str):
    print(msg, flush=True)
