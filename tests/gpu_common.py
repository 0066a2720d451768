"""Shared plumbing of the GPU parity tests: device tensors from the seeded
generators, raw-bit views, and the tolerances the tests hold the HIP path to.

Inputs come from `workloads` (numpy, seeded) and reach both sides: the HIP
library through device tensors, the oracle as exact float64 copies. Nothing
the HIP library writes is ever fed to the oracle.
"""
import numpy as np
import torch

import decoder_attention_rope_amd as gqa

DEV = "cuda"
# Max abs error allowed against the fp64 oracle: bf16 inputs with f32
# accumulation, and the all-f32 path.
TOL = {"bf16": 2e-2, "f32": 1e-4}
TORCH_DT = {"bf16": torch.bfloat16, "f32": torch.float32}
CODE = {"bf16": gqa.GQA_BF16, "f32": gqa.GQA_F32}


def host_values(x_f32, dtype):
    """float32 samples -> exact T values (CPU tensor of T, and float64 copy)."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32)).to(TORCH_DT[dtype])
    return t, t.to(torch.float64).numpy()


def dev(t):
    return t.to(DEV)


def i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def bits(t):
    """Raw bit pattern of a T tensor as int64 numpy (for bitwise compares)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().astype(np.int64) & 0xFFFF
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().astype(np.int64) & 0xFFFFFFFF
    raise TypeError(t.dtype)


def f64(t):
    return t.detach().cpu().to(torch.float64).numpy()


def workspace(nbytes):
    n = max(int(nbytes), 256)
    return torch.empty(n, dtype=torch.uint8, device=DEV), n


def poison_like(shape, dtype):
    """NaN-filled T tensor on the device: any stray read shows up."""
    return torch.full(shape, float("nan"), dtype=TORCH_DT[dtype], device=DEV)


def max_err(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    if got.size == 0:
        return 0.0
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(np.max(np.abs(got - ref)))


def assert_close(got, ref, dtype, what):
    err = max_err(got, ref)
    print(f"[parity] {what}: max abs err {err:.3e} (tol {TOL[dtype]:.0e})", flush=True)
    assert err <= TOL[dtype], f"{what}: max abs err {err:.3e} > {TOL[dtype]:.0e}"
