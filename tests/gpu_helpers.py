"""Helpers for GPU parity tests: move seeded host inputs to the device and
compare library outputs with the oracle's."""
import sys

import numpy as np

from trainable_block_sparse_gate_amd import workloads as wl

# parity tolerances: max-abs 2e-2 for bf16 paths, 1e-4 for fp32 paths
TOL = {"bf16": 2e-2, "f32": 1e-4}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_tensor(arr_f32, bits, dtype, device="cuda"):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(arr_f32, np.float32)).to(device)


def case_to_device(case: wl.VarlenCase, device="cuda"):
    import torch
    out = {}
    for nm in ("q", "k", "v", "dO"):
        arr = getattr(case, nm)
        if arr is None:
            continue
        out[nm] = dev_tensor(arr, case.bits.get(nm), case.dtype, device)
    out["logits"] = torch.from_numpy(case.logits).to(device)
    return out


def max_abs(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


def assert_close(name, got, want, tol):
    err = max_abs(got, want)
    scale = float(np.max(np.abs(want))) if np.size(want) else 0.0
    say(f"  {name}: max_abs={err:.3e} (max|ref|={scale:.3e}, tol={tol:g})")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    assert err <= tol, f"{name}: max_abs {err} > {tol}"


def summaries_f32(ksum):
    """Block summaries as the fp32 values they stand for, indexed [batch][kv
    head][block][channel] (fp8 summaries are stored as e4m3 codes in uint8;
    torch's float8_e4m3fn decodes them exactly)."""
    import torch
    from trainable_block_sparse_gate_amd import sas
    ksum = sas.summaries_by_block(ksum)  # [batch][hkv][block][channel]
    if ksum.dtype == torch.uint8:
        return ksum.view(torch.float8_e4m3fn).float().cpu().numpy()
    return ksum.float().cpu().numpy()
