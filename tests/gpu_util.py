"""Helpers shared by the GPU parity tests (imports torch lazily)."""

import numpy as np


def tolerance_report(got, want):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    err = np.abs(got - want)
    max_abs = float(err.max()) if err.size else 0.0
    rel_l2 = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-300))
    return max_abs, rel_l2


def assert_attention_close(got, want, max_abs=2e-3, rel_l2=1e-3, what=""):
    """The attention bar: max-abs <= 2e-3 and relative L2 <= 1e-3 against the
    float64 oracle (rounded to float32)."""
    want32 = np.asarray(want, np.float64).astype(np.float32)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ma, rl = tolerance_report(got, want32)
    assert ma <= max_abs and rl <= rel_l2, f"{what}: max_abs={ma:.3g} rel_l2={rl:.3g}"
    return ma, rl


def cuda(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def bf16_cuda(x):
    """float32 values that are exactly bfloat16 -> a bfloat16 CUDA tensor."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    b = t.to(torch.bfloat16)
    assert torch.equal(b.to(torch.float32), t), "input is not bf16-exact"
    return b.cuda()
