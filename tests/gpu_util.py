"""Helpers for GPU parity tests: move seeded numpy inputs to the device in the
dtype the C ABI expects, and compare against the fp64 oracle."""
import numpy as np

TOL_BF16 = 2e-3   # relative L2 bound for bf16 q/k/v inputs
TOL_F32 = 1e-5    # relative L2 bound for the fp32 path


def torch_mod():
    import torch
    return torch


def dev(x, bf16=False):
    """float32 numpy array -> contiguous device tensor (bf16 when asked; the
    values are already bf16-exact, so the cast is exact)."""
    torch = torch_mod()
    if x is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if bf16:
        t = t.to(torch.bfloat16)
    return t.to("cuda").contiguous()


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def report(name, **errs):
    print("[parity] %s %s" % (name, " ".join("%s=%.3e" % kv for kv in errs.items())), flush=True)
