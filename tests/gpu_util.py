"""Shared helpers of the GPU tests: seeded inputs on both sides, the oracle
call, and the parity bar.

Parity bar (element by element against the fp64 oracle):
  bf16 storage: max-abs <= 2e-2 and relative L2 <= 5e-3
  fp32 storage: max-abs <= 1e-4 and relative L2 <= 1e-4
Cache bytes, untouched slots, lengths and mask placement: bit-exact.
"""
import json
import os
import sys

import torch

import oracle
from phase_aware_swa_amd import inputs

TOL = {torch.bfloat16: (2e-2, 5e-3), torch.float32: (1e-4, 1e-4)}


def say(*a):
    """Names the case on stdout before a GPU step (flushed)."""
    print(*a, flush=True)
    sys.stdout.flush()


def errors(gpu, ref, chunk=1 << 24):
    """(max-abs, relative L2) of gpu against ref, accumulated in fp64 over
    slices of the first dimension so that full-size outputs need no fp64
    copy of their own."""
    g_all = gpu.detach()
    n = g_all.shape[0] if g_all.dim() else 1
    per = max(1, g_all[0].numel() if g_all.dim() else 1)
    step = max(1, chunk // per)
    max_abs, dsq, rsq = 0.0, 0.0, 0.0
    for i in range(0, n, step):
        g = (g_all[i:i + step] if g_all.dim() else g_all).to("cpu", torch.float64)
        r = (ref[i:i + step] if ref.dim() else ref).to(torch.float64)
        assert torch.isfinite(g).all(), "non-finite values in the GPU output"
        d = g - r
        if d.numel():
            max_abs = max(max_abs, d.abs().max().item())
        dsq += float((d * d).sum())
        rsq += float((r * r).sum())
    rel = (dsq ** 0.5) / (rsq ** 0.5) if rsq > 0 else dsq ** 0.5
    return max_abs, rel


def record(case, what, max_abs, rel, n):
    """Appends one parity result to the JSON-lines file named by
    ORTHROS_PARITY_LOG (nothing when it is unset)."""
    path = os.environ.get("ORTHROS_PARITY_LOG")
    if not path:
        return
    with open(path, "a") as f:
        f.write(json.dumps(dict(case=case, output=what, max_abs=max_abs, rel_l2=rel, elements=n)) + "\n")


def assert_parity(gpu, ref, dtype, what="", case=None):
    max_abs, rel = errors(gpu, ref)
    if case:
        record(case, what, max_abs, rel, int(ref.numel()))
    tol_abs, tol_rel = TOL[dtype]
    assert max_abs <= tol_abs and rel <= tol_rel, (
        f"{what}: max-abs {max_abs:.3e} (<= {tol_abs}) rel-L2 {rel:.3e} (<= {tol_rel})")
    return max_abs, rel


def to_cpu(x):
    return {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in x.items()}


def to_dev(x, device="cuda"):
    return {k: (v.to(device) if torch.is_tensor(v) and k != "needle_pos" else v) for k, v in x.items()}


def oracle_prefill(xc, window, swa=True, cap=None, softmax_scale=None):
    """The oracle on CPU copies of the inputs; caches start as sentinels."""
    B, T = xc["q"].shape[:2]
    Hkv, d = xc["k"].shape[2], xc["k"].shape[3]
    cap = cap or T
    kc = inputs.empty_cache(B, Hkv, cap, d, xc["q"].dtype)
    vc = inputs.empty_cache(B, Hkv, cap, d, xc["q"].dtype)
    return oracle.prefill(xc["q"], xc["q_out"], xc["out_pos"], xc["k"], xc["v"], xc["alpha"], xc["beta"],
                          xc["alpha_out"], xc["beta_out"], window, softmax_scale=softmax_scale,
                          k_cache=kc, v_cache=vc, swa=swa)


def bits(t):
    """Raw bit view for byte-exact comparisons."""
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def SENTINEL_CHECK(t):
    """True when every element of a bf16 tensor still holds the sentinel bit pattern."""
    return bool((bits(t.cpu()) == inputs.SENTINEL_BF16_BITS).all()) if t.numel() else True
