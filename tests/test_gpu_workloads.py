"""Parity at the full workload sizes, in the launch configuration the
benchmark times (MI355X only).  Where the oracle cannot redo a whole
workload in seconds it checks sampled outputs one by one; cache bytes,
sentinels and lengths are checked in full."""
import pytest
import torch

import oracle
from gpu_util import assert_parity, bits, say, to_cpu
from phase_aware_swa_amd import inputs
from phase_aware_swa_amd.runner import Decode, Prefill

pytestmark = pytest.mark.gpu


def sample_rows(B, T, Hq, n_random, edge, seed):
    g = torch.Generator().manual_seed(seed)
    rows = []
    for b in range(B):
        ts = torch.cat([torch.arange(min(edge, T)), torch.randint(0, T, (n_random,), generator=g),
                        torch.arange(max(0, T - edge), T)]).unique()
        for t in ts.tolist():
            for h in range(Hq):
                rows.append((b, t, h))
    return torch.tensor(rows, dtype=torch.int64)


def test_gqa_8b_prefill_128k_workload():
    """B2, 32/8 heads, d128, T131072, w128, bf16, one needle per (b, KV head)."""
    cfg = dict(inputs.WORKLOADS["gqa_8b_prefill_128k"])
    T = cfg["T"]
    say("workload gqa_8b_prefill_128k: generate")
    x = inputs.prefill_inputs(seed=2, device="cuda", **cfg)
    run = Prefill(cfg, x, cap=T + 64)
    say("workload gqa_8b_prefill_128k: prefill")
    run.run()
    torch.cuda.synchronize()
    # cache: every slot bit-exact, the spare slots untouched
    assert torch.equal(bits(run.k_cache[:, :, :T]), bits(x["k"].transpose(1, 2)))
    assert torch.equal(bits(run.v_cache[:, :, :T]), bits(x["v"].transpose(1, 2)))
    assert bool((bits(run.k_cache[:, :, T:]) == inputs.SENTINEL_BF16_BITS).all())
    say("workload gqa_8b_prefill_128k: oracle (global in full, sampled SWA rows)")
    xc = to_cpu(x)
    ref = oracle.prefill(xc["q"], xc["q_out"], xc["out_pos"], xc["k"], xc["v"], xc["alpha"], xc["beta"],
                         xc["alpha_out"], xc["beta_out"], cfg["window"], swa=False)
    assert_parity(run.o_out, ref["o_out"], torch.bfloat16, "o_out")
    G = cfg["n_q_heads"] // cfg["n_kv_heads"]
    for b in range(cfg["batch"]):
        for g in range(cfg["n_kv_heads"]):
            p = int(xc["needle_pos"][b, g])
            assert (run.o_out[b, g * G].cpu().double() - xc["v"][b, p, g].double()).abs().max() < 0.05
    rows = sample_rows(cfg["batch"], T, cfg["n_q_heads"], 2048, 128, seed=2)
    ref_rows = oracle.swa_rows(xc["q"], xc["k"], xc["v"], xc["alpha"], xc["beta"], cfg["window"], rows)
    o_cpu = run.o.cpu()
    got = o_cpu[rows[:, 0], rows[:, 1], rows[:, 2]]
    assert_parity(got, ref_rows, torch.bfloat16, "o (sampled rows)")


def test_gqa_8b_decode_b16_workload():
    """B16, 32/8 heads, d128, w128, bf16, lengths U[8192, 131072], 1024 steps:
    sampled steps against the oracle, final caches and lengths in full."""
    cfg = dict(inputs.WORKLOADS["gqa_8b_decode_b16"])
    steps = cfg["steps"]
    say("workload gqa_8b_decode_b16: generate")
    x = inputs.decode_inputs(seed=4, device="cuda", **cfg)
    xc = to_cpu(x)
    max_hint = int(xc["cache_len"].max()) + steps - 1
    dec = Decode(cfg, x["k_cache"], x["v_cache"], x["cache_len"], max_hint, x["alpha"], x["beta"],
                 x["alpha_out"], x["beta_out"])
    check = {0, 517, steps - 1}
    got = {}
    say("workload gqa_8b_decode_b16: 1024 steps")
    for s in range(steps):
        dec.step(x["q"][s], x["q_out"][s], x["k_new"][s], x["v_new"][s])
        if s in check:
            got[s] = (dec.o.cpu(), dec.o_out.cpu())
    torch.cuda.synchronize()
    say("workload gqa_8b_decode_b16: oracle")
    kc, vc, lc = xc["k_cache"], xc["v_cache"], xc["cache_len"].clone()
    for s in range(steps):
        o, o_out = oracle.decode_step(xc["q"][s], xc["q_out"][s], xc["k_new"][s], xc["v_new"][s], xc["alpha"],
                                      xc["beta"], xc["alpha_out"], xc["beta_out"], cfg["window"], kc, vc, lc,
                                      compute=s in check)
        if s in check:
            assert_parity(got[s][0], o, torch.bfloat16, f"o step {s}")
            assert_parity(got[s][1], o_out, torch.bfloat16, f"o_out step {s}")
    assert torch.equal(dec.cache_len.cpu(), lc)
    assert torch.equal(bits(dec.k_cache.cpu()), bits(kc))
    assert torch.equal(bits(dec.v_cache.cpu()), bits(vc))
