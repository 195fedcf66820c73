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


def test_gqa_8b_prefill_1m_36_layers_resident():
    """B1, 32/8 heads, d128, T = 2^20, w128, 36 layers whose caches (144 GiB)
    all stay resident.  Every layer: cache bytes against its own K/V, and a
    checksum re-read after all 36 layers (no layer overwrites another).
    Layers 0, 17, 35: the copy's global query against the oracle in full and
    Eq. (4) rows of three 512-row segments (start, middle, end)."""
    cfg = dict(inputs.WORKLOADS["gqa_8b_prefill_1m"])
    T, L, B, Hkv, d = cfg["T"], cfg["layers"], cfg["batch"], cfg["n_kv_heads"], cfg["head_dim"]
    w = cfg["window"]
    say("workload gqa_8b_prefill_1m: allocate 36 resident caches")
    kc_all = torch.empty(L, B, Hkv, T, d, dtype=torch.bfloat16, device="cuda")
    vc_all = torch.empty_like(kc_all)
    sums = []
    checked = {0, 17, 35}
    for layer in range(L):
        say(f"workload gqa_8b_prefill_1m: layer {layer}")
        x = inputs.prefill_inputs(seed=1000 + layer, device="cuda", **cfg)
        run = Prefill(cfg, x, k_cache=kc_all[layer], v_cache=vc_all[layer])
        run.run()
        torch.cuda.synchronize()
        assert torch.equal(bits(kc_all[layer]), bits(x["k"].transpose(1, 2)))
        assert torch.equal(bits(vc_all[layer]), bits(x["v"].transpose(1, 2)))
        sums.append((bits(kc_all[layer]).sum().item(), bits(vc_all[layer]).sum().item()))
        if layer in checked:
            k_h, v_h = x["k"].cpu(), x["v"].cpu()
            q_out = x["q_out"].cpu()
            ab = [x[n].cpu() for n in ("alpha", "beta", "alpha_out", "beta_out")]
            ref = oracle.prefill(None, q_out, x["out_pos"], k_h, v_h, *ab, w, swa=False)
            assert_parity(run.o_out, ref["o_out"], torch.bfloat16, f"layer {layer} o_out")
            for s in (0, T // 2, T - 512):
                lo = max(0, s - w + 1)
                qs = x["q"][:, lo:s + 512].cpu().contiguous()
                rows = torch.tensor([(0, t - lo, h) for t in range(s, s + 512) for h in range(cfg["n_q_heads"])])
                ref_rows = oracle.swa_rows(qs, k_h[:, lo:s + 512].contiguous(), v_h[:, lo:s + 512].contiguous(),
                                           ab[0], ab[1], w, rows)
                got = run.o[0, s:s + 512].cpu().reshape(-1, d)
                assert_parity(got, ref_rows, torch.bfloat16, f"layer {layer} o rows {s}..{s + 511}")
        del run, x
        torch.cuda.empty_cache()
    say("workload gqa_8b_prefill_1m: re-read all caches")
    for layer in range(L):
        assert sums[layer] == (bits(kc_all[layer]).sum().item(), bits(vc_all[layer]).sum().item())


@pytest.mark.parametrize("name", ["gqa_8b_sft_32k", "gqa_8b_pt_16k"])
def test_copies_workload(name):
    """The many-copy workloads in the launch configuration the benchmark
    times: the library's SWA pass fills the cache, orthros_copies runs over
    all T_out copies, and 96 sampled copies (the first, the last, and random
    ones) are checked against the oracle for every head."""
    from phase_aware_swa_amd.runner import Copies
    cfg = dict(inputs.WORKLOADS[name])
    B, T, T_out, Hq, d = cfg["batch"], cfg["T"], cfg["T_out"], cfg["n_q_heads"], cfg["head_dim"]
    say(f"workload {name}: generate")
    x = inputs.prefill_inputs(seed=7, device="cuda", **cfg)
    pre = Prefill(cfg, x)
    pre.run_swa()
    q_out, pos = inputs.copies_inputs(B, Hq, d, T, T_out, torch.bfloat16, seed=8, device="cuda")
    cp = Copies(cfg, T, q_out, pos, x["alpha_out"], x["beta_out"], pre.k_cache, pre.v_cache)
    say(f"workload {name}: copies")
    cp.run()
    torch.cuda.synchronize()
    g = torch.Generator().manual_seed(9)
    pick = torch.cat([torch.tensor([0, T_out - 1]), torch.randint(0, T_out, (94,), generator=g)]).unique()
    say(f"workload {name}: oracle on {pick.numel()} copies x {B} sequences")
    kc, vc = pre.k_cache.cpu(), pre.v_cache.cpu()
    ref = oracle.copies(q_out[:, pick].cpu().contiguous(), pos[:, pick].cpu(), x["alpha_out"].cpu(),
                        x["beta_out"].cpu(), kc, vc, T)
    assert_parity(cp.o_out[:, pick], ref, torch.bfloat16, f"{name} o_out (sampled copies)")
