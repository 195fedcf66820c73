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


def test_gqa_8b_prefill_128k_workload():
    """B2, 32/8 heads, d128, T131072, w128, bf16, one needle per (b, KV head).
    Every output against the oracle: Eq. (4) for all 2 x 131072 x 32 rows
    and the copy's global query; the cache byte for byte."""
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
    say("workload gqa_8b_prefill_128k: oracle (every row)")
    xc = to_cpu(x)
    ref = oracle.prefill(xc["q"], xc["q_out"], xc["out_pos"], xc["k"], xc["v"], xc["alpha"], xc["beta"],
                         xc["alpha_out"], xc["beta_out"], cfg["window"])
    case = "gqa_8b_prefill_128k"
    assert_parity(run.o_out, ref["o_out"], torch.bfloat16, "o_out", case=case)
    G = cfg["n_q_heads"] // cfg["n_kv_heads"]
    for b in range(cfg["batch"]):
        for g in range(cfg["n_kv_heads"]):
            p = int(xc["needle_pos"][b, g])
            assert (run.o_out[b, g * G].cpu().double() - xc["v"][b, p, g].double()).abs().max() < 0.05
    assert_parity(run.o, ref["o"], torch.bfloat16, "o", case=case)


def test_gqa_8b_decode_b16_workload():
    """B16, 32/8 heads, d128, w128, bf16, lengths U[8192, 131072], 1024 steps:
    every step of the first 64 and every 16th step after them (and the last)
    against the oracle, which appends every step; final caches and lengths
    in full."""
    cfg = dict(inputs.WORKLOADS["gqa_8b_decode_b16"])
    steps = cfg["steps"]
    say("workload gqa_8b_decode_b16: generate")
    x = inputs.decode_inputs(seed=4, device="cuda", **cfg)
    xc = to_cpu(x)
    max_hint = int(xc["cache_len"].max()) + steps - 1
    dec = Decode(cfg, x["k_cache"], x["v_cache"], x["cache_len"], max_hint, x["alpha"], x["beta"],
                 x["alpha_out"], x["beta_out"])
    check = set(range(64)) | set(range(64, steps, 16)) | {steps - 1}
    got = {}
    say(f"workload gqa_8b_decode_b16: {steps} steps")
    for s in range(steps):
        dec.step(x["q"][s], x["q_out"][s], x["k_new"][s], x["v_new"][s])
        if s in check:
            got[s] = (dec.o.cpu(), dec.o_out.cpu())
    torch.cuda.synchronize()
    say(f"workload gqa_8b_decode_b16: oracle on {len(check)} steps")
    kc, vc, lc = xc["k_cache"], xc["v_cache"], xc["cache_len"].clone()
    all_g, all_r = [], []
    for s in range(steps):
        o, o_out = oracle.decode_step(xc["q"][s], xc["q_out"][s], xc["k_new"][s], xc["v_new"][s], xc["alpha"],
                                      xc["beta"], xc["alpha_out"], xc["beta_out"], cfg["window"], kc, vc, lc,
                                      compute=s in check)
        if s in check:
            assert_parity(got[s][0], o, torch.bfloat16, f"o step {s}")
            assert_parity(got[s][1], o_out, torch.bfloat16, f"o_out step {s}")
            all_g.append(torch.stack(got[s]))
            all_r.append(torch.stack([o, o_out]))
    g_, r_ = torch.stack(all_g), torch.stack(all_r)
    case = f"gqa_8b_decode_b16 ({len(check)} of {steps} steps)"
    assert_parity(g_[:, 0], r_[:, 0], torch.bfloat16, "o", case=case)
    assert_parity(g_[:, 1], r_[:, 1], torch.bfloat16, "o_out", case=case)
    assert torch.equal(dec.cache_len.cpu(), lc)
    assert torch.equal(bits(dec.k_cache.cpu()), bits(kc))
    assert torch.equal(bits(dec.v_cache.cpu()), bits(vc))


@pytest.mark.timeout(900)
def test_gqa_8b_prefill_1m_36_layers_resident():
    """B1, 32/8 heads, d128, T = 2^20, w128, 36 layers whose caches (144 GiB)
    all stay resident.  Every layer: cache bytes against its own K/V; the
    copy's global query over all 2^20 keys against the oracle in full; Eq.
    (4) against the oracle on a stratified row sample (rows 0-255, 4096
    random rows, the last 256 rows, every head); and a checksum re-read of
    every cache after the last layer (no layer overwrites another)."""
    cfg = dict(inputs.WORKLOADS["gqa_8b_prefill_1m"])
    T, L, B, Hq, Hkv, d = (cfg[k] for k in ("T", "layers", "batch", "n_q_heads", "n_kv_heads", "head_dim"))
    w = cfg["window"]
    say("workload gqa_8b_prefill_1m: allocate 36 resident caches")
    kc_all = torch.empty(L, B, Hkv, T, d, dtype=torch.bfloat16, device="cuda")
    vc_all = torch.empty_like(kc_all)
    # host buffers reused by every layer: K/V as drawn (pinned) and the oracle's caches
    kh = torch.empty(B, T, Hkv, d, dtype=torch.bfloat16, pin_memory=True)
    vh = torch.empty_like(kh, pin_memory=True)
    kc_h = torch.empty(B, Hkv, T, d, dtype=torch.bfloat16)
    vc_h = torch.empty_like(kc_h)
    sums = []
    g = torch.Generator().manual_seed(36)
    case = "gqa_8b_prefill_1m (36 layers)"
    acc = {"o_out": ([], []), "o": ([], [])}
    for layer in range(L):
        say(f"workload gqa_8b_prefill_1m: layer {layer}")
        x = inputs.prefill_inputs(seed=1000 + layer, device="cuda", **cfg)
        run = Prefill(cfg, x, k_cache=kc_all[layer], v_cache=vc_all[layer])
        run.run()
        torch.cuda.synchronize()
        assert torch.equal(bits(kc_all[layer]), bits(x["k"].transpose(1, 2)))
        assert torch.equal(bits(vc_all[layer]), bits(x["v"].transpose(1, 2)))
        sums.append((bits(kc_all[layer]).sum().item(), bits(vc_all[layer]).sum().item()))
        kh.copy_(x["k"])
        vh.copy_(x["v"])
        ab = [x[n].cpu() for n in ("alpha", "beta", "alpha_out", "beta_out")]
        ref = oracle.prefill(None, x["q_out"].cpu(), x["out_pos"], kh, vh, *ab, w, swa=False, k_cache=kc_h,
                             v_cache=vc_h)
        assert_parity(run.o_out, ref["o_out"], torch.bfloat16, f"layer {layer} o_out")
        acc["o_out"][0].append(run.o_out.cpu())
        acc["o_out"][1].append(ref["o_out"])
        ts = torch.cat([torch.arange(256), torch.randint(0, T, (4096,), generator=g),
                        torch.arange(T - 256, T)]).unique()
        tsd = ts.cuda()
        qrows = x["q"][0, tsd].reshape(-1, d).cpu()
        rows = torch.stack([torch.zeros_like(ts).repeat_interleave(Hq), ts.repeat_interleave(Hq),
                            torch.arange(Hq).repeat(ts.numel())], dim=1)
        ref_rows = oracle.swa_rows_given_q(qrows, kh, vh, ab[0], ab[1], w, rows, n_q_heads=Hq)
        got = run.o[0, tsd].reshape(-1, d).cpu()
        assert_parity(got, ref_rows, torch.bfloat16, f"layer {layer} o ({ts.numel()} rows x {Hq} heads)")
        acc["o"][0].append(got)
        acc["o"][1].append(ref_rows)
        del run, x
        torch.cuda.empty_cache()
    for what, (gs, rs) in acc.items():
        assert_parity(torch.cat(gs), torch.cat(rs), torch.bfloat16,
                      what + (" (stratified rows)" if what == "o" else ""), case=case)
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
