"""GPU parity of orthros_prefill / orthros_swa_prefill / orthros_global_xattn
against the fp64 oracle, through the C ABI (MI355X only)."""
import pytest
import torch

from gpu_util import TOL, assert_parity, bits, oracle_prefill, say, to_cpu, to_dev
from phase_aware_swa_amd import binding, inputs
from phase_aware_swa_amd.runner import Prefill

pytestmark = pytest.mark.gpu


def make_cfg(B, Hq, Hkv, d, w, dtype):
    return dict(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=w, dtype=dtype)


def run_case(cfg, T, seed, out_pos=None, cap_extra=0, check_cache=True, case=None):
    cfg = {k: v for k, v in cfg.items() if k not in ("T", "kind")}
    say(f"prefill case {cfg} T={T} seed={seed} out_pos={out_pos} cap_extra={cap_extra}")
    xc = inputs.prefill_inputs(T=T, seed=seed, **cfg)
    if out_pos is not None:
        xc["out_pos"] = out_pos
    x = to_dev(xc)
    run = Prefill(cfg, x, cap=T + cap_extra)
    run.run()
    torch.cuda.synchronize()
    ref = oracle_prefill(xc, cfg["window"], cap=T + cap_extra)
    assert_parity(run.o, ref["o"], cfg["dtype"], "o", case=case)
    assert_parity(run.o_out, ref["o_out"], cfg["dtype"], "o_out", case=case)
    if check_cache:
        assert torch.equal(bits(run.k_cache.cpu()), bits(ref["k_cache"]))
        assert torch.equal(bits(run.v_cache.cpu()), bits(ref["v_cache"]))
    return run, ref, xc


# Shapes spanning several tiles, ragged tails, window edges, GQA groups and both head dims.
CASES = [
    # B, Hq, Hkv, d, w, T
    (1, 4, 4, 64, 128, 2048),
    (1, 4, 1, 128, 128, 1000),
    (2, 8, 2, 128, 128, 777),
    (1, 2, 2, 128, 128, 1),
    (1, 2, 2, 128, 128, 2),
    (1, 4, 4, 128, 128, 31),
    (1, 4, 4, 128, 128, 33),
    (3, 6, 2, 64, 17, 300),
    (1, 3, 1, 128, 1, 130),
    (1, 8, 1, 128, 129, 515),
    (1, 16, 2, 64, 300, 700),
    (1, 2, 1, 128, 2000, 1500),
    (2, 4, 2, 128, 5, 96),
    # GQA groups of 4 / 8 with w <= 129 (the streaming kernel), incl. segment edges
    (1, 4, 1, 64, 128, 300),
    (2, 8, 2, 128, 1, 100),
    (1, 4, 1, 128, 128, 1),
    (1, 4, 1, 128, 128, 33),
    (1, 4, 1, 128, 64, 4100),
    (1, 8, 1, 128, 100, 2000),
    (1, 4, 1, 128, 128, 40000),
    # other groups with w <= 129 (the streaming kernel: blocks of 2 or 1 heads)
    (2, 8, 8, 128, 128, 3000),
    (1, 4, 2, 64, 128, 1000),
    (1, 12, 2, 128, 128, 700),
    (2, 3, 3, 64, 129, 333),
    (1, 4, 4, 128, 128, 40000),
    (1, 8, 4, 64, 100, 20000),
    # groups of 1 and 3 past w = 129 (the generic kernel)
    (1, 4, 4, 128, 200, 700),
    (2, 6, 2, 128, 130, 500),
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("B,Hq,Hkv,d,w,T", CASES)
def test_prefill_parity(B, Hq, Hkv, d, w, T, dtype):
    cfg = make_cfg(B, Hq, Hkv, d, w, dtype)
    run_case(cfg, T, seed=1000 + T + w, cap_extra=37)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_copy_masked_by_original_position(dtype):
    """out_pos < T-1: the copy reads [0, out_pos], not the whole prompt."""
    cfg = make_cfg(3, 8, 2, 128, 128, dtype)
    run_case(cfg, 1500, seed=7, out_pos=[0, 700, 1499])


def test_tiny_fp32_workload():
    """Full parity at the tiny fp32 workload (B1, 4/4 heads, d64, T2048, w128)."""
    cfg = dict(inputs.WORKLOADS["tiny_fp32_prefill"])
    run_case(cfg, cfg["T"], seed=0, cap_extra=64, case="tiny_fp32_prefill")


def test_mha_1p3b_8k_workload():
    """Full parity at the 1.3B-class MHA workload (B1, 16/16, d128, T8192, w128, bf16)."""
    cfg = dict(inputs.WORKLOADS["mha_1p3b_prefill_8k"])
    run_case(cfg, cfg["T"], seed=1, cap_extra=64, case="mha_1p3b_prefill_8k")


def test_run_to_run_identical():
    cfg = make_cfg(2, 8, 2, 128, 128, torch.bfloat16)
    say("determinism case")
    x = to_dev(inputs.prefill_inputs(T=3000, seed=11, **cfg))
    run = Prefill(cfg, x)
    run.run()
    o1, oo1 = run.o.clone(), run.o_out.clone()
    run.run()
    torch.cuda.synchronize()
    assert torch.equal(bits(run.o), bits(o1)) and torch.equal(bits(run.o_out), bits(oo1))


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_window_one_and_first_row_exact(dtype):
    """w = 1: o = v exactly.  Row 0 and a copy at position 0 see only key 0."""
    cfg = make_cfg(2, 4, 2, 128, 1, dtype)
    say("w=1 exactness", dtype)
    xc = inputs.prefill_inputs(T=200, seed=12, **cfg)
    xc["out_pos"] = [0, 0]
    x = to_dev(xc)
    run = Prefill(cfg, x)
    run.run()
    torch.cuda.synchronize()
    v = xc["v"].repeat_interleave(2, dim=2)
    assert torch.equal(bits(run.o.cpu()), bits(v))
    assert torch.equal(bits(run.o_out.cpu()), bits(xc["v"][:, 0].repeat_interleave(2, dim=1).contiguous()))
    cfg["window"] = 128
    run2 = Prefill(cfg, x)
    run2.run()
    torch.cuda.synchronize()
    assert torch.equal(bits(run2.o[:, 0].cpu()), bits(xc["v"][:, 0].repeat_interleave(2, dim=1).contiguous()))


def test_mask_probe_bit_exact():
    """alpha = beta = 0 gives uniform weights.  V[j] = one-hot (j mod 127):
    a full 128-key window holds residue t mod 127 twice, so each row is
    exactly 2/128 there and 1/128 at the other 126 residues; the copy at P
    with P+1 = 1024 and V = one-hot (j mod 128) is exactly 1/128 everywhere.
    A shifted or resized window, or a copy masked by slot, breaks it."""
    T, d = 1500, 128
    cfg = make_cfg(1, 4, 2, d, 128, torch.bfloat16)
    say("mask probe")
    xc = inputs.prefill_inputs(T=T, seed=13, **cfg)
    for key in ("alpha", "beta", "alpha_out", "beta_out"):
        xc[key].zero_()
    j = torch.arange(T)
    xc["v"].zero_()
    xc["v"][0, j, :, j % 127] = 1.0
    xc["out_pos"] = [1023]
    x = to_dev(xc)
    run = Prefill(cfg, x)
    run.run()
    torch.cuda.synchronize()
    o = run.o.cpu().float()
    for t in range(127, T):
        exp = torch.full((d,), 1 / 128)
        exp[127] = 0.0
        exp[t % 127] = 2 / 128
        assert torch.equal(o[0, t, 0], exp) and torch.equal(o[0, t, 3], exp), f"row {t}"
    # global probe: V = one-hot (j mod 128) on the first 1024 keys
    xc["v"].zero_()
    xc["v"][0, j, :, j % 128] = 1.0
    run.x = to_dev(xc)
    run.run()
    torch.cuda.synchronize()
    assert torch.equal(run.o_out.cpu().float(), torch.full((1, 4, d), 1 / 128))


@pytest.mark.parametrize("Hq,Hkv,w", [(4, 4, 1), (4, 4, 3), (4, 2, 16), (4, 4, 128), (2, 1, 129), (4, 2, 300)],
                         ids=["G1-w1", "G1-w3", "G2-w16", "G1-w128", "G2-w129", "G2-w300"])
def test_fp32_moment_probe(Hq, Hkv, w):
    """The fp32 path's mask placement.  alpha = beta = 0 gives every admissible
    key the same weight; V rows [1, j, j^2, 0, ...] (j <= 299, so every sum
    of the row's weighted values is an integer below 2^24, exact in fp32)
    make each output the mean of 1, j and j^2 over the row's key set.  The
    count n and the first index lo of that set then follow exactly after
    rounding: n^2 = 12 (mean j^2 - mean j^2) + 1, lo = mean j - (n - 1) / 2.
    Every base row's set must be [max(0, t - w + 1), t]; the copy at 157
    must see [0, 157]."""
    T, d = 300, 64
    cfg = make_cfg(1, Hq, Hkv, d, w, torch.float32)
    say("fp32 moment probe", cfg)
    xc = inputs.prefill_inputs(T=T, seed=21, **cfg)
    for key in ("alpha", "beta", "alpha_out", "beta_out"):
        xc[key].zero_()
    j = torch.arange(T, dtype=torch.float32)
    xc["v"].zero_()
    xc["v"][0, :, :, 0] = 1.0
    xc["v"][0, :, :, 1] = j[:, None]
    xc["v"][0, :, :, 2] = (j * j)[:, None]
    xc["out_pos"] = [157]
    run = Prefill(cfg, to_dev(xc))
    run.run()
    torch.cuda.synchronize()

    def key_set(m):
        m = m.double()
        n = torch.round(torch.sqrt(12 * (m[..., 2] - m[..., 1] ** 2) + 1))
        lo = torch.round(m[..., 1] - (n - 1) / 2)
        return n, lo

    o = run.o.cpu()[0]                                   # [T, Hq, d]
    assert torch.allclose(o[..., 0], torch.ones_like(o[..., 0]), rtol=0, atol=1e-6)
    n, lo = key_set(o)
    t = torch.arange(T, dtype=torch.float64)[:, None].expand(T, Hq)
    lo_exp = torch.clamp(t - w + 1, min=0)
    assert torch.equal(lo, lo_exp), "first keys of the windows"
    assert torch.equal(n, t - lo_exp + 1), "window sizes"
    n_c, lo_c = key_set(run.o_out.cpu()[0])
    assert torch.equal(n_c, torch.full((Hq,), 158.0, dtype=torch.float64)) and torch.equal(lo_c, torch.zeros(Hq, dtype=torch.float64))


def test_base_stream_isolated_from_output_stream():
    """Perturbing q_out, alpha', beta' leaves the cache and o bit-identical."""
    cfg = make_cfg(2, 8, 2, 128, 128, torch.bfloat16)
    say("isolation case")
    xc = inputs.prefill_inputs(T=900, seed=14, **cfg)
    x = to_dev(xc)
    run = Prefill(cfg, x)
    run.run()
    torch.cuda.synchronize()
    o, kc, vc, oo = run.o.clone(), run.k_cache.clone(), run.v_cache.clone(), run.o_out.clone()
    x2 = dict(x)
    x2["q_out"] = (x["q_out"] * 3 + 1).contiguous()
    x2["alpha_out"] = (-x["alpha_out"]).contiguous()
    x2["beta_out"] = (x["beta_out"] + 5).contiguous()
    run.x = x2
    run.run()
    torch.cuda.synchronize()
    assert torch.equal(bits(run.o), bits(o))
    assert torch.equal(bits(run.k_cache), bits(kc)) and torch.equal(bits(run.v_cache), bits(vc))
    assert not torch.equal(bits(run.o_out), bits(oo))


@pytest.mark.parametrize("G,w", [(4, 128), (2, 128), (1, 128), (2, 200)],
                         ids=["fused-G4", "fused-G2", "fused-G1", "separate-G2-w200"])
def test_stages_match_one_call(G, w):
    """orthros_swa_prefill then orthros_global_xattn against orthros_prefill.
    o and the caches are bit-identical.  With w <= 129 the one call takes the
    fused path (the copy's query rides on the streaming SWA kernel, other
    key splits), so o_out of both is checked against the oracle; with
    w = 200 the one call runs the same two kernels and o_out is
    bit-identical."""
    cfg = make_cfg(2, 2 * G, 2, 128, w, torch.bfloat16)
    say("stages vs one call, G =", G, "w =", w)
    xc = inputs.prefill_inputs(T=1234, seed=15, **cfg)
    xc["out_pos"] = [1233, 600]
    x = to_dev(xc)
    a = Prefill(cfg, x)
    a.run()
    b = Prefill(cfg, x)
    b.run_swa()
    b.run_xattn()
    torch.cuda.synchronize()
    assert torch.equal(bits(a.o), bits(b.o))
    assert torch.equal(bits(a.k_cache), bits(b.k_cache)) and torch.equal(bits(a.v_cache), bits(b.v_cache))
    if w > 129:
        assert torch.equal(bits(a.o_out), bits(b.o_out))
    else:
        ref = oracle_prefill(xc, w)
        assert_parity(a.o_out, ref["o_out"], torch.bfloat16, "o_out (one call)")
        assert_parity(b.o_out, ref["o_out"], torch.bfloat16, "o_out (stages)")


def test_fused_copy_positions_at_segment_edges():
    """Fused path, 8 sequences whose copies sit at 0, inside the first pair,
    on both sides of pair and segment boundaries, mid-prompt and at T-1.
    (B8 x 2 KV heads x one 4-head block = 16 streams -> 32 segments of
    5 tiles = 160 keys at T = 5000.)"""
    cfg = make_cfg(8, 8, 2, 128, 128, torch.bfloat16)
    run_case(cfg, 5000, seed=18, out_pos=[0, 31, 32, 159, 160, 161, 2501, 4999])


@pytest.mark.parametrize("Hq,Hkv", [(4, 1), (2, 1), (2, 2)], ids=["G4", "G2", "G1"])
def test_fused_more_sequences_than_one_launch(Hq, Hkv):
    """67 sequences: the fused kernel takes copy positions 64 per launch
    (blocks of 4, 2 and 1 heads)."""
    cfg = make_cfg(67, Hq, Hkv, 64, 16, torch.bfloat16)
    g = torch.Generator().manual_seed(19)
    run_case(cfg, 70, seed=19 + Hq + Hkv, out_pos=torch.randint(0, 70, (67,), generator=g).tolist())


def test_explicit_softmax_scale():
    cfg = make_cfg(1, 4, 2, 64, 64, torch.float32)
    say("explicit scale")
    xc = inputs.prefill_inputs(T=500, seed=16, **cfg)
    x = to_dev(xc)
    run = Prefill(cfg, x, softmax_scale=0.05)
    run.run()
    torch.cuda.synchronize()
    ref = oracle_prefill(xc, 64, softmax_scale=0.05)
    assert_parity(run.o, ref["o"], torch.float32, "o")
    assert_parity(run.o_out, ref["o_out"], torch.float32, "o_out")


def test_status_errors_launch_nothing():
    """Bad arguments return a negative status and leave every buffer alone."""
    cfg = make_cfg(1, 4, 2, 128, 128, torch.bfloat16)
    x = to_dev(inputs.prefill_inputs(T=100, seed=17, **cfg))
    run = Prefill(cfg, x)
    run.o.zero_()
    x["out_pos"] = [100]
    with pytest.raises(binding.OrthrosError) as e:
        run.run()
    assert e.value.status == -4
    small = torch.empty(8, dtype=torch.uint8, device="cuda")
    run.x["out_pos"] = [99]
    run.workspace = small
    with pytest.raises(binding.OrthrosError) as e:
        run.run()
    assert e.value.status == -6
    torch.cuda.synchronize()
    assert int(run.o.abs().sum().item()) == 0
    assert bool((bits(run.k_cache) == inputs.SENTINEL_BF16_BITS).all())
