"""GPU parity of orthros_project -- the projections either side of the
attention step ("Orthros:阶段感知异构注意力精读笔记" §2.1-§2.2: K/V from the
base input for every position, written into the cache; both streams'
queries from the one shared W_Q with per-stream scale-offset) -- against the
fp64 oracle, through the C ABI (MI355X only)."""
import pytest
import torch

from gpu_util import SENTINEL_CHECK, assert_parity, bits, say
from oracle.project import cache_rows, project
from phase_aware_swa_amd import binding, inputs
from phase_aware_swa_amd.runner import Project, desc_for

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def make_cfg(B, Hq, Hkv, d, T, T_out, dm):
    return dict(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, T=T, T_out=T_out, d_model=dm, window=128,
                dtype=BF16)


def oracle_of(cfg, xc, scale_offset=True):
    so = {k: xc[k] for k in ("alpha", "beta", "alpha_out", "beta_out")}
    if not scale_offset:
        so = {"alpha": torch.ones_like(xc["alpha"]), "beta": torch.zeros_like(xc["beta"]),
              "alpha_out": torch.ones_like(xc["alpha"]), "beta_out": torch.zeros_like(xc["beta"])}
    return project(xc["x"], xc["x_out"], xc["w_q"], xc["w_k"], xc["w_v"], n_q_heads=cfg["n_q_heads"],
                   n_kv_heads=cfg["n_kv_heads"], head_dim=cfg["head_dim"], **so)


def run_case(cfg, seed, cap_extra=5, scale_offset=True):
    say(f"project case {cfg} seed={seed} cap_extra={cap_extra} scale_offset={scale_offset}")
    xc = inputs.project_inputs(seed=seed, **cfg)
    x = {k: v.cuda() for k, v in xc.items()}
    T = cfg["T"]
    run = Project(cfg, x, cap=T + cap_extra, scale_offset=scale_offset)
    run.run()
    torch.cuda.synchronize()
    ref = oracle_of(cfg, xc, scale_offset)
    assert_parity(run.q, ref["q"], BF16, "q")
    if cfg["T_out"]:
        assert_parity(run.q_out, ref["q_out"], BF16, "q_out")
    kc, vc = run.k_cache.cpu(), run.v_cache.cpu()
    assert_parity(kc[:, :, :T], cache_rows(ref["k"]), BF16, "k_cache")
    assert_parity(vc[:, :, :T], cache_rows(ref["v"]), BF16, "v_cache")
    # slots past T are untouched (still the sentinel bit pattern)
    assert SENTINEL_CHECK(kc[:, :, T:]) and SENTINEL_CHECK(vc[:, :, T:]), "a cache slot past T was written"
    return run, ref


@pytest.mark.parametrize("B,Hq,Hkv,d,T,T_out,dm", [
    (2, 8, 2, 128, 300, 3, 256),      # ragged row tile, several column tiles of each kind
    (1, 4, 1, 128, 256, 1, 64),       # exactly one row tile, the prefill copy, shallow K
    (2, 4, 2, 64, 513, 7, 96),        # d = 64 (two heads per column tile), K = 3 stages
    (3, 8, 8, 128, 77, 40, 160),      # MHA, ragged row tiles in both regions
    (1, 16, 4, 128, 1000, 600, 512),  # copy rows spanning three row tiles
])
def test_project_parity(B, Hq, Hkv, d, T, T_out, dm):
    run_case(make_cfg(B, Hq, Hkv, d, T, T_out, dm), seed=100 + T + dm)


def test_project_without_scale_offset():
    """alpha/beta NULL: the raw projections (what orthros_prefill takes)."""
    run_case(make_cfg(2, 8, 2, 128, 300, 3, 256), seed=7, scale_offset=False)


def test_project_no_copies():
    """T_out = 0: no copy rows, x_out and q_out may be NULL."""
    run_case(make_cfg(2, 8, 2, 128, 130, 0, 128), seed=8)


def test_project_one_row():
    run_case(make_cfg(1, 4, 1, 128, 1, 1, 32), seed=9, cap_extra=3)


def test_project_feeds_prefill():
    """orthros_project (no scale-offset) then orthros_prefill on its q and
    cache equals the oracle's projections followed by the oracle's prefill."""
    import oracle
    cfg = make_cfg(1, 8, 2, 128, 400, 1, 256)
    say(f"project -> prefill case {cfg}")
    xc = inputs.project_inputs(seed=11, **cfg)
    x = {k: v.cuda() for k, v in xc.items()}
    run = Project(cfg, x, cap=400, scale_offset=False)
    run.run()
    desc = desc_for(cfg)
    B, T, Hq, d = 1, 400, 8, 128
    o = torch.empty(B, T, Hq, d, dtype=BF16, device="cuda")
    o_out = torch.empty(B, Hq, d, dtype=BF16, device="cuda")
    ws = torch.empty(binding.prefill_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
    # K/V for orthros_prefill come from the cache the projection wrote ([B,T,Hkv,d] views of it)
    k = run.k_cache.transpose(1, 2).contiguous()
    v = run.v_cache.transpose(1, 2).contiguous()
    kc = inputs.empty_cache(B, 2, T, d, BF16, "cuda")
    vc = inputs.empty_cache(B, 2, T, d, BF16, "cuda")
    binding.prefill(desc, T, run.q, run.q_out[:, 0].contiguous(), [T - 1], k, v, x["alpha"], x["beta"],
                    x["alpha_out"], x["beta_out"], kc, vc, o, o_out, ws)
    torch.cuda.synchronize()
    assert torch.equal(bits(kc), bits(run.k_cache)), "prefill's cache copy differs from the projected cache"
    # the oracle chain on the projections the GPU produced (their bf16 values)
    ref = oracle.prefill(run.q.cpu(), run.q_out[:, 0].cpu(), [T - 1], k.cpu(), v.cpu(), xc["alpha"], xc["beta"],
                         xc["alpha_out"], xc["beta_out"], 128, cap=T)
    assert_parity(o, ref["o"], BF16, "o")
    assert_parity(o_out, ref["o_out"], BF16, "o_out")
    # and the projections themselves against the oracle's
    pr = oracle_of(cfg, xc, scale_offset=False)
    assert_parity(run.q, pr["q"], BF16, "q")


def test_project_run_to_run_identical():
    cfg = make_cfg(2, 8, 2, 128, 300, 3, 256)
    say(f"project determinism {cfg}")
    xc = inputs.project_inputs(seed=12, **cfg)
    x = {k: v.cuda() for k, v in xc.items()}
    a = Project(cfg, x, cap=300)
    a.run()
    q1, k1 = a.q.clone(), a.k_cache.clone()
    a.run()
    torch.cuda.synchronize()
    assert torch.equal(bits(a.q), bits(q1)) and torch.equal(bits(a.k_cache), bits(k1))


def test_project_workload_sampled():
    """The 8B-class layer's projections over the 128K prefill (d_model 4096,
    32/8 heads, B2 x T131072, one copy row each), in the launch the benchmark
    times; 64 sampled rows of q and of the cache against the oracle."""
    cfg = dict(inputs.WORKLOADS["gqa_8b_project_128k"])
    say(f"project workload {cfg}")
    x = inputs.project_inputs(seed=21, device="cuda", **cfg)
    run = Project(cfg, x, cap=cfg["T"])
    run.run()
    torch.cuda.synchronize()
    B, T = cfg["batch"], cfg["T"]
    g = torch.Generator().manual_seed(5)
    rows = torch.randint(0, B * T, (64,), generator=g).tolist() + [0, T - 1, T, B * T - 1]
    xs = x["x"].reshape(B * T, -1)[rows].cpu()[None]
    xc = {k: v.cpu() for k, v in x.items() if k != "x"}
    ref = project(xs, xc["x_out"], xc["w_q"], xc["w_k"], xc["w_v"], xc["alpha"], xc["beta"], xc["alpha_out"],
                  xc["beta_out"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"])
    qg = run.q.reshape(B * T, cfg["n_q_heads"], cfg["head_dim"])[rows].cpu()
    assert_parity(qg, ref["q"][0], BF16, "q rows")
    kg = torch.stack([run.k_cache[r // T, :, r % T] for r in rows]).cpu()
    vg = torch.stack([run.v_cache[r // T, :, r % T] for r in rows]).cpu()
    assert_parity(kg, ref["k"][0], BF16, "k rows")
    assert_parity(vg, ref["v"][0], BF16, "v rows")
    assert_parity(run.q_out.cpu(), ref["q_out"], BF16, "q_out")
