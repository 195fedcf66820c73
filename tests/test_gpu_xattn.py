"""GPU parity of orthros_global_xattn on its own -- the output copy's
full-history causal cross-attention over a filled cache
("Orthros:阶段感知异构注意力精读笔记" §2.3 Eq. (5), §2.4: keys [0, P] of the
copy's original position P) -- against the fp64 oracle, through the C ABI
(MI355X only).

The caches are filled by plain copies of K/V ([B][T][Hkv][d] -> [B][Hkv][cap][d]),
so only the cross-attention kernels run.  bf16 with groups of 4 (or any
group, once the copies read at least 2^20 keys over all streams) takes the
LDS-streamed MFMA kernel (streams of 4, 2 or 1 query heads per KV head;
stages of 128 keys at d = 128, 256 at d = 64; each workgroup takes an equal
run of the launch's keys, at least 256, in (sequence, stream, key) order, so
runs cross stream boundaries); the rest takes the lane-parallel chunk
kernel (power-of-two chunks).
Positions sit on both sides of pair (32), stage and chunk edges."""
import pytest
import torch

import oracle
from gpu_util import assert_parity, say, to_cpu
from phase_aware_swa_amd import inputs
from phase_aware_swa_amd.runner import Prefill

pytestmark = pytest.mark.gpu

BF16 = torch.bfloat16


def run_xattn_case(B, Hq, Hkv, d, T, out_pos, dtype=BF16, seed=0, cap_extra=3):
    cfg = dict(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=128, dtype=dtype)
    say(f"xattn case B={B} Hq={Hq} Hkv={Hkv} d={d} T={T} dtype={dtype} pos={out_pos[:8]}")
    x = inputs.prefill_inputs(T=T, seed=seed, device="cuda", **cfg)
    x["out_pos"] = list(out_pos)
    cap = T + cap_extra
    kc = inputs.empty_cache(B, Hkv, cap, d, dtype, "cuda")
    vc = inputs.empty_cache(B, Hkv, cap, d, dtype, "cuda")
    kc[:, :, :T] = x["k"].transpose(1, 2)
    vc[:, :, :T] = x["v"].transpose(1, 2)
    run = Prefill(cfg, x, k_cache=kc, v_cache=vc)
    run.run_xattn()
    torch.cuda.synchronize()
    xc = to_cpu(x)
    ref = oracle.prefill(None, xc["q_out"], xc["out_pos"], xc["k"], xc["v"], xc["alpha"], xc["beta"],
                         xc["alpha_out"], xc["beta_out"], 128, swa=False)
    assert_parity(run.o_out, ref["o_out"], dtype, "o_out")
    return run, xc


@pytest.mark.parametrize("B,Hq,Hkv,d,T,pos", [
    (1, 4, 1, 128, 1, [0]),                      # one key
    (6, 4, 1, 128, 300, [0, 31, 32, 127, 128, 299]),   # pair and stage edges (d = 128: 128 keys)
    (5, 8, 2, 64, 1000, [255, 256, 257, 511, 999]),    # stage edges (d = 64: 256 keys)
    (3, 16, 4, 128, 3000, [2999, 1, 1500]),      # 4 heads per group, several blocks of 4
    (2, 32, 4, 128, 2500, [2047, 2048]),         # 8 heads per group: two 4-head blocks
    (2, 8, 2, 128, 1234, [1233, 600]),
    (2, 4, 2, 128, 700, [699, 100]),             # G = 2, few keys: the lane-parallel kernel
    (3, 3, 3, 64, 900, [899, 0, 450]),           # MHA, d = 64: the lane-parallel kernel
    (1, 8, 8, 128, 140000, [139999]),            # MHA, 1.1M keys: the LDS kernel, 1-head streams
    (2, 4, 2, 64, 300000, [299999, 123456]),     # G = 2, d = 64, 1.2M keys: the LDS kernel, 2-head streams
    (2, 6, 2, 128, 180000, [179999, 90000]),     # G = 3: 1-head streams, three per KV head
])
def test_xattn_parity(B, Hq, Hkv, d, T, pos):
    run_xattn_case(B, Hq, Hkv, d, T, pos, seed=T + B)


def test_xattn_fp32():
    run_xattn_case(2, 8, 2, 128, 900, [899, 333], dtype=torch.float32, seed=3)


def test_xattn_more_sequences_than_one_launch():
    """67 sequences: positions travel 64 per launch; short streams, so each
    workgroup's run of 256 keys spans several of them."""
    g = torch.Generator().manual_seed(4)
    run_xattn_case(67, 4, 1, 128, 200, torch.randint(0, 200, (67,), generator=g).tolist(), seed=4)


@pytest.mark.parametrize("d", [128, 64])
def test_xattn_long_chunks(d):
    """One stream over 300000 keys: runs of 1172 keys per workgroup (a
    ragged last stage in each, at an offset that moves from run to run)."""
    run_xattn_case(1, 4, 1, d, 300000, [299999 - 77 * (d == 64)], seed=5 + d)


def test_xattn_workload_128k():
    """The 8B-class layer's copies over the whole 128K cache (B2, 32/8 heads,
    d128, one needle per (sequence, KV head)), in the launch the benchmark
    times; o_out in full against the oracle, and each needle head's output
    close to the needle's value row."""
    cfg = dict(inputs.WORKLOADS["gqa_8b_prefill_128k"])
    T = cfg["T"]
    say("xattn workload gqa_8b_prefill_128k")
    x = inputs.prefill_inputs(seed=6, device="cuda", **cfg)
    kc = x["k"].transpose(1, 2).contiguous()
    vc = x["v"].transpose(1, 2).contiguous()
    run = Prefill(cfg, x, k_cache=kc, v_cache=vc)
    run.run_xattn()
    torch.cuda.synchronize()
    xc = {k: (v.cpu() if torch.is_tensor(v) else v) for k, v in x.items() if k != "q"}
    ref = oracle.prefill(None, xc["q_out"], xc["out_pos"], xc["k"], xc["v"], xc["alpha"],
                         xc["beta"], xc["alpha_out"], xc["beta_out"], cfg["window"], swa=False)
    assert_parity(run.o_out, ref["o_out"], BF16, "o_out")
    G = cfg["n_q_heads"] // cfg["n_kv_heads"]
    for b in range(cfg["batch"]):
        for g in range(cfg["n_kv_heads"]):
            p = int(xc["needle_pos"][b, g])
            assert (run.o_out[b, g * G].cpu().double() - xc["v"][b, p, g].double()).abs().max() < 0.05
