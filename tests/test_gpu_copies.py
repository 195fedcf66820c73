"""GPU parity of orthros_copies -- output copies at many positions per
sequence, the PT and SFT modes of "Orthros:阶段感知异构注意力精读笔记" §2.5 --
against the fp64 oracle, through the C ABI (MI355X only).  The cache is the
one the library's own SWA pass wrote, in stream order before the copies."""
import pytest
import torch

import oracle
from gpu_util import assert_parity, bits, say
from phase_aware_swa_amd import binding, inputs
from phase_aware_swa_amd.runner import desc_for

pytestmark = pytest.mark.gpu


def make_cfg(B, Hq, Hkv, d, dtype, w=128):
    return dict(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=w, dtype=dtype)


def oracle_cache(xc, cap):
    B, T, Hkv, d = xc["k"].shape
    kc = torch.zeros(B, Hkv, cap, d, dtype=xc["k"].dtype)
    vc = torch.zeros(B, Hkv, cap, d, dtype=xc["k"].dtype)
    kc[:, :, :T] = xc["k"].transpose(1, 2)
    vc[:, :, :T] = xc["v"].transpose(1, 2)
    return kc, vc


def gpu_copies(cfg, T, xc, q_out, pos, cap):
    """The library's SWA pass writes the cache, then orthros_copies reads it."""
    B, Hq, Hkv, d, dt = cfg["batch"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["dtype"]
    desc = desc_for(cfg)
    x = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in xc.items()}
    kc = inputs.empty_cache(B, Hkv, cap, d, dt, "cuda")
    vc = inputs.empty_cache(B, Hkv, cap, d, dt, "cuda")
    o = torch.empty(B, T, Hq, d, dtype=dt, device="cuda")
    binding.swa_prefill(desc, T, x["q"], x["k"], x["v"], x["alpha"], x["beta"], kc, vc, o)
    o_out = torch.empty(B, q_out.shape[1], Hq, d, dtype=dt, device="cuda")
    binding.copies(desc, T, q_out.cuda(), pos.cuda(), x["alpha_out"], x["beta_out"], kc, vc, o_out)
    torch.cuda.synchronize()
    return o_out, kc, vc


def run_case(cfg, T, T_out, seed, positions="tail", pos=None, cap_extra=5):
    B, Hq, d, dt = cfg["batch"], cfg["n_q_heads"], cfg["head_dim"], cfg["dtype"]
    say(f"copies case {cfg} T={T} T_out={T_out} positions={positions} seed={seed}")
    xc = inputs.prefill_inputs(T=T, seed=seed, **cfg)
    q_out, p = inputs.copies_inputs(B, Hq, d, T, T_out, dt, seed + 1, positions=positions)
    if pos is not None:
        p = torch.tensor(pos, dtype=torch.int32).reshape(B, T_out)
    o_out, _, _ = gpu_copies(cfg, T, xc, q_out, p, T + cap_extra)
    kc, vc = oracle_cache(xc, T + cap_extra)
    ref = oracle.copies(q_out, p, xc["alpha_out"], xc["beta_out"], kc, vc, T)
    assert_parity(o_out, ref, dt, "o_out")
    return o_out, ref


# B, Hq, Hkv, d, T, T_out, positions
CASES = [
    (1, 4, 4, 64, 300, 300, "tail"),        # PT: every position copied
    (1, 4, 1, 128, 700, 700, "tail"),       # PT, one KV head for 4 query heads
    (2, 8, 2, 128, 777, 100, "tail"),       # SFT: an answer span at the end
    (2, 32, 8, 128, 1500, 257, "random"),   # positions unsorted, with repeats
    (1, 6, 2, 64, 200, 50, "random"),       # G = 3
    (1, 8, 1, 128, 1000, 64, "tail"),       # G = 8
    (3, 2, 2, 64, 90, 1, "random"),         # one copy (the prefill shape) per sequence
    (1, 4, 2, 128, 33, 33, "tail"),         # short prompt, ragged tiles
    # bf16 with groups of 4 / 8 takes the MFMA flash kernel: many two-pair steps
    (1, 8, 2, 64, 2100, 2100, "tail"),      # PT, d = 64
    (2, 8, 1, 128, 3000, 333, "random"),    # G = 8, a ragged last tile of copies
    (1, 4, 1, 128, 4096, 40, "tail"),       # SFT: one tile, positions 4056..4095
]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("B,Hq,Hkv,d,T,T_out,positions", CASES)
def test_copies_parity(B, Hq, Hkv, d, T, T_out, positions, dtype):
    run_case(make_cfg(B, Hq, Hkv, d, dtype), T, T_out, seed=500 + T + T_out, positions=positions)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_copies_at_first_and_last_position(dtype):
    """Copies at 0 read key 0 only: o_out = v_0 exactly (one weight of 1);
    a copy at T-1 reads every key."""
    cfg = make_cfg(2, 8, 2, 128, dtype)
    T = 400
    o_out, ref = run_case(cfg, T, 4, seed=41, pos=[0, T - 1, 0, 5, 0, 0, T - 1, 200])
    xc = inputs.prefill_inputs(T=T, seed=41, **cfg)
    v0 = xc["v"][:, 0].repeat_interleave(4, dim=1)          # [B, Hq, d]
    assert torch.equal(bits(o_out[0, 0].cpu()), bits(v0[0]))
    assert torch.equal(bits(o_out[1, 1].cpu()), bits(v0[1]))


def test_copies_invalid_positions_give_nan_and_leave_the_rest():
    """Positions outside [0, T) read nothing and give NaN for that copy only."""
    cfg = make_cfg(2, 8, 2, 128, torch.bfloat16)
    T, T_out = 300, 6
    say("copies with invalid positions")
    xc = inputs.prefill_inputs(T=T, seed=42, **cfg)
    q_out, _ = inputs.copies_inputs(2, 8, 128, T, T_out, torch.bfloat16, 43, positions="random")
    pos = torch.tensor([[5, -1, 299, 300, 150, 1 << 30], [0, 10, -7, 20, 299, 299]], dtype=torch.int32)
    o_out, kcg, _ = gpu_copies(cfg, T, xc, q_out, pos, T)
    bad = (pos < 0) | (pos >= T)
    assert torch.isnan(o_out.cpu()[bad].float()).all()
    good_pos = torch.where(bad, torch.zeros_like(pos), pos)
    kc, vc = oracle_cache(xc, T)
    ref = oracle.copies(q_out, good_pos, xc["alpha_out"], xc["beta_out"], kc, vc, T)
    assert_parity(o_out.cpu()[~bad], ref[~bad], torch.bfloat16, "valid copies")
    # the copies read the cache only
    assert torch.equal(bits(kcg[:, :, :T].cpu()), bits(xc["k"].transpose(1, 2)))


def test_copies_run_to_run_identical():
    cfg = make_cfg(2, 8, 2, 128, torch.bfloat16)
    T, T_out = 2000, 300
    say("copies determinism")
    xc = inputs.prefill_inputs(T=T, seed=44, **cfg)
    q_out, pos = inputs.copies_inputs(2, 8, 128, T, T_out, torch.bfloat16, 45, positions="random")
    a, _, _ = gpu_copies(cfg, T, xc, q_out, pos, T)
    b, _, _ = gpu_copies(cfg, T, xc, q_out, pos, T)
    assert torch.equal(bits(a), bits(b))
