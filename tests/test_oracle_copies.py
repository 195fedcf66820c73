"""Pins of the oracle's many-copy form (the PT and SFT modes of
"Orthros:阶段感知异构注意力精读笔记" §2.5: output copies at arbitrary
original positions, each the Eq. (5) query of its position) to things other
than itself: torch's SDPA in fp64, the one-copy prefill path, and
invariants.  CPU only."""
import pytest
import torch
import torch.nn.functional as F

import oracle
from phase_aware_swa_amd import inputs

f64 = torch.float64


def make(B, T, Hq, Hkv, d, T_out, seed, dtype=torch.float32, cap_extra=3):
    """Base K/V in a cache of capacity T + cap_extra, and T_out raw copy queries."""
    x = inputs.prefill_inputs(B, Hq, Hkv, d, T, dtype, seed)
    g = torch.Generator().manual_seed(seed + 1)
    q_out = torch.randn(B, T_out, Hq, d, generator=g).to(dtype)
    cap = T + cap_extra
    kc = torch.zeros(B, Hkv, cap, d, dtype=dtype)
    vc = torch.zeros(B, Hkv, cap, d, dtype=dtype)
    kc[:, :, :T] = x["k"].transpose(1, 2)
    vc[:, :, :T] = x["v"].transpose(1, 2)
    return x, q_out, kc, vc


def sdpa_masked(q, k, v, pos, scale):
    """q [n,d] at original positions pos [n]; k, v [T,d]; key j allowed iff j <= pos."""
    T = k.shape[0]
    mask = torch.arange(T)[None, :] <= torch.as_tensor(pos)[:, None]
    return F.scaled_dot_product_attention(q[None, None], k[None, None], v[None, None],
                                          attn_mask=mask[None, None], scale=scale)[0, 0]


@pytest.mark.parametrize("B,T,G,d", [(1, 50, 1, 16), (2, 33, 2, 8), (1, 64, 4, 32)])
def test_pt_mode_is_causal_attention(B, T, G, d):
    """PT copies every position: with alpha' = 1, beta' = 0 the copies are
    plain causal attention of q_out against the base K/V.  Catches j < t for
    j <= t, a wrong KV-head map, a wrong scale, copies reading each other."""
    Hkv = 2
    x, q_out, kc, vc = make(B, T, G * Hkv, Hkv, d, T, seed=20 + T)
    a1 = torch.ones_like(x["alpha_out"])
    b0 = torch.zeros_like(x["beta_out"])
    pos = torch.arange(T).repeat(B, 1)
    o = oracle.copies(q_out, pos, a1, b0, kc, vc, T)
    for b in range(B):
        for h in range(G * Hkv):
            ref = F.scaled_dot_product_attention(
                q_out[b, :, h].to(f64)[None, None], x["k"][b, :, h // G].to(f64)[None, None],
                x["v"][b, :, h // G].to(f64)[None, None], is_causal=True, scale=d ** -0.5)[0, 0]
            torch.testing.assert_close(o[b, :, h], ref, rtol=0, atol=1e-12)


def test_sft_positions_follow_original_position_not_slot():
    """SFT copies at answer positions, given here unsorted and with repeats:
    copy i reads keys [0, pos_i], whatever its slot i.  Catches a mask by
    slot, a mask shifted by the prompt length, sorted-position assumptions."""
    B, T, Hq, Hkv, d, T_out = 2, 60, 4, 2, 16, 9
    x, q_out, kc, vc = make(B, T, Hq, Hkv, d, T_out, seed=31)
    pos = torch.tensor([[59, 0, 17, 17, 40, 3, 58, 31, 12], [5, 5, 59, 22, 0, 1, 44, 30, 58]])
    a1 = torch.ones_like(x["alpha_out"])
    b0 = torch.zeros_like(x["beta_out"])
    o = oracle.copies(q_out, pos, a1, b0, kc, vc, T)
    for b in range(B):
        for h in range(Hq):
            ref = sdpa_masked(q_out[b, :, h].to(f64), x["k"][b, :, h // 2].to(f64),
                              x["v"][b, :, h // 2].to(f64), pos[b], d ** -0.5)
            torch.testing.assert_close(o[b, :, h], ref, rtol=0, atol=1e-12)


def test_copies_scale_offset_alpha_zero_gives_beta_query():
    """alpha' = 0 leaves the copy query beta', whatever q_out is: each copy is
    SDPA with query beta'_h at its position.  Catches the base stream's
    alpha/beta used for the copies, (q + beta) * alpha."""
    B, T, Hq, Hkv, d, T_out = 1, 40, 4, 2, 8, 5
    x, q_out, kc, vc = make(B, T, Hq, Hkv, d, T_out, seed=32)
    pos = torch.tensor([[39, 10, 0, 25, 7]])
    o = oracle.copies(q_out, pos, torch.zeros_like(x["alpha_out"]), x["beta_out"], kc, vc, T)
    for h in range(Hq):
        qb = x["beta_out"][h].to(f64).expand(T_out, d).contiguous()
        ref = sdpa_masked(qb, x["k"][0, :, h // 2].to(f64), x["v"][0, :, h // 2].to(f64), pos[0], d ** -0.5)
        torch.testing.assert_close(o[0, :, h], ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_one_copy_equals_prefill_copy(dtype):
    """A single copy at position P gives the bits of the one-copy prefill path
    (Eq. (5) with out_pos = P), with its own alpha', beta'."""
    B, T, Hq, Hkv, d = 2, 45, 4, 1, 16
    x, q_out, kc, vc = make(B, T, Hq, Hkv, d, 1, seed=33, dtype=dtype)
    pos = torch.tensor([[44], [19]])
    o = oracle.copies(q_out, pos, x["alpha_out"], x["beta_out"], kc, vc, T)
    r = oracle.prefill(None, q_out[:, 0].contiguous(), [44, 19], x["k"], x["v"], x["alpha"], x["beta"],
                       x["alpha_out"], x["beta_out"], 8, swa=False)
    assert torch.equal(o[:, 0], r["o_out"])


def test_copies_gqa_equals_mha_with_repeated_kv():
    """G = 4 query heads per KV head equals MHA with the KV heads repeated."""
    B, T, Hq, Hkv, d, T_out = 1, 30, 8, 2, 8, 6
    x, q_out, kc, vc = make(B, T, Hq, Hkv, d, T_out, seed=34)
    pos = torch.tensor([[29, 3, 14, 0, 22, 8]])
    o = oracle.copies(q_out, pos, x["alpha_out"], x["beta_out"], kc, vc, T)
    o_mha = oracle.copies(q_out, pos, x["alpha_out"], x["beta_out"], kc.repeat_interleave(4, dim=1).contiguous(),
                          vc.repeat_interleave(4, dim=1).contiguous(), T)
    assert torch.equal(o, o_mha)


def test_copies_reject_positions_outside_prompt():
    B, T, Hq, Hkv, d = 1, 10, 2, 1, 8
    x, q_out, kc, vc = make(B, T, Hq, Hkv, d, 2, seed=35)
    for bad in ([[3, 10]], [[-1, 0]]):
        with pytest.raises(ValueError):
            oracle.copies(q_out, torch.tensor(bad), x["alpha_out"], x["beta_out"], kc, vc, T)
