"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test fixes one part of the definition in "Orthros:阶段感知异构注意力精读笔记"
against a library routine (torch SDPA in fp64), the dense-matrix brute
force, a closed form, or an invariant the pages state.  The plausible
mistakes each one catches are named in its docstring.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import brute
from phase_aware_swa_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
f64 = torch.float64


def rand_case(B, T, Hq, Hkv, d, seed, dtype=torch.float32):
    return inputs.prefill_inputs(B, Hq, Hkv, d, T, dtype, seed)


def sdpa_causal(q, k, v, scale):
    """Full causal attention, torch's routine in fp64.  q [T,d], k/v [T,d]."""
    return F.scaled_dot_product_attention(q[None, None], k[None, None], v[None, None],
                                          is_causal=True, scale=scale)[0, 0]


def run_oracle(x, window, **kw):
    return oracle.prefill(x["q"], x["q_out"], x["out_pos"], x["k"], x["v"], x["alpha"],
                          x["beta"], x["alpha_out"], x["beta_out"], window, **kw)


# ------------------------------------------------------------------ P1 / SO

@pytest.mark.parametrize("T,d,G", [(64, 16, 1), (100, 32, 2), (37, 8, 4)])
def test_swa_full_window_is_causal_attention(T, d, G):
    """P1: a window w >= T keeps every causal key, so Eq. (4) is plain causal
    attention.  alpha = 1, beta = 0 makes q_hat = q.  Catches an off-by-one
    upper bound (j < t), a wrong KV-head map, a wrong scale."""
    x = rand_case(1, T, 2 * G, 2, d, seed=1)
    x["alpha"].fill_(1.0)
    x["beta"].zero_()
    for w in (T, T + 7):
        r = run_oracle(x, w)
        for h in range(2 * G):
            ref = sdpa_causal(x["q"][0, :, h].to(f64), x["k"][0, :, h // G].to(f64),
                              x["v"][0, :, h // G].to(f64), d ** -0.5)
            torch.testing.assert_close(r["o"][0, :, h], ref, rtol=0, atol=1e-12)


def test_scale_offset_alpha_zero_gives_beta_query():
    """SO: alpha = 0 leaves q_hat = beta for every row, whatever q is.
    Catches (q + beta) * alpha and a swapped alpha/beta."""
    T, d = 40, 16
    x = rand_case(1, T, 2, 2, d, seed=2)
    x["alpha"].zero_()
    r = run_oracle(x, window=T)
    for h in range(2):
        qb = x["beta"][h].to(f64).expand(T, d).contiguous()
        ref = sdpa_causal(qb, x["k"][0, :, h].to(f64), x["v"][0, :, h].to(f64), d ** -0.5)
        torch.testing.assert_close(r["o"][0, :, h], ref, rtol=0, atol=1e-12)


def test_scale_offset_is_per_query_head():
    """SO: alpha = c_h (one constant per head), beta = 0 is attention with the
    queries scaled by c_h.  With G = 2 two heads share a KV head but not
    alpha, so using the KV head's (or another head's) alpha fails."""
    T, d = 50, 8
    x = rand_case(1, T, 4, 2, d, seed=3)
    c = [0.5, 2.0, -1.0, 3.0]
    for h in range(4):
        x["alpha"][h].fill_(c[h])
    x["beta"].zero_()
    r = run_oracle(x, window=T)
    for h in range(4):
        ref = sdpa_causal(c[h] * x["q"][0, :, h].to(f64), x["k"][0, :, h // 2].to(f64),
                          x["v"][0, :, h // 2].to(f64), d ** -0.5)
        torch.testing.assert_close(r["o"][0, :, h], ref, rtol=0, atol=1e-12)


def test_output_stream_uses_its_own_scale_offset():
    """SO: base stream alpha = beta = 0 (uniform weights), output stream
    alpha' = 1, beta' = 0: the copy must equal the causal row of raw q_out.
    Catches the copy using the base stream's alpha/beta or vice versa."""
    T, d = 33, 16
    x = rand_case(1, T, 1, 1, d, seed=4)
    x["alpha"].zero_()
    x["beta"].zero_()
    x["alpha_out"].fill_(1.0)
    x["beta_out"].zero_()
    r = run_oracle(x, window=T)
    qfull = x["q"][0, :, 0].to(f64).clone()
    qfull[T - 1] = x["q_out"][0, 0].to(f64)
    ref = sdpa_causal(qfull, x["k"][0, :, 0].to(f64), x["v"][0, :, 0].to(f64), d ** -0.5)
    torch.testing.assert_close(r["o_out"][0, 0], ref[T - 1], rtol=0, atol=1e-12)
    # uniform weights: the base row t is the mean of v_0..v_t
    vm = torch.cumsum(x["v"][0, :, 0].to(f64), 0) / torch.arange(1, T + 1, dtype=f64)[:, None]
    torch.testing.assert_close(r["o"][0, :, 0], vm, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------- P2

@pytest.mark.parametrize("P", [0, 1, 17, 63])
def test_global_is_row_P_of_causal_attention(P):
    """P2: the copy at original position P (Eq. (5), j <= P) equals row P of
    full causal attention whose query row P is the copy's query.  P < T-1
    also pins masking by original position, not by slot index (§2.4)."""
    T, d = 64, 32
    x = rand_case(2, T, 2, 1, d, seed=5)
    x["alpha_out"].fill_(1.0)
    x["beta_out"].zero_()
    x["out_pos"] = [P, T - 1]
    r = run_oracle(x, window=8)
    for b, pos in ((0, P), (1, T - 1)):
        for h in range(2):
            qfull = x["q"][b, :, h].to(f64).clone()
            qfull[pos] = x["q_out"][b, h].to(f64)
            ref = sdpa_causal(qfull, x["k"][b, :, 0].to(f64), x["v"][b, :, 0].to(f64), d ** -0.5)
            torch.testing.assert_close(r["o_out"][b, h], ref[pos], rtol=0, atol=1e-12)


# ----------------------------------------------------------------------- P3

def test_base_stream_does_not_depend_on_output_stream():
    """P3: the base K/V cache and the base outputs never depend on the output
    stream (§2.4).  Perturbing q_out, alpha', beta' leaves them bit-identical."""
    T, d = 80, 16
    x = rand_case(1, T, 4, 2, d, seed=6, dtype=torch.bfloat16)
    r1 = run_oracle(x, window=16)
    y = dict(x)
    y["q_out"] = x["q_out"] * 3 + 1
    y["alpha_out"] = -x["alpha_out"]
    y["beta_out"] = x["beta_out"] + 5
    r2 = run_oracle(y, window=16)
    assert torch.equal(r1["o"], r2["o"])
    assert torch.equal(r1["k_cache"].view(torch.int16), r2["k_cache"].view(torch.int16))
    assert torch.equal(r1["v_cache"].view(torch.int16), r2["v_cache"].view(torch.int16))
    assert not torch.equal(r1["o_out"], r2["o_out"])


# ----------------------------------------------------------------------- P4

def test_walkthrough_prefill_then_decode():
    """P4: the §2.4 teaching example.  prefill([A,B,C]) with copy C', then one
    decode step with D / D', equals prefill([A,B,C,D]) with the copy at D:
    the same cache bytes, the same base output at D and the same copy output."""
    spec = json.load(open(os.path.join(GOLDEN, "walkthrough.json")))
    assert spec["cache_after"] == spec["equivalent_prefill"]["prompt"]
    n = len(spec["tokens"])                      # 4 tokens A, B, C, D
    d, Hq, Hkv, w = 16, 4, 2, 2
    x = rand_case(1, n, Hq, Hkv, d, seed=7, dtype=torch.bfloat16)
    cap = 8
    full = run_oracle(x, window=w, cap=cap, k_cache=inputs.empty_cache(1, Hkv, cap, d, torch.bfloat16),
                      v_cache=inputs.empty_cache(1, Hkv, cap, d, torch.bfloat16))
    # prefill of the prompt A, B, C with its copy at C (position 2)
    p = {key: (val[:, : n - 1].contiguous() if key in ("q", "k", "v") else val) for key, val in x.items()}
    p["out_pos"] = [n - 2]
    kc = inputs.empty_cache(1, Hkv, cap, d, torch.bfloat16)
    vc = inputs.empty_cache(1, Hkv, cap, d, torch.bfloat16)
    first = run_oracle(p, window=w, k_cache=kc, v_cache=vc)
    torch.testing.assert_close(first["o"][0], full["o"][0, : n - 1], rtol=0, atol=0)
    # decode step: base token D and its copy D'
    L = torch.tensor([n - 1], dtype=torch.int32)
    o, o_out = oracle.decode_step(x["q"][:, n - 1].contiguous(), x["q_out"], x["k"][:, n - 1].contiguous(),
                                  x["v"][:, n - 1].contiguous(), x["alpha"], x["beta"], x["alpha_out"],
                                  x["beta_out"], w, kc, vc, L)
    assert L.item() == n
    assert torch.equal(kc.view(torch.int16), full["k_cache"].view(torch.int16))
    assert torch.equal(vc.view(torch.int16), full["v_cache"].view(torch.int16))
    assert torch.equal(o, full["o"][:, n - 1])
    assert torch.equal(o_out, full["o_out"])


def test_decode_step_equals_prefill_of_extended_sequence():
    """P4 at a length beyond the window: a decode step at L equals prefill of
    the L+1 tokens with the copy at L (base row L and the copy)."""
    L0, d, Hq, Hkv, w = 45, 8, 2, 1, 6
    x = rand_case(1, L0 + 1, Hq, Hkv, d, seed=8)
    full = run_oracle(x, window=w)
    cap = L0 + 3
    kc = torch.zeros(1, Hkv, cap, d)
    vc = torch.zeros(1, Hkv, cap, d)
    kc[0, :, :L0] = x["k"][0, :L0].transpose(0, 1)
    vc[0, :, :L0] = x["v"][0, :L0].transpose(0, 1)
    L = torch.tensor([L0], dtype=torch.int32)
    o, o_out = oracle.decode_step(x["q"][:, L0].contiguous(), x["q_out"], x["k"][:, L0].contiguous(),
                                  x["v"][:, L0].contiguous(), x["alpha"], x["beta"], x["alpha_out"],
                                  x["beta_out"], w, kc, vc, L)
    assert torch.equal(o, full["o"][:, L0])
    assert torch.equal(o_out, full["o_out"])
    assert torch.equal(kc[0, :, : L0 + 1], full["k_cache"][0])


# ----------------------------------------------------------------------- P5

@pytest.mark.parametrize("T", [1, 2, 3, 17, 64])
@pytest.mark.parametrize("wsel", ["1", "2", "5", "T", "T+5"])
@pytest.mark.parametrize("G", [1, 2, 4])
def test_brute_force_tiny(T, wsel, G):
    """P5: the loop form (oracle.c) against the dense T x T mask form
    (brute.py) on every small (T, w, G).  Catches any window-edge, GQA or
    copy-position slip that only shows at some sizes."""
    w = {"1": 1, "2": 2, "5": 5, "T": T, "T+5": T + 5}[wsel]
    d = 8
    x = rand_case(2, T, 2 * G, 2, d, seed=100 + T * 7 + G)
    x["out_pos"] = [T - 1, T // 2]
    r = run_oracle(x, window=w)
    npx = {key: x[key].double().numpy() for key in ("q", "q_out", "k", "v", "alpha", "beta",
                                                     "alpha_out", "beta_out")}
    o, o_out = brute.prefill(npx["q"], npx["q_out"], x["out_pos"], npx["k"], npx["v"], npx["alpha"],
                             npx["beta"], npx["alpha_out"], npx["beta_out"], w, d ** -0.5)
    np.testing.assert_allclose(r["o"].numpy(), o, rtol=0, atol=1e-12)
    np.testing.assert_allclose(r["o_out"].numpy(), o_out, rtol=0, atol=1e-12)


# ------------------------------------------------------------------- P6, P7

def test_window_one_returns_own_value_exactly():
    """P6: w = 1 leaves one key (the row itself) with weight exactly 1."""
    x = rand_case(1, 30, 4, 2, 16, seed=9, dtype=torch.bfloat16)
    r = run_oracle(x, window=1)
    for h in range(4):
        assert torch.equal(r["o"][0, :, h], x["v"][0, :, h // 2].to(f64))


def test_first_position_returns_v0_exactly():
    """P7: row 0 and a copy at position 0 each see only key 0."""
    x = rand_case(2, 30, 2, 2, 16, seed=10, dtype=torch.bfloat16)
    x["out_pos"] = [0, 0]
    r = run_oracle(x, window=128)
    for b in range(2):
        for h in range(2):
            assert torch.equal(r["o"][b, 0, h], x["v"][b, 0, h].to(f64))
            assert torch.equal(r["o_out"][b, h], x["v"][b, 0, h].to(f64))


# ----------------------------------------------------------------------- P8

@pytest.mark.parametrize("w", [1, 3, 16, 128])
def test_mask_probe_recovers_key_sets(w):
    """P8: with alpha = beta = 0 every admissible key gets the same weight, so
    with V rows [1, j, j^2] the output is the mean over the key set; its
    count and first index follow in closed form.  Any shifted or resized
    window, or a copy masked by slot instead of position, moves them."""
    T, d = 300, 3
    x = rand_case(1, T, 1, 1, d, seed=11)
    for key in ("alpha", "beta", "alpha_out", "beta_out"):
        x[key].zero_()
    j = torch.arange(T, dtype=torch.float32)
    x["v"][0, :, 0] = torch.stack([torch.ones(T), j, j * j], 1)
    x["out_pos"] = [157]
    r = run_oracle(x, window=w)
    for t in range(T):
        lo = max(0, t - w + 1)
        n = t - lo + 1
        mean_j = (lo + t) / 2
        mean_j2 = sum(i * i for i in range(lo, t + 1)) / n
        torch.testing.assert_close(r["o"][0, t, 0], torch.tensor([1.0, mean_j, mean_j2], dtype=f64),
                                   rtol=1e-13, atol=1e-9)
    torch.testing.assert_close(r["o_out"][0, 0],
                               torch.tensor([1.0, 157 / 2, sum(i * i for i in range(158)) / 158], dtype=f64),
                               rtol=1e-13, atol=1e-9)


# ---------------------------------------------------------------- P9, P10

def test_gqa_equals_mha_with_repeated_kv():
    """P9: query head h reads KV head h // G; the same result comes from MHA
    with each KV head repeated G times (repeat_interleave)."""
    G = 4
    x = rand_case(1, 40, 8, 2, 16, seed=12)
    r = run_oracle(x, window=7)
    y = dict(x)
    y["k"] = x["k"].repeat_interleave(G, dim=2).contiguous()
    y["v"] = x["v"].repeat_interleave(G, dim=2).contiguous()
    r2 = run_oracle(y, window=7)
    torch.testing.assert_close(r["o"], r2["o"], rtol=0, atol=1e-13)
    torch.testing.assert_close(r["o_out"], r2["o_out"], rtol=0, atol=1e-13)


def test_shift_invariance_of_keys():
    """P10: adding one vector u to every key adds <q, u> to all scores of a
    query; softmax is unchanged.  Catches a missing max subtraction that
    overflows, or a normaliser summed over the wrong set."""
    x = rand_case(1, 50, 2, 1, 16, seed=13)
    # keys on a 2^-8 grid and an integer shift keep k + u exact in fp32
    x["k"] = (x["k"] * 256).round() / 256
    r = run_oracle(x, window=9)
    y = dict(x)
    u = torch.randint(-40, 41, (16,), generator=torch.Generator().manual_seed(0)).float()
    y["k"] = (x["k"] + u).contiguous()
    r2 = run_oracle(y, window=9)
    torch.testing.assert_close(r["o"], r2["o"], rtol=0, atol=1e-9)
    torch.testing.assert_close(r["o_out"], r2["o_out"], rtol=0, atol=1e-9)


# ---------------------------------------------------------------------- P11

def test_cache_bytes_and_untouched_slots():
    """P11: slot j of KV head g holds k[b, j, g] byte for byte; slots >= T
    keep the sentinel."""
    B, T, Hkv, d, cap = 2, 37, 3, 16, 50
    x = rand_case(B, T, 6, Hkv, d, seed=14, dtype=torch.bfloat16)
    kc = inputs.empty_cache(B, Hkv, cap, d, torch.bfloat16)
    vc = inputs.empty_cache(B, Hkv, cap, d, torch.bfloat16)
    run_oracle(x, window=5, k_cache=kc, v_cache=vc)
    assert torch.equal(kc[:, :, :T].view(torch.int16), x["k"].transpose(1, 2).contiguous().view(torch.int16))
    assert torch.equal(vc[:, :, :T].view(torch.int16), x["v"].transpose(1, 2).contiguous().view(torch.int16))
    assert bool((kc[:, :, T:].view(torch.int16) == inputs.SENTINEL_BF16_BITS).all())
    assert bool((vc[:, :, T:].view(torch.int16) == inputs.SENTINEL_BF16_BITS).all())


def test_decode_appends_at_length_only():
    """P11 for decode: the step writes slot len[b] of every KV head and no
    other slot, then increments len[b]."""
    B, Hq, Hkv, d, cap = 3, 4, 2, 8, 20
    g = torch.Generator().manual_seed(15)
    kc = inputs.empty_cache(B, Hkv, cap, d, torch.bfloat16)
    vc = inputs.empty_cache(B, Hkv, cap, d, torch.bfloat16)
    lens = torch.tensor([3, 0, 11], dtype=torch.int32)
    for b in range(B):
        kc[b, :, : lens[b]] = torch.randn(Hkv, int(lens[b]), d, generator=g).bfloat16()
        vc[b, :, : lens[b]] = torch.randn(Hkv, int(lens[b]), d, generator=g).bfloat16()
    before_k, before_v = kc.clone(), vc.clone()
    mk = lambda *s: torch.randn(*s, generator=g).bfloat16()
    k_new, v_new = mk(B, Hkv, d), mk(B, Hkv, d)
    o, o_out = oracle.decode_step(mk(B, Hq, d), mk(B, Hq, d), k_new, v_new, mk(Hq, d), mk(Hq, d),
                                  mk(Hq, d), mk(Hq, d), 4, kc, vc, lens)
    assert lens.tolist() == [4, 1, 12]
    for b, L in enumerate([3, 0, 11]):
        assert torch.equal(kc[b, :, L].view(torch.int16), k_new[b].view(torch.int16))
        assert torch.equal(vc[b, :, L].view(torch.int16), v_new[b].view(torch.int16))
        keep = [s for s in range(cap) if s != L]
        assert torch.equal(kc[b, :, keep].view(torch.int16), before_k[b, :, keep].view(torch.int16))
        assert torch.equal(vc[b, :, keep].view(torch.int16), before_v[b, :, keep].view(torch.int16))
    assert torch.isfinite(o).all() and torch.isfinite(o_out).all()


# ---------------------------------------------------------------------- P12

def test_needle_dominates_copy_softmax():
    """P12: the planted needle key takes >= 0.99 of the planting head's copy
    softmax, so that head's output is within 1% of the needle's value row
    (checked on a shortened sequence of the 128K workload's shape)."""
    cfg = dict(inputs.WORKLOADS["gqa_8b_prefill_128k"])
    cfg.update(T=4096)
    x = inputs.prefill_inputs(**cfg, seed=2)
    r = run_oracle(x, window=cfg["window"], swa=False)
    G = cfg["n_q_heads"] // cfg["n_kv_heads"]
    for b in range(cfg["batch"]):
        for g in range(cfg["n_kv_heads"]):
            p = int(x["needle_pos"][b, g])
            vn = x["v"][b, p, g].to(f64)
            other = x["v"][b, :, g].to(f64)
            spread = (other - vn).abs().max()
            assert (r["o_out"][b, g * G] - vn).abs().max() <= 0.01 * spread


# ------------------------------------------------------------- golden, dtype

def test_golden_closed_form():
    """Hand-derived closed forms for a 3-token case with nontrivial alpha,
    beta, alpha', beta' (tests/golden/tiny_closed_form.json)."""
    spec = json.load(open(os.path.join(GOLDEN, "tiny_closed_form.json")))
    sh = spec["shape"]
    T = sh["T"]
    t = lambda key, shape: torch.tensor(spec[key], dtype=torch.float32).reshape(shape).contiguous()
    x = dict(q=t("q", (1, T, 1, 2)), k=t("k", (1, T, 1, 2)), v=t("v", (1, T, 1, 2)),
             alpha=t("alpha", (1, 2)), beta=t("beta", (1, 2)), q_out=t("q_out", (1, 1, 2)),
             alpha_out=t("alpha_out", (1, 2)), beta_out=t("beta_out", (1, 2)))
    env = {"e": math.e}
    ev = lambda key: torch.tensor([eval(s, {}, env) for s in spec["expected"][key]], dtype=f64)
    for P in (2, 1, 0):
        x["out_pos"] = [P]
        r = run_oracle(x, window=sh["window"], softmax_scale=sh["softmax_scale"])
        for row in range(T):
            torch.testing.assert_close(r["o"][0, row, 0], ev(f"o[{row}]"), rtol=0, atol=1e-12)
        torch.testing.assert_close(r["o_out"][0, 0], ev(f"o_out(pos={P})"), rtol=0, atol=1e-12)


def test_bf16_storage_promotes_exactly():
    """bf16 inputs are read as their exact values: the oracle on bf16 storage
    equals the oracle on the same values stored as fp32, bit for bit."""
    x = rand_case(1, 25, 2, 1, 16, seed=16, dtype=torch.bfloat16)
    y = {key: (val.float() if torch.is_tensor(val) else val) for key, val in x.items()}
    r1 = run_oracle(x, window=4)
    r2 = run_oracle(y, window=4)
    assert torch.equal(r1["o"], r2["o"]) and torch.equal(r1["o_out"], r2["o_out"])


def test_explicit_softmax_scale():
    """softmax_scale = 0 in the shape means 1/sqrt(d); an explicit value is
    used as given (SDPA with that scale)."""
    T, d = 20, 16
    x = rand_case(1, T, 1, 1, d, seed=17)
    x["alpha"].fill_(1.0)
    x["beta"].zero_()
    r = run_oracle(x, window=T, softmax_scale=0.3)
    ref = sdpa_causal(x["q"][0, :, 0].to(f64), x["k"][0, :, 0].to(f64), x["v"][0, :, 0].to(f64), 0.3)
    torch.testing.assert_close(r["o"][0, :, 0], ref, rtol=0, atol=1e-12)


def test_swa_rows_match_full_prefill():
    """The sampled-row entry computes the same Eq. (4) rows as the full call."""
    x = rand_case(2, 70, 4, 2, 16, seed=18, dtype=torch.bfloat16)
    r = run_oracle(x, window=9)
    rows = torch.tensor([[0, 0, 0], [1, 69, 3], [0, 8, 1], [1, 9, 2], [0, 40, 3]])
    out = oracle.swa_rows(x["q"], x["k"], x["v"], x["alpha"], x["beta"], 9, rows)
    for i, (b, tt, h) in enumerate(rows.tolist()):
        assert torch.equal(out[i], r["o"][b, tt, h])


def test_swa_rows_given_q_match_full_prefill():
    """Rows whose queries are passed one by one give the full call's rows bit
    for bit (a row paired with the wrong query or head would not)."""
    x = rand_case(2, 70, 4, 2, 16, seed=19, dtype=torch.bfloat16)
    r = run_oracle(x, window=9)
    rows = torch.tensor([[0, 0, 0], [1, 69, 3], [0, 8, 1], [1, 9, 2], [0, 40, 3], [1, 40, 0]])
    qrows = torch.stack([x["q"][b, t, h] for b, t, h in rows.tolist()]).contiguous()
    out = oracle.swa_rows_given_q(qrows, x["k"], x["v"], x["alpha"], x["beta"], 9, rows, n_q_heads=4)
    for i, (b, tt, h) in enumerate(rows.tolist()):
        assert torch.equal(out[i], r["o"][b, tt, h])


def test_probe_closed_form_counts():
    """The mask probes' closed form (tests/probe_util.py) against brute
    force: residue counts of key intervals, and exact bf16 ratios."""
    import sys
    sys.path.insert(0, os.path.dirname(__file__))
    from probe_util import assert_probe, residue_counts
    for m, d in ((127, 128), (127, 64)):
        for lo in range(0, 260, 37):
            for hi in range(lo - 1, lo + 300, 41):
                for sh in (0, 5, 126):
                    c = residue_counts(torch.tensor(lo), torch.tensor(hi), torch.tensor(sh), m, d)
                    ref = torch.zeros(d, dtype=torch.int64)
                    for j in range(lo, hi + 1):
                        if (j + sh) % m < d:
                            ref[(j + sh) % m] += 1
                    assert torch.equal(c, ref), (m, d, lo, hi, sh)
    # a window of 128 keys over V = one-hot (j mod 127): 2/128 and 1/128 exactly
    cnt = residue_counts(torch.tensor([500]), torch.tensor([627]), torch.tensor([0]), 127, 128)
    vals = (cnt.double() / 128).bfloat16()
    assert assert_probe(vals, cnt, torch.tensor([128]), "closed form") == 0
    assert sorted(set(vals.float()[0].tolist())) == [0.0, 1 / 128, 2 / 128]
    bad = vals.clone()
    bad[0, 3] = (cnt[0, 3].double() / 129).bfloat16()
    with pytest.raises(AssertionError):
        assert_probe(bad, cnt, torch.tensor([128]), "a key too many")
