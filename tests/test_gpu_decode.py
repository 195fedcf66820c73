"""GPU parity of orthros_decode_step against the fp64 oracle, through the C
ABI (MI355X only)."""
import pytest
import torch

import oracle
from gpu_util import assert_parity, bits, say, to_cpu, to_dev
from phase_aware_swa_amd import inputs
from phase_aware_swa_amd.runner import Decode, Prefill

pytestmark = pytest.mark.gpu


def small_decode_inputs(B, Hq, Hkv, d, dtype, lens, steps, seed):
    g = torch.Generator().manual_seed(seed)
    cap = max(lens) + steps + 5
    mk = lambda *s: torch.randn(*s, generator=g).to(dtype)
    kc = inputs.empty_cache(B, Hkv, cap, d, dtype)
    vc = inputs.empty_cache(B, Hkv, cap, d, dtype)
    for b, L in enumerate(lens):
        kc[b, :, :L] = mk(Hkv, L, d)
        vc[b, :, :L] = mk(Hkv, L, d)
    x = dict(k_cache=kc, v_cache=vc, cache_len=torch.tensor(lens, dtype=torch.int32),
             q=mk(steps, B, Hq, d), q_out=mk(steps, B, Hq, d), k_new=mk(steps, B, Hkv, d),
             v_new=mk(steps, B, Hkv, d), alpha=(1 + 0.1 * torch.randn(Hq, d, generator=g)).to(dtype),
             beta=(0.1 * torch.randn(Hq, d, generator=g)).to(dtype),
             alpha_out=(1 + 0.1 * torch.randn(Hq, d, generator=g)).to(dtype),
             beta_out=(0.1 * torch.randn(Hq, d, generator=g)).to(dtype))
    return x, cap


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("Hq,Hkv,d,w", [(8, 2, 128, 128), (4, 4, 64, 5), (6, 2, 128, 1), (4, 1, 64, 300)])
def test_decode_steps_parity(Hq, Hkv, d, w, dtype):
    """Every step of a short run against the oracle, lengths 0 (empty history),
    below the window, and across several split chunks."""
    lens = [0, 5, 300, 1100]
    steps = 12
    say(f"decode case Hq={Hq} Hkv={Hkv} d={d} w={w} {dtype} lens={lens}")
    xc, cap = small_decode_inputs(len(lens), Hq, Hkv, d, dtype, lens, steps, seed=21)
    cfg = dict(batch=len(lens), n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=w, dtype=dtype)
    x = to_dev(xc)
    dec = Decode(cfg, x["k_cache"], x["v_cache"], x["cache_len"], max(lens) + steps, x["alpha"], x["beta"],
                 x["alpha_out"], x["beta_out"])
    kc, vc, lc = xc["k_cache"].clone(), xc["v_cache"].clone(), xc["cache_len"].clone()
    for s in range(steps):
        dec.step(x["q"][s], x["q_out"][s], x["k_new"][s], x["v_new"][s])
        torch.cuda.synchronize()
        o, o_out = oracle.decode_step(xc["q"][s], xc["q_out"][s], xc["k_new"][s], xc["v_new"][s], xc["alpha"],
                                      xc["beta"], xc["alpha_out"], xc["beta_out"], w, kc, vc, lc)
        assert_parity(dec.o, o, dtype, f"o step {s}")
        assert_parity(dec.o_out, o_out, dtype, f"o_out step {s}")
    assert torch.equal(dec.cache_len.cpu(), lc)
    assert torch.equal(bits(dec.k_cache.cpu()), bits(kc))
    assert torch.equal(bits(dec.v_cache.cpu()), bits(vc))


@pytest.mark.parametrize("d", [128, 64])
def test_decode_lengths_at_stage_and_chunk_edges(d):
    """bf16, 4-head groups, short histories (the LDS-streamed kernel, at
    d = 128 and d = 64): lengths whose new key L is
    the first or last key of a 128- or 256-key block and of a 256-key chunk,
    and one that leaves the last chunk a single key; 3 steps each."""
    lens = [0, 127, 128, 255, 256, 511, 1023, 4095]
    steps = 3
    Hq, Hkv, w = 8, 2, 128
    dtype = torch.bfloat16
    say(f"decode edges d={d} lens={lens}")
    xc, cap = small_decode_inputs(len(lens), Hq, Hkv, d, dtype, lens, steps, seed=25 + d)
    cfg = dict(batch=len(lens), n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=w, dtype=dtype)
    x = to_dev(xc)
    dec = Decode(cfg, x["k_cache"], x["v_cache"], x["cache_len"], max(lens) + steps, x["alpha"], x["beta"],
                 x["alpha_out"], x["beta_out"])
    kc, vc, lc = xc["k_cache"].clone(), xc["v_cache"].clone(), xc["cache_len"].clone()
    for s in range(steps):
        dec.step(x["q"][s], x["q_out"][s], x["k_new"][s], x["v_new"][s])
        torch.cuda.synchronize()
        o, o_out = oracle.decode_step(xc["q"][s], xc["q_out"][s], xc["k_new"][s], xc["v_new"][s], xc["alpha"],
                                      xc["beta"], xc["alpha_out"], xc["beta_out"], w, kc, vc, lc)
        assert_parity(dec.o, o, dtype, f"o step {s}")
        assert_parity(dec.o_out, o_out, dtype, f"o_out step {s}")
    assert torch.equal(dec.cache_len.cpu(), lc)
    assert torch.equal(bits(dec.k_cache.cpu()), bits(kc))
    assert torch.equal(bits(dec.v_cache.cpu()), bits(vc))


@pytest.mark.parametrize("keys", [4096, 4097], ids=["one-launch-32-chunks", "two-launches"])
def test_decode_short_kernel_edge(keys):
    """bf16 steps of at most 32 chunks of 128 keys run as one launch of the
    short-history kernel; a key more and they run on the LDS-streamed kernel
    (append, stream, merge): the step whose longest history makes
    max_len_hint + 1 = 4096 keys and the one a key longer, three steps each,
    against the oracle."""
    steps = 3
    lens = [keys - steps, 1, 4000]
    Hq, Hkv, d, w = 8, 2, 128, 128
    dtype = torch.bfloat16
    say(f"decode split-count edge keys={keys}")
    xc, cap = small_decode_inputs(len(lens), Hq, Hkv, d, dtype, lens, steps, seed=27 + keys)
    cfg = dict(batch=len(lens), n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=w, dtype=dtype)
    x = to_dev(xc)
    hint = max(lens) + steps - 1
    assert hint + 1 == keys
    dec = Decode(cfg, x["k_cache"], x["v_cache"], x["cache_len"], hint, x["alpha"], x["beta"],
                 x["alpha_out"], x["beta_out"])
    kc, vc, lc = xc["k_cache"].clone(), xc["v_cache"].clone(), xc["cache_len"].clone()
    for s in range(steps):
        dec.step(x["q"][s], x["q_out"][s], x["k_new"][s], x["v_new"][s])
        torch.cuda.synchronize()
        o, o_out = oracle.decode_step(xc["q"][s], xc["q_out"][s], xc["k_new"][s], xc["v_new"][s], xc["alpha"],
                                      xc["beta"], xc["alpha_out"], xc["beta_out"], w, kc, vc, lc)
        assert_parity(dec.o, o, dtype, f"o step {s}")
        assert_parity(dec.o_out, o_out, dtype, f"o_out step {s}")
    assert torch.equal(dec.cache_len.cpu(), lc)
    assert torch.equal(bits(dec.k_cache.cpu()), bits(kc))
    assert torch.equal(bits(dec.v_cache.cpu()), bits(vc))


@pytest.mark.parametrize("B,Hq,len_lo,len_hi,steps,w", [(32, 32, 66000, 70000, 2, 128),
                                                      (80, 32, 20000, 24000, 1, 128),
                                                      (32, 32, 66000, 70000, 1, 5000),
                                                      (16, 64, 66000, 70000, 1, 128),
                                                      (80, 16, 20000, 24000, 1, 128),
                                                      (80, 8, 20000, 24000, 2, 300)],
                         ids=["B32-70K", "B80-24K-two-launches", "B32-70K-window-5000",
                              "B16-70K-G8-two-head-blocks", "B80-24K-G2-two-launches",
                              "B80-24K-MHA-two-launches-w300"])
def test_decode_lds_kernel_long_histories(B, Hq, len_lo, len_hi, steps, w):
    """bf16, 8 KV heads, d128: 32 sequences (32 query heads) with histories
    up to 70K keys, 16 with 64 query heads (two 4-head blocks per KV head),
    or 80 (two launches of 64 and 16 sequences) up to 24K, with groups of 4,
    2 (2-head streams) and 1 -- large enough that the step runs on the
    LDS-streamed kernel (equal runs of the step's keys per workgroup).  Lengths include 0 and the edges of a 128-key
    stage; windows of 128 and 5000 keys.  Unused cache slots hold the NaN
    sentinel, and one sequence's length is past the hint.  Every step
    against the oracle, caches and lengths in full."""
    Hkv, d = 8, 128
    cfg = dict(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=w, dtype=torch.bfloat16,
               len_lo=len_lo, len_hi=len_hi, steps=steps)
    say("decode lds long histories: generate")
    x = inputs.decode_inputs(seed=31, device="cuda", **cfg)
    edges = [0, 1, 127, 128, 4095, 4096, 4100, 8191, len_lo - 1, len_lo]
    lens = x["cache_len"].clone()
    lens[:len(edges)] = torch.tensor(edges, dtype=torch.int32, device="cuda")
    slot = torch.arange(x["cap"], device="cuda")
    unused = (slot[None, :] >= lens[:, None].long())[:, None, :].expand(B, Hkv, x["cap"])
    inputs.fill_sentinel(x["k_cache"], unused)
    inputs.fill_sentinel(x["v_cache"], unused)
    # sequence 10 is past the hint: NaN outputs, its cache and length untouched
    big = 10
    max_hint = int(torch.cat([lens[:big], lens[big + 1:]]).max()) + steps - 1
    lens[big] = max_hint + 1
    x["cache_len"] = lens
    xc = to_cpu(x)
    dec = Decode(cfg, x["k_cache"], x["v_cache"], x["cache_len"], max_hint, x["alpha"], x["beta"],
                 x["alpha_out"], x["beta_out"])
    from phase_aware_swa_amd import binding
    from phase_aware_swa_amd.runner import desc_for
    # the LDS-streamed kernel's workspace (at least 12 * 2^20 keys over all
    # streams): counters, lengths, 3 record ids per stream, then 2 x 4
    # records of d + 32 floats per id (every stream of a launch of up to 64
    # sequences, plus 512)
    G = Hq // Hkv
    S = Hkv * (G // (4 if G % 4 == 0 else 2 if G % 2 == 0 else 1))
    assert (max_hint + 1) * B * S >= 12 << 20
    len_bytes = -(-B * 4 // 256) * 256         # the per-sequence lengths, 256-byte aligned
    cnt_bytes = -(-B * (S + 1) * 4 // 256) * 256     # arrival counters
    rng_bytes = -(-B * S * 3 * 4 // 256) * 256
    ids = -(-B // 64) * (min(B, 64) * S + 512)
    assert binding.decode_workspace_size(desc_for(cfg), max_hint) == (cnt_bytes + len_bytes + rng_bytes +
                                                                      ids * 2 * 4 * (d + 32) * 4)
    kc, vc, lc = xc["k_cache"], xc["v_cache"], xc["cache_len"].clone()
    for s in range(steps):
        say(f"decode lds long histories: step {s}")
        dec.step(x["q"][s], x["q_out"][s], x["k_new"][s], x["v_new"][s])
        torch.cuda.synchronize()
        keep = [t_[big].clone() for t_ in (kc, vc, lc)]
        lc[big] = 0          # the oracle steps it from an empty history; restored below
        o, o_out = oracle.decode_step(xc["q"][s], xc["q_out"][s], xc["k_new"][s], xc["v_new"][s], xc["alpha"],
                                      xc["beta"], xc["alpha_out"], xc["beta_out"], w, kc, vc, lc)
        kc[big], vc[big], lc[big] = keep
        ok = torch.arange(B) != big
        assert_parity(dec.o[ok], o[ok], torch.bfloat16, f"o step {s}")
        assert_parity(dec.o_out[ok], o_out[ok], torch.bfloat16, f"o_out step {s}")
        assert torch.isnan(dec.o[big].float()).all() and torch.isnan(dec.o_out[big].float()).all()
    assert torch.equal(dec.cache_len.cpu(), lc)
    assert torch.equal(bits(dec.k_cache.cpu()), bits(kc))
    assert torch.equal(bits(dec.v_cache.cpu()), bits(vc))


@pytest.mark.parametrize("Hq", [4, 8], ids=["G2", "G4"])
def test_decode_length_beyond_hint_is_left_alone(Hq):
    """A sequence whose length exceeds max_len_hint gets NaN outputs, no cache
    write and no length update; the others step normally."""
    lens = [10, 60]
    xc, cap = small_decode_inputs(2, Hq, 2, 128, torch.bfloat16, lens, 1, seed=22)
    cfg = dict(batch=2, n_q_heads=Hq, n_kv_heads=2, head_dim=128, window=128, dtype=torch.bfloat16)
    say(f"decode beyond hint Hq={Hq}")
    x = to_dev(xc)
    dec = Decode(cfg, x["k_cache"], x["v_cache"], x["cache_len"], 40, x["alpha"], x["beta"], x["alpha_out"],
                 x["beta_out"])
    before = x["k_cache"].clone()
    dec.step(x["q"][0], x["q_out"][0], x["k_new"][0], x["v_new"][0])
    torch.cuda.synchronize()
    assert dec.cache_len.cpu().tolist() == [11, 60]
    assert torch.isnan(dec.o[1].float()).all() and torch.isnan(dec.o_out[1].float()).all()
    assert torch.isfinite(dec.o[0].float()).all()
    assert torch.equal(bits(dec.k_cache[1]), bits(before[1]))


def test_decode_resume_from_host_copy():
    """The cache and lengths are the whole state: n steps, a round trip of the
    state through host memory, then n more steps gives the bits of 2n
    straight steps."""
    lens = [100, 2000, 4097]
    n = 6
    xc, cap = small_decode_inputs(3, 8, 2, 128, torch.bfloat16, lens, 2 * n, seed=23)
    cfg = dict(batch=3, n_q_heads=8, n_kv_heads=2, head_dim=128, window=128, dtype=torch.bfloat16)
    say("decode resume")
    outs = []
    for resume in (False, True):
        x = to_dev(xc)
        dec = Decode(cfg, x["k_cache"], x["v_cache"], x["cache_len"], max(lens) + 2 * n, x["alpha"], x["beta"],
                     x["alpha_out"], x["beta_out"])
        o_all = []
        for s in range(2 * n):
            if resume and s == n:
                torch.cuda.synchronize()
                k_h, v_h, l_h = dec.k_cache.cpu(), dec.v_cache.cpu(), dec.cache_len.cpu()
                dec.k_cache.copy_(torch.zeros_like(dec.k_cache))
                dec.k_cache.copy_(k_h.cuda())
                dec.v_cache.copy_(v_h.cuda())
                dec.cache_len.copy_(l_h.cuda())
            dec.step(x["q"][s], x["q_out"][s], x["k_new"][s], x["v_new"][s])
            o_all.append((dec.o.clone(), dec.o_out.clone()))
        torch.cuda.synchronize()
        outs.append((o_all, dec.k_cache.clone(), dec.cache_len.clone()))
    (a, ka, la), (b, kb, lb) = outs
    assert torch.equal(la, lb) and torch.equal(bits(ka), bits(kb))
    for (o1, oo1), (o2, oo2) in zip(a, b):
        assert torch.equal(bits(o1), bits(o2)) and torch.equal(bits(oo1), bits(oo2))


def test_walkthrough_prefill_then_decode_gpu():
    """prefill([A..C]) with its copy at C, then one decode step with D / D',
    against prefill([A..D]) with its copy at D: the same cache bytes; the
    base output at D and the copy's output within the parity bar."""
    T = 700
    cfg = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, window=128, dtype=torch.bfloat16)
    say("walkthrough gpu")
    xc = inputs.prefill_inputs(T=T, seed=24, **cfg)
    x = to_dev(xc)
    full = Prefill(cfg, x, cap=T + 8)
    full.run()
    part_x = {k: (v[:, : T - 1].contiguous() if k in ("q", "k", "v") else v) for k, v in x.items()}
    part_x["out_pos"] = [T - 2, T - 2]
    part = Prefill(cfg, part_x, cap=T + 8)
    part.run()
    lens = torch.full((2,), T - 1, dtype=torch.int32, device="cuda")
    dec = Decode(cfg, part.k_cache, part.v_cache, lens, T - 1, x["alpha"], x["beta"], x["alpha_out"],
                 x["beta_out"])
    dec.step(x["q"][:, T - 1].contiguous(), x["q_out"], x["k"][:, T - 1].contiguous(),
             x["v"][:, T - 1].contiguous())
    torch.cuda.synchronize()
    assert torch.equal(bits(part.k_cache), bits(full.k_cache))
    assert torch.equal(bits(part.v_cache), bits(full.v_cache))
    assert lens.cpu().tolist() == [T, T]
    ref_o = full.o[:, T - 1].cpu().double()
    assert_parity(dec.o, ref_o, torch.bfloat16, "base output at D")
    assert_parity(dec.o_out, full.o_out.cpu().double(), torch.bfloat16, "copy output at D'")
