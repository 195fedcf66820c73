"""Bit-exact mask placement on every kernel that serves the bf16 workloads
("Orthros:阶段感知异构注意力精读笔记" §2.3: the window W_t of Eq. (4) and
the copy's j <= t of Eq. (5); §2.4: the copy is masked by its original
position, not by its slot).

alpha = beta = alpha' = beta' = 0 makes every score zero, so each output is
the plain mean of V over the admissible keys.  V rows are one-hot: key j of
(sequence b, KV head g) marks column (j + s_bg) mod 127, with a shift s_bg
that differs between sequences and KV heads (a stream mix-up moves the
pattern).  Every output element is then count / |S| for the key set S
of its row, compared bit for bit (tests/probe_util.py).  Kernels covered:

  prefill, fused streaming kernel (groups of 4 and 8 query heads, w <= 129,
    d 128 and 64), copies on segment edges and below T-1;
  prefill, the fused streaming kernel for groups of 1, 2, 3 and 6
    (w <= 129: blocks of 2 heads, or of 1 with the head dims split);
  prefill, generic sliding-window kernel + LDS-streamed cross-attention
    (w > 129, groups of 4; and groups of 2 and 1), and
    orthros_global_xattn on its own;
  decode, LDS-streamed kernel (32 sequences; each workgroup takes an equal
    run of the step's keys, in (sequence, KV head, key) order): the base
    token's window straddling run boundaries at w = 128 and spanning several
    runs at w = 4096 and 5000, and the copy over ~64K-key histories with
    marked keys on both sides of every run boundary;
  decode, one-launch short-history kernel (groups of 1, 2, 3, 4 and 8,
    d 128 and 64, windows 1, 128 and 300), and the LDS-streamed kernel past
    4096 keys with groups of 1, 2 and 3 and d = 64.
(MI355X only.)"""
import pytest
import torch

from gpu_util import bits, say
from phase_aware_swa_amd import inputs
from phase_aware_swa_amd.runner import Decode, Prefill
from probe_util import assert_probe, marker, residue_counts

pytestmark = pytest.mark.gpu

M = 127
BF16 = torch.bfloat16


def shifts(B, Hkv):
    b = torch.arange(B)[:, None]
    g = torch.arange(Hkv)[None, :]
    return (5 * b + 17 * g) % M                                     # [B, Hkv]


def zero_scale_offset(x):
    for k in ("alpha", "beta", "alpha_out", "beta_out"):
        x[k] = torch.zeros_like(x[k])


def onehot_rows(cols, d, dtype=BF16):
    """[..., d] rows with a 1 at cols (where cols < d), else 0."""
    v = torch.zeros(*cols.shape, d + 1, dtype=dtype, device=cols.device)
    v.scatter_(-1, cols.clamp(max=d)[..., None], 1.0)
    return v[..., :d].contiguous()


def decode_split_of(B, Hq, Hkv, d, hint):
    """(uses the LDS-streamed kernel, workspace bytes) of a bf16 decode step,
    from the split rule of orthros_decode_step: 128-key chunks when that
    makes at most 32 (the one-launch kernel, records of d + 4 floats, two
    kinds per query head); else the LDS-streamed kernel (record-id table,
    then 2 x 4 records of d + 32 floats per id: every stream -- a KV head's
    block of 4, 2 or 1 query heads -- of a launch of up to 64 sequences plus
    512) when the group is a multiple of 4, the keys over all streams reach
    3 x 2^19 or the history 2^16 keys; else the lane-parallel kernel
    (power-of-two chunks >= 256 keys for about 16384 workgroups, records of
    d + 2 floats); arrival counters and lengths first."""
    G = Hq // Hkv
    hpw = 4 if G % 4 == 0 else 2 if G % 2 == 0 else 1
    S = Hkv * (G // hpw)
    streams = B * S
    keys = hint + 1
    head = -(-B * (S + 1) * 4 // 256) * 256 + -(-B * 4 // 256) * 256
    if keys <= 32 * 128:
        n_split = -(-keys // 128)                # short steps: one launch over 128-key chunks
        return False, head + B * Hq * 2 * n_split * (d + 4) * 4
    if G % 4 == 0 or keys * streams >= 3 << 19 or keys >= 1 << 16:
        ids = -(-B // 64) * (min(B, 64) * S + 512)
        return True, head + -(-streams * 3 * 4 // 256) * 256 + ids * 2 * 4 * (d + 32) * 4
    chunk = 256
    while chunk < -(-keys * streams // 16384):
        chunk *= 2
    return False, head + B * Hq * 2 * -(-keys // chunk) * (d + 2) * 4


def lds_run_starts(lens, S, hint):
    """Where the LDS-streamed decode kernel's runs start, per (sequence,
    stream): the history keys 0 .. L - 1 of a step with cache lengths `lens`
    (the new key L is added by the merge) in (sequence, stream, key) order,
    cut into equal runs of E = max(ceil(total / grid), 256) keys, grid =
    min(CUs, 512, ceil(B * S * (hint + 1) / 256)).  Returns {(b, stream):
    [keys]}."""
    B = len(lens)
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    grid = max(1, min(ncu, 512, -(-B * S * (hint + 1) // 256)))
    total = sum(L * S for L in lens)
    E = max(-(-total // grid), 256)
    starts, P = {}, 0
    for b, L in enumerate(lens):
        for j in range(S):
            n = L
            first = -(-P // E) * E                      # the first run start at or after P
            starts[(b, j)] = list(range(first - P, n, E))
            P += n
    return starts


# ------------------------------------------------------------------ prefill

def prefill_probe(B, Hq, Hkv, d, w, T, out_pos, seed, stages=False):
    cfg = dict(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=w, dtype=BF16)
    say(f"prefill probe {cfg} T={T} out_pos={out_pos} stages={stages}")
    xc = inputs.prefill_inputs(T=T, seed=seed, **cfg)
    zero_scale_offset(xc)
    sh = shifts(B, Hkv)
    j = torch.arange(T)
    xc["v"] = onehot_rows(marker(j[None, :, None], sh[:, None, :], M), d)          # [B, T, Hkv, d]
    xc["out_pos"] = out_pos
    x = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in xc.items()}
    run = Prefill(cfg, x, cap=T + 16)
    if stages:
        run.run_swa()
        run.run_xattn()
    else:
        run.run()
    torch.cuda.synchronize()
    G = Hq // Hkv
    # base rows: key set [max(0, t-w+1), t] of KV head h // G
    t = torch.arange(T)
    lo = (t - w + 1).clamp(min=0)
    shp = (B, T, Hkv)
    cnt = residue_counts(lo[None, :, None].expand(shp), t[None, :, None].expand(shp), sh[:, None, :].expand(shp),
                         M, d)
    n = (t - lo + 1)[None, :, None].expand(shp)
    o = run.o.view(B, T, Hkv, G, d)
    und = assert_probe(o, cnt[:, :, :, None, :].expand(B, T, Hkv, G, d), n[..., None].expand(B, T, Hkv, G),
                       "o (base rows)")
    # copies: key set [0, out_pos[b]]
    P = torch.tensor(out_pos, dtype=torch.int64)
    cnt = residue_counts(torch.zeros(B, Hkv, dtype=torch.int64), P[:, None].expand(B, Hkv), sh, M, d)
    und += assert_probe(run.o_out.view(B, Hkv, G, d), cnt[:, :, None, :].expand(B, Hkv, G, d),
                        (P + 1)[:, None, None].expand(B, Hkv, G), "o_out (copies)")
    # the cache is still written byte for byte
    assert torch.equal(bits(run.v_cache[:, :, :T].cpu()), bits(xc["v"].transpose(1, 2).contiguous()))
    say(f"prefill probe ok ({und} elements next to a bf16 midpoint)")


# Fused streaming kernel at T = 4096, B8, groups of 4: 16 streams, 32
# segments of 128 keys, so copies at 127, 255, 1023, 2047 end a segment and
# 128, 256 start one.
def test_probe_fused_g4_segment_edges():
    prefill_probe(8, 8, 2, 128, 128, 4096, [127, 128, 255, 256, 1023, 2047, 3000, 4095], seed=301)


# Groups of 8 (two 4-head blocks per KV head), ragged T: 160-key segments.
def test_probe_fused_g8_ragged():
    prefill_probe(4, 16, 2, 128, 128, 4100, [0, 159, 160, 4099], seed=302)


@pytest.mark.parametrize("w", [1, 2, 64, 129])
def test_probe_fused_windows(w):
    prefill_probe(2, 8, 2, 128, w, 1500, [1499, 700], seed=303 + w)


def test_probe_fused_d64():
    prefill_probe(2, 8, 2, 64, 128, 3000, [2999, 31], seed=310)


# w > 129: the generic sliding-window kernel, then the LDS-streamed
# cross-attention kernel for the copy (groups of 4).
def test_probe_generic_swa_and_lds_xattn():
    prefill_probe(3, 8, 2, 128, 200, 3000, [2999, 1024, 255], seed=311)


# orthros_swa_prefill then orthros_global_xattn (LDS-streamed, groups of 4).
def test_probe_stages_lds_xattn():
    prefill_probe(4, 32, 8, 128, 128, 4096, [4095, 2048, 2047, 5], seed=312, stages=True)


# The fused streaming kernel for other groups: groups of 2 (a head a wave),
# 1 and 3 (the waves of a sub-tile split the head dims), 6 (three 2-head
# blocks per KV head); the copy's query on the first waves of the block.
@pytest.mark.parametrize("B,Hq,Hkv,d,w,T,pos", [(2, 4, 2, 128, 128, 1500, [1499, 999]),
                                                (2, 4, 4, 128, 128, 1500, [1499, 31]),
                                                (2, 2, 2, 64, 129, 1100, [1099, 640]),
                                                (2, 6, 2, 128, 100, 1000, [999, 128]),
                                                (1, 12, 2, 128, 128, 700, [699])],
                         ids=["G2", "G1", "G1-d64-w129", "G3-w100", "G6"])
def test_probe_streaming_other_groups(B, Hq, Hkv, d, w, T, pos):
    prefill_probe(B, Hq, Hkv, d, w, T, pos, seed=313 + Hq + d + w)


# Groups of 2 and 1 on the generic kernels (w > 129).
@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (4, 4)], ids=["G2", "G1"])
def test_probe_generic_g2_g1(Hq, Hkv):
    prefill_probe(2, Hq, Hkv, 128, 200, 1500, [1499, 999], seed=330 + Hq + Hkv)


@pytest.mark.parametrize("Hq,Hkv", [(4, 2), (8, 2), (16, 2), (4, 4), (6, 2)], ids=["G2", "G4", "G8", "G1", "G3"])
def test_window_one_and_first_position_exact(Hq, Hkv):
    """Random inputs.  w = 1: o = v exactly (one key, weight 1).  A copy at
    position 0 and base row 0 (w = 128) see key 0 alone: exactly v_0."""
    G = Hq // Hkv
    cfg = dict(batch=2, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=128, window=1, dtype=BF16)
    say(f"w=1 exactness Hq={Hq} Hkv={Hkv}")
    xc = inputs.prefill_inputs(T=300, seed=320 + G, **cfg)
    xc["out_pos"] = [0, 0]
    x = {k: (v.cuda() if torch.is_tensor(v) else v) for k, v in xc.items()}
    run = Prefill(cfg, x)
    run.run()
    torch.cuda.synchronize()
    v = xc["v"].repeat_interleave(G, dim=2)
    assert torch.equal(bits(run.o.cpu()), bits(v))
    v0 = xc["v"][:, 0].repeat_interleave(G, dim=1).contiguous()
    assert torch.equal(bits(run.o_out.cpu()), bits(v0))
    cfg["window"] = 128
    run2 = Prefill(cfg, x)
    run2.run()
    torch.cuda.synchronize()
    assert torch.equal(bits(run2.o[:, 0].cpu()), bits(v0))
    assert torch.equal(bits(run2.o_out.cpu()), bits(v0))


# ------------------------------------------------------------------- decode

def decode_probe(B, Hq, Hkv, d, w, lens, steps, seed, marked=False, expect_lds=None, hint=None):
    """Decode steps from histories `lens` with one-hot V (every key, or in
    `marked` mode only keys 0 and 1, the two keys either side of every run
    boundary of the LDS-streamed kernel in any stream of the sequence at any
    step, and the last keys of the history up to the step's new key, each
    with a column of its own).  Every step's o and o_out against count / |S|;
    the caches and lengths byte for byte.  `hint` (max_len_hint) defaults to
    the longest history at the last step."""
    cfg = dict(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=w, dtype=BF16)
    say(f"decode probe {cfg} lens[:12]={lens[:12]} steps={steps} marked={marked}")
    lens_t = torch.tensor(lens, dtype=torch.int64)
    hint = int(lens_t.max()) + steps - 1 if hint is None else hint
    cap = max(int(lens_t.max()) + steps + 3, hint + 1)
    sh = shifts(B, Hkv)
    slot = torch.arange(cap)
    if marked:
        # column of each marked slot per sequence, -1 for unmarked (zero rows)
        col = torch.full((B, cap), -1, dtype=torch.int64)
        S = Hkv * (Hq // Hkv // 4)
        edges = [set() for _ in range(B)]
        for s in range(steps):
            for (b, j), ks in lds_run_starts([L + s for L in lens], S, hint).items():
                edges[b] |= {k + e for k in ks if k > 0 for e in (-1, 0)}
        for b, L in enumerate(lens):
            last = L + steps - 1                        # the last step's new key
            keys = {0, 1} | edges[b]
            assert len(keys) <= d - 16, "too many marked run edges for the columns"
            keys |= set(range(max(0, last - (d - 1 - len(keys)) + 1), last + 1))
            keys = sorted(k for k in keys if k <= last)[:d]
            for c, k in enumerate(keys):
                col[b, k] = c
        cols = col[:, None, :].expand(B, Hkv, cap).clone()
        cols[cols < 0] = d                               # d: no column (zero row)
    else:
        cols = marker(slot[None, None, :], sh[:, :, None], M).expand(B, Hkv, cap).clone()
    dev = "cuda"
    v_full = onehot_rows(cols.to(dev), d)                                          # [B, Hkv, cap, d]
    g = torch.Generator(device=dev).manual_seed(seed)
    k_full = torch.randn(B, Hkv, cap, d, generator=g, device=dev).to(BF16)
    # the history in the caches, the sentinel after it; the new keys come per step
    kc, vc = k_full.clone(), v_full.clone()
    unused = (slot.to(dev)[None, :] >= lens_t.to(dev)[:, None])[:, None, :].expand(B, Hkv, cap)
    inputs.fill_sentinel(kc, unused)
    inputs.fill_sentinel(vc, unused)
    q = torch.randn(steps, B, Hq, d, generator=g, device=dev).to(BF16)
    q_out = torch.randn(steps, B, Hq, d, generator=g, device=dev).to(BF16)
    z = torch.zeros(Hq, d, dtype=BF16, device=dev)
    clen = lens_t.to(torch.int32).to(dev)
    dec = Decode(cfg, kc, vc, clen, hint, z, z, z, z)
    if expect_lds is not None:
        from phase_aware_swa_amd import binding
        from phase_aware_swa_amd.runner import desc_for
        lds, ws = decode_split_of(B, Hq, Hkv, d, hint)
        assert lds == expect_lds
        assert binding.decode_workspace_size(desc_for(cfg), hint) == ws
    G = Hq // Hkv
    und = 0
    cols_c = cols
    for s in range(steps):
        L = lens_t + s                                                              # [B]
        ar, Ld = torch.arange(B, device=dev), L.to(dev)
        k_new = k_full[ar, :, Ld].contiguous()                                      # [B, Hkv, d]
        v_new = v_full[ar, :, Ld].contiguous()
        dec.step(q[s], q_out[s], k_new, v_new)
        torch.cuda.synchronize()
        # expected counts by brute force over the key sets (small d x sets)
        for kind, lo in (("o", (L - w + 1).clamp(min=0)), ("o_out", torch.zeros_like(L))):
            cnt = torch.zeros(B, Hkv, d, dtype=torch.int64)
            for b in range(B):
                cb = cols_c[b, :, lo[b]:L[b] + 1]                                    # [Hkv, n]
                for gg in range(Hkv):
                    c = cb[gg]
                    c = c[c < d]
                    cnt[b, gg] += torch.bincount(c, minlength=d)[:d]
            n = (L - lo + 1)[:, None, None].expand(B, Hkv, G)
            got = (dec.o if kind == "o" else dec.o_out).view(B, Hkv, G, d)
            und += assert_probe(got, cnt[:, :, None, :].expand(B, Hkv, G, d), n, f"{kind} step {s}")
    assert torch.equal(dec.cache_len.cpu(), (lens_t + steps).to(torch.int32))
    filled = (slot.to(dev)[None, :] < (lens_t + steps).to(dev)[:, None])[:, None, :].expand(B, Hkv, cap)
    ref_k, ref_v = k_full.clone(), v_full.clone()
    inputs.fill_sentinel(ref_k, ~filled)
    inputs.fill_sentinel(ref_v, ~filled)
    assert torch.equal(bits(dec.k_cache), bits(ref_k)) and torch.equal(bits(dec.v_cache), bits(ref_v))
    say(f"decode probe ok ({und} elements next to a bf16 midpoint)")


def lds_lens(B, base=65536):
    """Histories for the LDS-streamed decode kernel: edge lengths first, then
    the rest spread below base."""
    lens = [0, 1, 127, 128, 129, 255, 256, 4096 + 126]
    g = torch.Generator().manual_seed(B)
    while len(lens) < B:
        lens.append(int(torch.randint(8192, base, (1,), generator=g)))
    return lens[:B]


def straddling_windows(lens, S, hint, w):
    """(b, stream) pairs whose window's history keys [L - w + 1, L - 1] hold
    a run start past their first key at the first step."""
    out = []
    for (b, j), ks in lds_run_starts(lens, S, hint).items():
        lo = max(0, lens[b] - w + 1)
        if any(lo < k <= lens[b] - 1 for k in ks):
            out.append((b, j))
    return out


def test_probe_decode_lds_window_straddles_runs():
    """w = 128 on the LDS-streamed kernel with short histories (1-3K keys)
    under a large max_len_hint (the kernel is chosen by the hint): runs of a
    few thousand keys, so run boundaries fall inside many streams' windows;
    two steps (the second window holds the first step's appended key)."""
    g = torch.Generator().manual_seed(7)
    lens = [0, 1, 127, 128, 129] + [int(x) for x in torch.randint(1000, 3000, (27,), generator=g)]
    hint = 65535
    assert len(straddling_windows(lens, 8, hint, 128)) >= 8
    decode_probe(32, 32, 8, 128, 128, lens, 2, seed=330, expect_lds=True, hint=hint)


@pytest.mark.parametrize("w", [4096, 5000])
def test_probe_decode_lds_window_spans_runs(w):
    """Windows longer than a run (runs of ~2K keys): the base token's
    partials come from several workgroups."""
    g = torch.Generator().manual_seed(w)
    lens = [0, 1, 4095, 4096, 5000] + [int(x) for x in torch.randint(1000, 9000, (27,), generator=g)]
    hint = 65535
    assert len(straddling_windows(lens, 8, hint, w)) >= 32
    decode_probe(32, 32, 8, 128, w, lens, 1, seed=331, expect_lds=True, hint=hint)


def test_probe_decode_lds_copy_marked_run_edges():
    """The copy over ~64K keys: only keys 0, 1, both sides of every run
    boundary and the last keys carry a column, so a key dropped or doubled
    where one workgroup's run ends and the next begins, or a stray read past
    the new key (a NaN sentinel), changes the output."""
    lens = lds_lens(32)
    decode_probe(32, 32, 8, 128, 128, lens, 2, seed=332, marked=True, expect_lds=True)


@pytest.mark.parametrize("Hq,Hkv,d,w,longest,hint,lds",
                         [(8, 2, 128, 128, 4095, None, False), (8, 2, 128, 1, 4095, None, False),
                          (8, 2, 64, 300, 4095, None, False), (4, 2, 128, 128, 4095, None, False),
                          (16, 2, 128, 128, 4095, None, False), (4, 2, 128, 128, 9000, None, False),
                          (4, 2, 128, 128, 9000, 65535, True), (2, 2, 64, 128, 9000, 65535, True),
                          (8, 2, 64, 128, 9000, None, True), (4, 1, 128, 128, 4095, None, False),
                          (4, 1, 64, 300, 4095, None, False), (2, 1, 128, 1, 4095, None, False),
                          (1, 1, 128, 128, 4095, None, False), (6, 2, 128, 128, 4095, None, False),
                          (6, 2, 128, 300, 9000, 65535, True)],
                         ids=["G4", "G4-w1", "G4-d64-w300", "G2", "G8", "G2-lane", "G2-lds", "MHA-d64-lds",
                              "G4-d64-lds", "G4-Hkv1", "G4-d64-w300-Hkv1", "G2-w1-Hkv1", "MHA-Hkv1", "G3",
                              "G3-w300-lds"])
def test_probe_decode_short_kernel(Hq, Hkv, d, w, longest, hint, lds):
    """Short histories: lengths 0, 1, around the window, and on the edges of
    128- and 256-key chunks; three steps.  Up to 4096 keys the step is one
    launch of the short-history kernel (128-key chunks, merged in the
    launch; with one KV head, groups of 4, 2 and 1 give merges by one, two
    and four waves per head); with a 9000-key history it is the
    LDS-streamed kernel for
    groups of 4 (d = 64: 8 pairs per stage) and, for other groups, the
    lane-parallel kernel -- or the LDS-streamed one once max_len_hint + 1
    reaches 2^16 keys (2- and 1-head streams)."""
    lens = [0, 1, 126, 127, 128, 255, 256, 1000, longest]
    if longest == 4095:
        lens[-1] = 4093                          # keys = max_len_hint + 1 = 4096: the one-launch kernel
    decode_probe(len(lens), Hq, Hkv, d, w, lens, 3, seed=340 + w + d + Hq, expect_lds=lds, hint=hint)
