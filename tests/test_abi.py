"""The C-ABI library on the CPU: it loads, exports every symbol the header
declares, and rejects bad arguments with the documented status before any
HIP call (no GPU needed: validation never reaches the runtime)."""
import ctypes
import os
import re

import pytest

from phase_aware_swa_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "orthros.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(orthros_\w+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"orthros_prefill", "orthros_decode_step", "orthros_swa_prefill", "orthros_global_xattn",
            "orthros_copies"} <= set(names)
    lib = binding.lib()
    for n in names:
        assert hasattr(lib, n), f"{n} declared in orthros.h but not exported"


def test_abi_version_and_status_text():
    assert binding.abi_version() == 3
    text = open(HEADER).read()
    assert "#define ORTHROS_ABI_VERSION 3" in text
    for code, name in binding.STATUS.items():
        assert binding.status_str(code) == name
        assert re.search(rf"\b{name}\s*=\s*{code}\b", text) or code == 0


D = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, window=128, dtype=binding.BF16)
FAKE = 1 << 20   # aligned, never dereferenced: every call below fails validation first


def prefill_call(desc, T=100, cap=100, out_pos=(99, 99), ptr=FAKE, ws_bytes=1 << 30, ws=FAKE):
    pos = (ctypes.c_int64 * len(out_pos))(*out_pos)
    p = ctypes.c_void_p(ptr)
    return binding.lib().orthros_prefill(ctypes.byref(desc), T, p, p, pos, p, p, p, p, p, p, p, p, cap, p, p,
                                         ctypes.c_void_p(ws), ws_bytes, None)


def mk(**kw):
    d = dict(D)
    d.update(kw)
    return binding.Desc(d["batch"], d["n_q_heads"], d["n_kv_heads"], d["head_dim"], d["window"],
                        d.get("softmax_scale", 0.0), d["dtype"])


@pytest.mark.parametrize("change,status", [
    (dict(dtype=7), -3),
    (dict(batch=0), -2),
    (dict(n_q_heads=9), -2),
    (dict(head_dim=96), -2),
    (dict(window=0), -2),
    (dict(softmax_scale=-1.0), -2),
    (dict(softmax_scale=float("inf")), -2),
])
def test_bad_desc(change, status):
    assert prefill_call(mk(**change)) == status
    assert binding.lib().orthros_last_error()


def test_bad_call_arguments():
    d = mk()
    assert prefill_call(d, T=0) == -2
    assert prefill_call(d, T=100, cap=99) == -5
    assert prefill_call(d, out_pos=(99, 100)) == -4
    assert prefill_call(d, out_pos=(-1, 5)) == -4
    assert prefill_call(d, ptr=0) == -1
    assert prefill_call(d, ptr=FAKE + 8) == -8
    assert prefill_call(d, ws=0) == -6
    assert prefill_call(d, ws_bytes=16) == -6
    assert b"workspace" in binding.lib().orthros_last_error()
    n = None
    assert binding.lib().orthros_prefill(None, 100, n, n, n, n, n, n, n, n, n, n, n, 100, n, n, n, 0, n) == -1


def test_decode_bad_arguments():
    L = binding.lib()
    d = mk()
    p = ctypes.c_void_p(FAKE)
    call = lambda cap, hint, ws=FAKE, wsb=1 << 30: L.orthros_decode_step(
        ctypes.byref(d), p, p, p, p, p, p, p, p, p, p, cap, p, hint, p, p, ctypes.c_void_p(ws), wsb, None)
    assert call(cap=100, hint=100) == -5
    assert call(cap=100, hint=-1) == -2
    assert call(cap=100, hint=50, ws=0) == -6
    assert call(cap=100, hint=50, wsb=8) == -6


@pytest.mark.parametrize("B,Hq,Hkv,d,hint,kind", [(16, 32, 8, 128, 132095, "lds"), (4, 32, 8, 128, 32767, "lds"),
                                                 (1, 32, 8, 128, 4095, "short"), (1, 32, 8, 128, 4096, "lds"),
                                                 (80, 32, 8, 128, 24575, "lds"), (8, 16, 8, 128, 32767, "lds"),
                                                 (4, 16, 8, 128, 32767, "lane16"), (4, 16, 8, 128, 65535, "lds"),
                                                 (11, 32, 8, 64, 131071, "lds"), (3, 16, 8, 64, 4095, "short"),
                                                 (5, 8, 8, 128, 65535, "lds"), (5, 8, 8, 128, 9000, "lane16"),
                                                 (4, 32, 8, 128, 32767, "lane"), (3, 16, 8, 64, 4095, "lane")],
                         ids=["B16-128K-lds", "B4-32K-lds", "B1-4K-short", "B1-4K-plus-one-lds",
                              "B80-24K-lds-two-launches", "B8-32K-G2-lds", "B4-32K-G2-bf16-lane", "B4-64K-G2-lds",
                              "B11-128K-d64-lds", "B3-4K-G2-d64-short", "B5-64K-MHA-lds", "B5-9K-MHA-bf16-lane",
                              "B4-32K-f32-lane", "B3-4K-G2-d64-f32-lane"])
def test_decode_workspace_layout(B, Hq, Hkv, d, hint, kind):
    """The decode workspace: 256-byte-aligned arrival counters and lengths,
    then the partials.  bf16 steps of at most 32 chunks of 128 keys run on
    the one-launch short kernel (two kinds of records of d + 4 floats per
    chunk and query head); longer bf16 ones on the LDS-streamed kernel (a
    256-byte-aligned table of 3 record ids per stream -- a stream being a
    KV head's block of 4, 2 or 1 query heads -- then 2 kinds x 4 head slots
    x (d + 32) floats per id, ids for every stream of a launch of up to 64
    sequences plus one per workgroup, 512 at most) when the group is a
    multiple of 4, the keys over all streams reach 3 x 2^19 or the history 2^16
    keys; the rest (fp32 among them) on the lane kernel (power-of-two
    chunks >= 256 keys for about 16384 workgroups, two kinds of records of
    d + 2 floats per chunk and query head).  A workspace one byte short is
    rejected before anything runs."""
    dt = binding.F32 if kind == "lane" else binding.BF16
    desc = mk(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=128, dtype=dt)
    keys, G = hint + 1, Hq // Hkv
    S = Hkv * (G // (4 if G % 4 == 0 else 2 if G % 2 == 0 else 1))
    streams = B * S
    counters = -(-B * (S + 1) * 4 // 256) * 256      # one per head block, one per sequence
    lens = -(-B * 4 // 256) * 256
    if kind == "lds":
        ids = -(-B // 64) * (min(B, 64) * S + 512)
        need = counters + lens + -(-streams * 3 * 4 // 256) * 256 + ids * 2 * 4 * (d + 32) * 4
    else:
        if kind == "short":
            assert keys <= 32 * 128
            chunk, rec = 128, d + 4
        else:
            chunk, rec = 256, d + 2
            while chunk < -(-keys * streams // 16384):
                chunk *= 2
        n_split = -(-keys // chunk)
        need = counters + lens + B * Hq * 2 * n_split * rec * 4
    assert binding.decode_workspace_size(desc, hint) == need
    p = ctypes.c_void_p(FAKE)
    st = binding.lib().orthros_decode_step(ctypes.byref(desc), p, p, p, p, p, p, p, p, p, p, hint + 1, p, hint, p, p,
                                           p, need - 1, None)
    assert st == -6


def test_prefill_workspace_layout():
    """The prefill workspace of the separate cross-attention (orthros_global_xattn).
    On the LDS-streamed kernel -- bf16 groups that are multiples of 4, and
    other bf16 groups once the copies read at least 2^20 keys over all
    streams -- lengths, the record-id table (3 per stream), then records of 4
    head slots x (d + 32) floats for every stream of a launch of up to 64
    sequences plus 512, independent of T; else lengths and partials of
    d + 2 floats per power-of-two chunk (>= 256 keys, about 2048 workgroups)
    and query head.  (The fused prefill, window <= 129, may need more: its
    size is the larger; window 200 here.)"""
    for B, Hq, Hkv, d in ((2, 32, 8, 128), (70, 16, 2, 64), (3, 8, 4, 128), (2, 16, 16, 128)):
        desc = mk(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d, window=200, dtype=binding.BF16)
        G = Hq // Hkv
        S = Hkv * (G // (4 if G % 4 == 0 else 2 if G % 2 == 0 else 1))
        lens = -(-B * 4 // 256) * 256
        for T in (1000, 131072):
            if G % 4 == 0 or T * B * S >= 1 << 20:
                ids = -(-B // 64) * (min(B, 64) * S + 512)
                need = lens + -(-B * S * 3 * 4 // 256) * 256 + ids * 4 * (d + 32) * 4
            else:
                chunk = 256
                while chunk < -(-T * B * S // 2048):
                    chunk *= 2
                need = lens + B * Hq * -(-T // chunk) * (d + 2) * 4
            assert binding.prefill_workspace_size(desc, T) == need, (B, Hq, Hkv, d, T)


def test_workspace_sizes():
    d = mk()
    w1 = binding.prefill_workspace_size(d, 1000)
    w2 = binding.prefill_workspace_size(d, 131072)
    assert 0 < w1 <= w2
    assert binding.prefill_workspace_size(mk(head_dim=5), 100) == 0
    assert binding.prefill_workspace_size(d, 0) == 0
    assert 0 < binding.decode_workspace_size(d, 10) <= binding.decode_workspace_size(d, 100000)
    assert binding.decode_workspace_size(d, -1) == 0


def copies_call(desc, T=100, T_out=4, cap=100, ptr=FAKE, pos=FAKE):
    p = ctypes.c_void_p(ptr)
    return binding.lib().orthros_copies(ctypes.byref(desc), T, T_out, p, ctypes.c_void_p(pos), p, p, p, p, cap,
                                        p, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T_out=0), -2),
    (dict(T=0), -2),
    (dict(cap=50), -5),
    (dict(ptr=0), -1),
    (dict(pos=0), -1),
    (dict(ptr=FAKE + 8), -8),
    (dict(pos=FAKE + 2), -8),
])
def test_copies_rejects_bad_arguments(kw, status):
    assert copies_call(mk(), **kw) == status
    assert binding.lib().orthros_last_error().decode()


def test_copies_rejects_bad_desc():
    assert copies_call(mk(dtype=5)) == -3
    assert copies_call(mk(head_dim=96)) == -2


def project_call(desc, T=100, T_out=2, d_model=256, cap=100, ptr=FAKE, x_out=FAKE, q_out=FAKE, alpha=FAKE,
                 beta=FAKE, alpha_out=FAKE, beta_out=FAKE):
    p = ctypes.c_void_p(ptr)
    v = ctypes.c_void_p
    return binding.lib().orthros_project(ctypes.byref(desc), T, T_out, d_model, p, v(x_out), p, p, p, v(alpha),
                                         v(beta), v(alpha_out), v(beta_out), p, v(q_out), p, p, cap, None)


@pytest.mark.parametrize("kw,status", [
    (dict(T=0), -2),
    (dict(T_out=-1), -2),
    (dict(cap=50), -5),
    (dict(d_model=0), -2),
    (dict(d_model=100), -2),          # not a multiple of 32
    (dict(d_model=65536 + 32), -2),
    (dict(ptr=0), -1),
    (dict(x_out=0), -1),              # T_out > 0 needs the copy rows
    (dict(q_out=0), -1),
    (dict(alpha=0), -1),              # alpha without beta
    (dict(beta_out=0), -1),
    (dict(ptr=FAKE + 8), -8),
    (dict(alpha=FAKE + 4, beta=FAKE + 4), -8),
])
def test_project_rejects_bad_arguments(kw, status):
    assert project_call(mk(), **kw) == status
    assert binding.lib().orthros_last_error().decode()


def test_project_rejects_bad_desc():
    assert project_call(mk(dtype=0)) == -3              # fp32: the projection is bf16 only
    assert project_call(mk(dtype=9)) == -3
    assert project_call(mk(n_q_heads=2, n_kv_heads=1, head_dim=64)) == -2    # Hq * d = 128 but Hkv * d = 64


def test_project_accepts_optional_pointers():
    """T_out = 0 with NULL copy rows, and NULL scale-offsets, pass the pointer
    checks: a later check (alignment) is the one that fails, so nothing is
    ever launched on these fake pointers."""
    assert project_call(mk(), T_out=0, x_out=0, q_out=0, alpha=FAKE + 4, beta=FAKE + 4) == -8
    assert project_call(mk(), alpha=0, beta=0, alpha_out=FAKE + 4, beta_out=FAKE + 4) == -8


def test_decode_noalloc_rejects_without_touching_the_gpu():
    """The allocation-free decode step validates like orthros_decode_step and
    refuses a step whose partials exceed its 64 MiB scratch array, before
    any HIP call (so this runs without a GPU)."""
    L = binding.lib()
    p = ctypes.c_void_p(FAKE)
    call = lambda d, cap, hint: L.orthros_decode_step_noalloc(ctypes.byref(d), p, p, p, p, p, p, p, p, p, p, cap, p,
                                                              hint, p, p, None)
    d = mk()
    assert call(d, cap=100, hint=100) == -5
    assert call(d, cap=100, hint=-1) == -2
    assert call(mk(head_dim=96), cap=100, hint=50) == -2
    big = mk(batch=2048, n_q_heads=32, n_kv_heads=8, head_dim=128)      # 2048 sequences of 1K keys
    hint = 1000
    assert binding.decode_workspace_size(big, hint) > 64 << 20
    assert call(big, cap=hint + 1, hint=hint) == -6
    assert b"scratch" in L.orthros_last_error()
    # the 1024-step batch-16 workload (128K-key histories) fits, and so does batch 64
    for B in (16, 64):
        assert binding.decode_workspace_size(mk(batch=B, n_q_heads=32, n_kv_heads=8, head_dim=128),
                                             131072 + 1023) <= 64 << 20
