"""Seeded synthetic inputs for the Orthros attention step.

This module only draws random tensors of the right shapes, value
distributions and structure.  It holds none of the method's arithmetic: no
scale-offset, no attention, no masking.  Both the GPU path (tests, bench)
and the CPU oracle (tests) consume the tensors it returns.

Workloads (the shapes the pages' measurements are run at; values N(0,1)):

  tiny_fp32_prefill      fp32, B1, 4/4 heads, d64, T2048, w128  (parity only)
  mha_1p3b_prefill_8k    bf16, B1, 16/16 heads (MHA), d128, T8192, w128
  gqa_8b_prefill_128k    bf16, B2, 32/8 heads (GQA), d128, T131072, w128,
                         one planted "needle" key per (sequence, KV head)
  gqa_8b_prefill_1m      bf16, B1, 32/8, d128, T1048576, w128, 36 layers
  gqa_8b_decode_b16      bf16, B16, 32/8, d128, w128, cache lengths
                         uniform in [8192, 131072], 1024 decode steps

Draw order for one prefill call: q, q_out, k, v, alpha, beta, alpha_out,
beta_out, then (needle workloads) the needle positions.  alpha ~ 1 + 0.1 N,
beta ~ 0.1 N.  Values are drawn in fp32 and rounded to the storage type.
"""
import torch

WORKLOADS = {
    "tiny_fp32_prefill": dict(kind="prefill", dtype=torch.float32, batch=1, n_q_heads=4,
                              n_kv_heads=4, head_dim=64, T=2048, window=128),
    "mha_1p3b_prefill_8k": dict(kind="prefill", dtype=torch.bfloat16, batch=1, n_q_heads=16,
                                n_kv_heads=16, head_dim=128, T=8192, window=128),
    "gqa_8b_prefill_128k": dict(kind="prefill", dtype=torch.bfloat16, batch=2, n_q_heads=32,
                                n_kv_heads=8, head_dim=128, T=131072, window=128, needle=True),
    "gqa_8b_prefill_1m": dict(kind="prefill", dtype=torch.bfloat16, batch=1, n_q_heads=32,
                              n_kv_heads=8, head_dim=128, T=1048576, window=128, layers=36),
    "gqa_8b_decode_b16": dict(kind="decode", dtype=torch.bfloat16, batch=16, n_q_heads=32,
                              n_kv_heads=8, head_dim=128, window=128, len_lo=8192,
                              len_hi=131072, steps=1024),
    # output copies at many positions (the SFT and PT modes): an answer span
    # of 4096 copies after a 28K prompt, and every position of a 16K sequence
    "gqa_8b_sft_32k": dict(kind="copies", dtype=torch.bfloat16, batch=2, n_q_heads=32, n_kv_heads=8,
                           head_dim=128, T=32768, T_out=4096, window=128),
    "gqa_8b_pt_16k": dict(kind="copies", dtype=torch.bfloat16, batch=1, n_q_heads=32, n_kv_heads=8,
                          head_dim=128, T=16384, T_out=16384, window=128),
    # decode over a stack of 36 resident layers with short histories, where
    # the per-layer step is short enough for launch overhead to matter
    "gqa_8b_decode_36l_b4": dict(kind="decode_layers", dtype=torch.bfloat16, batch=4, n_q_heads=32, n_kv_heads=8,
                                 head_dim=128, window=128, len_lo=8192, len_hi=32768, steps=64, layers=36),
    "gqa_8b_decode_36l_b1_short": dict(kind="decode_layers", dtype=torch.bfloat16, batch=1, n_q_heads=32,
                                       n_kv_heads=8, head_dim=128, window=128, len_lo=1024, len_hi=4096, steps=64,
                                       layers=36),
    # the projections either side of the 8B-class layer's attention (d_model
    # 4096) over the 128K prefill: X of both sequences, one copy row each
    "gqa_8b_project_128k": dict(kind="project", dtype=torch.bfloat16, batch=2, n_q_heads=32, n_kv_heads=8,
                                head_dim=128, T=131072, T_out=1, d_model=4096, window=128),
}

# A bf16 NaN bit pattern written into cache slots that must never be read or
# written; any read of one poisons the output, any write changes the bytes.
SENTINEL_BF16_BITS = 0x7FC1


def _gen(seed, device):
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def _normal(shape, g, device, dtype, mean=0.0, std=1.0):
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x.mul_(std)
    if mean != 0.0:
        x.add_(mean)
    return x.to(dtype)


def prefill_inputs(batch, n_q_heads, n_kv_heads, head_dim, T, dtype, seed,
                   device="cpu", needle=False, **_):
    """Tensors for one prefill call (one layer).

    q [B,T,Hq,d]: the base stream's projected queries; q_out [B,Hq,d]: the
    output copy's projected query; k, v [B,T,Hkv,d]; alpha, beta, alpha_out,
    beta_out [Hq,d]; out_pos: list of B ints, the copy's original position
    (T-1, the last prompt token).

    needle=True plants one key per (sequence, KV head g): at a uniformly
    drawn position p, k[b,p,g] is set to 4x the output copy's projected query
    of the group's first head, q_out[b, g*G] (read as the raw projection;
    with alpha' ~ 1 and beta' ~ 0 that key dominates the copy's softmax).
    V is left as drawn.
    """
    g = _gen(seed, device)
    B, Hq, Hkv, d = batch, n_q_heads, n_kv_heads, head_dim
    x = {}
    x["q"] = _normal((B, T, Hq, d), g, device, dtype)
    x["q_out"] = _normal((B, Hq, d), g, device, dtype)
    x["k"] = _normal((B, T, Hkv, d), g, device, dtype)
    x["v"] = _normal((B, T, Hkv, d), g, device, dtype)
    x["alpha"] = _normal((Hq, d), g, device, dtype, mean=1.0, std=0.1)
    x["beta"] = _normal((Hq, d), g, device, dtype, std=0.1)
    x["alpha_out"] = _normal((Hq, d), g, device, dtype, mean=1.0, std=0.1)
    x["beta_out"] = _normal((Hq, d), g, device, dtype, std=0.1)
    x["out_pos"] = [T - 1] * B
    if needle:
        G = Hq // Hkv
        pos = torch.randint(0, T, (B, Hkv), generator=g, device=device)
        for b in range(B):
            for kv in range(Hkv):
                x["k"][b, pos[b, kv], kv] = x["q_out"][b, kv * G] * 4
        x["needle_pos"] = pos.cpu()
    return x


def copies_inputs(batch, n_q_heads, head_dim, T, T_out, dtype, seed, device="cpu", positions="tail"):
    """The output copies of the PT / SFT modes: raw projected copy queries
    q_out [B,T_out,Hq,d] ~ N(0,1) and their original positions pos
    [B,T_out] (int32).  positions="tail": the last T_out positions in
    order (an SFT answer span; T_out = T is PT); "random": uniform draws
    over [0, T), unsorted, repeats allowed."""
    g = _gen(seed, device)
    q_out = _normal((batch, T_out, n_q_heads, head_dim), g, device, dtype)
    if positions == "tail":
        pos = torch.arange(T - T_out, T, device=device, dtype=torch.int32).repeat(batch, 1)
    else:
        pos = torch.randint(0, T, (batch, T_out), generator=g, device=device).to(torch.int32)
    return q_out, pos.contiguous()


def project_inputs(batch, n_q_heads, n_kv_heads, head_dim, T, T_out, d_model, seed, device="cpu",
                   dtype=torch.bfloat16, **_):
    """Inputs of the projections: x [B,T,d_model] and x_out [B,T_out,d_model]
    ~ N(0,1); w_q [Hq*d, d_model], w_k, w_v [Hkv*d, d_model] ~ N(0, 1/d_model)
    (so each projected value is ~ N(0,1)); alpha, alpha_out ~ 1 + 0.1 N,
    beta, beta_out ~ 0.1 N, each [Hq, d].  Drawn in this order."""
    g = _gen(seed, device)
    B, Hq, Hkv, d = batch, n_q_heads, n_kv_heads, head_dim
    s = d_model ** -0.5
    x = {}
    x["x"] = _normal((B, T, d_model), g, device, dtype)
    x["x_out"] = _normal((B, T_out, d_model), g, device, dtype)
    x["w_q"] = _normal((Hq * d, d_model), g, device, dtype, std=s)
    x["w_k"] = _normal((Hkv * d, d_model), g, device, dtype, std=s)
    x["w_v"] = _normal((Hkv * d, d_model), g, device, dtype, std=s)
    x["alpha"] = _normal((Hq, d), g, device, dtype, mean=1.0, std=0.1)
    x["beta"] = _normal((Hq, d), g, device, dtype, std=0.1)
    x["alpha_out"] = _normal((Hq, d), g, device, dtype, mean=1.0, std=0.1)
    x["beta_out"] = _normal((Hq, d), g, device, dtype, std=0.1)
    return x


def decode_inputs(batch, n_q_heads, n_kv_heads, head_dim, dtype, seed, steps,
                  len_lo, len_hi, device="cpu", **_):
    """Tensors for a run of decode steps.

    cache_len [B] int32 ~ U{len_lo..len_hi}; cap = max(cache_len) + steps;
    k_cache, v_cache [B,Hkv,cap,d] hold N(0,1) in slots [0, len_b) and the
    sentinel bit pattern in every later slot.  Per step s: q[s], q_out[s]
    [B,Hq,d], k_new[s], v_new[s] [B,Hkv,d].  alpha..beta_out [Hq,d].
    """
    g = _gen(seed, device)
    B, Hq, Hkv, d = batch, n_q_heads, n_kv_heads, head_dim
    x = {}
    lens = torch.randint(len_lo, len_hi + 1, (B,), generator=g, device=device)
    cap = int(lens.max().item()) + steps
    x["cache_len"] = lens.to(torch.int32)
    x["cap"] = cap
    for name in ("k_cache", "v_cache"):
        c = _normal((B, Hkv, cap, d), g, device, dtype)
        slot = torch.arange(cap, device=device)
        unused = slot[None, :] >= lens[:, None]          # [B, cap]
        fill_sentinel(c, unused[:, None, :].expand(B, Hkv, cap))
        x[name] = c
    x["q"] = _normal((steps, B, Hq, d), g, device, dtype)
    x["q_out"] = _normal((steps, B, Hq, d), g, device, dtype)
    x["k_new"] = _normal((steps, B, Hkv, d), g, device, dtype)
    x["v_new"] = _normal((steps, B, Hkv, d), g, device, dtype)
    x["alpha"] = _normal((Hq, d), g, device, dtype, mean=1.0, std=0.1)
    x["beta"] = _normal((Hq, d), g, device, dtype, std=0.1)
    x["alpha_out"] = _normal((Hq, d), g, device, dtype, mean=1.0, std=0.1)
    x["beta_out"] = _normal((Hq, d), g, device, dtype, std=0.1)
    return x


def fill_sentinel(cache, where=None):
    """Writes the sentinel bit pattern into cache rows (bf16: a NaN; fp32: a NaN).

    where: bool tensor broadcastable to cache.shape[:-1], or None for all rows.
    """
    if cache.dtype == torch.bfloat16:
        bits = torch.tensor(SENTINEL_BF16_BITS, dtype=torch.int16)
        val = bits.view(torch.bfloat16).to(cache.device)
    else:
        val = torch.tensor(float("nan"), dtype=cache.dtype, device=cache.device)
    if where is None:
        cache.copy_(val.expand_as(cache))
    else:
        cache.masked_fill_(where[..., None], val)


def empty_cache(batch, n_kv_heads, cap, head_dim, dtype, device="cpu"):
    """A [B,Hkv,cap,d] cache with every slot holding the sentinel."""
    c = torch.empty(batch, n_kv_heads, cap, head_dim, dtype=dtype, device=device)
    fill_sentinel(c)
    return c
