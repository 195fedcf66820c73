"""fp64 CPU oracle of the projections on either side of the attention step.

TEST INFRASTRUCTURE ONLY.  Only the tests and the benchmark's CPU-baseline
leg may import this module; the GPU library never does, and this module
imports nothing from it.

"Orthros:阶段感知异构注意力精读笔记" §2.1-§2.2: every layer keeps two
residual streams, the base input X and the output copies' input X'.  The
base stream's keys and values come from X for every position (k = x W_K,
v = x W_V, the layer's cache rows); both streams' queries come from the one
shared W_Q and then take their own elementwise scale-offset:
q = (x W_Q) * alpha + beta, q' = (x' W_Q) * alpha' + beta'.

The weights are stored as [out][in] (the row-major form of a linear layer:
y = x W^T), so W_Q is [Hq*d][d_model] and W_K, W_V are [Hkv*d][d_model].
Inputs are promoted exactly to fp64; one fp64 matrix product per weight
(a library primitive) is the whole contraction.  Outputs are fp64:
  q      [B][T][Hq][d]         q_out   [B][T_out][Hq][d]
  k, v   [B][T][Hkv][d]        (cache rows: k_cache[b][g][t] = k[b][t][g])
"""
import torch


def _proj(x, w, heads, d):
    """x [B][T][d_model] -> (x W^T) as [B][T][heads][d] in fp64."""
    B, T, dm = x.shape
    y = x.double().reshape(B * T, dm) @ w.double().t()
    return y.reshape(B, T, heads, d)


def project(x, x_out, w_q, w_k, w_v, alpha, beta, alpha_out, beta_out, n_q_heads, n_kv_heads, head_dim):
    """The base stream's q, k, v from X and the copies' q' from X' ([N] §2.1-§2.2).

    x [B][T][d_model], x_out [B][T_out][d_model] (T_out may be 0); alpha..beta_out [Hq][d].
    Returns dict(q, q_out, k, v) in fp64.
    """
    d = head_dim
    q = _proj(x, w_q, n_q_heads, d) * alpha.double() + beta.double()
    q_out = _proj(x_out, w_q, n_q_heads, d) * alpha_out.double() + beta_out.double()
    k = _proj(x, w_k, n_kv_heads, d)
    v = _proj(x, w_v, n_kv_heads, d)
    return {"q": q, "q_out": q_out, "k": k, "v": v}


def cache_rows(kv):
    """[B][T][Hkv][d] -> the cache layout [B][Hkv][T][d] (slots 0..T-1)."""
    return kv.permute(0, 2, 1, 3).contiguous()
