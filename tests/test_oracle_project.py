"""Pins of the projection oracle ("Orthros:阶段感知异构注意力精读笔记"
§2.1-§2.2: K/V from the base input X for every position; both streams'
queries from the one shared W_Q, each with its own elementwise
scale-offset) to things other than itself: a hand-worked example, permutation
and one-hot weights, the shared weight across streams, linearity and the
cache placement.  CPU only."""
import torch

from oracle.project import cache_rows, project

f64 = torch.float64


def rand_case(B=2, T=5, T_out=3, dm=24, Hq=4, Hkv=2, d=6, seed=0):
    g = torch.Generator().manual_seed(seed)
    r = lambda *s: torch.randn(*s, generator=g)
    return dict(x=r(B, T, dm), x_out=r(B, T_out, dm), w_q=r(Hq * d, dm), w_k=r(Hkv * d, dm), w_v=r(Hkv * d, dm),
                alpha=1 + 0.1 * r(Hq, d), beta=0.1 * r(Hq, d), alpha_out=1 + 0.1 * r(Hq, d),
                beta_out=0.1 * r(Hq, d), n_q_heads=Hq, n_kv_heads=Hkv, head_dim=d)


def test_hand_worked_example():
    """x = [1, 2], W_Q = [[1, 0], [1, 1]] ([out][in]): x W_Q^T = [1, 3];
    alpha = [2, 3], beta = [1, -1] -> q = [3, 8].  (Using W_Q untransposed
    would give [3, 2] -> [7, 5].)  K with W_K = [[0, 1], [2, 0]] -> [2, 2];
    V with W_V = [[1, -1], [0, 3]] -> [-1, 6]."""
    x = torch.tensor([[[1.0, 2.0]]])
    c = dict(x=x, x_out=x.clone(), w_q=torch.tensor([[1.0, 0.0], [1.0, 1.0]]),
             w_k=torch.tensor([[0.0, 1.0], [2.0, 0.0]]), w_v=torch.tensor([[1.0, -1.0], [0.0, 3.0]]),
             alpha=torch.tensor([[2.0, 3.0]]), beta=torch.tensor([[1.0, -1.0]]),
             alpha_out=torch.tensor([[1.0, 1.0]]), beta_out=torch.tensor([[0.0, 0.0]]),
             n_q_heads=1, n_kv_heads=1, head_dim=2)
    r = project(**c)
    assert r["q"].flatten().tolist() == [3.0, 8.0]
    assert r["q_out"].flatten().tolist() == [1.0, 3.0]
    assert r["k"].flatten().tolist() == [2.0, 2.0]
    assert r["v"].flatten().tolist() == [-1.0, 6.0]


def test_permutation_weights_select_inputs():
    """W = the permutation matrix with W[j][perm[j]] = 1: output column j is
    input column perm[j] (a transposed W would give perm^-1).  Elementwise
    check against the inputs, no matrix product."""
    c = rand_case(dm=8, Hq=2, Hkv=1, d=4, seed=1)
    perm = torch.tensor([3, 0, 6, 1, 7, 2, 5, 4])
    assert not torch.equal(perm[perm], torch.arange(8))       # not an involution
    P = torch.zeros(8, 8)
    P[torch.arange(8), perm] = 1.0
    c["w_q"] = P
    c["w_k"] = P[:4].clone()
    c["w_v"] = P[4:].clone()
    r = project(**c)
    x, xo = c["x"].double(), c["x_out"].double()
    a, b, ao, bo = (c[k].double().flatten() for k in ("alpha", "beta", "alpha_out", "beta_out"))
    for j in range(8):
        assert torch.equal(r["q"].flatten(2)[..., j], x[..., perm[j]] * a[j] + b[j])
        assert torch.equal(r["q_out"].flatten(2)[..., j], xo[..., perm[j]] * ao[j] + bo[j])
    for j in range(4):
        assert torch.equal(r["k"].flatten(2)[..., j], x[..., perm[j]])
        assert torch.equal(r["v"].flatten(2)[..., j], x[..., perm[4 + j]])


def test_one_hot_rows_read_weight_columns():
    """x = e_i: x W^T is column i of W, head-split as [heads][d]."""
    c = rand_case(B=1, T=6, T_out=6, dm=6, seed=2)
    c["x"] = torch.eye(6)[None]
    c["x_out"] = torch.eye(6)[None]
    c["alpha"] = torch.ones_like(c["alpha"])
    c["beta"] = torch.zeros_like(c["beta"])
    r = project(**c)
    for i in range(6):
        assert torch.equal(r["q"][0, i].flatten(), c["w_q"][:, i].double())
        assert torch.equal(r["k"][0, i].flatten(), c["w_k"][:, i].double())
        assert torch.equal(r["v"][0, i].flatten(), c["w_v"][:, i].double())


def test_shared_weight_separate_scale_offset():
    """Both streams use the one W_Q: the same input in both streams differs
    only by the scale-offset (q' - beta') / alpha' == (q - beta) / alpha."""
    c = rand_case(T=4, T_out=4, seed=3)
    c["x_out"] = c["x"].clone()
    r = project(**c)
    raw = (r["q"] - c["beta"].double()) / c["alpha"].double()
    raw_out = (r["q_out"] - c["beta_out"].double()) / c["alpha_out"].double()
    assert torch.allclose(raw, raw_out, rtol=1e-12, atol=1e-12)
    assert not torch.allclose(r["q"], r["q_out"])


def test_linear_in_x():
    c = rand_case(seed=4)
    for k in ("alpha", "alpha_out"):
        c[k] = torch.ones_like(c[k])
    for k in ("beta", "beta_out"):
        c[k] = torch.zeros_like(c[k])
    x1 = c["x"].double()
    x2 = torch.randn(c["x"].shape, generator=torch.Generator().manual_seed(9), dtype=f64)
    r1 = project(**{**c, "x": x1})
    r2 = project(**{**c, "x": x2})
    r3 = project(**{**c, "x": 2 * x1 - 3 * x2})
    for k in ("q", "k", "v"):
        assert torch.allclose(r3[k], 2 * r1[k] - 3 * r2[k], rtol=1e-10, atol=1e-10)


def test_output_stream_does_not_touch_base_kv():
    """[N] §2.4: the base K/V never depend on the output stream's input."""
    c = rand_case(seed=5)
    r1 = project(**c)
    r2 = project(**{**c, "x_out": 100 * torch.randn(c["x_out"].shape)})
    assert torch.equal(r1["k"], r2["k"]) and torch.equal(r1["v"], r2["v"]) and torch.equal(r1["q"], r2["q"])


def test_cache_rows_layout():
    k = torch.arange(2 * 3 * 2 * 4, dtype=f64).reshape(2, 3, 2, 4)     # [B][T][Hkv][d]
    c = cache_rows(k)
    for b in range(2):
        for t in range(3):
            for g in range(2):
                assert torch.equal(c[b, g, t], k[b, t, g])


def test_empty_output_stream():
    c = rand_case(T_out=0, seed=6)
    r = project(**c)
    assert r["q_out"].shape == (2, 0, 4, 6)
