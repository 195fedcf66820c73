"""Closed forms of the mask probes ("Orthros:阶段感知异构注意力精读笔记"
§2.3 Eqs. (4)-(5): the window W_t and the copy's j <= t; §2.4: the copy is
masked by its original position).

With alpha = beta = 0 (both streams) every query is zero, so every score is
zero and the softmax weights are uniform over the admissible key set S: the
output is the mean of V over S.  When V rows are one-hot (key j marks column
c(j), or no column at all), output column c is exactly count_c(S) / |S|, a
ratio of small integers: a key too many or too few in S changes a count
(and |S|) and so the bits of the output.  The kernels form the output as
(sum of exact ones) times an fp32 reciprocal of |S|, so the bf16 result is
the round-to-nearest-even of count / |S| except when that ratio lies within
a few fp32 ulps of a bf16 rounding midpoint; those rare elements are flagged
here and may take either neighbour, every other element must match exactly.
"""
import torch


def marker(j, shift, m):
    """Column marked by key j: (j + shift) mod m."""
    return (j + shift) % m


def residue_counts(lo, hi, shift, m, d):
    """counts[..., c] = #{j in [lo, hi] : (j + shift) mod m == c} for c < d
    (0 for c >= m).  lo, hi, shift: int64 tensors of one shape (hi >= lo - 1;
    an empty set gives zeros)."""
    lo, hi, shift = (torch.as_tensor(x, dtype=torch.int64) for x in (lo, hi, shift))
    c = torch.arange(d, dtype=torch.int64)
    r = (c - shift[..., None]) % m                       # residue of j for column c
    f = lambda x: torch.div(x, m, rounding_mode="floor")
    cnt = f(hi[..., None] - r) - f(lo[..., None] - 1 - r)
    cnt[..., m:] = 0
    return cnt


def expected_bf16(counts, n):
    """(values, either_ok): values = bf16(counts / n); either_ok marks the
    elements whose ratio sits so close to a bf16 rounding midpoint that an
    fp32 reciprocal-and-multiply may round them either way."""
    x = counts.double() / torch.as_tensor(n, dtype=torch.float64)[..., None]
    lo = (x * (1 - 2.0 ** -20)).float().bfloat16()
    hi = (x * (1 + 2.0 ** -20)).float().bfloat16()
    return x.float().bfloat16(), lo.float() != hi.float()


def assert_probe(got, counts, n, what):
    """Bit-exact comparison of a bf16 output against count / n (see the
    module text); got and counts have the same shape, n one dim less."""
    got = got.detach().cpu()
    assert got.dtype == torch.bfloat16
    exp, either = expected_bf16(counts, n)
    g, e = got.float(), exp.float()
    ok = (g == e)
    if either.any():
        # the two bf16 neighbours of the ratio
        x = counts.double() / torch.as_tensor(n, dtype=torch.float64)[..., None]
        a = (x * (1 - 2.0 ** -20)).float().bfloat16().float()
        b = (x * (1 + 2.0 ** -20)).float().bfloat16().float()
        ok = ok | (either & ((g == a) | (g == b)))
    if not bool(ok.all()):
        bad = (~ok).nonzero()[:5].tolist()
        detail = [(tuple(i), got[tuple(i)].item(), exp[tuple(i)].item(), counts[tuple(i)].item()) for i in bad]
        raise AssertionError(f"{what}: {int((~ok).sum())} elements differ from count / n; first (index, got, "
                             f"expected, count): {detail}")
    return int(either.sum())
