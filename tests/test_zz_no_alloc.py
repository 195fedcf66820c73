"""orthros_decode_step_noalloc (the decode step on the library's own scratch
array, for callers that cannot allocate) against orthros_decode_step with a
caller workspace: the same kernels, so outputs, caches and lengths must
match bit for bit.  Three calls in a row, each with a smaller workspace than
the one before (MI355X only)."""
import pytest
import torch

from gpu_util import bits, say
from phase_aware_swa_amd import binding, inputs
from phase_aware_swa_amd.runner import Decode, desc_for

pytestmark = pytest.mark.gpu


def clone(x):
    return {k: (v.clone() if torch.is_tensor(v) else v) for k, v in x.items()}


def run_both(cfg, seed, steps):
    say(f"no-alloc decode vs workspace decode: {cfg} steps={steps}")
    x = inputs.decode_inputs(seed=seed, device="cuda", **cfg)
    y = clone(x)
    hint = int(x["cache_len"].max().item()) + steps - 1
    ref = Decode(cfg, x["k_cache"], x["v_cache"], x["cache_len"], hint, x["alpha"], x["beta"], x["alpha_out"],
                 x["beta_out"])
    desc = desc_for(cfg)
    o = torch.empty_like(ref.o)
    o_out = torch.empty_like(ref.o_out)
    for s in range(steps):
        ref.step(x["q"][s], x["q_out"][s], x["k_new"][s], x["v_new"][s])
        binding.decode_step_noalloc(desc, y["q"][s], y["q_out"][s], y["k_new"][s], y["v_new"][s], y["alpha"],
                                    y["beta"], y["alpha_out"], y["beta_out"], y["k_cache"], y["v_cache"],
                                    y["cache_len"], hint, o, o_out)
        torch.cuda.synchronize()
        assert torch.equal(bits(o), bits(ref.o)), f"step {s}: o"
        assert torch.equal(bits(o_out), bits(ref.o_out)), f"step {s}: o_out"
    assert torch.equal(y["cache_len"], x["cache_len"])
    assert torch.equal(bits(y["k_cache"]), bits(x["k_cache"]))
    assert torch.equal(bits(y["v_cache"]), bits(x["v_cache"]))
    return binding.decode_workspace_size(desc, hint)


def test_noalloc_decode_matches_workspace_decode():
    # first call: fp32, batch 16, 32/8 heads, d128, histories of 100K-120K
    # keys -- the lane-parallel kernel, about 60 MB of partials in the
    # scratch array
    lane = dict(batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, window=128, dtype=torch.float32,
                len_lo=100000, len_hi=120000, steps=2)
    ws_lane = run_both(lane, seed=70, steps=2)
    assert 32 << 20 < ws_lane <= 64 << 20
    # second call, smaller workspace: batch 16, histories of 98K-110K keys --
    # the LDS-streamed kernel, over what the first call left in the array
    big = dict(batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, window=128, dtype=torch.bfloat16,
               len_lo=98000, len_hi=110000, steps=2)
    ws_big = run_both(big, seed=71, steps=2)
    assert ws_big < ws_lane
    # third call, smaller still: batch 3, 8/2 heads, short histories -- the
    # one-launch short-history kernel
    small = dict(batch=3, n_q_heads=8, n_kv_heads=2, head_dim=128, window=128, dtype=torch.bfloat16,
                 len_lo=100, len_hi=3000, steps=2)
    ws_small = run_both(small, seed=72, steps=2)
    assert ws_small < ws_big
