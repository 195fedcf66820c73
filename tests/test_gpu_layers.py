"""Multi-layer decode ("Orthros:阶段感知异构注意力精读笔记" §2.5 decode row,
§2.6: every layer keeps its own full cache): a stack of resident layers, each
step running every layer's orthros_decode_step, eager and as one captured
HIP graph.  Every graph replay is checked bit for bit against the eager run of
the same step, with the program's own eager work and synchronisations
between replays (MI355X only)."""
import pytest
import torch

from gpu_util import bits, say
from phase_aware_swa_amd import inputs
from phase_aware_swa_amd.runner import LayerStack

pytestmark = pytest.mark.gpu


def make_stack(cfg, seeds):
    layers = [inputs.decode_inputs(seed=s, device="cuda", **cfg) for s in seeds]
    return LayerStack(cfg, layers, cfg["steps"]), layers


def clone_layers(layers):
    return [{k: (v.clone() if torch.is_tensor(v) else v) for k, v in x.items()} for x in layers]


@pytest.mark.parametrize("B,Hq,Hkv", [(2, 8, 2), (3, 4, 4)])
def test_graph_replay_matches_eager(B, Hq, Hkv):
    cfg = dict(batch=B, n_q_heads=Hq, n_kv_heads=Hkv, head_dim=128, window=128, dtype=torch.bfloat16,
               len_lo=200, len_hi=700, steps=4)
    say(f"layer stack graph case {cfg}")
    eager, layers = make_stack(cfg, seeds=[31, 32, 33])
    len0 = [x["cache_len"].clone() for x in layers]
    gstack = LayerStack(cfg, clone_layers(layers), cfg["steps"])
    graph = gstack.capture()                    # records only; nothing runs yet
    torch.cuda.synchronize()
    for s in range(cfg["steps"]):
        eager.set_inputs(s)
        eager.step()
        gstack.set_inputs(s)
        graph.replay()
        # the program's own eager work between replays
        junk = torch.randn(4096, device="cuda").mul_(2).sum()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for l, (de, dg) in enumerate(zip(eager.decs, gstack.decs)):
            assert torch.equal(de.cache_len, dg.cache_len), f"step {s} layer {l}: lengths"
            assert torch.equal(bits(de.o), bits(dg.o)), f"step {s} layer {l}: o"
            assert torch.equal(bits(de.o_out), bits(dg.o_out)), f"step {s} layer {l}: o_out"
            assert torch.equal(bits(de.k_cache), bits(dg.k_cache)), f"step {s} layer {l}: k_cache"
            assert torch.equal(bits(de.v_cache), bits(dg.v_cache)), f"step {s} layer {l}: v_cache"
    # every layer advanced by exactly one slot per step
    for l, (l0, dg) in enumerate(zip(len0, gstack.decs)):
        assert torch.equal(dg.cache_len.cpu(), l0.cpu() + cfg["steps"]), f"layer {l}: final lengths"


def test_layers_are_independent():
    """A stack step equals each layer's single-layer step run alone."""
    cfg = dict(batch=2, n_q_heads=8, n_kv_heads=2, head_dim=128, window=128, dtype=torch.bfloat16, len_lo=100,
               len_hi=400, steps=2)
    say(f"layer stack independence {cfg}")
    stack, layers = make_stack(cfg, seeds=[41, 42])
    solo, _ = make_stack(cfg, seeds=[42])
    for s in range(2):
        stack.set_inputs(s)
        stack.step()
        solo.set_inputs(s)
        solo.step()
    torch.cuda.synchronize()
    assert torch.equal(bits(stack.decs[1].o_out), bits(solo.decs[0].o_out))
    assert torch.equal(bits(stack.decs[1].k_cache), bits(solo.decs[0].k_cache))
