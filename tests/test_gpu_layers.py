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


def oracle_stack_check(stack, layers, steps, replay, case):
    """Runs `steps` multi-layer steps through `replay` (eager step or graph
    replay) and checks every layer's o, o_out, caches and lengths against
    the oracle stepping the same layers."""
    import oracle
    from gpu_util import assert_parity, to_cpu
    hosts = [to_cpu(x) for x in layers]
    state = [(h["k_cache"].clone(), h["v_cache"].clone(), h["cache_len"].clone()) for h in hosts]
    for s in range(steps):
        stack.set_inputs(s)
        replay()
        junk = torch.randn(4096, device="cuda").mul_(2).sum()     # the program's own work between steps
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        for l, (h, (kc, vc, lc), dec) in enumerate(zip(hosts, state, stack.decs)):
            o, o_out = oracle.decode_step(h["q"][s], h["q_out"][s], h["k_new"][s], h["v_new"][s], h["alpha"],
                                          h["beta"], h["alpha_out"], h["beta_out"], 128, kc, vc, lc)
            assert_parity(dec.o, o, torch.bfloat16, f"{case} step {s} layer {l} o")
            assert_parity(dec.o_out, o_out, torch.bfloat16, f"{case} step {s} layer {l} o_out")
            assert torch.equal(dec.cache_len.cpu(), lc), f"step {s} layer {l}: lengths"
    for l, ((kc, vc, _), dec) in enumerate(zip(state, stack.decs)):
        assert torch.equal(bits(dec.k_cache.cpu()), bits(kc)), f"layer {l}: k_cache"
        assert torch.equal(bits(dec.v_cache.cpu()), bits(vc)), f"layer {l}: v_cache"


def test_graph_36_layers_against_oracle():
    """36 resident layers (B2, 32/8 heads, d128, histories 200-2000), the
    whole multi-layer step captured once and replayed 3 times: every
    layer's outputs, caches and lengths against the oracle after every
    replay."""
    cfg = dict(batch=2, n_q_heads=32, n_kv_heads=8, head_dim=128, window=128, dtype=torch.bfloat16,
               len_lo=200, len_hi=2000, steps=3)
    say(f"36-layer graph vs oracle {cfg}")
    stack, layers = make_stack(cfg, seeds=list(range(500, 536)))
    graph = stack.capture()
    torch.cuda.synchronize()
    oracle_stack_check(stack, layers, cfg["steps"], graph.replay, "36-layer graph")


def test_graph_lds_path_matches_eager_and_oracle():
    """Histories long enough for the LDS-streamed decode kernel (B32, 32/8
    heads, 60K-66K keys): a 2-layer step captured in a HIP graph, replayed
    twice, bit for bit against the eager step, then one more replay against
    the oracle (which steps the same layers from their initial state)."""
    import oracle
    from gpu_util import assert_parity, to_cpu
    cfg = dict(batch=32, n_q_heads=32, n_kv_heads=8, head_dim=128, window=128, dtype=torch.bfloat16,
               len_lo=60000, len_hi=66000, steps=3)
    say(f"LDS-path graph case {cfg}")
    eager, layers = make_stack(cfg, seeds=[61, 62])
    hosts = [to_cpu(x) for x in layers]                     # the initial state, for the oracle
    gstack = LayerStack(cfg, clone_layers(layers), cfg["steps"])
    graph = gstack.capture()
    torch.cuda.synchronize()
    for s in range(2):
        eager.set_inputs(s)
        eager.step()
        gstack.set_inputs(s)
        graph.replay()
        torch.cuda.synchronize()
        for l, (de, dg) in enumerate(zip(eager.decs, gstack.decs)):
            assert torch.equal(de.cache_len, dg.cache_len), f"step {s} layer {l}: lengths"
            assert torch.equal(bits(de.o), bits(dg.o)), f"step {s} layer {l}: o"
            assert torch.equal(bits(de.o_out), bits(dg.o_out)), f"step {s} layer {l}: o_out"
    del eager
    gstack.set_inputs(2)
    graph.replay()
    torch.cuda.synchronize()
    for l, (h, dec) in enumerate(zip(hosts, gstack.decs)):
        kc, vc, lc = h["k_cache"], h["v_cache"], h["cache_len"].clone()
        for s in range(3):
            o, o_out = oracle.decode_step(h["q"][s], h["q_out"][s], h["k_new"][s], h["v_new"][s], h["alpha"],
                                          h["beta"], h["alpha_out"], h["beta_out"], 128, kc, vc, lc,
                                          compute=s == 2)
        assert_parity(dec.o, o, torch.bfloat16, f"LDS graph layer {l} o")
        assert_parity(dec.o_out, o_out, torch.bfloat16, f"LDS graph layer {l} o_out")
        assert torch.equal(dec.cache_len.cpu(), lc)
        assert torch.equal(bits(dec.k_cache.cpu()), bits(kc)) and torch.equal(bits(dec.v_cache.cpu()), bits(vc))
