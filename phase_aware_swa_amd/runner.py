"""Device-buffer plumbing around the binding: allocates outputs, caches and
workspaces with torch (device memory only) and calls the C ABI.

Nothing here computes: every step of the attention runs in liborthros.so.
"""
import torch

from . import binding
from .inputs import empty_cache


def desc_for(cfg, softmax_scale=0.0):
    return binding.make_desc(cfg["batch"], cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"],
                             cfg["window"], cfg["dtype"], softmax_scale)


class Prefill:
    """Buffers for repeated prefill calls of one shape on one device.

    x: the input dict of inputs.prefill_inputs (tensors already on `device`).
    cap: cache capacity (>= T); slots [T, cap) hold the sentinel and must
    stay untouched.  k_cache / v_cache: caller-owned caches to write into
    instead (their capacity is used).
    """

    def __init__(self, cfg, x, device="cuda", cap=None, softmax_scale=0.0, k_cache=None, v_cache=None):
        self.cfg = cfg
        self.x = x
        B, T = cfg["batch"], x["q"].shape[1]
        Hq, Hkv, d, dt = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"], cfg["dtype"]
        self.T = T
        self.desc = desc_for(cfg, softmax_scale)
        if k_cache is not None:
            self.k_cache, self.v_cache = k_cache, v_cache
            self.cap = k_cache.shape[2]
        else:
            self.cap = cap or T
            self.k_cache = empty_cache(B, Hkv, self.cap, d, dt, device)
            self.v_cache = empty_cache(B, Hkv, self.cap, d, dt, device)
        self.o = torch.empty(B, T, Hq, d, dtype=dt, device=device)
        self.o_out = torch.empty(B, Hq, d, dtype=dt, device=device)
        ws = binding.prefill_workspace_size(self.desc, T)
        self.workspace = torch.empty(max(ws, 16), dtype=torch.uint8, device=device)

    def run(self, stream=None):
        x = self.x
        binding.prefill(self.desc, self.T, x["q"], x["q_out"], x["out_pos"], x["k"], x["v"], x["alpha"],
                        x["beta"], x["alpha_out"], x["beta_out"], self.k_cache, self.v_cache, self.o,
                        self.o_out, self.workspace, stream)

    def run_swa(self, stream=None):
        x = self.x
        binding.swa_prefill(self.desc, self.T, x["q"], x["k"], x["v"], x["alpha"], x["beta"], self.k_cache,
                            self.v_cache, self.o, stream)

    def run_xattn(self, stream=None):
        x = self.x
        binding.global_xattn(self.desc, self.T, x["q_out"], x["out_pos"], x["alpha_out"], x["beta_out"],
                             self.k_cache, self.v_cache, self.o_out, self.workspace, stream)


class Decode:
    """Buffers for a run of decode steps over caches the caller owns.

    k_cache, v_cache, cache_len: device tensors, updated in place by step().
    max_len_hint: host bound of every cache length for the whole run.
    """

    def __init__(self, cfg, k_cache, v_cache, cache_len, max_len_hint, alpha, beta, alpha_out, beta_out,
                 softmax_scale=0.0):
        B, Hq, d, dt = cfg["batch"], cfg["n_q_heads"], cfg["head_dim"], cfg["dtype"]
        dev = k_cache.device
        self.desc = desc_for(cfg, softmax_scale)
        self.k_cache, self.v_cache, self.cache_len = k_cache, v_cache, cache_len
        self.max_len_hint = max_len_hint
        self.alpha, self.beta, self.alpha_out, self.beta_out = alpha, beta, alpha_out, beta_out
        self.o = torch.empty(B, Hq, d, dtype=dt, device=dev)
        self.o_out = torch.empty(B, Hq, d, dtype=dt, device=dev)
        ws = binding.decode_workspace_size(self.desc, max_len_hint)
        # zero-filled once: the step's arrival counters start at zero (each step leaves them so)
        self.workspace = torch.zeros(max(ws, 16), dtype=torch.uint8, device=dev)

    def step(self, q, q_out, k_new, v_new, o=None, o_out=None, stream=None):
        binding.decode_step(self.desc, q, q_out, k_new, v_new, self.alpha, self.beta, self.alpha_out,
                            self.beta_out, self.k_cache, self.v_cache, self.cache_len, self.max_len_hint,
                            self.o if o is None else o, self.o_out if o_out is None else o_out,
                            self.workspace, stream)


class LayerStack:
    """Decode state of a stack of resident layers (one model's layers, each
    with its own cache, lengths, workspace and step inputs) for the
    multi-layer decode step.

    layers: list of inputs.decode_inputs dicts already on the device (the
    step inputs of layer l at step s are x["q"][s] etc.); steps: how many
    steps the stack will run (bounds each layer's lengths).  set_inputs(s)
    copies step s's inputs into fixed per-layer buffers; step() runs every
    layer's orthros_decode_step in order on the current stream, reading those
    buffers; capture() records one step() into a HIP graph, whose replay()
    then runs the whole multi-layer step as one graph launch (every launch's
    arguments are fixed; the step inputs change through the buffers, the
    lengths through the device arrays the step itself advances).
    """

    def __init__(self, cfg, layers, steps):
        self.xs = layers
        # each layer's own bound of its lengths over `steps` steps (its cache capacity)
        self.decs = [Decode(cfg, x["k_cache"], x["v_cache"], x["cache_len"],
                            int(x["cache_len"].max().item()) + steps - 1, x["alpha"], x["beta"], x["alpha_out"],
                            x["beta_out"]) for x in layers]
        self.buf = [{k: torch.empty_like(x[k][0]) for k in ("q", "q_out", "k_new", "v_new")} for x in layers]

    def set_inputs(self, s):
        for x, b in zip(self.xs, self.buf):
            for k, t in b.items():
                t.copy_(x[k][s])

    def step(self):
        for dec, b in zip(self.decs, self.buf):
            dec.step(b["q"], b["q_out"], b["k_new"], b["v_new"])

    def capture(self):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.step()
        return g


class Project:
    """Buffers for orthros_project: q [B,T,Hq,d], q_out [B,T_out,Hq,d] and
    (unless given) caches of capacity cap filled with the sentinel."""

    def __init__(self, cfg, x, k_cache=None, v_cache=None, cap=None, scale_offset=True):
        self.desc = desc_for(cfg)
        B, T, dm = x["x"].shape
        T_out = x["x_out"].shape[1]
        Hq, Hkv, d = cfg["n_q_heads"], cfg["n_kv_heads"], cfg["head_dim"]
        dev = x["x"].device
        self.x, self.T, self.d_model = x, T, dm
        self.so = scale_offset
        self.q = torch.empty(B, T, Hq, d, dtype=torch.bfloat16, device=dev)
        self.q_out = torch.empty(B, T_out, Hq, d, dtype=torch.bfloat16, device=dev)
        cap = cap or T
        self.k_cache = k_cache if k_cache is not None else empty_cache(B, Hkv, cap, d, torch.bfloat16, dev)
        self.v_cache = v_cache if v_cache is not None else empty_cache(B, Hkv, cap, d, torch.bfloat16, dev)

    def run(self, stream=None):
        x = self.x
        so = (x["alpha"], x["beta"], x["alpha_out"], x["beta_out"]) if self.so else (None,) * 4
        binding.project(self.desc, self.T, self.d_model, x["x"], x["x_out"] if x["x_out"].shape[1] else None,
                        x["w_q"], x["w_k"], x["w_v"], *so, self.q, self.q_out if self.q_out.shape[1] else None,
                        self.k_cache, self.v_cache, stream)


class Copies:
    """Buffers for orthros_copies over caches filled by a prior SWA pass.

    q_out [B,T_out,Hq,d] and pos [B,T_out] (int32) on the device.
    """

    def __init__(self, cfg, T, q_out, pos, alpha_out, beta_out, k_cache, v_cache, softmax_scale=0.0):
        self.desc = desc_for(cfg, softmax_scale)
        self.T = T
        self.q_out, self.pos, self.alpha_out, self.beta_out = q_out, pos, alpha_out, beta_out
        self.k_cache, self.v_cache = k_cache, v_cache
        self.o_out = torch.empty_like(q_out)

    def run(self, stream=None):
        binding.copies(self.desc, self.T, self.q_out, self.pos, self.alpha_out, self.beta_out, self.k_cache,
                       self.v_cache, self.o_out, stream)
