"""Oracle: the whole MoE layer for m tokens, composed from the C stages.

TEST INFRASTRUCTURE ONLY. Per token (each token is independent, so m > 1 and
prefill are defined exactly as m = 1 repeated):
  1. q8_1 of the bf16 input row                       [moe_v41.rs, module doc]
  2. router logits, scores, top-k, weights, header   [moe_v41.rs, fn route_from_logits]
  3. per picked expert in plan order (ascending id):
     Q2_K gate/up GEMV, clamped SwiGLU, q8_1, Q3_K down GEMV
  4. acc = sum over the plan of w*y (f32, in plan order), then + shared expert
     output, out = bf16(acc)                           [moe_v41.rs, fn shared_side]
The shared expert is either resident bf16 (a dense MLP whose SwiGLU output is
rounded to bf16) or K-quant blocks run exactly as one more routed expert
(q8_1 of x, Q2_K gate/up, clamped SwiGLU, q8_1 of h, Q3_K down) whose output
is added after the routed sum [moe_v41.rs, struct MoeV41LayerWeights: the
shared matrices as bf16 or the GGUF's Q2_K/Q3_K blocks].
A stack of layers (one decode step through them, [step_seg.rs, module doc])
adds each layer's output to its input in f32 and rounds to bf16.
"""
from __future__ import annotations

import numpy as np

import synth
from . import (bf16_to_f32, combine, expert, f32_to_bf16, header_fields, q8_1, router_logits, select, shared)


class ExpertCache:
    """Host copies of the experts' raw blocks, generated on demand from the spec."""

    def __init__(self, spec: synth.LayerSpec):
        self.spec = spec
        self._c = {}

    def __call__(self, e: int):
        if e not in self._c:
            self._c[e] = tuple(synth.expert_blocks(self.spec, e, w) for w in ("gate", "up", "down"))
        return self._c[e]


def route(spec: synth.LayerSpec, x_bf16: np.ndarray, gate_w=None, bias=None) -> dict:
    gate_w = synth.gate_w(spec) if gate_w is None else gate_w
    bias = synth.bias(spec) if bias is None else bias
    logits = router_logits(x_bf16, gate_w)
    hdr, sc = select(spec.shape, logits, bias)
    return {"logits": logits, "scores": sc, "header": hdr}


def layer_forward(spec: synth.LayerSpec, x_bf16: np.ndarray, *, with_shared: bool = True, experts=None,
                  gate_w=None, bias=None, shared_w=None, shared_q=None, keep_experts: bool = True) -> dict:
    """Full layer for the bf16 rows x [m, dim]. Returns per-token results.
    The shared expert is K-quant when spec.shared_quant or shared_q (its
    (gate, up, down) raw blocks) is given, else bf16 (shared_w = (w1, w3, w2))."""
    s = spec.shape
    x_bf16 = np.ascontiguousarray(x_bf16, np.uint16).reshape(-1, s.dim)
    m = x_bf16.shape[0]
    experts = experts or ExpertCache(spec)
    r = route(spec, x_bf16, gate_w, bias)
    status, picks, wts, plan = header_fields(r["header"], s.topk)
    quant_shared = with_shared and (shared_q is not None or spec.shared_quant)
    if quant_shared:
        shared_q = shared_q or tuple(synth.shared_q_blocks(spec, w) for w in ("gate", "up", "down"))
    elif with_shared:
        shared_w = shared_w or tuple(synth.shared_w(spec, w) for w in ("w1", "w3", "w2"))
    out = dict(r)
    out.update(xq=[], xd16=[], tok=[], y_routed=np.empty((m, s.dim), np.float32),
               out_f32=np.empty((m, s.dim), np.float32), out_bf16=np.empty((m, s.dim), np.uint16), shared=[])
    for t in range(m):
        xq, xd = q8_1(bf16_to_f32(x_bf16[t]))
        out["xq"].append(xq)
        out["xd16"].append(xd)
        # plan-order weights: the pick-order weights permuted to ascending id
        order = np.argsort(picks[t], kind="stable")
        ids = picks[t][order]
        assert np.array_equal(ids, plan[t])
        w_plan = wts[t][order]
        per = []
        for e in ids:
            per.append(expert(s, xq, xd, *experts(int(e))))
        ys = np.stack([p["y"] for p in per])
        out["y_routed"][t], _ = combine(ys, w_plan)
        sd = None
        if quant_shared:   # one more expert on the same q8_1(x), output added after the routed sum
            sh = expert(s, xq, xd, *shared_q)
            out["shared"].append(sh)
            sd = sh["y"]
        elif with_shared:
            sh = shared(s, x_bf16[t], *shared_w)
            out["shared"].append(sh)
            sd = sh["sd"]
        out["out_f32"][t], out["out_bf16"][t] = combine(ys, w_plan, sd)
        out["tok"].append({"ids": ids, "w_plan": w_plan, "experts": per if keep_experts else None})
    return out


def residual(x_bf16: np.ndarray, out_f32: np.ndarray) -> np.ndarray:
    """The residual stream between stacked layers (the reading stated in the
    layer-stack entry point: no norm is named, none is applied):
    x_next = bf16(f32(x) + out), one f32 addition rounded to nearest."""
    return f32_to_bf16(bf16_to_f32(x_bf16) + np.asarray(out_f32, np.float32))


def stack_forward(specs, x0_bf16: np.ndarray, xs_given=None, layer_kwargs=None) -> dict:
    """One decode step through the layers of `specs` in order. Each layer is
    layer_forward on x_l; x_{l+1} = residual(x_l, out_l). With `xs_given`
    ([n_layers+1, m, dim] bf16), layer l reads xs_given[l] instead of its own
    x_l (teacher forcing: every layer checked on the same input as the
    device's). layer_kwargs: per-layer keyword arguments for layer_forward
    (weights given explicitly instead of generated from the spec)."""
    x = np.ascontiguousarray(x0_bf16, np.uint16)
    xs, outs, headers = [x], [], []
    for l, spec in enumerate(specs):
        xin = xs_given[l] if xs_given is not None else x
        kw = dict(layer_kwargs[l]) if layer_kwargs is not None else {}
        r = layer_forward(spec, xin, keep_experts=False, **kw)
        outs.append(r["out_f32"])
        headers.append(r["header"])
        x = residual(xin, r["out_f32"])
        xs.append(x)
    return {"xs": np.stack(xs), "out_f32": np.stack(outs), "headers": np.stack(headers)}
