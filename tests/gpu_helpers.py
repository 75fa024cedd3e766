"""Helpers for the GPU parity tests (device buffers, workspace views, the
acceptance rule for float64-accumulated GEMV outputs)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import routing_quant_expert_amd as R
import synth


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def workspace(cfg, m):
    n = R.workspace_bytes(cfg, m)
    assert n > 0
    ws = torch.empty(n + 256, dtype=torch.uint8, device="cuda")
    off = (-ws.data_ptr()) % 256
    ws = ws[off:off + n]
    R.workspace_init(cfg, m, ws)
    return ws


def ws_array(ws, layout: dict, name: str, dtype, count: int) -> np.ndarray:
    nbytes = np.dtype(dtype).itemsize * count
    off = layout[name]
    raw = ws[off:off + nbytes].cpu().numpy()
    return raw.view(dtype)


def to_np_u16(t) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def plan_tables(ws, layout, m, topk):
    P = layout["max_pairs"]
    words = ws_array(ws, layout, "plan", np.int32, layout["plan_words"])
    n_u, n_pairs = int(words[0]), int(words[1])
    base = 2
    tab = {}
    for name in ("u_expert", "u_first", "u_npairs", "pair_tok", "pair_expert", "pair_w"):
        tab[name] = words[base:base + P]
        base += P
    tab["pair_w"] = tab["pair_w"].view(np.float32)
    # a token's plan entries: its picks in ascending id, then its K-quant shared expert's pair (-1 = none)
    tab["tok_pairs"] = words[base:base + m * (topk + 1)].reshape(m, topk + 1)
    tab["n_u"], tab["n_pairs"] = n_u, n_pairs
    return tab


def f32_accept(got: np.ndarray, want: np.ndarray, near: np.ndarray, what: str) -> int:
    """got must equal want bit for bit, except where the exact value lies near
    an f32 midpoint (near=1): there the neighbour is also a correct rounding.
    Returns the number of such accepted neighbours."""
    g = got.view(np.uint32).astype(np.int64)
    w = want.view(np.uint32).astype(np.int64)
    diff = g != w
    if not diff.any():
        return 0
    ulp1 = np.abs(np.nextafter(want, np.float32(np.inf)) - want)
    one_ulp = np.abs(got.astype(np.float64) - want.astype(np.float64)) <= np.maximum(
        ulp1, np.abs(want - np.nextafter(want, np.float32(-np.inf)))).astype(np.float64)
    ok = diff & (near.astype(bool)) & one_ulp
    bad = diff & ~ok
    if bad.any():
        i = np.nonzero(bad)[0][:5]
        raise AssertionError(f"{what}: {int(bad.sum())} outputs differ: idx {i} got {got[i]} want {want[i]} "
                             f"near {near[i]}")
    return int(ok.sum())


def rel_l2(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.sqrt(((a - b) ** 2).sum() / max((b ** 2).sum(), 1e-300)))


def host_spec(shape, seed=1, layer=0, zipf=False):
    return synth.LayerSpec(shape, seed=seed, layer=layer, zipf_bias=zipf)


def oracle_header(spec, x_np, bias=None):
    lg = oracle.router_logits(x_np, synth.gate_w(spec))
    hdr, sc = oracle.select(spec.shape, lg, synth.bias(spec) if bias is None else bias)
    return lg, hdr, sc


def check_combine_bits(ws, layout: dict, tab: dict, m: int, topk: int, out_f32: np.ndarray, with_shared: bool,
                       tokens=None):
    """The combine order, bit for bit at any size: each token's f32 output
    must equal the oracle's combine applied to the device's own per-pair
    expert outputs y (in plan order, ascending expert id) with the plan
    weights, and then the device's own shared-expert output sd added after
    the routed sum [moe_v41.rs, fn shared_side] (a K-quant shared expert is
    the token's last plan entry, weight 1). The inputs are the device's,
    so no rounding of the GEMVs can blur a wrong summation order."""
    P, dim = layout["max_pairs"], out_f32.shape[1]
    y = ws_array(ws, layout, "y", np.float32, P * dim).reshape(P, dim)
    sd = ws_array(ws, layout, "sd", np.float32, m * dim).reshape(m, dim) if with_shared else None
    for t in (range(m) if tokens is None else tokens):
        pairs = [int(p) for p in tab["tok_pairs"][t] if p >= 0]   # a K-quant shared expert last, weight 1
        ys = np.stack([y[p] for p in pairs])
        w = np.array([tab["pair_w"][p] for p in pairs], np.float32)
        want, _ = oracle.combine(ys, w, None if sd is None else sd[t])
        got = np.ascontiguousarray(out_f32[t], np.float32)
        bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
        assert bad.size == 0, f"combine of token {t}: {bad.size} outputs differ, first at {bad[:4]}"
