#!/usr/bin/env python3
"""Benchmark: MoE-layer decode tokens/s at m=1 on one MI355X, and the HBM
roofline fraction of the layer kernel on its weight bytes.

Workload: one DeepSeek-V4.1-Flash-style MoE layer, dim 4096, inter 2048,
384 routed experts (Q2_K gate/up, Q3_K down, all resident: 3.5 GB), top-6,
bf16 router and bf16 shared expert; seeded synthetic inputs. A step is one
whole layer forward (route, select, routed experts, shared expert, combine)
for one token; steps cycle through `--tokens` distinct input rows so that
consecutive tokens pick mostly different experts (the 256 MB last-level
cache cannot hold a token's 54.7 MB of expert blocks from one step to the
next). Every second step's routed gate/up dispatch (the layer's largest
kernel) records HIP start/end events of its own, in the warm-up and in the
timed loop alike, so the tokens/s of a short run and a long one agree; the
roofline line is that kernel's. The three kernels (front, gate/up, down with
the combine) are timed once more in 64 steps after the timed region, and a
read-only streaming kernel gives the box's achievable HBM read rate.

--m 2..8 runs the multi-token path instead (correlated token rows, the
union of their picks read once); its gate/up kernel is the one timed.
"""
import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0   # dense int8 MFMA
# a kernel's source file and every header it includes (the counters are tied to these)
KERNEL_SOURCES = ("moe_decode1.hip", "moe_front.h", "moe_kquant.h", "moe_math.h", "moe_internal.h", "moe_select.h",
                  "moe_wave.h", "../../include/moe.h")
UNION_SOURCES = ("moe_experts.hip", "moe_kquant.h", "moe_math.h", "moe_internal.h", "moe_wave.h", "../../include/moe.h")
PREFILL_SOURCES = ("moe_prefill.hip", "moe_prefill.h", "moe_front.h", "moe_kquant.h", "moe_math.h", "moe_internal.h",
                   "moe_wave.h", "../../include/moe.h")


def source_text_key(text: bytes) -> bytes:
    """A source file's code with its comments dropped and whitespace runs
    collapsed: edits to comments leave a kernel's key unchanged."""
    import re
    tok = re.compile(rb'"(?:\\.|[^"\\\n])*"|\'(?:\\.|[^\'\\\n])*\'|//[^\n]*|/\*.*?\*/', re.S)
    code = tok.sub(lambda mt: mt.group(0) if mt.group(0)[:1] in (b'"', b"'") else b" ", text)
    return re.sub(rb"\s+", b" ", code).strip()


def kernel_source_sha(sources=KERNEL_SOURCES) -> str:
    """Hash of a kernel's sources without their comments (ties measured
    counters to a kernel version)."""
    import hashlib
    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "routing_quant_expert_amd", "csrc", f), "rb") as fh:
            h.update(source_text_key(fh.read()))
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, summary: str = "hbm_traffic_decode_m1_dim4096.md", sources=KERNEL_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; else None."""
    import re
    path = os.path.join(ROOT, "profiles", summary)
    if not os.path.exists(path):
        return None
    m = re.search(r"```json\n(\{.*?\})\n```", open(path).read(), re.S)
    if not m:
        return None
    d = json.loads(m.group(1))
    if d.get("kernel") != kernel or d.get("source_sha") != kernel_source_sha(sources):
        return None
    return d.get("traffic_bytes")


class HipEvents:
    """Raw HIP events (created up front, recorded by the library's hook)."""

    def __init__(self):
        self.h = ctypes.CDLL("libamdhip64.so")
        self.h.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.h.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.h.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.h.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.h.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e)
        return out

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.h.hipEventSynchronize(b) == 0
        assert self.h.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)

    def destroy(self, evs):
        for e in evs:
            self.h.hipEventDestroy(e)


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(spec, seconds: float, note: str = ""):
    """The oracle (plain C, as it stands) on host cores: whole-layer forward of
    successive tokens of the same workload, at all host threads for about 60%
    of `seconds`, then at one thread for the rest."""
    import oracle
    import synth
    from oracle import layer as olayer
    gw, b = synth.gate_w(spec), synth.bias(spec)
    sw = tuple(synth.shared_w(spec, w) for w in ("w1", "w3", "w2"))
    cache = olayer.ExpertCache(spec)

    def sample(budget, t_first):
        ntok, t_total = 0, 0.0
        while t_total < budget and ntok < 256:
            x = synth.tokens(spec, t_first + ntok, 1)
            r = olayer.route(spec, x, gw, b)
            for e in r["header"][0, 1:1 + spec.shape.topk]:
                cache(int(e))                      # input generation stays outside the timed part
            t0 = time.perf_counter()
            olayer.layer_forward(spec, x, experts=cache, gate_w=gw, bias=b, shared_w=sw, keep_experts=False)
            t_total += time.perf_counter() - t0
            ntok += 1
            cache._c.clear()
        return ntok, t_total

    threads = oracle.num_threads()
    n_all, t_all = sample(0.6 * seconds, 0)
    oracle.set_num_threads(1)
    try:
        n_one, t_one = sample(0.4 * seconds, 1000)
    finally:
        oracle.set_num_threads(threads)
    return {"value": n_all / t_all, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{n_all} tokens of the same layer (m=1), whole-layer forward, {t_all:.1f} s at {threads} "
                      f"threads; input generation excluded{note}",
            "single_thread": {"value": n_one / t_one, "unit": "tokens/s", "cores": 1,
                              "sample": f"{n_one} further tokens, {t_one:.1f} s at one thread"},
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count()}


def hbm_ceiling(blocks: int = 16384):
    """The box's achievable HBM read rate: the library's plain read-only
    streaming kernel (16-byte loads, a contiguous share per workgroup) over windows that the
    256 MB last-level cache cannot hold, each launch timed by the events of
    its own dispatch. 1 GiB windows alternate over 2 GiB; 64 MiB windows (the
    size of the m = 1 gate/up kernel's weights) rotate over 32 places."""
    import numpy as np
    import torch

    import routing_quant_expert_amd as R
    GiB = 1 << 30
    buf = torch.zeros(2 * GiB, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    ev = HipEvents()
    L = R.lib()
    res = {}
    for name, size, nwin, reps in (("1GiB", GiB, 2, 12), ("64MiB", 64 << 20, 32, 64)):
        evs = ev.create(2 * reps)
        for i in range(4):                      # warm-up, hook included
            L.moe_time_next_launch(R.MOE_K_READ_PROBE, evs[0], evs[1])
            R.read_probe(buf[(i % nwin) * size:], size, sink, blocks)
        torch.cuda.synchronize()
        for i in range(reps):
            L.moe_time_next_launch(R.MOE_K_READ_PROBE, evs[2 * i], evs[2 * i + 1])
            R.read_probe(buf[(i % nwin) * size:], size, sink, blocks)
        torch.cuda.synchronize()
        us = np.array([ev.elapsed_ms(evs[2 * i], evs[2 * i + 1]) for i in range(reps)]) * 1e3
        ev.destroy(evs)
        res[name] = {"GBs": size / float(np.median(us)) / 1e3, "median_us": float(np.median(us)), "launches": reps}
    del buf
    torch.cuda.empty_cache()
    return res


def stack_bench(args):
    """One token (or m) per step through a stack of `--layers` dim-4096 layers,
    all resident; the residual stream between layers runs on the device."""
    import numpy as np
    import torch

    import routing_quant_expert_amd as R
    import synth
    from synth.device import DeviceLayer

    n, m = args.layers, args.m
    specs = [synth.LayerSpec(synth.SHAPE_DS41, seed=args.seed, layer=l) for l in range(n)]
    s = specs[0].shape
    print(f"bench: generating {n} layers on the device", file=sys.stderr, flush=True)
    dls = [DeviceLayer(sp) for sp in specs]
    layers = [d.layer for d in dls]
    cfg = dls[0].cfg
    nt_tok = max(1, args.tokens)
    xs_all = torch.empty((nt_tok, n + 1, m, s.dim), dtype=torch.uint16, device="cuda")
    for t in range(nt_tok):
        x0 = synth.tokens(specs[0], t * m, m) if m == 1 else synth.correlated_tokens(specs[0], m, group=t)
        xs_all[t, 0] = torch.from_numpy(x0).cuda()
    ws = torch.empty(R.workspace_bytes(cfg, m), dtype=torch.uint8, device="cuda")
    R.workspace_init(cfg, m, ws)
    hdrs = torch.empty((n, m, R.header_words(cfg)), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    def step(i):
        R.stack_forward(cfg, layers, xs_all[i % nt_tok], ws, headers=hdrs)

    if args.graph:
        # one captured step per distinct input; before timing, each graph's
        # first replay must give the eager step's residual stream and headers
        ref = []
        for t in range(nt_tok):
            step(t)
            torch.cuda.synchronize()
            ref.append((xs_all[t].clone(), hdrs.clone()))
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        graphs = []
        with torch.cuda.stream(side):
            for t in range(nt_tok):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    R.stack_forward(cfg, layers, xs_all[t], ws, headers=hdrs, stream=side.cuda_stream)
                graphs.append(g)
        torch.cuda.synchronize()
        for t in range(nt_tok):
            xs_all[t, 1:].fill_(0)
            hdrs.fill_(0)
            graphs[t].replay()
            torch.cuda.synchronize()
            if not (torch.equal(xs_all[t], ref[t][0]) and torch.equal(hdrs, ref[t][1])):
                sys.exit(f"bench: graph replay of input {t} differs from the eager step")
        del ref

        def step(i):   # noqa: F811
            graphs[i % nt_tok].replay()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    K = args.steps
    t0 = time.perf_counter()
    for i in range(K):
        step(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall = t1 - t0
    layer_bytes = s.n_routed * s.dim * 2 + 3 * s.inter * s.dim * 2 + s.topk * (2 * s.gate_bytes + s.down_bytes)
    step_bytes = n * layer_bytes if m == 1 else None
    res = {
        "metric": "MoE-layer decode tokens/s at m=1 and % of HBM peak on expert-weight bytes",
        "value": K * m / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": f"moe_stack{n}_decode_m{m}_dim4096_inter2048_e384_top6", "layers": n, "m": m,
                   "launch": "graph replay" if args.graph else "eager",
                   "dim": s.dim, "inter": s.inter, "n_routed": s.n_routed, "topk": s.topk,
                   "resident_weight_bytes": n * (s.n_routed * s.expert_stride + 3 * s.inter * s.dim * 2 +
                                                 s.n_routed * s.dim * 2), "seed": args.seed},
        "detail": {"us_per_layer": wall * 1e6 / K / n},
    }
    if step_bytes:
        gbs = step_bytes / (wall / K) / 1e9
        res["roofline"] = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                           "frac": gbs / HBM_PEAK_GBS, "traffic": None, "kernel": "whole step (all launches)",
                           "bytes_per_launch": step_bytes}
    print(json.dumps(res), flush=True)


def cache_bench(args):
    """Decode through `--layers` dim-4096 layers whose routed experts live in
    pinned host memory, with an expert cache of `--cache-slots` device slots
    (the experts stream in over the host link on a miss); `--prefetch-k`
    predicted experts of the next layer are copied in ahead."""
    import numpy as np
    import torch

    import routing_quant_expert_amd as R
    import synth
    from synth.device import DeviceLayer, host_arena

    n, m = args.layers, args.m
    specs = [synth.LayerSpec(synth.SHAPE_DS41, seed=args.seed, layer=l) for l in range(n)]
    s = specs[0].shape
    print(f"bench: generating {n} layers, experts in pinned host memory ({n * s.n_routed * s.expert_stride / 1e9:.1f} GB)",
          file=sys.stderr, flush=True)
    scratch = torch.empty(s.n_routed * s.expert_stride, dtype=torch.uint8, device="cuda")
    hosts = [host_arena(sp, scratch) for sp in specs]
    del scratch
    torch.cuda.empty_cache()
    dls = [DeviceLayer(sp, experts_on_device=False) for sp in specs]
    cfg = dls[0].cfg
    cache = R.ExpertCache(cfg, hosts, s.expert_stride, s.gate_off, s.up_off, s.down_off, args.cache_slots, m)
    nt_tok = max(1, args.tokens)
    xs_all = torch.empty((nt_tok, n + 1, m, s.dim), dtype=torch.uint16, device="cuda")
    for t in range(nt_tok):
        xs_all[t, 0] = torch.from_numpy(synth.tokens(specs[0], t * m, m)).cuda()
    ws = torch.empty(R.workspace_bytes(cfg, m), dtype=torch.uint8, device="cuda")
    R.workspace_init(cfg, m, ws)
    layers = [d.layer for d in dls]
    torch.cuda.synchronize()
    for i in range(args.warmup):
        cache.forward(layers, xs_all[i % nt_tok], ws, prefetch_k=args.prefetch_k)
    torch.cuda.synchronize()
    st0 = cache.stats()
    K = args.steps
    t0 = time.perf_counter()
    for i in range(K):
        cache.forward(layers, xs_all[(args.warmup + i) % nt_tok], ws, prefetch_k=args.prefetch_k)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    st = {k: v - st0[k] for k, v in cache.stats().items()}
    cache.close()
    picks = st["hits"] + st["misses"]
    res = {
        "metric": "MoE-layer decode tokens/s at m=1 with the routed experts streamed from host memory",
        "value": K * m / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": f"moe_stack{n}_decode_m{m}_dim4096_inter2048_e384_top6_cache{args.cache_slots}"
                               f"_prefetch{args.prefetch_k}", "layers": n, "m": m, "cache_slots": args.cache_slots,
                   "prefetch_k": args.prefetch_k, "tokens_cycled": nt_tok, "host_expert_bytes": n * s.n_routed * s.expert_stride,
                   "seed": args.seed},
        "detail": {"stats": st, "hit_rate": st["hits"] / max(picks, 1),
                   "prefetch_used_rate": st["prefetch_used"] / max(st["prefetched"], 1),
                   "copied_bytes_per_step": st["bytes_copied"] / K,
                   "copy_gbs": st["bytes_copied"] / wall / 1e9},
    }
    print(json.dumps(res), flush=True)


def prefill_bench(args):
    """m > 8 tokens per step through the prefill kernels: the dim-4096 layer
    with the Zipf-skewed correction bias, m independent N(0,1) token rows."""
    import numpy as np
    import torch

    import routing_quant_expert_amd as R
    import synth
    from synth.device import DeviceLayer

    m = args.m
    spec = synth.LayerSpec(synth.SHAPE_DS41, seed=args.seed, zipf_bias=True, shared_quant=args.shared_quant)
    s = spec.shape
    shq = 1 if args.shared_quant else 0
    print(f"bench: generating the layer (dim {s.dim}, inter {s.inter}, {s.n_routed} experts, Zipf bias)",
          file=sys.stderr, flush=True)
    dl = DeviceLayer(spec)
    glibc = use_score_mode(args, dl)
    nb = max(1, min(args.tokens, 4))   # distinct batches cycled through
    if nb * m <= 4096:
        xs = torch.from_numpy(synth.tokens(spec, 0, nb * m)).cuda()
    else:   # large batches: the same rows generated on the device
        from synth.device import tokens_into
        xs = torch.empty((nb * m, s.dim), dtype=torch.uint16, device="cuda")
        tokens_into(spec, xs)
    ws = torch.empty(R.workspace_bytes(dl.cfg, m), dtype=torch.uint8, device="cuda")
    R.workspace_init(dl.cfg, m, ws)
    out = torch.empty((m, s.dim), dtype=torch.uint16, device="cuda")
    hw = R.header_words(dl.cfg)
    hdrs = torch.empty((nb, m, hw), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    def step(i):
        b = i % nb
        R.layer_forward(dl.cfg, dl.layer, xs[b * m:(b + 1) * m], out, ws, header=hdrs[b])

    ev = HipEvents()
    K = args.steps
    every = max(1, min(args.time_every, 2))
    nt = (K + every - 1) // every
    kinds = (("router", R.MOE_K_ROUTER), ("gateup", R.MOE_K_GATEUP), ("gateup2", R.MOE_K_GATEUP2),
             ("down", R.MOE_K_DOWN), ("down2", R.MOE_K_DOWN2), ("shared_gu", R.MOE_K_SHARED_GU),
             ("shared_down", R.MOE_K_SHARED_DOWN))
    if shq:   # the K-quant shared expert runs inside the expert launches: no bf16 shared GEMMs
        kinds = tuple(kv for kv in kinds if not kv[0].startswith("shared"))
    evs = {k: ev.create(2 * nt) for k, _ in kinds}
    scratch = {k: ev.create(2) for k, _ in kinds}
    L = R.lib()
    for i in range(args.warmup):   # the same event-bracketed dispatches as the timed loop
        if i % every == 0:
            for k, which in kinds:
                L.moe_time_next_launch(which, scratch[k][0], scratch[k][1])
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        if i % every == 0:
            j = i // every
            for k, which in kinds:
                L.moe_time_next_launch(which, evs[k][2 * j], evs[k][2 * j + 1])
        step(args.warmup + i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    k_ms = {k: np.array([ev.elapsed_ms(evs[k][2 * j], evs[k][2 * j + 1]) for j in range(nt)]) for k, _ in kinds}
    # the expert stage: its four launches (the experts with more than 8 pairs, then the others, on the caller's
    # stream), timed as the span from the first launch's start to the last one's end, each taken against the
    # router's start in the same step
    def at(k, j, end):
        return ev.elapsed_ms(evs["router"][2 * j], evs[k][2 * j + end])
    span_ms = np.array([max(at(k, j, 1) for k in ("gateup", "gateup2", "down", "down2")) -
                        min(at(k, j, 0) for k in ("gateup", "gateup2")) for j in range(nt)])
    for k, _ in kinds:
        ev.destroy(evs[k])
        ev.destroy(scratch[k])
    wall = t1 - t0
    picks = hdrs[:, :, 1:1 + s.topk].cpu().numpy()
    n_u = np.array([len(np.unique(p)) for p in picks])
    counts = np.bincount(picks[0].reshape(-1), minlength=s.n_routed)
    # the gate/up and the down stage are two launches each: the experts with at most 8 pairs, then the others
    split = {"gateup_small": float(k_ms["gateup"].mean()) * 1e3, "gateup_large": float(k_ms["gateup2"].mean()) * 1e3,
             "down_small": float(k_ms["down"].mean()) * 1e3, "down_large": float(k_ms["down2"].mean()) * 1e3}
    k_ms["gateup"] = k_ms["gateup"] + k_ms.pop("gateup2")
    k_ms["down"] = k_ms["down"] + k_ms.pop("down2")
    kinds = tuple(kv for kv in kinds if kv[0] not in ("gateup2", "down2"))
    us = {k: float(v.mean()) * 1e3 for k, v in k_ms.items()}
    nu = float(n_u.mean())
    pairs = m * s.topk
    nx = nu + shq        # expert groups the stage reads (the K-quant shared one included)
    px = pairs + shq * m  # (token, expert) pairs of the stage
    kbytes = {"router": s.n_routed * s.dim * 2, "gateup": nx * 2 * s.gate_bytes, "down": nx * s.down_bytes,
              "shared_gu": 2 * s.inter * s.dim * 2, "shared_down": s.inter * s.dim * 2}
    kops = {"router": 2 * m * s.n_routed * s.dim, "gateup": 2 * px * 2 * s.inter * s.dim,
            "down": 2 * px * s.dim * s.inter, "shared_gu": 2 * m * 2 * s.inter * s.dim,
            "shared_down": 2 * m * s.dim * s.inter}
    kern = {k: {"avg_us": us[k], "weight_bytes": kbytes[k], "gbs": kbytes[k] / us[k] / 1e3,
                "tops": kops[k] / us[k] / 1e6} for k, _ in kinds}
    launch_bytes = kbytes["gateup"] + kbytes["down"]
    launch_ops = kops["gateup"] + kops["down"]
    k_avg = float(span_ms.mean()) * 1e-3
    achieved = launch_bytes / k_avg / 1e9
    # the stage's bound: its weight bytes at the HBM peak, or its int8 work at the int8 MFMA peak, whichever
    # takes longer (a few thousand tokens move it from the first to the second)
    mfma_bound = launch_ops / (INT8_PEAK_TOPS * 1e12) > launch_bytes / (HBM_PEAK_GBS * 1e9)
    tops = launch_ops / k_avg / 1e12
    bound = ({"bound": "mfma", "achieved": tops, "peak": INT8_PEAK_TOPS, "unit": "TOP/s", "frac": tops / INT8_PEAK_TOPS}
             if mfma_bound else
             {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS})
    step_bytes = sum(v for k, v in kbytes.items() if not (shq and k.startswith("shared")))
    res = {
        "metric": (f"MoE-layer prefill tokens/s at m={m} and % of int8 MFMA peak on the expert stage's work"
                   if mfma_bound else f"MoE-layer prefill tokens/s at m={m} and % of HBM peak on expert-weight bytes"),
        "value": K * m / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall * 1e3 / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": f"moe_layer_prefill_m{m}_zipf_dim4096_inter2048_e384_top6" +
                               ("_shared_q2k_q3k" if shq else "") + ("_glibc_scores" if glibc else ""), "dim": s.dim,
                   "shared_expert": "Q2_K/Q3_K blocks" if shq else "bf16",
                   "scores": "glibc" if glibc else "correctly rounded",
                   "inter": s.inter, "n_routed": s.n_routed, "topk": s.topk, "m": m, "batches_cycled": nb,
                   "expert_arena_bytes": s.n_routed * s.expert_stride, "seed": args.seed},
        "roofline": {**bound,
                     "traffic": measured_traffic("expert stage", "hbm_traffic_prefill_m512_dim4096.md",
                                                 PREFILL_SOURCES) if m == 512 and not shq else None,
                     "kernel": "expert stage (k_gateup_pf, k_down_pf, k_gateup_pf_small, k_down_pf_small)",
                     "bytes_per_launch": launch_bytes, "avg_launch_us": k_avg * 1e6, "timed_launches": int(nt),
                     "launch_p10_p90_us": [float(np.percentile(span_ms, 10) * 1e3),
                                           float(np.percentile(span_ms, 90) * 1e3)],
                     "hbm_gbs": achieved, "int8_mfma_tops": tops, "int8_mfma_peak_tops": INT8_PEAK_TOPS},
        "detail": {"kernels": kern, "split_launch_us": split, "union_experts_mean": nu,
                   "largest_group": int(counts.max()),
                   "step_weight_bytes": step_bytes, "step_gbs": step_bytes / (wall / K) / 1e9,
                   "kernel_us_sum": sum(us.values()), "expert_stage_us": k_avg * 1e6,
                   "note": "the bf16 shared expert's GEMMs run on a second stream beside the router and selection: "
                           "their times include that sharing"},
    }
    if not args.no_cpu:
        print("bench: timing the oracle on the host", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(spec, args.cpu_seconds, "; the oracle defines each prefill token's output as its single-token output, so tokens/s of the two compare")
    print(json.dumps(res), flush=True)


def use_score_mode(args, dl) -> bool:
    """--score-mode glibc: register the glibc score table on the device and
    switch the layer's configuration to it (outside any timed region)."""
    if args.score_mode != "glibc":
        return False
    import routing_quant_expert_amd as R
    print("bench: building the glibc score table", file=sys.stderr, flush=True)
    R.enable_glibc_scores()
    dl.cfg.score_mode = R.MOE_SCORE_GLIBC
    return True


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--tokens", type=int, default=64, help="distinct input rows cycled through")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--time-every", type=int, default=2,
                    help="bracket every n-th step's gate/up dispatch with events (the same in warm-up and timed loop)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the read-only HBM streaming measurement")
    ap.add_argument("--cache-slots", type=int, default=0,
                    help="with --layers: stream the routed experts from pinned host memory through an expert cache of "
                         "this many device slots")
    ap.add_argument("--prefetch-k", type=int, default=0, help="with --cache-slots: predicted experts prefetched per token")
    ap.add_argument("--shared-quant", action="store_true",
                    help="the layer's shared expert as Q2_K/Q3_K blocks (run as one more expert) instead of bf16")
    ap.add_argument("--m", type=int, default=1, help="tokens per step (1: the single-token kernels; 2..8: the "
                                                     "multi-token decode path on correlated rows; > 8: the "
                                                     "prefill path, Zipf-skewed bias)")
    ap.add_argument("--layers", type=int, default=1,
                    help="decode through a stack of this many layers per step (each its own seeded weights)")
    ap.add_argument("--graph", action="store_true",
                    help="with --layers: replay each step from a captured graph (checked against eager first)")
    ap.add_argument("--score-mode", choices=("cr", "glibc"), default="cr",
                    help="router scores: correctly rounded (default) or the host glibc's, through the library's "
                         "exception table")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only copy 256 MiB device-to-device three times (calibrates the HBM byte counters)")
    args = ap.parse_args()
    if args.copy_probe:
        import torch
        src = torch.full((256 << 20,), 3, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(f"copied {src.numel()} bytes x3", flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py: the layer is measured on one GPU (asked for --gpus {args.gpus}); its sharding across "
              f"GPUs is a design note, not a measured path.", file=sys.stderr)
        sys.exit(2)
    if args.m < 1:
        print("bench.py: --m must be >= 1", file=sys.stderr)
        sys.exit(2)
    if args.m > 8:
        import torch
        torch.cuda.set_device(0)
        return prefill_bench(args)

    import numpy as np
    import torch

    import routing_quant_expert_amd as R
    import synth
    from synth.device import DeviceLayer

    torch.cuda.set_device(0)
    spec = synth.LayerSpec(synth.SHAPE_DS41, seed=args.seed, shared_quant=args.shared_quant)
    s = spec.shape
    m = args.m
    shq = 1 if args.shared_quant else 0
    print(f"bench: generating the layer (dim {s.dim}, inter {s.inter}, {s.n_routed} experts) on the device",
          file=sys.stderr, flush=True)
    if args.cache_slots > 0:
        return cache_bench(args)
    if args.layers > 1:
        return stack_bench(args)
    dl = DeviceLayer(spec)
    glibc = use_score_mode(args, dl)
    if m == 1:
        xs = torch.from_numpy(synth.tokens(spec, 0, args.tokens)).cuda()
    else:
        groups = [synth.correlated_tokens(spec, m, group=g) for g in range(args.tokens)]
        xs = torch.from_numpy(np.concatenate(groups)).cuda()
    ws = torch.empty(R.workspace_bytes(dl.cfg, m), dtype=torch.uint8, device="cuda")
    R.workspace_init(dl.cfg, m, ws)
    out = torch.empty((m, s.dim), dtype=torch.uint16, device="cuda")
    hw = R.header_words(dl.cfg)
    K = args.steps
    hdrs = torch.empty((K, m, hw), dtype=torch.int32, device="cuda")
    hdr_w = torch.empty((m, hw), dtype=torch.int32, device="cuda")
    torch.cuda.synchronize()

    # a step is one moe_layer_forward call through the C ABI; its arguments are marshalled once per cycled input
    L = R.lib()
    cfg_p, layer_p = ctypes.byref(dl.cfg), ctypes.byref(dl.layer)
    x_p = [ctypes.c_void_p(xs[t * m].data_ptr()) for t in range(args.tokens)]
    out_p, ws_p = ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr())
    ws_n = ctypes.c_size_t(ws.numel())
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    hdr_p = [ctypes.c_void_p(hdrs[i].data_ptr()) for i in range(K)]
    hdr_wp = ctypes.c_void_p(hdr_w.data_ptr())

    def step(i, hdr):
        rc = L.moe_layer_forward(cfg_p, layer_p, x_p[i % args.tokens], m, out_p, None, hdr, ws_p, ws_n, stream)
        if rc:
            raise R.MoeError(rc, L.moe_last_error().decode())

    # the box's read ceiling first: its streaming launches (a few ms) also bring the clocks up before the warm-up
    ceiling = None if args.no_ceiling else hbm_ceiling()
    ev = HipEvents()
    every = max(1, args.time_every)
    nt = (K + every - 1) // every
    evs = ev.create(2 * nt)
    scratch = ev.create(2)
    # warm-up: the same launches and the same event-bracketed dispatches as the timed loop
    for i in range(args.warmup):
        if i % every == 0:
            L.moe_time_next_launch(R.MOE_K_GATEUP, scratch[0], scratch[1])
        step(i, hdr_wp)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        if i % every == 0:          # every `every`-th step's gate/up dispatch records its own start and end
            j = i // every
            L.moe_time_next_launch(R.MOE_K_GATEUP, evs[2 * j], evs[2 * j + 1])
        step(args.warmup + i, hdr_p[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    gu_ms = np.array([ev.elapsed_ms(evs[2 * j], evs[2 * j + 1]) for j in range(nt)])
    ev.destroy(evs)

    # after the timed region: the three kernels of a further 64 steps, each bracketed on every second step
    kinds = (("front", R.MOE_K_ROUTER), ("gateup", R.MOE_K_GATEUP), ("down", R.MOE_K_DOWN))
    n_pass = 64
    kev = {k: ev.create(n_pass) for k, _ in kinds}
    for i in range(n_pass):
        if i % 2 == 0:
            for k, which in kinds:
                L.moe_time_next_launch(which, kev[k][i], kev[k][i + 1])
        step(args.warmup + K + i, hdr_wp)
    torch.cuda.synchronize()
    k_ms = {k: np.array([ev.elapsed_ms(kev[k][i], kev[k][i + 1]) for i in range(0, n_pass, 2)]) for k, _ in kinds}
    for k, _ in kinds:
        ev.destroy(kev[k])
    ev.destroy(scratch)

    wall = t1 - t0
    ms_per_step = wall * 1e3 / K
    router_bytes = s.n_routed * s.dim * 2
    # the shared expert: bf16 matrices, or (--shared-quant) K-quant blocks read as one more expert of the step
    shared_gu_bytes = 0 if shq else 2 * s.inter * s.dim * 2
    shared_down_bytes = 0 if shq else s.inter * s.dim * 2
    expert_bytes = 2 * s.gate_bytes + s.down_bytes
    us = {k: float(v.mean()) * 1e3 for k, v in k_ms.items()}
    sfx = ("_shared_q2k_q3k" if shq else "") + ("_glibc_scores" if glibc else "")
    if m == 1:
        kernel = "k_gateup_m1"
        n_u = np.full(1, s.topk)
        workload = f"moe_layer_decode_m1_dim4096_inter2048_e384_top6{sfx}"
    else:
        picks = hdrs[:, :, 1:1 + s.topk].cpu().numpy()
        n_u = np.array([len(np.unique(p)) for p in picks[::every]])   # the timed steps' unions
        kernel = "k_gateup"
        workload = f"moe_layer_decode_m{m}_correlated_dim4096_inter2048_e384_top6{sfx}"
    n_x = n_u.astype(np.float64) + shq   # experts whose blocks the step reads (the K-quant shared one included)
    if m == 1:   # the single-token launches: router | selection, routed + shared gate/up | down + combine
        kbytes = {"front": router_bytes,
                  "gateup": float(n_x.mean()) * 2 * s.gate_bytes + shared_gu_bytes,
                  "down": float(n_x.mean()) * s.down_bytes + shared_down_bytes}
    else:
        kbytes = {"front": router_bytes + shared_gu_bytes,
                  "gateup": float(n_x.mean()) * 2 * s.gate_bytes,
                  "down": float(n_x.mean()) * s.down_bytes + shared_down_bytes}
    launch_bytes = kbytes["gateup"]
    k_avg = float(gu_ms.mean()) * 1e-3
    extra = {"kernels_after_timed_region": {k: {"avg_us": us[k], "weight_bytes": kbytes[k],
                                                "gbs": kbytes[k] / us[k] / 1e3} for k, _ in kinds},
             "layer_weight_bytes": sum(kbytes.values()),
             "layer_kernels_us": sum(us.values()),
             "layer_kernels_gbs": sum(kbytes.values()) / sum(us.values()) / 1e3,
             "expert_kernels_gbs": (kbytes["gateup"] + kbytes["down"]) / (us["gateup"] + us["down"]) / 1e3,
             "step_gbs": sum(kbytes.values()) / (wall / K) / 1e9,
             "timing_note": f"every {every}-th step's gate/up dispatch carries start/end events, in the warm-up "
                            "and the timed loop alike; the per-kernel figures come from 64 further steps"}
    if m > 1:
        extra["union_experts_mean"] = float(n_u.mean())
    routed_bytes = float(n_u.mean()) * expert_bytes
    extra["routed_expert_bytes"] = routed_bytes
    achieved = launch_bytes / k_avg / 1e9
    res = {
        "metric": "MoE-layer decode tokens/s at m=1 and % of HBM peak on expert-weight bytes",
        "value": K * m / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "i8",
        "data": "synthetic",
        "config": {"workload": workload, "dim": s.dim, "inter": s.inter,
                   "n_routed": s.n_routed, "topk": s.topk, "m": m, "tokens_cycled": args.tokens,
                   "shared_expert": "Q2_K/Q3_K blocks" if shq else "bf16",
                   "scores": "glibc" if glibc else "correctly rounded",
                   "expert_arena_bytes": s.n_routed * s.expert_stride, "seed": args.seed},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS,
                     "traffic": (None if glibc else
                                 measured_traffic(kernel, "hbm_traffic_decode_m1_shared_kquant_dim4096.md")
                                 if shq and m == 1 else None if shq else measured_traffic(kernel) if m == 1 else
                                 measured_traffic(kernel, "hbm_traffic_decode_m8_dim4096.md", UNION_SOURCES) if m == 8
                                 else None), "kernel": kernel,
                     "bytes_per_launch": launch_bytes, "avg_launch_us": k_avg * 1e6, "timed_launches": int(nt),
                     "launch_p10_p90_us": [float(np.percentile(gu_ms, 10) * 1e3),
                                           float(np.percentile(gu_ms, 90) * 1e3)]},
        "detail": extra,
    }
    if ceiling:
        res["roofline"]["hbm_read_probe"] = ceiling
        res["roofline"]["frac_of_read_probe_64MiB"] = achieved / ceiling["64MiB"]["GBs"]
    if not args.no_cpu and m == 1:
        print("bench: timing the oracle on the host", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(spec, args.cpu_seconds)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
