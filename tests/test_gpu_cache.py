"""GPU checks of the expert cache (experts streamed from host memory into a
fixed number of device slots) [device_route.rs, module doc, fn
route_device_m1; moe_v41.rs, module doc; fn prefetch_k]. The cache's forward
must give the resident stack's results bit for bit (residual stream, layer
outputs, picks and weights: the same kernels on the same values, only the
blocks' addresses differ); its headers add the miss flag and the picks'
slots. Evictions across layers and steps, prefetching, the union and
prefill paths, a K-quant shared expert and the too-few-slots error."""
import numpy as np
import pytest
import torch

import oracle
import routing_quant_expert_amd as R
import synth
from synth.device import DeviceLayer
from tests.gpu_helpers import say, to_np_u16, workspace

pytestmark = pytest.mark.gpu

TINY = synth.SHAPE_TINY


def host_arena(spec):
    """Every expert's raw blocks in pinned host memory (the arena layout of the device layer)."""
    s = spec.shape
    t = torch.empty(s.n_routed * s.expert_stride, dtype=torch.uint8, pin_memory=True)
    a = t.numpy()
    for e in range(s.n_routed):
        a[e * s.expert_stride:(e + 1) * s.expert_stride] = synth.expert_bytes(spec, e)
    return t


class Stack:
    def __init__(self, n, seed, shared_quant=False):
        self.specs = [synth.LayerSpec(TINY, seed=seed, layer=l, shared_quant=shared_quant) for l in range(n)]
        self.dls = [DeviceLayer(sp) for sp in self.specs]
        self.hosts = [host_arena(sp) for sp in self.specs]
        self.cfg = self.dls[0].cfg
        self.layers = [d.layer for d in self.dls]

    def cache(self, n_slots, max_m):
        s = TINY
        return R.ExpertCache(self.cfg, self.hosts, s.expert_stride, s.gate_off, s.up_off, s.down_off, n_slots, max_m)


def _run(stk, x0, cache=None, prefetch_k=0, ws=None):
    n, (m, dim) = len(stk.layers), x0.shape
    xs = torch.empty((n + 1, m, dim), dtype=torch.uint16, device="cuda")
    xs[0] = torch.from_numpy(x0).cuda()
    out = torch.empty((n, m, dim), dtype=torch.float32, device="cuda")
    hdr = torch.empty((n, m, R.header_words(stk.cfg)), dtype=torch.int32, device="cuda")
    ws = workspace(stk.cfg, m) if ws is None else ws
    if cache is None:
        R.stack_forward(stk.cfg, stk.layers, xs, ws, out_f32=out, headers=hdr)
    else:
        cache.forward(stk.layers, xs, ws, out_f32=out, headers=hdr, prefetch_k=prefetch_k)
    torch.cuda.synchronize()
    return to_np_u16(xs), out.cpu().numpy(), hdr.cpu().numpy()


def _same_as_resident(ref, got, topk):
    xs_r, out_r, h_r = ref
    xs_c, out_c, h_c = got
    assert np.array_equal(xs_c, xs_r)
    assert np.array_equal(out_c.view(np.uint32), out_r.view(np.uint32))
    assert np.array_equal(h_c[..., 1:1 + 2 * topk], h_r[..., 1:1 + 2 * topk])   # picks and weight bits
    slots = h_c[..., 1 + 2 * topk:]
    miss = (h_c[..., 0] & R.MOE_STATUS_MISS) != 0
    assert np.array_equal(miss, (slots < 0).any(axis=-1))                       # the miss flag
    assert np.array_equal(h_c[..., 0] & ~R.MOE_STATUS_MISS, h_r[..., 0])
    return slots, miss


@pytest.mark.parametrize("prefetch_k", [0, 3])
def test_cache_single_tokens_with_evictions(prefetch_k):
    """Six tokens, one at a time, through three layers with 10 slots (a step
    needs 18): every step evicts, results bit-equal to the resident stack."""
    stk = Stack(3, seed=41)
    cache = stk.cache(n_slots=10, max_m=1)
    try:
        ws = workspace(stk.cfg, 1)
        for t in range(6):
            x0 = synth.tokens(stk.specs[0], 300 + t, 1)
            say(f"cache prefetch_k={prefetch_k}: token {t}")
            _same_as_resident(_run(stk, x0), _run(stk, x0, cache, prefetch_k, ws), TINY.topk)
        st = cache.stats()
        say(f"  stats {st}")
        assert st["hits"] + st["misses"] == 6 * 3 * TINY.topk and st["reads_back"] == 6 * 3
        assert st["bytes_copied"] == (st["misses"] + st["prefetched"]) * TINY.expert_stride
        if prefetch_k:
            assert st["prefetched"] > 0
        else:
            assert st["prefetched"] == 0
    finally:
        cache.close()


def test_cache_hits_and_slots_in_the_header():
    """An empty cache: every pick misses (slot words -1, miss flag set); the
    same token again: every pick hits, the slot words are the picks' slots."""
    stk = Stack(2, seed=42)
    cache = stk.cache(n_slots=64, max_m=1)
    try:
        x0 = synth.tokens(stk.specs[0], 7, 1)
        ref = _run(stk, x0)
        slots, miss = _same_as_resident(ref, _run(stk, x0, cache), TINY.topk)
        assert miss.all() and (slots == -1).all()
        slots, miss = _same_as_resident(ref, _run(stk, x0, cache), TINY.topk)
        assert not miss.any()
        for l in range(2):
            res = cache.resident(l)
            plan = ref[2][l, 0, 1 + 2 * TINY.topk:]
            assert np.array_equal(slots[l, 0], res[plan])
        st = cache.stats()
        assert st["misses"] == 2 * TINY.topk and st["hits"] == 2 * TINY.topk
    finally:
        cache.close()


@pytest.mark.parametrize("m", [3, 40])
def test_cache_multi_token_and_prefill_paths(m):
    stk = Stack(2, seed=43)
    cache = stk.cache(n_slots=256, max_m=m)
    try:
        for rep in range(2):
            x0 = synth.tokens(stk.specs[0], 500 + 50 * rep, m)
            say(f"cache m={m} rep {rep}")
            _same_as_resident(_run(stk, x0), _run(stk, x0, cache, prefetch_k=2), TINY.topk)
    finally:
        cache.close()


def test_cache_kquant_shared_expert():
    stk = Stack(2, seed=44, shared_quant=True)
    cache = stk.cache(n_slots=24, max_m=3)
    try:
        for m in (1, 3):
            x0 = synth.tokens(stk.specs[0], 80, m)
            say(f"cache with a K-quant shared expert m={m}")
            _same_as_resident(_run(stk, x0), _run(stk, x0, cache), TINY.topk)
    finally:
        cache.close()


def test_cache_too_few_slots_is_an_error():
    stk = Stack(1, seed=45)
    cache = stk.cache(n_slots=4, max_m=1)
    try:
        with pytest.raises(R.MoeError) as ei:
            _run(stk, synth.tokens(stk.specs[0], 0, 1), cache)
        assert ei.value.code == -2
        torch.cuda.synchronize()
    finally:
        cache.close()
