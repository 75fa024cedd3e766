"""CPU checks of libmoe.so: it loads, exports every symbol include/moe.h
declares, rejects bad arguments before touching a GPU, and its own
arithmetic (the device score/SwiGLU code compiled for the host) matches the
oracle bit for bit."""
import os
import re

import numpy as np
import pytest

import oracle
import routing_quant_expert_amd as R
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "moe.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[\w\s\*]+?\b(moe_\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = _declared_functions()
    assert len(names) >= 10, names
    L = R.lib()
    missing = [n for n in names if not hasattr(L, n)]
    assert not missing, missing


def test_workspace_queries():
    c = R.cfg_from_shape(synth.SHAPE_DS41)
    n1, n8 = R.workspace_bytes(c, 1), R.workspace_bytes(c, 8)
    assert 0 < n1 < n8
    L = R.workspace_layout(c, 8)
    offs = [L[k] for k in ("ctl", "xq", "xd", "xs", "logits", "scores", "plan", "g", "u", "h", "hq", "hd", "hs",
                           "y", "sg", "su", "sh", "sd", "yr", "status", "grp", "xd64", "hd64")]
    assert all(o % 256 == 0 for o in offs) and offs == sorted(offs) and L["total"] == n8
    assert L["max_pairs"] == 56   # 8 tokens x (6 picks + a K-quant shared expert)
    assert R.header_words(c) == 19
    # the control words sit at the start for every m, so a workspace initialised for max_m serves smaller calls
    assert all(R.workspace_layout(c, m)["ctl"] == 0 for m in (1, 3, 8, 512))
    assert R.workspace_bytes(c, 512) > n8 and R.workspace_layout(c, 512)["max_pairs"] == 3584


@pytest.mark.parametrize("field,value", [("dim", 300), ("dim", 256 * 3), ("dim", 256 * 32), ("inter", 0),
                                         ("inter", 256 * 32), ("topk", 9), ("n_routed", 2000)])
def test_unsupported_shapes_are_rejected(field, value):
    c = R.cfg_from_shape(synth.SHAPE_TINY)
    setattr(c, field, value)
    assert R.workspace_bytes(c, 1) == 0
    with pytest.raises(R.MoeError) as ei:
        R.workspace_layout(c, 1)
    assert ei.value.code in (-1, -2)


class _FakePtr:
    """Stands in for a device tensor in calls that must fail validation."""

    def __init__(self, addr, n=1, shape=(1,)):
        self.addr, self.n, self.shape = addr, n, shape

    def data_ptr(self):
        return self.addr

    def numel(self):
        return self.n

    def element_size(self):
        return 1


def test_argument_errors_before_any_launch():
    c = R.cfg_from_shape(synth.SHAPE_TINY)
    need = R.workspace_bytes(c, 1)
    x = _FakePtr(4096, shape=(1, 512))
    small = _FakePtr(1 << 20, n=need - 256)
    with pytest.raises(R.MoeError) as ei:   # workspace too small
        R.route_select(c, x, _FakePtr(8192), _FakePtr(16384), _FakePtr(32768), small, stream=0)
    assert ei.value.code == -3
    with pytest.raises(R.MoeError) as ei:   # misaligned workspace
        R.route_select(c, x, _FakePtr(8192), _FakePtr(16384), _FakePtr(32768), _FakePtr((1 << 20) + 4, n=need),
                       stream=0)
    assert ei.value.code == -1
    with pytest.raises(R.MoeError) as ei:   # decode m > 8
        R.experts_decode(c, _FakePtr(4096, shape=(9, 512)), _FakePtr(8192), R.Experts(1 << 20, 0, 0, 0, 0),
                         _FakePtr(16384), _FakePtr(1 << 24, n=1 << 30), stream=0)
    assert ei.value.code == -1
    with pytest.raises(R.MoeError) as ei:   # misaligned expert arena
        R.experts_decode(c, x, _FakePtr(8192), R.Experts((1 << 20) + 8, 0, 0, 0, 0), _FakePtr(16384),
                         _FakePtr(1 << 24, n=1 << 30), stream=0)
    assert ei.value.code == -1
    with pytest.raises(R.MoeError) as ei:   # prefill: misaligned expert arena
        R.experts_prefill(c, _FakePtr(4096, shape=(64, 512)), _FakePtr(8192), R.Experts((1 << 20) + 8, 0, 0, 0, 0),
                          _FakePtr(16384), _FakePtr(1 << 24, n=1 << 30), stream=0)
    assert ei.value.code == -1
    with pytest.raises(R.MoeError) as ei:   # prefill: workspace sized for fewer tokens
        R.experts_prefill(c, _FakePtr(4096, shape=(64, 512)), _FakePtr(8192), R.Experts(1 << 20, 0, 0, 0, 0),
                          _FakePtr(16384), _FakePtr(1 << 24, n=R.workspace_bytes(c, 63)), stream=0)
    assert ei.value.code == -3


def test_library_score_chain_matches_oracle_on_host():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.normal(0, 1.28, 400_000), rng.uniform(-110, 25, 300_000), rng.normal(0, 8, 100_000),
                        np.ldexp(rng.uniform(-1, 1, 100_000), rng.integers(-140, 5, 100_000))]).astype(np.float32)
    want = oracle.scores(x, 1.0)
    for flags in (0, 1):           # 1: every exp/log1p through the double-double path
        got = R.scores_host(x, 1.0, flags)
        bad = np.nonzero(got.view(np.uint32) != want.view(np.uint32))[0]
        assert bad.size == 0, (flags, x[bad[:5]], got[bad[:5]], want[bad[:5]])
    got = R.scores_host(x[:100_000], 0.7)
    assert np.array_equal(got.view(np.uint32), oracle.scores(x[:100_000], 0.7).view(np.uint32))


def test_library_exp_step_matches_oracle_on_host():
    """The exp step (flags bit 2) on one input in 2,000 of every f32 in
    [-104, 89] plus the ends: the straight-line estimate with Ziv's test
    equals the extended path and the oracle's correctly rounded exp."""
    lo, hi = np.float32(-104.0).view(np.uint32), np.float32(89.0).view(np.uint32)
    neg = np.arange(0x80000000, lo + 1, 2000, dtype=np.uint64).astype(np.uint32)
    pos = np.arange(0, hi + 1, 2000, dtype=np.uint64).astype(np.uint32)
    x = np.concatenate([neg.view(np.float32), pos.view(np.float32),
                        np.array([-104.0, 89.0, 20.0, 20.000002, -87.33655, -0.0, 1e-45, -1e-45], np.float32)])
    fast = R.scores_host(x, 1.0, R.SCORES_EXP_ONLY)
    slow = R.scores_host(x, 1.0, R.SCORES_EXP_ONLY | R.SCORES_EXTENDED)
    assert np.array_equal(fast.view(np.uint32), slow.view(np.uint32))
    want = oracle.exp_cr(x)
    bad = np.nonzero(fast.view(np.uint32) != want.view(np.uint32))[0]
    assert bad.size == 0, (x[bad[:5]], fast[bad[:5]], want[bad[:5]])
    with pytest.raises(R.MoeError):
        R.scores_host(x[:4], 1.0, R.SCORES_EXP_ONLY | R.SCORES_GLIBC)
    # another temperature: the step's input is RN32(logit / temp)
    lg = np.random.default_rng(8).normal(0, 6, 50_000).astype(np.float32)
    z = (lg.astype(np.float64) / np.float64(np.float32(0.7))).astype(np.float32)
    assert np.array_equal(R.scores_host(lg, 0.7, R.SCORES_EXP_ONLY).view(np.uint32), oracle.exp_cr(z).view(np.uint32))


def test_library_swiglu_matches_oracle_on_host():
    rng = np.random.default_rng(6)
    g = np.concatenate([rng.normal(0, 2, 200_000), rng.uniform(-120, 20, 50_000)]).astype(np.float32)
    u = rng.normal(0, 4, g.size).astype(np.float32)
    assert np.array_equal(R.swiglu_host(g, u, 7.0).view(np.uint32), oracle.swiglu(g, u, 7.0).view(np.uint32))


def test_empty_batch_is_rejected_by_every_entry_point():
    """m = 0 is out of range for every call (MOE_EINVAL, checked before any
    launch); so is a stack of zero layers."""
    c = R.cfg_from_shape(synth.SHAPE_TINY)
    ws = _FakePtr(1 << 20, n=1 << 30)
    x0 = _FakePtr(4096, shape=(0, 512))
    ex = R.Experts(1 << 20, 0, 0, 0, 0)
    layer = R.Layer(8192, 16384, ex, 1 << 21, 1 << 22, 1 << 23)
    calls = [
        lambda: R.route_select(c, x0, _FakePtr(8192), _FakePtr(16384), _FakePtr(32768), ws, stream=0),
        lambda: R.experts_decode(c, x0, _FakePtr(8192), ex, _FakePtr(16384), ws, stream=0),
        lambda: R.experts_prefill(c, x0, _FakePtr(8192), ex, _FakePtr(16384), ws, stream=0),
        lambda: R.layer_forward(c, layer, x0, _FakePtr(16384), ws, stream=0),
        lambda: R.stack_forward(c, [layer], _FakePtr(4096, shape=(2, 0, 512)), ws, stream=0),
        lambda: R.stack_forward(c, [], _FakePtr(4096, shape=(1, 1, 512)), ws, stream=0),
    ]
    for i, call in enumerate(calls):
        with pytest.raises(R.MoeError) as ei:
            call()
        assert ei.value.code == -1, i
    assert R.workspace_bytes(c, 0) == 0


def test_token_count_bound_is_enforced_before_any_launch():
    """The kernels index per-pair activations with 32-bit offsets and put
    tokens on a grid dimension: m above 65535, or with m * (topk + 1) *
    max(dim, inter) >= 2^31 (topk + 1: a K-quant shared expert is one more
    entry per token), is MOE_EUNSUPPORTED for every entry point, and
    the workspace size query returns 0 there."""
    ex = R.Experts(1 << 20, 0, 0, 0, 0)
    layer = R.Layer(8192, 16384, ex, 1 << 21, 1 << 22, 1 << 23)
    ws = _FakePtr(1 << 24, n=1 << 40)
    for shape, m in ((synth.SHAPE_TINY, 65536), (synth.SHAPE_DS41, 74899)):
        c = R.cfg_from_shape(shape)
        assert R.workspace_bytes(c, m) == 0
        x = _FakePtr(4096, shape=(m, shape.dim))
        calls = [
            lambda: R.workspace_layout(c, m),
            lambda: R.route_select(c, x, _FakePtr(8192), _FakePtr(16384), _FakePtr(32768), ws, stream=0),
            lambda: R.experts_prefill(c, x, _FakePtr(8192), ex, _FakePtr(16384), ws, stream=0),
            lambda: R.layer_forward(c, layer, x, _FakePtr(16384), ws, stream=0),
            lambda: R.stack_forward(c, [layer], _FakePtr(4096, shape=(2, m, shape.dim)), ws, stream=0),
        ]
        for i, call in enumerate(calls):
            with pytest.raises(R.MoeError) as ei:
                call()
            assert ei.value.code == -2, (shape.dim, i)
    # the largest accepted counts still size a workspace
    assert R.workspace_bytes(R.cfg_from_shape(synth.SHAPE_TINY), 65535) > 0
    assert R.workspace_bytes(R.cfg_from_shape(synth.SHAPE_DS41), 65535) > 0
