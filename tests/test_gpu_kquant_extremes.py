"""Layer outputs on K-quant blocks at the ends of their ranges, against the
oracle on the same bytes: Q2_K sub-block scales and mins of 15 (every byte
0xFF, or random scales under mins of 15), Q3_K 6-bit scales of 63 and 0 (the
signed extremes +31 and -32) or random, hmask all clear or all set, and
tokens whose q8_1 codes are +127 throughout (per-16 code sums of 2,032, the
largest the activation sums take) or +-127 with random signs. The
single-token kernels (m = 1), the multi-token ones (m = 5) and the prefill
ones (m = 40) all run [k-quant block formats: Q2_K 84 bytes (scales[16], qs[64], d, dmin), Q3_K
110 bytes (hmask[32], qs[64], scales[12], d)]."""
import numpy as np
import pytest
import torch

import oracle
import routing_quant_expert_amd as R
import synth
from synth.device import DeviceLayer
from tests.gpu_helpers import rel_l2, say, to_np_u16, workspace

pytestmark = pytest.mark.gpu

Q2K, Q3K = 84, 110


def _craft(host: np.ndarray, shape, rng) -> None:
    """Rewrite every routed expert's blocks in the host arena (d and dmin kept)."""
    s = shape
    nsb_gu, nsb_dn = s.dim // 256, s.inter // 256
    for e in range(s.n_routed):
        base = e * s.expert_stride
        for off in (s.gate_off, s.up_off):
            b = host[base + off: base + off + s.inter * nsb_gu * Q2K].reshape(-1, Q2K)
            if e % 2 == 0:
                b[:, :16] = 0xFF                                               # scale 15, min 15
            else:
                b[:, :16] = 0xF0 | rng.integers(0, 16, (b.shape[0], 16), dtype=np.uint8)   # min 15
            b[:, 16:80] = rng.integers(0, 256, (b.shape[0], 64), dtype=np.uint8)
        d = host[base + s.down_off: base + s.down_off + s.dim * nsb_dn * Q3K].reshape(-1, Q3K)
        d[:, :32] = 0x00 if e % 4 < 2 else 0xFF                                 # hmask
        d[:, 32:96] = rng.integers(0, 256, (d.shape[0], 64), dtype=np.uint8)
        if e % 3 == 0:
            d[:, 96:108] = 0xFF                                                 # every 6-bit scale 63
        elif e % 3 == 1:
            d[:, 96:108] = 0x00                                                 # every 6-bit scale 0
        else:
            d[:, 96:108] = rng.integers(0, 256, (d.shape[0], 12), dtype=np.uint8)


def _tokens(shape, m, rng) -> np.ndarray:
    x = np.full((m, shape.dim), 0.5, np.float32)
    for t in range(1, m, 2):
        x[t] *= np.where(rng.random(shape.dim) < 0.5, -1.0, 1.0)
    return oracle.f32_to_bf16(x)


@pytest.fixture(scope="module")
def crafted_layer():
    sh = synth.SHAPE_TINY
    rng = np.random.default_rng(43)
    say("generating and rewriting a small layer's expert blocks")
    dl = DeviceLayer(synth.LayerSpec(sh, seed=43))
    host = dl.arena.cpu().numpy().copy()
    _craft(host, sh, rng)
    dl.arena.copy_(torch.from_numpy(host))
    torch.cuda.synchronize()
    gw = oracle.f32_to_bf16(rng.normal(0.0, 0.05, (sh.n_routed, sh.dim)).astype(np.float32))
    return sh, dl, host, gw, rng


@pytest.mark.parametrize("m", [1, 5, 40])
def test_layer_on_kquant_range_ends(crafted_layer, m):
    sh, dl, host, gw, rng = crafted_layer
    x = _tokens(sh, m, rng)
    bias = np.zeros(sh.n_routed, np.float32)
    c = R.cfg_from_shape(sh)
    gwd = torch.from_numpy(gw.view(np.int16)).cuda()
    bd = torch.from_numpy(bias).cuda()
    L = R.Layer.from_buffer_copy(dl.layer)
    L.gate_w, L.bias = gwd.data_ptr(), bd.data_ptr()
    ob = torch.empty((m, sh.dim), dtype=torch.uint16, device="cuda")
    of = torch.empty((m, sh.dim), dtype=torch.float32, device="cuda")
    hdr = torch.empty((m, R.header_words(c)), dtype=torch.int32, device="cuda")
    xd = torch.from_numpy(x.view(np.int16)).cuda()
    say(f"layer on crafted blocks m={m}")
    R.layer_forward(c, L, xd, ob, workspace(c, m), out_f32=of, header=hdr)
    torch.cuda.synchronize()
    rb, rf, rh = oracle.ref_layer_forward(sh, x, gw, bias, host, sh.expert_stride, sh.gate_off, sh.up_off,
                                          sh.down_off,
                                          shared_bf16=tuple(to_np_u16(t) for t in (dl.sh_w1, dl.sh_w3, dl.sh_w2)))
    assert np.array_equal(hdr.cpu().numpy(), rh)
    got = of.cpu().numpy()
    assert np.all(np.isfinite(got))
    for t in range(m):
        assert rel_l2(got[t], rf[t]) <= 1e-3 and np.abs(got[t] - rf[t]).max() <= 1e-2 * max(1.0, np.abs(rf[t]).max()), t
