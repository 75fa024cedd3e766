"""GPU check of the entry point that allocates nothing
(moe_layer_forward_noalloc, for callers that cannot allocate): through the
C ABI, its output must equal the workspace entry point's (moe_layer_forward)
on the same inputs: headers bit for bit and the layer output bit for bit
(the same kernels run, only the workspace differs), which puts it within the
oracle's bar as well. Two calls in a row on one GPU, the second with fewer
tokens (the fixed scratch keeps the first call's contents), at dim 512 and
4096, plus the rejection of m outside 1..8."""
import numpy as np
import pytest
import torch

import routing_quant_expert_amd as R
import synth
from oracle import layer as olayer
from synth.device import DeviceLayer
from tests.gpu_helpers import rel_l2, say, to_np_u16, workspace

pytestmark = pytest.mark.gpu


def _forward(dl, x, noalloc):
    c, dim = dl.cfg, dl.spec.shape.dim
    m = x.shape[0]
    out = torch.full((m, dim), 0x7FC0, dtype=torch.uint16, device="cuda")
    out32 = torch.full((m, dim), float("nan"), dtype=torch.float32, device="cuda")
    hdr = torch.full((m, R.header_words(c)), -7, dtype=torch.int32, device="cuda")
    if noalloc:
        R.layer_forward_noalloc(c, dl.layer, x, out, out_f32=out32, header=hdr)
    else:
        R.layer_forward(c, dl.layer, x, out, workspace(c, m), out_f32=out32, header=hdr)
    torch.cuda.synchronize()
    return hdr.cpu().numpy(), out32.cpu().numpy(), to_np_u16(out)


@pytest.mark.parametrize("shape", [synth.SHAPE_TINY, synth.SHAPE_DS41], ids=lambda s: f"dim{s.dim}")
def test_noalloc_equals_workspace_entry_point(shape):
    spec = synth.LayerSpec(shape, seed=6)
    say(f"no-alloc entry point: generating layer dim {shape.dim}")
    dl = DeviceLayer(spec)
    try:
        for m, t0 in ((8, 0), (3, 50), (1, 90)):     # consecutive calls, each smaller than the one before
            x_np = synth.tokens(spec, t0, m)
            x = torch.from_numpy(x_np).cuda()
            say(f"  m={m}")
            h_n, o_n, b_n = _forward(dl, x, True)
            h_w, o_w, b_w = _forward(dl, x, False)
            assert np.array_equal(h_n, h_w), m
            assert np.array_equal(o_n.view(np.uint32), o_w.view(np.uint32)), m
            assert np.array_equal(b_n, b_w), m
            if shape == synth.SHAPE_TINY:
                ref = olayer.layer_forward(spec, x_np)
                assert np.array_equal(h_n, ref["header"])
                for t in range(m):
                    assert rel_l2(o_n[t], ref["out_f32"][t]) <= 1e-3
                    assert np.abs(o_n[t] - ref["out_f32"][t]).max() <= 1e-2
        # token counts outside 1..8 are refused before any launch
        for m in (0, 9):
            x = torch.zeros((max(m, 1), shape.dim), dtype=torch.uint16, device="cuda")[:m]
            out = torch.empty((max(m, 1), shape.dim), dtype=torch.uint16, device="cuda")
            with pytest.raises(R.MoeError) as ei:
                R.layer_forward_noalloc(dl.cfg, dl.layer, x, out)
            assert ei.value.code == -1
    finally:
        del dl
        torch.cuda.empty_cache()
