"""moe_w4_block_noalloc (the block on the library's own device scratch, for callers
that cannot allocate) against moe_w4_block with a caller workspace, through the
C ABI.  Two calls in a row on the shared scratch, the second smaller: a
full-size T=300 call (grouped path: tiled router, tile queues in the scratch's
control block), then T=2 (the three-kernel decode block).  Routing must be
bit-identical, routing weights within 1e-5 and outputs within
max|a - b| / max|b| <= 1e-2.
"""
import numpy as np
import pytest
import torch

from w4_dequant_grouped_amd import moe_w4 as B
from w4_dequant_grouped_amd import synth

from parity_util import OUT_TOL, WEIGHT_TOL, make_inputs, note

pytestmark = pytest.mark.gpu

S = synth.BlockShape


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


def _compare(ra: B.Routing, oa: torch.Tensor, rb: B.Routing, ob: torch.Tensor, what: str) -> None:
    for name in ("ids", "counts", "offsets", "perm"):
        assert torch.equal(getattr(ra, name), getattr(rb, name)), f"{what}: {name} differ"
    werr = (ra.weights - rb.weights).abs().max().item()
    assert werr <= WEIGHT_TOL, f"{what}: routing weight difference {werr}"
    a = oa.float().cpu().numpy().astype(np.float64)
    b = ob.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(a).all(), f"{what}: non-finite output"
    err = float(np.abs(a - b).max() / np.abs(b).max())
    note(f"  {what}: max|noalloc - block| / max|block| = {err:.3e}")
    assert err <= OUT_TOL, f"{what}: relative difference {err}"


def test_noalloc_matches_block_on_two_calls_in_a_row():
    full = S(T=1, H=2048, I=512, E=256, top_k=8)
    layer = synth.draw_layer(full, 600)
    lg = layer.to("cuda")
    rs = B.weights_struct(lg.routed)
    ss = B.weights_struct(lg.shared)
    for T, seed in ((300, 601), (2, 602)):
        shape = S(T=T, H=2048, I=512, E=256, top_k=8)
        note(f"[gpu] noalloc vs block: {synth.describe(shape)} seed={seed}")
        _, x = make_inputs(shape, seed, layer)
        x = x.cuda()
        dims = B.make_dims(T, 2048, 512, 256, 8)
        ra, oa = B.alloc_routing(T, 256, 8), torch.empty((T, 2048), dtype=torch.bfloat16, device="cuda")
        B.moe_w4_block_noalloc(dims, x, lg.router_w, lg.router_b, rs, ss, ra, oa)
        rb, ob = B.alloc_routing(T, 256, 8), torch.empty_like(oa)
        ws = B.alloc_workspace(dims)
        B.moe_w4_block(dims, x, lg.router_w, lg.router_b, rs, ss, rb, ob, ws)
        torch.cuda.synchronize()
        _compare(ra, oa, rb, ob, f"T={T}")


def test_noalloc_rejects_a_shape_beyond_its_scratch():
    layer = synth.draw_layer(S(T=1, H=2048, I=512, E=256, top_k=8), 603).to("cuda")
    T = 2048
    x = torch.zeros((T, 2048), dtype=torch.bfloat16, device="cuda")
    r, out = B.alloc_routing(T, 256, 8), torch.empty((T, 2048), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(RuntimeError, match="-9"):
        B.moe_w4_block_noalloc(B.make_dims(T, 2048, 512, 256, 8), x, layer.router_w, None,
                               B.weights_struct(layer.routed), B.weights_struct(layer.shared), r, out)
