"""GPU parity of the Gated DeltaNet scan, through the C ABI.

Every case compares moe_w4_gdn_scan (the register-resident scan) or
moe_w4_gdn_scan_chunked (the chunked MFMA form) with the float64 oracle on the
same seeded inputs.  Outputs: max|gpu - ref| / max|ref| <= 5e-3 (one round-to-nearest to
bf16 moves a value by at most half an ulp, 2^-8 ~ 3.9e-3 of itself; the fp32
recurrence adds errors near 1e-6).  Final state:
<= 1e-4 (fp32 throughout; the decay forgets old rounding errors within a few
dozen tokens).  The chunked form splits fp32 operands into bf16 hi + lo pairs,
about 16 significant bits per product term, inside the same state bound.
"""
import numpy as np
import pytest
import torch

from oracle import gdn_oracle as D
from w4_dequant_grouped_amd import moe_w4 as B
from w4_dequant_grouped_amd import synth_gdn as SG

pytestmark = pytest.mark.gpu

OUT_TOL = 5e-3
STATE_TOL = 1e-4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


def gpu_scan(x, chunked=False):
    g = x.to("cuda")
    out = torch.empty_like(g.v)
    state = g.state.clone()
    scan = B.moe_w4_gdn_scan_chunked if chunked else B.moe_w4_gdn_scan
    scan(g.q, g.k, g.v, g.g, g.beta, state, out)
    torch.cuda.synchronize()
    return out, state


def check(shape, seed, what, chunked=False):
    what = f"{'chunked ' if chunked else ''}{what}"
    print(f"[gpu-gdn] {what}: T={shape.T} Hv={shape.n_v_heads} Hk={shape.n_k_heads} seed={seed}", flush=True)
    x = SG.draw_gdn(shape, seed)
    out, state = gpu_scan(x, chunked)
    ref_o, ref_s = D.gdn_scan(x.q, x.k, x.v, x.g, x.beta, x.state)
    got_o = out.float().cpu().numpy().astype(np.float64)
    got_s = state.cpu().numpy().astype(np.float64)
    eo, es = D.relative_error(got_o, ref_o), D.relative_error(got_s, ref_s)
    print(f"  out {eo:.3e}  state {es:.3e}", flush=True)
    assert np.isfinite(got_o).all() and np.isfinite(got_s).all()
    assert eo <= OUT_TOL, f"{what}: output error {eo}"
    assert es <= STATE_TOL, f"{what}: state error {es}"


def test_tiny():
    shape, seed = SG.GDN_WORKLOADS["tiny"]
    check(shape, seed, "tiny")


@pytest.mark.parametrize("T", [1, 2, 31, 32, 33, 100])
def test_chunk_boundaries(T):
    check(SG.GdnShape(T=T), 400 + T, f"T={T}")


@pytest.mark.parametrize("Hv,Hk", [(8, 8), (8, 2), (6, 3)])
def test_head_mappings(Hv, Hk):
    check(SG.GdnShape(T=77, n_v_heads=Hv, n_k_heads=Hk), 500 + Hv + Hk, f"Hv={Hv} Hk={Hk}")


@pytest.mark.parametrize("name", ["decode", "prefill512", "prefill2048"])
def test_workloads(name):
    shape, seed = SG.GDN_WORKLOADS[name]
    check(shape, seed, name)


def test_split_sequence_is_bitwise_identical():
    # two calls with the state carried through memory give exactly the one-call result
    x = SG.draw_gdn(SG.GdnShape(T=300), 600).to("cuda")
    out1 = torch.empty_like(x.v)
    s1 = x.state.clone()
    B.moe_w4_gdn_scan(x.q, x.k, x.v, x.g, x.beta, s1, out1)
    out2 = torch.empty_like(x.v)
    s2 = x.state.clone()
    for a, b in ((0, 123), (123, 300)):
        o = torch.empty_like(x.v[a:b])
        B.moe_w4_gdn_scan(x.q[a:b].contiguous(), x.k[a:b].contiguous(), x.v[a:b].contiguous(),
                          x.g[a:b].contiguous(), x.beta[a:b].contiguous(), s2, o)
        out2[a:b] = o
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(s1, s2)


def test_zero_tokens_leave_the_state():
    x = SG.draw_gdn(SG.GdnShape(T=1), 601).to("cuda")
    s = x.state.clone()
    e = lambda n: torch.empty((0,) + n, device="cuda")   # noqa: E731
    B.moe_w4_gdn_scan(e((16, 128)).bfloat16(), e((16, 128)).bfloat16(), e((32, 128)).bfloat16(),
                      e((32,)).float(), e((32,)).float(), s, e((32, 128)).bfloat16())
    torch.cuda.synchronize()
    assert torch.equal(s, x.state)


def test_graph_replays_match_eager():
    x = SG.draw_gdn(SG.GdnShape(T=64), 602).to("cuda")
    out = torch.empty_like(x.v)
    state = x.state.clone()

    def step():
        state.copy_(x.state)
        B.moe_w4_gdn_scan(x.q, x.k, x.v, x.g, x.beta, state, out)

    step()
    torch.cuda.synchronize()
    ref_o, ref_s = out.clone(), state.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step()
    for r in range(3):
        out.zero_()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(state, ref_s), r
        x.v.mul_(-1.0)           # eager work on other inputs in between
        step()
        torch.cuda.synchronize()
        x.v.mul_(-1.0)


# --- the chunked MFMA form ---------------------------------------------------------

def test_chunked_tiny():
    shape, seed = SG.GDN_WORKLOADS["tiny"]
    check(shape, seed, "tiny", chunked=True)


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 100, 1000, 2047, 2048, 2049])
def test_chunked_chunk_and_segment_boundaries(T):
    # 64-token chunks, 2048-token segments (two launches each); a lone token past both
    check(SG.GdnShape(T=T), 700 + T, f"T={T}", chunked=True)


@pytest.mark.parametrize("Hv,Hk", [(8, 8), (8, 2), (6, 3)])
def test_chunked_head_mappings(Hv, Hk):
    check(SG.GdnShape(T=130, n_v_heads=Hv, n_k_heads=Hk), 800 + Hv + Hk, f"Hv={Hv} Hk={Hk}", chunked=True)


@pytest.mark.parametrize("name", ["prefill512", "prefill2048"])
def test_chunked_workloads(name):
    shape, seed = SG.GDN_WORKLOADS[name]
    check(shape, seed, name, chunked=True)


def test_chunked_split_sequence_carries_the_state():
    """Two chunked calls with the state carried through memory (the split falls
    inside a chunk) give the one-call result within the tolerances."""
    x = SG.draw_gdn(SG.GdnShape(T=300), 900).to("cuda")
    out1 = torch.empty_like(x.v)
    s1 = x.state.clone()
    B.moe_w4_gdn_scan_chunked(x.q, x.k, x.v, x.g, x.beta, s1, out1)
    out2 = torch.empty_like(x.v)
    s2 = x.state.clone()
    for a, b in ((0, 123), (123, 300)):
        o = torch.empty_like(x.v[a:b])
        B.moe_w4_gdn_scan_chunked(x.q[a:b].contiguous(), x.k[a:b].contiguous(), x.v[a:b].contiguous(),
                                  x.g[a:b].contiguous(), x.beta[a:b].contiguous(), s2, o)
        out2[a:b] = o
    torch.cuda.synchronize()
    eo = (out1.float() - out2.float()).abs().max().item() / out1.float().abs().max().item()
    es = (s1 - s2).abs().max().item() / s1.abs().max().item()
    assert eo <= OUT_TOL and es <= STATE_TOL, (eo, es)


def test_chunked_workspace_size_and_graph_replays():
    """The workspace the library asks for (one 2048-token segment at most), and
    three graph replays of a chunked call equal to the eager call bit for bit."""
    # per chunk: 20608 words per value head (-W, Pm and Vt fragments, gamma, d) and
    # 8192 per key head (K^T and Q fragments)
    per_chunk = (32 * 20608 + 16 * 8192) * 4
    assert B.moe_w4_gdn_chunked_workspace_bytes(1, 32, 16) == per_chunk
    assert B.moe_w4_gdn_chunked_workspace_bytes(5000, 32, 16) == 32 * per_chunk
    x = SG.draw_gdn(SG.GdnShape(T=200), 901).to("cuda")
    out = torch.empty_like(x.v)
    state = x.state.clone()
    ws = torch.empty(B.moe_w4_gdn_chunked_workspace_bytes(200, 32, 16), dtype=torch.uint8, device="cuda")

    def step():
        state.copy_(x.state)
        B.moe_w4_gdn_scan_chunked(x.q, x.k, x.v, x.g, x.beta, state, out, ws)

    step()
    torch.cuda.synchronize()
    ref_o, ref_s = out.clone(), state.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        step()
    for r in range(3):
        out.zero_()
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(state, ref_s), r
