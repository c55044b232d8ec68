"""GPU parity of decode attention over a paged KV cache, through the C ABI.

Every case compares moe_w4_attn_decode with the float64 oracle on the same seeded
inputs.  Tolerance: max|gpu - ref| / max|ref| <= 5e-3.  The output is rounded
once to bf16 (round to nearest moves a value by at most half an ulp, 2^-8 ~
3.9e-3 of itself); the softmax weights enter the p.V sums rounded to bf16 too,
but their rounding errors average out over the keys; scores and sums are fp32.
"""
import numpy as np
import pytest
import torch

from oracle import attn_oracle as A
from w4_dequant_grouped_amd import moe_w4 as B
from w4_dequant_grouped_amd import synth_attn as SA

pytestmark = pytest.mark.gpu

TOL = 5e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


def note(msg):
    print(msg, flush=True)


def run(shape, x_cpu):
    x = x_cpu.to("cuda")
    step = B.AttnDecode(shape, x)
    out = step()
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), step


def check(shape, seed, what, x=None):
    note(f"[gpu-attn] {what}: n_ctx={shape.n_ctx} Hq={shape.n_q_heads} Hkv={shape.n_kv_heads} seed={seed}")
    x = x if x is not None else SA.draw_attn(shape, seed)
    got, _ = run(shape, x)
    ref = A.decode_attention(x.q, x.k_pool, x.v_pool, x.table, shape.n_ctx)
    err = A.relative_error(got, ref)
    note(f"  max|gpu-ref|/max|ref| = {err:.3e}")
    assert np.isfinite(got).all(), what
    assert err <= TOL, f"{what}: {err}"
    return err


def test_tiny():
    shape, seed = SA.ATTN_WORKLOADS["tiny"]
    check(shape, seed, "tiny")


@pytest.mark.parametrize("n_ctx", [1, 2, 63, 64, 65, 200, 257, 1000, 4097])
def test_ragged_contexts(n_ctx):
    check(SA.AttnShape(n_ctx=n_ctx), 100 + n_ctx, f"ragged {n_ctx}")


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 4), (16, 1), (6, 3), (12, 1), (64, 8)])
def test_group_sizes(Hq, Hkv):
    # the pages also speak of four query heads per group; G = 1, 2, 4, 8, 12, 16
    check(SA.AttnShape(n_ctx=777, n_q_heads=Hq, n_kv_heads=Hkv), 200 + Hq + Hkv, f"G={Hq // Hkv}")


def test_nan_in_unused_slots_and_blocks():
    shape = SA.AttnShape(n_ctx=1000, poison_tail=True)
    x = SA.draw_attn(shape, 300)
    assert torch.isnan(x.k_pool.float()).any()
    check(shape, 300, "poisoned tail", x)


def test_dominant_key():
    shape = SA.AttnShape(n_ctx=5000)
    x = SA.draw_attn(shape, 301)
    n_star = 3210
    phys, slot = int(x.table[n_star // 64]), n_star % 64
    # cache head 1, aligned with query head 8 (first head of group 1)
    x.k_pool[phys, 1, slot] = (8 * x.q[8].float()).to(torch.bfloat16)
    err = check(shape, 301, "dominant key", x)
    got, _ = run(shape, x)
    v_star = x.v_pool[phys, 1, slot].double().numpy()
    assert np.abs(got[8] - v_star).max() <= 0.02 * np.abs(v_star).max()
    assert err <= TOL


@pytest.mark.parametrize("name", ["ctx32k", "ctx128k"])
def test_long_contexts(name):
    shape, seed = SA.ATTN_WORKLOADS[name]
    check(shape, seed, name)


def test_split_size_boundary():
    # 1025 blocks: the first context that takes 8 blocks per workgroup
    check(SA.AttnShape(n_ctx=1025 * 64 - 5), 302, "8 blocks per workgroup")


def test_repeat_calls_are_bitwise_identical():
    shape = SA.AttnShape(n_ctx=20000)
    x = SA.draw_attn(shape, 303).to("cuda")
    step = B.AttnDecode(shape, x)
    a = step().clone()
    b = step().clone()
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_graph_replays_match_eager():
    shape = SA.AttnShape(n_ctx=9000)
    x = SA.draw_attn(shape, 304).to("cuda")
    step = B.AttnDecode(shape, x)
    eager = step().clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    q2 = x.q.clone()
    for r in range(3):
        step.out.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(step.out, eager), r
        x.q.copy_(torch.flip(q2, [0]))        # eager work on other inputs in between
        step()
        torch.cuda.synchronize()
        x.q.copy_(q2)
