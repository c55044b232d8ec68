"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Block calls go through moe_w4_block (route + forward in one library call); the
split tests call moe_w4_route and moe_w4_forward separately.

Routing ids, counts, offsets and the permutation are compared bit for bit on
inputs whose k-th/(k+1)-th logit gap is at least 1e-3; routing weights within
1e-5; block outputs within max|gpu - ref| / max|ref| <= 1e-2.
"""
import numpy as np
import pytest
import torch

from oracle import moe_w4_oracle as O
from w4_dequant_grouped_amd import moe_w4 as B
from w4_dequant_grouped_amd import synth

from parity_util import (GAP, check_output, check_routing, full_check, make_inputs, note,
                         run_block, sampled_rows)

pytestmark = pytest.mark.gpu

S = synth.BlockShape


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    B.load_library()


# --- small configurations, full oracle -------------------------------------------

def test_tiny_workload():
    wl = synth.WORKLOADS["tiny"]
    full_check(wl.shape, wl.seed, what="tiny")


@pytest.mark.parametrize("T", [1, 2, 3, 5, 6, 7])
def test_decode_small_dims(T):
    full_check(S(T=T, H=512, I=256, E=32, top_k=4), 40 + T, what=f"decode-small T={T}")


@pytest.mark.parametrize("T", [8, 9, 33])
def test_grouped_small_dims(T):
    # T=8: smallest grouped call and last one-launch router; T=9: first tiled router
    full_check(S(T=T, H=512, I=256, E=32, top_k=4), 50 + T, what=f"grouped-small T={T}")


@pytest.mark.parametrize("T", [1, 2, 5])
def test_forced_grouped_path_small_T(T):
    # the grouped MFMA path below its default threshold (single M-tile, mostly padding)
    full_check(S(T=T, H=512, I=256, E=32, top_k=4), 70 + T, what=f"forced grouped T={T}",
               flags=B.MOE_W4_FORWARD_GROUPED)


@pytest.mark.parametrize("T", [4, 8])
def test_forced_gemv_path_up_to_8(T):
    # the GEMV path above its default threshold, up to the largest row count it is built for
    full_check(S(T=T, H=512, I=256, E=32, top_k=4), 80 + T, what=f"forced gemv T={T}",
               flags=B.MOE_W4_FORWARD_GEMV)


def test_grouped_multi_tile_ragged():
    # 1200 routed rows over 32 experts, shared expert 300 rows = 3 M-tiles (ragged)
    full_check(S(T=300, H=512, I=256, E=32, top_k=4), 61, what="multi-tile")


@pytest.mark.parametrize("T", [2, 5, 100, 300])
def test_tile_counts_not_powers_of_two(T):
    # H=768, I=384: six N-tiles per M-tile in both grouped GEMMs, 6 and 3 K-chunks, the
    # tiled router's fallback logits kernel (H/8 = 96); T=300 gives every routed expert
    # two M-tiles and the shared expert five (a block of four and a partial block)
    full_check(S(T=T, H=768, I=384, E=12, top_k=3), 90 + T, what=f"H=768 I=384 T={T}")


@pytest.mark.parametrize("T", [9, 130])
def test_partial_expert_tile(T):
    # E=100 at H=512: the tiled router's LDS logits kernel (H/8 = 64) with a second
    # tile of 36 experts (its weight rows past E clamped), two registers of logits per
    # lane in the top-k
    full_check(S(T=T, H=512, I=256, E=100, top_k=6), 105 + T, what=f"E=100 T={T}")


@pytest.mark.parametrize("T", [3, 9, 200])
def test_long_rows(T):
    # H=4352, I=640: gate/up rows of 34 K-chunks (eight full four-chunk blocks of
    # scale/bias words, then a block of two), down rows of 5 (one block, then one);
    # H/8 = 544 takes the tiled router's fallback logits kernel
    full_check(S(T=T, H=4352, I=640, E=8, top_k=2), 95 + T, what=f"H=4352 I=640 T={T}")


def test_one_expert_takes_every_token():
    shape = S(T=700, H=256, I=128, E=8, top_k=2)
    layer = synth.draw_layer(shape, 62)
    layer.router_b = torch.zeros(8, dtype=torch.float32)
    layer.router_b[3] = 40.0            # every token picks expert 3: 700 rows, 6 M-tiles
    full_check(shape, 62, layer=layer, what="one hot expert")


@pytest.mark.parametrize("T", [1, 2, 40])
def test_all_experts_selected(T):
    full_check(S(T=T, H=256, I=128, E=8, top_k=8), 63 + T, what=f"k=E T={T}")


@pytest.mark.parametrize("T", [1, 2, 20])
def test_top1_no_shared(T):
    full_check(S(T=T, H=256, I=128, E=16, top_k=1, shared=False), 65 + T, what=f"top1 T={T}")


@pytest.mark.parametrize("T", [2, 4, 64])
def test_top16(T):
    full_check(S(T=T, H=256, I=128, E=64, top_k=16), 67 + T, what=f"top16 T={T}")


def test_zero_tokens_is_a_no_op():
    shape = S(T=0, H=256, I=128, E=8, top_k=2)
    layer = synth.draw_layer(S(T=1, H=256, I=128, E=8, top_k=2), 70).to("cuda")
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    dims = B.make_dims(0, 256, 128, 8, 2)
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    r = B.alloc_routing(0, 8, 2)
    B.moe_w4_route(dims, x, layer.router_w, None, r, ws)
    out = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    B.moe_w4_forward(dims, x, layer.routed, layer.shared, r, out, ws)
    B.moe_w4_block(dims, x, layer.router_w, None, B.weights_struct(layer.routed),
                   B.weights_struct(layer.shared), r, out, ws)
    torch.cuda.synchronize()


@pytest.mark.parametrize("T", [1, 2])
def test_decode_router_bias_small_h(T):
    # H=256: only 8 of 64 lanes hold gate/up codes; Zipf router bias
    full_check(S(T=T, H=256, I=256, E=64, top_k=8, router_bias="zipf"), 72 + T,
               what=f"bias H=256 T={T}")


# --- full-size configurations ---------------------------------------------------------

@pytest.fixture(scope="module")
def full_layer():
    note("[gpu] drawing one full-size layer (H=2048, I=512, E=256)")
    return synth.draw_layer(S(T=1, H=2048, I=512, E=256, top_k=8), synth.WORKLOADS["decode"].seed)


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 7])
def test_decode_full_size(full_layer, T):
    shape = S(T=T, H=2048, I=512, E=256, top_k=8)
    full_check(shape, 100 + T, layer=full_layer, what=f"decode full T={T}")


def test_two_equal_rows_share_every_expert(full_layer):
    """T=2 with both token rows equal: both tokens pick the same eight experts, so
    every routed slot of the single-call decode block holds two h rows, and the down
    kernel takes both rows' tokens and weights from the slot table.  Routing
    bit-exact, both output rows within the tolerance (block and split calls)."""
    shape = S(T=2, H=2048, I=512, E=256, top_k=8)
    x1, _ = O.gap_conditioned_x(lambda rd: synth.draw_x(1, shape.H, 96, redraws=rd), 1,
                                full_layer.router_w, full_layer.router_b, shape.top_k, GAP)
    x = torch.cat([x1, x1], 0)
    ref = O.route(x, full_layer.router_w, full_layer.router_b, shape.top_k)
    assert (ref.ids[0] == ref.ids[1]).all() and (ref.counts[ref.counts > 0] == 2).all()
    lg = full_layer.to("cuda")
    y = O.forward_grouped(x, full_layer, ref, shape.group)
    for split in (False, True):
        r, out = run_block(lg, x.cuda(), shape, split=split)
        check_routing(r, ref, f"equal rows {'split' if split else 'block'}")
        check_output(out, y, what=f"equal rows {'split' if split else 'block'}")


@pytest.mark.parametrize("T,flags", [(1, B.MOE_W4_FORWARD_GROUPED), (4, B.MOE_W4_FORWARD_GROUPED),
                                     (8, B.MOE_W4_FORWARD_GEMV)])
def test_forced_paths_full_size(full_layer, T, flags):
    shape = S(T=T, H=2048, I=512, E=256, top_k=8)
    full_check(shape, 130 + T, layer=full_layer, what=f"forced flags={flags} full T={T}", flags=flags)


def _sampled_full(shape, seed, layer, what, nrows=12):
    note(f"[gpu] {what}: {synth.describe(shape)} seed={seed}")
    layer, x = make_inputs(shape, seed, layer)
    ref_r = O.route(x, layer.router_w, layer.router_b, shape.top_k)
    r, out = run_block(layer.to("cuda"), x.cuda(), shape)
    check_routing(r, ref_r, what)
    rows = sampled_rows(shape.T, nrows, seed)
    y = O.forward_dense(x, layer, ref_r, shape.group, rows=rows)
    check_output(out, y, rows=rows, what=what)
    return ref_r


def test_prefill_512_full_size(full_layer):
    """T=512 prefill at full size: routing bit-exact and the whole [512, 2048]
    output against the oracle's grouped form (every expert dequantised once)."""
    wl = synth.WORKLOADS["prefill512"]
    full_check(wl.shape, wl.seed, layer=full_layer, what="prefill T=512 (whole output)")


def test_prefill_2048_zipf_full_size():
    """T=2048 prefill with the Zipf router bias at full size: routing bit-exact and
    the whole [2048, 2048] output against the oracle; the routing has empty
    experts and experts above four times the mean load, so the grouped GEMMs run
    one-block tiles, full four-tile blocks of heavy experts and skipped segments."""
    wl = synth.WORKLOADS["prefill2048_zipf"]
    layer = synth.draw_layer(wl.shape, wl.seed)
    _, x = make_inputs(wl.shape, wl.seed, layer)
    counts = O.route(x, layer.router_w, layer.router_b, wl.shape.top_k).counts
    assert (counts == 0).any() and counts.max() > 4 * counts.mean()
    full_check(wl.shape, wl.seed, layer=layer, what="prefill T=2048 zipf (whole output)")


# --- properties -------------------------------------------------------------------------

def test_repeat_calls_and_workspace_reuse(full_layer):
    """Same workspace for a T=2048 call, then T=1, then T=2048 again: the control
    block returns to zero and results repeat (routing bit-identical)."""
    big = S(T=2048, H=2048, I=512, E=256, top_k=8)
    layer = full_layer.to("cuda")
    _, xb = make_inputs(big, 301, full_layer)
    _, x1 = make_inputs(S(T=1, H=2048, I=512, E=256, top_k=8), 302, full_layer)
    ws = B.alloc_workspace(B.make_dims(2048, 2048, 512, 256, 8))
    r1, o1 = run_block(layer, xb.cuda(), big, workspace=ws)
    r1 = [t.clone() for t in (r1.ids, r1.counts, r1.offsets, r1.perm)]
    o1 = o1.clone()
    rs, os_ = run_block(layer, x1.cuda(), S(T=1, H=2048, I=512, E=256, top_k=8), workspace=ws)
    ref1 = O.route(x1, full_layer.router_w, None, 8)
    check_routing(rs, ref1, "T=1 after T=2048")
    assert int(ws[:B.MOE_W4_CONTROL_BYTES].cpu().sum()) == 0
    r2, o2 = run_block(layer, xb.cuda(), big, workspace=ws)
    for a, b in zip(r1, (r2.ids, r2.counts, r2.offsets, r2.perm)):
        assert torch.equal(a, b)
    diff = (o1.float() - o2.float()).abs().max().item()
    assert diff <= 1e-2 * o1.float().abs().max().item()


def test_decode_is_deterministic(full_layer):
    shape = S(T=3, H=2048, I=512, E=256, top_k=8)
    layer = full_layer.to("cuda")
    _, x = make_inputs(shape, 303, full_layer)
    _, o1 = run_block(layer, x.cuda(), shape)
    o1 = o1.clone()
    _, o2 = run_block(layer, x.cuda(), shape)
    assert torch.equal(o1, o2)


def test_grouped_is_deterministic():
    """The grouped path gives bit-identical outputs on repeated calls, whatever order
    the workgroups take tiles in: every output row of the down GEMM has one writer and
    the combine sums each token's rows in slot order.  A call of another size in
    between changes which workgroups run which tiles."""
    wl = synth.WORKLOADS["prefill2048_zipf"]
    layer = synth.draw_layer(wl.shape, wl.seed)
    lg = layer.to("cuda")
    _, x = make_inputs(wl.shape, 305, layer)
    _, o1 = run_block(lg, x.cuda(), wl.shape)
    o1 = o1.clone()
    small = S(T=300, H=2048, I=512, E=256, top_k=8, router_bias="zipf")
    _, xs = make_inputs(small, 306, layer)
    run_block(lg, xs.cuda(), small)
    _, o2 = run_block(lg, x.cuda(), wl.shape)
    assert torch.equal(o1, o2)


# Control-block words of the grouped GEMMs (uint32 index): gate/up tile queues at
# 32 + 32 q, down queues at 288 + 32 q, 64-bit exit words at 544 and 576; the
# error counter is the block's last word (MOE_W4_CONTROL_ERRORS_OFFSET).
_CTL_GATEUP_QUEUE0 = 32
_CTL_ERRORS = B.MOE_W4_CONTROL_ERRORS_OFFSET // 4


@pytest.mark.parametrize("dirt", ["one queue advanced", "garbage"])
def test_dirty_control_block_is_counted_and_repaired(dirt):
    """The workspace rule broken on purpose from the host: the control block is not
    zero when a grouped forward starts, either one gate/up queue word already five
    tiles in (those tiles would be skipped silently) or the whole block filled with
    random words (a workspace that was never zero-filled).  The call adds to the
    error counter and its last kernel clears the queue and exit words, so the next
    call on the same workspace matches the oracle and adds no error."""
    shape = S(T=300, H=512, I=256, E=32, top_k=4)
    layer, x = make_inputs(shape, 700)
    lg, xg = layer.to("cuda"), x.cuda()
    blk = B.Block(lg, shape.T, shape.top_k)
    ctl = blk.workspace[:B.MOE_W4_CONTROL_BYTES].view(torch.int32)
    if dirt == "garbage":
        g = torch.Generator().manual_seed(701)
        ctl.copy_(torch.randint(-2 ** 31, 2 ** 31 - 1, (ctl.numel(),), generator=g, dtype=torch.int32))
        ctl[_CTL_ERRORS] = 0
    else:
        ctl[_CTL_GATEUP_QUEUE0] = 5
    blk(xg)
    torch.cuda.synchronize()
    errors = int(ctl[_CTL_ERRORS].item())
    assert errors >= 1, f"{dirt}: dirty control block not counted"
    if dirt != "garbage":
        rest = torch.cat([ctl[:_CTL_ERRORS], ctl[_CTL_ERRORS + 1:]])
        assert int(rest.abs().sum().item()) == 0, "control block not cleared"
    r, out = blk.routing, blk(xg)
    torch.cuda.synchronize()
    assert int(ctl[_CTL_ERRORS].item()) == errors, "a clean call counted an error"
    ref_r = O.route(x, layer.router_w, layer.router_b, shape.top_k)
    check_routing(r, ref_r, f"after {dirt}")
    check_output(out, O.forward_grouped(x, layer, ref_r, shape.group), what=f"after {dirt}")


def test_token_permutation_invariance_gpu():
    shape = S(T=96, H=512, I=256, E=32, top_k=4)
    layer, x = make_inputs(shape, 304)
    p = torch.randperm(shape.T, generator=synth.generator(5))
    lg = layer.to("cuda")
    r1, o1 = run_block(lg, x.cuda(), shape)
    o1 = o1.clone()
    c1 = r1.counts.clone()
    r2, o2 = run_block(lg, x[p].cuda(), shape)
    assert torch.equal(r2.counts, c1)
    ref = o1.float()[p.cuda()]
    assert (o2.float() - ref).abs().max().item() <= 1e-2 * ref.abs().max().item()


# --- the single-call entry point against the two separate calls ---------------------

@pytest.mark.parametrize("T", [1, 2])
def test_split_entry_points_full_size(full_layer, T):
    shape = S(T=T, H=2048, I=512, E=256, top_k=8)
    full_check(shape, 110 + T, layer=full_layer, what=f"split full T={T}", split=True)


@pytest.mark.parametrize("T", [1, 2])
def test_block_and_split_agree(full_layer, T):
    shape = S(T=T, H=2048, I=512, E=256, top_k=8)
    layer = full_layer.to("cuda")
    _, x = make_inputs(shape, 120 + T, full_layer)
    ra, oa = run_block(layer, x.cuda(), shape)
    ra = [t.clone() for t in (ra.ids, ra.weights, ra.counts, ra.offsets, ra.perm)]
    oa = oa.clone()
    rb, ob = run_block(layer, x.cuda(), shape, split=True)
    for a, b in zip(ra, (rb.ids, rb.weights, rb.counts, rb.offsets, rb.perm)):
        assert torch.equal(a, b)
    diff = (oa.float() - ob.float()).abs().max().item()
    assert diff <= 1e-2 * ob.float().abs().max().item()


def test_block_calls_leave_control_block_clear(full_layer):
    """Forty single-call blocks in a row on one workspace (T = 1, 2, 1, ...) with
    fresh inputs: sampled results match the oracle's routing, and the control
    block ends all zero."""
    layer = full_layer.to("cuda")
    dims2 = B.make_dims(2, 2048, 512, 256, 8)
    ws = B.alloc_workspace(dims2)
    for i in range(40):
        T = 1 + (i % 2)
        shape = S(T=T, H=2048, I=512, E=256, top_k=8)
        _, x = make_inputs(shape, 200 + i, full_layer)
        r, _ = run_block(layer, x.cuda(), shape, workspace=ws)
        if i % 8 == 0:
            check_routing(r, O.route(x, full_layer.router_w, None, 8), f"call {i}")
    assert int(ws[:B.MOE_W4_CONTROL_BYTES].cpu().sum()) == 0


# --- the 40-layer stack's layer size, and exact ties ------------------------------------

def test_stack_layer_T16384_sampled():
    """One layer of the 40-layer stack workload (T=16384, Zipf router bias): routing
    bit-exact against the oracle over all 16384 tokens, 12 sampled output rows."""
    wl = synth.WORKLOADS["stack40"]
    layer = synth.draw_layer(wl.shape, wl.seed)
    _sampled_full(wl.shape, wl.seed, layer, "stack layer T=16384")


@pytest.mark.parametrize("T", [1, 2, 16])
def test_boundary_ties_go_to_the_lower_expert(T):
    """Experts 5 and 9 have identical router rows and biases, so their logits tie
    exactly; with experts 0 and 1 far above and the rest far below, the k=3 choice
    must take 5 and leave 9 (one-launch router at T=1, 2; single-call block at
    T=1, 2; tiled router at T=16)."""
    shape = S(T=T, H=256, I=128, E=16, top_k=3)
    layer = synth.draw_layer(shape, 80 + T)
    layer.router_w[9] = layer.router_w[5]
    bias = torch.full((16,), -40.0, dtype=torch.float32)
    bias[0], bias[1], bias[5], bias[9] = 40.0, 30.0, 10.0, 10.0
    layer.router_b = bias
    x = synth.draw_x(T, 256, 80 + T)
    ref = O.route(x, layer.router_w, layer.router_b, 3)
    assert (ref.ids == np.array([0, 1, 5])).all()
    lg = layer.to("cuda")
    for split in (False, True):
        r, out = run_block(lg, x.cuda(), shape, split=split)
        check_routing(r, ref, f"ties T={T} {'split' if split else 'block'}")
        y = O.forward_grouped(x, layer, ref, shape.group)
        check_output(out, y, what=f"ties T={T}")


@pytest.mark.parametrize("T", [1, 2, 16])
def test_six_way_tie_across_the_top12_boundary(T):
    """top-12 of 64 experts: nine far above, six with identical router rows and
    biases spread over several lane groups, the rest far below.  Only the three
    lowest-id tied experts may be chosen, which the selection can settle only at
    full key depth."""
    shape = S(T=T, H=256, I=128, E=64, top_k=12)
    layer = synth.draw_layer(shape, 90 + T)
    tied = [12, 20, 33, 47, 58, 61]
    for e in tied[1:]:
        layer.router_w[e] = layer.router_w[tied[0]]
    bias = torch.full((64,), -40.0, dtype=torch.float32)
    bias[:9] = 40.0
    bias[tied] = 10.0
    layer.router_b = bias
    x = synth.draw_x(T, 256, 90 + T)
    ref = O.route(x, layer.router_w, layer.router_b, 12)
    assert (ref.ids == np.array(list(range(9)) + tied[:3])).all()
    lg = layer.to("cuda")
    for split in (False, True):
        r, out = run_block(lg, x.cuda(), shape, split=split)
        check_routing(r, ref, f"6-way tie T={T} {'split' if split else 'block'}")
        check_output(out, O.forward_grouped(x, layer, ref, shape.group), what=f"6-way tie T={T}")


@pytest.mark.parametrize("T,shared", [(9, True), (131, False)])
def test_byte_id_grouping_at_256_experts(T, shared):
    """E = 256 with top-8 and T*k not a multiple of 16 (72 and 1048 entries): the
    grouping kernel reads the chosen ids as bytes, where every byte value is a
    real expert id, so the padding of the last 16-byte piece must be masked by
    position. Without a shared expert (T=131) the tile sequence starts with a
    routed expert instead of the shared one."""
    full_check(S(T=T, H=256, I=128, E=256, top_k=8, shared=shared), 120 + T,
               what=f"E=256 byte ids T={T} shared={shared}")


@pytest.mark.parametrize("T", [16384, 16386])
def test_byte_id_grouping_batch_boundary(T):
    """The byte-id grouping at the edge of one batch per thread: T*k = 131072 fills
    exactly one batch of 16-byte loads per thread, kept in registers for the writing
    pass; T*k = 131088 needs a second batch, so both passes read the ids again."""
    full_check(S(T=T, H=256, I=128, E=256, top_k=8), 130 + T % 7,
               what=f"E=256 byte ids batch boundary T={T}")


@pytest.mark.parametrize("T", [8192, 8193])
def test_int32_id_grouping_batch_boundary(T):
    """E = 512 keeps the grouping on int32 ids: T*k = 65536 fills exactly one batch of
    16-byte loads per thread, kept in registers for the writing pass; T*k = 65544
    needs a second batch."""
    full_check(S(T=T, H=256, I=128, E=512, top_k=8), 140 + T % 7,
               what=f"E=512 int32 ids batch boundary T={T}")


# --- largest sizes the ABI accepts ------------------------------------------------------

@pytest.mark.parametrize("T", [2, 4, 64])
def test_max_experts_and_top_k(T):
    """E = 1024 experts (the largest accepted) with top-16: the 16-per-lane top-k,
    1025 segments in the grouped tile list, and the single-call decode block (at
    T=4 its 64 selected slots and 68 h rows take the down kernel's slot table in
    two passes of 64 lanes)."""
    full_check(S(T=T, H=256, I=128, E=1024, top_k=16), 70 + T, what=f"E=1024 top16 T={T}")


def test_max_tokens_T65536_sampled(full_layer):
    """T = 65536 (the largest accepted) at full size: routing bit-exact over all
    65536 tokens against the oracle, 12 sampled output rows."""
    _sampled_full(S(T=65536, H=2048, I=512, E=256, top_k=8), 71, full_layer, "T=65536")


# --- graph capture ------------------------------------------------------------------------

@pytest.mark.parametrize("T", [1, 2, 64])
def test_graph_replays_match_eager(full_layer, T):
    """Two block calls sharing one workspace, captured as a HIP graph: three
    replays, with eager calls on other inputs and a synchronisation between them,
    each equal bit for bit to the eager calls on the same inputs; the first
    replay's routing is bit-exact and its output within tolerance against the
    oracle; the control block ends all zero."""
    shape = S(T=T, H=2048, I=512, E=256, top_k=8)
    layer = full_layer.to("cuda")
    ws = B.alloc_workspace(B.make_dims(T, 2048, 512, 256, 8))
    blocks = [B.Block(layer, T, 8, workspace=ws) for _ in range(2)]
    _, xa = make_inputs(shape, 400 + T, full_layer)
    _, xb = make_inputs(shape, 500 + T, full_layer)
    xa, xb = xa.cuda(), xb.cuda()
    xin = torch.empty_like(xa)

    def body():
        for blk in blocks:
            blk(xin)

    xin.copy_(xa)
    body()
    torch.cuda.synchronize()
    ref = [(blk.out.clone(), blk.routing.perm.clone(), blk.routing.ids.clone()) for blk in blocks]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        body()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        body()
    for rep in range(3):
        xin.copy_(xa)
        graph.replay()
        torch.cuda.synchronize()
        for (o, p, i), blk in zip(ref, blocks):
            assert torch.equal(blk.routing.ids, i), f"replay {rep}: ids"
            assert torch.equal(blk.routing.perm, p), f"replay {rep}: perm"
            assert torch.equal(blk.out, o), f"replay {rep}: output"
        if rep == 0:
            # the replayed layer against the oracle itself, not only the eager call
            xa_cpu = xa.cpu()
            ref_r = O.route(xa_cpu, full_layer.router_w, None, 8)
            check_routing(blocks[1].routing, ref_r, f"graph replay T={T}")
            rows = None if T <= 2 else sampled_rows(T, 6, 400 + T)
            y = O.forward_dense(xa_cpu, full_layer, ref_r, 64, rows=rows)
            check_output(blocks[1].out, y, rows=rows, what=f"graph replay T={T}")
        xin.copy_(xb)
        body()
        torch.cuda.synchronize()
    assert int(ws[:B.MOE_W4_CONTROL_BYTES].cpu().sum()) == 0
