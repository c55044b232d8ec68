"""Shared plumbing of the GPU parity tests: seeded inputs, one block call through
the C ABI, and comparison against the CPU oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import moe_w4_oracle as O
from w4_dequant_grouped_amd import moe_w4 as B
from w4_dequant_grouped_amd import synth

OUT_TOL = 1e-2      # max|gpu - ref| / max|ref| on the block output
WEIGHT_TOL = 1e-5   # absolute, on the routing weights
GAP = 1e-3          # minimum k-th / (k+1)-th logit gap of parity inputs


def note(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def make_inputs(shape: synth.BlockShape, seed: int, layer=None, condition: bool = True):
    """CPU layer and gap-conditioned x (bf16 [T, H])."""
    if layer is None:
        layer = synth.draw_layer(shape, seed)
    if condition and shape.T > 0:
        x, _ = O.gap_conditioned_x(lambda rd: synth.draw_x(shape.T, shape.H, seed, redraws=rd),
                                   shape.T, layer.router_w, layer.router_b, shape.top_k, GAP)
    else:
        x = synth.draw_x(shape.T, shape.H, seed)
    return layer, x


def run_block(layer_gpu, x_gpu, shape: synth.BlockShape, workspace=None, split: bool = False,
              flags: int = 0):
    """One block call: moe_w4_block, or moe_w4_route then moe_w4_forward (split).
    flags picks the forward path (0: by T)."""
    blk = B.Block(layer_gpu, shape.T, shape.top_k, shape.group, workspace=workspace, flags=flags)
    out = blk.split(x_gpu) if split else blk(x_gpu)
    torch.cuda.synchronize()
    return blk.routing, out


def routing_to_cpu(r: B.Routing):
    return B.Routing(*(t.cpu() for t in (r.ids, r.weights, r.counts, r.offsets, r.perm)))


def check_routing(r_gpu: B.Routing, ref: O.Routing, what: str = "") -> None:
    g = routing_to_cpu(r_gpu)
    assert np.array_equal(g.ids.numpy(), ref.ids), f"{what}: topk ids differ"
    assert np.array_equal(g.counts.numpy(), ref.counts), f"{what}: counts differ"
    assert np.array_equal(g.offsets.numpy(), ref.offsets), f"{what}: offsets differ"
    assert np.array_equal(g.perm.numpy(), ref.perm), f"{what}: permutation differs"
    err = np.abs(g.weights.numpy().astype(np.float64) - ref.weights).max() if ref.weights.size else 0.0
    assert err <= WEIGHT_TOL, f"{what}: routing weight error {err}"


def check_output(out_gpu: torch.Tensor, ref: np.ndarray, rows=None, what: str = "") -> float:
    got = out_gpu.float().cpu().numpy().astype(np.float64)
    if rows is not None:
        got = got[list(rows)]
    err = O.relative_error(got, ref)
    note(f"  {what}: max|gpu-ref|/max|ref| = {err:.3e} (max|ref| = {np.abs(ref).max():.3f})")
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    assert err <= OUT_TOL, f"{what}: relative error {err} > {OUT_TOL}"
    return err


def full_check(shape: synth.BlockShape, seed: int, layer=None, what: str = "", condition=True,
               split: bool = False, flags: int = 0):
    """Route + forward on the GPU and compare everything with the full oracle."""
    note(f"[gpu] {what}: {synth.describe(shape)} seed={seed} {'split' if split else 'block'}")
    layer, x = make_inputs(shape, seed, layer, condition)
    ref_r = O.route(x, layer.router_w, layer.router_b, shape.top_k)
    r, out = run_block(layer.to("cuda"), x.cuda(), shape, split=split, flags=flags)
    if condition:
        check_routing(r, ref_r, what)
    y = O.forward_grouped(x, layer, ref_r, shape.group)
    return check_output(out, y, what=what)


def sampled_rows(T: int, n: int, seed: int):
    """n token rows: the first, the last, and a seeded spread in between."""
    g = torch.Generator().manual_seed(seed)
    inner = torch.randperm(max(T - 2, 0), generator=g)[: max(n - 2, 0)] + 1
    rows = sorted(set([0, T - 1] + inner.tolist()))
    return rows
