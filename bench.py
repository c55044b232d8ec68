#!/usr/bin/env python3
"""Benchmark of the W4 mixture-of-experts block on one MI355X.

Default workload (one JSON line on stdout): decode, T=1 token per layer-call,
hidden 2048, 256 experts top-8 + one shared expert, intermediate 512, 4-bit
weights in groups of 64, over 40 independently seeded layers used in rotation
(18.3 GB of packed weights, so every layer-call reads its experts from HBM, not
from the 256 MiB Infinity Cache) with a fresh activation row per layer-call.

A step is one decode token through all 40 layers: 40 x (route + forward).
value = MoE-layer tokens per second = 40 * T * steps / elapsed.

The same line carries:
  roofline      the dominant kernel's algorithmic bytes (or flops) per launch over
                its average duration, timed with HIP events that the library passes
                to each kernel's dispatch as start/stop events (hipExtLaunchKernelGGL)
                in a second pass over the same steps
  cpu_baseline  the CPU oracle (float64 NumPy) timed on a bounded sample of the
                same workload on this host
  prefill       the T=2048 Zipf-skewed prefill layer-call (8 layers rotated):
                tokens/s and the MFMA roofline of its dominant kernel

Other modes (their own JSON line):
  --crossover   verification batches: GEMV vs grouped path per T (1..64)
  --stack       the 40-layer stack: T=16384 prefill, then T=1 decode steps
  --attn        decode attention over a paged KV cache (16 query heads over 2
                key/value heads, head dim 128, 64-token blocks) at 32K, 64K and
                128K tokens of context, 10 caches in rotation
  --gdn         the Gated DeltaNet scan (32 value heads over 16 query/key heads,
                dimension 128): prefill T=512 and T=2048 on the chunked MFMA form
                (the register-resident scan timed beside it), and T=1 decode
                steps of the register scan over 30 layer states in rotation
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "MoE-layer tokens/sec + %HBM roofline (T=1) and %MFMA peak (T=2048)"

# the tiled router at H/8 a multiple of 64 (the bench shapes): the logits kernel
# splits the fp32 router weight into its bf16 planes itself
ROUTE_LARGE = ["router_logits", "router_topk", "router_group"]
BLOCK_DECODE = ["decode_logits_shared", "decode_route_gateup", "decode_down"]
FWD_GROUPED = ["grouped_gateup", "grouped_down", "finalize"]
ATTN = ["attn_split", "attn_combine"]
VALU_FP32_PEAK_TFLOPS = 157.3   # MI355X fp32 vector peak (256 CUs x 2.4 GHz), TFLOP/s


# ---------------------------------------------------------------------------
# HIP events through the runtime's C API (the library dispatches each timed
# kernel with one event pair as its start/stop events)
# ---------------------------------------------------------------------------
class HipEvents:
    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            rc = self.hip.hipEventCreate(ctypes.byref(e))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed: {rc}")
            evs.append(e.value)
        return evs

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed: {rc}")
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def source_hash() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "w4_dequant_grouped_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload: str, launches_per_unit=1):
    """HBM bytes per launch measured with rocprofv3 counters, if a summary for this
    kernel, this workload and the current kernel sources exists under profiles/."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        doc = json.load(f)
    ent = doc.get(f"{workload}:{kernel}")
    if not ent or ent.get("source_hash") != source_hash():
        return None
    return ent.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------
def expert_bytes(H, I, G=64):
    mat = lambda N, K: N * K // 2 + 2 * 2 * N * (K // G)   # noqa: E731
    return mat(I, H), mat(H, I)      # one of gate/up, down


def make_layers(shape, n_layers, seed0, device):
    from w4_dequant_grouped_amd import synth
    return [synth.draw_layer(shape, seed0 + l, device=device) for l in range(n_layers)]


def time_steps(step_fn, steps, warmup):
    import torch
    for _ in range(warmup):
        step_fn()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step_fn(i)
    torch.cuda.synchronize()
    return time.perf_counter() - t0


class DecodeGraph:
    """One decode step (every layer's block call) captured as a HIP graph.

    Each layer reads its activations from a fixed input buffer; a step copies that
    step's activations in (one device copy) and replays the graph.  Before it is
    used, every replay is checked against the eager step on the same inputs, with
    eager work and synchronisation between the replays."""

    def __init__(self, blocks, T, H):
        import torch
        self.blocks = blocks
        L = len(blocks)
        self.x = torch.zeros((L, T, H), dtype=torch.bfloat16, device="cuda")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            self._body()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self._body()
        torch.cuda.synchronize()

    def _body(self):
        for l, blk in enumerate(self.blocks):
            blk(self.x[l])

    def step(self, xstack):
        self.x.copy_(xstack)
        self.graph.replay()

    def eager(self, xstack):
        self.x.copy_(xstack)
        self._body()

    def check(self, xa, xb, replays=3):
        """Replays on xa must equal the eager step on xa bit for bit; an eager step
        on xb runs between replays."""
        import torch
        self.eager(xa)
        torch.cuda.synchronize()
        ref = [blk.out.clone() for blk in self.blocks]
        for r in range(replays):
            self.step(xa)
            torch.cuda.synchronize()
            for l, blk in enumerate(self.blocks):
                if not torch.equal(blk.out, ref[l]):
                    raise RuntimeError(f"graph replay {r} differs from the eager step at layer {l}")
            self.eager(xb)
            torch.cuda.synchronize()


def step_percentiles(step_fn, n):
    """p10 / p50 / p90 of n single-step durations (ms), each bracketed by torch events."""
    import torch
    pairs = []
    for i in range(n):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        step_fn(i)
        b.record()
        pairs.append((a, b))
    torch.cuda.synchronize()
    t = sorted(a.elapsed_time(b) for a, b in pairs)
    pick = lambda q: t[min(len(t) - 1, int(round(q * (len(t) - 1))))]   # noqa: E731
    return [round(pick(0.1), 4), round(pick(0.5), 4), round(pick(0.9), 4)]


def measure_ceilings():
    """Secondary denominators measured on this GPU: a plain device copy (bytes read
    plus written per second), a plain read (row sums over the same buffer, the
    fastest of the torch reductions measured: the weight streams of the MoE kernels
    only read) and a large bf16 GEMM through torch (hipBLASLt)."""
    import torch
    n = 1 << 28                                   # 1 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(2):
        dst.copy_(src)
    a.record()
    for _ in range(10):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    copy_gbps = 10 * 2 * 4 * n / (a.elapsed_time(b) * 1e-3) / 1e9
    del dst
    rows = src.view(-1, 4096)
    for _ in range(2):
        s = rows.sum(1)
    a.record()
    for _ in range(10):
        s = rows.sum(1)
    b.record()
    torch.cuda.synchronize()
    read_gbps = 10 * 4 * n / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, rows, s
    m = 8192
    g = torch.Generator(device="cuda").manual_seed(5)
    x = torch.randn((m, m), generator=g, device="cuda").to(torch.bfloat16)
    w = torch.randn((m, m), generator=g, device="cuda").to(torch.bfloat16)
    for _ in range(2):
        y = x @ w
    a.record()
    for _ in range(10):
        y = x @ w
    b.record()
    torch.cuda.synchronize()
    gemm_tflops = 10 * 2.0 * m ** 3 / (a.elapsed_time(b) * 1e-3) / 1e12
    del x, w, y
    torch.cuda.empty_cache()
    return {"copy_GBps": round(copy_gbps, 1), "read_GBps": round(read_gbps, 1),
            "bf16_gemm_TFLOPs": round(gemm_tflops, 1),
            "copy": "1 GiB fp32 device copy (read + write bytes)",
            "read": "row sums (4096 floats a row) over the same 1 GiB fp32 buffer (bytes read)",
            "gemm": f"{m}x{m}x{m} bf16 matmul (torch / hipBLASLt)"}


def kernel_times(blocks, xs, steps, ev: HipEvents, names, timed):
    """Average duration per kernel name over `steps` passes over all blocks.

    ``timed(block, x, events)`` runs one block call with an event pair per kernel
    and returns the kernel count.  The library dispatches each kernel with its
    pair as start/stop events (hipExtLaunchKernelGGL), so a pair spans that
    kernel's own execution, as rocprofv3's kernel trace does."""
    import torch
    n = len(names)
    events = []
    for s in range(steps):
        for l, blk in enumerate(blocks):
            e = ev.create(2 * n)
            got = timed(blk, xs[s % len(xs)][l], e)
            assert got == n, (got, names)
            events.append(e)
    torch.cuda.synchronize()
    sums = {name: 0.0 for name in names}
    for e in events:
        for i, name in enumerate(names):
            sums[name] += ev.elapsed_ms(e[2 * i], e[2 * i + 1])
        ev.destroy(e)
    return {name: 1e3 * v / len(events) for name, v in sums.items()}   # microseconds per launch


def split_timed(nr):
    """Timing callback of route + forward as two calls (first nr event pairs: route)."""
    def timed(blk, x, e):
        kr, kf = blk.timed(x, e[:2 * nr], e[2 * nr:])
        return kr + kf
    return timed


def run_decode(args, ev):
    import torch
    from w4_dequant_grouped_amd import moe_w4 as B
    from w4_dequant_grouped_amd import synth

    T, H, I, E, k = args.tokens, 2048, 512, 256, 8
    L = args.layers
    shape = synth.BlockShape(T=T, H=H, I=I, E=E, top_k=k)
    layers = make_layers(shape, L, 1000, "cuda")
    ws = B.alloc_workspace(B.make_dims(T, H, I, E, k))
    blocks = [B.Block(layer, T, k, workspace=ws) for layer in layers]
    nx = args.steps + args.warmup
    g = synth.generator(77, "cuda")
    xstk = torch.randn((nx, L, T, H), generator=g, device="cuda").to(torch.bfloat16)
    xs = [[xstk[i, l] for l in range(L)] for i in range(nx)]

    split = getattr(args, "entry", "block") == "split"
    use_graph = not split and not getattr(args, "no_graph", False)
    if use_graph:
        dg = DecodeGraph(blocks, T, H)
        dg.check(xstk[0], xstk[1 % nx])

        def step(i=0):
            dg.step(xstk[i % nx])
    else:
        def step(i=0):
            for l, blk in enumerate(blocks):
                if split:
                    blk.split(xs[i % nx][l])
                else:
                    blk(xs[i % nx][l])

    elapsed = time_steps(step, args.steps, args.warmup)
    ms_per_step = 1e3 * elapsed / args.steps
    value = L * T * args.steps / elapsed
    pcts = step_percentiles(step, min(args.steps, 20))

    names = BLOCK_DECODE
    kt = kernel_times(blocks, xs, min(args.steps, 10), ev, names,
                      lambda blk, x, e: blk.block_timed(x, e))
    # algorithmic bytes per launch from the routing each layer produced
    gu_b, dn_b = expert_bytes(H, I)
    active = []
    for blk in blocks:
        active.append(int((blk.routing.counts > 0).sum().item()))
    n_act = sum(active) / len(active)
    routing_bytes = T * k * 8 + (2 * E + 1 + T * k) * 4
    layer_bytes = E * H * 4 + (n_act + 1) * (2 * gu_b + dn_b) + 2 * T * H * 2 + routing_bytes
    # per kernel: every byte it must read or write once (weights, activations,
    # logits, h rows, routing)
    alg = {
        "decode_logits_shared": E * H * 4 + T * H * 2 + 2 * gu_b + T * E * 4 + T * I * 2,
        "decode_route_gateup": T * E * 4 + n_act * 2 * gu_b + T * H * 2 + T * k * I * 2 + routing_bytes,
        "decode_down": (n_act + 1) * dn_b + (T * k + T) * I * 2 + T * k * 8 + T * H * 2,
    }
    dom = max(names, key=lambda n: kt[n])
    achieved = alg[dom] / (kt[dom] * 1e-6) / 1e9
    roofline = {
        "bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
        "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": traffic_from_profiles(dom, "decode"),
        "alg_bytes_per_launch": int(alg[dom]), "avg_launch_us": round(kt[dom], 3),
        "kernel_us": {n: round(v, 3) for n, v in kt.items()},
        "layer_call_alg_bytes": int(layer_bytes),
        "layer_call_hbm_frac": round(layer_bytes / (ms_per_step / L * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "active_experts_per_call": n_act,
        "step_ms_p10_p50_p90": pcts,
    }
    config = {"workload": f"decode T={T} (40-layer rotation), H={H}, I={I}, E={E} top-{k} + shared, "
                          f"W4 group 64", "T": T, "H": H, "I": I, "E": E, "top_k": k,
              "layers": L, "shared_expert": True,
              "step": "hip graph of the 40 block calls (replays checked against eager)" if use_graph
              else ("route + forward calls" if split else "eager block calls")}
    return value, ms_per_step, roofline, config


def run_prefill(args, ev, T=2048, L=8, steps=5, warmup=2, zipf=True):
    """One prefill layer-call of T tokens over an L-layer rotation: tokens/s, %MFMA
    over the layer and of the dominant kernel, and %HBM of the layer-call's
    algorithmic bytes (W_r, every active expert's W4 bytes once, x and out)."""
    import torch
    from w4_dequant_grouped_amd import moe_w4 as B
    from w4_dequant_grouped_amd import synth

    H, I, E, k = 2048, 512, 256, 8
    shape = synth.BlockShape(T=T, H=H, I=I, E=E, top_k=k, router_bias="zipf" if zipf else "none")
    layers = make_layers(shape, L, 3000, "cuda")
    ws = B.alloc_workspace(B.make_dims(T, H, I, E, k))
    blocks = [B.Block(layer, T, k, workspace=ws) for layer in layers]
    g = synth.generator(78, "cuda")
    xs = [[torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16) for _ in range(L)]]

    def step(i=0):
        for l, blk in enumerate(blocks):
            blk(xs[0][l])

    elapsed = time_steps(step, steps, warmup)
    per_call_ms = 1e3 * elapsed / (steps * L)
    pcts = step_percentiles(lambda i: blocks[i % L](xs[0][i % L]), 16)
    kt = kernel_times(blocks, xs, steps, ev, ROUTE_LARGE + FWD_GROUPED, split_timed(len(ROUTE_LARGE)))
    rows = T * k + T
    # active experts of each layer's routing (after the last call on its input)
    active = []
    for l, blk in enumerate(blocks):
        blk(xs[0][l])
        off = blk.routing.offsets.cpu()
        active.append(int(((off[1:] - off[:-1]) > 0).sum()))
    gu, dn = expert_bytes(H, I)
    layer_bytes = sum(E * H * 4 + (a + 1) * (2 * gu + dn) + 2 * T * H * 2 for a in active) / L
    layer_bytes = float(layer_bytes)
    flops = {"grouped_gateup": 2.0 * rows * H * 2 * I, "grouped_down": 2.0 * rows * I * H}
    dom = max(flops, key=lambda n: kt[n])
    tflops = flops[dom] / (kt[dom] * 1e-6) / 1e12
    layer_flops = flops["grouped_gateup"] + flops["grouped_down"]
    a_mean = sum(active) / L
    # algorithmic bytes per launch: every active expert's (and the shared one's)
    # weights once, the activations read once, the expert-sorted outputs once
    kbytes = {"grouped_gateup": (a_mean + 1) * 2 * gu + T * H * 2 + rows * I * 2,
              "grouped_down": (a_mean + 1) * dn + rows * I * 2 + rows * H * 2}
    tkey = "prefill" if zipf else f"prefill{T}"
    if T >= 2048:
        # the MFMA target of the large prefill layer (the roofline's ridge is near
        # 312 flop/B; this layer sits at about 250)
        roof = {"bound": "mfma", "kernel": dom, "achieved": round(tflops, 2),
                "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                "traffic": traffic_from_profiles(dom, tkey),
                "alg_flops_per_launch": flops[dom]}
    else:
        # at this size the layer's arithmetic intensity (about 64 flop/B) is far
        # below the ridge point, so HBM bounds it
        gbs = kbytes[dom] / (kt[dom] * 1e-6) / 1e9
        roof = {"bound": "hbm", "kernel": dom, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                "traffic": traffic_from_profiles(dom, tkey),
                "alg_bytes_per_launch": int(kbytes[dom]),
                "mfma_frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4)}
    return {
        "workload": (f"prefill T={T} " + ("Zipf-skewed router bias" if zipf else "uniform-ish routing (no bias)")
                     + f", {L}-layer rotation, same shapes"),
        "tokens_per_s": round(T / (per_call_ms * 1e-3), 1),
        "ms_per_layer_call": round(per_call_ms, 4),
        "layer_call_mfma_frac": round(layer_flops / (per_call_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "active_experts_per_call": round(sum(active) / L, 2),
        "layer_call_alg_bytes": int(layer_bytes),
        "layer_call_hbm_frac": round(layer_bytes / (per_call_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "layer_call_ms_p10_p50_p90": pcts,
        "roofline": dict(roof, avg_launch_us=round(kt[dom], 3),
                         kernel_us={n: round(v, 3) for n, v in kt.items()}),
    }


def run_tiny(args, steps=200, warmup=20):
    """The tiny block (T=16, hidden 256, 16 experts top-2 + shared, intermediate 128):
    a correctness-sized workload, launch-bound, reported as block calls and tokens/s."""
    import torch
    from w4_dequant_grouped_amd import moe_w4 as B
    from w4_dequant_grouped_amd import synth

    wl = synth.WORKLOADS["tiny"]
    sh = wl.shape
    layer = synth.draw_layer(sh, wl.seed, device="cuda")
    blk = B.Block(layer, sh.T, sh.top_k, sh.group)
    x = synth.draw_x(sh.T, sh.H, wl.seed, device="cuda")

    def step(i=0):
        blk(x)

    elapsed = time_steps(step, steps, warmup)
    us = 1e6 * elapsed / steps
    return {"workload": "tiny block: " + wl.note, "us_per_call": round(us, 2),
            "tokens_per_s": round(sh.T / (us * 1e-6), 1),
            "call_us_p10_p50_p90": [round(1e3 * v, 2) for v in step_percentiles(step, 50)],
            "path": "moe_w4_block (grouped path at T=16: four router launches and three forward launches)"}


def run_stack(args, ev):
    """The 40-layer stack: T=16384 prefill through 40 independently seeded layers
    (Zipf-biased routers, the same activations into every layer, no chaining),
    then T=1 decode steps over the same 40 layers as one captured graph."""
    import torch
    from w4_dequant_grouped_amd import moe_w4 as B
    from w4_dequant_grouped_amd import synth

    T, H, I, E, k, L = args.stack_tokens, 2048, 512, 256, 8, 40
    shape = synth.BlockShape(T=T, H=H, I=I, E=E, top_k=k, router_bias="zipf")
    layers = make_layers(shape, L, 4000, "cuda")
    gu_b, dn_b = expert_bytes(H, I)
    per_expert = 2 * gu_b + dn_b

    # prefill
    ws = B.alloc_workspace(B.make_dims(T, H, I, E, k))
    blocks = [B.Block(layer, T, k, workspace=ws) for layer in layers]
    x = torch.randn((T, H), generator=synth.generator(4, "cuda"), device="cuda").to(torch.bfloat16)

    def pstep(i=0):
        for blk in blocks:
            blk(x)

    steps = 3
    elapsed = time_steps(pstep, steps, 1)
    stack_s = elapsed / steps
    active = [int((blk.routing.counts > 0).sum().item()) for blk in blocks]
    flops = 6.0 * (T * k + T) * H * I * L          # bf16 expert GEMMs
    pbytes = sum(E * H * 4 + (a + 1) * per_expert + 2 * T * H * 2 for a in active)
    kt = kernel_times(blocks, [[x] * L], 1, ev, ROUTE_LARGE + FWD_GROUPED, split_timed(len(ROUTE_LARGE)))
    gemm_flops = {"grouped_gateup": 2.0 * (T * k + T) * H * 2 * I, "grouped_down": 2.0 * (T * k + T) * I * H}
    prefill = {
        "T": T, "stack_ms": round(1e3 * stack_s, 3), "ms_per_layer": round(1e3 * stack_s / L, 4),
        "tokens_per_s": round(T / stack_s, 1),
        "mfma_frac": round(flops / stack_s / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "alg_GBps": round(pbytes / stack_s / 1e9, 1),
        "kernel_us": {n: round(v, 3) for n, v in kt.items()},
        "gemm_mfma_frac": {n: round(f / (kt[n] * 1e-6) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)
                           for n, f in gemm_flops.items()},
        "active_experts_per_layer": sum(active) / L,
    }
    del blocks, ws
    torch.cuda.empty_cache()

    # decode
    nd, warm = args.stack_decode_steps, 5
    ws1 = B.alloc_workspace(B.make_dims(1, H, I, E, k))
    dblocks = [B.Block(layer, 1, k, workspace=ws1) for layer in layers]
    xstk = torch.randn((nd + warm, L, 1, H), generator=synth.generator(5, "cuda"),
                       device="cuda").to(torch.bfloat16)
    dg = DecodeGraph(dblocks, 1, H)
    dg.check(xstk[0], xstk[1])
    elapsed = time_steps(lambda i=0: dg.step(xstk[i % (nd + warm)]), nd, warm)
    step_s = elapsed / nd
    dact = [int((blk.routing.counts > 0).sum().item()) for blk in dblocks]
    dbytes = sum(E * H * 4 + (a + 1) * per_expert + 2 * H * 2 for a in dact)
    decode = {
        "steps": nd, "us_per_step": round(1e6 * step_s, 2), "us_per_layer": round(1e6 * step_s / L, 3),
        "layer_tokens_per_s": round(L / step_s, 1),
        "alg_GBps": round(dbytes / step_s / 1e9, 1),
        "hbm_frac": round(dbytes / step_s / 1e9 / HBM_PEAK_GBS, 4),
    }
    return {"workload": f"stack of 40 seeded layers (Zipf-biased routers): T={T} prefill, "
                        f"then {nd} T=1 decode steps (captured graph)",
            "weights_GB": round(L * (E * H * 4 + (E + 1) * per_expert) / 1e9, 2),
            "prefill": prefill, "decode": decode}


def run_crossover(args, ev):
    """Verification-batch study: one decode step (40 layers, captured graph) at each
    T, through the GEMV path (T <= 8) and through the grouped MFMA path, with the
    expert union |U| each T activates and the bytes it must stream."""
    import torch
    from w4_dequant_grouped_amd import moe_w4 as B
    from w4_dequant_grouped_amd import synth

    H, I, E, k, L = 2048, 512, 256, 8, args.layers
    Ts = [int(t) for t in args.crossover_tokens.split(",")]
    shape = synth.BlockShape(T=1, H=H, I=I, E=E, top_k=k)
    layers = make_layers(shape, L, 1000, "cuda")
    gu_b, dn_b = expert_bytes(H, I)
    per_expert = 2 * gu_b + dn_b
    ws = B.alloc_workspace(B.make_dims(max(Ts), H, I, E, k))
    steps, warm = args.steps, args.warmup
    rows = []
    for T in Ts:
        nx = steps + warm
        xstk = torch.randn((nx, L, T, H), generator=synth.generator(700 + T, "cuda"),
                           device="cuda").to(torch.bfloat16)
        paths = [("gemv", B.MOE_W4_FORWARD_GEMV)] if T <= B.MOE_W4_GEMV_MAX_T else []
        paths.append(("grouped", B.MOE_W4_FORWARD_GROUPED))
        row = {"T": T}
        for name, flags in paths:
            print(f"[bench] crossover T={T} {name}", file=sys.stderr, flush=True)
            blocks = [B.Block(layer, T, k, workspace=ws, flags=flags) for layer in layers]
            dg = DecodeGraph(blocks, T, H)
            dg.check(xstk[0], xstk[1 % nx])
            elapsed = time_steps(lambda i=0: dg.step(xstk[i % nx]), steps, warm)
            step_s = elapsed / steps
            active = [int((blk.routing.counts > 0).sum().item()) for blk in blocks]
            nbytes = sum(E * H * 4 + (a + 1) * per_expert + 2 * T * H * 2 for a in active)
            row["active_experts"] = sum(active) / L
            row["alg_MB_per_layer"] = round(nbytes / L / 1e6, 3)
            row[name] = {"us_per_layer": round(1e6 * step_s / L, 3),
                         "tokens_per_s": round(L * T / step_s, 1),
                         "alg_GBps": round(nbytes / step_s / 1e9, 1),
                         "hbm_frac": round(nbytes / step_s / 1e9 / HBM_PEAK_GBS, 4)}
            del dg, blocks
            torch.cuda.empty_cache()
        row["faster"] = min((n for n, _ in paths), key=lambda n: row[n]["us_per_layer"])
        rows.append(row)
    base = rows[0]
    for row in rows:
        best = min(row[n]["us_per_layer"] for n in ("gemv", "grouped") if n in row)
        b0 = min(base[n]["us_per_layer"] for n in ("gemv", "grouped") if n in base)
        row["time_vs_T%d" % base["T"]] = round(best / b0, 3)
        row["bytes_vs_T%d" % base["T"]] = round(row["alg_MB_per_layer"] / base["alg_MB_per_layer"], 3)
    return {"workload": f"decode steps of {L} seeded layers (uniform-logit routers) at T rows per "
                        f"layer-call, GEMV path vs grouped MFMA path, each step a captured graph",
            "steps": steps, "warmup": warm, "default_gemv_max_T": B.MOE_W4_DECODE_MAX_T, "rows": rows}


def run_attn(args, ev):
    """Decode attention: one query token over n_ctx cached tokens, for the model's
    10 full-attention layers (10 caches used in rotation, so a step reads every
    cache from HBM).  Each step is the 10 calls captured as a HIP graph."""
    import torch
    from w4_dequant_grouped_amd import moe_w4 as B
    from w4_dequant_grouped_amd import synth_attn as SA

    L = 10
    rows = []
    for name in args.attn_contexts.split(","):
        shape, seed = SA.ATTN_WORKLOADS[name]
        print(f"[bench] attn {name}", file=sys.stderr, flush=True)
        res = {"workload": name, "n_ctx": shape.n_ctx}
        for variant in args.attn_variants.split(","):
            if variant == "unpacked":
                # every query head with its own copy of its cache head: the reads an
                # unpacked kernel makes (G times the bytes)
                sh = SA.AttnShape(n_ctx=shape.n_ctx, n_q_heads=16, n_kv_heads=16)
            else:
                sh = shape
            steps = []
            for l in range(L):
                x = SA.draw_attn(sh, seed + 1000 * l, device="cuda")
                if variant == "contiguous":
                    x.table = torch.arange(sh.n_blocks, dtype=torch.int32, device="cuda")
                steps.append(B.AttnDecode(sh, x))
            for st in steps:
                st()
            torch.cuda.synchronize()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                for st in steps:
                    st()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            ref = [st.out.clone() for st in steps]
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for st in steps:
                    st()
            g.replay()
            torch.cuda.synchronize()
            for st, r in zip(steps, ref):
                if not torch.equal(st.out, r):
                    raise RuntimeError("attention graph replay differs from the eager calls")
            elapsed = time_steps(lambda i=0: g.replay(), args.steps, args.warmup)
            us = 1e6 * elapsed / (args.steps * L)
            nbytes = SA.attn_bytes(sh)
            ent = {"us_per_layer": round(us, 3), "alg_MB": round(nbytes / 1e6, 2),
                   "alg_GBps": round(nbytes / (us * 1e-6) / 1e9, 1),
                   "hbm_frac": round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)}
            if variant == "paged":
                kt = {n: 0.0 for n in ATTN}
                reps = 5
                evs = []
                for r in range(reps):
                    for st in steps:
                        e = ev.create(4)
                        assert st.timed(e) == 2
                        evs.append(e)
                torch.cuda.synchronize()
                for e in evs:
                    kt["attn_split"] += ev.elapsed_ms(e[0], e[1])
                    kt["attn_combine"] += ev.elapsed_ms(e[2], e[3])
                    ev.destroy(e)
                kt = {n: 1e3 * v / len(evs) for n, v in kt.items()}
                split_bytes = nbytes - 2 * sh.n_q_heads * sh.head_dim * 2   # K, V, q, table
                ach = split_bytes / (kt["attn_split"] * 1e-6) / 1e9
                ent["roofline"] = {"bound": "hbm", "kernel": "attn_split", "achieved": round(ach, 1),
                                   "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                                   "traffic": traffic_from_profiles("attn_split", name),
                                   "alg_bytes_per_launch": int(split_bytes),
                                   "avg_launch_us": round(kt["attn_split"], 3),
                                   "kernel_us": {n: round(v, 3) for n, v in kt.items()}}
            res[variant] = ent
            del steps, g
            torch.cuda.empty_cache()
        if "unpacked" in res and "paged" in res:
            res["packing_speedup"] = round(res["unpacked"]["us_per_layer"] / res["paged"]["us_per_layer"], 3)
        if "contiguous" in res and "paged" in res:
            res["paged_vs_contiguous"] = round(res["contiguous"]["us_per_layer"] / res["paged"]["us_per_layer"], 3)
        rows.append(res)
    return rows


def gdn_chunked_scan_bytes(shape) -> int:
    """Bytes the chunked scan kernel streams per launch: the operand fragments the
    prep kernel wrote (per chunk and value head: -W 32 KiB, the six Pm fragments
    on or below the diagonal 12 KiB, Vt 32 KiB, the decays 512 B; per chunk and
    key head: K^T and Q fragments 32 KiB), the outputs, and the state in and out."""
    T, Hv, Hk, d = shape.T, shape.n_v_heads, shape.n_k_heads, shape.dim
    nch = (T + 63) // 64
    return nch * (Hv * (32768 + 12288 + 32768 + 512) + Hk * 32768) + T * Hv * d * 2 + 2 * Hv * d * d * 4


def gdn_prep_bytes(shape) -> int:
    """Bytes the chunked form's prep kernel moves per launch: q, k, v, the decays
    and write strengths in, the operand fragments out."""
    T, Hv, Hk, d = shape.T, shape.n_v_heads, shape.n_k_heads, shape.dim
    nch = (T + 63) // 64
    return 2 * T * Hk * d * 2 + T * Hv * d * 2 + 2 * T * Hv * 4 + \
        nch * (Hv * (32768 + 12288 + 32768 + 512) + Hk * 32768)


def run_gdn(args, ev):
    """Gated DeltaNet scan: prefill scans (T=512, 2048) over 4 layers in rotation on
    the chunked MFMA form (the register-resident scan timed on the same inputs),
    and T=1 decode steps of the register scan over 30 layer states in rotation (a
    step is the 30 scans).  Each is captured as a HIP graph and checked against
    the eager calls."""
    import torch
    from w4_dequant_grouped_amd import moe_w4 as B
    from w4_dequant_grouped_amd import synth_gdn as SG

    res = {}
    layers = {"prefill512": 4, "prefill2048": 4, "decode": 30}
    for name in args.gdn_workloads.split(","):
        L = layers[name]
        shape, seed = SG.GDN_WORKLOADS[name]
        print(f"[bench] gdn {name}", file=sys.stderr, flush=True)
        xs = [SG.draw_gdn(shape, seed + 100 * l, device="cuda") for l in range(L)]
        outs = [torch.empty_like(x.v) for x in xs]
        states = [x.state.clone() for x in xs]
        ws = torch.empty(max(B.moe_w4_gdn_chunked_workspace_bytes(shape.T, shape.n_v_heads, shape.n_k_heads), 16),
                         dtype=torch.uint8, device="cuda")

        def scan(chunked, x, st, o, events=None):
            if chunked:
                return B.moe_w4_gdn_scan_chunked(x.q, x.k, x.v, x.g, x.beta, st, o, ws, events=events)
            return B.moe_w4_gdn_scan(x.q, x.k, x.v, x.g, x.beta, st, o, events=events)

        def measure(chunked):
            def body():
                for x, o, st in zip(xs, outs, states):
                    scan(chunked, x, st, o)

            body()
            torch.cuda.synchronize()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                body()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                body()
            # a replay must equal the eager calls from the same states
            snap = [st.clone() for st in states]
            body()
            torch.cuda.synchronize()
            ref = [o.clone() for o in outs] + [st.clone() for st in states]
            for st, s0 in zip(states, snap):
                st.copy_(s0)
            g.replay()
            torch.cuda.synchronize()
            if not all(torch.equal(a, b) for a, b in zip(outs + states, ref)):
                raise RuntimeError("Gated DeltaNet graph replay differs from the eager calls")
            steps = args.steps if name == "decode" else max(5, args.steps // 10)
            elapsed = time_steps(lambda i=0: g.replay(), steps, args.warmup)
            us = 1e6 * elapsed / (steps * L)
            # per-kernel durations: kernel i of each call (prep, scan per segment)
            per = {}
            for r in range(3):
                for x, o, st in zip(xs, outs, states):
                    e = ev.create(16)
                    n = scan(chunked, x, st, o, events=e)
                    torch.cuda.synchronize()
                    for i in range(n):
                        per.setdefault(i, []).append(1e3 * ev.elapsed_ms(e[2 * i], e[2 * i + 1]))
                    ev.destroy(e)
            del g
            return us, {i: sum(v) / len(v) for i, v in per.items()}

        nbytes, flops = SG.gdn_bytes(shape), SG.gdn_flops(shape)
        if name == "decode":
            us, per = measure(False)
            k_us = per[0]
            ach = nbytes / (k_us * 1e-6) / 1e9
            ent = {"T": shape.T, "layers": L, "path": "register scan", "us_per_layer": round(us, 3),
                   "tokens_per_s": round(shape.T / (us * 1e-6), 1), "alg_MB": round(nbytes / 1e6, 3),
                   "alg_GFLOP": round(flops / 1e9, 3), "kernel_us": round(k_us, 3)}
            ent["roofline"] = {"bound": "hbm", "kernel": "gdn_scan", "achieved": round(ach, 1),
                               "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                               "traffic": traffic_from_profiles("gdn_scan", name),
                               "alg_bytes_per_launch": int(nbytes), "avg_launch_us": round(k_us, 3)}
        else:
            r_us, r_per = measure(False)
            c_us, c_per = measure(True)
            nseg = len(c_per) // 2
            prep_us = sum(c_per[2 * i] for i in range(nseg)) / nseg
            scan_us = sum(c_per[2 * i + 1] for i in range(nseg)) / nseg
            sb, pb = gdn_chunked_scan_bytes(shape), gdn_prep_bytes(shape)
            ent = {"T": shape.T, "layers": L, "path": "chunked MFMA form (prep + chunk scan)",
                   "us_per_layer": round(c_us, 3), "tokens_per_s": round(shape.T / (c_us * 1e-6), 1),
                   "register_us_per_layer": round(r_us, 3),
                   "register_tokens_per_s": round(shape.T / (r_us * 1e-6), 1),
                   "speedup_vs_register": round(r_us / c_us, 2),
                   "alg_MB": round(nbytes / 1e6, 3), "alg_GFLOP": round(flops / 1e9, 3),
                   "kernels_us": {"gdn_prep": round(prep_us, 2), "gdn_chunk_scan": round(scan_us, 2),
                                  "launches_per_kind": nseg}}
            ach = sb / (scan_us * 1e-6) / 1e9
            ent["roofline"] = {"bound": "hbm", "kernel": "gdn_chunk_scan", "achieved": round(ach, 1),
                               "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4),
                               "traffic": traffic_from_profiles("gdn_chunk_scan", name),
                               "alg_bytes_per_launch": int(sb), "avg_launch_us": round(scan_us, 3)}
            pach = pb / (prep_us * 1e-6) / 1e9
            ent["prep_roofline"] = {"bound": "hbm", "kernel": "gdn_prep", "achieved": round(pach, 1),
                                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(pach / HBM_PEAK_GBS, 4),
                                    "traffic": traffic_from_profiles("gdn_prep", name),
                                    "alg_bytes_per_launch": int(pb), "avg_launch_us": round(prep_us, 3)}
            rk = r_per[0]
            rach = flops / (rk * 1e-6) / 1e12
            ent["register_roofline"] = {"bound": "alu", "kernel": "gdn_scan", "achieved": round(rach, 2),
                                        "peak": VALU_FP32_PEAK_TFLOPS, "unit": "TFLOP/s",
                                        "frac": round(rach / VALU_FP32_PEAK_TFLOPS, 4),
                                        "alg_flops_per_launch": int(flops), "avg_launch_us": round(rk, 3)}
        res[name] = ent
        del xs, outs, states, ws
        torch.cuda.empty_cache()
    return res


def gdn_cpu_baseline(budget_s=15.0):
    """The scan oracle on this host, on a bounded sample (T=512, full heads)."""
    from threadpoolctl import threadpool_info

    from oracle import gdn_oracle as D
    from w4_dequant_grouped_amd import synth_gdn as SG

    shape, seed = SG.GDN_WORKLOADS["prefill512"]
    x = SG.draw_gdn(shape, seed)
    calls = 0
    t0 = time.perf_counter()
    while calls < 10 and time.perf_counter() - t0 < budget_s:
        D.gdn_scan(x.q, x.k, x.v, x.g, x.beta, x.state)
        calls += 1
    el = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(calls * shape.T / el, 1), "unit": "tokens/s (one layer, T=512)", "cores": threads,
            "kind": "oracle", "sample": f"{calls} scans of T=512 over 32 value heads, float64 NumPy oracle, "
                                        f"{el:.1f} s"}


def attn_cpu_baseline(budget_s=15.0):
    """The attention oracle on this host, on a bounded sample (32K context)."""
    from threadpoolctl import threadpool_info

    from oracle import attn_oracle as A
    from w4_dequant_grouped_amd import synth_attn as SA

    shape, seed = SA.ATTN_WORKLOADS["ctx32k"]
    x = SA.draw_attn(shape, seed)
    calls = 0
    t0 = time.perf_counter()
    while calls < 20 and time.perf_counter() - t0 < budget_s:
        A.decode_attention(x.q, x.k_pool, x.v_pool, x.table, shape.n_ctx)
        calls += 1
    el = time.perf_counter() - t0
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    return {"value": round(calls / el, 3), "unit": "layer-steps/s (32K context)", "cores": threads,
            "kind": "oracle", "sample": f"{calls} decode-attention steps at 32K context, float64 NumPy "
                                        f"oracle, {el:.1f} s"}


def _thread_counts():
    """Threads of the host's BLAS and OpenMP pools (threadpoolctl), and the CPU count."""
    from threadpoolctl import threadpool_info
    info = threadpool_info()
    blas = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "blas"] + [1])
    omp = max([i.get("num_threads", 1) for i in info if i.get("user_api") == "openmp"] + [0])
    return blas, omp, os.cpu_count()


def cpu_baseline(shape=None, seed=1000, max_calls=24, budget_s=20.0, what="decode"):
    """The oracle as it stands, on this host's cores, on a bounded sample: whole
    layer-calls (route + grouped forward) of one seeded layer of ``shape`` with
    fresh activations per call, until ``max_calls`` calls or ``budget_s`` seconds.
    The oracle's matrix products run on the BLAS pool; its dequantisation and
    routing loops run on one thread."""
    from oracle import moe_w4_oracle as O
    from w4_dequant_grouped_amd import synth

    if shape is None:
        shape = synth.BlockShape(T=1, H=2048, I=512, E=256, top_k=8)
    layer = synth.draw_layer(shape, seed, device="cpu")
    calls = 0
    t0 = time.perf_counter()
    while calls < max_calls and (calls == 0 or time.perf_counter() - t0 < budget_s):
        x = synth.draw_x(shape.T, shape.H, 500 + calls)
        r = O.route(x, layer.router_w, layer.router_b, shape.top_k)
        O.forward_grouped(x, layer, r, shape.group)
        calls += 1
    el = time.perf_counter() - t0
    blas, omp, ncpu = _thread_counts()
    unit = "layer-tokens/s" if shape.T == 1 else "tokens/s"
    return {"value": round(calls * shape.T / el, 3), "unit": unit, "cores": blas,
            "blas_threads": blas, "openmp_threads": omp, "host_cpus": ncpu, "kind": "oracle",
            "sample": f"{calls} whole {what} layer-call(s) ({synth.describe(shape)}) of one seeded "
                      f"layer, float64 NumPy oracle (route + grouped forward), {el:.1f} s; matrix "
                      f"products on {blas} BLAS threads, dequantisation and routing on one"}


def stack_cpu_baseline(nrows=16, budget_s=20.0):
    """The oracle on a fixed sample of the 40-layer stack workload: nrows token rows
    of one T=16384 layer (Zipf-biased router), routed over all 16384 tokens and then
    run through the per-token dense form, one row at a time."""
    from oracle import moe_w4_oracle as O
    from w4_dequant_grouped_amd import synth

    wl = synth.WORKLOADS["stack40"]
    layer = synth.draw_layer(wl.shape, 4000, device="cpu")
    x = synth.draw_x(wl.shape.T, wl.shape.H, 4)
    t0 = time.perf_counter()
    r = O.route(x, layer.router_w, layer.router_b, wl.shape.top_k)
    t_route = time.perf_counter() - t0
    rows, cache, done = list(range(0, wl.shape.T, wl.shape.T // nrows))[:nrows], {}, 0
    t1 = time.perf_counter()
    for t in rows:
        O.forward_dense(x, layer, r, wl.shape.group, rows=[t], cache=cache)
        done += 1
        if time.perf_counter() - t1 > budget_s:
            break
    el = time.perf_counter() - t1
    blas, omp, ncpu = _thread_counts()
    return {"value": round(done / el, 3), "unit": "token rows/s (sampled, per layer)", "cores": blas,
            "blas_threads": blas, "openmp_threads": omp, "host_cpus": ncpu, "kind": "oracle",
            "sample": f"routing of all {wl.shape.T} tokens of one seeded stack layer ({t_route:.1f} s), then "
                      f"{done} evenly spaced token rows through the per-token dense form ({el:.1f} s), "
                      f"float64 NumPy oracle; sampled, not a whole layer-call"}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--tokens", type=int, default=1, help="decode rows per layer-call (1..5)")
    ap.add_argument("--entry", choices=("block", "split"), default="block",
                    help="decode through moe_w4_block (default) or moe_w4_route + moe_w4_forward "
                         "(throughput only; kernel timings always use moe_w4_block)")
    ap.add_argument("--layers", type=int, default=40)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--prefill-only", type=int, default=0, metavar="T",
                    help="run only the prefill layer-call at T tokens (2048: Zipf-skewed router; "
                         "any other T: uniform-ish routing) and print its JSON")
    ap.add_argument("--no-graph", action="store_true",
                    help="time the decode step as eager block calls instead of a captured graph")
    ap.add_argument("--stack", action="store_true",
                    help="only run the 40-layer stack (T=16384 prefill + T=1 decode steps)")
    ap.add_argument("--stack-tokens", type=int, default=16384)
    ap.add_argument("--stack-decode-steps", type=int, default=256)
    ap.add_argument("--gdn", action="store_true",
                    help="only run the Gated DeltaNet scan (prefill T=512/2048, T=1 decode steps)")
    ap.add_argument("--gdn-workloads", default="prefill512,prefill2048,decode")
    ap.add_argument("--attn", action="store_true",
                    help="only run decode attention over a paged KV cache (32K/64K/128K context)")
    ap.add_argument("--attn-contexts", default="ctx32k,ctx64k,ctx128k")
    ap.add_argument("--attn-variants", default="paged,contiguous,unpacked",
                    help="paged: seeded block table; contiguous: identity table; unpacked: every "
                         "query head with its own cache head (the reads of an unpacked kernel)")
    ap.add_argument("--crossover", action="store_true",
                    help="only run the verification-batch study: GEMV vs grouped path per T")
    ap.add_argument("--crossover-tokens", default="1,2,3,4,5,6,7,8,12,16,24,32,48,64")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy (fp32 negate) of MIB MiB three times: the "
                         "reference kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the block's multi-GPU sharding is a design note, not built).", file=sys.stderr)
        sys.exit(2)

    import torch
    from w4_dequant_grouped_amd import moe_w4 as B
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_probe:
        n = args.copy_probe << 18                      # fp32 elements in MIB MiB
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            torch.neg(src, out=dst)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes_read": 4 * n, "copy_probe_bytes_written": 4 * n,
                          "launches": 3}), flush=True)
        return
    B.load_library()          # raises if the HIP library is missing: there is no fallback
    ev = HipEvents()
    if args.gdn:
        line = {"gated_deltanet": run_gdn(args, ev), "n_gpus": 1, "dtype": "fp32 state, bf16 io",
                "data": "synthetic (seeded q, k, v, decays, write strengths, states)",
                "source_hash": source_hash()}
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = gdn_cpu_baseline()
        print(json.dumps(line), flush=True)
        return
    if args.attn:
        line = {"attention": run_attn(args, ev), "n_gpus": 1, "dtype": "bf16",
                "data": "synthetic (seeded bf16 q, K, V; seeded block tables)", "source_hash": source_hash()}
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = attn_cpu_baseline()
        print(json.dumps(line), flush=True)
        return
    if args.crossover:
        line = {"crossover": run_crossover(args, ev), "n_gpus": 1, "dtype": "bf16",
                "data": "synthetic (seeded W4 layers and activations)", "source_hash": source_hash()}
        print(json.dumps(line), flush=True)
        return
    if args.prefill_only:
        T = args.prefill_only
        line = {"prefill": run_prefill(args, ev, T=T, zipf=(T == 2048)), "n_gpus": 1, "dtype": "bf16",
                "data": "synthetic (seeded W4 layers and activations)", "source_hash": source_hash()}
        print(json.dumps(line), flush=True)
        return
    if args.stack:
        print("[bench] stack: 40 layers", file=sys.stderr, flush=True)
        line = {"stack": run_stack(args, ev), "n_gpus": 1, "dtype": "bf16",
                "data": "synthetic (seeded W4 layers and activations)", "source_hash": source_hash()}
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = stack_cpu_baseline()
        print(json.dumps(line), flush=True)
        return

    print(f"[bench] decode: {args.layers} layers, T={args.tokens}, steps={args.steps}", file=sys.stderr, flush=True)
    value, ms_per_step, roofline, config = run_decode(args, ev)
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "layer-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded W4 layers and activations)", "config": config,
        "roofline": roofline,
    }
    torch.cuda.empty_cache()
    if not args.no_prefill:
        print("[bench] prefill T=2048 zipf", file=sys.stderr, flush=True)
        line["prefill"] = run_prefill(args, ev)
        torch.cuda.empty_cache()
        print("[bench] prefill T=512 uniform", file=sys.stderr, flush=True)
        line["prefill_T512"] = run_prefill(args, ev, T=512, zipf=False)
        torch.cuda.empty_cache()
        print("[bench] prefill T=2048 uniform", file=sys.stderr, flush=True)
        line["prefill_T2048_uniform"] = run_prefill(args, ev, T=2048, zipf=False)
        torch.cuda.empty_cache()
        print("[bench] tiny block", file=sys.stderr, flush=True)
        line["tiny"] = run_tiny(args)
    if not args.no_cpu_baseline:
        from w4_dequant_grouped_amd import synth
        print("[bench] cpu baseline (oracle): decode", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(synth.BlockShape(T=args.tokens, H=2048, I=512, E=256, top_k=8),
                                            what="decode")
        if "prefill" in line:
            print("[bench] cpu baseline (oracle): prefill", file=sys.stderr, flush=True)
            line["prefill"]["cpu_baseline"] = cpu_baseline(
                synth.WORKLOADS["prefill2048_zipf"].shape, seed=3000, max_calls=1, what="prefill T=2048 Zipf")
            line["prefill_T512"]["cpu_baseline"] = cpu_baseline(
                synth.WORKLOADS["prefill512"].shape, seed=3000, max_calls=1, what="prefill T=512")
            line["prefill_T2048_uniform"]["cpu_baseline"] = {
                "same_as": "prefill.cpu_baseline",
                "note": "the oracle's cost does not depend on the routing skew; not timed twice"}
            wl = synth.WORKLOADS["tiny"]
            line["tiny"]["cpu_baseline"] = cpu_baseline(wl.shape, seed=wl.seed, max_calls=200, budget_s=5.0,
                                                        what="tiny")
    print("[bench] measured ceilings", file=sys.stderr, flush=True)
    ceil = measure_ceilings()
    line["ceilings"] = ceil
    rf = line["roofline"]
    rf["frac_of_measured_copy"] = round(rf["achieved"] / ceil["copy_GBps"], 4)
    rf["frac_of_measured_read"] = round(rf["achieved"] / ceil["read_GBps"], 4)
    if "prefill_T512" in line:
        p5 = line["prefill_T512"]["roofline"]
        p5["frac_of_measured_read"] = round(p5["achieved"] / ceil["read_GBps"], 4)
    if "prefill" in line:
        pr = line["prefill"]["roofline"]
        pr["frac_of_measured_gemm"] = round(pr["achieved"] / ceil["bf16_gemm_TFLOPs"], 4)
    line["source_hash"] = source_hash()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
