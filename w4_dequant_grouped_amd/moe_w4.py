"""Python binding of libmoe_w4.so (argument marshalling only).

The names mirror the C ABI declared in include/moe_w4.h and include/moe_w4_attn.h.  torch tensors supply
device memory and the current HIP stream; every step of the block runs in the
library's HIP kernels.  There is no fallback: if the library is missing, the
calls raise.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_w4.so")

MOE_W4_DECODE_MAX_T = 7
MOE_W4_GEMV_MAX_T = 8
MOE_W4_FORWARD_GEMV = 1
MOE_W4_FORWARD_GROUPED = 2
MOE_W4_CONTROL_BYTES = 4096
MOE_W4_CONTROL_ERRORS_OFFSET = 4092
MOE_W4_NOALLOC_SCRATCH_BYTES = 32 << 20


class moe_w4_dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32),
                ("E", ctypes.c_int32), ("top_k", ctypes.c_int32), ("group", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class moe_w4_mat(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p), ("biases", ctypes.c_void_p)]


class moe_w4_weights(ctypes.Structure):
    _fields_ = [("gate", moe_w4_mat), ("up", moe_w4_mat), ("down", moe_w4_mat)]


class moe_w4_attn_dims(ctypes.Structure):
    _fields_ = [("n_ctx", ctypes.c_int32), ("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block", ctypes.c_int32),
                ("n_pool_blocks", ctypes.c_int32), ("flags", ctypes.c_uint32)]


MOE_W4_ATTN_MAX_CTX = 1 << 20


class moe_w4_gdn_dims(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("n_v_heads", ctypes.c_int32), ("n_k_heads", ctypes.c_int32),
                ("dim", ctypes.c_int32), ("flags", ctypes.c_uint32)]


MOE_W4_GDN_MAX_T = 1 << 20

EXPORTS = ("moe_w4_workspace_bytes", "moe_w4_route", "moe_w4_forward", "moe_w4_block",
           "moe_w4_route_timed", "moe_w4_forward_timed", "moe_w4_block_timed", "moe_w4_block_noalloc",
           "moe_w4_status_string", "moe_w4_last_error",
           "moe_w4_attn_workspace_bytes", "moe_w4_attn_decode", "moe_w4_attn_decode_timed",
           "moe_w4_gdn_scan", "moe_w4_gdn_scan_timed", "moe_w4_gdn_chunked_workspace_bytes",
           "moe_w4_gdn_scan_chunked", "moe_w4_gdn_scan_chunked_timed")

_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m w4_dequant_grouped_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.moe_w4_workspace_bytes.argtypes = [ctypes.POINTER(moe_w4_dims)]
    lib.moe_w4_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_w4_route.argtypes = [ctypes.POINTER(moe_w4_dims), P, P, P, P, P, P, P, P, P,
                                 ctypes.c_size_t, P]
    lib.moe_w4_route.restype = ctypes.c_int
    lib.moe_w4_forward.argtypes = [ctypes.POINTER(moe_w4_dims), P, ctypes.POINTER(moe_w4_weights),
                                   ctypes.POINTER(moe_w4_weights), P, P, P, P, P, P,
                                   ctypes.c_size_t, P]
    lib.moe_w4_forward.restype = ctypes.c_int
    W = ctypes.POINTER(moe_w4_weights)
    lib.moe_w4_block.argtypes = [ctypes.POINTER(moe_w4_dims), P, P, P, W, W, P, P, P, P, P, P, P,
                                 ctypes.c_size_t, P]
    lib.moe_w4_block.restype = ctypes.c_int
    lib.moe_w4_block_timed.argtypes = lib.moe_w4_block.argtypes + [P, ctypes.c_int, P]
    lib.moe_w4_block_timed.restype = ctypes.c_int
    lib.moe_w4_block_noalloc.argtypes = [ctypes.POINTER(moe_w4_dims), P, P, P, W, W, P, P, P, P, P, P, P]
    lib.moe_w4_block_noalloc.restype = ctypes.c_int
    lib.moe_w4_route_timed.argtypes = lib.moe_w4_route.argtypes + [P, ctypes.c_int, P]
    lib.moe_w4_route_timed.restype = ctypes.c_int
    lib.moe_w4_forward_timed.argtypes = lib.moe_w4_forward.argtypes + [P, ctypes.c_int, P]
    lib.moe_w4_forward_timed.restype = ctypes.c_int
    lib.moe_w4_status_string.argtypes = [ctypes.c_int]
    lib.moe_w4_status_string.restype = ctypes.c_char_p
    lib.moe_w4_last_error.argtypes = []
    lib.moe_w4_last_error.restype = ctypes.c_char_p
    A = ctypes.POINTER(moe_w4_attn_dims)
    lib.moe_w4_attn_workspace_bytes.argtypes = [A]
    lib.moe_w4_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_w4_attn_decode.argtypes = [A, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_w4_attn_decode.restype = ctypes.c_int
    lib.moe_w4_attn_decode_timed.argtypes = lib.moe_w4_attn_decode.argtypes + [P, ctypes.c_int, P]
    lib.moe_w4_attn_decode_timed.restype = ctypes.c_int
    D = ctypes.POINTER(moe_w4_gdn_dims)
    lib.moe_w4_gdn_scan.argtypes = [D, P, P, P, P, P, P, P, P]
    lib.moe_w4_gdn_scan.restype = ctypes.c_int
    lib.moe_w4_gdn_scan_timed.argtypes = lib.moe_w4_gdn_scan.argtypes + [P, ctypes.c_int, P]
    lib.moe_w4_gdn_scan_timed.restype = ctypes.c_int
    lib.moe_w4_gdn_chunked_workspace_bytes.argtypes = [D]
    lib.moe_w4_gdn_chunked_workspace_bytes.restype = ctypes.c_size_t
    lib.moe_w4_gdn_scan_chunked.argtypes = [D, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.moe_w4_gdn_scan_chunked.restype = ctypes.c_int
    lib.moe_w4_gdn_scan_chunked_timed.argtypes = lib.moe_w4_gdn_scan_chunked.argtypes + [P, ctypes.c_int, P]
    lib.moe_w4_gdn_scan_chunked_timed.restype = ctypes.c_int
    _lib = lib
    return lib


def make_dims(T: int, H: int, I: int, E: int, top_k: int, group: int = 64, flags: int = 0) -> moe_w4_dims:
    return moe_w4_dims(T, H, I, E, top_k, group, flags)


def moe_w4_status_string(status: int) -> str:
    return load_library().moe_w4_status_string(status).decode()


def moe_w4_last_error() -> str:
    return load_library().moe_w4_last_error().decode()


def _check(status: int, what: str) -> None:
    if status != 0:
        msg = moe_w4_status_string(status)
        extra = moe_w4_last_error() if status == -7 else ""
        raise RuntimeError(f"{what} failed ({status}): {msg} {extra}".strip())


def moe_w4_workspace_bytes(dims: moe_w4_dims) -> int:
    return int(load_library().moe_w4_workspace_bytes(ctypes.byref(dims)))


def alloc_workspace(dims: moe_w4_dims, device="cuda") -> torch.Tensor:
    """A zero-filled workspace of the size the library asks for."""
    n = moe_w4_workspace_bytes(dims)
    if n == 0:
        raise ValueError("invalid dims")
    return torch.zeros(n, dtype=torch.uint8, device=device)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, dtype, name: str) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


@dataclass
class Routing:
    ids: torch.Tensor       # int32 [T, k]
    weights: torch.Tensor   # float32 [T, k]
    counts: torch.Tensor    # int32 [E]
    offsets: torch.Tensor   # int32 [E + 1]
    perm: torch.Tensor      # int32 [T * k]


def alloc_routing(T: int, E: int, top_k: int, device="cuda") -> Routing:
    return Routing(torch.empty((T, top_k), dtype=torch.int32, device=device),
                   torch.empty((T, top_k), dtype=torch.float32, device=device),
                   torch.empty((E,), dtype=torch.int32, device=device),
                   torch.empty((E + 1,), dtype=torch.int32, device=device),
                   torch.empty((T * top_k,), dtype=torch.int32, device=device))


def moe_w4_route(dims: moe_w4_dims, x: torch.Tensor, router_w: torch.Tensor,
                 router_b: Optional[torch.Tensor], routing: Routing, workspace: torch.Tensor) -> Routing:
    """Enqueue the router on the current stream; fills ``routing`` in place."""
    _dev(x, torch.bfloat16, "x")
    _dev(router_w, torch.float32, "router_w")
    if router_b is not None:
        _dev(router_b, torch.float32, "router_b")
    for name in ("ids", "counts", "offsets", "perm"):
        _dev(getattr(routing, name), torch.int32, name)
    _dev(routing.weights, torch.float32, "weights")
    _dev(workspace, torch.uint8, "workspace")
    lib = load_library()
    st = lib.moe_w4_route(ctypes.byref(dims), _ptr(x), _ptr(router_w), _ptr(router_b),
                          _ptr(routing.ids), _ptr(routing.weights), _ptr(routing.counts),
                          _ptr(routing.offsets), _ptr(routing.perm), _ptr(workspace),
                          workspace.numel(), _stream())
    _check(st, "moe_w4_route")
    return routing


def weights_struct(experts) -> moe_w4_weights:
    """ctypes descriptor of a set of W4 experts (objects with gate/up/down having
    codes uint8, scales bf16 and biases bf16 device tensors)."""
    mats = []
    for name in ("gate", "up", "down"):
        m = getattr(experts, name)
        _dev(m.codes, torch.uint8, f"{name}.codes")
        _dev(m.scales, torch.bfloat16, f"{name}.scales")
        _dev(m.biases, torch.bfloat16, f"{name}.biases")
        mats.append(moe_w4_mat(_ptr(m.codes), _ptr(m.scales), _ptr(m.biases)))
    return moe_w4_weights(*mats)


def moe_w4_forward(dims: moe_w4_dims, x: torch.Tensor, routed, shared, routing: Routing,
                   out: torch.Tensor, workspace: torch.Tensor,
                   routed_struct: Optional[moe_w4_weights] = None,
                   shared_struct: Optional[moe_w4_weights] = None) -> torch.Tensor:
    """Enqueue the block on the current stream; writes ``out`` (bf16 [T, H]).

    ``routed_struct`` / ``shared_struct`` may carry prebuilt descriptors so a
    timing loop does not rebuild them."""
    _dev(x, torch.bfloat16, "x")
    _dev(out, torch.bfloat16, "out")
    _dev(workspace, torch.uint8, "workspace")
    rs = routed_struct if routed_struct is not None else weights_struct(routed)
    ss = shared_struct if shared_struct is not None else (
        None if shared is None else weights_struct(shared))
    lib = load_library()
    st = lib.moe_w4_forward(ctypes.byref(dims), _ptr(x), ctypes.byref(rs),
                            None if ss is None else ctypes.byref(ss),
                            _ptr(routing.ids), _ptr(routing.weights), _ptr(routing.offsets),
                            _ptr(routing.perm), _ptr(out), _ptr(workspace), workspace.numel(),
                            _stream())
    _check(st, "moe_w4_forward")
    return out


def _check_routing(routing: Routing) -> None:
    for name in ("ids", "counts", "offsets", "perm"):
        _dev(getattr(routing, name), torch.int32, name)
    _dev(routing.weights, torch.float32, "weights")


def moe_w4_block(dims: moe_w4_dims, x: torch.Tensor, router_w: torch.Tensor,
                 router_b: Optional[torch.Tensor], routed_struct: moe_w4_weights,
                 shared_struct: Optional[moe_w4_weights], routing: Routing, out: torch.Tensor,
                 workspace: torch.Tensor, events=None) -> int:
    """Route and forward in one library call.

    With ``events`` (hipEvent handles) the call records them around each kernel
    and returns the kernel count; otherwise returns 0."""
    _dev(x, torch.bfloat16, "x")
    _dev(router_w, torch.float32, "router_w")
    if router_b is not None:
        _dev(router_b, torch.float32, "router_b")
    _check_routing(routing)
    _dev(out, torch.bfloat16, "out")
    _dev(workspace, torch.uint8, "workspace")
    lib = load_library()
    args = (ctypes.byref(dims), _ptr(x), _ptr(router_w), _ptr(router_b), ctypes.byref(routed_struct),
            None if shared_struct is None else ctypes.byref(shared_struct), _ptr(routing.ids),
            _ptr(routing.weights), _ptr(routing.counts), _ptr(routing.offsets), _ptr(routing.perm),
            _ptr(out), _ptr(workspace), workspace.numel(), _stream())
    if events is None:
        _check(lib.moe_w4_block(*args), "moe_w4_block")
        return 0
    arr, cap = _events_arg(events)
    n = ctypes.c_int(0)
    _check(lib.moe_w4_block_timed(*args, arr, cap, ctypes.byref(n)), "moe_w4_block_timed")
    return n.value


def moe_w4_block_noalloc(dims: moe_w4_dims, x: torch.Tensor, router_w: torch.Tensor,
                         router_b: Optional[torch.Tensor], routed_struct: moe_w4_weights,
                         shared_struct: Optional[moe_w4_weights], routing: Routing,
                         out: torch.Tensor) -> None:
    """Route and forward in one library call on the library's own device scratch
    (no workspace argument; the call allocates nothing)."""
    _dev(x, torch.bfloat16, "x")
    _dev(router_w, torch.float32, "router_w")
    if router_b is not None:
        _dev(router_b, torch.float32, "router_b")
    _check_routing(routing)
    _dev(out, torch.bfloat16, "out")
    st = load_library().moe_w4_block_noalloc(
        ctypes.byref(dims), _ptr(x), _ptr(router_w), _ptr(router_b), ctypes.byref(routed_struct),
        None if shared_struct is None else ctypes.byref(shared_struct), _ptr(routing.ids),
        _ptr(routing.weights), _ptr(routing.counts), _ptr(routing.offsets), _ptr(routing.perm),
        _ptr(out), _stream())
    _check(st, "moe_w4_block_noalloc")


def _events_arg(events):
    if events is None:
        return None, 0
    arr = (ctypes.c_void_p * len(events))(*events)
    return arr, len(events)


def moe_w4_route_timed(dims: moe_w4_dims, x: torch.Tensor, router_w: torch.Tensor,
                       router_b: Optional[torch.Tensor], routing: Routing, workspace: torch.Tensor,
                       events=None) -> int:
    """moe_w4_route with hipEvent handles recorded around each kernel; returns the kernel count."""
    arr, cap = _events_arg(events)
    n = ctypes.c_int(0)
    st = load_library().moe_w4_route_timed(
        ctypes.byref(dims), _ptr(x), _ptr(router_w), _ptr(router_b), _ptr(routing.ids),
        _ptr(routing.weights), _ptr(routing.counts), _ptr(routing.offsets), _ptr(routing.perm),
        _ptr(workspace), workspace.numel(), _stream(), arr, cap, ctypes.byref(n))
    _check(st, "moe_w4_route_timed")
    return n.value


def moe_w4_forward_timed(dims: moe_w4_dims, x: torch.Tensor, routed_struct: moe_w4_weights,
                         shared_struct: Optional[moe_w4_weights], routing: Routing,
                         out: torch.Tensor, workspace: torch.Tensor, events=None) -> int:
    """moe_w4_forward with hipEvent handles recorded around each kernel; returns the kernel count."""
    arr, cap = _events_arg(events)
    n = ctypes.c_int(0)
    st = load_library().moe_w4_forward_timed(
        ctypes.byref(dims), _ptr(x), ctypes.byref(routed_struct),
        None if shared_struct is None else ctypes.byref(shared_struct), _ptr(routing.ids),
        _ptr(routing.weights), _ptr(routing.offsets), _ptr(routing.perm), _ptr(out),
        _ptr(workspace), workspace.numel(), _stream(), arr, cap, ctypes.byref(n))
    _check(st, "moe_w4_forward_timed")
    return n.value


class Block:
    """One layer's routed + shared W4 experts and router, bound for repeated calls."""

    def __init__(self, layer, T: int, top_k: int, group: int = 64, workspace: Optional[torch.Tensor] = None,
                 flags: int = 0):
        self.layer = layer
        E, I, H = layer.routed.gate.codes.shape[0], layer.routed.gate.codes.shape[1], layer.router_w.shape[1]
        self.dims = make_dims(T, H, I, E, top_k, group, flags)
        self.routed_struct = weights_struct(layer.routed)
        self.shared_struct = None if layer.shared is None else weights_struct(layer.shared)
        dev = layer.router_w.device
        self.workspace = workspace if workspace is not None else alloc_workspace(self.dims, dev)
        self.routing = alloc_routing(T, E, top_k, dev)
        self.out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)

    def __call__(self, x: torch.Tensor) -> torch.Tensor:
        """Route + forward through the single-call entry point."""
        moe_w4_block(self.dims, x, self.layer.router_w, self.layer.router_b, self.routed_struct,
                     self.shared_struct, self.routing, self.out, self.workspace)
        return self.out

    def split(self, x: torch.Tensor) -> torch.Tensor:
        """Route, then forward, as two separate library calls."""
        moe_w4_route(self.dims, x, self.layer.router_w, self.layer.router_b, self.routing, self.workspace)
        moe_w4_forward(self.dims, x, self.layer.routed, self.layer.shared, self.routing, self.out,
                       self.workspace, self.routed_struct, self.shared_struct)
        return self.out

    def block_timed(self, x: torch.Tensor, events) -> int:
        """One single-call block recording events around every kernel; returns the kernel count."""
        return moe_w4_block(self.dims, x, self.layer.router_w, self.layer.router_b, self.routed_struct,
                            self.shared_struct, self.routing, self.out, self.workspace, events)

    def timed(self, x: torch.Tensor, route_events, forward_events):
        """One call recording events around every kernel; returns (route kernels, forward kernels)."""
        nr = moe_w4_route_timed(self.dims, x, self.layer.router_w, self.layer.router_b, self.routing,
                                self.workspace, route_events)
        nf = moe_w4_forward_timed(self.dims, x, self.routed_struct, self.shared_struct, self.routing,
                                  self.out, self.workspace, forward_events)
        return nr, nf


# ---------------------------------------------------------------------------
# decode attention over a paged KV cache (include/moe_w4_attn.h)
# ---------------------------------------------------------------------------
def make_attn_dims(n_ctx: int, n_q_heads: int, n_kv_heads: int, n_pool_blocks: int,
                   head_dim: int = 128, block: int = 64, flags: int = 0) -> moe_w4_attn_dims:
    return moe_w4_attn_dims(n_ctx, n_q_heads, n_kv_heads, head_dim, block, n_pool_blocks, flags)


def moe_w4_attn_workspace_bytes(dims: moe_w4_attn_dims) -> int:
    return int(load_library().moe_w4_attn_workspace_bytes(ctypes.byref(dims)))


def moe_w4_attn_decode(dims: moe_w4_attn_dims, q: torch.Tensor, k_pool: torch.Tensor,
                       v_pool: torch.Tensor, table: torch.Tensor, out: torch.Tensor,
                       workspace: torch.Tensor, events=None) -> int:
    """One decode-attention step on the current stream; returns the kernel count."""
    for t, dt, name in ((q, torch.bfloat16, "q"), (k_pool, torch.bfloat16, "k_pool"),
                        (v_pool, torch.bfloat16, "v_pool"), (table, torch.int32, "table"),
                        (out, torch.bfloat16, "out"), (workspace, torch.uint8, "workspace")):
        _dev(t, dt, name)
    if table.numel() < (dims.n_ctx + dims.block - 1) // dims.block:
        raise ValueError("block table shorter than the context")
    arr, cap = _events_arg(events)
    n = ctypes.c_int(0)
    st = load_library().moe_w4_attn_decode_timed(
        ctypes.byref(dims), _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(table), _ptr(out),
        _ptr(workspace), workspace.numel(), _stream(), arr, cap, ctypes.byref(n))
    _check(st, "moe_w4_attn_decode")
    return n.value


class AttnDecode:
    """One decode-attention step bound to its cache, for repeated calls."""

    def __init__(self, shape, inputs):
        self.inputs = inputs
        self.dims = make_attn_dims(shape.n_ctx, shape.n_q_heads, shape.n_kv_heads,
                                   inputs.k_pool.shape[0], shape.head_dim, shape.block)
        n = moe_w4_attn_workspace_bytes(self.dims)
        if n == 0:
            raise ValueError("invalid attention dims")
        dev = inputs.q.device
        self.workspace = torch.zeros(n, dtype=torch.uint8, device=dev)
        self.out = torch.empty_like(inputs.q)

    def __call__(self) -> torch.Tensor:
        x = self.inputs
        moe_w4_attn_decode(self.dims, x.q, x.k_pool, x.v_pool, x.table, self.out, self.workspace)
        return self.out

    def timed(self, events) -> int:
        """One call with an event pair per kernel; returns the kernel count."""
        x = self.inputs
        return moe_w4_attn_decode(self.dims, x.q, x.k_pool, x.v_pool, x.table, self.out, self.workspace,
                                  events)


# ---------------------------------------------------------------------------
# Gated DeltaNet scan (include/moe_w4_gdn.h)
# ---------------------------------------------------------------------------
def moe_w4_gdn_scan(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                    beta: torch.Tensor, state: torch.Tensor, out: torch.Tensor, events=None) -> int:
    """One scan on the current stream: state is updated in place, out overwritten.
    Returns the kernel count."""
    for t, dt, name in ((q, torch.bfloat16, "q"), (k, torch.bfloat16, "k"), (v, torch.bfloat16, "v"),
                        (g, torch.float32, "g"), (beta, torch.float32, "beta"),
                        (state, torch.float32, "state"), (out, torch.bfloat16, "out")):
        _dev(t, dt, name)
    T, Hk, d = q.shape
    Hv = v.shape[1]
    if k.shape != q.shape or v.shape != (T, Hv, d) or g.shape != (T, Hv) or beta.shape != (T, Hv) \
            or state.shape != (Hv, d, d) or out.shape != (T, Hv, d):
        raise ValueError("inconsistent Gated DeltaNet shapes")
    dims = moe_w4_gdn_dims(T, Hv, Hk, d, 0)
    arr, cap = _events_arg(events)
    n = ctypes.c_int(0)
    st = load_library().moe_w4_gdn_scan_timed(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(out),
        _stream(), arr, cap, ctypes.byref(n))
    _check(st, "moe_w4_gdn_scan")
    return n.value


def moe_w4_gdn_chunked_workspace_bytes(T: int, n_v_heads: int, n_k_heads: int, dim: int = 128) -> int:
    return int(load_library().moe_w4_gdn_chunked_workspace_bytes(
        ctypes.byref(moe_w4_gdn_dims(T, n_v_heads, n_k_heads, dim, 0))))


def moe_w4_gdn_scan_chunked(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, g: torch.Tensor,
                            beta: torch.Tensor, state: torch.Tensor, out: torch.Tensor,
                            workspace: Optional[torch.Tensor] = None, events=None) -> int:
    """The chunked scan on the current stream (same arguments as moe_w4_gdn_scan plus a
    workspace; one is allocated when none is given).  Returns the kernel count."""
    for t, dt, name in ((q, torch.bfloat16, "q"), (k, torch.bfloat16, "k"), (v, torch.bfloat16, "v"),
                        (g, torch.float32, "g"), (beta, torch.float32, "beta"),
                        (state, torch.float32, "state"), (out, torch.bfloat16, "out")):
        _dev(t, dt, name)
    T, Hk, d = q.shape
    Hv = v.shape[1]
    if k.shape != q.shape or v.shape != (T, Hv, d) or g.shape != (T, Hv) or beta.shape != (T, Hv) \
            or state.shape != (Hv, d, d) or out.shape != (T, Hv, d):
        raise ValueError("inconsistent Gated DeltaNet shapes")
    dims = moe_w4_gdn_dims(T, Hv, Hk, d, 0)
    if workspace is None:
        workspace = torch.empty(max(moe_w4_gdn_chunked_workspace_bytes(T, Hv, Hk, d), 16),
                                dtype=torch.uint8, device=q.device)
    _dev(workspace, torch.uint8, "workspace")
    arr, cap = _events_arg(events)
    n = ctypes.c_int(0)
    st = load_library().moe_w4_gdn_scan_chunked_timed(
        ctypes.byref(dims), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(out),
        _ptr(workspace), workspace.numel(), _stream(), arr, cap, ctypes.byref(n))
    _check(st, "moe_w4_gdn_scan_chunked")
    return n.value
