"""The C ABI on the host: the library loads, exports what include/moe_w4.h
declares, sizes its workspace, and rejects bad arguments before launching
anything.  No call here reaches a kernel launch (each has one defect that the
host-side checks catch first), so these run without a GPU."""
import ctypes
import os
import re

import pytest

from w4_dequant_grouped_amd import moe_w4 as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_w4.h")
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

OK, ERR_NULL, ERR_DIMS, ERR_TOPK, ERR_GROUP, ERR_ALIGN, ERR_WS, ERR_LAUNCH, ERR_FLAGS, ERR_SCRATCH = \
    0, -1, -2, -3, -4, -5, -6, -7, -8, -9

FAKE = 0x7F0000000000          # aligned, never dereferenced: every call below fails validation


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(B.LIB_PATH):
        pytest.skip("library not built")
    return B.load_library()


def declared_functions():
    names = set()
    for path in HEADERS:
        text = open(path).read()
        names |= set(re.findall(r"^\s*(?:const\s+)?[\w\s\*]+?\b(moe_w4_\w+)\s*\(", text, re.M))
    return sorted(names)


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert names == sorted(B.EXPORTS), names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in (OK, ERR_NULL, ERR_DIMS, ERR_TOPK, ERR_GROUP, ERR_ALIGN, ERR_WS, ERR_LAUNCH, ERR_FLAGS,
                 ERR_SCRATCH):
        s = B.moe_w4_status_string(code)
        assert s and s != "unknown status"
    assert B.moe_w4_status_string(12345) == "unknown status"
    assert B.moe_w4_last_error() == ""


def _dims(**kw):
    d = dict(T=16, H=256, I=128, E=16, top_k=2, group=64, flags=0)
    d.update(kw)
    return B.make_dims(**d)


def test_workspace_bytes(lib):
    small = B.moe_w4_workspace_bytes(_dims())
    big = B.moe_w4_workspace_bytes(_dims(T=2048, H=2048, I=512, E=256, top_k=8))
    assert small > 0 and small % 256 == 0
    # K-split partial logits + bf16 split of the router weight + the chosen ids as bytes +
    # h (T*k + T rows of I) + per-(token, slot) bf16 output rows (T*k + T rows of H); no term
    # for expanded expert weights
    T, H, I, E, k = 2048, 2048, 512, 256, 8
    expect_min = (B.MOE_W4_CONTROL_BYTES + 8 * T * E * 4 + 3 * E * H * 2 + T * k
                  + (T * k + T) * I * 2 + (T * k + T) * H * 2)
    assert expect_min <= big <= expect_min + 256 * 8
    # far below a bf16 expansion of the routed gate, up and down weights (1.6 GB)
    assert big < 3 * E * I * H * 2 // 10
    for bad in (_dims(group=32), _dims(H=300), _dims(I=100), _dims(top_k=0), _dims(top_k=17),
                _dims(E=1025), _dims(T=-1), _dims(flags=1), _dims(top_k=20, E=16)):
        assert B.moe_w4_workspace_bytes(bad) == 0


def _route(lib, dims, x=FAKE, wr=FAKE, br=None, ids=FAKE, w=FAKE, cnt=FAKE, off=FAKE, perm=FAKE,
           ws=FAKE, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 1 << 40
    return lib.moe_w4_route(ctypes.byref(dims) if dims is not None else None, x, wr, br, ids, w, cnt,
                            off, perm, ws, ws_bytes, stream)


def _weights(codes=FAKE, scales=FAKE, biases=FAKE):
    m = B.moe_w4_mat(codes, scales, biases)
    good = B.moe_w4_mat(FAKE, FAKE, FAKE)
    return B.moe_w4_weights(m, good, good)


def _forward(lib, dims, x=FAKE, routed=None, shared=None, w=FAKE, off=FAKE, perm=FAKE, out=FAKE + 4096,
             ws=FAKE, ws_bytes=None):
    routed = routed if routed is not None else _weights()
    if ws_bytes is None:
        ws_bytes = 1 << 40
    return lib.moe_w4_forward(ctypes.byref(dims) if dims is not None else None, x,
                              ctypes.byref(routed), None if shared is None else ctypes.byref(shared),
                              None, w, off, perm, out, ws, ws_bytes, None)


def test_route_rejects_bad_arguments(lib):
    assert _route(lib, None) == ERR_NULL
    assert _route(lib, _dims(T=0)) == OK                    # empty batch: nothing to do
    assert _route(lib, _dims(flags=4)) == ERR_FLAGS
    assert _route(lib, _dims(flags=3)) == ERR_FLAGS         # both forward paths
    assert _route(lib, _dims(T=0, flags=B.MOE_W4_FORWARD_GROUPED)) == OK
    assert _route(lib, _dims(T=70000)) == ERR_DIMS
    assert _route(lib, _dims(E=0)) == ERR_DIMS
    assert _route(lib, _dims(top_k=17)) == ERR_TOPK
    assert _route(lib, _dims(top_k=17, E=32)) == ERR_TOPK
    assert _route(lib, _dims(top_k=0)) == ERR_TOPK
    assert _route(lib, _dims(group=128)) == ERR_GROUP
    assert _route(lib, _dims(H=384)) == ERR_GROUP
    assert _route(lib, _dims(), x=None) == ERR_NULL
    assert _route(lib, _dims(), wr=None) == ERR_NULL
    assert _route(lib, _dims(), perm=None) == ERR_NULL
    assert _route(lib, _dims(), ws=None) == ERR_NULL
    assert _route(lib, _dims(), x=FAKE + 2) == ERR_ALIGN
    assert _route(lib, _dims(), wr=FAKE + 4) == ERR_ALIGN
    assert _route(lib, _dims(), ws=FAKE + 64) == ERR_ALIGN
    assert _route(lib, _dims(), br=FAKE + 1) == ERR_ALIGN
    d = _dims()
    assert _route(lib, d, ws_bytes=B.moe_w4_workspace_bytes(d) - 1) == ERR_WS


def test_forward_rejects_bad_arguments(lib):
    assert _forward(lib, None) == ERR_NULL
    assert _forward(lib, _dims(T=0)) == OK
    assert _forward(lib, _dims(flags=1)) == ERR_FLAGS         # GEMV path asked for T=16 > 8
    assert _forward(lib, _dims(flags=8)) == ERR_FLAGS
    assert _forward(lib, _dims(T=8, flags=B.MOE_W4_FORWARD_GEMV), ws_bytes=0) == ERR_WS   # accepted flags
    assert _forward(lib, _dims(I=192)) == ERR_GROUP
    assert _forward(lib, _dims(top_k=3, E=2)) == ERR_TOPK
    assert _forward(lib, _dims(), x=None) == ERR_NULL
    assert _forward(lib, _dims(), out=None) == ERR_NULL
    assert _forward(lib, _dims(), routed=_weights(codes=None)) == ERR_NULL
    assert _forward(lib, _dims(), routed=_weights(scales=None)) == ERR_NULL
    assert _forward(lib, _dims(), shared=_weights(biases=None)) == ERR_NULL
    assert _forward(lib, _dims(), routed=_weights(codes=FAKE + 8)) == ERR_ALIGN
    assert _forward(lib, _dims(), shared=_weights(scales=FAKE + 1)) == ERR_ALIGN
    assert _forward(lib, _dims(), routed=_weights(biases=FAKE + 2)) == ERR_ALIGN
    assert _forward(lib, _dims(), out=FAKE + 2) == ERR_ALIGN
    assert _forward(lib, _dims(), x=FAKE + 8) == ERR_ALIGN
    d = _dims()
    assert _forward(lib, d, ws_bytes=B.moe_w4_workspace_bytes(d) - 256) == ERR_WS


def _noalloc(lib, dims, x=FAKE, wr=FAKE, br=None, routed=None, shared=None, ids=FAKE, w=FAKE, cnt=FAKE,
             off=FAKE, perm=FAKE, out=FAKE + 4096):
    routed = routed if routed is not None else _weights()
    return lib.moe_w4_block_noalloc(ctypes.byref(dims) if dims is not None else None, x, wr, br,
                                    ctypes.byref(routed), None if shared is None else ctypes.byref(shared),
                                    ids, w, cnt, off, perm, out, None)


def test_noalloc_rejects_bad_arguments_before_touching_the_gpu(lib):
    """Every rejection below happens on the host, before the device scratch is
    looked up; shapes whose workspace would not fit the scratch get their own
    status."""
    assert _noalloc(lib, None) == ERR_NULL
    assert _noalloc(lib, _dims(T=0)) == OK
    assert _noalloc(lib, _dims(flags=3)) == ERR_FLAGS
    assert _noalloc(lib, _dims(top_k=0)) == ERR_TOPK
    assert _noalloc(lib, _dims(group=32)) == ERR_GROUP
    full = dict(H=2048, I=512, E=256, top_k=8)
    assert _noalloc(lib, _dims(T=2048, **full)) == ERR_SCRATCH
    assert _noalloc(lib, _dims(), x=None) == ERR_NULL
    assert _noalloc(lib, _dims(), out=None) == ERR_NULL
    assert _noalloc(lib, _dims(), routed=_weights(codes=None)) == ERR_NULL
    assert _noalloc(lib, _dims(), x=FAKE + 2) == ERR_ALIGN
    assert _noalloc(lib, _dims(), routed=_weights(codes=FAKE + 8)) == ERR_ALIGN
    assert _noalloc(lib, _dims(), perm=FAKE + 1) == ERR_ALIGN
    # the largest accepted T at the full-size shape is the one the header states
    fits = [T for T in (512, 560, 561, 580, 600, 1024)
            if B.moe_w4_workspace_bytes(_dims(T=T, **full)) <= B.MOE_W4_NOALLOC_SCRATCH_BYTES]
    assert max(fits) == 560
    assert _noalloc(lib, _dims(T=561, **full)) == ERR_SCRATCH


def test_binding_constants_match_the_header():
    text = open(os.path.join(ROOT, "include", "moe_w4.h")).read()
    for name in ("MOE_W4_DECODE_MAX_T", "MOE_W4_GEMV_MAX_T", "MOE_W4_CONTROL_BYTES", "MOE_W4_FORWARD_GEMV",
                 "MOE_W4_FORWARD_GROUPED", "MOE_W4_CONTROL_ERRORS_OFFSET"):
        m = re.search(r"#define\s+%s\s+(\d+)u?\b" % name, text)
        assert m, name
        assert int(m.group(1)) == getattr(B, name), name
    m = re.search(r"#define\s+MOE_W4_NOALLOC_SCRATCH_BYTES\s+\((\d+)u << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == B.MOE_W4_NOALLOC_SCRATCH_BYTES


# --- decode attention (include/moe_w4_attn.h) ------------------------------------

def _adims(**kw):
    d = dict(n_ctx=1000, n_q_heads=16, n_kv_heads=2, n_pool_blocks=20, head_dim=128, block=64, flags=0)
    d.update(kw)
    return B.make_attn_dims(**d)


def _attn(lib, dims, q=FAKE, k=FAKE, v=FAKE, table=FAKE, out=FAKE + 4096, ws=FAKE, ws_bytes=1 << 40):
    return lib.moe_w4_attn_decode(ctypes.byref(dims) if dims is not None else None, q, k, v, table, out,
                                  ws, ws_bytes, None)


def test_attn_workspace_bytes(lib):
    n32 = B.moe_w4_attn_workspace_bytes(_adims(n_ctx=32768))
    n128 = B.moe_w4_attn_workspace_bytes(_adims(n_ctx=131072))
    assert n32 > 0 and n32 % 256 == 0
    # at most 256 splits per key/value head: (max, sum) x 16 + 8 x 128 numerators each
    assert n128 <= 2 * 256 * (2 * 16 + 8 * 128) * 4 + 3 * 256
    for bad in (_adims(n_ctx=0), _adims(n_ctx=B.MOE_W4_ATTN_MAX_CTX + 1), _adims(n_kv_heads=3),
                _adims(n_q_heads=32, n_kv_heads=1), _adims(head_dim=64), _adims(block=32),
                _adims(n_pool_blocks=0), _adims(flags=1)):
        assert B.moe_w4_attn_workspace_bytes(bad) == 0


def test_attn_rejects_bad_arguments(lib):
    assert _attn(lib, None) == ERR_NULL
    assert _attn(lib, _adims(flags=2)) == ERR_FLAGS
    assert _attn(lib, _adims(n_ctx=0)) == ERR_DIMS
    assert _attn(lib, _adims(n_kv_heads=5)) == ERR_DIMS
    assert _attn(lib, _adims(head_dim=256)) == ERR_GROUP
    assert _attn(lib, _adims(block=128)) == ERR_GROUP
    assert _attn(lib, _adims(), q=None) == ERR_NULL
    assert _attn(lib, _adims(), table=None) == ERR_NULL
    assert _attn(lib, _adims(), ws=None) == ERR_NULL
    assert _attn(lib, _adims(), q=FAKE + 8) == ERR_ALIGN
    assert _attn(lib, _adims(), k=FAKE + 2) == ERR_ALIGN
    assert _attn(lib, _adims(), table=FAKE + 2) == ERR_ALIGN
    assert _attn(lib, _adims(), ws=FAKE + 16) == ERR_ALIGN
    d = _adims()
    assert _attn(lib, d, ws_bytes=B.moe_w4_attn_workspace_bytes(d) - 1) == ERR_WS


# --- Gated DeltaNet scan (include/moe_w4_gdn.h) -----------------------------------

def _gdims(**kw):
    d = dict(T=100, n_v_heads=32, n_k_heads=16, dim=128, flags=0)
    d.update(kw)
    return B.moe_w4_gdn_dims(d["T"], d["n_v_heads"], d["n_k_heads"], d["dim"], d["flags"])


def _gdn(lib, dims, q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, state=FAKE, out=FAKE + 4096):
    return lib.moe_w4_gdn_scan(ctypes.byref(dims) if dims is not None else None, q, k, v, g, beta, state,
                               out, None)


def test_gdn_rejects_bad_arguments(lib):
    assert _gdn(lib, None) == ERR_NULL
    assert _gdn(lib, _gdims(flags=1)) == ERR_FLAGS
    assert _gdn(lib, _gdims(T=-1)) == ERR_DIMS
    assert _gdn(lib, _gdims(T=B.MOE_W4_GDN_MAX_T + 1)) == ERR_DIMS
    assert _gdn(lib, _gdims(n_k_heads=5)) == ERR_DIMS
    assert _gdn(lib, _gdims(n_v_heads=0)) == ERR_DIMS
    assert _gdn(lib, _gdims(dim=64)) == ERR_GROUP
    assert _gdn(lib, _gdims(T=0)) == OK                 # nothing to do
    assert _gdn(lib, _gdims(), q=None) == ERR_NULL
    assert _gdn(lib, _gdims(), state=None) == ERR_NULL
    assert _gdn(lib, _gdims(), q=FAKE + 8) == ERR_ALIGN
    assert _gdn(lib, _gdims(), g=FAKE + 2) == ERR_ALIGN
    assert _gdn(lib, _gdims(), state=FAKE + 4) == ERR_ALIGN
    assert _gdn(lib, _gdims(), out=FAKE + 2) == ERR_ALIGN


def _gdn_chunked(lib, dims, ws=FAKE + 8192, ws_bytes=1 << 40, q=FAKE, state=FAKE, out=FAKE + 4096):
    return lib.moe_w4_gdn_scan_chunked(ctypes.byref(dims) if dims is not None else None, q, FAKE, FAKE, FAKE,
                                       FAKE, state, out, ws, ws_bytes, None)


def test_gdn_chunked_workspace_bytes(lib):
    """One 2048-token segment at most: per 64-token chunk 82,432 bytes per value head
    (-W, Pm and Vt operand fragments, the decays) and 32,768 per key head (K^T and Q
    fragments); zero for invalid dims."""
    def wsb(**kw):
        return lib.moe_w4_gdn_chunked_workspace_bytes(ctypes.byref(_gdims(**kw)))
    per_chunk = 32 * 82432 + 16 * 32768
    assert wsb(T=1) == per_chunk
    assert wsb(T=64) == per_chunk
    assert wsb(T=65) == 2 * per_chunk
    assert wsb(T=2048) == 32 * per_chunk
    assert wsb(T=B.MOE_W4_GDN_MAX_T) == 32 * per_chunk
    assert wsb(T=100, n_v_heads=8, n_k_heads=2) == 2 * (8 * 82432 + 2 * 32768)
    assert wsb(T=0) == 0
    assert wsb(n_k_heads=5) == 0
    assert wsb(dim=64) == 0
    assert lib.moe_w4_gdn_chunked_workspace_bytes(None) == 0


def test_gdn_chunked_rejects_bad_arguments(lib):
    need = lib.moe_w4_gdn_chunked_workspace_bytes(ctypes.byref(_gdims()))
    assert _gdn_chunked(lib, None) == ERR_NULL
    assert _gdn_chunked(lib, _gdims(flags=1)) == ERR_FLAGS
    assert _gdn_chunked(lib, _gdims(T=B.MOE_W4_GDN_MAX_T + 1)) == ERR_DIMS
    assert _gdn_chunked(lib, _gdims(n_k_heads=3)) == ERR_DIMS
    assert _gdn_chunked(lib, _gdims(dim=64)) == ERR_GROUP
    assert _gdn_chunked(lib, _gdims(T=0), ws=None, ws_bytes=0) == OK      # nothing to do
    assert _gdn_chunked(lib, _gdims(), ws=None) == ERR_NULL
    assert _gdn_chunked(lib, _gdims(), q=None) == ERR_NULL
    assert _gdn_chunked(lib, _gdims(), ws=FAKE + 8) == ERR_ALIGN
    assert _gdn_chunked(lib, _gdims(), state=FAKE + 4) == ERR_ALIGN
    assert _gdn_chunked(lib, _gdims(), ws_bytes=need - 1) == ERR_WS
    assert _gdn_chunked(lib, _gdims(), ws_bytes=0) == ERR_WS


def test_size_limits_match_the_headers():
    for header, name, value in (("moe_w4_attn.h", "MOE_W4_ATTN_MAX_CTX", B.MOE_W4_ATTN_MAX_CTX),
                                ("moe_w4_gdn.h", "MOE_W4_GDN_MAX_T", B.MOE_W4_GDN_MAX_T)):
        text = open(os.path.join(ROOT, "include", header)).read()
        m = re.search(r"#define\s+%s\s+\(1 << (\d+)\)" % name, text)
        assert m and (1 << int(m.group(1))) == value, name
