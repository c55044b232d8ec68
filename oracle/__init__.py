"""CPU oracle for the W4 mixture-of-experts block -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import anything from here.  The product path (the HIP library
and its Python binding) never imports, links or calls this package.
"""
from .moe_w4_oracle import *  # noqa: F401,F403
from .moe_w4_oracle import Routing, route, forward_grouped, forward_dense, dequant  # noqa: F401
