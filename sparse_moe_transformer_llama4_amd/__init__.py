"""Llama 4 mixture-of-experts feed-forward block on AMD MI355X (gfx950).

The block runs in hand-written HIP kernels behind the C ABI of libmoe355
(include/moe.h); `moe` is a thin ctypes binding with the same entry points.
PyTorch is used only for device memory and streams.
"""
from .moe import (  # noqa: F401
    MOE_F32, MOE_BF16, MOE_E4M3, MoeError, Plan, load_library, moe_forward, moe_plan,
    moe_route, moe_status_string, moe_version, moe_workspace_size, symbols,
)
