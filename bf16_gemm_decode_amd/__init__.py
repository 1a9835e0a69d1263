"""MI355X (gfx950) column-major GEMM and decode GEMV behind a C ABI.

The computation runs in hand-written HIP kernels in ``libmigemm.so``
(``csrc/``); this package only binds them (``binding``) and holds the FLOP /
byte / roofline arithmetic used for reports (``roofline``).
"""
from .binding import (MigemmError, gemm, gemv, hbm_read, hbm_read_sink_words, lib,  # noqa: F401
                      gemm_f16_ptr, gemm_bf16_ptr, gemm_ex_ptr, gemv_bf16_ptr,
                      gemv_bf16_ex_ptr, tile_coord, gemm_plan, F16, BF16)
from . import roofline  # noqa: F401

__all__ = ["gemm", "gemv", "hbm_read", "lib", "tile_coord", "gemm_plan", "roofline",
           "MigemmError"]
