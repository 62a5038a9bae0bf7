"""BaKron two-sided-Hessian adaptive rounding on MI355X (gfx950).

The compute path is libbakron.so (HIP kernels behind the C ABI in
include/bakron.h); this package is its thin Python binding.
"""
from ._binding import (BakronError, GridError, LIB_PATH, check_grid, factor, factor_workspace_bytes, gptq,
                       gptq_workspace_bytes, kfac_factors, lib, moment, quantize, quantize_workspace_bytes,
                       row_sqnorms, shampoo_factors, solve, solve_antidiagonal, solve_batch, solve_noalloc,
                       solve_workspace_bytes, strerror, version)

__all__ = ["BakronError", "GridError", "LIB_PATH", "check_grid", "factor", "factor_workspace_bytes", "gptq",
           "gptq_workspace_bytes", "kfac_factors", "lib", "moment", "quantize", "quantize_workspace_bytes",
           "row_sqnorms", "shampoo_factors", "solve", "solve_antidiagonal", "solve_batch", "solve_noalloc",
           "solve_workspace_bytes", "strerror",
           "version"]
