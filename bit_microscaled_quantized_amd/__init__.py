"""NVFP4 quantize-and-contract on MI355X (gfx950).

The work runs in the HIP library libnvfp4.so (C ABI declared in include/nvfp4.h);
bit_microscaled_quantized_amd.nvfp4 marshals torch tensors into its calls.
Importing this package does not load the library; the first call does, and it
raises if the library has not been built.
"""
from .nvfp4 import (  # noqa: F401
    NVFP4_BF16, NVFP4_F32, NVFP4_RNE, NVFP4_SR, NVFP4_ROW_1D, NVFP4_COL_1D, NVFP4_TILE_2D,
    Nvfp4Error, library_path, load_library, nvfp4_dequantize, nvfp4_gemm, nvfp4_gemm_bf16,
    nvfp4_gemm_noalloc, nvfp4_gemm_workspace_size, nvfp4_set_quantize_passes,
    nvfp4_set_sync_spin_limit, nvfp4_single_pass_stats,
    nvfp4_quantize, nvfp4_quantize_row_rht, nvfp4_rht_quantize, nvfp4_status_str,
    mxfp4_gemm, mxfp4_quantize,
)
