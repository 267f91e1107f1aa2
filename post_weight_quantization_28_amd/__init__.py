"""MI355X (gfx950) GPTQ layer quantizer: Hessian accumulation, damped
Cholesky factor of the inverse, blocked column sweep with error feedback and
lazy-batch trailing updates, and code packing, in hand-written HIP kernels
behind a C ABI (include/gptq.h); and, for inference, the dequantising product
of a packed layer. This package is its Python binding."""
from .gptq import (BF16, F32, GPTQError, NOALLOC_SCRATCH_BYTES, QuantResult, accumulate_hessian, dequant_matmul,
                   dequant_matmul_noalloc, eora, eora_workspace_bytes, refine_lowrank,
                   refine_workspace_bytes, quantize_rtn,
                   dequant_matmul_workspace_bytes, factor_hinv, hessian_workspace_bytes, load, make_params, pack_codes, profile_collect,
                   profile_enable, quantize_layer, repack_act_order, unpack_codes, workspace_bytes, LIB_PATH,
                   PROF_CLASSES)

__all__ = ["BF16", "F32", "GPTQError", "NOALLOC_SCRATCH_BYTES", "QuantResult", "accumulate_hessian",
           "dequant_matmul", "dequant_matmul_noalloc", "eora", "eora_workspace_bytes", "refine_lowrank",
           "refine_workspace_bytes", "quantize_rtn",
           "dequant_matmul_workspace_bytes", "factor_hinv",
           "hessian_workspace_bytes", "load", "make_params", "pack_codes", "profile_collect",
           "profile_enable", "quantize_layer", "repack_act_order", "unpack_codes", "workspace_bytes", "LIB_PATH",
           "PROF_CLASSES"]
