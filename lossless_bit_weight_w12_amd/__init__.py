"""W12 on MI355X: lossless 12-bit BF16 weights decoded inside the GEMM, plus greedy
verification with a certified exact-argmax LM head.  The compute lives in libw12.so
(HIP kernels for gfx950 behind a C ABI, declared in include/w12.h); this package is its
thin Python binding."""
from .w12 import (Prepared, prepare_gemm, prepare_rms, prepare_verify, W12Desc, W12Error, W12Tensor, decode, encode, gemm, gemm_bf16, lib, lib_path,
                  lmhead_verify, rms_rescale, status_str, tiles_bytes, verify_candidates, verify_pass1,
                  workspace, workspace_bytes, EXPORTS, MAX_M, OP_DECODE, OP_ENCODE, OP_GEMM,
                  OP_GEMM_BF16, OP_VERIFY)

__all__ = ["Prepared", "prepare_gemm", "prepare_rms", "prepare_verify", "W12Desc", "W12Error", "W12Tensor", "decode", "encode", "gemm", "gemm_bf16", "lib",
           "lib_path", "lmhead_verify", "rms_rescale", "status_str", "tiles_bytes",
           "verify_candidates", "verify_pass1", "workspace", "workspace_bytes", "EXPORTS", "MAX_M", "OP_DECODE",
           "OP_ENCODE", "OP_GEMM", "OP_GEMM_BF16", "OP_VERIFY"]
