"""W12 on MI355X: lossless 12-bit BF16 weights decoded inside the GEMM, plus greedy
verification with a certified exact-argmax LM head, in one pass over the W12 head or in
two levels (an 8-bit screen copy first), and the GEMMs of FP8 targets (E4M3 weights with
128 x 128 block scales) in the same kernel family.  The compute lives in libw12.so (HIP
kernels for gfx950 behind a C ABI, declared in include/w12.h); this package is its thin
Python binding."""
from .w12 import (ENCODE_TOTAL_OFFSET, EXPORTS, F8Tensor, MAX_GROUP, MAX_M,
                  NOALLOC_SCRATCH_BYTES, OP_DECODE, OP_ENCODE, OP_GEMM, OP_GEMM_BF16,
                  OP_GEMM_F8, OP_GEMM_GROUP, OP_VERIFY, OP_VERIFY2, Prepared, ScreenCopy,
                  W12Desc, W12Error, W12Tensor, bf16_tile, decode, encode, f8_encode,
                  f8_tile, gemm, gemm_bf16, gemm_bf16_tiled, gemm_f8, gemm_f8_group,
                  gemm_group, gemm_noalloc, lib, lib_path, lmhead_verify, lmhead_verify2,
                  lmhead_verify2_batched, lmhead_verify_batched, logits_f32, prepare_gemm,
                  prepare_gemm_f8, prepare_gemm_f8_group, prepare_gemm_group, prepare_rms,
                  prepare_verify, prepare_verify2, prepare_verify2_batched,
                  prepare_verify_batched, rms_rescale, screen_encode, screen_logits_f32,
                  status_str, stream_read, tiles_bytes, verify2_candidates,
                  verify_candidates, workspace, workspace_bytes)

__all__ = ["ENCODE_TOTAL_OFFSET", "EXPORTS", "F8Tensor", "MAX_GROUP", "MAX_M",
           "NOALLOC_SCRATCH_BYTES", "OP_DECODE", "OP_ENCODE", "OP_GEMM", "OP_GEMM_BF16",
           "OP_GEMM_F8", "OP_GEMM_GROUP", "OP_VERIFY", "OP_VERIFY2", "Prepared",
           "ScreenCopy", "W12Desc", "W12Error", "W12Tensor", "bf16_tile", "decode",
           "encode", "f8_encode", "f8_tile", "gemm", "gemm_bf16", "gemm_bf16_tiled",
           "gemm_f8", "gemm_f8_group", "gemm_group", "gemm_noalloc", "lib", "lib_path",
           "lmhead_verify", "lmhead_verify2", "lmhead_verify2_batched",
           "lmhead_verify_batched", "logits_f32", "prepare_gemm", "prepare_gemm_f8",
           "prepare_gemm_f8_group", "prepare_gemm_group", "prepare_rms", "prepare_verify",
           "prepare_verify2", "prepare_verify2_batched", "prepare_verify_batched",
           "rms_rescale", "screen_encode", "screen_logits_f32", "status_str", "stream_read",
           "tiles_bytes", "verify2_candidates", "verify_candidates", "workspace",
           "workspace_bytes"]
