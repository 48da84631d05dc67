"""FP8_DYNAMIC W8A8 Linear for AMD Instinct MI355X (gfx950).

Per-token dynamic E4M3 activations x channel-wise static E4M3 weights, float32
accumulation, token-scale x channel-scale epilogue to bfloat16, as in the
FP8-Dynamic recipe of the MOSS-VL quantization README, and the BF16 RMSNorm
ahead of the q/k/v and gate/up Linears and the MLP activation ahead of
down_proj, each fused with the per-token quantization of its output, and the
key/value-cache codecs (FP8 E4M3; INT8 group-wise with a BF16 residual
window), and a grouped few-token call on weights in MFMA-tile order.  The
work happens in hand-written HIP kernels behind the C ABI
of ``include/fp8w8a8.h``; this package is its Python binding (argument
marshalling only).
"""

from .binding import (LIBRARY_PATH, SIGNATURES, Fp8W8A8Error, fp8_linear, fp8_linear_requant,
                      fp8_linear_group, fp8_linear_group_requant, init_workspace,
                      kv_dequantize_fp8, kv_quantize_fp8, kv_quantize_int8, kv_read_int8,
                      load_library,
                      quant_linear, quant_linear_group_m1, quant_linear_noalloc,
                      quantize_act_group, quantize_act_per_token,
                      rmsnorm_quant_linear,
                      swiglu_quant_linear, tile_weights,
                      quantize_weight_channelwise, rmsnorm_quantize, swiglu_quantize,
                      workspace_bytes)

__all__ = ["LIBRARY_PATH", "SIGNATURES", "Fp8W8A8Error", "fp8_linear",
           "fp8_linear_group", "fp8_linear_group_requant", "tile_weights",
           "fp8_linear_requant",
           "init_workspace", "kv_dequantize_fp8", "kv_quantize_fp8",
           "kv_quantize_int8", "kv_read_int8",
           "load_library", "quant_linear", "quant_linear_group_m1",
           "quant_linear_noalloc",
           "quantize_act_group", "quantize_act_per_token", "quantize_weight_channelwise",
           "rmsnorm_quantize", "rmsnorm_quant_linear", "swiglu_quantize",
           "swiglu_quant_linear", "workspace_bytes"]
