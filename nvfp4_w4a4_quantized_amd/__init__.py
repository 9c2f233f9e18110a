"""MI355X-native NVFP4 W4A4 MoE expert path (per-token NVFP4 quantize + MoE
permute -> W4A4 grouped GEMM FC1 -> SwiGLU/requantize -> FC2 -> combine)."""
