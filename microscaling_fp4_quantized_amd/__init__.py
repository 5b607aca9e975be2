"""MI355X-native online FP4 path: block-Hadamard rotate + MXFP4/NVFP4 quantize + W4A4 GEMM."""
