"""MI355X-native online FP4 path: block-Hadamard rotate + MXFP4/NVFP4 quantize + W4A4 GEMM.

The compute path is the HIP library libfp4.so (C ABI in include/fp4.h); the
Python names mirror the C calls and only marshal arguments:

    from microscaling_fp4_quantized_amd import fp4_rotate_quantize, fp4_quantize_weights, fp4_linear

Importing the package does not load the library; the first call does, and
raises if it is not built.
"""


def __getattr__(name):
    if name in ("fp4_rotate_quantize", "fp4_quantize_weights", "fp4_linear", "fp4_rotate_quantize_linear",
                "fp4_abi_version", "Fp4Error", "load_library", "library_path", "group_size", "FP4_MXFP4",
                "FP4_NVFP4"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
