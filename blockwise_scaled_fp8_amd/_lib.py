"""ctypes loader for libfp8bw.so and the prototypes of its C ABI
(include/fp8bw.h).  No fallback exists: if the library is not built, every
entry point raises."""

import ctypes
import os

LIB_NAME = "libfp8bw.so"
_LIB = None

c_i64 = ctypes.c_int64
c_int = ctypes.c_int
c_size = ctypes.c_size_t
c_ptr = ctypes.c_void_p

ABI_VERSION = 2   # fp8bw_abi_version() of the sources these prototypes mirror

# name -> (restype, argtypes), mirroring include/fp8bw.h
PROTOTYPES = {
    "fp8bw_abi_version": (c_int, []),
    "fp8bw_status_str": (ctypes.c_char_p, [c_int]),
    "fp8bw_last_error": (ctypes.c_char_p, []),
    "fp8_blockwise_quant": (c_int, [c_ptr, c_i64, c_i64, c_i64, c_int, c_int, c_ptr, c_i64,
                                    c_ptr, c_i64, c_i64, c_ptr]),
    "fp8_blockwise_quant_dual": (c_int, [c_ptr, c_i64, c_i64, c_i64, c_int, c_ptr, c_i64, c_ptr,
                                         c_i64, c_i64, c_ptr, c_i64, c_ptr, c_i64, c_i64, c_int,
                                         c_ptr]),
    "fp8bw_tensorwise_quant_ws_bytes": (c_size, [c_i64, c_i64]),
    "fp8_tensorwise_quant": (c_int, [c_ptr, c_i64, c_i64, c_i64, c_ptr, c_i64, c_ptr, c_ptr,
                                     c_size, c_ptr]),
    "fp8_tensorwise_quant_noalloc": (c_int, [c_ptr, c_i64, c_i64, c_i64, c_ptr, c_i64, c_ptr,
                                             c_ptr]),
    "fp8bw_gemm_blockwise_ws_bytes": (c_size, [c_i64, c_i64, c_i64]),
    "fp8_scaled_gemm_blockwise": (c_int, [c_ptr, c_i64, c_ptr, c_i64, c_i64, c_ptr, c_i64, c_ptr,
                                          c_i64, c_i64, c_int, c_i64, c_i64, c_i64, c_ptr, c_i64,
                                          c_int, c_ptr, c_size, c_ptr]),
    "fp8_scaled_gemm_blockwise_kn": (c_int, [c_ptr, c_i64, c_ptr, c_i64, c_i64, c_ptr, c_i64,
                                             c_ptr, c_i64, c_i64, c_int, c_i64, c_i64, c_i64,
                                             c_ptr, c_i64, c_int, c_ptr, c_size, c_ptr]),
    "fp8bw_gemm_num_configs": (c_int, []),
    "fp8bw_gemm_blockwise_plan": (c_int, [c_i64, c_i64, c_i64, c_int, c_ptr]),
    "fp8bw_gemm_ws_bytes_for_split": (c_size, [c_i64, c_i64, c_int]),
    "fp8_scaled_gemm_blockwise_cfg": (c_int, [c_ptr, c_i64, c_ptr, c_i64, c_i64, c_ptr, c_i64,
                                              c_ptr, c_i64, c_i64, c_int, c_i64, c_i64, c_i64,
                                              c_ptr, c_i64, c_int, c_int, c_int, c_ptr, c_size,
                                              c_ptr]),
    "fp8_scaled_gemm_tensorwise": (c_int, [c_ptr, c_i64, c_ptr, c_ptr, c_i64, c_ptr, c_i64, c_i64,
                                           c_i64, c_ptr, c_i64, c_int, c_ptr]),
    "fp8_scaled_gemm_blockwise_bias": (c_int, [c_ptr, c_i64, c_ptr, c_i64, c_i64, c_ptr, c_i64,
                                               c_ptr, c_i64, c_i64, c_int, c_i64, c_i64, c_i64,
                                               c_ptr, c_ptr, c_i64, c_int, c_ptr, c_size, c_ptr]),
    "fp8_scaled_gemm_tensorwise_bias": (c_int, [c_ptr, c_i64, c_ptr, c_ptr, c_i64, c_ptr, c_i64,
                                                c_i64, c_i64, c_ptr, c_ptr, c_i64, c_int, c_ptr]),
    "fp8_scaled_grouped_gemm_blockwise": (c_int, [c_ptr, c_i64, c_ptr, c_i64, c_ptr, c_i64, c_i64,
                                                  c_ptr, c_i64, c_i64, c_i64, c_int, c_ptr, c_i64,
                                                  c_i64, c_i64, c_ptr, c_i64, c_int, c_ptr]),
    "fp8bw_linear_ws_bytes": (c_size, [c_i64, c_i64, c_i64, c_int]),
    "fp8_linear_fwd": (c_int, [c_ptr, c_ptr, c_ptr, c_i64, c_i64, c_i64, c_ptr, c_size, c_ptr]),
    "fp8_linear_dgrad": (c_int, [c_ptr, c_ptr, c_ptr, c_i64, c_i64, c_i64, c_ptr, c_size, c_ptr]),
    "fp8_linear_wgrad": (c_int, [c_ptr, c_ptr, c_ptr, c_i64, c_i64, c_i64, c_ptr, c_size, c_ptr]),
    "fp8bw_linear_saved_bytes": (c_size, [c_i64, c_i64, c_i64]),
    "fp8_linear_fwd_save": (c_int, [c_ptr, c_ptr, c_ptr, c_i64, c_i64, c_i64, c_ptr, c_size, c_ptr,
                                    c_size, c_ptr]),
    "fp8_linear_bwd": (c_int, [c_ptr, c_ptr, c_ptr, c_size, c_ptr, c_ptr, c_i64, c_i64, c_i64,
                               c_ptr, c_size, c_ptr]),
}

STATUS = {0: "FP8BW_OK", 1: "FP8BW_ERR_NULL", 2: "FP8BW_ERR_SHAPE", 3: "FP8BW_ERR_LAYOUT",
          4: "FP8BW_ERR_ALIGN", 5: "FP8BW_ERR_UNSUPPORTED", 6: "FP8BW_ERR_WORKSPACE",
          7: "FP8BW_ERR_HIP"}


class FP8BWError(RuntimeError):
    """A non-OK status from the C ABI (message from fp8bw_last_error)."""

    def __init__(self, status, message):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {message}")


def lib_path():
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)


def load_library():
    """Load libfp8bw.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(
                f"{path} is not built: run `python -m blockwise_scaled_fp8_amd.build` "
                "(hipcc --offload-arch=gfx950).  There is no fallback implementation.")
        lib = ctypes.CDLL(path)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        # The prototypes above describe one version of the ABI; a library
        # built from other sources would be called with the wrong arguments.
        if lib.fp8bw_abi_version() != ABI_VERSION:
            raise RuntimeError(f"{path} has ABI version {lib.fp8bw_abi_version()}, this binding "
                               f"expects {ABI_VERSION}: rebuild it")
        _LIB = lib
    return _LIB


def check(status):
    if status != 0:
        msg = load_library().fp8bw_last_error().decode()
        raise FP8BWError(status, msg)
