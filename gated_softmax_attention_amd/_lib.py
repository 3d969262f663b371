"""ctypes view of libgsa.so: loads the library and declares the C ABI of include/gsa.h."""
import ctypes
import os

# GSA_LIBRARY_PATH selects another build of the same library (e.g. a tuning variant)
LIB_PATH = os.environ.get("GSA_LIBRARY_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgsa.so")

GSA_OK = 0
GSA_ERR_INVALID_ARG = 1
GSA_ERR_UNSUPPORTED = 2
GSA_ERR_MISALIGNED = 3
GSA_ERR_WORKSPACE = 4
GSA_ERR_NO_DEVICE = 5
GSA_ERR_HIP = 6

GSA_FP32 = 0
GSA_BF16 = 1

GSA_GATE_NONE = 0
GSA_GATE_ELEMENTWISE = 1
GSA_GATE_HEADWISE = 2
GSA_GATE_SHARED = 3

GSA_ACT_IDENTITY = 0
GSA_ACT_SIGMOID = 1
GSA_ACT_NS_SIGMOID = 2
GSA_ACT_SILU = 3

GSA_COMBINE_MUL = 0
GSA_COMBINE_ADD = 1
GSA_NORM_NONE = 0
GSA_NORM_RMS = 1

# name -> (restype, argtypes); the exported surface of include/gsa.h
_P, _I64, _I, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
SIGNATURES = {
    "gsa_version": (_I, []),
    "gsa_status_string": (ctypes.c_char_p, [_I]),
    "gsa_last_error_message": (ctypes.c_char_p, []),
    "gsa_gate_logits": (_I, [_P, _P, _P, _I64, _I64, _I64, _I, _I, _P]),
    "gsa_gate_logits_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I]),
    "gsa_gate_logits_ws": (_I, [_P, _P, _P, _I64, _I64, _I64, _I, _I, _P, _SZ, _P]),
    "gsa_forward": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _I, _P]),
    "gsa_forward_lse": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _I, _P]),
    "gsa_decode_num_splits": (_I64, [_I64, _I64, _I64, _I64, _I64, _I]),
    "gsa_decode_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I64, _I]),
    "gsa_decode": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _I, _I, _P, _SZ, _P]),
    "gsa_noalloc_scratch_bytes": (_SZ, []),
    "gsa_decode_noalloc": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _I, _I, _P]),
    "gsa_gated_decode_workspace_bytes": (_SZ, [_I64] * 6 + [_I, _I, _I]),
    "gsa_gated_decode": (_I, [_P] * 6 + [_I64] * 6 + [_I, _I, _I, _P, _SZ, _P]),
    "gsa_backward_workspace_bytes": (_SZ, [_I64, _I64, _I64, _I64, _I64, _I64, _I]),
    "gsa_backward": (_I, [_P] * 14 + [_I64] * 6 + [_I, _I, _P, _SZ, _P]),
    "gsa_forward_variant": (_I, [_P] * 6 + [_I64] * 5 + [_I, _I, _I, _I, _P]),
    "gsa_decode_variant": (_I, [_P] * 5 + [_I64] * 5 + [_I, _I, _I, _I, _I, _P, _SZ, _P]),
    "gsa_gate_head_mean": (_I, [_P, _P, _I64, _I64, _I64, _P]),
    "gsa_forward_value_gated": (_I, [_P] * 6 + [_I64] * 5 + [_I, _I, _P]),
    "gsa_value_gate": (_I, [_P, _P, _P, _I64, _I64, _I64, _I64, _I, _I, _P]),
    "gsa_project_qkvg": (_I, [_P] * 6 + [_I64] * 6 + [_I, _P]),
    "gsa_first_token_attention": (_I, [_P, _P, _P, _P, _P, _I64, _I64, _I64, _I64, _I64, _I, _P]),
}

_lib = None


class GsaError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__(f"{status_name(status)}: {message}")


def load(path: str = LIB_PATH):
    """Load libgsa.so once; raise if it has not been built (there is no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libgsa.so not found at {path}; build it with "
                           "`python -m gated_softmax_attention_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_name(status: int) -> str:
    return load().gsa_status_string(status).decode()


def check(status: int):
    if status != GSA_OK:
        raise GsaError(status, load().gsa_last_error_message().decode())
