"""ctypes binding of libminikv.so: argument marshalling only.

Every computation runs in the library's HIP kernels.  If the shared library is
missing this module raises; there is no fallback path.
"""

import ctypes
import os

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libminikv.so")

OK = 0
ERR_NULL = -1
ERR_SHAPE = -2
ERR_UNSUPPORTED = -3
ERR_ALIGN = -4
ERR_WORKSPACE = -5
ERR_LAUNCH = -6
F32 = 0
BF16 = 1
GROUP = 32
DECODE_SCRATCH_BYTES = 32 << 20  # MINIKV_DECODE_SCRATCH_BYTES
DECODE_TICKET_BYTES = 16384      # MINIKV_DECODE_TICKET_BYTES

# Every function the header declares, with its ctypes signature.
_vp, _i, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
_ip = ctypes.POINTER(ctypes.c_int)


class PackedT(ctypes.Structure):
    """Mirror of minikv_packed_t."""

    _fields_ = [
        ("k_codes", _vp),
        ("k_sz", _vp),
        ("v_codes", _vp),
        ("v_sz", _vp),
        ("B", ctypes.c_int32),
        ("Hkv", ctypes.c_int32),
        ("n_keep", ctypes.c_int32),
        ("D", ctypes.c_int32),
        ("group", ctypes.c_int32),
    ]


SIGNATURES = {
    "minikv_prefill_attn": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp]),
    "minikv_window_scores": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _vp]),
    "minikv_prefill_attn_scores": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _f, _vp, _vp, _vp, _vp]),
    "minikv_prefill_fuses_scores": (_i, [_i, _i, _i, _i, _i]),
    "minikv_select_topk": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _vp, _sz, _vp]),
    "minikv_select_ws_bytes": (_sz, [_i, _i, _i]),
    "minikv_quant_pack": (_i, [_vp, _vp, _i, _vp, _i, _i, _i, _i, _i, ctypes.POINTER(PackedT), _vp]),
    "minikv_decode_attn": (_i, [_vp, ctypes.POINTER(PackedT), _i, _f, _vp, _vp, _sz, _vp]),
    "minikv_decode_attn_noalloc": (_i, [_vp, ctypes.POINTER(PackedT), _i, _f, _vp, _vp]),
    "minikv_stream_pack": (_i, [_vp, _vp, _i, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp]),
    "minikv_stream_append": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp]),
    "minikv_stream_decode": (_i, [_vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _i, _f, _vp, _vp,
                                  _sz, _vp]),
    "minikv_stream_decode_ws_bytes": (_sz, [_i, _i, _i, _i, _i, _i]),
    "minikv_stream_init": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _ip, _ip, _vp]),
    "minikv_stream_append_token": (_i, [_vp, _vp, _i, _i, _i, _i, _ip, _ip, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "minikv_stream_set_counts": (_i, [_vp, _i, _i, _i, _vp]),
    "minikv_stream_step_append": (_i, [_vp, _vp, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "minikv_stream_step_decode_ws_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "minikv_stream_step_decode": (_i, [_vp, _i, _i, _i, _i, _i, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _f, _vp, _vp, _sz,
                                       _vp]),
    "minikv_packed_bytes": (_sz, [_i, _i, _i, _i]),
    "minikv_decode_ws_bytes": (_sz, [_i, _i, _i, _i, _i]),
    "minikv_keep_count": (_i, [_i, _i]),
    "minikv_pyramid_keep": (_i, [_i, _i, _i, _i, _i]),
    "minikv_split_heavy_recent": (_i, [_i, ctypes.POINTER(ctypes.c_int), ctypes.POINTER(ctypes.c_int)]),
    "minikv_status_string": (ctypes.c_char_p, [_i]),
    "minikv_build_id": (ctypes.c_char_p, []),
    "minikv_read_probe": (_i, [_vp, _sz, _vp, _vp]),
}

_lib = None


class MinikvError(RuntimeError):
    def __init__(self, fn, status):
        super().__init__(f"{fn} failed: status {status} ({status_string(status)})")
        self.status = status


def lib():
    """Load the in-tree libminikv.so once.

    Raises if it has not been built, or if its build id (a hash of the sources
    it was compiled from) is not that of the sources beside it: a stale binary
    is never used.
    """
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} not found: build it with `python -m bit_quantized_kv_quant_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        built, want = handle.minikv_build_id().decode(), _build.source_hash()
        if built != want:
            raise RuntimeError(f"{LIB_PATH} was built from other sources ({built}, sources are {want}): "
                               "rebuild it with `python -m bit_quantized_kv_quant_amd.build`")
        _lib = handle
    return _lib


def build_id():
    """Source hash the loaded library was built from."""
    return lib().minikv_build_id().decode()


def lib_path():
    return LIB_PATH


def status_string(status):
    return lib().minikv_status_string(int(status)).decode()


def check(fn, status):
    if status != OK:
        raise MinikvError(fn, status)
