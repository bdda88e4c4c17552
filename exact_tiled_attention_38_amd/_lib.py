"""ctypes loader for libfa.so. Argument marshalling only.

The library is loaded on first use; if it has not been built, every call
raises instead of falling back to anything else.
"""

import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfa.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "fa.h")

_lib = None

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float

SIGNATURES = {
    "fa_forward": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p]),
    "fa_forward_gqa": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _p]),
    "fa_forward_f32": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _f, _p]),
    "fa_forward_block_sparse": (_i, [_p] * 7 + [_i] * 7 + [_f, _p]),
    "fa_forward_fp8": (_i, [_p] * 5 + [_f] * 3 + [_i] * 6 + [_f, _p]),
    "fa_backward_workspace_bytes": (ctypes.c_size_t, [_i, _i, _i, _i]),
    "fa_backward": (_i, [_p] * 10 + [_i, _i, _i, _i, _i, _f, _p]),
    "fa_backward_gqa": (_i, [_p] * 10 + [_i, _i, _i, _i, _i, _i, _f, _p]),
    "fa_decode_workspace_bytes": (ctypes.c_size_t, [_i] * 6),
    "fa_decode": (_i, [_p] * 6 + [_i] * 7 + [_f, _p]),
    "fa_decode_noalloc": (_i, [_p] * 5 + [_i] * 7 + [_f, _p]),
    "fa_merge": (_i, [_p] * 4 + [_i, ctypes.c_longlong, _i, _p]),
    "fa_status_string": (ctypes.c_char_p, [_i]),
}


def status_codes():
    """Parse the FA_* status enum from include/fa.h."""
    text = open(HEADER_PATH).read()
    return {m.group(1): int(m.group(2)) for m in re.finditer(r"\b(FA_[A-Z_]+)\s*=\s*(\d+)", text)}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'` "
                "or `python -m exact_tiled_attention_38_amd.csrc.build`"
            )
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def status_string(code):
    return lib().fa_status_string(int(code)).decode()


def check(code, what):
    if code != 0:
        raise RuntimeError(f"{what}: {status_string(code)} (status {code})")
