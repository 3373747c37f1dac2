"""ctypes view of libflce.so (the C-ABI declared in include/flce.h)."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libflce.so")

F32, BF16 = 0, 1
SUM, MEAN = 0, 1
OK, ERR_ARG, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP, ERR_LABEL, ERR_SCRATCH = range(7)
# bytes of the fixed scratch array behind flce_forward_noalloc (FLCE_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 96 << 20

# Every symbol the header declares, with its ctypes signature.
_c = ctypes
_vp, _i64, _i32, _f32, _sz = _c.c_void_p, _c.c_int64, _c.c_int, _c.c_float, _c.c_size_t
_FB_ARGS = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _i32, _i64, _vp, _vp, _vp, _vp,
            _vp, _i32, _f32, _i32, _vp, _sz, _vp, _vp]
_F_ARGS = [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _i32, _i64, _vp, _vp, _vp, _i32,
           _f32, _vp, _sz, _vp, _vp]
SIGNATURES = {
    "flce_workspace_size": (_sz, [_i64, _i64, _i64, _i32]),
    "flce_check_args": (_i32, _FB_ARGS),
    "flce_forward_backward": (_i32, _FB_ARGS),
    "flce_workspace_size_ex": (_sz, [_i64, _i64, _i64, _i32, _i32]),
    "flce_vocab_chunk_ex": (_i64, [_i64, _i64, _i64, _i32, _i32]),
    "flce_check_args_ex": (_i32, _FB_ARGS + [_i32]),
    "flce_forward_backward_ex": (_i32, _FB_ARGS + [_i32]),
    "flce_workspace_size_nr": (_sz, [_i64, _i64, _i64, _i32, _i64]),
    "flce_token_chunk_nr": (_i64, [_i64, _i64, _i64, _i32, _i64]),
    "flce_check_args_nr": (_i32, _FB_ARGS + [_i64]),
    "flce_forward_backward_nr": (_i32, _FB_ARGS + [_i64]),
    "flce_forward_workspace_size": (_sz, [_i64, _i64, _i64, _i32]),
    "flce_forward_check_args": (_i32, _F_ARGS),
    "flce_forward": (_i32, _F_ARGS),
    "flce_forward_noalloc": (_i32, [_vp, _vp, _vp, _i64, _i64, _i64, _i64, _f32, _i32, _i64,
                                    _vp, _vp, _vp, _i32, _f32, _vp, _vp]),
    "flce_forward_logits_check_args": (_i32, _F_ARGS + [_vp, _i64, _i32]),
    "flce_forward_logits": (_i32, _F_ARGS + [_vp, _i64, _i32]),
    "flce_status_string": (_c.c_char_p, [_i32]),
    "flce_vocab_chunk": (_i64, [_i64, _i64, _i64, _i32]),
    "flce_kept_chunks": (_i64, [_i64, _i64, _i64, _i32, _i32]),
    "flce_profile_begin": (_i32, []),
    "flce_profile_end": (_i32, []),
    "flce_profile_kinds": (_i32, []),
    "flce_kernel_kind_name": (_c.c_char_p, [_i32]),
    "flce_profile_query": (_i32, [_i32, _c.POINTER(_c.c_double), _c.POINTER(_c.c_int64)]),
}

_lib = None


def load() -> ctypes.CDLL:
    """Load libflce.so; raises if it has not been built (no fallback path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m lm_head_linear_amd.build` "
            "(there is no non-HIP fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
