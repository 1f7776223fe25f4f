"""ctypes declarations of libstc (include/stc.h). Loading fails loudly when
the library has not been built: there is no fallback path."""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libstc.so")
DEBUG_LIB_PATH = os.path.join(HERE, "libstc_debug.so")  # the same library with device index checks

D = 128
STC_OK, STC_EINVAL, STC_EUNSUPPORTED, STC_EBUDGET, STC_EWORKSPACE, STC_EDEVICE = 0, -1, -2, -3, -4, -5
F32, BF16 = 0, 1
XFORM_EIGEN, XFORM_IDENTITY, XFORM_RHT = 0, 1, 2

c_i32, c_i64, c_u8, c_f32, c_f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_uint8, ctypes.c_float, ctypes.c_double
c_size, c_vp, c_cp = ctypes.c_size_t, ctypes.c_void_p, ctypes.c_char_p


class HeadInfo(ctypes.Structure):
    _fields_ = [("d", c_i32), ("xform", c_i32), ("total_bits", c_i32), ("n_kept", c_i32),
                ("bits", c_u8 * D), ("lam", c_f64 * D), ("steps", c_f64 * D), ("sketch_bits", c_i32)]


P = ctypes.POINTER
# name: (restype, argtypes)
SIGNATURES = {
    "stc_state_bytes": (c_size, []),
    "stc_packed_bytes": (c_size, [c_i32, c_i64]),
    "stc_attend_workspace_bytes": (c_size, [c_i64, c_i32, c_i64]),
    "stc_total_bits": (c_i32, [c_f32, c_i32]),
    "stc_delta_star": (c_f64, [c_i32]),
    "stc_water_fill": (c_i32, [c_i32, P(c_f64), c_i32, P(c_u8)]),
    "stc_allocate_bits": (c_i32, [c_i32, P(c_f64), c_i32, c_i32, c_f64, P(c_u8)]),
    "stc_eigh": (c_i32, [c_i32, P(c_f64), P(c_f64), P(c_f64)]),
    "stc_lloyd_max": (c_i32, [P(c_f64), c_i64, c_i32, c_f64, c_i32, P(c_f64), P(c_i32)]),
    "stc_state_init": (c_i32, [c_i32, c_i32, P(c_f64), P(c_f64), P(c_u8), P(c_f64), P(HeadInfo), c_vp, c_vp]),
    "stc_rht_state_init": (c_i32, [c_i32, P(ctypes.c_int8), P(c_f32), P(HeadInfo), c_vp, c_vp]),
    "stc_calibrate_head": (c_i32, [c_i32, c_i64, c_vp, c_i32, c_i64, c_f32, P(c_u8), c_i32, P(HeadInfo),
                                   c_vp, c_vp]),
    "stc_calibrate_heads_batched": (c_i32, [c_i32, c_i64, c_i64, c_vp, c_i32, c_i64, c_i64, c_f32, c_i32,
                                            P(HeadInfo), c_vp, c_vp]),
    "stc_state_basis": (c_i32, [c_vp, P(c_f32), c_vp]),
    "stc_encode_kv_batched": (c_i32, [c_vp, c_i64, c_vp, P(HeadInfo), c_i64, c_i64, c_vp, c_i32, c_i64, c_i64,
                                      c_vp, c_i64, c_vp, c_vp]),
    "stc_decode_kv_batched": (c_i32, [c_vp, c_i64, c_vp, P(HeadInfo), c_i64, c_i64, c_vp, c_i64, c_vp, c_vp,
                                      c_i32, c_i64, c_i64, c_vp]),
    "stc_append_kv_batched": (c_i32, [c_vp, c_i64, c_vp, P(HeadInfo), c_i64, c_i64, c_i64, c_vp, c_i32, c_i64,
                                      c_i64, c_vp, c_i64, c_vp, c_i64, c_vp]),
    "stc_append_rht_sketch_batched": (c_i32, [c_vp, c_i64, c_vp, P(HeadInfo), c_i64, c_i64, c_i64, c_vp, c_i64,
                                              c_i64, c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp, c_i64, c_vp]),
    "stc_rht_sketch_state_init": (c_i32, [c_i32, P(ctypes.c_int8), P(c_f32), P(c_f32), P(HeadInfo), c_vp, c_vp]),
    "stc_state_init_sketch": (c_i32, [c_i32, c_i32, P(c_f64), P(c_f64), P(c_u8), P(c_f64), P(c_f32), P(HeadInfo),
                                      c_vp, c_vp]),
    "stc_sketch_kv_batched": (c_i32, [c_vp, c_i64, c_vp, P(HeadInfo), c_i64, c_i64, c_i64, c_vp, c_i64, c_i64, c_vp,
                                      c_i64, c_vp, c_i64, c_vp]),
    "stc_attend_compressed_sketch_batched": (c_i32, [c_vp, c_i64, c_vp, c_vp, P(HeadInfo), c_i64, c_i64, c_vp, c_vp,
                                                     c_i64, c_vp, c_vp, c_i64, c_i64, c_i32, c_vp, c_vp, c_f32, c_vp,
                                                     c_size, c_vp]),
    "stc_encode_kv": (c_i32, [P(HeadInfo), c_vp, c_i64, c_vp, c_i32, c_i64, c_vp, c_vp, c_vp]),
    "stc_decode_kv": (c_i32, [P(HeadInfo), c_vp, c_i64, c_vp, c_vp, c_vp, c_i32, c_i64, c_vp]),
    "stc_quantize_pack_f32": (c_i32, [P(HeadInfo), c_vp, c_i64, c_vp, c_vp, c_vp]),
    "stc_attend_compressed_batched": (c_i32, [c_vp, c_i64, c_vp, c_vp, P(HeadInfo), c_i64, c_i64, c_vp, c_vp,
                                              c_i64, c_i32, c_vp, c_vp, c_f32, c_vp, c_size, c_vp]),
    "stc_attend_compressed_batched_noalloc": (c_i32, [c_vp, c_i64, c_vp, c_vp, P(HeadInfo), c_i64, c_i64, c_vp,
                                                      c_vp, c_i64, c_i32, c_vp, c_vp, c_f32, c_vp]),
    "stc_attend_noalloc_max_bytes": (c_size, []),
    "stc_attend_compressed": (c_i32, [P(HeadInfo), c_vp, P(HeadInfo), c_vp, c_i64, c_vp, c_vp, c_i32, c_vp,
                                      c_vp, c_f32, c_vp, c_size, c_vp]),
    "stc_attend_rht_batched": (c_i32, [c_vp, c_i64, c_vp, c_vp, P(HeadInfo), c_i64, c_i64, c_vp, c_vp, c_vp, c_vp,
                                       c_i64, c_i64, c_vp, c_vp, c_i64, c_i64, c_i32, c_vp, c_vp, c_f32, c_vp,
                                       c_size, c_vp]),
    "stc_decode_step_batched": (c_i32, [c_vp, c_i64, c_vp, c_vp, P(HeadInfo), c_i64, c_i64, c_vp, c_vp, c_i32,
                                        c_vp, c_vp, c_i64, c_i32, c_vp, c_vp, c_f32, c_vp, c_size, c_vp]),
    "stc_check_state_map": (c_i32, [c_vp, c_i64, c_i64, c_vp]),
    "stc_set_rht_encode_kernel": (c_i32, [c_i32]),
    "stc_get_rht_encode_kernel": (c_i32, []),
    "stc_debug_build": (c_i32, []),
    "stc_stream_copy": (c_i32, [c_vp, c_vp, c_i64, c_vp]),
    "stc_debug_flags": (c_i32, [P(ctypes.c_uint32), c_vp]),
    "stc_status_str": (c_cp, [c_i32]),
    "stc_last_error": (c_cp, []),
}

_lib = None
_loaded = {}


def load(path):
    """The library at `path` with every declared signature (loaded once)."""
    if path not in _loaded:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() "
                               "(python -m spectral_transform_codec_amd.build)")
        h = ctypes.CDLL(path)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(h, name)
            f.restype = res
            f.argtypes = args
        _loaded[path] = h
    return _loaded[path]


def lib():
    global _lib
    if _lib is None:
        _lib = load(LIB_PATH)
    return _lib


class use_library:
    """Route the binding's calls to the library at `path` inside a `with`
    block (for the debug build), then back to the one before."""

    def __init__(self, path):
        self.path = path

    def __enter__(self):
        global _lib
        self.prev = _lib
        _lib = load(self.path)
        return _lib

    def __exit__(self, *exc):
        global _lib
        _lib = self.prev
        return False


class StcError(RuntimeError):
    def __init__(self, call, status):
        L = lib()
        msg = L.stc_last_error().decode()
        super().__init__(f"{call}: {L.stc_status_str(status).decode()} ({status}): {msg}")
        self.status = status


def check(call, status):
    if status != STC_OK:
        raise StcError(call, status)
