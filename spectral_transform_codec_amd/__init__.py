"""Spectral transform KV-cache codec for MI355X: Python binding of libstc.

Every step of the codec runs in the HIP library (include/stc.h); this module
only marshals arguments. PyTorch provides device memory and the current HIP
stream. Names follow the C ABI: calibrate_head, encode_kv, decode_kv,
attend_compressed (plus batched forms, state construction and host math).
"""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence

import numpy as np
import torch

from . import _abi
from ._abi import (BF16, D, F32, XFORM_EIGEN, XFORM_IDENTITY, XFORM_RHT, HeadInfo, StcError,  # noqa: F401
                   check, lib)

__all__ = [
    "State", "StateArray", "calibrate_head", "state_init", "rht_state_init", "encode_kv", "decode_kv",
    "encode_kv_batched", "decode_kv_batched", "attend_compressed", "attend_compressed_batched",
    "quantize_pack_f32", "state_bytes", "packed_bytes", "attend_workspace_bytes", "total_bits",
    "delta_star", "water_fill", "eigh", "lloyd_max", "StcError", "set_rht_encode_kernel",
    "get_rht_encode_kernel", "RHT_ENCODE_MFMA", "RHT_ENCODE_BUTTERFLY", "calibrate_heads_batched",
]

_P = ctypes.POINTER


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t: Optional[torch.Tensor]):
    return ctypes.c_void_p(0 if t is None else t.data_ptr())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"K/V tensors must be bfloat16 or float32, got {t.dtype}")


def _np_ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(_P(ctype))


# ------------------------------------------------------------------ sizes
def state_bytes() -> int:
    return int(lib().stc_state_bytes())


def packed_bytes(total_bits: int, n_tokens: int) -> int:
    return int(lib().stc_packed_bytes(int(total_bits), int(n_tokens)))


def attend_workspace_bytes(n_pairs: int, group: int, n_tokens: int) -> int:
    return int(lib().stc_attend_workspace_bytes(int(n_pairs), int(group), int(n_tokens)))


# -------------------------------------------------------------- host math
def total_bits(avg_bits: float, d: int = D) -> int:
    return int(lib().stc_total_bits(float(avg_bits), int(d)))


def delta_star(bits: int) -> float:
    return float(lib().stc_delta_star(int(bits)))


def water_fill(lam: np.ndarray, total: int) -> np.ndarray:
    lam = np.ascontiguousarray(lam, dtype=np.float64)
    out = np.zeros(lam.shape[0], dtype=np.uint8)
    check("stc_water_fill", lib().stc_water_fill(lam.shape[0], _np_ptr(lam, ctypes.c_double), int(total),
                                                 _np_ptr(out, ctypes.c_uint8)))
    return out


ALLOC_VARIANTS = {"greedy": 0, "operational": 1, "grouped": 2, "floor": 3, "gap": 4}


def allocate_bits(lam: np.ndarray, total: int, variant: str = "greedy", param: float = 0.0) -> np.ndarray:
    lam = np.ascontiguousarray(lam, dtype=np.float64)
    out = np.zeros(lam.shape[0], dtype=np.uint8)
    check("stc_allocate_bits", lib().stc_allocate_bits(lam.shape[0], _np_ptr(lam, ctypes.c_double), int(total),
                                                       ALLOC_VARIANTS[variant], float(param),
                                                       _np_ptr(out, ctypes.c_uint8)))
    return out


def eigh(a: np.ndarray):
    a = np.ascontiguousarray(a, dtype=np.float64)
    d = a.shape[0]
    u = np.zeros((d, d), np.float64)
    lam = np.zeros(d, np.float64)
    check("stc_eigh", lib().stc_eigh(d, _np_ptr(a, ctypes.c_double), _np_ptr(u, ctypes.c_double),
                                     _np_ptr(lam, ctypes.c_double)))
    return u, lam


def lloyd_max(samples: np.ndarray, levels: int = 8, tol: float = 1e-12, max_iter: int = 10000):
    y = np.ascontiguousarray(samples, dtype=np.float64)
    c = np.zeros(levels, np.float64)
    it = ctypes.c_int32(0)
    check("stc_lloyd_max", lib().stc_lloyd_max(_np_ptr(y, ctypes.c_double), y.shape[0], levels, tol, max_iter,
                                               _np_ptr(c, ctypes.c_double), ctypes.byref(it)))
    return c, int(it.value)


# ----------------------------------------------------------------- states
class State:
    """One codec state: a device blob (torch uint8 tensor, owned here) plus
    its host summary."""

    def __init__(self, blob: torch.Tensor, info: HeadInfo):
        self.blob = blob
        self.info = info

    @property
    def total_bits(self) -> int:
        return int(self.info.total_bits)

    @property
    def bits(self) -> np.ndarray:
        return np.frombuffer(bytes(self.info.bits), dtype=np.uint8).copy()

    @property
    def lam(self) -> np.ndarray:
        return np.array(self.info.lam[:], dtype=np.float64)

    @property
    def steps(self) -> np.ndarray:
        return np.array(self.info.steps[:], dtype=np.float64)

    @property
    def xform(self) -> int:
        return int(self.info.xform)

    def basis(self) -> np.ndarray:
        u = np.zeros((D, D), np.float32)
        check("stc_state_basis", lib().stc_state_basis(_ptr(self.blob), _np_ptr(u, ctypes.c_float), _stream()))
        return u


def _new_blob(device) -> torch.Tensor:
    # torch's caching allocator returns 512-byte aligned blocks
    return torch.zeros(state_bytes(), dtype=torch.uint8, device=device)


def state_init(u: Optional[np.ndarray], lam: np.ndarray, bits: np.ndarray, steps: Optional[np.ndarray] = None,
               xform: int = XFORM_EIGEN, device="cuda", sketch: Optional[np.ndarray] = None) -> State:
    """sketch: S [128][128] fp32 to attach the keys' selective residual sketch."""
    info = HeadInfo()
    blob = _new_blob(device)
    lam = np.ascontiguousarray(lam, np.float64)
    bits = np.ascontiguousarray(bits, np.uint8)
    u_p = None if u is None else np.ascontiguousarray(u, np.float64)
    s_p = None if steps is None else np.ascontiguousarray(steps, np.float64)
    args = (D, xform, None if u_p is None else _np_ptr(u_p, ctypes.c_double), _np_ptr(lam, ctypes.c_double),
            _np_ptr(bits, ctypes.c_uint8), None if s_p is None else _np_ptr(s_p, ctypes.c_double))
    if sketch is None:
        check("stc_state_init", lib().stc_state_init(*args, ctypes.byref(info), _ptr(blob), _stream()))
    else:
        sk = np.ascontiguousarray(sketch, np.float32)
        assert sk.shape == (128, D)
        check("stc_state_init_sketch", lib().stc_state_init_sketch(*args, _np_ptr(sk, ctypes.c_float),
                                                                   ctypes.byref(info), _ptr(blob), _stream()))
    return State(blob, info)


def rht_state_init(signs: np.ndarray, codebook: np.ndarray, device="cuda") -> State:
    info = HeadInfo()
    blob = _new_blob(device)
    sg = np.ascontiguousarray(signs, np.int8)
    cb = np.ascontiguousarray(codebook, np.float32)
    check("stc_rht_state_init", lib().stc_rht_state_init(D, _np_ptr(sg, ctypes.c_int8), _np_ptr(cb, ctypes.c_float),
                                                         ctypes.byref(info), _ptr(blob), _stream()))
    return State(blob, info)


def rht_sketch_state_init(signs: np.ndarray, codebook: np.ndarray, sketch: np.ndarray, device="cuda") -> State:
    """Walsh-Hadamard state whose keys carry the residual sketch; sketch = S [128][128] fp32."""
    info = HeadInfo()
    blob = _new_blob(device)
    sg = np.ascontiguousarray(signs, np.int8)
    cb = np.ascontiguousarray(codebook, np.float32)
    sk = np.ascontiguousarray(sketch, np.float32)
    assert sk.shape == (128, D)
    check("stc_rht_sketch_state_init", lib().stc_rht_sketch_state_init(
        D, _np_ptr(sg, ctypes.c_int8), _np_ptr(cb, ctypes.c_float), _np_ptr(sk, ctypes.c_float), ctypes.byref(info),
        _ptr(blob), _stream()))
    return State(blob, info)


def calibrate_head(x: torch.Tensor, n_calib: int, avg_bits: float, bits: Optional[np.ndarray] = None,
                   xform: int = XFORM_EIGEN) -> State:
    """x: [n][128] (row stride may exceed 128) bf16/fp32 on the GPU."""
    assert x.dim() == 2 and x.shape[1] == D and x.stride(1) == 1
    info = HeadInfo()
    blob = _new_blob(x.device)
    b = None if bits is None else np.ascontiguousarray(bits, np.uint8)
    check("stc_calibrate_head", lib().stc_calibrate_head(
        D, int(n_calib), _ptr(x), _dtype_code(x), x.stride(0), float(avg_bits),
        None if b is None else _np_ptr(b, ctypes.c_uint8), xform, ctypes.byref(info), _ptr(blob), _stream()))
    return State(blob, info)


class StateArray:
    """States laid out back to back in one device tensor, for batched calls."""

    def __init__(self, states: Sequence[State]):
        assert len(states) > 0
        self.blob = torch.stack([s.blob for s in states]).contiguous()
        self.infos = (HeadInfo * len(states))()
        for i, s in enumerate(states):
            ctypes.memmove(ctypes.byref(self.infos[i]), ctypes.byref(s.info), ctypes.sizeof(HeadInfo))
        self.states = list(states)
        self.n = len(states)
        self.max_bits = max(int(s.info.total_bits) for s in states)
        self.xform = int(states[0].info.xform)

    @classmethod
    def _from_blob(cls, blob: torch.Tensor, infos) -> "StateArray":
        """An array over an existing [n][state_bytes] blob and its summaries
        (the states are views of the blob)."""
        self = cls.__new__(cls)
        self.blob = blob
        self.infos = infos
        self.n = blob.shape[0]
        self.states = []
        for i in range(self.n):
            info = HeadInfo()
            ctypes.memmove(ctypes.byref(info), ctypes.byref(infos[i]), ctypes.sizeof(HeadInfo))
            self.states.append(State(blob[i], info))
        self.max_bits = max(int(infos[i].total_bits) for i in range(self.n))
        self.xform = int(infos[0].xform)
        return self


def calibrate_heads_batched(x: torch.Tensor, n_calib: int, avg_bits: float, xform: int = XFORM_EIGEN) -> StateArray:
    """x: [S][n][128] bf16/fp32 on the GPU (row and stream strides from the
    tensor): one state per stream from its first n_calib rows, in one call."""
    assert x.dim() == 3 and x.shape[2] == D and x.stride(2) == 1 and x.shape[1] >= n_calib
    S = x.shape[0]
    infos = (HeadInfo * S)()
    blob = torch.zeros((S, state_bytes()), dtype=torch.uint8, device=x.device)
    check("stc_calibrate_heads_batched", lib().stc_calibrate_heads_batched(
        D, S, int(n_calib), _ptr(x), _dtype_code(x), x.stride(1), x.stride(0), float(avg_bits), xform, infos,
        _ptr(blob), _stream()))
    return StateArray._from_blob(blob, infos)


# ------------------------------------------------------------------ codec
def encode_kv(state: State, x: torch.Tensor):
    """x: [n][128] bf16/fp32 -> (packed uint8 [packed_bytes], norms fp32 [n] or None)."""
    assert x.dim() == 2 and x.shape[1] == D and x.stride(1) == 1
    n = x.shape[0]
    packed = torch.empty(packed_bytes(state.total_bits, n), dtype=torch.uint8, device=x.device)
    norms = torch.empty(n, dtype=torch.float32, device=x.device) if state.xform == XFORM_RHT else None
    check("stc_encode_kv", lib().stc_encode_kv(ctypes.byref(state.info), _ptr(state.blob), n, _ptr(x),
                                               _dtype_code(x), x.stride(0), _ptr(packed), _ptr(norms), _stream()))
    return packed, norms


def decode_kv(state: State, packed: torch.Tensor, n: int, norms: Optional[torch.Tensor] = None,
              dtype=torch.bfloat16, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    if out is None:
        out = torch.empty((n, D), dtype=dtype, device=packed.device)
    check("stc_decode_kv", lib().stc_decode_kv(ctypes.byref(state.info), _ptr(state.blob), n, _ptr(packed),
                                               _ptr(norms), _ptr(out), _dtype_code(out), out.stride(0), _stream()))
    return out


def quantize_pack_f32(state: State, coeffs: torch.Tensor) -> torch.Tensor:
    """coeffs: fp32 [n][128] latent coefficients -> packed bytes."""
    assert coeffs.dtype == torch.float32 and coeffs.is_contiguous() and coeffs.shape[1] == D
    n = coeffs.shape[0]
    packed = torch.empty(packed_bytes(state.total_bits, n), dtype=torch.uint8, device=coeffs.device)
    check("stc_quantize_pack_f32", lib().stc_quantize_pack_f32(ctypes.byref(state.info), _ptr(state.blob), n,
                                                               _ptr(coeffs), _ptr(packed), _stream()))
    return packed


def _map_arg(m):
    if m is None:
        return None
    assert m.dtype == torch.int32 and m.is_contiguous()
    return m


def check_state_map(state_of_stream: torch.Tensor, n_states: int) -> None:
    """Raise StcError if an entry of the int32 device map lies outside
    [0, n_states) (synchronizes the current stream)."""
    m = _map_arg(state_of_stream)
    check("stc_check_state_map", lib().stc_check_state_map(_ptr(m), m.numel(), int(n_states), _stream()))


RHT_ENCODE_MFMA = 0
RHT_ENCODE_BUTTERFLY = 1


def set_rht_encode_kernel(kind: int) -> None:
    """Walsh-Hadamard encode kernel for later launches: RHT_ENCODE_MFMA (the +-1
    matrix on the matrix cores) or RHT_ENCODE_BUTTERFLY (register butterflies)."""
    check("stc_set_rht_encode_kernel", lib().stc_set_rht_encode_kernel(int(kind)))


def get_rht_encode_kernel() -> int:
    return int(lib().stc_get_rht_encode_kernel())


def stream_copy(dst: torch.Tensor, src: torch.Tensor) -> None:
    """Measurement helper: copy src's bytes into dst (both contiguous, same
    byte size, a multiple of 16) with the library's streaming copy kernel."""
    assert dst.is_contiguous() and src.is_contiguous()
    nb = src.numel() * src.element_size()
    assert dst.numel() * dst.element_size() == nb
    check("stc_stream_copy", lib().stc_stream_copy(_ptr(dst), _ptr(src), nb, _stream()))


def encode_kv_batched(states: StateArray, x: torch.Tensor, state_of_stream: Optional[torch.Tensor] = None,
                      packed: Optional[torch.Tensor] = None, norms: Optional[torch.Tensor] = None):
    """x: [S][n][128] (row and stream strides from the tensor) -> packed [S][stride] uint8
    (stride = packed_bytes(max bits, n)), norms [S][n] for Walsh-Hadamard states."""
    assert x.dim() == 3 and x.shape[2] == D and x.stride(2) == 1
    S, n = x.shape[0], x.shape[1]
    stride = packed_bytes(states.max_bits, n)
    if packed is None:
        packed = torch.empty((S, stride), dtype=torch.uint8, device=x.device)
    if states.xform == XFORM_RHT and norms is None:
        norms = torch.empty((S, n), dtype=torch.float32, device=x.device)
    m = _map_arg(state_of_stream)
    check("stc_encode_kv_batched", lib().stc_encode_kv_batched(
        _ptr(states.blob), states.n, _ptr(m), states.infos, S, n, _ptr(x), _dtype_code(x), x.stride(1),
        x.stride(0), _ptr(packed), packed.stride(0), _ptr(norms), _stream()))
    return packed, norms


def append_kv_batched(states: StateArray, x: torch.Tensor, n_old: int, packed: torch.Tensor,
                      state_of_stream: Optional[torch.Tensor] = None, norms: Optional[torch.Tensor] = None):
    """Append x [S][m][128] (tokens n_old .. n_old+m-1 of every stream) to packed [S][stride]
    uint8 streams holding n_old tokens; stride must fit n_old + m. Walsh-Hadamard states write
    norms [S][>= n_old + m] at columns n_old .. n_old+m-1. Returns packed."""
    assert x.dim() == 3 and x.shape[2] == D and x.stride(2) == 1
    S, m = x.shape[0], x.shape[1]
    if states.xform == XFORM_RHT:
        assert norms is not None and norms.dim() == 2 and norms.stride(1) == 1
    ns = 0 if norms is None else norms.stride(0)
    check("stc_append_kv_batched", lib().stc_append_kv_batched(
        _ptr(states.blob), states.n, _ptr(_map_arg(state_of_stream)), states.infos, S, n_old, m, _ptr(x),
        _dtype_code(x), x.stride(1), x.stride(0), _ptr(packed), packed.stride(0), _ptr(norms), ns, _stream()))
    return packed


def attend_rht_batched(states: StateArray, k_state_of_pair: torch.Tensor, v_state_of_pair: torch.Tensor,
                       k_packed: torch.Tensor, k_norms: torch.Tensor, v_packed: torch.Tensor,
                       v_norms: torch.Tensor, n: int, q: torch.Tensor, scale: Optional[float] = None,
                       ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                       k_sketch: Optional[torch.Tensor] = None, k_rnorm: Optional[torch.Tensor] = None):
    """Attention over Walsh-Hadamard caches: k_packed, v_packed [P][stride] uint8 (same
    stride), k_norms, v_norms fp32 [P][>= n] (same stride); q fp32 [P][g][128]. With
    k_sketch uint8 [P][>= 16 n] and k_rnorm fp32 [P][>= n] the key residual sketch corrects
    the scores."""
    Pn, g = q.shape[0], q.shape[1]
    assert k_packed.stride(0) == v_packed.stride(0) and k_norms.stride(0) == v_norms.stride(0)
    assert k_norms.dtype == torch.float32 and k_norms.stride(1) == 1 and v_norms.stride(1) == 1
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    if out is None:
        out = torch.empty((Pn, g, D), dtype=torch.float32, device=q.device)
    need = attend_workspace_bytes(Pn, g, n)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    check("stc_attend_rht_batched", lib().stc_attend_rht_batched(
        _ptr(states.blob), states.n, _ptr(_map_arg(k_state_of_pair)), _ptr(_map_arg(v_state_of_pair)),
        states.infos, Pn, n, _ptr(k_packed), _ptr(k_norms), _ptr(v_packed), _ptr(v_norms), k_packed.stride(0),
        k_norms.stride(0), _ptr(k_sketch), _ptr(k_rnorm), 0 if k_sketch is None else k_sketch.stride(0),
        0 if k_rnorm is None else k_rnorm.stride(0), g, _ptr(q), _ptr(out), float(scale), _ptr(ws), ws.numel(),
        _stream()))
    return out


def decode_step_batched(states: StateArray, k_state_of_pair: torch.Tensor, v_state_of_pair: torch.Tensor,
                        n_old: int, k_new: torch.Tensor, v_new: torch.Tensor, k_packed: torch.Tensor,
                        v_packed: torch.Tensor, q: torch.Tensor, scale: Optional[float] = None,
                        ws: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None):
    """One generation step: append k_new, v_new [P][128] to the P KV heads' packed K and V
    streams (n_old tokens each, room for one more), then attend q fp32 [P][g][128] over
    all n_old + 1 tokens. Returns out fp32 [P][g][128]."""
    Pn, g = q.shape[0], q.shape[1]
    assert k_new.shape == (Pn, D) and v_new.shape == (Pn, D) and k_new.dtype == v_new.dtype
    assert k_new.is_contiguous() and v_new.is_contiguous() and q.is_contiguous()
    assert k_packed.stride(0) == v_packed.stride(0)
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    if out is None:
        out = torch.empty((Pn, g, D), dtype=torch.float32, device=q.device)
    need = attend_workspace_bytes(Pn, g, n_old + 1)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    check("stc_decode_step_batched", lib().stc_decode_step_batched(
        _ptr(states.blob), states.n, _ptr(_map_arg(k_state_of_pair)), _ptr(_map_arg(v_state_of_pair)),
        states.infos, Pn, n_old, _ptr(k_new), _ptr(v_new), _dtype_code(k_new), _ptr(k_packed), _ptr(v_packed),
        k_packed.stride(0), g, _ptr(q), _ptr(out), float(scale), _ptr(ws), ws.numel(), _stream()))
    return out


def append_rht_sketch_batched(states: StateArray, x: torch.Tensor, n_old: int, packed: torch.Tensor,
                              norms: torch.Tensor, sketch: torch.Tensor, rnorm: torch.Tensor,
                              state_of_stream: Optional[torch.Tensor] = None):
    """Walsh-Hadamard encode/append with the key residual sketch: x [S][m][128] bf16 are tokens
    n_old .. n_old+m-1; packed [S][>= 48 (n_old+m)], norms and rnorm fp32 [S][>= n_old+m],
    sketch uint8 [S][>= 16 (n_old+m)]."""
    assert x.dim() == 3 and x.shape[2] == D and x.stride(2) == 1 and x.dtype == torch.bfloat16
    S, m = x.shape[0], x.shape[1]
    for t in (norms, rnorm):
        assert t.dtype == torch.float32 and t.stride(1) == 1
    check("stc_append_rht_sketch_batched", lib().stc_append_rht_sketch_batched(
        _ptr(states.blob), states.n, _ptr(_map_arg(state_of_stream)), states.infos, S, n_old, m, _ptr(x),
        x.stride(1), x.stride(0), _ptr(packed), packed.stride(0), _ptr(norms), norms.stride(0), _ptr(sketch),
        sketch.stride(0), _ptr(rnorm), rnorm.stride(0), _stream()))
    return packed


def sketch_kv_batched(states: StateArray, x: torch.Tensor, n_old: int, sketch: torch.Tensor, rnorm: torch.Tensor,
                      state_of_stream: Optional[torch.Tensor] = None):
    """Selective residual sketch of eigen keys: x [S][m][128] bf16 are tokens n_old .. n_old+m-1;
    sketch uint8 [S][>= 16 (n_old+m)], rnorm fp32 [S][>= n_old+m]."""
    assert x.dim() == 3 and x.shape[2] == D and x.stride(2) == 1 and x.dtype == torch.bfloat16
    assert rnorm.dtype == torch.float32 and rnorm.stride(1) == 1
    check("stc_sketch_kv_batched", lib().stc_sketch_kv_batched(
        _ptr(states.blob), states.n, _ptr(_map_arg(state_of_stream)), states.infos, x.shape[0], n_old, x.shape[1],
        _ptr(x), x.stride(1), x.stride(0), _ptr(sketch), sketch.stride(0), _ptr(rnorm), rnorm.stride(0), _stream()))
    return sketch


def attend_compressed_sketch_batched(states: StateArray, k_state_of_pair: torch.Tensor,
                                     v_state_of_pair: torch.Tensor, k_packed: torch.Tensor, v_packed: torch.Tensor,
                                     k_sketch: torch.Tensor, k_rnorm: torch.Tensor, n: int, q: torch.Tensor,
                                     scale: Optional[float] = None, ws: Optional[torch.Tensor] = None,
                                     out: Optional[torch.Tensor] = None):
    Pn, g = q.shape[0], q.shape[1]
    assert k_packed.stride(0) == v_packed.stride(0)
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    if out is None:
        out = torch.empty((Pn, g, D), dtype=torch.float32, device=q.device)
    need = attend_workspace_bytes(Pn, g, n)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    check("stc_attend_compressed_sketch_batched", lib().stc_attend_compressed_sketch_batched(
        _ptr(states.blob), states.n, _ptr(_map_arg(k_state_of_pair)), _ptr(_map_arg(v_state_of_pair)),
        states.infos, Pn, n, _ptr(k_packed), _ptr(v_packed), k_packed.stride(0), _ptr(k_sketch), _ptr(k_rnorm),
        k_sketch.stride(0), k_rnorm.stride(0), g, _ptr(q), _ptr(out), float(scale), _ptr(ws), ws.numel(),
        _stream()))
    return out


def decode_kv_batched(states: StateArray, packed: torch.Tensor, n: int, norms: Optional[torch.Tensor] = None,
                      state_of_stream: Optional[torch.Tensor] = None, dtype=torch.bfloat16,
                      out: Optional[torch.Tensor] = None) -> torch.Tensor:
    S = packed.shape[0]
    if out is None:
        out = torch.empty((S, n, D), dtype=dtype, device=packed.device)
    m = _map_arg(state_of_stream)
    check("stc_decode_kv_batched", lib().stc_decode_kv_batched(
        _ptr(states.blob), states.n, _ptr(m), states.infos, S, n, _ptr(packed), packed.stride(0), _ptr(norms),
        _ptr(out), _dtype_code(out), out.stride(1), out.stride(0), _stream()))
    return out


def attend_compressed(k_state: State, v_state: State, k_packed: torch.Tensor, v_packed: torch.Tensor, n: int,
                      q: torch.Tensor, scale: Optional[float] = None, ws: Optional[torch.Tensor] = None):
    """q: fp32 [g][128] -> out fp32 [g][128]."""
    g = q.shape[0]
    assert q.dtype == torch.float32 and q.is_contiguous() and q.shape[1] == D
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    out = torch.empty((g, D), dtype=torch.float32, device=q.device)
    need = attend_workspace_bytes(1, g, n)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    check("stc_attend_compressed", lib().stc_attend_compressed(
        ctypes.byref(k_state.info), _ptr(k_state.blob), ctypes.byref(v_state.info), _ptr(v_state.blob), n,
        _ptr(k_packed), _ptr(v_packed), g, _ptr(q), _ptr(out), float(scale), _ptr(ws), ws.numel(), _stream()))
    return out


def attend_compressed_batched(states: StateArray, k_state_of_pair: torch.Tensor, v_state_of_pair: torch.Tensor,
                              k_packed: torch.Tensor, v_packed: torch.Tensor, n: int, q: torch.Tensor,
                              scale: Optional[float] = None, ws: Optional[torch.Tensor] = None,
                              out: Optional[torch.Tensor] = None):
    """k_packed, v_packed: [P][stride] uint8 (same stride); q: fp32 [P][g][128]."""
    Pn, g = q.shape[0], q.shape[1]
    assert k_packed.stride(0) == v_packed.stride(0)
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    if out is None:
        out = torch.empty((Pn, g, D), dtype=torch.float32, device=q.device)
    need = attend_workspace_bytes(Pn, g, n)
    if ws is None or ws.numel() < need:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    check("stc_attend_compressed_batched", lib().stc_attend_compressed_batched(
        _ptr(states.blob), states.n, _ptr(_map_arg(k_state_of_pair)), _ptr(_map_arg(v_state_of_pair)),
        states.infos, Pn, n, _ptr(k_packed), _ptr(v_packed), k_packed.stride(0), g, _ptr(q), _ptr(out),
        float(scale), _ptr(ws), ws.numel(), _stream()))
    return out


def attend_noalloc_max_bytes() -> int:
    return int(lib().stc_attend_noalloc_max_bytes())


def attend_compressed_batched_noalloc(states: StateArray, k_state_of_pair: torch.Tensor,
                                      v_state_of_pair: torch.Tensor, k_packed: torch.Tensor, v_packed: torch.Tensor,
                                      n: int, q: torch.Tensor, out: torch.Tensor, scale: Optional[float] = None):
    """attend_compressed_batched with the library's static scratch instead of
    a workspace: out fp32 [P][g][128] must be given (the call allocates
    nothing)."""
    Pn, g = q.shape[0], q.shape[1]
    assert k_packed.stride(0) == v_packed.stride(0)
    scale = (1.0 / np.sqrt(D)) if scale is None else scale
    check("stc_attend_compressed_batched_noalloc", lib().stc_attend_compressed_batched_noalloc(
        _ptr(states.blob), states.n, _ptr(_map_arg(k_state_of_pair)), _ptr(_map_arg(v_state_of_pair)),
        states.infos, Pn, n, _ptr(k_packed), _ptr(v_packed), k_packed.stride(0), g, _ptr(q), _ptr(out),
        float(scale), _stream()))
    return out
