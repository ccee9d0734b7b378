"""ctypes binding of libstarattn: the C ABI's calls under the same names.

Argument marshalling only: tensors become device pointers, the stream becomes
a hipStream_t, non-zero return codes become ``StarAttnError``. All work runs in
the HIP library; when the library is missing every call fails loudly.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libstarattn.so")
HEADER_PATH = os.path.join(os.path.dirname(HERE), "include", "starattn.h")

SA_OK, SA_EINVAL, SA_ENOTSUP, SA_EWORKSPACE, SA_EHIP = 0, -1, -2, -3, -4
SA_F32, SA_BF16 = 0, 1
SA_CALL_PHASE1, SA_CALL_PHASE2 = 1, 2
SA_ANCHOR_FIRST, SA_ANCHOR_PREVIOUS = 0, 1
ERROR_NAMES = {SA_EINVAL: "SA_EINVAL", SA_ENOTSUP: "SA_ENOTSUP", SA_EWORKSPACE: "SA_EWORKSPACE",
               SA_EHIP: "SA_EHIP"}


class StarAttnError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {message}")
        self.code = code


class sa_attn_desc(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("rope_theta", ctypes.c_double), ("softmax_scale", ctypes.c_float),
                ("reserved", ctypes.c_int32)]


SA_MAX_BATCH = 16


class sa_decode_seq(ctypes.Structure):
    _fields_ = [("q", ctypes.c_void_p), ("k_new", ctypes.c_void_p), ("v_new", ctypes.c_void_p),
                ("k_cache", ctypes.c_void_p), ("v_cache", ctypes.c_void_p), ("k_tail", ctypes.c_void_p),
                ("v_tail", ctypes.c_void_p), ("out", ctypes.c_void_p), ("lse", ctypes.c_void_p),
                ("ctx_len", ctypes.c_int64), ("block_len", ctypes.c_int64), ("tail_cap", ctypes.c_int64),
                ("tail_len", ctypes.c_int64)]


def make_desc(n_q_heads: int, n_kv_heads: int, head_dim: int, dtype: int, rope_theta: float,
              softmax_scale: float) -> sa_attn_desc:
    return sa_attn_desc(n_q_heads, n_kv_heads, head_dim, dtype, rope_theta, softmax_scale, 0)


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_SIGS = {
    "sa_phase1_encode": (ctypes.c_int, [ctypes.POINTER(sa_attn_desc), _I64, _I64, _I64, _P, _P, _P, _P, _P, _P, _P,
                                        ctypes.c_size_t, _P]),
    "sa_phase1_encode_anchor": (ctypes.c_int, [ctypes.POINTER(sa_attn_desc), _I64, _I64, _I64, _I32, _P, _P, _P, _P,
                                               _P, _P, _P, ctypes.c_size_t, _P]),
    "sa_phase1_encode_anchor_at": (ctypes.c_int, [ctypes.POINTER(sa_attn_desc), _I64, _I64, _I64,
                                                  ctypes.POINTER(_I64), _P, _P, _P, _P, _P, _P, _P, ctypes.c_size_t,
                                                  _P]),
    "sa_anchor_at_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(sa_attn_desc), _I64, _I64, _I64]),
    "sa_decode_append": (ctypes.c_int, [ctypes.POINTER(sa_attn_desc), _P, _P, _I64, _I64, _P, _P, _I64, _I64, _P]),
    "sa_phase2_partial": (ctypes.c_int, [ctypes.POINTER(sa_attn_desc), _P, _I64, _I64, _P, _P, _I64, _I64, _P, _P,
                                         _I64, _I64, _I64, _P, _P, _P, ctypes.c_size_t, _P]),
    "sa_phase2_step": (ctypes.c_int, [ctypes.POINTER(sa_attn_desc), _P, _P, _P, _I64, _P, _P, _I64, _I64, _P, _P,
                                      _I64, _I64, _P, _P, _P, ctypes.c_size_t, _P]),
    "sa_phase2_step_noalloc": (ctypes.c_int, [ctypes.POINTER(sa_attn_desc), _P, _P, _P, _I64, _P, _P, _I64, _I64, _P,
                                              _P, _I64, _I64, _P, _P, _P]),
    "sa_decode_batch_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(sa_attn_desc), _I32,
                                                         ctypes.POINTER(sa_decode_seq)]),
    "sa_decode_step_batched": (ctypes.c_int, [ctypes.POINTER(sa_attn_desc), _I32, ctypes.POINTER(sa_decode_seq), _P,
                                              ctypes.c_size_t, _P]),
    "sa_phase2_merge": (ctypes.c_int, [_I32, _I64, _I32, _I32, _P, _P, _P, _I32, _P, _P]),
    "sa_workspace_bytes": (ctypes.c_size_t, [_I32, ctypes.POINTER(sa_attn_desc), _I64, _I64, _I64, _I64]),
    "sa_calibrate_stream_read": (ctypes.c_int, [_P, ctypes.c_size_t, _P, _P]),
    "sa_calibrate_mfma": (ctypes.c_int, [_I32, _I32, _P, _P]),
    "sa_device_info": (ctypes.c_int, [ctypes.POINTER(ctypes.c_int32)] * 4),
    "sa_last_error": (ctypes.c_char_p, []),
    "sa_abi_version": (ctypes.c_int32, []),
}


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libstarattn.so not built at {LIB_PATH}; run python -m long_context_attention_amd.build")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(l, name)
            f.restype, f.argtypes = res, args
        _lib = l
    return _lib


def header_symbols() -> list[str]:
    """Function names declared in include/starattn.h."""
    text = open(HEADER_PATH).read()
    return sorted(set(re.findall(r"^\s*(?:int|int32_t|size_t|const char\*)\s+(sa_\w+)\s*\(", text, re.M)))


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x or None
    return x.data_ptr() or None


def _nbytes(x) -> int:
    if x is None:
        return 0
    if isinstance(x, int):
        raise TypeError("pass the workspace as a tensor (its size is taken from it)")
    return x.numel() * x.element_size()


def _stream(stream):
    if stream is None:
        import torch
        if not torch.cuda.is_available():
            return None
        return torch.cuda.current_stream().cuda_stream or None
    if isinstance(stream, int):
        return stream or None
    return stream.cuda_stream or None


def _check(rc: int) -> None:
    if rc != SA_OK:
        raise StarAttnError(rc, lib().sa_last_error().decode())


def sa_abi_version() -> int:
    return int(lib().sa_abi_version())


def sa_last_error() -> str:
    return lib().sa_last_error().decode()


def sa_workspace_bytes(which_call: int, desc: sa_attn_desc, ctx_len: int, block_len: int, t_q: int,
                       tail_cap: int) -> int:
    return int(lib().sa_workspace_bytes(which_call, ctypes.byref(desc), ctx_len, block_len, t_q, tail_cap))


def sa_phase1_encode(desc, ctx_len, block_len, anchor_len, q_ctx, k_ctx, v_ctx, out_ctx, k_cache, v_cache,
                     workspace=None, stream=None) -> None:
    _check(lib().sa_phase1_encode(ctypes.byref(desc), ctx_len, block_len, anchor_len, _ptr(q_ctx), _ptr(k_ctx),
                                  _ptr(v_ctx), _ptr(out_ctx), _ptr(k_cache), _ptr(v_cache), _ptr(workspace),
                                  _nbytes(workspace), _stream(stream)))


def sa_phase1_encode_anchor(desc, ctx_len, block_len, anchor_len, anchor_kind, q_ctx, k_ctx, v_ctx, out_ctx,
                            k_cache, v_cache, workspace=None, stream=None) -> None:
    _check(lib().sa_phase1_encode_anchor(ctypes.byref(desc), ctx_len, block_len, anchor_len, anchor_kind, _ptr(q_ctx),
                                         _ptr(k_ctx), _ptr(v_ctx), _ptr(out_ctx), _ptr(k_cache), _ptr(v_cache),
                                         _ptr(workspace), _nbytes(workspace), _stream(stream)))


def sa_anchor_at_workspace_bytes(desc, ctx_len, block_len, anchor_len) -> int:
    return int(lib().sa_anchor_at_workspace_bytes(ctypes.byref(desc), ctx_len, block_len, anchor_len))


def sa_phase1_encode_anchor_at(desc, ctx_len, block_len, anchor_len, anchor_pos, q_ctx, k_ctx, v_ctx, out_ctx,
                               k_cache, v_cache, workspace=None, stream=None) -> None:
    """``anchor_pos``: a sequence of ctx_len // block_len ints (copied into a host int64 array), or None."""
    pos = None if anchor_pos is None else (_I64 * len(anchor_pos))(*[int(p) for p in anchor_pos])
    _check(lib().sa_phase1_encode_anchor_at(ctypes.byref(desc), ctx_len, block_len, anchor_len, pos, _ptr(q_ctx),
                                            _ptr(k_ctx), _ptr(v_ctx), _ptr(out_ctx), _ptr(k_cache), _ptr(v_cache),
                                            _ptr(workspace), _nbytes(workspace), _stream(stream)))


def sa_decode_append(desc, k_new, v_new, t_new, pos0, k_tail, v_tail, tail_cap, tail_len, stream=None) -> None:
    _check(lib().sa_decode_append(ctypes.byref(desc), _ptr(k_new), _ptr(v_new), t_new, pos0, _ptr(k_tail),
                                  _ptr(v_tail), tail_cap, tail_len, _stream(stream)))


def sa_phase2_partial(desc, q, t_q, q_pos0, k_cache, v_cache, ctx_len, block_len, k_tail, v_tail, tail_cap,
                      tail_len, tail_pos0, out_part, lse_part, workspace=None, stream=None) -> None:
    _check(lib().sa_phase2_partial(ctypes.byref(desc), _ptr(q), t_q, q_pos0, _ptr(k_cache), _ptr(v_cache), ctx_len,
                                   block_len, _ptr(k_tail), _ptr(v_tail), tail_cap, tail_len, tail_pos0,
                                   _ptr(out_part), _ptr(lse_part), _ptr(workspace), _nbytes(workspace),
                                   _stream(stream)))


def sa_phase2_step(desc, q, k_new, v_new, t, k_cache, v_cache, ctx_len, block_len, k_tail, v_tail, tail_cap,
                   tail_len, out, lse=None, workspace=None, stream=None) -> None:
    _check(lib().sa_phase2_step(ctypes.byref(desc), _ptr(q), _ptr(k_new), _ptr(v_new), t, _ptr(k_cache),
                                _ptr(v_cache), ctx_len, block_len, _ptr(k_tail), _ptr(v_tail), tail_cap, tail_len,
                                _ptr(out), _ptr(lse), _ptr(workspace), _nbytes(workspace), _stream(stream)))


def sa_phase2_step_noalloc(desc, q, k_new, v_new, t, k_cache, v_cache, ctx_len, block_len, k_tail, v_tail, tail_cap,
                           tail_len, out, lse=None, stream=None) -> None:
    _check(lib().sa_phase2_step_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k_new), _ptr(v_new), t, _ptr(k_cache),
                                        _ptr(v_cache), ctx_len, block_len, _ptr(k_tail), _ptr(v_tail), tail_cap,
                                        tail_len, _ptr(out), _ptr(lse), _stream(stream)))


SA_NOALLOC_SCRATCH_BYTES = 64 << 20


def decode_seqs(seqs) -> ctypes.Array:
    """A C array of sa_decode_seq from dicts with the struct's field names
    (tensors for the pointers, ints for the sizes; lse may be missing)."""
    arr = (sa_decode_seq * len(seqs))()
    for i, d in enumerate(seqs):
        for name, _ in sa_decode_seq._fields_:
            v = d.get(name)
            setattr(arr[i], name, v if name in ("ctx_len", "block_len", "tail_cap", "tail_len") else _ptr(v))
    return arr


def sa_decode_batch_workspace_bytes(desc, seqs) -> int:
    arr = seqs if isinstance(seqs, ctypes.Array) else decode_seqs(seqs)
    return int(lib().sa_decode_batch_workspace_bytes(ctypes.byref(desc), len(arr), arr))


def sa_decode_step_batched(desc, seqs, workspace, stream=None) -> None:
    arr = seqs if isinstance(seqs, ctypes.Array) else decode_seqs(seqs)
    _check(lib().sa_decode_step_batched(ctypes.byref(desc), len(arr), arr, _ptr(workspace), _nbytes(workspace),
                                        _stream(stream)))


def sa_phase2_merge(n_parts, t_q, n_q_heads, head_dim, out_part, lse_part, out, out_dtype, lse=None,
                    stream=None) -> None:
    _check(lib().sa_phase2_merge(n_parts, t_q, n_q_heads, head_dim, _ptr(out_part), _ptr(lse_part), _ptr(out),
                                 out_dtype, _ptr(lse), _stream(stream)))


def sa_calibrate_stream_read(buf, sink, stream=None) -> None:
    _check(lib().sa_calibrate_stream_read(_ptr(buf), _nbytes(buf), _ptr(sink), _stream(stream)))


def sa_calibrate_mfma(iters, n_workgroups, sink, stream=None) -> None:
    _check(lib().sa_calibrate_mfma(iters, n_workgroups, _ptr(sink), _stream(stream)))


def sa_device_info() -> dict:
    """Compute units, peak shader and memory clocks (kHz) and memory bus width (bits) of the current device."""
    v = [ctypes.c_int32() for _ in range(4)]
    _check(lib().sa_device_info(*[ctypes.byref(x) for x in v]))
    return {"n_cus": v[0].value, "clock_khz": v[1].value, "mem_clock_khz": v[2].value, "mem_bus_bits": v[3].value}
