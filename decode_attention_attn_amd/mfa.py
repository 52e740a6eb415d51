"""Python binding of libmfa (ctypes): the C entry points under the same names.

Argument marshalling only: torch tensors are passed as device pointers
(``data_ptr()``), sizes and scalars as host values, the stream as the current
torch stream unless given. Every step of the computation runs in the HIP
kernels of ``libmfa.so``; there is no fallback. Importing this module raises
``ImportError`` when the library has not been built
(``python -m decode_attention_attn_amd.build``).
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmfa.so")

# PyTorch-ROCm ships its own HIP runtime (libamdhip64.so, soname .so.7). Load it
# before libmfa.so so that libmfa's dependency resolves to that same runtime;
# loading libmfa first would bring in a second HIP runtime from /opt/rocm whose
# streams and allocations are foreign to torch's.
try:
    import torch  # noqa: F401
except ImportError:  # pragma: no cover - torch is a dependency of the binding
    pass

if not os.path.exists(LIB_PATH):
    raise ImportError(f"libmfa.so not built at {LIB_PATH}; run `python -m decode_attention_attn_amd.build`")
try:
    _lib = ctypes.CDLL(LIB_PATH)
except OSError as e:  # pragma: no cover - depends on the ROCm install
    raise ImportError(f"cannot load {LIB_PATH}: {e}") from e

# mfa_dtype
MFA_F32, MFA_BF16, MFA_FP8_E4M3 = 0, 1, 2
# status codes
MFA_OK, MFA_ERR_INVALID_ARG, MFA_ERR_UNSUPPORTED, MFA_ERR_ALIGNMENT, MFA_ERR_WORKSPACE, MFA_ERR_HIP = 0, -1, -2, -3, -4, -5
MFA_HIDDEN, MFA_RANK, MFA_HEADS, MFA_HEAD_DIM = 7168, 2048, 64, 256
MFA_QDIM = MFA_HEADS * MFA_HEAD_DIM
MFA_MAX_BATCH = 65536
MFA_MAX_TOKENS = 4

_P, _I, _F, _Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t

_lib.mfa_version.restype = _I
_lib.mfa_version.argtypes = []
_lib.mfa_status_string.restype = ctypes.c_char_p
_lib.mfa_status_string.argtypes = [_I]
_lib.mfa_last_hip_error.restype = _I
_lib.mfa_last_hip_error.argtypes = []
_lib.mfa_qproj_workspace_size.restype = _Z
_lib.mfa_qproj_workspace_size.argtypes = [_I, _I]
_lib.mfa_qproj.restype = _I
_lib.mfa_qproj.argtypes = [_P, _P, _P, _F, _P, _P, _P, _Z, _I, _I, _P]
_lib.mfa_kv_append_workspace_size.restype = _Z
_lib.mfa_kv_append_workspace_size.argtypes = [_I, _I]
_lib.mfa_kv_append.restype = _I
_lib.mfa_kv_append.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _Z, _I, _I, _I, _P]
_lib.mfa_kv_append_fp8.restype = _I
_lib.mfa_kv_append_fp8.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _F, _F, _P, _Z, _I, _I, _P]
_lib.mfa_qproj_kv_append_workspace_size.restype = _Z
_lib.mfa_qproj_kv_append_workspace_size.argtypes = [_I]
_lib.mfa_qproj_kv_append.restype = _I
_lib.mfa_qproj_kv_append.argtypes = [_P, _P, _P, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P, _F, _F, _P, _Z, _I, _I, _P]
_lib.mfa_decode_attn_workspace_size.restype = _Z
_lib.mfa_decode_attn_workspace_size.argtypes = [_I, _I]
_lib.mfa_decode_attn.restype = _I
_lib.mfa_decode_attn.argtypes = [_P, _P, _P, _P, _P, _F, _F, _F, _P, _P, _P, _Z, _I, _I, _I, _I, _P]
_lib.mfa_decode_attn_noalloc.restype = _I
_lib.mfa_decode_attn_noalloc.argtypes = [_P, _P, _P, _P, _P, _F, _F, _F, _P, _P, _I, _I, _I, _I, _P]
_lib.mfa_decode_attn_mt_workspace_size.restype = _Z
_lib.mfa_decode_attn_mt_workspace_size.argtypes = [_I, _I, _I]
_lib.mfa_decode_attn_mt.restype = _I
_lib.mfa_decode_attn_mt.argtypes = [_P, _P, _P, _P, _P, _I, _F, _F, _F, _P, _P, _P, _Z, _I, _I, _I, _I, _P]
_lib.mfa_decode_attn_paged.restype = _I
_lib.mfa_decode_attn_paged.argtypes = [_P, _P, _P, _P, _I, _I, _P, _F, _F, _F, _P, _P, _P, _Z, _I, _I, _I, _I, _P]
_lib.mfa_decode_attn_paged_mt.restype = _I
_lib.mfa_decode_attn_paged_mt.argtypes = [_P, _P, _P, _P, _I, _I, _P, _I, _F, _F, _F, _P, _P, _P, _Z, _I, _I, _I, _I,
                                          _P]
_lib.mfa_qproj_w8.restype = _I
_lib.mfa_qproj_w8.argtypes = [_P, _P, _P, _P, _F, _P, _P, _P, _P, _Z, _I, _P]
_lib.mfa_kv_append_w8.restype = _I
_lib.mfa_kv_append_w8.argtypes = [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _I, _F, _F, _P, _Z, _I, _P]
_lib.mfa_oproj_w8.restype = _I
_lib.mfa_oproj_w8.argtypes = [_P, _P, _P, _P, _P, _Z, _I, _P]
_lib.mfa_qproj_kv_append_w8.restype = _I
_lib.mfa_qproj_kv_append_w8.argtypes = [_P, _P, _P, _P, _F, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _F, _F,
                                        _P, _Z, _I, _I, _P]
_lib.mfa_bw_probe.restype = _I
_lib.mfa_bw_probe.argtypes = [_P, _Z, _P, _I, _P]
_lib.mfa_oproj_workspace_size.restype = _Z
_lib.mfa_oproj_workspace_size.argtypes = [_I, _I]
_lib.mfa_oproj.restype = _I
_lib.mfa_oproj.argtypes = [_P, _P, _P, _P, _Z, _I, _I, _P]

EXPORTED = [
    "mfa_version", "mfa_status_string", "mfa_last_hip_error",
    "mfa_qproj_workspace_size", "mfa_qproj",
    "mfa_kv_append_workspace_size", "mfa_kv_append", "mfa_kv_append_fp8",
    "mfa_qproj_kv_append_workspace_size", "mfa_qproj_kv_append",
    "mfa_decode_attn_workspace_size", "mfa_decode_attn", "mfa_decode_attn_noalloc", "mfa_decode_attn_paged",
    "mfa_decode_attn_paged_mt",
    "mfa_decode_attn_mt_workspace_size", "mfa_decode_attn_mt",
    "mfa_oproj_workspace_size", "mfa_oproj",
    "mfa_qproj_w8", "mfa_kv_append_w8", "mfa_oproj_w8", "mfa_qproj_kv_append_w8", "mfa_bw_probe",
]


class MfaError(RuntimeError):
    def __init__(self, status: int, where: str):
        detail = f" [hipError_t {mfa_last_hip_error()}]" if status == MFA_ERR_HIP else ""
        super().__init__(f"{where}: {mfa_status_string(status)} ({status}){detail}")
        self.status = status


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t):
    if t is None:
        return 0
    return t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def check(status: int, where: str = "libmfa") -> None:
    if status != MFA_OK:
        raise MfaError(status, where)


def mfa_version() -> int:
    return _lib.mfa_version()


def mfa_status_string(status: int) -> str:
    return _lib.mfa_status_string(status).decode()


def mfa_last_hip_error() -> int:
    return _lib.mfa_last_hip_error()


def mfa_qproj_workspace_size(B: int, dt: int) -> int:
    return _lib.mfa_qproj_workspace_size(B, dt)


def mfa_qproj(x, w_dq, gamma, eps, w_uq, q_out, ws, B, dt, stream=None) -> int:
    return _lib.mfa_qproj(_ptr(x), _ptr(w_dq), _ptr(gamma), eps, _ptr(w_uq), _ptr(q_out), _ptr(ws), _nbytes(ws),
                          B, dt, _stream(stream))


def mfa_kv_append_workspace_size(B: int, act_dt: int) -> int:
    return _lib.mfa_kv_append_workspace_size(B, act_dt)


def mfa_kv_append(x, w_k, w_v, k_cache, v_cache, seq_off, seq_len, ws, B, act_dt, cache_dt, stream=None,
                  seq_len_out=None) -> int:
    return _lib.mfa_kv_append(_ptr(x), _ptr(w_k), _ptr(w_v), _ptr(k_cache), _ptr(v_cache), _ptr(seq_off),
                              _ptr(seq_len), _ptr(seq_len_out), _ptr(ws), _nbytes(ws), B, act_dt, cache_dt,
                              _stream(stream))


def mfa_kv_append_fp8(x, w_k, w_v, k_cache, v_cache, seq_off, seq_len, k_scale, v_scale, ws, B, act_dt,
                      stream=None, seq_len_out=None) -> int:
    return _lib.mfa_kv_append_fp8(_ptr(x), _ptr(w_k), _ptr(w_v), _ptr(k_cache), _ptr(v_cache), _ptr(seq_off),
                                  _ptr(seq_len), _ptr(seq_len_out), float(k_scale), float(v_scale), _ptr(ws),
                                  _nbytes(ws), B, act_dt, _stream(stream))


def mfa_qproj_kv_append_workspace_size(B: int) -> int:
    return _lib.mfa_qproj_kv_append_workspace_size(B)


def mfa_qproj_kv_append(x, w_dq, gamma, eps, w_uq, w_k, w_v, q_out, k_cache, v_cache, seq_off, seq_len, k_scale,
                        v_scale, ws, B, cache_dt, stream=None, seq_len_out=None) -> int:
    return _lib.mfa_qproj_kv_append(_ptr(x), _ptr(w_dq), _ptr(gamma), eps, _ptr(w_uq), _ptr(w_k), _ptr(w_v),
                                    _ptr(q_out), _ptr(k_cache), _ptr(v_cache), _ptr(seq_off), _ptr(seq_len),
                                    _ptr(seq_len_out), float(k_scale), float(v_scale), _ptr(ws), _nbytes(ws), B,
                                    cache_dt, _stream(stream))


def mfa_decode_attn_workspace_size(B: int, num_workgroups: int = 0) -> int:
    return _lib.mfa_decode_attn_workspace_size(B, num_workgroups)


def mfa_decode_attn(q, k_cache, v_cache, seq_off, seq_len, softmax_scale, k_scale, v_scale, out, lse, ws, B,
                    num_workgroups, q_dt, kv_dt, stream=None) -> int:
    return _lib.mfa_decode_attn(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_off), _ptr(seq_len),
                                softmax_scale, k_scale, v_scale, _ptr(out), _ptr(lse), _ptr(ws), _nbytes(ws), B,
                                num_workgroups, q_dt, kv_dt, _stream(stream))


MFA_NOALLOC_SCRATCH_BYTES = 40 << 20


def mfa_decode_attn_noalloc(q, k_cache, v_cache, seq_off, seq_len, softmax_scale, k_scale, v_scale, out, lse, B,
                            num_workgroups, q_dt, kv_dt, stream=None) -> int:
    return _lib.mfa_decode_attn_noalloc(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_off), _ptr(seq_len),
                                        softmax_scale, k_scale, v_scale, _ptr(out), _ptr(lse), B, num_workgroups,
                                        q_dt, kv_dt, _stream(stream))


def mfa_decode_attn_mt_workspace_size(B: int, n_tokens: int, num_workgroups: int = 0) -> int:
    return _lib.mfa_decode_attn_mt_workspace_size(B, n_tokens, num_workgroups)


def mfa_decode_attn_mt(q, k_cache, v_cache, seq_off, seq_len, n_tokens, softmax_scale, k_scale, v_scale, out, lse,
                       ws, B, num_workgroups, q_dt, kv_dt, stream=None) -> int:
    return _lib.mfa_decode_attn_mt(_ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(seq_off), _ptr(seq_len), n_tokens,
                                   softmax_scale, k_scale, v_scale, _ptr(out), _ptr(lse), _ptr(ws), _nbytes(ws), B,
                                   num_workgroups, q_dt, kv_dt, _stream(stream))


def mfa_decode_attn_paged(q, k_pages, v_pages, block_table, max_blocks, page_rows, seq_len, softmax_scale, k_scale,
                          v_scale, out, lse, ws, B, num_workgroups, q_dt, kv_dt, stream=None) -> int:
    return _lib.mfa_decode_attn_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), max_blocks,
                                      page_rows, _ptr(seq_len), softmax_scale, k_scale, v_scale, _ptr(out),
                                      _ptr(lse), _ptr(ws), _nbytes(ws), B, num_workgroups, q_dt, kv_dt,
                                      _stream(stream))


def mfa_decode_attn_paged_mt(q, k_pages, v_pages, block_table, max_blocks, page_rows, seq_len, n_tokens,
                             softmax_scale, k_scale, v_scale, out, lse, ws, B, num_workgroups, q_dt, kv_dt,
                             stream=None) -> int:
    return _lib.mfa_decode_attn_paged_mt(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(block_table), max_blocks,
                                         page_rows, _ptr(seq_len), n_tokens, softmax_scale, k_scale, v_scale,
                                         _ptr(out), _ptr(lse), _ptr(ws), _nbytes(ws), B, num_workgroups, q_dt, kv_dt,
                                         _stream(stream))


def mfa_oproj_workspace_size(B: int, dt: int) -> int:
    return _lib.mfa_oproj_workspace_size(B, dt)


def mfa_oproj(attn, w_o, y, ws, B, dt, stream=None) -> int:
    return _lib.mfa_oproj(_ptr(attn), _ptr(w_o), _ptr(y), _ptr(ws), _nbytes(ws), B, dt, _stream(stream))


def raw_function(name: str):
    """The ctypes function object of an exported symbol (for ABI tests)."""
    return getattr(_lib, name)


def mfa_qproj_w8(x, w_dq, s_dq, gamma, eps, w_uq, s_uq, q_out, ws, B, stream=None) -> int:
    return _lib.mfa_qproj_w8(_ptr(x), _ptr(w_dq), _ptr(s_dq), _ptr(gamma), eps, _ptr(w_uq), _ptr(s_uq), _ptr(q_out),
                             _ptr(ws), _nbytes(ws), B, _stream(stream))


def mfa_kv_append_w8(x, w_k, s_k, w_v, s_v, k_cache, v_cache, seq_off, seq_len, cache_dt, k_scale, v_scale, ws, B,
                     stream=None, seq_len_out=None) -> int:
    return _lib.mfa_kv_append_w8(_ptr(x), _ptr(w_k), _ptr(s_k), _ptr(w_v), _ptr(s_v), _ptr(k_cache), _ptr(v_cache),
                                 _ptr(seq_off), _ptr(seq_len), _ptr(seq_len_out), cache_dt, float(k_scale),
                                 float(v_scale), _ptr(ws), _nbytes(ws), B, _stream(stream))


def mfa_oproj_w8(attn, w_o, s_o, y, ws, B, stream=None) -> int:
    return _lib.mfa_oproj_w8(_ptr(attn), _ptr(w_o), _ptr(s_o), _ptr(y), _ptr(ws), _nbytes(ws), B, _stream(stream))


def mfa_qproj_kv_append_w8(x, w_dq, s_dq, gamma, eps, w_uq, s_uq, w_k, s_k, w_v, s_v, q_out, k_cache, v_cache,
                           seq_off, seq_len, k_scale, v_scale, ws, B, cache_dt, stream=None, seq_len_out=None) -> int:
    return _lib.mfa_qproj_kv_append_w8(_ptr(x), _ptr(w_dq), _ptr(s_dq), _ptr(gamma), eps, _ptr(w_uq), _ptr(s_uq),
                                       _ptr(w_k), _ptr(s_k), _ptr(w_v), _ptr(s_v), _ptr(q_out), _ptr(k_cache),
                                       _ptr(v_cache), _ptr(seq_off), _ptr(seq_len), _ptr(seq_len_out),
                                       float(k_scale), float(v_scale), _ptr(ws), _nbytes(ws), B, cache_dt,
                                       _stream(stream))


def mfa_bw_probe(buf, sink, num_workgroups=0, stream=None) -> int:
    return _lib.mfa_bw_probe(_ptr(buf), _nbytes(buf), _ptr(sink), num_workgroups, _stream(stream))
