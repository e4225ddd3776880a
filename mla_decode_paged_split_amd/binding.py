"""Thin ctypes binding over libmla_decode.so (argument marshalling only).

Every entry point keeps the C name from ``include/mla_decode.h``.  torch is
used only to own device memory and to name the current stream; all of the
computation happens in the library's HIP kernels.  There is no fallback: if
the library is missing or a call fails, a RuntimeError is raised.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "MLA_OK",
    "MLA_ERR_INVALID_ARG",
    "MLA_ERR_UNSUPPORTED",
    "MLA_ERR_WORKSPACE",
    "MLA_ERR_HIP",
    "MLA_DTYPE_BF16",
    "MLA_DTYPE_FP8_E4M3FN",
    "MLA_FLAG_FUSED_MERGE",
    "MLA_FLAG_FUSED_Q_CAST",
    "MLA_FLAG_CAUSAL",
    "MlaDecodeParams",
    "MlaDecodePlan",
    "library_path",
    "lib",
    "mla_status_string",
    "mla_decode_abi_version",
    "mla_read_probe",
    "MLA_READ_PROBE_BYTES_PER_WORD",
    "read_probe_sink_words",
    "mla_decode_workspace_size",
    "mla_decode_plan",
    "mla_decode_run",
    "mla_decode_run_paged",
    "mla_decode_attend",
    "mla_decode_merge",
    "mla_decode_quantize_q",
    "mla_decode_quantize_q_dynamic",
    "MLA_QUANT_DYNAMIC_SCRATCH_BYTES",
    "mla_decode_reduce",
    "mla_decode_run_noalloc",
    "MLA_NOALLOC_SCRATCH_BYTES",
    "make_params",
    "Decoder",
]

MLA_OK = 0
MLA_ERR_INVALID_ARG = 1
MLA_ERR_UNSUPPORTED = 2
MLA_ERR_WORKSPACE = 3
MLA_ERR_HIP = 4
MLA_DTYPE_BF16 = 0
MLA_DTYPE_FP8_E4M3FN = 1
MLA_FLAG_FUSED_MERGE = 1
MLA_FLAG_FUSED_Q_CAST = 2
MLA_FLAG_CAUSAL = 4
MLA_QUANT_DYNAMIC_SCRATCH_BYTES = 1024
MLA_NOALLOC_SCRATCH_BYTES = 26 << 20

_DTYPES = {"bf16": MLA_DTYPE_BF16, "fp8": MLA_DTYPE_FP8_E4M3FN}


class MlaDecodeParams(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("num_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("qk_dim", ctypes.c_int32),
        ("v_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("num_units", ctypes.c_int32),
        ("min_chunk", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
        ("max_q_len", ctypes.c_int32),
        ("logit_cap", ctypes.c_float),
    ]


class MlaDecodePlan(ctypes.Structure):
    _fields_ = [
        ("params", MlaDecodeParams),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("device", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("off_counters", ctypes.c_uint64),
        ("off_part_o", ctypes.c_uint64),
        ("off_part_lse", ctypes.c_uint64),
    ]


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmla_decode.so")


_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    """Load the built library once; raise if it has not been built."""
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with __graft_entry__.build() (hipcc, gfx950)")
        L = ctypes.CDLL(path)
        vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        L.mla_status_string.argtypes = [ctypes.c_int]
        L.mla_status_string.restype = ctypes.c_char_p
        L.mla_decode_abi_version.argtypes = []
        L.mla_decode_abi_version.restype = i32
        L.mla_read_probe.argtypes = [vp, sz, vp, sz, vp]
        L.mla_read_probe.restype = ctypes.c_int
        L.mla_decode_workspace_size.argtypes = [ctypes.POINTER(MlaDecodeParams)]
        L.mla_decode_workspace_size.restype = sz
        L.mla_decode_plan.argtypes = [ctypes.POINTER(MlaDecodeParams), vp, sz, vp, ctypes.POINTER(MlaDecodePlan)]
        L.mla_decode_plan.restype = ctypes.c_int
        L.mla_decode_run.argtypes = [ctypes.POINTER(MlaDecodePlan), vp, vp, vp, vp, vp, vp, vp, f32, vp, vp]
        L.mla_decode_run.restype = ctypes.c_int
        L.mla_decode_run_paged.argtypes = [ctypes.POINTER(MlaDecodePlan), vp, vp, vp, vp, vp, vp, vp, vp, f32, vp,
                                           vp, vp]
        L.mla_decode_run_paged.restype = ctypes.c_int
        L.mla_decode_attend.argtypes = L.mla_decode_run_paged.argtypes
        L.mla_decode_attend.restype = ctypes.c_int
        L.mla_decode_merge.argtypes = [ctypes.POINTER(MlaDecodePlan), vp, vp, vp, vp, vp]
        L.mla_decode_merge.restype = ctypes.c_int
        L.mla_decode_quantize_q.argtypes = [vp, vp, i64, vp]
        L.mla_decode_quantize_q.restype = ctypes.c_int
        L.mla_decode_quantize_q_dynamic.argtypes = [vp, vp, vp, vp, sz, i64, vp]
        L.mla_decode_quantize_q_dynamic.restype = ctypes.c_int
        L.mla_decode_reduce.argtypes = [vp, vp, vp, i32, vp, vp, vp]
        L.mla_decode_reduce.restype = ctypes.c_int
        L.mla_decode_run_noalloc.argtypes = [ctypes.POINTER(MlaDecodeParams), vp, vp, vp, vp, vp, vp, vp, vp, f32,
                                             vp, vp, vp]
        L.mla_decode_run_noalloc.restype = ctypes.c_int
        _LIB = L
    return _LIB


def _check(code: int, what: str) -> None:
    if code != MLA_OK:
        raise RuntimeError(f"{what} failed: {mla_status_string(code)}")


_PLACEHOLDERS: dict = {}


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    if t.numel() == 0:
        # torch gives zero-element tensors a null address; the C ABI rejects null,
        # and a zero-element buffer is never read, so pass a small live allocation
        ph = _PLACEHOLDERS.get(t.device)
        if ph is None:
            ph = _PLACEHOLDERS[t.device] = torch.zeros(16, dtype=torch.uint8, device=t.device)
        return ph.data_ptr()
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def mla_status_string(code: int) -> str:
    return lib().mla_status_string(int(code)).decode()


def mla_decode_abi_version() -> int:
    return int(lib().mla_decode_abi_version())


MLA_READ_PROBE_BYTES_PER_WORD = 32768


def read_probe_sink_words(nbytes: int) -> int:
    """Sink words mla_read_probe needs for a buffer of nbytes: one per probe workgroup."""
    return -(-nbytes // MLA_READ_PROBE_BYTES_PER_WORD)


def mla_read_probe(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Diagnostic streaming read of all of `buf` (see the header); `sink` holds one int32 per probe workgroup."""
    nbytes = buf.numel() * buf.element_size()
    if sink.dtype != torch.int32 or sink.numel() < read_probe_sink_words(nbytes):
        raise ValueError(f"sink must be int32 with at least {read_probe_sink_words(nbytes)} elements")
    code = lib().mla_read_probe(_ptr(buf), nbytes, _ptr(sink), sink.numel(), _stream(stream))
    _check(code, "mla_read_probe")


def make_params(batch: int, q_dtype: str, kv_dtype: str, *, total_q: Optional[int] = None, num_units: int = 0,
                min_chunk: int = 0, flags: int = 0, num_heads: int = 16, num_kv_heads: int = 1, qk_dim: int = 576,
                v_dim: int = 512, page_size: int = 1, max_q_len: int = 0, logit_cap: float = 0.0) -> MlaDecodeParams:
    return MlaDecodeParams(
        batch=batch, total_q=batch if total_q is None else total_q, num_heads=num_heads, num_kv_heads=num_kv_heads,
        qk_dim=qk_dim, v_dim=v_dim, page_size=page_size,
        q_dtype=_DTYPES.get(q_dtype, q_dtype) if isinstance(q_dtype, str) else q_dtype,
        kv_dtype=_DTYPES.get(kv_dtype, kv_dtype) if isinstance(kv_dtype, str) else kv_dtype,
        num_units=num_units, min_chunk=min_chunk, flags=flags, max_q_len=max_q_len, logit_cap=logit_cap,
    )


def mla_decode_workspace_size(params: MlaDecodeParams) -> int:
    return int(lib().mla_decode_workspace_size(ctypes.byref(params)))


def mla_decode_plan(params: MlaDecodeParams, workspace: torch.Tensor, stream=None) -> MlaDecodePlan:
    plan = MlaDecodePlan()
    code = lib().mla_decode_plan(ctypes.byref(params), _ptr(workspace), workspace.numel() * workspace.element_size(),
                                 _stream(stream), ctypes.byref(plan))
    _check(code, "mla_decode_plan")
    return plan


def _check_index_args(out, lse_out=None, **ints) -> None:
    for name, t in ints.items():
        if t is not None and t.dtype != torch.int32:
            raise ValueError(f"{name} must be int32")
    if out.dtype != torch.bfloat16:
        raise ValueError("out must be bf16")
    if lse_out is not None and (lse_out.dtype != torch.float32 or lse_out.numel() * 512 < out.numel()):
        raise ValueError("lse_out must be float32 with one value per token and head")


def mla_decode_run(plan: MlaDecodePlan, q: torch.Tensor, kv: torch.Tensor, qo_indptr: torch.Tensor,
                   kv_indptr: torch.Tensor, kv_indices: torch.Tensor, q_scale: Optional[torch.Tensor],
                   kv_scale: Optional[torch.Tensor], sm_scale: float, out: torch.Tensor, stream=None) -> None:
    _check_index_args(out, qo_indptr=qo_indptr, kv_indptr=kv_indptr, kv_indices=kv_indices)
    code = lib().mla_decode_run(ctypes.byref(plan), _ptr(q), _ptr(kv), _ptr(qo_indptr), _ptr(kv_indptr),
                                _ptr(kv_indices), _ptr(q_scale), _ptr(kv_scale), float(sm_scale), _ptr(out),
                                _stream(stream))
    _check(code, "mla_decode_run")


def mla_decode_run_paged(plan: MlaDecodePlan, q: torch.Tensor, kv: torch.Tensor, qo_indptr: torch.Tensor,
                         kv_indptr: torch.Tensor, kv_indices: torch.Tensor, kv_last_page_len: Optional[torch.Tensor],
                         q_scale: Optional[torch.Tensor], kv_scale: Optional[torch.Tensor], sm_scale: float,
                         out: torch.Tensor, lse_out: Optional[torch.Tensor] = None, stream=None) -> None:
    _check_index_args(out, lse_out, qo_indptr=qo_indptr, kv_indptr=kv_indptr, kv_indices=kv_indices,
                      kv_last_page_len=kv_last_page_len)
    code = lib().mla_decode_run_paged(ctypes.byref(plan), _ptr(q), _ptr(kv), _ptr(qo_indptr), _ptr(kv_indptr),
                                      _ptr(kv_indices), _ptr(kv_last_page_len), _ptr(q_scale), _ptr(kv_scale),
                                      float(sm_scale), _ptr(out), _ptr(lse_out), _stream(stream))
    _check(code, "mla_decode_run_paged")


def mla_decode_attend(plan: MlaDecodePlan, q: torch.Tensor, kv: torch.Tensor, qo_indptr: torch.Tensor,
                      kv_indptr: torch.Tensor, kv_indices: torch.Tensor, kv_last_page_len: Optional[torch.Tensor],
                      q_scale: Optional[torch.Tensor], kv_scale: Optional[torch.Tensor], sm_scale: float,
                      out: torch.Tensor, lse_out: Optional[torch.Tensor] = None, stream=None) -> None:
    _check_index_args(out, lse_out, qo_indptr=qo_indptr, kv_indptr=kv_indptr, kv_indices=kv_indices,
                      kv_last_page_len=kv_last_page_len)
    code = lib().mla_decode_attend(ctypes.byref(plan), _ptr(q), _ptr(kv), _ptr(qo_indptr), _ptr(kv_indptr),
                                   _ptr(kv_indices), _ptr(kv_last_page_len), _ptr(q_scale), _ptr(kv_scale),
                                   float(sm_scale), _ptr(out), _ptr(lse_out), _stream(stream))
    _check(code, "mla_decode_attend")


def mla_decode_merge(plan: MlaDecodePlan, qo_indptr: torch.Tensor, kv_indptr: torch.Tensor, out: torch.Tensor,
                     lse_out: Optional[torch.Tensor] = None, stream=None) -> None:
    _check_index_args(out, lse_out, qo_indptr=qo_indptr, kv_indptr=kv_indptr)
    code = lib().mla_decode_merge(ctypes.byref(plan), _ptr(qo_indptr), _ptr(kv_indptr), _ptr(out), _ptr(lse_out),
                                  _stream(stream))
    _check(code, "mla_decode_merge")


def mla_decode_quantize_q(q_bf16: torch.Tensor, q_fp8: torch.Tensor, stream=None) -> None:
    if q_bf16.dtype != torch.bfloat16 or q_fp8.element_size() != 1 or q_fp8.numel() != q_bf16.numel():
        raise ValueError("expected bf16 input and a 1-byte output of the same size")
    code = lib().mla_decode_quantize_q(_ptr(q_bf16), _ptr(q_fp8), q_bf16.numel(), _stream(stream))
    _check(code, "mla_decode_quantize_q")


def mla_decode_quantize_q_dynamic(q_bf16: torch.Tensor, q_fp8: torch.Tensor, q_scale: torch.Tensor,
                                  scratch: torch.Tensor, stream=None) -> None:
    if q_bf16.dtype != torch.bfloat16 or q_fp8.element_size() != 1 or q_fp8.numel() != q_bf16.numel():
        raise ValueError("expected bf16 input and a 1-byte output of the same size")
    if q_scale.dtype != torch.float32 or q_scale.numel() < 1:
        raise ValueError("q_scale must be a float32 tensor of at least one element")
    code = lib().mla_decode_quantize_q_dynamic(_ptr(q_bf16), _ptr(q_fp8), _ptr(q_scale), _ptr(scratch),
                                               scratch.numel() * scratch.element_size(), q_bf16.numel(),
                                               _stream(stream))
    _check(code, "mla_decode_quantize_q_dynamic")


def mla_decode_reduce(part_o: torch.Tensor, part_lse: torch.Tensor, part_indptr: torch.Tensor, out: torch.Tensor,
                      lse_out: Optional[torch.Tensor] = None, stream=None) -> None:
    if part_o.dtype != torch.float32 or part_lse.dtype != torch.float32 or part_indptr.dtype != torch.int32:
        raise ValueError("partials must be float32 and part_indptr int32")
    if lse_out is not None and (lse_out.dtype != torch.float32 or lse_out.numel() * 512 < out.numel()):
        raise ValueError("lse_out must be float32 with one value per sequence and head")
    batch = part_indptr.numel() - 1
    code = lib().mla_decode_reduce(_ptr(part_o), _ptr(part_lse), _ptr(part_indptr), batch, _ptr(out),
                                   _ptr(lse_out), _stream(stream))
    _check(code, "mla_decode_reduce")


def mla_decode_run_noalloc(params: MlaDecodeParams, q: torch.Tensor, kv: torch.Tensor, qo_indptr: torch.Tensor,
                           kv_indptr: torch.Tensor, kv_indices: torch.Tensor, kv_last_page_len: Optional[torch.Tensor],
                           q_scale: Optional[torch.Tensor], kv_scale: Optional[torch.Tensor], sm_scale: float,
                           out: torch.Tensor, lse_out: Optional[torch.Tensor] = None, stream=None) -> None:
    """One decode step with the library's own scratch array as the workspace (no plan, no allocation)."""
    _check_index_args(out, lse_out, qo_indptr=qo_indptr, kv_indptr=kv_indptr, kv_indices=kv_indices,
                      kv_last_page_len=kv_last_page_len)
    code = lib().mla_decode_run_noalloc(ctypes.byref(params), _ptr(q), _ptr(kv), _ptr(qo_indptr), _ptr(kv_indptr),
                                        _ptr(kv_indices), _ptr(kv_last_page_len), _ptr(q_scale), _ptr(kv_scale),
                                        float(sm_scale), _ptr(out), _ptr(lse_out), _stream(stream))
    _check(code, "mla_decode_run_noalloc")


class Decoder:
    """Owns one workspace and plan for a (batch, dtype pair); run() is one decode step."""

    def __init__(self, batch: int, q_dtype: str, kv_dtype: str, device: torch.device | str = "cuda", *,
                 num_units: int = 0, min_chunk: int = 0, flags: int = 0, page_size: int = 1, max_q_len: int = 0,
                 total_q: Optional[int] = None, logit_cap: float = 0.0, stream=None):
        self.params = make_params(batch, q_dtype, kv_dtype, num_units=num_units, min_chunk=min_chunk, flags=flags,
                                  page_size=page_size, max_q_len=max_q_len, total_q=total_q, logit_cap=logit_cap)
        nbytes = mla_decode_workspace_size(self.params)
        if nbytes == 0:
            raise RuntimeError("mla_decode_workspace_size rejected the parameters")
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.plan = mla_decode_plan(self.params, self.workspace, stream)
        self.q_dtype = q_dtype
        self.kv_dtype = kv_dtype

    def run(self, q, kv, qo_indptr, kv_indptr, kv_indices, q_scale, kv_scale, sm_scale, out, stream=None,
            kv_last_page_len=None, lse_out=None):
        if lse_out is not None:
            mla_decode_run_paged(self.plan, q, kv, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, q_scale,
                                 kv_scale, sm_scale, out, lse_out, stream)
        elif kv_last_page_len is None:
            mla_decode_run(self.plan, q, kv, qo_indptr, kv_indptr, kv_indices, q_scale, kv_scale, sm_scale, out,
                           stream)
        else:
            mla_decode_run_paged(self.plan, q, kv, qo_indptr, kv_indptr, kv_indices, kv_last_page_len, q_scale,
                                 kv_scale, sm_scale, out, None, stream)
        return out
