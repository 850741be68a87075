"""Python binding of libgsattn (ctypes).  Argument marshalling only.

Every step of the sub-layer runs in the library's HIP kernels; PyTorch only
provides device memory and the current stream.  The names follow the C ABI in
include/gsattn.h.  If the library is missing the calls raise: there is no
fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("GSATTN_LIB", os.path.join(HERE, "libgsattn.so"))

GS_OK, GS_ERR_INVALID_ARGUMENT, GS_ERR_UNSUPPORTED, GS_ERR_WORKSPACE_TOO_SMALL, GS_ERR_HIP = range(5)
GS_F32, GS_BF16 = 0, 1

EXPORTS = (
    "gs_block_mhsa_workspace_bytes", "gs_block_mhsa_fwd", "gs_block_mhsa_fwd_padded",
    "gs_block_mhsa_fwd_noalloc",
    "gs_block_mhsa_padded_workspace_bytes",
    "gs_qkv_proj", "gs_block_attn",
    "gs_block_attn_workspace_bytes", "gs_out_proj_residual", "gs_status_string",
    "gs_last_error_detail", "gs_version", "gs_window_xattn_workspace_bytes",
    "gs_window_xattn_fwd", "gs_bpe_ctc_workspace_bytes", "gs_bpe_pool_ctc_greedy",
)


class GsError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__(f"{name}: {detail}")
        self.status = status
        self.name = name
        self.detail = detail


class _Desc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_frames", ctypes.c_int64),
        ("d_model", ctypes.c_int32),
        ("dtype", ctypes.c_int),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("kernel_events", ctypes.c_void_p),
        ("flags", ctypes.c_uint32),
    ]


GS_FWD_REUSE_UNIT_TABLE = 1


class _XattnDesc(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_frames", ctypes.c_int64),
        ("feat_dim", ctypes.c_int32),
        ("d_q", ctypes.c_int32),
        ("num_windows", ctypes.c_int32),
        ("queries", ctypes.c_int32),
        ("dtype", ctypes.c_int),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
        ("kernel_events", ctypes.c_void_p),
    ]


_lib = None


def load(path: Optional[str] = None):
    """The loaded library (raises OSError if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise OSError(f"libgsattn not built: {p} is missing (run __graft_entry__.build())")
    lib = ctypes.CDLL(p)
    P, I32, I64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.gs_block_mhsa_workspace_bytes.restype = ctypes.c_size_t
    lib.gs_block_mhsa_workspace_bytes.argtypes = [I64, I32, ctypes.c_int]
    lib.gs_block_mhsa_fwd.restype = ctypes.c_int
    lib.gs_block_mhsa_fwd.argtypes = [P, P, P, P, I32, I32, P, P, ctypes.POINTER(_Desc)]
    lib.gs_block_mhsa_fwd_noalloc.restype = ctypes.c_int
    lib.gs_block_mhsa_fwd_noalloc.argtypes = [P, P, P, P, I32, I32, P, P, I32, I64, I32,
                                              ctypes.c_int]
    lib.gs_block_mhsa_padded_workspace_bytes.restype = ctypes.c_size_t
    lib.gs_block_mhsa_padded_workspace_bytes.argtypes = [I32, I32, I32, ctypes.c_int]
    lib.gs_block_mhsa_fwd_padded.restype = ctypes.c_int
    lib.gs_block_mhsa_fwd_padded.argtypes = [P, P, I32, P, P, I32, I32, P, P,
                                             ctypes.POINTER(_Desc)]
    lib.gs_window_xattn_workspace_bytes.restype = ctypes.c_size_t
    lib.gs_window_xattn_workspace_bytes.argtypes = [I64, I32, I32, I32]
    lib.gs_window_xattn_fwd.restype = ctypes.c_int
    lib.gs_window_xattn_fwd.argtypes = [P, P, P, P, P, P, I32, I32, P, P,
                                        ctypes.POINTER(_XattnDesc)]
    lib.gs_bpe_ctc_workspace_bytes.restype = ctypes.c_size_t
    lib.gs_bpe_ctc_workspace_bytes.argtypes = [I32, I32]
    lib.gs_bpe_pool_ctc_greedy.restype = ctypes.c_int
    lib.gs_bpe_pool_ctc_greedy.argtypes = [P, I64, P, P, I32, I64, I32, I32, I32, I32, P, P, P, P,
                                           ctypes.c_size_t, P]
    lib.gs_qkv_proj.restype = ctypes.c_int
    lib.gs_qkv_proj.argtypes = [P, P, P, I64, I32, ctypes.c_int, P]
    lib.gs_block_attn.restype = ctypes.c_int
    lib.gs_block_attn.argtypes = [P, P, I32, I64, I32, I32, I32, ctypes.c_int, P, P, ctypes.c_size_t, P]
    lib.gs_block_attn_workspace_bytes.restype = ctypes.c_size_t
    lib.gs_block_attn_workspace_bytes.argtypes = [I64]
    lib.gs_out_proj_residual.restype = ctypes.c_int
    lib.gs_out_proj_residual.argtypes = [P, P, P, P, I64, I32, ctypes.c_int, P]
    lib.gs_status_string.restype = ctypes.c_char_p
    lib.gs_status_string.argtypes = [ctypes.c_int]
    lib.gs_last_error_detail.restype = ctypes.c_char_p
    lib.gs_last_error_detail.argtypes = []
    lib.gs_version.restype = ctypes.c_int32
    lib.gs_version.argtypes = []
    if path is None:
        _lib = lib
    return lib


def _check(status: int):
    if status != GS_OK:
        lib = load()
        raise GsError(status, lib.gs_status_string(status).decode(),
                      lib.gs_last_error_detail().decode())


def _gs_dtype(t: torch.dtype) -> int:
    if t == torch.bfloat16:
        return GS_BF16
    if t == torch.float32:
        return GS_F32
    raise TypeError(f"unsupported dtype {t}")


def _dev(t: torch.Tensor, name: str, dtype: Optional[torch.dtype] = None) -> int:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


def workspace_bytes(total_frames: int, d_model: int, dtype: torch.dtype) -> int:
    return int(load().gs_block_mhsa_workspace_bytes(int(total_frames), int(d_model), _gs_dtype(dtype)))


def alloc_workspace(total_frames: int, d_model: int, dtype: torch.dtype, device=None) -> torch.Tensor:
    n = workspace_bytes(total_frames, d_model, dtype)
    return torch.empty(max(n, 256), dtype=torch.uint8, device=device or "cuda")


def block_mhsa_fwd(x: torch.Tensor, cu_seqlens: torch.Tensor, wqkv: torch.Tensor, wo: torch.Tensor,
                   block_frames: int, heads: int, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None, stream=None,
                   kernel_events: Optional["HipEvents"] = None,
                   reuse_unit_table: bool = False) -> torch.Tensor:
    """out = x + BlockMHSA(x), enqueued on `stream` (default: torch's current stream).
    reuse_unit_table: the workspace holds the attention work-unit table of an
    earlier call with the same cu_seqlens, sizes and block length (e.g. the
    previous layer of a stack), which is then not rebuilt."""
    lib = load()
    n, d = x.shape
    dt = _gs_dtype(x.dtype)
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = alloc_workspace(n, d, x.dtype, x.device)
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    desc = _Desc(int(cu_seqlens.numel()) - 1, int(n), int(d), dt, workspace.data_ptr(),
                 int(workspace.numel()), kernel_events.handle_array() if kernel_events else None,
                 GS_FWD_REUSE_UNIT_TABLE if reuse_unit_table else 0)
    _check(lib.gs_block_mhsa_fwd(
        _dev(x, "x"), _dev(cu_seqlens, "cu_seqlens"), _dev(wqkv, "Wqkv", x.dtype),
        _dev(wo, "Wo", x.dtype), int(block_frames), int(heads), _dev(out, "out", x.dtype),
        _stream(stream), ctypes.byref(desc)))
    return out


NOALLOC_SCRATCH_BYTES = 64 << 20  # GS_NOALLOC_SCRATCH_BYTES


def block_mhsa_fwd_noalloc(x: torch.Tensor, cu_seqlens: torch.Tensor, wqkv: torch.Tensor,
                           wo: torch.Tensor, block_frames: int, heads: int,
                           out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """block_mhsa_fwd with the library's static per-GPU scratch as its
    workspace (no device allocation by the library; `out` is allocated here
    only if not given)."""
    lib = load()
    n, d = x.shape
    if out is None:
        out = torch.empty_like(x)
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    _check(lib.gs_block_mhsa_fwd_noalloc(
        _dev(x, "x"), _dev(cu_seqlens, "cu_seqlens"), _dev(wqkv, "Wqkv", x.dtype),
        _dev(wo, "Wo", x.dtype), int(block_frames), int(heads), _dev(out, "out", x.dtype),
        _stream(stream), int(cu_seqlens.numel()) - 1, int(n), int(d), _gs_dtype(x.dtype)))
    return out


def block_mhsa_fwd_padded(x: torch.Tensor, lengths: torch.Tensor, wqkv: torch.Tensor,
                          wo: torch.Tensor, block_frames: int, heads: int,
                          out: Optional[torch.Tensor] = None,
                          workspace: Optional[torch.Tensor] = None, stream=None,
                          kernel_events: Optional["HipEvents"] = None) -> torch.Tensor:
    """The sub-layer on padded buckets: x [S, T, d], lengths int32 [S] (valid
    rows per bucket).  Padding rows come back equal to x."""
    lib = load()
    if x.dim() != 3:
        raise ValueError("x must be [buckets, bucket_frames, d_model]")
    s, t, d = x.shape
    dt = _gs_dtype(x.dtype)
    if out is None:
        out = torch.empty_like(x)
    if workspace is None:
        workspace = torch.empty(max(lib.gs_block_mhsa_padded_workspace_bytes(s, t, d, dt), 1),
                                dtype=torch.uint8, device=x.device)
    if lengths.dtype != torch.int32 or lengths.numel() != s:
        raise TypeError("lengths must be int32 with one entry per bucket")
    desc = _Desc(int(s), int(s * t), int(d), dt, workspace.data_ptr(), int(workspace.numel()),
                 kernel_events.handle_array() if kernel_events else None)
    _check(lib.gs_block_mhsa_fwd_padded(
        _dev(x, "x"), _dev(lengths, "lengths"), int(t), _dev(wqkv, "Wqkv", x.dtype),
        _dev(wo, "Wo", x.dtype), int(block_frames), int(heads), _dev(out, "out", x.dtype),
        _stream(stream), ctypes.byref(desc)))
    return out


def window_xattn_fwd(hcat: torch.Tensor, cu_seqlens: torch.Tensor, xq: torch.Tensor,
                     wq: torch.Tensor, wkv: torch.Tensor, wo: torch.Tensor, window_frames: int,
                     heads: int, out: Optional[torch.Tensor] = None,
                     workspace: Optional[torch.Tensor] = None, stream=None,
                     kernel_events: Optional["HipEvents"] = None) -> torch.Tensor:
    """Window cross-attention: hcat [N, F], xq [W, nq, dq] -> out [W, nq, dq]."""
    lib = load()
    n, f = hcat.shape
    nw, nq, dq = xq.shape
    dt = _gs_dtype(xq.dtype)
    if out is None:
        out = torch.empty_like(xq)
    if workspace is None:
        nb = lib.gs_window_xattn_workspace_bytes(n, dq, nw, nq)
        workspace = torch.empty(max(nb, 1), dtype=torch.uint8, device=xq.device)
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    desc = _XattnDesc(int(cu_seqlens.numel()) - 1, int(n), int(f), int(dq), int(nw), int(nq), dt,
                      workspace.data_ptr(), int(workspace.numel()),
                      kernel_events.handle_array() if kernel_events else None)
    _check(lib.gs_window_xattn_fwd(
        _dev(hcat, "hcat", xq.dtype), _dev(cu_seqlens, "cu_seqlens"), _dev(xq, "xq"),
        _dev(wq, "Wq", xq.dtype), _dev(wkv, "Wkv", xq.dtype), _dev(wo, "Wo", xq.dtype),
        int(window_frames), int(heads), _dev(out, "out", xq.dtype), _stream(stream),
        ctypes.byref(desc)))
    return out


def bpe_pool_ctc_greedy(logits: torch.Tensor, blank_prob: torch.Tensor, cu_seqlens: torch.Tensor,
                        num_classes: int, num_positions: int, window: int = 4, stride: int = 2,
                        workspace=None, stream=None, out=None):
    """Pooled argmax and CTC greedy tokens.  logits [N, ld] bf16 (the first
    num_classes columns are the classes), blank_prob [N] fp32, num_positions
    the pooled positions of all sequences (sum of ceil(len / stride), or
    more).  Returns (argmax [P], tokens [P], token_counts [S]) int32 device
    tensors; sequence s's tokens start at its first position (the prefix sum
    of the position counts)."""
    lib = load()
    n, ld = logits.shape
    s = int(cu_seqlens.numel()) - 1
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    num_positions = int(num_positions)
    dev = logits.device
    if out is None:
        out = (torch.empty(max(num_positions, 1), dtype=torch.int32, device=dev),
               torch.empty(max(num_positions, 1), dtype=torch.int32, device=dev),
               torch.empty(max(s, 1), dtype=torch.int32, device=dev))
    am, tok, cnt = out
    if workspace is None:
        workspace = torch.empty(lib.gs_bpe_ctc_workspace_bytes(s, num_positions),
                                dtype=torch.uint8, device=dev)
    _check(lib.gs_bpe_pool_ctc_greedy(
        _dev(logits, "logits", torch.bfloat16), int(ld), _dev(blank_prob, "blank_prob", torch.float32),
        _dev(cu_seqlens, "cu_seqlens"), s, int(n), int(num_classes), int(window), int(stride),
        int(num_positions), _dev(am, "argmax", torch.int32), _dev(tok, "tokens", torch.int32),
        _dev(cnt, "token_counts", torch.int32), workspace.data_ptr(), int(workspace.numel()),
        _stream(stream)))
    return am[:num_positions], tok[:num_positions], cnt[:s]


def qkv_proj(x: torch.Tensor, wqkv: torch.Tensor, qkv: Optional[torch.Tensor] = None, stream=None):
    n, d = x.shape
    if qkv is None:
        qkv = torch.empty((n, 3 * d), dtype=x.dtype, device=x.device)
    _check(load().gs_qkv_proj(_dev(x, "x"), _dev(wqkv, "Wqkv", x.dtype), _dev(qkv, "qkv", x.dtype),
                              int(n), int(d), _gs_dtype(x.dtype), _stream(stream)))
    return qkv


def block_attn(qkv: torch.Tensor, cu_seqlens: torch.Tensor, heads: int, block_frames: int,
               o: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
               stream=None):
    lib = load()
    n, d3 = qkv.shape
    d = d3 // 3
    if o is None:
        o = torch.empty((n, d), dtype=qkv.dtype, device=qkv.device)
    if workspace is None:
        nb = int(lib.gs_block_attn_workspace_bytes(int(n)))
        workspace = torch.empty(max(nb, 256), dtype=torch.uint8, device=qkv.device)
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    _check(lib.gs_block_attn(_dev(qkv, "qkv"), _dev(cu_seqlens, "cu_seqlens"),
                             int(cu_seqlens.numel()) - 1, int(n), int(d), int(heads),
                             int(block_frames), _gs_dtype(qkv.dtype), _dev(o, "o", qkv.dtype),
                             _dev(workspace, "workspace"), int(workspace.numel()), _stream(stream)))
    return o


def out_proj_residual(o: torch.Tensor, wo: torch.Tensor, x: torch.Tensor,
                      out: Optional[torch.Tensor] = None, stream=None):
    n, d = x.shape
    if out is None:
        out = torch.empty_like(x)
    _check(load().gs_out_proj_residual(_dev(o, "o", x.dtype), _dev(wo, "Wo", x.dtype), _dev(x, "x"),
                                       _dev(out, "out", x.dtype), int(n), int(d),
                                       _gs_dtype(x.dtype), _stream(stream)))
    return out


class HipEvents:
    """A few raw hipEvent_t handles (for the library's per-kernel timing hook)."""

    def __init__(self, count: int = 4):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self._hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self._hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                  ctypes.c_void_p]
        self._hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self._hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self._arr = (ctypes.c_void_p * count)()
        for i in range(count):
            h = ctypes.c_void_p()
            if self._hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self._arr[i] = h
        self.count = count

    def handle_array(self, offset: int = 0) -> int:
        """Address of the hipEvent_t array starting at event `offset`."""
        if not 0 <= offset < self.count:
            raise IndexError(offset)
        return ctypes.addressof(self._arr) + offset * ctypes.sizeof(ctypes.c_void_p)

    def view(self, offset: int) -> "_EventView":
        """The events offset..offset+3, as the library's four timing events."""
        if offset + 4 > self.count:
            raise IndexError(offset)
        return _EventView(self, offset)

    def record(self, i: int, stream=None) -> None:
        """Record event i on `stream` (a torch stream, a raw handle, or None
        for the null stream)."""
        h = getattr(stream, "cuda_stream", stream) or 0
        if self._hip.hipEventRecord(self._arr[i], ctypes.c_void_p(int(h))) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_ms(self, i: int, j: int) -> float:
        """Milliseconds between events i and j (waits for j)."""
        if self._hip.hipEventSynchronize(self._arr[j]) != 0:
            raise RuntimeError("hipEventSynchronize failed")
        ms = ctypes.c_float()
        if self._hip.hipEventElapsedTime(ctypes.byref(ms), self._arr[i], self._arr[j]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def __del__(self):
        try:
            for i in range(self.count):
                self._hip.hipEventDestroy(self._arr[i])
        except Exception:
            pass


class _EventView:
    def __init__(self, events: HipEvents, offset: int):
        self.events, self.offset = events, offset

    def handle_array(self) -> int:
        return self.events.handle_array(self.offset)
