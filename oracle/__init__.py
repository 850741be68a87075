"""CPU oracle for the block-local MHSA sub-layer (ctypes wrapper over gs_oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg are the only users.  The product package never imports this.

Everything here is IEEE double; callers widen bf16/fp32 inputs exactly with
`.double()` / `np.float64` before calling.  Parity is pinned by the tests in
tests/test_oracle_pins.py (closed forms, a library attention routine, a
brute-force masked reference, exact invariances).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gs_oracle.c")
LIB = os.path.join(HERE, "libgs_oracle.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-pthread"]


def build(src: str = SRC, out: str = LIB, extra=()) -> str:
    """Compile the oracle with gcc (plain IEEE double, no FMA contraction)."""
    cmd = ["gcc", *CFLAGS, *extra, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def host_threads() -> int:
    """Threads the oracle runs on by default: the cores this process may use
    (its CPU affinity), or OMP_NUM_THREADS where the machine sets it to the
    share of cores allotted to the job.  The result is the same bits at any
    thread count."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        return int(env)
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # (no affinity call on this platform)
        return os.cpu_count() or 1


_P = ctypes.c_void_p
_I32, _I64 = ctypes.c_int32, ctypes.c_int64


class Oracle:
    """Handle on one compiled copy of the oracle library."""

    def __init__(self, path: str = LIB):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.gso_count_blocks.restype = _I64
        lib.gso_count_blocks.argtypes = [_P, _I32, _I32]
        lib.gso_block_table.restype = ctypes.c_int
        lib.gso_block_table.argtypes = [_P, _I32, _I32, _P, _P]
        lib.gso_qkv_proj.restype = ctypes.c_int
        lib.gso_qkv_proj.argtypes = [_P, _P, _I64, _I32, _P, _P, ctypes.c_int]
        lib.gso_block_attn.restype = ctypes.c_int
        lib.gso_block_attn.argtypes = [_P, _P, _I32, _I32, _I32, _I32, _P, _P, ctypes.c_int]
        lib.gso_out_proj_residual.restype = ctypes.c_int
        lib.gso_out_proj_residual.argtypes = [_P, _P, _P, _I64, _I32, _P, _P, ctypes.c_int]
        lib.gso_block_mhsa.restype = ctypes.c_int
        lib.gso_block_mhsa.argtypes = [_P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, ctypes.c_int]
        self.lib = lib

    # -- helpers ----------------------------------------------------------
    @staticmethod
    def _f64(a) -> np.ndarray:
        if hasattr(a, "detach"):  # torch tensor
            a = a.detach().cpu().double().numpy()
        return np.ascontiguousarray(a, dtype=np.float64)

    @staticmethod
    def _cu(cu) -> np.ndarray:
        if hasattr(cu, "detach"):
            cu = cu.detach().cpu().numpy()
        return np.ascontiguousarray(cu, dtype=np.int32)

    @staticmethod
    def _mask(mask, n: int) -> Optional[np.ndarray]:
        if mask is None:
            return None
        m = np.ascontiguousarray(mask, dtype=np.uint8)
        if m.shape != (n,):
            raise ValueError("row mask must have one entry per row")
        return m

    @staticmethod
    def _ptr(a) -> Optional[int]:
        return None if a is None else a.ctypes.data

    @staticmethod
    def threads(n: Optional[int]) -> int:
        return int(n) if n else host_threads()

    @staticmethod
    def _check(rc: int, what: str):
        if rc != 0:
            raise RuntimeError(f"oracle {what} failed with code {rc}")

    # -- the steps ----------------------------------------------------------
    def count_blocks(self, cu, block_frames: int) -> int:
        cu = self._cu(cu)
        return int(self.lib.gso_count_blocks(cu.ctypes.data, len(cu) - 1, int(block_frames)))

    def block_table(self, cu, block_frames: int):
        cu = self._cu(cu)
        nb = self.count_blocks(cu, block_frames)
        if nb < 0:
            raise ValueError("malformed cu_seqlens")
        st = np.zeros(max(nb, 1), np.int64)
        ln = np.zeros(max(nb, 1), np.int64)
        self._check(self.lib.gso_block_table(cu.ctypes.data, len(cu) - 1, int(block_frames),
                                             st.ctypes.data, ln.ctypes.data), "block_table")
        return st[:nb], ln[:nb]

    def qkv_proj(self, x, wqkv, mask=None, nthreads=None) -> np.ndarray:
        x, w = self._f64(x), self._f64(wqkv)
        n, d = x.shape
        assert w.shape == (3 * d, d)
        m = self._mask(mask, n)
        y = np.zeros((n, 3 * d), np.float64)
        self._check(self.lib.gso_qkv_proj(x.ctypes.data, w.ctypes.data, n, d, self._ptr(m),
                                          y.ctypes.data, self.threads(nthreads)), "qkv_proj")
        return y

    def block_attn(self, qkv, cu, heads: int, block_frames: int, mask=None, nthreads=None):
        qkv, cu = self._f64(qkv), self._cu(cu)
        n, d3 = qkv.shape
        d = d3 // 3
        m = self._mask(mask, n)
        o = np.zeros((n, d), np.float64)
        self._check(self.lib.gso_block_attn(qkv.ctypes.data, cu.ctypes.data, len(cu) - 1, d,
                                            int(heads), int(block_frames), self._ptr(m),
                                            o.ctypes.data, self.threads(nthreads)), "block_attn")
        return o

    def out_proj_residual(self, o, wo, x, mask=None, nthreads=None) -> np.ndarray:
        o, w, x = self._f64(o), self._f64(wo), self._f64(x)
        n, d = x.shape
        m = self._mask(mask, n)
        out = np.zeros((n, d), np.float64)
        self._check(self.lib.gso_out_proj_residual(o.ctypes.data, w.ctypes.data, x.ctypes.data,
                                                   n, d, self._ptr(m), out.ctypes.data,
                                                   self.threads(nthreads)), "out_proj")
        return out

    def block_mhsa(self, x, cu, wqkv, wo, block_frames: int, heads: int, mask=None,
                   nthreads=None) -> np.ndarray:
        """The whole sub-layer.  Rows outside `mask` (if given) come back as NaN."""
        x, cu, w1, w2 = self._f64(x), self._cu(cu), self._f64(wqkv), self._f64(wo)
        n, d = x.shape
        if int(cu[-1]) != n:
            raise ValueError("cu_seqlens[-1] must equal the number of rows")
        m = self._mask(mask, n)
        out = np.full((n, d), np.nan, np.float64)
        self._check(self.lib.gso_block_mhsa(x.ctypes.data, cu.ctypes.data, len(cu) - 1, d,
                                            int(heads), int(block_frames), w1.ctypes.data,
                                            w2.ctypes.data, self._ptr(m), out.ctypes.data,
                                            self.threads(nthreads)), "block_mhsa")
        return out


    def block_mhsa_padded(self, x, lengths, bucket_frames: int, wqkv, wo, block_frames: int,
                          heads: int, mask=None, nthreads=None) -> np.ndarray:
        """The sub-layer on fixed-length padded buckets (the fixed 800-frame
        encoder bucket of the portable INT4 export, README "What Changed"
        item 4; the treatment of padding is a reading: padding rows are
        neither queries nor keys, and their output is x).

        x is [S*T, d] (or [S, T, d]); the first lengths[b] rows of bucket b
        (clamped to [0, T]) are sequence b.  By that definition the valid rows,
        taken bucket by bucket, are a packed batch whose offsets are the prefix
        sums of the lengths: they are computed as such, and padding rows copy
        x.  Rows outside `mask` (if given) among the valid ones come back as
        NaN; padding rows always hold x."""
        x = self._f64(x)
        t = int(bucket_frames)
        x = x.reshape(-1, x.shape[-1])
        n, d = x.shape
        lengths = np.asarray(lengths, np.int64)
        if t < 1 or n != len(lengths) * t:
            raise ValueError("x must hold len(lengths) buckets of bucket_frames rows")
        ln = np.clip(lengths, 0, t)
        idx = np.concatenate([b * t + np.arange(ln[b]) for b in range(len(ln))] +
                             [np.zeros(0, np.int64)]).astype(np.int64)
        out = x.copy()
        if idx.size:
            cu = np.zeros(len(ln) + 1, np.int32)
            cu[1:] = np.cumsum(ln)
            m = None if mask is None else np.asarray(mask, np.uint8).reshape(-1)[idx]
            out[idx] = self.block_mhsa(np.ascontiguousarray(x[idx]), cu, wqkv, wo, block_frames,
                                       heads, mask=m, nthreads=nthreads)
        return out


_default: Optional[Oracle] = None


def load() -> Oracle:
    """The default oracle; compiled on first use if the library is missing."""
    global _default
    if _default is None:
        if not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
            build()
        _default = Oracle(LIB)
    return _default
