"""The C-ABI library loads and exports what include/gsattn.h declares; host-side
checks reject bad arguments before any device work (CPU only)."""
import ctypes
import os
import re

import pytest

from conformer_block_attention_amd import gsattn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gsattn.h")

FAKE = 0x10000  # a non-null, 256-byte aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gs_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return gsattn.load()


def test_exports_every_declared_function(lib):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(gsattn.EXPORTS) == names


def test_version_and_status_strings(lib):
    assert lib.gs_version() >= 10000
    for code, name in enumerate(["GS_OK", "GS_ERR_INVALID_ARGUMENT", "GS_ERR_UNSUPPORTED",
                                 "GS_ERR_WORKSPACE_TOO_SMALL", "GS_ERR_HIP"]):
        assert lib.gs_status_string(code).decode() == name


def test_workspace_bytes(lib):
    n, d = 1000, 1024
    al = lambda v: (v + 255) // 256 * 256  # noqa: E731
    # unit table (16 B per unit) and a flag word per unit, units <= n + 1
    attn = al(16 * (n + 1)) + al(8 * (n + 1))
    assert lib.gs_block_attn_workspace_bytes(n) == attn
    for dt, e in ((gsattn.GS_BF16, 2), (gsattn.GS_F32, 4)):
        got = lib.gs_block_mhsa_workspace_bytes(n, d, dt)
        assert got == al(n * 3 * d * e) + al(n * d * e) + attn + 256
    assert lib.gs_block_mhsa_workspace_bytes(-1, d, gsattn.GS_BF16) == 0
    assert lib.gs_block_mhsa_workspace_bytes(n, d, 7) == 0


def _desc(S=2, N=400, d=1024, dt=gsattn.GS_BF16, ws=FAKE, wsb=1 << 40):
    return gsattn._Desc(S, N, d, dt, ws, wsb, None)


def _fwd(lib, desc, x=FAKE, cu=FAKE, wqkv=FAKE, wo=FAKE, B=200, H=8, out=FAKE + (1 << 30)):
    d = ctypes.byref(desc) if desc is not None else None
    st = lib.gs_block_mhsa_fwd(x, cu, wqkv, wo, B, H, out, None, d)
    return st, lib.gs_last_error_detail().decode()


@pytest.mark.parametrize("kw,desc_kw,code", [
    ({}, None, gsattn.GS_ERR_INVALID_ARGUMENT),                       # desc NULL
    ({"x": None}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({"cu": None}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({"wqkv": None}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({"wo": None}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({"out": None}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({"x": FAKE + 2}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),            # misaligned
    ({"B": 0}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({"H": 0}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({"H": 3}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),                   # 1024 % 3
    ({"H": 16}, {}, gsattn.GS_ERR_UNSUPPORTED),                       # dh = 64
    ({}, {"S": 0}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({}, {"N": -5}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({}, {"d": 1000}, gsattn.GS_ERR_UNSUPPORTED),
    ({}, {"dt": 9}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({}, {"ws": None}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({}, {"ws": FAKE + 16}, gsattn.GS_ERR_INVALID_ARGUMENT),          # workspace alignment
    ({}, {"wsb": 1000}, gsattn.GS_ERR_WORKSPACE_TOO_SMALL),
    ({"out": FAKE + 4096}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),       # partial overlap with x
])
def test_argument_errors(lib, kw, desc_kw, code):
    desc = None if desc_kw is None else _desc(**desc_kw)
    st, detail = _fwd(lib, desc, **kw)
    assert st == code, (st, detail)
    assert detail


def test_unknown_desc_flags_are_rejected(lib):
    desc = _desc()
    desc.flags = 0x4
    st, detail = _fwd(lib, desc)
    assert st == gsattn.GS_ERR_INVALID_ARGUMENT and "flags" in detail


def test_empty_input_is_noop(lib):
    # N = 0 returns before touching any pointer or the device
    st, _ = _fwd(lib, _desc(N=0, ws=None, wsb=0), x=None, wqkv=None, wo=None, out=None)
    assert st == gsattn.GS_OK


def test_stage_argument_errors(lib):
    assert lib.gs_qkv_proj(None, FAKE, FAKE, 10, 1024, gsattn.GS_BF16, None) == gsattn.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_qkv_proj(FAKE, FAKE, FAKE, 10, 96, gsattn.GS_BF16, None) == gsattn.GS_ERR_UNSUPPORTED
    W, WB = FAKE * 16, 1 << 20
    assert lib.gs_block_attn(FAKE, FAKE, 0, 10, 1024, 8, 200, gsattn.GS_BF16, FAKE, W, WB, None) == gsattn.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_block_attn(FAKE, None, 1, 10, 1024, 8, 200, gsattn.GS_BF16, FAKE, W, WB, None) == gsattn.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_block_attn(FAKE, FAKE, 1, 10, 1024, 8, 0, gsattn.GS_BF16, FAKE, W, WB, None) == gsattn.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_block_attn(FAKE, FAKE, 1, 10, 1024, 8, 200, gsattn.GS_BF16, FAKE, None, WB, None) == gsattn.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_block_attn(FAKE, FAKE, 1, 10, 1024, 8, 200, gsattn.GS_BF16, FAKE, W + 8, WB, None) == gsattn.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_block_attn(FAKE, FAKE, 1, 10, 1024, 8, 200, gsattn.GS_BF16, FAKE, W, 16, None) == gsattn.GS_ERR_WORKSPACE_TOO_SMALL
    assert lib.gs_out_proj_residual(FAKE, FAKE, None, FAKE, 10, 1024, gsattn.GS_F32, None) == gsattn.GS_ERR_INVALID_ARGUMENT
    assert lib.gs_qkv_proj(FAKE, FAKE, FAKE, 1 << 31, 1024, gsattn.GS_BF16, None) == gsattn.GS_ERR_UNSUPPORTED


def test_noalloc_refusals_before_any_device_work(lib):
    """Checks of gs_block_mhsa_fwd_noalloc that need no GPU: a workspace past
    the static scratch, bad dtype or sizes."""
    def call(N=400, d=1024, dt=gsattn.GS_BF16, S=2):
        return lib.gs_block_mhsa_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, 200, 8, FAKE + (1 << 30),
                                             None, S, N, d, dt)
    assert call(N=8169) == gsattn.GS_ERR_UNSUPPORTED
    assert "static scratch" in lib.gs_last_error_detail().decode()
    assert call(N=4090, dt=gsattn.GS_F32) == gsattn.GS_ERR_UNSUPPORTED
    assert call(dt=9) == gsattn.GS_ERR_INVALID_ARGUMENT
    assert call(N=-1) == gsattn.GS_ERR_INVALID_ARGUMENT
    assert call(d=1000) == gsattn.GS_ERR_UNSUPPORTED


def _fwd_padded(lib, desc, x=FAKE, lengths=FAKE, T=200, wqkv=FAKE, wo=FAKE, B=200, H=8,
                out=FAKE + (1 << 30)):
    d = ctypes.byref(desc) if desc is not None else None
    st = lib.gs_block_mhsa_fwd_padded(x, lengths, T, wqkv, wo, B, H, out, None, d)
    return st, lib.gs_last_error_detail().decode()


@pytest.mark.parametrize("kw,desc_kw,code", [
    ({}, None, gsattn.GS_ERR_INVALID_ARGUMENT),                       # desc NULL
    ({"lengths": None}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({"T": 0}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({"T": 300}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),                 # S * T != N
    ({"x": None}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({"out": FAKE + 4096}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),       # partial overlap with x
    ({"H": 16}, {}, gsattn.GS_ERR_UNSUPPORTED),
    ({"B": 0}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({}, {"S": 0}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({}, {"wsb": 1000}, gsattn.GS_ERR_WORKSPACE_TOO_SMALL),
])
def test_padded_argument_errors(lib, kw, desc_kw, code):
    desc = None if desc_kw is None else _desc(**desc_kw)
    st, detail = _fwd_padded(lib, desc, **kw)
    assert st == code, (st, detail)
    assert detail


def test_padded_zero_rows_is_rejected(lib):
    # S >= 1 buckets of T >= 1 rows never hold 0 rows: total_frames = 0 is a mismatch
    st, detail = _fwd_padded(lib, _desc(S=1, N=0, ws=None, wsb=0), x=None, T=1, wqkv=None,
                             wo=None, out=None)
    assert st == gsattn.GS_ERR_INVALID_ARGUMENT and "bucket_frames" in detail


def _xdesc(S=2, N=400, F=4096, dq=2048, W=30, nq=3, dt=gsattn.GS_BF16, ws=FAKE, wsb=1 << 40):
    return gsattn._XattnDesc(S, N, F, dq, W, nq, dt, ws, wsb, None)


def _xfwd(lib, desc, hcat=FAKE, cu=FAKE, xq=FAKE, wq=FAKE, wkv=FAKE, wo=FAKE, win=15, H=16,
          out=FAKE + (1 << 30)):
    d = ctypes.byref(desc) if desc is not None else None
    st = lib.gs_window_xattn_fwd(hcat, cu, xq, wq, wkv, wo, win, H, out, None, d)
    return st, lib.gs_last_error_detail().decode()


@pytest.mark.parametrize("kw,desc_kw,code", [
    ({}, None, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({}, {"dt": gsattn.GS_F32}, gsattn.GS_ERR_UNSUPPORTED),
    ({"cu": None}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({"xq": None}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({"wkv": FAKE + 8}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({"hcat": None}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({"win": 0}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({"H": 3}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),            # 2048 % 3
    ({"H": 32}, {}, gsattn.GS_ERR_UNSUPPORTED),                # dh = 64
    ({}, {"nq": 5}, gsattn.GS_ERR_UNSUPPORTED),
    ({}, {"dq": 128 * 3, "S": 2}, gsattn.GS_ERR_UNSUPPORTED),  # dq % 256
    ({"H": 3}, {"dq": 384}, gsattn.GS_ERR_UNSUPPORTED),
    ({}, {"F": 100}, gsattn.GS_ERR_UNSUPPORTED),
    ({}, {"W": -1}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({}, {"S": 0}, gsattn.GS_ERR_INVALID_ARGUMENT),
    ({}, {"wsb": 4096}, gsattn.GS_ERR_WORKSPACE_TOO_SMALL),
    ({"out": FAKE + 4096}, {}, gsattn.GS_ERR_INVALID_ARGUMENT),  # partial overlap with xq
])
def test_window_xattn_argument_errors(lib, kw, desc_kw, code):
    desc = None if desc_kw is None else _xdesc(**desc_kw)
    st, detail = _xfwd(lib, desc, **kw)
    assert st == code, (st, detail)
    assert detail


def test_window_xattn_no_windows_is_noop(lib):
    st, _ = _xfwd(lib, _xdesc(N=0, W=0, ws=None, wsb=0), hcat=None, xq=None, wq=None, wkv=None,
                  wo=None, out=None)
    assert st == gsattn.GS_OK


def test_window_xattn_workspace_bytes(lib):
    al = lambda v: (v + 255) // 256 * 256  # noqa: E731
    n, dq, w, nq = 1000, 2048, 70, 3
    assert lib.gs_window_xattn_workspace_bytes(n, dq, w, nq) == (
        al(n * 2 * dq * 2) + 2 * al(w * nq * dq * 2) + al(8 * w + 4) + 256)
    assert lib.gs_window_xattn_workspace_bytes(-1, dq, w, nq) == 0
