"""The C-ABI boundary on the CPU: the library loads, exports every symbol that
include/swa.h declares, and rejects bad arguments with the documented status
codes before any HIP call (so no GPU is touched).  The Python binding rejects
bad tensors before reaching the library."""

import ctypes
import os
import re
import subprocess

import pytest
import torch

import sliding_window_causal_amd as swa
from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "swa.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_entry_points():
    names = _declared_functions()
    for n in ("swa_forward", "swa_decode", "swa_ring_append", "swa_status_string",
              "swa_abi_version", "swa_chunk_forward", "swa_ring_append_chunk",
              "swa_forward_strided", "swa_decode_workspace_bytes", "swa_decode_split",
              "swa_decode_append", "swa_mha_forward", "swa_mha_workspace_bytes",
              "swa_backward", "swa_backward_workspace_bytes", "swa_forward_lse",
              "swa_chunk_forward_split", "swa_chunk_workspace_bytes"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = swa.lib()
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_exported_symbols_are_c_linkage():
    out = os.popen(f"nm -D --defined-only {swa.LIB_PATH}").read()
    exported = set(re.findall(r"\b(swa_[a-z_0-9]+)\b", out))
    assert set(_declared_functions()) <= exported


def test_abi_version_and_status_strings():
    assert swa.abi_version() == 2
    for code in (swa.SWA_OK, swa.SWA_ERR_INVALID_ARG, swa.SWA_ERR_UNSUPPORTED,
                 swa.SWA_ERR_LAUNCH, swa.SWA_ERR_SCRATCH_LIMIT, 99):
        s = swa.status_string(code)
        assert isinstance(s, str) and s


DUMMY = ctypes.c_void_p(0x1000)   # never dereferenced: every case below fails validation


def _fwd(q=DUMMY, k=DUMMY, v=DUMMY, o=DUMMY, B=1, H=1, T=8, D=64, W=4, dt=swa.SWA_BF16):
    return swa.lib().swa_forward(q, k, v, o, B, H, T, D, W, dt, None)


def _dec(q=DUMMY, kr=DUMMY, vr=DUMMY, pos=DUMMY, o=DUMMY, S=1, H=1, D=64, W=4, dt=swa.SWA_BF16):
    return swa.lib().swa_decode(q, kr, vr, pos, o, S, H, D, W, dt, None)


def _app(kn=DUMMY, vn=DUMMY, kr=DUMMY, vr=DUMMY, pos=DUMMY, S=1, H=1, D=64, W=4, dt=swa.SWA_BF16):
    return swa.lib().swa_ring_append(kn, vn, kr, vr, pos, S, H, D, W, dt, None)


@pytest.mark.parametrize("kw", [dict(q=None), dict(k=None), dict(v=None), dict(o=None),
                                dict(B=0), dict(H=0), dict(T=0), dict(D=0), dict(W=0),
                                dict(W=-3), dict(T=-1)])
def test_forward_invalid_args(kw):
    assert _fwd(**kw) == swa.SWA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(dt=7), dict(dt=-1), dict(D=96), dict(D=256),
                                dict(D=32), dict(dt=swa.SWA_F32, D=257)])
def test_forward_unsupported(kw):
    assert _fwd(**kw) == swa.SWA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(q=None), dict(kr=None), dict(vr=None), dict(pos=None),
                                dict(o=None), dict(S=0), dict(H=0), dict(D=0), dict(W=0)])
def test_decode_invalid_args(kw):
    assert _dec(**kw) == swa.SWA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(dt=3), dict(D=80), dict(dt=swa.SWA_F32, D=300)])
def test_decode_unsupported(kw):
    assert _dec(**kw) == swa.SWA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(kn=None), dict(vn=None), dict(kr=None), dict(vr=None),
                                dict(pos=None), dict(S=0), dict(W=0), dict(D=0)])
def test_append_invalid_args(kw):
    assert _app(**kw) == swa.SWA_ERR_INVALID_ARG


def test_append_unsupported_dtype():
    assert _app(dt=5) == swa.SWA_ERR_UNSUPPORTED


CONTIG = (ctypes.c_int64 * 12)(*([4 * 8 * 64, 8 * 64, 64] * 4))


def _fwds(q=DUMMY, k=DUMMY, v=DUMMY, o=DUMMY, B=1, H=4, T=8, D=64, W=4, st=CONTIG, scale=0.0,
          dt=swa.SWA_BF16):
    return swa.lib().swa_forward_strided(q, k, v, o, B, H, T, D, W, st, scale, dt, None)


def _neg_stride(i):
    a = list(CONTIG)
    a[i] = -1
    return (ctypes.c_int64 * 12)(*a)


@pytest.mark.parametrize("kw", [dict(q=None), dict(o=None), dict(st=None), dict(B=0), dict(T=0),
                                dict(W=0), dict(scale=float("nan")), dict(scale=float("inf")),
                                dict(scale=-float("inf")), dict(st=_neg_stride(0)),
                                dict(st=_neg_stride(5)), dict(st=_neg_stride(11))])
def test_forward_strided_invalid_args(kw):
    assert _fwds(**kw) == swa.SWA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(dt=5), dict(D=96), dict(D=32), dict(dt=swa.SWA_F32, D=257)])
def test_forward_strided_unsupported(kw):
    assert _fwds(**kw) == swa.SWA_ERR_UNSUPPORTED


@pytest.mark.parametrize("scale,exc", [(0, ValueError), (float("nan"), ValueError),
                                       (float("inf"), ValueError), ("0.1", TypeError),
                                       (True, TypeError)])
def test_binding_rejects_bad_scale(scale, exc, monkeypatch):
    # device checks are bypassed so that the scale check itself is reached
    monkeypatch.setattr(swa, "_check_device", lambda *a, **k: None)
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(exc):
        swa.swa_forward_strided(x, x, x, x.clone(), 4, scale=scale)


def test_binding_rejects_bad_layout():
    x = torch.zeros(1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        swa.sliding_window_attention(x, x, x, 4, layout="tbd")
    with pytest.raises(ValueError):
        swa.sliding_window_attention(x, x, x, 4, layout="bshd")


def _dsplit(ws=DUMMY, nb=1 << 30, S=1, H=4, D=128, W=4096, dt=swa.SWA_BF16, q=DUMMY):
    return swa.lib().swa_decode_split(q, DUMMY, DUMMY, DUMMY, DUMMY, S, H, D, W, dt, ws, nb, None)


def _dapp(ws=DUMMY, nb=1 << 30, S=1, H=4, D=128, W=4096, dt=swa.SWA_BF16, kn=DUMMY):
    return swa.lib().swa_decode_append(DUMMY, kn, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, S, H, D, W,
                                       dt, ws, nb, None)


def test_decode_workspace_bytes():
    L = swa.lib()
    need = L.swa_decode_workspace_bytes(1, 4, 128, 4096, swa.SWA_BF16)
    assert need > 0 and need % 4 == 0
    assert L.swa_decode_workspace_bytes(1024, 4, 128, 4096, swa.SWA_BF16) == 0
    # fp32 splits for the head sizes of its matrix-path kernel, at the same sizes
    assert L.swa_decode_workspace_bytes(1, 4, 128, 4096, swa.SWA_F32) == need
    assert L.swa_decode_workspace_bytes(1, 4, 32, 4096, swa.SWA_F32) > 0
    assert L.swa_decode_workspace_bytes(1, 4, 48, 4096, swa.SWA_F32) == 0
    assert L.swa_decode_workspace_bytes(1, 4, 128, 16385, swa.SWA_F32) == 0
    assert L.swa_decode_workspace_bytes(0, 4, 128, 4096, swa.SWA_BF16) == -swa.SWA_ERR_INVALID_ARG
    assert L.swa_decode_workspace_bytes(1, 4, 128, -1, swa.SWA_BF16) == -swa.SWA_ERR_INVALID_ARG


@pytest.mark.parametrize("fn", [_dsplit, _dapp])
@pytest.mark.parametrize("kw", [dict(ws=None), dict(nb=16), dict(nb=-1),
                                dict(ws=ctypes.c_void_p(0x1004)), dict(S=0), dict(W=0)])
def test_decode_workspace_entries_reject(fn, kw):
    assert fn(**kw) == swa.SWA_ERR_INVALID_ARG


@pytest.mark.parametrize("fn", [_dsplit, _dapp])
@pytest.mark.parametrize("kw", [dict(dt=3), dict(D=96), dict(dt=swa.SWA_F32, D=300)])
def test_decode_workspace_entries_unsupported(fn, kw):
    assert fn(**kw) == swa.SWA_ERR_UNSUPPORTED


def test_decode_append_rejects_null_token():
    assert _dapp(kn=None) == swa.SWA_ERR_INVALID_ARG


def _mha(x=DUMMY, wq=DUMMY, out=DUMMY, ws=DUMMY, nb=1 << 40, B=1, T=16, dm=256, H=2, W=8,
         dt=swa.SWA_BF16):
    return swa.lib().swa_mha_forward(x, wq, None, DUMMY, None, DUMMY, None, DUMMY, None, out, B,
                                     T, dm, H, W, dt, ws, nb, None)


def test_mha_workspace_bytes():
    L = swa.lib()
    assert L.swa_mha_workspace_bytes(2, 16, 256, swa.SWA_BF16) == 2 * 16 * 4 * 256 * 2
    assert L.swa_mha_workspace_bytes(2, 16, 256, swa.SWA_F32) == 2 * 16 * 4 * 256 * 4
    assert L.swa_mha_workspace_bytes(0, 16, 256, swa.SWA_F32) == -swa.SWA_ERR_INVALID_ARG
    assert L.swa_mha_workspace_bytes(1, 16, 256, 7) == -swa.SWA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(x=None), dict(wq=None), dict(out=None), dict(ws=None),
                                dict(B=0), dict(T=0), dict(dm=0), dict(H=0), dict(W=0),
                                dict(H=3), dict(nb=100), dict(nb=-1),
                                dict(ws=ctypes.c_void_p(0x1008))])
def test_mha_invalid_args(kw):
    assert _mha(**kw) == swa.SWA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(dt=4), dict(dm=192, H=2), dict(dm=64, H=2),
                                dict(dt=swa.SWA_F32, dm=1024, H=2)])
def test_mha_unsupported(kw):
    assert _mha(**kw) == swa.SWA_ERR_UNSUPPORTED


def _bwd(q=DUMMY, dq=DUMMY, ws=DUMMY, nb=1 << 40, B=1, H=1, T=8, D=64, W=4, scale=0.0,
         dt=swa.SWA_F32):
    return swa.lib().swa_backward(q, DUMMY, DUMMY, DUMMY, DUMMY, None, dq, DUMMY, DUMMY, B, H, T,
                                  D, W, scale, dt, ws, nb, None)


def _flse(q=DUMMY, lse=DUMMY, B=1, H=1, T=8, D=64, W=4, scale=0.0, dt=swa.SWA_BF16):
    return swa.lib().swa_forward_lse(q, DUMMY, DUMMY, DUMMY, lse, B, H, T, D, W, scale, dt, None)


@pytest.mark.parametrize("kw", [dict(q=None), dict(lse=None), dict(T=0), dict(W=0),
                                dict(scale=float("inf"))])
def test_forward_lse_invalid_args(kw):
    assert _flse(**kw) == swa.SWA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(dt=3), dict(D=96)])
def test_forward_lse_unsupported(kw):
    assert _flse(**kw) == swa.SWA_ERR_UNSUPPORTED


def test_backward_workspace_bytes():
    assert swa.lib().swa_backward_workspace_bytes(2, 3, 5) == 2 * 3 * 5 * 8
    assert swa.lib().swa_backward_workspace_bytes(0, 3, 5) == -swa.SWA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(q=None), dict(dq=None), dict(ws=None), dict(B=0), dict(T=0),
                                dict(W=0), dict(nb=8), dict(nb=-1), dict(scale=float("nan")),
                                dict(ws=ctypes.c_void_p(0x1002))])
def test_backward_invalid_args(kw):
    assert _bwd(**kw) == swa.SWA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(dt=2), dict(D=300)])
def test_backward_unsupported(kw):
    assert _bwd(**kw) == swa.SWA_ERR_UNSUPPORTED


def _chunk(q=DUMMY, kc=DUMMY, vc=DUMMY, kr=DUMMY, vr=DUMMY, pos=DUMMY, o=DUMMY, S=1, H=1, C=4,
           D=64, W=8, dt=swa.SWA_BF16):
    return swa.lib().swa_chunk_forward(q, kc, vc, kr, vr, pos, o, S, H, C, D, W, dt, None)


def _app_chunk(kc=DUMMY, vc=DUMMY, kr=DUMMY, vr=DUMMY, pos=DUMMY, S=1, H=1, C=4, D=64, W=8,
               dt=swa.SWA_BF16):
    return swa.lib().swa_ring_append_chunk(kc, vc, kr, vr, pos, S, H, C, D, W, dt, None)


@pytest.mark.parametrize("kw", [dict(q=None), dict(kc=None), dict(vc=None), dict(kr=None),
                                dict(vr=None), dict(pos=None), dict(o=None), dict(S=0), dict(H=0),
                                dict(C=0), dict(D=0), dict(W=0)])
def test_chunk_invalid_args(kw):
    assert _chunk(**kw) == swa.SWA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(dt=9), dict(D=300)])
def test_chunk_unsupported(kw):
    assert _chunk(**kw) == swa.SWA_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw", [dict(kc=None), dict(vr=None), dict(pos=None), dict(C=0),
                                dict(W=-2)])
def test_append_chunk_invalid_args(kw):
    assert _app_chunk(**kw) == swa.SWA_ERR_INVALID_ARG


def test_append_chunk_unsupported_dtype():
    assert _app_chunk(dt=4) == swa.SWA_ERR_UNSUPPORTED


def test_chunk_workspace_bytes():
    L = swa.lib()
    n = L.swa_chunk_workspace_bytes(1, 4, 128, 128, 4096, swa.SWA_BF16)
    assert n > 0 and n % (4 * (128 + 2)) == 0
    assert L.swa_chunk_workspace_bytes(64, 32, 2048, 128, 4096, swa.SWA_BF16) == 0
    assert L.swa_chunk_workspace_bytes(1, 4, 128, 128, 4096, swa.SWA_F32) == 0
    assert L.swa_chunk_workspace_bytes(0, 4, 128, 128, 4096, swa.SWA_BF16) == -swa.SWA_ERR_INVALID_ARG


@pytest.mark.parametrize("kw", [dict(ws=None), dict(nb=64), dict(nb=-1),
                                dict(ws=ctypes.c_void_p(0x1004)), dict(C=0)])
def test_chunk_split_invalid_args(kw):
    a = dict(ws=DUMMY, nb=1 << 40, C=128)
    a.update(kw)
    rc = swa.lib().swa_chunk_forward_split(DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, DUMMY, 1, 4,
                                           a["C"], 128, 4096, swa.SWA_BF16, a["ws"], a["nb"], None)
    assert rc == swa.SWA_ERR_INVALID_ARG


def test_oversized_grid_is_unsupported():
    assert _fwd(B=1 << 20, H=1 << 10, T=1 << 10, D=64) == swa.SWA_ERR_UNSUPPORTED


# ---- Python-level checks (no library call is reached) ----------------------

def test_binding_rejects_cpu_tensors():
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        swa.swa_forward(x, x, x, x.clone(), 4)


@pytest.mark.parametrize("W,exc", [(0, ValueError), (-1, ValueError), (True, TypeError),
                                   (2.0, TypeError)])
def test_binding_rejects_bad_window(W, exc):
    x = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(exc):
        swa.swa_forward(x, x, x, x.clone(), W)


def test_error_is_raised_with_status():
    err = swa.SWAError(swa.SWA_ERR_UNSUPPORTED, swa.status_string(swa.SWA_ERR_UNSUPPORTED))
    assert err.status == swa.SWA_ERR_UNSUPPORTED and "unsupported" in str(err)


def test_product_package_does_not_import_oracle():
    pkg = os.path.join(ROOT, "sliding_window_causal_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in text.replace("no fallback", ""), f


def _dnoalloc(q=DUMMY, kr=DUMMY, vr=DUMMY, pos=DUMMY, o=DUMMY, S=1, H=4, D=128, W=4096,
              dt=swa.SWA_BF16):
    return swa.lib().swa_decode_split_noalloc(q, kr, vr, pos, o, S, H, D, W, dt, None)


@pytest.mark.parametrize("kw,code", [(dict(q=None), swa.SWA_ERR_INVALID_ARG),
                                     (dict(kr=None), swa.SWA_ERR_INVALID_ARG),
                                     (dict(pos=None), swa.SWA_ERR_INVALID_ARG),
                                     (dict(o=None), swa.SWA_ERR_INVALID_ARG),
                                     (dict(S=0), swa.SWA_ERR_INVALID_ARG),
                                     (dict(W=-2), swa.SWA_ERR_INVALID_ARG),
                                     (dict(dt=7, S=1024), swa.SWA_ERR_UNSUPPORTED),
                                     (dict(D=96, S=1024), swa.SWA_ERR_UNSUPPORTED)])
def test_noalloc_decode_rejects_before_any_hip_call(kw, code):
    assert _dnoalloc(**kw) == code


def test_noalloc_scratch_covers_every_split_size():
    """The static scratch holds the split's partials for every size the split
    policy produces (splits stop at 512 (stream, head) pairs, 2048 workgroups
    and 64 splits), so swa_decode_split_noalloc never returns
    SWA_ERR_SCRATCH_LIMIT for a size swa_decode_split takes."""
    L = swa.lib()
    worst = 0
    for sh in range(1, 600):
        for dtype, D in ((swa.SWA_BF16, 64), (swa.SWA_BF16, 128), (swa.SWA_F32, 32),
                         (swa.SWA_F32, 64), (swa.SWA_F32, 128)):
            for W in (1, 255, 256, 257, 1000, 4096, 8191, 16384):
                n = L.swa_decode_workspace_bytes(1, sh, D, W, dtype)
                assert n >= 0
                worst = max(worst, n)
    assert 0 < worst <= swa.NOALLOC_SCRATCH_BYTES


def test_header_compiles_as_c_and_a_c_program_links(tmp_path):
    """include/swa.h is plain C: a C99 program that includes it (with -Wall
    -Werror -pedantic) links against libswa.so and gets the documented status
    codes from calls that fail validation, so no GPU is touched."""
    src = tmp_path / "abi.c"
    src.write_text(r'''
#include <stdio.h>
#include <string.h>
#include "swa.h"

int main(void) {
    int bad = 0;
    int rc;
    if (swa_abi_version() != 2) bad |= 1;
    if (strlen(swa_status_string(SWA_ERR_INVALID_ARG)) == 0) bad |= 2;
    rc = swa_forward(NULL, NULL, NULL, NULL, 1, 1, 8, 64, 4, SWA_BF16, NULL);
    if (rc != SWA_ERR_INVALID_ARG) bad |= 4;
    rc = swa_decode((void*)0x1000, (void*)0x1000, (void*)0x1000, (const int64_t*)0x1000,
                    (void*)0x1000, 1, 1, 64, 0, SWA_BF16, NULL);
    if (rc != SWA_ERR_INVALID_ARG) bad |= 8;
    rc = swa_forward((void*)0x1000, (void*)0x1000, (void*)0x1000, (void*)0x1000,
                     1, 1, 8, 64, 4, 7, NULL);
    if (rc != SWA_ERR_UNSUPPORTED) bad |= 16;
    if (swa_decode_workspace_bytes(0, 1, 64, 8, SWA_BF16) >= 0) bad |= 32;
    printf("%d\n", bad);
    return bad;
}
''')
    exe = tmp_path / "abi"
    libdir = os.path.dirname(swa.LIB_PATH)
    cc = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-pedantic", str(src),
                         "-I", os.path.join(ROOT, "include"), "-L", libdir, "-lswa",
                         f"-Wl,-rpath,{libdir}", "-o", str(exe)],
                        stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert cc.returncode == 0, cc.stdout
    run = subprocess.run([str(exe)], stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                         timeout=120)
    assert run.returncode == 0, run.stdout


def test_missing_library_raises_instead_of_falling_back(monkeypatch, tmp_path):
    """There is no CPU or other fallback: without libswa.so every entry point
    raises (here with the library path pointed at a file that does not exist
    and the loaded handle dropped)."""
    monkeypatch.setattr(swa, "LIB_PATH", str(tmp_path / "libswa.so"))
    monkeypatch.setattr(swa, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        swa.lib()
    with pytest.raises(RuntimeError, match="missing"):
        swa.abi_version()
