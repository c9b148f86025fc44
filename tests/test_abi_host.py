"""Host-side checks of libmla.so that need no GPU: the library loads, exports
every function include/mla_decode.h declares, and rejects invalid arguments
with the documented status codes before touching the device."""

import ctypes
import os
import subprocess

import pytest

from mla_latent_kv_05_amd import binding

pytestmark = pytest.mark.skipif(not os.path.exists(binding.LIB_PATH),
                                reason="libmla.so not built (python -m mla_latent_kv_05_amd.build)")

OK, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE = 0, -1, -2, -3, -4


def test_header_functions_exported():
    names = binding.header_functions()
    assert set(names) == {"mla_absorb_q", "mla_decode_workspace_bytes", "mla_decode_absorbed",
                          "mla_combine_lse", "mla_up_proj_v", "mla_status_string",
                          "mla_cache_append", "mla_cache_append_workspace_bytes", "mla_expand_kv", "mla_gqa_decode", "mla_decode_step",
                          "mla_decode_step_stages", "mla_decode_step_noalloc",
                          "mla_decode_step_workspace_bytes",
                          "mla_prefill_mha"}
    L = binding.lib()
    for n in names:
        assert hasattr(L, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", binding.LIB_PATH], capture_output=True, text=True).stdout
    for n in names:
        assert f" T {n}" in out, n


def test_library_is_gfx950_code():
    """The embedded device code bundle targets gfx950 (and nothing else)."""
    blob = open(binding.LIB_PATH, "rb").read()
    assert b"amdgcn-amd-amdhsa--gfx950" in blob
    for other in (b"--gfx942", b"--gfx90a", b"--gfx1100"):
        assert other not in blob


def test_status_strings():
    for code in (OK, INVALID, UNSUPPORTED, MISALIGNED, WORKSPACE, -5, -6):
        s = binding.status_string(code)
        assert s and s != "unknown status"
    assert binding.status_string(12345) == "unknown status"


FAKE = 0x1000  # never dereferenced: validation fails before any device access


def _decode(**over):
    a = dict(q_lat=FAKE, q_rope=FAKE, kv=FAKE, table=FAKE, max_blocks=4, lens=FAKE, B=2, s_q=1, n_h=128, d_c=512,
             d_r=64, bs=64, scale=0.072, qdt=1, kvdt=1, odt=1, splits=0, ws=FAKE, ws_bytes=1 << 30, out=FAKE,
             lse=None, flags=0)
    a.update(over)
    return binding.lib().mla_decode_absorbed(a["q_lat"], a["q_rope"], a["kv"], a["table"], a["max_blocks"],
                                             a["lens"], a["B"], a["s_q"], a["n_h"], a["d_c"], a["d_r"], a["bs"],
                                             a["scale"], a["qdt"], a["kvdt"], a["odt"], a["splits"], a["ws"],
                                             a["ws_bytes"], a["out"], a["lse"], a["flags"], None)


@pytest.mark.parametrize("over,code", [
    (dict(q_lat=None), INVALID), (dict(kv=None), INVALID), (dict(table=None), INVALID),
    (dict(lens=None), INVALID), (dict(out=None), INVALID), (dict(q_rope=None), INVALID),
    (dict(B=0), INVALID), (dict(s_q=0), INVALID), (dict(n_h=-1), INVALID), (dict(bs=0), INVALID),
    (dict(max_blocks=0), INVALID), (dict(scale=0.0), INVALID), (dict(scale=float("nan")), INVALID),
    (dict(qdt=2), INVALID), (dict(kvdt=7), INVALID), (dict(odt=2), INVALID), (dict(splits=-1), INVALID),
    (dict(flags=8), INVALID), (dict(s_q=17), UNSUPPORTED), (dict(d_c=4096), UNSUPPORTED),
    (dict(d_c=510), UNSUPPORTED), (dict(d_r=300), UNSUPPORTED), (dict(kvdt=2, d_r=60), UNSUPPORTED),
    (dict(out=FAKE + 4), MISALIGNED), (dict(ws=None), WORKSPACE),
])
def test_decode_argument_validation(over, code):
    assert _decode(**over) == code


def test_projection_argument_validation():
    L = binding.lib()
    # absorb: T_q=0 is a no-op even with null pointers
    assert L.mla_absorb_q(None, 0, None, None, 0, 0, 128, 128, 512, 1, 1, 1, None) == OK
    assert L.mla_absorb_q(None, 16384, FAKE, FAKE, 65536, 4, 128, 128, 512, 1, 1, 1, None) == INVALID
    assert L.mla_absorb_q(FAKE, 100, FAKE, FAKE, 65536, 4, 128, 128, 512, 1, 1, 1, None) == INVALID  # stride
    assert L.mla_absorb_q(FAKE, 16384, FAKE, FAKE, 65536, 4, 128, 128, 512, 2, 1, 1, None) == INVALID  # dtype
    assert L.mla_absorb_q(FAKE, 16384, FAKE, FAKE, 65536, 4, 128, 120, 512, 1, 1, 1, None) == UNSUPPORTED
    assert L.mla_absorb_q(FAKE + 2, 16384, FAKE, FAKE, 65536, 4, 128, 128, 512, 1, 1, 1, None) == MISALIGNED
    assert L.mla_up_proj_v(None, 0, None, None, 0, 0, 128, 512, 128, 1, 1, 1, None) == OK
    assert L.mla_up_proj_v(FAKE, 65536, None, FAKE, 16384, 4, 128, 512, 128, 1, 1, 1, None) == INVALID
    assert L.mla_up_proj_v(FAKE, 65536, FAKE, FAKE, 16384, 4, 128, 512, 100, 1, 1, 1, None) == UNSUPPORTED
    assert L.mla_up_proj_v(FAKE, 65540, FAKE, FAKE, 16384, 4, 128, 512, 128, 1, 1, 1, None) == MISALIGNED


def test_combine_argument_validation():
    L = binding.lib()
    assert L.mla_combine_lse(None, None, None, 0, 4, 512, None, None, 0, None) == OK
    assert L.mla_combine_lse(None, FAKE, None, 8, 4, 512, FAKE, None, 0, None) == INVALID
    assert L.mla_combine_lse(FAKE, FAKE, None, 8, 0, 512, FAKE, None, 0, None) == INVALID
    assert L.mla_combine_lse(FAKE, FAKE, None, 8, 4, 510, FAKE, None, 0, None) == UNSUPPORTED
    assert L.mla_combine_lse(FAKE + 8, FAKE, None, 8, 4, 512, FAKE, None, 0, None) == MISALIGNED


def test_workspace_bytes_invalid():
    L = binding.lib()
    assert L.mla_decode_workspace_bytes(0, 1, 128, 512, 4, 0) == 0
    assert L.mla_decode_workspace_bytes(2, 1, 128, 512, 4, -1) == 0


def test_cache_append_argument_validation():
    L = binding.lib()
    ws_n = L.mla_cache_append_workspace_bytes(64, 7168, 512, 64)
    assert ws_n >= 14 * 64 * 576 * 4
    assert L.mla_cache_append_workspace_bytes(0, 7168, 512, 64) == 0
    args = dict(h=FAKE, st=7168, w=FAKE, pos=FAKE, slots=FAKE, cache=FAKE, T=64, d=7168, d_c=512, d_r=64, bs=64,
                base=10000.0, idt=1, kdt=1, ws=FAKE, wsn=ws_n)

    def call(**over):
        a = dict(args, **over)
        return L.mla_cache_append(a["h"], a["st"], a["w"], a["pos"], a["slots"], a["cache"], a["T"], a["d"],
                                  a["d_c"], a["d_r"], a["bs"], a["base"], a["idt"], a["kdt"], a["ws"], a["wsn"], None)
    assert call(T=0, h=None, w=None) == OK
    assert call(h=None) == INVALID
    assert call(st=100) == INVALID
    assert call(d_r=63) == INVALID
    assert call(base=0.0) == INVALID
    assert call(idt=2) == INVALID
    assert call(kdt=5) == INVALID
    assert call(kdt=2, idt=0) == UNSUPPORTED
    assert call(wsn=ws_n - 4) == WORKSPACE
    assert call(ws=None) == WORKSPACE
    assert call(ws=FAKE + 4) == MISALIGNED


def test_prefill_and_expand_argument_validation():
    L = binding.lib()
    assert L.mla_prefill_mha(None, None, None, None, None, None, 0, 128, 128, 64, 0.07, 1, 1, None) == OK
    assert L.mla_prefill_mha(FAKE, FAKE, FAKE, FAKE, None, None, 8, 128, 128, 64, 0.07, 1, 1, None) == INVALID
    assert L.mla_prefill_mha(FAKE, FAKE, FAKE, FAKE, FAKE, None, 8, 128, 128, 64, 0.0, 1, 1, None) == INVALID
    assert L.mla_prefill_mha(FAKE, FAKE, None, FAKE, FAKE, None, 8, 128, 128, 64, 0.07, 1, 1, None) == INVALID
    assert L.mla_prefill_mha(FAKE, FAKE, FAKE, FAKE, FAKE, None, 8, 128, 256, 64, 0.07, 1, 1, None) == UNSUPPORTED
    assert L.mla_prefill_mha(FAKE, FAKE, FAKE, FAKE, FAKE + 4, None, 8, 128, 128, 64, 0.07, 1, 1, None) == MISALIGNED
    assert L.mla_expand_kv(None, 0, None, None, None, None, 0, 128, 512, 128, 1, 1, 1, None) == OK
    assert L.mla_expand_kv(FAKE, 100, FAKE, FAKE, FAKE, FAKE, 4, 128, 512, 128, 1, 1, 1, None) == INVALID
    assert L.mla_expand_kv(FAKE, 512, FAKE, FAKE, FAKE, FAKE, 4, 128, 512, 100, 1, 1, 1, None) == UNSUPPORTED
    assert L.mla_expand_kv(FAKE + 2, 512, FAKE, FAKE, FAKE, FAKE, 4, 128, 512, 128, 1, 1, 1, None) == MISALIGNED


def test_int_cache_argument_validation():
    """Low-bit kv dtypes need d_c and d_r in multiples of the 32-value group."""
    L = binding.lib()
    args = lambda kv, d_c, d_r: (FAKE, FAKE, FAKE, FAKE, 4, FAKE, 2, 1, 8, d_c, d_r, 64, 0.1, 1, kv, 1, 0,
                                 FAKE, 1 << 30, FAKE, None, 0, None)
    assert L.mla_decode_absorbed(*args(5, 128, 32)) == INVALID
    assert L.mla_decode_absorbed(*args(binding.MLA_INT4, 112, 32)) == UNSUPPORTED
    assert L.mla_decode_absorbed(*args(binding.MLA_INT2, 128, 16)) == UNSUPPORTED


def test_gqa_decode_argument_validation():
    L = binding.lib()
    args = lambda **k: tuple({**dict(q_c=FAKE, q_r=FAKE, kv=FAKE, tab=FAKE, mb=4, lens=FAKE, B=2, s_q=2, n_h=128,
                                     n_g=8, d_h=128, d_r=64, bs=64, sc=0.07, qd=1, kd=1, od=1, o=FAKE, lse=None,
                                     flags=0, st=None), **k}.values())
    assert L.mla_gqa_decode(*args(n_g=7)) == INVALID          # n_h not a multiple of n_g
    assert L.mla_gqa_decode(*args(o=None)) == INVALID
    assert L.mla_gqa_decode(*args(sc=0.0)) == INVALID
    assert L.mla_gqa_decode(*args(kd=2)) == INVALID           # fp8 is not a GQA-path cache type
    assert L.mla_gqa_decode(*args(d_h=256, d_r=64)) == UNSUPPORTED
    assert L.mla_gqa_decode(*args(flags=4)) == INVALID


def test_decode_step_argument_validation():
    L = binding.lib()
    base = L.mla_decode_workspace_bytes(4, 2, 128, 512, 16, 0)
    step = L.mla_decode_step_workspace_bytes(4, 2, 128, 512, 16, 0)
    if base:  # sizes need the device's compute-unit count
        assert step >= base + 4 * 2 * 128 * 512 * 2
    else:
        assert step == 0
        step = 1 << 30
    args = lambda **k: tuple({**dict(qn=FAKE, wuk=FAKE, qr=FAKE, kv=FAKE, tab=FAKE, mb=16, lens=FAKE, wuv=FAKE, B=4,
                                     s_q=2, n_h=128, d_h=128, d_c=512, d_r=64, bs=64, sc=0.07, kd=1, ns=0, ws=FAKE,
                                     wsb=step, o=FAKE, lse=None, st=None), **k}.values())
    assert L.mla_decode_step(*args(wuv=None)) == INVALID
    assert L.mla_decode_step(*args(d_h=64)) == UNSUPPORTED       # the fused up-projection is for d_h = 128
    assert L.mla_decode_step(*args(n_h=64)) == UNSUPPORTED       # off the MFMA attention shape
    assert L.mla_decode_step(*args(o=FAKE + 8)) == MISALIGNED
    assert L.mla_decode_step(*args(ws=None)) == WORKSPACE
    st = lambda stages, **k: L.mla_decode_step_stages(*args(**k)[:-1], stages, None)
    assert st(0) == INVALID
    assert st(8) == INVALID
    assert st(-1) == INVALID
    assert st(binding.MLA_STAGE_ATTEND, wuv=None) == INVALID
    assert st(binding.MLA_STAGE_MERGE, d_h=64) == UNSUPPORTED
    assert st(binding.MLA_STAGE_ALL, ws=None) == WORKSPACE


def test_decode_step_noalloc_argument_validation():
    """The no-allocation step checks its arguments like mla_decode_step
    before it looks at the device (no workspace arguments to check)."""
    L = binding.lib()
    args = lambda **k: tuple({**dict(qn=FAKE, wuk=FAKE, qr=FAKE, kv=FAKE, tab=FAKE, mb=16, lens=FAKE, wuv=FAKE, B=4,
                                     s_q=2, n_h=128, d_h=128, d_c=512, d_r=64, bs=64, sc=0.07, kd=1, ns=0, o=FAKE,
                                     lse=None, st=None), **k}.values())
    assert L.mla_decode_step_noalloc(*args(o=None)) == INVALID
    assert L.mla_decode_step_noalloc(*args(B=0)) == INVALID
    assert L.mla_decode_step_noalloc(*args(kd=9)) == INVALID
    assert L.mla_decode_step_noalloc(*args(sc=0.0)) == INVALID
    assert L.mla_decode_step_noalloc(*args(d_h=64)) == UNSUPPORTED
    assert L.mla_decode_step_noalloc(*args(n_h=64)) == UNSUPPORTED
    assert L.mla_decode_step_noalloc(*args(qn=FAKE + 8)) == MISALIGNED
    assert L.mla_decode_step_noalloc(*args(o=FAKE + 8)) == MISALIGNED
