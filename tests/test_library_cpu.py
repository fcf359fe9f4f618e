"""Host-side checks of libw12.so that need no GPU: it builds for gfx950, loads, exports
every symbol include/w12.h declares, and rejects bad arguments before any HIP call."""
import ctypes
import os
import re

import pytest

import lossless_bit_weight_w12_amd as w12
from lossless_bit_weight_w12_amd import w12 as B

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "w12.h")


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(w12.lib_path()):
        from lossless_bit_weight_w12_amd import build
        build.build(verbose=False)
    return w12.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(w12_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert set(names) == set(B.EXPORTS)
    for nm in names:
        assert hasattr(L, nm), nm


def test_status_strings(L):
    for code in range(-7, 1):
        assert w12.status_str(code) and w12.status_str(code) != "unknown status"
    assert w12.status_str(-99) == "unknown status"
    assert L.w12_version() == 0x000100


@pytest.mark.parametrize("n,k", [(16, 128), (1024, 1024), (151936, 5120), (5120, 17408)])
def test_tiles_bytes_closed_form(L, n, k):
    assert w12.tiles_bytes(n, k) == (n // 16) * (k // 128) * 3072 == 3 * 2 * n * k // 4


@pytest.mark.parametrize("n,k", [(0, 128), (15, 128), (16, 100), (16, 1 << 20), (17, 128)])
def test_bad_shapes_report_zero(L, n, k):
    assert w12.tiles_bytes(n, k) == 0
    assert w12.workspace_bytes(w12.OP_GEMM, 1, n, k) == 0


def test_workspace_sizes(L):
    assert w12.workspace_bytes(w12.OP_GEMM, 0, 1024, 1024) == 0
    assert w12.workspace_bytes(w12.OP_GEMM, w12.MAX_M + 1, 1024, 1024) == 0
    assert w12.workspace_bytes(w12.OP_VERIFY, w12.MAX_M, 1 << 25, 128) == 0   # m * n >= 2^32
    assert w12.workspace_bytes(99, 1, 1024, 1024) == 0
    n, k, m = 151936, 5120, 16
    v = w12.workspace_bytes(w12.OP_VERIFY, m, n, k)
    assert v >= 16 * m * (n // 16) + 4 * m * n + 8 * m   # block records, candidate lists, counts
    assert v < 8 * m * n                                  # no full logits or S
    assert w12.workspace_bytes(w12.OP_ENCODE, 1, n, k) >= 8 * (n // 16) * (k // 128)


FAKE = 0x10000          # non-null, 256-byte aligned, never dereferenced (validation fails first)


def desc(n=1024, k=1024, cb=tuple(range(100, 116)), e_max=120, n_esc=0):
    d = B.W12Desc()
    d.n, d.k, d.n_esc = n, k, n_esc
    for i, c in enumerate(cb):
        d.codebook[i] = c
    d.e_max = e_max
    d.tiles = FAKE
    d.esc_off = FAKE
    d.esc = FAKE if n_esc else None
    return d


def gemm(L, x=FAKE, m=1, d=None, y=FAKE, ws=FAKE, wsb=1 << 30):
    d = d or desc()
    return L.w12_gemm(x, m, ctypes.byref(d), y, ws, wsb, None)


def test_gemm_validation(L):
    assert gemm(L, x=None) == -1
    assert gemm(L, y=None) == -1
    assert L.w12_gemm(FAKE, 1, None, FAKE, FAKE, 1 << 30, None) == -1
    assert gemm(L, d=desc(n=1000)) == -2
    assert gemm(L, d=desc(k=1000)) == -2
    assert gemm(L, d=desc(k=1 << 20)) == -2
    assert gemm(L, m=0) == -3
    assert gemm(L, m=129) == -3
    assert gemm(L, m=128, d=desc(n=1 << 25, k=128)) == -2      # m * n >= 2^32
    assert gemm(L, m=127, d=desc(n=1 << 25, k=128), x=FAKE + 2) == -7   # shape passes
    assert gemm(L, d=desc(cb=(5,) * 16)) == -4
    assert gemm(L, d=desc(cb=tuple(range(115, 99, -1)))) == -4
    assert gemm(L, d=desc(e_max=255)) == -4
    bad = desc(n_esc=4)
    bad.esc = None
    assert gemm(L, d=bad) == -1
    assert gemm(L, m=16, wsb=0, d=desc(n=64, k=4096)) == -5     # split-K needs partials
    assert gemm(L, x=FAKE + 2) == -7
    assert gemm(L, ws=FAKE + 16) == -7
    assert gemm(L, y=FAKE + 8) == -7          # y must be 16-byte aligned
    mis = desc()
    mis.tiles = FAKE + 4
    assert gemm(L, d=mis) == -7


def test_gemm_rms_validation(L):
    """The RMS entry points validate exactly as their plain counterparts."""
    d = desc()
    assert L.w12_gemm_rms(None, 1, ctypes.byref(d), FAKE, FAKE, 1 << 30, None) == -1
    assert L.w12_gemm_rms(FAKE, 129, ctypes.byref(d), FAKE, FAKE, 1 << 30, None) == -3
    assert L.w12_gemm_rms(FAKE, 1, ctypes.byref(desc(n=1000)), FAKE, FAKE, 1 << 30, None) == -2
    assert L.w12_gemm_rms(FAKE, 1, ctypes.byref(d), FAKE + 8, FAKE, 1 << 30, None) == -7
    assert L.w12_gemm_rms(FAKE, 16, ctypes.byref(desc(n=64, k=4096)), FAKE, FAKE, 0, None) == -5
    darr = (ctypes.POINTER(B.W12Desc) * 2)(ctypes.pointer(desc()), ctypes.pointer(desc()))
    yarr = (ctypes.c_void_p * 2)(FAKE, FAKE)
    f = L.w12_gemm_group_rms
    assert f(FAKE, 1, darr, 0, yarr, FAKE, 1 << 30, None) == -3
    assert f(FAKE + 2, 1, darr, 2, yarr, FAKE, 1 << 30, None) == -7
    odd = (ctypes.POINTER(B.W12Desc) * 2)(ctypes.pointer(desc(k=1024)), ctypes.pointer(desc(k=2048)))
    assert f(FAKE, 1, odd, 2, yarr, FAKE, 1 << 30, None) == -2


def test_gemm_group_validation(L):
    f = L.w12_gemm_group
    ds = [desc(n=1024, k=1024), desc(n=256, k=1024), desc(n=256, k=1024)]
    darr = (ctypes.POINTER(B.W12Desc) * 3)(*[ctypes.pointer(d) for d in ds])
    yarr = (ctypes.c_void_p * 3)(FAKE, FAKE, FAKE)
    big = 1 << 30
    assert f(None, 1, darr, 3, yarr, FAKE, big, None) == -1
    assert f(FAKE, 1, None, 3, yarr, FAKE, big, None) == -1
    assert f(FAKE, 1, darr, 3, None, FAKE, big, None) == -1
    assert f(FAKE, 1, darr, 0, yarr, FAKE, big, None) == -3
    assert f(FAKE, 1, darr, 5, yarr, FAKE, big, None) == -3
    assert f(FAKE, 129, darr, 3, yarr, FAKE, big, None) == -3
    assert f(FAKE, 1, darr, 3, yarr, FAKE, 0, None) == -5           # split-K needs partials
    assert f(FAKE + 2, 1, darr, 3, yarr, FAKE, big, None) == -7
    yarr[2] = FAKE + 8
    assert f(FAKE, 1, darr, 3, yarr, FAKE, big, None) == -7
    yarr[2] = FAKE
    yarr[1] = None
    assert f(FAKE, 1, darr, 3, yarr, FAKE, big, None) == -1
    yarr[1] = FAKE
    odd = (ctypes.POINTER(B.W12Desc) * 2)(ctypes.pointer(desc(k=1024)), ctypes.pointer(desc(k=2048)))
    assert f(FAKE, 1, odd, 2, yarr, FAKE, big, None) == -2           # different k
    badcb = (ctypes.POINTER(B.W12Desc) * 2)(ctypes.pointer(desc()), ctypes.pointer(desc(cb=(5,) * 16)))
    assert f(FAKE, 1, badcb, 2, yarr, FAKE, big, None) == -4
    assert w12.workspace_bytes(w12.OP_GEMM_GROUP, 24, 7168, 5120) >= \
        w12.workspace_bytes(w12.OP_GEMM, 24, 7168, 5120)


def test_gemm_bf16_validation(L):
    f = L.w12_gemm_bf16
    assert f(None, 1, FAKE, 1024, 1024, FAKE, FAKE, 1 << 30, None) == -1
    assert f(FAKE, 1, FAKE, 1000, 1024, FAKE, FAKE, 1 << 30, None) == -2
    assert f(FAKE, 129, FAKE, 1024, 1024, FAKE, FAKE, 1 << 30, None) == -3
    assert f(FAKE, 1, FAKE + 8, 1024, 1024, FAKE, FAKE, 1 << 30, None) == -7
    assert f(FAKE, 1, FAKE, 1024, 1024, FAKE + 8, FAKE, 1 << 30, None) == -7


def test_bf16_tiled_validation(L):
    assert L.w12_bf16_tile(None, 1024, 1024, FAKE, None) == -1
    assert L.w12_bf16_tile(FAKE, 1000, 1024, FAKE, None) == -2
    assert L.w12_bf16_tile(FAKE, 1024, 1024, FAKE + 8, None) == -7
    f = L.w12_gemm_bf16_tiled
    assert f(FAKE, 1, None, 1024, 1024, FAKE, FAKE, 1 << 30, None) == -1
    assert f(FAKE, 1, FAKE, 1024, 100, FAKE, FAKE, 1 << 30, None) == -2
    assert f(FAKE, 0, FAKE, 1024, 1024, FAKE, FAKE, 1 << 30, None) == -3
    assert f(FAKE, 1, FAKE + 4, 1024, 1024, FAKE, FAKE, 1 << 30, None) == -7


def test_f8_validation(L):
    assert L.w12_f8_tile(None, 1024, 1024, FAKE, None) == -1
    assert L.w12_f8_tile(FAKE, 1000, 1024, FAKE, None) == -2
    assert L.w12_f8_tile(FAKE, 1024, 1024, FAKE + 8, None) == -7
    f = L.w12_gemm_f8
    assert f(FAKE, 1, FAKE, None, 1024, 1024, FAKE, FAKE, 1 << 30, None) == -1     # no scales
    assert f(FAKE, 1, None, FAKE, 1024, 1024, FAKE, FAKE, 1 << 30, None) == -1
    assert f(FAKE, 1, FAKE, FAKE, 1024, 100, FAKE, FAKE, 1 << 30, None) == -2
    assert f(FAKE, 0, FAKE, FAKE, 1024, 1024, FAKE, FAKE, 1 << 30, None) == -3
    assert f(FAKE, 129, FAKE, FAKE, 1024, 1024, FAKE, FAKE, 1 << 30, None) == -3
    assert f(FAKE, 1, FAKE + 4, FAKE, 1024, 1024, FAKE, FAKE, 1 << 30, None) == -7
    assert f(FAKE, 1, FAKE, FAKE + 2, 1024, 1024, FAKE, FAKE, 1 << 30, None) == -7
    need = w12.workspace_bytes(w12.OP_GEMM_F8, 1, 1024, 4096)
    assert need == w12.workspace_bytes(w12.OP_GEMM, 1, 1024, 4096) and need > 0   # (K split)
    assert f(FAKE, 1, FAKE, FAKE, 1024, 4096, FAKE, FAKE, need - 1, None) == -5
    assert f(FAKE, 1, FAKE, FAKE, 1024, 4096, FAKE, None, need, None) == -1


def test_f8_group_validation(L):
    P = lambda *v: (ctypes.c_void_p * len(v))(*v)
    N = lambda *v: (ctypes.c_uint64 * len(v))(*v)
    f = L.w12_gemm_f8_group
    ok = dict(x=FAKE, m=1, w=P(FAKE, FAKE), s=P(FAKE, FAKE), n=N(1024, 512), nw=2, k=1024,
              y=P(FAKE, FAKE), ws=FAKE, wsb=1 << 30)

    def call(**kw):
        a = {**ok, **kw}
        return f(a["x"], a["m"], a["w"], a["s"], a["n"], a["nw"], a["k"], a["y"], a["ws"], a["wsb"], None)
    assert call(x=None) == -1
    assert call(s=P(FAKE, None)) == -1
    assert call(y=P(None, FAKE)) == -1
    assert call(nw=0) == -3 and call(nw=5) == -3 and call(m=0) == -3 and call(m=129) == -3
    assert call(n=N(1024, 1000)) == -2
    assert call(k=100) == -2
    assert call(w=P(FAKE, FAKE + 8)) == -7
    assert call(s=P(FAKE + 2, FAKE)) == -7
    assert call(x=FAKE + 8) == -7
    need = w12.workspace_bytes(w12.OP_GEMM_GROUP, 1, 1536, 1024)
    assert need > 0 and call(wsb=need - 1) == -5 and call(ws=None, wsb=need) == -1


def test_verify_validation(L):
    f = L.w12_lmhead_verify
    d = desc(n=2048, k=512)
    big = 1 << 34
    assert f(FAKE, 4, ctypes.byref(d), FAKE, 4, None, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 4, ctypes.byref(d), None, 2, FAKE, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 4, ctypes.byref(d), FAKE, 5, FAKE, FAKE, FAKE, big, None) == -3   # n_draft > m
    assert f(FAKE, 0, ctypes.byref(d), FAKE, 0, FAKE, FAKE, FAKE, big, None) == -3
    assert f(FAKE, 4, ctypes.byref(d), FAKE, 4, FAKE, FAKE, FAKE, 100, None) == -5


def test_verify_batched_validation(L):
    f = L.w12_lmhead_verify_batched
    d = desc(n=2048, k=512)
    big = 1 << 34
    #      x     m  desc            off   nd    nreq draft argmax acc   ws    wsb
    assert f(None, 8, ctypes.byref(d), FAKE, FAKE, 3, FAKE, FAKE, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 8, ctypes.byref(d), None, FAKE, 3, FAKE, FAKE, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 8, ctypes.byref(d), FAKE, None, 3, FAKE, FAKE, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 8, ctypes.byref(d), FAKE, FAKE, 3, None, FAKE, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 8, ctypes.byref(d), FAKE, FAKE, 3, FAKE, None, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 8, ctypes.byref(d), FAKE, FAKE, 3, FAKE, FAKE, None, FAKE, big, None) == -1
    assert f(FAKE, 8, ctypes.byref(d), FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, big, None) == -3
    assert f(FAKE, 8, ctypes.byref(d), FAKE, FAKE, 9, FAKE, FAKE, FAKE, FAKE, big, None) == -3   # n_req > m
    assert f(FAKE, 129, ctypes.byref(d), FAKE, FAKE, 3, FAKE, FAKE, FAKE, FAKE, big, None) == -3
    assert f(FAKE, 8, ctypes.byref(d), FAKE + 2, FAKE, 3, FAKE, FAKE, FAKE, FAKE, big, None) == -7
    assert f(FAKE, 8, ctypes.byref(d), FAKE, FAKE, 3, FAKE, FAKE, FAKE, FAKE, 100, None) == -5
    assert f(FAKE, 8, ctypes.byref(desc(n=1000, k=512)), FAKE, FAKE, 3, FAKE, FAKE, FAKE, FAKE, big,
             None) == -2


def test_logits_f32_validation(L):
    f = L.w12_logits_f32
    d = desc(n=2048, k=512)
    big = 1 << 34
    assert f(None, 4, ctypes.byref(d), FAKE, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 4, ctypes.byref(d), None, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 4, ctypes.byref(d), FAKE, FAKE, None, big, None) == -1
    assert f(FAKE, 4, None, FAKE, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 0, ctypes.byref(d), FAKE, FAKE, FAKE, big, None) == -3
    assert f(FAKE, 129, ctypes.byref(d), FAKE, FAKE, FAKE, big, None) == -3
    assert f(FAKE, 4, ctypes.byref(desc(n=1000, k=512)), FAKE, FAKE, FAKE, big, None) == -2
    assert f(FAKE, 4, ctypes.byref(d), FAKE, FAKE, FAKE, 100, None) == -5
    assert f(FAKE, 4, ctypes.byref(d), FAKE + 8, FAKE, FAKE, big, None) == -7
    assert f(FAKE, 4, ctypes.byref(d), FAKE, FAKE + 4, FAKE, big, None) == -7


def test_encode_decode_validation(L):
    cb = (ctypes.c_uint8 * 16)()
    em = ctypes.c_uint8()
    ne = ctypes.c_uint64()
    f = L.w12_encode_count
    assert f(None, 16, 128, cb, ctypes.byref(em), ctypes.byref(ne), FAKE, 1 << 20, None) == -1
    assert f(FAKE, 16, 100, cb, ctypes.byref(em), ctypes.byref(ne), FAKE, 1 << 20, None) == -2
    assert f(FAKE, 16, 128, cb, ctypes.byref(em), ctypes.byref(ne), FAKE, 16, None) == -5
    assert f(FAKE + 2, 16, 128, cb, ctypes.byref(em), ctypes.byref(ne), FAKE, 1 << 20, None) == -7
    d = desc()
    assert L.w12_encode(FAKE, ctypes.byref(d), FAKE, 16, None) == -5
    assert L.w12_encode(None, ctypes.byref(d), FAKE, 1 << 30, None) == -1
    assert L.w12_decode(ctypes.byref(desc(k=100)), FAKE, None) == -2
    assert L.w12_decode(ctypes.byref(desc()), None, None) == -1
    assert L.w12_rms_rescale(FAKE, 0, 128, FAKE, None) == -3
    assert L.w12_rms_rescale(FAKE, 4, 100, FAKE, None) == -2        # k % 8 != 0
    assert L.w12_rms_rescale(FAKE + 8, 4, 128, FAKE, None) == -7    # x not 16-byte aligned
    assert L.w12_workspace_init(None, 64, None) == -1


def test_library_binds_to_torchs_hip_runtime():
    """The binding loads torch before libw12.so, so that the library's NEEDED
    libamdhip64.so.7 resolves to the runtime torch already holds (torch bundles its own);
    checked in a fresh interpreter that asks for the library before importing torch."""
    import subprocess
    import sys
    code = ("import sys; sys.path.insert(0, %r)\n"
            "import lossless_bit_weight_w12_amd as w12\n"
            "w12.lib()\n"
            "import torch, os\n"
            "maps = open('/proc/self/maps').read()\n"
            "paths = {l.split()[-1] for l in maps.splitlines() if 'libamdhip64.so' in l}\n"
            "print(len(paths))\n") % (os.path.dirname(os.path.dirname(os.path.abspath(__file__))),)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300)
    assert out.returncode == 0, out.stderr[-2000:]
    assert out.stdout.strip().splitlines()[-1] == "1"      # one HIP runtime in the process


def test_stream_read_validation(L):
    assert L.w12_stream_read(None, 1024, 16, FAKE, None) == -1
    assert L.w12_stream_read(FAKE, 1024, 16, None, None) == -1
    assert L.w12_stream_read(FAKE, 0, 16, FAKE, None) == -2
    assert L.w12_stream_read(FAKE, 1000, 16, FAKE, None) == -2
    assert L.w12_stream_read(FAKE, 1 << 32, 16, FAKE, None) == -2
    assert L.w12_stream_read(FAKE, 1024, 0, FAKE, None) == -3
    assert L.w12_stream_read(FAKE, 1024, 65537, FAKE, None) == -3
    assert L.w12_stream_read(FAKE + 8, 1024, 16, FAKE, None) == -7


def test_header_constants_match_binding():
    """The binding's copies of the header's numeric constants agree with include/w12.h."""
    import re
    from lossless_bit_weight_w12_amd import w12 as b
    text = open(HEADER).read()

    def define(name):
        m = re.search(r"#define\s+%s\s+\(?(\d+)u?(?:\s*<<\s*(\d+))?\)?" % name, text)
        assert m, name
        return int(m.group(1)) << int(m.group(2) or 0)

    assert define("W12_ENCODE_TOTAL_OFFSET") == b.ENCODE_TOTAL_OFFSET
    assert define("W12_NOALLOC_SCRATCH_BYTES") == b.NOALLOC_SCRATCH_BYTES
    assert define("W12_MAX_M") == b.MAX_M
    for name, val in [("W12_OP_ENCODE", b.OP_ENCODE), ("W12_OP_DECODE", b.OP_DECODE),
                      ("W12_OP_GEMM", b.OP_GEMM), ("W12_OP_GEMM_BF16", b.OP_GEMM_BF16),
                      ("W12_OP_VERIFY", b.OP_VERIFY), ("W12_OP_GEMM_GROUP", b.OP_GEMM_GROUP),
                      ("W12_OP_VERIFY2", b.OP_VERIFY2), ("W12_OP_GEMM_F8", b.OP_GEMM_F8)]:
        assert define(name) == val, name


def _screen_bytes_closed_form(n, k):
    a = lambda v: (v + 255) // 256 * 256
    return a((n // 16) * (k // 128) * 2176) + 2 * a(4 * n)


@pytest.mark.parametrize("n,k", [(16, 128), (2048, 512), (151936, 5120), (16400, 512)])
def test_screen_bytes_closed_form(L, n, k):
    assert L.w12_screen_bytes(n, k) == _screen_bytes_closed_form(n, k)
    # the screen tiles are 17/24 of the W12 tiles (2176 against 3072 bytes per 16 x 128)
    assert (n // 16) * (k // 128) * 2176 * 24 == w12.tiles_bytes(n, k) * 17


@pytest.mark.parametrize("n,k", [(0, 128), (15, 128), (16, 100), (16, 1 << 20)])
def test_screen_bad_shapes(L, n, k):
    assert L.w12_screen_bytes(n, k) == 0
    assert w12.workspace_bytes(w12.OP_VERIFY2, 1, n, k) == 0


def test_screen_encode_validation(L):
    f = L.w12_screen_encode
    big = 1 << 34
    assert f(None, 2048, 512, FAKE, big, None) == -1
    assert f(FAKE, 2048, 512, None, big, None) == -1
    assert f(FAKE, 2008, 512, FAKE, big, None) == -2
    assert f(FAKE, 2048, 500, FAKE, big, None) == -2
    assert f(FAKE, 2048, 512, FAKE, L.w12_screen_bytes(2048, 512) - 1, None) == -5
    assert f(FAKE + 8, 2048, 512, FAKE, big, None) == -7
    assert f(FAKE, 2048, 512, FAKE + 16, big, None) == -7


def test_verify2_workspace_sizes(L):
    assert w12.workspace_bytes(w12.OP_VERIFY2, 0, 2048, 512) == 0
    assert w12.workspace_bytes(w12.OP_VERIFY2, w12.MAX_M + 1, 2048, 512) == 0
    assert w12.workspace_bytes(w12.OP_VERIFY2, w12.MAX_M, 1 << 25, 128) == 0   # m * n >= 2^32
    a = lambda v: (v + 255) // 256 * 256
    for m, n in [(1, 2048), (16, 151936), (120, 151936), (5, 16400)]:
        nb = n // 16
        ngrp = (nb + 7) // 8
        slices = 32 if m <= 16 else 16 if m <= 32 else 8 if m <= 64 else 4
        cap = 16 * 8 * ((ngrp + slices - 1) // slices)
        sl, ent = m * slices, m * slices * cap
        want = (4096 + a(8 * m) + 3 * a(4 * m * nb) + 2 * a(4 * m * ngrp) + a(4 * sl) + a(8 * sl)
                + a(4 * ent) + 2 * a(8 * ent) + a(4 * m * n))
        assert w12.workspace_bytes(w12.OP_VERIFY2, m, n, 512) == want, (m, n)


def test_verify2_validation(L):
    f = L.w12_lmhead_verify2
    d = desc(n=2048, k=512)
    big = 1 << 34
    #        x     m  desc            screen draft nd argmax acc   ws    wsb
    assert f(None, 4, ctypes.byref(d), FAKE, FAKE, 4, FAKE, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 4, ctypes.byref(d), None, FAKE, 4, FAKE, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 4, ctypes.byref(d), FAKE, None, 2, FAKE, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 4, ctypes.byref(d), FAKE, FAKE, 4, None, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 4, ctypes.byref(d), FAKE, FAKE, 4, FAKE, None, FAKE, big, None) == -1
    assert f(FAKE, 4, ctypes.byref(d), FAKE, FAKE, 4, FAKE, FAKE, None, big, None) == -1
    assert f(FAKE, 4, None, FAKE, FAKE, 4, FAKE, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 4, ctypes.byref(d), FAKE, FAKE, 5, FAKE, FAKE, FAKE, big, None) == -3   # n_draft > m
    assert f(FAKE, 0, ctypes.byref(d), FAKE, FAKE, 0, FAKE, FAKE, FAKE, big, None) == -3
    assert f(FAKE, 129, ctypes.byref(d), FAKE, FAKE, 4, FAKE, FAKE, FAKE, big, None) == -3
    assert f(FAKE, 4, ctypes.byref(desc(n=1000, k=512)), FAKE, FAKE, 4, FAKE, FAKE, FAKE, big, None) == -2
    need = w12.workspace_bytes(w12.OP_VERIFY2, 4, 2048, 512)
    assert f(FAKE, 4, ctypes.byref(d), FAKE, FAKE, 4, FAKE, FAKE, FAKE, need - 1, None) == -5
    assert f(FAKE + 8, 4, ctypes.byref(d), FAKE, FAKE, 4, FAKE, FAKE, FAKE, big, None) == -7
    assert f(FAKE, 4, ctypes.byref(d), FAKE + 16, FAKE, 4, FAKE, FAKE, FAKE, big, None) == -7
    assert f(FAKE, 4, ctypes.byref(d), FAKE, FAKE, 4, FAKE, FAKE, FAKE + 16, big, None) == -7
    assert f(FAKE, 4, ctypes.byref(d), FAKE, FAKE, 4, FAKE + 2, FAKE, FAKE, big, None) == -7


def test_verify2_batched_and_logits_validation(L):
    f = L.w12_lmhead_verify2_batched
    d = desc(n=2048, k=512)
    big = 1 << 34
    #        x     m  desc            screen off   nd    nreq draft argmax acc   ws    wsb
    assert f(FAKE, 8, ctypes.byref(d), FAKE, None, FAKE, 3, FAKE, FAKE, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 8, ctypes.byref(d), FAKE, FAKE, None, 3, FAKE, FAKE, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 8, ctypes.byref(d), FAKE, FAKE, FAKE, 3, None, FAKE, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 8, ctypes.byref(d), None, FAKE, FAKE, 3, FAKE, FAKE, FAKE, FAKE, big, None) == -1
    assert f(FAKE, 8, ctypes.byref(d), FAKE, FAKE, FAKE, 0, FAKE, FAKE, FAKE, FAKE, big, None) == -3
    assert f(FAKE, 8, ctypes.byref(d), FAKE, FAKE, FAKE, 9, FAKE, FAKE, FAKE, FAKE, big, None) == -3
    assert f(FAKE, 8, ctypes.byref(d), FAKE, FAKE + 2, FAKE, 3, FAKE, FAKE, FAKE, FAKE, big, None) == -7
    assert f(FAKE, 8, ctypes.byref(d), FAKE, FAKE, FAKE, 3, FAKE, FAKE, FAKE, FAKE, 100, None) == -5
    g = L.w12_screen_logits_f32
    assert g(FAKE, 4, ctypes.byref(d), FAKE, None, FAKE, FAKE, big, None) == -1
    assert g(FAKE, 4, ctypes.byref(d), FAKE, FAKE, None, FAKE, big, None) == -1
    assert g(FAKE, 4, ctypes.byref(d), None, FAKE, FAKE, FAKE, big, None) == -1
    assert g(FAKE, 0, ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, big, None) == -3
    assert g(FAKE, 4, ctypes.byref(d), FAKE, FAKE, FAKE, FAKE, 100, None) == -5
    assert g(FAKE, 4, ctypes.byref(d), FAKE, FAKE + 8, FAKE, FAKE, big, None) == -7


def test_gemm_routing_refusals_need_no_device():
    """The binding's routing by weight format refuses a mixed W12 / FP8 group before
    touching any tensor."""
    t8 = B.F8Tensor(n=16, k=128, tiles=None, scale=None)
    t12 = B.W12Tensor(n=16, k=128, n_esc=0, codebook=tuple(range(16)), e_max=0, tiles=None,
                      esc_off=None, esc=None)
    with pytest.raises(ValueError):
        w12.gemm_group(None, [t8, t12])
    with pytest.raises(ValueError):
        w12.gemm_group(None, [t12, t8], rms=True)


def test_f8_rms_validation(L):
    f = L.w12_gemm_f8_rms
    assert f(FAKE, 1, FAKE, None, 1024, 1024, FAKE, FAKE, 1 << 30, None) == -1
    assert f(FAKE, 0, FAKE, FAKE, 1024, 1024, FAKE, FAKE, 1 << 30, None) == -3
    assert f(FAKE, 1, FAKE, FAKE, 1000, 1024, FAKE, FAKE, 1 << 30, None) == -2
    P = lambda *v: (ctypes.c_void_p * len(v))(*v)
    N = lambda *v: (ctypes.c_uint64 * len(v))(*v)
    g = L.w12_gemm_f8_group_rms
    assert g(FAKE, 1, P(FAKE), P(None), N(1024), 1, 1024, P(FAKE), FAKE, 1 << 30, None) == -1
    assert g(FAKE, 1, P(FAKE), P(FAKE), N(1024), 5, 1024, P(FAKE), FAKE, 1 << 30, None) == -3
