"""Thin Python binding of libw12.so (ctypes).

Argument marshalling only: torch supplies device memory and the current HIP stream;
every step of encode, decode, GEMM and verification runs in the library's HIP kernels.
There is no CPU fallback: without the built library (or without a GPU) the calls raise.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_int, c_int32, c_size_t, c_uint8, c_uint32, c_uint64, c_void_p
from dataclasses import dataclass

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw12.so")
_LIB = None

OP_ENCODE, OP_DECODE, OP_GEMM, OP_GEMM_BF16, OP_VERIFY, OP_GEMM_GROUP, OP_VERIFY2, OP_GEMM_F8 = \
    0, 1, 2, 3, 4, 5, 6, 7
MAX_M = 128
MAX_GROUP = 4
STATUS = {0: "W12_OK", -1: "W12_ERR_NULL", -2: "W12_ERR_SHAPE", -3: "W12_ERR_RANGE",
          -4: "W12_ERR_FORMAT", -5: "W12_ERR_WORKSPACE", -6: "W12_ERR_HIP", -7: "W12_ERR_ALIGN"}
EXPORTS = ("w12_tiles_bytes", "w12_workspace_bytes", "w12_workspace_init", "w12_encode_count",
           "w12_encode", "w12_decode", "w12_gemm", "w12_gemm_group", "w12_gemm_rms",
           "w12_gemm_group_rms", "w12_gemm_bf16", "w12_bf16_tile",
           "w12_gemm_bf16_tiled", "w12_lmhead_verify", "w12_lmhead_verify_batched",
           "w12_logits_f32",
           "w12_rms_rescale", "w12_status_str", "w12_version", "w12_gemm_noalloc", "w12_stream_read",
           "w12_screen_bytes", "w12_screen_encode", "w12_lmhead_verify2", "w12_lmhead_verify2_batched",
           "w12_screen_logits_f32", "w12_f8_tile", "w12_gemm_f8", "w12_gemm_f8_group",
           "w12_gemm_f8_rms", "w12_gemm_f8_group_rms")
NOALLOC_SCRATCH_BYTES = 32 << 20   # W12_NOALLOC_SCRATCH_BYTES
ENCODE_TOTAL_OFFSET = 2112   # W12_ENCODE_TOTAL_OFFSET: true escape count in an encode workspace


class W12Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS.get(status, status)} ({status_str(status)})")


class W12Desc(ctypes.Structure):
    _fields_ = [("n", c_uint64), ("k", c_uint64), ("n_esc", c_uint64),
                ("codebook", c_uint8 * 16), ("e_max", c_uint8), ("reserved", c_uint8 * 7),
                ("tiles", c_void_p), ("esc_off", c_void_p), ("esc", c_void_p)]


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load libw12.so; raises if it has not been built (no silent fallback)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run "
                               "`python -m lossless_bit_weight_w12_amd.build` first")
        # torch ships its own HIP runtime (soname libamdhip64.so.7, the one libw12.so needs).
        # Loaded first, it is the runtime the library binds to; the other way round the
        # process would hold two HIP runtimes, and the library's launches on torch's
        # streams and memory would fail.
        import torch  # noqa: F401
        L = ctypes.CDLL(_LIB_PATH)
        L.w12_tiles_bytes.restype = c_size_t
        L.w12_tiles_bytes.argtypes = [c_uint64, c_uint64]
        L.w12_workspace_bytes.restype = c_size_t
        L.w12_workspace_bytes.argtypes = [c_int, c_uint32, c_uint64, c_uint64]
        L.w12_workspace_init.restype = c_int32
        L.w12_workspace_init.argtypes = [c_void_p, c_size_t, c_void_p]
        L.w12_encode_count.restype = c_int32
        L.w12_encode_count.argtypes = [c_void_p, c_uint64, c_uint64, c_void_p, c_void_p, c_void_p,
                                       c_void_p, c_size_t, c_void_p]
        L.w12_encode.restype = c_int32
        L.w12_encode.argtypes = [c_void_p, ctypes.POINTER(W12Desc), c_void_p, c_size_t, c_void_p]
        L.w12_decode.restype = c_int32
        L.w12_decode.argtypes = [ctypes.POINTER(W12Desc), c_void_p, c_void_p]
        L.w12_gemm.restype = c_int32
        L.w12_gemm.argtypes = [c_void_p, c_uint32, ctypes.POINTER(W12Desc), c_void_p, c_void_p,
                               c_size_t, c_void_p]
        L.w12_gemm_group.restype = c_int32
        L.w12_gemm_group.argtypes = [c_void_p, c_uint32, c_void_p, c_uint32, c_void_p, c_void_p,
                                     c_size_t, c_void_p]
        L.w12_gemm_noalloc.restype = c_int32
        L.w12_gemm_noalloc.argtypes = [c_void_p, c_uint32, ctypes.POINTER(W12Desc), c_void_p, c_void_p]
        L.w12_stream_read.restype = c_int32
        L.w12_stream_read.argtypes = [c_void_p, c_uint64, c_uint32, c_void_p, c_void_p]
        L.w12_gemm_rms.restype = c_int32
        L.w12_gemm_rms.argtypes = L.w12_gemm.argtypes
        L.w12_gemm_group_rms.restype = c_int32
        L.w12_gemm_group_rms.argtypes = L.w12_gemm_group.argtypes
        L.w12_gemm_bf16.restype = c_int32
        L.w12_gemm_bf16.argtypes = [c_void_p, c_uint32, c_void_p, c_uint64, c_uint64, c_void_p,
                                    c_void_p, c_size_t, c_void_p]
        L.w12_bf16_tile.restype = c_int32
        L.w12_bf16_tile.argtypes = [c_void_p, c_uint64, c_uint64, c_void_p, c_void_p]
        L.w12_gemm_bf16_tiled.restype = c_int32
        L.w12_gemm_bf16_tiled.argtypes = [c_void_p, c_uint32, c_void_p, c_uint64, c_uint64,
                                          c_void_p, c_void_p, c_size_t, c_void_p]
        L.w12_f8_tile.restype = c_int32
        L.w12_f8_tile.argtypes = [c_void_p, c_uint64, c_uint64, c_void_p, c_void_p]
        L.w12_gemm_f8.restype = c_int32
        L.w12_gemm_f8.argtypes = [c_void_p, c_uint32, c_void_p, c_void_p, c_uint64, c_uint64,
                                  c_void_p, c_void_p, c_size_t, c_void_p]
        L.w12_gemm_f8_group.restype = c_int32
        L.w12_gemm_f8_group.argtypes = [c_void_p, c_uint32, c_void_p, c_void_p, c_void_p, c_uint32,
                                        c_uint64, c_void_p, c_void_p, c_size_t, c_void_p]
        L.w12_gemm_f8_rms.restype = c_int32
        L.w12_gemm_f8_rms.argtypes = L.w12_gemm_f8.argtypes
        L.w12_gemm_f8_group_rms.restype = c_int32
        L.w12_gemm_f8_group_rms.argtypes = L.w12_gemm_f8_group.argtypes
        L.w12_lmhead_verify.restype = c_int32
        L.w12_lmhead_verify.argtypes = [c_void_p, c_uint32, ctypes.POINTER(W12Desc), c_void_p,
                                        c_uint32, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.w12_lmhead_verify_batched.restype = c_int32
        L.w12_lmhead_verify_batched.argtypes = [c_void_p, c_uint32, ctypes.POINTER(W12Desc), c_void_p,
                                                c_void_p, c_uint32, c_void_p, c_void_p, c_void_p,
                                                c_void_p, c_size_t, c_void_p]
        L.w12_logits_f32.restype = c_int32
        L.w12_logits_f32.argtypes = [c_void_p, c_uint32, ctypes.POINTER(W12Desc), c_void_p,
                                     c_void_p, c_void_p, c_size_t, c_void_p]
        L.w12_screen_bytes.restype = c_size_t
        L.w12_screen_bytes.argtypes = [c_uint64, c_uint64]
        L.w12_screen_encode.restype = c_int32
        L.w12_screen_encode.argtypes = [c_void_p, c_uint64, c_uint64, c_void_p, c_size_t, c_void_p]
        L.w12_lmhead_verify2.restype = c_int32
        L.w12_lmhead_verify2.argtypes = [c_void_p, c_uint32, ctypes.POINTER(W12Desc), c_void_p,
                                         c_void_p, c_uint32, c_void_p, c_void_p, c_void_p,
                                         c_size_t, c_void_p]
        L.w12_lmhead_verify2_batched.restype = c_int32
        L.w12_lmhead_verify2_batched.argtypes = [c_void_p, c_uint32, ctypes.POINTER(W12Desc),
                                                 c_void_p, c_void_p, c_void_p, c_uint32, c_void_p,
                                                 c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.w12_screen_logits_f32.restype = c_int32
        L.w12_screen_logits_f32.argtypes = [c_void_p, c_uint32, ctypes.POINTER(W12Desc), c_void_p,
                                            c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]
        L.w12_rms_rescale.restype = c_int32
        L.w12_rms_rescale.argtypes = [c_void_p, c_uint32, c_uint64, c_void_p, c_void_p]
        L.w12_status_str.restype = ctypes.c_char_p
        L.w12_status_str.argtypes = [c_int32]
        L.w12_version.restype = c_uint32
        L.w12_version.argtypes = []
        _LIB = L
    return _LIB


def status_str(s: int) -> str:
    return lib().w12_status_str(int(s)).decode()


def _check(fn: str, st: int):
    if st != 0:
        raise W12Error(fn, st)


def tiles_bytes(n: int, k: int) -> int:
    return int(lib().w12_tiles_bytes(n, k))


def workspace_bytes(op: int, m: int, n: int, k: int) -> int:
    return int(lib().w12_workspace_bytes(op, m, n, k))


# ----------------------------------------------------------------------------- torch glue
def _torch():
    import torch
    return torch


def _stream(dev):
    return c_void_p(_torch().cuda.current_stream(dev).cuda_stream)


def _ptr(t) -> c_void_p:
    return c_void_p(t.data_ptr())


def _as_bits(t):
    """View a BF16 / int16 / uint16 CUDA tensor as 16-bit storage (no copy)."""
    torch = _torch()
    if not t.is_cuda:
        raise ValueError("W12 calls need CUDA (HIP) tensors")
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise ValueError(f"expected BF16 bits, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return t


_WS = {}


def workspace(nbytes: int, device, purpose: str = "gemm"):
    """A workspace of at least nbytes on `device`, cached per purpose ("gemm" for both
    GEMM entry points, "verify", "encode") so that calls of different kinds queued on
    one stream never share scratch memory; grown on demand."""
    torch = _torch()
    dev = torch.device(device)
    key = (dev.index if dev.index is not None else torch.cuda.current_device(), purpose)
    buf = _WS.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=dev)
        _WS[key] = buf
    return buf


@dataclass
class W12Tensor:
    """A W12-encoded weight [n, k] resident on the GPU."""
    n: int
    k: int
    n_esc: int
    codebook: tuple
    e_max: int
    tiles: object      # torch.uint8 [tiles_bytes]
    esc_off: object    # torch.int32 [n/16 + 1]
    esc: object        # torch.int32 [max(n_esc, 1)]

    def desc(self) -> W12Desc:
        d = W12Desc()
        d.n, d.k, d.n_esc = self.n, self.k, self.n_esc
        for i, c in enumerate(self.codebook):
            d.codebook[i] = c
        d.e_max = self.e_max
        d.tiles = self.tiles.data_ptr()
        d.esc_off = self.esc_off.data_ptr()
        d.esc = self.esc.data_ptr()
        return d

    @property
    def device(self):
        return self.tiles.device

    def nbytes(self) -> int:
        """Bytes of the format: tiles + escapes + offsets + the 64-byte header."""
        return self.tiles.numel() + 4 * self.n_esc + 4 * (self.n // 16 + 1) + 64

    def bits_per_weight(self) -> float:
        return 8.0 * self.nbytes() / (self.n * self.k)


def encode(w) -> W12Tensor:
    """Encode BF16 weights w [n, k] (CUDA) to W12 on the same device."""
    torch = _torch()
    w = _as_bits(w)
    n, k = w.shape
    L = lib()
    dev = w.device
    ws = workspace(workspace_bytes(OP_ENCODE, 1, n, k), dev, "encode")
    cb = (c_uint8 * 16)()
    emax = c_uint8()
    nesc = c_uint64()
    s = _stream(dev)
    _check("w12_encode_count", L.w12_encode_count(_ptr(w), n, k, ctypes.byref(cb), ctypes.byref(emax),
                                                  ctypes.byref(nesc), _ptr(ws), ws.numel(), s))
    t = W12Tensor(n=n, k=k, n_esc=int(nesc.value), codebook=tuple(cb), e_max=int(emax.value),
                  tiles=torch.empty(tiles_bytes(n, k), dtype=torch.uint8, device=dev),
                  esc_off=torch.empty(n // 16 + 1, dtype=torch.int32, device=dev),
                  esc=torch.empty(max(int(nesc.value), 1), dtype=torch.int32, device=dev))
    d = t.desc()
    _check("w12_encode", L.w12_encode(_ptr(w), ctypes.byref(d), _ptr(ws), ws.numel(), s))
    return t


def decode(t: W12Tensor, out=None):
    torch = _torch()
    if out is None:
        out = torch.empty((t.n, t.k), dtype=torch.bfloat16, device=t.device)
    d = t.desc()
    _check("w12_decode", lib().w12_decode(ctypes.byref(d), _ptr(_as_bits(out)), _stream(t.device)))
    return out


@dataclass
class F8Tensor:
    """An FP8 weight [n, k] of an FP8 target resident on the GPU: E4M3 codes in the GEMM's
    2 KB tiles (w12_f8_tile) and FP32 scales per 128 x 128 block [ceil(n/128), k/128]."""
    n: int
    k: int
    tiles: object      # torch.uint8 [n*k]
    scale: object      # torch.float32 [ceil(n/128), k/128]

    def nbytes(self) -> int:
        return self.tiles.numel() + 4 * self.scale.numel()


def f8_encode(q, scale) -> F8Tensor:
    """F8Tensor of row-major E4M3 codes q [n, k] (uint8, CUDA) and their block scales."""
    torch = _torch()
    n, k = q.shape
    if scale.dtype != torch.float32 or tuple(scale.shape) != ((n + 127) // 128, k // 128):
        raise ValueError("f8_encode: scale must be float32 [ceil(n/128), k/128]")
    return F8Tensor(n, k, f8_tile(q), scale.contiguous())


def gemm(x, t, out=None, rms: bool = False):
    """y = x . W^T, x BF16 [m, k] (m <= MAX_M), y BF16 [m, n].  rms: each output row divided
    by the RMS of its x row (w12_gemm_rms).  A GEMM is routed by its weight's format: a
    W12Tensor to w12_gemm, an F8Tensor (the weight of an FP8 target) to w12_gemm_f8 (FP8 GEMM
    routing, review page "The mechanisms it found")."""
    torch = _torch()
    if isinstance(t, F8Tensor):
        return gemm_f8(x, t.tiles, t.scale, t.n, t.k, out, rms=rms)
    x = _as_bits(x)
    m = x.shape[0]
    if x.shape[1] != t.k:
        raise ValueError(f"x has {x.shape[1]} columns, W has k = {t.k}")
    if out is None:
        out = torch.empty((m, t.n), dtype=torch.bfloat16, device=x.device)
    ws = workspace(max(workspace_bytes(OP_GEMM, m, t.n, t.k), 256), x.device)
    d = t.desc()
    fn = "w12_gemm_rms" if rms else "w12_gemm"
    _check(fn, getattr(lib(), fn)(_ptr(x), m, ctypes.byref(d), _ptr(_as_bits(out)), _ptr(ws),
                                  ws.numel(), _stream(x.device)))
    return out


def gemm_noalloc(x, t: W12Tensor, out=None):
    """y = x . W^T through w12_gemm_noalloc: the library's own fixed scratch array instead
    of a workspace (for callers that cannot allocate; `out` must then be given)."""
    torch = _torch()
    x = _as_bits(x)
    m = x.shape[0]
    if x.shape[1] != t.k:
        raise ValueError(f"x has {x.shape[1]} columns, W has k = {t.k}")
    if out is None:
        out = torch.empty((m, t.n), dtype=torch.bfloat16, device=x.device)
    d = t.desc()
    _check("w12_gemm_noalloc", lib().w12_gemm_noalloc(_ptr(x), m, ctypes.byref(d), _ptr(_as_bits(out)),
                                                      _stream(x.device)))
    return out


def stream_read(buf, offset: int, nbytes: int, workgroups: int, sink):
    """The streaming-read probe (w12_stream_read) over bytes [offset, offset + nbytes) of the
    uint8 device tensor buf; sink: int32 device tensor of at least 4 * workgroups."""
    if offset < 0 or offset + nbytes > buf.numel() or sink.numel() < 4 * workgroups:
        raise ValueError("stream_read: range outside buf, or sink too small")
    _check("w12_stream_read", lib().w12_stream_read(c_void_p(buf.data_ptr() + offset), nbytes,
                                                    workgroups, _ptr(sink), _stream(buf.device)))


def _group_args(x, ts, outs):
    torch = _torch()
    x = _as_bits(x)
    m = x.shape[0]
    if not 1 <= len(ts) <= MAX_GROUP:
        raise ValueError(f"a group holds 1..{MAX_GROUP} weights")
    if any(t.k != x.shape[1] for t in ts):
        raise ValueError("every weight of a group must have k = x.shape[1]")
    if outs is None:
        outs = [torch.empty((m, t.n), dtype=torch.bfloat16, device=x.device) for t in ts]
    descs = [t.desc() for t in ts]
    darr = (ctypes.POINTER(W12Desc) * len(ts))(*[ctypes.pointer(d) for d in descs])
    yarr = (c_void_p * len(ts))(*[_as_bits(o).data_ptr() for o in outs])
    ws = workspace(max(workspace_bytes(OP_GEMM_GROUP, m, sum(t.n for t in ts), ts[0].k), 256),
                   x.device)
    args = (_ptr(x), m, ctypes.cast(darr, c_void_p), len(ts), ctypes.cast(yarr, c_void_p), _ptr(ws),
            ws.numel(), _stream(x.device))
    return args, outs, (x, ts, outs, ws, descs, darr, yarr)


def gemm_group(x, ts, outs=None, rms: bool = False):
    """y_i = x . W_i^T for the weights ts (1..4, same k) in one launch per codebook kind;
    rms as for gemm (w12_gemm_group_rms).  A group of F8Tensors goes to w12_gemm_f8_group."""
    if ts and all(isinstance(t, F8Tensor) for t in ts):
        return gemm_f8_group(x, [(t.tiles, t.scale, t.n) for t in ts], ts[0].k, outs, rms=rms)
    if any(isinstance(t, F8Tensor) for t in ts):
        raise ValueError("gemm_group: a group holds W12 weights or FP8 weights, not both")
    args, outs, keep = _group_args(x, ts, outs)
    fn = "w12_gemm_group_rms" if rms else "w12_gemm_group"
    _check(fn, getattr(lib(), fn)(*args))
    return outs


def gemm_bf16(x, w, out=None):
    """The same kernel family on plain BF16 weights w [n, k]."""
    torch = _torch()
    x = _as_bits(x)
    w = _as_bits(w)
    m = x.shape[0]
    n, k = w.shape
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    ws = workspace(max(workspace_bytes(OP_GEMM_BF16, m, n, k), 256), x.device)
    _check("w12_gemm_bf16", lib().w12_gemm_bf16(_ptr(x), m, _ptr(w), n, k, _ptr(_as_bits(out)),
                                                _ptr(ws), ws.numel(), _stream(x.device)))
    return out


def bf16_tile(w):
    """4 KB-tiled copy of BF16 weights w [n, k] (the second baseline's layout)."""
    torch = _torch()
    w = _as_bits(w)
    n, k = w.shape
    out = torch.empty(n * k * 2, dtype=torch.uint8, device=w.device)
    _check("w12_bf16_tile", lib().w12_bf16_tile(_ptr(w), n, k, _ptr(out), _stream(w.device)))
    return out


def gemm_bf16_tiled(x, w_tiled, n: int, k: int, out=None):
    """The same kernel family on 4 KB-tiled BF16 weights (from bf16_tile)."""
    torch = _torch()
    x = _as_bits(x)
    m = x.shape[0]
    if x.shape[1] != k or w_tiled.numel() * w_tiled.element_size() != 2 * n * k:
        raise ValueError("gemm_bf16_tiled: x must be [m, k] and w_tiled n*k*2 bytes")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    ws = workspace(max(workspace_bytes(OP_GEMM_BF16, m, n, k), 256), x.device)
    _check("w12_gemm_bf16_tiled", lib().w12_gemm_bf16_tiled(
        _ptr(x), m, _ptr(w_tiled), n, k, _ptr(_as_bits(out)), _ptr(ws), ws.numel(), _stream(x.device)))
    return out


def f8_tile(q):
    """2 KB-tiled copy of FP8 E4M3 codes q [n, k] (uint8 storage) for gemm_f8."""
    torch = _torch()
    if not q.is_cuda or q.dtype != torch.uint8 or not q.is_contiguous() or q.dim() != 2:
        raise ValueError("f8_tile: q must be a contiguous uint8 CUDA tensor [n, k]")
    n, k = q.shape
    out = torch.empty(n * k, dtype=torch.uint8, device=q.device)
    _check("w12_f8_tile", lib().w12_f8_tile(_ptr(q), n, k, _ptr(out), _stream(q.device)))
    return out


def gemm_f8(x, q_tiled, scale, n: int, k: int, out=None, rms: bool = False):
    """y = x . W^T for the FP8 weight W = E4M3(q) * block scale: q_tiled from f8_tile,
    scale float32 [ceil(n/128), k/128].  rms: each output row divided by the RMS of its x
    row (w12_gemm_f8_rms)."""
    torch = _torch()
    x = _as_bits(x)
    m = x.shape[0]
    if x.shape[1] != k or q_tiled.numel() * q_tiled.element_size() != n * k:
        raise ValueError("gemm_f8: x must be [m, k] and q_tiled n*k bytes")
    if (not scale.is_cuda or scale.dtype != torch.float32 or not scale.is_contiguous()
            or scale.numel() != ((n + 127) // 128) * (k // 128)):
        raise ValueError("gemm_f8: scale must be a contiguous float32 CUDA tensor "
                         "[ceil(n/128), k/128]")
    if out is None:
        out = torch.empty((m, n), dtype=torch.bfloat16, device=x.device)
    ws = workspace(max(workspace_bytes(OP_GEMM_F8, m, n, k), 256), x.device)
    fn = "w12_gemm_f8_rms" if rms else "w12_gemm_f8"
    _check(fn, getattr(lib(), fn)(
        _ptr(x), m, _ptr(q_tiled), _ptr(scale), n, k, _ptr(_as_bits(out)), _ptr(ws), ws.numel(),
        _stream(x.device)))
    return out


def _f8_group_args(x, weights, k: int, outs):
    torch = _torch()
    x = _as_bits(x)
    m = x.shape[0]
    if x.shape[1] != k or not 1 <= len(weights) <= MAX_GROUP:
        raise ValueError("gemm_f8_group: x must be [m, k] and 1..MAX_GROUP weights given")
    for qt, sc, n in weights:
        if qt.numel() * qt.element_size() != n * k or sc.dtype != torch.float32 or \
                not sc.is_contiguous() or sc.numel() != ((n + 127) // 128) * (k // 128):
            raise ValueError("gemm_f8_group: each weight is (q_tiled of n*k bytes, float32 "
                             "scale [ceil(n/128), k/128], n)")
    if outs is None:
        outs = [torch.empty((m, n), dtype=torch.bfloat16, device=x.device) for _, _, n in weights]
    nw = len(weights)
    ptrs = (c_void_p * nw)(*[qt.data_ptr() for qt, _, _ in weights])
    scs = (c_void_p * nw)(*[sc.data_ptr() for _, sc, _ in weights])
    ns = (c_uint64 * nw)(*[n for _, _, n in weights])
    ys = (c_void_p * nw)(*[_as_bits(o).data_ptr() for o in outs])
    n_total = sum(n for _, _, n in weights)
    ws = workspace(max(workspace_bytes(OP_GEMM_GROUP, m, n_total, k), 256), x.device)
    args = (_ptr(x), m, ctypes.cast(ptrs, c_void_p), ctypes.cast(scs, c_void_p),
            ctypes.cast(ns, c_void_p), nw, k, ctypes.cast(ys, c_void_p), _ptr(ws), ws.numel(),
            _stream(x.device))
    return args, outs, (x, weights, outs, ws, ptrs, scs, ns, ys)


def gemm_f8_group(x, weights, k: int, outs=None, rms: bool = False):
    """One launch over up to MAX_GROUP FP8 weights that read x: weights is a list of
    (q_tiled, scale, n) as gemm_f8 takes them; returns the outputs [m, n_i].  rms as for
    gemm_f8 (w12_gemm_f8_group_rms)."""
    args, outs, _keep = _f8_group_args(x, weights, k, outs)
    fn = "w12_gemm_f8_group_rms" if rms else "w12_gemm_f8_group"
    _check(fn, getattr(lib(), fn)(*args))
    return outs


def lmhead_verify(x, t: W12Tensor, draft, argmax_out=None, accepted_out=None):
    """Exact-logit argmax per row (lowest index on ties) and accepted-prefix length."""
    torch = _torch()
    x = _as_bits(x)
    m = x.shape[0]
    if argmax_out is None:
        argmax_out = torch.empty(m, dtype=torch.int32, device=x.device)
    if accepted_out is None:
        accepted_out = torch.empty(1, dtype=torch.int32, device=x.device)
    n_draft = int(draft.numel())
    ws = workspace(workspace_bytes(OP_VERIFY, m, t.n, t.k), x.device, "verify")
    d = t.desc()
    _check("w12_lmhead_verify", lib().w12_lmhead_verify(
        _ptr(x), m, ctypes.byref(d), _ptr(draft) if n_draft else None, n_draft, _ptr(argmax_out),
        _ptr(accepted_out), _ptr(ws), ws.numel(), _stream(x.device)))
    return argmax_out, accepted_out


def _batched_checked(x, t: W12Tensor, req_off, req_ndraft, draft, argmax_out, accepted_out):
    """Validated batched-verification tensors (the outputs allocated when not given)."""
    torch = _torch()
    x = _as_bits(x)
    m = x.shape[0]
    n_req = int(req_ndraft.numel())
    for name, a, size in (("req_off", req_off, n_req + 1), ("req_ndraft", req_ndraft, n_req),
                          ("draft", draft, m)):
        if a.dtype != torch.int32 or a.numel() != size or a.device != x.device:
            raise ValueError(f"lmhead_verify_batched: {name} must be int32 [{size}] on {x.device}")
    if argmax_out is None:
        argmax_out = torch.empty(m, dtype=torch.int32, device=x.device)
    if accepted_out is None:
        accepted_out = torch.empty(n_req, dtype=torch.int32, device=x.device)
    return x, m, n_req, argmax_out, accepted_out


def _batched_args(x, t: W12Tensor, req_off, req_ndraft, draft, argmax_out, accepted_out):
    x, m, n_req, argmax_out, accepted_out = _batched_checked(x, t, req_off, req_ndraft, draft,
                                                             argmax_out, accepted_out)
    ws = workspace(workspace_bytes(OP_VERIFY, m, t.n, t.k), x.device, "verify")
    d = t.desc()
    args = (_ptr(x), m, ctypes.byref(d), _ptr(req_off), _ptr(req_ndraft), n_req, _ptr(draft),
            _ptr(argmax_out), _ptr(accepted_out), _ptr(ws), ws.numel(), _stream(x.device))
    return args, (x, t, req_off, req_ndraft, draft, argmax_out, accepted_out, ws, d)


def lmhead_verify_batched(x, t: W12Tensor, req_off, req_ndraft, draft, argmax_out=None,
                          accepted_out=None):
    """Several requests verified in one pass: request r owns rows req_off[r] ..
    req_off[r+1]-1 and drafts draft[req_off[r] + i] for i < req_ndraft[r] (int32 device
    tensors [n_req+1], [n_req], [m]).  Returns (argmax [m], accepted [n_req]); an invalid
    request entry gets accepted -1."""
    args, keep = _batched_args(x, t, req_off, req_ndraft, draft, argmax_out, accepted_out)
    _check("w12_lmhead_verify_batched", lib().w12_lmhead_verify_batched(*args))
    return keep[5], keep[6]


@dataclass
class ScreenCopy:
    """The screen copy of an LM head for two-level verification (w12_screen_encode):
    8-bit codes with a BF16 scale per 32 columns, plus the per-row bound constants."""
    n: int
    k: int
    buf: object        # torch.uint8 [w12_screen_bytes(n, k)]

    def nbytes(self) -> int:
        return int(self.buf.numel())


def screen_encode(w) -> ScreenCopy:
    """Screen copy of BF16 weights w [n, k] (CUDA) on the same device."""
    torch = _torch()
    w = _as_bits(w)
    n, k = w.shape
    nbytes = int(lib().w12_screen_bytes(n, k))
    if nbytes == 0:
        raise ValueError(f"screen copy needs n % 16 == 0, k % 128 == 0, 0 < k < 2^20 (got {n}x{k})")
    buf = torch.empty(nbytes, dtype=torch.uint8, device=w.device)
    _check("w12_screen_encode", lib().w12_screen_encode(_ptr(w), n, k, _ptr(buf), nbytes,
                                                        _stream(w.device)))
    return ScreenCopy(n=n, k=k, buf=buf)


def _verify2_ws(m: int, t: W12Tensor, dev):
    # zero-filled on allocation: its row tickets start at zero (every call leaves them so)
    return workspace(workspace_bytes(OP_VERIFY2, m, t.n, t.k), dev, "verify2")


def _check_screen(t: W12Tensor, sc: ScreenCopy):
    if (sc.n, sc.k) != (t.n, t.k):
        raise ValueError(f"screen copy is {sc.n}x{sc.k}, the head {t.n}x{t.k}")


def lmhead_verify2(x, t: W12Tensor, sc: ScreenCopy, draft, argmax_out=None, accepted_out=None):
    """Two-level verification: the same results as lmhead_verify, from the screen copy
    first and the W12 head for the logits it cannot rule out."""
    torch = _torch()
    _check_screen(t, sc)
    x = _as_bits(x)
    m = x.shape[0]
    if argmax_out is None:
        argmax_out = torch.empty(m, dtype=torch.int32, device=x.device)
    if accepted_out is None:
        accepted_out = torch.empty(1, dtype=torch.int32, device=x.device)
    n_draft = int(draft.numel())
    ws = _verify2_ws(m, t, x.device)
    d = t.desc()
    _check("w12_lmhead_verify2", lib().w12_lmhead_verify2(
        _ptr(x), m, ctypes.byref(d), _ptr(sc.buf), _ptr(draft) if n_draft else None, n_draft,
        _ptr(argmax_out), _ptr(accepted_out), _ptr(ws), ws.numel(), _stream(x.device)))
    return argmax_out, accepted_out


def _batched2_args(x, t: W12Tensor, sc: ScreenCopy, req_off, req_ndraft, draft, argmax_out,
                   accepted_out):
    _check_screen(t, sc)
    x, m, n_req, argmax_out, accepted_out = _batched_checked(x, t, req_off, req_ndraft, draft,
                                                             argmax_out, accepted_out)
    ws = _verify2_ws(m, t, x.device)
    d = t.desc()
    args = (_ptr(x), m, ctypes.byref(d), _ptr(sc.buf), _ptr(req_off), _ptr(req_ndraft), n_req,
            _ptr(draft), _ptr(argmax_out), _ptr(accepted_out), _ptr(ws), ws.numel(),
            _stream(x.device))
    return args, (x, t, sc, req_off, req_ndraft, draft, argmax_out, accepted_out, ws, d)


def lmhead_verify2_batched(x, t: W12Tensor, sc: ScreenCopy, req_off, req_ndraft, draft,
                           argmax_out=None, accepted_out=None):
    """Several requests in one two-level pass (requests as lmhead_verify_batched)."""
    args, keep = _batched2_args(x, t, sc, req_off, req_ndraft, draft, argmax_out, accepted_out)
    _check("w12_lmhead_verify2_batched", lib().w12_lmhead_verify2_batched(*args))
    return keep[6], keep[7]


def screen_logits_f32(x, t: W12Tensor, sc: ScreenCopy):
    """The screen logits z8^ [m, n] and their certified bounds [m, n] (FP32) from the first
    pass of the two-level verification."""
    torch = _torch()
    _check_screen(t, sc)
    x = _as_bits(x)
    m = x.shape[0]
    z = torch.empty((m, t.n), dtype=torch.float32, device=x.device)
    bnd = torch.empty((m, t.n), dtype=torch.float32, device=x.device)
    ws = _verify2_ws(m, t, x.device)
    d = t.desc()
    _check("w12_screen_logits_f32", lib().w12_screen_logits_f32(
        _ptr(x), m, ctypes.byref(d), _ptr(sc.buf), _ptr(z), _ptr(bnd), _ptr(ws), ws.numel(),
        _stream(x.device)))
    return z, bnd


def verify2_candidates(t: W12Tensor, m: int):
    """Per-row diagnostic counts of the last two-level verification on this device's
    workspace: int32 [m, 2] = (logits the screen could not rule out, those left after the
    FP64 recomputation; 1 means no exact sum was needed)."""
    torch = _torch()
    ws = _verify2_ws(m, t, t.device)
    return ws[4096:4096 + 8 * m].view(torch.int32).view(m, 2).clone()


def verify_candidates(t: W12Tensor, m: int):
    """Per-row diagnostic counts of the last verification on this device's workspace:
    int32 [m, 2] = (candidate logits screened in FP64, those left after the screen; 1
    means no exact sum was needed)."""
    torch = _torch()
    ws = workspace(workspace_bytes(OP_VERIFY, m, t.n, t.k), t.device, "verify")
    return ws[:8 * m].view(torch.int32).view(m, 2).clone()   # the counts open the workspace


def logits_f32(x, t: W12Tensor):
    """FP32 logits z^ [m, n] and error scales S [m, n] from the first pass of the
    verification (same kernels, same summation order).  S = X_m W_v rounded up, an upper
    bound of sum_k |x_k||w_vk| (Cauchy-Schwarz): W_v the first pass's bound of
    ||w_v||_2, X_m the second pass's bound of ||x_m||_2."""
    torch = _torch()
    x = _as_bits(x)
    m = x.shape[0]
    z = torch.empty((m, t.n), dtype=torch.float32, device=x.device)
    s = torch.empty((m, t.n), dtype=torch.float32, device=x.device)
    ws = workspace(workspace_bytes(OP_VERIFY, m, t.n, t.k), x.device, "verify")
    d = t.desc()
    _check("w12_logits_f32", lib().w12_logits_f32(_ptr(x), m, ctypes.byref(d), _ptr(z), _ptr(s),
                                                  _ptr(ws), ws.numel(), _stream(x.device)))
    return z, s


def rms_rescale(x, out=None):
    torch = _torch()
    x = _as_bits(x)
    m, k = x.shape
    if out is None:
        out = torch.empty_like(x)
    _check("w12_rms_rescale", lib().w12_rms_rescale(_ptr(x), m, k, _ptr(_as_bits(out)), _stream(x.device)))
    return out


# ----------------------------------------------------------------------------- prepared calls
class Prepared:
    """One library call with its arguments marshalled once (device pointers, descriptor,
    workspace, stream); calling it re-issues the call with no other Python work.  The
    tensors it refers to must stay alive, and the stream is the one current when it was
    prepared."""

    def __init__(self, name: str, fn, args, keep):
        self.name, self._fn, self._args, self._keep = name, fn, args, keep

    def __call__(self):
        st = self._fn(*self._args)
        if st != 0:
            raise W12Error(self.name, st)


def prepare_gemm(x, t: W12Tensor, out, rms: bool = False) -> Prepared:
    x, out = _as_bits(x), _as_bits(out)
    m = x.shape[0]
    if x.shape[1] != t.k or tuple(out.shape) != (m, t.n):
        raise ValueError("prepare_gemm: x must be [m, k] and out [m, n]")
    ws = workspace(max(workspace_bytes(OP_GEMM, m, t.n, t.k), 256), x.device)
    d = t.desc()
    args = (_ptr(x), m, ctypes.byref(d), _ptr(out), _ptr(ws), ws.numel(), _stream(x.device))
    fn = "w12_gemm_rms" if rms else "w12_gemm"
    return Prepared(fn, getattr(lib(), fn), args, (x, t, out, ws, d))


def prepare_gemm_group(x, ts, outs, rms: bool = False) -> Prepared:
    args, outs, keep = _group_args(x, ts, outs)
    fn = "w12_gemm_group_rms" if rms else "w12_gemm_group"
    return Prepared(fn, getattr(lib(), fn), args, keep)


def prepare_gemm_f8(x, q_tiled, scale, n: int, k: int, out, rms: bool = False) -> Prepared:
    x, out = _as_bits(x), _as_bits(out)
    m = x.shape[0]
    if x.shape[1] != k or tuple(out.shape) != (m, n) or q_tiled.numel() * q_tiled.element_size() != n * k:
        raise ValueError("prepare_gemm_f8: x must be [m, k], out [m, n], q_tiled n*k bytes")
    ws = workspace(max(workspace_bytes(OP_GEMM_F8, m, n, k), 256), x.device)
    args = (_ptr(x), m, _ptr(q_tiled), _ptr(scale), n, k, _ptr(out), _ptr(ws), ws.numel(),
            _stream(x.device))
    fn = "w12_gemm_f8_rms" if rms else "w12_gemm_f8"
    return Prepared(fn, getattr(lib(), fn), args, (x, q_tiled, scale, out, ws))


def prepare_gemm_f8_group(x, weights, k: int, outs, rms: bool = False) -> Prepared:
    args, outs, keep = _f8_group_args(x, weights, k, outs)
    fn = "w12_gemm_f8_group_rms" if rms else "w12_gemm_f8_group"
    return Prepared(fn, getattr(lib(), fn), args, keep)


def prepare_rms(x, out) -> Prepared:
    x, out = _as_bits(x), _as_bits(out)
    m, k = x.shape
    args = (_ptr(x), m, k, _ptr(out), _stream(x.device))
    return Prepared("w12_rms_rescale", lib().w12_rms_rescale, args, (x, out))


def prepare_verify(x, t: W12Tensor, draft, argmax_out, accepted_out) -> Prepared:
    x = _as_bits(x)
    m = x.shape[0]
    n_draft = int(draft.numel())
    ws = workspace(workspace_bytes(OP_VERIFY, m, t.n, t.k), x.device, "verify")
    d = t.desc()
    args = (_ptr(x), m, ctypes.byref(d), _ptr(draft) if n_draft else None, n_draft,
            _ptr(argmax_out), _ptr(accepted_out), _ptr(ws), ws.numel(), _stream(x.device))
    return Prepared("w12_lmhead_verify", lib().w12_lmhead_verify, args,
                    (x, t, draft, argmax_out, accepted_out, ws, d))


def prepare_verify2(x, t: W12Tensor, sc: ScreenCopy, draft, argmax_out, accepted_out) -> Prepared:
    _check_screen(t, sc)
    x = _as_bits(x)
    m = x.shape[0]
    n_draft = int(draft.numel())
    ws = _verify2_ws(m, t, x.device)
    d = t.desc()
    args = (_ptr(x), m, ctypes.byref(d), _ptr(sc.buf), _ptr(draft) if n_draft else None, n_draft,
            _ptr(argmax_out), _ptr(accepted_out), _ptr(ws), ws.numel(), _stream(x.device))
    return Prepared("w12_lmhead_verify2", lib().w12_lmhead_verify2, args,
                    (x, t, sc, draft, argmax_out, accepted_out, ws, d))


def prepare_verify2_batched(x, t: W12Tensor, sc: ScreenCopy, req_off, req_ndraft, draft,
                            argmax_out, accepted_out) -> Prepared:
    args, keep = _batched2_args(x, t, sc, req_off, req_ndraft, draft, argmax_out, accepted_out)
    return Prepared("w12_lmhead_verify2_batched", lib().w12_lmhead_verify2_batched, args, keep)


def prepare_verify_batched(x, t: W12Tensor, req_off, req_ndraft, draft, argmax_out,
                           accepted_out) -> Prepared:
    args, keep = _batched_args(x, t, req_off, req_ndraft, draft, argmax_out, accepted_out)
    return Prepared("w12_lmhead_verify_batched", lib().w12_lmhead_verify_batched, args, keep)
