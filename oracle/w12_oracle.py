"""CPU oracle for W12: the plain, slow, obviously-correct definition of every result
the HIP library computes.  TEST INFRASTRUCTURE ONLY: nothing in the product path
(the ``lossless_bit_weight_w12_amd`` package, its C-ABI library or kernels) may import,
call or link this file; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, tables or constants
generators with the HIP path.

What the pages fix, and where (pages are cited by title and section):

* "StargazerX0/SpecPilot" (hotrepo.ai repo digest), section "What it is": W12 is a
  12-bit weight format whose decode inside the GEMM is bit-exact, and decoding is
  greedy with the target model choosing every token.
* "SpecPilot" (fasttoolhub glossary), section "Differentiation": the 12-bit format is
  general and lossless.
* "SpecPilot: an agent doubled speculative decoding speed, and the 10.87x needs
  context" (ai.jakubjirak.com review), section "The mechanisms it found": about
  12.01-12.02 bits per weight on dense models, decoded in GEMM registers; 12 instead
  of 16 bits cuts weight traffic by a quarter; the LM head's argmax is certified
  exact.  Section "The caveats the README states": batched kernels reduce in another
  order, so near-ties can flip -- which is why argmax here is defined on exact logits.
* "StargazerX0/SpecPilot", section "Results and verification": each committed token
  must be the target's own choice (the accepted-prefix rule below).

The pages give no bit layout.  W12 v1 (defined here and implemented independently on
the GPU) is the plainest layout with 12 = 1 sign + 7 mantissa + 4 code bits per weight
and a per-tensor codebook (a per-group codebook would cost about one extra bit per
weight, contradicting the 12.01-12.02 figure):

  fields     BF16 b: s = b>>15, e = (b>>7)&0xFF, m = b&0x7F, sm = (s<<7)|m
  histogram  H[e] over all N*K elements (e = 0..255)
  codebook   the 16 exponents with the largest H[e], ties to the smaller e (H = 0 is
             eligible), then sorted ascending -> C[0..15]
  codes      code = j with C[j] = e; e not in C -> escape: code 0 is stored and the
             true exponent goes to the escape list
  tiles      W [N out, K in] row-major, N % 16 == 0, K % 128 == 0.  Tile (b, g)
             covers rows 16b..16b+15 and columns 128g..128g+127, 3072 bytes at offset
             (g*(N/16) + b)*3072 (column-major tile order: the tiles of one column of
             every row-block are adjacent).  Lane slot l = 0..63: r = l % 16, q = l // 16.
             Element t = 0..31 of slot l: j = t // 8, i = t % 8,
             kappa = 32j + 8q + i  (row 16b + r, column 128g + kappa).
             sm byte at 1024*(t // 16) + 16*l + (t % 16);
             code nibble in the little-endian u32 at 2048 + 16*l + 4*j, at bit
             4*(i // 2) + 16*(i % 2)  (even i in the low half-word, odd i in the high).
  escapes    u32 record (r<<28) | (k<<8) | e per escape; the records of row-block b
             are esc[esc_off[b] : esc_off[b+1]], sorted ascending by (k, r);
             esc_off[0] = 0, esc_off[N/16] = n_esc.
  header     64 bytes LE: "W12\\0", version 1 (u32), N, K, n_esc (u64), C[16],
             e_max (u8: largest exponent field < 255 present, 0 if none), 15 zero bytes.
  size       bytes = 3072*(N/16)*(K/128) + 4*n_esc + 4*(N/16 + 1) + 64
"""
from __future__ import annotations

from dataclasses import dataclass
import numpy as np

TILE_ROWS = 16
TILE_K = 128
TILE_BYTES = 3072
HEADER_BYTES = 64
# GEMM acceptance rule: |y - z| <= REL_TOL * sum_k |x_k||w_k| + ABS_TOL per element
REL_TOL = 2e-3
ABS_TOL = 1e-6


# ----------------------------------------------------------------------------- fields
def split_fields(w: np.ndarray):
    """Sign, exponent field, mantissa and the sign/mantissa byte of BF16 bit patterns."""
    b = np.asarray(w, dtype=np.uint16).astype(np.uint32)
    s = b >> 15
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    sm = (s << 7) | m
    return s, e, m, sm


def join_fields(sm: np.ndarray, e: np.ndarray) -> np.ndarray:
    """BF16 bits from the sm byte and the exponent field: (s<<15) | (e<<7) | m."""
    sm = np.asarray(sm, dtype=np.uint32)
    e = np.asarray(e, dtype=np.uint32)
    return (((sm >> 7) << 15) | (e << 7) | (sm & 0x7F)).astype(np.uint16)


def exponent_histogram(w: np.ndarray) -> np.ndarray:
    _, e, _, _ = split_fields(w.reshape(-1))
    return np.bincount(e.astype(np.int64), minlength=256).astype(np.int64)


def choose_codebook(hist: np.ndarray) -> np.ndarray:
    """Top-16 exponents by count, ties to the smaller exponent, returned ascending."""
    order = sorted(range(256), key=lambda ex: (-int(hist[ex]), ex))
    return np.array(sorted(order[:16]), dtype=np.uint8)


def finite_e_max(hist: np.ndarray) -> int:
    present = [ex for ex in range(255) if hist[ex] > 0]
    return max(present) if present else 0


# ----------------------------------------------------------------------------- layout
def slot_layout():
    """Per (lane slot l, element t): row r, column offset kappa, sm byte offset, code
    word offset and code bit position inside that word.  Arrays of shape [64, 32]."""
    l = np.arange(64)[:, None] * np.ones((1, 32), dtype=np.int64)
    t = np.ones((64, 1), dtype=np.int64) * np.arange(32)[None, :]
    r = l % 16
    q = l // 16
    j = t // 8
    i = t % 8
    kappa = 32 * j + 8 * q + i
    sm_pos = 1024 * (t // 16) + 16 * l + (t % 16)
    word_pos = 2048 + 16 * l + 4 * j
    bit = 4 * (i // 2) + 16 * (i % 2)
    return r, kappa, sm_pos, word_pos, bit


@dataclass
class W12Blob:
    n: int
    k: int
    codebook: np.ndarray      # uint8[16], ascending
    e_max: int
    tiles: np.ndarray         # uint8[(n/16)*(k/128)*3072]
    esc_off: np.ndarray       # uint32[n/16 + 1]
    esc: np.ndarray           # uint32[n_esc]

    @property
    def n_esc(self) -> int:
        return int(self.esc.size)


def check_shape(n: int, k: int):
    if n <= 0 or k <= 0 or n % TILE_ROWS or k % TILE_K or k >= (1 << 20):
        raise ValueError(f"W12 v1 needs N % 16 == 0, K % 128 == 0, 0 < K < 2^20 (got {n}x{k})")


# ----------------------------------------------------------------------------- encode
def encode(w: np.ndarray, rows_per_chunk: int = 4096, codebook=None) -> W12Blob:
    """W12 v1 encode of BF16 bits w [N, K] (uint16).

    The bytes of a row-block's tiles depend only on its 16 rows and the tensor's
    codebook, so passing the codebook of a larger tensor encodes a band of its row-blocks
    exactly as the whole-tensor encode would: the band's tiles are those of rows
    b0..b1-1 in every column (escape offsets then count from the band's start; e_max
    stays that of the rows given)."""
    w = np.ascontiguousarray(w, dtype=np.uint16)
    n, k = w.shape
    check_shape(n, k)
    hist = exponent_histogram(w)
    cb = choose_codebook(hist) if codebook is None else np.asarray(codebook, dtype=np.uint8)
    if cb.shape != (16,) or np.any(np.diff(cb.astype(np.int64)) <= 0):
        raise ValueError("codebook must be 16 strictly ascending exponents")
    code_of = np.full(256, -1, dtype=np.int64)
    code_of[cb.astype(np.int64)] = np.arange(16)
    nb, gk = n // TILE_ROWS, k // TILE_K
    r_ix, kap, sm_pos, word_pos, bit = slot_layout()
    tiles = np.zeros((nb, gk, TILE_BYTES), dtype=np.uint8)
    esc_parts = []
    rows_per_chunk = max(16, rows_per_chunk - rows_per_chunk % 16)
    for n0 in range(0, n, rows_per_chunk):
        n1 = min(n, n0 + rows_per_chunk)
        _, e, _, sm = split_fields(w[n0:n1])
        code = code_of[e]
        is_esc = code < 0
        code = np.where(is_esc, 0, code)
        b0, b1 = n0 // 16, n1 // 16
        # [blocks, 16 rows, gk, 128] -> [blocks, gk, 16, 128]
        sm4 = sm.reshape(b1 - b0, 16, gk, 128).transpose(0, 2, 1, 3)
        cd4 = code.reshape(b1 - b0, 16, gk, 128).transpose(0, 2, 1, 3)
        sm_slots = sm4[:, :, r_ix, kap]            # [blocks, gk, 64, 32]
        cd_slots = cd4[:, :, r_ix, kap]
        tb = tiles[b0:b1]
        tb[:, :, sm_pos.reshape(-1)] = sm_slots.reshape(b1 - b0, gk, -1).astype(np.uint8)
        # code words: 4 words of 8 nibbles per slot
        words = np.zeros((b1 - b0, gk, 64, 4), dtype=np.uint32)
        for t in range(32):
            words[:, :, :, t // 8] |= (cd_slots[:, :, :, t].astype(np.uint32)
                                       << np.uint32(bit[0, t]))
        wb = words.reshape(b1 - b0, gk, 64 * 4).astype("<u4").view(np.uint8)
        wb = wb.reshape(b1 - b0, gk, 64, 4, 4)     # [.., l, j, byte]
        for jj in range(4):
            for by in range(4):
                tb[:, :, 2048 + 16 * np.arange(64) + 4 * jj + by] = wb[:, :, :, jj, by]
        # escapes of this chunk, as (row, col, exponent)
        rr, cc = np.nonzero(is_esc)
        if rr.size:
            esc_parts.append((rr + n0, cc, e[rr, cc]))
    if esc_parts:
        rows = np.concatenate([p[0] for p in esc_parts]).astype(np.int64)
        cols = np.concatenate([p[1] for p in esc_parts]).astype(np.int64)
        exps = np.concatenate([p[2] for p in esc_parts]).astype(np.int64)
    else:
        rows = cols = exps = np.zeros(0, dtype=np.int64)
    blk = rows // 16
    rr = rows % 16
    order = np.lexsort((rr, cols, blk))            # by block, then k, then r
    blk, rr, cols, exps = blk[order], rr[order], cols[order], exps[order]
    esc = ((rr << 28) | (cols << 8) | exps).astype(np.uint32)
    counts = np.bincount(blk, minlength=nb) if blk.size else np.zeros(nb, dtype=np.int64)
    esc_off = np.zeros(nb + 1, dtype=np.uint32)
    esc_off[1:] = np.cumsum(counts)
    # stored column-major: tile (b, g) at (g*nb + b)*3072
    return W12Blob(n=n, k=k, codebook=cb, e_max=finite_e_max(hist),
                   tiles=np.ascontiguousarray(tiles.transpose(1, 0, 2)).reshape(-1),
                   esc_off=esc_off, esc=esc)


def band_tiles(tiles: np.ndarray, n: int, k: int, b0: int, b1: int) -> np.ndarray:
    """The tile bytes of row-blocks b0..b1-1 of an [n, k] tensor's (column-major) tile
    array, in the order a band encode of those rows stores them."""
    t = np.asarray(tiles).reshape(k // TILE_K, n // TILE_ROWS, TILE_BYTES)
    return np.ascontiguousarray(t[:, b0:b1]).reshape(-1)


# ----------------------------------------------------------------------------- decode
def decode(blob: W12Blob, blocks_per_chunk: int = 256) -> np.ndarray:
    """Inverse of encode: BF16 bits [N, K]."""
    n, k = blob.n, blob.k
    nb, gk = n // 16, k // 128
    r_ix, kap, sm_pos, word_pos, bit = slot_layout()
    tiles_all = blob.tiles.reshape(gk, nb, TILE_BYTES).transpose(1, 0, 2)   # [b, g, byte]
    out = np.empty((n, k), dtype=np.uint16)
    for b0 in range(0, nb, blocks_per_chunk):
        b1 = min(nb, b0 + blocks_per_chunk)
        cb = b1 - b0
        tiles = tiles_all[b0:b1]
        sm_slots = tiles[:, :, sm_pos.reshape(-1)].reshape(cb, gk, 64, 32).astype(np.uint32)
        wbytes = tiles[:, :, 2048:3072].reshape(cb, gk, 64, 4, 4).astype(np.uint32)
        words = (wbytes[..., 0] | (wbytes[..., 1] << 8) | (wbytes[..., 2] << 16)
                 | (wbytes[..., 3] << 24))                           # [cb, gk, 64, 4]
        codes = np.empty((cb, gk, 64, 32), dtype=np.uint32)
        for t in range(32):
            codes[:, :, :, t] = (words[:, :, :, t // 8] >> np.uint32(bit[0, t])) & 0xF
        e_slots = blob.codebook.astype(np.uint32)[codes]
        sm = np.empty((cb, gk, 16, 128), dtype=np.uint32)
        ex = np.empty((cb, gk, 16, 128), dtype=np.uint32)
        sm[:, :, r_ix, kap] = sm_slots
        ex[:, :, r_ix, kap] = e_slots
        sm = sm.transpose(0, 2, 1, 3).reshape(cb * 16, k)
        ex = ex.transpose(0, 2, 1, 3).reshape(cb * 16, k)
        for b in range(b0, b1):
            for rec in blob.esc[blob.esc_off[b]:blob.esc_off[b + 1]]:
                rec = int(rec)
                r, kk, e = rec >> 28, (rec >> 8) & 0xFFFFF, rec & 0xFF
                ex[16 * (b - b0) + r, kk] = e
        out[16 * b0:16 * b1] = join_fields(sm, ex)
    return out


# ----------------------------------------------------------------------------- sizes
def header(blob: W12Blob) -> bytes:
    h = bytearray(HEADER_BYTES)
    h[0:4] = b"W12\x00"
    h[4:8] = (1).to_bytes(4, "little")
    h[8:16] = blob.n.to_bytes(8, "little")
    h[16:24] = blob.k.to_bytes(8, "little")
    h[24:32] = blob.n_esc.to_bytes(8, "little")
    h[32:48] = bytes(blob.codebook.tolist())
    h[48] = blob.e_max
    return bytes(h)


def serialize(blob: W12Blob) -> bytes:
    return (header(blob) + blob.tiles.tobytes() + blob.esc_off.astype("<u4").tobytes()
            + blob.esc.astype("<u4").tobytes())


def blob_bytes(blob: W12Blob) -> int:
    return len(serialize(blob))


def bits_per_weight(blob: W12Blob) -> float:
    return 8.0 * blob_bytes(blob) / (blob.n * blob.k)


# ----------------------------------------------------------------------------- GEMM
def bf16_to_f64(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gemm_reference(x: np.ndarray, w: np.ndarray, rows_per_chunk: int = 8192):
    """z = x . W^T and S = |x| . |W|^T in float64 for BF16 bits x [M, K], w [N, K].
    Each BF16 product is exact in float64; the float64 sum is within K*2^-53*S of the
    exact value, negligible against the acceptance rule."""
    xf = bf16_to_f64(x)
    n = w.shape[0]
    z = np.empty((x.shape[0], n))
    s = np.empty((x.shape[0], n))
    for n0 in range(0, n, rows_per_chunk):
        wf = bf16_to_f64(w[n0:n0 + rows_per_chunk])
        z[:, n0:n0 + wf.shape[0]] = xf @ wf.T
        s[:, n0:n0 + wf.shape[0]] = np.abs(xf) @ np.abs(wf).T
    return z, s


def gemm_w12(x: np.ndarray, blob: W12Blob):
    """The W12 GEMM as the pages describe it: decode the weights bit-exactly, then the
    plain BF16 product (FP64 here)."""
    return gemm_reference(x, decode(blob))


def gemm_rows(x: np.ndarray, w_rows: np.ndarray):
    """z and S for selected weight rows (sampled checks at full size)."""
    return gemm_reference(x, w_rows)


def within_tolerance(y_bits: np.ndarray, z: np.ndarray, s: np.ndarray):
    """Literal acceptance |y - z| <= 2e-3*S + 1e-6 per element for BF16 outputs y."""
    y = bf16_to_f64(y_bits)
    return np.abs(y - z) <= REL_TOL * s + ABS_TOL


def bf16_round(v: np.ndarray) -> np.ndarray:
    """Round float64 values to BF16 (round to nearest, ties to even) directly, without
    an intermediate float32 rounding.  Returns uint16 bits.  Finite inputs only."""
    v = np.asarray(v, dtype=np.float64)
    mant, ex = np.frexp(v)                       # v = mant * 2^ex, 0.5 <= |mant| < 1
    step = np.maximum(ex - 8, -133)              # BF16 grid spacing exponent (subnormals: 2^-133)
    q = np.rint(np.ldexp(v, -step))              # exact scaling; rint = ties to even
    r = np.ldexp(q, step)
    r = np.where(np.abs(r) >= 2.0 ** 128, np.copysign(np.inf, v), r)
    b = r.astype(np.float32).view(np.uint32)     # exact: r has at most 8 significant bits
    return (b >> 16).astype(np.uint16)


def within_tolerance_rounded(y_bits: np.ndarray, z: np.ndarray, s: np.ndarray):
    """Rounding-aware acceptance: y is the BF16 rounding of some t with
    |t - z| <= 2e-3*S + 1e-6, i.e. RNE(z - tau) <= y <= RNE(z + tau) (RNE is monotone).
    A BF16 y that meets the literal rule is its own rounding (RNE(y) = y), so this set
    contains the literal one; it adds at most the half BF16 step that the final
    rounding of an in-tolerance accumulator can add.  Where one product dominates a
    row (|z| close to S) the BF16 step exceeds 2e-3*S and no BF16 value may meet the
    literal rule at all; this rule still accepts the roundings of in-tolerance sums."""
    tau = REL_TOL * s + ABS_TOL
    y = bf16_to_f64(y_bits)
    lo = bf16_to_f64(bf16_round(z - tau))
    hi = bf16_to_f64(bf16_round(z + tau))
    return (lo <= y) & (y <= hi)


def gemm_accept(y_bits: np.ndarray, z: np.ndarray, s: np.ndarray):
    """Per-element GEMM acceptance of a BF16 output: the tolerance bounds the FP32
    accumulation before its final round-to-nearest-even, so y is accepted iff it is the
    BF16 rounding of a value within 2e-3*S + 1e-6 of the exact z
    (within_tolerance_rounded; every y the literal rule accepts is accepted too)."""
    return within_tolerance_rounded(y_bits, z, s)


# ----------------------------------------------------------------------------- exact
def exact_parts(b: np.ndarray):
    """Integer form of finite BF16 values: value = sign * M * 2^E with
    normal (e >= 1): M = 128 + m, E = e - 134; zero/subnormal (e = 0): M = m, E = -133."""
    s, e, m, _ = split_fields(b)
    s = s.astype(np.int64)
    e = e.astype(np.int64)
    m = m.astype(np.int64)
    if np.any(e == 255):
        raise ValueError("exact logits are defined for finite BF16 only")
    mant = np.where(e > 0, m + 128, m)
    ex = np.where(e > 0, e - 134, -133)
    sign = 1 - 2 * s
    return sign, mant, ex


EXACT_SHIFT = 266   # -(smallest product exponent): every product is an integer at 2^-266


def exact_logit(x_row: np.ndarray, w_row: np.ndarray) -> int:
    """Z = sum_k x_k * w_k * 2^266 as an exact Python integer."""
    sx, mx, ex = exact_parts(x_row)
    sw, mw, ew = exact_parts(w_row)
    prod = sx * sw * mx * mw                 # |prod| < 2^16
    sh = ex + ew + EXACT_SHIFT               # 0 .. 506
    total = 0
    for shv in np.unique(sh):
        part = int(prod[sh == shv].sum())    # |part| < K * 2^16, exact in int64
        total += part << int(shv)
    return total


def fp64_filter_width(k: int, s_max: float) -> float:
    """Width of the rigorous float64 filter of argmax_exact: any summation order of K
    products, each exact in float64, is within gamma*S of the exact sum with
    gamma = (K+2)*2^-52; two logits (the maximum's and a candidate's) each carry that
    error, so 2*gamma*max S covers every row."""
    return 2.0 * (k + 2) * 2.0 ** -52 * s_max


def argmax_exact(x: np.ndarray, w: np.ndarray, rows_per_chunk: int = 8192):
    """Per row m: the index v maximising the exact logit sum_k x[m,k]*W[v,k], lowest
    index on an exact tie.  Steps: float64 logits z64 and S64 for every v; a rigorous
    filter keeps v with z64_v >= max z64 - fp64_filter_width(K, max S64) (the float64
    error of any summation order is below gamma*S); exact integer logits of the
    survivors decide.  Returns (argmax int64[M], candidate counts)."""
    k = x.shape[1]
    z64, s64 = gemm_reference(x, w, rows_per_chunk)
    out = np.empty(x.shape[0], dtype=np.int64)
    ncand = np.empty(x.shape[0], dtype=np.int64)
    for mi in range(x.shape[0]):
        zmax = z64[mi].max()
        thr = zmax - fp64_filter_width(k, s64[mi].max())
        cand = np.nonzero(z64[mi] >= thr)[0]
        ncand[mi] = cand.size
        best_v, best_z = -1, None
        for v in cand:                        # ascending: lowest index kept on ties
            zv = exact_logit(x[mi], w[v])
            if best_z is None or zv > best_z:
                best_v, best_z = int(v), zv
        out[mi] = best_v
    return out, ncand


def accepted_length(argmax: np.ndarray, draft: np.ndarray) -> int:
    """Greedy verification: the number of leading draft tokens equal to the target's
    own choice (first mismatch position, or n_draft if none)."""
    for i in range(len(draft)):
        if int(argmax[i]) != int(draft[i]):
            return i
    return len(draft)


def accepted_lengths_batched(argmax: np.ndarray, draft: np.ndarray, row_off, n_draft):
    """Greedy verification of a batch of requests sharing one LM-head pass ("SpecPilot:
    an agent doubled speculative decoding speed, and the 10.87x needs context", sections
    "Where the numbers come from" -- batched rows with 16, 20 and 24 requests -- and "The
    mechanisms it found" -- per-request drafter block lengths, ragged drafts).  Request r
    owns rows row_off[r] .. row_off[r+1]-1; its draft tokens sit at the same rows, the
    first n_draft[r] of them.  Each request's accepted length is the single-request rule
    (accepted_length) on its own rows; requests do not see one another."""
    out = []
    for r in range(len(n_draft)):
        a, nd = int(row_off[r]), int(n_draft[r])
        out.append(accepted_length(argmax[a:a + nd], draft[a:a + nd]))
    return np.array(out, dtype=np.int64)


# ----------------------------------------------------------------------------- screen copy
# Two-level verification ("SpecPilot: an agent doubled speculative decoding speed, and the
# 10.87x needs context", section "The mechanisms it found": verification in two levels,
# with an 8-bit copy of the head; "SpecPilot" glossary, "Differentiation"): a first pass
# over an 8-bit copy of the LM head rules out the logits that cannot be the argmax, and
# only the rest are computed from the exact (W12) weights.  The pages give the idea and
# the bit width only.  Screen copy v1 (defined here; implemented independently on the GPU):
#
#   groups   32 consecutive columns of a row: group g holds columns 32g .. 32g+31
#   scale    s_vg = the smallest BF16 value >= (largest |w| over the group's finite
#            weights) / 127, and at least 2^-100 (so a group of zeros gets 2^-100)
#   code     q_vk = w_vk / s_vg rounded to the nearest integer, ties to even
#            (|q| <= 127 by the choice of s); 0 for a non-finite weight
#   tile     16 rows x 128 columns, 2176 bytes at (g*(N/16) + b)*2176 (column-major tile
#            order, as W12): the int8 code of element t of lane slot l (the W12 slot
#            layout: row r = l % 16, column 128g + 32(t//8) + 8(l//16) + t%8) at the W12
#            sign/mantissa byte position 1024*(t//16) + 16*l + t%16, then the tile's 64
#            scales, BF16 little-endian, row 4a+i (a, i = 0..3) and 32-column group j of
#            the tile at 2048 + 32a + 8i + 2j
#   rows     the per-row constants the screen's error bound needs are upper bounds of
#            ||r_v||_2 + gamma*||w^_v||_2 (r = w - w^, w^ = q*s); they are not unique
#            and are checked against the exact sums below, not stored here.
#
# The screen bound: for any x, z_v = sum_k x_k w_vk = z8_v + sum_k x_k r_vk with
# z8_v = sum_k x_k w^_vk, and |sum_k x_k r_vk| <= ||x||_2 ||r_v||_2 (Cauchy-Schwarz).  z8
# is evaluated in FP32 as sum_g s_vg (sum_{k in g} x_k q_vk): a 32-term sum of exact
# products per group (at most 31 additions), then one scaled addition per group into the
# running total (at most K/32 more), so each term passes through at most D = K/32 + 64
# additions (with slack); in any such order the result is within gamma*S8 (gamma =
# D*2^-23/(1 - D*2^-23), S8 = sum_k |x_k||w^_vk| <= ||x||_2 ||w^_v||_2) of z8, plus
# underflow terms.
SCREEN_GROUP = 32
SCREEN_QMAX = 127
SCREEN_S_MIN = 2.0 ** -100
SCREEN_TILE_BYTES = 2176


def bf16_round_up(v: np.ndarray) -> np.ndarray:
    """The smallest BF16 value >= v for positive finite float64 v in the normal BF16
    range, as uint16 bits: the significand rounded up to 8 bits."""
    v = np.asarray(v, dtype=np.float64)
    mant, ex = np.frexp(v)                                 # v = mant * 2^ex, 0.5 <= mant < 1
    r = np.ldexp(np.ceil(np.ldexp(mant, 8)), ex - 8)       # at most 8 significant bits
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def screen_encode(w: np.ndarray):
    """Screen copy v1 of BF16 bits w [N, K]: codes q (int8 [N, K]), scale bits (uint16
    [N, K/32]) and whether every weight of a row is finite (bool [N]).  The quotient
    w/s is correctly rounded in float64 and cannot cross or land on a half-integer it
    does not equal (w and s have 8-bit significands), so rint gives the exact
    round-to-nearest-even of w/s; likewise for the scale's quotient by 127."""
    n, k = w.shape
    check_shape(n, k)
    wf = bf16_to_f64(w).reshape(n, k // SCREEN_GROUP, SCREEN_GROUP)
    fin = np.isfinite(wf)
    wz = np.where(fin, wf, 0.0)
    amax = np.abs(wz).max(axis=2)
    s_bits = bf16_round_up(np.maximum(amax / SCREEN_QMAX, SCREEN_S_MIN))
    s = bf16_to_f64(s_bits)[:, :, None]
    q = np.rint(wz / s)
    return q.astype(np.int8).reshape(n, k), s_bits, fin.reshape(n, k).all(axis=1)


def screen_weights(q: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    """w^ = q * s in float64 (exact: a 7-bit integer times a BF16 value)."""
    n, k = q.shape
    s = bf16_to_f64(s_bits).reshape(n, k // SCREEN_GROUP, 1)
    return (q.astype(np.float64).reshape(n, k // SCREEN_GROUP, SCREEN_GROUP) * s).reshape(n, k)


def screen_pack(q: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    """Tile bytes of the screen copy (uint8 [(N/16)*(K/128)*2176]), layout above."""
    n, k = q.shape
    nb, gk = n // TILE_ROWS, k // TILE_K
    r, kappa, pos, _, _ = slot_layout()
    out = np.zeros((gk, nb, SCREEN_TILE_BYTES), dtype=np.uint8)
    qt = q.view(np.uint8).reshape(nb, TILE_ROWS, gk, TILE_K).transpose(2, 0, 1, 3)   # [g, b, r, kappa]
    out[:, :, pos.ravel()] = qt[:, :, r.ravel(), kappa.ravel()]
    st = s_bits.reshape(nb, TILE_ROWS, gk, 4).transpose(2, 0, 1, 3)                 # [g, b, row, j]
    sb = st.astype("<u2").view(np.uint8).reshape(gk, nb, TILE_ROWS, 4, 2)
    for row in range(TILE_ROWS):
        a, i = row // 4, row % 4
        for j in range(4):
            off = 2048 + 32 * a + 8 * i + 2 * j
            out[:, :, off:off + 2] = sb[:, :, row, j, :]
    return out.reshape(-1)


def screen_row_sums_exact(w_row: np.ndarray, q_row: np.ndarray, s_row_bits: np.ndarray):
    """Exact R2 = sum_k (w_k - w^_k)^2 and Q2 = sum_k w^_k^2 of one row with finite
    weights, as Python integers in units of 2^-266 (every BF16 value and every w^ is a
    multiple of 2^-133, and r = w - w^ is exact in float64: it has at most 8 significant
    bits)."""
    wf = bf16_to_f64(w_row)
    what = screen_weights(q_row[None, :], s_row_bits[None, :])[0]
    r = wf - what
    r2 = sum(int(v) ** 2 for v in np.ldexp(r, 133))
    q2 = sum(int(v) ** 2 for v in np.ldexp(what, 133))
    return r2, q2


def screen_gamma(k: int) -> float:
    """gamma of the screen bound for K columns (D = K/32 + 64 additions per term: one
    32-term group sum, then one scaled addition per group)."""
    d = (k // SCREEN_GROUP + 64) * 2.0 ** -23
    return d / (1.0 - d)


def screen_logits_reference(x: np.ndarray, q: np.ndarray, s_bits: np.ndarray):
    """z8 = x . w^T and S8 = |x| . |w^|^T in float64 for BF16 bits x [M, K] (each product
    is exact in float64: 8-bit x 15-bit significands)."""
    xf = bf16_to_f64(x)
    what = screen_weights(q, s_bits)
    return xf @ what.T, np.abs(xf) @ np.abs(what).T


# ----------------------------------------------------------------------------- FP8 GEMM
# FP8 GEMM routing ("SpecPilot: an agent doubled speculative decoding speed, and the
# 10.87x needs context", section "The mechanisms it found": FP8 GEMM routing is one of
# the batching mechanisms; "StargazerX0/SpecPilot", section "What it is": three of the
# batching settings run FP8 targets).  The pages give no format.  Reading taken here:
# the target's own FP8 weights in the usual checkpoint form, and BF16 activations --
#   codes    q[n][k], one OCP FP8 E4M3 byte per weight: sign bit, 4 exponent bits
#            (bias 7), 3 mantissa bits; exponent field 0 is subnormal (m/8 * 2^-6);
#            no infinities; S.1111.111 is NaN (the largest finite is 448)
#   scales   s[n // 128][k // 128], one FP32 value per 128 x 128 block
#   weight   W[n][k] = E4M3(q[n][k]) * s[n // 128][k // 128]
#   product  y = x . W^T, accepted by the same rule as every other GEMM here
#   tiles    16 rows x 128 columns, 2048 bytes at (g*(N/16) + b)*2048 (column-major
#            tile order, as W12): the code of element t of lane slot l (the W12 slot
#            layout) at the W12 sign/mantissa byte position 1024*(t//16) + 16*l + t%16.
# For such a target this product is the target's own (lossless): no weight is changed.
F8_TILE_BYTES = 2048
F8_BLOCK = 128


def f8_e4m3_to_f64(b: np.ndarray) -> np.ndarray:
    """Values of E4M3 bytes (float64; NaN for S.1111.111)."""
    b = np.asarray(b, dtype=np.uint8).astype(np.int64)
    sign = np.where(b >> 7, -1.0, 1.0)
    e = (b >> 3) & 0xF
    m = b & 0x7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    return np.where((e == 0xF) & (m == 0x7), np.nan, sign * mag)


def f8_weights(q: np.ndarray, s: np.ndarray) -> np.ndarray:
    """W = E4M3(q) * block scale in float64 (exact: a 4-bit significand times an FP32
    value).  q uint8 [N, K], s float32 [ceil(N/128), K/128]."""
    n, k = q.shape
    srow = np.asarray(s, dtype=np.float64)[np.arange(n) // F8_BLOCK]           # [N, K/128]
    return f8_e4m3_to_f64(q) * np.repeat(srow, F8_BLOCK, axis=1)[:, :k]


def f8_pack(q: np.ndarray) -> np.ndarray:
    """Tile bytes of FP8 codes q uint8 [N, K] (uint8 [(N/16)*(K/128)*2048]), layout above."""
    n, k = q.shape
    check_shape(n, k)
    nb, gk = n // TILE_ROWS, k // TILE_K
    r, kappa, pos, _, _ = slot_layout()
    out = np.zeros((gk, nb, F8_TILE_BYTES), dtype=np.uint8)
    qt = np.asarray(q, dtype=np.uint8).reshape(nb, TILE_ROWS, gk, TILE_K).transpose(2, 0, 1, 3)
    out[:, :, pos.ravel()] = qt[:, :, r.ravel(), kappa.ravel()]
    return out.reshape(-1)


def gemm_f8_reference(x: np.ndarray, q: np.ndarray, s: np.ndarray, rows_per_chunk: int = 8192):
    """z = x . W^T and S = |x| . |W|^T in float64 for BF16 bits x [M, K] and the FP8 weight
    (q, s).  Each product x*W has at most 8 + 4 + 24 significant bits, exact in float64;
    the float64 sum is within K*2^-53*S of the exact value."""
    if rows_per_chunk % F8_BLOCK:
        raise ValueError("rows_per_chunk must be a multiple of 128")
    xf = bf16_to_f64(x)
    n = q.shape[0]
    z = np.empty((x.shape[0], n))
    sa = np.empty((x.shape[0], n))
    for n0 in range(0, n, rows_per_chunk):
        n1 = min(n, n0 + rows_per_chunk)
        wf = f8_weights(q[n0:n1], s[n0 // F8_BLOCK:(n1 + F8_BLOCK - 1) // F8_BLOCK])
        z[:, n0:n1] = xf @ wf.T
        sa[:, n0:n1] = np.abs(xf) @ np.abs(wf).T
    return z, sa
