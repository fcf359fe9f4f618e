// The W12 decode/verification GEMM kernel family for gfx950 (MI355X).
//
// y[m][n] = sum_k x[m][k] * W[n][k] for m < M <= 32, W streamed once from HBM.
// W12 weights are decoded to BF16 pairs in registers ("StargazerX0/SpecPilot", "What
// it is": decoding happens bit-exactly inside the GEMM; review page, "The mechanisms
// it found": 12 instead of 16 bits per weight cuts the weight traffic by a quarter).
//
// A launch multiplies one x by up to kMaxSeg weights that share K (a group: q, k and
// v of a layer, or gate and up); their row-blocks are numbered consecutively and each
// wave looks up the weight its row-block belongs to (tiles, escapes, codebook, y).  A
// single GEMM is a group of one.
//
// Kernel shapes
//   k_gemm (wave columns): a workgroup of NWV waves owns RBW consecutive row-blocks and
//   a K-range [ga, gb) (blockIdx.y selects the split); wave w streams tile columns
//   ga+w, ga+w+NWV, ... with its own x column in LDS, so no workgroup barrier is needed;
//   the waves' partial sums meet in LDS at the end.
//   k_gemm_cs (column synchronous, MFMA): a workgroup of NW waves owns NW row-blocks,
//   one per wave; all waves walk the same columns and share each x column through LDS
//   (one barrier per column).
// Per tile, lane l (row r = l%16, k-group q = l/16) holds the 32 weights of its slot:
//   three coalesced 16-byte loads per lane (1 KB per wave instruction), unpacked into
//   16 BF16 pairs P[4j+p] = {w(k0+2p), w(k0+2p+1)} with k0 = 32j + 8q.  Those 8 BF16 of
//   group j are exactly the lane's A operand of v_mfma_f32_16x16x32_bf16 (row r,
//   k = 8q..8q+7 of the 32-wide step), and adjacent-k pairs for v_dot2_f32_bf16.
// m < W12_MFMA_MIN_M: VALU path, v_dot2 (2 MACs per instruction) with x pairs read from
//   LDS as broadcast ds_read_b128; partial sums are reduced across the 4 lanes that
//   share a row with cross-lane shuffles, then across waves.
// Otherwise MFMA: W tile as the 16-row A operand, x as the B operand (16 or 32 columns;
//   padding columns carry a copy of the last x row or zeros and are never stored).
// Escapes (exponents outside the codebook) are patched into the unpacked registers by
//   the owning lane, walking the row-block's sorted escape list through a 4-record
//   window in scalar registers.
// Split-K (gridDim.y > 1): FP32 partials go to the workspace at device scope and the
//   split that finishes last in its row-block group sums them in split order
//   (deterministic; see split_last).
// RMS launches (p.rms; the column-synchronous kernel's EPI_RMS instantiations): the
//   output rows are divided by the RMS of their x rows, summed from the staged x
//   (harness op of the layer chain, not the W12 method).
// FP8 tiles (SRC_F8: E4M3 weights of an FP8 checkpoint with one FP32 scale per 128 x 128
//   block) take the column-synchronous path with the BF16 and RMS epilogues: each byte
//   pair is converted exactly to a BF16 pair, each tile column is summed from zero and
//   enters the running sum times its block scale.
// The logits epilogue (verification pass 1) sums every tile column from zero before
//   adding it to the running sum, and keeps per row-block the two largest logits, the
//   index of the largest and the largest bound of a row's 2-norm; the full FP32 logits
//   only when the caller passes a buffer for them.
#pragma once

#include "w12_internal.h"

namespace w12 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// Plain BF16 sources (row-major or tiled): no decode, no escapes.
constexpr bool plain_bf16(int src) { return src == SRC_BF16 || src == SRC_BF16T; }
// W12 sources: sign/mantissa bytes, exponent codes and escapes.
constexpr bool w12_src(int src) { return src == SRC_RUN || src == SRC_LUT; }
// Bytes of one 16 x 128 tile, and the 16-byte loads per lane that read it.
constexpr uint32_t tile_bytes(int src) {
  return src == SRC_BF16T ? 4096u : src == SRC_F8 ? 2048u : 3072u;
}
constexpr int tile_loads(int src) { return plain_bf16(src) ? 4 : src == SRC_F8 ? 2 : 3; }

// BF16 per LDS row of an x column: +16 B pad (3.2 bank-conflict cycles per MFMA B read,
// measured; +32 B has none but is no faster up to 64 columns), +32 B for the 64- and
// 128-column tiles of k_gemm_cs, where the B reads bound the kernel (4% at 128 columns).
constexpr int kXsStride = 128 + 8;
constexpr int xs_stride(int mt) { return mt >= 64 ? 128 + 16 : kXsStride; }


// The weight a row-block belongs to, selected from the launch's table with constant
// indices only (the table stays in the kernel-argument segment; for a wave-uniform b
// every field is a scalar).
struct SegView {
  const uint8_t* w;
  const uint32_t* esc_off;
  const uint32_t* esc;
  uint16_t* y;
  uint32_t rb0, n, basepair;
  uint32_t lut[4];
  const float* scale;
};

__device__ __forceinline__ SegView seg_view(const GemmParams& p, uint32_t b) {
  SegView v;
  v.w = p.seg[0].w;
  v.esc_off = p.seg[0].esc_off;
  v.esc = p.seg[0].esc;
  v.y = p.seg[0].y;
  v.rb0 = p.seg[0].rb0;
  v.n = p.seg[0].n;
  v.basepair = p.seg[0].basepair;
  v.scale = p.seg[0].scale;
#pragma unroll
  for (int i = 0; i < 4; ++i) v.lut[i] = p.seg[0].lut[i];
#pragma unroll
  for (int s = 1; s < kMaxSeg; ++s) {
    const bool here = (uint32_t)s < p.nseg && b >= p.seg[s].rb0;
    v.w = here ? p.seg[s].w : v.w;
    v.esc_off = here ? p.seg[s].esc_off : v.esc_off;
    v.esc = here ? p.seg[s].esc : v.esc;
    v.y = here ? p.seg[s].y : v.y;
    v.rb0 = here ? p.seg[s].rb0 : v.rb0;
    v.n = here ? p.seg[s].n : v.n;
    v.basepair = here ? p.seg[s].basepair : v.basepair;
    v.scale = here ? p.seg[s].scale : v.scale;
#pragma unroll
    for (int i = 0; i < 4; ++i) v.lut[i] = here ? p.seg[s].lut[i] : v.lut[i];
  }
  return v;
}

// BF16 pair view of a 32-bit word.  Taken by value on purpose: this compiler
// miscompiles __builtin_bit_cast applied directly to an ext-vector element (it reads
// element 0 whatever the index), so vector elements must pass through a scalar first.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

__device__ __forceinline__ uint32_t vperm(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) return (uint16_t)((u >> 16) | 0x0040u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// 16-entry byte lookup of four codes (each byte 0..15) in the codebook held as four
// dwords: two byte permutes pick C[c & 7] from C[0..7] and C[8..15], a third builds
// the per-byte select mask from bit 3 (selector 4 -> 0x00, 5 -> 0xFF).
__device__ __forceinline__ uint32_t lut16(uint32_t c, uint32_t t0, uint32_t t1, uint32_t t2,
                                          uint32_t t3) {
  const uint32_t c7 = c & 0x07070707u;
  const uint32_t lo = vperm(t1, t0, c7);
  const uint32_t hi = vperm(t3, t2, c7);
  const uint32_t msel = ((c >> 3) & 0x01010101u) | 0x04040404u;
  const uint32_t msk = vperm(0x0000FF00u, 0u, msel);
  return (hi & msk) | (lo & ~msk);
}

template <int SRC>
struct TileRegs {
  u32x4 v[tile_loads(SRC)];
  float sc;   // SRC_F8: the tile's block scale
};

// Tile (b, g) of a weight of nbw row-blocks: W12 and 4 KB BF16 tiles are stored column
// by column, tile (b, g) at (g * nbw + b) * tile bytes, so the workgroups streaming one
// column at a time read adjacent tiles.
template <int SRC>
__device__ __forceinline__ void load_tile(TileRegs<SRC>& t, const uint8_t* __restrict__ w,
                                          const GemmParams& p, uint32_t b, uint32_t g, int lane,
                                          uint32_t nbw) {
  if constexpr (SRC == SRC_BF16) {
    const int r = lane & 15, q = lane >> 4;
    const uint8_t* base = w + ((size_t)(16u * b + r) * p.k + 128u * g + 8u * q) * 2u;
#pragma unroll
    // plain loads: each instruction covers half of every 128-byte line it touches, and
    // the other half is read by the next instruction from L2
    for (int j = 0; j < 4; ++j) t.v[j] = *reinterpret_cast<const u32x4*>(base + 64 * j);
  } else if constexpr (SRC == SRC_BF16T) {
    // 4 KB tiles: the lane's 16 bytes of group j at 1024 j + 16 lane, so every wave
    // instruction reads 1 KB of whole lines (streaming loads, as for W12 tiles)
    const uint8_t* base = w + ((size_t)g * nbw + b) * 4096u + (uint32_t)lane * 16u;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      t.v[j] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + 1024 * j));
  } else {
    const uint8_t* base = w + ((size_t)g * nbw + b) * 3072u + (uint32_t)lane * 16u;
#pragma unroll
    // streaming (nontemporal) loads: every instruction reads 1 KB of whole lines
    for (int s = 0; s < 3; ++s)
      t.v[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(base + 1024 * s));
  }
}

// Raw buffer resources (gfx9 layout: 48-bit base, stride 0, size in bytes, dword 3 =
// 32-bit data format, which untyped loads ignore).  A load past the size returns zeros.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kCpolNT = 2;   // cache policy of a buffer load: nontemporal (streaming)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}

// Split-K completion inside the GEMM launch.  The K splits of one row-block group run on
// any XCDs, whose L2 caches are not coherent with one another for plain accesses.  Every
// split writes its FP32 partials (and, on RMS launches, its rows' sums of x^2) with
// device-scope stores (cache policy sc1: written through to device-coherent memory),
// waits until they are complete, and then takes a ticket with a device-scope atomic; the
// split that takes the last ticket resets it to zero for the next launch and reads every
// split's partials with device-scope loads (sc1: never served from a stale cache line),
// summing them in split order, so the result is the same whichever split finishes last.
// No workgroup ever waits for another.  Tickets start at zero (a zeroed workspace) and
// every launch leaves them at zero.
constexpr int kCpolDevice = 16;   // sc1: coherent at device scope
__device__ __forceinline__ void st_dev(__amdgpu_buffer_rsrc_t rs, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, off, 0, kCpolDevice);
}
__device__ __forceinline__ void st_dev(__amdgpu_buffer_rsrc_t rs, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, off, 0, kCpolDevice);
}
__device__ __forceinline__ f32x4 ld_dev4(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, kCpolDevice));
}
__device__ __forceinline__ float ld_dev1(__amdgpu_buffer_rsrc_t rs, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, kCpolDevice));
}

// Called by every thread of a split workgroup after its device-scope stores: true in the
// workgroup that finished last among the gridDim.y splits of row-block group `grp`.
__device__ __forceinline__ bool split_last(uint32_t* tickets, uint32_t grp) {
  __shared__ uint32_t s_last;
  // this thread's device-scope stores are complete (visible at device scope) ...
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();   // ... and so are every other thread's of the workgroup
  if (threadIdx.x == 0) {
    const uint32_t old = __hip_atomic_fetch_add(tickets + grp, 1u, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old + 1u == gridDim.y;
    if (last) __hip_atomic_store(tickets + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last ? 1u : 0u;
  }
  __syncthreads();
  return s_last != 0u;
}

// One tile (W12, FP8 or 4 KB BF16) through a buffer resource over exactly its bytes,
// built from a wave-uniform address: advancing a column changes scalar registers only,
// and the lanes' offsets stay fixed.
template <int SRC>
__device__ __forceinline__ void load_tile_rs(TileRegs<SRC>& t, const uint8_t* tile, int lane) {
  static_assert(SRC != SRC_BF16, "row-major BF16 rows are not tiles");
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(tile, tile_bytes(SRC));
#pragma unroll
  for (int s = 0; s < tile_loads(SRC); ++s)
    t.v[s] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)lane * 16u + 1024u * s, 0, kCpolNT);
}

// Registers -> 16 BF16 pairs (P[4j+p] = element 2p in the low half, 2p+1 in the high).
template <int SRC>
__device__ __forceinline__ void unpack_tile(const TileRegs<SRC>& t, const SegView& a,
                                            uint32_t P[16]) {
  if constexpr (plain_bf16(SRC)) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int p = 0; p < 4; ++p) P[4 * j + p] = t.v[j][p];
  } else if constexpr (SRC == SRC_F8) {
    // FP8 E4M3 bytes in the W12 sign/mantissa byte order (group j in dwords 2(j&1),
    // 2(j&1)+1 of load j/2): one v_cvt_scalef32_pk_bf16_fp8 per pair, at scale 1.  Every
    // E4M3 value (normal 2^-6..448 with 3 mantissa bits, subnormal multiples of 2^-9) is
    // a BF16 value, so the conversion is exact; the block scale is applied to the FP32
    // column sums.
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4& S = t.v[j >> 1];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t wd = S[2 * (j & 1) + h];
        P[4 * j + 2 * h] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd, 1.0f, false));
        P[4 * j + 2 * h + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(wd, 1.0f, true));
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4& S = (j < 2) ? t.v[0] : t.v[1];
      const uint32_t sa = S[2 * (j & 1)], sb = S[2 * (j & 1) + 1];
      const uint32_t cw = t.v[2][j];
      uint32_t E[4];
      if constexpr (SRC == SRC_RUN) {
#pragma unroll
        for (int p = 0; p < 4; ++p) E[p] = (((cw >> (4 * p)) & 0x000F000Fu) + a.basepair) << 7;
      } else {
        const uint32_t elo = lut16(cw & 0x0F0F0F0Fu, a.lut[0], a.lut[1], a.lut[2], a.lut[3]);
        const uint32_t ehi = lut16((cw >> 4) & 0x0F0F0F0Fu, a.lut[0], a.lut[1], a.lut[2], a.lut[3]);
        E[0] = (elo & 0x00FF00FFu) << 7;
        E[1] = (ehi & 0x00FF00FFu) << 7;
        E[2] = ((elo >> 8) & 0x00FF00FFu) << 7;
        E[3] = ((ehi >> 8) & 0x00FF00FFu) << 7;
      }
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t s = (p < 2) ? sa : sb;
        // bytes {sm(odd), sm(odd), sm(even), sm(even)}: sign -> bit 15/31, mantissa ->
        // bits 0-6/16-22 after the mask; the exponent fills bits 7-14/23-30.
        const uint32_t dup = vperm(s, s, (p & 1) ? 0x03030202u : 0x01010000u);
        P[4 * j + p] = (dup & 0x807F807Fu) | E[p];
      }
    }
  }
}

// Escape cursor of one row-block, wave-uniform (scalar registers): records [pos, end)
// not yet consumed, and a window w[] holding records pos..pos+3 (a sentinel, whose
// column is past any K, beyond end).  Scalar loads share a wait counter with LDS, so
// the window is refilled only after the tile's last LDS read (esc_refill), never in
// front of one; a tile with more than four escapes in one row-block refills inline.
constexpr int kEscWin = 4;
struct EscCursor {
  uint32_t pos, end;
  uint32_t w[kEscWin];   // records pos .. pos + nwin - 1, then sentinels
  uint32_t nwin;
  bool stale;            // records consumed since the last refill
};

constexpr uint32_t kEscSentinel = 0xFFFFFFFFu;

__device__ __forceinline__ uint32_t esc_col(uint32_t rec) { return (rec >> 8) & 0xFFFFFu; }

// Escape records are read-only for the whole launch and addressed uniformly: reading
// them through the constant address space makes them scalar (SMEM) loads, which do not
// share the vector-memory counter with the tile prefetch.
typedef const __attribute__((address_space(4))) uint32_t* const_u32_ptr;

__device__ __forceinline__ uint32_t sload(const uint32_t* p, uint32_t i) {
  return ((const_u32_ptr)p)[i];
}

__device__ __forceinline__ void esc_refill(EscCursor& c, const uint32_t* __restrict__ esc) {
#pragma unroll
  for (int i = 0; i < kEscWin; ++i) c.w[i] = c.pos + i < c.end ? sload(esc, c.pos + i) : kEscSentinel;
  c.nwin = min(c.end - c.pos, (uint32_t)kEscWin);
  c.stale = false;
}

// Start the cursor at the first record of row-block b with column >= kmin (binary
// search over the row-block's records, which are sorted by column).
__device__ __forceinline__ void esc_begin(EscCursor& c, const uint32_t* __restrict__ esc_off,
                                          const uint32_t* __restrict__ esc, uint32_t b,
                                          uint32_t kmin) {
  uint32_t lo = sload(esc_off, b);
  const uint32_t end = sload(esc_off, b + 1);
  if (kmin > 0u) {
    uint32_t hi = end;
    while (lo < hi) {
      const uint32_t mid = lo + ((hi - lo) >> 1);
      if (esc_col(sload(esc, mid)) < kmin) lo = mid + 1; else hi = mid;
    }
  }
  c.pos = lo;
  c.end = end;
  esc_refill(c, esc);
}

__device__ __forceinline__ void patch_pair(uint32_t P[16], uint32_t pi, uint32_t sh, uint32_t e,
                                           bool mine) {
#pragma unroll
  for (int z = 0; z < 16; ++z) {
    if ((uint32_t)z == pi) {
      const uint32_t v = P[z];
      const uint32_t nv = (v & ~(0xFFu << sh)) | (e << sh);
      P[z] = mine ? nv : v;
    }
  }
}

// Patch the escapes of tile column g into P.  Records of columns below g (other
// waves' columns) are skipped; consumption stops at the first record past the tile.
// The window is shifted as records are consumed and refilled inline only when it runs
// dry inside a tile (more than four escapes of one row-block in one tile).
__device__ __forceinline__ void esc_apply(EscCursor& c, const uint32_t* __restrict__ esc,
                                          uint32_t g, int lane, uint32_t P[16]) {
  const uint32_t klo = g * 128u, khi = klo + 128u;
  while (esc_col(c.w[0]) < khi) {
    const uint32_t rec = c.w[0];
    if (esc_col(rec) >= klo) {
      const uint32_t rr = rec >> 28;
      const uint32_t kap = esc_col(rec) - klo;
      const uint32_t j = kap >> 5, qq = (kap >> 3) & 3u, ii = kap & 7u;
      patch_pair(P, 4u * j + (ii >> 1), 7u + 16u * (ii & 1u), rec & 0xFFu,
                 (uint32_t)lane == 16u * qq + rr);
    }
#pragma unroll
    for (int i = 0; i + 1 < kEscWin; ++i) c.w[i] = c.w[i + 1];
    c.w[kEscWin - 1] = kEscSentinel;
    ++c.pos;
    --c.nwin;
    c.stale = true;
    if (c.nwin == 0u && c.pos < c.end) esc_refill(c, esc);
  }
}

// Sum of squares of the 8 BF16 of a 16-byte x unit, in FP32, in a fixed order (RMS
// launches: the row's mean square is accumulated from the staged x units).
__device__ __forceinline__ float unit_sumsq(const u32x4& v) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float lo = __uint_as_float(v[i] << 16), hi = __uint_as_float(v[i] & 0xFFFF0000u);
    s += lo * lo + hi * hi;
  }
  return s;
}

// 1 / RMS of a row from its sum of squares over K (the RMS rescale's formula).
__device__ __forceinline__ float rms_of(float ss, uint32_t k) { return sqrtf(ss / (float)k); }

// One wave's x column: MT rows x 128 BF16 = 16*MT units of 16 bytes over 64 lanes.
template <int MT>
struct XStage {
  static constexpr int kUnits = (16 * MT + 63) / 64;
  u32x4 v[kUnits];
};

// Every lane issues the same loads on every path, with the row clamped to m_rows - 1 and
// the column to the last one of the K-range, so the compiler's wait counts stay exact.
// The loaded values are used as they are: a clamped row only feeds MFMA output columns
// m >= m_rows, which are never stored (each output column depends on its own x row
// only), and a column past the range is never multiplied.  Zeroing them would put a
// select on the load result next to the load, and the compiler then waits for the load
// right there, in front of the next prefetch.
template <int MT>
__device__ __forceinline__ void x_load(XStage<MT>& st, const uint16_t* __restrict__ x,
                                       uint32_t k, uint32_t m_rows, uint32_t g, uint32_t gb,
                                       int lane) {
#pragma unroll
  for (int i = 0; i < XStage<MT>::kUnits; ++i) {
    const uint32_t u = (uint32_t)lane + 64u * i;
    const uint32_t uu = u < 16u * MT ? u : u % (16u * MT);
    const uint32_t m = uu >> 4, cu = uu & 15u;
    const uint32_t ml = min(m, m_rows - 1u), gl = min(g, gb - 1u);
    st.v[i] = *reinterpret_cast<const u32x4*>(x + (size_t)ml * k + 128u * gl + 8u * cu);
  }
}

template <int MT>
__device__ __forceinline__ void x_store(const XStage<MT>& st, uint16_t* xw, int lane) {
#pragma unroll
  for (int i = 0; i < XStage<MT>::kUnits; ++i) {
    const uint32_t u = (uint32_t)lane + 64u * i;
    if (u < 16u * MT) {
      const uint32_t m = u >> 4, cu = u & 15u;
      *reinterpret_cast<u32x4*>(xw + m * kXsStride + 8u * cu) = st.v[i];
    }
  }
}

// M: x rows staged (compile-time; the VALU path's rows, or for MFMA 4, 8 or 16 of the
// MT = 16 columns of the B operand); MT: LDS rows.
// EPI_BF16 with gridDim.y > 1 writes FP32 partials [split][m][n] and the last split of
// the workgroup's row-block group writes y; with one split it writes y directly.
template <int M, int MT, bool MF, int RBW, int NWV, int SRC, int EPI>
__global__ __launch_bounds__(NWV * 64) void k_gemm(
    const uint16_t* __restrict__ x, float* __restrict__ out_f32, float* __restrict__ out_s,
    BlockMax bm,
    GemmParams p) {
  constexpr int NH = MF ? MT / 16 : 1;
  static_assert(SRC != SRC_F8, "FP8 tiles run column-synchronous only");
  // the logits epilogue (VALU path only: from W12_MFMA_MIN_M rows on it runs in k_gemm_cs)
  // also records per weight row an upper bound of ||w_v||_2 (the scale of its
  // rounding-error bound is ||x||_2 ||w_v||_2, verification pass 2 supplies ||x||_2): the
  // squares summed by v_dot2 of the weights with themselves
  constexpr bool kWn = EPI == EPI_LOGITS;
  static_assert(!(kWn && MF), "the logits epilogue runs column-synchronous with MFMA");
  __shared__ __align__(16) uint16_t xs[NWV * MT * kXsStride];   // one x column per wave
  __shared__ float fin[kWn ? RBW * MT * 16 : 1];
  __shared__ float s_wn[kWn ? RBW * 16 : 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform, in an SGPR
  const int r = lane & 15, q = lane >> 4;
  const uint32_t rbg = blockIdx.x, split = blockIdx.y;
  const uint32_t b0 = rbg * RBW;
  // split s of S covers tile columns [s*G/S, (s+1)*G/S): the K range dealt evenly
  const uint32_t ga = (uint32_t)(((uint64_t)split * p.g_cols) / gridDim.y);
  const uint32_t gb = (uint32_t)(((uint64_t)(split + 1u) * p.g_cols) / gridDim.y);
  const uint32_t m_rows = MF ? p.m : (uint32_t)M;

  float vacc[RBW][MF ? 1 : M];
  f32x4 macc[RBW][NH];
  float wsq[RBW];     // kWn: this lane's sum of squares of row r's weights
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
#pragma unroll
    for (int m = 0; m < (MF ? 1 : M); ++m) vacc[rb][m] = 0.f;
#pragma unroll
    for (int h = 0; h < NH; ++h) macc[rb][h] = f32x4{0.f, 0.f, 0.f, 0.f};
    wsq[rb] = 0.f;
  }

  EscCursor ec[RBW];
  SegView sv[RBW];          // the weight of each row-block (launch numbering b0 + rb)
  uint32_t bl[RBW];         // the row-block inside that weight (clamped into range)
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
    const uint32_t bg = min(b0 + rb, p.nb - 1u);
    sv[rb] = seg_view(p, bg);
    bl[rb] = bg - sv[rb].rb0;
  }

  TileRegs<SRC> tA[RBW], tB[RBW];
  XStage<M> xr;      // only the M staged rows (MFMA: 4, 8 or 16 of the 16 padded)

  uint16_t* xw = xs + wave * MT * kXsStride;   // this wave's x column in LDS

  auto load_tiles = [&](TileRegs<SRC>* t, uint32_t g) {
    const uint32_t gl = min(g, gb - 1u);
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) load_tile<SRC>(t[rb], sv[rb].w, p, bl[rb], gl, lane, sv[rb].n / 16u);
  };

  auto compute = [&](const TileRegs<SRC>* t, uint32_t g) {
    uint32_t P[RBW][16];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      unpack_tile<SRC>(t[rb], sv[rb], P[rb]);
      if constexpr (w12_src(SRC)) {
        if (b0 + rb < p.nb) esc_apply(ec[rb], sv[rb].esc, g, lane, P[rb]);
      }
    }
    const uint16_t* xrow = xw + 8 * q;
    // logits: the column's sums chain from zero and are then added to the running sums,
    // so a product meets at most 16 v_dot2 (2 roundings each, whatever their internal
    // order) and one addition per later column: the certified bound's depth
    float vcol[RBW][MF ? 1 : M];
    auto vc = [&](int rb, int m) -> float& { return kWn ? vcol[rb][m] : vacc[rb][m]; };
    if constexpr (kWn) {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int m = 0; m < (MF ? 1 : M); ++m) vcol[rb][m] = 0.f;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (MF) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          // rows past the M staged ones are padding: their LDS rows are never written
          // or read, and the B operand gets zeros there
          const u32x4 xv = (16 * h + r) < M
              ? *reinterpret_cast<const u32x4*>(xrow + (16 * h + r) * kXsStride + 32 * j)
              : u32x4{0u, 0u, 0u, 0u};
          const bf16x8_t bv = __builtin_bit_cast(bf16x8_t, xv);
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb) {
            const u32x4 av = {P[rb][4 * j], P[rb][4 * j + 1], P[rb][4 * j + 2], P[rb][4 * j + 3]};
            macc[rb][h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8_t, av), bv, macc[rb][h], 0, 0, 0);
          }
        }
      } else {
#pragma unroll
        for (int m = 0; m < M; ++m) {
          const u32x4 xv = *reinterpret_cast<const u32x4*>(xrow + m * kXsStride + 32 * j);
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int pp = 0; pp < 4; ++pp) {
              vc(rb, m) = __builtin_amdgcn_fdot2_f32_bf16(
                  as_bf16x2(P[rb][4 * j + pp]), as_bf16x2(xv[pp]), vc(rb, m), false);
            }
        }
        if constexpr (kWn) {
#pragma unroll
          for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
            for (int pp = 0; pp < 4; ++pp)
              wsq[rb] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(P[rb][4 * j + pp]),
                                                        as_bf16x2(P[rb][4 * j + pp]), wsq[rb], false);
        }
      }
    }
    if constexpr (kWn) {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int m = 0; m < (MF ? 1 : M); ++m) vacc[rb][m] += vcol[rb][m];
    }
    if constexpr (w12_src(SRC)) {
      // refill after the tile's last LDS read: a pending scalar load would otherwise
      // hold up the LDS waits (they share one counter)
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
        if (ec[rb].stale) esc_refill(ec[rb], sv[rb].esc);
    }
  };

  // ---- main loop.  Wave w streams tile columns ga+w, ga+w+4, ... of its row-blocks
  // independently of the other waves (x goes through the wave's own LDS slot, so no
  // workgroup barrier).  In source order column g+4's x and tiles are requested before
  // column g is computed; every iteration issues the same loads (past the last column
  // the addresses are clamped to the last tile column, still in L2, and the values are
  // never used).  The compiler is left free to sink part of the next column's loads
  // below the compute to reuse registers: pinning the full one-column-ahead schedule
  // with scheduling barriers (and a single-exit loop) measured slower on these shapes
  // (M1 down -5 %, M16 / M32 gate+up -3 to -4 %), the memory system being saturated by
  // fewer requests in flight per wave.  (No RMS launch runs here: W12 launches with the
  // BF16 epilogue are column-synchronous, and the BF16 sources have no RMS form.)
  uint32_t g = ga + (uint32_t)wave;
  if (g < gb) {
    x_load<M>(xr, x, p.k, m_rows, g, gb, lane);
    load_tiles(tA, g);
    // escape cursors start after the first tiles are requested: their scalar loads
    // (one or two dependent round trips) overlap the first tile fetch
    if constexpr (w12_src(SRC)) {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb) esc_begin(ec[rb], sv[rb].esc_off, sv[rb].esc, bl[rb], ga * 128u);
    }
    x_store<M>(xr, xw, lane);
    __builtin_amdgcn_wave_barrier();
    for (;;) {
      x_load<M>(xr, x, p.k, m_rows, g + NWV, gb, lane);
      load_tiles(tB, g + NWV);
      compute(tA, g);
      __builtin_amdgcn_wave_barrier();
      x_store<M>(xr, xw, lane);
      __builtin_amdgcn_wave_barrier();
      g += NWV;
      if (g >= gb) break;
      x_load<M>(xr, x, p.k, m_rows, g + NWV, gb, lane);
      load_tiles(tA, g + NWV);
      compute(tB, g);
      __builtin_amdgcn_wave_barrier();
      x_store<M>(xr, xw, lane);
      __builtin_amdgcn_wave_barrier();
      g += NWV;
      if (g >= gb) break;
    }
  }
  __syncthreads();   // LDS x no longer read: reuse it for the cross-wave reduction

  // ---- cross-lane / cross-wave reduction into red[] (aliases xs); the row sums of
  // squares, when kept, follow as [wave][rb][row]
  float* red = reinterpret_cast<float*>(xs);
  constexpr int kRed = MF ? NWV * RBW * NH * 4 * 64 : NWV * RBW * M * 16;
  static_assert((kRed + (kWn ? NWV * RBW * 16 : 0)) * sizeof(float) <= sizeof(xs), "reduction fits in xs");
  auto to_red = [&](float* dst, float (*va)[MF ? 1 : M], f32x4 (*ma)[NH]) {
    if constexpr (MF) {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int h = 0; h < NH; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            dst[(((wave * RBW + rb) * NH + h) * 4 + i) * 64 + lane] = ma[rb][h][i];
    } else {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
        for (int m = 0; m < M; ++m) {
          float v = va[rb][m];
          v += __shfl_xor(v, 16);
          v += __shfl_xor(v, 32);
          if (q == 0) dst[((wave * RBW + rb) * M + m) * 16 + r] = v;
        }
    }
  };
  to_red(red, vacc, macc);
  if constexpr (kWn) {
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      float v = wsq[rb];
      v += __shfl_xor(v, 16);
      v += __shfl_xor(v, 32);
      if (q == 0) red[kRed + (wave * RBW + rb) * 16 + r] = v;
    }
  }
  __syncthreads();

  constexpr int kOut = RBW * MT * 16;   // (rb, m, row) outputs of this workgroup
  auto final_value = [&](const float* src, int o) -> float {
    const int rb = o / (MT * 16), rem = o % (MT * 16), m = rem >> 4, rr = rem & 15;
    float s = 0.f;
#pragma unroll
    for (int wv = 0; wv < NWV; ++wv) {
      if constexpr (MF) {
        const int h = m >> 4, ln = 16 * (rr >> 2) + (m & 15), i = rr & 3;
        s += src[(((wv * RBW + rb) * NH + h) * 4 + i) * 64 + ln];
      } else {
        s += src[((wv * RBW + rb) * M + m) * 16 + rr];
      }
    }
    return s;
  };

  if constexpr (EPI == EPI_LOGITS) {
    if (tid < RBW * 16) {   // the waves' partial sums of squares in wave order
      float t = 0.f;
#pragma unroll
      for (int wv = 0; wv < NWV; ++wv) t += red[kRed + (wv * RBW + (tid >> 4)) * 16 + (tid & 15)];
      s_wn[tid] = l2_norm_up(t, p.k);
    }
    for (int o = tid; o < kOut; o += (NWV * 64)) fin[o] = final_value(red, o);
    __syncthreads();
    if (out_f32) {   // full logits and norms only when asked for
      for (int o = tid; o < kOut; o += (NWV * 64)) {
        const int rb = o / (MT * 16), rem = o % (MT * 16), m = rem >> 4, rr = rem & 15;
        const uint32_t b = b0 + rb;
        if (b >= p.nb || (uint32_t)m >= m_rows) continue;
        out_f32[(size_t)m * p.n + 16u * b + rr] = fin[o];
        out_s[(size_t)m * p.n + 16u * b + rr] = s_wn[rb * 16 + rr];
      }
    }
    if (bm.accepted && blockIdx.x == 0 && blockIdx.y == 0)
      accept_init(bm, p.m, (uint32_t)tid, NWV * 64u);   // verification pass 2 lowers them
    // per (row-block, output row) records, kept in LDS for the workgroup's group record
    __shared__ float s_gv[RBW][MT], s_gv2[RBW][MT], s_gs[RBW][MT];
    __shared__ int32_t s_gi[RBW][MT];
    for (int o = tid; o < RBW * MT; o += (NWV * 64)) {
      const int rb = o / MT, m = o % MT;
      const uint32_t b = b0 + rb;
      const bool live = b < p.nb && (uint32_t)m < m_rows;
      // largest (lowest row on ties) and second largest logit of the block
      float best = fin[o * 16], second = -__builtin_inff(), smax = s_wn[rb * 16];
      int bi = 0;
      bool finite = __builtin_isfinite(best);
      for (int rr = 1; rr < 16; ++rr) {
        const float v = fin[o * 16 + rr];
        finite = finite && __builtin_isfinite(v);
        if (v > best) { second = best; best = v; bi = rr; }
        else if (v > second) second = v;
        smax = fmaxf(smax, s_wn[rb * 16 + rr]);
      }
      s_gv[rb][m] = !live ? -__builtin_inff() : (finite ? best : __builtin_nanf(""));
      s_gv2[rb][m] = !live ? -__builtin_inff() : second;
      s_gi[rb][m] = (int32_t)(16u * b + bi);
      s_gs[rb][m] = live ? smax : 0.f;
      if (!live) continue;
      bm.v[(size_t)m * p.nb + b] = finite ? best : __builtin_nanf("");
      bm.v2[(size_t)m * p.nb + b] = finite ? second : __builtin_nanf("");
      bm.s[(size_t)m * p.nb + b] = smax;
      bm.i[(size_t)m * p.nb + b] = (int32_t)(16u * b + bi);
    }
    __syncthreads();
    if ((uint32_t)tid < MT && (uint32_t)tid < m_rows) {
      // the group's two largest logits: a block whose best beats the current best brings
      // its own second, an equal best makes the second equal to it (a tie)
      float v = s_gv[0][tid], v2 = s_gv2[0][tid], sv = s_gs[0][tid], wg = s_gs[0][tid];
      int32_t vi = s_gi[0][tid];
      bool nan = v != v;
#pragma unroll
      for (int rb = 1; rb < RBW; ++rb) {
        const float vw = s_gv[rb][tid];
        nan = nan || vw != vw;
        if (vw > v) { v2 = fmaxf(v, s_gv2[rb][tid]); v = vw; vi = s_gi[rb][tid]; sv = s_gs[rb][tid]; }   // ties: the lower row-block
        else v2 = fmaxf(v2, vw);
        wg = fmaxf(wg, s_gs[rb][tid]);
      }
      const size_t og = (size_t)tid * bm.ngrp + blockIdx.x;
      bm.gv[og] = nan ? __builtin_nanf("") : v;
      bm.gv2[og] = nan ? __builtin_nanf("") : v2;
      bm.gi[og] = vi;
      bm.gs[og] = sv;
      bm.gw[og] = wg;
    }
  } else {
    auto store_y = [&](int rb, int m, int rr, float v) {
      const bool second = RBW == 2 && rb == 1;     // per-thread: pick the row-block's weight
      uint16_t* yy = second ? sv[RBW - 1].y : sv[0].y;
      const uint32_t nn = second ? sv[RBW - 1].n : sv[0].n;
      const uint32_t bb = second ? bl[RBW - 1] : bl[0];
      yy[(size_t)m * nn + 16u * bb + rr] = f32_to_bf16_rne(v);
    };
    if (gridDim.y == 1) {
      for (int o = tid; o < kOut; o += (NWV * 64)) {
        const int rb = o / (MT * 16), rem = o % (MT * 16), m = rem >> 4, rr = rem & 15;
        const float v = final_value(red, o);
        if (b0 + rb >= p.nb || (uint32_t)m >= m_rows) continue;
        store_y(rb, m, rr, v);
      }
    } else {
      // K split: this split's partials [split][m][n] at device scope; the split that
      // completes the group sums all of them in split order
      const __amdgpu_buffer_rsrc_t prs = make_rsrc(out_f32, gridDim.y * m_rows * p.n * 4u);
      for (int o = tid; o < kOut; o += (NWV * 64)) {
        const int rb = o / (MT * 16), rem = o % (MT * 16), m = rem >> 4, rr = rem & 15;
        const uint32_t b = b0 + rb;
        const float v = final_value(red, o);
        if (b >= p.nb || (uint32_t)m >= m_rows) continue;
        st_dev(prs, ((split * m_rows + m) * p.n + 16u * b + rr) * 4u, v);
      }
      if (split_last(p.tickets, blockIdx.x)) {
        for (int o = tid; o < kOut; o += (NWV * 64)) {
          const int rb = o / (MT * 16), rem = o % (MT * 16), m = rem >> 4, rr = rem & 15;
          const uint32_t b = b0 + rb;
          if (b >= p.nb || (uint32_t)m >= m_rows) continue;
          float v[kMaxSplit];
#pragma unroll
          for (uint32_t sp = 0; sp < kMaxSplit; ++sp) {   // every load in flight before the adds
            const uint32_t spl = min(sp, gridDim.y - 1u);
            v[sp] = ld_dev1(prs, ((spl * m_rows + m) * p.n + 16u * b + rr) * 4u);
          }
          float t = 0.f;
#pragma unroll
          for (uint32_t sp = 0; sp < kMaxSplit; ++sp)
            if (sp < gridDim.y) t += v[sp];
          store_y(rb, m, rr, t);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// Column-synchronous MFMA kernel (m >= W12_MFMA_MIN_M).  A workgroup of NW waves covers
// NW consecutive row-blocks, one per wave, and all waves walk the same tile columns of
// the K-range together.  The x column (MT rows x 128 BF16) is loaded once per
// workgroup -- each thread a slice -- into one of two LDS slots, so one barrier per
// column suffices (the slot written for column g+1 was last read for column g-1, which
// every wave finished before the previous barrier).  Compared with a wave per column
// this divides the x traffic per tile by NW.  Each wave owns its row-block's outputs:
// lane l holds D[4q+i][l%16 + 16h], i.e. rows 16b+4q..16b+4q+3 of output column m.
template <int MT, int NW, int SRC, int EPI>
__global__ __launch_bounds__(NW * 64) void k_gemm_cs(
    const uint16_t* __restrict__ x, float* __restrict__ out_f32, float* __restrict__ out_s,
    BlockMax bm,
    GemmParams p) {
  constexpr int NH = MT / 16;
  // The logits epilogue records, per weight row, an upper bound of ||w_v||_2 (the error
  // scale is ||x||_2 ||w_v||_2 >= sum_k |x_k||w_vk| by Cauchy-Schwarz, and verification
  // pass 2 supplies ||x||_2).  The squares are summed by an MFMA of the A operand with
  // itself (its diagonal): one per 32 columns, whatever the number of x columns, where
  // a second MFMA on sign-cleared operands took one per x column block, and no x norms
  // here (summing them in every workgroup cost more than the rest of the bound).
  constexpr bool kWn = EPI == EPI_LOGITS;
  constexpr int NT = NW * 64;
  constexpr int kUnits = (16 * MT + NT - 1) / NT;     // 16-byte x units per thread
  constexpr int kXs = xs_stride(MT);
  __shared__ __align__(16) uint16_t xs[2][MT * kXs];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const uint32_t b = blockIdx.x * NW + (uint32_t)wave;
  const bool bvalid = b < p.nb;
  const SegView sv = seg_view(p, min(b, p.nb - 1u));
  const uint32_t bl = min(b, p.nb - 1u) - sv.rb0;   // row-block inside its weight
  const uint32_t split = blockIdx.y;
  // split s of S covers tile columns [s*G/S, (s+1)*G/S): the K range dealt evenly
  const uint32_t ga = (uint32_t)(((uint64_t)split * p.g_cols) / gridDim.y);
  const uint32_t gb = (uint32_t)(((uint64_t)(split + 1u) * p.g_cols) / gridDim.y);
  const uint32_t m_rows = p.m;

  f32x4 acc[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 nacc = {0.f, 0.f, 0.f, 0.f};   // kWn: D = W W^T over the K-range, diagonal used
  TileRegs<SRC> tA, tB;
  u32x4 xr[2][kUnits];   // x units of the column being staged (two sets up to 32 columns)
  EscCursor ec;

  // Loads go through buffer resources (the current tile, x) with fixed lane offsets and
  // the column in scalar registers: with 64-bit per-lane addresses recomputed every
  // column, the compiler waited for the previous column's loads before issuing the next
  // column's.
  constexpr bool kRs = SRC != SRC_BF16;
  constexpr uint32_t kTileB = tile_bytes(SRC);
  const uint32_t nbw = sv.n / 16u;   // row-blocks of this wave's weight (tile column stride)
  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x, m_rows * (uint32_t)p.k * 2u);
  uint32_t xoff[kUnits];   // byte offset of the thread's x units in column 0
#pragma unroll
  for (int i = 0; i < kUnits; ++i) {
    const uint32_t u = (uint32_t)tid + NT * i;
    const uint32_t uu = u < 16u * MT ? u : u % (16u * MT);
    const uint32_t m = uu >> 4, cu = uu & 15u;
    // clamped row / column, used unzeroed (see x_load)
    xoff[i] = (min(m, m_rows - 1u) * (uint32_t)p.k + 8u * cu) * 2u;
  }
  auto xload = [&](int set, uint32_t g) {
    const uint32_t gl = min(g, gb - 1u);
#pragma unroll
    for (int i = 0; i < kUnits; ++i)
      xr[set][i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff[i], 256u * gl, 0);
  };
  // FP8: the block scale of the wave's tile, one uniform load beside the tile's (the
  // 16 rows of a row-block lie in one 128-row scale block)
  constexpr bool kF8 = SRC == SRC_F8;
  const __amdgpu_buffer_rsrc_t scrs =
      make_rsrc(kF8 ? sv.scale : nullptr, kF8 ? ((nbw + 7u) / 8u) * p.g_cols * 4u : 0u);
  const uint32_t scrow = (bl / 8u) * p.g_cols * 4u;
  auto tload = [&](TileRegs<SRC>& t, uint32_t g) {
    if constexpr (kRs) load_tile_rs<SRC>(t, sv.w + ((size_t)g * nbw + bl) * kTileB, lane);
    else load_tile<SRC>(t, sv.w, p, bl, g, lane, nbw);
    if constexpr (kF8)
      t.sc = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(scrs, 0u, scrow + 4u * g, 0));
  };

  // RMS launches sum each row's x^2 over the K-range.  Up to 32 columns (the EPI_RMS
  // instantiations) by an MFMA of the x fragments with themselves (waves 0..3 take one of
  // the column's four 32-column steps each; the diagonal is kept), on matrix cores that
  // are otherwise 90 % idle: the decode chain's gate/up and o launches at M = 24 49.2 /
  // 16.4 -> 47.2 / 16.0 us against per-unit VALU sums.  At 64 and 128 columns, where the
  // MFMA accumulators would spill, the BF16 instantiation sums per unit on the VALU in
  // column order under the runtime flag (the compiler then keeps a separate copy of the
  // main loop for plain launches, which measured faster for them than the lone loop of a
  // compile-time form: gate+up / down M128 83.3 / 65.5 against 91.6 / 69.5 us).
  constexpr bool kRmsMF = EPI == EPI_RMS;
  static_assert(!kRmsMF || MT <= 32, "the RMS epilogue is instantiated up to 32 columns");
  const bool rms_valu = EPI == EPI_BF16 && MT >= 64 && p.rms;
  const bool rms_on = kRmsMF || rms_valu;
  float ssq[kUnits];
#pragma unroll
  for (int i = 0; i < kUnits; ++i) ssq[i] = 0.f;
  f32x4 racc[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) racc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto xsumsq = [&](int set, bool in_range) {
    if (rms_valu && in_range) {
#pragma unroll
      for (int i = 0; i < kUnits; ++i) ssq[i] += unit_sumsq(xr[set][i]);
    }
  };
  auto xstore = [&](int set, uint32_t slot) {
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
      const uint32_t u = (uint32_t)tid + NT * i;
      // (a compile-time true test when the units divide evenly: no exec-masked branch)
      if (kUnits * NT == 16 * MT || u < 16u * MT) {
        const uint32_t m = u >> 4, cu = u & 15u;
        *reinterpret_cast<u32x4*>(&xs[slot][m * kXs + 8u * cu]) = xr[set][i];
      }
    }
  };
  // The column's x fragments are read from LDS before the tile is decoded, so their
  // latency hides under the decode instead of stalling the MFMAs (the compiler placed
  // the reads after the decode, each pair waited for before its MFMAs): MLP gate+up
  // M1 / M16 / M32 41.8 / 42.2 / 46.1 -> 40.5 / 41.0 / 44.7 us.  Only where the extra
  // registers keep the occupancy the launches need: 16 columns, 32 with one x unit per
  // thread and the BF16 epilogue (with 5 or 7 waves, or the logits epilogue, the
  // 32-column kernel reached 129-135 VGPRs and lost a workgroup per CU: down M32
  // 28.2 -> 39.2 us), and 64 in the 10-wave workgroups that run one per CU (163 VGPRs;
  // gate+up M48 / M64 58.9 / 58.8 -> 56.6 / 57.8 us).
  constexpr bool kEarlyX = MT == 16 || (MT == 32 && kUnits == 1 && EPI != EPI_LOGITS) ||
                           (MT == 64 && NW == 10 && EPI == EPI_BF16);
  auto compute = [&](const TileRegs<SRC>& t, uint32_t g) {
    const uint16_t* xrow = &xs[g & 1u][8 * q];
    u32x4 xvs[4][NH];
    if constexpr (kEarlyX) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int h = 0; h < NH; ++h)
          xvs[j][h] = *reinterpret_cast<const u32x4*>(xrow + (16 * h + r) * kXs + 32 * j);
      __builtin_amdgcn_sched_barrier(0);
    }
    uint32_t P[16];
    unpack_tile<SRC>(t, sv, P);
    if constexpr (w12_src(SRC)) {
      if (bvalid) esc_apply(ec, sv.esc, g, lane, P);
    }
    // logits: the column's 4 MFMAs chain from zero and the column sum is added to the
    // running sum, so a product meets at most 4 MFMA accumulations (whatever their
    // internal order) and one addition per later column: the certified bound's depth
    f32x4 col[NH];
    if constexpr (kF8) {
      // FP8: each x column block's chain over the tile column (one 128-column scale
      // block) starts from zero and enters the running sum times the block scale (one
      // FMA); written block by block, and from 64 columns scheduled two blocks at a time
      // (with every block's chain interleaved the 128-column kernel spilled 72 bytes per
      // lane; scheduled freely, 8 bytes but gate+up M128 71.0 -> 77.0 us; in pairs, 16)
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const u32x4 av = {P[4 * j], P[4 * j + 1], P[4 * j + 2], P[4 * j + 3]};
          const u32x4 xv =
              kEarlyX ? xvs[j][h] : *reinterpret_cast<const u32x4*>(xrow + (16 * h + r) * kXs + 32 * j);
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                      __builtin_bit_cast(bf16x8_t, xv), c, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[h][i] = __builtin_fmaf(t.sc, c[i], acc[h][i]);
        if (MT >= 64 && (h & 1) == 1) __builtin_amdgcn_sched_barrier(0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 av = {P[4 * j], P[4 * j + 1], P[4 * j + 2], P[4 * j + 3]};
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const u32x4 xv =
              kEarlyX ? xvs[j][h] : *reinterpret_cast<const u32x4*>(xrow + (16 * h + r) * kXs + 32 * j);
          f32x4& c = kWn ? col[h] : acc[h];
          c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, xv),
                                                      (kWn && j == 0) ? f32x4{0.f, 0.f, 0.f, 0.f} : c, 0, 0, 0);
        }
      }
    }
    if constexpr (kWn) {
#pragma unroll
      for (int h = 0; h < NH; ++h) acc[h] += col[h];
    }
    if constexpr (kRmsMF) {
      if (wave < 4) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (wave == j) {   // (wave-uniform)
#pragma unroll
            for (int h = 0; h < NH; ++h) {
              const u32x4 xv =
                  kEarlyX ? xvs[j][h] : *reinterpret_cast<const u32x4*>(xrow + (16 * h + r) * kXs + 32 * j);
              racc[h] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, xv),
                                                                __builtin_bit_cast(bf16x8_t, xv), racc[h], 0, 0, 0);
            }
          }
      }
    }
    if constexpr (kWn) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x4 av = {P[4 * j], P[4 * j + 1], P[4 * j + 2], P[4 * j + 3]};
        nacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, av),
                                                       __builtin_bit_cast(bf16x8_t, av), nacc, 0, 0, 0);
      }
    }
    if constexpr (w12_src(SRC)) {
      __builtin_amdgcn_sched_barrier(0);
      if (ec.stale) esc_refill(ec, sv.esc);
    }
  };

  // ---- main loop: every iteration but the last issues the same loads (the next column's
  // x and tiles), so each wait is a fixed count; one barrier per column.  Up to 32
  // columns the last column is computed without a prefetch (a uniform branch): a dead
  // prefetch past the end would hold the workgroup's exit and its split completion, which
  // wait for every load (gate+up M32 47.2 -> 45.7 us, down and the decode chain's small
  // launches 0.2-0.6 us faster).
  // As in k_gemm, the compiler's schedule (which may wait for tile g before issuing
  // tile g+1) measured faster than a pinned deeper prefetch.
  // x two columns ahead (staged into LDS one column ahead) for the plain sources, and for
  // FP8 up to 32 columns and in the 10-wave 64-column kernel: all workgroups read the same x column at about the same time,
  // so its loads miss together, and waiting for them one column ahead put a memory
  // latency on every column (FP8 gate+up M1 / M32 / M64 38.2 / 40.6 / 46.7 -> 27.1 / 30.2 /
  // 42.7 us; tiled BF16 gate+up M32 / M64 / M128 74.6 / 87.4 / 132.4 -> 66.4 / 81.9 /
  // 121.9 us).  The W12 launches, bound by their larger tile stream, measured no gain (the
  // 4-8 more registers cost them 0.1-0.6 us), and FP8 in the 5-wave 64-column and in the
  // 128-column kernels lost more to the registers (down M64 32.7 -> 41.2 us, gate+up M128
  // 70.6 -> 106.7 us, spilling): they keep x one column ahead.
  constexpr bool kXAhead = !w12_src(SRC) && (MT <= 32 || SRC != SRC_F8 || (MT == 64 && NW == 10));
  uint32_t g = ga;
  xload(0, g);
  tload(tA, g);
  if constexpr (kXAhead) xload(1, g + 1);
  if constexpr (w12_src(SRC)) esc_begin(ec, sv.esc_off, sv.esc, bl, ga * 128u);
  xsumsq(0, true);
  xstore(0, g & 1u);
  __syncthreads();
  constexpr int kA = kXAhead ? 1 : 0;   // register set of the x column staged next
  if constexpr (MT <= 32) {
    // (no RMS sums here: up to 32 columns they come from the MFMA path)
    for (;;) {
      if (g + 1 >= gb) { compute(tA, g); break; }
      xload(0, kXAhead ? g + 2 : g + 1);
      tload(tB, g + 1);
      compute(tA, g);
      xstore(kA, (g + 1) & 1u);
      __syncthreads();
      ++g;
      if (g + 1 >= gb) { compute(tB, g); break; }
      xload(kA, kXAhead ? g + 2 : g + 1);
      tload(tA, g + 1);
      compute(tB, g);
      xstore(0, (g + 1) & 1u);
      __syncthreads();
      ++g;
    }
    __syncthreads();   // every wave is done with the x slots
  } else {
    // 64 and 128 columns: the peeled column's second copy of the compute raised these
    // instantiations' registers past an occupancy step (the tiled BF16 kernel at 64 rows:
    // 94 -> 130 VGPRs, down 41 -> 54 us), so the loop keeps a clamped dead prefetch
    for (;;) {
      xload(0, kXAhead ? g + 2 : g + 1);
      tload(tB, min(g + 1, gb - 1u));
      compute(tA, g);
      xsumsq(kA, g + 1 < gb);
      xstore(kA, (g + 1) & 1u);
      __syncthreads();
      if (++g >= gb) break;
      xload(kA, kXAhead ? g + 2 : g + 1);
      tload(tA, min(g + 1, gb - 1u));
      compute(tB, g);
      xsumsq(0, g + 1 < gb);
      xstore(0, (g + 1) & 1u);
      __syncthreads();
      if (++g >= gb) break;
    }
  }

  // RMS launches: each row's sum of x^2 over the K-range, one value per row in LDS: the
  // four MFMA partials' diagonals (D[c][c] sits in lane c + 16 (c / 4), element c % 4)
  // added in wave order, or the 16 threads of a row's units meeting in a fixed shuffle
  // tree.  With K split, every workgroup also leaves its split's value in its group's
  // slot ss[group][split][row] for the split that completes the group (device scope).
  __shared__ float s_ss[MT];
  const __amdgpu_buffer_rsrc_t ssrs = make_rsrc(p.ss, gridDim.x * gridDim.y * m_rows * 4u);
  if constexpr (kRmsMF) {
    __shared__ float s_xs[4][MT];
    if (wave < 4) {
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (r == 4 * q + i) s_xs[wave][16 * h + r] = racc[h][i];
    }
    __syncthreads();
    if ((uint32_t)tid < MT) {
      const float v = (s_xs[0][tid] + s_xs[1][tid]) + (s_xs[2][tid] + s_xs[3][tid]);
      s_ss[tid] = v;
      if (gridDim.y > 1 && (uint32_t)tid < m_rows)
        st_dev(ssrs, ((blockIdx.x * gridDim.y + blockIdx.y) * m_rows + tid) * 4u, v);
    }
    __syncthreads();
  } else if (rms_valu) {
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
      float v = ssq[i];
#pragma unroll
      for (int off = 8; off >= 1; off >>= 1) v += __shfl_xor(v, off);
      const uint32_t u = (uint32_t)tid + NT * i;
      if ((kUnits * NT == 16 * MT || u < 16u * MT) && (u & 15u) == 0u) {
        s_ss[u >> 4] = v;
        if (gridDim.y > 1 && (u >> 4) < m_rows)
          st_dev(ssrs, ((blockIdx.x * gridDim.y + blockIdx.y) * m_rows + (u >> 4)) * 4u, v);
      }
    }
    __syncthreads();
  }

  const uint32_t n0 = 16u * b + 4u * (uint32_t)q;       // launch numbering (logits, partials)
  const uint32_t n0l = 16u * bl + 4u * (uint32_t)q;     // inside the weight (y)
  if constexpr (EPI == EPI_LOGITS) {
    if (bm.accepted && blockIdx.x == 0 && blockIdx.y == 0)
      accept_init(bm, p.m, (uint32_t)tid, NT);   // verification pass 2 lowers them
    // the workgroup's group record per output row: its waves' row-blocks in order
    __shared__ float s_gv[NW][MT], s_gv2[NW][MT], s_gs[NW][MT];
    __shared__ int32_t s_gi[NW][MT];
    // ||w_v||_2 bounds of the lane's rows 4q+i: D[c][c] sits in lane c + 16 (c / 4),
    // element c % 4
    f32x4 wn;
#pragma unroll
    for (int i = 0; i < 4; ++i) wn[i] = l2_norm_up(__shfl(nacc[i], 20 * q + i), p.k);
    float wmax = fmaxf(fmaxf(wn[0], wn[1]), fmaxf(wn[2], wn[3]));
    wmax = fmaxf(wmax, __shfl_xor(wmax, 16));
    wmax = fmaxf(wmax, __shfl_xor(wmax, 32));   // the row-block's largest
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      const uint32_t m = 16u * h + (uint32_t)r;
      // largest (lowest row on ties) and second largest of this lane's 4 rows;
      // non-finite poisons the block
      float best = acc[h][0], second = -__builtin_inff();
      int bi = 0;
      bool finite = __builtin_isfinite(acc[h][0]);
#pragma unroll
      for (int i = 1; i < 4; ++i) {
        finite = finite && __builtin_isfinite(acc[h][i]);
        if (acc[h][i] > best) { second = best; best = acc[h][i]; bi = i; }
        else if (acc[h][i] > second) second = acc[h][i];
      }
      int row = 4 * q + bi;
      // merge with the lanes holding the block's other rows: the better first wins,
      // the second is the larger of its own second and the other's first
#pragma unroll
      for (int off = 16; off <= 32; off <<= 1) {
        const float ob = __shfl_xor(best, off);
        const float o2 = __shfl_xor(second, off);
        const int orow = __shfl_xor(row, off);
        const int ofin = __shfl_xor((int)finite, off);
        finite = finite && ofin;
        if (ob > best || (ob == best && orow < row)) {
          second = fmaxf(o2, best);
          best = ob;
          row = orow;
        } else {
          second = fmaxf(second, ob);
        }
      }
      if (m < m_rows && bvalid) {
        if (out_f32) {   // full logits and norms only when asked for (verification needs the maxima)
          *reinterpret_cast<f32x4*>(out_f32 + (size_t)m * p.n + n0) = acc[h];
          *reinterpret_cast<f32x4*>(out_s + (size_t)m * p.n + n0) = wn;
        }
        if (q == 0) {
          bm.v[(size_t)m * p.nb + b] = finite ? best : __builtin_nanf("");
          bm.v2[(size_t)m * p.nb + b] = finite ? second : __builtin_nanf("");
          bm.s[(size_t)m * p.nb + b] = wmax;
          bm.i[(size_t)m * p.nb + b] = (int32_t)(16u * b + row);
        }
      }
      if (q == 0) {   // a row-block past the end takes no part in the group record
        const bool live = bvalid && m < m_rows;
        s_gv[wave][m] = !live ? -__builtin_inff() : (finite ? best : __builtin_nanf(""));
        s_gv2[wave][m] = !live ? -__builtin_inff() : second;
        s_gi[wave][m] = (int32_t)(16u * b + row);
        s_gs[wave][m] = live ? wmax : 0.f;
      }
    }
    __syncthreads();
    if ((uint32_t)tid < MT && (uint32_t)tid < m_rows) {
      // the group's two largest logits: a block whose best beats the current best brings
      // its own second, an equal best makes the second equal to it (a tie)
      float v = s_gv[0][tid], v2 = s_gv2[0][tid], sv = s_gs[0][tid], wg = s_gs[0][tid];
      int32_t vi = s_gi[0][tid];
      bool nan = v != v;
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const float vw = s_gv[w][tid];
        nan = nan || vw != vw;
        if (vw > v) { v2 = fmaxf(v, s_gv2[w][tid]); v = vw; vi = s_gi[w][tid]; sv = s_gs[w][tid]; }   // ties: the lower row-block
        else v2 = fmaxf(v2, vw);
        wg = fmaxf(wg, s_gs[w][tid]);
      }
      const size_t o = (size_t)tid * bm.ngrp + blockIdx.x;
      bm.gv[o] = nan ? __builtin_nanf("") : v;
      bm.gv2[o] = nan ? __builtin_nanf("") : v2;
      bm.gi[o] = vi;
      bm.gs[o] = sv;
      bm.gw[o] = wg;
    }
  } else {
    auto store_y = [&](uint32_t m, f32x4 v, float ss) {
      if (rms_on) {
        const float rms = rms_of(ss, p.k);
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = v[i] / rms;
      }
      const uint32_t lo = (uint32_t)f32_to_bf16_rne(v[0]) | ((uint32_t)f32_to_bf16_rne(v[1]) << 16);
      const uint32_t hi = (uint32_t)f32_to_bf16_rne(v[2]) | ((uint32_t)f32_to_bf16_rne(v[3]) << 16);
      *reinterpret_cast<uint2*>(sv.y + (size_t)m * sv.n + n0l) = make_uint2(lo, hi);
    };
    if (gridDim.y == 1) {
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const uint32_t m = 16u * h + (uint32_t)r;
        if (m < m_rows && bvalid) store_y(m, acc[h], rms_on ? s_ss[m] : 0.f);
      }
    } else {
      // K split: this split's partials [split][m][n] (launch numbering) at device scope;
      // the split that completes the group sums all of them in split order
      const __amdgpu_buffer_rsrc_t prs = make_rsrc(out_f32, gridDim.y * m_rows * p.n * 4u);
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const uint32_t m = 16u * h + (uint32_t)r;
        if (m < m_rows && bvalid) st_dev(prs, ((split * m_rows + m) * p.n + n0) * 4u, acc[h]);
      }
      if (split_last(p.tickets, blockIdx.x)) {
        // two 16-row halves at a time have every split's partials requested before any is
        // used (one round trip per pair: the halves one after the other cost the decode
        // chain's split launches a round trip each).  Rows past m read the last row's
        // partials, a wave past the last row-block reads past them (inside the resource,
        // or beyond it, which returns zeros without an access); neither is stored.
        constexpr int kHC = NH < 2 ? NH : 2;
#pragma unroll
        for (int h0 = 0; h0 < NH; h0 += kHC) {
          f32x4 v[kHC][kMaxSplit];
          float ssp[kHC][kMaxSplit];
#pragma unroll
          for (int hh = 0; hh < kHC; ++hh) {
            const uint32_t m = min(16u * (h0 + hh) + (uint32_t)r, m_rows - 1u);
#pragma unroll
            for (uint32_t sp = 0; sp < kMaxSplit; ++sp) {
              const uint32_t spl = min(sp, gridDim.y - 1u);
              v[hh][sp] = ld_dev4(prs, ((spl * m_rows + m) * p.n + n0) * 4u);
              ssp[hh][sp] = rms_on ? ld_dev1(ssrs, ((blockIdx.x * gridDim.y + spl) * m_rows + m) * 4u) : 0.f;
            }
          }
#pragma unroll
          for (int hh = 0; hh < kHC; ++hh) {
            const uint32_t m = 16u * (h0 + hh) + (uint32_t)r;
            if (m >= m_rows || !bvalid) continue;
            f32x4 t = {0.f, 0.f, 0.f, 0.f};
            float ss = 0.f;
#pragma unroll
            for (uint32_t sp = 0; sp < kMaxSplit; ++sp)
              if (sp < gridDim.y) { t += v[hh][sp]; ss += ssp[hh][sp]; }
            store_y(m, t, ss);
          }
        }
      }
    }
  }
}

// Host-side launcher for one weight source: dispatch on m (exact for the VALU path,
// 16 or 32 columns for MFMA), rbw and epilogue.
template <int SRC>
hipError_t launch_gemm_src(const GemmArgs& a, int epi, const GemmPlan& pl, hipStream_t s) {
  dim3 grid(pl.n_rbg, pl.nsplit);
  const GemmParams& p = a.p;
  float* f32 = epi == EPI_LOGITS ? a.logits : a.partial;
#define W12_L(M_, MT_, MF_, RBW_, NWV_, EPI_)                                                     \
  hipLaunchKernelGGL((k_gemm<M_, MT_, MF_, RBW_, NWV_, SRC, EPI_>), grid, dim3(NWV_ * 64), 0, s, \
                     a.x, f32, a.sabs, a.bm, p)
#define W12_RBW(M_, MT_, MF_, EPI_)                   \
  do {                                                \
    if (pl.rbw == 2) W12_L(M_, MT_, MF_, 2, 4, EPI_); \
    else W12_L(M_, MT_, MF_, 1, 4, EPI_);             \
  } while (0)
// (W12 GEMMs with BF16 output, and the logits epilogue from W12_MFMA_MIN_M rows on, always
// run column-synchronous, and the BF16 sources have no logits epilogue: none of them is
// instantiated here)
#define W12_EPI(M_, MT_, MF_)                                                 \
  do {                                                                        \
    if constexpr (SRC == SRC_F8) {                                            \
      return hipErrorInvalidValue; /* FP8 runs column-synchronous only */     \
    } else if constexpr (plain_bf16(SRC)) {                                   \
      if (epi != EPI_BF16) return hipErrorInvalidValue;                       \
      W12_RBW(M_, MT_, MF_, EPI_BF16);                                        \
    } else if constexpr (!MF_) {                                              \
      if (epi != EPI_LOGITS) return hipErrorInvalidValue;                     \
      W12_RBW(M_, MT_, MF_, EPI_LOGITS);                                      \
    } else {                                                                  \
      return hipErrorInvalidValue;                                            \
    }                                                                         \
  } while (0)
#define W12_CS(MT_, EPI_)                                                                     \
  do {                                                                                        \
    if (pl.nw == 10) {                                                                        \
      if constexpr (EPI_ != EPI_LOGITS && (MT_ >= 32 || (MT_ == 16 && plain_bf16(SRC))))       \
        hipLaunchKernelGGL((k_gemm_cs<MT_, 10, SRC, EPI_>), grid, dim3(640), 0, s, a.x, f32,   \
                           a.sabs, a.bm, p);                                                  \
      else                                                                                    \
        return hipErrorInvalidValue; /* not instantiated: the plan never asks for it */      \
    } else if (pl.nw == 8) {                                                                  \
      if constexpr (EPI_ == EPI_LOGITS)                                                       \
        hipLaunchKernelGGL((k_gemm_cs<MT_, 8, SRC, EPI_LOGITS>), grid, dim3(512), 0, s, a.x, f32, \
                           a.sabs, a.bm, p);                                                  \
      else                                                                                    \
        return hipErrorInvalidValue; /* not instantiated: the plan never asks for it */      \
    } else if (pl.nw == 9 || pl.nw == 7) {                                                    \
      if constexpr (EPI_ != EPI_LOGITS && MT_ <= 32 && !plain_bf16(SRC)) {                      \
        if (pl.nw == 9)                                                                       \
          hipLaunchKernelGGL((k_gemm_cs<MT_, 9, SRC, EPI_>), grid, dim3(576), 0, s, a.x, f32,  \
                             a.sabs, a.bm, p);                                                \
        else                                                                                  \
          hipLaunchKernelGGL((k_gemm_cs<MT_, 7, SRC, EPI_>), grid, dim3(448), 0, s, a.x, f32,  \
                             a.sabs, a.bm, p);                                                \
      } else {                                                                                \
        return hipErrorInvalidValue; /* not instantiated: the plan never asks for it */      \
      }                                                                                       \
    } else if (pl.nw == 5)                                                                    \
      hipLaunchKernelGGL((k_gemm_cs<MT_, 5, SRC, EPI_>), grid, dim3(320), 0, s, a.x, f32,     \
                         a.sabs, a.bm, p);                         \
    else                                                                                      \
      hipLaunchKernelGGL((k_gemm_cs<MT_, 4, SRC, EPI_>), grid, dim3(256), 0, s, a.x, f32,     \
                         a.sabs, a.bm, p);                         \
  } while (0)
// (the RMS launches, GemmParams.rms with the BF16 epilogue, run their own instantiation
// up to 32 columns and the BF16 one's runtime path from 64; the BF16 sources have neither
// RMS nor logits launches, FP8 no logits launches)
#define W12_CS_EPI(MT_)                                                     \
  do {                                                                      \
    if (epi == EPI_BF16 && (!p.rms || MT_ >= 64)) W12_CS(MT_, EPI_BF16);   \
    else if constexpr (plain_bf16(SRC)) return hipErrorInvalidValue;       \
    else if constexpr (SRC == SRC_F8) {                                     \
      if (epi == EPI_LOGITS) return hipErrorInvalidValue;                   \
      if constexpr (MT_ <= 32) W12_CS(MT_, EPI_RMS);                        \
      else return hipErrorInvalidValue;                                     \
    }                                                                       \
    else if (epi == EPI_LOGITS) W12_CS(MT_, EPI_LOGITS);                    \
    else if constexpr (MT_ <= 32) W12_CS(MT_, EPI_RMS);                     \
    else return hipErrorInvalidValue;                                       \
  } while (0)
  if (pl.kind != KIND_COLUMN_SYNC && p.rms) return hipErrorInvalidValue;   // (never planned)
  if (pl.kind == KIND_COLUMN_SYNC) {
    if (p.m <= 16) W12_CS_EPI(16);
    else if (p.m <= 32) W12_CS_EPI(32);
    else if (p.m <= 64) W12_CS_EPI(64);
    else W12_CS_EPI(128);
  } else if (pl.mfma) {
    if (p.m <= 4) W12_EPI(4, 16, true);
    else if (p.m <= 8) W12_EPI(8, 16, true);
    else W12_EPI(16, 16, true);
  } else {
#define W12_VCASE(M_)                                          \
  case M_:                                                     \
    if constexpr (M_ < W12_MFMA_MIN_M) W12_EPI(M_, M_, false); \
    break;
    switch (p.m) {
      W12_VCASE(1) W12_VCASE(2) W12_VCASE(3) W12_VCASE(4) W12_VCASE(5)
      W12_VCASE(6) W12_VCASE(7) W12_VCASE(8) W12_VCASE(9) W12_VCASE(10)
      W12_VCASE(11) W12_VCASE(12) W12_VCASE(13) W12_VCASE(14) W12_VCASE(15)
      default: break;
    }
#undef W12_VCASE
  }
#undef W12_CS_EPI
#undef W12_CS
#undef W12_EPI
#undef W12_RBW
#undef W12_L
  return hipGetLastError();
}

}  // namespace w12
