// The W12 decode/verification GEMM kernel family for gfx950 (MI355X).
//
// y[m][n] = sum_k x[m][k] * W[n][k] for m < M <= 32, W streamed once from HBM.
// W12 weights are decoded to BF16 pairs in registers ("StargazerX0/SpecPilot", "What
// it is": decoding happens bit-exactly inside the GEMM; review page, "The mechanisms
// it found": 12 instead of 16 bits per weight cuts the weight traffic by a quarter).
//
// Work decomposition
//   workgroup = 4 waves = RBW consecutive row-blocks (16 rows each) x a K-range of
//   tile columns [ga, gb) (blockIdx.y selects the split).  The K-range is processed in
//   chunks of 4 tile columns; wave w takes column c0 + w of each chunk, so the four
//   waves stream four adjacent 3 KB tiles per row-block.  x for the chunk is staged
//   through LDS (register prefetch one chunk ahead, so the global x loads are issued
//   before the tile prefetch and never make a wait on the tiles necessary).
//   Tile loads are issued one chunk ahead (double-buffered registers).
// Per tile, lane l (row r = l%16, k-group q = l/16) holds the 32 weights of its slot:
//   three coalesced 16-byte loads per lane (1 KB per wave instruction), unpacked into
//   16 BF16 pairs P[4j+p] = {w(k0+2p), w(k0+2p+1)} with k0 = 32j + 8q.  Those 8 BF16 of
//   group j are exactly the lane's A operand of v_mfma_f32_16x16x32_bf16 (row r,
//   k = 8q..8q+7 of the 32-wide step), and adjacent-k pairs for v_dot2_f32_bf16.
// M <= 15: VALU path, v_dot2 (2 MACs per instruction) with x pairs read from LDS as
//   broadcast ds_read_b128 (16 lanes share each address); partial sums are reduced
//   across the 4 lanes that share a row with cross-lane shuffles, then across waves.
// M >= 16: MFMA path, W tile as the 16-row A operand, x as the B operand (16 or 32
//   columns, rows >= M zero-filled in LDS).
// Escapes (exponents outside the codebook) are patched into the unpacked registers by
//   the owning lane, walking the row-block's sorted escape list with a 64-record
//   window held one record per lane (ballot selects the records of the current tile).
// Split-K (blockIdx.y > 0 exists): FP32 partials go to the workspace and the last
//   workgroup to arrive (ticket counter) sums them in split order -- deterministic --
//   and resets the counter to zero for the next call.
#pragma once

#include "w12_internal.h"

namespace w12 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

constexpr int kWaves = 4;
constexpr int kThreads = 256;
constexpr int kChunk = 4;                        // tile columns per LDS x chunk
constexpr int kXsStride = kChunk * 128 + 8;      // BF16 per LDS row (+16 B pad: no bank
                                                 // conflicts for the MFMA B reads)

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
  u32x4 v[SRC == SRC_BF16 ? 4 : 3];
};

template <int SRC>
__device__ __forceinline__ void load_tile(TileRegs<SRC>& t, const GemmArgs& a, uint32_t b,
                                          uint32_t g, int lane) {
  if constexpr (SRC == SRC_BF16) {
    const int r = lane & 15, q = lane >> 4;
    const uint8_t* base = a.w + ((size_t)(16u * b + r) * a.k + 128u * g + 8u * q) * 2u;
#pragma unroll
    for (int j = 0; j < 4; ++j) t.v[j] = *reinterpret_cast<const u32x4*>(base + 64 * j);
  } else {
    const uint8_t* base = a.w + ((size_t)b * a.g_cols + g) * 3072u + (uint32_t)lane * 16u;
#pragma unroll
    for (int s = 0; s < 3; ++s) t.v[s] = *reinterpret_cast<const u32x4*>(base + 1024 * s);
  }
}

// Registers -> 16 BF16 pairs (P[4j+p] = element 2p in the low half, 2p+1 in the high).
template <int SRC>
__device__ __forceinline__ void unpack_tile(const TileRegs<SRC>& t, const GemmArgs& a,
                                            uint32_t P[16]) {
  if constexpr (SRC == SRC_BF16) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int p = 0; p < 4; ++p) P[4 * j + p] = t.v[j][p];
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

// Escape cursor of one row-block: records [pos, end) not yet consumed; lane i of `win`
// holds record wb + i.
struct EscCursor {
  uint32_t pos, end, wb, win;
};

__device__ __forceinline__ void esc_load_window(EscCursor& c, const uint32_t* esc, int lane) {
  c.wb = c.pos;
  const uint32_t idx = c.pos + (uint32_t)lane;
  c.win = (idx < c.end) ? esc[idx] : 0xFFFFFFFFu;
}

// Position the cursor at the first record with column >= kmin.
__device__ __forceinline__ void esc_seek(EscCursor& c, const uint32_t* esc, uint32_t kmin,
                                         int lane) {
  for (;;) {
    esc_load_window(c, esc, lane);
    if (kmin == 0u || c.pos >= c.end) return;
    const uint32_t kk = (c.win >> 8) & 0xFFFFFu;
    const bool below = (c.wb + (uint32_t)lane < c.end) && kk < kmin;
    const uint32_t nbelow = (uint32_t)__builtin_popcountll(__builtin_amdgcn_ballot_w64(below));
    c.pos += nbelow;
    if (nbelow < 64u) return;
  }
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

// Patch the escapes of tile column g into P (records sorted by column, then row).
__device__ __forceinline__ void esc_apply(EscCursor& c, const uint32_t* esc, uint32_t g,
                                          int lane, uint32_t P[16]) {
  if (c.pos >= c.end) return;
  const uint32_t klo = g * 128u, khi = klo + 128u;
  for (;;) {
    const uint32_t li = c.pos - c.wb;
    const uint32_t kk = (c.win >> 8) & 0xFFFFFu;
    const bool valid = ((uint32_t)lane >= li) && (c.wb + (uint32_t)lane < c.end);
    const uint64_t below = __builtin_amdgcn_ballot_w64(valid && kk < khi);
    uint64_t hit = __builtin_amdgcn_ballot_w64(valid && kk >= klo && kk < khi);
    while (hit) {
      const int bit = __builtin_ctzll(hit);
      hit &= hit - 1;
      const uint32_t rec = __builtin_amdgcn_readlane(c.win, bit);
      const uint32_t rr = rec >> 28;
      const uint32_t kap = ((rec >> 8) & 0xFFFFFu) - klo;
      const uint32_t j = kap >> 5, qq = (kap >> 3) & 3u, i = kap & 7u;
      const uint32_t owner = 16u * qq + rr;
      patch_pair(P, 4u * j + (i >> 1), 7u + 16u * (i & 1u), rec & 0xFFu, (uint32_t)lane == owner);
    }
    c.pos += (uint32_t)__builtin_popcountll(below);
    if (c.pos >= c.end || c.pos - c.wb < 64u) return;
    esc_load_window(c, esc, lane);   // window used up: the next records may still be < khi
  }
}

template <int MT>
struct XStage {
  static constexpr int kUnits = (MT * 64 + kThreads - 1) / kThreads;   // 16-byte units
  u32x4 v[kUnits];
};

template <int MT>
__device__ __forceinline__ void x_load(XStage<MT>& st, const GemmArgs& a, uint32_t m_rows,
                                       uint32_t c0, uint32_t gb, int tid) {
#pragma unroll
  for (int i = 0; i < XStage<MT>::kUnits; ++i) {
    const uint32_t u = (uint32_t)tid + kThreads * i;
    const uint32_t m = u >> 6, cu = u & 63u;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (u < MT * 64u && m < m_rows && c0 + (cu >> 4) < gb)
      v = *reinterpret_cast<const u32x4*>(a.x + (size_t)m * a.k + 128u * c0 + 8u * cu);
    st.v[i] = v;
  }
}

template <int MT>
__device__ __forceinline__ void x_store(const XStage<MT>& st, uint16_t* xs, int tid) {
#pragma unroll
  for (int i = 0; i < XStage<MT>::kUnits; ++i) {
    const uint32_t u = (uint32_t)tid + kThreads * i;
    if (u < MT * 64u) {
      const uint32_t m = u >> 6, cu = u & 63u;
      *reinterpret_cast<u32x4*>(xs + m * kXsStride + 8u * cu) = st.v[i];
    }
  }
}

// M: rows for the VALU path (compile-time); MT: LDS rows (= M, or 16/32 for MFMA).
template <int M, int MT, bool MF, int RBW, int SRC, int EPI>
__global__ __launch_bounds__(kThreads) void k_gemm(GemmArgs a) {
  constexpr int NH = MF ? MT / 16 : 1;
  __shared__ __align__(16) uint16_t xs[MT * kXsStride];
  __shared__ float fin[RBW * MT * 16];
  __shared__ uint32_t s_last;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, q = lane >> 4;
  const uint32_t rbg = blockIdx.x, split = blockIdx.y;
  const uint32_t b0 = rbg * RBW;
  const uint32_t ga = split * a.cols_per_split;
  const uint32_t gb = min(a.g_cols, ga + a.cols_per_split);
  const uint32_t m_rows = MF ? a.m : (uint32_t)M;

  float vacc[RBW][MF ? 1 : M];
  f32x4 macc[RBW][NH];
#pragma unroll
  for (int rb = 0; rb < RBW; ++rb) {
#pragma unroll
    for (int m = 0; m < (MF ? 1 : M); ++m) vacc[rb][m] = 0.f;
#pragma unroll
    for (int h = 0; h < NH; ++h) macc[rb][h] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  EscCursor ec[RBW];
  if constexpr (SRC != SRC_BF16) {
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      const uint32_t b = b0 + rb;
      if (b < a.nb) {
        ec[rb].pos = __builtin_amdgcn_readfirstlane(a.esc_off[b]);
        ec[rb].end = __builtin_amdgcn_readfirstlane(a.esc_off[b + 1]);
        esc_seek(ec[rb], a.esc, ga * 128u, lane);
      } else {
        ec[rb].pos = ec[rb].end = ec[rb].wb = 0u;
        ec[rb].win = 0xFFFFFFFFu;
      }
    }
  }

  TileRegs<SRC> tA[RBW], tB[RBW];
  XStage<MT> xr;

  auto load_tiles = [&](TileRegs<SRC>* t, uint32_t g) {
    if (g < gb) {
#pragma unroll
      for (int rb = 0; rb < RBW; ++rb)
        if (b0 + rb < a.nb) load_tile<SRC>(t[rb], a, b0 + rb, g, lane);
    }
  };

  auto compute = [&](const TileRegs<SRC>* t, uint32_t g) {
    if (g >= gb) return;
    uint32_t P[RBW][16];
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb) {
      unpack_tile<SRC>(t[rb], a, P[rb]);
      if constexpr (SRC != SRC_BF16) esc_apply(ec[rb], a.esc, g, lane, P[rb]);
    }
    const uint16_t* xrow = xs + 128 * wave + 8 * q;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (MF) {
#pragma unroll
        for (int h = 0; h < NH; ++h) {
          const u32x4 xv = *reinterpret_cast<const u32x4*>(xrow + (16 * h + r) * kXsStride + 32 * j);
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
            for (int p = 0; p < 4; ++p)
              vacc[rb][m] = __builtin_amdgcn_fdot2_f32_bf16(
                  as_bf16x2(P[rb][4 * j + p]), as_bf16x2(xv[p]), vacc[rb][m], false);
        }
      }
    }
  };

  // ---- main loop: chunk c0 computes from LDS while chunk c0+4 is in flight
  uint32_t c0 = ga;
  x_load<MT>(xr, a, m_rows, c0, gb, tid);
  load_tiles(tA, c0 + wave);
  x_store<MT>(xr, xs, tid);
  __syncthreads();
  for (;;) {
    uint32_t c1 = c0 + kChunk;
    if (c1 < gb) {
      x_load<MT>(xr, a, m_rows, c1, gb, tid);
      load_tiles(tB, c1 + wave);
    }
    compute(tA, c0 + wave);
    if (c1 >= gb) break;
    __syncthreads();
    x_store<MT>(xr, xs, tid);
    __syncthreads();
    c0 = c1;
    c1 = c0 + kChunk;
    if (c1 < gb) {
      x_load<MT>(xr, a, m_rows, c1, gb, tid);
      load_tiles(tA, c1 + wave);
    }
    compute(tB, c0 + wave);
    if (c1 >= gb) break;
    __syncthreads();
    x_store<MT>(xr, xs, tid);
    __syncthreads();
    c0 = c1;
  }
  __syncthreads();   // LDS x no longer read: reuse it for the cross-wave reduction

  // ---- cross-lane / cross-wave reduction into red[] (aliases xs)
  float* red = reinterpret_cast<float*>(xs);
  if constexpr (MF) {
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
      for (int h = 0; h < NH; ++h)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          red[(((wave * RBW + rb) * NH + h) * 4 + i) * 64 + lane] = macc[rb][h][i];
  } else {
#pragma unroll
    for (int rb = 0; rb < RBW; ++rb)
#pragma unroll
      for (int m = 0; m < M; ++m) {
        float v = vacc[rb][m];
        v += __shfl_xor(v, 16);
        v += __shfl_xor(v, 32);
        if (q == 0) red[((wave * RBW + rb) * M + m) * 16 + r] = v;
      }
  }
  __syncthreads();

  constexpr int kOut = RBW * MT * 16;   // (rb, m, row) outputs of this workgroup
  auto final_value = [&](int o) -> float {
    const int rb = o / (MT * 16), rem = o % (MT * 16), m = rem >> 4, rr = rem & 15;
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      if constexpr (MF) {
        const int h = m >> 4, ln = 16 * (rr >> 2) + (m & 15), i = rr & 3;
        s += red[(((w * RBW + rb) * NH + h) * 4 + i) * 64 + ln];
      } else {
        s += red[((w * RBW + rb) * M + m) * 16 + rr];
      }
    }
    return s;
  };

  if constexpr (EPI == EPI_LOGITS) {
    for (int o = tid; o < kOut; o += kThreads) {
      const int rb = o / (MT * 16), rem = o % (MT * 16), m = rem >> 4, rr = rem & 15;
      const uint32_t b = b0 + rb;
      const float v = final_value(o);
      fin[o] = v;
      if (b < a.nb && (uint32_t)m < m_rows) a.logits[(size_t)m * a.n + 16u * b + rr] = v;
    }
    __syncthreads();
    for (int o = tid; o < RBW * MT; o += kThreads) {
      const int rb = o / MT, m = o % MT;
      const uint32_t b = b0 + rb;
      if (b >= a.nb || (uint32_t)m >= m_rows) continue;
      float best = fin[o * 16];
      int bi = 0;
      bool finite = __builtin_isfinite(best);
      for (int rr = 1; rr < 16; ++rr) {
        const float v = fin[o * 16 + rr];
        finite = finite && __builtin_isfinite(v);
        if (v > best) { best = v; bi = rr; }
      }
      a.rbmax_v[(size_t)m * a.nb + b] = finite ? best : __builtin_nanf("");
      a.rbmax_i[(size_t)m * a.nb + b] = (int32_t)(16u * b + bi);
    }
    return;
  } else {
    if (a.nsplit == 1) {
      for (int o = tid; o < kOut; o += kThreads) {
        const int rb = o / (MT * 16), rem = o % (MT * 16), m = rem >> 4, rr = rem & 15;
        const uint32_t b = b0 + rb;
        const float v = final_value(o);
        if (b < a.nb && (uint32_t)m < m_rows) a.y[(size_t)m * a.n + 16u * b + rr] = f32_to_bf16_rne(v);
      }
      return;
    }
    for (int o = tid; o < kOut; o += kThreads) {
      const int rb = o / (MT * 16), rem = o % (MT * 16), m = rem >> 4, rr = rem & 15;
      const uint32_t b = b0 + rb;
      const float v = final_value(o);
      if (b < a.nb && (uint32_t)m < m_rows)
        __hip_atomic_store(a.partial + ((size_t)split * m_rows + m) * a.n + 16u * b + rr, v,
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
      const uint32_t t = __hip_atomic_fetch_add(a.counters + rbg, 1u, __ATOMIC_ACQ_REL,
                                                __HIP_MEMORY_SCOPE_AGENT);
      s_last = (t == a.nsplit - 1u) ? 1u : 0u;
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    for (int o = tid; o < kOut; o += kThreads) {
      const int rb = o / (MT * 16), rem = o % (MT * 16), m = rem >> 4, rr = rem & 15;
      const uint32_t b = b0 + rb;
      if (b >= a.nb || (uint32_t)m >= m_rows) continue;
      float s = 0.f;
      for (uint32_t sp = 0; sp < a.nsplit; ++sp)
        s += __hip_atomic_load(a.partial + ((size_t)sp * m_rows + m) * a.n + 16u * b + rr,
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      a.y[(size_t)m * a.n + 16u * b + rr] = f32_to_bf16_rne(s);
    }
    if (tid == 0)
      __hip_atomic_store(a.counters + rbg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Host-side launcher for one weight source: dispatch on m (exact for the VALU path,
// 16 or 32 columns for MFMA), rbw and epilogue.
template <int SRC>
hipError_t launch_gemm_src(const GemmArgs& a, int epi, const GemmPlan& p, hipStream_t s) {
  dim3 grid(p.n_rbg, p.nsplit), block(kThreads);
#define W12_L(M_, MT_, MF_, RBW_, EPI_) \
  hipLaunchKernelGGL((k_gemm<M_, MT_, MF_, RBW_, SRC, EPI_>), grid, block, 0, s, a)
#define W12_RBW(M_, MT_, MF_, EPI_)            \
  do {                                         \
    if (p.rbw == 1) W12_L(M_, MT_, MF_, 1, EPI_); \
    else W12_L(M_, MT_, MF_, 2, EPI_);          \
  } while (0)
#define W12_EPI(M_, MT_, MF_)                                       \
  do {                                                              \
    if (epi == EPI_BF16) W12_RBW(M_, MT_, MF_, EPI_BF16);          \
    else if constexpr (SRC != SRC_BF16) W12_RBW(M_, MT_, MF_, EPI_LOGITS); \
  } while (0)
  switch (a.m) {
    case 1: W12_EPI(1, 1, false); break;
    case 2: W12_EPI(2, 2, false); break;
    case 3: W12_EPI(3, 3, false); break;
    case 4: W12_EPI(4, 4, false); break;
    case 5: W12_EPI(5, 5, false); break;
    case 6: W12_EPI(6, 6, false); break;
    case 7: W12_EPI(7, 7, false); break;
    case 8: W12_EPI(8, 8, false); break;
    case 9: W12_EPI(9, 9, false); break;
    case 10: W12_EPI(10, 10, false); break;
    case 11: W12_EPI(11, 11, false); break;
    case 12: W12_EPI(12, 12, false); break;
    case 13: W12_EPI(13, 13, false); break;
    case 14: W12_EPI(14, 14, false); break;
    case 15: W12_EPI(15, 15, false); break;
    case 16: W12_EPI(16, 16, true); break;
    default: W12_EPI(32, 32, true); break;
  }
#undef W12_EPI
#undef W12_RBW
#undef W12_L
  return hipGetLastError();
}

}  // namespace w12
