// Exact logits of LM-head rows from the W12 tiles, shared by the verification kernels:
// a BF16 product is +-Mx Mw 2^(Ex+Ew) with 8-bit significands, so sum_k x_k w_vk is an
// integer in units of 2^-266 (review page "SpecPilot: an agent doubled speculative
// decoding speed, and the 10.87x needs context", "The mechanisms it found": certified
// exact-argmax LM head; its caveats: reduction order flips near-ties, which the exact sum
// removes).
#pragma once

#include "w12_internal.h"

namespace w12 {

constexpr int kLimbs = 18;            // 18 x 32 bits > 542 bits (largest |sum| for K < 2^20)
constexpr uint32_t kExactWaves = 8;   // the verification workgroups have 512 threads

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bool exact_parts(uint32_t bits, int& sgn, uint32_t& mant, int& ex) {
  const uint32_t e = (bits >> 7) & 0xFFu, m = bits & 0x7Fu;
  sgn = (bits >> 15) ? -1 : 1;
  mant = e ? (m | 0x80u) : m;
  ex = e ? (int)e - 134 : -133;
  return e != 0xFFu;
}

// Weight (v, kk) of a head of nb row-blocks (tile (b, g) at (g * nb + b) * 3072).
__device__ __forceinline__ uint32_t decode_w(const uint8_t* tiles, uint32_t nb, uint32_t v,
                                             uint32_t kk, const uint32_t lut[4]) {
  const uint32_t b = v >> 4, r = v & 15u, g = kk >> 7, kap = kk & 127u;
  const uint32_t q = (kap >> 3) & 3u, j = kap >> 5, i = kap & 7u;
  const uint32_t l = 16u * q + r, t = 8u * j + i;
  const uint8_t* tb = tiles + ((uint64_t)g * nb + b) * 3072u;
  const uint32_t sm = tb[1024u * (t >> 4) + 16u * l + (t & 15u)];
  const uint32_t cw = *reinterpret_cast<const uint32_t*>(tb + 2048u + 16u * l + 4u * j);
  const uint32_t code = (cw >> (4u * (i >> 1) + 16u * (i & 1u))) & 0xFu;
  const uint32_t e = (lut[code >> 2] >> (8u * (code & 3u))) & 0xFFu;
  return ((sm & 0x80u) << 8) | (e << 7) | (sm & 0x7Fu);
}

// The BF16 weight of element t (0..31) of lane slot l from the slot's sign/mantissa
// words (s_lo: t < 16, s_hi: t >= 16) and its four code words.
__device__ __forceinline__ uint32_t slot_weight(const u32x4& s_lo, const u32x4& s_hi,
                                                const u32x4& cw, uint32_t t,
                                                const uint32_t lut[4]) {
  const uint32_t jj = t >> 3, i = t & 7u;
  const uint32_t sword = t < 16u ? s_lo[(t & 15u) >> 2] : s_hi[(t & 15u) >> 2];
  const uint32_t sm = (sword >> (8u * (t & 3u))) & 0xFFu;
  const uint32_t code = (cw[jj] >> (4u * (i >> 1) + 16u * (i & 1u))) & 0xFu;
  const uint32_t e = (lut[code >> 2] >> (8u * (code & 3u))) & 0xFFu;
  return ((sm & 0x80u) << 8) | (e << 7) | (sm & 0x7Fu);
}

// Add sign * x * w (BF16 bits) to a lane's column of limbs (units of 2^-266); false if
// either value is not finite.
__device__ __forceinline__ bool limb_term(unsigned long long* col, uint32_t xb, uint32_t wb,
                                          bool subtract) {
  int sx, sw, ex, ew;
  uint32_t mx, mw;
  const bool okx = exact_parts(xb, sx, mx, ex), okw = exact_parts(wb, sw, mw, ew);
  const uint32_t prod = mx * mw;   // < 2^16
  if (prod != 0u) {
    const int sh = ex + ew + 266;   // 0 .. 506
    const unsigned long long v = (unsigned long long)prod << (sh & 31);
    long long lo = (long long)(v & 0xFFFFFFFFull), hi = (long long)(v >> 32);
    if (((sx * sw) < 0) != subtract) { lo = -lo; hi = -hi; }
    const int idx = sh >> 5;
    col[idx * 64] += (unsigned long long)lo;
    col[(idx + 1) * 64] += (unsigned long long)hi;
  }
  return okx && okw;
}

// LDS of the exact stage: one limb column per lane of each wave, the survivors' digits.
struct ExactShared {
  unsigned long long limb[kExactWaves][kLimbs * 64];
  uint32_t dig[kExactWaves][kLimbs];
  int32_t sgn[kExactWaves], vid[kExactWaves];
  uint32_t best[kLimbs];
  int32_t best_v, best_sign;
  uint32_t bad;
};

// One x row against the W12 head.
struct ExactRow {
  const uint16_t* xr;       // [k] BF16
  const uint8_t* tiles;
  const uint32_t* esc;
  uint32_t nb, g_cols, k;
  const uint32_t* lut;      // [4]: the codebook as a byte lookup
};

// The exact argmax over ns candidate rows, called by every thread of a workgroup of
// kExactWaves waves: get(c) is candidate c's row, range(c, e0, e1) its row-block's escape
// range.  Each candidate's sum_k x_k w_vk is accumulated as an integer in units of 2^-266,
// one wave per candidate (kExactWaves at a time): lane l adds its products into limb column
// l (no two lanes share a word), escapes replace the product decoded with code 0, then 18
// lanes sum the columns and lane 0 carries them into 32-bit digits and a sign.  Returns,
// in every thread, the row with the largest exact sum (lowest index on an exact tie), or
// -1 if a value is not finite.
template <class Get, class Range>
__device__ int32_t exact_best(ExactShared& ex, const ExactRow& c, uint32_t ns, Get get,
                              Range range) {
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  if (tid == 0) { ex.best_v = -1; ex.best_sign = 0; ex.bad = 0; }
  __syncthreads();
  for (uint32_t c0i = 0; c0i < ns; c0i += kExactWaves) {
    const uint32_t ci = c0i + wave;
    unsigned long long* col = &ex.limb[wave][lane];
#pragma unroll
    for (int i = 0; i < kLimbs; ++i) col[i * 64] = 0ull;
    bool ok = true;
    if (ci < ns) {
      const uint32_t v = (uint32_t)get(ci), b = v >> 4, r = v & 15u;
      for (uint32_t j = lane; j < 4u * c.g_cols; j += 64u) {
        const uint32_t g = j >> 2, q = j & 3u, l = 16u * q + r;
        const uint8_t* tb = c.tiles + ((uint64_t)g * c.nb + b) * 3072u + 16u * l;
        const u32x4 s_lo = *reinterpret_cast<const u32x4*>(tb);
        const u32x4 s_hi = *reinterpret_cast<const u32x4*>(tb + 1024);
        const u32x4 cw = *reinterpret_cast<const u32x4*>(tb + 2048);
#pragma unroll
        for (uint32_t jj = 0; jj < 4; ++jj) {
          const u32x4 xv = *reinterpret_cast<const u32x4*>(c.xr + 128u * g + 32u * jj + 8u * q);
#pragma unroll
          for (uint32_t i = 0; i < 8; ++i) {
            const uint32_t wb = slot_weight(s_lo, s_hi, cw, 8u * jj + i, c.lut);
            const uint32_t xb = (xv[i >> 1] >> (16u * (i & 1u))) & 0xFFFFu;
            ok = limb_term(col, xb, wb, false) && ok;
          }
        }
      }
      uint32_t e0, e1;
      range(ci, e0, e1);
      for (uint32_t i = e0 + lane; i < e1; i += 64u) {
        const uint32_t rec = c.esc[i];
        const uint32_t kk = (rec >> 8) & 0xFFFFFu;
        if ((rec >> 28) != r || kk >= c.k) continue;   // another row, or malformed
        const uint32_t wb = decode_w(c.tiles, c.nb, v, kk, c.lut);
        const uint32_t wt = (wb & 0x807Fu) | ((rec & 0xFFu) << 7);
        limb_term(col, c.xr[kk], wb, true);
        ok = limb_term(col, c.xr[kk], wt, false) && ok;
      }
      if (!ok) atomicOr(&ex.bad, 1u);
    }
    __syncthreads();   // every lane's column is written
    if (ci < ns && lane < (uint32_t)kLimbs) {
      long long t = 0;
      for (uint32_t l = 0; l < 64u; ++l) t += (long long)ex.limb[wave][lane * 64u + l];
      ex.limb[wave][lane * 64u] = (unsigned long long)t;   // column 0 of limb `lane`: the row sum
    }
    __syncthreads();   // the column sums are written
    if (ci < ns && lane == 0) {
      // normalise to 32-bit digits; the final carry is the sign (0 or -1)
      long long carry = 0;
      for (int i = 0; i < kLimbs; ++i) {
        const long long t = (long long)ex.limb[wave][i * 64] + carry;
        ex.dig[wave][i] = (uint32_t)(t & 0xFFFFFFFFll);
        carry = t >> 32;
      }
      ex.sgn[wave] = (int32_t)carry;
      ex.vid[wave] = (int32_t)get(ci);
    }
    __syncthreads();
    if (tid == 0) {   // this batch of candidates (one per wave) against the best so far
      for (uint32_t w = 0; w < kExactWaves && c0i + w < ns; ++w) {
        bool better;
        if (ex.best_v < 0) {
          better = true;
        } else if (ex.sgn[w] != ex.best_sign) {
          better = ex.sgn[w] > ex.best_sign;
        } else {
          int cmp = 0;
          for (int i = kLimbs - 1; i >= 0 && cmp == 0; --i)
            cmp = ex.dig[w][i] > ex.best[i] ? 1 : (ex.dig[w][i] < ex.best[i] ? -1 : 0);
          better = cmp > 0 || (cmp == 0 && ex.vid[w] < ex.best_v);
        }
        if (better) {
          for (int i = 0; i < kLimbs; ++i) ex.best[i] = ex.dig[w][i];
          ex.best_sign = ex.sgn[w];
          ex.best_v = ex.vid[w];
        }
      }
    }
    __syncthreads();
  }
  return ex.bad ? -1 : ex.best_v;
}

}  // namespace w12
