// Greedy verification epilogue: certified exact argmax over the LM-head logits and
// the accepted-prefix length.
//
// Pass 1 (the GEMM kernel family with the logits epilogue) leaves, per row and per
// 16-row block of the head, the largest FP32 logit z^ (with its index), the second
// largest, and the largest S^ = the same kernel's FP32 sum of |x_k||w_vk| over the
// block's rows.  Pass 2 (one workgroup per row):
//   1. z* = max z^ over the block maxima (lowest index on ties), S* the largest S^ of
//      its block (an upper bound of its own S^);
//   2. the error bound.  A product of two BF16 values is exact in FP32 unless it
//      underflows.  Whatever the summation order, each of the K products of a logit
//      passes through at most D = K + 64 additions (the slack covers the accumulators'
//      zero starts and the cross-wave sums), each with relative error below
//      eps = 2^-23 (round-to-nearest or toward zero), so with g = D eps / (1 - D eps)
//        |z^ - z| <= g S + A,   S = sum_k |x_k w_k|,
//      A = D 2^-126 (1 + Xmax + Wmax) covering flushed denormal inputs, products and
//      partial sums (Xmax = max |x_k|, Wmax = 2^(e_max-126) > |w|).  S^ sums the same
//      nonnegative terms, so S <= S^/(1-g) + A, and B(S^) = g (S^/(1-g) + A) + A,
//      inflated by 2^-20 for its FP64 evaluation, bounds |z^ - z|; B grows with S^;
//   3. L = z* - B(S*) is below the true maximum, so every v with z^_v + B(S^_v) >= L
//      is a candidate (the exact argmax always is).  With the block's largest S^ in B,
//      a block adds its largest logit when that reaches L, and all of its rows when its
//      second largest does too (otherwise no other row of it can);
//   4. FP64 screen: each candidate's logit is recomputed from the W12 tiles in FP64 (a
//      BF16 product is exact in FP64; escape corrections add two terms each), within
//      g64 S64 of the exact value; only the candidates whose FP64 upper bound reaches
//      the largest FP64 lower bound survive;
//   5. when more than one survives, each survivor's logit is recomputed exactly:
//      sum_k x_k w_vk as an integer in units of 2^-266 (a BF16 product is
//      +-Mx*Mw*2^(Ex+Ew) with 8-bit significands), accumulated in 64-bit LDS limbs; the
//      largest exact value wins, lowest index on an exact tie.
// The review page ("The mechanisms it found") names a certified exact-argmax LM head,
// and its caveats note that reduction order can flip near-ties: the exact logit makes
// the answer independent of the order.  Accept: first i < n_draft with
// argmax[i] != draft[i], else n_draft ("StargazerX0/SpecPilot", "Results and
// verification": every committed token is the target's own choice): pass 1 sets it to
// n_draft and every row i < n_draft whose argmax differs from the draft lowers it to i
// with an atomic minimum.  Batched, each request applies the same rule to its own rows
// (its i counted from its first row), with its own accepted length.
#include "w12_internal.h"

namespace w12 {

constexpr int kLimbs = 18;   // 18 x 32 bits > 542 bits (largest |sum| for K < 2^20)
constexpr uint32_t kScreenMax = 512;   // candidates screened in FP64 (more: all go exact)
constexpr uint32_t kGroup = 4;         // candidates screened at once, kT / kGroup threads each
constexpr uint32_t kCache = 9728;      // block maxima kept in LDS for the candidate scan

__device__ __forceinline__ bool exact_parts(uint32_t bits, int& sgn, uint32_t& mant, int& ex) {
  const uint32_t e = (bits >> 7) & 0xFFu, m = bits & 0x7Fu;
  sgn = (bits >> 15) ? -1 : 1;
  mant = e ? (m | 0x80u) : m;
  ex = e ? (int)e - 134 : -133;
  return e != 0xFFu;
}

// Weight (v, kk) of a head of nb row-blocks (tile (b, g) at (g * nb + b) * 3072).
__device__ __forceinline__ uint32_t decode_w(const uint8_t* tiles, uint32_t nb, uint32_t v,
                                             uint32_t kk, const uint32_t lut[4],
                                             uint32_t* code_out) {
  const uint32_t b = v >> 4, r = v & 15u, g = kk >> 7, kap = kk & 127u;
  const uint32_t q = (kap >> 3) & 3u, j = kap >> 5, i = kap & 7u;
  const uint32_t l = 16u * q + r, t = 8u * j + i;
  const uint8_t* tb = tiles + ((uint64_t)g * nb + b) * 3072u;
  const uint32_t sm = tb[1024u * (t >> 4) + 16u * l + (t & 15u)];
  const uint32_t cw = *reinterpret_cast<const uint32_t*>(tb + 2048u + 16u * l + 4u * j);
  const uint32_t code = (cw >> (4u * (i >> 1) + 16u * (i & 1u))) & 0xFu;
  const uint32_t e = (lut[code >> 2] >> (8u * (code & 3u))) & 0xFFu;
  *code_out = code;
  return ((sm & 0x80u) << 8) | (e << 7) | (sm & 0x7Fu);
}

__device__ __forceinline__ void limb_add(unsigned long long* limbs, int sgn, uint32_t prod, int sh,
                                         bool subtract) {
  if (prod == 0) return;
  const unsigned long long v = (unsigned long long)prod << (sh & 31);
  const int idx = sh >> 5;
  long long lo = (long long)(v & 0xFFFFFFFFull), hi = (long long)(v >> 32);
  if ((sgn < 0) != subtract) { lo = -lo; hi = -hi; }
  if (lo) atomicAdd(limbs + idx, (unsigned long long)lo);
  if (hi) atomicAdd(limbs + idx + 1, (unsigned long long)hi);
}

constexpr uint32_t kT = 512;   // threads of the pass-2 workgroup (one workgroup per row)

__global__ __launch_bounds__(kT) void k_verify_pass2(VerifyArgs a) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __shared__ float s_bv[kT];
  __shared__ int32_t s_bi[kT];
  __shared__ double s_d0[kT], s_d1[kT];
  __shared__ uint32_t s_u0[kT];
  __shared__ unsigned long long limbs[kLimbs];
  __shared__ uint32_t best[kLimbs];
  __shared__ int32_t s_best_v, s_best_sign;
  __shared__ uint32_t s_cnt, s_bad, s_nsurv;
  __shared__ double s_z64[kScreenMax], s_b64[kScreenMax];
  __shared__ float s_rv[kCache], s_rs[kCache];
  __shared__ int32_t s_cand[kScreenMax];   // the first candidates (the rest in global memory)
  const uint32_t row = blockIdx.x, tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint16_t* xr = a.x + (uint64_t)row * a.k;
  const float* rv = a.rbmax_v + (uint64_t)row * a.nb;
  const float* rv2 = a.rbmax_v2 + (uint64_t)row * a.nb;
  const float* rs = a.rbmax_s + (uint64_t)row * a.nb;
  const int32_t* ri = a.rbmax_i + (uint64_t)row * a.nb;
  int32_t* cand = a.cand + (uint64_t)row * a.n;
  auto put = [&](uint32_t c, int32_t v) { if (c < kScreenMax) s_cand[c] = v; else cand[c] = v; };
  auto get = [&](uint32_t c) { return c < kScreenMax ? s_cand[c] : cand[c]; };
  int32_t result = -1;
  uint32_t ncand = 0, nsurv = 0;

  // 1. z* and its index over the block maxima (NaN marks a non-finite block); the
  // maxima and their S are kept in LDS for the candidate scan (up to kCache blocks)
  float bv = -__builtin_inff();
  int32_t bi = 0x7FFFFFFF;
  bool bad = false;
  auto take = [&](uint32_t b, float v, int32_t i, float sb) {
    if (b < kCache) { s_rv[b] = v; s_rs[b] = sb; }
    if (v != v) bad = true;
    else if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
  };
  // Every scan below issues all of a thread's loads of a chunk (clamped indices) before
  // using any, so a chunk costs one memory latency; the result does not depend on the
  // order (largest value, lowest index on ties).
  if ((a.nb & 3u) == 0u) {   // rows start on 16-byte boundaries: four blocks per load
    typedef float f32x4v __attribute__((ext_vector_type(4)));
    typedef int32_t i32x4v __attribute__((ext_vector_type(4)));
    constexpr uint32_t kU = 6;
    const uint32_t nb4 = a.nb / 4u;
    for (uint32_t base = 0; base < nb4; base += kT * kU) {
      f32x4v v[kU], sb[kU];
      i32x4v iv[kU];
#pragma unroll
      for (uint32_t u = 0; u < kU; ++u) {
        const uint32_t b4 = min(base + u * kT + tid, nb4 - 1u);
        v[u] = reinterpret_cast<const f32x4v*>(rv)[b4];
        iv[u] = reinterpret_cast<const i32x4v*>(ri)[b4];
        sb[u] = reinterpret_cast<const f32x4v*>(rs)[b4];
      }
#pragma unroll
      for (uint32_t u = 0; u < kU; ++u) {
        const uint32_t b4 = base + u * kT + tid;
        if (b4 < nb4) {
#pragma unroll
          for (uint32_t j = 0; j < 4; ++j) take(4u * b4 + j, v[u][j], iv[u][j], sb[u][j]);
        }
      }
    }
  } else {
    constexpr uint32_t kU = 8;
    for (uint32_t base = 0; base < a.nb; base += kT * kU) {
      float v[kU], sb[kU];
      int32_t iv[kU];
#pragma unroll
      for (uint32_t u = 0; u < kU; ++u) {
        const uint32_t b = min(base + u * kT + tid, a.nb - 1u);
        v[u] = rv[b];
        iv[u] = ri[b];
        sb[u] = rs[b];
      }
#pragma unroll
      for (uint32_t u = 0; u < kU; ++u)
        if (base + u * kT + tid < a.nb) take(base + u * kT + tid, v[u], iv[u], sb[u]);
    }
  }
  // 2. Xmax (and finiteness of x), eight BF16 per load (k is a multiple of 128)
  double xm = 0.0;
  {
    constexpr uint32_t kU = 4;
    const uint32_t nx = a.k / 8u;
    for (uint32_t base = 0; base < nx; base += kT * kU) {
      u32x4 xv[kU];
#pragma unroll
      for (uint32_t u = 0; u < kU; ++u)
        xv[u] = reinterpret_cast<const u32x4*>(xr)[min(base + u * kT + tid, nx - 1u)];
#pragma unroll
      for (uint32_t u = 0; u < kU; ++u) {
        if (base + u * kT + tid >= nx) continue;
#pragma unroll
        for (uint32_t h = 0; h < 8; ++h) {
          const uint32_t bits = (xv[u][h >> 1] >> (16u * (h & 1u))) & 0xFFFFu;
          if (((bits >> 7) & 0xFFu) == 0xFFu) bad = true;
          xm = fmax(xm, fabs((double)__uint_as_float(bits << 16)));
        }
      }
    }
  }
  // wave trees (fixed pattern; every lane ends with the wave's result), then the waves'
  // results in wave order
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float v2 = __shfl_xor(bv, off);
    const int32_t i2 = __shfl_xor(bi, off);
    if (v2 > bv || (v2 == bv && i2 < bi)) { bv = v2; bi = i2; }
    xm = fmax(xm, __shfl_xor(xm, off));
  }
  if (tid == 0) { s_cnt = 0; s_bad = 0; s_best_v = -1; }
  if (lane == 0) { s_bv[wave] = bv; s_bi[wave] = bi; s_d0[wave] = xm; }
  __syncthreads();
  if (bad) atomicOr(&s_bad, 1u);
  bv = s_bv[0];
  bi = s_bi[0];
  xm = s_d0[0];
  for (uint32_t w = 1; w < kT / 64u; ++w) {
    if (s_bv[w] > bv || (s_bv[w] == bv && s_bi[w] < bi)) { bv = s_bv[w]; bi = s_bi[w]; }
    xm = fmax(xm, s_d0[w]);
  }
  __syncthreads();   // s_bad complete; s_bv / s_bi / s_d0 free again
  const float zmax = bv;
  const double dd = (double)a.k + 64.0;
  const double gam = dd * ldexp(1.0, -23) / (1.0 - dd * ldexp(1.0, -23));
  const double wmax = ldexp(1.0, (int)a.e_max - 126);
  const double absb = dd * ldexp(1.0, -126) * (1.0 + xm + wmax);
  const double infl = 1.0 + ldexp(1.0, -20);
  // B(S^) = (g (S^/(1-g) + A) + A) * infl = c1 S^ + c0
  const double c1 = gam / (1.0 - gam) * infl, c0 = (gam * absb + absb) * infl;
  const uint32_t bstar = bi >= 0 && (uint32_t)bi < a.n ? (uint32_t)bi >> 4 : 0u;
  const double lo = (double)zmax - (c1 * (double)rs[bstar] + c0);
  const bool row_ok = !s_bad && __builtin_isfinite(zmax) && lo == lo;
  if (row_ok) {
    // 3. candidates: a block's largest logit, and all its rows when its second largest
    // also reaches L
#pragma unroll 8
    for (uint32_t b = tid; b < a.nb; b += kT) {
      const double bb = c1 * (double)(b < kCache ? s_rs[b] : rs[b]) + c0;
      if ((double)(b < kCache ? s_rv[b] : rv[b]) + bb < lo) continue;
      const int32_t i1 = ri[b];
      const float v2 = rv2[b];   // (both loads in flight together)
      put(atomicAdd(&s_cnt, 1u), i1);
      if ((double)v2 + bb >= lo)
        for (uint32_t rr = 0; rr < 16; ++rr)
          if ((int32_t)(16u * b + rr) != i1) put(atomicAdd(&s_cnt, 1u), (int32_t)(16u * b + rr));
    }
    __syncthreads();
    ncand = s_cnt;

    // 4. FP64 screen, up to kGroup candidates at a time (one or two when there are no
    // more, so each has more threads and its loads take fewer rounds), per threads each;
    // a candidate's escape offsets are requested with its tile loads.  Thread u of a
    // candidate v = 16b + r takes lane slots (g, q) = j / 4, j % 4 for j = u, u + per,
    // ...: slot l = 16q + r of tile (b, g) holds row r's columns 128g + 32jj + 8q + i
    // (jj < 4, i < 8), sign/mantissa bytes at 16l and 1024 + 16l, code nibbles in the
    // dwords at 2048 + 16l.  The threads also take the block's escape records of row r
    // (the product decoded with code 0 is replaced).  Partial sums meet in fixed
    // shuffle and LDS trees, so the screen is deterministic.  Summed in any order, the K
    // products and two terms per escape (K' terms) give an FP64 logit within g64 S64 of
    // the exact one, g64 = (K'+8) 2^-53 / (1 - (K'+8) 2^-53), S64 the sum of the terms'
    // magnitudes.
    const bool screen = ncand <= kScreenMax;
    if (screen) {
      const uint32_t grp = ncand <= 1u ? 1u : (ncand <= 2u ? 2u : kGroup);
      const uint32_t per = kT / grp, cc = tid / per, u = tid % per;
      for (uint32_t c0i = 0; c0i < ncand; c0i += grp) {
        const uint32_t c = c0i + cc;
        const bool active = c < ncand;
        double z = 0.0, sa = 0.0;
        uint32_t nesc = 0;
        if (active) {
          const uint32_t v = (uint32_t)s_cand[c], b = v >> 4, r = v & 15u;
          const uint32_t e0 = a.esc_off[b], e1 = a.esc_off[b + 1];
          for (uint32_t j = u; j < 4u * a.g_cols; j += per) {
            const uint32_t g = j >> 2, q = j & 3u, l = 16u * q + r;
            const uint8_t* tb = a.tiles + ((uint64_t)g * a.nb + b) * 3072u + 16u * l;
            const u32x4 s_lo = *reinterpret_cast<const u32x4*>(tb);
            const u32x4 s_hi = *reinterpret_cast<const u32x4*>(tb + 1024);
            const u32x4 cw = *reinterpret_cast<const u32x4*>(tb + 2048);
#pragma unroll
            for (uint32_t jj = 0; jj < 4; ++jj) {
              const u32x4 xv = *reinterpret_cast<const u32x4*>(xr + 128u * g + 32u * jj + 8u * q);
#pragma unroll
              for (uint32_t i = 0; i < 8; ++i) {
                const uint32_t t = 8u * jj + i;
                const uint32_t sword = t < 16u ? s_lo[(t & 15u) >> 2] : s_hi[(t & 15u) >> 2];
                const uint32_t sm = (sword >> (8u * (t & 3u))) & 0xFFu;
                const uint32_t code = (cw[jj] >> (4u * (i >> 1) + 16u * (i & 1u))) & 0xFu;
                const uint32_t e = (a.lut[code >> 2] >> (8u * (code & 3u))) & 0xFFu;
                const uint32_t wb = ((sm & 0x80u) << 8) | (e << 7) | (sm & 0x7Fu);
                const uint32_t xb = (xv[i >> 1] >> (16u * (i & 1u))) & 0xFFFFu;
                const double pr = (double)__uint_as_float(xb << 16) * (double)__uint_as_float(wb << 16);
                z += pr;
                sa += fabs(pr);
              }
            }
          }
          for (uint32_t i = e0 + u; i < e1; i += per) {
            const uint32_t rec = a.esc[i];
            const uint32_t kk = (rec >> 8) & 0xFFFFFu;
            if ((rec >> 28) != r || kk >= a.k) continue;   // another row, or malformed
            uint32_t code;
            const uint32_t wb = decode_w(a.tiles, a.nb, v, kk, a.lut, &code);
            const uint32_t wt = (wb & 0x807Fu) | ((rec & 0xFFu) << 7);
            const double xv = (double)__uint_as_float((uint32_t)xr[kk] << 16);
            const double pw = xv * (double)__uint_as_float(wb << 16);
            const double pt = xv * (double)__uint_as_float(wt << 16);
            z += pt - pw;
            sa += fabs(pt) + fabs(pw);
            ++nesc;
          }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          z += __shfl_xor(z, off);
          sa += __shfl_xor(sa, off);
          nesc += __shfl_xor(nesc, off);
        }
        if (lane == 0) { s_d0[wave] = z; s_d1[wave] = sa; s_u0[wave] = nesc; }
        __syncthreads();
        if (active && u == 0) {
          const uint32_t w0 = cc * (per / 64u);
          double zz = 0.0, ss = 0.0;
          uint32_t ne = 0;
          for (uint32_t w = 0; w < per / 64u; ++w) { zz += s_d0[w0 + w]; ss += s_d1[w0 + w]; ne += s_u0[w0 + w]; }
          const double kk2 = (double)a.k + 2.0 * (double)ne + 8.0;
          const double g64 = kk2 * ldexp(1.0, -53) / (1.0 - kk2 * ldexp(1.0, -53));
          s_z64[c] = zz;
          s_b64[c] = g64 * ss / (1.0 - g64) * infl;
        }
        __syncthreads();
      }
      // survivors: every candidate whose upper bound reaches the largest lower bound
      if (tid == 0) {
        double lo64 = -__builtin_inf();
        for (uint32_t c = 0; c < ncand; ++c) lo64 = fmax(lo64, s_z64[c] - s_b64[c]);
        uint32_t ns = 0;
        for (uint32_t c = 0; c < ncand; ++c)
          if (s_z64[c] + s_b64[c] >= lo64) s_cand[ns++] = s_cand[c];
        s_nsurv = ns;
      }
    } else if (tid == 0) {
      s_nsurv = ncand;   // too many to screen: every candidate goes exact
    }
    __syncthreads();
    nsurv = s_nsurv;
    if (nsurv == 1u) {
      result = get(0);
    } else {
      // 5. exact recompute of the survivors
      for (uint32_t c = 0; c < nsurv; ++c) {
        const uint32_t v = (uint32_t)get(c);
        if (tid < kLimbs) limbs[tid] = 0ull;
        __syncthreads();
        uint32_t code;
        for (uint32_t kk = tid; kk < a.k; kk += kT) {
          const uint32_t wb = decode_w(a.tiles, a.nb, v, kk, a.lut, &code);
          int sx_, sw_, ex_, ew_;
          uint32_t mx_, mw_;
          const bool okx = exact_parts(xr[kk], sx_, mx_, ex_);
          const bool okw = exact_parts(wb, sw_, mw_, ew_);
          if (!okx || !okw) atomicOr(&s_bad, 1u);
          limb_add(limbs, sx_ * sw_, mx_ * mw_, ex_ + ew_ + 266, false);
        }
        // escapes of this row: replace the product decoded with the stored code
        const uint32_t b = v >> 4, r = v & 15u;
        const uint32_t e0 = a.esc_off[b], e1 = a.esc_off[b + 1];
        for (uint32_t i = e0 + tid; i < e1; i += kT) {
          const uint32_t rec = a.esc[i];
          if ((rec >> 28) != r || ((rec >> 8) & 0xFFFFFu) >= a.k) continue;
          const uint32_t kk = (rec >> 8) & 0xFFFFFu;
          const uint32_t wb = decode_w(a.tiles, a.nb, v, kk, a.lut, &code);
          const uint32_t wt = (wb & 0x807Fu) | ((rec & 0xFFu) << 7);
          int sx_, sw_, ex_, ew_;
          uint32_t mx_, mw_;
          exact_parts(xr[kk], sx_, mx_, ex_);
          if (exact_parts(wb, sw_, mw_, ew_)) limb_add(limbs, sx_ * sw_, mx_ * mw_, ex_ + ew_ + 266, true);
          if (!exact_parts(wt, sw_, mw_, ew_)) atomicOr(&s_bad, 1u);
          limb_add(limbs, sx_ * sw_, mx_ * mw_, ex_ + ew_ + 266, false);
        }
        __syncthreads();
        if (tid == 0) {
          // normalise to 32-bit digits; the final carry is the sign (0 or -1)
          uint32_t dig[kLimbs];
          long long carry = 0;
          for (int i = 0; i < kLimbs; ++i) {
            const long long t = (long long)limbs[i] + carry;
            dig[i] = (uint32_t)(t & 0xFFFFFFFFll);
            carry = t >> 32;
          }
          bool better;
          if (s_best_v < 0) {
            better = true;
          } else if ((int32_t)carry != s_best_sign) {
            better = (int32_t)carry > s_best_sign;
          } else {
            int cmp = 0;
            for (int i = kLimbs - 1; i >= 0 && cmp == 0; --i)
              cmp = dig[i] > best[i] ? 1 : (dig[i] < best[i] ? -1 : 0);
            better = cmp > 0 || (cmp == 0 && (int32_t)v < s_best_v);
          }
          if (better) {
            for (int i = 0; i < kLimbs; ++i) best[i] = dig[i];
            s_best_sign = (int32_t)carry;
            s_best_v = (int32_t)v;
          }
        }
        __syncthreads();
      }
      result = s_bad ? -1 : s_best_v;
    }
  }
  __shared__ int32_t s_result;
  if (tid == 0) {
    a.argmax[row] = result;
    if (a.ncand) { a.ncand[2 * row] = (int32_t)ncand; a.ncand[2 * row + 1] = (int32_t)nsurv; }
    s_result = result;
  }
  __syncthreads();
  result = s_result;
  // accepted-prefix lengths: pass 1 set each to its draft length; the first mismatching
  // row of a request wins.  One request over all rows, or one thread per request entry.
  if (!a.req_off) {
    if (tid == 0 && row < a.n_draft && result != a.draft[row]) atomicMin(a.accepted, (int32_t)row);
  } else {
    for (uint32_t r = tid; r < a.n_req; r += kT) {
      int32_t lo, nd;
      if (req_entry(a.req_off, a.req_ndraft, r, a.m, lo, nd) && (int32_t)row >= lo &&
          (int32_t)row < lo + nd && result != a.draft[row])
        atomicMin(a.accepted + r, (int32_t)row - lo);
    }
  }
}

hipError_t launch_verify_pass2(const VerifyArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_verify_pass2, dim3(a.m), dim3(kT), 0, s, a);
  return hipGetLastError();
}

}  // namespace w12
