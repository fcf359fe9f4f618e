// Greedy verification epilogue: certified exact argmax over the LM-head logits and
// the accepted-prefix length.
//
// Pass 1 (the GEMM kernel family with the logits epilogue) leaves FP32 logits z^[m][v],
// S^[m][v] = the same kernel's FP32 sum of |x_k||w_vk|, and per 16-row block the
// largest z^ (with its index) and the largest S^.  Pass 2 (one workgroup per row):
//   1. z* = max z^ over the block maxima (lowest index on ties), S* its S^;
//   2. the error bound.  A product of two BF16 values is exact in FP32 unless it
//      underflows.  Whatever the summation order, each of the K products of a logit
//      passes through at most D = K + 64 additions (the slack covers the accumulators'
//      zero starts and the cross-wave sums), each with relative error below
//      eps = 2^-23 (round-to-nearest or toward zero), so with g = D eps / (1 - D eps)
//        |z^ - z| <= g S + A,   S = sum_k |x_k w_k|,
//      A = D 2^-126 (1 + Xmax + Wmax) covering flushed denormal inputs, products and
//      partial sums (Xmax = max |x_k|, Wmax = 2^(e_max-126) > |w|).  S^ sums the same
//      nonnegative terms, so S <= S^/(1-g) + A, and B(S^) = g (S^/(1-g) + A) + A,
//      inflated by 2^-20 for its FP64 evaluation, bounds |z^ - z|;
//   3. L = z* - B(S*) is below the true maximum, so every v with z^_v + B(S^_v) >= L is
//      a candidate (the exact argmax always is); whole blocks are skipped when their
//      largest z^ plus B(largest S^) falls below L;
//   4. each candidate's logit is recomputed exactly: sum_k x_k w_vk as an integer in
//      units of 2^-266 (a BF16 product is +-Mx*Mw*2^(Ex+Ew) with 8-bit significands),
//      accumulated in 64-bit LDS limbs; the largest exact value wins, lowest index on
//      an exact tie.
// The review page ("The mechanisms it found") names a certified exact-argmax LM head,
// and its caveats note that reduction order can flip near-ties: the exact logit makes
// the answer independent of the order.  Accept: first i < n_draft with
// argmax[i] != draft[i], else n_draft ("StargazerX0/SpecPilot", "Results and
// verification": every committed token is the target's own choice).
#include "w12_internal.h"

namespace w12 {

constexpr int kLimbs = 18;   // 18 x 32 bits > 542 bits (largest |sum| for K < 2^20)

__device__ __forceinline__ bool exact_parts(uint32_t bits, int& sgn, uint32_t& mant, int& ex) {
  const uint32_t e = (bits >> 7) & 0xFFu, m = bits & 0x7Fu;
  sgn = (bits >> 15) ? -1 : 1;
  mant = e ? (m | 0x80u) : m;
  ex = e ? (int)e - 134 : -133;
  return e != 0xFFu;
}

__device__ __forceinline__ uint32_t decode_w(const uint8_t* tiles, uint32_t g_cols, uint32_t v,
                                             uint32_t kk, const uint32_t lut[4],
                                             uint32_t* code_out) {
  const uint32_t b = v >> 4, r = v & 15u, g = kk >> 7, kap = kk & 127u;
  const uint32_t q = (kap >> 3) & 3u, j = kap >> 5, i = kap & 7u;
  const uint32_t l = 16u * q + r, t = 8u * j + i;
  const uint8_t* tb = tiles + ((uint64_t)b * g_cols + g) * 3072u;
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

__global__ __launch_bounds__(256) void k_verify_pass2(VerifyArgs a) {
  __shared__ float s_bv[256];
  __shared__ int32_t s_bi[256];
  __shared__ double s_xm[256];
  __shared__ unsigned long long limbs[kLimbs];
  __shared__ uint32_t best[kLimbs];
  __shared__ int32_t s_best_v, s_best_sign;
  __shared__ uint32_t s_cnt, s_bad;
  const uint32_t row = blockIdx.x, tid = threadIdx.x;
  const uint16_t* xr = a.x + (uint64_t)row * a.k;

  // 1. z* and its index over the block maxima (NaN marks a non-finite block)
  float bv = -__builtin_inff();
  int32_t bi = 0x7FFFFFFF;
  bool bad = false;
  for (uint32_t b = tid; b < a.nb; b += 256) {
    const float v = a.rbmax_v[(uint64_t)row * a.nb + b];
    const int32_t i = a.rbmax_i[(uint64_t)row * a.nb + b];
    if (v != v) bad = true;
    else if (v > bv || (v == bv && i < bi)) { bv = v; bi = i; }
  }
  // 2. Xmax (and finiteness of x)
  double xm = 0.0;
  for (uint32_t i = tid; i < a.k; i += 256) {
    const uint32_t bits = xr[i];
    if (((bits >> 7) & 0xFFu) == 0xFFu) bad = true;
    xm = fmax(xm, fabs((double)__uint_as_float(bits << 16)));
  }
  s_bv[tid] = bv;
  s_bi[tid] = bi;
  s_xm[tid] = xm;
  if (tid == 0) { s_cnt = 0; s_bad = 0; }
  __syncthreads();
  if (bad) atomicOr(&s_bad, 1u);
  for (uint32_t off = 128; off > 0; off >>= 1) {
    if (tid < off) {
      const float v2 = s_bv[tid + off];
      const int32_t i2 = s_bi[tid + off];
      if (v2 > s_bv[tid] || (v2 == s_bv[tid] && i2 < s_bi[tid])) { s_bv[tid] = v2; s_bi[tid] = i2; }
      s_xm[tid] = fmax(s_xm[tid], s_xm[tid + off]);
    }
    __syncthreads();
  }
  const float zmax = s_bv[0];
  const double dd = (double)a.k + 64.0;
  const double gam = dd * ldexp(1.0, -23) / (1.0 - dd * ldexp(1.0, -23));
  const double wmax = ldexp(1.0, (int)a.e_max - 126);
  const double absb = dd * ldexp(1.0, -126) * (1.0 + s_xm[0] + wmax);
  const double infl = 1.0 + ldexp(1.0, -20);
  auto bound = [&](float s_hat) -> double {
    return (gam * ((double)s_hat / (1.0 - gam) + absb) + absb) * infl;
  };
  const uint64_t vstar = s_bi[0] >= 0 && (uint32_t)s_bi[0] < a.n ? (uint32_t)s_bi[0] : 0u;
  const double lo = (double)zmax - bound(a.sabs[(uint64_t)row * a.n + vstar]);
  if (s_bad || !__builtin_isfinite(zmax) || lo != lo) {
    if (tid == 0) { a.argmax[row] = -1; if (a.ncand) a.ncand[row] = 0; }
    return;
  }
  // 3. candidates
  int32_t* cand = a.cand + (uint64_t)row * a.n;
  for (uint32_t b = tid; b < a.nb; b += 256) {
    const uint64_t bo = (uint64_t)row * a.nb + b;
    if ((double)a.rbmax_v[bo] + bound(a.rbmax_s[bo]) < lo) continue;
    for (uint32_t rr = 0; rr < 16; ++rr) {
      const uint64_t vo = (uint64_t)row * a.n + 16u * b + rr;
      if ((double)a.logits[vo] + bound(a.sabs[vo]) >= lo)
        cand[atomicAdd(&s_cnt, 1u)] = (int32_t)(16u * b + rr);
    }
  }
  __syncthreads();
  const uint32_t ncand = s_cnt;
  if (tid == 0) { s_best_v = -1; if (a.ncand) a.ncand[row] = (int32_t)ncand; }
  // 4. exact recompute of every candidate
  for (uint32_t c = 0; c < ncand; ++c) {
    const uint32_t v = (uint32_t)cand[c];
    if (tid < kLimbs) limbs[tid] = 0ull;
    __syncthreads();
    uint32_t code;
    for (uint32_t kk = tid; kk < a.k; kk += 256) {
      const uint32_t wb = decode_w(a.tiles, a.g_cols, v, kk, a.lut, &code);
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
    for (uint32_t i = e0 + tid; i < e1; i += 256) {
      const uint32_t rec = a.esc[i];
      if ((rec >> 28) != r) continue;
      const uint32_t kk = (rec >> 8) & 0xFFFFFu;
      const uint32_t wb = decode_w(a.tiles, a.g_cols, v, kk, a.lut, &code);
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
  if (tid == 0) a.argmax[row] = s_bad ? -1 : s_best_v;
}

__global__ void k_accept(const int32_t* argmax, const int32_t* draft, uint32_t n_draft,
                         int32_t* accepted) {
  if (threadIdx.x != 0) return;
  uint32_t i = 0;
  while (i < n_draft && argmax[i] == draft[i]) ++i;
  *accepted = (int32_t)i;
}

hipError_t launch_verify_pass2(const VerifyArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_verify_pass2, dim3(a.m), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_accept(const VerifyArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_accept, dim3(1), dim3(64), 0, s, a.argmax, a.draft, a.n_draft, a.accepted);
  return hipGetLastError();
}

}  // namespace w12
