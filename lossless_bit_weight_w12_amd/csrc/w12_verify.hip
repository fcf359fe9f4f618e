// Greedy verification epilogue: certified exact argmax over the LM-head logits and
// the accepted-prefix length.
//
// Pass 1 (the GEMM kernel family with the logits epilogue) leaves, per row and per
// 16-row block of the head, the largest FP32 logit z^ (with its index), the second
// largest, and W_b = the largest FP32 upper bound of ||w_v||_2 over the block's rows
// (the same kernel sums the squares of the weights it streams); and per workgroup of
// pass 1 (a group of consecutive row-blocks) the group's largest and second largest
// logit, the index of the largest, that block's W_b, and the group's largest W_b.  Pass 2
// (one workgroup per row):
//   1. z* = max z^ over the group records (lowest index on ties), W* the W_b of its
//      block; X >= ||x||_2 from the FP64 sum of the exact squares of x;
//   2. the error bound.  A product of two BF16 values is exact in FP32 unless it
//      underflows.  Each of the K products of a logit passes through at most
//      D = bound_depth(K) = K/128 + 192 additions (pass 1 sums every tile column from
//      zero and then adds it to the running sum, so the undocumented order inside an
//      MFMA costs at most 32 roundings per instruction of the column's chain of 4),
//      each with relative error below eps = 2^-23 (round-to-nearest or toward zero), so
//      with g = D eps / (1 - D eps)
//        |z^ - z| <= g S + A,   S = sum_k |x_k w_k| <= ||x||_2 ||w_v||_2 <= X W_v
//      (Cauchy-Schwarz), A = (2K + D) 2^-126 (1 + Xmax + Wmax) covering flushed denormal
//      inputs and products (K terms) and partial sums (at most K + D additions), each
//      losing less than 2^-126 (1 + Xmax + Wmax) (Xmax = max |x_k|,
//      Wmax = 2^(e_max-126) > |w|).
//      B(S') = c1 S' + c0 with c1 = bound_slope(K) >= g and c0 = (g A + A) 2^-20-inflated
//      is at least g S + A for any S' >= S, the inflation covering its FP64 evaluation;
//      S' = X W_b for a row of block b;
//   3. L = z* - B(X W*) is below the true maximum, so every v with z^_v + B(X W_v) >= L
//      is a candidate (the exact argmax always is).  A group whose largest logit plus
//      B(X times its largest W_b) is below L holds none; in the others, with W_b in B,
//      a block adds its largest logit when that reaches L, and all of its rows when its
//      second largest does too (otherwise no other row of it can).  The group holding z*
//      adds z* alone, without reading its block records, when its second largest logit
//      plus B(X times its largest W_b) is below L;
//   4. a single candidate is the argmax.  Otherwise the FP64 screen: each candidate's
//      logit is recomputed from the W12 tiles in FP64 (a
//      BF16 product is exact in FP64; escape corrections add two terms each), within
//      g64 S64 of the exact value; only the candidates whose FP64 upper bound reaches
//      the largest FP64 lower bound survive.  Candidates are screened in chunks, so
//      any number of them is screened (a first sweep finds the largest lower bound, a
//      second keeps the survivors); a survivor whose bound g64 S64 is zero has an exact
//      FP64 sum (every term is zero);
//   5. when more than one survives and not all of them are exact in FP64, each
//      survivor's logit is recomputed exactly: sum_k x_k w_vk as an integer in units of
//      2^-266 (a BF16 product is +-Mx*Mw*2^(Ex+Ew) with 8-bit significands), one wave
//      per survivor, each lane adding its products into its own column of 64-bit limbs
//      in LDS, the columns then summed and carried; the largest exact value wins,
//      lowest index on an exact tie.
// A row of x whose every entry is +-0 has every exact logit 0: its argmax is index 0.
// The review page ("The mechanisms it found") names a certified exact-argmax LM head,
// and its caveats note that reduction order can flip near-ties: the exact logit makes
// the answer independent of the order.  Accept: first i < n_draft with
// argmax[i] != draft[i], else n_draft ("StargazerX0/SpecPilot", "Results and
// verification": every committed token is the target's own choice): pass 1 sets it to
// n_draft and every row i < n_draft whose argmax differs from the draft lowers it to i
// with an atomic minimum.  Batched, each request applies the same rule to its own rows
// (its i counted from its first row), with its own accepted length.
#include "w12_exact.h"

namespace w12 {

constexpr uint32_t kT = 512;           // threads of the pass-2 workgroup (one workgroup per row)
constexpr uint32_t kWaves = kT / 64u;
static_assert(kWaves == kExactWaves, "the exact stage runs one wave per candidate");
constexpr uint32_t kScreenMax = 512;   // candidates screened per chunk (ids and results in LDS)
constexpr uint32_t kGCache = 6144;     // group records (largest logit, norm) kept in LDS for the scan
constexpr uint32_t kEscUnread = 0xFFFFFFFFu;   // a candidate's escape range not read yet

__global__ __launch_bounds__(kT) void k_verify_pass2(VerifyArgs a) {
  __shared__ float s_gvc[kGCache], s_gwc[kGCache];
  __shared__ int32_t s_cand[kScreenMax];   // the first candidates (the rest in global memory)
  __shared__ uint32_t s_ce0[kScreenMax], s_ce1[kScreenMax];   // their escape ranges
  __shared__ int32_t s_chunk[kScreenMax];  // ids of the chunk being screened
  __shared__ uint32_t s_ke0[kScreenMax], s_ke1[kScreenMax];   // the chunk's escape ranges
  __shared__ double s_z64[kScreenMax], s_b64[kScreenMax];
  __shared__ double s_d0[kWaves], s_d1[kWaves];
  __shared__ float s_wv[kWaves], s_ws[kWaves], s_w2[kWaves];
  __shared__ int32_t s_wi[kWaves];
  __shared__ uint32_t s_u0[kWaves];
  __shared__ ExactShared s_ex;
  __shared__ uint32_t s_cnt, s_bad, s_nsurv, s_allexact;
  __shared__ double s_lo64;
  __shared__ int32_t s_result;
  const uint32_t row = blockIdx.x, tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint16_t* xr = a.x + (uint64_t)row * a.k;
  const float* gv = a.grp_v + (uint64_t)row * a.ngrp;
  const float* gv2 = a.grp_v2 + (uint64_t)row * a.ngrp;
  const int32_t* gi = a.grp_i + (uint64_t)row * a.ngrp;
  const float* gs = a.grp_s + (uint64_t)row * a.ngrp;
  const float* gw = a.grp_w + (uint64_t)row * a.ngrp;
  const float* rv = a.rbmax_v + (uint64_t)row * a.nb;
  const float* rv2 = a.rbmax_v2 + (uint64_t)row * a.nb;
  const float* rs = a.rbmax_s + (uint64_t)row * a.nb;
  const int32_t* ri = a.rbmax_i + (uint64_t)row * a.nb;
  int32_t* cand = a.cand + (uint64_t)row * a.n;
  // candidate ids; the first kScreenMax also keep their row-block's escape range
  auto put = [&](uint32_t c, int32_t v, uint32_t e0, uint32_t e1) {
    if (c < kScreenMax) { s_cand[c] = v; s_ce0[c] = e0; s_ce1[c] = e1; } else cand[c] = v;
  };
  auto get = [&](uint32_t c) { return c < kScreenMax ? s_cand[c] : cand[c]; };
  uint32_t ncand = 0, nsurv = 0;
  if (tid == 0) { s_cnt = 0; s_bad = 0; s_result = -1; }

  // 1. z*, its index, W* and the second largest logit of its group over the group
  // records (NaN marks a group with a non-finite logit), which stay in LDS for the scan,
  // and Xmax, ||x||_2^2 and the finiteness of x.  Every scan issues all of a thread's
  // loads of a round before using any; the result does not depend on the order (largest
  // value, lowest index on ties).
  float bv = -__builtin_inff(), bs = 0.f, b2 = -__builtin_inff();
  int32_t bi = 0x7FFFFFFF;
  bool bad = false;
  double xm = 0.0;    // Xmax, eight BF16 per load (k is a multiple of 128)
  double ssx = 0.0;   // sum of x_k^2 (each square exact in FP64)
  {
    constexpr uint32_t kU = 10, kXU = 2;   // 5120 groups per round: 151936 rows in one at 2 row-blocks per group
    const uint32_t nx = a.k / 8u;
    const uint32_t rounds = max((a.ngrp + kT * kU - 1) / (kT * kU), (nx + kT * kXU - 1) / (kT * kXU));
    for (uint32_t rd = 0; rd < rounds; ++rd) {
      const uint32_t base = rd * kT * kU, xbase = rd * kT * kXU;
      // largest logit, second largest, its block's norm, the group's largest norm
      float v[kU], vs2[kU], s[kU], u[kU];
      int32_t iv[kU];
      u32x4 xv[kXU];
#pragma unroll
      for (uint32_t q = 0; q < kXU; ++q)
        xv[q] = reinterpret_cast<const u32x4*>(xr)[min(xbase + q * kT + tid, nx - 1u)];
#pragma unroll
      for (uint32_t q = 0; q < kU; ++q) {
        const uint32_t G = base + q * kT + tid;
        if (G < a.ngrp) {   // (uniform over a wave but the last: no duplicate loads)
          v[q] = gv[G];
          vs2[q] = gv2[G];
          iv[q] = gi[G];
          s[q] = gs[G];
          u[q] = gw[G];
        }
      }
#pragma unroll
      for (uint32_t q = 0; q < kU; ++q) {
        const uint32_t G = base + q * kT + tid;
        if (G >= a.ngrp) continue;
        if (G < kGCache) { s_gvc[G] = v[q]; s_gwc[G] = u[q]; }
        if (v[q] != v[q]) bad = true;
        else if (v[q] > bv || (v[q] == bv && iv[q] < bi)) { bv = v[q]; bi = iv[q]; bs = s[q]; b2 = vs2[q]; }
      }
#pragma unroll
      for (uint32_t q = 0; q < kXU; ++q) {
        if (xbase + q * kT + tid >= nx) continue;
#pragma unroll
        for (uint32_t h = 0; h < 8; ++h) {
          const uint32_t bits = (xv[q][h >> 1] >> (16u * (h & 1u))) & 0xFFFFu;
          if (((bits >> 7) & 0xFFu) == 0xFFu) bad = true;
          const double xv64 = (double)__uint_as_float(bits << 16);
          xm = fmax(xm, fabs(xv64));
          ssx += xv64 * xv64;
        }
      }
    }
  }
  // wave trees (fixed pattern; every lane ends with the wave's result), then the waves'
  // results in wave order
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const float v2 = __shfl_xor(bv, off), s2 = __shfl_xor(bs, off), t2 = __shfl_xor(b2, off);
    const int32_t i2 = __shfl_xor(bi, off);
    if (v2 > bv || (v2 == bv && i2 < bi)) { bv = v2; bi = i2; bs = s2; b2 = t2; }
    xm = fmax(xm, __shfl_xor(xm, off));
    ssx += __shfl_xor(ssx, off);
  }
  __syncthreads();   // s_cnt, s_bad initialised
  if (bad) atomicOr(&s_bad, 1u);
  if (lane == 0) {
    s_wv[wave] = bv;
    s_wi[wave] = bi;
    s_ws[wave] = bs;
    s_w2[wave] = b2;
    s_d0[wave] = xm;
    s_d1[wave] = ssx;
  }
  __syncthreads();
  bv = s_wv[0];
  bi = s_wi[0];
  bs = s_ws[0];
  b2 = s_w2[0];
  xm = s_d0[0];
  ssx = s_d1[0];
  for (uint32_t w = 1; w < kWaves; ++w) {
    if (s_wv[w] > bv || (s_wv[w] == bv && s_wi[w] < bi)) { bv = s_wv[w]; bi = s_wi[w]; bs = s_ws[w]; b2 = s_w2[w]; }
    xm = fmax(xm, s_d0[w]);
    ssx += s_d1[w];
  }
  const float zmax = bv;
  const double dd = bound_depth(a.k);
  const double gam = dd * ldexp(1.0, -23) / (1.0 - dd * ldexp(1.0, -23));
  const double wmax = ldexp(1.0, (int)a.e_max - 126);
  const double absb = (2.0 * (double)a.k + dd) * ldexp(1.0, -126) * (1.0 + xm + wmax);
  const double infl = 1.0 + ldexp(1.0, -20);
  const double c1 = bound_slope(a.k), c0 = (gam * absb + absb) * infl;
  const double xn = x_norm_up(ssx);   // >= ||x||_2: the scale of row v is xn * W_v
  const double lo = (double)zmax - (c1 * (xn * (double)bs) + c0);
  const bool row_ok = !s_bad && __builtin_isfinite(zmax) && lo == lo;
  const bool zero_row = row_ok && xm == 0.0;   // every product is +-0: every logit is 0
  if (row_ok && !zero_row) {
    // 2. candidates from the groups whose bound reaches L: a block's largest logit, and
    // all its rows when its second largest also reaches L
    const uint32_t gstar = ((uint32_t)bi >> 4) / a.bpg;   // the group holding z*
    for (uint32_t G = tid; G < a.ngrp; G += kT) {
      const float gzv = G < kGCache ? s_gvc[G] : gv[G];
      const float gwv = G < kGCache ? s_gwc[G] : gw[G];
      const double gbound = c1 * (xn * (double)gwv) + c0;
      if ((double)gzv + gbound < lo) continue;   // none of its rows reaches L
      if (G == gstar && (double)b2 + gbound < lo) {
        // every other row of z*'s group is at most its second largest logit and has at
        // most its largest norm: z* alone, without the block records (its escape range
        // is read later, only if the FP64 screen needs it)
        put(atomicAdd(&s_cnt, 1u), bi, kEscUnread, kEscUnread);
        continue;
      }
      const uint32_t b0 = G * a.bpg;
      float v[kMaxBpg], v2[kMaxBpg], sb[kMaxBpg];
      int32_t i1[kMaxBpg];
      uint32_t eo[kMaxBpg + 1];   // eo[q] = esc_off[b0 + q] (index clamped to nb)
#pragma unroll
      for (uint32_t q = 0; q < kMaxBpg; ++q) {   // every load of the group in flight at once
        const uint32_t b = min(b0 + min(q, a.bpg - 1u), a.nb - 1u);
        v[q] = rv[b];
        v2[q] = rv2[b];
        sb[q] = rs[b];
        i1[q] = ri[b];
      }
#pragma unroll
      for (uint32_t q = 0; q <= kMaxBpg; ++q) eo[q] = a.esc_off[min(b0 + q, a.nb)];
#pragma unroll
      for (uint32_t q = 0; q < kMaxBpg; ++q) {
        const uint32_t b = b0 + q;
        if (q >= a.bpg || b >= a.nb) continue;
        const uint32_t e1 = eo[q + 1];   // esc_off[b + 1]
        const double bb = c1 * (xn * (double)sb[q]) + c0;
        if ((double)v[q] + bb < lo) continue;
        put(atomicAdd(&s_cnt, 1u), i1[q], eo[q], e1);
        if ((double)v2[q] + bb >= lo)
          for (uint32_t rr = 0; rr < 16; ++rr)
            if ((int32_t)(16u * b + rr) != i1[q]) put(atomicAdd(&s_cnt, 1u), (int32_t)(16u * b + rr), eo[q], e1);
      }
    }
    __syncthreads();
    ncand = s_cnt;

    // 3. FP64 screen of the chunk's candidates [c0i, c0i + nc): up to 8 at a time (fewer
    // when there are fewer, so each has more threads and its loads take fewer rounds),
    // kT / grp threads each.  Thread u of a candidate v = 16b + r takes 8-weight units
    // U = u, u + per, ... of lane slots (g, q) = (U / 4) / 4, (U / 4) % 4: slot
    // l = 16q + r of tile (b, g) holds row r's columns 128g + 32jj + 8q + i (jj < 4,
    // i < 8), sign/mantissa bytes at 16l and 1024 + 16l, code nibbles in the dwords at
    // 2048 + 16l.  The threads also
    // take the block's escape records of row r (the product decoded with code 0 is
    // replaced).  Partial sums meet in fixed shuffle and LDS trees, so the screen is
    // deterministic.  Summed in any order, the K products and two terms per escape (K'
    // terms) give an FP64 logit within g64 S64 of the exact one, g64 = (K'+8) 2^-53 /
    // (1 - (K'+8) 2^-53), S64 the sum of the terms' magnitudes.
    auto screen = [&](uint32_t nc) {   // ids in s_chunk[0, nc) -> s_z64, s_b64
      const uint32_t grp = nc <= 1u ? 1u : (nc <= 2u ? 2u : (nc <= 4u ? 4u : 8u));
      const uint32_t per = kT / grp, cc = tid / per, u = tid % per;
      for (uint32_t c0i = 0; c0i < nc; c0i += grp) {
        const uint32_t c = c0i + cc;
        const bool active = c < nc;
        double z = 0.0, sa = 0.0;
        uint32_t nesc = 0;
        if (active) {
          const uint32_t v = (uint32_t)s_chunk[c], b = v >> 4, r = v & 15u;
          const uint32_t e0 = s_ke0[c], e1 = s_ke1[c];
          // the thread's first escape record, requested with its tiles
          const uint32_t rec0 = e0 + u < e1 ? a.esc[e0 + u] : 0u;
          // units of 8 weights: unit U = 4j + jj of slot j = (g, q) is group jj of row r's
          // columns 128g + 32jj + 8q .. +7: its sign/mantissa bytes are 8 consecutive bytes
          // of the slot's 16-byte row (t = 8jj + i: bytes 16l + (t & 15) + 1024 (t >= 16)),
          // its codes one dword at 2048 + 16l + 4jj, its x values one 16-byte load
          // kSB units per thread have their loads in flight together (the tiles come
          // from HBM: one round trip per unit made the screen latency-bound); a unit past
          // the end loads the last one again and is not used
          constexpr uint32_t kSB = 4;
          const uint32_t nU = 16u * a.g_cols;
          for (uint32_t U0 = u; U0 < nU; U0 += kSB * per) {
            uint2 smv[kSB];
            uint32_t cwj[kSB];
            u32x4 xv[kSB];
#pragma unroll
            for (uint32_t sb = 0; sb < kSB; ++sb) {
              const uint32_t U = min(U0 + sb * per, nU - 1u);
              const uint32_t j = U >> 2, jj = U & 3u, g = j >> 2, q = j & 3u, l = 16u * q + r;
              const uint8_t* tb = a.tiles + ((uint64_t)g * a.nb + b) * 3072u + 16u * l;
              smv[sb] = *reinterpret_cast<const uint2*>(tb + 1024u * (jj >> 1) + 8u * (jj & 1u));
              cwj[sb] = *reinterpret_cast<const uint32_t*>(tb + 2048u + 4u * jj);
              xv[sb] = *reinterpret_cast<const u32x4*>(xr + 128u * g + 32u * jj + 8u * q);
            }
#pragma unroll
            for (uint32_t sb = 0; sb < kSB; ++sb) {
              if (U0 + sb * per >= nU) break;
#pragma unroll
              for (uint32_t i = 0; i < 8; ++i) {
                const uint32_t sm = ((i < 4u ? smv[sb].x : smv[sb].y) >> (8u * (i & 3u))) & 0xFFu;
                const uint32_t code = (cwj[sb] >> (4u * (i >> 1) + 16u * (i & 1u))) & 0xFu;
                const uint32_t e = (a.lut[code >> 2] >> (8u * (code & 3u))) & 0xFFu;
                const uint32_t wb = ((sm & 0x80u) << 8) | (e << 7) | (sm & 0x7Fu);
                const uint32_t xb = (xv[sb][i >> 1] >> (16u * (i & 1u))) & 0xFFFFu;
                const double pr = (double)__uint_as_float(xb << 16) * (double)__uint_as_float(wb << 16);
                z += pr;
                sa += fabs(pr);
              }
            }
          }
          for (uint32_t i = e0 + u; i < e1; i += per) {
            const uint32_t rec = i == e0 + u ? rec0 : a.esc[i];
            const uint32_t kk = (rec >> 8) & 0xFFFFFu;
            if ((rec >> 28) != r || kk >= a.k) continue;   // another row, or malformed
            const uint32_t wb = decode_w(a.tiles, a.nb, v, kk, a.lut);
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
    };
    // first sweep: the largest FP64 lower bound; second sweep: the survivors, compacted
    // into the candidate list (a survivor's position never passes its own, so the
    // chunk's ids, copied to s_chunk first, are never overwritten before they are read).
    // A survivor whose bound is zero has S64 = 0: every term is zero and its logit is
    // exactly 0; when every survivor is such, the lowest index among them wins.
    // A single candidate is the argmax (the exact argmax is always a candidate).
    if (tid == 0) {
      s_lo64 = -__builtin_inf();
      s_nsurv = ncand == 1u ? 1u : 0u;
      s_allexact = 1;
      s_result = 0x7FFFFFFF;
    }
    const bool one_chunk = ncand <= kScreenMax;
    for (int sweep = ncand == 1u ? 2 : (one_chunk ? 1 : 0); sweep < 2; ++sweep) {
      for (uint32_t cb = 0; cb < ncand; cb += kScreenMax) {
        const uint32_t nc = min(ncand - cb, kScreenMax);
        __syncthreads();   // the previous chunk's ids and results are consumed
        for (uint32_t c = tid; c < nc; c += kT) {
          const uint32_t cc = cb + c;
          const int32_t v = get(cc);
          s_chunk[c] = v;
          const bool known = cc < kScreenMax && s_ce0[cc] != kEscUnread;
          s_ke0[c] = known ? s_ce0[cc] : a.esc_off[(uint32_t)v >> 4];
          s_ke1[c] = known ? s_ce1[cc] : a.esc_off[((uint32_t)v >> 4) + 1u];
        }
        __syncthreads();
        screen(nc);
        if (tid == 0) {
          if (sweep == 0 || one_chunk) {
            double l64 = s_lo64;
            for (uint32_t c = 0; c < nc; ++c) l64 = fmax(l64, s_z64[c] - s_b64[c]);
            s_lo64 = l64;
          }
          if (sweep == 1) {
            const double l64 = s_lo64;
            uint32_t ns = s_nsurv;
            for (uint32_t c = 0; c < nc; ++c) {
              if (s_z64[c] + s_b64[c] < l64) continue;
              put(ns++, s_chunk[c], s_ke0[c], s_ke1[c]);
              if (s_b64[c] != 0.0) s_allexact = 0;
              s_result = min(s_result, s_chunk[c]);   // the lowest survivor
            }
            s_nsurv = ns;
          }
        }
      }
    }
    __syncthreads();
    nsurv = s_nsurv;
    const bool need_exact = nsurv > 1u && !s_allexact;
    const int32_t lowest = s_result;
    __syncthreads();   // every thread has read s_result before it is rewritten
    if (!need_exact) {
      if (tid == 0) s_result = nsurv == 1u ? get(0) : lowest;
    } else {
      // 4. exact recompute of the survivors (w12_exact.h), one wave each
      const ExactRow er{xr, a.tiles, a.esc, a.nb, a.g_cols, a.k, a.lut};
      const int32_t rbest = exact_best(s_ex, er, nsurv, get, [&](uint32_t c, uint32_t& e0, uint32_t& e1) {
        const uint32_t b = (uint32_t)get(c) >> 4;
        const bool known = c < kScreenMax && s_ce0[c] != kEscUnread;
        e0 = known ? s_ce0[c] : a.esc_off[b];
        e1 = known ? s_ce1[c] : a.esc_off[b + 1];
      });
      if (tid == 0) s_result = rbest;
    }
  } else if (tid == 0) {
    s_result = zero_row ? 0 : -1;
  }
  __syncthreads();
  const int32_t result = s_result;
  if (tid == 0) {
    a.argmax[row] = result;
    if (a.ncand) { a.ncand[2 * row] = (int32_t)ncand; a.ncand[2 * row + 1] = (int32_t)nsurv; }
  }
  // accepted-prefix lengths: pass 1 set each to its draft length; the first mismatching
  // row of a request wins.  One request over all rows, or one thread per request entry.
  if (!a.req_off) {
    if (tid == 0 && row < a.n_draft && result != a.draft[row]) atomicMin(a.accepted, (int32_t)row);
  } else {
    for (uint32_t r = tid; r < a.n_req; r += kT) {
      int32_t lo_r, nd;
      if (req_entry(a.req_off, a.req_ndraft, r, a.m, lo_r, nd) && (int32_t)row >= lo_r &&
          (int32_t)row < lo_r + nd && result != a.draft[row])
        atomicMin(a.accepted + r, (int32_t)row - lo_r);
    }
  }
}

hipError_t launch_verify_pass2(const VerifyArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_verify_pass2, dim3(a.m), dim3(kT), 0, s, a);
  return hipGetLastError();
}

// The full first-pass output's error scales: row m of s holds the row norms W_v (the
// same for every row) and becomes X_m W_v rounded up to FP32, X_m the bound of ||x_m||_2
// that pass 2 uses (one workgroup per row; x finite, as verification requires).
__global__ __launch_bounds__(256) void k_scale_norms(const uint16_t* __restrict__ x, uint32_t k,
                                                     float* __restrict__ s, uint32_t n) {
  __shared__ double s_part[4];
  const uint32_t row = blockIdx.x, tid = threadIdx.x;
  const uint16_t* xr = x + (uint64_t)row * k;
  double ss = 0.0;
  for (uint32_t i = tid; i < k; i += 256u) {
    const double v = (double)__uint_as_float((uint32_t)xr[i] << 16);
    ss += v * v;
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if ((tid & 63u) == 0u) s_part[tid >> 6] = ss;
  __syncthreads();
  const double xn = x_norm_up((s_part[0] + s_part[1]) + (s_part[2] + s_part[3]));
  float* sr = s + (uint64_t)row * n;
  for (uint32_t v = tid; v < n; v += 256u) sr[v] = f32_round_up(xn * (double)sr[v] * (1.0 + 0x1p-50));
}

hipError_t launch_scale_norms(const uint16_t* x, uint32_t m, uint32_t k, float* s, uint32_t n,
                              hipStream_t st) {
  hipLaunchKernelGGL(k_scale_norms, dim3(m), dim3(256), 0, st, x, k, s, n);
  return hipGetLastError();
}

}  // namespace w12
