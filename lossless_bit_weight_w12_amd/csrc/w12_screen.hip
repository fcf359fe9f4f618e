// Two-level greedy verification over the LM head ("SpecPilot: an agent doubled
// speculative decoding speed, and the 10.87x needs context", section "The mechanisms it
// found": verification in two levels with an 8-bit copy of the head; "SpecPilot"
// glossary, "Differentiation").  The pages name the idea and the bit width; the copy's
// format and the certificate are defined here.
//
// Screen copy v1 (built by k_screen_encode): per row v and 32-column group g a scale
// s_vg = the smallest BF16 value >= max |w| / 127 over the group's finite weights (at
// least 2^-100) and codes q = rne(w / s) (int8, |q| <= 127, 0 for a non-finite w), in
// tiles of 16 rows x 128 columns (2176 bytes: the codes at the W12 sign/mantissa byte
// positions, then the tile's 64 scales); per row C_v >= ||r_v||_2 + gamma ||w^_v||_2
// (w^ = q s, r = w - w^, gamma = D 2^-23 / (1 - D 2^-23), D = K/32 + 64; +Inf for a row with a
// non-finite weight) and A_v = (K/32)(max_g s_vg 2^-113 + 2^-125), rounded up.
//
// Why the interval holds: z_v = sum_k x_k w_vk = z8_v + sum_k x_k r_vk with z8 = x . w^,
// and |sum_k x_k r_vk| <= ||x||_2 ||r_v||_2 (Cauchy-Schwarz).  The first pass computes
// z8^ = sum_g s_vg (sum_{k in g} x_k q_vk): each inner sum is one MFMA step on exact
// products (a BF16 x times an integer |q| <= 127 is exact in FP32; at most 31 additions),
// scaled and added to the running total with one FMA (at most K/32 more), so each term
// passes through at most D = K/32 + 64 additions with relative error below 2^-23 and
// |z8^ - z8| <= gamma S8 + A_v with S8 = sum_k |x_k||w^_vk| <= ||x||_2 ||w^_v||_2
// (A_v covers flushed denormal products, partial sums and scaled sums).  With X >= ||x||_2
// (from the staged x, rounded up), |z8^ - z_v| <= X C_v + A_v.  A non-finite z8^ (FP32
// overflow) gives the interval (-Inf, +Inf).
//
// Pass 1 (k_screen, one wave per 16-row block, 8 per workgroup, column-synchronous like
// the GEMM): per x row and block, the largest and second largest upper end hi of the
// block's intervals and the row of the largest; per workgroup ("group") the largest hi
// and the largest lower end lo.  Pass 2 (k_screen_select, 32 workgroups per x row): L =
// the largest lo of the row; a row v with hi_v < L is below some logit, so it is not the
// argmax; the others (a block's best row, all 16 when its second best also reaches L)
// are recomputed in FP64 from the W12 tiles, one wave each (within g64 S64 of the exact
// value, as in the single-level verification); the workgroup finishing last for a row
// keeps those whose FP64 interval reaches the largest FP64 lower bound, and when more
// than one is left and any is inexact, sums them exactly (w12_exact.h).  Lowest index on
// exact ties; the accepted length as in the single-level verification.
#include "w12_exact.h"
#include "w12_gemm_kernel.h"

namespace w12 {

// ------------------------------------------------------------------ rounding helpers
__device__ __forceinline__ float f32_round_down(double d) { return -f32_round_up(-d); }

// Upper bound of a + b for FP32 a, b (one FP64 addition, whose relative error is below
// 2^-53, widened by 2^-51 and rounded up).
__device__ __forceinline__ float add_up(float a, float b) {
  const double h = (double)a + (double)b;
  return f32_round_up(h + fabs(h) * 0x1p-51);
}
__device__ __forceinline__ float sub_down(float a, float b) {
  const double l = (double)a - (double)b;
  return f32_round_down(l - fabs(l) * 0x1p-51);
}

// Four int8 codes (one dword) -> four BF16 values (two dwords); exact (|q| <= 127).
__device__ __forceinline__ void i8x4_to_bf16(uint32_t w, uint32_t& lo, uint32_t& hi) {
  const uint32_t f0 = __float_as_uint((float)(int32_t)(int8_t)(w & 0xFFu));
  const uint32_t f1 = __float_as_uint((float)(int32_t)(int8_t)((w >> 8) & 0xFFu));
  const uint32_t f2 = __float_as_uint((float)(int32_t)(int8_t)((w >> 16) & 0xFFu));
  const uint32_t f3 = __float_as_uint((float)(int32_t)(int8_t)(w >> 24));
  lo = __builtin_amdgcn_perm(f1, f0, 0x07060302u);   // high halves: bf16(f0) | bf16(f1) << 16
  hi = __builtin_amdgcn_perm(f3, f2, 0x07060302u);
}

// ------------------------------------------------------------------ encode
// One workgroup of 256 threads per 16-row block, walking the block's tile columns.
// Thread t: row r = t / 16, 32-column group j = (t / 4) % 4 of the tile, columns
// 32j + 8u .. +7 with u = t % 4 (lane slot 16u + r, elements 8j .. 8j+7).  A group's four
// threads are consecutive lanes (shuffles xor 1, 2); a row's sixteen too (xor 1..8).
__global__ __launch_bounds__(256) void k_screen_encode(const uint16_t* w, uint32_t nb,
                                                       uint32_t g_cols, uint8_t* tiles,
                                                       float* coef, float* abse) {
  const uint32_t b = blockIdx.x, t = threadIdx.x;
  const uint32_t r = t >> 4, j = (t >> 2) & 3u, u = t & 3u;
  const uint32_t k = g_cols * 128u;
  const uint16_t* wr = w + (uint64_t)(16u * b + r) * k + 32u * j + 8u * u;
  double r2 = 0.0, q2 = 0.0, smax = 0.0;
  bool finite = true;
  for (uint32_t g = 0; g < g_cols; ++g) {
    const u32x4 v = *reinterpret_cast<const u32x4*>(wr + 128u * g);
    double wd[8];
    bool fin[8];
    double amax = 0.0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t bits = (v[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
      fin[i] = ((bits >> 7) & 0xFFu) != 0xFFu;
      wd[i] = fin[i] ? (double)__uint_as_float(bits << 16) : 0.0;
      amax = fmax(amax, fabs(wd[i]));
      finite = finite && fin[i];
    }
    amax = fmax(amax, __shfl_xor(amax, 1));
    amax = fmax(amax, __shfl_xor(amax, 2));
    // the smallest BF16 value >= max(amax / 127, 2^-100): the smallest FP32 value >= it,
    // then its low half rounded up (BF16 values are FP32 values)
    uint32_t sb = __float_as_uint(f32_round_up(fmax(amax / 127.0, 0x1p-100)));
    if (sb & 0xFFFFu) sb = (sb + 0x10000u) & 0xFFFF0000u;
    const double s = (double)__uint_as_float(sb);
    smax = fmax(smax, s);
    uint32_t c0 = 0, c1 = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // w / s is correctly rounded in FP64 and cannot reach a half-integer it does not
      // equal (8-bit significands), so rint gives the exact nearest-even code
      const double qd = fin[i] ? rint(wd[i] / s) : 0.0;
      const double wh = qd * s;            // exact: a 7-bit integer times a BF16 value
      const double rr = wd[i] - wh;        // exact: at most 8 significant bits
      r2 += rr * rr;
      q2 += wh * wh;
      const uint32_t byte = (uint32_t)(int32_t)qd & 0xFFu;
      if (i < 4) c0 |= byte << (8 * i);
      else c1 |= byte << (8 * (i - 4));
    }
    uint8_t* tb = tiles + ((uint64_t)g * nb + b) * kScreenTileBytes;
    const uint32_t l = 16u * u + r;
    *reinterpret_cast<uint2*>(tb + 1024u * (j >> 1) + 16u * l + 8u * (j & 1u)) = make_uint2(c0, c1);
    if (u == 0)
      *reinterpret_cast<uint16_t*>(tb + 2048u + 32u * (r >> 2) + 8u * (r & 3u) + 2u * j) = (uint16_t)(sb >> 16);
  }
  // the row's sums over its sixteen threads (a fixed tree: deterministic)
#pragma unroll
  for (int off = 1; off <= 8; off <<= 1) {
    r2 += __shfl_xor(r2, off);
    q2 += __shfl_xor(q2, off);
    smax = fmax(smax, __shfl_xor(smax, off));
    finite = __shfl_xor((int)finite, off) && finite;
  }
  if ((t & 15u) == 0) {
    // each square is exact (at most 16 significant bits); K terms summed in FP64 are
    // within K 2^-53 < 2^-33 of the exact sums, and sqrt, the product and the sum add a
    // few units of 2^-53: widened by 2^-30 and 2^-50, rounded up to FP32
    const double dd = (double)(k / 32u) + 64.0;   // D of the screen sum (see above)
    const double gam = dd * 0x1p-23 / (1.0 - dd * 0x1p-23);
    const double rn = sqrt(r2 * (1.0 + 0x1p-30)) * (1.0 + 0x1p-50);
    const double qn = sqrt(q2 * (1.0 + 0x1p-30)) * (1.0 + 0x1p-50);
    const double c = (rn + gam * qn) * (1.0 + 0x1p-50);
    const double ab = ((double)(k / 32u) * (smax * 0x1p-113 + 0x1p-125)) * (1.0 + 0x1p-50);
    coef[16u * b + r] = finite ? f32_round_up(c) : __builtin_inff();
    abse[16u * b + r] = f32_round_up(ab);
  }
}

hipError_t launch_screen_encode(const uint16_t* w, uint32_t nb, uint32_t g_cols, uint8_t* tiles,
                                float* coef, float* abse, hipStream_t s) {
  hipLaunchKernelGGL(k_screen_encode, dim3(nb), dim3(256), 0, s, w, nb, g_cols, tiles, coef, abse);
  return hipGetLastError();
}

// ------------------------------------------------------------------ pass 1
// MFMA layout as the GEMM: lane l holds D[4q+i][l%16 + 16h] (q = l / 16), i.e. rows
// 16b + 4q + i of the block for x row m = l%16 + 16h; its A operand of step j is slot l's
// elements 8j .. 8j+7.  Each step's products are summed from zero and added to the
// accumulator times the row's scale of that 32-column group.
template <int MT, bool FULL>
__global__ __launch_bounds__(kScreenNW * 64) void k_screen(ScreenArgs a) {
  constexpr int NW = kScreenNW, NH = MT / 16, NT = NW * 64;
  constexpr int kUnits = (16 * MT + NT - 1) / NT;     // 16-byte x units per thread
  constexpr int kXs = xs_stride(MT);
  __shared__ __align__(16) uint16_t xs[2][MT * kXs];
  __shared__ float s_ss[MT];
  __shared__ float s_gh[NW][MT], s_gl[NW][MT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, q = lane >> 4;
  const uint32_t b = blockIdx.x * NW + (uint32_t)wave;
  const bool bvalid = b < a.nb;
  const uint32_t bl = min(b, a.nb - 1u);
  const uint32_t m_rows = a.m, gb = a.g_cols;

  f32x4 acc[NH];
#pragma unroll
  for (int h = 0; h < NH; ++h) acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x4 tA[4], tB[4];
  u32x4 xr[kUnits];

  const __amdgpu_buffer_rsrc_t xrs = make_rsrc(a.x, m_rows * a.k * 2u);
  uint32_t xoff[kUnits];
#pragma unroll
  for (int i = 0; i < kUnits; ++i) {
    const uint32_t u = (uint32_t)tid + NT * i;
    const uint32_t uu = u < 16u * MT ? u : u % (16u * MT);
    const uint32_t m = uu >> 4, cu = uu & 15u;
    xoff[i] = (min(m, m_rows - 1u) * a.k + 8u * cu) * 2u;   // padding rows repeat the last
  }
  auto xload = [&](uint32_t g) {
    const uint32_t gl = min(g, gb - 1u);
#pragma unroll
    for (int i = 0; i < kUnits; ++i) xr[i] = __builtin_amdgcn_raw_buffer_load_b128(xrs, xoff[i], 256u * gl, 0);
  };
  auto tload = [&](u32x4 (&t)[4], uint32_t g) {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(a.tiles + ((size_t)g * a.nb + bl) * kScreenTileBytes, kScreenTileBytes);
    t[0] = __builtin_amdgcn_raw_buffer_load_b128(rs, (uint32_t)lane * 16u, 0, kCpolNT);
    t[1] = __builtin_amdgcn_raw_buffer_load_b128(rs, 1024u + (uint32_t)lane * 16u, 0, kCpolNT);
    t[2] = __builtin_amdgcn_raw_buffer_load_b128(rs, 2048u + 32u * (uint32_t)q, 0, kCpolNT);
    t[3] = __builtin_amdgcn_raw_buffer_load_b128(rs, 2064u + 32u * (uint32_t)q, 0, kCpolNT);
  };
  float ssq[kUnits];
#pragma unroll
  for (int i = 0; i < kUnits; ++i) ssq[i] = 0.f;
  auto xsumsq = [&](bool in_range) {
    if (in_range) {
#pragma unroll
      for (int i = 0; i < kUnits; ++i) ssq[i] += unit_sumsq(xr[i]);
    }
  };
  auto xstore = [&](uint32_t slot) {
#pragma unroll
    for (int i = 0; i < kUnits; ++i) {
      const uint32_t u = (uint32_t)tid + NT * i;
      if (kUnits * NT == 16 * MT || u < 16u * MT) {
        const uint32_t m = u >> 4, cu = u & 15u;
        *reinterpret_cast<u32x4*>(&xs[slot][m * kXs + 8u * cu]) = xr[i];
      }
    }
  };
  auto compute = [&](const u32x4 (&t)[4], uint32_t slot) {
    // scale of row 4q+i, group j: bytes 8i + 2j of the lane's 32 scale bytes
    float sc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d = 2 * i + (j >> 1);
        const uint32_t dw = t[2 + (d >> 2)][d & 3];
        sc[i][j] = __uint_as_float((j & 1) ? (dw & 0xFFFF0000u) : (dw << 16));
      }
    const uint16_t* xrow = &xs[slot][8 * q];
    // up to 32 columns the column's x fragments are read from LDS before the codes are
    // converted, so their latency hides under the conversion (two levels at M = 32:
    // 222 -> 208 us; 16 columns within 1 %); at 64 and 128 columns the registers are
    // not there
    constexpr bool kEarly = MT <= 32;
    u32x4 xvs[4][NH];
    if constexpr (kEarly) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int h = 0; h < NH; ++h)
          xvs[j][h] = *reinterpret_cast<const u32x4*>(xrow + (16 * h + r) * kXs + 32 * j);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const u32x4 cw = t[j >> 1];
      uint32_t a0, a1, a2, a3;
      i8x4_to_bf16(cw[2 * (j & 1)], a0, a1);
      i8x4_to_bf16(cw[2 * (j & 1) + 1], a2, a3);
      const u32x4 av = {a0, a1, a2, a3};
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const u32x4 xv =
            kEarly ? xvs[j][h] : *reinterpret_cast<const u32x4*>(xrow + (16 * h + r) * kXs + 32 * j);
        const f32x4 part = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8_t, av), __builtin_bit_cast(bf16x8_t, xv),
            f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[h][i] = fmaf(sc[i][j], part[i], acc[h][i]);
      }
    }
  };

  uint32_t g = 0;
  xload(g);
  tload(tA, g);
  xsumsq(true);
  xstore(0);
  __syncthreads();
  // every iteration issues the same loads (the next column, clamped past the end): fixed
  // wait counts.  (Peeling the last column, as the GEMM does, raised this kernel's
  // registers from 68 to 104 and slowed it by about 10 %.)
  for (;;) {
    xload(g + 1);
    tload(tB, min(g + 1, gb - 1u));
    compute(tA, g & 1u);
    xsumsq(g + 1 < gb);
    xstore((g + 1) & 1u);
    __syncthreads();
    if (++g >= gb) break;
    xload(g + 1);
    tload(tA, min(g + 1, gb - 1u));
    compute(tB, g & 1u);
    xsumsq(g + 1 < gb);
    xstore((g + 1) & 1u);
    __syncthreads();
    if (++g >= gb) break;
  }

  // ||x_m||^2 per x row: the 16 threads of a row's units meet in a fixed shuffle tree
#pragma unroll
  for (int i = 0; i < kUnits; ++i) {
    float v = ssq[i];
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) v += __shfl_xor(v, off);
    const uint32_t u = (uint32_t)tid + NT * i;
    if ((kUnits * NT == 16 * MT || u < 16u * MT) && (u & 15u) == 0u) s_ss[u >> 4] = v;
  }
  if (a.acc.accepted && blockIdx.x == 0) accept_init(a.acc, m_rows, (uint32_t)tid, NT);
  __syncthreads();

  const uint32_t v0 = 16u * bl + 4u * (uint32_t)q;
  const f32x4 cc = *reinterpret_cast<const f32x4*>(a.coef + v0);
  const f32x4 aa = *reinterpret_cast<const f32x4*>(a.abse + v0);
#pragma unroll
  for (int h = 0; h < NH; ++h) {
    const uint32_t m = 16u * h + (uint32_t)r;
    const float X = l2_norm_up(s_ss[m], a.k);   // >= ||x||_2
    float hi[4], lo[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      bf[i] = f32_round_up(((double)X * (double)cc[i] + (double)aa[i]) * (1.0 + 0x1p-50));
      if (__builtin_isfinite(acc[h][i])) {
        hi[i] = add_up(acc[h][i], bf[i]);
        lo[i] = sub_down(acc[h][i], bf[i]);
      } else {
        hi[i] = __builtin_inff();
        lo[i] = -__builtin_inff();
      }
    }
    // largest hi (lowest row on ties), second largest, largest lo over the block's rows:
    // this lane's four, then the lanes holding the other rows of column m
    float best = hi[0], second = -__builtin_inff(), lmax = lo[0];
    int bi = 0;
#pragma unroll
    for (int i = 1; i < 4; ++i) {
      if (hi[i] > best) { second = best; best = hi[i]; bi = i; }
      else if (hi[i] > second) second = hi[i];
      lmax = fmaxf(lmax, lo[i]);
    }
    int row = 4 * q + bi;
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float ob = __shfl_xor(best, off);
      const float o2 = __shfl_xor(second, off);
      const int orow = __shfl_xor(row, off);
      lmax = fmaxf(lmax, __shfl_xor(lmax, off));
      if (ob > best || (ob == best && orow < row)) {
        second = fmaxf(o2, best);
        best = ob;
        row = orow;
      } else {
        second = fmaxf(second, ob);
      }
    }
    const bool live = bvalid && m < m_rows;
    if (live) {
      if constexpr (FULL) {
        *reinterpret_cast<f32x4*>(a.full_z + (size_t)m * a.n + v0) = acc[h];
        *reinterpret_cast<f32x4*>(a.full_b + (size_t)m * a.n + v0) = f32x4{bf[0], bf[1], bf[2], bf[3]};
      }
      if (q == 0) {
        a.hi1[(size_t)m * a.nb + b] = best;
        a.hi2[(size_t)m * a.nb + b] = second;
        a.idx[(size_t)m * a.nb + b] = (int32_t)(16u * b + row);
      }
    }
    if (q == 0) {
      s_gh[wave][m] = live ? best : -__builtin_inff();
      s_gl[wave][m] = live ? lmax : -__builtin_inff();
    }
  }
  __syncthreads();
  if (tid < MT && (uint32_t)tid < m_rows) {
    float gh = s_gh[0][tid], gl = s_gl[0][tid];
#pragma unroll
    for (int w = 1; w < NW; ++w) { gh = fmaxf(gh, s_gh[w][tid]); gl = fmaxf(gl, s_gl[w][tid]); }
    a.gh[(size_t)tid * a.ngrp + blockIdx.x] = gh;
    a.gl[(size_t)tid * a.ngrp + blockIdx.x] = gl;
  }
}

hipError_t launch_screen_pass1(const ScreenArgs& a, hipStream_t s) {
  const dim3 grid(a.ngrp), block(kScreenNW * 64);
  const bool full = a.full_z != nullptr;
#define W12_SCREEN(MT_)                                                             \
  do {                                                                              \
    if (full) hipLaunchKernelGGL((k_screen<MT_, true>), grid, block, 0, s, a);      \
    else hipLaunchKernelGGL((k_screen<MT_, false>), grid, block, 0, s, a);          \
  } while (0)
  if (a.m <= 16) W12_SCREEN(16);
  else if (a.m <= 32) W12_SCREEN(32);
  else if (a.m <= 64) W12_SCREEN(64);
  else W12_SCREEN(128);
#undef W12_SCREEN
  return hipGetLastError();
}

// ------------------------------------------------------------------ pass 2
constexpr uint32_t kSelT = 512;
constexpr uint32_t kSelW = kSelT / 64u;
constexpr uint32_t kSelMaxSlices = 32;
constexpr uint32_t kUnitChunk = 8;    // 8-weight units per thread with loads in flight together
constexpr uint32_t kSelCandLds = 512; // candidate ids of a slice kept in LDS (the rest re-read)
static_assert(kSelW == kExactWaves, "the exact stage runs one wave per candidate");

// Device-scope (agent) stores and loads: the data one workgroup leaves for the workgroup
// that completes the row, which may run on another XCD.
template <class T>
__device__ __forceinline__ void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T ld_agent(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// FP64 logits of candidates [0, nc) of this workgroup (ids from get(c)) from the W12 tiles:
// up to 8 candidates at a time, kSelT / G threads each (G = candidates of the round, a
// power of two), so that a thread's share of a row (8-weight units U = u, u + per, ... of
// row r's lane slots (g, q) = (U / 4) / 4, (U / 4) % 4, group jj = U % 4) is at most a
// chunk or two, its loads issued together.  Each product is exact in FP64; summed in any
// order, the K products and two terms per escape (K' terms) are within g64 S64 of the exact
// logit, g64 = (K'+8) 2^-53 / (1 - (K'+8) 2^-53), S64 the sum of the terms' magnitudes.
// Partial sums meet in fixed shuffle and LDS trees.  put(c, z, b64) runs in one thread per
// candidate.
template <class Get, class Put>
__device__ void fp64_logits_wg(const ExactRow& c, const uint32_t* esc_off, uint32_t nc, Get get,
                               Put put, double* s_d0, double* s_d1, uint32_t* s_u0) {
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  const uint32_t nunits = 16u * c.g_cols;
  for (uint32_t c0 = 0; c0 < nc; c0 += 8u) {
    const uint32_t left = nc - c0;
    const uint32_t G = left >= 8u ? 8u : (left > 4u ? 8u : (left > 2u ? 4u : left));
    const uint32_t per = kSelT / G, cc = tid / per, u = tid % per;
    const bool active = cc < left;
    double z = 0.0, sa = 0.0;
    uint32_t nesc = 0;
    if (active) {
      const uint32_t v = (uint32_t)get(c0 + cc), b = v >> 4, r = v & 15u;
      const uint32_t e0 = esc_off[b], e1 = esc_off[b + 1];
      for (uint32_t U0 = u; U0 < nunits; U0 += kUnitChunk * per) {
        uint2 smv[kUnitChunk];
        uint32_t cwv[kUnitChunk];
        u32x4 xv[kUnitChunk];
#pragma unroll
        for (uint32_t i = 0; i < kUnitChunk; ++i) {
          const uint32_t U = min(U0 + i * per, nunits - 1u);   // clamped: loaded, not added
          const uint32_t j = U >> 2, jj = U & 3u, g = j >> 2, q = j & 3u, l = 16u * q + r;
          const uint8_t* tb = c.tiles + ((uint64_t)g * c.nb + b) * 3072u + 16u * l;
          smv[i] = *reinterpret_cast<const uint2*>(tb + 1024u * (jj >> 1) + 8u * (jj & 1u));
          cwv[i] = *reinterpret_cast<const uint32_t*>(tb + 2048u + 4u * jj);
          xv[i] = *reinterpret_cast<const u32x4*>(c.xr + 128u * g + 32u * jj + 8u * q);
        }
#pragma unroll
        for (uint32_t i = 0; i < kUnitChunk; ++i) {
          if (U0 + i * per >= nunits) continue;
#pragma unroll
          for (uint32_t e = 0; e < 8; ++e) {
            const uint32_t sm = ((e < 4u ? smv[i].x : smv[i].y) >> (8u * (e & 3u))) & 0xFFu;
            const uint32_t code = (cwv[i] >> (4u * (e >> 1) + 16u * (e & 1u))) & 0xFu;
            const uint32_t ex = (c.lut[code >> 2] >> (8u * (code & 3u))) & 0xFFu;
            const uint32_t wb = ((sm & 0x80u) << 8) | (ex << 7) | (sm & 0x7Fu);
            const uint32_t xb = (xv[i][e >> 1] >> (16u * (e & 1u))) & 0xFFFFu;
            const double pr = (double)__uint_as_float(xb << 16) * (double)__uint_as_float(wb << 16);
            z += pr;
            sa += fabs(pr);
          }
        }
      }
      for (uint32_t i = e0 + u; i < e1; i += per) {
        const uint32_t rec = c.esc[i];
        const uint32_t kk = (rec >> 8) & 0xFFFFFu;
        if ((rec >> 28) != r || kk >= c.k) continue;   // another row, or malformed
        const uint32_t wb = decode_w(c.tiles, c.nb, v, kk, c.lut);
        const uint32_t wt = (wb & 0x807Fu) | ((rec & 0xFFu) << 7);
        const double xd = (double)__uint_as_float((uint32_t)c.xr[kk] << 16);
        const double pw = xd * (double)__uint_as_float(wb << 16);
        const double pt = xd * (double)__uint_as_float(wt << 16);
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
      const double kk2 = (double)c.k + 2.0 * (double)ne + 8.0;
      const double g64 = kk2 * 0x1p-53 / (1.0 - kk2 * 0x1p-53);
      put(c0 + cc, zz, g64 * ss / (1.0 - g64) * (1.0 + 0x1p-20));
    }
    __syncthreads();   // s_d0.. are rewritten by the next round
  }
}

__global__ __launch_bounds__(kSelT) void k_screen_select(SelectArgs a) {
  __shared__ ExactShared s_ex;
  __shared__ int32_t s_cand[kSelCandLds];   // this slice's first candidates (all in sc_v too)
  __shared__ float s_lf[kSelW];
  __shared__ double s_d0[kSelW], s_d1[kSelW];
  __shared__ uint32_t s_u0[kSelW];
  __shared__ double s_lo64[8];
  __shared__ int32_t s_scnt[kSelMaxSlices], s_soff[kSelMaxSlices + 1];
  __shared__ double s_slo[kSelMaxSlices];
  __shared__ uint32_t s_flag, s_cnt, s_last, s_nsurv, s_allexact;
  __shared__ int32_t s_low;
  const uint32_t slice = blockIdx.x, row = blockIdx.y, tid = threadIdx.x;
  const uint32_t lane = tid & 63u, wave = tid >> 6;
  const uint32_t S = gridDim.x;
  const uint16_t* xr = a.x + (uint64_t)row * a.k;
  const size_t sbase = ((size_t)row * S + slice) * a.cap;
  if (tid == 0) { s_flag = 0; s_cnt = 0; }
  if (tid < 8) s_lo64[tid] = -__builtin_inf();
  __syncthreads();

  // 1. the x row: nonzero (bit 0) and non-finite (bit 1) entries; L = the row's largest
  // lower end over the group records (all loads of a thread issued before any use)
  uint32_t fl = 0;
  float lm = -__builtin_inff();
  {
    constexpr uint32_t kXU = 2, kGU = 4;
    const uint32_t nx = a.k / 8u;
    // round r covers x units [r * kXU * kSelT, +kXU * kSelT) and groups [r * kGU * kSelT, +kGU * kSelT)
    static_assert(kGU == 2 * kXU, "one round covers half as many x units as groups");
    for (uint32_t base = 0; base < max(2u * nx, a.ngrp); base += kSelT * kGU) {
      u32x4 xv[kXU];
      float gv[kGU];
#pragma unroll
      for (uint32_t i = 0; i < kXU; ++i) xv[i] = reinterpret_cast<const u32x4*>(xr)[min(base / 2u + i * kSelT + tid, nx - 1u)];
#pragma unroll
      for (uint32_t i = 0; i < kGU; ++i) gv[i] = a.gl[(size_t)row * a.ngrp + min(base + i * kSelT + tid, a.ngrp - 1u)];
#pragma unroll
      for (uint32_t i = 0; i < kXU; ++i) {
        if (base / 2u + i * kSelT + tid >= nx) continue;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t bits = (xv[i][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
          if (bits & 0x7FFFu) fl |= 1u;
          if (((bits >> 7) & 0xFFu) == 0xFFu) fl |= 2u;
        }
      }
#pragma unroll
      for (uint32_t i = 0; i < kGU; ++i) lm = fmaxf(lm, gv[i]);   // clamped repeats are harmless
    }
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) lm = fmaxf(lm, __shfl_xor(lm, off));
  if (fl) atomicOr(&s_flag, fl);
  if (lane == 0) s_lf[wave] = lm;
  __syncthreads();
  float L = s_lf[0];
  for (uint32_t w = 1; w < kSelW; ++w) L = fmaxf(L, s_lf[w]);
  const uint32_t flags = s_flag;
  const bool work = (flags & 1u) && !(flags & 2u);   // nonzero and finite

  if (work) {
    // 2. candidates of this slice's groups (slice, slice + S, ...): a row v whose upper
    // end hi_v is below L is not the argmax; a block holds such rows only, its best row,
    // or (second best reaching L) possibly any row
    auto put = [&](int32_t v) {
      const uint32_t c = atomicAdd(&s_cnt, 1u);
      if (c < kSelCandLds) s_cand[c] = v;
      st_agent(a.sc_v + sbase + c, v);
    };
    for (uint32_t t0 = 0; slice + S * t0 < a.ngrp; t0 += kSelT) {
      const uint32_t G = slice + S * (t0 + tid);
      if (G < a.ngrp) {
        // the group's upper end and its blocks' records, all requested at once
        const float gh = a.gh[(size_t)row * a.ngrp + G];
        const uint32_t b0 = G * a.bpg;
        float h1[kMaxBpg], h2[kMaxBpg];
        int32_t i1[kMaxBpg];
#pragma unroll
        for (uint32_t qb = 0; qb < kMaxBpg; ++qb) {
          const size_t o = (size_t)row * a.nb + min(b0 + min(qb, a.bpg - 1u), a.nb - 1u);
          h1[qb] = a.hi1[o];
          h2[qb] = a.hi2[o];
          i1[qb] = a.idx[o];
        }
        if (gh >= L) {
#pragma unroll
          for (uint32_t qb = 0; qb < kMaxBpg; ++qb) {
            const uint32_t b = b0 + qb;
            if (qb >= a.bpg || b >= a.nb || !(h1[qb] >= L)) continue;
            put(i1[qb]);
            if (h2[qb] >= L)
              for (uint32_t rr = 0; rr < 16; ++rr)
                if ((int32_t)(16u * b + rr) != i1[qb]) put((int32_t)(16u * b + rr));
          }
        }
      }
    }
    __syncthreads();
    const uint32_t nc = s_cnt;
    // 3. their FP64 logits, the whole workgroup on up to 8 at a time
    const ExactRow er{xr, a.tiles, a.esc, a.nb, a.g_cols, a.k, a.lut};
    fp64_logits_wg(er, a.esc_off, nc,
                   [&](uint32_t c) { return c < kSelCandLds ? s_cand[c] : ld_agent(a.sc_v + sbase + c); },
                   [&](uint32_t c, double z, double b64) {
                     st_agent(a.sc_z + sbase + c, z);
                     st_agent(a.sc_b + sbase + c, b64);
                     const double lo = (__builtin_isfinite(z) && __builtin_isfinite(b64)) ? z - b64 : __builtin_nan("");
                     double& slot = s_lo64[c & 7u];   // one writer per slot and round
                     slot = (slot != slot || lo != lo) ? __builtin_nan("") : fmax(slot, lo);
                   },
                   s_d0, s_d1, s_u0);
    if (tid == 0) {
      double lo = s_lo64[0];
      for (uint32_t w = 1; w < 8; ++w) lo = (lo != lo || s_lo64[w] != s_lo64[w]) ? __builtin_nan("") : fmax(lo, s_lo64[w]);
      st_agent(a.sc_cnt + (size_t)row * S + slice, (int32_t)nc);
      st_agent(a.sc_lo + (size_t)row * S + slice, lo);
    }
  }

  // 4. the row's ticket: the workgroup that takes the last one completes the row
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (tid == 0) {
    const uint32_t old = __hip_atomic_fetch_add(a.tickets + row, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old + 1u == S;
    if (last) __hip_atomic_store(a.tickets + row, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last ? 1u : 0u;
  }
  __syncthreads();
  if (!s_last) return;

  int32_t result;
  uint32_t ntot = 0, nsurv = 0;
  if (!work) {
    result = (flags & 2u) ? -1 : 0;   // non-finite x: -1; all +-0: every logit is 0
  } else {
    // 5. the slices' counts and largest FP64 lower bounds (one thread each), then the
    // survivors: candidates whose FP64 interval reaches the largest lower bound
    if (tid < S) {
      const int32_t cnt = ld_agent(a.sc_cnt + (size_t)row * S + tid);
      s_scnt[tid] = max(cnt, 0);
      s_slo[tid] = cnt > 0 ? ld_agent(a.sc_lo + (size_t)row * S + tid) : -__builtin_inf();
    }
    if (tid == 0) { s_nsurv = 0; s_allexact = 1; s_low = 0x7FFFFFFF; }
    __syncthreads();
    double L64 = -__builtin_inf();
    bool bad = false;
    for (uint32_t s = 0; s < S; ++s) {
      if (s_slo[s] != s_slo[s]) bad = true;
      else L64 = fmax(L64, s_slo[s]);
      ntot += (uint32_t)s_scnt[s];
    }
    if (tid == 0) {
      int32_t acc = 0;
      for (uint32_t s = 0; s < S; ++s) { s_soff[s] = acc; acc += s_scnt[s]; }
      s_soff[S] = acc;
    }
    __syncthreads();
    if (!bad) {
      int32_t* surv = a.surv + (size_t)row * a.n;
      for (uint32_t i = tid; i < ntot; i += kSelT) {
        uint32_t s = 0;
        while ((uint32_t)s_soff[s + 1] <= i) ++s;
        const size_t e = ((size_t)row * S + s) * a.cap + (i - (uint32_t)s_soff[s]);
        const double z = ld_agent(a.sc_z + e), bb = ld_agent(a.sc_b + e);
        const int32_t v = ld_agent(a.sc_v + e);
        if (z + bb < L64) continue;
        surv[atomicAdd(&s_nsurv, 1u)] = v;
        if (bb != 0.0) s_allexact = 0;
        atomicMin(&s_low, v);
      }
    }
    __syncthreads();
    nsurv = s_nsurv;
    if (bad || nsurv == 0) {
      result = -1;
    } else if (nsurv == 1 || s_allexact) {
      result = s_low;   // one survivor, or survivors whose FP64 sums are exact and equal
    } else {
      const int32_t* surv = a.surv + (size_t)row * a.n;
      const ExactRow er{xr, a.tiles, a.esc, a.nb, a.g_cols, a.k, a.lut};
      result = exact_best(s_ex, er, nsurv, [&](uint32_t c) { return surv[c]; },
                          [&](uint32_t c, uint32_t& e0, uint32_t& e1) {
                            const uint32_t b = (uint32_t)surv[c] >> 4;
                            e0 = a.esc_off[b];
                            e1 = a.esc_off[b + 1];
                          });
    }
  }
  if (tid == 0) {
    a.argmax[row] = result;
    if (a.ncand) { a.ncand[2 * row] = (int32_t)ntot; a.ncand[2 * row + 1] = (int32_t)nsurv; }
  }
  // accepted-prefix lengths: pass 1 set each to its draft length; the first mismatching
  // row of a request lowers it.  One request over all rows, or one thread per request.
  if (!a.req_off) {
    if (tid == 0 && row < a.n_draft && result != a.draft[row]) atomicMin(a.accepted, (int32_t)row);
  } else {
    for (uint32_t rq = tid; rq < a.n_req; rq += kSelT) {
      int32_t lo_r, nd;
      if (req_entry(a.req_off, a.req_ndraft, rq, a.m, lo_r, nd) && (int32_t)row >= lo_r &&
          (int32_t)row < lo_r + nd && result != a.draft[row])
        atomicMin(a.accepted + rq, (int32_t)row - lo_r);
    }
  }
}

hipError_t launch_screen_pass2(const SelectArgs& a, hipStream_t s) {
  if (a.slices < 1 || a.slices > kSelMaxSlices) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_screen_select, dim3(a.slices, a.m), dim3(kSelT), 0, s, a);
  return hipGetLastError();
}

}  // namespace w12
