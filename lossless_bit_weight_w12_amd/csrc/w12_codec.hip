// W12 v1 encode and decode kernels for gfx950.
//
// Encode ("SpecPilot" glossary, "Differentiation": a general lossless 12-bit format):
//   1. exponent histogram (per-wave LDS bins, then 64-bit global atomics),
//   2. codebook = 16 most frequent exponent fields, ties to the smaller field, ascending;
//      e_max and the escape count come from the same histogram (one workgroup),
//   3. escapes per 16x128 tile, 4. exclusive scan over tiles (tile and row-block
//      escape offsets), 5. pack: sm bytes and code nibbles in the slot layout, escape
//      records written in (column, row) order within each tile.
// Decode: tiles + escapes -> BF16 rows, bit-exact.
#include "w12_internal.h"

namespace w12 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__global__ void k_fill_zero(uint8_t* p, size_t bytes) {
  const size_t n16 = bytes / 16;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    reinterpret_cast<u32x4*>(p)[i] = u32x4{0u, 0u, 0u, 0u};
  if (blockIdx.x == 0 && threadIdx.x < (bytes & 15)) p[n16 * 16 + threadIdx.x] = 0;
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  size_t blocks = (bytes / 16 + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(k_fill_zero, dim3((unsigned)blocks), dim3(256), 0, s, (uint8_t*)p, bytes);
  return hipGetLastError();
}

// ---------------------------------------------------------------- 1. histogram
__global__ __launch_bounds__(256) void k_hist(const uint16_t* w, uint64_t count,
                                              unsigned long long* hist) {
  __shared__ uint32_t bins[4][256];
  const int tid = threadIdx.x, wave = tid >> 6;
  for (int i = tid; i < 4 * 256; i += 256) (&bins[0][0])[i] = 0;
  __syncthreads();
  const uint64_t n8 = count / 8;   // count is a multiple of 2048
  const uint64_t stride = (uint64_t)gridDim.x * 256u;
  for (uint64_t i = (uint64_t)blockIdx.x * 256u + tid; i < n8; i += stride) {
    const u32x4 v = reinterpret_cast<const u32x4*>(w)[i];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      atomicAdd(&bins[wave][(v[d] >> 7) & 0xFFu], 1u);
      atomicAdd(&bins[wave][(v[d] >> 23) & 0xFFu], 1u);
    }
  }
  __syncthreads();
  const uint32_t c = bins[0][tid] + bins[1][tid] + bins[2][tid] + bins[3][tid];
  if (c) atomicAdd(hist + tid, (unsigned long long)c);
}

hipError_t launch_encode_hist(const uint16_t* w, uint64_t count, unsigned long long* hist,
                              hipStream_t s) {
  uint64_t blocks = (count / 8 + 255) / 256;
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(k_hist, dim3((unsigned)blocks), dim3(256), 0, s, w, count, hist);
  return hipGetLastError();
}

// ---------------------------------------------------------------- 2. codebook
// result layout: [0..15] codebook, [16] e_max, [24..31] n_esc (u64),
//                [32..63] 256-bit membership mask (8 x u32)
__global__ __launch_bounds__(256) void k_codebook(const unsigned long long* hist,
                                                  uint8_t* result) {
  __shared__ unsigned long long h[256];
  __shared__ uint32_t chosen[256];
  __shared__ unsigned long long esc_part[256];
  __shared__ uint32_t emax_part[256];
  const int e = threadIdx.x;
  h[e] = hist[e];
  __syncthreads();
  const unsigned long long he = h[e];
  uint32_t rank = 0;
  for (int d = 0; d < 256; ++d) {
    const unsigned long long hd = h[d];
    rank += (hd > he || (hd == he && d < e)) ? 1u : 0u;
  }
  const uint32_t sel = rank < 16u ? 1u : 0u;
  chosen[e] = sel;
  esc_part[e] = sel ? 0ull : he;
  emax_part[e] = (e < 255 && he > 0) ? (uint32_t)e : 0u;
  __syncthreads();
  if (sel) {
    uint32_t pos = 0;
    for (int d = 0; d < e; ++d) pos += chosen[d];
    result[pos] = (uint8_t)e;
  }
  for (int off = 128; off > 0; off >>= 1) {
    if (e < off) {
      esc_part[e] += esc_part[e + off];
      emax_part[e] = max(emax_part[e], emax_part[e + off]);
    }
    __syncthreads();
  }
  if (e == 0) {
    result[16] = (uint8_t)emax_part[0];
    *reinterpret_cast<unsigned long long*>(result + 24) = esc_part[0];
  }
  if (e < 8) {
    uint32_t m = 0;
    for (int b = 0; b < 32; ++b) m |= chosen[32 * e + b] << b;
    reinterpret_cast<uint32_t*>(result + 32)[e] = m;
  }
}

hipError_t launch_encode_codebook(const unsigned long long* hist, uint8_t* result,
                                  hipStream_t s) {
  hipLaunchKernelGGL(k_codebook, dim3(1), dim3(256), 0, s, hist, result);
  return hipGetLastError();
}

// ---------------------------------------------------------------- 3. escapes per tile
// Thread t reads 8 consecutive elements: row 16b + t/16, columns 128g + 8*(t%16) + 0..7.
__global__ __launch_bounds__(256) void k_count_tiles(const uint16_t* w, uint32_t g_cols,
                                                     Mask256 mask, uint32_t* tile_cnt) {
  __shared__ uint32_t msk[8];
  __shared__ uint32_t wsum[4];
  const int tid = threadIdx.x;
  if (tid < 8) msk[tid] = mask.m[tid];
  __syncthreads();
  const uint64_t tile = blockIdx.x;
  const uint32_t b = (uint32_t)(tile / g_cols), g = (uint32_t)(tile % g_cols);
  const uint64_t k = (uint64_t)g_cols * 128u;
  const uint16_t* row = w + (uint64_t)(16u * b + (tid >> 4)) * k + 128u * g + 8u * (tid & 15);
  const u32x4 v = *reinterpret_cast<const u32x4*>(row);
  uint32_t c = 0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const uint32_t e0 = (v[d] >> 7) & 0xFFu, e1 = (v[d] >> 23) & 0xFFu;
    c += ((msk[e0 >> 5] >> (e0 & 31)) & 1u) ? 0u : 1u;
    c += ((msk[e1 >> 5] >> (e1 & 31)) & 1u) ? 0u : 1u;
  }
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off);
  if ((tid & 63) == 0) wsum[tid >> 6] = c;
  __syncthreads();
  if (tid == 0) tile_cnt[tile] = wsum[0] + wsum[1] + wsum[2] + wsum[3];
}

hipError_t launch_encode_count_tiles(const uint16_t* w, uint32_t nb, uint32_t g_cols,
                                     const Mask256& member, uint32_t* tile_cnt, hipStream_t s) {
  const uint64_t tiles = (uint64_t)nb * g_cols;
  hipLaunchKernelGGL(k_count_tiles, dim3((unsigned)tiles), dim3(256), 0, s, w, g_cols, member,
                     tile_cnt);
  return hipGetLastError();
}

// ---------------------------------------------------------------- 4. scan over tiles
// One workgroup walks the counts in chunks of 8192: each chunk is read coalesced into
// LDS, every thread scans 8 consecutive counts in registers, the 1024 thread sums are
// scanned with wave shuffles and a 16-entry LDS step, and the running total carries
// into the next chunk.  Row-block offsets are clamped to the escape array's capacity, so
// a descriptor whose n_esc is smaller than the true count never leads a later reader past
// the end of `esc`; `total` receives the true count.
constexpr uint32_t kScanChunk = 8192;
__global__ __launch_bounds__(1024) void k_scan(const uint32_t* tile_cnt, uint32_t n_tiles,
                                               uint32_t g_cols, uint32_t* tile_off,
                                               uint32_t* esc_off, uint32_t esc_cap,
                                               uint32_t* total) {
  __shared__ uint32_t buf[kScanChunk];
  __shared__ uint32_t wsum[16];
  const uint32_t tid = threadIdx.x, lane = tid & 63u, wave = tid >> 6;
  uint32_t carry = 0;
  for (uint32_t base = 0; base < n_tiles; base += kScanChunk) {
#pragma unroll
    for (uint32_t j = 0; j < 8; ++j) {
      const uint32_t i = base + j * 1024u + tid;
      buf[j * 1024u + tid] = i < n_tiles ? tile_cnt[i] : 0u;
    }
    __syncthreads();
    uint32_t v[8], run = 0;
#pragma unroll
    for (uint32_t e = 0; e < 8; ++e) { v[e] = run; run += buf[8u * tid + e]; }   // exclusive
    // inclusive scan of the thread sums across the wave
    uint32_t inc = run;
#pragma unroll
    for (uint32_t off = 1; off < 64; off <<= 1) {
      const uint32_t o = __shfl_up(inc, off);
      if (lane >= off) inc += o;
    }
    if (lane == 63) wsum[wave] = inc;
    __syncthreads();
    uint32_t before = 0, chunk_total = 0;
    for (uint32_t w = 0; w < 16; ++w) {
      const uint32_t t = wsum[w];
      before += w < wave ? t : 0u;
      chunk_total += t;
    }
    const uint32_t excl = carry + before + inc - run;
#pragma unroll
    for (uint32_t e = 0; e < 8; ++e) {
      const uint32_t i = base + 8u * tid + e;
      if (i < n_tiles) {
        tile_off[i] = excl + v[e];
        if (i % g_cols == 0) esc_off[i / g_cols] = min(excl + v[e], esc_cap);
      }
    }
    carry += chunk_total;
    __syncthreads();   // buf and wsum are rewritten by the next chunk
  }
  if (tid == 0) {
    esc_off[n_tiles / g_cols] = min(carry, esc_cap);
    *total = carry;
  }
}

hipError_t launch_encode_scan(const uint32_t* tile_cnt, uint32_t n_tiles, uint32_t g_cols,
                              uint32_t* tile_off, uint32_t* esc_off, uint32_t esc_cap,
                              uint32_t* total, hipStream_t s) {
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, tile_cnt, n_tiles, g_cols, tile_off,
                     esc_off, esc_cap, total);
  return hipGetLastError();
}

// ---------------------------------------------------------------- 5. pack
// One workgroup per tile, numbered row-block major (the escape order); the tile's bytes
// go to its column-major place, (g * nb + b) * 3072.
// Thread t = 4l + j builds slot l's elements 8j..8j+7: columns 32j + 8q + 0..7 of row r.
__global__ __launch_bounds__(256) void k_pack(const uint16_t* w, uint32_t nb, uint32_t g_cols,
                                              Codebook16 codebook,
                                              const uint32_t* tile_off, uint8_t* tiles,
                                              uint32_t* esc, uint64_t esc_cap) {
  __shared__ uint8_t code_of[256];
  __shared__ uint16_t ex[2048];       // exponent of an escape at order index kappa*16 + r
  __shared__ uint32_t wsum[4];
  const int tid = threadIdx.x;
  code_of[tid] = 0xFF;
  __syncthreads();
  if (tid < 16) code_of[codebook.c[tid]] = (uint8_t)tid;
  __syncthreads();
  const uint64_t tile = blockIdx.x;
  const uint32_t b = (uint32_t)(tile / g_cols), g = (uint32_t)(tile % g_cols);
  const uint64_t k = (uint64_t)g_cols * 128u;
  const int l = tid >> 2, j = tid & 3, r = l & 15, q = l >> 4;
  const uint32_t kap0 = 32u * j + 8u * q;
  const u32x4 v = *reinterpret_cast<const u32x4*>(w + (uint64_t)(16u * b + r) * k + 128u * g + kap0);
  uint32_t sm_lo = 0, sm_hi = 0, cw = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t bits = (i & 1) ? (v[i >> 1] >> 16) : (v[i >> 1] & 0xFFFFu);
    const uint32_t e = (bits >> 7) & 0xFFu;
    const uint32_t sm = ((bits >> 8) & 0x80u) | (bits & 0x7Fu);
    const uint32_t cd = code_of[e];
    const bool is_esc = cd == 0xFFu;
    if (i < 4) sm_lo |= sm << (8 * i);
    else sm_hi |= sm << (8 * (i - 4));
    cw |= (is_esc ? 0u : cd) << (4 * (i >> 1) + 16 * (i & 1));
    ex[(kap0 + i) * 16 + r] = is_esc ? (uint16_t)e : (uint16_t)0xFFFF;
  }
  uint8_t* tb = tiles + ((uint64_t)g * nb + b) * 3072u;
  *reinterpret_cast<u32x2*>(tb + 1024 * (j >> 1) + 16 * l + 8 * (j & 1)) = u32x2{sm_lo, sm_hi};
  *reinterpret_cast<uint32_t*>(tb + 2048 + 16 * l + 4 * j) = cw;
  __syncthreads();
  // escape records in (kappa, r) order: thread t owns order indices 8t..8t+7
  uint32_t c = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) c += ex[8 * tid + u] != 0xFFFF ? 1u : 0u;
  // block exclusive scan of c
  uint32_t incl = c;
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t t = __shfl_up(incl, off);
    if ((tid & 63) >= off) incl += t;
  }
  if ((tid & 63) == 63) wsum[tid >> 6] = incl;
  __syncthreads();
  uint32_t base = 0;
  for (int wv = 0; wv < (tid >> 6); ++wv) base += wsum[wv];
  uint32_t rank = base + incl - c;
  if (c) {
    const uint64_t t0 = tile_off[tile];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const uint32_t p = 8u * tid + u;
      const uint16_t e = ex[p];
      if (e != 0xFFFF) {
        const uint32_t kap = p >> 4, rr = p & 15u;
        const uint64_t idx = t0 + rank;
        if (idx < esc_cap) esc[idx] = (rr << 28) | ((128u * g + kap) << 8) | e;
        ++rank;
      }
    }
  }
}

hipError_t launch_encode_pack(const uint16_t* w, uint32_t nb, uint32_t g_cols,
                              const Codebook16& codebook, const uint32_t* tile_off,
                              uint8_t* tiles, uint32_t* esc, uint64_t esc_cap,
                              hipStream_t s) {
  const uint64_t n_tiles = (uint64_t)nb * g_cols;
  hipLaunchKernelGGL(k_pack, dim3((unsigned)n_tiles), dim3(256), 0, s, w, nb, g_cols, codebook,
                     tile_off, tiles, esc, esc_cap);
  return hipGetLastError();
}

// ---------------------------------------------------------------- decode
__global__ __launch_bounds__(256) void k_decode(const uint8_t* tiles, const uint32_t* esc_off,
                                                const uint32_t* esc, uint32_t nb, uint32_t g_cols,
                                                Codebook16 cb, uint16_t* w_out) {
  __shared__ uint16_t ovr[2048];     // escape exponent at kappa*16 + r, 0xFFFF = none
  __shared__ uint32_t s_range[2];
  const int tid = threadIdx.x;
  const uint64_t tile = blockIdx.x;
  const uint32_t b = (uint32_t)(tile / g_cols), g = (uint32_t)(tile % g_cols);
  for (int i = tid; i < 2048; i += 256) ovr[i] = 0xFFFF;
  if (tid == 0) {
    // records of row-block b with column in [128g, 128g + 128): binary search on column
    const uint32_t lo0 = esc_off[b], hi0 = esc_off[b + 1];
    uint32_t lo = lo0, hi = hi0;
    while (lo < hi) {
      const uint32_t mid = lo + (hi - lo) / 2;
      if (((esc[mid] >> 8) & 0xFFFFFu) < 128u * g) lo = mid + 1; else hi = mid;
    }
    uint32_t lo2 = lo, hi2 = hi0;
    while (lo2 < hi2) {
      const uint32_t mid = lo2 + (hi2 - lo2) / 2;
      if (((esc[mid] >> 8) & 0xFFFFFu) < 128u * (g + 1)) lo2 = mid + 1; else hi2 = mid;
    }
    s_range[0] = lo;
    s_range[1] = lo2;
  }
  __syncthreads();
  for (uint32_t i = s_range[0] + tid; i < s_range[1]; i += 256) {
    const uint32_t rec = esc[i];
    const uint32_t kap = ((rec >> 8) & 0xFFFFFu) - 128u * g;
    ovr[kap * 16 + (rec >> 28)] = (uint16_t)(rec & 0xFFu);
  }
  __syncthreads();
  const int l = tid >> 2, j = tid & 3, r = l & 15, q = l >> 4;
  const uint32_t kap0 = 32u * j + 8u * q;
  const uint8_t* tb = tiles + ((uint64_t)g * nb + b) * 3072u;
  const u32x2 sm = *reinterpret_cast<const u32x2*>(tb + 1024 * (j >> 1) + 16 * l + 8 * (j & 1));
  const uint32_t cw = *reinterpret_cast<const uint32_t*>(tb + 2048 + 16 * l + 4 * j);
  uint32_t out[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t s8 = ((i < 4 ? sm[0] : sm[1]) >> (8 * (i & 3))) & 0xFFu;
    const uint32_t code = (cw >> (4 * (i >> 1) + 16 * (i & 1))) & 0xFu;
    const uint16_t o = ovr[(kap0 + i) * 16 + r];
    const uint32_t e = (o != 0xFFFF) ? (uint32_t)o : (uint32_t)cb.c[code];
    const uint32_t bits = ((s8 & 0x80u) << 8) | (e << 7) | (s8 & 0x7Fu);
    out[i >> 1] |= bits << (16 * (i & 1));
  }
  const uint64_t k = (uint64_t)g_cols * 128u;
  *reinterpret_cast<u32x4*>(w_out + (uint64_t)(16u * b + r) * k + 128u * g + kap0) =
      u32x4{out[0], out[1], out[2], out[3]};
}

hipError_t launch_decode(const uint8_t* tiles, const uint32_t* esc_off, const uint32_t* esc,
                         uint32_t nb, uint32_t g_cols, const Codebook16& cb,
                         uint16_t* w_out, hipStream_t s) {
  const uint64_t n_tiles = (uint64_t)nb * g_cols;
  hipLaunchKernelGGL(k_decode, dim3((unsigned)n_tiles), dim3(256), 0, s, tiles, esc_off, esc,
                     nb, g_cols, cb, w_out);
  return hipGetLastError();
}

// ---------------------------------------------------------------- RMS rescale (chain)
// One workgroup per row; k % 8 == 0 and 16-byte aligned rows, so every thread moves
// 8 BF16 per load and store.  The sum of squares is reduced in a fixed order (per
// thread, then a fixed tree), so the result is deterministic.
__global__ __launch_bounds__(256) void k_rms(const uint16_t* __restrict__ x, uint32_t k,
                                             uint16_t* __restrict__ y) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  __shared__ float part[4];
  const uint32_t row = blockIdx.x, tid = threadIdx.x, units = k >> 3;
  const u32x4* xr = reinterpret_cast<const u32x4*>(x + (uint64_t)row * k);
  u32x4* yr = reinterpret_cast<u32x4*>(y + (uint64_t)row * k);
  float s = 0.f;
  for (uint32_t u = tid; u < units; u += 256) {
    const u32x4 v = xr[u];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(v[i] << 16), hi = __uint_as_float(v[i] & 0xFFFF0000u);
      s += lo * lo + hi * hi;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if ((tid & 63) == 0) part[tid >> 6] = s;
  __syncthreads();
  const float rms = sqrtf(((part[0] + part[1]) + (part[2] + part[3])) / (float)k);
  auto rne = [](float f) -> uint32_t {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7F800000u) == 0x7F800000u && (u & 0x007FFFFFu)) u |= 0x00400000u;
    else u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
  };
  for (uint32_t u = tid; u < units; u += 256) {
    const u32x4 v = xr[u];
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float lo = __uint_as_float(v[i] << 16) / rms, hi = __uint_as_float(v[i] & 0xFFFF0000u) / rms;
      o[i] = rne(lo) | (rne(hi) << 16);
    }
    yr[u] = o;
  }
}

// Row-major BF16 -> 4 KB tiles: tile (b, g) at (g * nb + b) * 4096 (column-major, as
// the W12 tiles), lane slot l
// (r = l % 16, q = l / 16) of group j at 1024 j + 16 l holding row 16b + r, columns
// 128g + 32j + 8q .. +7.  One thread per 16-byte unit.
__global__ __launch_bounds__(256) void k_bf16_tile(const uint16_t* __restrict__ w, uint32_t nb,
                                                   uint32_t g_cols, uint8_t* __restrict__ out) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const uint64_t units = (uint64_t)nb * g_cols * 256u;
  const uint64_t k = (uint64_t)g_cols * 128u;
  for (uint64_t u = (uint64_t)blockIdx.x * 256u + threadIdx.x; u < units;
       u += (uint64_t)gridDim.x * 256u) {
    const uint64_t tile = u >> 8;
    const uint32_t within = (uint32_t)(u & 255u), j = within >> 6, l = within & 63u;
    const uint64_t b = tile / g_cols, g = tile % g_cols;
    const uint32_t r = l & 15u, q = l >> 4;
    const u32x4 v = *reinterpret_cast<const u32x4*>(w + (16u * b + r) * k + 128u * g + 32u * j + 8u * q);
    *reinterpret_cast<u32x4*>(out + (g * nb + b) * 4096u + 1024u * j + 16u * l) = v;
  }
}

hipError_t launch_bf16_tile(const uint16_t* w, uint32_t nb, uint32_t g_cols, uint8_t* out,
                            hipStream_t s) {
  const uint64_t units = (uint64_t)nb * g_cols * 256u;
  uint64_t blocks = (units + 255u) / 256u;
  if (blocks > 65536u) blocks = 65536u;
  hipLaunchKernelGGL(k_bf16_tile, dim3((uint32_t)blocks), dim3(256), 0, s, w, nb, g_cols, out);
  return hipGetLastError();
}

// Row-major FP8 bytes -> 2 KB tiles: tile (b, g) at (g * nb + b) * 2048, the 8 bytes of
// lane slot l (r = l % 16, q = l / 16) in group j (row 16b + r, columns
// 128g + 32j + 8q .. +7) at 1024 (j / 2) + 16 l + 8 (j % 2): the byte order of the W12
// sign/mantissa bytes, so that each wave instruction of the GEMM reads 1 KB of whole
// lines.  One thread per 8-byte unit.
__global__ __launch_bounds__(256) void k_f8_tile(const uint8_t* __restrict__ w, uint32_t nb,
                                                 uint32_t g_cols, uint8_t* __restrict__ out) {
  const uint64_t units = (uint64_t)nb * g_cols * 256u;
  const uint64_t k = (uint64_t)g_cols * 128u;
  for (uint64_t u = (uint64_t)blockIdx.x * 256u + threadIdx.x; u < units;
       u += (uint64_t)gridDim.x * 256u) {
    const uint64_t tile = u >> 8;
    const uint32_t within = (uint32_t)(u & 255u), j = within >> 6, l = within & 63u;
    const uint64_t b = tile / g_cols, g = tile % g_cols;
    const uint32_t r = l & 15u, q = l >> 4;
    const uint2 v = *reinterpret_cast<const uint2*>(w + (16u * b + r) * k + 128u * g + 32u * j + 8u * q);
    *reinterpret_cast<uint2*>(out + (g * nb + b) * 2048u + 1024u * (j >> 1) + 16u * l + 8u * (j & 1u)) = v;
  }
}

hipError_t launch_f8_tile(const uint8_t* w, uint32_t nb, uint32_t g_cols, uint8_t* out,
                          hipStream_t s) {
  const uint64_t units = (uint64_t)nb * g_cols * 256u;
  uint64_t blocks = (units + 255u) / 256u;
  if (blocks > 65536u) blocks = 65536u;
  hipLaunchKernelGGL(k_f8_tile, dim3((uint32_t)blocks), dim3(256), 0, s, w, nb, g_cols, out);
  return hipGetLastError();
}

hipError_t launch_rms_rescale(const uint16_t* x, uint32_t m, uint32_t k, uint16_t* y,
                              hipStream_t s) {
  hipLaunchKernelGGL(k_rms, dim3(m), dim3(256), 0, s, x, k, y);
  return hipGetLastError();
}

}  // namespace w12
