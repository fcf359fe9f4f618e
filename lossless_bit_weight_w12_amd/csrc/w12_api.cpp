// C-ABI host layer of libw12.so: argument validation (before any HIP call), workspace
// layout, kernel-family dispatch and launch.  No HIP call happens at load time.
#include "w12.h"
#include "w12_internal.h"

#include <string.h>

#include <algorithm>

using namespace w12;

namespace {

constexpr uint64_t kMaxK = 1ull << 20;
constexpr uint64_t kMaxN = 1ull << 31;
#ifndef W12_TARGET_WG
#define W12_TARGET_WG 1024
#endif
#ifndef W12_CS_FEW_NW
#define W12_CS_FEW_NW 5
#endif
#ifndef W12_CS_NW
#define W12_CS_NW 5
#endif
#ifndef W12_CS_NW32
#define W12_CS_NW32 10   // 17..128 x columns on 2048..2560 row-blocks
#endif
static_assert((W12_CS_NW == 4 || W12_CS_NW == 5) && (W12_CS_FEW_NW == 4 || W12_CS_FEW_NW == 5) &&
              (W12_CS_NW32 == 5 || W12_CS_NW32 == 10),
              "column-synchronous launches are instantiated for 4 and 5 waves (and 10 from 32 columns)");
#ifndef W12_NS_CAP
#define W12_NS_CAP 8
#endif
static_assert(W12_NS_CAP >= 1 && W12_NS_CAP <= w12::kMaxSplit, "split cap within the completing split's limit");
#ifndef W12_CS_MIN_COLS
#define W12_CS_MIN_COLS 4
#endif
constexpr int kTargetWorkgroups = W12_TARGET_WG;   // 4-wave workgroups: 4 per CU on 256 CUs

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

inline bool shape_ok(uint64_t n, uint64_t k) {
  return n > 0 && k > 0 && n % 16 == 0 && k % 128 == 0 && k < kMaxK && n < kMaxN &&
         (n / 16) * (k / 128) < (1ull << 31);
}

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Element counts of [m][n] outputs and workspaces stay below 2^32 (32-bit indexing).
inline bool mn_ok(uint32_t m, uint64_t n) { return (uint64_t)m * n < (1ull << 32); }

w12_status check_desc(const w12_desc* d, bool need_data) {
  if (!d) return W12_ERR_NULL;
  if (!shape_ok(d->n, d->k)) return W12_ERR_SHAPE;
  for (int i = 1; i < 16; ++i)
    if (d->codebook[i] <= d->codebook[i - 1]) return W12_ERR_FORMAT;
  if (d->e_max >= 255) return W12_ERR_FORMAT;
  if (d->n_esc > (uint64_t)d->n * d->k || d->n_esc >= (1ull << 32)) return W12_ERR_FORMAT;
  if (need_data) {
    if (!d->tiles || !d->esc_off) return W12_ERR_NULL;
    if (d->n_esc > 0 && !d->esc) return W12_ERR_NULL;
    if (!aligned(d->tiles, 16)) return W12_ERR_ALIGN;
  }
  return W12_OK;
}

inline bool codebook_is_run(const uint8_t* c) {
  for (int i = 1; i < 16; ++i)
    if (c[i] != (uint8_t)(c[0] + i)) return false;
  return true;
}

#ifndef W12_RBW2_MIN_NB
#define W12_RBW2_MIN_NB 1024   // row-blocks from which workgroups take two row-blocks
#endif

// Work split: row-blocks per workgroup and K splits so that the grid holds enough
// workgroups to keep 256 CUs streaming; splits keep at least one column per wave.
// Kernel choice, measured on the MLP-block shapes (gate+up 2176 row-blocks x 40 tile
// columns, down 320 x 136):
//  - m < W12_MFMA_MIN_M: VALU path, waves stream their own columns;
//  - few row-blocks (long K): column-synchronous MFMA, K split;
//  - many row-blocks: wave-column MFMA below m = 16 (no per-column barrier), column-
//    synchronous from m = 16 (x traffic dominates).
// W12 launches with the BF16 epilogue take the column-synchronous kernel at every m: with
// 5-wave workgroups it beats the wave-column kernels there too (gate+up M1 / M4 / M8
// 47.2 / 47.5 / 48.6 -> 43.4 / 43.5 / 43.5 us, down M1 26.6 -> 25.8 us).  The BF16
// baselines and the logits epilogue keep the wave-column kernels below m = 16, which are
// faster for them (tiled BF16 gate+up M1 57.1 us against 61.9; LM-head verification M1
// 193 us against 201).
// Column-synchronous workgroups take 5 row-blocks (5 waves).  Every workgroup of a launch
// is resident at once, so the CU holding the most row-blocks sets the time: gate+up with
// 4 per workgroup is 544 workgroups, up to 3 on a CU (12 row-blocks against 8.5 on
// average); with 5 it is 436, at most 2 (10).  Measured: gate+up M16 / M24 / M32 5.44 /
// 4.87 / 4.60 -> 5.82 / 5.21 / 5.13 TB/s, and the split down launches (64 groups x 8
// splits = 2 workgroups per CU) M32 4.18 -> 4.44; 6 or 7 waves (12 and 14 row-blocks per
// CU) are slower, 3 ties on gate+up and loses on down, 8 (272 workgroups) loses.  With
// 32-column x tiles on 2048..2560 row-blocks, 10 waves (at most one workgroup per CU, K
// whole, half the x requests per row-block) are faster: gate+up M32 tiled BF16 69.2 ->
// 64.0 us, row-major BF16 86.3 -> 78.4 us, W12 M24 / M32 49.3 / 48.9 -> 48.0 / 48.5 us;
// at 16 columns the BF16 baselines gain too (tiled 62.0 -> 58.5 us, row-major 79.3 ->
// 75.1 us) and W12 does not (43.3 us either way); at 64 and 128 columns both gain (W12
// gate+up M64 / M128 63.5 / 128.8 -> 59.7 / 84.3 us, tiled BF16 84.0 / 122.7 -> 73.1 /
// 107.8 us).  The logits epilogue takes 8 waves (LM head, M = 16: 214 us with 4 waves, 200
// with 8, 208 with 10, 5 slower than 4; M = 24: 238 / 222 / 246 us; M = 120: 793 / 519 /
// 522 us, 933 with 16; M = 64: 358 / 292 / 329 / 317 us).  Few row-blocks at 65..128 columns (K split 8 ways)
// take 10 waves as well, one workgroup per CU (down M128 W12 65.1 -> 48.6 us, tiled BF16
// 69.2 -> 50.7 us; at 64 columns 5 stays ahead); other shapes keep 4 at 128 columns (74 KB
// of LDS per workgroup; gate+up M128 135 -> 164 us with 5).
// W12 launches with the BF16 epilogue at 1..32 rows choose the wave count among 5, 7 and
// 9 by the same residency argument, counted in tiles: every workgroup is resident, so the
// launch takes as long as the CU with the most tiles to stream, ceil(workgroups / 256) x
// waves x tile columns per split; the larger wave count wins a tie (fewer x requests per
// row-block).  Measured (one box, interleaved): the decode chain's q/k/v group (448
// row-blocks, K split 8 ways; 5 -> 7 waves, 720 -> 512 workgroups) 19.95 -> 17.48 us at
// M = 24, 20.42 -> 19.09 us with the RMS rescale; its gate/up group (2176 row-blocks;
// 5 or 10 -> 9 waves, 242 workgroups) 50.78 -> 49.63 us with the RMS rescale at M = 24,
// the MLP gate+up within 1 % at M = 1..32; down and o (320 row-blocks) keep 5.
GemmPlan make_plan(uint32_t m, uint64_t n, uint64_t k, int epi, bool bf16_src = false) {
  GemmPlan p;
  const uint64_t nb = n / 16, g = k / 128;
  uint64_t min_cols;   // tile columns a split keeps at least
  p.kind = KIND_WAVE_COLUMNS;
  p.mfma = m >= W12_MFMA_MIN_M;
  p.rbw = 1;
  p.nw = 4;
  const bool few_rows = nb < W12_RBW2_MIN_NB;
  const bool w12_bf16_out = !bf16_src && epi == EPI_BF16;
  // K splits of a launch of `groups` row-block groups (units: 4-wave workgroup equivalents)
  auto splits = [&](uint64_t units, int kind) -> uint64_t {
    // W12 column-synchronous launches that already fill the chip (>= 512 four-wave
    // workgroups) keep K whole: the partials and their completion cost more than the
    // extra parallelism gains.  The BF16 kernel (4 KB tiles) is faster split: measured
    // on the MLP gate+up at M16 / M32, 81 / 92 us split in two against 87 / 100 us whole.
    const bool keep_k = !bf16_src && kind == KIND_COLUMN_SYNC &&
                        units >= (uint64_t)kTargetWorkgroups / 2;
    if (epi != EPI_BF16 || keep_k) return 1;
    // enough splits to reach the workgroup target, each keeping >= min_cols columns
    uint64_t ns = ((uint64_t)kTargetWorkgroups + units - 1) / units;
    ns = std::min<uint64_t>(ns, std::min<uint64_t>(W12_NS_CAP, g / min_cols));
    return std::max<uint64_t>(ns, 1);
  };
  uint64_t units;
  // the logits epilogue runs column-synchronous from 4 rows on (151936-row LM head:
  // M4 / M8 196.6 / 205.6 -> 192.6 / 192.4 us against the wave-column MFMA kernel); at
  // 1..3 rows the wave-column VALU kernel is 1 us faster (189.2 against 190.3 us)
  if (w12_bf16_out || (p.mfma && (epi == EPI_LOGITS || few_rows || m >= 16))) {
    p.kind = KIND_COLUMN_SYNC;
    min_cols = W12_CS_MIN_COLS;
    if (w12_bf16_out && m <= 32) {
      uint64_t best = ~0ull;
      for (int nw : {5, 7, 9}) {
        const uint64_t groups = (nb + nw - 1) / nw;
        const uint64_t ns = splits(groups * nw / 4, KIND_COLUMN_SYNC);
        const uint64_t tiles = (groups * ns + 255) / 256 * nw * ((g + ns - 1) / ns);
        if (tiles <= best) { best = tiles; p.nw = nw; }
      }
    } else {
      // 17..128 columns (16..128 for the BF16 baselines): 10 waves where that is at most
      // one workgroup per CU with K whole
      const bool ten = (m > 16 || bf16_src) && nb >= 2048 && (nb + 9) / 10 <= 256;
      p.nw = epi != EPI_BF16 ? 8
             : few_rows ? (m > 64 ? W12_CS_NW32 : W12_CS_FEW_NW)
             : ten ? W12_CS_NW32 : (m > 64 ? 4 : W12_CS_NW);
    }
    p.n_rbg = (uint32_t)((nb + p.nw - 1) / p.nw);
    units = (uint64_t)p.n_rbg * p.nw / 4;
  } else {
    min_cols = 4;
    p.rbw = few_rows ? 1 : 2;
    p.n_rbg = (uint32_t)((nb + p.rbw - 1) / p.rbw);
    units = p.n_rbg;
  }
  p.nsplit = (uint32_t)splits(units, p.kind);   // the kernels deal the K range evenly
  return p;
}

// GEMM workspace when K is split: the row-block groups' tickets (a fixed 4 KB region at the
// start: they must be zero before the first split launch and every launch leaves them
// zero), the FP32 partials [nsplit][m][n], and (RMS launches) each group's per-split sums
// of x^2 [groups][nsplit][m].  A split launch has fewer than 1024 row-block groups (it is
// split because it has fewer than kTargetWorkgroups four-wave workgroup equivalents).
constexpr size_t kTicketBytes = 4096;
constexpr uint32_t kMaxTickets = kTicketBytes / 4;

size_t split_ws_bytes(uint64_t nsplit, uint32_t m, uint64_t n, uint64_t groups) {
  return nsplit > 1 ? kTicketBytes + align256((size_t)nsplit * m * n * 4) +
                          align256((size_t)groups * nsplit * m * 4)
                    : 0;
}

size_t gemm_ws_bytes(uint32_t m, uint64_t n, uint64_t k, bool bf16_src = false) {
  const GemmPlan p = make_plan(m, n, k, EPI_BF16, bf16_src);
  return split_ws_bytes(p.nsplit, m, n, p.n_rbg);
}

// A group may run as two launches (one per codebook kind), each over part of the rows:
// enough for the most splits any part can take, and for the most row-block groups (W12
// launches take at least four row-blocks per workgroup).
size_t group_ws_bytes(uint32_t m, uint64_t n_total, uint64_t k) {
  const uint64_t g = k / 128;
  const uint64_t cap = std::min<uint64_t>(W12_NS_CAP, std::max<uint64_t>(g / 4, 1));
  const uint64_t groups = std::min<uint64_t>((n_total / 16 + 3) / 4, kMaxTickets);
  return split_ws_bytes(cap, m, n_total, groups);
}

// Point a launch's split-K state into the workspace (nothing when K is whole).
bool set_split_ws(GemmArgs& a, void* ws, const GemmPlan& p, uint32_t m, uint64_t n) {
  if (p.nsplit <= 1) return true;
  if (p.n_rbg > kMaxTickets) return false;   // (no plan splits that many groups)
  a.p.tickets = (uint32_t*)ws;
  a.partial = (float*)((uint8_t*)ws + kTicketBytes);
  a.p.ss = (float*)((uint8_t*)a.partial + align256((size_t)p.nsplit * m * n * 4));
  return true;
}

// Verify workspace: per-row diagnostic counts first (a fixed place), then the
// per-row-block records of pass 1, its group records (one per workgroup of pass 1: at
// most one per row-block) and the candidate lists of pass 2.
struct VerifyLayout {
  size_t ncand, bm_v, bm_v2, bm_s, bm_i, g_v, g_v2, g_i, g_s, g_w, cand, total;
};

VerifyLayout verify_layout(uint32_t m, uint64_t n) {
  VerifyLayout L;
  const uint64_t nb = n / 16;
  const size_t rec = align256((size_t)m * nb * 4);
  L.ncand = 0;
  L.bm_v = L.ncand + align256((size_t)m * 8);
  L.bm_v2 = L.bm_v + rec;
  L.bm_s = L.bm_v2 + rec;
  L.bm_i = L.bm_s + rec;
  L.g_v = L.bm_i + rec;
  L.g_v2 = L.g_v + rec;
  L.g_i = L.g_v2 + rec;
  L.g_s = L.g_i + rec;
  L.g_w = L.g_s + rec;
  L.cand = L.g_w + rec;
  L.total = L.cand + align256((size_t)m * n * 4);
  return L;
}

// Records of pass 1 for a launch of plan p (group records: one per row-block group).
BlockMax block_max(uint8_t* base, const VerifyLayout& L, const GemmPlan& p) {
  BlockMax bm;
  memset(&bm, 0, sizeof(bm));   // no accept, no request table
  bm.v = (float*)(base + L.bm_v);
  bm.v2 = (float*)(base + L.bm_v2);
  bm.s = (float*)(base + L.bm_s);
  bm.i = (int32_t*)(base + L.bm_i);
  bm.gv = (float*)(base + L.g_v);
  bm.gv2 = (float*)(base + L.g_v2);
  bm.gi = (int32_t*)(base + L.g_i);
  bm.gs = (float*)(base + L.g_s);
  bm.gw = (float*)(base + L.g_w);
  bm.ngrp = p.n_rbg;
  return bm;
}

// Row-blocks per group record of a logits launch.
inline uint32_t blocks_per_group(const GemmPlan& p) {
  return p.kind == KIND_COLUMN_SYNC ? (uint32_t)p.nw : (uint32_t)p.rbw;
}

struct EncodeLayout {
  size_t hist, result, total, tile_cnt, tile_off, bytes;
};

EncodeLayout encode_layout(uint64_t n, uint64_t k) {
  EncodeLayout L;
  const uint64_t tiles = (n / 16) * (k / 128);
  L.hist = 0;                 // 256 x u64
  L.result = 2048;            // 64 bytes
  L.total = W12_ENCODE_TOTAL_OFFSET;   // u32: the true escape count (w12_encode)
  L.tile_cnt = 4096;
  L.tile_off = L.tile_cnt + align256((size_t)tiles * 4);
  L.bytes = L.tile_off + align256((size_t)tiles * 4);
  return L;
}

inline w12_status hip_status(hipError_t e) { return e == hipSuccess ? W12_OK : W12_ERR_HIP; }

// Segment of a launch for a W12 weight (codebook as kernel arguments).
Seg w12_seg(const w12_desc* d, uint16_t* y, uint32_t rb0) {
  Seg g;
  memset(&g, 0, sizeof(g));
  g.w = (const uint8_t*)d->tiles;
  g.esc_off = d->esc_off;
  g.esc = d->esc;
  g.y = y;
  g.rb0 = rb0;
  g.n = (uint32_t)d->n;
  for (int i = 0; i < 4; ++i)
    g.lut[i] = (uint32_t)d->codebook[4 * i] | ((uint32_t)d->codebook[4 * i + 1] << 8) |
               ((uint32_t)d->codebook[4 * i + 2] << 16) | ((uint32_t)d->codebook[4 * i + 3] << 24);
  g.basepair = (uint32_t)d->codebook[0] | ((uint32_t)d->codebook[0] << 16);
  return g;
}

// Launch parameters common to every segment.
void fill_params(GemmParams& p, uint32_t m, uint64_t k, uint64_t n_total, uint32_t nseg) {
  p.m = m;
  p.k = (uint32_t)k;
  p.g_cols = (uint32_t)(k / 128);
  p.n = (uint32_t)n_total;
  p.nb = (uint32_t)(n_total / 16);
  p.nseg = nseg;
  p.rms = 0;
  p.ss = nullptr;
  p.tickets = nullptr;
}

// One launch over segments ds[0..nseg) (same k, same codebook kind): y_i = x . W_i^T,
// each row divided by the RMS of its x row when rms is set.
hipError_t launch_w12_group(const uint16_t* x, uint32_t m, const w12_desc* const* ds,
                            uint16_t* const* ys, uint32_t nseg, void* ws, hipStream_t s,
                            bool rms) {
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  uint64_t n_total = 0;
  for (uint32_t i = 0; i < nseg; ++i) {
    a.p.seg[i] = w12_seg(ds[i], ys[i], (uint32_t)(n_total / 16));
    n_total += ds[i]->n;
  }
  fill_params(a.p, m, ds[0]->k, n_total, nseg);
  const GemmPlan p = make_plan(m, n_total, ds[0]->k, EPI_BF16);
  a.p.rms = rms ? 1u : 0u;
  if (!set_split_ws(a, ws, p, m, n_total)) return hipErrorInvalidValue;
  const int src = codebook_is_run(ds[0]->codebook) ? SRC_RUN : SRC_LUT;
  return launch_gemm(a, src, EPI_BF16, p, s);
}

}  // namespace

// The argument checks of w12_gemm other than the workspace's (host only, no HIP call);
// *need = the workspace bytes the call takes.
w12_status w12::gemm_check(const uint16_t* x, uint32_t m, const w12_desc* d, const uint16_t* y,
                           size_t* need) {
  if (!x || !y) return W12_ERR_NULL;
  w12_status st = check_desc(d, true);
  if (st != W12_OK) return st;
  if (m < 1 || m > W12_MAX_M) return W12_ERR_RANGE;
  if (!mn_ok(m, d->n)) return W12_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(y, 16)) return W12_ERR_ALIGN;
  *need = gemm_ws_bytes(m, d->n, d->k);
  return W12_OK;
}

// w12_gemm after its checks: launch on a workspace of at least the needed bytes.
w12_status w12::gemm_launch(const uint16_t* x, uint32_t m, const w12_desc* d, uint16_t* y,
                            void* ws, void* stream, bool rms) {
  return hip_status(launch_w12_group(x, m, &d, &y, 1, ws, (hipStream_t)stream, rms));
}

namespace {

w12_status gemm_impl(const uint16_t* x, uint32_t m, const w12_desc* d, uint16_t* y, void* ws,
                     size_t ws_bytes, void* stream, bool rms) {
  size_t need = 0;
  const w12_status st = gemm_check(x, m, d, y, &need);
  if (st != W12_OK) return st;
  if (ws_bytes < need) return W12_ERR_WORKSPACE;
  if (need > 0 && !ws) return W12_ERR_NULL;
  if (!aligned(ws, 256)) return W12_ERR_ALIGN;
  return gemm_launch(x, m, d, y, ws, stream, rms);
}

w12_status gemm_group_impl(const uint16_t* x, uint32_t m, const w12_desc* const* descs,
                           uint32_t n_w, uint16_t* const* ys, void* ws, size_t ws_bytes,
                           void* stream, bool rms) {
  if (!x || !descs || !ys) return W12_ERR_NULL;
  if (n_w < 1 || n_w > W12_MAX_GROUP || m < 1 || m > W12_MAX_M) return W12_ERR_RANGE;
  uint64_t n_total = 0;
  for (uint32_t i = 0; i < n_w; ++i) {
    w12_status st = check_desc(descs[i], true);
    if (st != W12_OK) return st;
    if (!ys[i]) return W12_ERR_NULL;
    if (descs[i]->k != descs[0]->k) return W12_ERR_SHAPE;
    if (!aligned(ys[i], 16)) return W12_ERR_ALIGN;
    n_total += descs[i]->n;
  }
  if (n_total >= kMaxN || !mn_ok(m, n_total)) return W12_ERR_SHAPE;
  const size_t need = group_ws_bytes(m, n_total, descs[0]->k);
  if (ws_bytes < need) return W12_ERR_WORKSPACE;
  if (need > 0 && !ws) return W12_ERR_NULL;
  if (!aligned(x, 16) || !aligned(ws, 256)) return W12_ERR_ALIGN;
  // one launch per codebook kind (run / lookup table), in the callers' order within each
  const w12_desc* dd[2][W12_MAX_GROUP];
  uint16_t* yy[2][W12_MAX_GROUP];
  uint32_t cnt[2] = {0, 0};
  for (uint32_t i = 0; i < n_w; ++i) {
    const int kind = codebook_is_run(descs[i]->codebook) ? 0 : 1;
    dd[kind][cnt[kind]] = descs[i];
    yy[kind][cnt[kind]++] = ys[i];
  }
  hipError_t e = hipSuccess;
  for (int kind = 0; kind < 2 && e == hipSuccess; ++kind)
    if (cnt[kind])
      e = launch_w12_group(x, m, dd[kind], yy[kind], cnt[kind], ws, (hipStream_t)stream, rms);
  return hip_status(e);
}

// Both verification entry points: one request over all rows (req_off NULL, n_draft
// tokens) or a request table (req_off, req_ndraft: n_req entries, device).
w12_status verify_impl(const uint16_t* x, uint32_t m, const w12_desc* d, const int32_t* draft,
                       uint32_t n_draft, const int32_t* req_off, const int32_t* req_ndraft,
                       uint32_t n_req, int32_t* argmax_out, int32_t* accepted_out, void* ws,
                       size_t ws_bytes, void* stream) {
  if (!x || !argmax_out || !accepted_out || !ws) return W12_ERR_NULL;
  w12_status st = check_desc(d, true);
  if (st != W12_OK) return st;
  if (m < 1 || m > W12_MAX_M) return W12_ERR_RANGE;
  if (!mn_ok(m, d->n)) return W12_ERR_SHAPE;
  const VerifyLayout L = verify_layout(m, d->n);
  if (ws_bytes < L.total) return W12_ERR_WORKSPACE;
  if (!aligned(x, 16) || !aligned(ws, 256) || !aligned(argmax_out, 4) || !aligned(accepted_out, 4))
    return W12_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* base = (uint8_t*)ws;
  GemmPlan p = make_plan(m, d->n, d->k, EPI_LOGITS);
  if (blocks_per_group(p) > kMaxBpg) return W12_ERR_HIP;   // (no plan asks for more)
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.p.seg[0] = w12_seg(d, nullptr, 0);
  fill_params(a.p, m, d->k, d->n, 1);
  a.logits = nullptr;          // pass 2 works from the block records and the tiles
  a.sabs = nullptr;
  a.bm = block_max(base, L, p);
  a.bm.accepted = accepted_out;   // pass 1 sets the draft lengths, pass 2 lowers them
  a.bm.n_draft = n_draft;
  a.bm.req_off = req_off;
  a.bm.req_ndraft = req_ndraft;
  a.bm.n_req = n_req;
  const int src = codebook_is_run(d->codebook) ? SRC_RUN : SRC_LUT;
  hipError_t e = launch_gemm(a, src, EPI_LOGITS, p, s);
  VerifyArgs v;
  memset(&v, 0, sizeof(v));
  v.x = x;
  v.tiles = (const uint8_t*)d->tiles;
  v.esc_off = d->esc_off;
  v.esc = d->esc;
  v.rbmax_v = a.bm.v;
  v.rbmax_v2 = a.bm.v2;
  v.rbmax_s = a.bm.s;
  v.rbmax_i = a.bm.i;
  v.grp_v = a.bm.gv;
  v.grp_v2 = a.bm.gv2;
  v.grp_i = a.bm.gi;
  v.grp_s = a.bm.gs;
  v.grp_w = a.bm.gw;
  v.ngrp = a.bm.ngrp;
  v.bpg = blocks_per_group(p);
  v.cand = (int32_t*)(base + L.cand);
  v.ncand = (int32_t*)(base + L.ncand);
  v.argmax = argmax_out;
  v.draft = draft;
  v.accepted = accepted_out;
  v.m = m;
  v.n = a.p.n;
  v.k = a.p.k;
  v.g_cols = a.p.g_cols;
  v.nb = a.p.nb;
  v.n_draft = n_draft;
  v.req_off = req_off;
  v.req_ndraft = req_ndraft;
  v.n_req = n_req;
  v.e_max = d->e_max;
  for (int i = 0; i < 4; ++i) v.lut[i] = a.p.seg[0].lut[i];
  if (e == hipSuccess) e = launch_verify_pass2(v, s);
  return hip_status(e);
}

// Screen copy of a head: tiles, then C [n], then A [n] (each from a 256-byte boundary).
struct ScreenLayout {
  size_t coef, abse, total;
};

ScreenLayout screen_layout(uint64_t n, uint64_t k) {
  ScreenLayout L;
  L.coef = align256((size_t)(n / 16) * (k / 128) * kScreenTileBytes);
  L.abse = L.coef + align256((size_t)n * 4);
  L.total = L.abse + align256((size_t)n * 4);
  return L;
}

// Two-level verification workspace: the row tickets (a fixed 4 KB region at the start,
// zero before the first use, left zero by every call), diagnostic counts, the first
// pass's block and group records, each slice's candidates with their FP64 values, and
// each row's survivors.  A slice holds at most 16 rows of each block of its groups.
struct Verify2Layout {
  size_t ncand, hi1, hi2, idx, gh, gl, sc_cnt, sc_lo, sc_v, sc_z, sc_b, surv, total;
  uint32_t ngrp, cap, slices;
};

Verify2Layout verify2_layout(uint32_t m, uint64_t n) {
  Verify2Layout L;
  const uint64_t nb = n / 16;
  L.ngrp = (uint32_t)((nb + kScreenNW - 1) / kScreenNW);
  L.slices = screen_slices(m);
  L.cap = 16u * kScreenNW * ((L.ngrp + L.slices - 1) / L.slices);
  const size_t rec = align256((size_t)m * nb * 4), grec = align256((size_t)m * L.ngrp * 4);
  const size_t sl = (size_t)m * L.slices, ent = sl * L.cap;
  L.ncand = kTicketBytes;
  L.hi1 = L.ncand + align256((size_t)m * 8);
  L.hi2 = L.hi1 + rec;
  L.idx = L.hi2 + rec;
  L.gh = L.idx + rec;
  L.gl = L.gh + grec;
  L.sc_cnt = L.gl + grec;
  L.sc_lo = L.sc_cnt + align256(sl * 4);
  L.sc_v = L.sc_lo + align256(sl * 8);
  L.sc_z = L.sc_v + align256(ent * 4);
  L.sc_b = L.sc_z + align256(ent * 8);
  L.surv = L.sc_b + align256(ent * 8);
  L.total = L.surv + align256((size_t)m * n * 4);
  return L;
}

// Two-level verification (pass 1 only when full_z is set: the screen logits and bounds).
w12_status verify2_impl(const uint16_t* x, uint32_t m, const w12_desc* d, const void* screen,
                        const int32_t* draft, uint32_t n_draft, const int32_t* req_off,
                        const int32_t* req_ndraft, uint32_t n_req, int32_t* argmax_out,
                        int32_t* accepted_out, void* ws, size_t ws_bytes, void* stream,
                        float* full_z, float* full_b) {
  if (!x || !screen || !ws) return W12_ERR_NULL;
  if (!full_z && (!argmax_out || !accepted_out)) return W12_ERR_NULL;
  w12_status st = check_desc(d, !full_z);
  if (st != W12_OK) return st;
  if (m < 1 || m > W12_MAX_M) return W12_ERR_RANGE;
  if (!mn_ok(m, d->n)) return W12_ERR_SHAPE;
  const Verify2Layout L = verify2_layout(m, d->n);
  if (ws_bytes < L.total) return W12_ERR_WORKSPACE;
  if (!aligned(x, 16) || !aligned(ws, 256) || !aligned(screen, 256)) return W12_ERR_ALIGN;
  if (full_z && (!aligned(full_z, 16) || !aligned(full_b, 16))) return W12_ERR_ALIGN;
  if (!full_z && (!aligned(argmax_out, 4) || !aligned(accepted_out, 4))) return W12_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* base = (uint8_t*)ws;
  const ScreenLayout SL = screen_layout(d->n, d->k);
  ScreenArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.tiles = (const uint8_t*)screen;
  a.coef = (const float*)((const uint8_t*)screen + SL.coef);
  a.abse = (const float*)((const uint8_t*)screen + SL.abse);
  a.hi1 = (float*)(base + L.hi1);
  a.hi2 = (float*)(base + L.hi2);
  a.idx = (int32_t*)(base + L.idx);
  a.gh = (float*)(base + L.gh);
  a.gl = (float*)(base + L.gl);
  a.full_z = full_z;
  a.full_b = full_b;
  if (!full_z) {
    a.acc.accepted = accepted_out;   // pass 1 sets the draft lengths, pass 2 lowers them
    a.acc.n_draft = n_draft;
    a.acc.req_off = req_off;
    a.acc.req_ndraft = req_ndraft;
    a.acc.n_req = n_req;
  }
  a.m = m;
  a.n = (uint32_t)d->n;
  a.k = (uint32_t)d->k;
  a.nb = (uint32_t)(d->n / 16);
  a.g_cols = (uint32_t)(d->k / 128);
  a.ngrp = L.ngrp;
  hipError_t e = launch_screen_pass1(a, s);
  if (full_z || e != hipSuccess) return hip_status(e);
  SelectArgs v;
  memset(&v, 0, sizeof(v));
  v.x = x;
  v.tiles = (const uint8_t*)d->tiles;
  v.esc_off = d->esc_off;
  v.esc = d->esc;
  v.hi1 = a.hi1;
  v.hi2 = a.hi2;
  v.idx = a.idx;
  v.gh = a.gh;
  v.gl = a.gl;
  v.tickets = (uint32_t*)base;
  v.sc_cnt = (int32_t*)(base + L.sc_cnt);
  v.sc_lo = (double*)(base + L.sc_lo);
  v.sc_v = (int32_t*)(base + L.sc_v);
  v.sc_z = (double*)(base + L.sc_z);
  v.sc_b = (double*)(base + L.sc_b);
  v.surv = (int32_t*)(base + L.surv);
  v.cap = L.cap;
  v.slices = L.slices;
  v.argmax = argmax_out;
  v.ncand = (int32_t*)(base + L.ncand);
  v.draft = draft;
  v.accepted = accepted_out;
  v.req_off = req_off;
  v.req_ndraft = req_ndraft;
  v.n_req = n_req;
  v.m = m;
  v.n = a.n;
  v.k = a.k;
  v.g_cols = a.g_cols;
  v.nb = a.nb;
  v.ngrp = L.ngrp;
  v.bpg = kScreenNW;
  v.n_draft = n_draft;
  const Seg sg = w12_seg(d, nullptr, 0);
  for (int i = 0; i < 4; ++i) v.lut[i] = sg.lut[i];
  return hip_status(launch_screen_pass2(v, s));
}

}  // namespace

extern "C" {

size_t w12_tiles_bytes(uint64_t n, uint64_t k) {
  if (!shape_ok(n, k)) return 0;
  return (size_t)(n / 16) * (k / 128) * 3072u;
}

size_t w12_workspace_bytes(int op, uint32_t m, uint64_t n, uint64_t k) {
  if (!shape_ok(n, k)) return 0;
  switch (op) {
    case W12_OP_ENCODE: return encode_layout(n, k).bytes;
    case W12_OP_DECODE: return 0;
    case W12_OP_GEMM:
    case W12_OP_GEMM_BF16:
    case W12_OP_GEMM_F8:   // (FP8 tiles are planned as W12 tiles)
      if (m < 1 || m > W12_MAX_M || !mn_ok(m, n)) return 0;
      return gemm_ws_bytes(m, n, k, op == W12_OP_GEMM_BF16);
    case W12_OP_VERIFY:
      if (m < 1 || m > W12_MAX_M || !mn_ok(m, n)) return 0;
      return verify_layout(m, n).total;
    case W12_OP_GEMM_GROUP:
      if (m < 1 || m > W12_MAX_M || !mn_ok(m, n)) return 0;
      return group_ws_bytes(m, n, k);
    case W12_OP_VERIFY2:
      if (m < 1 || m > W12_MAX_M || !mn_ok(m, n)) return 0;
      return verify2_layout(m, n).total;
    default: return 0;
  }
}

w12_status w12_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (ws_bytes == 0) return W12_OK;
  if (!ws) return W12_ERR_NULL;
  if (!aligned(ws, 16)) return W12_ERR_ALIGN;
  return hip_status(launch_fill_zero(ws, ws_bytes, (hipStream_t)stream));
}

w12_status w12_encode_count(const uint16_t* w, uint64_t n, uint64_t k, uint8_t codebook_out[16],
                            uint8_t* e_max_out, uint64_t* n_esc_out, void* ws, size_t ws_bytes,
                            void* stream) {
  if (!w || !codebook_out || !e_max_out || !n_esc_out || !ws) return W12_ERR_NULL;
  if (!shape_ok(n, k)) return W12_ERR_SHAPE;
  if (ws_bytes < encode_layout(n, k).bytes) return W12_ERR_WORKSPACE;
  if (!aligned(w, 16) || !aligned(ws, 256)) return W12_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  const EncodeLayout L = encode_layout(n, k);
  uint8_t* base = (uint8_t*)ws;
  hipError_t e = launch_fill_zero(base, 4096, s);
  if (e == hipSuccess) e = launch_encode_hist(w, n * k, (unsigned long long*)(base + L.hist), s);
  if (e == hipSuccess) e = launch_encode_codebook((const unsigned long long*)(base + L.hist), base + L.result, s);
  uint8_t res[64];
  if (e == hipSuccess) e = hipMemcpyAsync(res, base + L.result, 64, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return W12_ERR_HIP;
  memcpy(codebook_out, res, 16);
  *e_max_out = res[16];
  uint64_t ne;
  memcpy(&ne, res + 24, 8);
  *n_esc_out = ne;
  return W12_OK;
}

w12_status w12_encode(const uint16_t* w, const w12_desc* d, void* ws, size_t ws_bytes,
                      void* stream) {
  if (!w || !ws) return W12_ERR_NULL;
  w12_status st = check_desc(d, true);
  if (st != W12_OK) return st;
  const EncodeLayout L = encode_layout(d->n, d->k);
  if (ws_bytes < L.bytes) return W12_ERR_WORKSPACE;
  if (!aligned(w, 16) || !aligned(ws, 256)) return W12_ERR_ALIGN;
  hipStream_t s = (hipStream_t)stream;
  uint8_t* base = (uint8_t*)ws;
  const uint32_t nb = (uint32_t)(d->n / 16), g = (uint32_t)(d->k / 128);
  Mask256 mask;
  memset(&mask, 0, sizeof(mask));
  Codebook16 cb;
  for (int i = 0; i < 16; ++i) {
    cb.c[i] = d->codebook[i];
    mask.m[d->codebook[i] >> 5] |= 1u << (d->codebook[i] & 31);
  }
  uint32_t* tile_cnt = (uint32_t*)(base + L.tile_cnt);
  uint32_t* tile_off = (uint32_t*)(base + L.tile_off);
  hipError_t e = launch_encode_count_tiles(w, nb, g, mask, tile_cnt, s);
  if (e == hipSuccess)
    e = launch_encode_scan(tile_cnt, nb * g, g, tile_off, d->esc_off, (uint32_t)d->n_esc,
                           (uint32_t*)(base + L.total), s);
  if (e == hipSuccess)
    e = launch_encode_pack(w, nb, g, cb, tile_off, (uint8_t*)d->tiles, d->esc, d->n_esc, s);
  return hip_status(e);
}

w12_status w12_decode(const w12_desc* d, uint16_t* w_out, void* stream) {
  if (!w_out) return W12_ERR_NULL;
  w12_status st = check_desc(d, true);
  if (st != W12_OK) return st;
  if (!aligned(w_out, 16)) return W12_ERR_ALIGN;
  Codebook16 cb;
  for (int i = 0; i < 16; ++i) cb.c[i] = d->codebook[i];
  return hip_status(launch_decode((const uint8_t*)d->tiles, d->esc_off, d->esc,
                                  (uint32_t)(d->n / 16), (uint32_t)(d->k / 128), cb, w_out,
                                  (hipStream_t)stream));
}

w12_status w12_gemm(const uint16_t* x, uint32_t m, const w12_desc* d, uint16_t* y, void* ws,
                    size_t ws_bytes, void* stream) {
  return gemm_impl(x, m, d, y, ws, ws_bytes, stream, false);
}

w12_status w12_gemm_rms(const uint16_t* x, uint32_t m, const w12_desc* d, uint16_t* y, void* ws,
                        size_t ws_bytes, void* stream) {
  return gemm_impl(x, m, d, y, ws, ws_bytes, stream, true);
}

w12_status w12_gemm_group(const uint16_t* x, uint32_t m, const w12_desc* const* descs,
                          uint32_t n_w, uint16_t* const* ys, void* ws, size_t ws_bytes,
                          void* stream) {
  return gemm_group_impl(x, m, descs, n_w, ys, ws, ws_bytes, stream, false);
}

w12_status w12_gemm_group_rms(const uint16_t* x, uint32_t m, const w12_desc* const* descs,
                              uint32_t n_w, uint16_t* const* ys, void* ws, size_t ws_bytes,
                              void* stream) {
  return gemm_group_impl(x, m, descs, n_w, ys, ws, ws_bytes, stream, true);
}

w12_status w12_gemm_bf16(const uint16_t* x, uint32_t m, const uint16_t* w, uint64_t n,
                         uint64_t k, uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !w || !y) return W12_ERR_NULL;
  if (!shape_ok(n, k)) return W12_ERR_SHAPE;
  if (m < 1 || m > W12_MAX_M) return W12_ERR_RANGE;
  if (!mn_ok(m, n)) return W12_ERR_SHAPE;
  const size_t need = gemm_ws_bytes(m, n, k, true);
  if (ws_bytes < need) return W12_ERR_WORKSPACE;
  if (need > 0 && !ws) return W12_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16) || !aligned(ws, 256)) return W12_ERR_ALIGN;
  const GemmPlan p = make_plan(m, n, k, EPI_BF16, true);
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.p.seg[0].w = (const uint8_t*)w;
  a.p.seg[0].y = y;
  a.p.seg[0].n = (uint32_t)n;
  fill_params(a.p, m, k, n, 1);
  if (!set_split_ws(a, ws, p, m, n)) return W12_ERR_HIP;
  return hip_status(launch_gemm(a, SRC_BF16, EPI_BF16, p, (hipStream_t)stream));
}

w12_status w12_bf16_tile(const uint16_t* w, uint64_t n, uint64_t k, void* w_tiled, void* stream) {
  if (!w || !w_tiled) return W12_ERR_NULL;
  if (!shape_ok(n, k)) return W12_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(w_tiled, 16)) return W12_ERR_ALIGN;
  return hip_status(launch_bf16_tile(w, (uint32_t)(n / 16), (uint32_t)(k / 128),
                                     (uint8_t*)w_tiled, (hipStream_t)stream));
}

w12_status w12_gemm_bf16_tiled(const uint16_t* x, uint32_t m, const void* w_tiled, uint64_t n,
                               uint64_t k, uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !w_tiled || !y) return W12_ERR_NULL;
  if (!shape_ok(n, k)) return W12_ERR_SHAPE;
  if (m < 1 || m > W12_MAX_M) return W12_ERR_RANGE;
  if (!mn_ok(m, n)) return W12_ERR_SHAPE;
  const size_t need = gemm_ws_bytes(m, n, k, true);
  if (ws_bytes < need) return W12_ERR_WORKSPACE;
  if (need > 0 && !ws) return W12_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_tiled, 16) || !aligned(y, 16) || !aligned(ws, 256)) return W12_ERR_ALIGN;
  const GemmPlan p = make_plan(m, n, k, EPI_BF16, true);
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.p.seg[0].w = (const uint8_t*)w_tiled;
  a.p.seg[0].y = y;
  a.p.seg[0].n = (uint32_t)n;
  fill_params(a.p, m, k, n, 1);
  if (!set_split_ws(a, ws, p, m, n)) return W12_ERR_HIP;
  return hip_status(launch_gemm(a, SRC_BF16T, EPI_BF16, p, (hipStream_t)stream));
}

w12_status w12_f8_tile(const uint8_t* w, uint64_t n, uint64_t k, void* w_tiled, void* stream) {
  if (!w || !w_tiled) return W12_ERR_NULL;
  if (!shape_ok(n, k)) return W12_ERR_SHAPE;
  if (!aligned(w, 16) || !aligned(w_tiled, 16)) return W12_ERR_ALIGN;
  return hip_status(launch_f8_tile(w, (uint32_t)(n / 16), (uint32_t)(k / 128), (uint8_t*)w_tiled,
                                   (hipStream_t)stream));
}

}  // extern "C"

namespace {

w12_status gemm_f8_impl(const uint16_t* x, uint32_t m, const void* w_tiled, const float* scale,
                        uint64_t n, uint64_t k, uint16_t* y, void* ws, size_t ws_bytes,
                        void* stream, bool rms) {
  if (!x || !w_tiled || !scale || !y) return W12_ERR_NULL;
  if (!shape_ok(n, k)) return W12_ERR_SHAPE;
  if (m < 1 || m > W12_MAX_M) return W12_ERR_RANGE;
  if (!mn_ok(m, n)) return W12_ERR_SHAPE;
  const size_t need = gemm_ws_bytes(m, n, k, false);
  if (ws_bytes < need) return W12_ERR_WORKSPACE;
  if (need > 0 && !ws) return W12_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_tiled, 16) || !aligned(scale, 4) || !aligned(y, 16) ||
      !aligned(ws, 256))
    return W12_ERR_ALIGN;
  const GemmPlan p = make_plan(m, n, k, EPI_BF16, false);
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.p.seg[0].w = (const uint8_t*)w_tiled;
  a.p.seg[0].scale = scale;
  a.p.seg[0].y = y;
  a.p.seg[0].n = (uint32_t)n;
  fill_params(a.p, m, k, n, 1);
  a.p.rms = rms ? 1u : 0u;
  if (!set_split_ws(a, ws, p, m, n)) return W12_ERR_HIP;
  return hip_status(launch_gemm(a, SRC_F8, EPI_BF16, p, (hipStream_t)stream));
}

w12_status gemm_f8_group_impl(const uint16_t* x, uint32_t m, const void* const* w_tiled,
                              const float* const* scales, const uint64_t* ns, uint32_t n_w,
                              uint64_t k, uint16_t* const* ys, void* ws, size_t ws_bytes,
                              void* stream, bool rms) {
  if (!x || !w_tiled || !scales || !ns || !ys) return W12_ERR_NULL;
  if (n_w < 1 || n_w > W12_MAX_GROUP || m < 1 || m > W12_MAX_M) return W12_ERR_RANGE;
  uint64_t n_total = 0;
  for (uint32_t i = 0; i < n_w; ++i) {
    if (!w_tiled[i] || !scales[i] || !ys[i]) return W12_ERR_NULL;
    if (!shape_ok(ns[i], k)) return W12_ERR_SHAPE;
    if (!aligned(w_tiled[i], 16) || !aligned(scales[i], 4) || !aligned(ys[i], 16))
      return W12_ERR_ALIGN;
    n_total += ns[i];
  }
  if (n_total >= kMaxN || !mn_ok(m, n_total)) return W12_ERR_SHAPE;
  const size_t need = group_ws_bytes(m, n_total, k);
  if (ws_bytes < need) return W12_ERR_WORKSPACE;
  if (need > 0 && !ws) return W12_ERR_NULL;
  if (!aligned(x, 16) || !aligned(ws, 256)) return W12_ERR_ALIGN;
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  n_total = 0;
  for (uint32_t i = 0; i < n_w; ++i) {
    a.p.seg[i].w = (const uint8_t*)w_tiled[i];
    a.p.seg[i].scale = scales[i];
    a.p.seg[i].y = ys[i];
    a.p.seg[i].n = (uint32_t)ns[i];
    a.p.seg[i].rb0 = (uint32_t)(n_total / 16);
    n_total += ns[i];
  }
  fill_params(a.p, m, k, n_total, n_w);
  a.p.rms = rms ? 1u : 0u;
  const GemmPlan p = make_plan(m, n_total, k, EPI_BF16, false);
  if (!set_split_ws(a, ws, p, m, n_total)) return W12_ERR_HIP;
  return hip_status(launch_gemm(a, SRC_F8, EPI_BF16, p, (hipStream_t)stream));
}

}  // namespace

extern "C" {

w12_status w12_gemm_f8(const uint16_t* x, uint32_t m, const void* w_tiled, const float* scale,
                       uint64_t n, uint64_t k, uint16_t* y, void* ws, size_t ws_bytes,
                       void* stream) {
  return gemm_f8_impl(x, m, w_tiled, scale, n, k, y, ws, ws_bytes, stream, false);
}

w12_status w12_gemm_f8_rms(const uint16_t* x, uint32_t m, const void* w_tiled, const float* scale,
                           uint64_t n, uint64_t k, uint16_t* y, void* ws, size_t ws_bytes,
                           void* stream) {
  return gemm_f8_impl(x, m, w_tiled, scale, n, k, y, ws, ws_bytes, stream, true);
}

w12_status w12_gemm_f8_group(const uint16_t* x, uint32_t m, const void* const* w_tiled,
                             const float* const* scales, const uint64_t* ns, uint32_t n_w,
                             uint64_t k, uint16_t* const* ys, void* ws, size_t ws_bytes,
                             void* stream) {
  return gemm_f8_group_impl(x, m, w_tiled, scales, ns, n_w, k, ys, ws, ws_bytes, stream, false);
}

w12_status w12_gemm_f8_group_rms(const uint16_t* x, uint32_t m, const void* const* w_tiled,
                                 const float* const* scales, const uint64_t* ns, uint32_t n_w,
                                 uint64_t k, uint16_t* const* ys, void* ws, size_t ws_bytes,
                                 void* stream) {
  return gemm_f8_group_impl(x, m, w_tiled, scales, ns, n_w, k, ys, ws, ws_bytes, stream, true);
}

w12_status w12_lmhead_verify(const uint16_t* x, uint32_t m, const w12_desc* d, const int32_t* draft,
                             uint32_t n_draft, int32_t* argmax_out, int32_t* accepted_out,
                             void* ws, size_t ws_bytes, void* stream) {
  if (n_draft > 0 && !draft) return W12_ERR_NULL;
  if (m >= 1 && n_draft > m) return W12_ERR_RANGE;
  return verify_impl(x, m, d, draft, n_draft, nullptr, nullptr, 1, argmax_out, accepted_out,
                     ws, ws_bytes, stream);
}

w12_status w12_lmhead_verify_batched(const uint16_t* x, uint32_t m, const w12_desc* d,
                                     const int32_t* req_off, const int32_t* req_ndraft,
                                     uint32_t n_req, const int32_t* draft,
                                     int32_t* argmax_out, int32_t* accepted_out, void* ws,
                                     size_t ws_bytes, void* stream) {
  if (!req_off || !req_ndraft || !draft) return W12_ERR_NULL;
  if (n_req < 1 || n_req > m) return W12_ERR_RANGE;
  if (!aligned(req_off, 4) || !aligned(req_ndraft, 4) || !aligned(draft, 4)) return W12_ERR_ALIGN;
  return verify_impl(x, m, d, draft, 0, req_off, req_ndraft, n_req, argmax_out, accepted_out,
                     ws, ws_bytes, stream);
}

w12_status w12_logits_f32(const uint16_t* x, uint32_t m, const w12_desc* d, float* logits_out,
                          float* sabs_out, void* ws, size_t ws_bytes, void* stream) {
  if (!x || !logits_out || !sabs_out || !ws) return W12_ERR_NULL;
  w12_status st = check_desc(d, true);
  if (st != W12_OK) return st;
  if (m < 1 || m > W12_MAX_M) return W12_ERR_RANGE;
  if (!mn_ok(m, d->n)) return W12_ERR_SHAPE;
  const VerifyLayout L = verify_layout(m, d->n);
  if (ws_bytes < L.total) return W12_ERR_WORKSPACE;
  if (!aligned(x, 16) || !aligned(ws, 256) || !aligned(logits_out, 16) || !aligned(sabs_out, 16))
    return W12_ERR_ALIGN;
  uint8_t* base = (uint8_t*)ws;
  GemmPlan p = make_plan(m, d->n, d->k, EPI_LOGITS);
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.p.seg[0] = w12_seg(d, nullptr, 0);
  fill_params(a.p, m, d->k, d->n, 1);
  a.logits = logits_out;
  a.sabs = sabs_out;   // the row norms first, then scaled by each row's bound of ||x||_2
  a.bm = block_max(base, L, p);
  const int src = codebook_is_run(d->codebook) ? SRC_RUN : SRC_LUT;
  hipError_t e = launch_gemm(a, src, EPI_LOGITS, p, (hipStream_t)stream);
  if (e == hipSuccess) e = launch_scale_norms(x, m, d->k, sabs_out, (uint32_t)d->n, (hipStream_t)stream);
  return hip_status(e);
}

size_t w12_screen_bytes(uint64_t n, uint64_t k) {
  if (!shape_ok(n, k)) return 0;
  return screen_layout(n, k).total;
}

w12_status w12_screen_encode(const uint16_t* w, uint64_t n, uint64_t k, void* screen,
                             size_t screen_bytes, void* stream) {
  if (!w || !screen) return W12_ERR_NULL;
  if (!shape_ok(n, k)) return W12_ERR_SHAPE;
  const ScreenLayout L = screen_layout(n, k);
  if (screen_bytes < L.total) return W12_ERR_WORKSPACE;
  if (!aligned(w, 16) || !aligned(screen, 256)) return W12_ERR_ALIGN;
  uint8_t* base = (uint8_t*)screen;
  return hip_status(launch_screen_encode(w, (uint32_t)(n / 16), (uint32_t)(k / 128), base,
                                         (float*)(base + L.coef), (float*)(base + L.abse),
                                         (hipStream_t)stream));
}

w12_status w12_lmhead_verify2(const uint16_t* x, uint32_t m, const w12_desc* d,
                              const void* screen, const int32_t* draft, uint32_t n_draft,
                              int32_t* argmax_out, int32_t* accepted_out, void* ws,
                              size_t ws_bytes, void* stream) {
  if (n_draft > 0 && !draft) return W12_ERR_NULL;
  if (m >= 1 && n_draft > m) return W12_ERR_RANGE;
  return verify2_impl(x, m, d, screen, draft, n_draft, nullptr, nullptr, 1, argmax_out,
                      accepted_out, ws, ws_bytes, stream, nullptr, nullptr);
}

w12_status w12_lmhead_verify2_batched(const uint16_t* x, uint32_t m, const w12_desc* d,
                                      const void* screen, const int32_t* req_off,
                                      const int32_t* req_ndraft, uint32_t n_req,
                                      const int32_t* draft, int32_t* argmax_out,
                                      int32_t* accepted_out, void* ws, size_t ws_bytes,
                                      void* stream) {
  if (!req_off || !req_ndraft || !draft) return W12_ERR_NULL;
  if (n_req < 1 || n_req > m) return W12_ERR_RANGE;
  if (!aligned(req_off, 4) || !aligned(req_ndraft, 4) || !aligned(draft, 4)) return W12_ERR_ALIGN;
  return verify2_impl(x, m, d, screen, draft, 0, req_off, req_ndraft, n_req, argmax_out,
                      accepted_out, ws, ws_bytes, stream, nullptr, nullptr);
}

w12_status w12_screen_logits_f32(const uint16_t* x, uint32_t m, const w12_desc* d,
                                 const void* screen, float* logits_out, float* bound_out,
                                 void* ws, size_t ws_bytes, void* stream) {
  if (!logits_out || !bound_out) return W12_ERR_NULL;
  return verify2_impl(x, m, d, screen, nullptr, 0, nullptr, nullptr, 0, nullptr, nullptr, ws,
                      ws_bytes, stream, logits_out, bound_out);
}

w12_status w12_rms_rescale(const uint16_t* x, uint32_t m, uint64_t k, uint16_t* y, void* stream) {
  if (!x || !y) return W12_ERR_NULL;
  if (m < 1 || m > (1u << 20)) return W12_ERR_RANGE;
  if (k == 0 || k >= kMaxK || k % 8) return W12_ERR_SHAPE;
  if (!aligned(x, 16) || !aligned(y, 16)) return W12_ERR_ALIGN;
  return hip_status(launch_rms_rescale(x, m, (uint32_t)k, y, (hipStream_t)stream));
}

w12_status w12_stream_read(const void* buf, uint64_t bytes, uint32_t workgroups, uint32_t* sink,
                           void* stream) {
  if (!buf || !sink) return W12_ERR_NULL;
  if (bytes == 0 || bytes % 16 || bytes >= (1ull << 32)) return W12_ERR_SHAPE;
  if (workgroups < 1 || workgroups > 65536) return W12_ERR_RANGE;
  if (!aligned(buf, 16) || !aligned(sink, 4)) return W12_ERR_ALIGN;
  return hip_status(launch_stream_read(buf, (uint32_t)bytes, workgroups, sink, (hipStream_t)stream));
}

const char* w12_status_str(w12_status s) {
  switch (s) {
    case W12_OK: return "ok";
    case W12_ERR_NULL: return "null pointer";
    case W12_ERR_SHAPE: return "bad shape (n % 16, k % 128, 0 < k < 2^20)";
    case W12_ERR_RANGE: return "value out of range (m in 1..128, n_draft <= m, n_req in 1..m)";
    case W12_ERR_FORMAT: return "bad W12 descriptor (codebook not ascending, e_max, n_esc)";
    case W12_ERR_WORKSPACE: return "workspace too small";
    case W12_ERR_HIP: return "HIP runtime error";
    case W12_ERR_ALIGN: return "misaligned pointer";
    default: return "unknown status";
  }
}

uint32_t w12_version(void) { return 0x000100u; }

}  // extern "C"
