// Internal definitions shared by the host layer and the kernels of libw12.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

// m from which the MFMA path runs; below it the VALU v_dot2 path.  Measured on the MLP
// shapes: from m = 4 the VALU path is VALU-issue-bound and the MFMA path (x zero-padded
// to 16 rows) is faster.
struct w12_desc;   // the C ABI's weight descriptor (w12.h)

#ifndef W12_MFMA_MIN_M
#define W12_MFMA_MIN_M 4
#endif

namespace w12 {

// Weight source of the GEMM kernel family.
enum Src : int {
  SRC_RUN = 0,   // W12 tiles, codebook is a run C[j] = C[0] + j (exponent = base + code)
  SRC_LUT = 1,   // W12 tiles, arbitrary ascending codebook (16-entry byte LUT)
  SRC_BF16 = 2,  // plain BF16 rows [n][k]
  SRC_BF16T = 3, // plain BF16 in 4 KB tiles (the layout of w12_bf16_tile)
  SRC_F8 = 4,    // FP8 E4M3 in 2 KB tiles with one FP32 scale per 128 x 128 block (w12_f8_tile)
};

// Epilogue of the GEMM kernel family.
enum Epi : int {
  EPI_BF16 = 0,    // y = bf16(x . W^T)
  EPI_LOGITS = 1,  // per-row-block maxima (+ fp32 logits [m][n] when asked for): verification pass 1
  EPI_RMS = 2,     // y = bf16((x . W^T) / rms(x)) per row (GemmParams.rms launches, W12 sources)
};

// One weight of a launch.  A launch multiplies one x by up to kMaxSeg weights that
// share K (a group), their row-blocks numbered consecutively; a single GEMM is a group
// of one.
constexpr int kMaxSeg = 4;
// Most K splits a launch takes (the completing split keeps one partial per split in registers).
constexpr uint32_t kMaxSplit = 8;
// Most row-blocks in one group record of verification pass 1 (its workgroup's row-blocks).
constexpr uint32_t kMaxBpg = 8;
struct Seg {
  const uint8_t* w;         // W12 tiles, or BF16 rows [n][k]
  const uint32_t* esc_off;  // [n/16 + 1] (W12)
  const uint32_t* esc;      // [n_esc] (W12)
  uint16_t* y;              // [m][n] BF16 (EPI_BF16)
  uint32_t rb0;             // first row-block of this weight in the launch
  uint32_t n;               // rows of this weight
  uint32_t basepair;        // SRC_RUN: C[0] | C[0] << 16
  uint32_t lut[4];          // SRC_LUT: codebook bytes C[0..15]
  const float* scale;       // SRC_F8: block scales [ceil(n/128)][k/128]
};

// Scalar parameters of one launch (a kernel argument).
struct GemmParams {
  uint32_t m, k, g_cols;
  uint32_t nb, n;           // row-blocks and rows of all the launch's weights together
  uint32_t nseg;
  // RMS launches (rms = 1): y = (x . W^T) / sqrt(mean_k x^2) per row; when K is split,
  // each workgroup leaves its split's sum of x^2 per row in ss[group][split][m]
  uint32_t rms;
  float* ss;
  // K split: one ticket per row-block group (zero before the launch, zero after it)
  uint32_t* tickets;
  Seg seg[kMaxSeg];
};

// Depth of the certified bound on an FP32 logit of verification pass 1 (derivation in
// w12_verify.hip): the logits kernels sum each 128-column tile column from zero, 4 MFMAs
// or 16 v_dot2 in a chain, then add it to the running sum.  Whatever order the hardware
// adds inside one instruction (not documented), a value entering an MFMA meets at most
// 32 roundings in it and one entering a v_dot2 at most 2, so a product meets at most 128
// within its column, then one addition per column (K/128 of them), then at most 64 in
// the cross-lane and cross-wave sums: D = K/128 + 192.
__host__ __device__ inline double bound_depth(uint32_t k) { return (double)(k / 128u) + 192.0; }

// Slope of that bound, B(S) = c1 S + c0: g = D 2^-23 / (1 - D 2^-23), c1 = g / (1 - g),
// inflated by 2^-20 for its FP64 evaluation.
__host__ __device__ inline double bound_slope(uint32_t k) {
  const double dd = bound_depth(k);
  const double gam = dd * 0x1p-23 / (1.0 - dd * 0x1p-23);
  return gam / (1.0 - gam) * (1.0 + 0x1p-20);
}

// Smallest FP32 value >= d (finite or infinite d).
__device__ inline float f32_round_up(double d) {
  float f = (float)d;
  if ((double)f < d) {
    uint32_t u = __float_as_uint(f);
    if (f == 0.0f) u = 1u;          // +-0 -> the smallest positive subnormal
    else if (f > 0.0f) u += 1u;
    else u -= 1u;
    f = __uint_as_float(u);
  }
  return f;
}

// FP32 upper bound of the 2-norm of K BF16 values from the FP32 sum of their squares in
// any order: a square is exact unless it falls below 2^-126, each term passes through at
// most D = K + 64 additions with relative error below 2^-23, and flushes below 2^-126
// (squares and partial sums, 2D of them) lose less than 2^-126 each.
__device__ inline float l2_norm_up(float sumsq, uint32_t k) {
  const double dd = (double)k + 64.0;
  const double gam = dd * 0x1p-23 / (1.0 - dd * 0x1p-23);
  const double t = ((double)sumsq + 2.0 * dd * 0x1p-126) * (1.0 + 2.0 * gam);
  return f32_round_up(sqrt(t) * (1.0 + 0x1p-50));
}

// FP64 upper bound of ||x||_2 from the FP64 sum of the exact squares of K < 2^20 BF16
// values in any order (relative error below K 2^-53 < 2^-33, and sqrt and the product
// add below 2^-52).
__device__ inline double x_norm_up(double sumsq) {
  return sqrt(sumsq * (1.0 + 0x1p-30)) * (1.0 + 0x1p-50);
}

// Per-row-block records of the logits epilogue (verification pass 1), [m][nb] each, and
// one record per workgroup ("group": its consecutive row-blocks), [m][ngrp] each.
struct BlockMax {
  float* v;                 // largest logit of the row-block (NaN if any is not finite)
  float* v2;                // second largest (equal to v on a tie)
  float* s;                 // largest FP32 upper bound of ||w_v||_2 over the row-block
  int32_t* i;               // index of v, lowest on ties
  float* gv;                // group: largest logit (NaN if any of its logits is not finite)
  int32_t* gi;              // group: index of gv, lowest on ties
  float* gv2;               // group: second largest logit over its rows (gv on a tie)
  float* gs;                // group: s of the row-block holding gv
  float* gw;                // group: largest s over its row-blocks
  uint32_t ngrp;            // groups per row (the grid's row-block groups)
  int32_t* accepted;        // [n_req]: set by the first workgroup (NULL: untouched)
  uint32_t n_draft;         // one request over all rows (req_off NULL): its draft length
  const int32_t* req_off;   // batched: request r owns rows req_off[r] .. req_off[r+1]-1
  const int32_t* req_ndraft;   // batched: draft tokens of request r
  uint32_t n_req;
};

// Request r of a batched verification: its first row lo and draft length nd; false for
// an entry outside 0 <= req_off[r] <= req_off[r+1] <= m, 0 <= nd <= its row count.
__device__ __forceinline__ bool req_entry(const int32_t* req_off, const int32_t* req_ndraft,
                                          uint32_t r, uint32_t m, int32_t& lo, int32_t& nd) {
  lo = req_off[r];
  const int32_t hi = req_off[r + 1];
  nd = req_ndraft[r];
  return lo >= 0 && lo <= hi && hi <= (int32_t)m && nd >= 0 && nd <= hi - lo;
}

// Starting value of each request's accepted length, written by verification pass 1:
// the draft length (lowered by pass 2 at the first mismatch), -1 for an invalid entry.
__device__ __forceinline__ void accept_init(const BlockMax& bm, uint32_t m, uint32_t tid,
                                            uint32_t nthreads) {
  for (uint32_t r = tid; r < bm.n_req; r += nthreads) {
    int32_t lo, nd;
    bm.accepted[r] = !bm.req_off ? (int32_t)bm.n_draft
                                 : (req_entry(bm.req_off, bm.req_ndraft, r, m, lo, nd) ? nd : -1);
  }
}

struct GemmArgs {
  const uint16_t* x;        // [m][k] BF16
  float* logits;            // [m][n] (EPI_LOGITS; NULL: not written)
  float* sabs;              // [m][n] with logits: the row norm bound W_v in every row
  BlockMax bm;              // EPI_LOGITS
  float* partial;           // [nsplit][m][n] split-K partial sums (launch numbering)
  GemmParams p;
};

// Kernel shapes of the GEMM family.
enum Kind : int {
  KIND_WAVE_COLUMNS = 0,    // k_gemm: each wave streams its own tile columns (VALU or MFMA)
  KIND_COLUMN_SYNC = 1,     // k_gemm_cs: a workgroup's waves share each x column (MFMA)
};

struct GemmPlan {
  int kind;                 // Kind
  bool mfma;                // KIND_WAVE_COLUMNS: MFMA (m >= W12_MFMA_MIN_M) or VALU
  int rbw;                  // KIND_WAVE_COLUMNS: row-blocks per wave (1 or 2)
  int nw;                   // KIND_COLUMN_SYNC: waves (= row-blocks) per workgroup (4 or 8)
  uint32_t nsplit;          // K splits across workgroups
  uint32_t n_rbg;           // row-block groups = ceil(nb / rbw)
};

// Launch one GEMM (kernel family chosen by m, src, epi and plan.rbw).
hipError_t launch_gemm_run(const GemmArgs& a, int epi, const GemmPlan& p, hipStream_t s);
hipError_t launch_gemm_lut(const GemmArgs& a, int epi, const GemmPlan& p, hipStream_t s);
hipError_t launch_gemm_bf16_src(const GemmArgs& a, int epi, const GemmPlan& p, hipStream_t s);
hipError_t launch_gemm_bf16t_src(const GemmArgs& a, int epi, const GemmPlan& p, hipStream_t s);
hipError_t launch_gemm_f8_src(const GemmArgs& a, int epi, const GemmPlan& p, hipStream_t s);
inline hipError_t launch_gemm(const GemmArgs& a, int src, int epi, const GemmPlan& p,
                              hipStream_t s) {
  if (src == SRC_RUN) return launch_gemm_run(a, epi, p, s);
  if (src == SRC_LUT) return launch_gemm_lut(a, epi, p, s);
  if (src == SRC_BF16T) return launch_gemm_bf16t_src(a, epi, p, s);
  if (src == SRC_F8) return launch_gemm_f8_src(a, epi, p, s);
  return launch_gemm_bf16_src(a, epi, p, s);
}

// Codec kernels.
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);
hipError_t launch_encode_hist(const uint16_t* w, uint64_t count, unsigned long long* hist,
                              hipStream_t s);
hipError_t launch_encode_codebook(const unsigned long long* hist, uint8_t* result,
                                  hipStream_t s);
struct Mask256 {
  uint32_t m[8];
};
struct Codebook16 {
  uint8_t c[16];
};
hipError_t launch_encode_count_tiles(const uint16_t* w, uint32_t nb, uint32_t g_cols,
                                     const Mask256& member, uint32_t* tile_cnt, hipStream_t s);
hipError_t launch_encode_scan(const uint32_t* tile_cnt, uint32_t n_tiles, uint32_t g_cols,
                              uint32_t* tile_off, uint32_t* esc_off, uint32_t esc_cap,
                              uint32_t* total, hipStream_t s);
hipError_t launch_encode_pack(const uint16_t* w, uint32_t nb, uint32_t g_cols,
                              const Codebook16& cb, const uint32_t* tile_off,
                              uint8_t* tiles, uint32_t* esc, uint64_t esc_cap,
                              hipStream_t s);
hipError_t launch_bf16_tile(const uint16_t* w, uint32_t nb, uint32_t g_cols, uint8_t* out,
                            hipStream_t s);
hipError_t launch_f8_tile(const uint8_t* w, uint32_t nb, uint32_t g_cols, uint8_t* out,
                          hipStream_t s);
hipError_t launch_decode(const uint8_t* tiles, const uint32_t* esc_off, const uint32_t* esc,
                         uint32_t nb, uint32_t g_cols, const Codebook16& cb,
                         uint16_t* w_out, hipStream_t s);

// Verification pass 2 (certified exact argmax) and accept.
struct VerifyArgs {
  const uint16_t* x;
  const uint8_t* tiles;
  const uint32_t* esc_off;
  const uint32_t* esc;
  const float* rbmax_v;     // [m][nb]
  const float* rbmax_v2;    // [m][nb]
  const float* rbmax_s;     // [m][nb]
  const int32_t* rbmax_i;   // [m][nb]
  const float* grp_v;       // [m][ngrp] group records of pass 1
  const float* grp_v2;
  const int32_t* grp_i;
  const float* grp_s;
  const float* grp_w;
  uint32_t ngrp, bpg;       // groups per row, row-blocks per group (<= kMaxBpg)
  int32_t* cand;            // [m][n] candidate logits
  int32_t* argmax;          // [m]
  int32_t* ncand;           // [m][2]: candidate logits, those left after the FP64 screen
                            // (diagnostic; may be NULL)
  const int32_t* draft;     // [m] (batched) or [n_draft]
  int32_t* accepted;        // [n_req]
  const int32_t* req_off;   // NULL: one request over rows 0..m-1 with n_draft tokens
  const int32_t* req_ndraft;
  uint32_t n_req;
  uint32_t m, n, k, g_cols, nb, n_draft;
  uint32_t e_max;
  uint32_t lut[4];
};
hipError_t launch_verify_pass2(const VerifyArgs& a, hipStream_t s);
// s [m][n]: row norms W_v in every row -> X_m W_v (the first pass's full output)
hipError_t launch_scale_norms(const uint16_t* x, uint32_t m, uint32_t k, float* s, uint32_t n,
                              hipStream_t st);

// Two-level verification (w12_screen.hip): the screen copy of the head (8-bit codes, a
// BF16 scale per 32 columns) and its two passes.
constexpr uint32_t kScreenTileBytes = 2176;   // 2048 code bytes + 64 BF16 scales
// Workgroups per x row in the second pass: more for few rows (each workgroup takes the
// candidates of its share of the row's groups), fewer when many rows fill the chip anyway.
#ifndef W12_SCREEN_SLICES
#define W12_SCREEN_SLICES 32u, 16u, 8u, 4u   // m <= 16, <= 32, <= 64, more
#endif
__host__ __device__ inline uint32_t screen_slices(uint32_t m) {
  constexpr uint32_t t[4] = {W12_SCREEN_SLICES};
  return m <= 16 ? t[0] : (m <= 32 ? t[1] : (m <= 64 ? t[2] : t[3]));
}
constexpr uint32_t kScreenNW = 8;             // row-blocks (waves) per first-pass workgroup

struct ScreenArgs {         // first pass: the screen GEMM with the interval epilogue
  const uint16_t* x;        // [m][k]
  const uint8_t* tiles;     // screen tiles
  const float* coef;        // C [n]
  const float* abse;        // A [n]
  float* hi1;               // [m][nb] largest upper end of the row-block's intervals
  float* hi2;               // [m][nb] second largest
  int32_t* idx;             // [m][nb] row of hi1 (lowest on ties)
  float* gh;                // [m][ngrp] largest hi1 of the group (workgroup)
  float* gl;                // [m][ngrp] largest lower end of the group's intervals
  float* full_z;            // [m][n] screen logits (NULL: not written)
  float* full_b;            // [m][n] their bounds
  BlockMax acc;             // accept fields only (accepted, n_draft, req_*)
  uint32_t m, n, k, nb, g_cols, ngrp;
};

struct SelectArgs {         // second pass: candidates, FP64 from W12, exact, accept
  const uint16_t* x;
  const uint8_t* tiles;     // the W12 head
  const uint32_t* esc_off;
  const uint32_t* esc;
  const float* hi1;
  const float* hi2;
  const int32_t* idx;
  const float* gh;
  const float* gl;
  uint32_t* tickets;        // [m]: zero before the launch, zero after it
  int32_t* sc_cnt;          // [m][slices] survivors kept by each slice
  double* sc_lo;            // [m][slices] largest FP64 lower bound of each slice
  int32_t* sc_v;            // [m][slices][cap]
  double* sc_z;             // [m][slices][cap]
  double* sc_b;             // [m][slices][cap]
  int32_t* surv;            // [m][n] survivors of the row (the last workgroup)
  uint32_t cap, slices;      // entries per slice, slices per row (screen_slices(m))
  int32_t* argmax;          // [m]
  int32_t* ncand;           // [m][2]: candidates after the screen, after FP64 (may be NULL)
  const int32_t* draft;
  int32_t* accepted;
  const int32_t* req_off;
  const int32_t* req_ndraft;
  uint32_t n_req;
  uint32_t m, n, k, g_cols, nb, ngrp, bpg, n_draft;
  uint32_t lut[4];
};

hipError_t launch_screen_encode(const uint16_t* w, uint32_t nb, uint32_t g_cols, uint8_t* tiles,
                                float* coef, float* abse, hipStream_t s);
hipError_t launch_screen_pass1(const ScreenArgs& a, hipStream_t s);
hipError_t launch_screen_pass2(const SelectArgs& a, hipStream_t s);

hipError_t launch_rms_rescale(const uint16_t* x, uint32_t m, uint32_t k, uint16_t* y,
                              hipStream_t s);
hipError_t launch_stream_read(const void* buf, uint32_t bytes, uint32_t workgroups, uint32_t* sink,
                              hipStream_t s);

// w12_gemm in two halves (host layer): argument checks with the workspace bytes the call
// needs, then the launch on a workspace of at least that size.
int32_t gemm_check(const uint16_t* x, uint32_t m, const ::w12_desc* d, const uint16_t* y,
                   size_t* need);
int32_t gemm_launch(const uint16_t* x, uint32_t m, const ::w12_desc* d, uint16_t* y, void* ws,
                    void* stream, bool rms);

}  // namespace w12
