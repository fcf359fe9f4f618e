/*
 * w12.h -- C ABI of libw12.so: the W12 lossless 12-bit weight format on MI355X
 * (gfx950): encode, bit-exact decode, the memory-bound decode/verification GEMM
 * (M = 1..32 rows of BF16 x against W12 weights, FP32 accumulate, BF16 out; up to 128
 * rows for several requests verified together), the greedy verification epilogue
 * (exact-logit argmax per row, accepted-prefix length per request), and the same GEMM
 * for the FP8 weights of FP8 targets (E4M3 codes with 128 x 128 block scales).
 *
 * Sources (pages cited by title and section):
 *  - "StargazerX0/SpecPilot" (hotrepo.ai), "What it is": W12 is a 12-bit weight
 *    format decoded bit-exactly inside the GEMM; decoding is greedy and the target
 *    model decides each token.  "Results and verification": every committed token
 *    must be the target's own choice.
 *  - "SpecPilot" (fasttoolhub glossary), "Differentiation": the format is a general,
 *    lossless 12-bit weight format.
 *  - "SpecPilot: an agent doubled speculative decoding speed, and the 10.87x needs
 *    context", "The mechanisms it found": about 12.01-12.02 bits per weight, decoded
 *    in GEMM registers, a quarter less weight traffic than BF16 in memory-bound
 *    decode, and a certified exact-argmax LM head; "The caveats the README states":
 *    reduction order can flip near-ties (hence argmax on exact logits); FP8 GEMM
 *    routing among the batching mechanisms, with the "What it is" section of the digest
 *    placing three batching settings on FP8 targets.
 *
 * W12 v1 layout (the pages fix only its properties; this is the layout defined here):
 *  - W is [n out][k in] BF16, row-major; n % 16 == 0, k % 128 == 0, 0 < k < 2^20.
 *  - Per-tensor codebook C[16]: the 16 exponent fields with the largest counts (ties
 *    to the smaller field), strictly ascending.  Element code = index of its exponent
 *    in C; an exponent outside C is an escape (code 0 stored, true exponent listed).
 *  - Tile (b, g) = rows 16b..16b+15 x columns 128g..128g+127, 3072 bytes at byte
 *    offset (g*(n/16) + b)*3072: column-major tile order, so the row-blocks' tiles of
 *    one column are adjacent.  Lane slot l = 0..63 (r = l%16, q = l/16) holds
 *    32 elements t = 0..31 (j = t/8, i = t%8) at column 128g + 32j + 8q + i of row
 *    16b + r.  Byte 1024*(t/16) + 16l + t%16 holds sm = (sign<<7) | mantissa; the
 *    little-endian u32 at 2048 + 16l + 4j holds the 8 codes of j, code of i at bit
 *    4*(i/2) + 16*(i%2).  (Slot l's 8 elements of j are exactly lane l's 8 BF16 A-
 *    operand values of one v_mfma_f32_16x16x32_bf16 step.)
 *  - Escapes: u32 (r<<28) | (k<<8) | e per escape; row-block b owns
 *    esc[esc_off[b] .. esc_off[b+1]), sorted ascending by (k, r); esc_off has
 *    n/16 + 1 entries, esc_off[0] = 0, esc_off[n/16] = n_esc.
 *  - Bits per weight = 12 + 8*(4*n_esc + 4*(n/16 + 1) + 64)/(n*k) counting a 64-byte
 *    header; tile bytes are exactly 3/4 of the BF16 bytes.
 *
 * Conventions for every call:
 *  - Pointers marked "device" are HIP device memory owned by the caller; the library
 *    never allocates or frees device memory and never synchronises, except
 *    w12_encode_count (documented below).  Inputs must not alias outputs.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls are asynchronous;
 *    buffers must stay alive until the stream has passed the call.
 *  - Arguments are validated on the host before any HIP call; on error nothing is
 *    launched and outputs are untouched.  Launch failures return W12_ERR_HIP; device
 *    faults surface at the caller's next synchronisation.
 *  - The workspace `ws` (device, w12_workspace_bytes(op, ...) bytes, 256-byte aligned;
 *    may be NULL when that size is 0) holds intermediate results.  GEMM workspaces
 *    (W12_OP_GEMM, W12_OP_GEMM_BF16, W12_OP_GEMM_GROUP, W12_OP_GEMM_F8) begin with the
 *    split-K tickets
 *    (4096 bytes), which must be zero before the first call that uses the workspace
 *    (a zero-filled allocation, or w12_workspace_init); every call leaves them zero, so
 *    one zeroing serves every later call of any shape.  Nothing else in any workspace
 *    needs initialisation.  Two calls that run concurrently must not share a workspace.
 */
#ifndef W12_H
#define W12_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t w12_status;

#define W12_OK             0
#define W12_ERR_NULL      -1  /* a required pointer is NULL */
#define W12_ERR_SHAPE     -2  /* n % 16, k % 128, k >= 2^20, n == 0, m * n >= 2^32 */
#define W12_ERR_RANGE     -3  /* m outside 1..W12_MAX_M, n_draft > m, n_req outside 1..m */
#define W12_ERR_FORMAT    -4  /* codebook not strictly ascending, e_max >= 255 */
#define W12_ERR_WORKSPACE -5  /* workspace smaller than w12_workspace_bytes() */
#define W12_ERR_HIP       -6  /* a HIP runtime call or kernel launch failed */
#define W12_ERR_ALIGN     -7  /* tiles/x/w/y/ws not aligned as documented */

/* Rows of one call: decode-sized batches (1..32) and the batched regime of several
 * requests verified together (16 to 24 requests of a few draft tokens each). */
#define W12_MAX_M 128
#define W12_MAX_GROUP 4   /* weights of one w12_gemm_group or w12_gemm_f8_group call, at most */

/* Host-side descriptor of one W12 tensor (device buffers + host metadata). */
typedef struct w12_desc {
  uint64_t n;             /* output rows, multiple of 16 */
  uint64_t k;             /* input columns, multiple of 128, < 2^20 */
  uint64_t n_esc;         /* number of escape records */
  uint8_t codebook[16];   /* strictly ascending exponent fields */
  uint8_t e_max;          /* largest exponent field < 255 present in W (0 if none) */
  uint8_t reserved[7];
  void* tiles;            /* device, w12_tiles_bytes(n, k) bytes, 16-byte aligned */
  uint32_t* esc_off;      /* device, n/16 + 1 entries */
  uint32_t* esc;          /* device, n_esc entries (may be NULL when n_esc == 0) */
} w12_desc;

/* Operation ids for w12_workspace_bytes. */
#define W12_OP_ENCODE    0
#define W12_OP_DECODE    1
#define W12_OP_GEMM      2
#define W12_OP_GEMM_BF16 3
#define W12_OP_VERIFY    4
#define W12_OP_GEMM_GROUP 5   /* n = the group's rows added up */
#define W12_OP_VERIFY2   6   /* two-level verification (w12_lmhead_verify2) */
#define W12_OP_GEMM_F8   7   /* FP8 GEMM (w12_gemm_f8) */

/* Bytes of the tile array: (n/16)*(k/128)*3072; 0 if the shape is invalid. */
size_t w12_tiles_bytes(uint64_t n, uint64_t k);

/* Workspace bytes needed by `op` for m rows (ignored by ENCODE/DECODE) and an
 * n x k weight; 0 for an invalid op or shape, and 0 when the op needs none (DECODE,
 * and GEMM shapes that are not split along K).  GEMM split along K needs the tickets
 * (4096 bytes), FP32 partials [splits][m][n] and the row-block groups' row sums of x^2
 * [groups][splits][m] (RMS launches), each from a 256-byte boundary; VERIFY holds, each region starting on a 256-byte boundary
 * in this order: per-row diagnostic counts (int32 [m][2]: candidate logits, those left
 * after the FP64 screen), the per-row-block records of the first pass (largest FP32
 * logit, second largest, largest row norm bound W_v (w12_lmhead_verify), each FP32
 * [m][n/16]; index of the largest, int32 [m][n/16]), its per-workgroup group records
 * (largest logit, second largest, its index, that row-block's norm bound, the group's
 * largest norm bound: five arrays of [m][n/16] 4-byte entries, the first ngroups of each
 * row used) and the
 * candidate lists (int32 [m][n]); all readable after a call for diagnostics.  ENCODE holds the histogram and per-tile escape counts. */
size_t w12_workspace_bytes(int op, uint32_t m, uint64_t n, uint64_t k);

/* Zero-fills `ws` on `stream` with a kernel (no hipMemset): prepares a GEMM workspace
 * whose memory was not allocated zero-filled (its split-K tickets must start at zero). */
w12_status w12_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Encode, first half (exponent histogram -> codebook, e_max, n_esc).
 * w: device BF16 bits [n][k] row-major, 16-byte aligned.  Results land in host memory
 * (codebook_out[16], *e_max_out, *n_esc_out); this call SYNCHRONISES `stream` to
 * return them.  Defines the codebook rule of the W12 v1 layout above (lossless format
 * per "SpecPilot" glossary, "Differentiation"). */
w12_status w12_encode_count(const uint16_t* w, uint64_t n, uint64_t k,
                            uint8_t codebook_out[16], uint8_t* e_max_out,
                            uint64_t* n_esc_out, void* ws, size_t ws_bytes, void* stream);

/* Byte offset in an ENCODE workspace of the u32 where w12_encode leaves the true escape
 * count of its input for d->codebook (readable once the stream has reached the call). */
#define W12_ENCODE_TOTAL_OFFSET 2112

/* Encode, second half (the W12 v1 layout above; lossless 12-bit format per "SpecPilot"
 * glossary, "Differentiation", at about 12.01-12.02 bits per weight per the review's
 * "The mechanisms it found"): writes d->tiles, d->esc_off and d->esc for w [n][k] using
 * d->codebook.  d->n_esc must be the count w12_encode_count returned for that codebook.
 * The call does not synchronise, so it cannot check that: with a wrong n_esc the encoding
 * is wrong (escapes past n_esc are dropped) but memory-safe, since escape writes stop at
 * n_esc and every esc_off entry is clamped to n_esc, so no later call reads past `esc`;
 * compare the u32 at W12_ENCODE_TOTAL_OFFSET of ws with n_esc to detect it (equal for a
 * correct call).  Output bytes are identical to the CPU oracle's. */
w12_status w12_encode(const uint16_t* w, const w12_desc* d, void* ws, size_t ws_bytes,
                      void* stream);

/* Bit-exact inverse of w12_encode (lossless per "SpecPilot" glossary, "Differentiation"):
 * w_out device BF16 [n][k] row-major (16-byte aligned). */
w12_status w12_decode(const w12_desc* d, uint16_t* w_out, void* stream);

/* y = x . W^T with W decoded in registers ("StargazerX0/SpecPilot", "What it is"):
 * x device BF16 [m][k], y device BF16 [m][n] (row-major, 16-byte aligned), m in
 * 1..W12_MAX_M,
 * FP32 accumulation, round-to-nearest-even to BF16.  IEEE propagation for non-finite
 * inputs.  ws: w12_workspace_bytes(W12_OP_GEMM, ...) bytes (may be NULL when that is
 * 0; its tickets zeroed once, see above); calls that share a workspace must be ordered on
 * one stream.  The result is deterministic: when K is split, the split that finishes last
 * in each row-block group sums the FP32 partials of all splits in split order. */
w12_status w12_gemm(const uint16_t* x, uint32_t m, const w12_desc* d, uint16_t* y,
                    void* ws, size_t ws_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): w12_gemm with its K-split workspace
 * taken from a fixed array of W12_NOALLOC_SCRATCH_BYTES inside the library instead of a
 * caller's buffer; each GPU holds its own copy of the array from that GPU's first call
 * until the process ends.  Arguments (the caller still passes x and y), arithmetic,
 * results (bit-identical to w12_gemm: same kernels, same K split) and errors as w12_gemm;
 * W12_ERR_WORKSPACE when the call needs more workspace than the array holds
 * (w12_workspace_bytes(W12_OP_GEMM, m, n, k) > W12_NOALLOC_SCRATCH_BYTES), checked before
 * any HIP call.  Allocates nothing.  The stream's GPU must be the current device.  The
 * first call on a GPU looks up the array's device address (make it before capturing a
 * graph) and clears the array's split-K tickets on `stream`; every call leaves them at
 * zero.  All calls on one GPU share its array, which keeps the last call's contents:
 * calls ordered on one stream are safe, calls that overlap on one GPU (other streams,
 * other host threads) race and give undefined results. */
#define W12_NOALLOC_SCRATCH_BYTES (32u << 20)
w12_status w12_gemm_noalloc(const uint16_t* x, uint32_t m, const w12_desc* d, uint16_t* y,
                            void* stream);

/* Several W12 weights that read the same x (q, k and v of a layer; gate and up):
 * ys[i] = x . W_i^T for i < n_w (1..W12_MAX_GROUP), all with the same k, in one launch
 * per codebook kind (row-blocks of the weights numbered consecutively; a K split is
 * completed inside the launch, as in w12_gemm).  descs: host array of n_w descriptors; ys:
 * host array of n_w device BF16 outputs [m][n_i], each 16-byte aligned.  Same arithmetic, rounding and
 * determinism as w12_gemm (the K split can differ, so the last bit can too).
 * ws: w12_workspace_bytes(W12_OP_GEMM_GROUP, m, sum of n_i, k) bytes.  Errors: as
 * w12_gemm; W12_ERR_RANGE for n_w outside 1..W12_MAX_GROUP, W12_ERR_SHAPE for weights
 * of different k. */
w12_status w12_gemm_group(const uint16_t* x, uint32_t m, const w12_desc* const* descs,
                          uint32_t n_w, uint16_t* const* ys, void* ws, size_t ws_bytes,
                          void* stream);

/* The same products of the row-wise RMS-normalised input, for the layer chain whose
 * every GEMM consumes the RMS-rescaled output of the previous one (w12_rms_rescale):
 * y[row] = bf16((x[row] . W^T) / r), r = sqrt(mean_k x[row,k]^2) in FP32, the division
 * applied to the FP32 accumulators (equal to the product of the rescaled row up to
 * rounding; the rescaled row itself is never rounded to BF16).  r comes from the x values
 * each launch streams anyway (up to 32 rows as matrix-core products of x with itself,
 * from 33 rows per-unit sums), summed the same way on every call.  Arguments, workspace
 * (W12_OP_GEMM / W12_OP_GEMM_GROUP), errors and determinism as w12_gemm /
 * w12_gemm_group.  Not part of the W12 method itself. */
w12_status w12_gemm_rms(const uint16_t* x, uint32_t m, const w12_desc* d, uint16_t* y,
                        void* ws, size_t ws_bytes, void* stream);
w12_status w12_gemm_group_rms(const uint16_t* x, uint32_t m, const w12_desc* const* descs,
                              uint32_t n_w, uint16_t* const* ys, void* ws, size_t ws_bytes,
                              void* stream);

/* The same kernel family reading plain BF16 weights w [n][k] row-major (the baseline
 * W12 is measured against: plain BF16 decoding in "What it is").  Workspace as for
 * w12_gemm (W12_OP_GEMM_BF16). */
w12_status w12_gemm_bf16(const uint16_t* x, uint32_t m, const uint16_t* w, uint64_t n,
                         uint64_t k, uint16_t* y, void* ws, size_t ws_bytes, void* stream);

/* The second baseline: BF16 weights in 4 KB tiles, read by the same kernel family with
 * the same streaming loads as W12 tiles (every wave instruction reads 1 KB of whole
 * lines).  w12_bf16_tile writes the tiled copy of row-major w [n][k] (device, 16-byte
 * aligned) into w_tiled (device, n*k*2 bytes, 16-byte aligned): tile (b, g) at
 * (g*(n/16) + b)*4096 (column-major, as the W12 tiles), lane slot l (r = l%16,
 * q = l/16) of group j at 1024j + 16l holding row 16b + r, columns 128g + 32j + 8q .. +7.  w12_gemm_bf16_tiled takes that
 * copy; workspace as for w12_gemm_bf16 (W12_OP_GEMM_BF16).  Shapes and errors as
 * w12_gemm_bf16. */
w12_status w12_bf16_tile(const uint16_t* w, uint64_t n, uint64_t k, void* w_tiled, void* stream);
w12_status w12_gemm_bf16_tiled(const uint16_t* x, uint32_t m, const void* w_tiled, uint64_t n,
                               uint64_t k, uint16_t* y, void* ws, size_t ws_bytes,
                               void* stream);

/* FP8 GEMM routing (review page, "The mechanisms it found": FP8 GEMM routing among the
 * batching mechanisms; "StargazerX0/SpecPilot", "What it is": batching settings with FP8
 * targets).  The pages give no format; this library reads it as the target's own FP8
 * weights in the common checkpoint form: W[n][k] = q[n][k] * s[n/128][k/128], q one OCP
 * FP8 E4M3 byte per weight (bias 7, no infinities, S.1111.111 NaN), s one FP32 scale per
 * 128 x 128 block, with BF16 activations.  The product is the W12 GEMM's with those
 * weights: every x * q is exact in FP32, each 128-column block sum is multiplied by its
 * scale, the result rounded once to BF16, so it is lossless for such a target to the
 * same accumulation tolerance as w12_gemm.
 * w12_f8_tile writes the tiled copy of row-major q [n][k] (device, n*k bytes, 16-byte
 * aligned) into w_tiled (device, n*k bytes, 16-byte aligned): tile (b, g) at
 * (g*(n/16) + b)*2048 (column-major), the 8 bytes of lane slot l (r = l%16, q = l/16) in
 * group j (row 16b + r, columns 128g + 32j + 8q .. +7) at 1024*(j/2) + 16l + 8*(j%2).
 * w12_gemm_f8: y[row] = bf16(sum_k x[row,k] * q[n,k] * s[n/128][k/128]) for x device
 * BF16 [m][k] (m in 1..W12_MAX_M, 16-byte aligned), w_tiled as written by w12_f8_tile,
 * scale device FP32 [ceil(n/128)][k/128] row-major (4-byte aligned; the last block row
 * covers the rows past the last multiple of 128), y device BF16 [m][n].
 * ws: w12_workspace_bytes(W12_OP_GEMM_F8, m, n, k) bytes, as for w12_gemm.  Shapes,
 * errors and determinism as w12_gemm; finite x, q and s keep the result within that
 * tolerance, a NaN byte makes its rows' outputs NaN. */
w12_status w12_f8_tile(const uint8_t* w, uint64_t n, uint64_t k, void* w_tiled, void* stream);
w12_status w12_gemm_f8(const uint16_t* x, uint32_t m, const void* w_tiled, const float* scale,
                       uint64_t n, uint64_t k, uint16_t* y, void* ws, size_t ws_bytes,
                       void* stream);

/* Up to W12_MAX_GROUP FP8 weights that read one x (q, k and v of a layer, or gate and up)
 * in one launch: y_i = bf16(x . W_i^T) for weight i given by w_tiled[i] (from w12_f8_tile),
 * scales[i] (FP32 [ceil(ns[i]/128)][k/128]) and ns[i] rows, all with the same k; ys[i]
 * device BF16 [m][ns[i]].  The arrays of pointers and ns are host memory.
 * ws: w12_workspace_bytes(W12_OP_GEMM_GROUP, m, sum of ns[i], k) bytes.  Errors as
 * w12_gemm_f8; W12_ERR_RANGE for n_w outside 1..W12_MAX_GROUP. */
w12_status w12_gemm_f8_group(const uint16_t* x, uint32_t m, const void* const* w_tiled,
                             const float* const* scales, const uint64_t* ns, uint32_t n_w,
                             uint64_t k, uint16_t* const* ys, void* ws, size_t ws_bytes,
                             void* stream);

/* The same products of the row-wise RMS-normalised input, as w12_gemm_rms for W12
 * weights (harness op of a layer chain, not part of the FP8 routing itself):
 * y[row] = bf16((x[row] . W^T) / r), r = sqrt(mean_k x[row,k]^2) in FP32, the division
 * applied to the FP32 sums.  Arguments, workspace, errors and determinism as
 * w12_gemm_f8 / w12_gemm_f8_group. */
w12_status w12_gemm_f8_rms(const uint16_t* x, uint32_t m, const void* w_tiled, const float* scale,
                           uint64_t n, uint64_t k, uint16_t* y, void* ws, size_t ws_bytes,
                           void* stream);
w12_status w12_gemm_f8_group_rms(const uint16_t* x, uint32_t m, const void* const* w_tiled,
                                 const float* const* scales, const uint64_t* ns, uint32_t n_w,
                                 uint64_t k, uint16_t* const* ys, void* ws, size_t ws_bytes,
                                 void* stream);

/* Greedy verification over the LM head (review page, "The mechanisms it found":
 * certified exact-argmax LM head; "StargazerX0/SpecPilot", "Results and
 * verification": committed tokens are the target's own choice).
 * x device BF16 [m][k] (m in 1..W12_MAX_M, finite), W12 head d (finite weights), draft
 * device int32 [n_draft] (n_draft <= m).  Writes argmax_out device int32 [m]: the index
 * v maximising the EXACT logit sum_k x[row,k]*W[v,k], lowest index on exact ties; and
 * accepted_out device int32 [1]: the first i < n_draft with argmax[i] != draft[i], or
 * n_draft.  A first pass streams the head once and keeps, per 16-row block, the two
 * largest FP32 logits z^ and the largest FP32 upper bound W_v of ||w_v||_2 (the same pass
 * sums the squares of the weights it streams), and per workgroup of blocks their maxima.
 * The error scale of a logit is S = X W_v >= sum_k |x_k||w_vk| (Cauchy-Schwarz), X an
 * upper bound of ||x||_2 taken in the second pass.  With B(S) a bound on |z^ - z| for any summation
 * order, every logit whose z^ + B(S) can reach the lower bound z^* - B(S*) of the
 * computed maximum is a candidate; a single candidate is the answer, several are
 * recomputed in FP64 from the W12 tiles, and those that the FP64 intervals cannot
 * separate are summed exactly, so the result does not depend on the reduction order.
 * A row of x that is all +-0 gets index 0 (every logit is exactly 0) without a search;
 * any number of candidates is screened, in chunks (weights whose squares sum past the FP32
 * range, |w| of about 2^57 at k = 5120, make W_v infinite: the answer stays exact, but
 * every row of such a block, or of the whole head when it holds the largest logit, is
 * screened).  A row whose logits are not finite
 * gets argmax -1.  ws: w12_workspace_bytes(W12_OP_VERIFY, m, n, k). */
w12_status w12_lmhead_verify(const uint16_t* x, uint32_t m, const w12_desc* d,
                             const int32_t* draft, uint32_t n_draft, int32_t* argmax_out,
                             int32_t* accepted_out, void* ws, size_t ws_bytes,
                             void* stream);

/* Greedy verification of several requests in one pass over the LM head (review page,
 * "Where the numbers come from": batched decoding of 16, 20 and 24 requests; "The
 * mechanisms it found": ragged drafts, a drafter block length per request).  The
 * argmax is w12_lmhead_verify's over all m rows of x.  Request r (0 <= r < n_req,
 * 1 <= n_req <= m) owns rows req_off[r] .. req_off[r+1]-1, and its draft tokens are
 * draft[req_off[r] + i] for i < req_ndraft[r].  req_off (int32 [n_req + 1]), req_ndraft
 * (int32 [n_req]) and draft (int32 [m]) are device arrays read on the stream, so one
 * prepared call can serve new batches.  accepted_out (device int32 [n_req]) gets, per
 * request, the first i < req_ndraft[r] with argmax[req_off[r] + i] != draft[req_off[r]
 * + i], or req_ndraft[r] when there is none.  An entry is valid when 0 <= req_off[r] <=
 * req_off[r+1] <= m and 0 <= req_ndraft[r] <= req_off[r+1] - req_off[r]; an invalid one
 * gets accepted -1 (the kernels read nothing outside the three arrays).  Rows before
 * req_off[0] or from req_off[n_req] on belong to no request and are only argmax'd.
 * ws: w12_workspace_bytes(W12_OP_VERIFY, m, n, k).  Errors as w12_lmhead_verify, plus
 * W12_ERR_RANGE for n_req outside 1..m. */
w12_status w12_lmhead_verify_batched(const uint16_t* x, uint32_t m, const w12_desc* d,
                                     const int32_t* req_off, const int32_t* req_ndraft,
                                     uint32_t n_req, const int32_t* draft,
                                     int32_t* argmax_out, int32_t* accepted_out, void* ws,
                                     size_t ws_bytes, void* stream);

/* The first pass of w12_lmhead_verify with its full output (for tests of the certified
 * bound, and as an FP32-output GEMM): logits_out = FP32 z^ [m][n] and sabs_out = the
 * FP32 error scales S = X W_v [m][n] of w12_lmhead_verify, rounded up (device, 16-byte
 * aligned), from the same kernels in the same summation order as the verification; ws as
 * for W12_OP_VERIFY (its block maxima are overwritten).  Errors as w12_lmhead_verify. */
w12_status w12_logits_f32(const uint16_t* x, uint32_t m, const w12_desc* d, float* logits_out,
                          float* sabs_out, void* ws, size_t ws_bytes, void* stream);

/* ---- Two-level verification ("SpecPilot: an agent doubled speculative decoding speed,
 * and the 10.87x needs context", "The mechanisms it found": verification in two levels
 * with an 8-bit copy of the head; "SpecPilot" glossary, "Differentiation").  A screen
 * copy of the LM head (8-bit codes) is streamed first; a certified bound rules out every
 * logit that cannot be the argmax, and only the others are computed from the W12 head
 * (FP64, then exact sums where FP64 cannot separate them).
 *
 * Screen copy v1 (one device buffer of w12_screen_bytes(n, k) bytes):
 *  - per row v and group g of 32 consecutive columns, a scale s_vg = the smallest BF16
 *    value >= (largest |w| over the group's finite weights) / 127, and at least 2^-100;
 *    codes q = w / s_vg rounded to the nearest integer, ties to even (int8, |q| <= 127; 0
 *    for a non-finite w);
 *  - tiles of 16 rows x 128 columns, 2176 bytes, tile (b, g) at (g*(n/16) + b)*2176: the
 *    code of element t of lane slot l (the W12 slot layout above) at 1024*(t/16) + 16l +
 *    t%16, then the tile's 64 scales (BF16, little-endian), row 4a+i (a, i = 0..3) and
 *    32-column group j of the tile at 2048 + 32a + 8i + 2j;
 *  - from the next 256-byte boundary, FP32 C[n]: C_v >= ||w_v - q_v s_v||_2 +
 *    gamma ||q_v s_v||_2 (gamma = D 2^-23 / (1 - D 2^-23), D = k/32 + 64), +Inf for a row with
 *    a non-finite weight; from the next 256-byte boundary, FP32 A[n] >= (k/32)(max_g s_vg
 *    2^-113 + 2^-125), the allowance for flushed denormals.
 * For any x row and any FP32 evaluation of the screen logit z8^_v = sum_g s_vg (sum over
 * the group's 32 columns of x_k q_vk) in which each term passes through at most D
 * additions (a 32-term group sum, then one scaled addition per group),
 * |z8^_v - z_v| <= ||x||_2 C_v + A_v (z_v the exact logit): Cauchy-Schwarz on the code
 * residuals, plus the rounding of the sum. */
size_t w12_screen_bytes(uint64_t n, uint64_t k);

/* Builds the screen copy of BF16 weights w [n][k] (device, row-major, 16-byte aligned;
 * shape as W12: n % 16 == 0, k % 128 == 0, 0 < k < 2^20) into `screen` (device, 256-byte
 * aligned, screen_bytes >= w12_screen_bytes(n, k), else W12_ERR_WORKSPACE).  Codes and
 * scales are identical to the CPU oracle's; C and A are computed in FP64 with rounding
 * margins and rounded up (certified upper bounds, not unique values). */
w12_status w12_screen_encode(const uint16_t* w, uint64_t n, uint64_t k, void* screen,
                             size_t screen_bytes, void* stream);

/* Greedy verification in two levels: the same results as w12_lmhead_verify (the exact
 * argmax per row, lowest index on exact ties; the accepted length), from the W12 head d and
 * `screen`, its screen copy (w12_screen_encode of the same weights: the results are exact
 * only if it is).  Pass 1 streams the screen copy (0.71 of the W12 tile bytes) and keeps,
 * per x row and 16-row block, the certified intervals' largest and second largest upper
 * ends z8^ + ||x|| C + A (||x|| bounded from above from the staged x) and, per group of 8
 * blocks, the largest upper and lower ends; pass 2 (32 workgroups per x row) drops every
 * logit whose upper end is below the row's largest lower end, recomputes the others in
 * FP64 from the W12 tiles (one wave each), and the workgroup that finishes a row last keeps
 * those whose FP64 intervals reach the largest FP64 lower bound, summing them exactly when
 * more than one is left and any is inexact.  A row of x that is all +-0 gets 0; a row with
 * a non-finite x or candidate logit gets -1.  x, m, d, draft, n_draft, argmax_out and
 * accepted_out as for w12_lmhead_verify; screen 256-byte aligned.
 * ws: w12_workspace_bytes(W12_OP_VERIFY2, m, n, k) bytes, 256-byte aligned; it begins with
 * 4096 bytes of per-row tickets that must be zero before its first use
 * (w12_workspace_init) and that every call leaves zero; calls sharing a workspace must be
 * ordered on one stream.  Errors as w12_lmhead_verify. */
w12_status w12_lmhead_verify2(const uint16_t* x, uint32_t m, const w12_desc* d,
                              const void* screen, const int32_t* draft, uint32_t n_draft,
                              int32_t* argmax_out, int32_t* accepted_out, void* ws,
                              size_t ws_bytes, void* stream);

/* Several requests in one two-level pass: requests and results as
 * w12_lmhead_verify_batched, verification as w12_lmhead_verify2. */
w12_status w12_lmhead_verify2_batched(const uint16_t* x, uint32_t m, const w12_desc* d,
                                      const void* screen, const int32_t* req_off,
                                      const int32_t* req_ndraft, uint32_t n_req,
                                      const int32_t* draft, int32_t* argmax_out,
                                      int32_t* accepted_out, void* ws, size_t ws_bytes,
                                      void* stream);

/* Pass 1 of w12_lmhead_verify2 with its full output (for tests of the screen bound):
 * logits_out = the FP32 screen logits z8^ [m][n] and bound_out = their FP32 bounds
 * ||x|| C_v + A_v rounded up [m][n] (device, 16-byte aligned).  d supplies the shape only
 * (its buffers are not read).  ws as for W12_OP_VERIFY2 (its records are overwritten). */
w12_status w12_screen_logits_f32(const uint16_t* x, uint32_t m, const w12_desc* d,
                                 const void* screen, float* logits_out, float* bound_out,
                                 void* ws, size_t ws_bytes, void* stream);

/* Harness op for the layer chain: y[row] = bf16(x[row] / sqrt(mean(x[row]^2))) in FP32,
 * x, y device BF16 [m][k] (16-byte aligned, k % 8 == 0, 0 < k < 2^20, m <= 2^20;
 * otherwise W12_ERR_ALIGN / W12_ERR_SHAPE / W12_ERR_RANGE).  Not part of the W12
 * method itself. */
w12_status w12_rms_rescale(const uint16_t* x, uint32_t m, uint64_t k, uint16_t* y,
                           void* stream);

/* Measurement helper, not part of the W12 method: streams `bytes` (a multiple of 16,
 * below 2^32) of device memory at `buf` (16-byte aligned) with the nontemporal 16-byte
 * buffer loads the GEMM kernels use for W12 tiles, grid-stride over `workgroups`
 * (1..65536) workgroups of 256 threads; each wave stores the XOR of what it read in
 * sink[4 * workgroup + wave] (device, 4 * workgroups uint32, 4-byte aligned).  Its time is
 * the streaming-read ceiling a GEMM launch of the same size is compared with, and its
 * FETCH_SIZE counter scales the traffic counters for these loads.  Errors: W12_ERR_NULL,
 * W12_ERR_SHAPE (bytes), W12_ERR_RANGE (workgroups), W12_ERR_ALIGN. */
w12_status w12_stream_read(const void* buf, uint64_t bytes, uint32_t workgroups, uint32_t* sink,
                           void* stream);

/* Static description of a status code. */
const char* w12_status_str(w12_status s);

/* Library version: 0x000100 for W12 v1, library 0.1. */
uint32_t w12_version(void);

#ifdef __cplusplus
}
#endif

#endif /* W12_H */
