/*
 * detgrad.h - deterministic, atomic-free gradient reductions for AMD MI355X (gfx950).
 *
 * Four reductions that the pages make deterministic by the same pattern: each
 * workgroup writes its own FP32 partial sums into per-tile slots, and the slots
 * are then reduced in a fixed canonical order on the caller's stream
 * (Megatron-LM PR #8244, description; cudnn-frontend PR #521, first commit).
 * Every entry point takes an `atomic` flag: 0 runs the deterministic route,
 * 1 runs the non-deterministic comparison route that adds the same tile
 * partials into the output with hardware float atomics.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - All data pointers are device pointers (hipMalloc / torch CUDA tensors).
 *   `stream` is a hipStream_t passed as void* (NULL = the default stream).
 * - A call only enqueues work on `stream`. It never allocates, never
 *   synchronises with the host and keeps no state between calls; the caller
 *   owns every buffer, the workspace included.
 * - Outputs ACCUMULATE: out <- RN32(out + total), one rounding per element
 *   (cudnn-frontend PR #521: the slot reduction adds into the existing output
 *   instead of replacing it; FlashInfer PR #8924: bitwise AccumulateGrad of
 *   the deterministic dW). An empty problem leaves every output bit unchanged.
 * - `atomic` must be exactly 0 or 1, anything else is DET_ERR_INVALID_ARG
 *   (FlashInfer PR #8924, mode rules: only an explicit value selects a route).
 * - With atomic = 0 the output bits are a function of the inputs and the tile
 *   configuration only: identical from run to run, under any concurrent load.
 *   With atomic = 1 only closeness is promised.
 * - All arguments are checked on the host before anything is enqueued; a
 *   non-OK status means nothing was launched. det_last_error() then returns a
 *   thread-local description.
 *
 * Workspace
 * ---------
 * The deterministic routes need device scratch of det_*_workspace_size()
 * bytes (0 when a route keeps its partials on chip), 256-byte aligned. A
 * non-empty workspace starts with a 256-byte header; det_index_add keeps its
 * bad-id counter there, which every call leaves at zero again. Call
 * det_workspace_init() once on a new workspace (it enqueues a tiny fill
 * kernel on `stream`); it never needs another fill. The slot area behind the
 * header is never read before it is written in the same call, so it needs no
 * initial value. One workspace must not be used by two calls that can run at
 * the same time (for example on two streams without an event between them).
 */
#ifndef DETGRAD_H
#define DETGRAD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define DET_ABI_VERSION 1
#define DET_WS_HEADER_BYTES 256

typedef enum {
  DET_OK = 0,
  DET_ERR_INVALID_ARG = -1, /* bad size, stride, pointer, flag or config    */
  DET_ERR_UNSUPPORTED = -2, /* legal but not implemented (e.g. dtype)       */
  DET_ERR_WORKSPACE = -3,   /* workspace missing, too small or misaligned   */
  DET_ERR_OVERLAP = -4,     /* an output overlaps an input or the workspace */
  DET_ERR_HIP = -5          /* the HIP runtime reported an error            */
} det_status;

typedef enum { DET_BF16 = 0, DET_F32 = 1 } det_dtype;

/* ABI version of the loaded library (DET_ABI_VERSION). */
int det_abi_version(void);

/* Text of the last non-OK status returned on this thread ("" if none). */
const char* det_last_error(void);

/* Zero the counter header of a fresh workspace. Enqueued on `stream` as a
 * small fill kernel (no memset node, so it may be graph-captured).
 * ws: device pointer, 256-byte aligned; ws_bytes >= DET_WS_HEADER_BYTES. */
int det_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------
 * det_colsum: Gated-DeltaNet gate backward column sums.
 * Megatron-LM PR #8244 (ordered A_log/dt_bias reduction of the fused pre-GDR
 * gate backward): programs write FP32 partial sums and the caller reduces
 * them in order; the tile is picked by a shape-only rule that also sizes the
 * scratch and the launch, and explicit tile overrides are honoured.
 *
 *   x = a[t,h] + dt_bias[h],  g = -exp(A_log[h]) * softplus(x)
 *   dA_log[h]   += sum_t dg[t,h] * g
 *   ddt_bias[h] += sum_t dg[t,h] * (-exp(A_log[h])) * sigmoid(x)
 *
 * Canonical order: per tile of block_t rows and per head, the adjacent
 * pairwise tree over the tile's rows (rows >= T count as -0.0); the tiles'
 * slots folded left to right; one add into the output. exp, softplus and
 * sigmoid are fixed sequences of correctly rounded float32 operations
 * (threshold 20 for softplus), so the CPU oracle reproduces every bit.
 * block_h only shapes the launch; it never changes a bit.
 *
 * a, dg: [T, H] with element strides (st, sh) >= 1, any layout (for example
 *        a column slice of a wider tensor, or a transposed view); dtype
 *        DET_BF16 (widened exactly) or DET_F32, the same for both (the page
 *        tests both input precisions).
 * A_log, dt_bias: [H] float32, contiguous. dA_log, ddt_bias: [H] float32,
 *        accumulated, must not overlap the inputs, each other or ws.
 * cfg:   NULL selects det_colsum_select_cfg(T, H). block_t in {64,128,256},
 *        block_h in {8,16,32}.
 * ws:    det_colsum_workspace_size() bytes (0 for atomic = 1; ws may be NULL). */
typedef struct {
  int32_t block_t;
  int32_t block_h;
} det_colsum_cfg;

int det_colsum_select_cfg(int64_t T, int64_t H, det_colsum_cfg* out);
int det_colsum_workspace_size(int64_t T, int64_t H, const det_colsum_cfg* cfg, int atomic, size_t* bytes);
int det_colsum(const void* a, int64_t a_st, int64_t a_sh, const void* dg, int64_t dg_st, int64_t dg_sh,
               int in_dtype, const float* A_log, const float* dt_bias, int64_t T, int64_t H, float* dA_log,
               float* ddt_bias, const det_colsum_cfg* cfg, void* ws, size_t ws_bytes, int atomic, void* stream);

/* det_colsum_da: det_colsum that also writes the elementwise gradient of the
 * gate input (the same x depends on a and on dt_bias, so the term summed into
 * ddt_bias is da itself):
 *
 *   da[t,h] = dg[t,h] * (-exp(A_log[h])) * sigmoid(x)   (overwritten, not accumulated)
 *
 * computed in float32 exactly as the ddt_bias term and stored in in_dtype:
 * bf16 by round to nearest even (NaN stays NaN), float32 unchanged. The GDN
 * gate page names only the two parameter gradients; the elementwise output is
 * the gate-variants extension of the same kernel. dA_log and ddt_bias are
 * bitwise those of det_colsum, on both arms.
 * da: [T, H] with element strides (da_st, da_sh) >= 1 such that no two
 *     elements share an address (da_st >= H*da_sh or da_sh >= T*da_st); it
 *     must not overlap a, dg, A_log, dt_bias, dA_log, ddt_bias or ws.
 * Other arguments, errors and the workspace as for det_colsum. */
int det_colsum_da(const void* a, int64_t a_st, int64_t a_sh, const void* dg, int64_t dg_st, int64_t dg_sh,
                  int in_dtype, const float* A_log, const float* dt_bias, int64_t T, int64_t H, float* dA_log,
                  float* ddt_bias, void* da, int64_t da_st, int64_t da_sh, const det_colsum_cfg* cfg, void* ws,
                  size_t ws_bytes, int atomic, void* stream);

/* det_colsum_noalloc: det_colsum for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same arguments without a workspace, the same bits on
 * both arms. The slots live in a static device array of the library, 4 MiB
 * per GPU, held until the process ends. A problem whose slots need more
 * (256 + 2 * ceil(T / block_t) * H * 4 bytes, rounded up to 256 per slot
 * array) returns DET_ERR_WORKSPACE before any launch. The call allocates
 * nothing. Every call on one GPU shares that GPU's array, so two calls that
 * can run at the same time on one GPU (two streams, two threads) race and
 * must be ordered by the caller. */
int det_colsum_noalloc(const void* a, int64_t a_st, int64_t a_sh, const void* dg, int64_t dg_st, int64_t dg_sh,
                       int in_dtype, const float* A_log, const float* dt_bias, int64_t T, int64_t H, float* dA_log,
                       float* ddt_bias, const det_colsum_cfg* cfg, int atomic, void* stream);

/* ------------------------------------------------------------------------
 * det_index_add: out[ids[p]] += src[p] without float atomics.
 * Megatron-LM PR #7441 (DSv4 deterministic mode), source 3: the sparse-
 * indexer dK is accumulated by a deterministic index_add (stable sort +
 * prefix sum) instead of atomics; padding slots are dropped.
 *
 * Canonical order: pairs (ids[p], p) with 0 <= ids[p] < n_rows, stably sorted
 * by id (equal ids keep ascending p); each id's run cut into chunks of
 * chunk_rows rows; a chunk's partial is the left-to-right fold of its rows;
 * the chunk partials folded left to right and added once into out[id]. Ids
 * of -1 are padding. Any other out-of-range id is dropped and counted
 * (det_index_add_bad_ids). Ids with no rows leave out[id] untouched.
 *
 * out:  [n_rows, dim] float32, row stride out_ld >= dim (elements).
 * ids:  [n_src] int32. src: [n_src, dim], row stride src_ld >= dim, DET_BF16
 *       (widened exactly) or DET_F32 (the page tests the indexer dK in both).
 * dim must be a multiple of 8; out_ld, src_ld multiples of 8; src and out
 * 16-byte aligned (DET_ERR_UNSUPPORTED otherwise). n_rows <= 16384, dim <= 512.
 * cfg:  NULL = {chunk_rows = 256}; chunk_rows in [1, 65536].
 * ws:   det_index_add_workspace_size() bytes (0 for atomic = 1). */
typedef struct {
  int32_t chunk_rows;
} det_index_add_cfg;

int det_index_add_workspace_size(int64_t n_src, int64_t dim, int64_t n_rows, const det_index_add_cfg* cfg,
                                 int atomic, size_t* bytes);
int det_index_add(float* out, int64_t n_rows, int64_t dim, int64_t out_ld, const int32_t* ids, int64_t n_src,
                  const void* src, int64_t src_ld, int src_dtype, const det_index_add_cfg* cfg, void* ws,
                  size_t ws_bytes, int atomic, void* stream);
/* Number of ids dropped as out of range (not -1) by the last det_index_add
 * that used this workspace. Synchronises `stream`; for tests and debugging.
 * No kernel of det_index_add waits for another workgroup (each stage hands
 * its results to the next through a kernel boundary), so a call cannot stall
 * on a busy GPU. */
int det_index_add_bad_ids(const void* ws, size_t ws_bytes, int64_t* count, void* stream);

/* ------------------------------------------------------------------------
 * det_indexer_dk: the sparse-indexer dK with its source rows made on the fly.
 * Megatron-LM PR #7441 (DSv4 deterministic mode), source 3 and its fix: the
 * deterministic indexer backward computes the clipped-log KL gradient of the
 * indexer scores, predict * sum(kept_target) - kept_target with the targets
 * clamped at e^-100 and a valid-slot mask, normalised by
 * loss_coeff / (B * S_q) * sm_scale * grad_loss, and accumulates dK over the
 * key ids without atomics. Per query row r and top-k slot j:
 *
 *   valid   = 0 <= ids[r][j] < n_rows
 *   kept    = valid ? max(target[r][j], EPS) : 0    EPS = 27 * 2^-149, the float32 nearest e^-100
 *   S_r     = ((-0 + kept[r][0]) + kept[r][1]) + ...  (slot order)
 *   c       = RN32(RN32(RN32(predict[r][j] * S_r) - kept) * scale)
 *   src     = RN32(c * q[r][d])                       (source row of slot (r, j))
 *   dk[id] += the det_index_add canonical order over the src rows of valid slots
 *
 * (chunks of chunk_rows rows in stable id order, folded left to right, one
 * add into dk[id]). scale is the caller's float32 product of loss_coeff /
 * (B * S_q), sm_scale and grad_loss (the score being sm_scale * q . k). The
 * bits equal det_index_add on the explicit float32 source rows.
 *
 * ids: [Q, K] int32, predict, target: [Q, K] float32, all contiguous (row
 *      stride K); K <= 1024. q: [Q, dim] bf16 (q_dtype DET_BF16; DET_F32 is
 *      DET_ERR_UNSUPPORTED), row stride q_ld >= dim, a multiple of 8, 16-byte
 *      aligned. dk: [n_rows, dim] float32, row stride dk_ld >= dim (multiple
 *      of 4, 16-byte aligned), accumulated. dim in {128, 256, 512},
 *      n_rows <= 16384.
 * cfg: NULL = {chunk_rows = 256}; chunk_rows in [1, 1024].
 * ws:  det_indexer_dk_workspace_size() bytes: the det_index_add workspace
 *      plus one float32 coefficient per slot; the atomic arm (per-element
 *      float atomics of the same products, no sort) needs the coefficients
 *      only. Bad ids are counted as for det_index_add (det_index_add_bad_ids
 *      reads the count from this workspace). */
int det_indexer_dk_workspace_size(int64_t Q, int64_t K, int64_t dim, int64_t n_rows, const det_index_add_cfg* cfg,
                                  int atomic, size_t* bytes);
int det_indexer_dk(float* dk, int64_t n_rows, int64_t dim, int64_t dk_ld, const int32_t* ids, const float* predict,
                   const float* target, int64_t Q, int64_t K, const void* q, int64_t q_ld, int q_dtype, float scale,
                   const det_index_add_cfg* cfg, void* ws, size_t ws_bytes, int atomic, void* stream);

/* ------------------------------------------------------------------------
 * det_grouped_dprob: dprob of a grouped-GEMM dsReLU backward.
 * cudnn-frontend PR #521 (deterministic dprob): each N tile of a token gets
 * its own slot with a single writer, each subtile's partial is stored by its
 * subtile index, and the slots are folded in one fixed order and added into
 * the existing dprob.
 *
 *   dprob[m] += sum_n dY[m,n] * relu(C[m,n])^2     for offs[0] <= m < offs[E]
 *
 * Canonical order: term = dY * (c*c if c > 0 else +0); per 128-wide N tile
 * the adjacent pairwise tree of its terms (n >= N is -0.0); the tiles folded
 * left to right; one add into dprob[m]. Rows outside [offs[0], offs[E])
 * (clamped to [0, M]) are untouched. offs: [E+1] int32 device array, read
 * only by the kernel (no host sync); rows are independent, so the grouping
 * never changes a bit.
 *
 * dY, C: [M, N] bf16, row strides ldy, ldc >= N (elements).
 * dprob: [M] float32, accumulated.
 * cfg:   NULL = {tile_n = 128, rows_per_wg = 4}; tile_n must be 128;
 *        rows_per_wg in [1, 1024] only shapes the launch.
 * ws:    the deterministic route keeps every slot on chip and needs no
 *        workspace (size 0); ws may be NULL. */
typedef struct {
  int32_t tile_n;
  int32_t rows_per_wg;
} det_dprob_cfg;

int det_grouped_dprob_workspace_size(int64_t M, int64_t N, const det_dprob_cfg* cfg, int atomic, size_t* bytes);
int det_grouped_dprob(float* dprob, const void* dY, int64_t ldy, const void* C, int64_t ldc, int64_t M, int64_t N,
                      const int32_t* offs, int32_t E, const det_dprob_cfg* cfg, void* ws, size_t ws_bytes,
                      int atomic, void* stream);

/* ------------------------------------------------------------------------
 * det_grouped_dbias: dbias of a grouped-GEMM dsReLU backward.
 * cudnn-frontend PR #521, the commit that extends the determinism flag to
 * dbias: dbias contends across M tiles, so each (M block, column) gets its
 * own float32 slot with a single writer, followed by a per-expert segment sum
 * of the slots; experts start on M-tile boundaries, so no tile holds rows of
 * two experts.
 *
 *   dbias[e][n] += sum_{offs[e] <= m < offs[e+1]} dA[m][n]
 *
 * Canonical order: expert bounds b_0 = clamp(offs[0], 0, M), b_e =
 * clamp(offs[e], b_{e-1}, M) (read on the device only); expert e's rows cut
 * into tiles of block_m rows counted from b_e (with block_m-aligned experts
 * these are the absolute M blocks); per tile and column the adjacent pairwise
 * tree of its block_m values (rows past the expert are -0.0); the expert's
 * tile slots folded left to right; one add into dbias[e][n]. An expert with
 * no rows leaves dbias[e] untouched. block_m changes the bits; block_n only
 * shapes the launch.
 *
 * dA:    [M, N] bf16, row stride lda >= N; N and lda multiples of 8 and dA
 *        16-byte aligned (DET_ERR_UNSUPPORTED otherwise).
 * dbias: [E, N] float32, row stride ld_e >= N, accumulated.
 * offs:  [E+1] int32 device array; E <= 65535.
 * cfg:   block_m in {64, 128, 256}; block_n (columns per workgroup) in
 *        {128, 256, 512}. NULL = block_m 128 and the widest block_n that
 *        still gives (ceil(M / 128) + E) x ceil(N / block_n) >= 2048
 *        workgroups, else 128 (a shape-only rule; block_n never changes a
 *        bit).
 * ws:    the deterministic route needs det_grouped_dbias_workspace_size()
 *        bytes: the header, the per-expert tile starts and one float32 slot
 *        per possible tile and column, (ceil(M / block_m) + E) x N.
 *        atomic = 1 needs none (the tile partials are added with float
 *        atomics). */
typedef struct {
  int32_t block_m;
  int32_t block_n;
} det_dbias_cfg;

int det_grouped_dbias_workspace_size(int64_t M, int64_t N, int32_t E, const det_dbias_cfg* cfg, int atomic,
                                     size_t* bytes);
int det_grouped_dbias(float* dbias, int64_t ld_e, const void* dA, int64_t lda, int64_t M, int64_t N,
                      const int32_t* offs, int32_t E, const det_dbias_cfg* cfg, void* ws, size_t ws_bytes, int atomic,
                      void* stream);

/* ------------------------------------------------------------------------
 * det_grouped_wgrad_acc: main_grad[e] += G_e^T X_e with fixed-order split-K.
 * FlashInfer PR #8602 (fused fp32 weight-gradient accumulate into main_grad)
 * and #8924 (deterministic accumulate: bitwise AccumulateGrad of the
 * deterministic dW, identical from run to run; expert offsets on the device).
 *
 * Expert e owns token rows [offs[e], offs[e+1]) of G [T_total, M] and
 * X [T_total, N] (bf16, row strides ldg >= M, ldx >= N). Its rows are cut into
 * K tiles of k_tile (= 512) rows counted from the expert's first row, and
 * ktiles_per_split consecutive K tiles form one split (0 = one split per
 * expert). Each split's partial Q_s = G_s^T X_s is computed on the matrix
 * cores in ascending row order from +0.0; then
 *   main_grad[e] <- RN32(main_grad[e] + (((Q_0 + Q_1) + Q_2) + ...)).
 * block_m and block_n only shape the launch.
 *
 * main_grad: [E, M, N] float32, element (e,i,j) at e*ld_e + i*ld_m + j;
 *            ld_m >= N, ld_e >= M*ld_m (so an expanded tensor is rejected).
 * offs: [E+1] int32 device array, non-decreasing, offs[E] <= T_total.
 *       Values are read on the device only; out-of-range offsets are clamped.
 * M must be a multiple of 128 and N of block_n (the workgroup tile); ldg,
 * ldx, ld_m and ld_e keep every row 16-byte aligned, as do G, X and
 * main_grad; T_total < 2^30 and (T_total + 512) * max(ldg, ldx) * 2 < 2^31
 * (32-bit buffer offsets). Otherwise DET_ERR_UNSUPPORTED.
 * cfg:  NULL selects {block_m = 256, block_n = 256, k_tile = 512,
 *       ktiles_per_split = 0}; block_m x block_n must be 256 x 256, 128 x 256
 *       or 128 x 512 (the tile only shapes the launch: all give the same
 *       bits), k_tile 512, ktiles_per_split in [0, 2^20].
 * ws:   ktiles_per_split = 0 keeps each expert's partial in registers and
 *       needs no workspace (size 0); otherwise the 256-byte header plus one
 *       [M, N] float32 slot per possible split, ceil(T_total / (512 C)) + E
 *       slots. atomic = 1 needs none. */
typedef struct {
  int32_t block_m;
  int32_t block_n;
  int32_t k_tile;
  int32_t ktiles_per_split;
} det_wgrad_cfg;

int det_grouped_wgrad_acc_workspace_size(int64_t T_total, int32_t E, int64_t M, int64_t N, const det_wgrad_cfg* cfg,
                                         int atomic, size_t* bytes);
int det_grouped_wgrad_acc(float* main_grad, int64_t ld_e, int64_t ld_m, const void* G, int64_t ldg, const void* X,
                          int64_t ldx, const int32_t* offs, int32_t E, int64_t T_total, int64_t M, int64_t N,
                          const det_wgrad_cfg* cfg, void* ws, size_t ws_bytes, int atomic, void* stream);

/* det_grouped_wgrad_acc_bf16: the same grouped weight gradient accumulated
 * into a bf16 main_grad. FlashInfer PR #8924, "Design and numerics": for a
 * bf16 output the bf16 dW is added in bf16, bitwise the AccumulateGrad of the
 * deterministic dW. Here dW[e] is the float32 fold of the expert's split
 * partials exactly as in det_grouped_wgrad_acc; then, per element,
 *
 *   main_grad <- RN_bf16( RN32( main_grad + RN_bf16(dW) ) )
 *
 * (RN_bf16: round to nearest even, NaN kept). Experts with no rows keep their
 * bits. Every split's partial goes to the workspace (also with
 * ktiles_per_split = 0, one split per expert) and one fold kernel adds.
 * main_grad: [E, M, N] bf16 bits, strides (ld_e, ld_m, 1) in elements, both
 * multiples of 4, 8-byte aligned. No atomic arm. Other arguments and errors
 * as for det_grouped_wgrad_acc.
 * ws: det_grouped_wgrad_acc_bf16_workspace_size() bytes (max_splits x M x N
 *     float32: E x M x N with one split per expert). */
int det_grouped_wgrad_acc_bf16_workspace_size(int64_t T_total, int32_t E, int64_t M, int64_t N,
                                              const det_wgrad_cfg* cfg, size_t* bytes);
int det_grouped_wgrad_acc_bf16(uint16_t* main_grad, int64_t ld_e, int64_t ld_m, const void* G, int64_t ldg,
                               const void* X, int64_t ldx, const int32_t* offs, int32_t E, int64_t T_total,
                               int64_t M, int64_t N, const det_wgrad_cfg* cfg, void* ws, size_t ws_bytes,
                               void* stream);

/* ------------------------------------------------------------------------
 * det_topk_canonicalize: canonical order of a compact indexer top-k.
 * Megatron-LM PR #7441 (DSv4 deterministic mode), source 1 and its fix: a
 * row's selected ids, and so the terms of its softmax sum, came out in an
 * order that varied between runs; every row is put in one canonical order
 * (padding at the end, logits moved alongside), its softmax is summed again
 * in that order, and a row without a valid id gets probabilities of zero.
 *
 * Canonical order per row: slots with a valid id (>= 0) by ascending id,
 * equal ids by ascending slot, then the padding slots (negative ids) by slot.
 * ids_out and logits_out are the row's ids and logits in that order. With
 * m = the largest valid logit, e_j = exp32(logit_j - m) (the fixed float32
 * sequence of det_colsum), S = the left-to-right sum of the e_j in that order,
 * probs_j = e_j / S (one correctly rounded division) for valid slots and +0.0
 * for padding; a row with no valid id gets all +0.0. Distinct ids in any slot
 * order give the same bits.
 *
 * ids: [Q, K] int32, logits: [Q, K] float32, row stride ld >= K (elements).
 * ids_out: [Q, K] int32, logits_out, probs: [Q, K] float32, row stride
 *          ld_out >= K; outputs must not overlap the inputs or each other.
 * K <= 1024 (DET_ERR_UNSUPPORTED otherwise). No workspace. The entry point is
 * deterministic by construction and has no atomic arm. */
int det_topk_canonicalize(const int32_t* ids, const float* logits, int64_t Q, int64_t K, int64_t ld,
                          int32_t* ids_out, float* logits_out, float* probs, int64_t ld_out, void* stream);

/* ------------------------------------------------------------------------
 * Diagnostics (tests only). det_detmath_eval evaluates the device versions of
 * the gate's exp / log1p / softplus / sigmoid sequences elementwise:
 * fn = 0 exp32, 1 log1p32, 2 softplus32, 3 sigmoid32. x, y: [n] float32
 * device arrays that must not overlap. Lets a test compare the GPU's bits
 * with the CPU oracle's over any sample of inputs. */
int det_detmath_eval(const float* x, float* y, int64_t n, int fn, void* stream);

/* det_mfma_eval runs chains of the weight gradient's matrix-core instruction
 * (v_mfma_f32_32x32x16_bf16) on plain operands, for the tests that pin the
 * oracle's model of that instruction (the pages say nothing about matrix-core
 * rounding; FlashInfer PR #8924 makes the deterministic dW's bits part of the
 * contract). For q < n: acc = C[q]; for b = 0..kblocks-1,
 * acc = mfma(A[q][:, 16b:16b+16], B[q][16b:16b+16, :], acc); D[q] = acc.
 * k = 8 kg + e inside a block is the operand element e of lane group kg, which
 * is token row 16b + k of a weight-gradient block.
 * A: [n][32][16 kblocks] bf16 bits, B: [n][16 kblocks][32] bf16 bits,
 * C, D: [n][32][32] float32; all row-major, contiguous, device memory; D must
 * not overlap the inputs. kblocks in [1, 4096]. */
int det_mfma_eval(const uint16_t* A, const uint16_t* B, const float* C, float* D, int64_t n, int kblocks,
                  void* stream);

/* det_mfma_rate is a measurement aid, not part of any reduction: `blocks`
 * workgroups of four waves, each wave holding four A and four B fragments of
 * the weight gradient's instruction (bf16 values from `ops`, read once) and
 * running `iters` rounds of the 4 x 4 pattern of MFMAs into sixteen
 * accumulators, with no memory traffic in the loop: 16 * 32768 flops per wave
 * and round. It times the matrix cores on the caller's operand values (their
 * power, and so the clock they allow, depends on those values). out[w*64 + l]
 * receives lane l of wave w's accumulator sum.
 * ops: >= 64*64*64 bf16 values, device memory; out: >= 256 * blocks floats,
 * not overlapping ops. blocks in [1, 2^20], iters in [0, 2^24]. */
int det_mfma_rate(const uint16_t* ops, int64_t n_ops, float* out, int64_t n_out, int blocks, int iters, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DETGRAD_H */
