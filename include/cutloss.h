/*
 * cutloss — fused large-vocabulary classifier-head losses for AMD Instinct MI355X (gfx950).
 *
 * Computes the loss and gradients of a classifier head over the logits X = A E^T
 * (A[T,D] activations, E[V,D] item/class embeddings) without ever storing the
 * T x V logits in device memory: logit tiles are formed on chip, reduced, and
 * recomputed in the backward pass.
 *
 * Operations and the passages that define them:
 *  - Multi-label BCE over the whole vocabulary, split into a dense background
 *    sum_v softplus(x_tv) and a sparse correction -sum_{p in P_t} x_tp
 *    (Cut Binary Cross Entropy, paperpeel: §I-B "Fused Direct BCE Formulation",
 *    §III-A vocabulary chunking, §III-B custom-VJP rematerialization).
 *  - Softmax cross-entropy as logsumexp(x_t) - x_{t,y_t}, the target logit by an
 *    indexed dot product and the logsumexp by an online max/sum over vocabulary
 *    tiles (Cut Your Losses, abeam.tech article: the sections on splitting the
 *    loss into two needed quantities and on recomputing tiles in backward).
 *  - BCE backward fused with a momentum-free SGD step on the embeddings, so dE
 *    is never stored; E may be FP8 E4M3 (ELMO, ai.info summary: Key
 *    Contributions 1-2 and Methodology).
 *
 * Conventions
 *  - Every data pointer is a DEVICE pointer and must be 16-byte aligned. The
 *    caller owns every buffer; the library never allocates device memory. Scratch
 *    space comes from the caller's workspace, sized by the *_workspace_size query.
 *  - Matrices are row-major and dense: A is [T, D] bf16; E is [V, D] bf16 or OCP FP8
 *    E4M3FN (1 byte); dA is [T, D] bf16; dE is [V, D] bf16. D must be a positive
 *    multiple of 64 (at most 9216). loss/lse/dloss are [T] float32.
 *  - All work is enqueued on `stream` (a hipStream_t, NULL = default stream);
 *    no call synchronizes except cutloss_read_data_errors.
 *  - Host-detectable errors (bad sizes, NULL or misaligned pointers, too small a
 *    workspace, unsupported dtype) return a status before anything is launched.
 *    Data errors found on the device (IDs outside [0, V), malformed CSR rows) are
 *    counted in the workspace and the offending entries are ignored.
 *  - The per-row loss is the sum over the vocabulary; the library applies no
 *    batch reduction. A caller's mean or weighting is expressed through dloss
 *    (dloss_t = dL/dloss_t; NULL means 1 for every row).
 *  - Masked (BCE) and ignored (CE) rows give loss 0, a zero dA row and no dE
 *    contribution.
 *  - Results are deterministic: every reduction runs in a fixed order.
 *  - Paths: heads with D in {64, 128, 256} and bf16 E run fused logit-tile sweeps that
 *    never write a logit; every other head (any D that is a multiple of 64, or FP8 E)
 *    runs a chunked path that keeps one vocabulary chunk's bf16 gradient tile
 *    (T x Vc) in the workspace: Vc is at most ceil(V / 8) items rounded up to 256, so the
 *    tile holds at most about an eighth of the T x V logits, and the tile is at most
 *    2 GiB. A forward stores no tile and runs the vocabulary as one chunk. The environment
 *    variable CUTLOSS_MAX_CHUNK_ITEMS caps Vc further (read when a call or size query plans
 *    the work, so set it before both).
 */
#ifndef CUTLOSS_H
#define CUTLOSS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  CUTLOSS_OK = 0,
  CUTLOSS_ERR_INVALID_ARG = 1,  /* a NULL/misaligned pointer or a bad size */
  CUTLOSS_ERR_UNSUPPORTED = 2,  /* a valid request the library does not implement (e.g. D % 64 != 0) */
  CUTLOSS_ERR_WORKSPACE = 3,    /* workspace smaller than the size query returned */
  CUTLOSS_ERR_HIP = 4           /* a HIP launch/runtime error; text in cutloss_last_error() */
} cutloss_status;

typedef enum {
  CUTLOSS_BF16 = 0,
  CUTLOSS_FP8_E4M3 = 1          /* OCP E4M3FN: bias 7, no infinities, max 448 */
} cutloss_dtype;

/* Operation codes for the workspace queries. */
typedef enum {
  CUTLOSS_OP_FWD = 0,
  CUTLOSS_OP_BWD = 1,
  CUTLOSS_OP_BWD_SGD = 2,
  CUTLOSS_OP_FWD_METRICS = 3,
  CUTLOSS_OP_BWD_SGD_EX = 4
} cutloss_op;

/* Rounding of the SGD writeback. */
typedef enum {
  CUTLOSS_ROUND_NEAREST_EVEN = 0,
  CUTLOSS_ROUND_STOCHASTIC = 1
} cutloss_rounding;

/* Options of cutloss_bce_bwd_sgd_ex (NULL: nearest-even, bf16 x FP8 logits, as cutloss_bce_bwd_sgd). */
typedef struct {
  int32_t rounding;     /* cutloss_rounding */
  uint64_t seed;        /* stochastic rounding key: pass a new seed every step */
  int32_t fp8_logits;   /* 1: A is cast to FP8 E4M3FN for the logit product (FP8 E only) */
} cutloss_sgd_options;

/*
 * Multi-label BCE problem. The positives of row t are pos_ids[pos_row_ptr[t] ..
 * pos_row_ptr[t+1]) in any order; pad_id entries are not positives, repeats count
 * once (Cut BCE §III-B/§III-E/§IV-A). Rows with row_mask[t] == 0 are padding rows.
 */
typedef struct {
  int64_t T, D, V;
  const void* A;                 /* [T, D] bf16 */
  const void* E;                 /* [V, D] bf16 or fp8 (per e_dtype); updated in place by bwd_sgd */
  cutloss_dtype e_dtype;
  const int32_t* pos_row_ptr;    /* [T+1], pos_row_ptr[0] = 0, non-decreasing */
  const int32_t* pos_ids;        /* [nnz] item IDs */
  int64_t nnz;                   /* = pos_row_ptr[T]; passed by the caller (the host never reads device memory) */
  const uint8_t* row_mask;       /* [T], 1 = valid row; NULL = all rows valid */
  int32_t pad_id;                /* padding item ID (not a positive); < 0 = none */
} cutloss_bce_problem;

/* Softmax cross-entropy problem: one class target per row. */
typedef struct {
  int64_t T, D, V;
  const void* A;                 /* [T, D] bf16 */
  const void* E;                 /* [V, D] bf16 or fp8 */
  cutloss_dtype e_dtype;
  const int64_t* target;         /* [T] class IDs in [0, V), or ignore_index */
  int64_t ignore_index;          /* e.g. -100 */
} cutloss_ce_problem;

/*
 * Workspace size in bytes for `op` on problem `p` (0 if the problem is invalid).
 * On the fused-sweep path it grows with T, D, nnz and the vocabulary tile count, never
 * with T*V; the chunked path's backward adds one chunk's gradient tile (at most
 * T * ceil(V/8) bf16 values, at most 2 GiB) and the chunk's transposed E.
 */
size_t cutloss_bce_workspace_size(const cutloss_bce_problem* p, int32_t op);
size_t cutloss_ce_workspace_size(const cutloss_ce_problem* p, int32_t op);

/*
 * BCE forward: loss[t] = sum_v softplus(x_tv) - sum_{p in P_t} x_tp (0 on masked rows).
 * Cut BCE §I-B (dense background + sparse correction), §III-A (vocabulary tiles).
 */
cutloss_status cutloss_bce_fwd(const cutloss_bce_problem* p, float* loss,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * BCE forward with Cut Metrics (Cut Binary Cross Entropy, paperpeel, §III-D): besides
 * loss (as cutloss_bce_fwd), counts[t] = (TP, FP, FN, TN) for row t, the confusion
 * counts over the V items of the predictions sigmoid(x_tv) > 0.5, i.e. x_tv > 0, against
 * the canonical positive set P_t. Computed in the same pass as the loss; no logits are
 * stored. Masked rows give (0, 0, 0, 0). counts: int32 [T][4], device, 16-byte aligned.
 * A logit within fp32 rounding of 0 may be decided either way, and a positive's decision
 * may differ between the dense count and the indexed dot product (FP is kept >= 0).
 * Requires V < 2^24 (CUTLOSS_ERR_UNSUPPORTED otherwise).
 * Workspace: cutloss_bce_workspace_size(p, CUTLOSS_OP_FWD_METRICS).
 */
cutloss_status cutloss_bce_fwd_metrics(const cutloss_bce_problem* p, float* loss, int32_t* counts,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * BCE backward: with G = w (sigmoid(X) - Y), w_t = dloss_t * mask_t,
 * dA = G E (bf16 [T,D]) and dE = G^T A (bf16 [V,D]). Logit tiles are recomputed
 * (Cut BCE §III-B/§III-C). If loss_out is not NULL the forward loss is emitted by
 * the same pass (fused forward+backward). dA or dE may be NULL to skip it.
 */
cutloss_status cutloss_bce_bwd(const cutloss_bce_problem* p, const float* dloss,
                               void* dA, void* dE, float* loss_out,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * cutloss_bce_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation). Same arguments, outputs
 * and kernels, without a workspace argument: the scratch space is a fixed array inside the
 * library, 64 MiB per GPU (CUTLOSS_STATIC_SCRATCH_BYTES), created with the library's code
 * on each GPU it runs on and held until the process ends. Nothing is allocated by the call.
 * A problem whose cutloss_bce_workspace_size(p, CUTLOSS_OP_BWD) exceeds that size returns
 * CUTLOSS_ERR_WORKSPACE before anything is launched. The array belongs to the device that
 * is current when the call is made, and `stream` must belong to that device. Every call on
 * one GPU shares the array, which keeps the last call's contents (each call sets up what it
 * reads): calls that overlap on one GPU (on different streams, or from several host threads
 * without ordering) race and give undefined results. Data errors are counted but cannot be
 * read back (cutloss_read_data_errors needs a caller workspace).
 */
#define CUTLOSS_STATIC_SCRATCH_BYTES (64ull << 20)
cutloss_status cutloss_bce_bwd_noalloc(const cutloss_bce_problem* p, const float* dloss,
                                       void* dA, void* dE, float* loss_out, void* stream);

/*
 * BCE backward fused with SGD on E: E <- round(E - lr * dE), dE never stored
 * (ELMO summary, Key Contributions 2: gradient fusion; Methodology: momentum-free
 * SGD, FP8 E4M3 weights). Rounding to E's dtype is nearest-even; FP8 saturates at
 * +-448. E (p->E) is modified in place, so the call is not idempotent. dA (bf16)
 * and loss_out are optional outputs as in cutloss_bce_bwd.
 */
cutloss_status cutloss_bce_bwd_sgd(const cutloss_bce_problem* p, const float* dloss, float lr,
                                   void* dA, float* loss_out,
                                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * cutloss_bce_bwd_sgd with ELMO's low-precision options (ELMO summary, Key Contributions 1
 * and Methodology):
 *  - rounding = CUTLOSS_ROUND_STOCHASTIC rounds E' stochastically, so that small updates are
 *    kept on average. With y = E_vd - lr dE_vd (FP8: clamped to +-448) and lo <= y <= hi its
 *    neighbours on E's storage grid, E'_vd = hi exactly when u (hi - lo) < y - lo, where
 *    u = h / 2^16 and h is the 16-bit half-word (d mod 8) (low half first) of the
 *    Philox-4x32-10 output (Salmon et al., SC 2011) for counter (d / 8, v mod 2^32, v / 2^32,
 *    0) and key (seed mod 2^32, seed / 2^32). y on the grid is kept; zero is stored as +0. The
 *    result is a deterministic function of (seed, v, d) and the update. BF16 E assumes
 *    finite, normal-range values.
 *  - fp8_logits = 1 casts A to FP8 E4M3FN (nearest-even, saturating) for the matmul that
 *    produces the logits, which then runs on the FP8 MFMA with FP8 E; the loss and
 *    G = w (sigmoid(X) - Y) come from those logits, dA = G E, and dE = G^T A uses A itself.
 *    Requires FP8 E (CUTLOSS_ERR_UNSUPPORTED otherwise).
 * Runs the chunked path for every D. Workspace: cutloss_bce_workspace_size(p,
 * CUTLOSS_OP_BWD_SGD_EX), which covers every option.
 */
cutloss_status cutloss_bce_bwd_sgd_ex(const cutloss_bce_problem* p, const float* dloss, float lr,
                                      const cutloss_sgd_options* opt, void* dA, float* loss_out,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * Softmax CE forward: lse[t] = logsumexp_v x_tv (every row), loss[t] = lse[t] - x_{t,y_t}
 * (0 on ignored rows). Cut Your Losses article: target logit by an indexed dot
 * product, logsumexp by an online max/sum over vocabulary tiles.
 */
cutloss_status cutloss_ce_fwd(const cutloss_ce_problem* p, float* loss, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Softmax CE backward from the forward's lse: G = w (softmax(X) - onehot(y)),
 * dA = G E, dE = G^T A (bf16). dA or dE may be NULL to skip it.
 */
cutloss_status cutloss_ce_bwd(const cutloss_ce_problem* p, const float* lse, const float* dloss,
                              void* dA, void* dE,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Softmax CE backward with the gradient filter (Cut Your Losses article, the note that the
 * softmax tail below numerical precision contributes negligibly to the gradient and its
 * computation may be skipped). As cutloss_ce_bwd, except that the matrix work of a logit
 * tile whose entries all have |w_t softmax_tv| < grad_filter_eps is skipped for both dA and
 * dE (the tile's dense terms are dropped; the -1 target terms never are). Tiles are 32 x 32
 * per wave on the fused-sweep path (D in {64, 128, 256}) and the products' stage tiles on
 * the chunked path. An approximation by design: the dropped sum is bounded by
 * sum over entries below eps of |w_t softmax_tv| |E_v| (dA) or |A_t| (dE).
 * grad_filter_eps in [0, 1]; 0 gives the exact cutloss_ce_bwd result.
 * Workspace: cutloss_ce_workspace_size(p, CUTLOSS_OP_BWD).
 */
cutloss_status cutloss_ce_bwd_filtered(const cutloss_ce_problem* p, const float* lse, const float* dloss,
                                       void* dA, void* dE, float grad_filter_eps,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Number of data errors counted by the last call that used this workspace
 * (positive IDs / targets outside [0, V), malformed CSR rows). Synchronizes `stream`.
 */
cutloss_status cutloss_read_data_errors(const void* workspace, void* stream, int64_t* n_errors);

/*
 * Test hook: canonical positive sets of a BCE problem as computed on the device.
 * Writes the canonical CSR (crow[T+1], cids[nnz'] sorted ascending within rows, no
 * pads, repeats or masked rows) and the item-major pairs (items[nnz'], rows[nnz'],
 * ordered by item then row) into the given device buffers (each sized for nnz
 * entries), and *n_unique_pairs = nnz' (synchronizes `stream`).
 */
cutloss_status cutloss_bce_canonical_targets(const cutloss_bce_problem* p,
                                             int32_t* crow, int32_t* cids,
                                             int32_t* items, int32_t* rows, int64_t* n_unique_pairs,
                                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * Test hook: the sparse correction's positive logits as the loss computes them
 * (Cut Binary Cross Entropy, Section I-B, fused direct BCE formulation: the loss is the
 * dense softplus sum minus the sum of the logits of a row's positives).
 * Canonicalizes the positive sets as cutloss_bce_canonical_targets does, then writes
 * sum_x[t] = sum over the canonical positives p of row t of x_tp = A_t . E_p (fp32, summed
 * in ascending item order; 0 for masked rows and rows without positives) and, if x_pos is
 * not NULL, x_pos[e] = x_tp for every canonical pair e in the order of the canonical CSR
 * (rows ascending, items ascending within a row; at most nnz entries). sum_x holds T floats,
 * x_pos nnz floats, both device memory owned by the caller. The workspace holds only the
 * canonical targets: cutloss_bce_workspace_size(p, op) of any op suffices. Asynchronous on
 * `stream`; data errors are counted as by the other entry points.
 */
cutloss_status cutloss_bce_positive_logits(const cutloss_bce_problem* p, float* sum_x, float* x_pos,
                                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Profiling hook. While enabled (process-wide), every entry point records a HIP event
 * pair on the caller's stream around each of its kernel phases:
 *   0 target canonicalization, 1 rows sweep (loss/LSE partials, dA partials),
 *   2 row finalization (loss, lse, dA), 3 row weights + sparse item sums,
 *   4 cols sweep (dE or the fused SGD step); the chunked path records its three
 *   products per chunk as 5 logits + epilogue, 6 dA product, 7 dE product (or the
 *   fused SGD step; for FP8 E over at most 128 rows that step also forms dA, and phase 6
 *   records no launch).
 * cutloss_profile_read synchronizes on the recorded events, writes the summed
 * milliseconds and the number of recorded launches per phase (arrays of n entries),
 * and clears the records. Enabling costs one event record per phase boundary.
 */
enum { CUTLOSS_PHASE_TARGETS = 0, CUTLOSS_PHASE_ROWS = 1, CUTLOSS_PHASE_FINALIZE = 2,
       CUTLOSS_PHASE_ITEM_SUMS = 3, CUTLOSS_PHASE_COLS = 4, CUTLOSS_PHASE_CHUNK_LOGITS = 5,
       CUTLOSS_PHASE_CHUNK_DA = 6, CUTLOSS_PHASE_CHUNK_DE = 7, CUTLOSS_N_PHASES = 8 };
cutloss_status cutloss_profile_enable(int32_t enable);
cutloss_status cutloss_profile_read(float* ms, int32_t* launches, int32_t n);

const char* cutloss_status_string(cutloss_status s);
/* Text of the last error on the calling thread ("" if none). */
const char* cutloss_last_error(void);
/* Library version string. */
const char* cutloss_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CUTLOSS_H */
