// Internal launchers of the chunked GEMM path and of the row / item finalization shared by
// both paths (the fused sweeps need only common.h).
#pragma once
#include "common.h"

namespace cl {

// ----------------------------------------------------------------------------------
// Chunked path for wide heads (gemm.hip): three MFMA GEMMs per vocabulary chunk.
// An operand is stored row-major as [rows][cols] with leading dimension ld (elements):
// kc = 1 if its cols are the GEMM's K index (k contiguous), 0 if its rows are (k rows).
// Rows at or past rows_valid and column groups past cols_valid are read as copies of
// the last valid ones (never out of bounds); the GEMM masks or zero-pads them.
// ----------------------------------------------------------------------------------
struct GemmOperand {
  const void* p;
  int64_t ld, rows_valid, cols_valid;
  int kc;      // 1: [M or N][K]; 0: [K][M or N]
  int fp8;     // OCP E4M3FN storage (widened to bf16 when staged; with both operands FP8
               // and k-contiguous, copied as they are and multiplied by the FP8 MFMA)
  // bt > 0: blocked bf16 storage of the chunk's gradient tile P[t][v] (t = the stored row
  // index, v = the column): element (t, v) at ((t / bt) * nvb + v / 32) * bt * 32
  // + (t % bt) * 32 + v % 32, i.e. bt x 32 blocks, contiguous, ld unused
  int bt;
  int64_t nvb;
};

enum {
  GEMM_EPI_BCE_P = 0,     // logits (M = chunk items, N = rows): P = sigmoid(x) (unweighted), softplus partials
  GEMM_EPI_BCE_LOSS = 1,  // softplus partials only
  GEMM_EPI_CE_LSE = 2,    // running (max, sum) partials
  GEMM_EPI_CE_P = 3,      // P = w exp(x - lse)
  GEMM_EPI_ACC = 4,       // C (+)= acc into fp32 [M][N] (split-K slice per blockIdx.z)
  GEMM_EPI_DE = 5,        // dE rows of the chunk: acc - S_u, bf16
  GEMM_EPI_SGD = 6,       // E <- round(E - lr (acc - S_u)) in place
  GEMM_EPI_BCE_METRICS = 7  // softplus partials + counts of logits > 0 (as floats) in part_b
};

struct GemmParams {
  GemmOperand a, b;
  int64_t M, N, K;          // K a multiple of 32
  int64_t k_per_split;      // K range of one blockIdx.z slice (multiple of 32)
  int epi;
  // logits epilogues: chunk rows m map to items v0 + m (< V), cols n to rows t (< T)
  int64_t v0, V, T;
  const float* w;           // [T] row weights
  const float* lse;         // [T] CE logsumexp
  uint16_t* P;              // bf16 gradient tile of the chunk P[t][item], blocked as for a
  int p_bt;                 // GemmOperand with bt = p_bt, nvb = p_nvb; rows t < p_rows
  int64_t p_nvb, p_rows;
  float* part_a; float* part_b;  // [n_splits][T] row partials
  int64_t part_base;        // split index of this chunk's first item tile
  // ACC epilogue
  float* acc; int64_t ldacc; int64_t acc_slice;   // acc + z * acc_slice
  int acc_trans;            // 1: the product is dA^T (M = D, N = rows), stored as [row][d]
  int acc_first;            // 1: store, 0: add to the previous value
  // DE / SGD epilogues
  const int32_t* uitems; const int32_t* counts; const float* S_u; int64_t D;
  const int32_t* imap;      // [V] item -> unique-item index (-1: none); NULL: binary search of uitems
  void* dE; void* E_inplace; int e_fp8; float lr;
  int sr; uint64_t sr_seed;  // SGD: stochastic rounding keyed by (sr_seed, v, d) when sr != 0
  // CE gradient filter: the CE_P epilogue sets flags[tm * flag_ld + tn] = flag_gen for an
  // output tile (item tile tm, row tile tn of flag_bn rows) holding some |P| >= filter_eps;
  // the dA and dE products skip the matrix work of a k stage whose P tiles are unflagged.
  // flags == NULL: off.
  int32_t* flags; int64_t flag_ld; int flag_bn; int flag_gen; float filter_eps;
};
hipError_t launch_gemm(const GemmParams& p, hipStream_t st);
// A8 = E4M3FN(A), nearest-even, saturating at +-448; n a multiple of 8
hipError_t launch_cast_fp8(const uint16_t* A, int64_t n, uint8_t* A8, hipStream_t st);
// Et[d][v] = E[v][d] (bf16) for v < vlen, 0 for vlen <= v < mc; Et rows hold ld >= mc items.
// mc and D multiples of 64, ld a multiple of 8.
hipError_t launch_transpose_chunk(const uint16_t* E, int64_t vlen, int64_t mc, int64_t D, uint16_t* Et, int64_t ld,
                                  hipStream_t st);
int gemm_tile_m();                     // 256
int gemm_tile_n_of(int epi, int64_t M, int64_t N, int64_t D);   // 128 or 256 for that product

// ----------------------------------------------------------------------------------
// FP8 SGD product for heads of at most 128 rows (sgd_rows.hip): E <- E4M3(E - lr (P^T A_w
// - S)) with nearest-even or stochastic rounding, whole E rows of 32 items per workgroup.
// ----------------------------------------------------------------------------------
struct SgdRowsParams {
  int64_t V;             // items; rows at or past V are neither read for real nor written
  int64_t v0;            // first item of the chunk
  int64_t nblk;          // 32-item blocks of the chunk (the grid)
  int D;                 // a multiple of 128, at most 1024
  const uint16_t* P;     // the chunk's gradient tile in blocks of 128 rows x 32 items (bt = 128)
  const uint16_t* AwT;   // [D][128] bf16: bf16(w_t A[t][d]) for t < T, 0 past T
  const float* S_u;      // [unique items][D] positive-row sums
  const int32_t* imap;   // [V] item -> unique-item index, -1 for none
  uint8_t* E;            // [V][D] E4M3FN, updated in place
  float lr;
  int sr; uint64_t sr_seed;   // stochastic rounding keyed by (sr_seed, v, d) when sr != 0, else nearest-even
  // dA (optional): dA_part[r][t][d] (r < dA_splits, t < T) += sum over the items that block
  // row r of the chunk covers of P[t][v] E[v][d], E read before its update; dA_first: the
  // chunk starts the sums (its partials are stored, not added to). NULL: no dA.
  int64_t T;
  float* dA_part;
  int64_t dA_splits;
  int dA_first;
};
bool sgd_rows_supported(int64_t Tp, int64_t D);   // Tp: rows of the gradient tile (128)
// the dA partials of a head whose first chunk has nblk 32-item blocks: one per block row
int64_t sgd_rows_dA_splits(int64_t nblk, int64_t D, int sr);

// ----------------------------------------------------------------------------------
// BCE logits product for FP8 E and heads of at most 128 rows (logits_rows.hip): loss
// partials and (P != NULL) the unweighted sigmoid tile, streaming 32-item blocks of E.
// ----------------------------------------------------------------------------------
struct LogitsRowsParams {
  int64_t V, T;          // items, rows (1 .. 128)
  int64_t v0;            // first item of the chunk
  int64_t nblk;          // 32-item blocks of the chunk's P region: 8 * nslots
  int64_t nslots;        // the chunk's loss slots: its 256-item tiles
  int64_t part_base;     // the chunk's first slot (v0 / 256)
  int D;                 // a multiple of 128, at most 768
  const uint8_t* E;      // [V][D] E4M3FN
  const uint16_t* A;     // [T][D] bf16
  uint16_t* P;           // the chunk's gradient tile in 128 x 32 blocks, or NULL
  float* part_a;         // [slots][T] softplus partials
  float* part_b;         // [slots][T] counts of positive logits (Cut Metrics forward), or NULL
};
bool logits_rows_supported(int64_t Tp, int64_t D);
hipError_t launch_logits_rows(const LogitsRowsParams& p, hipStream_t st);
hipError_t launch_weighted_transpose(const void* A, const float* w, int64_t T, int64_t D, uint16_t* AwT,
                                     hipStream_t st);
hipError_t launch_sgd_rows(const SgdRowsParams& p, hipStream_t st);

struct FinalizeParams {
  int64_t T, D, V;
  const void* A; const void* E; int e_fp8;
  const int32_t* crow; const int32_t* cids;   // canonical positives / targets
  const float* dloss; const uint8_t* mask;     // BCE
  const int64_t* ce_target; int64_t ignore_index;  // CE
  int n_splits;             // loss / lse partials
  int n_splits_dA;          // dA partials
  int dA_weighted;          // 1: dA partials already carry w_t (chunked CE path)
  const float* part_a; const float* part_b; const float* part_dA;
  float* loss; float* lse; void* dA;
  const float* lse_in;      // CE backward: lse from the forward
  float* w_out;             // [T] weights for the cols sweep
  // positive-row terms computed before E changes (chunked path): if set, finalize reads
  // them instead of E: pos_dot[t] = sum_p A_t . E_p, pos_sum[t][d] = sum_p E_p[d]
  float* pos_dot; float* pos_sum;
  float* pos_x;             // k_row_positives only, if set: x_tp per canonical positive (cids order)
  // Cut Metrics: per-split counts of logits > 0 (floats, exact below 2^24) in part_c, the
  // per-row positives with a positive logit (pos_tp, from k_row_positives when set), and
  // the output counts[T][4] = (TP, FP, FN, TN)
  const float* part_c; int32_t* pos_tp; int32_t* counts;
  // FP8 logits: the activations' E4M3FN copy [T][D] that the logit product uses; the
  // positive rows' logits are taken from it as well
  const uint8_t* A8;
};
hipError_t launch_row_positives(const FinalizeParams& p, hipStream_t st);
// kind: 0 = BCE, 1 = CE
hipError_t launch_finalize_rows(const FinalizeParams& p, int kind, int want_loss, int want_dA, hipStream_t st);
// Reduces split partials pa (and pb) [S][N] into their split-0 slice in a fixed order
// (groups of 64 splits, then groups of group sums). mode 1 merges logsumexp (max, sum)
// pairs. tmp holds reduce_splits_tmp_floats(S, N, mode) floats.
size_t reduce_splits_tmp_floats(int64_t S, int64_t N, int mode);
hipError_t launch_reduce_splits(float* pa, float* pb, int64_t S, int64_t N, float* tmp, int mode, hipStream_t st);
hipError_t launch_row_weights(const FinalizeParams& p, int kind, hipStream_t st);
// Aw[t][d] = bf16(w[t] * A[t][d]): the activations weighted per row (the BCE dE product's
// operand, so that the gradient tile can hold the unweighted sigmoid)
hipError_t launch_scale_rows(const void* A, const float* w, int64_t T, int64_t D, uint16_t* Aw, hipStream_t st);
// Sparse dE term S_u (one row per unique positive item); `part` holds
// 2 * item_sum_parts(nnz_cap) * D floats of piece partials.
size_t item_sum_parts(int64_t nnz_cap);
hipError_t launch_item_sums(int64_t D, int64_t nnz_cap, const void* A, const float* w,
                            const int32_t* csc_rows, const int32_t* useg, const int32_t* counts,
                            float* S_u, float* part, hipStream_t st);

}  // namespace cl
