// Shared device helpers and internal launcher declarations for the cutloss HIP library (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cutloss.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

#define CL_LDS __attribute__((address_space(3)))

namespace cl {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kFp8Max = 448.0f;

// v_mfma_f32_32x32x16_bf16. Lane l supplies A[m = l%32][k = 8*(l/32) + j] and
// B[k = 8*(l/32) + j][n = l%32], j = 0..7; the result register i of lane l is
// C[m = 8*(i/4) + 4*(l/32) + i%4][n = l%32].
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16: within each 16-lane group, lane j supplies the address of 4
// consecutive 16-bit elements; lane i receives element (i%4) of lanes i/4, 4+i/4,
// 8+i/4, 12+i/4. Loading rows k0..k0+3 (4 lanes per row, 4 columns each) hands lane
// i column i of those 4 rows.
__device__ __forceinline__ s16x4 lds_read_tr16(const char* lds_generic_base, uint32_t byte_off) {
  const CL_LDS char* p = (const CL_LDS char*)((uintptr_t)lds_generic_base) + byte_off;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((CL_LDS s16x4*)p);
}

__device__ __forceinline__ bf16x8 cat_bf16(s16x4 lo, s16x4 hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// 8 OCP E4M3FN bytes -> 8 bf16 (exact: every E4M3 value is a bf16 value).
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint2 q) {
  f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.x, false);
  f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.x, true);
  f32x2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.y, false);
  f32x2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)q.y, true);
  bf16x8 r = {(__bf16)a[0], (__bf16)a[1], (__bf16)b[0], (__bf16)b[1],
              (__bf16)c[0], (__bf16)c[1], (__bf16)d[0], (__bf16)d[1]};
  return r;
}

__device__ __forceinline__ float fp8_to_f32(uint32_t byte) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)byte, false)[0];
}

// float -> E4M3FN byte, nearest-even, saturating at +-448 (the hardware conversion
// alone turns |x| > 464 into NaN, so the input is clamped first).
__device__ __forceinline__ uint32_t f32_to_fp8_sat(float x) {
  x = __builtin_fminf(__builtin_fmaxf(x, -kFp8Max), kFp8Max);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(x, 0.0f, 0, false) & 0xffu;
}

__device__ __forceinline__ uint32_t f32_to_bf16_bits(float x) {
  __bf16 h = (__bf16)x;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ float wave_sum(float v) {
  // fixed butterfly order: deterministic
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace cl

// ----------------------------------------------------------------------------------
// internal launchers (defined in the .hip translation units)
// ----------------------------------------------------------------------------------
namespace cl {

struct TargetsWs {
  // all device pointers inside the caller's workspace
  unsigned long long* err;   // data-error counter
  int32_t* cnt;              // [T + 1]
  int32_t* off;              // [T + 1]
  int32_t* keyA; int32_t* valA;
  int32_t* keyB; int32_t* valB;
  int32_t* flags;            // [nnz + 1]
  int32_t* fscan;            // [nnz + 1]
  int32_t* hist;             // [256 * nblk_max]
  int32_t* hscan;            // [256 * nblk_max + 1]
  int32_t* csc_items; int32_t* csc_rows;  // [nnz]
  int32_t* uitems;           // [nnz]
  int32_t* useg;             // [nnz + 1]
  int32_t* crow;             // [T + 1]
  int32_t* cids;             // [nnz]
  int32_t* counts;           // [4]: 0 = valid pairs, 1 = unique pairs, 2 = unique items
};

// Canonicalize multi-label positives (BCE) or single targets (CE, when targets != NULL).
hipError_t launch_targets(const TargetsWs& w, int64_t T, int64_t V, int64_t nnz,
                          const int32_t* row_ptr, const int32_t* ids, const uint8_t* mask, int32_t pad_id,
                          const int64_t* ce_target, int64_t ignore_index, hipStream_t st);
size_t targets_radix_blocks(int64_t nnz);

hipError_t launch_zero_u64(unsigned long long* p, int n, hipStream_t st);
// zero n bytes (n a multiple of 4) with a kernel
hipError_t launch_zero_bytes(void* p, size_t n, hipStream_t st);
// map[v] = index of v among the unique positive items, -1 for every other item v < V
hipError_t launch_item_map(const TargetsWs& w, int64_t V, int64_t cap, int32_t* map, hipStream_t st);

struct SweepParams {
  int64_t T, D, V;
  const void* A;            // bf16 [T, D]
  const void* E;            // bf16 / fp8 [V, D]
  int e_fp8;
  // rows sweep (stationary A, streaming E)
  int n_splits;             // vocabulary splits
  int64_t split_len;        // columns per split (multiple of 32)
  float* part_a;            // [n_splits][T]: BCE dense-sum partials / CE running max
  float* part_b;            // [n_splits][T]: CE running sum
  float* part_dA;           // [n_splits][T][D] fp32, or NULL
  // cols sweep (stationary E, streaming A)
  const float* w;           // [T] per-row weight (mask * dloss); cols sweep
  const float* lse;         // [T] CE logsumexp (cols sweep and CE rows-backward)
  const int32_t* uitems;    // sorted unique positive items
  const int32_t* counts;    // counts[2] = number of unique items
  const float* S_u;         // [n_unique][D] sparse dE correction
  void* dE;                 // bf16 [V, D] output or NULL
  void* E_inplace;          // SGD target (== E) or NULL
  float lr;
  // CE gradient filter: a wave skips its gradient product for a chunk whose |P| values
  // (bf16 bit patterns) are all below filter_bits; 0 = off
  uint32_t filter_bits;
};

// Rows sweep modes: 0 = BCE loss partials, 1 = BCE dA partials, 2 = BCE dA + loss partials,
// 3 = CE (max, sum) partials, 4 = CE dA partials.
// Cols sweep: kind 0 = BCE, 1 = CE; epi 0 = write dE (bf16), 1 = SGD step on E in place.
// sweep2.hip: LDS-DMA sweeps (bf16 streamed operand, D in {64, 128, 256}).
hipError_t launch_sweep2_rows(const SweepParams& p, int mode, hipStream_t st);
hipError_t launch_sweep2_cols(const SweepParams& p, int kind, int epi, hipStream_t st);
bool sweep2_rows_supported(int64_t D, int e_fp8);
bool sweep2_cols_supported(int64_t D);
int sweep2_rows_per_block(int64_t D);   // stationary rows per workgroup of the LDS-DMA rows sweep

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
  GEMM_EPI_BCE_P = 0,     // logits (M = chunk items, N = rows): P = w sigmoid(x), softplus partials
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
// Et[d][v] = E[v][d] (bf16) for v < vlen, 0 for vlen <= v < mc; Et rows hold ld >= mc items.
// mc and D multiples of 64, ld a multiple of 8.
// A8 = E4M3FN(A), nearest-even, saturating at +-448; n a multiple of 8
hipError_t launch_cast_fp8(const uint16_t* A, int64_t n, uint8_t* A8, hipStream_t st);
hipError_t launch_transpose_chunk(const uint16_t* E, int64_t vlen, int64_t mc, int64_t D, uint16_t* Et, int64_t ld,
                                  hipStream_t st);
int gemm_tile_m();                     // 256
int gemm_tile_n_of(int epi, int64_t M, int64_t N, int64_t D);   // 128 or 256 for that product
// waves along M of the logits product (row partials per item tile) for T rows, head D
int gemm_k1_warps_m(int64_t T, int64_t D, bool fp8_fp8 = false);

struct FinalizeParams {
  int64_t T, D, V;
  const void* A; const void* E; int e_fp8;
  const int32_t* crow; const int32_t* cids;   // canonical positives / targets
  const float* dloss; const uint8_t* mask;     // BCE
  const int64_t* ce_target; int64_t ignore_index;  // CE
  int n_splits;             // loss / lse partials
  int n_splits_dA;          // dA partials
  int dA_weighted;          // 1: dA partials already carry w_t (chunked path)
  const float* part_a; const float* part_b; const float* part_dA;
  float* loss; float* lse; void* dA;
  const float* lse_in;      // CE backward: lse from the forward
  float* w_out;             // [T] weights for the cols sweep
  // positive-row terms computed before E changes (chunked path): if set, finalize reads
  // them instead of E: pos_dot[t] = sum_p A_t . E_p, pos_sum[t][d] = sum_p E_p[d]
  float* pos_dot; float* pos_sum;
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
// Sparse dE term S_u (one row per unique positive item); `part` holds
// 2 * item_sum_parts(nnz_cap) * D floats of piece partials.
size_t item_sum_parts(int64_t nnz_cap);
hipError_t launch_item_sums(int64_t D, int64_t nnz_cap, const void* A, const float* w,
                            const int32_t* csc_rows, const int32_t* useg, const int32_t* counts,
                            float* S_u, float* part, hipStream_t st);

}  // namespace cl
