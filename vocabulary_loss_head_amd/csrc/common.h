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

// LDS DMA: each active lane copies 16 (or 4) bytes from global address sbase + voff to LDS
// byte address lds + 16 * lane (4 * lane). sbase and lds are wave-uniform. Written as inline
// asm so that the compiler's wait insertion does not track these copies: it would otherwise
// wait for every copy in flight before each transposing LDS read (ds_read_b64_tr_b16), which
// it cannot tell apart from the copies' destinations. Callers order every read of a
// destination after the copy with an explicit vmcnt wait and a workgroup barrier. The
// s_nop covers the M0-write to LDS-DMA hazard. M0 is a reserved register (the compiler warns
// about the clobber); in the kernels that use these copies nothing else reads M0 (no
// builtin LDS copies, no relative register addressing, no messages), which the generated
// code shows, so no value of the compiler's own is overwritten.
__device__ __forceinline__ void lds_dma16(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}
// The same copy with the non-temporal hint, for data read once in a pass (the E stream of
// the small-row heads): it is kept from displacing data the next kernel reads again.
__device__ __forceinline__ void lds_dma16_nt(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :: "v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(voff), "s"(sbase), "s"(lds) : "memory", "m0");
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// 8 OCP E4M3FN bytes -> 8 bf16 (exact: every E4M3 value is a bf16 value).
// Two E4M3FN values (bytes 0-1, or 2-3 with HI, of w) to a bf16 pair in one instruction,
// exactly (every E4M3FN value is a bf16 value; scale 1). Inline asm: the compiler's builtin
// for this instruction treats its result as 16 bits wide and drops the second element.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  uint32_t r;
  if constexpr (HI) asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0 op_sel:[1,0,0]" : "=v"(r) : "v"(w));
  else asm("v_cvt_scalef32_pk_bf16_fp8 %0, %1, 1.0" : "=v"(r) : "v"(w));
  return r;
}

__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint2 q) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 r = {fp8x2_to_bf16x2<false>(q.x), fp8x2_to_bf16x2<true>(q.x), fp8x2_to_bf16x2<false>(q.y),
                   fp8x2_to_bf16x2<true>(q.y)};
  return __builtin_bit_cast(bf16x8, r);
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
bool sweep2_cols_supported(int64_t D, int e_fp8);
int sweep2_rows_per_block(int64_t D);   // stationary rows per workgroup of the LDS-DMA rows sweep
int sweep2_waves_per_block(int64_t D);  // waves per workgroup of the LDS-DMA sweeps

}  // namespace cl
