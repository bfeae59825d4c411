// FP8 SGD product of the chunked path for heads of at most 128 rows (the XMC head: T = 128,
// D = 768, V = 3M): E <- round_E4M3(E - lr (P^T A_w - S)) over one vocabulary chunk, the
// classifier update applied where its gradient is formed so that dE is never stored (ELMO,
// ai.info summary, Key Contributions 2 and Methodology; the sparse term S as in Cut Binary
// Cross Entropy §III-C).
//
// With so few rows the product is a stream over E: an item's update reads and writes one
// D-byte row of E and costs 2 T D flops. The general GEMM runs two workgroups per CU, each
// doing its loads, its matrix work and its epilogue in turn, and E moves at about 3 TB/s.
// Here a workgroup owns one 128-column slice of D and sweeps 32-item blocks of the chunk:
//  * its four waves hold the slice's weighted activations, A_w^T [128 columns][128 rows]
//    bf16, as the MFMA's B operand in registers for the whole sweep (32 VGPRs a lane);
//  * the chunk's gradient tile P is stored in blocks of 128 rows x 32 items (launch.h); a
//    block (8 KB), the 32 items' 128-byte slices of E (4 KB) and their unique-item indices
//    are copied into LDS with global_load_lds one block ahead, into two buffers, and each
//    block waits only for its own copies (an explicit vmcnt);
//  * the block is read transposed as the A operand (rows = items, k = t): 8 MFMAs a wave;
//  * the 32 x 128 result passes through LDS so that each of the 256 threads updates one
//    contiguous 16-byte piece of a row.
#include "launch.h"

#include <algorithm>

namespace cl {

namespace {

constexpr int kSgdItems = 32;                      // items per block
constexpr int kSgdRows = 128;                      // rows (k) of a gradient-tile block
constexpr int kSgdCols = 128;                      // columns of a workgroup's slice (4 waves x 32)
constexpr int kPRow = 2 * kSgdItems + 16;          // LDS stride of a block row (bytes)
constexpr int kPImg = 12 * 1024;                   // LDS image of a block: 10 KB used, 3 copies a wave
constexpr int kEImg = kSgdItems * kSgdCols;        // the items' slices of E: 32 x 128 bytes
constexpr int kMapImg = 4 * 256;                   // unique-item indices: one 256-byte slot a wave
constexpr int kStageRow = 4 * kSgdCols + 16;       // fp32 result row (+16 bytes)
constexpr int kOffE = 2 * kPImg;
constexpr int kOffMap = kOffE + 2 * kEImg;
constexpr int kOffStage = kOffMap + 2 * kMapImg;
constexpr int kLds = kOffStage + kSgdItems * kStageRow;
constexpr int kCopies = 5;                         // copy instructions a wave issues per block

__device__ __forceinline__ uint32_t lds_u32(const void* p) { return (uint32_t)(uintptr_t)p; }

// s_waitcnt vmcnt(N): gfx9 encoding, vmcnt[3:0] at bits 3:0 and vmcnt[5:4] at 15:14
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0xF70 | (N & 15) | ((N >> 4) << 14));
}

__device__ __forceinline__ s16x4 read_tr16(uint32_t lds) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((CL_LDS s16x4*)(uintptr_t)lds);
}

// A_w^T[d][t] = bf16(w_t A[t][d]) for t < T and 0 for T <= t < 128: the same rounding of
// the same product as the row-major weighted activations of the general path.
__global__ __launch_bounds__(256) void k_weighted_t(const uint16_t* __restrict__ A, const float* __restrict__ w,
                                                    int64_t T, int64_t D, uint16_t* __restrict__ AwT) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= D * kSgdRows) return;
  const int64_t d = i / kSgdRows, t = i - d * kSgdRows;
  uint16_t v = 0;
  if (t < T) v = (uint16_t)f32_to_bf16_bits(w[t] * bf16_bits_to_f32(A[t * D + d]));
  AwT[i] = v;
}

// Workgroup g sweeps slice g % ns (ns = D / 128) over the blocks g / ns, g / ns + R, ...
// (R = gridDim.x / ns); every wave of it runs the same blocks, so the barriers match.
__global__ __launch_bounds__(256) void k_sgd_rows(const SgdRowsParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[kLds];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int D = p.D;
  const int ns = D / kSgdCols;
  const int c0 = kSgdCols * (int)(blockIdx.x % ns);
  const int64_t rstep = gridDim.x / ns;
  int64_t j = blockIdx.x / ns;
  if (j >= p.nblk) return;
  const uint32_t l0 = lds_u32(lds);

  // the held B operand: lane (column c0 + 32 wv + l32) with rows t = 16 ks + 8 h + 0..7
  bf16x8 bst[kSgdRows / 16];
  {
    const uint16_t* at = p.AwT + (int64_t)(c0 + 32 * wv + l32) * kSgdRows + 8 * h;
#pragma unroll
    for (int ks = 0; ks < kSgdRows / 16; ++ks) bst[ks] = *(const bf16x8*)(at + 16 * ks);
  }
  // copies of block jb into buffer q, kCopies per wave: image byte o of the P block holds
  // row o / kPRow, byte o % kPRow (pad bytes fetch byte 0); wave wv copies the 128-byte
  // slices of items 8 wv .. 8 wv + 7 and (in its own slot) the 32 items' indices. Rows
  // past V fetch row V - 1 and are not written back.
  auto issue = [&](int64_t jb, int q) {
    const uint16_t* blk = p.P + jb * (kSgdRows * kSgdItems);
#pragma unroll
    for (int x = 0; x < 3; ++x) {
      const int kb = wv + 4 * x;
      const int o = kb * 1024 + 16 * lane;
      const int r = o / kPRow, c = o - r * kPRow;
      const uint32_t src = (r < kSgdRows && c < 2 * kSgdItems) ? (uint32_t)(r * 2 * kSgdItems + c) : 0u;
      lds_dma16(blk, src, l0 + (uint32_t)(q * kPImg + kb * 1024));
    }
    const int64_t vb = p.v0 + jb * kSgdItems;
    {
      int64_t v = vb + 8 * wv + (lane >> 3);
      v = v < p.V ? v : p.V - 1;
      lds_dma16(p.E + vb * D, (uint32_t)((v - vb) * D + c0 + 16 * (lane & 7)),
                l0 + (uint32_t)(kOffE + q * kEImg + wv * 1024));
    }
    {
      int64_t v = vb + l32;
      v = v < p.V ? v : p.V - 1;
      lds_dma4(p.imap + vb, (uint32_t)(4 * (v - vb)), l0 + (uint32_t)(kOffMap + q * kMapImg + wv * 256));
    }
  };
  // the held operand's loads complete here: no wait of the compiler's own for them may
  // remain inside the loop, where it would also wait for the next block's copies
  wait_vm<0>();
  issue(j, 0);
  const int s = lane & 15;
  // transposed reads of a block: lane (item l32) receives rows 8 h + m and 8 h + 4 + m
  // (m = 0..3) of k step ks, from the 16-lane group's row and item offsets
  const uint32_t ta0 = (uint32_t)((8 * h + (s >> 2)) * kPRow + 2 * (4 * (s & 3) + 16 * ((lane >> 4) & 1)));
  const int it = tid >> 3, pc = tid & 7;         // the update's item and 16-column piece
  int q = 0;
  for (; j < p.nblk; j += rstep) {
    const bool more = j + rstep < p.nblk;        // uniform over the workgroup
    if (more) issue(j + rstep, q ^ 1);
    if (more) wait_vm<kCopies>(); else wait_vm<0>();
    __syncthreads();                             // block j's copies are visible

    const uint32_t ta = l0 + (uint32_t)(q * kPImg) + ta0;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kSgdRows / 16; ++ks) {
      const bf16x8 a = cat_bf16(read_tr16(ta + (uint32_t)(16 * ks * kPRow)),
                                read_tr16(ta + (uint32_t)((16 * ks + 4) * kPRow)));
      acc = mfma32(a, bst[ks], acc);
    }
    // result register i of a lane: item 8 (i >> 2) + 4 h + (i & 3), column 32 wv + l32
    char* const stage = lds + kOffStage;
#pragma unroll
    for (int i = 0; i < 16; ++i)
      *(float*)(stage + (8 * (i >> 2) + 4 * h + (i & 3)) * kStageRow + 4 * (32 * wv + l32)) = acc[i];
    __syncthreads();

    float g[16];
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      const f32x4 x = *(const f32x4*)(stage + it * kStageRow + 64 * pc + 16 * k4);
      g[4 * k4] = x[0]; g[4 * k4 + 1] = x[1]; g[4 * k4 + 2] = x[2]; g[4 * k4 + 3] = x[3];
    }
    const int u = *(const int*)(lds + kOffMap + q * kMapImg + 4 * it);
    if (u >= 0) {
      const float4* su = (const float4*)(p.S_u + (int64_t)u * D + c0 + 16 * pc);
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const float4 x = su[k4];
        g[4 * k4] -= x.x; g[4 * k4 + 1] -= x.y; g[4 * k4 + 2] -= x.z; g[4 * k4 + 3] -= x.w;
      }
    }
    const int64_t v = p.v0 + j * kSgdItems + it;
    if (v < p.V) {
      const uint4 e = *(const uint4*)(lds + kOffE + q * kEImg + it * kSgdCols + 16 * pc);
      const uint32_t w4[4] = {e.x, e.y, e.z, e.w};
      uint32_t o[4];
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        // two E4M3 values per conversion; the clamp to +-448 keeps the hardware conversion
        // from turning |x| > 464 into NaN (saturating nearest-even)
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w4[k4], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w4[k4], true);
        const float e0 = __builtin_amdgcn_fmed3f(__builtin_fmaf(-p.lr, g[4 * k4], lo[0]), -kFp8Max, kFp8Max);
        const float e1 = __builtin_amdgcn_fmed3f(__builtin_fmaf(-p.lr, g[4 * k4 + 1], lo[1]), -kFp8Max, kFp8Max);
        const float e2 = __builtin_amdgcn_fmed3f(__builtin_fmaf(-p.lr, g[4 * k4 + 2], hi[0]), -kFp8Max, kFp8Max);
        const float e3 = __builtin_amdgcn_fmed3f(__builtin_fmaf(-p.lr, g[4 * k4 + 3], hi[1]), -kFp8Max, kFp8Max);
        int rr = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
        rr = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, rr, true);
        o[k4] = (uint32_t)rr;
      }
      *(uint4*)(p.E + v * D + c0 + 16 * pc) = uint4{o[0], o[1], o[2], o[3]};
    }
    __syncthreads();                             // buffer q and the stage are free again
    q ^= 1;
  }
}

}  // namespace

bool sgd_rows_supported(int64_t Tp, int64_t D) { return Tp == kSgdRows && D % 128 == 0 && D >= 128 && D <= 1024; }

hipError_t launch_weighted_transpose(const void* A, const float* w, int64_t T, int64_t D, uint16_t* AwT,
                                     hipStream_t st) {
  if (T < 0 || T > kSgdRows || D <= 0) return hipErrorInvalidValue;
  const int64_t n = D * kSgdRows;
  k_weighted_t<<<(unsigned)((n + 255) / 256), 256, 0, st>>>((const uint16_t*)A, w, T, D, AwT);
  return hipGetLastError();
}

hipError_t launch_sgd_rows(const SgdRowsParams& p, hipStream_t st) {
  if (!sgd_rows_supported(kSgdRows, p.D) || p.nblk <= 0 || p.V <= 0 || p.v0 < 0 || p.v0 >= p.V ||
      p.P == nullptr || p.AwT == nullptr || p.E == nullptr || p.imap == nullptr)
    return hipErrorInvalidValue;
  // every block starts inside the vocabulary (the copies address rows relative to it)
  if (p.v0 + (p.nblk - 1) * kSgdItems >= p.V) return hipErrorInvalidValue;
  // about three workgroups per CU (51 KB of LDS each), every slice with the same block rows
  const int64_t ns = p.D / kSgdCols;
  const int64_t rows = std::max<int64_t>(1, std::min<int64_t>(p.nblk, 768 / ns));
  k_sgd_rows<<<(unsigned)(ns * rows), 256, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace cl
