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
//    contiguous 16-byte piece of a row;
//  * with dA requested, the same two LDS images also give the slice's share of the row
//    gradient, sum over the chunk's items of P[t][v] E[v][d] with E before its update (the
//    backward's G E, Cut Binary Cross Entropy §III-B): the block is read row-wise as the A
//    operand (rows t, k = items) and the E slice transposed (ds_read_b64_tr_b8, k = items) as
//    the B operand, each wave accumulating a 64 x 64 tile in registers over all of its
//    blocks. The workgroup's 128 x 128 tile is one split partial of dA; the partial carries
//    over from one chunk to the next (loaded at the start, stored at the end), so that the
//    separate dA product and its second pass over E and P are not needed.
#include "launch.h"
#include "sr.h"

#include <algorithm>

namespace cl {

namespace {

constexpr int kSgdItems = 32;                      // items per block
constexpr int kSgdRows = 128;                      // rows (k) of a gradient-tile block
constexpr int kSgdCols = 128;                      // columns of a workgroup's slice (4 waves x 32)
// LDS image of a gradient-tile block: rows of 64 bytes, unpadded, the 16-byte piece c of row
// r stored at piece c ^ ((r / 4) mod 4). The transposed reads of the SGD product take 4
// consecutive rows per half-wave (256 bytes, every bank once); the dA product's 16-byte reads
// take 16 consecutive rows, which the XOR spreads over the 16 slots.
constexpr int kPRow = 2 * kSgdItems;
constexpr int kPImg = kSgdRows * kPRow;            // 8 KB, two copies a wave
// the items' slices of E: 32 rows of 128 bytes, the 16-byte piece c of row v stored at piece
// c ^ (v & 7) of the row, so that the transposed reads (8 rows, one piece) meet 8 bank groups
constexpr int kEImg = kSgdItems * kSgdCols;
constexpr int kMapImg = 4 * 256;                   // unique-item indices: one 256-byte slot a wave
constexpr int kStageRow = 4 * kSgdCols + 16;       // fp32 result row (+16 bytes)
constexpr int kOffE = 2 * kPImg;
constexpr int kOffMap = kOffE + 2 * kEImg;
constexpr int kOffStage = kOffMap + 2 * kMapImg;
constexpr int kLds = kOffStage + kSgdItems * kStageRow;
constexpr int kCopies = 4;                         // copy instructions a wave issues per block

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

// 8 bytes of a transposed 8 x 16 byte block: within a 16-lane group, lane i receives byte
// i % 8 of the 8-byte rows that lanes i / 8, i / 8 + 2, ..., i / 8 + 14 address
__device__ __forceinline__ uint2 read_tr8(uint32_t lds) {
  typedef int i32x2 __attribute__((ext_vector_type(2)));
  const i32x2 r = __builtin_amdgcn_ds_read_tr8_b64_v2i32((CL_LDS i32x2*)(uintptr_t)lds);
  return uint2{(uint32_t)r[0], (uint32_t)r[1]};
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

// Workgroup (block row r, slice s) sweeps columns 128 s .. 128 s + 127 (s < ns = D / 128)
// over the blocks r, r + R, ... (R = gridDim.x / ns); every wave of it runs the same blocks,
// so the barriers match. The ns slices of a block row read the same gradient-tile blocks:
// consecutive workgroups go to the eight XCDs in turn, so when R is a multiple of 8 the
// slices of row r are workgroups 8 i + r % 8 (one XCD, one L2) and each P block comes from
// HBM once.
// SR: stochastic rounding (the uniforms' Philox work needs registers: two waves per SIMD)
template <bool SR>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(SR ? 2 : 3))) void k_sgd_rows(const SgdRowsParams p) {
  __shared__ __attribute__((aligned(1024))) char lds[kLds];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int D = p.D;
  const int ns = D / kSgdCols;
  const int64_t rstep = gridDim.x / ns;
  int64_t r, sl;
  if (rstep % 8 == 0) {
    const int64_t idx = blockIdx.x / 8;
    r = blockIdx.x % 8 + 8 * (idx / ns);
    sl = idx % ns;
  } else {
    r = blockIdx.x / ns;
    sl = blockIdx.x % ns;
  }
  const int c0 = kSgdCols * (int)sl;
  int64_t j = r;
  if (j >= p.nblk) return;
  const uint32_t l0 = lds_u32(lds);

  // the held B operand: lane (column c0 + 32 wv + l32) with rows t = 16 ks + 8 h + 0..7
  bf16x8 bst[kSgdRows / 16];
  {
    const uint16_t* at = p.AwT + (int64_t)(c0 + 32 * wv + l32) * kSgdRows + 8 * h;
#pragma unroll
    for (int ks = 0; ks < kSgdRows / 16; ++ks) bst[ks] = *(const bf16x8*)(at + 16 * ks);
  }
  // dA tile of the wave: rows 64 th .. 64 th + 63, columns c0 + 64 dh .. + 63; register i of
  // tile (mt, nt) holds row 64 th + 32 mt + 8 (i >> 2) + 4 h + (i & 3), column
  // c0 + 64 dh + 32 nt + l32 of split partial r
  const int th = wv & 1, dh = wv >> 1;
  const bool want_dA = p.dA_part != nullptr;
  float* const part = want_dA ? p.dA_part + r * p.T * D : nullptr;
  f32x16 dacc[2][2];
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      dacc[mt][nt] = f32x16{};
      if (want_dA && !p.dA_first) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t t = 64 * th + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
          if (t < p.T) dacc[mt][nt][i] = part[t * D + c0 + 64 * dh + 32 * nt + l32];
        }
      }
    }
  // copies of block jb into buffer q, kCopies per wave: image piece c' of row r holds the
  // block's piece c' ^ ((r / 4) mod 4) of that row; wave wv copies the 128-byte slices of
  // items 8 wv .. 8 wv + 7 and (in its own slot) the 32 items' indices. Rows past V fetch
  // row V - 1 and are not written back.
  auto issue = [&](int64_t jb, int q) {
    const uint16_t* blk = p.P + jb * (kSgdRows * kSgdItems);
#pragma unroll
    for (int x = 0; x < kPImg / 4096; ++x) {
      const int kb = wv + 4 * x;
      const int o = kb * 1024 + 16 * lane;
      const int r = o / kPRow, c = (o % kPRow) / 16;
      lds_dma16(blk, (uint32_t)(r * kPRow + 16 * (c ^ ((r >> 2) & 3))), l0 + (uint32_t)(q * kPImg + kb * 1024));
    }
    const int64_t vb = p.v0 + jb * kSgdItems;
    {
      // LDS piece lane & 7 of row 8 wv + (lane >> 3) holds the row's piece (lane & 7) ^ (lane >> 3)
      int64_t v = vb + 8 * wv + (lane >> 3);
      v = v < p.V ? v : p.V - 1;
      lds_dma16_nt(p.E + vb * D, (uint32_t)((v - vb) * D + c0 + 16 * ((lane & 7) ^ (lane >> 3))),
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
  // (m = 0..3) of k step ks, from the 16-lane group's row and item offsets: byte
  // 8 (s & 3) + 32 g of the row (g = (lane >> 4) & 1), i.e. piece (s & 3) / 2 + 2 g, which
  // those rows store at that piece ^ 2h and ^ (2h + 1)
  const int tpc = ((s & 3) >> 1) + 2 * ((lane >> 4) & 1);
  const uint32_t ta0 = (uint32_t)((8 * h + (s >> 2)) * kPRow + 16 * (tpc ^ (2 * h)) + 8 * (s & 1));
  const uint32_t tb0 = (uint32_t)((8 * h + 4 + (s >> 2)) * kPRow + 16 * (tpc ^ (2 * h + 1)) + 8 * (s & 1));
  const int it = tid >> 3, pc = tid & 7;         // the update's item and 16-column piece
  // dA operands: the block's rows 64 th + 32 mt + l32 at items 16 ks + 8 h (16 bytes), and
  // the E slice read transposed: in 16-lane group gq, lane s addresses item row
  // 16 ks + 8 h + (s >> 1), bytes 8 (s & 1) of piece 4 dh + 2 nt + (gq & 1) (swizzled)
  const uint32_t pa0 = (uint32_t)((64 * th + l32) * kPRow);
  const int pfl = (l32 >> 2) & 3;                // the rows' piece XOR
  const uint32_t pk0 = (uint32_t)(16 * (h ^ pfl)), pk1 = (uint32_t)(16 * ((2 + h) ^ pfl));
  const uint32_t eb0 = (uint32_t)((8 * h + (s >> 1)) * kSgdCols + 8 * (s & 1));
  const int epc = 4 * dh + ((lane >> 4) & 1);
  int q = 0;
  for (; j < p.nblk; j += rstep) {
    const bool more = j + rstep < p.nblk;        // uniform over the workgroup
    if (more) issue(j + rstep, q ^ 1);
    if (more) wait_vm<kCopies>(); else wait_vm<0>();
    __syncthreads();                             // block j's copies are visible

    const uint32_t ta = l0 + (uint32_t)(q * kPImg) + ta0, tb = l0 + (uint32_t)(q * kPImg) + tb0;
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < kSgdRows / 16; ++ks) {
      const bf16x8 a = cat_bf16(read_tr16(ta + (uint32_t)(16 * ks * kPRow)), read_tr16(tb + (uint32_t)(16 * ks * kPRow)));
      acc = mfma32(a, bst[ks], acc);
    }
    if (want_dA) {
      const uint32_t pb = l0 + (uint32_t)(q * kPImg) + pa0;
      const uint32_t eb = l0 + (uint32_t)(kOffE + q * kEImg) + eb0;
#pragma unroll
      for (int ks = 0; ks < kSgdItems / 16; ++ks) {
        bf16x8 pa[2], eb8[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          pa[mt] = *(const CL_LDS bf16x8*)(uintptr_t)(pb + (uint32_t)(32 * mt * kPRow) + (ks ? pk1 : pk0));
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          eb8[nt] = fp8x8_to_bf16x8(read_tr8(eb + (uint32_t)(16 * ks * kSgdCols + 16 * ((epc + 2 * nt) ^ (s >> 1)))));
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int nt = 0; nt < 2; ++nt) dacc[mt][nt] = mfma32(pa[mt], eb8[nt], dacc[mt][nt]);
      }
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
      const uint4 e = *(const uint4*)(lds + kOffE + q * kEImg + it * kSgdCols + 16 * (pc ^ (it & 7)));
      const uint32_t w4[4] = {e.x, e.y, e.z, e.w};
      uint32_t o[4];
      uint32_t hw[8];                            // SR: the uniforms of columns c0 + 16 pc .. + 15
      if constexpr (SR) sr_uniforms16(p.sr_seed, v, c0 + 16 * pc, hw);
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        // two E4M3 values per conversion; nearest-even: the clamp to +-448 keeps the hardware
        // conversion from turning |x| > 464 into NaN (saturating); stochastic: the rounded
        // values lie on the grid, so the conversion is exact
        const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w4[k4], false);
        const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w4[k4], true);
        const float y0 = __builtin_fmaf(-p.lr, g[4 * k4], lo[0]), y1 = __builtin_fmaf(-p.lr, g[4 * k4 + 1], lo[1]);
        const float y2 = __builtin_fmaf(-p.lr, g[4 * k4 + 2], hi[0]), y3 = __builtin_fmaf(-p.lr, g[4 * k4 + 3], hi[1]);
        float e0, e1, e2, e3;
        if constexpr (SR) {
          e0 = sr_fp8(y0, sr_h16(hw, 4 * k4));
          e1 = sr_fp8(y1, sr_h16(hw, 4 * k4 + 1));
          e2 = sr_fp8(y2, sr_h16(hw, 4 * k4 + 2));
          e3 = sr_fp8(y3, sr_h16(hw, 4 * k4 + 3));
        } else {
          e0 = __builtin_amdgcn_fmed3f(y0, -kFp8Max, kFp8Max);
          e1 = __builtin_amdgcn_fmed3f(y1, -kFp8Max, kFp8Max);
          e2 = __builtin_amdgcn_fmed3f(y2, -kFp8Max, kFp8Max);
          e3 = __builtin_amdgcn_fmed3f(y3, -kFp8Max, kFp8Max);
        }
        int rr = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
        rr = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, rr, true);
        o[k4] = (uint32_t)rr;
      }
      // each E piece is written once per pass: stored with the non-temporal hint, as it is read
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]}, (u32x4*)(p.E + v * D + c0 + 16 * pc));
    }
    __syncthreads();                             // buffer q and the stage are free again
    q ^= 1;
  }
  if (want_dA) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t t = 64 * th + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
          if (t < p.T) part[t * D + c0 + 64 * dh + 32 * nt + l32] = dacc[mt][nt][i];
        }
  }
}

}  // namespace

bool sgd_rows_supported(int64_t Tp, int64_t D) { return Tp == kSgdRows && D % 128 == 0 && D >= 128 && D <= 1024; }

// block rows of workgroups: three workgroups per CU (two with stochastic rounding), a
// multiple of 8 where there are that many, so that a row's slices share an XCD
static int64_t sgd_rows_max(int64_t ns, int sr) {
  const int64_t r = (sr ? 512 : 768) / ns;
  return r >= 8 ? r / 8 * 8 : r;
}

int64_t sgd_rows_dA_splits(int64_t nblk, int64_t D, int sr) {
  return std::max<int64_t>(1, std::min<int64_t>(nblk, sgd_rows_max(std::max<int64_t>(1, D / kSgdCols), sr)));
}

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
  // about three workgroups per CU (51 KB of LDS each; two with stochastic rounding), every
  // slice with the same block rows
  const int64_t ns = p.D / kSgdCols;
  int64_t rows = std::max<int64_t>(1, std::min<int64_t>(p.nblk, sgd_rows_max(ns, p.sr)));
  if (p.dA_part != nullptr) {
    // one dA partial per block row: the first chunk writes every one of them
    if (p.T < 1 || p.T > kSgdRows || p.dA_splits < 1 || p.dA_splits > sgd_rows_max(ns, p.sr)) return hipErrorInvalidValue;
    if (p.dA_first && p.nblk < p.dA_splits) return hipErrorInvalidValue;
    rows = std::min<int64_t>(p.nblk, p.dA_splits);
  }
  if (p.sr) k_sgd_rows<true><<<(unsigned)(ns * rows), 256, 0, st>>>(p);
  else k_sgd_rows<false><<<(unsigned)(ns * rows), 256, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace cl
