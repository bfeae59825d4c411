// Logits product of the chunked path for FP8 E and heads of at most 128 rows (the XMC head:
// T = 128, D = 768, V = 3M): per vocabulary chunk, every row's BCE softplus partial and, for a
// backward, the unweighted sigmoid tile P in its blocked layout, or, for the Cut Metrics
// forward, the row's count of positive logits (Cut Binary Cross Entropy §III-A/B: the dense
// softplus term, the gradient recomputed per tile; §III-D: the metrics' dense counts; ELMO,
// ai.info summary: FP8 E4M3 label weights, widened here exactly to bf16 for the MFMA).
//
// With so few rows the product is a stream over E (2D flops per logit, D bytes of E per item),
// so it is shaped like one:
//  * a workgroup has eight waves: wave w holds rows 32 (w % 4) .. + 32 of A over one half of D
//    in registers as the MFMA's B operand (D/8 VGPRs: 96 at D = 768), one workgroup per CU;
//  * persistent workgroups walk the chunk's 32-item blocks. A block's E rows (32 x D bytes)
//    are copied into LDS with global_load_lds up to four blocks ahead, into as many buffers
//    as fit, at a row stride of D + 16 bytes (an odd number of 16-byte bank slots), so that
//    the 16-byte fragment reads of 16 items at once meet distinct banks and every read is a
//    per-lane base plus an immediate;
//  * a wave widens each 8-byte half of a fragment (four instructions for 8 values) and
//    issues D/32 MFMAs per block; the two halves of a row quarter then exchange partial
//    logits through LDS, so that each finishes 16 of the 32 items;
//  * each lane sums its row's softplus terms in registers across blocks (the log taken once
//    per block); sigma goes through an LDS image of the block's P (128 rows x 32 items) and
//    out as one contiguous 8 KB run in 16-byte pieces;
//  * workgroup g of a chunk writes loss slot part_base + g and the chunk's slots past the
//    workgroups are zeroed, so the finalization sums the slots as it does for the GEMM's
//    per-tile partials.
#include "launch.h"

#include <algorithm>

namespace cl {

namespace {

constexpr int kLItems = 32;                    // items per block
constexpr int kLRows = 128;                    // rows of a P block (T at most)
constexpr int kLPRow = 2 * kLItems + 16;       // LDS stride of a P-image row (bytes)
constexpr int kLPImg = kLRows * kLPRow;
constexpr int kLMaxWorkgroups = 256;           // one per CU
constexpr int kLLds = 160 * 1024;              // LDS of a workgroup
constexpr float kLNegInf = -__builtin_inff();

__device__ __forceinline__ uint32_t lds_u32(const void* p) { return (uint32_t)(uintptr_t)p; }

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0xF70 | (N & 15) | ((N >> 4) << 14));
}

// MODE 0: loss partials; 1: loss partials and P; 2: loss partials and positive-logit counts
template <int D, int MODE>
__global__ __launch_bounds__(512, 1) void k_logits_rows(const LogitsRowsParams p) {
  constexpr bool WP = MODE == 1, CNT = MODE == 2;
  constexpr int DH = D / 2;                    // columns of a wave's half
  constexpr int KH = DH / 16;                  // its MFMA k steps
  constexpr int ER = D + 16;                   // LDS stride of an E row
  constexpr int NC = (kLItems * ER + 1023) / 1024;   // 1 KB copies of a block's image
  constexpr int EB = NC * 1024;
  constexpr int C0 = NC / 8;                   // copies per block of waves NC % 8 .. 7 (others + 1)
  // E buffers: as many as the LDS holds beside the other regions (at most 6), so that
  // NBUF - 1 blocks (98 KB at D = 768) are in flight beyond the current one
  constexpr int FIXED = (WP ? kLPImg : 0) + 8 * 8 * 64 * 4 + 8 * kLRows;
  constexpr int NBUF = std::min(6, (kLLds - FIXED) / EB);
  constexpr int LA = NBUF - 1;                 // blocks issued ahead
  static_assert(NBUF >= 3, "E buffers");
  constexpr int OFF_P = NBUF * EB;             // the P image
  constexpr int OFF_X = OFF_P + (WP ? kLPImg : 0);   // partial-logit exchange, [8 waves][8][64]
  constexpr int OFF_F = OFF_X + 8 * 8 * 64 * 4;      // loss (and count) exchange, [2][128]
  __shared__ __attribute__((aligned(1024))) char lds[OFF_F + 8 * kLRows];
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tq = wv & 3, dh = wv >> 2;
  const uint32_t dh_mask = dh ? 0xffffffffu : 0u;
  const int64_t g = blockIdx.x, ng = gridDim.x;
  const uint32_t l0 = lds_u32(lds);
  const int t = 32 * tq + l32;                 // this lane's row
  const bool t_ok = t < p.T;
  const uint32_t t_mask = t_ok ? 0xffffffffu : 0u;
  const int ncp = wv < NC % 8 ? C0 + 1 : C0;   // this wave's copies per block

  // the chunk's loss (and count) slots past the workgroups' own
  for (int64_t sl = ng + g; sl < p.nslots; sl += ng)
    for (int r = tid; r < p.T; r += 512) {
      p.part_a[(p.part_base + sl) * p.T + r] = 0.0f;
      if constexpr (CNT) p.part_b[(p.part_base + sl) * p.T + r] = 0.0f;
    }

  // the held B operand: row t of A; k step ks takes columns DH dh + 32 (ks / 2) + 16 h +
  // 8 (ks % 2) .. + 8 (zero past T), so that one 16-byte fragment read of E serves a pair of
  // k steps (the same k order on both operands)
  bf16x8 ast[KH];
#pragma unroll
  for (int ks = 0; ks < KH; ++ks)
    ast[ks] = t_ok ? *(const bf16x8*)(p.A + (int64_t)t * D + DH * dh + 32 * (ks >> 1) + 16 * h + 8 * (ks & 1))
                   : bf16x8{};

  // copies of block bb into buffer q, copy kb = wv + 8 x: image byte o holds item o / ER,
  // byte o % ER of its row (the pad bytes and the bytes past the image fetch the block's
  // first byte). Rows past V (the chunk's last blocks run to its 256-item rounding) fetch
  // row V - 1, from a base row clamped the same way, so every offset is non-negative.
  // A copy's item row and byte within the row are the same for every block: kept per copy
  // (row -1: a pad byte). With rb the block's first row clamped to V - 1, row r of the block
  // is read at offset min(r, rmax) D + c from row rb, rmax = clamp(V - 1 - vb, 0, 31).
  constexpr int NX = (NC + 7) / 8;
  int crow[NX], ccol[NX];
#pragma unroll
  for (int x = 0; x < NX; ++x) {
    const int kb = wv + 8 * x;
    const int o = kb * 1024 + 16 * lane;
    const int r = o / ER, c = o - r * ER;
    const bool in = kb < NC && r < kLItems && c < D;
    crow[x] = in ? r : -1;
    ccol[x] = in ? c : 0;
  }
  auto issue = [&](int64_t bb, int q) {
    const int64_t vb = p.v0 + bb * kLItems;
    const int64_t rb = vb < p.V ? vb : p.V - 1;
    const int rmax = (int)std::min<int64_t>(kLItems - 1, std::max<int64_t>(0, p.V - 1 - vb));
    const uint8_t* const base = p.E + rb * D;
#pragma unroll
    for (int x = 0; x < NX; ++x) {
      const int kb = wv + 8 * x;
      if (kb >= NC) break;
      const uint32_t src = crow[x] >= 0 ? (uint32_t)(min(crow[x], rmax) * D + ccol[x]) : 0u;
      lds_dma16_nt(base, src, l0 + (uint32_t)(q * EB + kb * 1024));
    }
  };
  // wait until block k's copies are in: n later blocks' copies (ncp each) may stay in flight
  // (every P store issued since also counts: the wait is then conservative, never short)
  auto wait_for = [&](int n) {
    const bool more = ncp == C0 + 1;
    switch (n) {
      case 5: if (more) wait_vm<5 * (C0 + 1)>(); else wait_vm<5 * C0>(); break;
      case 4: if (more) wait_vm<4 * (C0 + 1)>(); else wait_vm<4 * C0>(); break;
      case 3: if (more) wait_vm<3 * (C0 + 1)>(); else wait_vm<3 * C0>(); break;
      case 2: if (more) wait_vm<2 * (C0 + 1)>(); else wait_vm<2 * C0>(); break;
      case 1: if (more) wait_vm<C0 + 1>(); else wait_vm<C0>(); break;
      default: wait_vm<0>();
    }
  };
  // the held operand's loads complete here: no wait of the compiler's own for them may
  // remain inside the loop, where it would also wait for later blocks' copies
  wait_vm<0>();
  int64_t b = g;
#pragma unroll
  for (int k = 0; k < LA; ++k)
    if (b + k * ng < p.nblk) issue(b + k * ng, k);
  float relu = 0.0f, lg = 0.0f, cnt = 0.0f;
  int q = 0;
  float* const xb = (float*)(lds + OFF_X);
  char* const pimg = lds + OFF_P;

  // block b's copies are in and visible (later blocks' copies stay in flight)
  int left = (int)((p.nblk - 1 - b) / ng);      // the workgroup's blocks after the current one
  auto begin = [&]() {
    if (left >= LA) issue(b + LA * ng, q == 0 ? NBUF - 1 : q - 1);   // uniform
    wait_for(min(LA, left));
    __syncthreads();
  };
  // the wave's half of block b's logits, item l32 as the A operand
  auto product = [&]() {
    // lane (item l32, half h) reads 16 bytes, columns DH dh + 32 s + 16 h .. + 16, for k steps
    // 2 s and 2 s + 1: 16 lanes a cycle, 16 rows whose stride (D + 16 bytes, an odd number of
    // 16-byte slots) puts them in distinct banks
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const uint32_t eb = l0 + (uint32_t)(q * EB + l32 * ER + DH * dh + 16 * h);
    u32x4 raw[KH / 2];                           // every fragment read is issued up front
#pragma unroll
    for (int s2 = 0; s2 < KH / 2; ++s2) raw[s2] = *(const CL_LDS u32x4*)(uintptr_t)(eb + (uint32_t)(32 * s2));
    f32x16 acc = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KH; ++ks) {
      const u32x4& r = raw[ks >> 1];
      acc = mfma32(fp8x8_to_bf16x8((ks & 1) ? uint2{r[2], r[3]} : uint2{r[0], r[1]}), ast[ks], acc);
    }
    return acc;
  };
  // result register i holds item 8 (i >> 2) + 4 h + (i & 3): half dh keeps items
  // 16 dh .. 16 dh + 15 (registers 8 dh .. 8 dh + 7) and hands the others to its partner
  auto exchange = [&](const f32x16& acc, float (&x8)[8]) {
    // (register choice by bit masks: a select on dh would become indexed register access)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t lo = __float_as_uint(acc[j]), hi = __float_as_uint(acc[8 + j]);
      xb[(wv * 8 + j) * 64 + lane] = __uint_as_float((lo & dh_mask) | (hi & ~dh_mask));
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t lo = __float_as_uint(acc[j]), hi = __float_as_uint(acc[8 + j]);
      x8[j] = __uint_as_float((hi & dh_mask) | (lo & ~dh_mask)) + xb[((wv ^ 4) * 8 + j) * 64 + lane];
    }
  };
  // register j of block bb: item 16 dh + 8 (j >> 2) + 4 h + (j & 3), row t; items past V
  // become -inf, which adds 0 to both sums and gives sigma 0. sigma goes to the P image.
  auto epilogue = [&](const float (&x8)[8], int64_t bb) {
    const int lim = (int)std::min<int64_t>(kLItems, p.V - (p.v0 + bb * kLItems));   // items of the block in V
    float prod = 1.0f;
    float f[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int it = 16 * dh + 8 * (j >> 2) + 4 * h + (j & 3);
      const float x = it < lim ? x8[j] : kLNegInf;
      const float e = __builtin_amdgcn_exp2f(-__builtin_fabsf(x) * kLog2e);   // e^-|x| in [0, 1]
      const float qv = 1.0f + e;
      relu += __builtin_fmaxf(x, 0.0f);
      prod *= qv;
      if constexpr (CNT) cnt += x > 0.0f ? 1.0f : 0.0f;   // exact in fp32 below 2^24
      if constexpr (WP) {                        // unweighted: w enters through dA and A_w
        const float r = __builtin_amdgcn_rcpf(qv);
        f[j] = x >= 0.0f ? r : e * r;
      }
    }
    lg += __builtin_amdgcn_logf(prod);           // log2 of a product of 8 factors in [1, 2]
    if constexpr (WP) {
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        uint2 pk;                                // rows past T hold 0
        pk.x = (f32_to_bf16_bits(f[4 * jj]) | (f32_to_bf16_bits(f[4 * jj + 1]) << 16)) & t_mask;
        pk.y = (f32_to_bf16_bits(f[4 * jj + 2]) | (f32_to_bf16_bits(f[4 * jj + 3]) << 16)) & t_mask;
        *(uint2*)(pimg + t * kLPRow + 2 * (16 * dh + 8 * jj + 4 * h)) = pk;
      }
    }
  };
  // the P of block bb: 128 rows x 64 bytes, contiguous in the blocked layout; thread tid
  // copies 16-byte piece tid (row tid / 4, quarter tid % 4)
  auto store_p = [&](int64_t bb) {
    uint16_t* const pb = p.P + bb * (kLRows * kLItems);
    const int r = tid >> 2, qq = tid & 3;
    *(uint4*)(pb + r * kLItems + 8 * qq) = *(const uint4*)(pimg + r * kLPRow + 16 * qq);
  };

  // Software pipeline over the workgroup's blocks: the matrix work of block b runs beside
  // the transcendental epilogue of block b - ng, two barriers a block. The P image written
  // by an epilogue is stored after the next barrier; the exchange and the P image are not
  // written again before every thread has passed the following block's first barrier.
  float xp[8];
  begin();
  exchange(product(), xp);
  int64_t bp = b;
  q = q == NBUF - 1 ? 0 : q + 1;
  for (b += ng; b < p.nblk; b += ng) {
    --left;
    begin();                                     // also: the previous P store and exchange reads are done
    const f32x16 acc = product();
    epilogue(xp, bp);
    // one instruction stream for both: the fragment reads first, then each MFMA followed
    // by the widening of the next fragment and a share of the epilogue, so that the
    // vector ALU works while the matrix core runs
    __builtin_amdgcn_sched_group_barrier(0x100, KH / 2, 0);
#pragma unroll
    for (int i = 0; i < KH; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
    }
    float x8[8];
    exchange(acc, x8);                           // its barrier also completes the P image of block bp
    if constexpr (WP) store_p(bp);
#pragma unroll
    for (int j = 0; j < 8; ++j) xp[j] = x8[j];
    bp = b;
    q = q == NBUF - 1 ? 0 : q + 1;
  }
  if constexpr (WP) __syncthreads();             // the last loop's P store has read the image
  epilogue(xp, bp);
  if constexpr (WP) {
    __syncthreads();
    store_p(bp);
  }
  // a row's partial: the two halves of each wave, then the two column halves, in that order
  float vs = relu + lg * kLn2;
  vs += __shfl_xor(vs, 32, 64);
  float* const fb = (float*)(lds + OFF_F);
  if constexpr (CNT) cnt += __shfl_xor(cnt, 32, 64);
  if (dh == 1 && h == 0) {
    fb[t] = vs;
    if constexpr (CNT) fb[kLRows + t] = cnt;
  }
  __syncthreads();
  if (dh == 0 && h == 0 && t_ok) {
    p.part_a[(p.part_base + g) * p.T + t] = vs + fb[t];
    if constexpr (CNT) p.part_b[(p.part_base + g) * p.T + t] = cnt + fb[kLRows + t];
  }
}

template <int D>
hipError_t launch_d(const LogitsRowsParams& p, unsigned grid, hipStream_t st) {
  if (p.P != nullptr) k_logits_rows<D, 1><<<grid, 512, 0, st>>>(p);
  else if (p.part_b != nullptr) k_logits_rows<D, 2><<<grid, 512, 0, st>>>(p);
  else k_logits_rows<D, 0><<<grid, 512, 0, st>>>(p);
  return hipGetLastError();
}

}  // namespace

bool logits_rows_supported(int64_t Tp, int64_t D) { return Tp == kLRows && D % 128 == 0 && D >= 128 && D <= 768; }

hipError_t launch_logits_rows(const LogitsRowsParams& p, hipStream_t st) {
  if (!logits_rows_supported(kLRows, p.D) || p.T < 1 || p.T > kLRows || p.nslots < 1 || p.nblk != 8 * p.nslots ||
      p.V <= 0 || p.v0 < 0 || p.v0 >= p.V || p.E == nullptr || p.A == nullptr || p.part_a == nullptr ||
      (p.P != nullptr && p.part_b != nullptr))
    return hipErrorInvalidValue;
  const unsigned grid = (unsigned)std::min<int64_t>(kLMaxWorkgroups, p.nslots);
  switch (p.D) {
    case 128: return launch_d<128>(p, grid, st);
    case 256: return launch_d<256>(p, grid, st);
    case 384: return launch_d<384>(p, grid, st);
    case 512: return launch_d<512>(p, grid, st);
    case 640: return launch_d<640>(p, grid, st);
    case 768: return launch_d<768>(p, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cl
