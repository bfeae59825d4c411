// Chunked path for wide classifier heads (D > 256, or FP8 embeddings): per vocabulary
// chunk of Vc items, three MFMA GEMMs with fused epilogues.
//
//   K1  X^T = E_c A^T          (M = chunk items, N = rows, K = D)
//       BCE: P = w sigmoid(X) -> bf16 P[t][v] buffer, softplus row partials;
//       CE forward: (max, sum) row partials; CE backward: P = w exp(X - lse).
//   K2  dA (+)= P E_c          (M = rows, N = D, K = Vc), fp32 split-K partials
//   K3  dE_c = P^T A - S       (M = chunk items, N = D, K = rows): bf16 dE, or the
//       SGD step on E in place (ELMO summary, Key Contributions 2: gradient fused with
//       the update, never stored).
//
// Cut Binary Cross Entropy (paperpeel) §III-A forms the logits of one vocabulary block
// at a time and discards them; here only the chunk's gradient tile P (T x Vc bf16) is
// kept, long enough for K2 and K3 to consume it. The executed matrix work is 6 T V D
// (no recompute), and at D >= 512 each GEMM stays compute-bound with P in HBM.
//
// Kernel: 8 waves, 256 x (256 | 128) output tile, K stages of 32 in a 4-deep LDS ring.
// Every operand arrives by global_load_lds_dwordx4 (lane-linear 1 KB blocks) from a
// wave-uniform tile origin plus per-lane offsets fixed at kernel start. FP8 operands are
// copied as raw bytes and widened to bf16 (exactly) after the fragment read. An operand
// tile is either k-contiguous ([rows][32 k], read with ds_read_b128, or ds_read_b64 for
// FP8) or k-major ([32 k][cols], read transposed with ds_read_b64_tr_b16, or
// ds_read_b64_tr_b8 for FP8); every read pattern gives lane (l, h) the k values
// 16 kk + 8 h + 0..7, so any pair of modes composes.
//
// Workgroups take output tiles in an order that keeps each XCD (blockIdx % 8) on a
// contiguous run of tiles: 8 row tiles by all column tiles, so the 32 workgroups an XCD
// runs at once share their A and B tiles through that XCD's L2.
#include "launch.h"
#include "sr.h"


namespace cl {

namespace {

constexpr int kBK = 32;
typedef int i32x8 __attribute__((ext_vector_type(8)));
// Two workgroup shapes: NW = 8 waves with a 4-deep ring (one workgroup per CU), and NW = 4
// waves with 256 x 128 tiles and a 3-deep ring (72 KB of LDS, two workgroups per CU, so one
// can run its MFMAs while the other is in its epilogue).
template <int NW, int BN> struct Cfg {
  static constexpr int THREADS = 64 * NW;
  static constexpr int NST = NW == 4 ? 3 : 4;
};
constexpr int kBM = 256;
constexpr int kGroupM = 8;
constexpr int kMaxStages = 1024;
template <bool B> struct BoolC { static constexpr bool value = B; };      // k stages of one filtered dA / dE workgroup
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ int res_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// Swizzle of k-major tiles. One transposed read touches 4 rows at 64 logical bytes for
// each half wave, rows q..q+3 and q+8..q+11 (q = 0 or 4, + 16 for the second k16 half).
// s(r) sends rows with different r & 3 to different 64-byte groups of the 256-byte bank
// window and the two row quads to alternate 32-byte groups, so every 16- or 32-lane
// subset of the instruction reads distinct banks.
__device__ __forceinline__ int swz_kr(int r) { return ((r & 3) << 2) | (((r >> 3) & 1) << 1) | ((r >> 2) & 1); }

template <class T>
__device__ __forceinline__ const CL_LDS T* lds_ptr(uint32_t a) { return (const CL_LDS T*)(uintptr_t)a; }

// s_waitcnt vmcnt(N): gfx9 encoding, vmcnt[3:0] at bits 3:0 and vmcnt[5:4] at 15:14
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0xF70 | (N & 15) | ((N >> 4) << 14));
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// Wait until at most `later` stages of NPER copies each are in flight (L: the most there
// can be; more is waited down to L).
template <int NPER, int L>
__device__ __forceinline__ void wait_later(int later) {
  if constexpr (L <= 0) {
    wait_vm<0>();
  } else {
    if (later >= L) wait_vm<L * NPER>();
    else wait_later<NPER, L - 1>(later);
  }
}

__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// One stage of one operand: R rows (KC) or R columns (KR) by 32 k, in LDS as bf16 (ESZ 2)
// or as the raw bytes of an FP8 operand (ESZ 1).
template <int NW, int R, bool KC, int ESZ = 2>
struct Tile {
  static constexpr int BYTES = 32 * ESZ * R;
  static constexpr int KB = BYTES / 1024;
  static constexpr int PER_WAVE = KB / NW;            // DMA blocks per wave
  static constexpr int ROW = KC ? 32 * ESZ : ESZ * R; // bytes per LDS row
  static constexpr int NCH = ROW / 16;
  static_assert(PER_WAVE >= 1 && KB % NW == 0, "tile");
  // 16-byte piece lp of row r goes to piece phys(lp, r) of that row (an involution in lp).
  // FP8 k-contiguous rows are 32 bytes: rows r and r + 8 swap their two pieces, so a
  // fragment read (32 rows, one 8-byte half each) spreads over twice the banks. FP8 k-major
  // rows: the 8 rows one transposed read touches take 8 different pieces (16 over the wave).
  __device__ __forceinline__ static int phys(int lp, int r) {
    if constexpr (ESZ == 1) {
      if constexpr (KC) return lp ^ ((r >> 3) & 1);
      else return lp ^ (r & 15 & (NCH - 1));
    } else {
      if constexpr (KC) return lp ^ ((r >> 2) & 3);
      else return lp ^ (swz_kr(r) & (NCH - 1));
    }
  }
};

// Where the 8-element groups of one stage come from. The LDS byte of group j is fixed
// per lane; its source is origin(k0) + off[j] elements, origin(k0) being the wave-uniform
// address of element (outer0, k0) (KC) or (k0, outer0) (KR). Offsets clamp the outer
// index into the valid range once; a stage that reaches past the valid k range (only the
// last stages of some products) recomputes them with the k clamp as well.
template <int NW, int R, bool KC, bool F8, bool Q8 = false>
struct Loader {
  // F8: an FP8 operand copied as raw bytes (32 k per stage); Q8: FP8 x FP8 tiles (64 k per
  // stage, the bf16 tile's byte geometry)
  using TL = Tile<NW, R, KC, F8 ? 1 : 2>;
  static constexpr int N = TL::PER_WAVE;
  static constexpr int ESZ = (F8 || Q8) ? 1 : 2;
  static constexpr int EPP = (F8 || Q8) ? 16 : 8;      // elements per 16-byte LDS piece
  static constexpr int BK = Q8 ? 64 : kBK;             // k elements per stage
  uint32_t off[N];

  __device__ __forceinline__ static int byte_of(int j, int wv, int lane, int /*tid*/) {
    return (wv * TL::PER_WAVE + j) * 1024 + 16 * lane;
  }
  __device__ __forceinline__ static void rc(int byte, int& r, int& c) {
    r = byte / TL::ROW;
    c = EPP * TL::phys((byte % TL::ROW) / 16, r);
  }
  __device__ __forceinline__ void init(const GemmOperand& op, int64_t outer0, int wv, int lane, int tid) {
#pragma unroll
    for (int j = 0; j < N; ++j) {
      int r, c;
      rc(byte_of(j, wv, lane, tid), r, c);
      if (op.bt > 0) {
        // blocked P: the stage's k range is one 32-column block; KC: rows t of the tile
        // (clamped), KR: columns v of the tile, rows k0 + r inside one row block
        const int64_t bsz = (int64_t)op.bt * 32;
        if constexpr (KC) {
          const int64_t t = min(outer0 + r, op.rows_valid - 1);
          off[j] = (uint32_t)((t / op.bt) * op.nvb * bsz + (t % op.bt) * 32 + c);
        } else {
          const int64_t v = outer0 + c;
          off[j] = (uint32_t)((v >> 5) * bsz + r * 32 + (v & 31));
        }
      } else if constexpr (KC) {
        const int64_t row = min(outer0 + r, op.rows_valid - 1) - outer0;
        off[j] = (uint32_t)(row * op.ld + c);
      } else {
        const int64_t col = min(outer0 + c, op.cols_valid - EPP) - outer0;
        off[j] = (uint32_t)(r * op.ld + col);
      }
    }
  }
  __device__ __forceinline__ static const char* origin(const GemmOperand& op, int64_t outer0, int64_t k0) {
    if (op.bt > 0) {
      if constexpr (KC) return (const char*)op.p + k0 * op.bt * ESZ;          // column block k0 / 32
      else return (const char*)op.p + ((k0 / op.bt) * op.nvb * op.bt * 32 + (k0 % op.bt) * 32) * ESZ;
    }
    return (const char*)op.p + (KC ? outer0 * op.ld + k0 : k0 * op.ld + outer0) * ESZ;
  }
  // blocked operands are fully valid over the k range (checked by the launcher)
  __device__ __forceinline__ static bool tail(const GemmOperand& op, int64_t k0) {
    if (op.bt > 0) return false;
    return KC ? k0 + BK > op.cols_valid : k0 + BK > op.rows_valid;
  }
  // A k index at or below every clamped k index of the stage at k0: tail stages take their
  // origin there, so that each lane's offset (a 32-bit unsigned register for the LDS copy)
  // is non-negative even when the whole stage lies past the valid k range.
  __device__ __forceinline__ static int64_t tail_k(const GemmOperand& op, int64_t k0) {
    return KC ? min(k0, (int64_t)op.cols_valid - EPP) : min(k0, (int64_t)op.rows_valid - 1);
  }
  // element offset from origin(kb) of the stage at k0 with every index clamped (kb <= k0,
  // kb at or below every clamped k index)
  __device__ __forceinline__ static int64_t clamped(const GemmOperand& op, int64_t outer0, int64_t k0, int64_t kb, int byte) {
    int r, c;
    rc(byte, r, c);
    int64_t row, col;
    if constexpr (KC) {
      row = min(outer0 + r, op.rows_valid - 1);
      col = min(k0 + c, op.cols_valid - EPP);
      return (row - outer0) * op.ld + (col - kb);
    } else {
      row = min(k0 + r, op.rows_valid - 1);
      col = min(outer0 + c, op.cols_valid - EPP);
      return (row - kb) * op.ld + (col - outer0);
    }
  }
};

// Tail stages compute their clamped offsets from an opaque copy of the thread index, so
// that none of those terms is hoisted out of the main loop into registers held for the
// whole loop (they pushed register-heavy products into spilling).
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

// The copies are issued as inline asm (lds_dma16): every global load of a kernel's main loop
// is an LDS copy, and the loop's own waits count them.
template <int NW, int R, bool KC, bool F8, bool Q8>
__device__ __forceinline__ void dma_stage(const Loader<NW, R, KC, F8, Q8>& ld, const GemmOperand& op, int64_t outer0,
                                          int64_t k0, uint32_t lds, int wv, int lane) {
  using LD = Loader<NW, R, KC, F8, Q8>;
  using TL = typename LD::TL;
  const char* org = LD::origin(op, outer0, k0);
  if (!LD::tail(op, k0)) {
#pragma unroll
    for (int j = 0; j < TL::PER_WAVE; ++j) {
      const uint32_t dst = lds + (wv * TL::PER_WAVE + j) * 1024;
      lds_dma16(org, (uint32_t)(LD::ESZ * ld.off[j]), dst);
    }
  } else {
    const int ln = opaque(lane);
    const int64_t kt = LD::tail_k(op, k0);
    const char* orgt = LD::origin(op, outer0, kt);
#pragma unroll
    for (int j = 0; j < TL::PER_WAVE; ++j) {
      const int blk = wv * TL::PER_WAVE + j;
      const int64_t o = LD::clamped(op, outer0, k0, kt, blk * 1024 + 16 * ln);
      lds_dma16(orgt, (uint32_t)(LD::ESZ * o), lds + blk * 1024);
    }
  }
}

// MFMA operand fragments of a stage tile: lane (l32, h) gets index l32 of the 32-wide
// block `blk` and k = 16 kk + 8 h + 0..7.
// F8: the tile holds raw FP8 bytes, read 8 per lane and widened to bf16 (exact). A
// k-contiguous row read is one ds_read_b64; a k-major tile is read with ds_read_b64_tr_b8:
// in each 16-lane group g, lane i receives byte i mod 8 of the 8-byte reads of lanes
// floor(i/8) + 2j, j = 0..7, so lane s of the group reads row k0 + 8 (g >> 1) + (s >> 1),
// columns 16 (g & 1) + 8 (s & 1) + 0..7, and lane i gets column 16 (g & 1) + i of those
// 8 rows in k order.
template <int NW, int R, bool KC, bool F8 = false>
struct Frag {
  uint32_t base0, base1;   // KC: row-read base; KR: transposed-read bases (k rows +0..3, +4..7)
  __device__ __forceinline__ void init(uint32_t blk0_off, int lane) {
    using TL = Tile<NW, R, KC, F8 ? 1 : 2>;
    const int h = lane >> 5, l32 = lane & 31;
    if constexpr (F8) {
      if constexpr (KC) {
        const int r = l32;                       // + 32 blk leaves (r >> 3) & 1 unchanged
        base0 = blk0_off + r * TL::ROW + 16 * ((r >> 3) & 1) + 8 * h;
      } else {
        const int g = (lane >> 4) & 3, sl = lane & 15;
        const int kr = 8 * (g >> 1) + (sl >> 1);   // + 16 kk leaves kr & 15 unchanged
        base0 = blk0_off + kr * TL::ROW + 16 * ((g & 1) ^ (kr & 15 & (TL::NCH - 1))) + 8 * (sl & 1);
      }
      base1 = 0;
    } else if constexpr (KC) {
      const int r = l32;                         // + 32 blk: does not change (r >> 2) & 3
      const int sw = (r >> 2) & 3;
      base0 = blk0_off + r * TL::ROW + 16 * ((sw & 2) | (h ^ (sw & 1)));
      base1 = 0;
    } else {
      const int rsub = (lane & 15) >> 2;
      const int c0 = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
      const int co = 8 * (lane & 1);
      const int rA = 8 * h + rsub, rB = rA + 4;
      base0 = blk0_off + rA * TL::ROW + co + 16 * (c0 ^ (swz_kr(rA) & (TL::NCH - 1)));
      base1 = blk0_off + rB * TL::ROW + co + 16 * (c0 ^ (swz_kr(rB) & (TL::NCH - 1)));
    }
  }
  // blk: 32-wide block index within the tile's R; kk: 16-k half of the stage
  __device__ __forceinline__ bf16x8 read(uint32_t stage_off, int blk, int kk) const {
    using TL = Tile<NW, R, KC, F8 ? 1 : 2>;
    if constexpr (F8) {
      if constexpr (KC) {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        const u32x2 q = *lds_ptr<u32x2>(((base0 ^ (uint32_t)(16 * kk)) + (uint32_t)(blk * 32 * TL::ROW)) + stage_off);
        return fp8x8_to_bf16x8(uint2{q[0], q[1]});
      } else {
        typedef int i32x2 __attribute__((ext_vector_type(2)));
        const uint32_t o = (base0 ^ (uint32_t)(32 * blk)) + stage_off + (uint32_t)(kk * 16 * TL::ROW);
        const i32x2 q = __builtin_amdgcn_ds_read_tr8_b64_v2i32((CL_LDS i32x2*)(uintptr_t)o);
        return fp8x8_to_bf16x8(uint2{(uint32_t)q[0], (uint32_t)q[1]});
      }
    } else if constexpr (KC) {
      return *lds_ptr<bf16x8>(((base0 ^ (uint32_t)(32 * kk)) + (uint32_t)(blk * 32 * TL::ROW)) + stage_off);
    } else {
      const uint32_t o = stage_off + (uint32_t)(kk * 16 * TL::ROW);
      const s16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CL_LDS s16x4*)(uintptr_t)((base0 ^ (uint32_t)(64 * blk)) + o));
      const s16x4 b2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CL_LDS s16x4*)(uintptr_t)((base1 ^ (uint32_t)(64 * blk)) + o));
      return cat_bf16(b1, b2);
    }
  }
};

// FP8 x FP8 operand fragments (v_mfma_scale_f32_32x32x64_f8f6f4, both operands E4M3): a
// k-contiguous stage row holds 64 FP8 values in four 16-byte pieces, and lane (l32, h) takes
// row l32 of the block, k = 32 h + 0..31: logical pieces 2h and 2h + 1 (two ds_read_b128).
template <int NW, int R>
struct Frag8 {
  uint32_t p0, p1;
  __device__ __forceinline__ void init(uint32_t blk0_off, int lane) {
    using TL = Tile<NW, R, true>;
    const int h = lane >> 5, r = lane & 31;
    const int sw = (r >> 2) & 3;                 // + 32 blk leaves (r >> 2) & 3 unchanged
    p0 = blk0_off + r * TL::ROW + 16 * ((2 * h) ^ sw);
    p1 = blk0_off + r * TL::ROW + 16 * ((2 * h + 1) ^ sw);
  }
  __device__ __forceinline__ i32x8 read(uint32_t stage_off, int blk) const {
    using TL = Tile<NW, R, true>;
    const uint32_t o = stage_off + (uint32_t)(blk * 32 * TL::ROW);
    typedef int i32x4 __attribute__((ext_vector_type(4)));
    const i32x4 x = *lds_ptr<i32x4>(p0 + o);
    const i32x4 y = *lds_ptr<i32x4>(p1 + o);
    return i32x8{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  }
};

template <int NW, int BN> struct WaveGrid;
template <> struct WaveGrid<8, 256> { static constexpr int WM = 2, WN = 4; };
template <> struct WaveGrid<8, 128> { static constexpr int WM = 4, WN = 2; };
template <> struct WaveGrid<4, 128> { static constexpr int WM = 2, WN = 2; };

__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const bf16x2 v = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// Output tile of workgroup blockIdx.x (grid padded to a multiple of 8). Returns false for
// padding workgroups.
__device__ __forceinline__ bool map_tile(int gm, int gn, int gz, int& tm, int& tn, int& tz) {
  const int g = blockIdx.x;
  const int per = (int)(gridDim.x >> 3);
  const int L = (g & 7) * per + (g >> 3);
  const int plane = gm * gn;
  if (L >= plane * gz) return false;
  tz = L / plane;
  const int r = L - tz * plane;
  const int grp = r / (kGroupM * gn);
  const int rem = r - grp * (kGroupM * gn);
  const int gsz = min(kGroupM, gm - grp * kGroupM);
  tn = rem / gsz;
  tm = grp * kGroupM + (rem - tn * gsz);
  return true;
}

// Q8: both operands FP8 E4M3 and k-contiguous, copied to LDS as they are and multiplied by
// the FP8 MFMA (64 k per stage).
template <int NW, int BN, bool AKC, bool BKC, bool AF8, bool BF8, int EPI, bool Q8 = false>
__global__ __launch_bounds__(64 * NW, 2) void k_gemm(const GemmParams p) {
  static_assert(!Q8 || (AKC && BKC && !AF8 && !BF8), "fp8 x fp8 operands are k-contiguous DMA tiles");
  constexpr int BK = Q8 ? 64 : kBK;
  constexpr int kThreads = Cfg<NW, BN>::THREADS;
  using TA = Tile<NW, kBM, AKC, AF8 ? 1 : 2>;
  using TB = Tile<NW, BN, BKC, BF8 ? 1 : 2>;
  constexpr int WM = WaveGrid<NW, BN>::WM, WN = WaveGrid<NW, BN>::WN;
  constexpr int TM = kBM / WM, TN = BN / WN;
  constexpr int MT = TM / 32, NTW = TN / 32;
  constexpr int STAGE = TA::BYTES + TB::BYTES;
  constexpr int NPER = TA::PER_WAVE + TB::PER_WAVE;   // LDS copies per wave and stage
  // The ring keeps the size of the bf16 tiles' ring when an operand is FP8 (the epilogues
  // stage the P image and the dE tile through it). FP8 stages are smaller, but a deeper ring
  // in the same bytes measured no faster on the 3M-item head: its products are bound by
  // HBM bandwidth once the copies run ahead.
  constexpr int kNst = Cfg<NW, BN>::NST;
  constexpr int RING = kNst * (Tile<NW, kBM, AKC>::BYTES + Tile<NW, BN, BKC>::BYTES);
  static_assert(kNst * STAGE <= RING && (kNst - 1) * NPER < 64, "ring");
  __shared__ __attribute__((aligned(1024))) char ring[RING];

  int tm, tn, tz;
  if (!map_tile((int)((p.M + kBM - 1) / kBM), (int)((p.N + BN - 1) / BN),
                (int)((p.K + p.k_per_split - 1) / p.k_per_split), tm, tn, tz))
    return;

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv % WM, wn = wv / WM;
  const int64_t m0 = (int64_t)tm * kBM, n0 = (int64_t)tn * BN;
  const int64_t kz0 = (int64_t)tz * p.k_per_split;
  const int64_t klen = min(p.k_per_split, p.K - kz0);
  const int nk = klen > 0 ? (int)(klen / BK) : 0;
  const uint32_t ring0 = (uint32_t)(uintptr_t)ring;

  Loader<NW, kBM, AKC, AF8, Q8> la;
  Loader<NW, BN, BKC, BF8, Q8> lb;
  la.init(p.a, m0, wv, lane, tid);
  lb.init(p.b, n0, wv, lane, tid);

  Frag<NW, kBM, AKC, AF8> fa;
  Frag<NW, BN, BKC, BF8> fb;
  fa.init(ring0, lane);
  fb.init(ring0 + TA::BYTES, lane);
  const int ablk0 = (wm * TM) / 32, bblk0 = (wn * TN) / 32;

  f32x16 acc[MT][NTW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) acc[mt][nt] = f32x16{};

  // Gradient filter (dA and dE products): wave 0 lists, in order, the k stages whose P tile
  // the logits product flagged; the pipeline then runs over that list only.
  __shared__ int slist[kMaxStages];
  __shared__ int scount;
  bool filt = false;
  int nk_run = nk;
  if constexpr (EPI == GEMM_EPI_ACC || EPI == GEMM_EPI_DE) {
    if (p.flags != nullptr) {
      filt = true;
      if (wv == 0) {
        int cnt = 0;
        for (int b = 0; b < nk; b += 64) {
          const int st = b + lane;
          bool act = false;
          if (st < nk) {
            const int64_t k0 = kz0 + (int64_t)st * kBK;
            if constexpr (EPI == GEMM_EPI_ACC) {   // k = items, M tile = rows t
              const int64_t it = k0 >> 8;
              const int64_t t0 = m0 / p.flag_bn, t1 = min((m0 + kBM - 1) / p.flag_bn, p.flag_ld - 1);
              act = p.flags[it * p.flag_ld + t0] == p.flag_gen || p.flags[it * p.flag_ld + t1] == p.flag_gen;
            } else {                               // M tile = items, k = rows t
              act = p.flags[(m0 >> 8) * p.flag_ld + k0 / p.flag_bn] == p.flag_gen;
            }
          }
          const uint64_t m = __builtin_amdgcn_ballot_w64(act);
          if (act) slist[cnt + __builtin_popcountll(m & ((1ull << lane) - 1))] = st;
          cnt += __builtin_popcountll(m);
        }
        if (lane == 0) scount = cnt;
      }
      __syncthreads();
      nk_run = scount;
    }
  }
  auto stage_k = [&](int s) -> int64_t { return kz0 + (int64_t)(filt ? slist[s] : s) * BK; };

  // Every operand tile arrives by LDS copy, issued as inline asm so that the compiler's
  // waits do not count the copies; none of its own loads may then be left pending inside
  // the main loop.
  wait_vm<0>();

  // dE/SGD epilogue geometry: each wave stages MG row tiles at a time through its share of
  // the ring as fp32 rows of stride RS; a lane then owns SPL segments of 16 adjacent d
  constexpr int WREG = RING / NW;            // LDS bytes per wave
  constexpr int RS = TN * 4 + 16;            // fp32 row stride: 16 B pad spreads the 16-lane reads
  constexpr int MG = (WREG / (32 * RS)) < MT ? (WREG / (32 * RS)) : MT;
  constexpr int SEGS = TN / 16;
  constexpr int SPL = 32 * MG * SEGS / 64;    // segments per lane per group
  constexpr int NG = MT / MG > 0 ? MT / MG : 1;
  // FP8 SGD (either rounding): the E bytes of all the lane's segments are loaded here, before
  // the first stage's copies, so their HBM latency overlaps the pipeline's start and the
  // epilogue never waits for E
  constexpr bool PRE = EPI == GEMM_EPI_SGD;
  const bool pre = PRE && p.e_fp8;
  uint4 epre[PRE ? SPL * NG : 1];
  if constexpr (PRE) {
    if (pre) {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
          const int sg = lane + 64 * i, row = sg / SEGS, seg = sg - row * SEGS;
          const int64_t v = p.v0 + m0 + wm * TM + 32 * (gi * MG) + row;
          const int64_t d0 = n0 + wn * TN + 16 * seg;
          epre[gi * SPL + i] = (v < p.V && d0 < p.D)
                                   ? *(const uint4*)((const uint8_t*)p.E_inplace + v * p.D + d0)
                                   : uint4{0u, 0u, 0u, 0u};
        }
    }
  }
  auto issue = [&](int s) {
    const uint32_t so = ring0 + (uint32_t)((s % kNst) * STAGE);
    const int64_t k0 = stage_k(s);
    dma_stage<NW, kBM, AKC, AF8, Q8>(la, p.a, m0, k0, so, wv, lane);
    dma_stage<NW, BN, BKC, BF8, Q8>(lb, p.b, n0, k0, so + TA::BYTES, wv, lane);
  };

  if constexpr (Q8) {
    // The MFMAs of stage s are issued first and run in the matrix pipe while the wave waits
    // for stage s + 1, passes the barrier that retires stage s (its fragments are in
    // registers) and reads stage s + 1's fragments into the same registers.
    Frag8<NW, kBM> ga;
    Frag8<NW, BN> gb;
    ga.init(ring0, lane);
    gb.init(ring0 + TA::BYTES, lane);
    i32x8 xa[MT], xb[NTW];
    auto read8 = [&](int s) {
      const uint32_t so = (uint32_t)((s % kNst) * STAGE);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) xa[mt] = ga.read(so, ablk0 + mt);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) xb[nt] = gb.read(so, bblk0 + nt);
    };
    if (nk_run > 0) {
      for (int x = 0; x < kNst; ++x)
        if (x < nk_run) issue(x);
      const int later = min(nk_run - 1, kNst - 1);
      if (later >= 3) wait_vm<3 * NPER>(); else if (later == 2) wait_vm<2 * NPER>();
      else if (later == 1) wait_vm<NPER>(); else wait_vm<0>();
      block_sync();
      read8(0);
    }
    for (int s = 0; s < nk_run; ++s) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(xa[mt], xb[nt], acc[mt][nt], 0, 0, 0, 127, 0, 127);
      if (s + 1 < nk_run) {
        const int later = min(nk_run - 2 - s, kNst - 2);      // stages after s + 1 in flight
        if (later >= 2) wait_vm<2 * NPER>(); else if (later == 1) wait_vm<NPER>(); else wait_vm<0>();
        block_sync();
        if (s + kNst < nk_run) issue(s + kNst);
        read8(s + 1);
      }
    }
  } else {
  // Software pipeline, half a stage deep: the LDS reads of one k16 half are in flight while
  // the MFMAs of the other run, and the barrier that retires a ring slot sits between the
  // two MFMA halves of a stage. All kNst slots are in flight after the prologue.
  bf16x8 a0[MT], b0[NTW], a1[MT], b1[NTW];
  auto read_half = [&](int s, int kk, bf16x8* av, bf16x8* bv) {
    const uint32_t so = (uint32_t)((s % kNst) * STAGE);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) av[mt] = fa.read(so, ablk0 + mt, kk);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) bv[nt] = fb.read(so, bblk0 + nt, kk);
  };
  auto mma_half = [&](const bf16x8* av, const bf16x8* bv) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) acc[mt][nt] = mfma32(av[mt], bv[nt], acc[mt][nt]);
  };
  if (nk_run > 0) {
    for (int x = 0; x < kNst; ++x)
      if (x < nk_run) issue(x);
    wait_later<NPER, kNst - 1>(min(nk_run - 1, kNst - 1));   // stages after stage 0 in flight
    wait_lgkm0();
    block_sync();
    read_half(0, 0, a0, b0);
  }
  for (int s = 0; s < nk_run; ++s) {
    read_half(s, 1, a1, b1);
    mma_half(a0, b0);
    if (s + 1 < nk_run) {
      wait_later<NPER, kNst - 2>(min(nk_run - 2 - s, kNst - 2));   // stages after s + 1 in flight
      wait_lgkm0();
      block_sync();                          // stage s retired, stage s + 1 landed
      if (s + kNst < nk_run) issue(s + kNst);
      read_half(s + 1, 0, a0, b0);
    }
    mma_half(a1, b1);
  }
  }

  // ---------------------------------------------------------------- epilogues
  if constexpr (EPI == GEMM_EPI_BCE_P || EPI == GEMM_EPI_BCE_LOSS || EPI == GEMM_EPI_CE_LSE || EPI == GEMM_EPI_CE_P ||
                EPI == GEMM_EPI_BCE_METRICS) {
    constexpr bool BCE_SUM = EPI == GEMM_EPI_BCE_P || EPI == GEMM_EPI_BCE_LOSS || EPI == GEMM_EPI_BCE_METRICS;
    constexpr bool WRITES_P = EPI == GEMM_EPI_BCE_P || EPI == GEMM_EPI_CE_P;
    // row partials of the WM wave rows, combined in wave-row order into one partial per item
    // tile (half or a quarter of the split-reduction traffic)
    constexpr bool PARTS = BCE_SUM || EPI == GEMM_EPI_CE_LSE;
    constexpr bool TWO = EPI == GEMM_EPI_BCE_METRICS || EPI == GEMM_EPI_CE_LSE;
    __shared__ float comb_a[PARTS ? WM : 1][PARTS ? BN : 1];
    __shared__ float comb_b[TWO ? WM : 1][TWO ? BN : 1];
    // Tiles inside the valid item and row ranges skip the per-element masks.
    auto logit_tile = [&](auto tail_c) {
      constexpr bool TAIL = decltype(tail_c)::value;
      const int64_t mw = m0 + wm * TM;          // chunk-relative first item of the wave
      float pabs = 0.0f;                         // CE_P: largest |P| of the wave (gradient filter)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int64_t t = n0 + wn * TN + 32 * nt + l32;
        const bool t_ok = !TAIL || t < p.T;
        const bool t_st = !TAIL || t < p.p_rows; // the P buffer has this row
        float wt = 0.0f, lt = 0.0f;
        if constexpr (EPI == GEMM_EPI_CE_P) wt = t_ok ? p.w[t] : 0.0f;
        if constexpr (EPI == GEMM_EPI_CE_P) lt = t_ok ? p.lse[t] * kLog2e : 0.0f;
        (void)t_st;
        // P image in LDS: item block b, tile row r, 16-byte group j of the block row (XOR
        // swizzled by (r >> 2) & 3 so that 32 rows at once hit distinct banks), half h
        const int pr = (int)(t - n0);
        const uint32_t pimg = (uint32_t)(((int)((mw - m0) >> 5)) * (BN * 64) + pr * 64 + 8 * h);
        float relu = 0.0f, prod = 1.0f, lg = 0.0f, mx = kNegInf, sm = 0.0f, cnt = 0.0f;
        if constexpr (EPI == GEMM_EPI_CE_LSE) {
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int64_t v = p.v0 + mw + 32 * mt + res_row(i, h);
              mx = (!TAIL || (v < p.V && t_ok)) ? __builtin_fmaxf(mx, acc[mt][nt][i]) : mx;
            }
        }
        const float mb = mx == kNegInf ? 0.0f : mx * kLog2e;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float f[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const int i = 4 * j + q;
              const int64_t v = p.v0 + mw + 32 * mt + res_row(i, h);
              const bool ok = !TAIL || (v < p.V && t_ok);
              const float x = acc[mt][nt][i];
              f[q] = 0.0f;
              if constexpr (EPI == GEMM_EPI_BCE_METRICS) cnt += (ok && x > 0.0f) ? 1.0f : 0.0f;
              if constexpr (BCE_SUM) {
                const float e = __builtin_amdgcn_exp2f(-__builtin_fabsf(x) * kLog2e);
                const float qv = 1.0f + e;
                relu += ok ? __builtin_fmaxf(x, 0.0f) : 0.0f;
                prod *= ok ? qv : 1.0f;
                if constexpr (EPI == GEMM_EPI_BCE_P) {   // unweighted: w enters through dA and A_w
                  const float r = __builtin_amdgcn_rcpf(qv);
                  const float sig = x >= 0.0f ? r : e * r;
                  f[q] = ok ? sig : 0.0f;
                }
              } else if constexpr (EPI == GEMM_EPI_CE_LSE) {
                sm += ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -mb)) : 0.0f;
              } else {  // CE_P
                const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -lt));
                f[q] = ok && wt != 0.0f ? wt * e : 0.0f;
                pabs = __builtin_fmaxf(pabs, __builtin_fabsf(f[q]));
              }
            }
            if constexpr (WRITES_P) {
              uint2 pk;
              pk.x = pack2(f[0], f[1]);
              pk.y = pack2(f[2], f[3]);
              *(uint2*)(ring + pimg + mt * (BN * 64) + ((j ^ ((pr >> 2) & 3)) << 4)) = pk;
            }
          }
          if constexpr (BCE_SUM) {
            lg += __builtin_amdgcn_logf(prod);   // log2 of a product of 16 factors in [1, 2]
            prod = 1.0f;
          }
          __builtin_amdgcn_sched_barrier(0);     // one 32-row slice at a time
        }
        const int rr = wn * TN + 32 * nt + l32;   // row of the tile
        if constexpr (BCE_SUM) {
          float vsum = relu + lg * kLn2;
          vsum += __shfl_xor(vsum, 32, 64);
          if (h == 0) comb_a[wm][rr] = vsum;
        }
        if constexpr (EPI == GEMM_EPI_BCE_METRICS) {
          cnt += __shfl_xor(cnt, 32, 64);
          if (h == 0) comb_b[wm][rr] = cnt;
        }
        if constexpr (EPI == GEMM_EPI_CE_LSE) {
          const float m2 = __shfl_xor(mx, 32, 64);
          const float s2 = __shfl_xor(sm, 32, 64);
          const float mn = __builtin_fmaxf(mx, m2);
          float s = 0.0f;
          if (mn != kNegInf) s = sm * __builtin_amdgcn_exp2f((mx - mn) * kLog2e) + s2 * __builtin_amdgcn_exp2f((m2 - mn) * kLog2e);
          if (h == 0) {
            comb_a[wm][rr] = mn;
            comb_b[wm][rr] = s;
          }
        }
      }
      if constexpr (EPI == GEMM_EPI_CE_P) {
        // gradient filter: flag the output tile when some |P| of any wave reaches the threshold
        if (p.flags != nullptr && __builtin_amdgcn_ballot_w64(pabs >= p.filter_eps) != 0 && lane == 0)
          p.flags[(int64_t)tm * p.flag_ld + tn] = p.flag_gen;
      }
    };
    if constexpr (WRITES_P) block_sync();       // the ring becomes the P image
    // (the CE gradient epilogue keeps its masks: without them it runs out of registers)
    if (EPI != GEMM_EPI_CE_P && p.v0 + m0 + kBM <= p.V && n0 + BN <= p.T) logit_tile(BoolC<false>{});
    else logit_tile(BoolC<true>{});
    if constexpr (PARTS) {
      __syncthreads();
      const int64_t split = p.part_base + (int64_t)tm;
      for (int r = tid; r < BN; r += kThreads) {
        const int64_t t = n0 + r;
        if (t >= p.T) continue;
        if constexpr (EPI == GEMM_EPI_CE_LSE) {
          float mn = kNegInf;
#pragma unroll
          for (int q = 0; q < WM; ++q) mn = __builtin_fmaxf(mn, comb_a[q][r]);
          float sum = 0.0f;
          if (mn != kNegInf) {
#pragma unroll
            for (int q = 0; q < WM; ++q)
              if (comb_a[q][r] != kNegInf) sum += comb_b[q][r] * __builtin_amdgcn_exp2f((comb_a[q][r] - mn) * kLog2e);
          }
          p.part_a[split * p.T + t] = mn;
          p.part_b[split * p.T + t] = sum;
        } else {
          float va = 0.0f;
#pragma unroll
          for (int q = 0; q < WM; ++q) va += comb_a[q][r];
          p.part_a[split * p.T + t] = va;
          if constexpr (EPI == GEMM_EPI_BCE_METRICS) {
            float vb = 0.0f;
#pragma unroll
            for (int q = 0; q < WM; ++q) vb += comb_b[q][r];
            p.part_b[split * p.T + t] = vb;
          }
        }
      }
    }
    if constexpr (WRITES_P) {
      // The tile's P is 8 item blocks x BN rows x 64 bytes, and each item block's rows are one
      // contiguous run of the blocked layout (bt is a multiple of BN): copy it out in 16-byte
      // pieces, consecutive threads on consecutive bytes of a run.
      constexpr int IMG = 8 * BN * 64;
      static_assert(IMG <= RING, "P image fits the ring");
      block_sync();
      const int64_t pbs = (int64_t)p.p_bt * 32;
      // all BN rows of the tile lie in one row block of the layout (bt is a multiple of BN and
      // n0 of BN): its block index and first row offset are per-workgroup constants, so the
      // copy loop does no 64-bit division
      const int64_t tblk = n0 / p.p_bt;
      const int64_t toff = n0 - tblk * p.p_bt;
      uint16_t* const pblk = p.P + (tblk * p.p_nvb + (m0 >> 5)) * pbs + toff * 32;
      const int64_t rows_here = p.p_rows - n0;
#pragma unroll 4
      for (int k = tid; k < IMG / 16; k += kThreads) {
        const int b = (16 * k) / (BN * 64);
        const int rem = 16 * k - b * (BN * 64);
        const int r = rem >> 6;
        const int q = ((rem & 63) >> 4) ^ ((r >> 2) & 3);
        if (r < rows_here) {
          typedef int i32x4 __attribute__((ext_vector_type(4)));
          const i32x4 x = *lds_ptr<i32x4>(ring0 + (uint32_t)(16 * k));
          *(i32x4*)(pblk + (int64_t)b * pbs + r * 32 + 8 * q) = x;
        }
      }
    }
  } else if constexpr (EPI == GEMM_EPI_ACC) {
    float* out = p.acc + (int64_t)tz * p.acc_slice;
    if (p.acc_trans) {
      // dA^T tile: result registers 4q..4q+3 hold 4 consecutive d of row n = l32
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const int64_t n = n0 + wn * TN + 32 * nt + l32;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int64_t m = m0 + wm * TM + 32 * mt + 8 * q + 4 * h;
            if (n < p.T && m < p.D) {                // D is a multiple of 64: m .. m + 3 valid
              float4* o = (float4*)(out + n * p.ldacc + m);
              float4 x = {acc[mt][nt][4 * q], acc[mt][nt][4 * q + 1], acc[mt][nt][4 * q + 2], acc[mt][nt][4 * q + 3]};
              if (!p.acc_first) {
                const float4 y = *o;
                x.x += y.x; x.y += y.y; x.z += y.z; x.w += y.w;
              }
              *o = x;
            }
          }
        }
      return;
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int64_t n = n0 + wn * TN + 32 * nt + l32;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t m = m0 + wm * TM + 32 * mt + res_row(i, h);
          if (m < p.T && n < p.D) {
            float* o = out + m * p.ldacc + n;
            *o = p.acc_first ? acc[mt][nt][i] : *o + acc[mt][nt][i];
          }
        }
      }
  } else {  // DE / SGD: rows of the tile go through LDS so that each lane owns 16 adjacent d
    __shared__ int uix[kBM];
    block_sync();                              // every wave is done with the ring
    for (int k = tid; k < kBM; k += kThreads) {
      const int64_t v = p.v0 + m0 + k;
      if (p.imap != nullptr) {               // one load instead of a dependent search
        uix[k] = v < p.V ? p.imap[v] : -1;
        continue;
      }
      const int nu = p.counts[2];
      int lo = 0, hi = nu;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)p.uitems[mid] < v) lo = mid + 1;
        else hi = mid;
      }
      uix[k] = (lo < nu && (int64_t)p.uitems[lo] == v) ? lo : -1;
    }
    static_assert(MG >= 1 && MT % MG == 0 && TN % 16 == 0 && (32 * MG * SEGS) % 64 == 0, "epilogue staging");
    char* wbuf = ring + wv * WREG;
    const uint32_t wb = ring0 + (uint32_t)(wv * WREG);
#pragma unroll
    for (int g0 = 0; g0 < MT; g0 += MG) {
      __syncthreads();
#pragma unroll
      for (int mq = 0; mq < MG; ++mq)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt)
#pragma unroll
          for (int i = 0; i < 16; ++i)
            *(float*)(wbuf + (32 * mq + res_row(i, h)) * RS + 4 * (32 * nt + l32)) = acc[g0 + mq][nt][i];
      __syncthreads();
#pragma unroll
      for (int si = 0; si < SPL; ++si) {
        const int s = lane + 64 * si;
        const int row = s / SEGS, seg = s - row * SEGS;
        const int ml = wm * TM + 32 * g0 + row;
        const int64_t v = p.v0 + m0 + ml;
        const int64_t d0 = n0 + wn * TN + 16 * seg;
        if (v >= p.V || d0 >= p.D) continue;
        float g[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          typedef float f32x4 __attribute__((ext_vector_type(4)));
          const f32x4 x = *lds_ptr<f32x4>(wb + (uint32_t)(row * RS + 64 * seg + 16 * q));
          g[4 * q] = x[0]; g[4 * q + 1] = x[1]; g[4 * q + 2] = x[2]; g[4 * q + 3] = x[3];
        }
        const int u = uix[ml];
        if (u >= 0) {
          const float4* su = (const float4*)(p.S_u + (int64_t)u * p.D + d0);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float4 x = su[q];
            g[4 * q] -= x.x; g[4 * q + 1] -= x.y; g[4 * q + 2] -= x.z; g[4 * q + 3] -= x.w;
          }
        }
        if constexpr (EPI == GEMM_EPI_DE) {
          uint4 o0, o1;
          o0.x = pack2(g[0], g[1]); o0.y = pack2(g[2], g[3]); o0.z = pack2(g[4], g[5]); o0.w = pack2(g[6], g[7]);
          o1.x = pack2(g[8], g[9]); o1.y = pack2(g[10], g[11]); o1.z = pack2(g[12], g[13]); o1.w = pack2(g[14], g[15]);
          uint4* dst = (uint4*)((uint16_t*)p.dE + v * p.D + d0);
          dst[0] = o0;
          dst[1] = o1;
        } else if (p.sr) {
          // the 16 uniforms of d0 .. d0 + 15: Philox counters d / 8 (two of them), half-word d % 8
          uint32_t hw[8];
          sr_uniforms16(p.sr_seed, v, d0, hw);
          auto h16 = [&](int j) -> uint32_t { return sr_h16(hw, j); };
          if (p.e_fp8) {
            uint4* ep = (uint4*)((uint8_t*)p.E_inplace + v * p.D + d0);
            const uint4 e = pre ? epre[PRE ? (g0 / MG) * SPL + si : 0] : *ep;
            const uint32_t w[4] = {e.x, e.y, e.z, e.w};
            uint32_t o[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], false);
              const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], true);
              const float e0 = sr_fp8(__builtin_fmaf(-p.lr, g[4 * q], lo[0]), h16(4 * q));
              const float e1 = sr_fp8(__builtin_fmaf(-p.lr, g[4 * q + 1], lo[1]), h16(4 * q + 1));
              const float e2 = sr_fp8(__builtin_fmaf(-p.lr, g[4 * q + 2], hi[0]), h16(4 * q + 2));
              const float e3 = sr_fp8(__builtin_fmaf(-p.lr, g[4 * q + 3], hi[1]), h16(4 * q + 3));
              int r = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);   // exact: grid values
              r = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, r, true);
              o[q] = (uint32_t)r;
            }
            *ep = uint4{o[0], o[1], o[2], o[3]};
          } else {
            uint4* ep = (uint4*)((uint16_t*)p.E_inplace + v * p.D + d0);
#pragma unroll
            for (int q = 0; q < 2; ++q) {
              const uint4 e = ep[q];
              const uint32_t w[4] = {e.x, e.y, e.z, e.w};
              uint32_t o[4];
#pragma unroll
              for (int b = 0; b < 4; ++b) {
                const int j = 8 * q + 2 * b;
                const float lo = sr_bf16(__builtin_fmaf(-p.lr, g[j], bf16_bits_to_f32(w[b] & 0xffffu)), h16(j));
                const float hi = sr_bf16(__builtin_fmaf(-p.lr, g[j + 1], bf16_bits_to_f32(w[b] >> 16)), h16(j + 1));
                o[b] = (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);   // exact
              }
              ep[q] = uint4{o[0], o[1], o[2], o[3]};
            }
          }
        } else if (p.e_fp8) {
          uint4* ep = (uint4*)((uint8_t*)p.E_inplace + v * p.D + d0);
          const uint4 e = pre ? epre[PRE ? (g0 / MG) * SPL + si : 0] : *ep;
          const uint32_t w[4] = {e.x, e.y, e.z, e.w};
          uint32_t o[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // two E4M3 values per conversion; the clamp to +-448 keeps the hardware
            // conversion from turning |x| > 464 into NaN (saturating RNE)
            const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], false);
            const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[q], true);
            const float e0 = __builtin_amdgcn_fmed3f(__builtin_fmaf(-p.lr, g[4 * q], lo[0]), -kFp8Max, kFp8Max);
            const float e1 = __builtin_amdgcn_fmed3f(__builtin_fmaf(-p.lr, g[4 * q + 1], lo[1]), -kFp8Max, kFp8Max);
            const float e2 = __builtin_amdgcn_fmed3f(__builtin_fmaf(-p.lr, g[4 * q + 2], hi[0]), -kFp8Max, kFp8Max);
            const float e3 = __builtin_amdgcn_fmed3f(__builtin_fmaf(-p.lr, g[4 * q + 3], hi[1]), -kFp8Max, kFp8Max);
            int r = __builtin_amdgcn_cvt_pk_fp8_f32(e0, e1, 0, false);
            r = __builtin_amdgcn_cvt_pk_fp8_f32(e2, e3, r, true);
            o[q] = (uint32_t)r;
          }
          *ep = uint4{o[0], o[1], o[2], o[3]};
        } else {
          uint4* ep = (uint4*)((uint16_t*)p.E_inplace + v * p.D + d0);
#pragma unroll
          for (int q = 0; q < 2; ++q) {
            const uint4 e = ep[q];
            const uint32_t w[4] = {e.x, e.y, e.z, e.w};
            uint32_t o[4];
#pragma unroll
            for (int b = 0; b < 4; ++b) {
              const float lo = bf16_bits_to_f32(w[b] & 0xffffu) - p.lr * g[8 * q + 2 * b];
              const float hi = bf16_bits_to_f32(w[b] >> 16) - p.lr * g[8 * q + 2 * b + 1];
              o[b] = pack2(lo, hi);
            }
            ep[q] = uint4{o[0], o[1], o[2], o[3]};
          }
        }
      }
    }
  }
}

// The operand combinations the chunked path uses:
//   K1: A = E chunk (k-contiguous, bf16 or fp8), B = activations (k-contiguous); with FP8
//       logits both FP8 and multiplied as FP8
//   K2: A = P (k-contiguous), B = the transposed bf16 E chunk (k-contiguous) or the fp8
//       E chunk itself (k-major); for fp8 E and at most 128 rows, dA^T with A = the fp8 E
//       chunk (k-major) and B = P (k-contiguous)
//   K3: A = P (k-major), B = activations (k-major)
template <int NW, int BN>
hipError_t gemm_bn(const GemmParams& p, dim3 grid, hipStream_t st) {
  const bool akc = p.a.kc, bkc = p.b.kc, af8 = p.a.fp8, bf8 = p.b.fp8;
#define CL_G(AKC, BKC, AF8, BF8, E) k_gemm<NW, BN, AKC, BKC, AF8, BF8, E><<<grid, 64 * NW, 0, st>>>(p)
  if (akc && bkc && af8 && bf8) {              // K1 with FP8 activations and FP8 E (8 waves)
    if constexpr (NW == 8) {
      if (p.epi == GEMM_EPI_BCE_P) k_gemm<NW, BN, true, true, false, false, GEMM_EPI_BCE_P, true><<<grid, 64 * NW, 0, st>>>(p);
      else if (p.epi == GEMM_EPI_BCE_LOSS)
        k_gemm<NW, BN, true, true, false, false, GEMM_EPI_BCE_LOSS, true><<<grid, 64 * NW, 0, st>>>(p);
      else return hipErrorInvalidValue;
    } else {
      return hipErrorInvalidValue;
    }
  } else if (akc && bkc && !af8 && !bf8 && p.epi == GEMM_EPI_ACC) {   // K2, bf16 E
    CL_G(true, true, false, false, GEMM_EPI_ACC);
  } else if (akc && bkc && !bf8) {             // K1
    switch (p.epi) {
#define CL_K1(E) case E: if (af8) CL_G(true, true, true, false, E); else CL_G(true, true, false, false, E); break;
      CL_K1(GEMM_EPI_BCE_P) CL_K1(GEMM_EPI_BCE_LOSS) CL_K1(GEMM_EPI_CE_LSE) CL_K1(GEMM_EPI_CE_P)
      CL_K1(GEMM_EPI_BCE_METRICS)
#undef CL_K1
      default: return hipErrorInvalidValue;
    }
  } else if (akc && !bkc && !af8 && bf8 && p.epi == GEMM_EPI_ACC) {    // K2, fp8 E
    // the raw FP8 tile of BN columns must split into whole 1 KB copies per wave (the
    // planner never pairs an FP8 B tile of 128 columns with 8 waves)
    if constexpr (BN * 32 / 1024 >= NW && (BN * 32 / 1024) % NW == 0) CL_G(true, false, false, true, GEMM_EPI_ACC);
    else return hipErrorInvalidValue;
  } else if (!akc && bkc && af8 && !bf8 && p.epi == GEMM_EPI_ACC) {    // K2 as dA^T = E_c^T P^T, fp8 E
    CL_G(false, true, true, false, GEMM_EPI_ACC);
  } else if (!akc && !bkc && !af8 && !bf8) {   // K3: both operands k-major
    if (p.epi == GEMM_EPI_DE) {
      CL_G(false, false, false, false, GEMM_EPI_DE);
    } else if (p.epi == GEMM_EPI_SGD) {
      CL_G(false, false, false, false, GEMM_EPI_SGD);
    } else {
      return hipErrorInvalidValue;
    }
  } else {
    return hipErrorInvalidValue;
  }
#undef CL_G
  return hipGetLastError();
}

// Et[d][v] = E[v][d] for v < vlen and 0 for vlen <= v < mc: one 64 x 64 tile per
// workgroup, read as 128-byte row pieces of E and written as 128-byte row pieces of Et.
__global__ __launch_bounds__(256) void k_transpose_chunk(const uint16_t* __restrict__ E, int64_t vlen, int64_t D,
                                                         uint16_t* __restrict__ Et, int64_t ld) {
  // t[v][d] in 128-byte rows, the 16-byte chunk k of row v stored at chunk k ^ ((v / 8) mod 8):
  // written 16 bytes a lane (two rows x 8 chunks per 16 lanes: distinct slots) and read a
  // halfword a lane down a column (8 rows 8 apart per wave: 8 different chunks)
  __shared__ uint4 t[64 * 8];
  const int tid = threadIdx.x;
  const int64_t v0 = (int64_t)blockIdx.x * 64, d0 = (int64_t)blockIdx.y * 64;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = tid / 8 + 32 * h, k = tid % 8;
    uint4 x = {0u, 0u, 0u, 0u};
    if (v0 + r < vlen) x = *(const uint4*)(E + (v0 + r) * D + d0 + 8 * k);
    t[r * 8 + (k ^ ((r >> 3) & 7))] = x;
  }
  __syncthreads();
  const uint16_t* const th = (const uint16_t*)t;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int d = tid / 8 + 32 * h, k = tid % 8;   // rows 8 k .. 8 k + 7 (their v / 8 is k)
    const int col = 8 * ((d >> 3) ^ k) + (d & 7);
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = (uint32_t)th[(8 * k + 2 * i) * 64 + col] | ((uint32_t)th[(8 * k + 2 * i + 1) * 64 + col] << 16);
    *(uint4*)(Et + (d0 + d) * ld + v0 + 8 * k) = uint4{o[0], o[1], o[2], o[3]};
  }
}

// 8 activations per thread: 16 bytes in, 8 bytes out
__global__ __launch_bounds__(256) void k_cast_fp8(const uint16_t* __restrict__ A, int64_t n8, uint8_t* __restrict__ A8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const uint4 x = *(const uint4*)(A + 8 * i);
  const uint32_t w[4] = {x.x, x.y, x.z, x.w};
  uint32_t o[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const float a0 = __builtin_amdgcn_fmed3f(bf16_bits_to_f32(w[2 * q] & 0xffffu), -kFp8Max, kFp8Max);
    const float a1 = __builtin_amdgcn_fmed3f(bf16_bits_to_f32(w[2 * q] >> 16), -kFp8Max, kFp8Max);
    const float a2 = __builtin_amdgcn_fmed3f(bf16_bits_to_f32(w[2 * q + 1] & 0xffffu), -kFp8Max, kFp8Max);
    const float a3 = __builtin_amdgcn_fmed3f(bf16_bits_to_f32(w[2 * q + 1] >> 16), -kFp8Max, kFp8Max);
    int r = __builtin_amdgcn_cvt_pk_fp8_f32(a0, a1, 0, false);
    r = __builtin_amdgcn_cvt_pk_fp8_f32(a2, a3, r, true);
    o[q] = (uint32_t)r;
  }
  *(uint2*)(A8 + 8 * i) = uint2{o[0], o[1]};
}

}  // namespace

hipError_t launch_cast_fp8(const uint16_t* A, int64_t n, uint8_t* A8, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  if (n % 8 != 0) return hipErrorInvalidValue;
  const int64_t n8 = n / 8;
  k_cast_fp8<<<(unsigned)((n8 + 255) / 256), 256, 0, st>>>(A, n8, A8);
  return hipGetLastError();
}

hipError_t launch_transpose_chunk(const uint16_t* E, int64_t vlen, int64_t mc, int64_t D, uint16_t* Et, int64_t ld,
                                  hipStream_t st) {
  if (vlen <= 0 || mc % 64 != 0 || vlen > mc || D % 64 != 0 || ld < mc || ld % 8 != 0) return hipErrorInvalidValue;
  k_transpose_chunk<<<dim3((unsigned)(mc / 64), (unsigned)(D / 64)), 256, 0, st>>>(E, vlen, D, Et, ld);
  return hipGetLastError();
}

// Workgroup shape of a product: 4 waves (two workgroups per CU) for heads up to D = 1024,
// where the logits epilogue and the short k loops gain most from the overlap, except the
// dA product of very few rows (one row tile) or over D >= 512 columns, and FP8 x FP8 logits,
// which take 8 waves.
int gemm_waves(const GemmParams& p) {
  if (p.D > 1024) return 8;
  if (p.epi == GEMM_EPI_ACC && p.M <= 128) return 8;
  // dA product over a wide output (N = D >= 512): 256 x 256 tiles stream fewer operand bytes
  // per flop than two 256 x 128 workgroups
  if (p.epi == GEMM_EPI_ACC && p.N >= 512) return 8;
  if (p.a.fp8 && p.b.fp8) return 8;   // FP8 x FP8 logits: 4 waves would spill (two 8-register fragments per block)
  return 4;
}
int tile_n_for(int nw, int64_t N) { return (nw == 4 || N <= 128) ? 128 : 256; }

int gemm_tile_m() { return kBM; }
int gemm_tile_n_of(int epi, int64_t M, int64_t N, int64_t D) {
  GemmParams q{};
  q.epi = epi; q.M = M; q.N = N; q.D = D;
  return tile_n_for(gemm_waves(q), N);
}

hipError_t launch_gemm(const GemmParams& p, hipStream_t st) {
  if (p.M <= 0 || p.N <= 0 || p.K <= 0 || p.K % kBK != 0 || p.k_per_split % kBK != 0 || p.k_per_split <= 0)
    return hipErrorInvalidValue;
  // FP8 x FP8: 64 k per stage, no k tail, k-contiguous operands
  if (p.a.fp8 && p.b.fp8 && (p.K % 64 != 0 || p.k_per_split % 64 != 0 || !p.a.kc || !p.b.kc)) return hipErrorInvalidValue;
  const int nw = gemm_waves(p);
  const int bn = tile_n_for(nw, p.N);
  const int64_t gm = (p.M + kBM - 1) / kBM, gn = (p.N + bn - 1) / bn, gz = (p.K + p.k_per_split - 1) / p.k_per_split;
  // every tile's outer origin lies inside its operand (the loaders clamp relative to it);
  // operands have at least one row and one 8-element group per row
  const int64_t a_outer = p.a.kc ? p.a.rows_valid : p.a.cols_valid;
  const int64_t b_outer = p.b.kc ? p.b.rows_valid : p.b.cols_valid;
  if ((gm - 1) * kBM >= a_outer || (gn - 1) * bn >= b_outer || p.a.rows_valid < 1 || p.b.rows_valid < 1 ||
      p.a.cols_valid < 8 || p.b.cols_valid < 8)
    return hipErrorInvalidValue;
  // a 16-byte piece of an FP8 operand holds 16 elements: at least one whole piece per row
  // (the loaders clamp columns to cols_valid - 16)
  if ((p.a.fp8 && p.a.cols_valid < 16) || (p.b.fp8 && p.b.cols_valid < 16)) return hipErrorInvalidValue;
  // blocked operands (bf16 only): bt a multiple of 32 (a k stage of 32 stored rows stays in
  // one row block), the whole k range valid, and every column of a tile stored
  for (const GemmOperand* op : {&p.a, &p.b}) {
    if (op->bt <= 0) continue;
    const int64_t tile = op == &p.a ? kBM : bn;
    const int64_t outer_tiles = op == &p.a ? gm : gn;
    if (op->fp8 || op->bt % 32 != 0 || (op->kc ? p.K > op->cols_valid : p.K > op->rows_valid) ||
        (!op->kc && outer_tiles * tile > op->cols_valid))
      return hipErrorInvalidValue;
  }
  if (p.flags != nullptr && (p.epi == GEMM_EPI_ACC || p.epi == GEMM_EPI_DE) && p.k_per_split / kBK > kMaxStages)
    return hipErrorInvalidValue;
  const int64_t tiles = gm * gn * gz;
  if (tiles > ((int64_t)1 << 30)) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((tiles + 7) / 8 * 8));
  if (nw == 4) return gemm_bn<4, 128>(p, grid, st);
  return bn == 128 ? gemm_bn<8, 128>(p, grid, st) : gemm_bn<8, 256>(p, grid, st);
}

}  // namespace cl
