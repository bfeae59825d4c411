// Logit-tile sweeps for bf16 streamed operands and D in {64, 128, 256} (gfx950).
//
// The computation follows Cut Binary Cross Entropy §III-A..C (dense softplus term, sigmoid
// gradient recomputed per tile) and the Cut Your Losses article (online logsumexp, softmax
// gradient), arranged for measured CDNA4 limits:
//  * each wave holds MT 32-row tiles of the stationary matrix in VGPRs (MT = 2 for
//    D = 64; 1 for D = 128 and 256, where the 128 gradient accumulators and 64 stationary
//    registers of a D = 256 tile fill the 256 VGPRs of two waves per SIMD), so every LDS
//    read of a streamed chunk feeds MT MFMAs in the logit product and in the gradient
//    product;
//  * the logit and gradient products keep several LDS operand reads in flight ahead of
//    their MFMAs; the sigmoid/exp epilogue of one wave runs while the other wave of the
//    SIMD issues matrix work;
//  * streamed 32-row chunks go HBM/L2 -> LDS by global_load_lds_dwordx4 (no staging
//    registers, no ds_write) into a 4-buffer ring inside one LDS array. The copies are
//    issued as inline asm (lds_dma16): the compiler would otherwise wait for all copies in
//    flight before every transposing read. Each step waits for its own copies with an
//    explicit vmcnt, one s_barrier publishes the chunk to the workgroup and retires the
//    oldest buffer, and the next copies are issued right after;
//  * rows past the end of a range are fetched as copies of the last valid row (never
//    out of bounds) and their logits are set to -inf, which makes every epilogue
//    (softplus, sigmoid, exp) contribute exactly zero; only the last chunk of a range
//    can hold such rows, so only that chunk runs the masked epilogue.
//
// LDS layout of a chunk: rows at a stride of ROW + 16 bytes, so row r starts at bank
// slot r (mod 16) of the 256-byte bank window. A DMA instruction writes 1 KB
// lane-linearly: lane i of block kb fetches the piece that belongs at byte
// kb*1024 + 16 i (pad slots fetch a harmless copy), and a chunk takes 4 n + 1 blocks.
// Reads need no swizzle: a logits read (one 16-byte piece of 16 rows per 16 lanes)
// hits 16 distinct slots, and a transposed read touches rows 4 apart (4 q + 2 h + b,
// see pi_row) whose 64-byte windows tile the bank window. Every read address is a
// per-lane base plus an immediate offset.
#include "common.h"

#define CL_GAS __attribute__((address_space(1)))

namespace cl {

namespace {

constexpr int kRC = 32;          // streamed rows per chunk
// LDS buffers (a power of two). Eight (six chunks in flight instead of two) measured 0.3%
// faster sweeps but a 7% slower forward at T = 4096, D = 256 (more of E in flight per CU
// against the L2 reuse of each chunk by the row blocks).
#ifndef CL_SWEEP_RING
#define CL_SWEEP_RING 4
#endif
constexpr int kRing = CL_SWEEP_RING;
// LDS operand reads kept in flight ahead of their MFMAs: as many as the register budget
// of two waves per SIMD leaves without spilling inside the chunk loop
#ifndef CL_ROWS_READ_AHEAD
#define CL_ROWS_READ_AHEAD 4
#endif
#ifndef CL_COLS_LOGITS_READ_AHEAD
#define CL_COLS_LOGITS_READ_AHEAD 4
#endif
#ifndef CL_COLS_READ_AHEAD
#define CL_COLS_READ_AHEAD 2
#endif
constexpr float kNegInf = -__builtin_inff();

// For each D: MT stationary 32-row tiles per wave, NW waves per workgroup and WPE
// workgroups per CU (two waves per SIMD in every case). At D = 128, MT = 2 would need one
// wave per SIMD (the accumulators of two tiles exceed 256 registers); the epilogue then
// has no second wave to run beside, and the sweeps take 24% longer than with MT = 1 and
// two waves per SIMD (T = 16384, V = 100000). With NW = 8 the two waves of a
// SIMD belong to one workgroup and run out of phase (see sweep_loop).
template <int D> struct Tiling;
template <> struct Tiling<64> { static constexpr int MT = 2, NW = 4, WPE = 2; };
template <> struct Tiling<128> { static constexpr int MT = 1, NW = 8, WPE = 1; };
template <> struct Tiling<256> { static constexpr int MT = 1, NW = 8, WPE = 1; };

template <int D>
struct Geo {
  static constexpr int NCH = D / 8;             // 16-byte pieces per row
  static constexpr int ROW = 2 * D;             // bytes of row data
  static constexpr int ROWP = ROW + 16;         // LDS row stride
  static constexpr int KBP = (kRC * ROWP + 1023) / 1024;   // DMA blocks per chunk (4 n + 1)
  static constexpr int BUF = KBP * 1024;        // LDS bytes per ring buffer
  static constexpr int LPWP = KBP / Tiling<D>::NW;   // blocks of every wave; wave 0 also takes the last
  static_assert(KBP % Tiling<D>::NW == 1, "padded chunk layout");
};


__device__ __forceinline__ uint32_t lds_addr(const void* p) { return (uint32_t)(uintptr_t)p; }
template <class T>
__device__ __forceinline__ const CL_LDS T* lds_ptr(uint32_t a) { return (const CL_LDS T*)(uintptr_t)a; }

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt[3:0] and vmcnt[5:4] at bits 15:14, expcnt[6:4] = 7,
// lgkmcnt[11:8] = 15).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0xF70 | (N & 15) | ((N >> 4) << 14));
}
// wait until at most `later` chunks of P copies each are in flight (later <= K)
template <int P, int K>
__device__ __forceinline__ void wait_later(int later) {
  if constexpr (K > 0) {
    if (later >= K) {
      wait_vm<K * P>();
      return;
    }
    wait_later<P, K - 1>(later);
  } else {
    wait_vm<0>();
  }
}

__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// Chunk position of streamed row r: the logits read of lane l32 takes LDS row
// pi_row(l32), so the logit in result register i of half h belongs to LDS row
// pi_row(res_row(i, h)) = 16 (i >> 3) + 4 (i & 3) + 2 h + ((i >> 2) & 1), and the
// k-block of the gradient product that a transposed read serves is rows 4 q + 2 h + b.
__device__ __forceinline__ int pi_row(int r) {
  return (r & 16) | ((r & 3) << 2) | (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
}

// Source offsets (bf16 elements from the chunk's first row) of this lane's DMA blocks:
// blocks wv * LPWP + j, and for wave 0 also the last block. Pad slots and bytes past the
// chunk fetch element 0. `lim` clamps rows (the last valid row of a short chunk).
template <int D>
struct DmaOffsets {
  int32_t off[Geo<D>::LPWP + 1];
  __device__ __forceinline__ static int32_t at(int kb, int lane, int lim) {
    using G = Geo<D>;
    const int byte = kb * 1024 + 16 * lane;
    const int r = byte / G::ROWP;
    const int w = byte - r * G::ROWP;
    if (r >= kRC || w >= G::ROW) return 0;
    return min(r, lim) * D + (w >> 4) * 8;
  }
  __device__ __forceinline__ static int block(int j, int wv) {
    return j < Geo<D>::LPWP ? wv * Geo<D>::LPWP + j : Geo<D>::KBP - 1;
  }
  __device__ __forceinline__ void init(int wv, int lane) {
#pragma unroll
    for (int j = 0; j <= Geo<D>::LPWP; ++j) off[j] = at(block(j, wv), lane, kRC - 1);
  }
};

// Fetch rows [row0, row0 + 32) of a row-major bf16 [*, D] matrix into the LDS buffer at
// byte address `buf`; rows at or past `row_end` (> row0) are fetched as copies of
// row_end - 1. `wv` is wave-uniform, so each instruction's LDS destination is scalar.
template <int D>
__device__ __forceinline__ void dma_chunk(const DmaOffsets<D>& dof, const uint16_t* base, int64_t row0,
                                          int64_t row_end, uint32_t buf, int wv, int lane) {
  using G = Geo<D>;
  const char* cbase = (const char*)(base + row0 * D);       // wave-uniform
  const int lim = (int)min((int64_t)(kRC - 1), row_end - 1 - row0);
  const int nb = G::LPWP + (wv == 0 ? 1 : 0);
  if (lim == kRC - 1) {
#pragma unroll
    for (int j = 0; j <= G::LPWP; ++j) {
      if (j == G::LPWP && nb == G::LPWP) break;
      const int kb = DmaOffsets<D>::block(j, wv);
      lds_dma16(cbase, 2 * (uint32_t)dof.off[j], buf + kb * 1024);
    }
  } else {
    // the offsets of a short chunk are computed here from an opaque copy of the lane id,
    // so that none of their terms is hoisted out of the chunk loop into live registers
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int j = 0; j <= G::LPWP; ++j) {
      if (j == G::LPWP && nb == G::LPWP) break;
      const int kb = DmaOffsets<D>::block(j, wv);
      const int32_t o = DmaOffsets<D>::at(kb, ln, lim);
      lds_dma16(cbase, 2 * (uint32_t)o, buf + kb * 1024);
    }
  }
}

// 32 floats of v for the rows of a chunk (clamped to n - 1) into LDS at `buf`: slot j
// holds row row0 + pi_row(j), the row whose logits sit where result row j would be.
__device__ __forceinline__ void dma_vec(const float* v, int64_t row0, int64_t n, uint32_t buf, int lane) {
  int64_t r = row0 + pi_row(lane & 31);
  r = r < n ? r : n - 1;
  if (lane < 32) lds_dma4(v, 4 * (uint32_t)r, buf);
}

template <int D, bool FP8>
__device__ __forceinline__ void load_stationary(bf16x8 (&sf)[D / 16], const void* base, int64_t row, bool ok, int h) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    if (!ok) { sf[ks] = bf16x8{}; continue; }
    if constexpr (FP8) {
      const uint2 q = *(const uint2*)((const uint8_t*)base + row * D + 16 * ks + 8 * h);
      sf[ks] = fp8x8_to_bf16x8(q);
    } else {
      sf[ks] = *(const bf16x8*)((const uint16_t*)base + row * D + 16 * ks + 8 * h);
    }
  }
}

// chunk row held in result register i of a lane with half h
__device__ __forceinline__ int res_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

// Per-lane LDS read bases of a chunk at ring offset 0.
//  rowb: 16-byte read of piece 2 ks + h of LDS row pi_row(l32) = rowb + 32 ks
//  tr0/tr1: transposed 8-byte reads of column tile nt, LDS rows 4 q + 2 h (+ 1) with
//           q = (lane & 15) >> 2 = trX + 64 nt, plus 16 rows (kk = 1) = + 16 * ROWP
template <int D>
struct ReadBase {
  uint32_t rowb, tr0, tr1;
  __device__ __forceinline__ void init(uint32_t ring, int lane) {
    using G = Geo<D>;
    const int h = lane >> 5, l32 = lane & 31;
    rowb = ring + pi_row(l32) * G::ROWP + 16 * h;
    const int q = (lane & 15) >> 2;
    tr0 = ring + (4 * q + 2 * h) * G::ROWP + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);
    tr1 = tr0 + G::ROWP;
  }
};

template <int D>
__device__ __forceinline__ bf16x8 read_row_piece(const ReadBase<D>& rb, uint32_t boff, int ks) {
  return *lds_ptr<bf16x8>(rb.rowb + boff + (uint32_t)(32 * ks));
}

template <int D>
__device__ __forceinline__ bf16x8 read_col_piece(const ReadBase<D>& rb, uint32_t boff, int nt, int kk) {
  const uint32_t o = boff + (uint32_t)(64 * nt + kk * 16 * Geo<D>::ROWP);
  const s16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CL_LDS s16x4*)(uintptr_t)(rb.tr0 + o));
  const s16x4 b2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CL_LDS s16x4*)(uintptr_t)(rb.tr1 + o));
  return cat_bf16(b1, b2);
}

// Logits of chunk rows at or past `lim` (chunk-relative, wave-uniform) become -inf.
template <int MT>
__device__ __forceinline__ void mask_tail(f32x16 (&y)[MT], int lim, int h) {
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 16; ++i) y[mt][i] = (pi_row(res_row(i, h)) < lim) ? y[mt][i] : kNegInf;
}

// ------------------------------------------------------------------------------------
// Epilogue of one chunk for MT tiles, visited element by element so that a caller can
// interleave it with matrix work.
//   RM 0: BCE softplus sum + sigmoid (F)      RM 1: sigmoid only
//   RM 2: BCE softplus sum only                RM 3: CE running (max, sum)
//   RM 4: exp(x - lse_row) (CE rows gradient)  RM 5: w_r * sigmoid(x) (BCE cols)
//   RM 6: w_r * exp(x - lse_r) (CE cols)       RM 7: RM 2 + count of logits > 0
// ------------------------------------------------------------------------------------
template <int MT, int RM>
struct Epi {
  float relu[MT], lg[MT], prod[MT];
  float sx[MT], sa[MT];     // sums of x and |x| over full chunks: relu = (sx + sa) / 2
  float cnt[MT];            // RM 7: logits > 0 (exact in fp32 below 2^24)
  float run_m[MT], run_s[MT], mb[MT];
  float lse_s[MT];
  uint32_t vb = 0;          // LDS address of the chunk's per-row vectors (cols kinds)

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      relu[mt] = 0.0f; lg[mt] = 0.0f; prod[mt] = 1.0f; sx[mt] = 0.0f; sa[mt] = 0.0f; cnt[mt] = 0.0f;
      run_m[mt] = kNegInf; run_s[mt] = 0.0f; mb[mt] = 0.0f; lse_s[mt] = 0.0f;
    }
  }
  // before the elements of a chunk (CE needs the chunk max first)
  __device__ __forceinline__ void begin(const f32x16 (&y)[MT]) {
    if constexpr (RM == 3) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        float xm = y[mt][0];
#pragma unroll
        for (int i = 1; i < 16; ++i) xm = __builtin_fmaxf(xm, y[mt][i]);
        const float mn = __builtin_fmaxf(run_m[mt], xm);
        // rescale the running sum to the new max (0 while nothing finite has been seen)
        run_s[mt] = mn == kNegInf ? 0.0f : run_s[mt] * __builtin_amdgcn_exp2f((run_m[mt] - mn) * kLog2e);
        run_m[mt] = mn;
        mb[mt] = mn == kNegInf ? 0.0f : mn * kLog2e;
      }
    }
  }
  // per-row weight (and CE logsumexp) of result registers i, i+1 (adjacent chunk rows),
  // read from LDS where they are used
  __device__ __forceinline__ f32x2 row_pair(int i, int h, int which) const {
    return *lds_ptr<f32x2>(vb + 4 * (which * kRC + res_row(i, h)));
  }
  template <bool TAIL>
  __device__ __forceinline__ void elem2(int mt, int i, int h, float x0, float x1, float& f0, float& f1) {
    if constexpr (RM == 5) {
      const f32x2 w = row_pair(i, h, 0);
      f0 = w[0] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x0 * kLog2e));
      f1 = w[1] * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x1 * kLog2e));
    } else if constexpr (RM == 6) {
      const f32x2 w = row_pair(i, h, 0);
      const f32x2 l = row_pair(i, h, 1);
      const float e0 = __builtin_amdgcn_exp2f((x0 - l[0]) * kLog2e);
      const float e1 = __builtin_amdgcn_exp2f((x1 - l[1]) * kLog2e);
      f0 = w[0] != 0.0f ? w[0] * e0 : 0.0f;           // ignored rows: exactly 0
      f1 = w[1] != 0.0f ? w[1] * e1 : 0.0f;
    } else {
      f0 = elem<TAIL>(mt, i, x0);
      f1 = elem<TAIL>(mt, i + 1, x1);
    }
  }
  // TAIL: the chunk may hold -inf logits (rows past the range), which the sums of x and
  // |x| cannot take; other chunks hold finite logits only
  template <bool TAIL>
  __device__ __forceinline__ float elem(int mt, int i, float x) {
    if constexpr (RM == 7) cnt[mt] += x > 0.0f ? 1.0f : 0.0f;
    if constexpr (RM == 0 || RM == 2 || RM == 7) {
      const float e = __builtin_amdgcn_exp2f(-__builtin_fabsf(x) * kLog2e);   // e^-|x| in [0, 1]
      const float q = 1.0f + e;
      if constexpr (TAIL) {
        relu[mt] += __builtin_fmaxf(x, 0.0f);
      } else {
        sx[mt] += x;
        sa[mt] += __builtin_fabsf(x);
      }
      prod[mt] *= q;
      if constexpr (RM == 0) {
        const float r = __builtin_amdgcn_rcpf(q);
        return x >= 0.0f ? r : e * r;
      }
      return 0.0f;
    } else if constexpr (RM == 1) {
      // 1 / (1 + 2^(-x log2 e)): the exp overflows to +inf for x << 0, giving 0
      return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-x * kLog2e));
    } else if constexpr (RM == 3) {
      run_s[mt] += __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -mb[mt]));
      return 0.0f;
    } else if constexpr (RM == 4) {
      return __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -lse_s[mt]));
    }
    return 0.0f;    // RM 5, 6 go through elem2
  }
  __device__ __forceinline__ void end() {
    if constexpr (RM == 0 || RM == 2 || RM == 7) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        lg[mt] += __builtin_amdgcn_logf(prod[mt]);   // log2 of a product of 16 factors in [1, 2]
        prod[mt] = 1.0f;
      }
    }
  }
};

template <int RM> struct EpiHasF { static constexpr bool value = (RM == 0 || RM == 1 || (RM >= 4 && RM <= 6)); };

// packed bf16 operand of the gradient product: pw[mt][kk][j] = bf16 pair (F[8kk+2j], F[8kk+2j+1])
template <int MT>
struct FPack {
  uint32_t pw[MT][2][4];
  __device__ __forceinline__ bf16x8 op(int mt, int kk) const {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 v = {pw[mt][kk][0], pw[mt][kk][1], pw[mt][kk][2], pw[mt][kk][3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 v = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

// y = logits of the chunk in buffer `boff` for the MT stationary tiles.
template <int D, int MT, int RA>
__device__ __forceinline__ void chunk_logits(const bf16x8 (&sf)[MT][D / 16], f32x16 (&y)[MT], const ReadBase<D>& rb,
                                             uint32_t boff) {
  constexpr int KS = D / 16;
  constexpr int PF = KS < RA ? KS : RA;
  bf16x8 ra[PF];
#pragma unroll
  for (int j = 0; j < PF; ++j) ra[j] = read_row_piece<D>(rb, boff, j);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) y[mt] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const bf16x8 a = ra[ks % PF];
    if (ks + PF < KS) ra[ks % PF] = read_row_piece<D>(rb, boff, ks + PF);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) y[mt] = mfma32(a, sf[mt][ks], y[mt]);
  }
  // keep PF reads in flight: the first PF reads, then each step's MFMAs followed by the
  // read that refills the slot they consumed
  __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    __builtin_amdgcn_sched_group_barrier(0x008, MT, 0);
    if (ks + PF < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// Epilogue of the chunk whose logits are y, producing the packed gradient operand fo.
template <int MT, int RM, bool TAIL>
__device__ __forceinline__ void epilogue(const f32x16 (&y)[MT], Epi<MT, RM>& ep, FPack<MT>& fo, int h) {
  constexpr int NP = MT * 8;                    // element pairs per chunk
  constexpr bool HAS_F = EpiHasF<RM>::value;
  ep.begin(y);
#pragma unroll
  for (int e = 0; e < NP; ++e) {
    const int mt = e / 8, i = 2 * (e % 8);
    float f0, f1;
    ep.template elem2<TAIL>(mt, i, h, y[mt][i], y[mt][i + 1], f0, f1);
    if constexpr (HAS_F) fo.pw[mt][i / 8][(i % 8) / 2] = pack_bf16x2(f0, f1);
  }
  ep.end();
}

template <int D, int MT, int RA>
__device__ __forceinline__ void grad_only(f32x16 (&acc)[MT][D / 32], const FPack<MT>& fi, const ReadBase<D>& rb,
                                          uint32_t boff) {
  constexpr int NI = 2 * (D / 32);
  constexpr int PF = NI < RA ? NI : RA;
  bf16x8 rbuf[PF];
#pragma unroll
  for (int j = 0; j < PF; ++j) rbuf[j] = read_col_piece<D>(rb, boff, j % (D / 32), j / (D / 32));
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int nt = it % (D / 32), kk = it / (D / 32);
    const bf16x8 b = rbuf[it % PF];
    if (it + PF < NI) rbuf[it % PF] = read_col_piece<D>(rb, boff, (it + PF) % (D / 32), (it + PF) / (D / 32));
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) acc[mt][nt] = mfma32(fi.op(mt, kk), b, acc[mt][nt]);
  }
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * PF, 0);
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    __builtin_amdgcn_sched_group_barrier(0x008, MT, 0);
    if (it + PF < NI) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
}

// CE gradient filter (Cut Your Losses article, the note on the softmax tail below numerical
// precision): true when some |P| of the wave's chunk tile is at least the bf16 pattern
// `bits`; wave-uniform.
template <int MT>
__device__ __forceinline__ bool wave_any_at_least(const FPack<MT>& f, uint32_t bits) {
  uint32_t m = 0;
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t v = f.pw[mt][kk][j] & 0x7FFF7FFFu;
        m = max(m, max(v & 0xFFFFu, v >> 16));
      }
  return __builtin_amdgcn_ballot_w64(m >= bits) != 0;
}

// ------------------------------------------------------------------------------------
// The chunk loop shared by both sweeps. issue(c, boff) enqueues the DMA of chunk c into
// the buffer at ring offset boff (NPER0 instructions on wave 0, NPER on the others);
// prep(c, boff) points the epilogue at the chunk's per-row inputs.
// Per chunk a wave computes the logit tile (matrix work), its epilogue (VALU work) and the
// gradient product (matrix work). With 8-wave workgroups the second half of the waves
// lags by a chunk phase: in the period of chunk c it runs the epilogue and gradient
// product of chunk c - 1 and then the logits of chunk c, whose tile it keeps for the next
// period. The two waves that share a SIMD (wv and wv + 4) thus offer VALU work while the
// other issues MFMAs. The lagging waves still read chunk c - 1 during period c, so only
// two chunks are in flight beyond the current one; otherwise three.
// ------------------------------------------------------------------------------------
template <int D, int MT, int RM, bool TAIL>
__device__ __forceinline__ void epilogue_and_mask(f32x16 (&y)[MT], Epi<MT, RM>& ep, FPack<MT>& f, int64_t left, int h) {
  if (TAIL) mask_tail<MT>(y, (int)left, h);
  epilogue<MT, RM, TAIL>(y, ep, f, h);
}

template <int D, int MT, int RM, int NPER0, int NPER, int RAL, int RAG, class Issue, class Prep>
__device__ __forceinline__ void sweep_loop(int nch, int64_t rows_left0, const bf16x8 (&sf)[MT][D / 16],
                                           f32x16 (&acc)[MT][D / 32], Epi<MT, RM>& ep, const ReadBase<D>& rb,
                                           int h, int wv, uint32_t filter_bits, Issue issue, Prep prep) {
  using G = Geo<D>;
  constexpr bool HAS_F = EpiHasF<RM>::value;
  constexpr bool SHIFT = Tiling<D>::NW == 8;
  constexpr int AHEAD = SHIFT ? kRing - 2 : kRing - 1;
  static_assert((AHEAD - 1) * NPER0 < 64 && (kRing & (kRing - 1)) == 0 && AHEAD >= 2, "vmcnt / ring");
  if (nch <= 0) return;
  const bool lag = SHIFT && wv >= 4;       // wave-uniform
  // the stationary operand's loads complete here: the compiler does not count the LDS
  // copies, so no wait of its own may remain pending inside the loop
  wait_vm<0>();
#pragma unroll
  for (int k = 0; k < AHEAD; ++k)
    if (k < nch) issue(k, (uint32_t)(k * G::BUF));
  FPack<MT> f;
  f32x16 y[MT];
  // epilogue and gradient product of chunk k (buffer at ring offset bk), y holding its logits
  auto finish = [&](int k, uint32_t bk) {
    const int64_t left = rows_left0 - (int64_t)k * kRC;
    if (left < kRC) epilogue_and_mask<D, MT, RM, true>(y, ep, f, left, h);
    else epilogue_and_mask<D, MT, RM, false>(y, ep, f, left, h);
    if constexpr (HAS_F) {
      bool keep = true;
      if constexpr (RM == 4 || RM == 6) keep = filter_bits == 0 || wave_any_at_least(f, filter_bits);
      if (keep) grad_only<D, MT, RAG>(acc, f, rb, bk);
    }
  };
  // top of the period of chunk c: own copies of chunk c done, chunk c published, copies
  // of chunk c + AHEAD issued
  auto period = [&](int c) {
    const int later = min(nch - 1 - c, AHEAD - 1);   // own later chunks left in flight
    if (wv == 0) wait_later<NPER0, AHEAD - 1>(later);
    else wait_later<NPER, AHEAD - 1>(later);
    block_sync();
    if (c + AHEAD < nch) issue(c + AHEAD, (uint32_t)(((c + AHEAD) & (kRing - 1)) * G::BUF));
  };
  if (!lag) {
    for (int c = 0; c < nch; ++c) {
      const uint32_t boff = (uint32_t)((c & (kRing - 1)) * G::BUF);
      period(c);
      prep(c, boff);
      chunk_logits<D, MT, RAL>(sf, y, rb, boff);
      finish(c, boff);
    }
    return;
  }
  period(0);
  chunk_logits<D, MT, RAL>(sf, y, rb, 0);
  for (int c = 1; c < nch; ++c) {
    const uint32_t boff = (uint32_t)((c & (kRing - 1)) * G::BUF);
    const uint32_t bprev = (uint32_t)(((c - 1) & (kRing - 1)) * G::BUF);
    period(c);
    prep(c - 1, bprev);
    finish(c - 1, bprev);
    chunk_logits<D, MT, RAL>(sf, y, rb, boff);
  }
  {
    const uint32_t blast = (uint32_t)(((nch - 1) & (kRing - 1)) * G::BUF);
    prep(nch - 1, blast);
    finish(nch - 1, blast);
  }
}

// ------------------------------------------------------------------------------------
// rows sweep. MODE: 0 BCE loss partials, 1 BCE dA partials, 2 BCE dA + loss partials,
// 3 CE (max, sum) partials, 4 CE dA partials, 5 BCE loss partials + counts of logits > 0
// (the dense part of the Cut Metrics, Cut Binary Cross Entropy §III-D).
// ------------------------------------------------------------------------------------
template <int MODE> struct RowsRM;
template <> struct RowsRM<0> { static constexpr int RM = 2; };
template <> struct RowsRM<1> { static constexpr int RM = 1; };
template <> struct RowsRM<2> { static constexpr int RM = 0; };
template <> struct RowsRM<3> { static constexpr int RM = 3; };
template <> struct RowsRM<4> { static constexpr int RM = 4; };
template <> struct RowsRM<5> { static constexpr int RM = 7; };

template <int D, int MODE>
__global__ __launch_bounds__(64 * Tiling<D>::NW, Tiling<D>::WPE) void k_rows2(const SweepParams p) {
  using G = Geo<D>;
  constexpr int MT = Tiling<D>::MT;
  constexpr int RM = RowsRM<MODE>::RM;
  constexpr bool HAS_F = EpiHasF<RM>::value;
  constexpr int KS = D / 16, NT = D / 32;
  constexpr int SB = 32 * MT * Tiling<D>::NW;   // stationary rows per workgroup
  __shared__ __attribute__((aligned(1024))) char ring[kRing * G::BUF];

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nsb = (int)((p.T + SB - 1) / SB);
  const int g = blockIdx.x;
  int split, sb;
  if ((p.n_splits & 7) == 0) {          // workgroup g runs on XCD g % 8: one split per XCD
    const int loc = g >> 3;
    split = (g & 7) + 8 * (loc / nsb);
    sb = loc % nsb;
  } else {
    split = g / nsb;
    sb = g % nsb;
  }
  const int64_t s_wave = (int64_t)sb * SB + wv * 32 * MT;
  const int64_t r_begin = (int64_t)split * p.split_len;
  const int64_t r_end = min(p.V, r_begin + p.split_len);
  const int nch = r_end > r_begin ? (int)((r_end - r_begin + kRC - 1) / kRC) : 0;
  const uint16_t* E = (const uint16_t*)p.E;
  const uint32_t ring0 = lds_addr(ring);

  bf16x8 sf[MT][KS];
  Epi<MT, RM> ep;
  ep.init();
  f32x16 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int64_t srow = s_wave + 32 * mt + l32;
    load_stationary<D, false>(sf[mt], p.A, srow, srow < p.T, h);
    if constexpr (RM == 4) ep.lse_s[mt] = srow < p.T ? p.lse[srow] * kLog2e : 0.0f;
    if constexpr (HAS_F) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x16{};
    }
  }
  ReadBase<D> rb;
  rb.init(ring0, lane);
  DmaOffsets<D> dof;
  dof.init(wv, lane);

  auto issue = [&](int c, uint32_t boff) {
    dma_chunk<D>(dof, E, r_begin + (int64_t)c * kRC, r_end, ring0 + boff, wv, lane);
  };
  auto prep = [&](int, uint32_t) {};
  sweep_loop<D, MT, RM, G::LPWP + 1, G::LPWP, CL_ROWS_READ_AHEAD, CL_ROWS_READ_AHEAD>(nch, r_end - r_begin, sf, acc, ep, rb, h, wv, p.filter_bits, issue, prep);

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int64_t srow = s_wave + 32 * mt + l32;
    const bool s_ok = srow < p.T;
    if constexpr (RM == 0 || RM == 2 || RM == 7) {
      float v = ep.relu[mt] + 0.5f * (ep.sx[mt] + ep.sa[mt]) + ep.lg[mt] * kLn2;
      v += __shfl_xor(v, 32, 64);
      if (h == 0 && s_ok) p.part_a[(int64_t)split * p.T + srow] = v;
    }
    if constexpr (RM == 7) {
      float c = ep.cnt[mt];
      c += __shfl_xor(c, 32, 64);
      if (h == 0 && s_ok) p.part_b[(int64_t)split * p.T + srow] = c;
    }
    if constexpr (RM == 3) {
      const float m1 = ep.run_m[mt], s1 = ep.run_s[mt];
      const float m2 = __shfl_xor(m1, 32, 64);
      const float s2 = __shfl_xor(s1, 32, 64);
      const float mn = __builtin_fmaxf(m1, m2);
      float s = 0.0f;
      if (mn != kNegInf) s = s1 * __builtin_amdgcn_exp2f((m1 - mn) * kLog2e) + s2 * __builtin_amdgcn_exp2f((m2 - mn) * kLog2e);
      if (h == 0 && s_ok) {
        p.part_a[(int64_t)split * p.T + srow] = mn;
        p.part_b[(int64_t)split * p.T + srow] = s;
      }
    }
    if constexpr (HAS_F) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t s = s_wave + 32 * mt + res_row(i, h);
          if (s < p.T) p.part_dA[((int64_t)split * p.T + s) * D + 32 * nt + l32] = acc[mt][nt][i];
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// cols sweep: 128*MT stationary E rows per workgroup (bf16 E), A streamed with the row
// weights (and the CE logsumexp). KIND 0 BCE, 1 CE. EPI 0 writes dE (bf16), EPI 1 applies
// E <- bf16(E - lr dE) in place (nearest-even).
// ------------------------------------------------------------------------------------
template <int D, int KIND, int EPI>
__global__ __launch_bounds__(64 * Tiling<D>::NW, Tiling<D>::WPE) void k_cols2(const SweepParams p) {
  using G = Geo<D>;
  constexpr int MT = Tiling<D>::MT;
  constexpr int RM = KIND == 0 ? 5 : 6;
  constexpr int NT = D / 32, KS = D / 16;
  constexpr int NV = KIND == 1 ? 2 : 1;     // per-row vectors streamed with A: w (and lse)
  constexpr int SB = 32 * MT * Tiling<D>::NW;
  __shared__ __attribute__((aligned(1024))) char ring[kRing * G::BUF];
  __shared__ __attribute__((aligned(256))) float vecs[kRing][NV][kRC];
  __shared__ int uix[SB];

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t v_blk = (int64_t)blockIdx.x * SB;
  const int64_t s_wave = v_blk + wv * 32 * MT;
  const int nch = (int)((p.T + kRC - 1) / kRC);
  const uint16_t* A = (const uint16_t*)p.A;
  const uint32_t ring0 = lds_addr(ring);
  const uint32_t vec0 = lds_addr(vecs);

  bf16x8 sf[MT][KS];
  f32x16 acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int64_t srow = s_wave + 32 * mt + l32;
    load_stationary<D, false>(sf[mt], p.E, srow, srow < p.V, h);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = f32x16{};
  }
  Epi<MT, RM> ep;
  ep.init();
  ReadBase<D> rb;
  rb.init(ring0, lane);
  DmaOffsets<D> dof;
  dof.init(wv, lane);

  auto issue = [&](int c, uint32_t boff) {
    const int64_t r0 = (int64_t)c * kRC;
    const uint32_t vb = vec0 + (boff / G::BUF) * (NV * kRC * 4);
    dma_chunk<D>(dof, A, r0, p.T, ring0 + boff, wv, lane);
    dma_vec(p.w, r0, p.T, vb, lane);
    if constexpr (KIND == 1) dma_vec(p.lse, r0, p.T, vb + kRC * 4, lane);
  };
  auto prep = [&](int, uint32_t boff) { ep.vb = vec0 + (boff / G::BUF) * (NV * kRC * 4); };
  sweep_loop<D, MT, RM, G::LPWP + 1 + NV, G::LPWP + NV, CL_COLS_LOGITS_READ_AHEAD, CL_COLS_READ_AHEAD>(nch, p.T, sf, acc, ep, rb, h, wv, p.filter_bits, issue, prep);

  // sparse positive term: index of each item of the block in the sorted unique-item list
  for (int k = tid; k < SB; k += 64 * Tiling<D>::NW) {
    const int64_t v = v_blk + k;
    const int nu = p.counts[2];
    int lo = 0, hi = nu;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)p.uitems[mid] < v) lo = mid + 1;
      else hi = mid;
    }
    uix[k] = (lo < nu && (int64_t)p.uitems[lo] == v) ? lo : -1;
  }
  __syncthreads();

#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = wv * 32 * MT + 32 * mt + res_row(i, h);
      const int64_t v = v_blk + m;
      if (v >= p.V) continue;
      const int u = uix[m];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int d = 32 * nt + l32;
        float gv = acc[mt][nt][i];
        if (u >= 0) gv -= p.S_u[(int64_t)u * D + d];
        if constexpr (EPI == 0) {
          ((uint16_t*)p.dE)[v * D + d] = (uint16_t)f32_to_bf16_bits(gv);
        } else {
          uint16_t* e16 = (uint16_t*)p.E_inplace + v * D + d;
          *e16 = (uint16_t)f32_to_bf16_bits(bf16_bits_to_f32(*e16) - p.lr * gv);
        }
      }
    }
  }
}

template <int D>
hipError_t rows2_d(const SweepParams& p, int mode, hipStream_t st) {
  constexpr int SB = 32 * Tiling<D>::MT * Tiling<D>::NW;
  const int nsb = (int)((p.T + SB - 1) / SB);
  const dim3 grid((unsigned)(nsb * p.n_splits)), block(64 * Tiling<D>::NW);
  switch (mode) {
    case 0: k_rows2<D, 0><<<grid, block, 0, st>>>(p); break;
    case 1: k_rows2<D, 1><<<grid, block, 0, st>>>(p); break;
    case 2: k_rows2<D, 2><<<grid, block, 0, st>>>(p); break;
    case 3: k_rows2<D, 3><<<grid, block, 0, st>>>(p); break;
    case 4: k_rows2<D, 4><<<grid, block, 0, st>>>(p); break;
    case 5: k_rows2<D, 5><<<grid, block, 0, st>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t cols2_d(const SweepParams& p, int kind, int epi, hipStream_t st) {
  const int64_t sb = 32 * Tiling<D>::MT * Tiling<D>::NW;
  const dim3 grid((unsigned)((p.V + sb - 1) / sb)), block(64 * Tiling<D>::NW);
  if (p.e_fp8) return hipErrorInvalidValue;     // FP8 E runs the chunked path
  switch (kind * 2 + epi) {
    case 0: k_cols2<D, 0, 0><<<grid, block, 0, st>>>(p); break;
    case 1: k_cols2<D, 0, 1><<<grid, block, 0, st>>>(p); break;
    case 2: k_cols2<D, 1, 0><<<grid, block, 0, st>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool sweep2_rows_supported(int64_t D, int e_fp8) { return !e_fp8 && (D == 64 || D == 128 || D == 256); }
bool sweep2_cols_supported(int64_t D, int e_fp8) { return !e_fp8 && (D == 64 || D == 128 || D == 256); }
int sweep2_rows_per_block(int64_t D) {
  switch (D) {
    case 64: return 32 * Tiling<64>::MT * Tiling<64>::NW;
    case 128: return 32 * Tiling<128>::MT * Tiling<128>::NW;
    case 256: return 32 * Tiling<256>::MT * Tiling<256>::NW;
    default: return 128;
  }
}

int sweep2_waves_per_block(int64_t D) {
  switch (D) {
    case 64: return Tiling<64>::NW;
    case 128: return Tiling<128>::NW;
    case 256: return Tiling<256>::NW;
    default: return 4;
  }
}

hipError_t launch_sweep2_rows(const SweepParams& p, int mode, hipStream_t st) {
  switch (p.D) {
    case 64: return rows2_d<64>(p, mode, st);
    case 128: return rows2_d<128>(p, mode, st);
    case 256: return rows2_d<256>(p, mode, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_sweep2_cols(const SweepParams& p, int kind, int epi, hipStream_t st) {
  switch (p.D) {
    case 64: return cols2_d<64>(p, kind, epi, st);
    case 128: return cols2_d<128>(p, kind, epi, st);
    case 256: return cols2_d<256>(p, kind, epi, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cl
