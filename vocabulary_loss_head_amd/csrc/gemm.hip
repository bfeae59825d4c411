// Chunked path for wide classifier heads (D > 256, or FP8 embeddings): per vocabulary
// chunk of Vc items, three MFMA GEMMs with fused epilogues.
//
//   K1  X^T = E_c A^T          (M = chunk items, N = rows, K = D)
//       BCE: P = w sigmoid(X) -> bf16 [Vc][T] buffer, softplus row partials;
//       CE forward: (max, sum) row partials; CE backward: P = w exp(X - lse).
//   K2  dA (+)= P^T-chunk E_c   (M = rows, N = D, K = Vc), fp32 split-K partials
//   K3  dE_c = P A - S          (M = chunk items, N = D, K = rows): bf16 dE, or the
//       SGD step on E in place (ELMO summary, Key Contributions 2: gradient fused with
//       the update, never stored).
//
// Cut Binary Cross Entropy (paperpeel) §III-A forms the logits of one vocabulary block
// at a time and discards them; here only the chunk's gradient tile P (T x Vc bf16) is
// kept, long enough for K2 and K3 to consume it. The executed matrix work is 6 T V D
// (no recompute), and at D >= 512 each GEMM stays compute-bound with P in HBM.
//
// Kernel: 8 waves, 256 x (256 | 128) output tile, K stages of 32 in a 4-deep LDS ring.
// bf16 operands arrive by global_load_lds_dwordx4 (lane-linear 1 KB blocks); FP8
// operands go through registers and are widened to bf16 exactly on the way to LDS.
// An operand tile is either k-contiguous ([rows][32 k], read with ds_read_b128) or
// k-major ([32 k][cols], read transposed with ds_read_b64_tr_b16); both read patterns
// give lane (l, h) the k values 16 kk + 8 h + 0..7, so any pair of modes composes.
#include "common.h"

#define CL_GAS __attribute__((address_space(1)))

namespace cl {

namespace {

constexpr int kBK = 32;
constexpr int kNst = 4;
constexpr int kBM = 256;
constexpr int kThreads = 512;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ int swz_f(int r) { return ((r & 7) << 1) | ((r >> 3) & 1); }
__device__ __forceinline__ int res_row(int i, int h) { return 8 * (i >> 2) + 4 * h + (i & 3); }

template <class T>
__device__ __forceinline__ const CL_LDS T* lds_ptr(uint32_t a) { return (const CL_LDS T*)(uintptr_t)a; }

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt");
  __builtin_amdgcn_s_waitcnt(0xF70 | N);
}
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

__device__ __forceinline__ void block_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
}

// One stage of one operand: R rows (KC) or R columns (KR) by 32 k, bf16 in LDS.
template <int R, bool KC>
struct Tile {
  static constexpr int BYTES = 64 * R;
  static constexpr int KB = BYTES / 1024;
  static constexpr int PER_WAVE = KB / 8;             // DMA blocks per wave
  static constexpr int ROW = KC ? 64 : 2 * R;         // bytes per LDS row
  static constexpr int NCH = ROW / 16;
  static constexpr int PIECES = BYTES / 16 / kThreads;  // staged pieces per thread
  static_assert(PER_WAVE >= 1 && PIECES >= 1, "tile");
  __device__ __forceinline__ static int phys(int lp, int r) {   // an involution in lp
    if constexpr (KC) return lp ^ ((r >> 2) & 3);
    else return lp ^ (swz_f(r) & (NCH - 1));
  }
  // storage element offset of the 8-element group that belongs at LDS byte `byte`
  __device__ __forceinline__ static int64_t src(const GemmOperand& op, int64_t outer0, int64_t k0, int byte) {
    const int r = byte / ROW;
    const int lp = phys((byte % ROW) / 16, r);
    int64_t row, col;
    if constexpr (KC) {
      row = outer0 + r;
      col = k0 + 8 * lp;
    } else {
      row = k0 + r;
      col = outer0 + 8 * lp;
    }
    row = row < op.rows_valid ? row : op.rows_valid - 1;
    col = col <= op.cols_valid - 8 ? col : op.cols_valid - 8;
    return row * op.ld + col;
  }
};

template <int R, bool KC>
__device__ __forceinline__ void dma_tile(const GemmOperand& op, int64_t outer0, int64_t k0, uint32_t lds, int wv,
                                         int lane) {
  using TL = Tile<R, KC>;
  asm volatile("" : "+v"(lane));     // recompute the cheap per-lane offsets at every issue
#pragma unroll
  for (int j = 0; j < TL::PER_WAVE; ++j) {
    const int kb = wv * TL::PER_WAVE + j;
    const int64_t off = TL::src(op, outer0, k0, kb * 1024 + 16 * lane);
    __builtin_amdgcn_global_load_lds((const CL_GAS void*)((const uint16_t*)op.p + off),
                                     (CL_LDS void*)(uintptr_t)(lds + kb * 1024), 16, 0, 0);
  }
}

template <int R, bool KC>
struct Fp8Stage {
  uint2 q[Tile<R, KC>::PIECES];
  __device__ __forceinline__ void load(const GemmOperand& op, int64_t outer0, int64_t k0, int tid) {
#pragma unroll
    for (int i = 0; i < Tile<R, KC>::PIECES; ++i) {
      const int64_t off = Tile<R, KC>::src(op, outer0, k0, 16 * (tid + kThreads * i));
      q[i] = *(const uint2*)((const uint8_t*)op.p + off);
    }
  }
  __device__ __forceinline__ void store(uint32_t lds, int tid) const {
#pragma unroll
    for (int i = 0; i < Tile<R, KC>::PIECES; ++i)
      *(CL_LDS bf16x8*)(uintptr_t)(lds + 16 * (tid + kThreads * i)) = fp8x8_to_bf16x8(q[i]);
  }
};

// MFMA operand fragments of a stage tile: lane (l32, h) gets index l32 of the 32-wide
// block `blk` and k = 16 kk + 8 h + 0..7.
template <int R, bool KC>
struct Frag {
  uint32_t base0, base1;   // KC: row-read base; KR: transposed-read bases (k rows +0..3, +4..7)
  __device__ __forceinline__ void init(uint32_t blk0_off, int lane) {
    using TL = Tile<R, KC>;
    const int h = lane >> 5, l32 = lane & 31;
    if constexpr (KC) {
      const int r = l32;                         // + 32 blk: does not change (r >> 2) & 3
      const int sw = (r >> 2) & 3;
      base0 = blk0_off + r * TL::ROW + 16 * ((sw & 2) | (h ^ (sw & 1)));
      base1 = 0;
    } else {
      const int rsub = (lane & 15) >> 2;
      const int c0 = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
      const int co = 8 * (lane & 1);
      const int rA = 8 * h + rsub, rB = rA + 4;
      base0 = blk0_off + rA * TL::ROW + co + 16 * (c0 ^ (swz_f(rA) & (TL::NCH - 1)));
      base1 = blk0_off + rB * TL::ROW + co + 16 * (c0 ^ (swz_f(rB) & (TL::NCH - 1)));
    }
  }
  // blk: 32-wide block index within the tile's R; kk: 16-k half of the stage
  __device__ __forceinline__ bf16x8 read(uint32_t stage_off, int blk, int kk) const {
    using TL = Tile<R, KC>;
    if constexpr (KC) {
      return *lds_ptr<bf16x8>(((base0 ^ (uint32_t)(32 * kk)) + (uint32_t)(blk * 32 * TL::ROW)) + stage_off);
    } else {
      const uint32_t o = stage_off + (uint32_t)(kk * 16 * TL::ROW);
      const s16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CL_LDS s16x4*)(uintptr_t)((base0 ^ (uint32_t)(64 * blk)) + o));
      const s16x4 b2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((CL_LDS s16x4*)(uintptr_t)((base1 ^ (uint32_t)(64 * blk)) + o));
      return cat_bf16(b1, b2);
    }
  }
};

template <int BN> struct WaveGrid;
template <> struct WaveGrid<256> { static constexpr int WM = 2, WN = 4; };
template <> struct WaveGrid<128> { static constexpr int WM = 4, WN = 2; };

__device__ __forceinline__ uint16_t bf16_bits(float x) { return (uint16_t)f32_to_bf16_bits(x); }

template <int BN, bool AKC, bool BKC, bool AF8, bool BF8, int EPI>
__global__ __launch_bounds__(kThreads, 2) void k_gemm(const GemmParams p) {
  using TA = Tile<kBM, AKC>;
  using TB = Tile<BN, BKC>;
  constexpr int WM = WaveGrid<BN>::WM, WN = WaveGrid<BN>::WN;
  constexpr int TM = kBM / WM, TN = BN / WN;
  constexpr int MT = TM / 32, NTW = TN / 32;
  constexpr int STAGE = TA::BYTES + TB::BYTES;
  constexpr int NPER = (AF8 ? TA::PIECES : TA::PER_WAVE) + (BF8 ? TB::PIECES : TB::PER_WAVE);
  __shared__ __attribute__((aligned(1024))) char ring[kNst * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wv % WM, wn = wv / WM;
  const int64_t m0 = (int64_t)blockIdx.x * kBM, n0 = (int64_t)blockIdx.y * BN;
  const int64_t kz0 = (int64_t)blockIdx.z * p.k_per_split;
  const int64_t klen = min(p.k_per_split, p.K - kz0);
  const int nk = klen > 0 ? (int)(klen / kBK) : 0;
  const uint32_t ring0 = (uint32_t)(uintptr_t)ring;

  Frag<kBM, AKC> fa;
  Frag<BN, BKC> fb;
  fa.init(ring0, lane);
  fb.init(ring0 + TA::BYTES, lane);
  const int ablk0 = (wm * TM) / 32, bblk0 = (wn * TN) / 32;

  f32x16 acc[MT][NTW];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) acc[mt][nt] = f32x16{};

  Fp8Stage<kBM, AKC> sa;
  Fp8Stage<BN, BKC> sb;
  // fp8 register loads are issued before the stage's DMAs, so waiting for them at the
  // next step does not wait for those DMAs.
  auto issue = [&](int s) {
    const uint32_t so = ring0 + (uint32_t)((s % kNst) * STAGE);
    const int64_t k0 = kz0 + (int64_t)s * kBK;
    if constexpr (AF8) sa.load(p.a, m0, k0, tid);
    if constexpr (BF8) sb.load(p.b, n0, k0, tid);
    if constexpr (!AF8) dma_tile<kBM, AKC>(p.a, m0, k0, so, wv, lane);
    if constexpr (!BF8) dma_tile<BN, BKC>(p.b, n0, k0, so + TA::BYTES, wv, lane);
  };
  auto store_fp8 = [&](int s) {
    const uint32_t so = ring0 + (uint32_t)((s % kNst) * STAGE);
    if constexpr (AF8) sa.store(so, tid);
    if constexpr (BF8) sb.store(so + TA::BYTES, tid);
  };

  for (int s = 0; s < kNst - 1; ++s) {
    if (s < nk) {
      issue(s);
      store_fp8(s);
    }
  }
  for (int s = 0; s < nk; ++s) {
    if constexpr (AF8 || BF8) {
      if (s >= 1 && s + kNst - 2 < nk) store_fp8(s + kNst - 2);   // loaded at step s - 1
      wait_lgkm0();
    }
    const int later = min(nk - 1 - s, kNst - 2);
    if (later >= 2) wait_vm<2 * NPER>(); else if (later == 1) wait_vm<NPER>(); else wait_vm<0>();
    block_sync();
    if (s + kNst - 1 < nk) issue(s + kNst - 1);
    const uint32_t so = (uint32_t)((s % kNst) * STAGE);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 av[MT], bv[NTW];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) av[mt] = fa.read(so, ablk0 + mt, kk);
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) bv[nt] = fb.read(so, bblk0 + nt, kk);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) acc[mt][nt] = mfma32(av[mt], bv[nt], acc[mt][nt]);
    }
  }

  // ---------------------------------------------------------------- epilogues
  if constexpr (EPI == GEMM_EPI_BCE_P || EPI == GEMM_EPI_BCE_LOSS || EPI == GEMM_EPI_CE_LSE || EPI == GEMM_EPI_CE_P) {
    const int64_t split = p.part_base + (int64_t)blockIdx.x * WM + wm;
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) {
      const int64_t t = n0 + wn * TN + 32 * nt + l32;
      const bool t_ok = t < p.T;
      float wt = 0.0f, lt = 0.0f;
      if constexpr (EPI == GEMM_EPI_BCE_P || EPI == GEMM_EPI_CE_P) wt = t_ok ? p.w[t] : 0.0f;
      if constexpr (EPI == GEMM_EPI_CE_P) lt = t_ok ? p.lse[t] * kLog2e : 0.0f;
      float relu = 0.0f, prod = 1.0f, lg = 0.0f, mx = kNegInf, sm = 0.0f;
      if constexpr (EPI == GEMM_EPI_CE_LSE) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int64_t v = p.v0 + m0 + wm * TM + 32 * mt + res_row(i, h);
            mx = (v < p.V && t_ok) ? __builtin_fmaxf(mx, acc[mt][nt][i]) : mx;
          }
      }
      const float mb = mx == kNegInf ? 0.0f : mx * kLog2e;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int64_t ml = m0 + wm * TM + 32 * mt + res_row(i, h);
          const int64_t v = p.v0 + ml;
          const bool ok = v < p.V && t_ok;
          const float x = acc[mt][nt][i];
          if constexpr (EPI == GEMM_EPI_BCE_P || EPI == GEMM_EPI_BCE_LOSS) {
            const float e = __builtin_amdgcn_exp2f(-__builtin_fabsf(x) * kLog2e);
            const float q = 1.0f + e;
            relu += ok ? __builtin_fmaxf(x, 0.0f) : 0.0f;
            prod *= ok ? q : 1.0f;
            if constexpr (EPI == GEMM_EPI_BCE_P) {
              const float r = __builtin_amdgcn_rcpf(q);
              const float sig = x >= 0.0f ? r : e * r;
              if (t < p.ldp) p.P[ml * p.ldp + t] = bf16_bits(ok ? wt * sig : 0.0f);
            }
            if ((i & 15) == 15) {      // log2 of a product of 16 factors in [1, 2]
              lg += __builtin_amdgcn_logf(prod);
              prod = 1.0f;
            }
          } else if constexpr (EPI == GEMM_EPI_CE_LSE) {
            sm += ok ? __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -mb)) : 0.0f;
          } else {  // CE_P
            const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -lt));
            if (t < p.ldp) p.P[ml * p.ldp + t] = bf16_bits(ok && wt != 0.0f ? wt * e : 0.0f);
          }
        }
        __builtin_amdgcn_sched_barrier(0);     // one 32-row slice at a time
      }
      if constexpr (EPI == GEMM_EPI_BCE_P || EPI == GEMM_EPI_BCE_LOSS) {
        float vsum = relu + lg * kLn2;
        vsum += __shfl_xor(vsum, 32, 64);
        if (h == 0 && t_ok) p.part_a[split * p.T + t] = vsum;
      }
      if constexpr (EPI == GEMM_EPI_CE_LSE) {
        const float m2 = __shfl_xor(mx, 32, 64);
        const float s2 = __shfl_xor(sm, 32, 64);
        const float mn = __builtin_fmaxf(mx, m2);
        float s = 0.0f;
        if (mn != kNegInf) s = sm * __builtin_amdgcn_exp2f((mx - mn) * kLog2e) + s2 * __builtin_amdgcn_exp2f((m2 - mn) * kLog2e);
        if (h == 0 && t_ok) {
          p.part_a[split * p.T + t] = mn;
          p.part_b[split * p.T + t] = s;
        }
      }
    }
  } else if constexpr (EPI == GEMM_EPI_ACC) {
    float* out = p.acc + (int64_t)blockIdx.z * p.acc_slice;
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
  } else {  // DE / SGD
    block_sync();                              // the ring is free: reuse it for item indices
    int* uix = (int*)ring;
    for (int k = tid; k < kBM; k += kThreads) {
      const int64_t v = p.v0 + m0 + k;
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
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ml = wm * TM + 32 * mt + res_row(i, h);
        const int64_t v = p.v0 + m0 + ml;
        if (v >= p.V) continue;
        const int u = uix[ml];
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
          const int64_t d = n0 + wn * TN + 32 * nt + l32;
          if (d >= p.D) continue;
          float g = acc[mt][nt][i];
          if (u >= 0) g -= p.S_u[(int64_t)u * p.D + d];
          if constexpr (EPI == GEMM_EPI_DE) {
            ((uint16_t*)p.dE)[v * p.D + d] = bf16_bits(g);
          } else if (p.e_fp8) {
            uint8_t* e8 = (uint8_t*)p.E_inplace + v * p.D + d;
            *e8 = (uint8_t)f32_to_fp8_sat(fp8_to_f32(*e8) - p.lr * g);
          } else {
            uint16_t* e16 = (uint16_t*)p.E_inplace + v * p.D + d;
            *e16 = bf16_bits(bf16_bits_to_f32(*e16) - p.lr * g);
          }
        }
      }
  }
}

// The three operand combinations the chunked path uses:
//   K1: A = E chunk (k-contiguous, bf16 or fp8), B = activations (k-contiguous)
//   K2: A = P (k-major), B = E chunk (k-major, bf16 or fp8)
//   K3: A = P (k-contiguous), B = activations (k-major)
template <int BN>
hipError_t gemm_bn(const GemmParams& p, dim3 grid, hipStream_t st) {
  const bool akc = p.a.kc, bkc = p.b.kc, af8 = p.a.fp8, bf8 = p.b.fp8;
#define CL_G(AKC, BKC, AF8, BF8, E) k_gemm<BN, AKC, BKC, AF8, BF8, E><<<grid, kThreads, 0, st>>>(p)
  if (akc && bkc && !bf8) {                    // K1
    switch (p.epi) {
#define CL_K1(E) case E: if (af8) CL_G(true, true, true, false, E); else CL_G(true, true, false, false, E); break;
      CL_K1(GEMM_EPI_BCE_P) CL_K1(GEMM_EPI_BCE_LOSS) CL_K1(GEMM_EPI_CE_LSE) CL_K1(GEMM_EPI_CE_P)
#undef CL_K1
      default: return hipErrorInvalidValue;
    }
  } else if (!akc && !bkc && !af8 && p.epi == GEMM_EPI_ACC) {   // K2
    if (bf8) CL_G(false, false, false, true, GEMM_EPI_ACC);
    else CL_G(false, false, false, false, GEMM_EPI_ACC);
  } else if (akc && !bkc && !af8 && !bf8) {    // K3
    if (p.epi == GEMM_EPI_DE) CL_G(true, false, false, false, GEMM_EPI_DE);
    else if (p.epi == GEMM_EPI_SGD) CL_G(true, false, false, false, GEMM_EPI_SGD);
    else return hipErrorInvalidValue;
  } else {
    return hipErrorInvalidValue;
  }
#undef CL_G
  return hipGetLastError();
}

}  // namespace

int gemm_tile_m() { return kBM; }
int gemm_tile_n(int64_t N) { return N <= 128 ? 128 : 256; }
int gemm_warps_m(int64_t N) { return N <= 128 ? WaveGrid<128>::WM : WaveGrid<256>::WM; }

hipError_t launch_gemm(const GemmParams& p, hipStream_t st) {
  if (p.M <= 0 || p.N <= 0 || p.K <= 0 || p.K % kBK != 0 || p.k_per_split % kBK != 0 || p.k_per_split <= 0)
    return hipErrorInvalidValue;
  const int bn = gemm_tile_n(p.N);
  const dim3 grid((unsigned)((p.M + kBM - 1) / kBM), (unsigned)((p.N + bn - 1) / bn),
                  (unsigned)((p.K + p.k_per_split - 1) / p.k_per_split));
  return bn == 128 ? gemm_bn<128>(p, grid, st) : gemm_bn<256>(p, grid, st);
}

}  // namespace cl
