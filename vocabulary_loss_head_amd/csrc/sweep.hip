// Fused logit-tile sweeps for D <= 512 (gfx950, v_mfma_f32_32x32x16_bf16).
//
// Cut Binary Cross Entropy (paperpeel) §III-A tiles the vocabulary and never keeps a
// logit block; §III-B recomputes the blocks in the backward pass; §III-C accumulates
// the embedding gradient of a vocabulary block on chip across row tiles. Cut Your
// Losses (abeam.tech article) does the same for softmax CE with an online max/sum.
//
// Both sweeps share one structure. A workgroup of 4 waves holds 128 "stationary" rows
// (32 per wave) in VGPRs as MFMA operands and streams the other matrix through LDS in
// chunks of 32 rows:
//   Y  = R_chunk . S^T                 (M = streamed row r, N = stationary row s, K = D)
//   F  = f(Y)                          (sigmoid, exp(x - lse), softplus/LSE reductions)
//   dS += F^T . R_chunk                (M = s, N = d, K = r)
// Each lane of Y holds one stationary row s and 16 streamed rows r, so per-row
// reductions over r (the BCE dense sum, the CE max/sum) stay in the lane, and F is
// already laid out as the A operand of the dS product (K permuted consistently on
// both operands). The streamed chunk is stored once, row-major; the dS product reads
// it transposed with ds_read_b64_tr_b16.
//
//  rows sweep: S = A (rows t), R = E (items v)  -> per-row loss / LSE partials and dA
//              partials over a vocabulary split (XCD-grouped so the workgroups of one
//              split share E tiles in one L2).
//  cols sweep: S = E (items v), R = A (rows t)  -> dE for the 128 items, minus the sparse
//              positive term, written as bf16 or applied as an SGD step in place.
#include "common.h"

namespace cl {

namespace {

constexpr int kRC = 32;  // streamed rows per chunk

template <int D, bool FP8>
struct ChunkStager {
  static constexpr int NCH = D / 8;                  // 16-byte chunks per LDS row
  static constexpr int PPT = kRC * NCH / 256;        // 16-byte pieces per thread
  static_assert(PPT >= 1, "D too small");
  typedef typename std::conditional<FP8, uint2, uint4>::type raw_t;
  raw_t raw[PPT];

  __device__ __forceinline__ void load(const void* base, int64_t r0, int64_t r_end, int tid) {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int pc = tid + 256 * k;
      const int row = pc / NCH, c = pc % NCH;
      const int64_t gr = r0 + row;
      if (gr < r_end) {
        if constexpr (FP8) raw[k] = *(const uint2*)((const uint8_t*)base + gr * D + c * 8);
        else raw[k] = *(const uint4*)((const uint16_t*)base + gr * D + c * 8);
      } else {
        raw[k] = raw_t{};
      }
    }
  }
  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int k = 0; k < PPT; ++k) {
      const int pc = tid + 256 * k;
      const int row = pc / NCH, c = pc % NCH;
      uint4 v;
      if constexpr (FP8) v = __builtin_bit_cast(uint4, fp8x8_to_bf16x8(raw[k]));
      else v = raw[k];
      *(uint4*)(lds + row * (D * 2) + swz<NCH>(c, row) * 16) = v;
    }
  }
};

// Stationary operand: row `row` of `base`, the 8 K-values d = 16*ks + 8*h .. +7.
template <int D, bool FP8>
__device__ __forceinline__ void load_stationary(bf16x8 (&sf)[D / 16], const void* base, int64_t row, bool ok, int h) {
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    if (!ok) { sf[ks] = bf16x8{}; continue; }
    if constexpr (FP8) {
      uint2 q = *(const uint2*)((const uint8_t*)base + row * D + 16 * ks + 8 * h);
      sf[ks] = fp8x8_to_bf16x8(q);
    } else {
      sf[ks] = *(const bf16x8*)((const uint16_t*)base + row * D + 16 * ks + 8 * h);
    }
  }
}

// Y = R_chunk . S^T for one 32x32 tile.
template <int D>
__device__ __forceinline__ f32x16 tile_logits(const char* L, const bf16x8 (&sf)[D / 16], int l32, int h) {
  constexpr int NCH = D / 8;
  f32x16 y = {};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const bf16x8 ra = *(const bf16x8*)(L + l32 * (D * 2) + swz<NCH>(2 * ks + h, l32) * 16);
    y = mfma32(ra, sf[ks], y);
  }
  return y;
}

// dS[s][d] += sum_r F[s][r] R[r][d] over the 32 rows of the chunk.
template <int D>
__device__ __forceinline__ void tile_grad(f32x16 (&acc)[D / 32], const char* L, bf16x8 fa0, bf16x8 fa1, int lane) {
  constexpr int NCH = D / 8;
  const int h = lane >> 5;
  const int rsub = (lane & 15) >> 2;
  const int colq = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const CL_LDS char* Ls = (const CL_LDS char*)L;
#pragma unroll
  for (int nt = 0; nt < D / 32; ++nt) {
    const int col = 32 * nt + colq;
    const int cc = col >> 3, co = (col & 7) * 2;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int row1 = 16 * kk + 4 * h + rsub;
      const int row2 = row1 + 8;
      const s16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (CL_LDS s16x4*)(Ls + row1 * (D * 2) + swz<NCH>(cc, row1) * 16 + co));
      const s16x4 b2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (CL_LDS s16x4*)(Ls + row2 * (D * 2) + swz<NCH>(cc, row2) * 16 + co));
      acc[nt] = mfma32(kk ? fa1 : fa0, cat_bf16(b1, b2), acc[nt]);
    }
  }
}

__device__ __forceinline__ void pack_f(const float (&F)[16], bf16x8& fa0, bf16x8& fa1) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    fa0[j] = (__bf16)F[j];
    fa1[j] = (__bf16)F[8 + j];
  }
}

// sigmoid(x) and 1 + e^-|x| sharing one exp.
__device__ __forceinline__ void sigmoid_q(float x, float& sig, float& q) {
  const float e = __builtin_amdgcn_exp2f(-__builtin_fabsf(x) * kLog2e);
  q = 1.0f + e;
  const float r = __builtin_amdgcn_rcpf(q);
  sig = x >= 0.0f ? r : e * r;
}

// ------------------------------------------------------------------------------------
// rows sweep
// MODE: 0 BCE loss only, 1 BCE dA, 2 BCE dA + loss, 3 CE max/sum, 4 CE dA
// ------------------------------------------------------------------------------------
template <int D, int MODE, bool RFP8>
__global__ __launch_bounds__(256, 1) void k_sweep_rows(const SweepParams p) {
  constexpr bool WANT_DS = (MODE == 1 || MODE == 2 || MODE == 4);
  constexpr bool BCE_LOSS = (MODE == 0 || MODE == 2);
  constexpr bool CE_LSE = (MODE == 3);
  constexpr int KS = D / 16, NT = D / 32;
  __shared__ __attribute__((aligned(16))) char lds[2][kRC * D * 2];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int nsb = (int)((p.T + 127) / 128);
  const int g = blockIdx.x;
  int split, sb;
  if ((p.n_splits & 7) == 0) {          // workgroup g runs on XCD g % 8: keep a split on one XCD
    const int loc = g >> 3;
    split = (g & 7) + 8 * (loc / nsb);
    sb = loc % nsb;
  } else {
    split = g / nsb;
    sb = g % nsb;
  }
  const int64_t s_wave = (int64_t)sb * 128 + wv * 32;
  const int64_t srow = s_wave + l32;
  const bool s_ok = srow < p.T;
  const int64_t r_begin = (int64_t)split * p.split_len;
  const int64_t r_end = min(p.V, r_begin + p.split_len);
  const int nch = r_end > r_begin ? (int)((r_end - r_begin + kRC - 1) / kRC) : 0;

  bf16x8 sf[KS];
  load_stationary<D, false>(sf, p.A, srow, s_ok, h);
  float lse_s = 0.0f;
  if constexpr (MODE == 4) lse_s = s_ok ? p.lse[srow] * kLog2e : 0.0f;

  f32x16 acc[NT];
  if constexpr (WANT_DS) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x16{};
  }
  float relu = 0.0f, lg = 0.0f;                 // BCE loss state
  float run_m = -__builtin_inff(), run_s = 0.0f;  // CE state

  ChunkStager<D, RFP8> stg;
  if (nch > 0) {
    stg.load(p.E, r_begin, r_end, tid);
    stg.store(lds[0], tid);
  }
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    const int64_t r0 = r_begin + (int64_t)c * kRC;
    if (c + 1 < nch) stg.load(p.E, r0 + kRC, r_end, tid);
    const char* L = lds[c & 1];
    const f32x16 y = tile_logits<D>(L, sf, l32, h);

    float F[16];
    if constexpr (CE_LSE) {
      float xm = -__builtin_inff();
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = 8 * (i >> 2) + 4 * h + (i & 3);
        if (r0 + m < r_end) xm = __builtin_fmaxf(xm, y[i]);
      }
      const float mn = __builtin_fmaxf(run_m, xm);
      if (mn != -__builtin_inff()) {
        float s = run_s * __builtin_amdgcn_exp2f((run_m - mn) * kLog2e);
        const float mb = mn * kLog2e;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int m = 8 * (i >> 2) + 4 * h + (i & 3);
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(y[i], kLog2e, -mb));
          s += (r0 + m < r_end) ? e : 0.0f;
        }
        run_s = s;
        run_m = mn;
      }
    } else {
      float prod = 1.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = 8 * (i >> 2) + 4 * h + (i & 3);
        const bool ok = r0 + m < r_end;
        const float x = y[i];
        if constexpr (MODE == 4) {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -lse_s));
          F[i] = ok ? e : 0.0f;
        } else {
          float sig, q;
          sigmoid_q(x, sig, q);
          F[i] = ok ? sig : 0.0f;
          if constexpr (BCE_LOSS) {
            relu += ok ? __builtin_fmaxf(x, 0.0f) : 0.0f;
            prod *= ok ? q : 1.0f;
          }
        }
      }
      if constexpr (BCE_LOSS) lg += __builtin_amdgcn_logf(prod);  // log2 of a product in [1, 2^16]
    }
    if constexpr (WANT_DS) {
      bf16x8 fa0, fa1;
      pack_f(F, fa0, fa1);
      tile_grad<D>(acc, L, fa0, fa1, lane);
    }
    if (c + 1 < nch) stg.store(lds[(c + 1) & 1], tid);
    __syncthreads();
  }

  // ---- partial outputs of this split
  if constexpr (BCE_LOSS) {
    float v = relu + lg * kLn2;
    v += __shfl_xor(v, 32, 64);
    if (h == 0 && s_ok) p.part_a[(int64_t)split * p.T + srow] = v;
  }
  if constexpr (CE_LSE) {
    const float m2 = __shfl_xor(run_m, 32, 64);
    const float s2 = __shfl_xor(run_s, 32, 64);
    const float mn = __builtin_fmaxf(run_m, m2);
    float s = 0.0f;
    if (mn != -__builtin_inff()) {
      s = run_s * __builtin_amdgcn_exp2f((run_m - mn) * kLog2e) + s2 * __builtin_amdgcn_exp2f((m2 - mn) * kLog2e);
    }
    if (h == 0 && s_ok) {
      p.part_a[(int64_t)split * p.T + srow] = mn;
      p.part_b[(int64_t)split * p.T + srow] = s;
    }
  }
  if constexpr (WANT_DS) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int64_t s = s_wave + 8 * (i >> 2) + 4 * h + (i & 3);
        if (s < p.T) p.part_dA[((int64_t)split * p.T + s) * D + 32 * nt + l32] = acc[nt][i];
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// cols sweep. KIND: 0 BCE, 1 CE. EPI: 0 write dE (bf16), 1 SGD step on E in place.
// ------------------------------------------------------------------------------------
template <int D, int KIND, int EPI, bool SFP8>
__global__ __launch_bounds__(256, 1) void k_sweep_cols(const SweepParams p) {
  constexpr int KS = D / 16, NT = D / 32;
  __shared__ __attribute__((aligned(16))) char lds[2][kRC * D * 2];
  __shared__ __attribute__((aligned(16))) float lw[2][kRC];
  __shared__ __attribute__((aligned(16))) float ll[2][kRC];
  __shared__ int uix[128];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6, h = lane >> 5, l32 = lane & 31;
  const int64_t v_blk = (int64_t)blockIdx.x * 128;
  const int64_t s_wave = v_blk + wv * 32;
  const int64_t srow = s_wave + l32;
  const bool s_ok = srow < p.V;
  const int nch = (int)((p.T + kRC - 1) / kRC);

  bf16x8 sf[KS];
  load_stationary<D, SFP8>(sf, p.E, srow, s_ok, h);
  f32x16 acc[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) acc[nt] = f32x16{};

  ChunkStager<D, false> stg;
  float wreg = 0.0f, lreg = 0.0f;
  auto load_w = [&](int64_t r0) {
    if (tid < kRC) {
      const int64_t r = r0 + tid;
      wreg = r < p.T ? p.w[r] : 0.0f;
      if constexpr (KIND == 1) lreg = r < p.T ? p.lse[r] : 0.0f;
    }
  };
  auto store_w = [&](int b) {
    if (tid < kRC) {
      lw[b][tid] = wreg;
      if constexpr (KIND == 1) ll[b][tid] = lreg * kLog2e;
    }
  };
  if (nch > 0) {
    stg.load(p.A, 0, p.T, tid);
    load_w(0);
    stg.store(lds[0], tid);
    store_w(0);
  }
  __syncthreads();

  for (int c = 0; c < nch; ++c) {
    const int64_t r0 = (int64_t)c * kRC;
    if (c + 1 < nch) {
      stg.load(p.A, r0 + kRC, p.T, tid);
      load_w(r0 + kRC);
    }
    const int b = c & 1;
    const char* L = lds[b];
    const f32x16 y = tile_logits<D>(L, sf, l32, h);
    float F[16];
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const f32x4 w4 = *(const f32x4*)&lw[b][8 * q4 + 4 * h];
      f32x4 l4 = {};
      if constexpr (KIND == 1) l4 = *(const f32x4*)&ll[b][8 * q4 + 4 * h];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = 4 * q4 + j;
        const float x = y[i];
        if constexpr (KIND == 0) {
          float sig, q;
          sigmoid_q(x, sig, q);
          F[i] = w4[j] * sig;
        } else {
          const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(x, kLog2e, -l4[j]));
          F[i] = w4[j] != 0.0f ? w4[j] * e : 0.0f;
        }
      }
    }
    bf16x8 fa0, fa1;
    pack_f(F, fa0, fa1);
    tile_grad<D>(acc, L, fa0, fa1, lane);
    if (c + 1 < nch) {
      stg.store(lds[b ^ 1], tid);
      store_w(b ^ 1);
    }
    __syncthreads();
  }

  // ---- sparse positive term: index of each of the 128 items in the unique-item list
  if (tid < 128) {
    const int64_t v = v_blk + tid;
    const int nu = p.counts[2];
    int lo = 0, hi = nu;  // first index with uitems[idx] >= v
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if ((int64_t)p.uitems[mid] < v) lo = mid + 1;
      else hi = mid;
    }
    uix[tid] = (lo < nu && (int64_t)p.uitems[lo] == v) ? lo : -1;
  }
  __syncthreads();

#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = wv * 32 + 8 * (i >> 2) + 4 * h + (i & 3);
    const int64_t v = v_blk + m;
    if (v >= p.V) continue;
    const int u = uix[m];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int d = 32 * nt + l32;
      float g = acc[nt][i];
      if (u >= 0) g -= p.S_u[(int64_t)u * D + d];
      if constexpr (EPI == 0) {
        ((uint16_t*)p.dE)[v * D + d] = (uint16_t)f32_to_bf16_bits(g);
      } else {
        if constexpr (SFP8) {
          uint8_t* e8 = (uint8_t*)p.E_inplace + v * D + d;
          const float old = fp8_to_f32(*e8);
          *e8 = (uint8_t)f32_to_fp8_sat(old - p.lr * g);
        } else {
          uint16_t* e16 = (uint16_t*)p.E_inplace + v * D + d;
          const float old = bf16_bits_to_f32(*e16);
          *e16 = (uint16_t)f32_to_bf16_bits(old - p.lr * g);
        }
      }
    }
  }
}

// ------------------------------------------------------------------------------------
// host launchers
// ------------------------------------------------------------------------------------
template <int D>
hipError_t rows_d(const SweepParams& p, int mode, hipStream_t st) {
  const int nsb = (int)((p.T + 127) / 128);
  const dim3 grid((unsigned)(nsb * p.n_splits)), block(256);
#define CL_ROWS(M)                                                                        \
  case M:                                                                                 \
    if (p.e_fp8) k_sweep_rows<D, M, true><<<grid, block, 0, st>>>(p);                     \
    else k_sweep_rows<D, M, false><<<grid, block, 0, st>>>(p);                            \
    break;
  switch (mode) {
    CL_ROWS(0) CL_ROWS(1) CL_ROWS(2) CL_ROWS(3) CL_ROWS(4)
    default: return hipErrorInvalidValue;
  }
#undef CL_ROWS
  return hipGetLastError();
}

template <int D>
hipError_t cols_d(const SweepParams& p, int kind, int epi, hipStream_t st) {
  const dim3 grid((unsigned)((p.V + 127) / 128)), block(256);
  const int key = kind * 4 + epi * 2 + (p.e_fp8 ? 1 : 0);
  switch (key) {
    case 0: k_sweep_cols<D, 0, 0, false><<<grid, block, 0, st>>>(p); break;
    case 1: k_sweep_cols<D, 0, 0, true><<<grid, block, 0, st>>>(p); break;
    case 2: k_sweep_cols<D, 0, 1, false><<<grid, block, 0, st>>>(p); break;
    case 3: k_sweep_cols<D, 0, 1, true><<<grid, block, 0, st>>>(p); break;
    case 4: k_sweep_cols<D, 1, 0, false><<<grid, block, 0, st>>>(p); break;
    case 5: k_sweep_cols<D, 1, 0, true><<<grid, block, 0, st>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool sweep_supported(int64_t D) { return D == 64 || D == 128 || D == 256 || D == 512; }

hipError_t launch_sweep_rows(const SweepParams& p, int mode, hipStream_t st) {
  switch (p.D) {
    case 64: return rows_d<64>(p, mode, st);
    case 128: return rows_d<128>(p, mode, st);
    case 256: return rows_d<256>(p, mode, st);
    case 512: return rows_d<512>(p, mode, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_sweep_cols(const SweepParams& p, int kind, int epi, hipStream_t st) {
  switch (p.D) {
    case 64: return cols_d<64>(p, kind, epi, st);
    case 128: return cols_d<128>(p, kind, epi, st);
    case 256: return cols_d<256>(p, kind, epi, st);
    case 512: return cols_d<512>(p, kind, epi, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace cl
