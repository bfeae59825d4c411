// Per-row finalization and the sparse positive terms.
//
// BCE (Cut Binary Cross Entropy, paperpeel, §I-B): loss_t = sum_v softplus(x_tv)
// - sum_{p in P_t} x_tp. The dense sum arrives as partials over vocabulary splits;
// the positive logits x_tp = A_t . E_p are indexed dot products (the "indexed matrix
// multiplication" of the Cut Your Losses article). Gradient rows:
// dA_t = w_t (sum_v sigmoid(x_tv) E_v - sum_{p in P_t} E_p).
// CE (Cut Your Losses article): lse_t merges the per-split running (max, sum) pairs,
// loss_t = lse_t - x_{t,y_t}, dA_t = w_t (sum_v softmax_tv E_v - E_{y_t}).
// The dE sparse term S_v = sum_{t : v in P_t} w_t A_t is a segmented sum over the
// item-major pairs, in row order.
// All reductions run in a fixed order (no float atomics), so results are bitwise
// reproducible.
#include "common.h"

namespace cl {

namespace {

__device__ __forceinline__ float load_e(const void* E, int e_fp8, int64_t idx) {
  return e_fp8 ? fp8_to_f32(((const uint8_t*)E)[idx]) : bf16_bits_to_f32(((const uint16_t*)E)[idx]);
}

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o > 0; o >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ bool row_valid(const FinalizeParams& p, int kind, int64_t t) {
  if (kind == 0) return p.mask == nullptr || p.mask[t] != 0;
  const int64_t y = p.ce_target[t];
  return y != p.ignore_index && y >= 0 && y < p.V;
}

__device__ __forceinline__ float row_weight(const FinalizeParams& p, int kind, int64_t t) {
  if (!row_valid(p, kind, t)) return 0.0f;
  return p.dloss ? p.dloss[t] : 1.0f;
}

constexpr int kMaxDPerLane = 2304 / 64;

// One wave per row.
__global__ __launch_bounds__(256) void k_finalize_rows(const FinalizeParams p, int kind, int want_loss, int want_dA) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  const int64_t D = p.D;
  const int nd = (int)(D / 64);
  const bool valid = row_valid(p, kind, t);
  const uint16_t* A = (const uint16_t*)p.A;

  // positives: x_tp and the sum of E_p
  float corr[kMaxDPerLane];
  for (int k = 0; k < nd; ++k) corr[k] = 0.0f;
  float sum_x = 0.0f;
  const int32_t pb = p.crow[t], pe = p.crow[t + 1];
  for (int32_t e = pb; e < pe; ++e) {
    const int64_t v = p.cids[e];
    float part = 0.0f;
    for (int k = 0; k < nd; ++k) {
      const int64_t d = lane + 64 * k;
      const float ev = load_e(p.E, p.e_fp8, v * D + d);
      part += bf16_bits_to_f32(A[t * D + d]) * ev;
      corr[k] += ev;
    }
    sum_x += wave_sum(part);
  }

  if (want_loss) {
    if (kind == 0) {
      float part = 0.0f;
      for (int j = lane; j < p.n_splits; j += 64) part += p.part_a[(int64_t)j * p.T + t];
      const float dense = wave_sum(part);
      if (lane == 0) p.loss[t] = valid ? dense - sum_x : 0.0f;
    } else {
      float m = -__builtin_inff();
      for (int j = lane; j < p.n_splits; j += 64) m = __builtin_fmaxf(m, p.part_a[(int64_t)j * p.T + t]);
      const float M = wave_max(m);
      float s = 0.0f;
      for (int j = lane; j < p.n_splits; j += 64) {
        const float mj = p.part_a[(int64_t)j * p.T + t];
        if (mj != -__builtin_inff()) s += p.part_b[(int64_t)j * p.T + t] * __expf(mj - M);
      }
      const float S = wave_sum(s);
      const float lse = M + __logf(S);
      if (lane == 0) {
        p.lse[t] = lse;
        p.loss[t] = valid ? lse - sum_x : 0.0f;
      }
    }
  }

  if (want_dA) {
    const float w = row_weight(p, kind, t);
    uint16_t* dA = (uint16_t*)p.dA;
    for (int k = 0; k < nd; ++k) {
      const int64_t d = lane + 64 * k;
      float g = 0.0f;
      if (valid) {
        float acc = 0.0f;
        for (int j = 0; j < p.n_splits; ++j) acc += p.part_dA[((int64_t)j * p.T + t) * D + d];
        g = w * (acc - corr[k]);
      }
      dA[t * D + d] = (uint16_t)f32_to_bf16_bits(g);
    }
  }
}

__global__ void k_row_weights(const FinalizeParams p, int kind) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < p.T) p.w_out[t] = row_weight(p, kind, t);
}

// S_u[d] = sum over the item's pairs (in row order) of w_t A_t[d]
__global__ __launch_bounds__(256) void k_item_sums(int64_t D, const uint16_t* __restrict__ A, const float* __restrict__ w,
                                                   const int32_t* __restrict__ csc_rows, const int32_t* __restrict__ useg,
                                                   const int32_t* __restrict__ counts, float* __restrict__ S_u) {
  const int nu = counts[2];
  for (int u = blockIdx.x; u < nu; u += gridDim.x) {
    const int32_t b = useg[u], e = useg[u + 1];
    for (int64_t d = threadIdx.x; d < D; d += 256) {
      float acc = 0.0f;
      for (int32_t i = b; i < e; ++i) {
        const int64_t t = csc_rows[i];
        acc += w[t] * bf16_bits_to_f32(A[t * D + d]);
      }
      S_u[(int64_t)u * D + d] = acc;
    }
  }
}

}  // namespace

hipError_t launch_finalize_rows(const FinalizeParams& p, int kind, int want_loss, int want_dA, hipStream_t st) {
  if (p.T == 0) return hipSuccess;
  if (p.D / 64 > kMaxDPerLane) return hipErrorInvalidValue;
  k_finalize_rows<<<(unsigned)((p.T + 3) / 4), 256, 0, st>>>(p, kind, want_loss, want_dA);
  return hipGetLastError();
}

hipError_t launch_row_weights(const FinalizeParams& p, int kind, hipStream_t st) {
  if (p.T == 0) return hipSuccess;
  k_row_weights<<<(unsigned)((p.T + 255) / 256), 256, 0, st>>>(p, kind);
  return hipGetLastError();
}

hipError_t launch_item_sums(int64_t D, int64_t nnz_cap, const void* A, const float* w, const int32_t* csc_rows,
                            const int32_t* useg, const int32_t* counts, float* S_u, hipStream_t st) {
  if (nnz_cap <= 0) return hipSuccess;
  const unsigned grid = (unsigned)(nnz_cap < 4096 ? nnz_cap : 4096);
  k_item_sums<<<grid, 256, 0, st>>>(D, (const uint16_t*)A, w, csc_rows, useg, counts, S_u);
  return hipGetLastError();
}

}  // namespace cl
