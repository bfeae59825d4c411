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
#include "launch.h"

namespace cl {

namespace {

__device__ __forceinline__ float load_e(const void* E, int e_fp8, int64_t idx) {
  return e_fp8 ? fp8_to_f32(((const uint8_t*)E)[idx]) : bf16_bits_to_f32(((const uint16_t*)E)[idx]);
}

// four consecutive elements idx .. idx + 3 of E (idx a multiple of 4)
__device__ __forceinline__ f32x4 load_e4(const void* E, int e_fp8, int64_t idx) {
  if (e_fp8) {
    const uint32_t q = *(const uint32_t*)((const uint8_t*)E + idx);
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)q, false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)q, true);
    return f32x4{lo[0], lo[1], hi[0], hi[1]};
  }
  const uint2 q = *(const uint2*)((const uint16_t*)E + idx);
  return f32x4{__uint_as_float(q.x << 16), __uint_as_float(q.x & 0xffff0000u), __uint_as_float(q.y << 16),
               __uint_as_float(q.y & 0xffff0000u)};
}

// A_t[d .. d + 3] (bf16, or the FP8 copy of A when the logits run in FP8)
__device__ __forceinline__ f32x4 load_a4(const FinalizeParams& p, int64_t idx) {
  return p.A8 != nullptr ? load_e4(p.A8, 1, idx) : load_e4(p.A, 0, idx);
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

// This lane's share of the positive logit A_t . E_v: lane owns d = 4 lane + 256 k + 0..3.
__device__ __forceinline__ float pos_dot_part(const FinalizeParams& p, int64_t t, int64_t v, int lane) {
  float part = 0.0f;
  for (int64_t d = 4 * lane; d < p.D; d += 256) {
    const f32x4 a = load_a4(p, t * p.D + d);
    const f32x4 e = load_e4(p.E, p.e_fp8, v * p.D + d);
    part += a[0] * e[0];
    part += a[1] * e[1];
    part += a[2] * e[2];
    part += a[3] * e[3];
  }
  return part;
}

// One wave per row; lanes over d.
__global__ __launch_bounds__(256) void k_finalize_rows(const FinalizeParams p, int kind, int want_loss, int want_dA) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  const int64_t D = p.D;
  const bool valid = row_valid(p, kind, t);
  const int32_t pb = p.crow[t], pe = p.crow[t + 1];

  if (want_loss) {
    // positive logits x_tp = A_t . E_p (indexed dot products), summed in positive order;
    // tp counts the positives with x_tp > 0 (Cut Metrics)
    float sum_x = 0.0f;
    int tp = 0;
    if (p.pos_dot != nullptr) {
      sum_x = p.pos_dot[t];
      if (p.pos_tp != nullptr) tp = p.pos_tp[t];
    } else {
      for (int32_t e = pb; e < pe; ++e) {
        const float x = wave_sum(pos_dot_part(p, t, (int64_t)p.cids[e], lane));
        sum_x += x;
        tp += x > 0.0f ? 1 : 0;
      }
    }
    if (kind == 0) {
      float part = 0.0f;
      for (int j = lane; j < p.n_splits; j += 64) part += p.part_a[(int64_t)j * p.T + t];
      const float dense = wave_sum(part);
      if (lane == 0) p.loss[t] = valid ? dense - sum_x : 0.0f;
      if (p.counts != nullptr) {
        // confusion counts of the predictions x > 0 against the positive set; the dense
        // count sums integer-valued partials (exact in fp32 below 2^24)
        float c = 0.0f;
        for (int j = lane; j < p.n_splits; j += 64) c += p.part_c[(int64_t)j * p.T + t];
        const int64_t npos = (int64_t)(pe - pb);
        const int64_t pos_pred = (int64_t)wave_sum(c);
        if (lane == 0) {
          int32_t* o = p.counts + 4 * t;
          if (!valid) {
            o[0] = o[1] = o[2] = o[3] = 0;
          } else {
            // a positive whose logit sits within rounding of 0 can be decided differently
            // by the dense pass and the indexed dot product: keep FP >= 0
            const int64_t fp = pos_pred > tp ? pos_pred - tp : 0;
            o[0] = tp;
            o[1] = (int32_t)fp;
            o[2] = (int32_t)(npos - tp);
            o[3] = (int32_t)(p.V - npos - fp);
          }
        }
      }
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
    // lane owns 4 consecutive d per 256-wide slab: 16-byte partial loads, 8-byte stores; each
    // element is summed over the splits and the positives in the same order as before
    const float w = row_weight(p, kind, t);
    uint16_t* dA = (uint16_t*)p.dA;
    for (int64_t d = 4 * lane; d < D; d += 256) {
      f32x4 g = {0.0f, 0.0f, 0.0f, 0.0f};
      if (valid) {
        f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int j = 0; j < p.n_splits_dA; ++j) acc += *(const f32x4*)(p.part_dA + ((int64_t)j * p.T + t) * D + d);
        f32x4 corr = {0.0f, 0.0f, 0.0f, 0.0f};   // sum of E_p over the row's positives
        if (p.pos_sum != nullptr) corr = *(const f32x4*)(p.pos_sum + t * D + d);
        else for (int32_t e = pb; e < pe; ++e) corr += load_e4(p.E, p.e_fp8, (int64_t)p.cids[e] * D + d);
        g = p.dA_weighted ? acc - w * corr : w * (acc - corr);
      }
      const uint32_t lo = f32_to_bf16_bits(g[0]) | (f32_to_bf16_bits(g[1]) << 16);
      const uint32_t hi = f32_to_bf16_bits(g[2]) | (f32_to_bf16_bits(g[3]) << 16);
      *(uint2*)(dA + t * D + d) = uint2{lo, hi};
    }
  }
}

// pos_dot[t] = sum_p A_t . E_p and pos_sum[t][d] = sum_p E_p[d], one wave per row, in
// positive order (the same order finalize uses when it reads E directly). For D <= 256 NS
// the row of A stays in registers and the E rows of four positives are loaded together;
// every sum still runs over d slabs and positives in order.
constexpr int kPosBatch = 4;

template <int NS>
__device__ __forceinline__ void row_positives_held(const FinalizeParams& p, int64_t t, int lane) {
  const int64_t D = p.D;
  const int32_t pb = p.crow[t], pe = p.crow[t + 1];
  f32x4 a[NS], corr[NS];
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const int64_t d = 4 * lane + 256 * k;
    a[k] = d < D ? load_a4(p, t * D + d) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    corr[k] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }
  float sum_x = 0.0f;
  int tp = 0;
  for (int32_t e0 = pb; e0 < pe; e0 += kPosBatch) {
    f32x4 ev[kPosBatch][NS];
#pragma unroll
    for (int b = 0; b < kPosBatch; ++b) {
      const int64_t v = p.cids[min(e0 + b, pe - 1)];
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        const int64_t d = 4 * lane + 256 * k;
        ev[b][k] = d < D ? load_e4(p.E, p.e_fp8, v * D + d) : f32x4{0.0f, 0.0f, 0.0f, 0.0f};
      }
    }
#pragma unroll
    for (int b = 0; b < kPosBatch; ++b) {
      if (e0 + b >= pe) break;
      float part = 0.0f;
#pragma unroll
      for (int k = 0; k < NS; ++k) {
        if (4 * lane + 256 * k < D) {
          part += a[k][0] * ev[b][k][0];
          part += a[k][1] * ev[b][k][1];
          part += a[k][2] * ev[b][k][2];
          part += a[k][3] * ev[b][k][3];
          corr[k] += ev[b][k];
        }
      }
      const float x = wave_sum(part);
      if (p.pos_x != nullptr && lane == 0) p.pos_x[e0 + b] = x;
      sum_x += x;
      tp += x > 0.0f ? 1 : 0;
    }
  }
  if (lane == 0) p.pos_dot[t] = sum_x;
  if (lane == 0 && p.pos_tp != nullptr) p.pos_tp[t] = tp;
  if (p.pos_sum == nullptr) return;          // no dA requested
#pragma unroll
  for (int k = 0; k < NS; ++k) {
    const int64_t d = 4 * lane + 256 * k;
    if (d < D) *(f32x4*)(p.pos_sum + t * D + d) = corr[k];
  }
}

__global__ __launch_bounds__(256) void k_row_positives(const FinalizeParams p) {
  const int lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= p.T) return;
  const int64_t D = p.D;
  if (D <= 256) return row_positives_held<1>(p, t, lane);
  if (D <= 512) return row_positives_held<2>(p, t, lane);
  if (D <= 1024) return row_positives_held<4>(p, t, lane);
  const int32_t pb = p.crow[t], pe = p.crow[t + 1];
  float sum_x = 0.0f;
  int tp = 0;
  for (int32_t e = pb; e < pe; ++e) {
    const float x = wave_sum(pos_dot_part(p, t, (int64_t)p.cids[e], lane));
    if (p.pos_x != nullptr && lane == 0) p.pos_x[e] = x;
    sum_x += x;
    tp += x > 0.0f ? 1 : 0;
  }
  if (lane == 0) p.pos_dot[t] = sum_x;
  if (lane == 0 && p.pos_tp != nullptr) p.pos_tp[t] = tp;
  if (p.pos_sum == nullptr) return;          // no dA requested
  for (int64_t d = 4 * lane; d < D; d += 256) {
    f32x4 corr = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int32_t e = pb; e < pe; ++e) corr += load_e4(p.E, p.e_fp8, (int64_t)p.cids[e] * D + d);
    *(f32x4*)(p.pos_sum + t * D + d) = corr;
  }
}

__global__ __launch_bounds__(256) void k_scale_rows(const uint16_t* __restrict__ A, const float* __restrict__ w,
                                                    int64_t n4, int64_t D, uint16_t* __restrict__ Aw) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // 4 elements (one row: D % 4 == 0)
  if (i >= n4) return;
  const float wt = w[(4 * i) / D];
  const f32x4 a = load_e4(A, 0, 4 * i);
  const uint32_t lo = f32_to_bf16_bits(wt * a[0]) | (f32_to_bf16_bits(wt * a[1]) << 16);
  const uint32_t hi = f32_to_bf16_bits(wt * a[2]) | (f32_to_bf16_bits(wt * a[3]) << 16);
  *(uint2*)(Aw + 4 * i) = uint2{lo, hi};
}

__global__ void k_row_weights(const FinalizeParams p, int kind) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t < p.T) p.w_out[t] = row_weight(p, kind, t);
}

// Sparse dE term S_u = sum over the item's pairs (in row order) of w_t A_t, as a
// segmented sum over the item-major pairs. Pairs are cut into fixed pieces of kPiece;
// one wave sums each piece, lanes over d. An item lying inside one piece is finished
// there; an item crossing piece boundaries leaves its run at the end of its first
// piece in part[j][1], its runs covering or starting later pieces in part[j][0], and
// k_item_fixup adds them in piece order. Every sum runs in a fixed order.
constexpr int kPiece = 16;
constexpr int kPieceBatch = 8;     // pairs whose rows of A are loaded together
constexpr int kPieceSlabs = 4;     // 256-wide d slabs per pass over the piece (D <= 1024: one)

__device__ __forceinline__ int lane_i32(int32_t v, int i) { return __builtin_amdgcn_readlane(v, i); }
__device__ __forceinline__ float lane_f32(float v, int i) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), i));
}

// index of the unique item that holds pair i: the last u < nu with useg[u] <= i (useg
// ascending, useg[0] = 0 <= i < useg[nu]), narrowed 64 ways a step by the wave's lanes
__device__ __forceinline__ int item_of_wave(const int32_t* useg, int nu, int32_t i, int lane) {
  int lo = 0, hi = nu;
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int idx = lo + lane * step;
    const unsigned long long m = __ballot(idx < hi && useg[idx] <= i);   // a prefix of lanes, lane 0 set
    const int L = 63 - __clzll(m);
    const int nlo = lo + L * step;
    hi = min(hi, nlo + step);
    lo = nlo;
  }
  return lo;
}

// The piece's pairs sit one a lane (row t and weight w_t of pair a + i in lane i) and the
// ends of its items likewise, so that the rows of A of kPieceBatch pairs are requested
// together; the sum of each item still runs over its pairs in order.
__global__ __launch_bounds__(256) void k_item_pieces(int64_t D, const uint16_t* __restrict__ A, const float* __restrict__ w,
                                                     const int32_t* __restrict__ csc_rows, const int32_t* __restrict__ useg,
                                                     const int32_t* __restrict__ counts, float* __restrict__ S_u,
                                                     float* __restrict__ part) {
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int32_t n = counts[1], nu = counts[2];
  const int64_t a = j * kPiece;
  if (a >= n) return;
  const int64_t b = min(a + kPiece, (int64_t)n);
  const int u0 = item_of_wave(useg, nu, (int32_t)a, lane);   // pairs are item-major: later items follow in order
  int32_t tr = 0, ue = n;
  float wr = 0.0f;
  if (lane < kPiece) {
    if (a + lane < b) tr = csc_rows[a + lane];
    ue = useg[min(u0 + lane + 1, nu)];                       // end of item u0 + lane (useg[nu] = n)
  }
  if (lane < kPiece && a + lane < b) wr = w[tr];
  const int32_t us0 = useg[u0];
  const int ns = (int)((D + 255) / 256);                     // 256-wide d slabs; lane owns 4 d of each
  for (int k0 = 0; k0 < ns; k0 += kPieceSlabs) {
    f32x4 acc[kPieceSlabs];
#pragma unroll
    for (int kk = 0; kk < kPieceSlabs; ++kk) acc[kk] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    int k = 0;                                               // current item: u0 + k, pairs [s_k, e_k)
    int64_t s_k = us0, e_k = lane_i32(ue, 0);
    for (int64_t q0 = a; q0 < b; q0 += kPieceBatch) {
      uint2 raw[kPieceBatch][kPieceSlabs];
#pragma unroll
      for (int bq = 0; bq < kPieceBatch; ++bq) {
        const int i = (int)(q0 - a) + bq;
        const int64_t t = lane_i32(tr, min(i, kPiece - 1));
#pragma unroll
        for (int kk = 0; kk < kPieceSlabs; ++kk) {
          const int64_t d = 4 * lane + 256 * (k0 + kk);
          raw[bq][kk] = (q0 + bq < b && d < D) ? *(const uint2*)(A + t * D + d) : uint2{0u, 0u};
        }
      }
#pragma unroll
      for (int bq = 0; bq < kPieceBatch; ++bq) {
        const int64_t q = q0 + bq;
        if (q >= b) break;
        const float wt = lane_f32(wr, (int)(q - a));
#pragma unroll
        for (int kk = 0; kk < kPieceSlabs; ++kk) {
          const uint2 r = raw[bq][kk];
          const f32x4 x = {__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u), __uint_as_float(r.y << 16),
                           __uint_as_float(r.y & 0xffff0000u)};
          acc[kk] += wt * x;
        }
        if (q + 1 == e_k || q + 1 == b) {                    // the item's last pair in this piece
          float* dst;
          if (s_k >= a && e_k <= b) dst = S_u + (int64_t)(u0 + k) * D;   // complete inside this piece
          else if (s_k < a) dst = part + (j * 2 + 0) * D;                // began in an earlier piece
          else dst = part + (j * 2 + 1) * D;                             // continues into later pieces
#pragma unroll
          for (int kk = 0; kk < kPieceSlabs; ++kk) {
            const int64_t d = 4 * lane + 256 * (k0 + kk);
            if (d < D) *(f32x4*)(dst + d) = acc[kk];
            acc[kk] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
          }
          ++k;
          s_k = e_k;
          e_k = lane_i32(ue, min(k, kPiece - 1));
        }
      }
    }
  }
}

// One block per piece: if an item starts in piece j and continues past it, finish it.
__global__ __launch_bounds__(256) void k_item_fixup(int64_t D, const int32_t* __restrict__ useg,
                                                    const int32_t* __restrict__ counts, float* __restrict__ S_u,
                                                    const float* __restrict__ part) {
  const int64_t j = blockIdx.x;
  const int32_t n = counts[1], nu = counts[2];
  const int64_t a = j * kPiece;
  if (a >= n) return;
  const int64_t b = min(a + kPiece, (int64_t)n);
  const int u = item_of_wave(useg, nu, (int32_t)(b - 1), threadIdx.x & 63);
  const int64_t s = useg[u], e = useg[u + 1];
  if (!(e > b && s >= a)) return;
  const int64_t j1 = (e - 1) / kPiece;
  // 4 consecutive d per thread; the pieces j + 1 .. j1 go round-robin to four partial sums
  // (long chains: a popular item spans many pieces), combined in a fixed order
  for (int64_t d = 4 * (int64_t)threadIdx.x; d < D; d += 1024) {
    f32x4 a0 = *(const f32x4*)(part + (j * 2 + 1) * D + d);
    f32x4 a1 = {0.0f, 0.0f, 0.0f, 0.0f}, a2 = a1, a3 = a1;
    int64_t jj = j + 1;
    for (; jj + 3 <= j1; jj += 4) {
      a0 += *(const f32x4*)(part + (jj * 2 + 0) * D + d);
      a1 += *(const f32x4*)(part + ((jj + 1) * 2 + 0) * D + d);
      a2 += *(const f32x4*)(part + ((jj + 2) * 2 + 0) * D + d);
      a3 += *(const f32x4*)(part + ((jj + 3) * 2 + 0) * D + d);
    }
    for (; jj <= j1; ++jj) a0 += *(const f32x4*)(part + (jj * 2 + 0) * D + d);
    *(f32x4*)(S_u + (int64_t)u * D + d) = (a0 + a1) + (a2 + a3);
  }
}

// Fixed-order reduction of split partials [S][N] (row-major by split), one thread per
// column n: group g sums splits [64 g, 64 g + 64) in split order. mode 0: plain sums;
// mode 1: logsumexp pairs (a = running max, b = sum of exp(x - max)), merged to the
// group max. Reading and writing the same buffer is allowed: each thread reads all of
// its column before it writes it.
constexpr int kRedGroup = 64;

// All of a thread's loads are issued before its sums (indices clamped into the group), so
// that a level costs one round trip to memory; the sums skip the clamped copies and keep
// the split order.
__global__ __launch_bounds__(256) void k_reduce_splits(const float* pa, const float* pb, int64_t S, int64_t N, float* oa,
                                                       float* ob, int mode) {
  const int64_t n = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t g = blockIdx.y;
  if (n >= N) return;
  const int64_t s0 = g * kRedGroup;
  const int cnt = (int)(min(S, s0 + kRedGroup) - s0);
  const float* ca = pa + s0 * N + n;
  float va[kRedGroup];
#pragma unroll
  for (int i = 0; i < kRedGroup; ++i) va[i] = ca[(int64_t)min(i, cnt - 1) * N];
  if (mode == 0) {
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < kRedGroup; ++i)
      if (i < cnt) acc += va[i];
    oa[g * N + n] = acc;
  } else {
    const float* cb = pb + s0 * N + n;
    float vb[kRedGroup];
#pragma unroll
    for (int i = 0; i < kRedGroup; ++i) vb[i] = cb[(int64_t)min(i, cnt - 1) * N];
    float m = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < kRedGroup; ++i)
      if (i < cnt) m = __builtin_fmaxf(m, va[i]);
    float sum = 0.0f;
    if (m != -__builtin_inff()) {
#pragma unroll
      for (int i = 0; i < kRedGroup; ++i)
        if (i < cnt && va[i] != -__builtin_inff()) sum += vb[i] * __builtin_amdgcn_exp2f((va[i] - m) * kLog2e);
    }
    oa[g * N + n] = m;
    ob[g * N + n] = sum;
  }
}

int64_t red_groups(int64_t S) { return (S + kRedGroup - 1) / kRedGroup; }

}  // namespace

size_t reduce_splits_tmp_floats(int64_t S, int64_t N, int mode) {
  size_t f = 0;
  for (int64_t s = S; s > kRedGroup; s = red_groups(s)) f += (size_t)red_groups(s) * (size_t)N;
  return mode ? 2 * f : f;
}

hipError_t launch_reduce_splits(float* pa, float* pb, int64_t S, int64_t N, float* tmp, int mode, hipStream_t st) {
  if (S <= 1 || N <= 0) return hipSuccess;
  const unsigned bx = (unsigned)((N + 255) / 256);
  const float* ca = pa;
  const float* cb = pb;
  int64_t cs = S;
  while (cs > kRedGroup) {
    const int64_t g = red_groups(cs);
    float* ta = tmp;
    float* tb = mode ? tmp + g * N : nullptr;
    k_reduce_splits<<<dim3(bx, (unsigned)g), 256, 0, st>>>(ca, cb, cs, N, ta, tb, mode);
    tmp += (mode ? 2 : 1) * g * N;
    ca = ta;
    cb = tb;
    cs = g;
  }
  k_reduce_splits<<<dim3(bx, 1), 256, 0, st>>>(ca, cb, cs, N, pa, pb, mode);
  return hipGetLastError();
}

hipError_t launch_finalize_rows(const FinalizeParams& p, int kind, int want_loss, int want_dA, hipStream_t st) {
  if (p.T == 0) return hipSuccess;
  k_finalize_rows<<<(unsigned)((p.T + 3) / 4), 256, 0, st>>>(p, kind, want_loss, want_dA);
  return hipGetLastError();
}

hipError_t launch_row_positives(const FinalizeParams& p, hipStream_t st) {
  if (p.T == 0) return hipSuccess;
  k_row_positives<<<(unsigned)((p.T + 3) / 4), 256, 0, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_scale_rows(const void* A, const float* w, int64_t T, int64_t D, uint16_t* Aw, hipStream_t st) {
  const int64_t n4 = T * D / 4;
  if (n4 == 0) return hipSuccess;
  k_scale_rows<<<(unsigned)((n4 + 255) / 256), 256, 0, st>>>((const uint16_t*)A, w, n4, D, Aw);
  return hipGetLastError();
}

hipError_t launch_row_weights(const FinalizeParams& p, int kind, hipStream_t st) {
  if (p.T == 0) return hipSuccess;
  k_row_weights<<<(unsigned)((p.T + 255) / 256), 256, 0, st>>>(p, kind);
  return hipGetLastError();
}

size_t item_sum_parts(int64_t nnz_cap) { return (size_t)((nnz_cap + kPiece - 1) / kPiece); }

hipError_t launch_item_sums(int64_t D, int64_t nnz_cap, const void* A, const float* w, const int32_t* csc_rows,
                            const int32_t* useg, const int32_t* counts, float* S_u, float* part, hipStream_t st) {
  if (nnz_cap <= 0) return hipSuccess;
  const int64_t np = (int64_t)item_sum_parts(nnz_cap);
  k_item_pieces<<<(unsigned)((np + 3) / 4), 256, 0, st>>>(D, (const uint16_t*)A, w, csc_rows, useg, counts, S_u, part);
  k_item_fixup<<<(unsigned)np, 256, 0, st>>>(D, useg, counts, S_u, part);
  return hipGetLastError();
}

}  // namespace cl
