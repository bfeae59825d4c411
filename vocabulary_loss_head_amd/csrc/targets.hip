// Canonical positive sets on the device.
//
// Cut Binary Cross Entropy (paperpeel) keeps only the sparse target IDs of each row
// (§III-B), pads target lists and trains non-padding positions (§III-E), and tests
// padded and duplicate IDs (§IV-A). The label y_tv is 1 exactly when v is in row t's
// list, is not the padding ID and row t is valid; repeats count once. IDs outside
// [0, V) are counted as data errors and ignored. For softmax CE the single target of
// each non-ignored row is the one positive.
//
// Pipeline (every step deterministic, any row length):
//   1. count valid entries per row, scan, compact (item, row) pairs in row order;
//   2. stable LSD radix sort by item (8-bit digits) -> item-major order with
//      repeats adjacent; keep the first of each (item, row) run -> CSC pairs;
//   3. unique item list and its segment starts (for the dE sparse term);
//   4. stable radix sort of the unique pairs by row -> canonical CSR (items
//      ascending within a row).
#include <algorithm>
#include "launch.h"

namespace cl {

constexpr int RS_TILE = 1024;
constexpr int kRsOwnOffsetsMaxBlocks = 128;

size_t targets_radix_blocks(int64_t nnz) { return nnz <= 0 ? 1 : (size_t)((nnz + RS_TILE - 1) / RS_TILE); }

__global__ void k_zero_u64(unsigned long long* p, int n) {
  int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0ull;
}

hipError_t launch_zero_u64(unsigned long long* p, int n, hipStream_t st) {
  k_zero_u64<<<(n + 255) / 256, 256, 0, st>>>(p, n);
  return hipGetLastError();
}

// ---- step 1 -------------------------------------------------------------------------
__global__ void k_row_count(int64_t T, int64_t V, int64_t nnz, const int32_t* __restrict__ row_ptr,
                            const int32_t* __restrict__ ids, const uint8_t* __restrict__ mask, int32_t pad,
                            int32_t* __restrict__ cnt, unsigned long long* err) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  int64_t b = row_ptr[t], e = row_ptr[t + 1];
  if (b < 0 || e > nnz || e < b) {            // malformed row: a data error, no positives
    atomicAdd(err, 1ull);
    cnt[t] = 0;
    return;
  }
  if (mask != nullptr && mask[t] == 0) { cnt[t] = 0; return; }
  int c = 0;
  unsigned long long bad = 0;
  for (int64_t i = b; i < e; ++i) {
    int32_t v = ids[i];
    if (pad >= 0 && v == pad) continue;
    if (v < 0 || (int64_t)v >= V) { ++bad; continue; }
    ++c;
  }
  if (bad) atomicAdd(err, bad);
  cnt[t] = c;
}

__global__ void k_row_count_ce(int64_t T, int64_t V, const int64_t* __restrict__ target, int64_t ignore,
                               int32_t* __restrict__ cnt, unsigned long long* err) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  int64_t y = target[t];
  int c = 0;
  if (y != ignore) {
    if (y >= 0 && y < V) c = 1;
    else atomicAdd(err, 1ull);
  }
  cnt[t] = c;
}

__global__ void k_row_compact(int64_t T, int64_t V, int64_t nnz, const int32_t* __restrict__ row_ptr,
                              const int32_t* __restrict__ ids, const int32_t* __restrict__ cnt,
                              const int32_t* __restrict__ off, int32_t pad,
                              int32_t* __restrict__ key, int32_t* __restrict__ val) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  if (cnt[t] == 0) return;                    // masked, malformed or no valid entries
  int64_t b = row_ptr[t], e = row_ptr[t + 1];
  int64_t o = off[t];
  for (int64_t i = b; i < e; ++i) {
    int32_t v = ids[i];
    if (pad >= 0 && v == pad) continue;
    if (v < 0 || (int64_t)v >= V) continue;
    if (o >= nnz) break;                      // overlapping rows of a non-monotone row_ptr
    key[o] = v;
    val[o] = (int32_t)t;
    ++o;
  }
}

// Overlapping rows (a non-monotone row_ptr) can count more valid entries than nnz: the
// excess is a data error and the pair count is clamped to the array capacity.
__global__ void k_clamp_count(int32_t* counts, int64_t cap, unsigned long long* err) {
  if (threadIdx.x == 0 && blockIdx.x == 0 && (int64_t)counts[0] > cap) {
    atomicAdd(err, (unsigned long long)((int64_t)counts[0] - cap));
    counts[0] = (int32_t)cap;
  }
}

__global__ void k_row_compact_ce(int64_t T, const int64_t* __restrict__ target, const int32_t* __restrict__ cnt,
                                 const int32_t* __restrict__ off, int32_t* __restrict__ key, int32_t* __restrict__ val) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= T) return;
  if (cnt[t] == 0) return;
  key[off[t]] = (int32_t)target[t];
  val[off[t]] = (int32_t)t;
}

// Single-workgroup exclusive scan: out[i] = sum in[0..i), out[n] = total.
// If n_dev != NULL the length is min(n, *n_dev) and entries past it read as 0.
// Tiles of 16384 entries, 16 consecutive ones per thread (four 16-byte loads and stores
// where the buffers allow): each thread sums its entries, each wave scans its 64 thread
// sums with shuffles, the 16 wave totals meet in LDS, and a running carry links the tiles
// (two barriers per tile). The next tile is loaded while the current one is scanned, so
// a tile costs about one memory latency. Integer sums, so the result does not depend on
// the order.
constexpr int kScanPer = 16;
constexpr int64_t kScanTile = 1024 * kScanPer;

__device__ __forceinline__ void scan_load(const int32_t* __restrict__ in, int64_t i0, int64_t m, bool vec,
                                          int (&v)[kScanPer]) {
  if (vec && i0 + kScanPer <= m) {
    const int4* p = (const int4*)(in + i0);
#pragma unroll
    for (int q = 0; q < kScanPer / 4; ++q) {
      const int4 x = p[q];
      v[4 * q] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) v[j] = (i0 + j < m) ? in[i0 + j] : 0;
  }
}

__global__ __launch_bounds__(1024) void k_scan(const int32_t* __restrict__ in, int64_t n, const int32_t* n_dev,
                                               int32_t* __restrict__ out, int32_t* total_out) {
  __shared__ int32_t wsum[16];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int64_t m = n;
  if (n_dev != nullptr) m = min((int64_t)*n_dev, n);
  // 16-byte accesses need 16-byte aligned buffers (entry offsets are multiples of 16)
  const bool vin = ((uintptr_t)in & 15) == 0, vout = ((uintptr_t)out & 15) == 0;
  int32_t carry = 0;                      // the same value in every thread
  int vn[kScanPer];
  scan_load(in, (int64_t)tid * kScanPer, m, vin, vn);
  for (int64_t base = 0; base < n; base += kScanTile) {
    const int64_t i0 = base + (int64_t)tid * kScanPer;
    int v[kScanPer];
    int local = 0;
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      v[j] = vn[j];
      local += v[j];
    }
    if (base + kScanTile < n) scan_load(in, i0 + kScanTile, m, vin, vn);
    int x = local;                        // inclusive scan over the wave
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(x, o, 64);
      if (lane >= o) x += y;
    }
    if (lane == 63) wsum[wv] = x;
    __syncthreads();
    int wpre = 0, tot = 0;
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const int t = wsum[k];
      wpre += k < wv ? t : 0;
      tot += t;
    }
    int run = carry + wpre + x - local;
    int r[kScanPer];
#pragma unroll
    for (int j = 0; j < kScanPer; ++j) {
      r[j] = run;
      run += v[j];
    }
    if (vout && i0 + kScanPer <= n) {
      int4* q = (int4*)(out + i0);
#pragma unroll
      for (int k = 0; k < kScanPer / 4; ++k) q[k] = make_int4(r[4 * k], r[4 * k + 1], r[4 * k + 2], r[4 * k + 3]);
    } else {
#pragma unroll
      for (int j = 0; j < kScanPer; ++j)
        if (i0 + j < n) out[i0 + j] = r[j];
    }
    carry += tot;
    __syncthreads();                      // wsum is rewritten by the next tile
  }
  if (tid == 0) {
    out[n] = carry;
    if (total_out != nullptr) *total_out = carry;
  }
}

// ---- radix sort (stable, 8-bit digits) ------------------------------------------------
__global__ __launch_bounds__(256) void k_rs_hist(const int32_t* __restrict__ kin, const int32_t* n_dev, int shift,
                                                 int32_t* __restrict__ hist, int nblk) {
  __shared__ int32_t h[256];
  const int tid = threadIdx.x;
  h[tid] = 0;
  __syncthreads();
  const int64_t n = *n_dev;
  const int64_t b = blockIdx.x;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int64_t i = b * RS_TILE + j * 256 + tid;
    if (i < n) atomicAdd(&h[((uint32_t)kin[i] >> shift) & 255u], 1);
  }
  __syncthreads();
  hist[(int64_t)tid * nblk + b] = h[tid];
}

// First output slot of block b's keys with digit tid: the exclusive prefix of the block
// histograms taken in digit-major order (every block's count of smaller digits, then the
// count of digit tid in blocks before b). Each thread reads one digit's nblk counts; tmp is
// 256 ints of LDS.
__device__ __forceinline__ int32_t rs_block_offset(const int32_t* __restrict__ hist, int nblk, int64_t b, int tid,
                                                   int32_t* tmp) {
  const int32_t* row = hist + (int64_t)tid * nblk;
  int32_t tot = 0, pre = 0;
#pragma unroll 8
  for (int k = 0; k < nblk; ++k) {
    const int32_t c = row[k];
    tot += c;
    pre += k < b ? c : 0;
  }
  tmp[tid] = tot;
  __syncthreads();
  for (int o = 1; o < 256; o <<= 1) {          // inclusive scan of the digit totals
    const int32_t add = tid >= o ? tmp[tid - o] : 0;
    __syncthreads();
    tmp[tid] += add;
    __syncthreads();
  }
  return tmp[tid] - tot + pre;
}

// hscan: the scanned histograms, or null to derive block b's offsets from hist itself
__global__ __launch_bounds__(256) void k_rs_scatter(const int32_t* __restrict__ kin, const int32_t* __restrict__ vin,
                                                    int32_t* __restrict__ kout, int32_t* __restrict__ vout,
                                                    const int32_t* n_dev, int shift,
                                                    const int32_t* __restrict__ hscan,
                                                    const int32_t* __restrict__ hist, int nblk) {
  __shared__ int32_t run[256];
  __shared__ int32_t wcnt[4][256];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int64_t b = blockIdx.x;
  const int64_t n = *n_dev;
  if (hscan != nullptr) {
    run[tid] = hscan[(int64_t)tid * nblk + b];
  } else {
    const int32_t o = rs_block_offset(hist, nblk, b, tid, run);
    run[tid] = o;                                 // own slot, after the scan's last barrier
  }
  for (int j = 0; j < 4; ++j) {
#pragma unroll
    for (int k = 0; k < 4; ++k) wcnt[k][tid] = 0;
    __syncthreads();
    const int64_t i = b * RS_TILE + j * 256 + tid;
    const bool act = i < n;
    const int32_t key = act ? kin[i] : 0;
    const int32_t val = act ? vin[i] : 0;
    const uint32_t d = ((uint32_t)key >> shift) & 255u;
    unsigned long long peers = __ballot(act);
#pragma unroll
    for (int bit = 0; bit < 8; ++bit) {
      const bool on = (d >> bit) & 1u;
      const unsigned long long bb = __ballot(on);
      peers &= on ? bb : ~bb;
    }
    const int rank = __popcll(peers & ((1ull << lane) - 1ull));
    if (act && rank == 0) wcnt[w][d] = __popcll(peers);
    __syncthreads();
    if (act) {
      int pre = 0;
      for (int k = 0; k < w; ++k) pre += wcnt[k][d];
      const int pos = run[d] + pre + rank;
      kout[pos] = key;
      vout[pos] = val;
    }
    __syncthreads();
    run[tid] += wcnt[0][tid] + wcnt[1][tid] + wcnt[2][tid] + wcnt[3][tid];
    __syncthreads();
  }
}

// ---- dedupe / unique items / row pointers ------------------------------------------------
__global__ void k_flag_pairs(const int32_t* __restrict__ key, const int32_t* __restrict__ val, const int32_t* n_dev,
                             int64_t cap, int32_t* __restrict__ flags) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= cap) return;
  const int64_t n = *n_dev;
  int f = 0;
  if (i < n) f = (i == 0 || key[i] != key[i - 1] || val[i] != val[i - 1]) ? 1 : 0;
  flags[i] = f;
}

__global__ void k_compact_pairs(const int32_t* __restrict__ key, const int32_t* __restrict__ val,
                                const int32_t* __restrict__ flags, const int32_t* __restrict__ fscan,
                                const int32_t* n_dev, int64_t cap,
                                int32_t* __restrict__ items, int32_t* __restrict__ rows) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= cap || i >= *n_dev) return;
  if (flags[i]) {
    items[fscan[i]] = key[i];
    rows[fscan[i]] = val[i];
  }
}

__global__ void k_flag_items(const int32_t* __restrict__ items, const int32_t* n_dev, int64_t cap,
                             int32_t* __restrict__ flags) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= cap) return;
  const int64_t n = *n_dev;
  flags[i] = (i < n && (i == 0 || items[i] != items[i - 1])) ? 1 : 0;
}

__global__ void k_compact_items(const int32_t* __restrict__ items, const int32_t* __restrict__ flags,
                                const int32_t* __restrict__ fscan, const int32_t* n_dev, const int32_t* nu_dev,
                                int64_t cap, int32_t* __restrict__ uitems, int32_t* __restrict__ useg) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = *n_dev;
  if (i == 0) useg[*nu_dev] = (int32_t)n;
  if (i >= cap || i >= n) return;
  if (flags[i]) {
    uitems[fscan[i]] = items[i];
    useg[fscan[i]] = (int32_t)i;
  }
}

__global__ void k_copy2(const int32_t* __restrict__ a, const int32_t* __restrict__ b, const int32_t* n_dev,
                        int64_t cap, int32_t* __restrict__ a2, int32_t* __restrict__ b2) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= cap || i >= *n_dev) return;
  a2[i] = a[i];
  b2[i] = b[i];
}

__global__ void k_row_ptr(const int32_t* __restrict__ rows_sorted, const int32_t* n_dev, int64_t cap, int64_t T,
                          int32_t* __restrict__ crow) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t n = *n_dev;
  if (i > cap || i > n) return;
  const int64_t r_prev = (i == 0) ? -1 : rows_sorted[i - 1];
  const int64_t r_cur = (i == n) ? T : rows_sorted[i];
  for (int64_t r = r_prev + 1; r <= r_cur; ++r) crow[r] = (int32_t)i;
}

static int bits_for(int64_t n) {  // bits needed for values in [0, n)
  int b = 0;
  while (b < 62 && ((int64_t)1 << b) < n) ++b;
  return b;
}

static inline unsigned grid_for(int64_t n, int bs) { return (unsigned)((n + bs - 1) / bs > 0 ? (n + bs - 1) / bs : 1); }

// Radix-sort (key, val) pairs held in (kA, vA) by key bits [0, nbits); returns true if the
// result ended in (kB, vB).
static bool radix_sort(const TargetsWs& w, int32_t* kA, int32_t* vA, int32_t* kB, int32_t* vB,
                       const int32_t* n_dev, int64_t cap, int nbits, hipStream_t st) {
  const int nblk = (int)targets_radix_blocks(cap);
  bool inB = false;
  for (int shift = 0; shift < nbits; shift += 8) {
    const int32_t* ki = inB ? kB : kA;
    const int32_t* vi = inB ? vB : vA;
    int32_t* ko = inB ? kA : kB;
    int32_t* vo = inB ? vA : vB;
    k_rs_hist<<<nblk, 256, 0, st>>>(ki, n_dev, shift, w.hist, nblk);
    // up to 128 blocks each scatter block reads the whole histogram table (128 KB) and forms
    // its own offsets; larger sorts scan the table once in a kernel of its own
    const bool own = nblk <= kRsOwnOffsetsMaxBlocks;
    if (!own) k_scan<<<1, 1024, 0, st>>>(w.hist, (int64_t)256 * nblk, nullptr, w.hscan, nullptr);
    k_rs_scatter<<<nblk, 256, 0, st>>>(ki, vi, ko, vo, n_dev, shift, own ? nullptr : w.hscan, w.hist, nblk);
    inB = !inB;
  }
  return inB;
}

// ---- small problems: the whole pipeline in one workgroup ---------------------------------
// Up to kSmallPairs IDs and kSmallRows rows, the same steps run in LDS in one launch instead
// of about twenty: the (item, row) pairs are sorted as 64-bit keys by a bitonic network
// (equal keys are repeats of one pair, so the order matches the stable radix sorts), then
// the unique pairs as (row, item) keys. Every output equals the multi-kernel pipeline's.
constexpr int kSmallPairs = 4096;
constexpr int kSmallRows = 8192;
constexpr int kSmallThreads = 1024;

// exclusive scan of s[0 .. n) in place, s[n] = total (n <= 8 * kSmallThreads); returns the total
__device__ int small_scan(int* s, int n, int* wsum) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  constexpr int PER = 8;
  int v[PER];
  int sum = 0;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid * PER + k;
    v[k] = i < n ? s[i] : 0;
    sum += v[k];
  }
  int x = sum;                                  // inclusive scan over the wave's threads
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) wsum[wv] = x;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int k = 0; k < kSmallThreads / 64; ++k) {
      const int c = wsum[k];
      wsum[k] = run;
      run += c;
    }
    wsum[kSmallThreads / 64] = run;
  }
  __syncthreads();
  int base = wsum[wv] + x - sum;
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = tid * PER + k;
    if (i < n) s[i] = base;
    base += v[k];
  }
  const int total = wsum[kSmallThreads / 64];
  if (tid == 0) s[n] = total;
  __syncthreads();
  return total;
}

// ascending bitonic sort of a[0 .. N), N a power of two (entries past the data hold ~0)
__device__ void small_sort(unsigned long long* a, int N) {
  for (int k = 2; k <= N; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < N; i += kSmallThreads) {
        const int l = i ^ j;
        if (l > i) {
          const unsigned long long x = a[i], y = a[l];
          if ((x > y) == ((i & k) == 0)) {
            a[i] = y;
            a[l] = x;
          }
        }
      }
      __syncthreads();
    }
}

__device__ __forceinline__ unsigned long long shfl_xor_u64(unsigned long long v, int m) {
  const int lo = __shfl_xor((int)(uint32_t)v, m, 64), hi = __shfl_xor((int)(uint32_t)(v >> 32), m, 64);
  return ((unsigned long long)(uint32_t)hi << 32) | (uint32_t)lo;
}

// the same network for N <= kSmallThreads with one key per thread: exchanges between
// lanes of one wave go through shuffles, wider ones through LDS, so only the steps with
// partners 64 or more apart take barriers (10 of the 55 at N = 1024)
__device__ void small_sort_lanes(unsigned long long* a, int N) {
  const int i = threadIdx.x;
  unsigned long long x = i < N ? a[i] : ~0ull;
  for (int k = 2; k <= N; k <<= 1)
    for (int j = k >> 1; j > 0; j >>= 1) {
      unsigned long long y;
      if (j >= 64) {
        if (i < N) a[i] = x;
        __syncthreads();
        y = i < N ? a[i ^ j] : ~0ull;
        __syncthreads();
      } else {
        y = shfl_xor_u64(x, j);
      }
      // the lower index of a pair keeps the minimum in an ascending block, the maximum in
      // a descending one; the upper index the other
      const bool keep_min = ((i & j) == 0) == ((i & k) == 0);
      x = keep_min ? (x < y ? x : y) : (x < y ? y : x);
    }
  if (i < N) a[i] = x;
  __syncthreads();
}

__device__ __forceinline__ int small_pow2(int n) {
  int N = 2;
  while (N < n) N <<= 1;
  return N;
}

__global__ __launch_bounds__(kSmallThreads) void k_targets_small(int64_t T, int64_t V, int64_t nnz,
                                                                 const int32_t* __restrict__ row_ptr,
                                                                 const int32_t* __restrict__ ids,
                                                                 const uint8_t* __restrict__ mask, int32_t pad,
                                                                 const TargetsWs w) {
  __shared__ int s_off[kSmallRows + 1];                 // entries per row, then row offsets
  __shared__ int s_flag[kSmallPairs + 1];               // run starts, then their positions
  __shared__ unsigned long long s_key[kSmallPairs];     // (item, row) keys, then (row, item)
  __shared__ unsigned long long s_u[kSmallPairs];       // the unique (item, row) keys
  __shared__ int32_t s_ids[kSmallPairs];                // the IDs, read once
  __shared__ int s_wsum[kSmallThreads / 64 + 1];
  const int tid = threadIdx.x;
  const int nT = (int)T;
  unsigned long long bad = 0;
  for (int i = tid; i < (int)nnz; i += kSmallThreads) s_ids[i] = ids[i];
  __syncthreads();
  // 1. valid entries per row (malformed rows: one data error, no entries), their offsets,
  //    and the pairs in row order
  for (int t = tid; t < nT; t += kSmallThreads) {
    const int64_t b = row_ptr[t], e = row_ptr[t + 1];
    int c = 0;
    if (b < 0 || e > nnz || e < b) {
      ++bad;
    } else if (mask == nullptr || mask[t] != 0) {
      for (int64_t i = b; i < e; ++i) {
        const int32_t v = s_ids[i];
        if (pad >= 0 && v == pad) continue;
        if (v < 0 || (int64_t)v >= V) { ++bad; continue; }
        ++c;
      }
    }
    s_off[t] = c;
  }
  __syncthreads();
  const int n0 = small_scan(s_off, nT, s_wsum);
  const int n0c = (int64_t)n0 > nnz ? (int)nnz : n0;   // overlapping rows: the excess is an error
  if (tid == 0 && n0c < n0) bad += (unsigned long long)(n0 - n0c);
  for (int t = tid; t < nT; t += kSmallThreads) {
    if (s_off[t + 1] == s_off[t]) continue;
    const int64_t b = row_ptr[t], e = row_ptr[t + 1];
    int64_t o = s_off[t];
    for (int64_t i = b; i < e; ++i) {
      const int32_t v = s_ids[i];
      if (pad >= 0 && v == pad) continue;
      if (v < 0 || (int64_t)v >= V) continue;
      if (o >= nnz) break;
      s_key[o] = ((unsigned long long)(uint32_t)v << 32) | (uint32_t)t;
      ++o;
    }
  }
  // 2. item-major order; the first of each run of equal keys is a unique pair
  const int N0 = small_pow2(n0c);
  for (int i = n0c + tid; i < N0; i += kSmallThreads) s_key[i] = ~0ull;
  __syncthreads();
  if (n0c > 1) {
    if (N0 <= kSmallThreads) small_sort_lanes(s_key, N0);
    else small_sort(s_key, N0);
  }
  for (int i = tid; i < n0c; i += kSmallThreads) s_flag[i] = (i == 0 || s_key[i] != s_key[i - 1]) ? 1 : 0;
  __syncthreads();
  const int n = small_scan(s_flag, n0c, s_wsum);
  for (int i = tid; i < n0c; i += kSmallThreads) {
    if (i == 0 || s_key[i] != s_key[i - 1]) {
      const int q = s_flag[i];
      const unsigned long long k = s_key[i];
      s_u[q] = k;
      w.csc_items[q] = (int32_t)(k >> 32);
      w.csc_rows[q] = (int32_t)(k & 0xffffffffull);
    }
  }
  __syncthreads();
  // 3. unique items and their segment starts
  for (int j = tid; j < n; j += kSmallThreads) s_flag[j] = (j == 0 || (s_u[j] >> 32) != (s_u[j - 1] >> 32)) ? 1 : 0;
  __syncthreads();
  const int nu = small_scan(s_flag, n, s_wsum);
  for (int j = tid; j < n; j += kSmallThreads) {
    if (j == 0 || (s_u[j] >> 32) != (s_u[j - 1] >> 32)) {
      w.uitems[s_flag[j]] = (int32_t)(s_u[j] >> 32);
      w.useg[s_flag[j]] = j;
    }
  }
  if (tid == 0) w.useg[nu] = n;
  // 4. canonical CSR: the unique pairs by row, items ascending within a row
  const int N1 = small_pow2(n);
  for (int j = tid; j < N1; j += kSmallThreads)
    s_key[j] = j < n ? ((s_u[j] & 0xffffffffull) << 32) | (s_u[j] >> 32) : ~0ull;
  __syncthreads();
  if (n > 1) {
    if (N1 <= kSmallThreads) small_sort_lanes(s_key, N1);
    else small_sort(s_key, N1);
  }
  for (int j = tid; j < n; j += kSmallThreads) w.cids[j] = (int32_t)(s_key[j] & 0xffffffffull);
  for (int j = tid; j <= n; j += kSmallThreads) {
    const int r_prev = j == 0 ? -1 : (int)(s_key[j - 1] >> 32);
    const int r_cur = j == n ? nT : (int)(s_key[j] >> 32);
    for (int r = r_prev + 1; r <= r_cur; ++r) w.crow[r] = j;
  }
  if (tid == 0) {
    w.counts[0] = n0c;
    w.counts[1] = n;
    w.counts[2] = nu;
  }
  if (bad) atomicAdd(w.err, bad);
}

hipError_t launch_targets(const TargetsWs& w, int64_t T, int64_t V, int64_t nnz,
                          const int32_t* row_ptr, const int32_t* ids, const uint8_t* mask, int32_t pad_id,
                          const int64_t* ce_target, int64_t ignore_index, hipStream_t st) {
  if (ce_target == nullptr && nnz <= kSmallPairs && T <= kSmallRows) {
    k_targets_small<<<1, kSmallThreads, 0, st>>>(T, V, nnz, row_ptr, ids, mask, pad_id, w);
    return hipGetLastError();
  }
  const int64_t cap = ce_target ? T : nnz;     // capacity of every pair array
  // 1. valid entries per row, their offsets, compacted (item, row) pairs in row order
  if (ce_target) {
    k_row_count_ce<<<grid_for(T, 256), 256, 0, st>>>(T, V, ce_target, ignore_index, w.cnt, w.err);
  } else {
    k_row_count<<<grid_for(T, 256), 256, 0, st>>>(T, V, nnz, row_ptr, ids, mask, pad_id, w.cnt, w.err);
  }
  k_scan<<<1, 1024, 0, st>>>(w.cnt, T, nullptr, w.off, w.counts + 0);
  k_clamp_count<<<1, 64, 0, st>>>(w.counts, cap, w.err);
  if (ce_target) {
    k_row_compact_ce<<<grid_for(T, 256), 256, 0, st>>>(T, ce_target, w.cnt, w.off, w.keyA, w.valA);
  } else {
    k_row_compact<<<grid_for(T, 256), 256, 0, st>>>(T, V, nnz, row_ptr, ids, w.cnt, w.off, pad_id, w.keyA, w.valA);
  }
  // 2. item-major order, repeats removed
  const bool inB = radix_sort(w, w.keyA, w.valA, w.keyB, w.valB, w.counts + 0, cap, bits_for(V), st);
  const int32_t* ks = inB ? w.keyB : w.keyA;
  const int32_t* vs = inB ? w.valB : w.valA;
  const unsigned g = grid_for(cap + 1, 256);
  k_flag_pairs<<<g, 256, 0, st>>>(ks, vs, w.counts + 0, cap, w.flags);
  k_scan<<<1, 1024, 0, st>>>(w.flags, cap, nullptr, w.fscan, w.counts + 1);
  k_compact_pairs<<<g, 256, 0, st>>>(ks, vs, w.flags, w.fscan, w.counts + 0, cap, w.csc_items, w.csc_rows);
  // 3. unique items and segment starts
  k_flag_items<<<g, 256, 0, st>>>(w.csc_items, w.counts + 1, cap, w.flags);
  k_scan<<<1, 1024, 0, st>>>(w.flags, cap, nullptr, w.fscan, w.counts + 2);
  k_compact_items<<<g, 256, 0, st>>>(w.csc_items, w.flags, w.fscan, w.counts + 1, w.counts + 2, cap, w.uitems, w.useg);
  // 4. canonical CSR: stable sort of the unique pairs by row
  k_copy2<<<g, 256, 0, st>>>(w.csc_rows, w.csc_items, w.counts + 1, cap, w.keyA, w.valA);
  const bool inB2 = radix_sort(w, w.keyA, w.valA, w.keyB, w.valB, w.counts + 1, cap, bits_for(T), st);
  const int32_t* rs = inB2 ? w.keyB : w.keyA;
  const int32_t* is = inB2 ? w.valB : w.valA;
  k_copy2<<<g, 256, 0, st>>>(is, is, w.counts + 1, cap, w.cids, w.cids);
  k_row_ptr<<<grid_for(cap + 1, 256), 256, 0, st>>>(rs, w.counts + 1, cap, T, w.crow);
  return hipGetLastError();
}

namespace {
__global__ void k_fill_i32(int32_t* p, int64_t n, int32_t v) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}
__global__ void k_item_map(const int32_t* __restrict__ uitems, const int32_t* __restrict__ counts, int64_t cap,
                           int32_t* __restrict__ map) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < cap && i < counts[2]) map[uitems[i]] = (int32_t)i;
}
}  // namespace

hipError_t launch_zero_bytes(void* p, size_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  if (n % 4 != 0) return hipErrorInvalidValue;
  const int64_t n4 = (int64_t)(n / 4);
  k_fill_i32<<<(unsigned)std::min<int64_t>((n4 + 255) / 256, 4096), 256, 0, st>>>((int32_t*)p, n4, 0);
  return hipGetLastError();
}

hipError_t launch_item_map(const TargetsWs& w, int64_t V, int64_t cap, int32_t* map, hipStream_t st) {
  if (V <= 0) return hipSuccess;
  k_fill_i32<<<(unsigned)std::min<int64_t>((V + 255) / 256, 4096), 256, 0, st>>>(map, V, -1);
  if (cap > 0) k_item_map<<<grid_for(cap, 256), 256, 0, st>>>(w.uitems, w.counts, cap, map);
  return hipGetLastError();
}

}  // namespace cl
