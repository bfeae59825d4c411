// C ABI of the cutloss library: argument validation, workspace layout and kernel order.
// Every entry point validates on the host and returns before launching anything if a
// check fails; all work is then enqueued on the caller's stream without synchronizing.
#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "launch.h"

namespace {

// Heads with D in {64, 128, 256} and bf16 E run the fused LDS-DMA sweeps (sweep2.hip);
// every other supported head runs the chunked GEMM path (gemm.hip).
hipError_t rows_sweep(const cl::SweepParams& sp, int mode, hipStream_t st) { return cl::launch_sweep2_rows(sp, mode, st); }

hipError_t cols_sweep(const cl::SweepParams& sp, int kind, int epi, hipStream_t st) {
  return cl::launch_sweep2_cols(sp, kind, epi, st);
}

// ---- phase profiling (cutloss_profile_enable / cutloss_profile_read)
struct PhaseRec {
  int phase;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<PhaseRec> g_prof;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t prof_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

// RAII scope that brackets one phase with events when profiling is on.
struct Phase {
  int phase;
  hipStream_t st;
  hipEvent_t a = nullptr;
  Phase(int ph, hipStream_t s) : phase(ph), st(s) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    if (!g_prof_on) return;
    a = prof_event();
    if (a) hipEventRecord(a, st);
  }
  ~Phase() {
    std::lock_guard<std::mutex> g(g_prof_mu);
    if (!a) return;
    hipEvent_t b = prof_event();
    if (!b) return;
    hipEventRecord(b, st);
    g_prof.push_back({phase, a, b});
  }
};

thread_local std::string g_last_error;

cutloss_status fail(cutloss_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

cutloss_status hip_check(hipError_t e, const char* where) {
  if (e == hipSuccess) return CUTLOSS_OK;
  return fail(CUTLOSS_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

constexpr size_t kAlign = 256;
size_t up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }

// Workspace carving: a bump allocator over the caller's buffer (or a null base to size it).
struct Carver {
  char* base;
  size_t off = 0;
  explicit Carver(void* b) : base((char*)b) {}
  template <class T>
  T* take(size_t n) {
    T* p = base ? (T*)(base + off) : nullptr;
    off += up(sizeof(T) * (n > 0 ? n : 1));
    return p;
  }
};

struct Plan {
  int64_t T, D, V, cap;
  int n_splits;
  int64_t split_len;
};

// Vocabulary splits of the rows sweep: enough (row block, split) workgroups to fill the
// chip about twice; a multiple of 8 so each split maps to one XCD.
Plan make_plan(int64_t T, int64_t D, int64_t V, int64_t cap, int e_fp8) {
  Plan pl{T, D, V, cap, 1, 0};
  const bool sw = cl::sweep2_rows_supported(D, e_fp8);
  const int64_t rpb = sw ? cl::sweep2_rows_per_block(D) : 128;
  const int64_t target = 4096 / (sw ? cl::sweep2_waves_per_block(D) : 4);   // about 4096 waves
  const int64_t nsb = (T + rpb - 1) / rpb;
  int64_t ns = nsb > 0 ? (target + nsb - 1) / nsb : 1;
  const int64_t max_ns = (V + 31) / 32;
  if (ns > max_ns) ns = max_ns;
  if (ns > 256) ns = 256;
  if (ns >= 8) ns = ns / 8 * 8;
  if (ns < 1) ns = 1;
  int64_t sl = (V + ns - 1) / ns;
  sl = (sl + 31) / 32 * 32;
  pl.n_splits = (int)ns;
  pl.split_len = sl;
  return pl;
}

struct Ws {
  unsigned long long* err;
  cl::TargetsWs tw;
  float* w;
  float* part_a;
  float* part_b;
  float* part_dA;
  float* S_u;
  float* S_part;
  size_t bytes;
};

// op: 0 fwd (loss partials), 1 bwd (dA partials + S_u), 2 CE fwd (two partial arrays)
Ws carve(void* base, const Plan& pl, bool need_dA, bool need_Su, bool two_partials) {
  Carver c(base);
  Ws w{};
  w.err = c.take<unsigned long long>(4);
  const int64_t T = pl.T, cap = pl.cap;
  const size_t nblk = cl::targets_radix_blocks(cap);
  cl::TargetsWs& t = w.tw;
  t.err = w.err;
  t.counts = c.take<int32_t>(4);
  t.cnt = c.take<int32_t>(T + 1);
  t.off = c.take<int32_t>(T + 1);
  t.keyA = c.take<int32_t>(cap);
  t.valA = c.take<int32_t>(cap);
  t.keyB = c.take<int32_t>(cap);
  t.valB = c.take<int32_t>(cap);
  t.flags = c.take<int32_t>(cap + 1);
  t.fscan = c.take<int32_t>(cap + 1);
  t.hist = c.take<int32_t>(256 * nblk);
  t.hscan = c.take<int32_t>(256 * nblk + 1);
  t.csc_items = c.take<int32_t>(cap);
  t.csc_rows = c.take<int32_t>(cap);
  t.uitems = c.take<int32_t>(cap);
  t.useg = c.take<int32_t>(cap + 1);
  t.crow = c.take<int32_t>(T + 1);
  t.cids = c.take<int32_t>(cap);
  w.w = c.take<float>(T);
  w.part_a = c.take<float>((size_t)pl.n_splits * T);
  w.part_b = two_partials ? c.take<float>((size_t)pl.n_splits * T) : nullptr;
  w.part_dA = need_dA ? c.take<float>((size_t)pl.n_splits * T * pl.D) : nullptr;
  w.S_u = need_Su ? c.take<float>((size_t)cap * pl.D) : nullptr;
  w.S_part = need_Su ? c.take<float>(2 * cl::item_sum_parts(cap) * pl.D) : nullptr;
  w.bytes = c.off;
  return w;
}

// ---------------------------------------------------------------------------------
// Chunked path (wide heads, FP8 E): see gemm.hip.
// ---------------------------------------------------------------------------------
bool use_chunked(int64_t D, int e_fp8) {
  return !(cl::sweep2_rows_supported(D, e_fp8) && cl::sweep2_cols_supported(D, e_fp8));
}

int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }
int64_t ceil_div(int64_t x, int64_t a) { return (x + a - 1) / a; }

struct ChunkPlan {
  int64_t T, D, V, cap;
  int64_t Tp;         // rows of the P buffer P[t][item], a multiple of bt
  int64_t bt;         // P row-block height: 128 for T <= 128, else 256 (blocks of bt x 32)
  int64_t Vc;         // items per chunk (multiple of the item tile)
  int64_t n_chunks;
  int64_t n_splits;   // loss / lse partials: one per item tile
  int64_t sk;         // split-K slices of the dA product
  int64_t sk_rows;    // dA partials of the whole-row FP8 SGD product when it also forms dA (0: n/a)
  int64_t kps;        // items per slice
  int64_t flag_bn, flag_ld;   // gradient filter flags: row tile of the logits product, row tiles
  bool q8;            // FP8 logits: the logits product multiplies FP8 activations and FP8 E
  bool trans_dA;      // FP8 E, at most 128 rows: the dA product runs as dA^T = E_c^T P^T (M = D)
};

constexpr int64_t kChunkPBytes = 2ll << 30;     // P buffer budget
// at least this many vocabulary chunks whatever T is, so that the gradient tile of a chunk
// holds at most an eighth of the T x V logits (ELMO's 8-way label chunking of the logit
// buffer, ai.info summary, Main Findings)
constexpr int64_t kMinChunks = 8;

ChunkPlan make_chunk_plan(int64_t T, int64_t D, int64_t V, int64_t cap, bool q8 = false, bool e_fp8 = false,
                          bool no_tile = false) {
  ChunkPlan c{};
  c.T = T; c.D = D; c.V = V; c.cap = cap; c.q8 = q8;
  // a 256-row tile over at most 128 rows would waste half the dA product's MFMAs
  c.trans_dA = e_fp8 && T <= 128;
  const int64_t bm = cl::gemm_tile_m();
  c.bt = round_up(T > 0 ? T : 1, 128) <= 128 ? 128 : 256;
  c.Tp = round_up(T > 0 ? T : 1, c.bt);
  int64_t vc = kChunkPBytes / (c.Tp * 2) / bm * bm;
  vc = std::min(vc, round_up(ceil_div(V, kMinChunks), bm));
  // a call that stores no gradient tile (a forward) runs the whole vocabulary as one chunk
  if (no_tile) vc = round_up(V > 0 ? V : 1, bm);
  // CUTLOSS_MAX_CHUNK_ITEMS caps the chunk (rounded down to the item tile): a tuning knob,
  // and the way tests exercise several chunks on small problems
  if (const char* env = std::getenv("CUTLOSS_MAX_CHUNK_ITEMS")) {
    const long long cap_items = std::atoll(env);
    if (cap_items > 0 && cap_items / bm * bm < vc) vc = cap_items / bm * bm;
  }
  if (vc < bm) vc = bm;
  if (vc > round_up(V, bm)) vc = round_up(V, bm);
  c.Vc = vc;
  c.n_chunks = ceil_div(V, vc);
  c.n_splits = ceil_div(V, bm);   // one loss partial per item tile (its wave rows combined)
  // dA product: (row tiles) x (D tiles) x split-K slices. Every slice's partial [T][D] is
  // read and rewritten once per chunk, so fewer, longer slices move fewer bytes; heads up to
  // D = 1024 take about 512 workgroups, wider (compute-bound) ones about 1024. The
  // transposed product (3 tiles at D = 768) rounds down, so that its one-per-CU workgroups
  // fill whole waves (510 on 256 CUs; 1026 left a fifth wave of 2).
  const int64_t tiles = c.trans_dA
      ? ceil_div(D, bm) * ceil_div(T > 0 ? T : 1, cl::gemm_tile_n_of(cl::GEMM_EPI_ACC, D, T > 0 ? T : 1, D))
      : ceil_div(T > 0 ? T : 1, bm) * ceil_div(D, cl::gemm_tile_n_of(cl::GEMM_EPI_ACC, T, D, D));
  const int64_t blocks = D <= 1024 ? 512 : 1024;
  int64_t sk = c.trans_dA ? blocks / tiles : ceil_div(blocks, tiles);
  if (sk > vc / 32) sk = vc / 32;
  if (sk < 1) sk = 1;
  c.kps = round_up(ceil_div(vc, sk), 32);
  c.sk = ceil_div(vc, c.kps);
  // (the nearest-even shape has the most block rows, so its count bounds both roundings)
  c.sk_rows = e_fp8 && cl::sgd_rows_supported(c.Tp, D) ? cl::sgd_rows_dA_splits(ceil_div(std::min(vc, V), 32), D, 0) : 0;
  c.flag_bn = cl::gemm_tile_n_of(cl::GEMM_EPI_CE_P, vc, T > 0 ? T : 1, D);
  c.flag_ld = ceil_div(T > 0 ? T : 1, c.flag_bn);
  return c;
}

struct Ws2 {
  unsigned long long* err;
  cl::TargetsWs tw;
  float* w;
  float* part_a;
  float* part_b;
  uint16_t* P;
  float* part_dA;
  float* pos_dot;
  float* pos_sum;
  int32_t* pos_tp;
  float* S_u;
  float* S_part;
  float* red;         // staging of the split reductions
  int32_t* flags;     // gradient filter: [Vc / 256][flag_ld]
  int32_t* imap;      // [V] item -> unique-item index (dE / SGD epilogue)
  uint16_t* Et;       // the chunk's bf16 E transposed, [D][Vc] (the dA product's k-contiguous operand)
  uint8_t* A8;        // FP8 logits: E4M3FN copy of A [T][D]
  uint16_t* Aw;       // BCE dE product: the rows of A weighted by w, bf16 [T][D]
  uint16_t* AwT;      // the same transposed, [D][128] bf16 (FP8 SGD of heads of at most 128 rows)
  size_t bytes;
};

Ws2 carve_chunked(void* base, const ChunkPlan& pl, bool need_P, bool need_dA, bool need_Su, bool two_partials,
                  bool need_pos, bool need_Et) {
  Carver c(base);
  Ws2 w{};
  w.err = c.take<unsigned long long>(4);
  const int64_t T = pl.T, cap = pl.cap;
  const size_t nblk = cl::targets_radix_blocks(cap);
  cl::TargetsWs& t = w.tw;
  t.err = w.err;
  t.counts = c.take<int32_t>(4);
  t.cnt = c.take<int32_t>(T + 1);
  t.off = c.take<int32_t>(T + 1);
  t.keyA = c.take<int32_t>(cap);
  t.valA = c.take<int32_t>(cap);
  t.keyB = c.take<int32_t>(cap);
  t.valB = c.take<int32_t>(cap);
  t.flags = c.take<int32_t>(cap + 1);
  t.fscan = c.take<int32_t>(cap + 1);
  t.hist = c.take<int32_t>(256 * nblk);
  t.hscan = c.take<int32_t>(256 * nblk + 1);
  t.csc_items = c.take<int32_t>(cap);
  t.csc_rows = c.take<int32_t>(cap);
  t.uitems = c.take<int32_t>(cap);
  t.useg = c.take<int32_t>(cap + 1);
  t.crow = c.take<int32_t>(T + 1);
  t.cids = c.take<int32_t>(cap);
  w.w = c.take<float>(T);
  w.part_a = c.take<float>((size_t)pl.n_splits * T);
  w.part_b = two_partials ? c.take<float>((size_t)pl.n_splits * T) : nullptr;
  w.P = need_P ? c.take<uint16_t>((size_t)pl.Vc * pl.Tp) : nullptr;
  const int64_t n_dA = std::max(pl.sk, pl.sk_rows);
  w.part_dA = need_dA ? c.take<float>((size_t)n_dA * T * pl.D) : nullptr;
  w.pos_dot = need_pos ? c.take<float>(T) : nullptr;
  w.pos_sum = need_pos && need_dA ? c.take<float>((size_t)T * pl.D) : nullptr;
  w.pos_tp = need_pos ? c.take<int32_t>(T) : nullptr;
  w.S_u = need_Su ? c.take<float>((size_t)cap * pl.D) : nullptr;
  w.S_part = need_Su ? c.take<float>(2 * cl::item_sum_parts(cap) * pl.D) : nullptr;
  const size_t red_loss = cl::reduce_splits_tmp_floats(pl.n_splits, T, two_partials ? 1 : 0);
  const size_t red_dA = need_dA ? cl::reduce_splits_tmp_floats(n_dA, T * pl.D, 0) : 0;
  w.red = c.take<float>(std::max<size_t>(1, std::max(red_loss, red_dA)));
  w.flags = need_P ? c.take<int32_t>((size_t)(pl.Vc / 256) * pl.flag_ld) : nullptr;
  w.Et = need_dA && need_Et ? c.take<uint16_t>((size_t)pl.Vc * pl.D) : nullptr;
  w.A8 = pl.q8 ? c.take<uint8_t>((size_t)T * pl.D) : nullptr;
  w.imap = need_Su ? c.take<int32_t>((size_t)pl.V) : nullptr;
  w.Aw = need_Su ? c.take<uint16_t>((size_t)T * pl.D) : nullptr;
  w.AwT = need_Su && cl::sgd_rows_supported(pl.Tp, pl.D) ? c.take<uint16_t>((size_t)pl.D * pl.Tp) : nullptr;
  w.bytes = c.off;
  return w;
}

cl::GemmOperand operand(const void* p, int64_t ld, int64_t rows_valid, int64_t cols_valid, int kc, int fp8,
                        int bt = 0, int64_t nvb = 0) {
  cl::GemmOperand o;
  o.p = p; o.ld = ld; o.rows_valid = rows_valid; o.cols_valid = cols_valid; o.kc = kc; o.fp8 = fp8;
  o.bt = bt; o.nvb = nvb;
  return o;
}

cutloss_status check_common(int64_t T, int64_t D, int64_t V, const void* A, const void* E, int e_dtype) {
  if (T < 0 || D <= 0 || V <= 0) return fail(CUTLOSS_ERR_INVALID_ARG, "bad sizes T=%lld D=%lld V=%lld", (long long)T, (long long)D, (long long)V);
  if (T >= (1ll << 31) || V >= (1ll << 31)) return fail(CUTLOSS_ERR_INVALID_ARG, "T and V must be < 2^31");
  if (D % 64 != 0) return fail(CUTLOSS_ERR_UNSUPPORTED, "D=%lld must be a multiple of 64", (long long)D);
  if (D > 2304 * 4) return fail(CUTLOSS_ERR_UNSUPPORTED, "D=%lld too large", (long long)D);
  if (e_dtype != CUTLOSS_BF16 && e_dtype != CUTLOSS_FP8_E4M3) return fail(CUTLOSS_ERR_INVALID_ARG, "unknown e_dtype %d", e_dtype);
  if (T > 0 && (A == nullptr || !aligned(A, 16))) return fail(CUTLOSS_ERR_INVALID_ARG, "A must be a non-NULL 16-byte aligned device pointer");
  if (E == nullptr || !aligned(E, 16)) return fail(CUTLOSS_ERR_INVALID_ARG, "E must be a non-NULL 16-byte aligned device pointer");
  return CUTLOSS_OK;
}

cutloss_status check_bce(const cutloss_bce_problem* p) {
  if (p == nullptr) return fail(CUTLOSS_ERR_INVALID_ARG, "problem is NULL");
  cutloss_status s = check_common(p->T, p->D, p->V, p->A, p->E, p->e_dtype);
  if (s != CUTLOSS_OK) return s;
  if (p->nnz < 0 || p->nnz >= (1ll << 31)) return fail(CUTLOSS_ERR_INVALID_ARG, "bad nnz %lld", (long long)p->nnz);
  if (p->T > 0 && (p->pos_row_ptr == nullptr || !aligned(p->pos_row_ptr, 4))) return fail(CUTLOSS_ERR_INVALID_ARG, "pos_row_ptr must be a non-NULL aligned device pointer");
  if (p->nnz > 0 && (p->pos_ids == nullptr || !aligned(p->pos_ids, 4))) return fail(CUTLOSS_ERR_INVALID_ARG, "pos_ids must be a non-NULL aligned device pointer");
  return CUTLOSS_OK;
}

cutloss_status check_ce(const cutloss_ce_problem* p) {
  if (p == nullptr) return fail(CUTLOSS_ERR_INVALID_ARG, "problem is NULL");
  cutloss_status s = check_common(p->T, p->D, p->V, p->A, p->E, p->e_dtype);
  if (s != CUTLOSS_OK) return s;
  if (p->T > 0 && (p->target == nullptr || !aligned(p->target, 8))) return fail(CUTLOSS_ERR_INVALID_ARG, "target must be a non-NULL 8-byte aligned device pointer");
  return CUTLOSS_OK;
}

cutloss_status check_ws(void* ws, size_t have, size_t need) {
  if (have < need) return fail(CUTLOSS_ERR_WORKSPACE, "workspace too small: %zu < %zu bytes", have, need);
  if (need > 0 && (ws == nullptr || !aligned(ws, kAlign))) return fail(CUTLOSS_ERR_INVALID_ARG, "workspace must be a non-NULL 256-byte aligned device pointer");
  return CUTLOSS_OK;
}

cutloss_status check_out(const void* ptr, size_t align, const char* name, bool required) {
  if (ptr == nullptr) return required ? fail(CUTLOSS_ERR_INVALID_ARG, "%s is NULL", name) : CUTLOSS_OK;
  if (!aligned(ptr, align)) return fail(CUTLOSS_ERR_INVALID_ARG, "%s must be %zu-byte aligned", name, align);
  return CUTLOSS_OK;
}

#define CL_TRY(expr)                      \
  do {                                    \
    cutloss_status _s = (expr);           \
    if (_s != CUTLOSS_OK) return _s;      \
  } while (0)
#define CL_HIP(expr, where) CL_TRY(hip_check((expr), where))

// BCE pipeline shared by fwd / bwd / bwd_sgd.
// want_loss: emit loss; want_dA; dE_mode: 0 none, 1 write dE, 2 SGD in place
cutloss_status bce_run_chunked(const cutloss_bce_problem* p, const float* dloss, float* loss, void* dA, void* dE,
                               int dE_mode, float lr, void* ws, size_t ws_bytes, hipStream_t st, int32_t* counts,
                               int sr = 0, uint64_t sr_seed = 0, bool fp8_logits = false);
cutloss_status ce_run_chunked(const cutloss_ce_problem* p, const float* lse_in, const float* dloss, float* loss,
                              float* lse, void* dA, void* dE, void* ws, size_t ws_bytes, hipStream_t st,
                              float filter_eps);

// smallest bf16 bit pattern whose value is >= eps (eps > 0, finite); 0 = filter off
uint32_t filter_bits_of(float eps) {
  if (!(eps > 0.0f)) return 0u;
  uint32_t u;
  std::memcpy(&u, &eps, 4);
  const uint32_t hi = u >> 16;
  return (u & 0xFFFFu) ? hi + 1 : hi;
}

// counts != NULL (forward only): Cut Metrics in the same pass as the loss
cutloss_status bce_run(const cutloss_bce_problem* p, const float* dloss, float* loss, void* dA, void* dE,
                       int dE_mode, float lr, void* ws, size_t ws_bytes, hipStream_t st, int32_t* counts = nullptr) {
  if (use_chunked(p->D, p->e_dtype == CUTLOSS_FP8_E4M3))
    return bce_run_chunked(p, dloss, loss, dA, dE, dE_mode, lr, ws, ws_bytes, st, counts);
  const Plan pl = make_plan(p->T, p->D, p->V, p->nnz, p->e_dtype == CUTLOSS_FP8_E4M3);
  const bool rows_grad = dA != nullptr;
  const bool need_Su = dE_mode != 0;
  const Ws w = carve(ws, pl, rows_grad, need_Su, counts != nullptr);
  CL_TRY(check_ws(ws, ws_bytes, w.bytes));
  const int e_fp8 = p->e_dtype == CUTLOSS_FP8_E4M3;

  {
    Phase ph(CUTLOSS_PHASE_TARGETS, st);
    CL_HIP(cl::launch_zero_u64(w.err, 4, st), "zero counters");
    CL_HIP(cl::launch_targets(w.tw, p->T, p->V, p->nnz, p->pos_row_ptr, p->pos_ids, p->row_mask, p->pad_id,
                              nullptr, 0, st), "targets");
  }

  cl::FinalizeParams fp{};
  fp.T = p->T; fp.D = p->D; fp.V = p->V; fp.A = p->A; fp.E = p->E; fp.e_fp8 = e_fp8;
  fp.crow = w.tw.crow; fp.cids = w.tw.cids; fp.dloss = dloss; fp.mask = p->row_mask;
  fp.n_splits = pl.n_splits; fp.n_splits_dA = pl.n_splits; fp.part_a = w.part_a; fp.part_dA = w.part_dA;
  fp.loss = loss; fp.dA = dA; fp.w_out = w.w;
  fp.part_c = w.part_b; fp.counts = counts;

  cl::SweepParams sp{};
  sp.T = p->T; sp.D = p->D; sp.V = p->V; sp.A = p->A; sp.E = p->E; sp.e_fp8 = e_fp8;
  sp.n_splits = pl.n_splits; sp.split_len = pl.split_len;
  sp.part_a = w.part_a; sp.part_b = w.part_b; sp.part_dA = w.part_dA;
  sp.w = w.w; sp.uitems = w.tw.uitems; sp.counts = w.tw.counts; sp.S_u = w.S_u;
  sp.dE = dE_mode == 1 ? dE : nullptr; sp.E_inplace = dE_mode == 2 ? (void*)p->E : nullptr; sp.lr = lr;

  if (p->T > 0 && (loss != nullptr || rows_grad)) {
    const int mode = rows_grad ? (loss ? 2 : 1) : (counts ? 5 : 0);
    {
      Phase ph(CUTLOSS_PHASE_ROWS, st);
      CL_HIP(rows_sweep(sp, mode, st), "rows sweep");
    }
    Phase ph(CUTLOSS_PHASE_FINALIZE, st);
    CL_HIP(cl::launch_finalize_rows(fp, 0, loss != nullptr, rows_grad, st), "finalize rows");
  }
  if (dE_mode != 0) {
    {
      Phase ph(CUTLOSS_PHASE_ITEM_SUMS, st);
      CL_HIP(cl::launch_row_weights(fp, 0, st), "row weights");
      CL_HIP(cl::launch_item_sums(p->D, pl.cap, p->A, w.w, w.tw.csc_rows, w.tw.useg, w.tw.counts, w.S_u, w.S_part, st), "item sums");
    }
    Phase ph(CUTLOSS_PHASE_COLS, st);
    CL_HIP(cols_sweep(sp, 0, dE_mode == 2 ? 1 : 0, st), "cols sweep");
  }
  return CUTLOSS_OK;
}

// filter_eps > 0 (backward only): the CE gradient filter
cutloss_status ce_run(const cutloss_ce_problem* p, const float* lse_in, const float* dloss, float* loss, float* lse,
                      void* dA, void* dE, void* ws, size_t ws_bytes, hipStream_t st, float filter_eps = 0.0f) {
  if (use_chunked(p->D, p->e_dtype == CUTLOSS_FP8_E4M3))
    return ce_run_chunked(p, lse_in, dloss, loss, lse, dA, dE, ws, ws_bytes, st, filter_eps);
  const bool fwd = loss != nullptr;
  const Plan pl = make_plan(p->T, p->D, p->V, p->T, p->e_dtype == CUTLOSS_FP8_E4M3);
  const Ws w = carve(ws, pl, dA != nullptr, dE != nullptr, fwd);
  CL_TRY(check_ws(ws, ws_bytes, w.bytes));
  const int e_fp8 = p->e_dtype == CUTLOSS_FP8_E4M3;

  {
    Phase ph(CUTLOSS_PHASE_TARGETS, st);
    CL_HIP(cl::launch_zero_u64(w.err, 4, st), "zero counters");
    CL_HIP(cl::launch_targets(w.tw, p->T, p->V, p->T, nullptr, nullptr, nullptr, -1, p->target, p->ignore_index, st), "targets");
  }

  cl::FinalizeParams fp{};
  fp.T = p->T; fp.D = p->D; fp.V = p->V; fp.A = p->A; fp.E = p->E; fp.e_fp8 = e_fp8;
  fp.crow = w.tw.crow; fp.cids = w.tw.cids; fp.dloss = dloss; fp.ce_target = p->target; fp.ignore_index = p->ignore_index;
  fp.n_splits = pl.n_splits; fp.n_splits_dA = pl.n_splits; fp.part_a = w.part_a; fp.part_b = w.part_b; fp.part_dA = w.part_dA;
  fp.loss = loss; fp.lse = lse; fp.dA = dA; fp.w_out = w.w; fp.lse_in = lse_in;

  cl::SweepParams sp{};
  sp.T = p->T; sp.D = p->D; sp.V = p->V; sp.A = p->A; sp.E = p->E; sp.e_fp8 = e_fp8;
  sp.n_splits = pl.n_splits; sp.split_len = pl.split_len;
  sp.part_a = w.part_a; sp.part_b = w.part_b; sp.part_dA = w.part_dA;
  sp.w = w.w; sp.lse = lse_in; sp.uitems = w.tw.uitems; sp.counts = w.tw.counts; sp.S_u = w.S_u; sp.dE = dE;
  sp.filter_bits = fwd ? 0u : filter_bits_of(filter_eps);

  if (fwd) {
    if (p->T > 0) {
      {
        Phase ph(CUTLOSS_PHASE_ROWS, st);
        CL_HIP(rows_sweep(sp, 3, st), "rows sweep");
      }
      Phase ph(CUTLOSS_PHASE_FINALIZE, st);
      CL_HIP(cl::launch_finalize_rows(fp, 1, 1, 0, st), "finalize rows");
    }
    return CUTLOSS_OK;
  }
  if (dA != nullptr && p->T > 0) {
    {
      Phase ph(CUTLOSS_PHASE_ROWS, st);
      CL_HIP(rows_sweep(sp, 4, st), "rows sweep");
    }
    Phase ph(CUTLOSS_PHASE_FINALIZE, st);
    CL_HIP(cl::launch_finalize_rows(fp, 1, 0, 1, st), "finalize rows");
  }
  if (dE != nullptr) {
    {
      Phase ph(CUTLOSS_PHASE_ITEM_SUMS, st);
      CL_HIP(cl::launch_row_weights(fp, 1, st), "row weights");
      CL_HIP(cl::launch_item_sums(p->D, pl.cap, p->A, w.w, w.tw.csc_rows, w.tw.useg, w.tw.counts, w.S_u, w.S_part, st), "item sums");
    }
    Phase ph(CUTLOSS_PHASE_COLS, st);
    CL_HIP(cols_sweep(sp, 1, 0, st), "cols sweep");
  }
  return CUTLOSS_OK;
}

// One vocabulary chunk of the chunked path: K1 (logits + epilogue), then K2 (dA) and
// K3 (dE / SGD) on the chunk's P. Stream order keeps K2 reading E_c before K3 updates it.
struct ChunkJob {
  const ChunkPlan* pl;
  const void* A; const void* E; int e_fp8;
  int k1_epi;            // GEMM_EPI_*
  const float* w; const float* lse;
  uint16_t* P; float* part_a; float* part_b;
  float* part_dA;        // NULL: no dA
  uint16_t* Et;          // bf16 E: workspace for the transposed chunk
  const uint8_t* A8;     // FP8 logits: the activations' E4M3FN copy
  const void* A_dE;      // the dE product's activations operand (NULL: A)
  const uint16_t* AwT;   // non-NULL: the SGD product runs as whole-row updates (sgd_rows.hip)
  bool rows_dA;          // with AwT: that product also forms the dA partials (no separate dA product)
  int64_t dA_splits;     // rows_dA: its partial count
  bool rows_logits;      // the BCE logits product streams 32-item blocks (logits_rows.hip)
  int k3_epi;            // -1: none, GEMM_EPI_DE or GEMM_EPI_SGD
  const int32_t* uitems; const int32_t* counts; const float* S_u; const int32_t* imap;
  void* dE; float lr;
  int sr; uint64_t sr_seed;   // SGD: stochastic rounding
  int32_t* flags; int64_t flag_ld; int flag_bn; float filter_eps;   // gradient filter (flags NULL: off)
};

cutloss_status run_chunks(const ChunkJob& j, hipStream_t st) {
  const ChunkPlan& pl = *j.pl;
  const int64_t bm = cl::gemm_tile_m();
  const int64_t esz = j.e_fp8 ? 1 : 2;
  for (int64_t c = 0; c < pl.n_chunks; ++c) {
    const int64_t v0 = c * pl.Vc;
    const int64_t vlen = std::min(pl.Vc, pl.V - v0);
    const int64_t mc = round_up(vlen, bm);
    const void* Ec = (const char*)j.E + v0 * pl.D * esz;
    if (j.rows_logits) {
      Phase ph(CUTLOSS_PHASE_CHUNK_LOGITS, st);
      cl::LogitsRowsParams r{};
      r.V = pl.V; r.T = pl.T; r.v0 = v0; r.nblk = mc / 32; r.nslots = mc / bm; r.part_base = v0 / bm;
      r.D = (int)pl.D; r.E = (const uint8_t*)Ec - v0 * pl.D; r.A = (const uint16_t*)j.A;
      r.P = j.k1_epi == cl::GEMM_EPI_BCE_P ? j.P : nullptr; r.part_a = j.part_a;
      r.part_b = j.k1_epi == cl::GEMM_EPI_BCE_METRICS ? j.part_b : nullptr;
      CL_HIP(cl::launch_logits_rows(r, st), "chunk logits rows");
    } else {
      Phase ph(CUTLOSS_PHASE_CHUNK_LOGITS, st);
      cl::GemmParams g{};
      g.a = operand(Ec, pl.D, vlen, pl.D, 1, j.e_fp8);
      g.b = j.A8 != nullptr ? operand(j.A8, pl.D, pl.T, pl.D, 1, 1) : operand(j.A, pl.D, pl.T, pl.D, 1, 0);
      // columns t < T (tiles past T would start outside A); P rows T .. tile end are written as 0
      g.M = mc; g.N = pl.T; g.K = pl.D; g.k_per_split = pl.D;
      g.epi = j.k1_epi;
      g.v0 = v0; g.V = pl.V; g.T = pl.T; g.D = pl.D;
      g.w = j.w; g.lse = j.lse; g.P = j.P; g.p_bt = (int)pl.bt; g.p_nvb = pl.Vc / 32; g.p_rows = pl.Tp;
      g.part_a = j.part_a; g.part_b = j.part_b;
      g.part_base = v0 / bm;
      g.flags = j.flags; g.flag_ld = j.flag_ld; g.flag_bn = j.flag_bn; g.flag_gen = (int)(c + 1);
      g.filter_eps = j.filter_eps;
      CL_HIP(cl::launch_gemm(g, st), "chunk logits");
    }
    if (j.part_dA != nullptr && !j.rows_dA) {
      Phase ph(CUTLOSS_PHASE_CHUNK_DA, st);
      cl::GemmParams g{};
      g.epi = cl::GEMM_EPI_ACC;
      g.T = pl.T; g.D = pl.D;
      g.acc = j.part_dA; g.ldacc = pl.D; g.acc_slice = pl.T * pl.D; g.acc_first = c == 0;
      g.k_per_split = pl.kps; g.K = mc;
      if (j.e_fp8 && pl.trans_dA && j.flags == nullptr) {
        // dA^T = E_c^T P^T: M = D, N = rows, stored as [row][d]
        g.a = operand(Ec, pl.D, vlen, pl.D, 0, 1);
        g.b = operand(j.P, 0, pl.Tp, mc, 1, 0, (int)pl.bt, pl.Vc / 32);
        g.M = pl.D; g.N = pl.T; g.acc_trans = 1;
      } else {
        g.a = operand(j.P, 0, pl.Tp, mc, 1, 0, (int)pl.bt, pl.Vc / 32);
        if (j.e_fp8) {
          g.b = operand(Ec, pl.D, vlen, pl.D, 0, 1);
        } else {
          // k-contiguous copy of the chunk (zero past vlen): the product reads it with
          // full-width LDS reads instead of transposing reads
          CL_HIP(cl::launch_transpose_chunk((const uint16_t*)Ec, vlen, mc, pl.D, j.Et, pl.Vc, st), "chunk transpose");
          g.b = operand(j.Et, pl.Vc, pl.D, mc, 1, 0);
        }
        g.M = pl.T; g.N = pl.D;
        g.flags = j.flags; g.flag_ld = j.flag_ld; g.flag_bn = j.flag_bn; g.flag_gen = (int)(c + 1);
      }
      CL_HIP(cl::launch_gemm(g, st), "chunk dA");
    }
    if (j.k3_epi == cl::GEMM_EPI_SGD && j.AwT != nullptr) {
      Phase ph(CUTLOSS_PHASE_CHUNK_DE, st);
      cl::SgdRowsParams s{};
      s.V = pl.V; s.v0 = v0; s.nblk = ceil_div(vlen, 32); s.D = (int)pl.D;
      s.P = j.P; s.AwT = j.AwT; s.S_u = j.S_u; s.imap = j.imap; s.E = (uint8_t*)j.E; s.lr = j.lr;
      s.sr = j.sr; s.sr_seed = j.sr_seed;
      if (j.rows_dA) {
        s.T = pl.T; s.dA_part = j.part_dA; s.dA_splits = j.dA_splits; s.dA_first = c == 0;
      }
      CL_HIP(cl::launch_sgd_rows(s, st), "chunk SGD rows");
    } else if (j.k3_epi >= 0) {
      Phase ph(CUTLOSS_PHASE_CHUNK_DE, st);
      cl::GemmParams g{};
      g.a = operand(j.P, 0, pl.Tp, mc, 0, 0, (int)pl.bt, pl.Vc / 32);
      g.b = operand(j.A_dE != nullptr ? j.A_dE : j.A, pl.D, pl.T, pl.D, 0, 0);
      // k = t over the rows the logits product wrote (T rounded up to the k stage)
      g.M = mc; g.N = pl.D; g.K = round_up(pl.T, 32); g.k_per_split = g.K;
      g.epi = j.k3_epi;
      g.v0 = v0; g.V = pl.V; g.T = pl.T; g.D = pl.D;
      g.uitems = j.uitems; g.counts = j.counts; g.S_u = j.S_u; g.imap = j.imap;
      g.dE = j.dE; g.E_inplace = (void*)j.E; g.e_fp8 = j.e_fp8; g.lr = j.lr;
      g.sr = j.sr; g.sr_seed = j.sr_seed;
      g.flags = j.flags; g.flag_ld = j.flag_ld; g.flag_bn = j.flag_bn; g.flag_gen = (int)(c + 1);
      CL_HIP(cl::launch_gemm(g, st), "chunk dE");
    }
  }
  return CUTLOSS_OK;
}

cutloss_status bce_run_chunked(const cutloss_bce_problem* p, const float* dloss, float* loss, void* dA, void* dE,
                               int dE_mode, float lr, void* ws, size_t ws_bytes, hipStream_t st, int32_t* counts,
                               int sr, uint64_t sr_seed, bool fp8_logits) {
  const bool grad = dA != nullptr || dE_mode != 0;
  const ChunkPlan pl = make_chunk_plan(p->T, p->D, p->V, p->nnz, fp8_logits, p->e_dtype == CUTLOSS_FP8_E4M3, !grad);
  const int e_fp8 = p->e_dtype == CUTLOSS_FP8_E4M3;
  const Ws2 w = carve_chunked(ws, pl, grad, dA != nullptr, dE_mode != 0, counts != nullptr, true, !e_fp8);
  CL_TRY(check_ws(ws, ws_bytes, w.bytes));
  // FP8 SGD over at most 128 rows (either rounding): whole-row updates, which also form the
  // dA partials from the E they read before updating it
  const bool sgd_rows = dE_mode == 2 && e_fp8 && w.AwT != nullptr;
  const bool rows_dA = sgd_rows && dA != nullptr && pl.sk_rows > 0;
  const int64_t n_dA = rows_dA ? cl::sgd_rows_dA_splits(ceil_div(std::min(pl.Vc, pl.V), 32), pl.D, sr) : pl.sk;
  {
    Phase ph(CUTLOSS_PHASE_TARGETS, st);
    CL_HIP(cl::launch_zero_u64(w.err, 4, st), "zero counters");
    CL_HIP(cl::launch_targets(w.tw, p->T, p->V, p->nnz, p->pos_row_ptr, p->pos_ids, p->row_mask, p->pad_id,
                              nullptr, 0, st), "targets");
  }
  if (p->T == 0) {   // no rows: dE = 0, E unchanged by the SGD step
    if (dE_mode == 1) CL_HIP(cl::launch_zero_bytes(dE, (size_t)p->V * p->D * 2, st), "zero dE");
    return CUTLOSS_OK;
  }
  cl::FinalizeParams fp{};
  fp.T = p->T; fp.D = p->D; fp.V = p->V; fp.A = p->A; fp.E = p->E; fp.e_fp8 = e_fp8;
  fp.crow = w.tw.crow; fp.cids = w.tw.cids; fp.dloss = dloss; fp.mask = p->row_mask;
  // the gradient tile holds the unweighted sigmoid: w scales dA here and A in the dE product
  fp.n_splits = (int)pl.n_splits; fp.n_splits_dA = (int)n_dA; fp.dA_weighted = 0;
  fp.part_a = w.part_a; fp.part_dA = w.part_dA; fp.loss = loss; fp.dA = dA; fp.w_out = w.w;
  fp.pos_dot = w.pos_dot; fp.pos_sum = w.pos_sum;
  fp.part_c = w.part_b; fp.counts = counts; fp.pos_tp = counts ? w.pos_tp : nullptr;
  fp.A8 = w.A8;
  {
    Phase ph(CUTLOSS_PHASE_ITEM_SUMS, st);
    if (w.A8 != nullptr) CL_HIP(cl::launch_cast_fp8((const uint16_t*)p->A, p->T * p->D, w.A8, st), "fp8 activations");
    CL_HIP(cl::launch_row_weights(fp, 0, st), "row weights");
    // positive-row terms read E before any chunk's SGD step changes it
    CL_HIP(cl::launch_row_positives(fp, st), "row positives");
    if (dE_mode != 0) {
      CL_HIP(cl::launch_item_sums(p->D, pl.cap, p->A, w.w, w.tw.csc_rows, w.tw.useg, w.tw.counts, w.S_u, w.S_part, st),
             "item sums");
      CL_HIP(cl::launch_item_map(w.tw, p->V, pl.cap, w.imap, st), "item map");
      if (sgd_rows)
        CL_HIP(cl::launch_weighted_transpose(p->A, w.w, p->T, p->D, w.AwT, st), "weighted activations");
      else
        CL_HIP(cl::launch_scale_rows(p->A, w.w, p->T, p->D, w.Aw, st), "weighted activations");
    }
  }
  ChunkJob j{};
  j.pl = &pl; j.A = p->A; j.E = p->E; j.e_fp8 = e_fp8;
  j.A_dE = dE_mode != 0 ? w.Aw : nullptr;
  j.AwT = sgd_rows ? w.AwT : nullptr;
  j.rows_dA = rows_dA;
  j.dA_splits = n_dA;
  j.k1_epi = grad ? cl::GEMM_EPI_BCE_P : (counts ? cl::GEMM_EPI_BCE_METRICS : cl::GEMM_EPI_BCE_LOSS);
  // FP8 E over at most 128 rows (BCE loss, with P or with the metrics' counts): the
  // streaming logits product
  j.rows_logits = e_fp8 && !pl.q8 && cl::logits_rows_supported(pl.Tp, p->D);
  j.w = w.w; j.P = w.P; j.part_a = w.part_a; j.part_b = w.part_b; j.part_dA = w.part_dA; j.Et = w.Et;
  j.A8 = w.A8;
  j.k3_epi = dE_mode == 0 ? -1 : (dE_mode == 1 ? cl::GEMM_EPI_DE : cl::GEMM_EPI_SGD);
  j.uitems = w.tw.uitems; j.counts = w.tw.counts; j.S_u = w.S_u; j.imap = w.imap; j.dE = dE; j.lr = lr;
  j.sr = sr; j.sr_seed = sr_seed;
  CL_TRY(run_chunks(j, st));
  if (loss != nullptr || dA != nullptr) {
    Phase ph(CUTLOSS_PHASE_FINALIZE, st);
    if (loss != nullptr) {
      CL_HIP(cl::launch_reduce_splits(w.part_a, nullptr, pl.n_splits, p->T, w.red, 0, st), "loss partials");
      if (counts != nullptr)
        CL_HIP(cl::launch_reduce_splits(w.part_b, nullptr, pl.n_splits, p->T, w.red, 0, st), "count partials");
      fp.n_splits = 1;
    }
    if (dA != nullptr) {
      CL_HIP(cl::launch_reduce_splits(w.part_dA, nullptr, n_dA, p->T * p->D, w.red, 0, st), "dA partials");
      fp.n_splits_dA = 1;
    }
    CL_HIP(cl::launch_finalize_rows(fp, 0, loss != nullptr, dA != nullptr, st), "finalize rows");
  }
  return CUTLOSS_OK;
}

cutloss_status ce_run_chunked(const cutloss_ce_problem* p, const float* lse_in, const float* dloss, float* loss,
                              float* lse, void* dA, void* dE, void* ws, size_t ws_bytes, hipStream_t st,
                              float filter_eps) {
  const bool fwd = loss != nullptr;
  const bool grad = !fwd && (dA != nullptr || dE != nullptr);
  const ChunkPlan pl = make_chunk_plan(p->T, p->D, p->V, p->T, false, p->e_dtype == CUTLOSS_FP8_E4M3, !grad);
  const int e_fp8 = p->e_dtype == CUTLOSS_FP8_E4M3;
  const Ws2 w = carve_chunked(ws, pl, grad, !fwd && dA != nullptr, !fwd && dE != nullptr, fwd, false, !e_fp8);
  CL_TRY(check_ws(ws, ws_bytes, w.bytes));
  {
    Phase ph(CUTLOSS_PHASE_TARGETS, st);
    CL_HIP(cl::launch_zero_u64(w.err, 4, st), "zero counters");
    CL_HIP(cl::launch_targets(w.tw, p->T, p->V, p->T, nullptr, nullptr, nullptr, -1, p->target, p->ignore_index, st),
           "targets");
  }
  if (p->T == 0 && !fwd && dE != nullptr) CL_HIP(cl::launch_zero_bytes(dE, (size_t)p->V * p->D * 2, st), "zero dE");
  if (p->T == 0 || (!fwd && !grad)) return CUTLOSS_OK;
  cl::FinalizeParams fp{};
  fp.T = p->T; fp.D = p->D; fp.V = p->V; fp.A = p->A; fp.E = p->E; fp.e_fp8 = e_fp8;
  fp.crow = w.tw.crow; fp.cids = w.tw.cids; fp.dloss = dloss; fp.ce_target = p->target; fp.ignore_index = p->ignore_index;
  fp.n_splits = (int)pl.n_splits; fp.n_splits_dA = (int)pl.sk; fp.dA_weighted = 1;
  fp.part_a = w.part_a; fp.part_b = w.part_b; fp.part_dA = w.part_dA;
  fp.loss = loss; fp.lse = lse; fp.dA = dA; fp.w_out = w.w; fp.lse_in = lse_in;
  ChunkJob j{};
  j.pl = &pl; j.A = p->A; j.E = p->E; j.e_fp8 = e_fp8;
  j.w = w.w; j.lse = lse_in; j.P = w.P; j.part_a = w.part_a; j.part_b = w.part_b;
  j.uitems = w.tw.uitems; j.counts = w.tw.counts; j.S_u = w.S_u; j.imap = w.imap; j.dE = dE;
  if (fwd) {
    j.k1_epi = cl::GEMM_EPI_CE_LSE;
    j.k3_epi = -1;
    CL_TRY(run_chunks(j, st));
    Phase ph(CUTLOSS_PHASE_FINALIZE, st);
    CL_HIP(cl::launch_reduce_splits(w.part_a, w.part_b, pl.n_splits, p->T, w.red, 1, st), "lse partials");
    fp.n_splits = 1;
    CL_HIP(cl::launch_finalize_rows(fp, 1, 1, 0, st), "finalize rows");
    return CUTLOSS_OK;
  }
  {
    Phase ph(CUTLOSS_PHASE_ITEM_SUMS, st);
    CL_HIP(cl::launch_row_weights(fp, 1, st), "row weights");
    if (dE != nullptr) {
      CL_HIP(cl::launch_item_sums(p->D, pl.cap, p->A, w.w, w.tw.csc_rows, w.tw.useg, w.tw.counts, w.S_u, w.S_part, st),
             "item sums");
      CL_HIP(cl::launch_item_map(w.tw, p->V, pl.cap, w.imap, st), "item map");
    }
  }
  j.k1_epi = cl::GEMM_EPI_CE_P;
  j.part_dA = w.part_dA;
  j.Et = w.Et;
  // the filtered products list at most 1024 k stages per workgroup: beyond that the call
  // runs unfiltered (exact)
  if (filter_eps > 0.0f && pl.kps / 32 <= 1024 && round_up(pl.T, 32) / 32 <= 1024) {
    j.flags = w.flags; j.flag_ld = pl.flag_ld; j.flag_bn = (int)pl.flag_bn; j.filter_eps = filter_eps;
    // chunk c flags its tiles with c + 1: flags left in a reused workspace by an earlier call
    // would match, so the region starts at 0 in every call
    CL_HIP(cl::launch_zero_bytes(w.flags, (size_t)(pl.Vc / 256) * pl.flag_ld * sizeof(int32_t), st), "zero flags");
  }
  j.k3_epi = dE != nullptr ? cl::GEMM_EPI_DE : -1;
  CL_TRY(run_chunks(j, st));
  if (dA != nullptr) {
    Phase ph(CUTLOSS_PHASE_FINALIZE, st);
    CL_HIP(cl::launch_reduce_splits(w.part_dA, nullptr, pl.sk, p->T * p->D, w.red, 0, st), "dA partials");
    fp.n_splits_dA = 1;
    CL_HIP(cl::launch_finalize_rows(fp, 1, 0, 1, st), "finalize rows");
  }
  return CUTLOSS_OK;
}

// ---- allocation-free variant of cutloss_bce_bwd: the workspace is a fixed device array of
// the library (one copy per GPU, held until the process ends)
constexpr size_t kStaticScratchBytes = 64ull << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up on the first call on
// that device. In host code the array's name stands for a host-side shadow, never for the
// device memory, so only this address is passed to kernels.
cutloss_status scratch_of_current_device(void** out) {
  int dev = 0;
  CL_HIP(hipGetDevice(&dev), "current device");
  if (dev < 0 || dev >= kMaxDevices) return fail(CUTLOSS_ERR_UNSUPPORTED, "device index %d >= %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    CL_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)), "scratch array address");
    if (ptr == nullptr) return fail(CUTLOSS_ERR_HIP, "scratch array address is NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return CUTLOSS_OK;
}

}  // namespace

extern "C" {

size_t cutloss_bce_workspace_size(const cutloss_bce_problem* p, int32_t op) {
  if (check_bce(p) != CUTLOSS_OK) return 0;
  const bool metrics = op == CUTLOSS_OP_FWD_METRICS;
  const bool bwd = op != CUTLOSS_OP_FWD && !metrics;
  if (op == CUTLOSS_OP_BWD_SGD_EX) {   // either rounding, with or without FP8 logits
    size_t b = 0;
    for (const bool q8 : {false, true}) {
      if (q8 && p->e_dtype != CUTLOSS_FP8_E4M3) continue;
      const ChunkPlan cp = make_chunk_plan(p->T, p->D, p->V, p->nnz, q8, p->e_dtype == CUTLOSS_FP8_E4M3);
      b = std::max(b, carve_chunked(nullptr, cp, true, true, true, false, true, p->e_dtype != CUTLOSS_FP8_E4M3).bytes);
    }
    return b;
  }
  if (use_chunked(p->D, p->e_dtype == CUTLOSS_FP8_E4M3)) {
    const ChunkPlan cp = make_chunk_plan(p->T, p->D, p->V, p->nnz, false, p->e_dtype == CUTLOSS_FP8_E4M3, !bwd);
    return carve_chunked(nullptr, cp, bwd, bwd, bwd, metrics, true, p->e_dtype != CUTLOSS_FP8_E4M3).bytes;
  }
  const Plan pl = make_plan(p->T, p->D, p->V, p->nnz, p->e_dtype == CUTLOSS_FP8_E4M3);
  return carve(nullptr, pl, bwd, bwd, metrics).bytes;
}

size_t cutloss_ce_workspace_size(const cutloss_ce_problem* p, int32_t op) {
  if (check_ce(p) != CUTLOSS_OK) return 0;
  const bool bwd = op != CUTLOSS_OP_FWD;
  if (use_chunked(p->D, p->e_dtype == CUTLOSS_FP8_E4M3)) {
    const ChunkPlan cp = make_chunk_plan(p->T, p->D, p->V, p->T, false, p->e_dtype == CUTLOSS_FP8_E4M3, !bwd);
    return carve_chunked(nullptr, cp, bwd, bwd, bwd, !bwd, false, p->e_dtype != CUTLOSS_FP8_E4M3).bytes;
  }
  const Plan pl = make_plan(p->T, p->D, p->V, p->T, p->e_dtype == CUTLOSS_FP8_E4M3);
  return carve(nullptr, pl, bwd, bwd, !bwd).bytes;
}

cutloss_status cutloss_bce_fwd(const cutloss_bce_problem* p, float* loss, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  CL_TRY(check_bce(p));
  CL_TRY(check_out(loss, 4, "loss", p->T > 0));
  return bce_run(p, nullptr, loss, nullptr, nullptr, 0, 0.0f, ws, ws_bytes, (hipStream_t)stream);
}

cutloss_status cutloss_bce_fwd_metrics(const cutloss_bce_problem* p, float* loss, int32_t* counts, void* ws,
                                       size_t ws_bytes, void* stream) {
  g_last_error.clear();
  CL_TRY(check_bce(p));
  CL_TRY(check_out(loss, 4, "loss", p->T > 0));
  CL_TRY(check_out(counts, 16, "counts", p->T > 0));
  if (p->V >= (int64_t)1 << 24) return fail(CUTLOSS_ERR_UNSUPPORTED, "Cut Metrics need V < 2^24 (V = %lld)", (long long)p->V);
  return bce_run(p, nullptr, loss, nullptr, nullptr, 0, 0.0f, ws, ws_bytes, (hipStream_t)stream, counts);
}

cutloss_status cutloss_bce_bwd(const cutloss_bce_problem* p, const float* dloss, void* dA, void* dE, float* loss_out,
                               void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  CL_TRY(check_bce(p));
  CL_TRY(check_out(dloss, 4, "dloss", false));
  CL_TRY(check_out(dA, 16, "dA", false));
  CL_TRY(check_out(dE, 16, "dE", false));
  CL_TRY(check_out(loss_out, 4, "loss_out", false));
  return bce_run(p, dloss, loss_out, dA, dE, dE ? 1 : 0, 0.0f, ws, ws_bytes, (hipStream_t)stream);
}

cutloss_status cutloss_bce_bwd_noalloc(const cutloss_bce_problem* p, const float* dloss, void* dA, void* dE,
                                       float* loss_out, void* stream) {
  g_last_error.clear();
  CL_TRY(check_bce(p));
  CL_TRY(check_out(dloss, 4, "dloss", false));
  CL_TRY(check_out(dA, 16, "dA", false));
  CL_TRY(check_out(dE, 16, "dE", false));
  CL_TRY(check_out(loss_out, 4, "loss_out", false));
  const size_t need = cutloss_bce_workspace_size(p, CUTLOSS_OP_BWD);
  if (need > kStaticScratchBytes)
    return fail(CUTLOSS_ERR_WORKSPACE, "problem needs %zu bytes of scratch; the allocation-free call has %zu",
                need, kStaticScratchBytes);
  void* ws = nullptr;
  CL_TRY(scratch_of_current_device(&ws));
  return bce_run(p, dloss, loss_out, dA, dE, dE ? 1 : 0, 0.0f, ws, kStaticScratchBytes, (hipStream_t)stream);
}

cutloss_status cutloss_bce_bwd_sgd(const cutloss_bce_problem* p, const float* dloss, float lr, void* dA, float* loss_out,
                                   void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  CL_TRY(check_bce(p));
  CL_TRY(check_out(dloss, 4, "dloss", false));
  CL_TRY(check_out(dA, 16, "dA", false));
  CL_TRY(check_out(loss_out, 4, "loss_out", false));
  if (!(lr == lr)) return fail(CUTLOSS_ERR_INVALID_ARG, "lr is NaN");
  return bce_run(p, dloss, loss_out, dA, nullptr, 2, lr, ws, ws_bytes, (hipStream_t)stream);
}

cutloss_status cutloss_bce_bwd_sgd_ex(const cutloss_bce_problem* p, const float* dloss, float lr,
                                      const cutloss_sgd_options* opt, void* dA, float* loss_out, void* ws,
                                      size_t ws_bytes, void* stream) {
  g_last_error.clear();
  CL_TRY(check_bce(p));
  CL_TRY(check_out(dloss, 4, "dloss", false));
  CL_TRY(check_out(dA, 16, "dA", false));
  CL_TRY(check_out(loss_out, 4, "loss_out", false));
  if (!(lr == lr)) return fail(CUTLOSS_ERR_INVALID_ARG, "lr is NaN");
  const cutloss_sgd_options o = opt != nullptr ? *opt : cutloss_sgd_options{0, 0, 0};
  if (o.rounding != CUTLOSS_ROUND_NEAREST_EVEN && o.rounding != CUTLOSS_ROUND_STOCHASTIC)
    return fail(CUTLOSS_ERR_INVALID_ARG, "rounding must be CUTLOSS_ROUND_NEAREST_EVEN or CUTLOSS_ROUND_STOCHASTIC");
  if (o.fp8_logits != 0 && o.fp8_logits != 1) return fail(CUTLOSS_ERR_INVALID_ARG, "fp8_logits must be 0 or 1");
  if (o.fp8_logits && p->e_dtype != CUTLOSS_FP8_E4M3)
    return fail(CUTLOSS_ERR_UNSUPPORTED, "FP8 logits need FP8 E");
  // the chunked products carry both options, for every head width
  return bce_run_chunked(p, dloss, loss_out, dA, nullptr, 2, lr, ws, ws_bytes, (hipStream_t)stream, nullptr,
                         o.rounding == CUTLOSS_ROUND_STOCHASTIC, o.seed, o.fp8_logits != 0);
}

cutloss_status cutloss_ce_fwd(const cutloss_ce_problem* p, float* loss, float* lse, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  CL_TRY(check_ce(p));
  CL_TRY(check_out(loss, 4, "loss", p->T > 0));
  CL_TRY(check_out(lse, 4, "lse", p->T > 0));
  return ce_run(p, nullptr, nullptr, loss, lse, nullptr, nullptr, ws, ws_bytes, (hipStream_t)stream);
}

cutloss_status cutloss_ce_bwd_filtered(const cutloss_ce_problem* p, const float* lse, const float* dloss, void* dA,
                                       void* dE, float grad_filter_eps, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  if (!(grad_filter_eps >= 0.0f) || grad_filter_eps > 1.0f)
    return fail(CUTLOSS_ERR_INVALID_ARG, "grad_filter_eps must lie in [0, 1]");
  CL_TRY(check_ce(p));
  CL_TRY(check_out(lse, 4, "lse", p->T > 0));
  CL_TRY(check_out(dloss, 4, "dloss", false));
  CL_TRY(check_out(dA, 16, "dA", false));
  CL_TRY(check_out(dE, 16, "dE", false));
  return ce_run(p, lse, dloss, nullptr, nullptr, dA, dE, ws, ws_bytes, (hipStream_t)stream, grad_filter_eps);
}

cutloss_status cutloss_ce_bwd(const cutloss_ce_problem* p, const float* lse, const float* dloss, void* dA, void* dE,
                              void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  CL_TRY(check_ce(p));
  CL_TRY(check_out(lse, 4, "lse", p->T > 0));
  CL_TRY(check_out(dloss, 4, "dloss", false));
  CL_TRY(check_out(dA, 16, "dA", false));
  CL_TRY(check_out(dE, 16, "dE", false));
  return ce_run(p, lse, dloss, nullptr, nullptr, dA, dE, ws, ws_bytes, (hipStream_t)stream);
}

cutloss_status cutloss_read_data_errors(const void* ws, void* stream, int64_t* n_errors) {
  g_last_error.clear();
  if (ws == nullptr || n_errors == nullptr) return fail(CUTLOSS_ERR_INVALID_ARG, "NULL argument");
  unsigned long long v = 0;
  CL_HIP(hipMemcpyAsync(&v, ws, sizeof(v), hipMemcpyDeviceToHost, (hipStream_t)stream), "read error counter");
  CL_HIP(hipStreamSynchronize((hipStream_t)stream), "synchronize");
  *n_errors = (int64_t)v;
  return CUTLOSS_OK;
}

cutloss_status cutloss_bce_canonical_targets(const cutloss_bce_problem* p, int32_t* crow, int32_t* cids, int32_t* items,
                                             int32_t* rows, int64_t* n_unique_pairs, void* ws, size_t ws_bytes,
                                             void* stream) {
  g_last_error.clear();
  CL_TRY(check_bce(p));
  if (crow == nullptr || n_unique_pairs == nullptr || (p->nnz > 0 && (cids == nullptr || items == nullptr || rows == nullptr)))
    return fail(CUTLOSS_ERR_INVALID_ARG, "NULL output");
  hipStream_t st = (hipStream_t)stream;
  const Plan pl = make_plan(p->T, p->D, p->V, p->nnz, p->e_dtype == CUTLOSS_FP8_E4M3);
  const Ws w = carve(ws, pl, false, false, false);
  CL_TRY(check_ws(ws, ws_bytes, w.bytes));
  CL_HIP(cl::launch_zero_u64(w.err, 4, st), "zero counters");
  CL_HIP(cl::launch_targets(w.tw, p->T, p->V, p->nnz, p->pos_row_ptr, p->pos_ids, p->row_mask, p->pad_id, nullptr, 0, st), "targets");
  int32_t n = 0;
  CL_HIP(hipMemcpyAsync(&n, w.tw.counts + 1, sizeof(n), hipMemcpyDeviceToHost, st), "copy count");
  CL_HIP(hipMemcpyAsync(crow, w.tw.crow, sizeof(int32_t) * (p->T + 1), hipMemcpyDeviceToDevice, st), "copy crow");
  CL_HIP(hipStreamSynchronize(st), "synchronize");
  if (n > 0) {
    CL_HIP(hipMemcpyAsync(cids, w.tw.cids, sizeof(int32_t) * n, hipMemcpyDeviceToDevice, st), "copy cids");
    CL_HIP(hipMemcpyAsync(items, w.tw.csc_items, sizeof(int32_t) * n, hipMemcpyDeviceToDevice, st), "copy items");
    CL_HIP(hipMemcpyAsync(rows, w.tw.csc_rows, sizeof(int32_t) * n, hipMemcpyDeviceToDevice, st), "copy rows");
    CL_HIP(hipStreamSynchronize(st), "synchronize");
  }
  *n_unique_pairs = n;
  return CUTLOSS_OK;
}

cutloss_status cutloss_bce_positive_logits(const cutloss_bce_problem* p, float* sum_x, float* x_pos,
                                           void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  CL_TRY(check_bce(p));
  if (sum_x == nullptr) return fail(CUTLOSS_ERR_INVALID_ARG, "NULL output");
  hipStream_t st = (hipStream_t)stream;
  Plan pl = make_plan(p->T, p->D, p->V, p->nnz, p->e_dtype == CUTLOSS_FP8_E4M3);
  pl.n_splits = 0;   // the canonical targets only: a prefix of every operation's workspace
  const Ws w = carve(ws, pl, false, false, false);
  CL_TRY(check_ws(ws, ws_bytes, w.bytes));
  if (p->T == 0) return CUTLOSS_OK;
  CL_HIP(cl::launch_zero_u64(w.err, 4, st), "zero counters");
  CL_HIP(cl::launch_targets(w.tw, p->T, p->V, p->nnz, p->pos_row_ptr, p->pos_ids, p->row_mask, p->pad_id, nullptr, 0, st), "targets");
  cl::FinalizeParams fp{};
  fp.T = p->T; fp.D = p->D; fp.V = p->V;
  fp.A = p->A; fp.E = p->E; fp.e_fp8 = p->e_dtype == CUTLOSS_FP8_E4M3;
  fp.crow = w.tw.crow; fp.cids = w.tw.cids;
  fp.pos_dot = sum_x; fp.pos_x = x_pos;
  CL_HIP(cl::launch_row_positives(fp, st), "row positives");
  return CUTLOSS_OK;
}

cutloss_status cutloss_profile_enable(int32_t enable) {
  std::lock_guard<std::mutex> g(g_prof_mu);
  g_prof_on = enable != 0;
  return CUTLOSS_OK;
}

cutloss_status cutloss_profile_read(float* ms, int32_t* launches, int32_t n) {
  g_last_error.clear();
  if (n < 0 || (n > 0 && (ms == nullptr || launches == nullptr))) return fail(CUTLOSS_ERR_INVALID_ARG, "bad output arrays");
  std::vector<PhaseRec> recs;
  {
    std::lock_guard<std::mutex> g(g_prof_mu);
    recs.swap(g_prof);
  }
  for (int i = 0; i < n; ++i) { ms[i] = 0.0f; launches[i] = 0; }
  cutloss_status st = CUTLOSS_OK;
  for (const PhaseRec& r : recs) {
    if (st == CUTLOSS_OK) {
      hipError_t e = hipEventSynchronize(r.b);
      float t = 0.0f;
      if (e == hipSuccess) e = hipEventElapsedTime(&t, r.a, r.b);
      if (e != hipSuccess) st = hip_check(e, "profile events");
      else if (r.phase < n) { ms[r.phase] += t; launches[r.phase] += 1; }
    }
  }
  std::lock_guard<std::mutex> g(g_prof_mu);
  for (const PhaseRec& r : recs) { g_event_pool.push_back(r.a); g_event_pool.push_back(r.b); }
  return st;
}

const char* cutloss_status_string(cutloss_status s) {
  switch (s) {
    case CUTLOSS_OK: return "ok";
    case CUTLOSS_ERR_INVALID_ARG: return "invalid argument";
    case CUTLOSS_ERR_UNSUPPORTED: return "unsupported";
    case CUTLOSS_ERR_WORKSPACE: return "workspace too small";
    case CUTLOSS_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* cutloss_last_error(void) { return g_last_error.c_str(); }

const char* cutloss_version(void) { return "cutloss 0.1.0 gfx950"; }

}  // extern "C"
