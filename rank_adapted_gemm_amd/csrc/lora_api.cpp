// C-ABI entry points: argument checks, segment scheduling and kernel launches.
//
// Scheduling follows the request model of "two 27B models on a single RTX
// 5090" (section 4): requests naming the adapter and requests naming the base
// model share one batch, and the adapter applies only to the former.  The host
// turns the caller's segment table into a compact one (empty segments dropped,
// neighbours with the same adapter merged) that every kernel receives by value.
// Row tiles that hold no adapter row skip the shrink and the expand entirely,
// so base-only rows never read A or B.
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "lora_extract.h"
#include "lora_internal.h"

namespace {

using lora::AdapterTable;
using lora::ProjArgs;
using lora::SegTable;

constexpr int64_t kMaxOperandBytes = int64_t(1) << 31;

size_t in_elem_bytes(lora_dtype d) { return d == LORA_F32 ? 4 : 2; }
size_t out_elem_bytes(lora_dtype d) { return d == LORA_BF16 ? 2 : 4; }
bool dtype_ok(int d) { return d == LORA_BF16 || d == LORA_F32 || d == LORA_BF16_F32OUT; }
bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Bytes of the intermediate s X A^T: bf16 hi + lo parts, or fp32 — 4 bytes per
// element either way, rows indexed by global row.
size_t t_bytes(int64_t M, int64_t rank) { return size_t(M) * size_t(rank) * 4; }

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + nb && b0 < a0 + na;
}

// Test hook (lora_debug_handover_fault): decode calls wait for one T group more
// than exist, with a short spin, so the failure path runs and every block exits.
std::atomic<int> g_handover_fault{0};
constexpr uint32_t kSpinLimit = 1u << 22;   // polls (about 0.3 s) before a wait for T gives up

// Byte offset of the sticky error bits in a workspace.
constexpr size_t kErrOffset = LORA_WORKSPACE_COUNTER_BYTES - 8;

// The decode path's counters (one per 128 output columns, plus three) must fit
// the workspace's counter area below the error bits.
bool decode_counters_fit(int64_t N) { return ((N + 127) / 128 + 3) * 8 <= int64_t(kErrOffset); }

// Rows of each adapter and the first virtual row tile of each, for the
// adapter-sorted shrink (the segment table is already validated).
lora::ShrinkPlan shrink_plan(const SegTable& st, int32_t n_adapters) {
  lora::ShrinkPlan sp{};
  sp.n_adapters = n_adapters;
  sp.splits = 1;
  for (int g = 0; g < st.n; ++g)
    if (st.adapter[g] >= 0) sp.rows[st.adapter[g]] += st.start[g + 1] - st.start[g];
  sp.tile_off[0] = 0;
  for (int a = 0; a < n_adapters; ++a)
    sp.tile_off[a + 1] = sp.tile_off[a] + (sp.rows[a] + lora::kShrinkRows - 1) / lora::kShrinkRows;
  return sp;
}

lora_status check_shape(int64_t M, int64_t N, int64_t K, lora_dtype dtype) {
  if (!dtype_ok(dtype)) return LORA_EUNSUPPORTED;
  if (M < 0 || N < 1 || K < 1) return LORA_EINVAL;
  if (K % 8 != 0) return LORA_EUNSUPPORTED;
  if (dtype != LORA_F32 && M <= lora::kDecodeMaxRows && !decode_counters_fit(N)) return LORA_EUNSUPPORTED;
  const int64_t ie = int64_t(in_elem_bytes(dtype)), oe = int64_t(out_elem_bytes(dtype));
  if (M * K * ie >= kMaxOperandBytes || N * K * ie >= kMaxOperandBytes || M * N * oe >= kMaxOperandBytes)
    return LORA_EUNSUPPORTED;
  return LORA_OK;
}

bool rank_ok(int64_t rank) {
  return rank >= LORA_MIN_RANK && rank <= LORA_MAX_RANK && rank % 16 == 0;
}

bool small_m(int64_t M) { return M <= lora::kDecodeMaxRows; }

// The decode split is planned for the call's rank even when no row names an
// adapter (a call without adapters may pass any rank).
int64_t plan_rank(int64_t rank) { return rank_ok(rank) ? rank : 256; }



// Workspace of a call: the decode path keeps split-K partials for W and for each
// adapter named in the batch; the prefill path keeps s X A^T (4 bytes per
// element, bf16 hi + lo or fp32) for adapter rows, indexed by global row.  T is
// `slices` x rank wide.
size_t r256(size_t x) { return (x + 255) & ~size_t(255); }

// K splits of the bf16 shrink, from the shape alone (so calls that differ only
// in how their adapters are stored sum in the same order): enough blocks to
// cover the chip when the grid of 128 x 128 tiles, estimated as
// ceil(M/128) x ceil(trank/128), is small; at most 8, each split at least 8
// stages of 64, and the partials of up to LORA_MAX_ADAPTERS adapters' tiles
// within 128 MiB.
int shrink_splits(int64_t M, int64_t K, int64_t trank) {
  const int64_t rt = lora::kShrinkRows;
  const int64_t ntn = (trank + rt - 1) / rt, ntm = (M + rt - 1) / rt;
  const int64_t tiles = std::max<int64_t>(1, ntn * ntm), nk = (K + 63) / 64;
  int64_t s = std::min<int64_t>({lora::kShrinkMaxSplits, 256 / tiles, nk / 8});
  while (s > 1 && s * ntn * (ntm + LORA_MAX_ADAPTERS) * int64_t(lora::kShrinkPartBytes) > (int64_t(128) << 20)) --s;
  return int(std::max<int64_t>(1, s));
}

// Bytes of the split shrink's partials: one per (tile, split), the tiles of
// n_used adapters bounded by ceil(trank/128) x (ceil(M/128) + n_used).
size_t part_bytes(int64_t M, int64_t K, int64_t trank, int64_t n_used) {
  const int s = shrink_splits(M, K, trank);
  if (s == 1 || n_used == 0) return 0;
  const int64_t rt = lora::kShrinkRows;
  return size_t(s) * size_t((trank + rt - 1) / rt) * size_t((M + rt - 1) / rt + n_used) * lora::kShrinkPartBytes;
}

// The prefill path's regions after the counters: T (when an adapter is
// named), the bf16 copy of 4-bit weights, then the shrink's partials.
struct PrefillLayout {
  size_t off_w, off_part, part, total;
};
PrefillLayout prefill_layout(int64_t M, int64_t N, int64_t K, int64_t rank, int64_t slices, int64_t n_used, bool q4) {
  PrefillLayout l;
  const size_t tb = n_used ? t_bytes(M, slices * rank) : 0;
  l.off_w = LORA_WORKSPACE_COUNTER_BYTES + r256(tb);
  const size_t end = q4 ? l.off_w + size_t(N) * size_t(K) * 2 : LORA_WORKSPACE_COUNTER_BYTES + tb;
  l.part = part_bytes(M, K, slices * rank, n_used);
  l.off_part = l.part ? r256(end) : end;
  l.total = l.off_part + l.part;
  return l;
}

// With 4-bit weights the prefill path also keeps a bf16 copy of W after T.
size_t need_bytes(int64_t M, int64_t N, int64_t K, int64_t rank, int64_t slices, int64_t n_used, lora_dtype dtype,
                  bool q4 = false) {
  if (dtype != LORA_F32 && small_m(M))
    return lora::decode_plan(M, N, K, plan_rank(rank), slices * plan_rank(rank), n_used).total;
  if (!q4 && !n_used) return 0;
  if (dtype == LORA_F32) return LORA_WORKSPACE_COUNTER_BYTES + t_bytes(M, slices * rank);
  return prefill_layout(M, N, K, rank, slices, n_used, q4).total;
}

// Extra checks of a call with 4-bit weights: the bf16 kernels only, K a
// multiple of the 128-wide group.
lora_status check_q4(int64_t K, lora_dtype dtype) {
  if (dtype == LORA_F32) return LORA_EUNSUPPORTED;
  if (K % 128 != 0) return LORA_EUNSUPPORTED;
  return LORA_OK;
}

// Slice table of a call: one slice of width N for a plain call; otherwise
// 2 .. LORA_MAX_SLICES positive widths, each a multiple of LORA_SLICE_ALIGN,
// summing to N.
lora_status make_slices(int32_t n_slices, const int64_t* slice_n, int64_t N, lora::Slices& sl) {
  memset(&sl, 0, sizeof(sl));
  if (n_slices < 1 || n_slices > LORA_MAX_SLICES) return LORA_EUNSUPPORTED;
  if (n_slices == 1) {
    if (slice_n && slice_n[0] != N) return LORA_EINVAL;
    sl.n = 1;
    sl.end[0] = int32_t(N);
    return LORA_OK;
  }
  if (!slice_n) return LORA_EINVAL;
  int64_t end = 0;
  for (int s = 0; s < n_slices; ++s) {
    if (slice_n[s] < 1) return LORA_EINVAL;
    if (slice_n[s] % LORA_SLICE_ALIGN != 0) return LORA_EUNSUPPORTED;
    end += slice_n[s];
    if (end > N) return LORA_EINVAL;
    sl.end[s] = int32_t(end);
  }
  if (end != N) return LORA_EINVAL;
  sl.n = n_slices;
  return LORA_OK;
}

}  // namespace

extern "C" {

const char* lora_status_string(lora_status s) {
  switch (s) {
    case LORA_OK: return "ok";
    case LORA_EINVAL: return "invalid argument (null pointer, bad size, misalignment or overlapping output)";
    case LORA_ESEGMENTS: return "malformed segment table";
    case LORA_EADAPTER: return "adapter index out of range or adapter pointer missing";
    case LORA_EUNSUPPORTED: return "shape, rank, dtype or table size outside the supported limits";
    case LORA_EWORKSPACE: return "workspace missing or too small";
    case LORA_EHIP: return "HIP runtime error while enqueueing";
    case LORA_EHANDOVER: return "a decode call on this workspace lost a hand-over between blocks (its output holds NaN)";
  }
  return "unknown status";
}

size_t lora_proj_sliced_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t rank, int32_t n_slices,
                                        int32_t n_adapters, lora_dtype dtype) {
  if (check_shape(M, N, K, dtype) != LORA_OK) return 0;
  if (n_slices < 1 || n_slices > LORA_MAX_SLICES) return 0;
  if (n_slices > 1 && N % LORA_SLICE_ALIGN != 0) return 0;
  if (n_adapters < 0 || n_adapters > LORA_MAX_ADAPTERS) return 0;
  if (n_adapters > 0 && !rank_ok(rank)) return 0;
  const int64_t n_used = std::min<int64_t>(n_adapters, std::max<int64_t>(M, 1));
  return need_bytes(M, N, K, rank, n_slices, n_used, dtype);
}

size_t lora_proj_q4_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t rank, int32_t n_slices,
                                    int32_t n_adapters, lora_dtype dtype) {
  if (check_shape(M, N, K, dtype) != LORA_OK || check_q4(K, dtype) != LORA_OK) return 0;
  if (n_slices < 1 || n_slices > LORA_MAX_SLICES) return 0;
  if (n_slices > 1 && N % LORA_SLICE_ALIGN != 0) return 0;
  if (n_adapters < 0 || n_adapters > LORA_MAX_ADAPTERS) return 0;
  if (n_adapters > 0 && !rank_ok(rank)) return 0;
  const int64_t n_used = std::min<int64_t>(n_adapters, std::max<int64_t>(M, 1));
  return need_bytes(M, N, K, rank, n_slices, n_used, dtype, true);
}

size_t lora_proj_workspace_bytes(int64_t M, int64_t N, int64_t K, int32_t rank, int32_t n_adapters,
                                 lora_dtype dtype) {
  return lora_proj_sliced_workspace_bytes(M, N, K, rank, 1, n_adapters, dtype);
}

const char* lora_proj_path(int64_t M, int64_t N, int64_t K, int32_t rank, lora_dtype dtype) {
  if (check_shape(M, N, K, dtype) != LORA_OK) return "invalid";
  (void)rank;
  if (dtype == LORA_F32) return "f32";
  return small_m(M) ? "decode" : "prefill";
}

int32_t lora_proj_tile_rows(int64_t M, int64_t N, int64_t K, lora_dtype dtype) {
  if (check_shape(M, N, K, dtype) != LORA_OK || dtype == LORA_F32 || small_m(M)) return 0;
  return lora::main_tile_rows(int(M), int(N));
}

}  // extern "C"

namespace {

// One call.  scales[a] is adapter a's scale; when scales is NULL every adapter
// uses `scale`.  n_slices / slice_n cut the output columns into slices (NULL
// and 1 for a plain call).  WP non-null: W holds 4-bit codes and WP their
// params words (lora_proj_q4).
lora_status run_call(const void* X, const int32_t* seg_starts, const int32_t* seg_adapter, int32_t n_seg,
                     const void* W, const void* const* A, const void* const* B, int32_t n_adapters, int32_t rank,
                     const float* scales, float scale, int32_t n_slices, const int64_t* slice_n, void* Y,
                     int64_t M, int64_t N, int64_t K, lora_dtype dtype, void* workspace, size_t workspace_bytes,
                     hipStream_t stream, hipEvent_t main_start, hipEvent_t main_stop, const void* WP = nullptr,
                     bool clear_counters = false, const int32_t* ranks = nullptr) {
  lora_status st = check_shape(M, N, K, dtype);
  if (st != LORA_OK) return st;
  const bool q4 = WP != nullptr;
  if (q4 && (st = check_q4(K, dtype)) != LORA_OK) return st;
  lora::Slices sl;
  st = make_slices(n_slices, slice_n, N, sl);
  if (st != LORA_OK) return st;
  if (M == 0) return LORA_OK;
  if (!X || !W || !Y || !aligned16(X) || !aligned16(W) || !aligned16(Y)) return LORA_EINVAL;
  if (q4 && !aligned16(WP)) return LORA_EINVAL;
  if (n_adapters < 0) return LORA_EINVAL;
  if (n_adapters > LORA_MAX_ADAPTERS) return LORA_EUNSUPPORTED;
  if (n_adapters > 0 && (!A || !B)) return LORA_EINVAL;

  // ---- segment table: validate, drop empty segments, merge equal neighbours
  if (!seg_starts || !seg_adapter || n_seg < 1) return LORA_ESEGMENTS;
  if (seg_starts[0] != 0 || int64_t(seg_starts[n_seg]) != M) return LORA_ESEGMENTS;
  SegTable tbl;
  memset(&tbl, 0, sizeof(tbl));
  tbl.n = 0;
  bool used[LORA_MAX_ADAPTERS] = {};
  int64_t adapter_rows = 0;
  for (int32_t g = 0; g < n_seg; ++g) {
    const int32_t lo = seg_starts[g], hi = seg_starts[g + 1];
    if (hi < lo) return LORA_ESEGMENTS;
    const int32_t a = seg_adapter[g];
    if (a < -1 || a >= n_adapters) return LORA_EADAPTER;
    if (hi == lo) continue;
    if (a >= 0) {
      used[a] = true;
      adapter_rows += hi - lo;
    }
    if (tbl.n > 0 && tbl.adapter[tbl.n - 1] == a) {
      tbl.start[tbl.n] = hi;             // extend the previous segment
      continue;
    }
    if (tbl.n == LORA_MAX_SEGMENTS) return LORA_EUNSUPPORTED;
    tbl.start[tbl.n] = lo;
    tbl.adapter[tbl.n] = int8_t(a);
    ++tbl.n;
    tbl.start[tbl.n] = hi;
  }

  // ---- adapters named by non-empty segments, each at its own rank (ranks
  // NULL: every adapter at `rank`); from here on `rank` is the largest of them
  const bool has_adapter = adapter_rows > 0;
  const size_t ie = in_elem_bytes(dtype), oe = out_elem_bytes(dtype);
  AdapterTable at;
  memset(&at, 0, sizeof(at));
  if (has_adapter) {
    int32_t rmax = 0;
    for (int a = 0; a < n_adapters; ++a) {
      if (!used[a]) continue;
      const int32_t ra = ranks ? ranks[a] : rank;
      if (!rank_ok(ra)) return LORA_EUNSUPPORTED;
      const size_t ab = size_t(ra) * size_t(sl.n) * size_t(K) * ie, bb = size_t(N) * size_t(ra) * ie;
      if (int64_t(ab) >= kMaxOperandBytes || int64_t(bb) >= kMaxOperandBytes) return LORA_EUNSUPPORTED;
      if (!A[a] || !B[a]) return LORA_EADAPTER;
      if (!aligned16(A[a]) || !aligned16(B[a])) return LORA_EINVAL;
      at.A[a] = A[a];
      at.B[a] = B[a];
      at.scale[a] = scales ? scales[a] : scale;
      at.rank[a] = ra;
      at.a_bytes[a] = uint32_t(ab);
      at.b_bytes[a] = uint32_t(bb);
      rmax = ra > rmax ? ra : rmax;
    }
    rank = rmax;
  }

  // ---- workspace
  int n_used = 0;
  int8_t slot_of[LORA_MAX_ADAPTERS];
  int8_t slot_adapter[LORA_MAX_ADAPTERS] = {};
  for (int a = 0; a < LORA_MAX_ADAPTERS; ++a) slot_of[a] = -1;
  for (int a = 0; a < n_adapters; ++a)
    if (used[a]) {
      slot_of[a] = int8_t(n_used);
      slot_adapter[n_used++] = int8_t(a);
    }
  const bool decode = dtype != LORA_F32 && small_m(M);
  const size_t need = need_bytes(M, N, K, rank, sl.n, n_used, dtype, q4);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return LORA_EWORKSPACE;
    if (!aligned16(workspace)) return LORA_EINVAL;
    if (int64_t(need) >= kMaxOperandBytes) return LORA_EUNSUPPORTED;
  }

  // ---- the output may not overlap anything the call reads or the workspace
  const size_t y_bytes = size_t(M) * size_t(N) * oe;
  const size_t x_bytes = size_t(M) * size_t(K) * ie;
  const size_t w_bytes = q4 ? size_t(N) * size_t(K) / 2 : size_t(N) * size_t(K) * ie;
  const size_t wp_bytes = q4 ? size_t(K / 128) * size_t(N) * 4 : 0;
  if (overlaps(Y, y_bytes, X, x_bytes) || overlaps(Y, y_bytes, W, w_bytes)) return LORA_EINVAL;
  if (q4 && (overlaps(Y, y_bytes, WP, wp_bytes) || (need > 0 && overlaps(WP, wp_bytes, workspace, need))))
    return LORA_EINVAL;
  if (need > 0 && (overlaps(Y, y_bytes, workspace, need) || overlaps(X, x_bytes, workspace, need) ||
                   overlaps(W, w_bytes, workspace, need)))
    return LORA_EINVAL;
  if (has_adapter) {
    for (int a = 0; a < n_adapters; ++a) {
      if (!used[a]) continue;
      const size_t ab = at.a_bytes[a], bb = at.b_bytes[a];
      if (overlaps(Y, y_bytes, A[a], ab) || overlaps(Y, y_bytes, B[a], bb)) return LORA_EINVAL;
      if (overlaps(workspace, need, A[a], ab) || overlaps(workspace, need, B[a], bb)) return LORA_EINVAL;
    }
  }

  ProjArgs p;
  p.X = X;
  p.W = W;
  p.Y = Y;
  p.T = has_adapter && !decode ? static_cast<char*>(workspace) + LORA_WORKSPACE_COUNTER_BYTES : nullptr;
  p.M = int32_t(M);
  p.N = int32_t(N);
  p.K = int32_t(K);
  p.rank = has_adapter ? rank : 0;
  p.trank = p.rank * sl.n;
  p.sl = sl;
  p.x_bytes = uint32_t(x_bytes);
  p.w_bytes = uint32_t(w_bytes);
  p.y_bytes = uint32_t(y_bytes);
  p.t_bytes = has_adapter && !decode ? uint32_t(t_bytes(M, int64_t(rank) * sl.n)) : 0u;

  hipError_t e = hipSuccess;
  if (decode) {
    const lora::DecodePlan pl = lora::decode_plan(M, N, K, plan_rank(rank), sl.n * plan_rank(rank), n_used);
    lora::DecodeArgs d;
    memset(&d, 0, sizeof(d));
    char* ws = static_cast<char*>(workspace);
    d.X = X;
    d.W = W;
    d.WP = WP;
    d.wp_bytes = uint32_t(wp_bytes);
    d.Y = Y;
    d.cnt = reinterpret_cast<unsigned long long*>(ws + pl.off_cnt);
    d.err = reinterpret_cast<uint32_t*>(ws + kErrOffset);
    d.PA = reinterpret_cast<float*>(ws + pl.off_pa);
    d.PW = reinterpret_cast<float*>(ws + pl.off_pw);
    d.TH = reinterpret_cast<uint16_t*>(ws + pl.off_th);
    d.TL = reinterpret_cast<uint16_t*>(ws + pl.off_tl);
    d.x_bytes = uint32_t(x_bytes);
    d.w_bytes = uint32_t(w_bytes);
    d.y_bytes = uint32_t(y_bytes);
    d.t_bytes = uint32_t(pl.t_bytes);
    d.pa_bytes = uint32_t(pl.pa_bytes);
    d.ranks_differ = 0;
    for (int a = 0; a < n_adapters; ++a)
      if (used[a] && at.rank[a] != rank) d.ranks_differ = 1;
    d.a_bytes = has_adapter ? uint32_t(size_t(rank) * size_t(sl.n) * size_t(K) * ie) : 0u;
    d.b_bytes = has_adapter ? uint32_t(size_t(N) * size_t(rank) * ie) : 0u;
    d.pw_bytes = uint32_t(pl.pw_bytes);
    d.M = int32_t(M);
    d.N = int32_t(N);
    d.K = int32_t(K);
    d.rank = int32_t(plan_rank(rank));
    d.trank = d.rank * sl.n;
    d.sl = sl;
    d.nst = pl.nst;
    d.nrs = pl.nrs;
    d.n_used = pl.n_used;
    d.ntA = pl.ntA;
    d.ntW = pl.ntW;
    d.GA = pl.GA;
    d.GW = pl.GW;
    d.smaxW = pl.smaxW;
    d.spin_limit = kSpinLimit;
    d.fault = g_handover_fault.load(std::memory_order_relaxed);
    for (int g = 0; g < tbl.n; ++g)
      for (int32_t m = tbl.start[g]; m < tbl.start[g + 1]; ++m)
        d.row_slot[m] = tbl.adapter[g] < 0 ? int8_t(-1) : slot_of[tbl.adapter[g]];
    for (int i = 0; i < n_used; ++i) d.slot_adapter[i] = slot_adapter[i];
    if (clear_counters)   // every check has passed: from here on the call launches
      e = lora::launch_clear_words(reinterpret_cast<uint32_t*>(ws), int(LORA_WORKSPACE_COUNTER_BYTES / 4), stream);
    if (e == hipSuccess)
      e = lora::launch_decode(d, at, pl.MT, dtype == LORA_BF16_F32OUT, stream, main_start, main_stop);
  } else if (dtype == LORA_F32) {
    if (has_adapter) e = lora::launch_f32_shrink(p, tbl, at, stream);
    if (e == hipSuccess) e = lora::launch_f32_main(p, tbl, at, has_adapter, stream, main_start, main_stop);
  } else {
    const PrefillLayout lay = prefill_layout(M, N, K, rank, sl.n, n_used, q4);
    if (q4) {   // expand the 4-bit weights into a bf16 copy after T, then run the bf16 kernels
      char* wcopy = static_cast<char*>(workspace) + lay.off_w;
      e = lora::launch_q4_dequant(W, WP, wcopy, N, K, stream);
      p.W = wcopy;
      p.w_bytes = uint32_t(size_t(N) * size_t(K) * 2);
    }
    if (e == hipSuccess && has_adapter) {
      lora::ShrinkPlan sp = shrink_plan(tbl, n_adapters);
      sp.splits = lay.part ? shrink_splits(M, K, p.trank) : 1;
      sp.part = lay.part ? static_cast<char*>(workspace) + lay.off_part : nullptr;
      sp.part_bytes = uint32_t(lay.part);
      e = lora::launch_bf16_shrink(p, tbl, at, sp, stream);
    }
    if (e == hipSuccess)
      e = lora::launch_bf16_main(p, tbl, at, has_adapter, dtype == LORA_BF16_F32OUT, stream, main_start, main_stop);
  }
  return e == hipSuccess ? LORA_OK : LORA_EHIP;
}

}  // namespace

extern "C" {

lora_status lora_proj_ex(const void* X,
                         const int32_t* seg_starts, const int32_t* seg_adapter, int32_t n_seg,
                         const void* W,
                         const void* const* A, const void* const* B,
                         int32_t n_adapters, int32_t rank, float scale,
                         void* Y,
                         int64_t M, int64_t N, int64_t K,
                         lora_dtype dtype,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream,
                         hipEvent_t main_start, hipEvent_t main_stop) {
  return run_call(X, seg_starts, seg_adapter, n_seg, W, A, B, n_adapters, rank, nullptr, scale, 1, nullptr, Y, M, N,
                  K, dtype, workspace, workspace_bytes, stream, main_start, main_stop);
}

lora_status lora_proj(const void* X,
                      const int32_t* seg_starts, const int32_t* seg_adapter, int32_t n_seg,
                      const void* W,
                      const void* const* A, const void* const* B,
                      int32_t n_adapters, int32_t rank, float scale,
                      void* Y,
                      int64_t M, int64_t N, int64_t K,
                      lora_dtype dtype,
                      void* workspace, size_t workspace_bytes,
                      hipStream_t stream) {
  return run_call(X, seg_starts, seg_adapter, n_seg, W, A, B, n_adapters, rank, nullptr, scale, 1, nullptr, Y, M, N,
                  K, dtype, workspace, workspace_bytes, stream, nullptr, nullptr);
}

lora_status lora_proj_multi(const void* X,
                            const int32_t* seg_starts, const int32_t* seg_adapter, int32_t n_seg,
                            const void* W,
                            const void* const* A, const void* const* B,
                            int32_t n_adapters, int32_t rank, const float* scales,
                            void* Y,
                            int64_t M, int64_t N, int64_t K,
                            lora_dtype dtype,
                            void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  if (n_adapters > 0 && !scales) return LORA_EINVAL;
  return run_call(X, seg_starts, seg_adapter, n_seg, W, A, B, n_adapters, rank, scales, 0.0f, 1, nullptr, Y, M, N, K,
                  dtype, workspace, workspace_bytes, stream, nullptr, nullptr);
}

lora_status lora_proj_q4(const void* X,
                         const int32_t* seg_starts, const int32_t* seg_adapter, int32_t n_seg,
                         const void* Wq, const void* Wp,
                         const void* const* A, const void* const* B,
                         int32_t n_adapters, int32_t rank, const float* scales,
                         int32_t n_slices, const int64_t* slice_n,
                         void* Y,
                         int64_t M, int64_t N, int64_t K,
                         lora_dtype dtype,
                         void* workspace, size_t workspace_bytes,
                         hipStream_t stream) {
  if (!Wp) return LORA_EINVAL;
  if (n_adapters > 0 && !scales) return LORA_EINVAL;
  return run_call(X, seg_starts, seg_adapter, n_seg, Wq, A, B, n_adapters, rank, scales, 0.0f, n_slices, slice_n, Y,
                  M, N, K, dtype, workspace, workspace_bytes, stream, nullptr, nullptr, Wp);
}

lora_status lora_proj_sliced(const void* X,
                             const int32_t* seg_starts, const int32_t* seg_adapter, int32_t n_seg,
                             const void* W,
                             const void* const* A, const void* const* B,
                             int32_t n_adapters, int32_t rank, const float* scales,
                             int32_t n_slices, const int64_t* slice_n,
                             void* Y,
                             int64_t M, int64_t N, int64_t K,
                             lora_dtype dtype,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  if (n_adapters > 0 && !scales) return LORA_EINVAL;
  return run_call(X, seg_starts, seg_adapter, n_seg, W, A, B, n_adapters, rank, scales, 0.0f, n_slices, slice_n, Y,
                  M, N, K, dtype, workspace, workspace_bytes, stream, nullptr, nullptr);
}

lora_status lora_proj_ranked(const void* X,
                             const int32_t* seg_starts, const int32_t* seg_adapter, int32_t n_seg,
                             const void* W,
                             const void* const* A, const void* const* B,
                             int32_t n_adapters, const int32_t* ranks, const float* scales,
                             int32_t n_slices, const int64_t* slice_n,
                             void* Y,
                             int64_t M, int64_t N, int64_t K,
                             lora_dtype dtype,
                             void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  if (n_adapters > 0 && (!scales || !ranks)) return LORA_EINVAL;
  return run_call(X, seg_starts, seg_adapter, n_seg, W, A, B, n_adapters, LORA_MIN_RANK, scales, 0.0f, n_slices,
                  slice_n, Y, M, N, K, dtype, workspace, workspace_bytes, stream, nullptr, nullptr, nullptr, false,
                  ranks);
}

}  // extern "C"

namespace {

bool extract_args_ok(int64_t N, int64_t K, int32_t l, int32_t rank, int32_t power_iters) {
  return N >= 1 && K >= 1 && rank >= 1 && l >= rank && l <= 512 && l % 2 == 0 && l <= std::min(N, K) &&
         power_iters >= 0 && power_iters <= 8 && N * K * 4 < (int64_t(1) << 36);
}

}  // namespace

extern "C" {

size_t lora_extract_workspace_bytes(int64_t N, int64_t K, int32_t l, int32_t rank) {
  if (!extract_args_ok(N, K, l, rank, 0)) return 0;
  return lora::extract_workspace_bytes(N, K, l, rank);
}

lora_status lora_extract(const void* W_adapted, const void* W_base, int64_t N, int64_t K,
                         const float* omega, int32_t l, int32_t rank, int32_t power_iters,
                         float* B, float* A, float* sigma,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (N < 1 || K < 1) return LORA_EINVAL;
  if (!extract_args_ok(N, K, l, rank, power_iters)) return LORA_EUNSUPPORTED;
  const void* ptrs[] = {W_adapted, W_base, omega, B, A, sigma};
  for (const void* p : ptrs)
    if (!p || !aligned16(p)) return LORA_EINVAL;
  const size_t need = lora::extract_workspace_bytes(N, K, l, rank);
  if (!workspace || workspace_bytes < need) return LORA_EWORKSPACE;
  if (!aligned16(workspace)) return LORA_EINVAL;
  const size_t w = size_t(N) * size_t(K) * 2;
  const size_t outs[] = {size_t(N) * size_t(rank) * 4, size_t(rank) * size_t(K) * 4, size_t(rank) * 4};
  const void* out_ptrs[] = {B, A, sigma};
  const void* in_ptrs[] = {W_adapted, W_base, omega};
  const size_t ins[] = {w, w, size_t(K) * size_t(l) * 4};
  for (int i = 0; i < 3; ++i) {
    if (overlaps(workspace, need, in_ptrs[i], ins[i]) || overlaps(workspace, need, out_ptrs[i], outs[i]))
      return LORA_EINVAL;
    for (int j = 0; j < 3; ++j)
      if (overlaps(out_ptrs[i], outs[i], in_ptrs[j], ins[j]) || (i != j && overlaps(out_ptrs[i], outs[i], out_ptrs[j], outs[j])))
        return LORA_EINVAL;
  }
  const hipError_t e = lora::launch_extract(W_adapted, W_base, N, K, omega, l, rank, power_iters, B, A, sigma,
                                            workspace, stream);
  return e == hipSuccess ? LORA_OK : LORA_EHIP;
}

}  // extern "C"

extern "C" {

lora_status lora_workspace_status(void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!workspace || !aligned16(workspace) || workspace_bytes < LORA_WORKSPACE_COUNTER_BYTES) return LORA_EINVAL;
  uint32_t bits = 0;
  if (hipMemcpyAsync(&bits, static_cast<char*>(workspace) + kErrOffset, sizeof(bits), hipMemcpyDeviceToHost,
                     stream) != hipSuccess)
    return LORA_EHIP;
  if (hipStreamSynchronize(stream) != hipSuccess) return LORA_EHIP;
  if (bits == 0) return LORA_OK;
  // a call lost a hand-over: its counts may be anywhere, so restore the whole area
  if (lora::launch_clear_words(static_cast<uint32_t*>(workspace), int(LORA_WORKSPACE_COUNTER_BYTES / 4), stream) !=
          hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return LORA_EHIP;
  return LORA_EHANDOVER;
}

int32_t lora_debug_handover_fault(int32_t on) { return g_handover_fault.exchange(on ? 1 : 0); }

}  // extern "C"

extern "C" {

int32_t lora_decode_plan_describe(int64_t M, int64_t N, int64_t K, int32_t rank, int32_t n_slices,
                                  const int64_t* slice_n, int32_t n_used, int64_t* out, int32_t n_out) {
  if (check_shape(M, N, K, LORA_BF16) != LORA_OK || M < 1 || !small_m(M) || !out) return 0;
  if (n_used < 0 || n_used > LORA_MAX_ADAPTERS || (n_used > 0 && !rank_ok(rank))) return 0;
  lora::Slices sl;
  if (make_slices(n_slices, slice_n, N, sl) != LORA_OK) return 0;
  const int64_t r = plan_rank(rank);
  const lora::DecodePlan p = lora::decode_plan(M, N, K, r, sl.n * r, n_used);
  const int64_t v[] = {p.MT, p.nst, p.nrs, p.ntA, p.ntW, p.n_used, p.GA, p.GW, p.smaxW,
                       int64_t(p.off_cnt), int64_t(p.off_pa), int64_t(p.pa_bytes), int64_t(p.off_pw),
                       int64_t(p.pw_bytes), int64_t(p.off_th), int64_t(p.t_bytes), int64_t(p.off_tl),
                       int64_t(p.total)};
  const int32_t n = int32_t(sizeof(v) / sizeof(v[0]));
  for (int32_t i = 0; i < n && i < n_out; ++i) out[i] = v[i];
  return n;
}

}  // extern "C"

// ------------------------------------------------------------------ no allocation
// The entry point for callers that cannot allocate (code under graph capture,
// tight serving loops): its workspace is a fixed array in device memory, one
// copy per GPU, held from the library's load until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device copy: the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current.
static __device__ __align__(256) char scratch[LORA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch[kMaxDevices] = {};

// The current device's copy of `scratch` (null on a runtime error).
void* scratch_of_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_scratch[dev] = p;
  }
  return g_scratch[dev];
}

}  // namespace

extern "C" {

lora_status lora_proj_noalloc(const void* X,
                              const int32_t* seg_starts, const int32_t* seg_adapter, int32_t n_seg,
                              const void* W,
                              const void* const* A, const void* const* B,
                              int32_t n_adapters, int32_t rank, float scale,
                              void* Y,
                              int64_t M, int64_t N, int64_t K,
                              lora_dtype dtype,
                              hipStream_t stream) {
  void* ws = scratch_of_current_device();
  if (!ws) return LORA_EHIP;
  // the decode path's counters start from zero on every call: a failed earlier
  // call on this GPU cannot leave counts behind for this one
  return run_call(X, seg_starts, seg_adapter, n_seg, W, A, B, n_adapters, rank, nullptr, scale, 1, nullptr, Y, M, N,
                  K, dtype, ws, LORA_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr, nullptr, true);
}

}  // extern "C"
