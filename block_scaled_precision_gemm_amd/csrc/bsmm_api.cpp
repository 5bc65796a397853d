// Host front end of libbsmm: argument validation, plan selection and the C
// entry points declared in include/bsmm.h.  Everything here runs on the host
// before any HIP call, so every error path is testable without a GPU.

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "bsmm.h"
#include "bsmm_internal.h"
#include "bsmm_tuned.h"

namespace bsmm {
namespace {

thread_local char g_err[512] = "";

bsmm_status fail(bsmm_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

// ---- override (tests / tuning) and logging --------------------------------
// The environment is read once; after that the planning path takes no lock
// unless a variant or split is forced: `active` says whether one is, and
// `gen` changes on every setter call so that cached plans made under an
// earlier setting are not reused.
struct Override {
  std::mutex mu;                    // guards `variant`, `split` and the tail fields
  std::string variant;
  int split = 0;
  int m_split = 0;                  // forced M-split point (0: none)
  std::string m_tail;               // and its tail launch's kernel and K slices
  int m_tail_split = 1;
  std::atomic<int> active{0};       // a variant or split is forced
  std::atomic<unsigned> gen{1};     // bumped by every setter call
  std::atomic<int> sk_grid{0};      // stream-K grid (0: co-resident capacity)
  int log = 0;
  int tail_split_cap = 0;          // BSMM_TAIL_SPLIT: cap on the tail launch's K slices
  std::string tail_variant;        // BSMM_TAIL_VARIANT: kernel of the tail launch
};
Override& ovr() {
  static Override o;
  return o;
}
void read_env_once() {
  static std::once_flag once;
  std::call_once(once, [] {
    Override& o = ovr();
    std::lock_guard<std::mutex> g(o.mu);
    if (const char* v = getenv("BSMM_FORCE_VARIANT")) o.variant = v;
    if (const char* v = getenv("BSMM_FORCE_SPLITK")) o.split = atoi(v);
    if (const char* v = getenv("BSMM_LOG")) o.log = atoi(v);
    if (const char* v = getenv("BSMM_TAIL_SPLIT")) o.tail_split_cap = atoi(v);
    if (const char* v = getenv("BSMM_TAIL_VARIANT")) o.tail_variant = v;
    o.active.store(!o.variant.empty() || o.split > 0, std::memory_order_release);
  });
}

// Per-thread cache of recent plans, keyed by the problem, the workspace
// size and the override generation: a repeated call (a decode loop) skips
// the table search and the heuristic.  Direct-mapped, no allocation.
struct PlanKey {
  int op, dt, G, M, N, K;
  size_t ws;
  unsigned gen;
  bool operator==(const PlanKey& o) const {
    return op == o.op && dt == o.dt && G == o.G && M == o.M && N == o.N && K == o.K &&
           ws == o.ws && gen == o.gen;
  }
};
struct PlanSlot {
  PlanKey key{-1, -1, 0, 0, 0, 0, 0, 0};
  Plan plan;
};
constexpr int kPlanCache = 16;
thread_local PlanSlot t_plans[kPlanCache];
unsigned plan_hash(const PlanKey& k) {
  uint64_t h = (uint64_t)k.op * 0x9E3779B97F4A7C15ull;
  for (uint64_t v : {(uint64_t)k.dt, (uint64_t)k.G, (uint64_t)k.M, (uint64_t)k.N,
                     (uint64_t)k.K, (uint64_t)k.ws})
    h = (h ^ v) * 0x100000001B3ull;
  return (unsigned)(h >> 32) % kPlanCache;
}

constexpr int64_t kMaxDim = (int64_t)1 << 31;
constexpr int64_t kMaxLd = (int64_t)1 << 23;    // 256 rows * ld + K < 2^32
constexpr int64_t kMaxInt8K = 130944;           // largest multiple of 128 below 2^31 / 2^14

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

const char* op_name(bsmm_op op) {
  switch (op) {
    case BSMM_OP_INT8_ROWWISE: return "int8_rowwise";
    case BSMM_OP_FP8_BLOCKWISE: return "fp8_blockwise";
    case BSMM_OP_FP8_SCALED_MM: return "fp8_scaled_mm";
    case BSMM_OP_FP8_MX32_MM: return "fp8_mx32_mm";
    case BSMM_OP_FP8_GROUPWISE: return "fp8_groupwise";
    default: return "fp8_mx_bmm";
  }
}

}  // namespace

const Variant* find_variant(const char* name) {
  int n = 0;
  const Variant* v = variants(&n);
  for (int i = 0; i < n; ++i)
    if (strcmp(v[i].name, name) == 0) return &v[i];
  return nullptr;
}

size_t splitk_workspace(const Problem& p, int rows, int split) {
  if (split <= 1) return 0;
  return (size_t)split * (size_t)p.G * (size_t)rows * (size_t)p.N * 4u;
}

static size_t ws_bytes(int G, int rows, int N, int split) {
  if (split <= 1) return 0;
  return (size_t)split * (size_t)G * (size_t)rows * (size_t)N * 4u;
}

size_t persistent_workspace(const Variant* v, bsmm_op op) {
  (void)op;   // int32 and fp32 partials are both 4 bytes
  return (size_t)kPlanCUs * v->wg_per_cu * 2 * ((size_t)v->tile_m * v->tile_n * 4u + 8u);
}

static bool plan_packed(const Plan& pl, bsmm_op op) {
  return packable_scales(op) &&
         (pl.v->packed_scales || (pl.tail && pl.tail->packed_scales));
}

// Workspace of a plan: packed scale_a (packed-scale variants), then the
// split-K partials or stream-K slots of the bulk launch or of the tail
// launch (they run one after the other on the stream and share the space).
static size_t plan_ws(const Plan& pl, bsmm_op op, int G, int M, int N, int K) {
  const size_t pack = plan_packed(pl, op) ? packed_scale_bytes(op, G, M, K, N) : 0;
  const int rows = pl.m_split ? pl.m_split : M;
  auto launch_ws = [&](const Variant* v, int r, int split) {
    if (v->persistent) return persistent_workspace(v, op);
    if (v->kind == 3 || v->kind == 4) return narrow_workspace(G, N, v->tile_n, split);
    return ws_bytes(G, r, N, split);
  };
  size_t main = launch_ws(pl.v, rows, pl.split);
  if (pl.tail && pl.m_split) {
    const size_t t = launch_ws(pl.tail, M - pl.m_split, pl.tail_split);
    if (t > main) main = t;
  }
  return pack + main;
}

// Shrink a plan until its workspace fits: drop split-K, then the stream-K
// slots, then the packed scales.
static void fit_workspace(Plan& pl, bsmm_op op, int G, int M, int N, int K, bsmm_dtype dt,
                          size_t workspace_bytes) {
  pl.workspace = plan_ws(pl, op, G, M, N, K);
  if (pl.workspace <= workspace_bytes) return;
  pl.split = 1;
  pl.tail_split = 1;
  pl.workspace = plan_ws(pl, op, G, M, N, K);
  if (pl.workspace <= workspace_bytes) return;
  if (pl.v->persistent) {
    Plan h = make_plan_heuristic(op, G, M, N, K, dt);
    pl.v = h.v;
    pl.tail = h.tail;
    pl.m_split = h.m_split;
    pl.split = 1;
    pl.tail_split = 1;
    pl.workspace = plan_ws(pl, op, G, M, N, K);
    if (pl.workspace <= workspace_bytes) return;
  }
  if (pl.v->packed_scales && pl.v->unpacked) pl.v = find_variant(pl.v->unpacked);
  if (pl.tail && pl.tail->packed_scales && pl.tail->unpacked) pl.tail = find_variant(pl.tail->unpacked);
  pl.workspace = plan_ws(pl, op, G, M, N, K);
}

// Plan selection (bsmm_plan_info::source):
//  0  exact hit in the tuned table for (op, out dtype, G, N, K, M);
//  1  padded-M: the nearest tuned M bucket above M for the same (op, dtype,
//     G, N, K), run at the real M (every variant masks rows past M);
//  2  heuristic: tile by M; split-K when the grid would underfill the chip
//     and K is long compared with the tile (the "K much larger than m, n and
//     m, n small" rule of Inductor's use_decompose_k_choice); an M-split into
//     a tile-aligned bulk plus a short tail when the bulk work G*M_bulk is
//     at least 8192 rows (the break-even the aiter PR's dispatch uses);
//  3  override.
// A plan whose workspace exceeds workspace_bytes falls back to split 1.
static Plan make_plan_uncached(bsmm_op op, int G, int M, int N, int K, bsmm_dtype dt,
                               size_t workspace_bytes);

Plan make_plan(bsmm_op op, int G, int M, int N, int K, bsmm_dtype dt,
               size_t workspace_bytes) {
  read_env_once();
  Override& o = ovr();
  if (o.active.load(std::memory_order_acquire))
    return make_plan_uncached(op, G, M, N, K, dt, workspace_bytes);
  const PlanKey key{(int)op, (int)dt, G, M, N, K, workspace_bytes,
                    o.gen.load(std::memory_order_acquire)};
  PlanSlot& slot = t_plans[plan_hash(key)];
  if (slot.key == key) return slot.plan;
  slot.plan = make_plan_uncached(op, G, M, N, K, dt, workspace_bytes);
  slot.key = key;
  return slot.plan;
}

static Plan make_plan_uncached(bsmm_op op, int G, int M, int N, int K, bsmm_dtype dt,
                               size_t workspace_bytes) {
  Plan pl;
  const int KB = K / kBlockK;
  {
    Override& o = ovr();
    std::lock_guard<std::mutex> g(o.mu);
    if (!o.variant.empty() || o.split > 0 || o.m_split > 0) {
      Plan h = make_plan_heuristic(op, G, M, N, K, dt);
      const Variant* v = o.variant.empty() ? h.v : find_variant(o.variant.c_str());
      if (!v || (v->max_m && M > v->max_m)) v = h.v;
      pl.v = v;
      pl.split = o.split > 0 ? o.split : (o.variant.empty() ? h.split : 1);
      if (pl.split > KB) pl.split = KB > 0 ? KB : 1;
      // a forced M-split: bulk rows [0, m_split) on the main kernel, the rest
      // on the tail kernel (packed-scale kernels start on a 64-row boundary)
      const Variant* tv = o.m_tail.empty() ? nullptr : find_variant(o.m_tail.c_str());
      if (o.m_split > 0 && o.m_split < M && o.m_split % 64 == 0 && tv && !tv->max_m &&
          !pl.v->max_m) {
        pl.m_split = o.m_split;
        pl.tail = tv;
        pl.tail_split = o.m_tail_split > 0 ? o.m_tail_split : 1;
        if (pl.tail_split > KB) pl.tail_split = KB > 0 ? KB : 1;
        if (tv->persistent) pl.tail_split = 1;
      }
      pl.source = 3;
      if (pl.v->persistent || pl.v->kind == 2) pl.split = 1;   // no split-K in these kernels
      fit_workspace(pl, op, G, M, N, K, dt, workspace_bytes);
      return pl;
    }
  }
  const TunedEntry* best = nullptr;
  int ntab = 0;
  const TunedEntry* tab = tuned_table(&ntab);
  for (int i = 0; i < ntab; ++i) {
    const TunedEntry& e = tab[i];
    if (e.op != (int)op || e.out_dtype != (int)dt || e.G != G || e.N != N || e.K != K)
      continue;
    if (e.M == M) { best = &e; pl.source = 0; break; }
    if (e.M > M && (!best || e.M < best->M)) { best = &e; pl.source = 1; }
  }
  // a tuned entry is used only where its kernels take this M (the skinny
  // kernel takes M <= 16 in a single launch, so it is never a tail); a
  // padded-M bucket never displaces the skinny kernel for M <= 16
  const Variant* bv = best ? find_variant(best->variant) : nullptr;
  if (bv && bv->max_m && M > bv->max_m) bv = nullptr;
  if (bv && pl.source == 1 && M <= 16 && bv->max_m != 16) bv = nullptr;
  // stream-K entries serve their exact shape only: at another M the tile
  // count may leave a stream-K phase, whose K-skewed ranges lose L2 reuse
  if (bv && pl.source == 1 && bv->persistent) bv = nullptr;
  if (bv) {
    pl.v = bv;
    pl.split = best->split;
    const Variant* tv = best->tail_variant[0] ? find_variant(best->tail_variant) : nullptr;
    if (pl.source == 0 && tv && !tv->max_m && best->m_split > 0 && best->m_split < M) {
      pl.tail = tv;
      pl.m_split = best->m_split;
      pl.tail_split = best->tail_split > 0 ? best->tail_split : 1;
    }
  }
  if (!pl.v) {
    pl = make_plan_heuristic(op, G, M, N, K, dt);
    pl.source = 2;
  }
  if (pl.split > KB) pl.split = KB > 0 ? KB : 1;
  if (pl.v->persistent || pl.v->kind == 2) pl.split = 1;   // no split-K in these kernels
  fit_workspace(pl, op, G, M, N, K, dt, workspace_bytes);
  return pl;
}

Plan make_plan_heuristic(bsmm_op op, int G, int M, int N, int K, bsmm_dtype dt) {
  (void)dt;
  Plan pl;
  // fp8 with enough rows: the K loop reads scale_a repacked once per call
  // (one small load per wave and K block instead of one per row group)
  // mx32 reads twelve scale bytes per lane and K block unpacked, two words
  // packed: it packs whenever it runs the tile kernel.  groupwise has only
  // packed kernels (its K loop stages the packed scales through LDS).
  const bool gw = op == BSMM_OP_FP8_GROUPWISE;
  const bool pack = gw || (op == BSMM_OP_FP8_MX32_MM
                               ? M > 16
                               : packable_scales(op) && M > 128 && (int64_t)G * M >= 1024);
  const char* name;
  if (M <= 16 && !gw) {
    // decode-sized: one pass over B with K split inside each workgroup
    pl.v = find_variant("s16x16");
    return pl;
  }
  if (M <= 64 && !gw) name = N % 256 == 0 ? "t64x256" : "t64x128";
  else if (M <= 128)
    name = N % 256 == 0 ? (pack ? "t128x256p" : "t128x256") : (gw ? "t256x128p" : "t128x128");
  else if (N % 256 == 0) name = pack ? "t256x256p" : "t256x256";
  else name = pack ? "t256x128p" : "t256x128";
  pl.v = find_variant(name);
  const int KB = K / kBlockK;
  const int64_t tiles = (int64_t)((M + pl.v->tile_m - 1) / pl.v->tile_m) *
                        ((N + pl.v->tile_n - 1) / pl.v->tile_n) * G;
  pl.split = 1;
  // Split K only when one pass leaves most CUs idle and each slice keeps at
  // least 4 K blocks.
  if (tiles < 128 && KB >= 8) {
    int s = (int)((256 + tiles - 1) / tiles);
    if (s > KB / 4) s = KB / 4;
    if (s < 1) s = 1;
    pl.split = s;
  }
  const int bm = pl.v->tile_m;
  const int64_t per_row = (int64_t)((N + pl.v->tile_n - 1) / pl.v->tile_n) * G;
  const int64_t rounds = tiles / kPlanCUs, rem = tiles % kPlanCUs;
  if (rounds >= 1 && rem > 0 && rem <= kPlanCUs / 2 && KB >= 8) {
    // Whole rounds: the last round would leave most CUs idle.  The bulk
    // launch takes the tile rows that fill whole rounds; the remaining rows
    // run as a second launch of the same kernel with split K across the chip.
    const int64_t bulk_tile_rows = rounds * kPlanCUs / per_row;
    const int m_split = (int)(bulk_tile_rows * bm);
    if (bulk_tile_rows >= 1 && m_split < M) {
      const int64_t tail_tiles = (int64_t)((M - m_split + bm - 1) / bm) * per_row;
      int s = (int)(kPlanCUs / tail_tiles);     // tail_tiles * s fits one round
      if (s > KB / 4) s = KB / 4;
      if (ovr().tail_split_cap > 0 && s > ovr().tail_split_cap) s = ovr().tail_split_cap;
      if (s >= 2) {
        pl.m_split = m_split;
        pl.tail = pl.v;
        // A short tail (at most 32 bulk tiles) runs on narrower tiles with
        // fewer K slices, so fewer partial planes are reduced: 128 x 128
        // tiles with at most 4 slices, or for mx32 (whose unpacked K loop
        // is slow) the packed 256 x 128 tile with at most 6 (MI355X, the
        // 256-row tails of 16640 x 5120 x 8192 and 16640 x 8192 x 5120:
        // 1.2-2.5% per call).  Groupwise keeps its packed bulk tile.
        if (tail_tiles <= 32 && !gw) {
          const bool mx32 = op == BSMM_OP_FP8_MX32_MM;
          if (const Variant* tv = find_variant(mx32 ? "t256x128p" : "t128x128")) {
            pl.tail = tv;
            if (s > (mx32 ? 6 : 4)) s = mx32 ? 6 : 4;
          }
        }
        if (!ovr().tail_variant.empty())
          if (const Variant* tv = find_variant(ovr().tail_variant.c_str())) pl.tail = tv;
        pl.tail_split = s;
        return pl;
      }
    }
  }
  // M-split: aligned bulk on the big tile plus a narrow tail launch.
  const int bulk = (M / bm) * bm;
  const int tail = M - bulk;
  if (bm == 256 && tail > 0 && tail <= 64 && (int64_t)G * bulk >= 8192 && !gw) {
    pl.m_split = bulk;
    pl.tail = find_variant(N % 256 == 0 ? "t64x256" : "t64x128");
  }
  return pl;
}

static bsmm_status run(const Problem& p, size_t workspace_bytes, void* ws,
                       void* stream) {
  Plan pl = make_plan(p.op, p.G, p.M, p.N, p.K, p.out_dtype, workspace_bytes);
  if (ovr().log)
    fprintf(stderr, "[bsmm] %s G=%d M=%d N=%d K=%d out=%d -> %s split=%d m_split=%d tail=%s/%d src=%d\n",
            op_name(p.op), p.G, p.M, p.N, p.K, (int)p.out_dtype, pl.v->name, pl.split,
            pl.m_split, pl.tail ? pl.tail->name : "-", pl.tail_split, pl.source);
  // packed scale_a first (shared by both launches), then the launches, which
  // share the rest of the workspace
  if (p.op == BSMM_OP_FP8_GROUPWISE &&
      (!pl.v->packed_scales || (pl.m_split && pl.tail && !pl.tail->packed_scales)))
    return fail(BSMM_ERR_ARG,
                "fp8 groupwise runs packed-scale kernels only: it needs a workspace of %zu bytes "
                "(variant %s)",
                bsmm_workspace_bytes(p.op, p.G, p.M, p.N, p.K, p.out_dtype), pl.v->name);
  Launch l;
  l.psa = nullptr;
  l.stream = stream;
  l.ws = ws;
  l.ws_bytes = ws ? workspace_bytes : 0;
  l.sk_grid = ovr().sk_grid.load(std::memory_order_relaxed);
  if (plan_packed(pl, p.op) && p.K >= kBlockK) {
    const size_t pack = packed_scale_bytes(p.op, p.G, p.M, p.K, p.N);
    if (!ws || l.ws_bytes < pack) return fail(BSMM_ERR_ARG, "workspace too small for the plan");
    if (pack_scale_a(p, ws, stream)) return fail(BSMM_ERR_HIP, "scale packing launch failed");
    l.psa = ws;
    l.ws_bytes -= pack;
    l.ws = l.ws_bytes ? (void*)((uint8_t*)ws + pack) : nullptr;
  }
  l.row_begin = 0;
  l.row_end = pl.m_split ? pl.m_split : p.M;
  l.split = pl.split;
  const bool timed = timing_on();
  if (timed) timing_mark(stream, pl.v->name, true);
  if (pl.v->launch(p, l))
    return fail(BSMM_ERR_HIP, "kernel launch failed (%s)", pl.v->name);
  if (timed) timing_mark(stream, pl.v->name, false);
  if (pl.m_split && pl.m_split < p.M) {
    l.row_begin = pl.m_split;
    l.row_end = p.M;
    l.split = pl.tail_split;
    if (pl.tail->launch(p, l))
      return fail(BSMM_ERR_HIP, "kernel launch failed (%s)", pl.tail->name);
  }
  return BSMM_OK;
}

}  // namespace bsmm

using namespace bsmm;

#define CHECK(cond, status, ...) \
  do { if (!(cond)) return fail(status, __VA_ARGS__); } while (0)

extern "C" {

bsmm_status bsmm_int8_rowwise(const int8_t* a, int64_t lda, const int8_t* b,
                              int64_t ldb, const float* scale_a, int64_t sa_m,
                              const float* scale_b, int64_t sb_n, void* out,
                              int64_t ldo, bsmm_dtype out_dtype, int64_t M,
                              int64_t N, int64_t K, void* workspace,
                              size_t workspace_bytes, void* stream) {
  CHECK(M >= 0 && N >= 0 && K >= 0, BSMM_ERR_SHAPE, "negative size M=%lld N=%lld K=%lld",
        (long long)M, (long long)N, (long long)K);
  CHECK(M < kMaxDim && N < kMaxDim && K < kMaxDim, BSMM_ERR_UNSUPPORTED, "size beyond 2^31");
  CHECK(out_dtype == BSMM_I32 || out_dtype == BSMM_F32 || out_dtype == BSMM_BF16,
        BSMM_ERR_DTYPE, "unknown output dtype %d", (int)out_dtype);
  if (M == 0 || N == 0) return BSMM_OK;
  CHECK(K % kBlockK == 0, BSMM_ERR_UNSUPPORTED, "K=%lld is not a multiple of 128", (long long)K);
  // any int8 code, -128 included: |acc| <= K * 128^2 = K * 2^14 < 2^31
  CHECK(K <= kMaxInt8K, BSMM_ERR_UNSUPPORTED,
        "K=%lld may overflow the int32 accumulator (K * 2^14 >= 2^31)", (long long)K);
  CHECK(out != nullptr, BSMM_ERR_NULL, "out is NULL");
  CHECK(K == 0 || (a != nullptr && b != nullptr), BSMM_ERR_NULL, "a or b is NULL");
  if (out_dtype != BSMM_I32) {
    CHECK(scale_a != nullptr && scale_b != nullptr, BSMM_ERR_NULL,
          "scale_a / scale_b NULL with a scaled output dtype");
    CHECK(sa_m >= 0 && sb_n >= 0, BSMM_ERR_SCALE_SHAPE,
          "scale strides must be >= 0 (0 broadcasts one scalar)");
    CHECK(aligned(scale_a, 4) && aligned(scale_b, 4), BSMM_ERR_ALIGN, "scales not 4-byte aligned");
    CHECK((M - 1) * sa_m < ((int64_t)1 << 30) && (N - 1) * sb_n < ((int64_t)1 << 30),
          BSMM_ERR_UNSUPPORTED, "scale index range beyond 2^30");
  }
  CHECK(ldo >= N, BSMM_ERR_SHAPE, "ldo=%lld below N", (long long)ldo);
  if (K > 0) {   // operands are not read when K == 0
    CHECK(lda >= K && ldb >= K, BSMM_ERR_SHAPE, "leading dimensions lda=%lld ldb=%lld below K",
          (long long)lda, (long long)ldb);
    CHECK(lda % 16 == 0 && ldb % 16 == 0, BSMM_ERR_ALIGN, "lda / ldb not multiples of 16 bytes");
    CHECK(lda <= kMaxLd && ldb <= kMaxLd, BSMM_ERR_UNSUPPORTED, "leading dimension beyond 2^23");
  }
  CHECK(K == 0 || (aligned(a, 16) && aligned(b, 16)), BSMM_ERR_ALIGN, "a / b not 16-byte aligned");
  CHECK(aligned(out, 4), BSMM_ERR_ALIGN, "out not 4-byte aligned");
  Problem p{};
  p.op = BSMM_OP_INT8_ROWWISE;
  p.out_dtype = out_dtype;
  p.G = 1; p.M = (int)M; p.N = (int)N; p.K = (int)K;
  p.a = (const uint8_t*)a; p.lda = lda; p.a_sg = 0;
  p.b = (const uint8_t*)b; p.ldb = ldb; p.b_sg = 0;
  p.sa = scale_a; p.sa_m = sa_m; p.sa_sg = 0; p.sa_kb = 0;
  p.sb = scale_b; p.sb_n = sb_n; p.sb_sg = 0; p.sb_kb = 0;
  p.out = out; p.ldo = ldo; p.o_sg = 0;
  return run(p, workspace ? workspace_bytes : 0, workspace, stream);
}

bsmm_status bsmm_fp8_blockwise(const uint8_t* a, int64_t lda, const uint8_t* b,
                               int64_t ldb, const float* scale_a, int64_t sa_m,
                               int64_t sa_kb, const float* scale_b, int64_t sb_kb,
                               int64_t sb_nb, void* out, int64_t ldo,
                               bsmm_dtype out_dtype, int64_t M, int64_t N, int64_t K,
                               void* workspace, size_t workspace_bytes, void* stream) {
  CHECK(M >= 0 && N >= 0 && K >= 0, BSMM_ERR_SHAPE, "negative size M=%lld N=%lld K=%lld",
        (long long)M, (long long)N, (long long)K);
  CHECK(M < kMaxDim && N < kMaxDim && K < kMaxDim, BSMM_ERR_UNSUPPORTED, "size beyond 2^31");
  CHECK(out_dtype == BSMM_F32 || out_dtype == BSMM_BF16, BSMM_ERR_DTYPE,
        "fp8 blockwise writes fp32 or bf16 (got %d)", (int)out_dtype);
  if (M == 0 || N == 0) return BSMM_OK;
  CHECK(K % kBlockK == 0, BSMM_ERR_UNSUPPORTED, "K=%lld is not a multiple of 128", (long long)K);
  CHECK(N % kBlockK == 0, BSMM_ERR_UNSUPPORTED, "N=%lld is not a multiple of 128", (long long)N);
  CHECK(out != nullptr, BSMM_ERR_NULL, "out is NULL");
  if (K > 0) {
    CHECK(a != nullptr && b != nullptr, BSMM_ERR_NULL, "a or b is NULL");
    CHECK(scale_a != nullptr && scale_b != nullptr, BSMM_ERR_NULL, "scale_a / scale_b is NULL");
    CHECK(sa_m >= 0 && sa_kb >= 0 && sb_kb >= 0 && sb_nb >= 0, BSMM_ERR_SCALE_SHAPE,
          "scale strides must be >= 0 (0 broadcasts)");
    const int64_t KB = K / kBlockK, NB = N / kBlockK;
    CHECK(((M - 1) * sa_m + (KB - 1) * sa_kb) < ((int64_t)1 << 30) &&
              ((KB - 1) * sb_kb + (NB - 1) * sb_nb) < ((int64_t)1 << 30),
          BSMM_ERR_UNSUPPORTED, "scale index range beyond 2^30");
    CHECK(aligned(scale_a, 4) && aligned(scale_b, 4), BSMM_ERR_ALIGN, "scales not 4-byte aligned");
    CHECK(aligned(a, 16) && aligned(b, 16), BSMM_ERR_ALIGN, "a / b not 16-byte aligned");
  }
  CHECK(ldo >= N, BSMM_ERR_SHAPE, "ldo=%lld below N", (long long)ldo);
  if (K > 0) {   // operands are not read when K == 0
    CHECK(lda >= K && ldb >= K, BSMM_ERR_SHAPE, "leading dimensions lda=%lld ldb=%lld below K",
          (long long)lda, (long long)ldb);
    CHECK(lda % 16 == 0 && ldb % 16 == 0, BSMM_ERR_ALIGN, "lda / ldb not multiples of 16 bytes");
    CHECK(lda <= kMaxLd && ldb <= kMaxLd, BSMM_ERR_UNSUPPORTED, "leading dimension beyond 2^23");
  }
  CHECK(aligned(out, 4), BSMM_ERR_ALIGN, "out not 4-byte aligned");
  Problem p{};
  p.op = BSMM_OP_FP8_BLOCKWISE;
  p.out_dtype = out_dtype;
  p.G = 1; p.M = (int)M; p.N = (int)N; p.K = (int)K;
  p.a = a; p.lda = lda;
  p.b = b; p.ldb = ldb;
  p.sa = scale_a; p.sa_m = sa_m; p.sa_kb = sa_kb;
  p.sb = scale_b; p.sb_kb = sb_kb; p.sb_n = sb_nb;
  p.out = out; p.ldo = ldo;
  return run(p, workspace ? workspace_bytes : 0, workspace, stream);
}

bsmm_status bsmm_fp8_blockwise_scratch(const uint8_t* a, int64_t lda, const uint8_t* b,
                                       int64_t ldb, const float* scale_a, int64_t sa_m,
                                       int64_t sa_kb, const float* scale_b, int64_t sb_kb,
                                       int64_t sb_nb, void* out, int64_t ldo,
                                       bsmm_dtype out_dtype, int64_t M, int64_t N, int64_t K,
                                       void* stream) {
  // the workspace the fastest plan wants (0 for sizes the entry point
  // rejects or that launch nothing, which bsmm_fp8_blockwise then handles)
  const size_t need = bsmm_workspace_bytes(BSMM_OP_FP8_BLOCKWISE, 1, M, N, K, out_dtype);
  CHECK(need <= kScratchBytes, BSMM_ERR_UNSUPPORTED,
        "M=%lld N=%lld K=%lld needs %zu bytes of workspace; the static scratch holds %zu "
        "(use bsmm_fp8_blockwise with a workspace)",
        (long long)M, (long long)N, (long long)K, need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    int err = 0;
    ws = scratch_device_ptr(&err);
    CHECK(ws != nullptr, BSMM_ERR_HIP, "the static scratch's device address is unavailable "
          "(hipGetSymbolAddress: error %d)", err);
  }
  return bsmm_fp8_blockwise(a, lda, b, ldb, scale_a, sa_m, sa_kb, scale_b, sb_kb, sb_nb, out,
                            ldo, out_dtype, M, N, K, ws, need, stream);
}

bsmm_status bsmm_fp8_groupwise(const uint8_t* a, int64_t lda, const uint8_t* b,
                               int64_t ldb, const float* scale_a, int64_t sa_m,
                               int64_t sa_kb, const float* scale_b, int64_t sb_kb,
                               int64_t sb_n, void* out, int64_t ldo,
                               bsmm_dtype out_dtype, int64_t M, int64_t N, int64_t K,
                               void* workspace, size_t workspace_bytes, void* stream) {
  CHECK(M >= 0 && N >= 0 && K >= 0, BSMM_ERR_SHAPE, "negative size M=%lld N=%lld K=%lld",
        (long long)M, (long long)N, (long long)K);
  CHECK(M < kMaxDim && N < kMaxDim && K < kMaxDim, BSMM_ERR_UNSUPPORTED, "size beyond 2^31");
  CHECK(out_dtype == BSMM_F32 || out_dtype == BSMM_BF16, BSMM_ERR_DTYPE,
        "fp8 groupwise writes fp32 or bf16 (got %d)", (int)out_dtype);
  if (M == 0 || N == 0) return BSMM_OK;
  CHECK(K % kBlockK == 0, BSMM_ERR_UNSUPPORTED, "K=%lld is not a multiple of 128", (long long)K);
  CHECK(out != nullptr, BSMM_ERR_NULL, "out is NULL");
  if (K > 0) {
    CHECK(a != nullptr && b != nullptr, BSMM_ERR_NULL, "a or b is NULL");
    CHECK(scale_a != nullptr && scale_b != nullptr, BSMM_ERR_NULL, "scale_a / scale_b is NULL");
    CHECK(sa_m >= 0 && sa_kb >= 0 && sb_kb >= 0 && sb_n >= 0, BSMM_ERR_SCALE_SHAPE,
          "scale strides must be >= 0 (0 broadcasts)");
    const int64_t KB = K / kBlockK;
    CHECK(((M - 1) * sa_m + (KB - 1) * sa_kb) < ((int64_t)1 << 30) &&
              ((KB - 1) * sb_kb + (N - 1) * sb_n) < ((int64_t)1 << 30),
          BSMM_ERR_UNSUPPORTED, "scale index range beyond 2^30");
    // the K loop addresses the packed scales with 32-bit byte offsets
    CHECK(KB <= 65535 && packed_scale_bytes(BSMM_OP_FP8_GROUPWISE, 1, (int)M, (int)K, (int)N) <
                             ((size_t)1 << 31),
          BSMM_ERR_UNSUPPORTED, "packed scales beyond 2^31 bytes");
    CHECK(aligned(scale_a, 4) && aligned(scale_b, 4), BSMM_ERR_ALIGN, "scales not 4-byte aligned");
    CHECK(aligned(a, 16) && aligned(b, 16), BSMM_ERR_ALIGN, "a / b not 16-byte aligned");
    CHECK(lda >= K && ldb >= K, BSMM_ERR_SHAPE, "leading dimensions lda=%lld ldb=%lld below K",
          (long long)lda, (long long)ldb);
    CHECK(lda % 16 == 0 && ldb % 16 == 0, BSMM_ERR_ALIGN, "lda / ldb not multiples of 16 bytes");
    CHECK(lda <= kMaxLd && ldb <= kMaxLd, BSMM_ERR_UNSUPPORTED, "leading dimension beyond 2^23");
  }
  CHECK(ldo >= N, BSMM_ERR_SHAPE, "ldo=%lld below N", (long long)ldo);
  CHECK(aligned(out, 4), BSMM_ERR_ALIGN, "out not 4-byte aligned");
  Problem p{};
  p.op = BSMM_OP_FP8_GROUPWISE;
  p.out_dtype = out_dtype;
  p.G = 1; p.M = (int)M; p.N = (int)N; p.K = (int)K;
  p.a = a; p.lda = lda;
  p.b = b; p.ldb = ldb;
  p.sa = scale_a; p.sa_m = sa_m; p.sa_kb = sa_kb;
  p.sb = scale_b; p.sb_kb = sb_kb; p.sb_n = sb_n;
  p.out = out; p.ldo = ldo;
  return run(p, workspace ? workspace_bytes : 0, workspace, stream);
}

bsmm_status bsmm_fp8_mx_bmm(const uint8_t* x, int64_t x_sg, int64_t x_sm,
                            const uint8_t* w, int64_t w_sg, int64_t w_sn,
                            const uint8_t* x_scale, int64_t xs_sg, int64_t xs_sm,
                            const uint8_t* w_scale, int64_t ws_sg, int64_t ws_snb,
                            void* out, int64_t o_sg, int64_t o_sm, bsmm_dtype out_dtype,
                            int64_t G, int64_t M, int64_t N, int64_t K,
                            void* workspace, size_t workspace_bytes, void* stream) {
  CHECK(G >= 0 && M >= 0 && N >= 0 && K >= 0, BSMM_ERR_SHAPE,
        "negative size G=%lld M=%lld N=%lld K=%lld", (long long)G, (long long)M,
        (long long)N, (long long)K);
  CHECK(G < kMaxDim && M < kMaxDim && N < kMaxDim && K < kMaxDim, BSMM_ERR_UNSUPPORTED,
        "size beyond 2^31");
  CHECK(out_dtype == BSMM_F32 || out_dtype == BSMM_BF16, BSMM_ERR_DTYPE,
        "fp8 mx BMM writes fp32 or bf16 (got %d)", (int)out_dtype);
  if (G == 0 || M == 0 || N == 0) return BSMM_OK;
  CHECK(K % kBlockK == 0, BSMM_ERR_UNSUPPORTED, "K=%lld is not a multiple of 128", (long long)K);
  CHECK(N % kBlockK == 0, BSMM_ERR_UNSUPPORTED, "N=%lld is not a multiple of 128", (long long)N);
  CHECK(out != nullptr, BSMM_ERR_NULL, "out is NULL");
  CHECK(x_sg >= 0 && x_sm >= 0 && w_sg >= 0 && w_sn >= 0 && o_sg >= 0 && o_sm >= 0,
        BSMM_ERR_LAYOUT, "negative stride");
  CHECK(x_sm >= K && w_sn >= K && o_sm >= N, BSMM_ERR_LAYOUT,
        "row strides x_sm=%lld w_sn=%lld o_sm=%lld below K / N", (long long)x_sm,
        (long long)w_sn, (long long)o_sm);
  if (K > 0) {
    CHECK(x != nullptr && w != nullptr, BSMM_ERR_NULL, "x or w is NULL");
    CHECK(x_scale != nullptr && w_scale != nullptr, BSMM_ERR_NULL, "x_scale / w_scale is NULL");
    CHECK(xs_sg >= 0 && xs_sm >= 0 && ws_sg >= 0 && ws_snb >= 0, BSMM_ERR_SCALE_SHAPE,
          "scale strides must be >= 0");
    CHECK(aligned(x, 16) && aligned(w, 16) && x_sg % 16 == 0 && x_sm % 16 == 0 &&
              w_sg % 16 == 0 && w_sn % 16 == 0,
          BSMM_ERR_ALIGN, "x / w pointers or strides not 16-byte aligned");
    CHECK(x_sm <= kMaxLd && w_sn <= kMaxLd, BSMM_ERR_UNSUPPORTED, "row stride beyond 2^23");
  }
  CHECK(aligned(out, 4), BSMM_ERR_ALIGN, "out not 4-byte aligned");
  Problem p{};
  p.op = BSMM_OP_FP8_MX_BMM;
  p.out_dtype = out_dtype;
  p.G = (int)G; p.M = (int)M; p.N = (int)N; p.K = (int)K;
  p.a = x; p.a_sg = x_sg; p.lda = x_sm;
  p.b = w; p.b_sg = w_sg; p.ldb = w_sn;
  p.sa = x_scale; p.sa_sg = xs_sg; p.sa_m = xs_sm; p.sa_kb = 1;
  p.sb = w_scale; p.sb_sg = ws_sg; p.sb_n = ws_snb; p.sb_kb = 1;
  p.out = out; p.o_sg = o_sg; p.ldo = o_sm;
  return run(p, workspace ? workspace_bytes : 0, workspace, stream);
}

size_t bsmm_workspace_bytes(bsmm_op op, int64_t G, int64_t M, int64_t N, int64_t K,
                            bsmm_dtype out_dtype) {
  if (G <= 0 || M <= 0 || N <= 0 || K <= 0 || G >= kMaxDim || M >= kMaxDim ||
      N >= kMaxDim || K >= kMaxDim || K % kBlockK)
    return 0;
  Plan pl = make_plan(op, (int)G, (int)M, (int)N, (int)K, out_dtype, (size_t)-1);
  return pl.workspace;
}

bsmm_status bsmm_query_plan(bsmm_op op, int64_t G, int64_t M, int64_t N, int64_t K,
                            bsmm_dtype out_dtype, size_t workspace_bytes,
                            bsmm_plan_info* info) {
  CHECK(info != nullptr, BSMM_ERR_NULL, "info is NULL");
  CHECK(op == BSMM_OP_INT8_ROWWISE || op == BSMM_OP_FP8_BLOCKWISE || op == BSMM_OP_FP8_MX_BMM ||
            op == BSMM_OP_FP8_SCALED_MM || op == BSMM_OP_FP8_MX32_MM ||
            op == BSMM_OP_FP8_GROUPWISE,
        BSMM_ERR_ARG, "unknown op %d", (int)op);
  CHECK(G > 0 && M > 0 && N > 0 && K >= 0, BSMM_ERR_SHAPE, "sizes must be positive");
  CHECK(G < kMaxDim && M < kMaxDim && N < kMaxDim && K < kMaxDim, BSMM_ERR_UNSUPPORTED,
        "size beyond 2^31");
  CHECK(K % kBlockK == 0, BSMM_ERR_UNSUPPORTED, "K not a multiple of 128");
  Plan pl = make_plan(op, (int)G, (int)M, (int)N, (int)K, out_dtype, workspace_bytes);
  memset(info, 0, sizeof(*info));
  snprintf(info->variant, sizeof(info->variant), "%s", pl.v->name);
  info->tile_m = pl.v->tile_m;
  info->tile_n = pl.v->tile_n;
  info->split_k = pl.split;
  info->m_split = pl.m_split;
  info->workspace = (int64_t)pl.workspace;
  info->source = pl.source;
  snprintf(info->tail_variant, sizeof(info->tail_variant), "%s",
           pl.m_split && pl.tail ? pl.tail->name : "");
  info->tail_split_k = pl.m_split && pl.tail ? pl.tail_split : 0;
  return BSMM_OK;
}

bsmm_status bsmm_set_override(const char* variant, int split_k) {
  read_env_once();
  if (variant && variant[0] && !find_variant(variant))
    return fail(BSMM_ERR_ARG, "unknown variant '%s'", variant);
  Override& o = ovr();
  std::lock_guard<std::mutex> g(o.mu);
  o.variant = variant ? variant : "";
  o.split = split_k > 0 ? split_k : 0;
  o.active.store(!o.variant.empty() || o.split > 0 || o.m_split > 0, std::memory_order_release);
  o.gen.fetch_add(1, std::memory_order_acq_rel);
  return BSMM_OK;
}

bsmm_status bsmm_set_override_tail(int m_split, const char* tail_variant, int tail_split) {
  read_env_once();
  if (m_split > 0 && (!tail_variant || !tail_variant[0] || !find_variant(tail_variant)))
    return fail(BSMM_ERR_ARG, "unknown tail variant '%s'", tail_variant ? tail_variant : "");
  CHECK(m_split >= 0 && m_split % 64 == 0, BSMM_ERR_ARG,
        "the M-split point must be a non-negative multiple of 64 (got %d)", m_split);
  Override& o = ovr();
  std::lock_guard<std::mutex> g(o.mu);
  o.m_split = m_split;
  o.m_tail = m_split > 0 ? tail_variant : "";
  o.m_tail_split = tail_split > 0 ? tail_split : 1;
  o.active.store(!o.variant.empty() || o.split > 0 || o.m_split > 0, std::memory_order_release);
  o.gen.fetch_add(1, std::memory_order_acq_rel);
  return BSMM_OK;
}

bsmm_status bsmm_set_streamk_grid(int workgroups) {
  CHECK(workgroups >= 0, BSMM_ERR_ARG, "negative stream-K grid %d", workgroups);
  ovr().sk_grid.store(workgroups, std::memory_order_release);
  return BSMM_OK;
}

const char* bsmm_variant_names(void) {
  static std::string names = [] {
    std::string s;
    int n = 0;
    const Variant* v = variants(&n);
    for (int i = 0; i < n; ++i) {
      if (i) s += ",";
      s += v[i].name;
    }
    return s;
  }();
  return names.c_str();
}

bsmm_status bsmm_fp8_scaled_mm(const uint8_t* a, int64_t lda, const uint8_t* b, int64_t ldb,
                               const float* scale_a, int64_t sa_m, const float* scale_b,
                               int64_t sb_n, const void* bias, bsmm_dtype bias_dtype,
                               const float* scale_result, void* out, int64_t ldo,
                               bsmm_dtype out_dtype, int64_t M, int64_t N, int64_t K,
                               void* workspace, size_t workspace_bytes, void* stream) {
  CHECK(M >= 0 && N >= 0 && K >= 0, BSMM_ERR_SHAPE, "negative size M=%lld N=%lld K=%lld",
        (long long)M, (long long)N, (long long)K);
  CHECK(M < kMaxDim && N < kMaxDim && K < kMaxDim, BSMM_ERR_UNSUPPORTED, "size beyond 2^31");
  CHECK(out_dtype == BSMM_F32 || out_dtype == BSMM_BF16 || out_dtype == BSMM_E4M3,
        BSMM_ERR_DTYPE, "fp8 scaled_mm writes fp32, bf16 or e4m3 (got %d)", (int)out_dtype);
  if (M == 0 || N == 0) return BSMM_OK;
  CHECK(K % kBlockK == 0, BSMM_ERR_UNSUPPORTED, "K=%lld is not a multiple of 128", (long long)K);
  CHECK(out != nullptr, BSMM_ERR_NULL, "out is NULL");
  CHECK(scale_a != nullptr && scale_b != nullptr, BSMM_ERR_NULL, "scale_a / scale_b is NULL");
  CHECK(sa_m >= 0 && sb_n >= 0, BSMM_ERR_SCALE_SHAPE,
        "scale strides must be >= 0 (0: tensorwise, one scalar)");
  CHECK((M - 1) * sa_m < ((int64_t)1 << 30) && (N - 1) * sb_n < ((int64_t)1 << 30),
        BSMM_ERR_UNSUPPORTED, "scale index range beyond 2^30");
  CHECK(aligned(scale_a, 4) && aligned(scale_b, 4), BSMM_ERR_ALIGN, "scales not 4-byte aligned");
  if (bias) {
    CHECK(bias_dtype == BSMM_F32 || bias_dtype == BSMM_BF16, BSMM_ERR_DTYPE,
          "bias must be fp32 or bf16 (got %d)", (int)bias_dtype);
    CHECK(aligned(bias, bias_dtype == BSMM_F32 ? 4 : 2), BSMM_ERR_ALIGN, "bias misaligned");
  }
  CHECK(scale_result == nullptr || aligned(scale_result, 4), BSMM_ERR_ALIGN,
        "scale_result not 4-byte aligned");
  CHECK(ldo >= N, BSMM_ERR_SHAPE, "ldo=%lld below N", (long long)ldo);
  if (K > 0) {   // operands are not read when K == 0
    CHECK(a != nullptr && b != nullptr, BSMM_ERR_NULL, "a or b is NULL");
    CHECK(lda >= K && ldb >= K, BSMM_ERR_SHAPE, "leading dimensions lda=%lld ldb=%lld below K",
          (long long)lda, (long long)ldb);
    CHECK(lda % 16 == 0 && ldb % 16 == 0, BSMM_ERR_ALIGN, "lda / ldb not multiples of 16 bytes");
    CHECK(lda <= kMaxLd && ldb <= kMaxLd, BSMM_ERR_UNSUPPORTED, "leading dimension beyond 2^23");
    CHECK(aligned(a, 16) && aligned(b, 16), BSMM_ERR_ALIGN, "a / b not 16-byte aligned");
  }
  const uintptr_t osz = out_dtype == BSMM_F32 ? 4 : out_dtype == BSMM_BF16 ? 2 : 1;
  CHECK(aligned(out, osz), BSMM_ERR_ALIGN, "out not %d-byte aligned", (int)osz);
  Problem p{};
  p.op = BSMM_OP_FP8_SCALED_MM;
  p.out_dtype = out_dtype;
  p.G = 1; p.M = (int)M; p.N = (int)N; p.K = (int)K;
  p.a = a; p.lda = lda;
  p.b = b; p.ldb = ldb;
  p.sa = scale_a; p.sa_m = sa_m;
  p.sb = scale_b; p.sb_n = sb_n;
  p.out = out; p.ldo = ldo;
  p.bias = bias;
  p.bias_bf16 = bias && bias_dtype == BSMM_BF16;
  p.sr = scale_result;
  return run(p, workspace ? workspace_bytes : 0, workspace, stream);
}

bsmm_status bsmm_fp8_mx32_mm(const uint8_t* a, int64_t lda, const uint8_t* b, int64_t ldb,
                             const uint8_t* a_scale, int64_t as_m, const uint8_t* b_scale,
                             int64_t bs_n, void* out, int64_t ldo, bsmm_dtype out_dtype,
                             int64_t M, int64_t N, int64_t K, void* workspace,
                             size_t workspace_bytes, void* stream) {
  CHECK(M >= 0 && N >= 0 && K >= 0, BSMM_ERR_SHAPE, "negative size M=%lld N=%lld K=%lld",
        (long long)M, (long long)N, (long long)K);
  CHECK(M < kMaxDim && N < kMaxDim && K < kMaxDim, BSMM_ERR_UNSUPPORTED, "size beyond 2^31");
  CHECK(out_dtype == BSMM_F32 || out_dtype == BSMM_BF16, BSMM_ERR_DTYPE,
        "fp8 mx32 writes fp32 or bf16 (got %d)", (int)out_dtype);
  if (M == 0 || N == 0) return BSMM_OK;
  CHECK(K % kBlockK == 0, BSMM_ERR_UNSUPPORTED, "K=%lld is not a multiple of 128", (long long)K);
  CHECK(out != nullptr, BSMM_ERR_NULL, "out is NULL");
  CHECK(ldo >= N, BSMM_ERR_SHAPE, "ldo=%lld below N", (long long)ldo);
  if (K > 0) {
    const int64_t KC = K / 32;
    CHECK(a != nullptr && b != nullptr, BSMM_ERR_NULL, "a or b is NULL");
    CHECK(a_scale != nullptr && b_scale != nullptr, BSMM_ERR_NULL, "a_scale / b_scale is NULL");
    CHECK(as_m >= KC && bs_n >= KC, BSMM_ERR_SCALE_SHAPE,
          "scale rows of K/32 = %lld bytes need strides as_m=%lld bs_n=%lld >= K/32",
          (long long)KC, (long long)as_m, (long long)bs_n);
    CHECK((M - 1) * as_m + KC < ((int64_t)1 << 31) && (N - 1) * bs_n + KC < ((int64_t)1 << 31),
          BSMM_ERR_UNSUPPORTED, "scale index range beyond 2^31");
    CHECK(lda >= K && ldb >= K, BSMM_ERR_SHAPE, "leading dimensions lda=%lld ldb=%lld below K",
          (long long)lda, (long long)ldb);
    CHECK(lda % 16 == 0 && ldb % 16 == 0, BSMM_ERR_ALIGN, "lda / ldb not multiples of 16 bytes");
    CHECK(lda <= kMaxLd && ldb <= kMaxLd, BSMM_ERR_UNSUPPORTED, "leading dimension beyond 2^23");
    CHECK(aligned(a, 16) && aligned(b, 16), BSMM_ERR_ALIGN, "a / b not 16-byte aligned");
  }
  CHECK(aligned(out, 4), BSMM_ERR_ALIGN, "out not 4-byte aligned");
  Problem p{};
  p.op = BSMM_OP_FP8_MX32_MM;
  p.out_dtype = out_dtype;
  p.G = 1; p.M = (int)M; p.N = (int)N; p.K = (int)K;
  p.a = a; p.lda = lda;
  p.b = b; p.ldb = ldb;
  p.sa = a_scale; p.sa_m = as_m;
  p.sb = b_scale; p.sb_n = bs_n;
  p.out = out; p.ldo = ldo;
  return run(p, workspace ? workspace_bytes : 0, workspace, stream);
}

}  // extern "C"

namespace {

// Checks shared by the quantisers; `block` is 8 (int8 rows), 32 or 128.
bsmm_status quant_common(const void* x, int64_t ldx, bsmm_dtype x_dtype, const void* q,
                         int64_t ldq, const void* scale, int64_t s_m, int64_t s_kb,
                         int64_t M, int64_t K, int block, size_t scale_align) {
  CHECK(x_dtype == BSMM_F32 || x_dtype == BSMM_BF16, BSMM_ERR_DTYPE,
        "quantiser input must be fp32 or bf16 (got %d)", (int)x_dtype);
  CHECK(M >= 0 && K >= 0, BSMM_ERR_SHAPE, "negative size M=%lld K=%lld", (long long)M,
        (long long)K);
  CHECK(M < kMaxDim && K < kMaxDim, BSMM_ERR_UNSUPPORTED, "size beyond 2^31");
  CHECK(K % block == 0, BSMM_ERR_UNSUPPORTED, "K=%lld is not a multiple of %d", (long long)K,
        block);
  if (M == 0) return BSMM_OK;
  if (K == 0 && block != 8) return BSMM_OK;   // no blocks: nothing is written
  CHECK(scale != nullptr, BSMM_ERR_NULL, "scale is NULL");
  CHECK(aligned(scale, scale_align), BSMM_ERR_ALIGN, "scale not %d-byte aligned",
        (int)scale_align);
  CHECK(s_m >= 0 && s_kb >= 0, BSMM_ERR_SCALE_SHAPE, "scale strides must be >= 0");
  // every (row, block) must own its scale: the strides may not alias
  const int64_t KB = block == 8 ? 1 : K / block;
  if (KB > 0) {
    const bool rows_ok = M == 1 || s_m >= 1;
    const bool cols_ok = KB == 1 || s_kb >= 1;
    const bool disjoint = M == 1 || KB == 1 || s_m >= KB * s_kb || s_kb >= M * s_m;
    CHECK(rows_ok && cols_ok && disjoint, BSMM_ERR_SCALE_SHAPE,
          "scale strides s_m=%lld s_kb=%lld make two blocks share a scale", (long long)s_m,
          (long long)s_kb);
  }
  if (K == 0) return BSMM_OK;
  CHECK(x != nullptr && q != nullptr, BSMM_ERR_NULL, "x or q is NULL");
  CHECK(ldx >= K && ldq >= K, BSMM_ERR_SHAPE, "leading dimensions ldx=%lld ldq=%lld below K",
        (long long)ldx, (long long)ldq);
  CHECK(ldx % 8 == 0, BSMM_ERR_ALIGN, "ldx=%lld is not a multiple of 8 elements",
        (long long)ldx);
  CHECK(ldq % 8 == 0, BSMM_ERR_ALIGN, "ldq=%lld is not a multiple of 8 bytes",
        (long long)ldq);
  CHECK(aligned(x, 16), BSMM_ERR_ALIGN, "x not 16-byte aligned");
  CHECK(aligned(q, 8), BSMM_ERR_ALIGN, "q not 8-byte aligned");
  return BSMM_OK;
}

// Checks shared by the transposing quantisers of x [R, C]: R a multiple of
// 128, C of `cmult` (8 for the column groups, 128 with row or weight
// blocks); one scale per (128-row group, column) or, with `blocks`, per
// (128-row group, 128-column block).
bsmm_status quant_t_common(const void* x, int64_t ldx, bsmm_dtype x_dtype, const void* scale,
                           int64_t s_g, int64_t s_c, int64_t R, int64_t C, int cmult,
                           bool blocks) {
  CHECK(x_dtype == BSMM_F32 || x_dtype == BSMM_BF16, BSMM_ERR_DTYPE,
        "quantiser input must be fp32 or bf16 (got %d)", (int)x_dtype);
  CHECK(R >= 0 && C >= 0, BSMM_ERR_SHAPE, "negative size R=%lld C=%lld", (long long)R,
        (long long)C);
  CHECK(R < kMaxDim && C < kMaxDim, BSMM_ERR_UNSUPPORTED, "size beyond 2^31");
  CHECK(R % 128 == 0, BSMM_ERR_UNSUPPORTED, "R=%lld is not a multiple of 128", (long long)R);
  CHECK(C % cmult == 0, BSMM_ERR_UNSUPPORTED, "C=%lld is not a multiple of %d", (long long)C,
        cmult);
  if (R == 0 || C == 0) return BSMM_OK;
  CHECK(R / 128 <= 65535, BSMM_ERR_UNSUPPORTED, "R=%lld beyond 65535 groups of 128 rows",
        (long long)R);
  CHECK(scale != nullptr, BSMM_ERR_NULL, "scale is NULL");
  CHECK(aligned(scale, 4), BSMM_ERR_ALIGN, "scale not 4-byte aligned");
  CHECK(s_g >= 0 && s_c >= 0, BSMM_ERR_SCALE_SHAPE, "scale strides must be >= 0");
  const int64_t G = R / 128, NC = blocks ? C / 128 : C;
  const bool rows_ok = G == 1 || s_g >= 1;
  const bool cols_ok = NC == 1 || s_c >= 1;
  const bool disjoint = G == 1 || NC == 1 || s_g >= NC * s_c || s_c >= G * s_g;
  CHECK(rows_ok && cols_ok && disjoint, BSMM_ERR_SCALE_SHAPE,
        "scale strides s_g=%lld s_c=%lld make two groups share a scale", (long long)s_g,
        (long long)s_c);
  CHECK(x != nullptr, BSMM_ERR_NULL, "x is NULL");
  CHECK(ldx >= C, BSMM_ERR_SHAPE, "ldx=%lld below C", (long long)ldx);
  CHECK(ldx % 8 == 0 && aligned(x, 16), BSMM_ERR_ALIGN,
        "x not 16-byte aligned or ldx=%lld not a multiple of 8 elements", (long long)ldx);
  return BSMM_OK;
}

// transposed codes [C, R]: 16-byte row segments
bsmm_status check_qt(const void* q_t, int64_t ldqt, int64_t R) {
  CHECK(ldqt >= R, BSMM_ERR_SHAPE, "ldqt=%lld below R", (long long)ldqt);
  CHECK(ldqt % 16 == 0 && aligned(q_t, 16), BSMM_ERR_ALIGN, "q_t or ldqt not 16-byte aligned");
  return BSMM_OK;
}

bsmm_status quant_run(QuantArgs::Kind kind, const void* x, int64_t ldx, bsmm_dtype x_dtype,
                      void* q, int64_t ldq, void* scale, int64_t s_m, int64_t s_kb, int64_t M,
                      int64_t K, void* stream) {
  QuantArgs a{};
  a.kind = kind;
  a.x = x; a.ldx = ldx; a.x_dtype = x_dtype;
  a.q = q; a.ldq = ldq;
  a.scale = scale; a.s_m = s_m; a.s_kb = s_kb;
  a.M = M; a.K = K;
  if (launch_quant(a, stream) != 0) return fail(BSMM_ERR_HIP, "quantiser launch failed");
  return BSMM_OK;
}

}  // namespace

extern "C" {

bsmm_status bsmm_quant_int8_rowwise(const void* x, int64_t ldx, bsmm_dtype x_dtype,
                                    int8_t* q, int64_t ldq, float* scale, int64_t s_m,
                                    int64_t M, int64_t K, void* stream) {
  bsmm_status st = quant_common(x, ldx, x_dtype, q, ldq, scale, s_m, 0, M, K, 8, 4);
  if (st != BSMM_OK || M == 0) return st;
  CHECK(M <= ((int64_t)1 << 26), BSMM_ERR_UNSUPPORTED, "M=%lld beyond 2^26 rows",
        (long long)M);
  return quant_run(QuantArgs::kInt8Rows, x, ldx, x_dtype, q, ldq, scale, s_m, 0, M, K, stream);
}

bsmm_status bsmm_quant_fp8_blockwise(const void* x, int64_t ldx, bsmm_dtype x_dtype,
                                     uint8_t* q, int64_t ldq, float* scale, int64_t s_m,
                                     int64_t s_kb, int64_t M, int64_t K, void* stream) {
  bsmm_status st = quant_common(x, ldx, x_dtype, q, ldq, scale, s_m, s_kb, M, K, 128, 4);
  if (st != BSMM_OK || M == 0 || K == 0) return st;
  CHECK(M * (K / 128) < ((int64_t)1 << 30), BSMM_ERR_UNSUPPORTED,
        "M * K / 128 = %lld blocks beyond 2^30", (long long)(M * (K / 128)));
  return quant_run(QuantArgs::kFp8Blocks, x, ldx, x_dtype, q, ldq, scale, s_m, s_kb, M, K,
                   stream);
}

bsmm_status bsmm_quant_fp8_mx(const void* x, int64_t ldx, bsmm_dtype x_dtype, uint8_t* q,
                              int64_t ldq, uint8_t* scale, int64_t s_m, int64_t s_kb,
                              int64_t M, int64_t K, void* stream) {
  bsmm_status st = quant_common(x, ldx, x_dtype, q, ldq, scale, s_m, s_kb, M, K, 128, 1);
  if (st != BSMM_OK || M == 0 || K == 0) return st;
  CHECK(M * (K / 128) < ((int64_t)1 << 30), BSMM_ERR_UNSUPPORTED,
        "M * K / 128 = %lld blocks beyond 2^30", (long long)(M * (K / 128)));
  return quant_run(QuantArgs::kFp8Mx, x, ldx, x_dtype, q, ldq, scale, s_m, s_kb, M, K, stream);
}

bsmm_status bsmm_quant_fp8_mx32(const void* x, int64_t ldx, bsmm_dtype x_dtype, uint8_t* q,
                                int64_t ldq, uint8_t* scale, int64_t s_m, int64_t s_kb,
                                int64_t M, int64_t K, void* stream) {
  bsmm_status st = quant_common(x, ldx, x_dtype, q, ldq, scale, s_m, s_kb, M, K, 32, 1);
  if (st != BSMM_OK || M == 0 || K == 0) return st;
  CHECK(M * (K / 32) < ((int64_t)1 << 30), BSMM_ERR_UNSUPPORTED,
        "M * K / 32 = %lld blocks beyond 2^30", (long long)(M * (K / 32)));
  return quant_run(QuantArgs::kFp8Mx32, x, ldx, x_dtype, q, ldq, scale, s_m, s_kb, M, K,
                   stream);
}

bsmm_status bsmm_quant_fp8_columns(const void* x, int64_t ldx, bsmm_dtype x_dtype,
                                   uint8_t* q_t, int64_t ldqt, float* scale, int64_t s_g,
                                   int64_t s_c, int64_t R, int64_t C, void* stream) {
  bsmm_status st = quant_t_common(x, ldx, x_dtype, scale, s_g, s_c, R, C, 8, false);
  if (st != BSMM_OK || R == 0 || C == 0) return st;
  CHECK(q_t != nullptr, BSMM_ERR_NULL, "q_t is NULL");
  st = check_qt(q_t, ldqt, R);
  if (st != BSMM_OK) return st;
  QuantArgs a{};
  a.kind = QuantArgs::kFp8Columns;
  a.x = x; a.ldx = ldx; a.x_dtype = x_dtype;
  a.q = nullptr; a.ldq = 0;
  a.qt = q_t; a.ldqt = ldqt;
  a.scale = scale; a.s_m = s_g; a.s_kb = s_c;
  a.M = R; a.K = C;
  if (launch_quant(a, stream) != 0) return fail(BSMM_ERR_HIP, "quantiser launch failed");
  return BSMM_OK;
}

bsmm_status bsmm_quant_fp8_weight(const void* w, int64_t ldw, bsmm_dtype w_dtype, uint8_t* q,
                                  int64_t ldq, uint8_t* q_t, int64_t ldqt, float* scale,
                                  int64_t s_r, int64_t s_c, int64_t R, int64_t C, void* stream) {
  bsmm_status st = quant_t_common(w, ldw, w_dtype, scale, s_r, s_c, R, C, 128, true);
  if (st != BSMM_OK || R == 0 || C == 0) return st;
  CHECK(q != nullptr || q_t != nullptr, BSMM_ERR_NULL, "q and q_t are both NULL");
  if (q != nullptr) {
    CHECK(ldq >= C, BSMM_ERR_SHAPE, "ldq=%lld below C", (long long)ldq);
    CHECK(ldq % 8 == 0 && aligned(q, 8), BSMM_ERR_ALIGN, "q or ldq not 8-byte aligned");
  }
  if (q_t != nullptr) {
    st = check_qt(q_t, ldqt, R);
    if (st != BSMM_OK) return st;
  }
  QuantArgs a{};
  a.kind = QuantArgs::kFp8Weight;
  a.x = w; a.ldx = ldw; a.x_dtype = w_dtype;
  a.q = q; a.ldq = ldq;
  a.qt = q_t; a.ldqt = ldqt;
  a.scale = scale; a.s_m = s_r; a.s_kb = s_c;
  a.M = R; a.K = C;
  if (launch_quant(a, stream) != 0) return fail(BSMM_ERR_HIP, "quantiser launch failed");
  return BSMM_OK;
}

bsmm_status bsmm_quant_fp8_blockwise_columns(const void* x, int64_t ldx, bsmm_dtype x_dtype,
                                             uint8_t* q, int64_t ldq, float* s_rows,
                                             int64_t sr_m, int64_t sr_kb, uint8_t* q_t,
                                             int64_t ldqt, float* s_cols, int64_t sc_g,
                                             int64_t sc_c, int64_t R, int64_t C, void* stream) {
  bsmm_status st = quant_t_common(x, ldx, x_dtype, s_cols, sc_g, sc_c, R, C, 128, false);
  if (st != BSMM_OK || R == 0 || C == 0) return st;
  CHECK(q != nullptr && q_t != nullptr && s_rows != nullptr, BSMM_ERR_NULL,
        "q, q_t or s_rows is NULL");
  CHECK(ldq >= C, BSMM_ERR_SHAPE, "ldq=%lld below C", (long long)ldq);
  CHECK(ldq % 8 == 0 && aligned(q, 8), BSMM_ERR_ALIGN, "q or ldq not 8-byte aligned");
  st = check_qt(q_t, ldqt, R);
  if (st != BSMM_OK) return st;
  CHECK(aligned(s_rows, 4), BSMM_ERR_ALIGN, "s_rows not 4-byte aligned");
  CHECK(sr_m >= 0 && sr_kb >= 0, BSMM_ERR_SCALE_SHAPE, "scale strides must be >= 0");
  {
    const int64_t KB = C / 128;
    const bool rows_ok = R == 1 || sr_m >= 1;
    const bool cols_ok = KB == 1 || sr_kb >= 1;
    const bool disjoint = R == 1 || KB == 1 || sr_m >= KB * sr_kb || sr_kb >= R * sr_m;
    CHECK(rows_ok && cols_ok && disjoint, BSMM_ERR_SCALE_SHAPE,
          "row-scale strides sr_m=%lld sr_kb=%lld make two blocks share a scale",
          (long long)sr_m, (long long)sr_kb);
  }
  QuantArgs a{};
  a.kind = QuantArgs::kFp8RowsColumns;
  a.x = x; a.ldx = ldx; a.x_dtype = x_dtype;
  a.q = q; a.ldq = ldq;
  a.qt = q_t; a.ldqt = ldqt;
  a.scale = s_cols; a.s_m = sc_g; a.s_kb = sc_c;
  a.scale2 = s_rows; a.s2_m = sr_m; a.s2_kb = sr_kb;
  a.M = R; a.K = C;
  if (launch_quant(a, stream) != 0) return fail(BSMM_ERR_HIP, "quantiser launch failed");
  return BSMM_OK;
}

const char* bsmm_status_string(bsmm_status s) {
  switch (s) {
    case BSMM_OK: return "BSMM_OK";
    case BSMM_ERR_NULL: return "BSMM_ERR_NULL";
    case BSMM_ERR_SHAPE: return "BSMM_ERR_SHAPE";
    case BSMM_ERR_SCALE_SHAPE: return "BSMM_ERR_SCALE_SHAPE";
    case BSMM_ERR_LAYOUT: return "BSMM_ERR_LAYOUT";
    case BSMM_ERR_ALIGN: return "BSMM_ERR_ALIGN";
    case BSMM_ERR_DTYPE: return "BSMM_ERR_DTYPE";
    case BSMM_ERR_UNSUPPORTED: return "BSMM_ERR_UNSUPPORTED";
    case BSMM_ERR_HIP: return "BSMM_ERR_HIP";
    case BSMM_ERR_ARG: return "BSMM_ERR_ARG";
  }
  return "BSMM_ERR_UNKNOWN";
}

const char* bsmm_last_error(void) { return g_err; }

int bsmm_version(void) { return BSMM_VERSION; }

}  // extern "C"
