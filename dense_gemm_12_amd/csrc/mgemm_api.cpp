// The C ABI of libmgemm (declared in include/mgemm.h): argument validation,
// the shape-keyed planner (tuning table + cost model) and the launch
// on the caller's stream.  No allocation, no printing, no exceptions across
// the boundary.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <memory>
#include <string>
#include <vector>

#include "../../include/mgemm.h"
#include "gemm_params.hpp"
#include "split16.hpp"

using mg::GemmParams;
using mg::KernelEntry;

namespace {

thread_local int g_last_hip_error = 0;

constexpr int64_t kMaxDim = (int64_t)1 << 31;  // dimensions must be < 2^31
constexpr int64_t kMaxLd = (int64_t)1 << 21;   // per-slice byte offsets stay below 2^31
constexpr int kMaxSplits = 64;                  // split-K ranges per problem
constexpr int64_t kFillWorkgroups = 256;        // one workgroup per CU

int elem_size(int dtype) { return dtype == MG_F32 ? 4 : 2; }

const KernelEntry *entries(int in_type, int *n) {
  switch (in_type) {
    case MG_F32: return mg::entries_f32(n);
    case MG_F16: return mg::entries_f16(n);
    case MG_BF16: return mg::entries_bf16(n);
    default: *n = 0; return nullptr;
  }
}

// ----------------------------------------------------------- tuning table --
struct Rule {
  int in, c, ta, tb;
  int64_t M, N, K;
  std::string config;
  bool ws;     // tuned for the workspace path (split-K and operand repacking allowed)
  int splits;  // ws rules: the tuned split count (0: the planner's fill rule)
};
struct Table {
  std::vector<Rule> rules;
  // "rate" lines: the fraction of the input type's peak each configuration
  // reached at full occupancy when the table was tuned, and its workgroups
  // per CU on that device (index = config id; 0 where the table gives none).
  std::vector<float> rate[3];
  std::vector<int> occ[3];
};
// The loaded table.  A loader builds a new table and publishes it with one
// atomic store; every call plans with the snapshot it loads at its start, so
// loading a table while other threads run GEMMs is safe.
std::shared_ptr<const Table> g_table = std::make_shared<const Table>();

std::shared_ptr<const Table> table_snapshot() { return std::atomic_load(&g_table); }

int find_config(int in_type, const char *name) {
  int n = 0;
  const KernelEntry *e = entries(in_type, &n);
  for (int i = 0; i < n; ++i)
    if (strcmp(e[i].name, name) == 0) return i;
  return -1;
}

int parse_dtype(const char *s) {
  if (!strcmp(s, "f32")) return MG_F32;
  if (!strcmp(s, "f16")) return MG_F16;
  if (!strcmp(s, "bf16")) return MG_BF16;
  return -1;
}

// ----------------------------------------------------------- validation --
struct Problem {
  int in_type, c_type, ta, tb;
  int64_t M, N, K, lda, ldb, ldc;
  float alpha, beta;
  const void *A, *B;
  void *C;
  // A or B is a zero-padded copy made by the library (16-byte loads legal
  // even when the contiguous extent is not a whole number of chunks).
  bool a_padded = false, b_padded = false;
  bool ws_path = false;  // planning for a call that has a workspace
};

bool ranges_overlap(const void *p, int64_t pbytes, const void *q, int64_t qbytes) {
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + (uintptr_t)qbytes && b < a + (uintptr_t)pbytes;
}

// Bytes spanned by a stored rows x cols row-major matrix with leading dim ld.
int64_t span_bytes(int64_t rows, int64_t cols, int64_t ld, int es) {
  if (rows <= 0 || cols <= 0) return 0;
  return ((rows - 1) * ld + cols) * es;
}

mg_status validate(const Problem &p) {
  if (p.ta != MG_N && p.ta != MG_T) return MG_EINVAL;
  if (p.tb != MG_N && p.tb != MG_T) return MG_EINVAL;
  if (p.in_type == MG_F32 && p.c_type != MG_F32) return MG_EINVAL;
  if (p.in_type == MG_F16 && p.c_type != MG_F16 && p.c_type != MG_F32) return MG_EINVAL;
  if (p.in_type == MG_BF16 && p.c_type != MG_BF16 && p.c_type != MG_F32) return MG_EINVAL;
  if (p.M < 0 || p.N < 0 || p.K < 0) return MG_EINVAL;
  // stored shapes
  const int64_t a_rows = p.ta == MG_N ? p.M : p.K, a_cols = p.ta == MG_N ? p.K : p.M;
  const int64_t b_rows = p.tb == MG_N ? p.K : p.N, b_cols = p.tb == MG_N ? p.N : p.K;
  const int64_t one = 1;
  if (p.lda < (a_cols > one ? a_cols : one)) return MG_EINVAL;
  if (p.ldb < (b_cols > one ? b_cols : one)) return MG_EINVAL;
  if (p.ldc < (p.N > one ? p.N : one)) return MG_EINVAL;
  if (p.M == 0 || p.N == 0) return MG_OK;
  if (p.C == nullptr) return MG_EINVAL;
  const bool reads_ab = p.K > 0 && p.alpha != 0.0f;
  if (reads_ab && (p.A == nullptr || p.B == nullptr)) return MG_EINVAL;
  const int es = elem_size(p.in_type), ces = elem_size(p.c_type);
  const int64_t c_bytes = span_bytes(p.M, p.N, p.ldc, ces);
  if (reads_ab) {
    if (ranges_overlap(p.C, c_bytes, p.A, span_bytes(a_rows, a_cols, p.lda, es))) return MG_EINVAL;
    if (ranges_overlap(p.C, c_bytes, p.B, span_bytes(b_rows, b_cols, p.ldb, es))) return MG_EINVAL;
  }
  if (p.M >= kMaxDim || p.N >= kMaxDim || p.K >= kMaxDim) return MG_EUNSUPPORTED;
  if (p.ldc >= kMaxDim) return MG_EUNSUPPORTED;
  if (reads_ab && (p.lda > kMaxLd || p.ldb > kMaxLd)) return MG_EUNSUPPORTED;
  if ((p.M + 15) / 16 * ((p.N + 15) / 16) >= kMaxDim) return MG_EUNSUPPORTED;
  return MG_OK;
}

// 16-byte loads along an operand's contiguous dimension are legal: aligned
// base and pitch, and either whole chunks or a zero-padded library copy.
bool vec_ok(const void *base, int64_t ld, int64_t contiguous_extent, int es, bool padded) {
  const int v = 16 / es;
  return ((uintptr_t)base % 16 == 0) && ((ld * es) % 16 == 0) && (padded || contiguous_extent % v == 0);
}
bool a_vec_ok(const Problem &p) {
  return vec_ok(p.A, p.lda, p.ta == MG_N ? p.K : p.M, elem_size(p.in_type), p.a_padded);
}
bool b_vec_ok(const Problem &p) {
  return vec_ok(p.B, p.ldb, p.tb == MG_T ? p.K : p.N, elem_size(p.in_type), p.b_padded);
}

// ------------------------------------------------------------- planning --
struct Plan {
  int config;
  bool a_vec, b_vec;
  int splits;  // split count a workspace-path rule asks for (0: none)
};

int64_t tiles_for(int64_t M, int64_t N, int bm, int bn) {
  return ((M + bm - 1) / bm) * ((N + bn - 1) / bn);
}

// ----------------------------------------------------------- cost model --
// Workgroups of configuration i (input type in) that fit on one CU, asked of
// the HIP runtime once (-1 without a device).
int runtime_occupancy(int in, int i, const KernelEntry &k) {
  static std::atomic<int> cache[3][64];
  if (i < 64) {
    const int c = cache[in][i].load(std::memory_order_relaxed);
    if (c != 0) return c;
  }
  const int n = k.occupancy ? k.occupancy() : -1;
  if (i < 64) cache[in][i].store(n > 0 ? n : -1, std::memory_order_relaxed);
  return n > 0 ? n : -1;
}

// The table's figure (measured where it was tuned, so plans do not depend
// on whether a device is present), else the runtime's, else a rough figure
// from LDS and wave count.
int occupancy(const Table &t, int in, int i, const KernelEntry &k) {
  if (i < (int)t.occ[in].size() && t.occ[in][i] > 0) return t.occ[in][i];
  int n = runtime_occupancy(in, i, k);
  if (n <= 0) {
    const int by_lds = k.lds_bytes > 0 ? (160 * 1024) / k.lds_bytes : 8;
    const int by_waves = k.threads >= 512 ? 1 : 2;
    n = by_lds < by_waves ? by_lds : by_waves;
    if (n < 1) n = 1;
  }
  return n;
}

// Fraction of the type's peak configuration i reaches at full occupancy:
// the table's measured rate, else a default by kind that favours larger
// tiles (their data reuse grows with the tile's side).
double efficiency(const Table &t, int in, int i, const KernelEntry &k) {
  if (i < (int)t.rate[in].size() && t.rate[in][i] > 0.0f) return t.rate[in][i];
  const double base = k.kind == 1 ? 0.45 : (k.kind == 0 ? 0.30 : 0.40);
  return base * sqrt(sqrt((double)k.bm * k.bn / 65536.0));
}

// Estimated time of configuration i on problem p (units common to one input
// type): the grid runs in rounds of 256 CUs x occupancy workgroups, and a
// round takes (occupancy) tile times at the configuration's full-occupancy
// efficiency.  A partial round is charged as a full one: workgroups that
// share a CU with fewer others do not speed up in proportion.
double est_time(const Table &t, const Problem &p, int i, const KernelEntry &k) {
  const int occ = occupancy(t, p.in_type, i, k);
  const int64_t tiles = tiles_for(p.M, p.N, k.bm, k.bn);
  const int64_t slots = 256 * (int64_t)occ;
  const int64_t rounds = (tiles + slots - 1) / slots;
  return (double)rounds * occ * (2.0 * k.bm * k.bn * (double)(p.K > 0 ? p.K : 1)) / efficiency(t, p.in_type, i, k);
}

bool usable(const KernelEntry &k, const Problem &p) {
  const int c = p.c_type == MG_F32 ? 1 : 0, akc = p.ta == MG_N, bkc = p.tb == MG_T;
  return k.a_vec && k.b_vec && k.fn[c][akc][bkc] != nullptr;
}

// Built-in choice among the fully vectorised configurations that support the
// problem's layout: the least estimated time, ties to the larger tile, then
// table order.  The vector-ALU tiles (kind 2) run only when forced or named
// by the tuning table.
int model_config(const Table &t, const Problem &p, double *est = nullptr) {
  int n = 0;
  const KernelEntry *e = entries(p.in_type, &n);
  int best = -1;
  double best_t = 0.0;
  for (int i = 0; i < n; ++i) {
    if (!usable(e[i], p) || e[i].kind == 2 || e[i].sk) continue;
    const double ti = est_time(t, p, i, e[i]);
    if (best < 0 || ti < best_t * (1.0 - 1e-9) ||
        (ti <= best_t * (1.0 + 1e-9) && (int64_t)e[i].bm * e[i].bn > (int64_t)e[best].bm * e[best].bn)) {
      best = i;
      best_t = ti;
    }
  }
  if (est) *est = best_t;
  return best;
}

int table_config(const Table &t, const Problem &p, bool ws_rules, int *splits = nullptr, double *dist = nullptr) {
  const Rule *best = nullptr;
  double best_d = 1e300;
  for (const Rule &r : t.rules) {
    if (r.in != p.in_type || r.c != p.c_type || r.ta != p.ta || r.tb != p.tb || r.ws != ws_rules) continue;
    const double d = fabs(log2((double)(p.M + 1) / (r.M + 1))) +
                     fabs(log2((double)(p.N + 1) / (r.N + 1))) +
                     fabs(log2((double)(p.K + 1) / (r.K + 1)));
    if (d < best_d) {
      best_d = d;
      best = &r;
    }
  }
  if (!best || best_d > 1.5) return -1;  // only near neighbours are trusted
  if (splits) *splits = best->splits;
  if (dist) *dist = best_d;
  return find_config(p.in_type, best->config.c_str());
}

// The fallback configuration matching the operands' vector legality.
int elem_config(int in_type, bool a_vec, bool b_vec) {
  int n = 0;
  const KernelEntry *e = entries(in_type, &n);
  for (int i = 0; i < n; ++i)
    if (e[i].a_vec == a_vec && e[i].b_vec == b_vec && !(a_vec && b_vec)) return i;
  return -1;
}

Plan plan(const Problem &p) {
  Plan pl;
  pl.a_vec = a_vec_ok(p);
  pl.b_vec = b_vec_ok(p);
  pl.splits = 0;
  if (pl.a_vec && pl.b_vec) {
    const std::shared_ptr<const Table> t = table_snapshot();
    int n = 0;
    const KernelEntry *e = entries(p.in_type, &n);
    int c = p.ws_path ? table_config(*t, p, true, &pl.splits) : -1;
    double dist = 0.0;
    if (c < 0) {
      pl.splits = 0;
      c = table_config(*t, p, false, nullptr, &dist);
      // a rule for a neighbouring shape is kept unless the cost model expects
      // it to be clearly slower here (e.g. a tile that filled the GPU there
      // leaves CUs idle here)
      if (c >= 0 && dist > 0.0 && usable(e[c], p)) {
        double best_t = 0.0;
        const int m = model_config(*t, p, &best_t);
        if (m >= 0 && est_time(*t, p, c, e[c]) > 1.1 * best_t) c = m;
      }
    }
    // a rule naming an element-load variant was tuned on operands 16-byte
    // loads could not read; these can be, so the rule does not apply
    if (c >= 0 && !usable(e[c], p)) c = -1;
    // stream-K needs a workspace: only calls that bring one may use it
    if (c >= 0 && e[c].sk && !p.ws_path) c = -1;
    pl.config = c >= 0 ? c : model_config(*t, p);
  } else {
    pl.config = elem_config(p.in_type, pl.a_vec, pl.b_vec);
  }
  return pl;
}

}  // namespace

// Split-K shape: K cut into ranges of `chunk` (a multiple of bk) values;
// returns the number of ranges, which may be below the requested s.
static int split_shape(int64_t K, int bk, int s, int *chunk) {
  if (s <= 1 || K <= 0) {
    *chunk = (int)K;
    return 1;
  }
  const int64_t per = (K + s - 1) / s;
  const int64_t c = (per + bk - 1) / bk * bk;
  *chunk = (int)c;
  return (int)((K + c - 1) / c);
}

// The planner's split count: 1 unless the tile grid leaves CUs idle; then
// enough ranges to give every CU a workgroup, each at least two slices
// deep, and no more than the workspace holds.
static int auto_splits(const Problem &p, const KernelEntry &k, int64_t ws_bytes, int hint) {
  const int64_t t = tiles_for(p.M, p.N, k.bm, k.bn);
  if (p.K <= 0 || (hint == 0 && t >= kFillWorkgroups)) return 1;
  int64_t s = hint > 0 ? hint : (kFillWorkgroups + t - 1) / t;
  const int64_t by_k = p.K / (2 * (int64_t)k.bk);
  const int64_t by_ws = ws_bytes / (p.M * p.N * 4);
  if (s > by_k) s = by_k;
  if (s > by_ws) s = by_ws;
  if (s > kMaxSplits) s = kMaxSplits;
  return s < 2 ? 1 : (int)s;
}

// Operand repacking for the workspace path: an operand that 16-byte loads
// cannot read (misaligned base or pitch, or a contiguous extent that is not
// a whole number of chunks) is copied into the workspace with its pitch
// rounded up to a chunk and the padding zeroed.  Returns the bytes the copy
// takes (0 when the operand is already loadable or cannot be repacked).
struct Pack {
  int64_t rows, cols, pitch;
  size_t bytes;
};

static Pack pack_shape(const Problem &p, bool is_a) {
  Pack k{0, 0, 0, 0};
  if (is_a ? a_vec_ok(p) : b_vec_ok(p)) return k;
  const int es = elem_size(p.in_type), v = 16 / es;
  const bool kc = is_a ? p.ta == MG_N : p.tb == MG_T;
  const int64_t outer = is_a ? p.M : p.N;
  k.rows = kc ? outer : p.K;
  k.cols = kc ? p.K : outer;
  k.pitch = (k.cols + v - 1) / v * v;
  if (k.pitch > kMaxLd || k.rows <= 0 || k.cols <= 0) return Pack{0, 0, 0, 0};
  k.bytes = ((size_t)k.rows * k.pitch * es + 255) / 256 * 256;
  return k;
}

// Stream-K shape of configuration cfg on problem p: one round of the chip
// (256 CUs x the configuration's workgroups per CU, at most one workgroup
// per slice iteration) and the workspace it needs: 2 partial-tile slots of
// BM x BN floats per workgroup, then one arrival counter per tile.
struct SkShape {
  int grid, ipt, dp_tiles;
  int64_t tiles, total;
  size_t slots_bytes, bytes;
};

static SkShape sk_shape(const Table &t, const Problem &p, int cfg, const KernelEntry &k) {
  SkShape sh{};
  sh.tiles = tiles_for(p.M, p.N, k.bm, k.bn);
  sh.ipt = (int)((p.K + k.bk - 1) / k.bk);
  sh.total = sh.tiles * sh.ipt;
  int64_t g = kFillWorkgroups * (int64_t)occupancy(t, p.in_type, cfg, k);
  if (g > sh.total) g = sh.total;
  sh.grid = (int)(g < 1 ? 1 : g);
  // all rounds but the last two are data-parallel; the last one to two
  // rounds' worth of tiles is shared in slice ranges
  const int64_t rounds = sh.tiles / sh.grid;
  sh.dp_tiles = (int)(rounds >= 2 ? (rounds - 1) * sh.grid : 0);
  sh.slots_bytes = (size_t)2 * sh.grid * k.bm * k.bn * 4;
  sh.bytes = sh.slots_bytes + ((size_t)sh.tiles * 4 + 255) / 256 * 256;
  return sh;
}

// Implementation shared by the entry points.  splits: 0 = planner's choice
// (bounded by the workspace), 1 = no split, >= 2 = that many K ranges.
static mg_status run(const Problem &p, int forced, int splits, void *ws, size_t ws_bytes,
                     void *stream_v, const int *row_exp = nullptr, const int *col_exp = nullptr) {
  mg_status s = validate(p);
  if (s != MG_OK) return s;
  if (splits < 0 || splits > kMaxSplits) return MG_EINVAL;
  if (ws_bytes > 0 && (ws == nullptr || (uintptr_t)ws % 16 != 0)) return MG_EINVAL;
  if (splits > 1 && (int64_t)ws_bytes / splits < p.M * p.N * 4) return MG_EINVAL;
  if (ws_bytes > 0 && p.M > 0 && p.N > 0) {
    const int64_t wb = (int64_t)ws_bytes;
    const int es = elem_size(p.in_type);
    const int64_t a_rows = p.ta == MG_N ? p.M : p.K, a_cols = p.ta == MG_N ? p.K : p.M;
    const int64_t b_rows = p.tb == MG_N ? p.K : p.N, b_cols = p.tb == MG_N ? p.N : p.K;
    if (ranges_overlap(ws, wb, p.C, span_bytes(p.M, p.N, p.ldc, elem_size(p.c_type))) ||
        ranges_overlap(ws, wb, p.A, span_bytes(a_rows, a_cols, p.lda, es)) ||
        ranges_overlap(ws, wb, p.B, span_bytes(b_rows, b_cols, p.ldb, es)))
      return MG_EINVAL;
  }
  if (p.M == 0 || p.N == 0) return MG_OK;
  int n = 0;
  const KernelEntry *e = entries(p.in_type, &n);
  if (forced < -1 || forced >= n) return MG_EINVAL;
  hipStream_t stream = static_cast<hipStream_t>(stream_v);

  GemmParams gp{};
  gp.A = p.A;
  gp.B = p.B;
  gp.C = p.C;
  gp.lda = p.lda;
  gp.ldb = p.ldb;
  gp.ldc = p.ldc;
  gp.M = (int)p.M;
  gp.N = (int)p.N;
  gp.K = (int)p.K;
  gp.alpha = p.alpha;
  gp.beta = p.beta;
  gp.splits = 1;
  gp.k_chunk = (int)p.K;
  gp.ws = nullptr;
  gp.row_exp = row_exp;
  gp.col_exp = col_exp;
  const int ces = elem_size(p.c_type);
  // 1: four-element (16-byte fp32, 8-byte 16-bit) C accesses are legal;
  // 2: eight-element (16-byte) 16-bit C accesses too
  gp.c_vec = ((uintptr_t)p.C % (ces == 4 ? 16 : 8) == 0) && (p.ldc % 4 == 0);
  if (gp.c_vec && ces == 2 && (uintptr_t)p.C % 16 == 0 && p.ldc % 8 == 0) gp.c_vec = 2;
  const int c_idx = p.c_type == MG_F32 ? 0 : (p.c_type == MG_F16 ? 1 : 2);

  hipError_t err;
  if (p.K == 0 || p.alpha == 0.0f) {
    err = mg::scale_launcher(c_idx)(gp, stream);
  } else if (ws_bytes > 0 && !(p.ws_path)) {
    // Workspace path: repack what 16-byte loads cannot read (keeping room
    // for a forced split), then plan and split with the rest.
    Problem q = p;
    q.ws_path = true;
    char *w = static_cast<char *>(ws);
    size_t used = 0;
    const size_t reserve = splits > 1 ? (size_t)splits * p.M * p.N * 4 : 0;
    for (int side = 0; side < 2; ++side) {
      const Pack k = pack_shape(q, side == 0);
      if (k.bytes == 0 || used + k.bytes + reserve > ws_bytes) continue;
      const void *src = side == 0 ? q.A : q.B;
      const int64_t ld = side == 0 ? q.lda : q.ldb;
      err = mg::launch_pack(elem_size(q.in_type), src, ld, k.rows, k.cols, w + used, k.pitch, stream);
      if (err != hipSuccess) {
        g_last_hip_error = (int)err;
        return MG_EHIP;
      }
      if (side == 0) {
        q.A = w + used;
        q.lda = k.pitch;
        q.a_padded = true;
      } else {
        q.B = w + used;
        q.ldb = k.pitch;
        q.b_padded = true;
      }
      used += k.bytes;
    }
    return run(q, forced, splits, w + used, ws_bytes - used, stream_v, row_exp, col_exp);
  } else {
    Plan pl = plan(p);
    int cfg = forced >= 0 ? forced : pl.config;
    if (cfg < 0) return MG_EUNSUPPORTED;
    SkShape sk{};
    if (e[cfg].sk) {
      const std::shared_ptr<const Table> t = table_snapshot();
      sk = sk_shape(*t, p, cfg, e[cfg]);
      if (sk.total >= kMaxDim) return MG_EUNSUPPORTED;
      if (ws == nullptr || ws_bytes < sk.bytes) {
        if (forced >= 0) return MG_EUNSUPPORTED;
        cfg = model_config(*t, p);  // the planner's stream-K pick without room for it
        if (cfg < 0) return MG_EUNSUPPORTED;
      }
    }
    const KernelEntry &k = e[cfg];
    if ((k.a_vec && !pl.a_vec) || (k.b_vec && !pl.b_vec)) return MG_EUNSUPPORTED;
    const int ci = (p.c_type == MG_F32) ? 1 : 0, ak = p.ta == MG_N ? 1 : 0, bk = p.tb == MG_T ? 1 : 0;
    if (k.fn[ci][ak][bk] == nullptr) return MG_EUNSUPPORTED;
    gp.tiles_m = (int)((p.M + k.bm - 1) / k.bm);
    gp.tiles_n = (int)((p.N + k.bn - 1) / k.bn);
    gp.group_m = 8;
    const int c_is_f32 = (p.c_type == MG_F32) ? 1 : 0;
    const int a_kc = p.ta == MG_N ? 1 : 0, b_kc = p.tb == MG_T ? 1 : 0;
    if (k.sk) {
      // stream-K: partial-tile slots, then the zeroed arrival counters
      gp.ws = static_cast<float *>(ws);
      gp.sk_cnt = reinterpret_cast<int *>(static_cast<char *>(ws) + sk.slots_bytes);
      gp.sk_grid = sk.grid;
      gp.sk_ipt = sk.ipt;
      gp.sk_dp_tiles = sk.dp_tiles;
      err = mg::launch_zero_ints(gp.sk_cnt, (int)sk.tiles, stream);
      if (err == hipSuccess) err = k.fn[c_is_f32][a_kc][b_kc](gp, stream);
    } else {
      int chunk = 0;
      const int sp = split_shape(p.K, k.bk,
                                 splits == 0 ? auto_splits(p, k, (int64_t)ws_bytes, pl.splits) : splits, &chunk);
      if ((int64_t)gp.tiles_m * gp.tiles_n * sp >= kMaxDim) return MG_EUNSUPPORTED;
      gp.splits = sp;
      gp.k_chunk = chunk;
      gp.ws = static_cast<float *>(ws);
      err = k.fn[c_is_f32][a_kc][b_kc](gp, stream);
      if (err == hipSuccess && sp > 1) err = mg::reduce_launcher(c_idx)(gp, stream);
    }
  }
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return MG_EHIP;
  }
  return MG_OK;
}

// ---------------------------------------------- fp32 through split fp16 --
static constexpr int64_t kSplit16Max = (int64_t)1 << 22;  // grid-dimension limits of the split kernels

struct Split16Layout {
  int64_t Kp;
  int parts;
  size_t a, b, re, ce, pm, total;  // byte offsets of the workspace sections
};

static Split16Layout split16_layout(int64_t M, int64_t N, int64_t K) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  Split16Layout L{};
  L.Kp = (K + 63) / 64 * 64;
  L.parts = (int)(K / 64 < 1 ? 1 : (K / 64 > 64 ? 64 : K / 64));
  L.a = 0;
  L.b = L.a + up((size_t)M * 3 * L.Kp * 2);
  L.re = L.b + up((size_t)N * 3 * L.Kp * 2);
  L.ce = L.re + up((size_t)M * 4);
  L.pm = L.ce + up((size_t)N * 4);
  L.total = L.pm + up((size_t)L.parts * (M > N ? M : N) * 4);
  return L;
}

static mg_status split16_run(const Problem &p, void *ws, size_t ws_bytes, void *stream_v) {
  mg_status s = validate(p);
  if (s != MG_OK) return s;
  if (p.M == 0 || p.N == 0) return MG_OK;
  if (p.K == 0 || p.alpha == 0.0f) return run(p, -1, 1, nullptr, 0, stream_v);  // C = beta * C
  if (p.M > kSplit16Max || p.N > kSplit16Max || p.K > kSplit16Max) return MG_EUNSUPPORTED;
  const Split16Layout L = split16_layout(p.M, p.N, p.K);
  if (3 * L.Kp > kMaxLd) return MG_EUNSUPPORTED;
  if (ws == nullptr || (uintptr_t)ws % 16 != 0 || ws_bytes < L.total) return MG_EINVAL;
  {
    const int64_t wb = (int64_t)ws_bytes;
    const int64_t a_rows = p.ta == MG_N ? p.M : p.K, a_cols = p.ta == MG_N ? p.K : p.M;
    const int64_t b_rows = p.tb == MG_N ? p.K : p.N, b_cols = p.tb == MG_N ? p.N : p.K;
    if (ranges_overlap(ws, wb, p.C, span_bytes(p.M, p.N, p.ldc, 4)) ||
        ranges_overlap(ws, wb, p.A, span_bytes(a_rows, a_cols, p.lda, 4)) ||
        ranges_overlap(ws, wb, p.B, span_bytes(b_rows, b_cols, p.ldb, 4)))
      return MG_EINVAL;
  }
  char *w = static_cast<char *>(ws);
  mg::Split16Plan sp{};
  sp.A = static_cast<const float *>(p.A);
  sp.B = static_cast<const float *>(p.B);
  sp.lda = p.lda;
  sp.ldb = p.ldb;
  sp.M = (int)p.M;
  sp.N = (int)p.N;
  sp.K = (int)p.K;
  sp.Kp = (int)L.Kp;
  sp.a_rows_contiguous = p.ta == MG_N;
  sp.b_cols_contiguous = p.tb == MG_T;
  sp.parts = L.parts;
  sp.Ap = reinterpret_cast<uint16_t *>(w + L.a);
  sp.Bp = reinterpret_cast<uint16_t *>(w + L.b);
  sp.row_exp = reinterpret_cast<int *>(w + L.re);
  sp.col_exp = reinterpret_cast<int *>(w + L.ce);
  sp.pmax = reinterpret_cast<float *>(w + L.pm);
  hipError_t err = mg::split16_prepare(sp, static_cast<hipStream_t>(stream_v));
  if (err != hipSuccess) {
    g_last_hip_error = (int)err;
    return MG_EHIP;
  }
  // A' B'^T over K' = 3 Kp: the TN fp16 GEMM with fp32 C and the unscaling.
  const int64_t kq = 3 * L.Kp;
  Problem q{MG_F16, MG_F32, MG_N, MG_T, p.M, p.N, kq, kq, kq, p.ldc, p.alpha, p.beta, sp.Ap, sp.Bp, p.C};
  return run(q, -1, 1, nullptr, 0, stream_v, sp.row_exp, sp.col_exp);
}

extern "C" {

mg_status gemm_f32_split16(mg_op ta, mg_op tb, int64_t M, int64_t N, int64_t K, float alpha,
                           const float *A, int64_t lda, const float *B, int64_t ldb, float beta,
                           float *C, int64_t ldc, void *workspace, size_t workspace_bytes,
                           void *stream) {
  Problem p{MG_F32, MG_F32, (int)ta, (int)tb, M, N, K, lda, ldb, ldc, alpha, beta, A, B, C};
  return split16_run(p, workspace, workspace_bytes, stream);
}

size_t mg_split16_workspace_size(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return split16_layout(M, N, K).total;
}

mg_status gemm_f32_cfg(int config, mg_op ta, mg_op tb, int64_t M, int64_t N, int64_t K,
                       float alpha, const float *A, int64_t lda, const float *B, int64_t ldb,
                       float beta, float *C, int64_t ldc, void *stream) {
  Problem p{MG_F32, MG_F32, (int)ta, (int)tb, M, N, K, lda, ldb, ldc, alpha, beta, A, B, C};
  return run(p, config, 1, nullptr, 0, stream);
}

mg_status gemm_f16_cfg(int config, mg_op ta, mg_op tb, int64_t M, int64_t N, int64_t K,
                       float alpha, const uint16_t *A, int64_t lda, const uint16_t *B,
                       int64_t ldb, float beta, void *C, mg_dtype c_type, int64_t ldc,
                       void *stream) {
  Problem p{MG_F16, (int)c_type, (int)ta, (int)tb, M, N, K, lda, ldb, ldc, alpha, beta, A, B, C};
  return run(p, config, 1, nullptr, 0, stream);
}

mg_status gemm_bf16_cfg(int config, mg_op ta, mg_op tb, int64_t M, int64_t N, int64_t K,
                        float alpha, const uint16_t *A, int64_t lda, const uint16_t *B,
                        int64_t ldb, float beta, void *C, mg_dtype c_type, int64_t ldc,
                        void *stream) {
  Problem p{MG_BF16, (int)c_type, (int)ta, (int)tb, M, N, K, lda, ldb, ldc, alpha, beta, A, B, C};
  return run(p, config, 1, nullptr, 0, stream);
}

mg_status gemm_f32(mg_op ta, mg_op tb, int64_t M, int64_t N, int64_t K, float alpha,
                   const float *A, int64_t lda, const float *B, int64_t ldb, float beta, float *C,
                   int64_t ldc, void *stream) {
  return gemm_f32_cfg(-1, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

mg_status gemm_f16(mg_op ta, mg_op tb, int64_t M, int64_t N, int64_t K, float alpha,
                   const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, float beta,
                   void *C, mg_dtype c_type, int64_t ldc, void *stream) {
  return gemm_f16_cfg(-1, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream);
}

mg_status gemm_bf16(mg_op ta, mg_op tb, int64_t M, int64_t N, int64_t K, float alpha,
                    const uint16_t *A, int64_t lda, const uint16_t *B, int64_t ldb, float beta,
                    void *C, mg_dtype c_type, int64_t ldc, void *stream) {
  return gemm_bf16_cfg(-1, ta, tb, M, N, K, alpha, A, lda, B, ldb, beta, C, c_type, ldc, stream);
}

mg_status gemm_ex(mg_dtype in_type, mg_dtype c_type, mg_op ta, mg_op tb, int64_t M, int64_t N,
                  int64_t K, float alpha, const void *A, int64_t lda, const void *B, int64_t ldb,
                  float beta, void *C, int64_t ldc, void *workspace, size_t workspace_bytes,
                  int config, int splits, void *stream) {
  if ((int)in_type < MG_F32 || (int)in_type > MG_BF16) return MG_EINVAL;
  Problem p{(int)in_type, (int)c_type, (int)ta, (int)tb, M, N, K, lda, ldb, ldc, alpha, beta, A, B, C};
  return run(p, config, splits, workspace, workspace_bytes, stream);
}

size_t mg_workspace_size(mg_dtype in_type, mg_dtype c_type, mg_op ta, mg_op tb, int64_t M, int64_t N,
                         int64_t K, int64_t lda, int64_t ldb) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  if ((int)in_type < MG_F32 || (int)in_type > MG_BF16) return 0;
  // Planned as for 16-byte-aligned base pointers with the given leading dimensions.
  Problem p{(int)in_type, (int)c_type, (int)ta, (int)tb, M, N, K, lda, ldb, N, 1.0f, 0.0f,
            (const void *)(uintptr_t)4096, (const void *)(uintptr_t)4096, nullptr};
  p.ws_path = true;
  size_t packed = 0;
  for (int side = 0; side < 2; ++side) {
    const Pack k = pack_shape(p, side == 0);
    if (k.bytes == 0) continue;
    packed += k.bytes;
    if (side == 0) {
      p.lda = k.pitch;
      p.a_padded = true;
    } else {
      p.ldb = k.pitch;
      p.b_padded = true;
    }
  }
  const Plan pl = plan(p);
  if (pl.config < 0) return packed;
  int n = 0;
  const KernelEntry &k = entries(p.in_type, &n)[pl.config];
  if (k.sk) return packed + sk_shape(*table_snapshot(), p, pl.config, k).bytes;
  int chunk = 0;
  const int sp = split_shape(K, k.bk, auto_splits(p, k, INT64_MAX, pl.splits), &chunk);
  return packed + (sp > 1 ? (size_t)sp * (size_t)M * (size_t)N * 4 : 0);
}

int mg_chosen_config_ws(mg_dtype in_type, mg_dtype c_type, mg_op ta, mg_op tb, int64_t M, int64_t N,
                        int64_t K, int64_t lda, int64_t ldb) {
  if (M <= 0 || N <= 0 || K <= 0) return -1;
  if ((int)in_type < MG_F32 || (int)in_type > MG_BF16) return -1;
  Problem p{(int)in_type, (int)c_type, (int)ta, (int)tb, M, N, K, lda, ldb, N, 1.0f, 0.0f,
            (const void *)(uintptr_t)4096, (const void *)(uintptr_t)4096, nullptr};
  p.ws_path = true;
  for (int side = 0; side < 2; ++side) {
    const Pack k = pack_shape(p, side == 0);
    if (k.bytes == 0) continue;
    if (side == 0) {
      p.lda = k.pitch;
      p.a_padded = true;
    } else {
      p.ldb = k.pitch;
      p.b_padded = true;
    }
  }
  return plan(p).config;
}

int mg_num_configs(mg_dtype in_type) {
  int n = 0;
  entries((int)in_type, &n);
  return n;
}

const char *mg_config_name(mg_dtype in_type, int config) {
  int n = 0;
  const KernelEntry *e = entries((int)in_type, &n);
  if (config < 0 || config >= n) return nullptr;
  return e[config].name;
}

int mg_chosen_config(mg_dtype in_type, mg_dtype c_type, mg_op ta, mg_op tb, int64_t M, int64_t N,
                     int64_t K) {
  // Planned as for 16-byte-aligned operands with contiguous leading dimensions.
  const int64_t lda = ta == MG_N ? K : M, ldb = tb == MG_N ? N : K;
  Problem p{(int)in_type, (int)c_type, (int)ta, (int)tb, M, N, K, lda, ldb, N, 1.0f, 0.0f,
            (const void *)(uintptr_t)4096, (const void *)(uintptr_t)4096, nullptr};
  if (M <= 0 || N <= 0 || K <= 0) return -1;
  return plan(p).config;
}

mg_status mg_load_tune_table(const char *path) {
  if (!path) return MG_EINVAL;
  FILE *f = fopen(path, "r");
  if (!f) return MG_EINVAL;
  Table table;
  std::vector<Rule> &rules = table.rules;
  char line[512];
  bool ok = true;
  bool continuation = false;  // inside a line longer than the buffer
  while (fgets(line, sizeof line, f)) {
    const bool whole = strchr(line, '\n') != nullptr || feof(f);
    const bool skip = continuation || line[0] == '#' || line[0] == '\n' || line[0] == '\0';
    continuation = !whole;
    if (skip) continue;
    if (!whole) {  // a rule never needs this much text
      ok = false;
      break;
    }
    if (!strncmp(line, "rate ", 5)) {  // rate <in> <config> <fraction of peak> <workgroups per CU>
      char in[16], cfg[128];
      float frac = 0.0f;
      int occ = 0;
      const int in_t = sscanf(line, "rate %15s %127s %f %d", in, cfg, &frac, &occ) == 4 ? parse_dtype(in) : -1;
      const int id = in_t >= 0 ? find_config(in_t, cfg) : -1;
      if (id < 0 || !(frac > 0.0f && frac <= 1.0f) || occ < 1 || occ > 32) {
        ok = false;
        break;
      }
      if ((int)table.rate[in_t].size() <= id) {
        table.rate[in_t].resize(id + 1, 0.0f);
        table.occ[in_t].resize(id + 1, 0);
      }
      table.rate[in_t][id] = frac;
      table.occ[in_t][id] = occ;
      continue;
    }
    char in[16], c[16], ta[4], tb[4], cfg[128], tag[8] = {0}, sp[16] = {0};
    long long M, N, K;
    const int got = sscanf(line, "%15s %15s %3s %3s %lld %lld %lld %127s %7s %15s", in, c, ta, tb, &M, &N, &K,
                           cfg, tag, sp);
    int rule_splits = 0;
    if (got < 8 || (got >= 9 && strcmp(tag, "ws") != 0) ||
        (got == 10 && (sscanf(sp, "s=%d", &rule_splits) != 1 || rule_splits < 1 || rule_splits > kMaxSplits))) {
      ok = false;
      break;
    }
    Rule r;
    r.in = parse_dtype(in);
    r.c = parse_dtype(c);
    r.ta = !strcmp(ta, "N") ? MG_N : (!strcmp(ta, "T") ? MG_T : -1);
    r.tb = !strcmp(tb, "N") ? MG_N : (!strcmp(tb, "T") ? MG_T : -1);
    r.M = M;
    r.N = N;
    r.K = K;
    r.config = cfg;
    r.ws = got >= 9;
    r.splits = rule_splits;
    if (r.in < 0 || r.c < 0 || r.ta < 0 || r.tb < 0 || find_config(r.in, cfg) < 0) {
      ok = false;
      break;
    }
    rules.push_back(r);
  }
  fclose(f);
  if (!ok) return MG_EINVAL;
  std::atomic_store(&g_table, std::shared_ptr<const Table>(std::make_shared<const Table>(std::move(table))));
  return MG_OK;
}

int mg_tune_table_size(void) { return (int)table_snapshot()->rules.size(); }

int mg_config_occupancy(mg_dtype in_type, int config) {
  int n = 0;
  const KernelEntry *e = entries((int)in_type, &n);
  if (!e || config < 0 || config >= n) return -1;
  return runtime_occupancy((int)in_type, config, e[config]);
}

const char *mg_status_str(mg_status s) {
  switch (s) {
    case MG_OK: return "ok";
    case MG_EINVAL: return "invalid argument";
    case MG_EUNSUPPORTED: return "unsupported problem (outside the kernels' addressing range)";
    case MG_EHIP: return "HIP launch error";
    case MG_ESCRATCH: return "problem needs more scratch than the no-allocation entry point's fixed array holds";
    default: return "unknown status";
  }
}

int mg_last_hip_error(void) { return g_last_hip_error; }

const char *mg_version(void) { return "mgemm 0.1 (gfx950)"; }

}  // extern "C"
