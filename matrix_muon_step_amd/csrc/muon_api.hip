// C ABI of libmuon: argument validation, execution plan, workspace layout,
// descriptor upload and the grouped launch sequence of one Muon step
// (Muon synthesis note on papers.chlience.com, section 4).
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "muon.h"
#include "muon_internal.h"

using namespace muon;

// Workspace of muon_step_static: a file-scope device array, one copy per GPU
// the library runs on, held until the process ends.  In host code the
// array's name is only a host-side stand-in; its device address on the
// current device comes from hipGetSymbolAddress, taken once per device and
// kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[MUON_STATIC_WORKSPACE_BYTES];

namespace {

thread_local std::string g_last_error;

muon_status_t fail(muon_status_t st, const std::string& msg) {
  g_last_error = msg;
  return st;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x, size_t a = kAlign) { return (x + a - 1) / a * a; }
int64_t round_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

// One matrix as the planner sees it (host side, before pointers are bound).
struct Item {
  float* W;
  const void* G;   // gradient, or M in orthogonalise-only mode
  float* B;
  int64_t rows, cols;
  float lr_scale;
  float lr_wd;
  int32_t flags;
};

// Prefix tables uploaded after the descriptors.  Fixed ones first, then one
// table per kernel configuration for the symmetric stages (Gram and
// polynomial share it) and one per configuration for the BX stage.
enum Table { kTabMom = 0, kTabPrep, kTabUpd, kTabSmallGram, kTabSmallPoly, kTabFixed };
constexpr int kNumTables = kTabFixed + 2 * kNumCfg;
int tab_sym(int cfg) { return kTabFixed + cfg; }
int tab_bx(int cfg) { return kTabFixed + kNumCfg + cfg; }

struct Plan {
  std::vector<MatDesc> descs;
  std::vector<int32_t> pre[kNumTables];
  int64_t tot[kNumTables] = {};
  size_t table_bytes = 0;   // descriptors + prefix tables
  size_t total_bytes = 0;
  std::vector<int64_t> x_offset;
  int ns_steps = 0;
};

struct Range {
  uintptr_t lo, hi;
  bool writable;
  const char* what;
  int64_t idx;
};

muon_status_t check_aliasing(std::vector<Range>& rs) {
  std::sort(rs.begin(), rs.end(), [](const Range& a, const Range& b) { return a.lo < b.lo; });
  uintptr_t max_end_any = 0, max_end_w = 0;
  const Range* last_any = nullptr;
  const Range* last_w = nullptr;
  for (const Range& r : rs) {
    if (r.lo == r.hi) continue;
    if (r.lo < max_end_w) {
      return fail(MUON_ERR_ALIAS, std::string("muon: ") + r.what + " of matrix " +
                                      std::to_string(r.idx) + " overlaps " + last_w->what +
                                      " of matrix " + std::to_string(last_w->idx));
    }
    if (r.writable && r.lo < max_end_any) {
      return fail(MUON_ERR_ALIAS, std::string("muon: ") + r.what + " of matrix " +
                                      std::to_string(r.idx) + " overlaps " + last_any->what +
                                      " of matrix " + std::to_string(last_any->idx));
    }
    if (r.hi > max_end_any) { max_end_any = r.hi; last_any = &r; }
    if (r.writable && r.hi > max_end_w) { max_end_w = r.hi; last_w = &r; }
  }
  return MUON_OK;
}

bool finite(float x) { return isfinite(x); }

// Kernel configurations of one matrix: (symmetric stages, BX stage).
struct MatCfg {
  int sym, bx;
  int64_t m_pad, n_pad;
};

int64_t upper_tiles(int64_t mp, int t) {
  const int64_t nt = mp / t;
  return nt * (nt + 1) / 2;
}

// Choice of kernel configurations for a Gram side m and long side n: the
// combination with the least estimated time, i.e. padded matrix-core work
// (upper tiles for the symmetric products) divided by each configuration's
// relative sustained rate on gfx950, from measurements of these kernels:
// 32x32 256-tiles 1.10, 320x256 BX tiles 1.04, 160x256 BX tiles 1.00,
// 16x16 160-tiles 0.85, 128-tiles 0.70.  The choice depends on the shape
// alone; the one per-call change made afterwards (256-tiles to 128-tiles in
// a small call) keeps the arithmetic, so a matrix gives the same bits
// whatever else a call holds.
MatCfg choose_cfg(int64_t m, int64_t n) {
  struct Cand { int sym, bx; };
  static const Cand cands[] = {
      {kCfgG256, kCfgG256}, {kCfgT160, kCfgW160}, {kCfgT160, kCfgT160}, {kCfgT128, kCfgT128}, {kCfgT160, kCfgW320}};
  static const double rate[kNumCfg] = {1.10, 1.00, 0.85, 0.70, 1.04};
  MatCfg best{};
  double best_cost = 0.0;
  for (const Cand& c : cands) {
    const int64_t mp = round_up(m, kCfgRows[c.sym]);
    if (mp % kCfgRows[c.bx] != 0) continue;
    const int64_t np = round_up(n, kCfgCols[c.bx]);
    const int64_t kg = round_up(n, 32);
    const int t = kCfgRows[c.sym];
    const double sym_work = static_cast<double>(upper_tiles(mp, t)) * 2.0 * t * t * (kg + mp);
    const double bx_work = 2.0 * static_cast<double>(mp) * np * mp;
    const double cost = sym_work / rate[c.sym] + bx_work / rate[c.bx];
    if (best_cost == 0.0 || cost < best_cost) {
      best_cost = cost;
      best = MatCfg{c.sym, c.bx, mp, np};
    }
  }
  return best;
}

// A call whose 256-tile BX launch would have fewer tiles than this (two per
// CU of the 256-CU MI355X) runs its 256-tile matrices on 128-tiles.
constexpr int64_t kSmallCallTiles = 512;

// Gram-side tile rows per group of the BX tile order (wide-tile kernels):
// all of them, so the tiles of one long-side column run together and share
// their X^T panel in L2.
int bx_group(const MatCfg& cfg) { return static_cast<int>(cfg.m_pad / kCfgRows[cfg.bx]); }

// Validates shapes and scalars of every item and fills the plan (offsets
// relative to a workspace base of 0).  Pointer checks happen separately.
muon_status_t make_plan(const std::vector<Item>& items, int ns_steps, Plan& plan) {
  const int64_t n = static_cast<int64_t>(items.size());
  if (n > (1 << 20)) return fail(MUON_ERR_UNSUPPORTED, "muon: more than 2^20 matrices");
  plan = Plan();
  plan.ns_steps = ns_steps;
  plan.descs.resize(n);
  plan.x_offset.resize(n);
  for (auto& v : plan.pre) v.resize(n + 1);

  size_t off = 0;
  off += align_up(sizeof(MatDesc) * n);
  // prefix tables, then the call's count of matrices marked for the prep
  // pass (uploaded as zero with the table)
  off += align_up(sizeof(int32_t) * (kNumTables * (n + 1) + 1));
  plan.table_bytes = off;

  // Kernel configurations: by shape (choose_cfg), then, for a call whose
  // 256-tile BX launch would give the GPU fewer than two tiles per CU, the
  // same arithmetic on 128-tiles (G128 computes exactly what G256 does, so
  // the bits do not depend on the choice).
  std::vector<MatCfg> cfgs(n);
  int64_t g256_bx_tiles = 0;
  for (int64_t i = 0; i < n; ++i) {
    const Item& it = items[i];
    if (it.rows < 1 || it.cols < 1)
      return fail(MUON_ERR_INVALID_ARG, "muon: matrix " + std::to_string(i) + " has rows or cols < 1");
    if (it.rows > MUON_MAX_DIM || it.cols > MUON_MAX_DIM)
      return fail(MUON_ERR_UNSUPPORTED, "muon: matrix " + std::to_string(i) + " exceeds MUON_MAX_DIM");
    const int64_t m = std::min(it.rows, it.cols), nn = std::max(it.rows, it.cols);
    if (m > MUON_MAX_GRAM)
      return fail(MUON_ERR_UNSUPPORTED, "muon: matrix " + std::to_string(i) + " has min(rows, cols) > MUON_MAX_GRAM");
    if (!finite(it.lr_scale) || !finite(it.lr_wd))
      return fail(MUON_ERR_INVALID_ARG, "muon: matrix " + std::to_string(i) + " has a non-finite lr*scale or lr*weight_decay");
    cfgs[i] = m <= kSmallGram ? MatCfg{-1, -1, kSmallGram, round_up(nn, kSmallChunk)} : choose_cfg(m, nn);
    if (cfgs[i].bx == kCfgG256)
      g256_bx_tiles += (cfgs[i].m_pad / kCfgRows[kCfgG256]) * (cfgs[i].n_pad / kCfgCols[kCfgG256]);
  }
  if (g256_bx_tiles > 0 && g256_bx_tiles < kSmallCallTiles) {
    for (int64_t i = 0; i < n; ++i) {
      if (cfgs[i].bx != kCfgG256) continue;
      const int64_t m = std::min(items[i].rows, items[i].cols), nn = std::max(items[i].rows, items[i].cols);
      cfgs[i] = MatCfg{kCfgG128, kCfgG128, round_up(m, kCfgRows[kCfgG128]), round_up(nn, kCfgCols[kCfgG128])};
    }
  }

  int64_t total_partials = 0;
  int64_t total_slots = 0;
  for (int64_t i = 0; i < n; ++i) {
    const Item& it = items[i];
    const bool tr = it.rows > it.cols;
    const int64_t m = tr ? it.cols : it.rows;
    const int64_t nn = tr ? it.rows : it.cols;
    MatDesc& d = plan.descs[i];
    memset(&d, 0, sizeof(d));
    const bool small = m <= kSmallGram;
    const MatCfg cfg = cfgs[i];
    d.rows = it.rows;
    d.cols = it.cols;
    d.m = static_cast<int32_t>(m);
    d.n = static_cast<int32_t>(nn);
    d.sym_cfg = cfg.sym;
    d.bx_cfg = cfg.bx;
    d.m_pad = static_cast<int32_t>(cfg.m_pad);
    d.n_pad = static_cast<int32_t>(cfg.n_pad);
    d.k_gram = static_cast<int32_t>(round_up(nn, 32));
    d.bx_group = small ? 0 : bx_group(cfg);
    // The wide-tile BX kernels apply the update from their last launch.
    const bool fused = !small && ns_steps > 0 && cfg_wide(cfg.bx);
    // The normalisation is folded into the first iteration where there is
    // one and the iterate is the bf16 pair.
    const bool fold = !small && ns_steps > 0;
    d.flags = it.flags | (tr ? kTransposed : 0) | (small ? kSmall : 0) | (fused ? kFusedUpd : 0) |
              (fold ? kFold : 0);
    d.lr_scale = it.lr_scale;
    d.lr_wd = it.lr_wd;
    d.s_chunks = small ? d.n_pad / kSmallChunk : 0;
    int64_t work[kNumTables] = {};
    work[kTabPrep] = ((d.m_pad + kEwTile - 1) / kEwTile) * ((d.n_pad + kEwTile - 1) / kEwTile);
    work[kTabMom] = ((d.m_pad + mom_tile_i(tr) - 1) / mom_tile_i(tr)) *
                    ((d.n_pad + mom_tile_j(tr) - 1) / mom_tile_j(tr));
    d.mom_blocks = static_cast<int32_t>(work[kTabMom]);
    total_partials += d.mom_blocks;
    work[kTabUpd] = fused ? 0 : ((it.rows + kEwTile - 1) / kEwTile) * ((it.cols + kEwTile - 1) / kEwTile);
    if (small) {
      work[kTabSmallGram] = d.s_chunks;
      work[kTabSmallPoly] = 1;
    } else {
      work[tab_sym(cfg.sym)] = upper_tiles(d.m_pad, kCfgRows[cfg.sym]);
      work[tab_bx(cfg.bx)] = (d.m_pad / kCfgRows[cfg.bx]) * (d.n_pad / kCfgCols[cfg.bx]);
    }
    // Diagnostics partials: one per wave of the kernel that writes W.
    d.diag_slots = static_cast<int32_t>(fused ? work[tab_bx(cfg.bx)] * kCfgWaves[cfg.bx] : work[kTabUpd] * 4);
    total_slots += d.diag_slots;
    const int64_t lim = (int64_t{1} << 31) - 1;
    for (int k = 0; k < kNumTables; ++k) {
      plan.pre[k][i] = static_cast<int32_t>(plan.tot[k]);
      plan.tot[k] += work[k];
      if (plan.tot[k] > lim) return fail(MUON_ERR_UNSUPPORTED, "muon: too many work-groups for one launch");
    }
  }
  for (int k = 0; k < kNumTables; ++k) plan.pre[k][n] = static_cast<int32_t>(plan.tot[k]);

  // Partials and sigma, and the scratch of the diagnostics (always
  // reserved, so one workspace size serves muon_step and muon_step_diag).
  const size_t partial_off = off;
  off += align_up(sizeof(float) * total_partials);
  const size_t sigma_off = off;
  off += align_up(sizeof(float) * 4 * n);
  const size_t bad_off = off;
  off += align_up(sizeof(int32_t) * total_partials);
  const size_t mstat_off = off;
  off += align_up(sizeof(float) * 2 * n);
  const size_t slot_off = off;
  off += align_up(sizeof(DiagPart) * total_slots);
  int64_t pcur = 0, scur = 0;
  for (int64_t i = 0; i < n; ++i) {
    MatDesc& d = plan.descs[i];
    d.partials = reinterpret_cast<float*>(partial_off + sizeof(float) * pcur);
    d.mom_bad = reinterpret_cast<int32_t*>(bad_off + sizeof(int32_t) * pcur);
    pcur += d.mom_blocks;
    d.sigma = reinterpret_cast<float*>(sigma_off + sizeof(float) * 4 * i);
    d.mstat = reinterpret_cast<float*>(mstat_off + sizeof(float) * 2 * i);
    d.diag_part = reinterpret_cast<DiagPart*>(slot_off + sizeof(DiagPart) * scur);
    scur += d.diag_slots;
  }
  // Iterate and Gram buffers.
  for (int64_t i = 0; i < n; ++i) {
    MatDesc& d = plan.descs[i];
    plan.x_offset[i] = static_cast<int64_t>(off);
    if (d.flags & kSmall) {
      const size_t xb = align_up(sizeof(float) * static_cast<size_t>(d.m_pad) * d.n_pad);
      d.xf[0] = reinterpret_cast<float*>(off); off += xb;
      if (ns_steps > 0) {
        d.xf[1] = reinterpret_cast<float*>(off); off += xb;
        d.sgram = reinterpret_cast<float*>(off);
        off += align_up(sizeof(float) * static_cast<size_t>(d.s_chunks) * kSmallGram * kSmallGram);
        d.spoly = reinterpret_cast<float*>(off);
        off += align_up(sizeof(float) * kSmallGram * kSmallGram);
      }
      continue;
    }
    const size_t xb = align_up(sizeof(__bf16) * static_cast<size_t>(d.m_pad) * d.n_pad);
    const size_t gb = align_up(sizeof(__bf16) * static_cast<size_t>(d.m_pad) * d.m_pad);
    d.xt_hi[0] = reinterpret_cast<__bf16*>(off); off += xb;
    d.xt_lo[0] = reinterpret_cast<__bf16*>(off); off += xb;
    if (ns_steps > 0) {
      d.xt_hi[1] = reinterpret_cast<__bf16*>(off); off += xb;
      d.xt_lo[1] = reinterpret_cast<__bf16*>(off); off += xb;
      d.gram = reinterpret_cast<__bf16*>(off); off += gb;
      d.poly = reinterpret_cast<__bf16*>(off); off += gb;
    }
  }
  plan.total_bytes = off;
  return MUON_OK;
}

template <class T>
T* rebase(T* p, uintptr_t base) {
  return p ? reinterpret_cast<T*>(reinterpret_cast<uintptr_t>(p) + base) : nullptr;
}

void bind_workspace(Plan& plan, uintptr_t base) {
  for (MatDesc& d : plan.descs) {
    d.partials = rebase(d.partials, base);
    d.sigma = rebase(d.sigma, base);
    d.mom_bad = rebase(d.mom_bad, base);
    d.mstat = rebase(d.mstat, base);
    d.diag_part = rebase(d.diag_part, base);
    for (int b = 0; b < 2; ++b) {
      d.xt_hi[b] = rebase(d.xt_hi[b], base);
      d.xt_lo[b] = rebase(d.xt_lo[b], base);
      d.xf[b] = rebase(d.xf[b], base);
    }
    d.gram = rebase(d.gram, base);
    d.poly = rebase(d.poly, base);
    d.sgram = rebase(d.sgram, base);
    d.spoly = rebase(d.spoly, base);
  }
}

// ---------------------------------------------------------------- staging ring
// Pinned host slots for the descriptor table; a slot is reused only after the
// copy that last read it has completed (tracked by an event).
struct Slot {
  void* host = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool pending = false;
};

struct DeviceStaging {
  int device = -1;
  Slot slots[4];
  int cursor = 0;
};

std::mutex g_staging_mu;
std::vector<DeviceStaging> g_staging;

hipError_t upload_table(const void* src, size_t bytes, void* dst, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_staging_mu);
  DeviceStaging* ds = nullptr;
  for (auto& x : g_staging)
    if (x.device == dev) ds = &x;
  if (!ds) {
    g_staging.emplace_back();
    ds = &g_staging.back();
    ds->device = dev;
  }
  Slot& sl = ds->slots[ds->cursor];
  ds->cursor = (ds->cursor + 1) % 4;
  if (sl.pending) {
    e = hipEventSynchronize(sl.ev);
    if (e != hipSuccess) return e;
    sl.pending = false;
  }
  if (!sl.ev) {
    e = hipEventCreateWithFlags(&sl.ev, hipEventDisableTiming);
    if (e != hipSuccess) return e;
  }
  if (sl.cap < bytes) {
    if (sl.host) hipHostFree(sl.host);
    sl.host = nullptr;
    sl.cap = 0;
    const size_t cap = std::max<size_t>(bytes, 64 * 1024);
    e = hipHostMalloc(&sl.host, cap, hipHostMallocDefault);
    if (e != hipSuccess) return e;
    sl.cap = cap;
  }
  memcpy(sl.host, src, bytes);
  e = hipMemcpyAsync(dst, sl.host, bytes, hipMemcpyHostToDevice, s);
  if (e != hipSuccess) return e;
  e = hipEventRecord(sl.ev, s);
  if (e != hipSuccess) return e;
  sl.pending = true;
  return hipSuccess;
}

// ---------------------------------------------------------------- profiling
struct PendingEv {
  int stage;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<PendingEv> g_prof_pending;
std::vector<hipEvent_t> g_prof_pool;

hipEvent_t prof_event() {
  if (!g_prof_pool.empty()) {
    hipEvent_t e = g_prof_pool.back();
    g_prof_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

template <class F>
hipError_t run_stage(int stage, hipStream_t s, F&& f) {
  bool on;
  {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    on = g_prof_on;
  }
  if (!on) return f();
  hipEvent_t a, b;
  {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    a = prof_event();
    b = prof_event();
  }
  if (a) hipEventRecord(a, s);
  hipError_t e = f();
  if (b) hipEventRecord(b, s);
  if (a && b) {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    g_prof_pending.push_back({stage, a, b});
  }
  return e;
}

// Cost-balanced split of one grouped GEMM launch over the 8 XCDs.  A tile's
// cost is taken as its reduction length (tiles of one launch share their
// shape): k_gram for the Gram stage, m_pad for the polynomial and BX stages.
XcdSplit make_split(const Plan& plan, int tab, int mode) {
  const std::vector<int32_t>& pre = plan.pre[tab];
  const int n = static_cast<int>(plan.descs.size());
  double total = 0.0;
  for (int i = 0; i < n; ++i) {
    const double c = (mode == 0) ? plan.descs[i].k_gram : plan.descs[i].m_pad;
    total += static_cast<double>(pre[i + 1] - pre[i]) * c;
  }
  int32_t start[9];
  start[0] = 0;
  start[8] = pre[n];
  int i = 0;
  double before = 0.0;  // cost of matrices 0..i-1
  for (int x = 1; x < 8; ++x) {
    const double target = total * x / 8.0;
    while (i < n) {
      const double c = (mode == 0) ? plan.descs[i].k_gram : plan.descs[i].m_pad;
      const double mc = static_cast<double>(pre[i + 1] - pre[i]) * c;
      if (before + mc >= target) break;
      before += mc;
      ++i;
    }
    int w = pre[n];
    if (i < n) {
      const double c = (mode == 0) ? plan.descs[i].k_gram : plan.descs[i].m_pad;
      const int64_t k = static_cast<int64_t>((target - before) / c + 0.5);
      const int64_t lo = pre[i], hi = pre[i + 1];
      w = static_cast<int>(std::min(hi, std::max(lo, lo + k)));
    }
    start[x] = std::max(w, start[x - 1]);
  }
  XcdSplit sp;
  sp.max_len = 0;
  for (int x = 0; x < 8; ++x) {
    sp.begin[x] = start[x];
    sp.end[x] = start[x + 1];
    sp.max_len = std::max(sp.max_len, start[x + 1] - start[x]);
  }
  return sp;
}

muon_status_t hip_fail(hipError_t e, const char* where) {
  return fail(MUON_ERR_HIP, std::string("muon: ") + where + ": " + hipGetErrorString(e));
}

// Launch sequence of one call.  The descriptor table is uploaded into the
// workspace, then every stage is one grouped launch over all matrices.
// With `diag_out` (a device muon_diag_t array) the W-writing kernels also
// sum the diagnostics and a last launch reduces them.
// How execute() gets the descriptor table into the workspace.
enum Upload {
  // (a table of at most kTableArgBytes goes as the argument of one kernel
  // in the first two modes)
  kUploadPinned,    // through the pinned staging ring (allocated on first use)
  kUploadPageable,  // straight from this call's host memory (the copy has
                    // consumed it when hipMemcpyAsync returns); allocates nothing
  kUploadNone,      // already resident (a recorded plan): only the call's
                    // counter is zeroed, by a kernel; no profiling events
};

// The descriptor table of a bound plan (descriptors, then the prefix tables,
// then the zeroed counter of matrices marked for the prep pass).
std::vector<unsigned char> make_table(const Plan& plan) {
  const int n = static_cast<int>(plan.descs.size());
  std::vector<unsigned char> table(plan.table_bytes, 0);
  memcpy(table.data(), plan.descs.data(), sizeof(MatDesc) * n);
  int32_t* pre = reinterpret_cast<int32_t*>(table.data() + align_up(sizeof(MatDesc) * n));
  for (int k = 0; k < kNumTables; ++k)
    memcpy(pre + k * (n + 1), plan.pre[k].data(), sizeof(int32_t) * (n + 1));
  return table;
}

muon_status_t execute(Plan& plan, void* workspace, float mu, float eps, hipStream_t s,
                      void* diag_out = nullptr, Upload upload = kUploadPinned) {
  const int n = static_cast<int>(plan.descs.size());
  const uintptr_t base = reinterpret_cast<uintptr_t>(workspace);
  bind_workspace(plan, base);
  const bool diag = diag_out != nullptr;
  if (diag)
    for (MatDesc& d : plan.descs) d.flags |= kDiag;

  const size_t pre_off = align_up(sizeof(MatDesc) * n);
  const MatDesc* d_desc = reinterpret_cast<const MatDesc*>(base);
  const int32_t* d_pre = reinterpret_cast<const int32_t*>(base + pre_off);
  auto ptab = [&](int k) { return d_pre + k * (n + 1); };
  auto ttot = [&](int k) { return static_cast<int>(plan.tot[k]); };
  int32_t* d_prep_count = const_cast<int32_t*>(d_pre) + kNumTables * (n + 1);
  const bool recorded = upload == kUploadNone;
  // A recorded plan's launches carry no profiling events.
  auto stage = [&](int st, auto&& f) -> hipError_t { return recorded ? f() : run_stage(st, s, f); };

  hipError_t e;
  if (recorded) {
    e = launch_zero_counter(d_prep_count, s);
  } else {
    const std::vector<unsigned char> table = make_table(plan);
    e = stage(MUON_STAGE_UPLOAD, [&] {
      if (table.size() <= static_cast<size_t>(kTableArgBytes))
        return launch_table_write(workspace, table.data(), table.size(), s);
      return upload == kUploadPageable
                 ? hipMemcpyAsync(workspace, table.data(), table.size(), hipMemcpyHostToDevice, s)
                 : upload_table(table.data(), table.size(), workspace, s);
    });
  }
  if (e != hipSuccess) return hip_fail(e, "descriptor upload");
  e = stage(MUON_STAGE_MOMENTUM, [&] { return launch_momentum(d_desc, ptab(kTabMom), n, ttot(kTabMom), mu, s); });
  if (e != hipSuccess) return hip_fail(e, "momentum launch");
  e = stage(MUON_STAGE_NORM, [&] { return launch_norm(d_desc, n, eps, d_prep_count, s); });
  if (e != hipSuccess) return hip_fail(e, "norm launch");
  e = stage(MUON_STAGE_PREP, [&] {
    return launch_prep(d_desc, ptab(kTabPrep), n, ttot(kTabPrep), mu, d_prep_count, s);
  });
  if (e != hipSuccess) return hip_fail(e, "prep launch");
  int buf = 0;
  static const int stage_of_mode[3] = {MUON_STAGE_GRAM, MUON_STAGE_POLY, MUON_STAGE_BX};
  for (int it = 0; it < plan.ns_steps; ++it) {
    const bool last = it + 1 == plan.ns_steps;
    for (int mode = 0; mode < 3; ++mode) {
      for (int c = 0; c < kNumCfg; ++c) {
        const int tab = mode == 2 ? tab_bx(c) : tab_sym(c);
        if (plan.tot[tab] == 0) continue;
        const XcdSplit sp = make_split(plan, tab, mode);
        const bool wide = cfg_wide(c);
        // 3: BX with the update applied; 4: the same with diagnostics
        const int kmode = (wide && last && mode == 2) ? (diag ? 4 : 3) : mode;
        e = stage(kmode >= 3 ? MUON_STAGE_BX_UPDATE : stage_of_mode[mode], [&] {
          return wide ? launch_ns_gemm32(kmode, c, d_desc, ptab(tab), n, sp, buf, it == 0, s)
                      : launch_ns_gemm(mode, c, d_desc, ptab(tab), n, sp, buf, it == 0, s);
        });
        if (e != hipSuccess) return hip_fail(e, "matrix-core launch");
      }
    }
    if (plan.tot[kTabSmallGram] > 0) {
      e = stage(MUON_STAGE_GRAM, [&] {
        return launch_small_gram(d_desc, ptab(kTabSmallGram), n, ttot(kTabSmallGram), buf, s);
      });
      if (e != hipSuccess) return hip_fail(e, "small gram launch");
      e = stage(MUON_STAGE_POLY, [&] {
        return launch_small_poly(d_desc, ptab(kTabSmallPoly), n, ttot(kTabSmallPoly), s);
      });
      if (e != hipSuccess) return hip_fail(e, "small poly launch");
      e = stage(MUON_STAGE_BX, [&] {
        return launch_small_bx(d_desc, ptab(kTabSmallGram), n, ttot(kTabSmallGram), buf, s);
      });
      if (e != hipSuccess) return hip_fail(e, "small bx launch");
    }
    buf ^= 1;
  }
  if (plan.tot[kTabUpd] > 0) {
    e = stage(MUON_STAGE_UPDATE, [&] {
      return launch_update(d_desc, ptab(kTabUpd), n, ttot(kTabUpd), buf, diag, s);
    });
    if (e != hipSuccess) return hip_fail(e, "update launch");
  }
  if (diag) {
    e = stage(MUON_STAGE_DIAG, [&] { return launch_diag(d_desc, n, diag_out, s); });
    if (e != hipSuccess) return hip_fail(e, "diagnostics launch");
  }
  return MUON_OK;
}

muon_status_t check_hparams(const muon_hparams_t* hp) {
  if (!hp) return fail(MUON_ERR_INVALID_ARG, "muon: hp is NULL");
  if (!finite(hp->mu) || !finite(hp->lr) || !finite(hp->eps) || hp->eps < 0.f || !finite(hp->weight_decay))
    return fail(MUON_ERR_INVALID_ARG, "muon: mu, lr, eps and weight_decay must be finite and eps >= 0");
  if (hp->ns_steps < 0 || hp->ns_steps > MUON_MAX_NS_STEPS)
    return fail(MUON_ERR_INVALID_ARG, "muon: ns_steps outside 0..MUON_MAX_NS_STEPS");
  if (hp->nesterov != 0 && hp->nesterov != 1)
    return fail(MUON_ERR_INVALID_ARG, "muon: nesterov must be 0 or 1");
  if (hp->g_dtype != MUON_F32 && hp->g_dtype != MUON_BF16)
    return fail(MUON_ERR_INVALID_ARG, "muon: unknown g_dtype");
  return MUON_OK;
}

muon_status_t items_from_step(const muon_matrix_t* mats, int64_t n, const muon_hparams_t* hp,
                              bool check_ptrs, std::vector<Item>& items) {
  muon_status_t st = check_hparams(hp);
  if (st != MUON_OK) return st;
  if (n < 0) return fail(MUON_ERR_INVALID_ARG, "muon: n < 0");
  if (n > 0 && !mats) return fail(MUON_ERR_INVALID_ARG, "muon: mats is NULL");
  items.resize(n);
  for (int64_t i = 0; i < n; ++i) {
    const muon_matrix_t& mt = mats[i];
    if (check_ptrs) {
      if (!mt.W || !mt.G || !mt.B)
        return fail(MUON_ERR_INVALID_ARG, "muon: matrix " + std::to_string(i) + " has a NULL W, G or B");
      if ((reinterpret_cast<uintptr_t>(mt.W) | reinterpret_cast<uintptr_t>(mt.G) |
           reinterpret_cast<uintptr_t>(mt.B)) & 15u)
        return fail(MUON_ERR_ALIGN, "muon: matrix " + std::to_string(i) + " W, G or B is not 16-byte aligned");
    }
    if (!finite(mt.scale))
      return fail(MUON_ERR_INVALID_ARG, "muon: matrix " + std::to_string(i) + " has a non-finite scale");
    Item& it = items[i];
    it.W = mt.W;
    it.G = mt.G;
    it.B = mt.B;
    it.rows = mt.rows;
    it.cols = mt.cols;
    it.lr_scale = hp->lr * mt.scale;
    it.lr_wd = hp->lr * hp->weight_decay;
    it.flags = (hp->g_dtype == MUON_BF16 ? kGBf16 : 0) | (hp->nesterov ? kNesterov : 0);
  }
  return MUON_OK;
}

muon_status_t check_workspace(const Plan& plan, void* ws, size_t ws_bytes) {
  if (plan.total_bytes == 0) return MUON_OK;
  if (!ws) return fail(MUON_ERR_WORKSPACE, "muon: workspace is NULL");
  if (reinterpret_cast<uintptr_t>(ws) % kAlign)
    return fail(MUON_ERR_WORKSPACE, "muon: workspace is not 256-byte aligned");
  if (ws_bytes < plan.total_bytes)
    return fail(MUON_ERR_WORKSPACE, "muon: workspace has " + std::to_string(ws_bytes) +
                                        " bytes, needs " + std::to_string(plan.total_bytes));
  return MUON_OK;
}

void fill_ptrs(Plan& plan, const std::vector<Item>& items) {
  for (size_t i = 0; i < items.size(); ++i) {
    plan.descs[i].W = items[i].W;
    plan.descs[i].G = items[i].G;
    plan.descs[i].B = items[i].B;
  }
}

// Memory ranges of a step call (each matrix's W, B and G, the workspace the
// plan uses and the optional diagnostics array) checked for overlaps that
// the step forbids (see check_aliasing).
muon_status_t check_step_aliasing(const std::vector<Item>& items, const muon_hparams_t* hp, const void* workspace,
                                  size_t workspace_used, const muon_diag_t* diag) {
  std::vector<Range> rs;
  const size_t gsz = hp->g_dtype == MUON_BF16 ? 2 : 4;
  const int64_t n = static_cast<int64_t>(items.size());
  for (int64_t i = 0; i < n; ++i) {
    const uintptr_t e = static_cast<uintptr_t>(items[i].rows * items[i].cols);
    const uintptr_t w = reinterpret_cast<uintptr_t>(items[i].W), b = reinterpret_cast<uintptr_t>(items[i].B),
                    g = reinterpret_cast<uintptr_t>(items[i].G);
    rs.push_back({w, w + 4 * e, true, "W", i});
    rs.push_back({b, b + 4 * e, true, "B", i});
    rs.push_back({g, g + gsz * e, false, "G", i});
  }
  const uintptr_t ws = reinterpret_cast<uintptr_t>(workspace);
  rs.push_back({ws, ws + workspace_used, true, "workspace", -1});
  if (diag)
    rs.push_back({reinterpret_cast<uintptr_t>(diag), reinterpret_cast<uintptr_t>(diag + n), true, "diag", -1});
  return check_aliasing(rs);
}

// ---------------------------------------------------------------- static workspace
// Device address of `scratch` per device (looked up once per device).
std::mutex g_scratch_mu;
std::vector<std::pair<int, void*>> g_scratch_ptr;  // (device, address of scratch there)

muon_status_t static_workspace(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  for (const auto& p : g_scratch_ptr)
    if (p.first == dev) {
      *out = p.second;
      return MUON_OK;
    }
  void* ptr = nullptr;
  e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the static workspace");
  if (!ptr || reinterpret_cast<uintptr_t>(ptr) % kAlign)
    return fail(MUON_ERR_HIP, "muon: the static workspace has no 256-byte aligned device address");
  g_scratch_ptr.emplace_back(dev, ptr);
  *out = ptr;
  return MUON_OK;
}

}  // namespace

extern "C" {

size_t muon_workspace_bytes(const muon_matrix_t* mats, int64_t n, const muon_hparams_t* hp) {
  g_last_error.clear();
  std::vector<Item> items;
  if (items_from_step(mats, n, hp, false, items) != MUON_OK) return 0;
  if (n == 0) return 0;
  Plan plan;
  if (make_plan(items, hp->ns_steps, plan) != MUON_OK) return 0;
  return plan.total_bytes;
}

// use_static: the workspace is the library's static device array (after the
// plan is checked to fit it); `workspace` and `workspace_bytes` are ignored.
static muon_status_t step_impl(const muon_matrix_t* mats, int64_t n, const muon_hparams_t* hp,
                               muon_diag_t* diag, void* workspace, size_t workspace_bytes, void* stream,
                               bool use_static = false) {
  std::vector<Item> items;
  muon_status_t st = items_from_step(mats, n, hp, true, items);
  if (st != MUON_OK) return st;
  if (n == 0) return MUON_OK;
  Plan plan;
  st = make_plan(items, hp->ns_steps, plan);
  if (st != MUON_OK) return st;
  if (use_static) {
    if (plan.total_bytes > MUON_STATIC_WORKSPACE_BYTES)
      return fail(MUON_ERR_WORKSPACE, "muon: this call needs " + std::to_string(plan.total_bytes) +
                                          " bytes of workspace; the static workspace holds " +
                                          std::to_string(static_cast<size_t>(MUON_STATIC_WORKSPACE_BYTES)));
    st = static_workspace(&workspace);
    if (st != MUON_OK) return st;
    workspace_bytes = MUON_STATIC_WORKSPACE_BYTES;
  }
  st = check_workspace(plan, workspace, workspace_bytes);
  if (st != MUON_OK) return st;
  st = check_step_aliasing(items, hp, workspace, plan.total_bytes, diag);
  if (st != MUON_OK) return st;
  fill_ptrs(plan, items);
  return execute(plan, workspace, hp->mu, hp->eps, static_cast<hipStream_t>(stream), diag,
                 use_static ? kUploadPageable : kUploadPinned);
}

muon_status_t muon_step(const muon_matrix_t* mats, int64_t n, const muon_hparams_t* hp,
                        void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  return step_impl(mats, n, hp, nullptr, workspace, workspace_bytes, stream);
}

}  // extern "C"

struct muon_plan_s {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  hipEvent_t done = nullptr;  // recorded after each replay: the last one in flight
  hipStream_t last = nullptr;  // the stream `done` was last recorded on
  int device = -1;
};

extern "C" {

muon_status_t muon_plan_create(const muon_matrix_t* mats, int64_t n, const muon_hparams_t* hp, void* workspace,
                               size_t workspace_bytes, void* stream, muon_plan_t* out) {
  g_last_error.clear();
  if (!out) return fail(MUON_ERR_INVALID_ARG, "muon: out is NULL");
  *out = nullptr;
  if (n < 1) return fail(MUON_ERR_INVALID_ARG, "muon: a plan needs at least one matrix");
  std::vector<Item> items;
  muon_status_t st = items_from_step(mats, n, hp, true, items);
  if (st != MUON_OK) return st;
  Plan plan;
  st = make_plan(items, hp->ns_steps, plan);
  if (st != MUON_OK) return st;
  st = check_workspace(plan, workspace, workspace_bytes);
  if (st != MUON_OK) return st;
  st = check_step_aliasing(items, hp, workspace, plan.total_bytes, nullptr);
  if (st != MUON_OK) return st;
  fill_ptrs(plan, items);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  // The table, with the descriptors bound to the workspace, stays resident.
  {
    Plan bound = plan;
    bind_workspace(bound, reinterpret_cast<uintptr_t>(workspace));
    const std::vector<unsigned char> table = make_table(bound);
    e = hipMemcpyAsync(workspace, table.data(), table.size(), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) return hip_fail(e, "descriptor upload");
  }
  // Record the launch sequence on a private stream.
  hipStream_t cs = nullptr;
  e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e != hipSuccess) return hip_fail(e, "hipStreamCreateWithFlags");
  e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    hipStreamDestroy(cs);
    return hip_fail(e, "hipStreamBeginCapture");
  }
  const std::string before = g_last_error;
  st = execute(plan, workspace, hp->mu, hp->eps, cs, nullptr, kUploadNone);
  const std::string launch_error = g_last_error;
  hipGraph_t graph = nullptr;
  e = hipStreamEndCapture(cs, &graph);
  hipStreamDestroy(cs);
  if (st != MUON_OK) {
    if (graph) hipGraphDestroy(graph);
    return fail(st, launch_error);
  }
  if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
  if (e != hipSuccess) {
    hipGraphDestroy(graph);
    return hip_fail(e, "hipGraphInstantiate");
  }
  // Recorded once here (on the creation stream, idle since the table
  // upload), then after every replay.
  hipEvent_t done = nullptr;
  e = hipEventCreateWithFlags(&done, hipEventDisableTiming);
  if (e == hipSuccess) {
    e = hipEventRecord(done, s);
    if (e != hipSuccess) hipEventDestroy(done);
  }
  if (e != hipSuccess) {
    hipGraphExecDestroy(exec);
    hipGraphDestroy(graph);
    return hip_fail(e, "plan event");
  }
  muon_plan_s* p = new muon_plan_s;
  p->graph = graph;
  p->exec = exec;
  p->done = done;
  p->last = s;
  p->device = dev;
  *out = p;
  g_last_error = before;
  return MUON_OK;
}

muon_status_t muon_plan_step(muon_plan_t plan, void* stream) {
  g_last_error.clear();
  if (!plan) return fail(MUON_ERR_INVALID_ARG, "muon: plan is NULL");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != plan->device)
    return fail(MUON_ERR_INVALID_ARG, "muon: the plan was recorded on device " + std::to_string(plan->device) +
                                          ", the current device is " + std::to_string(dev));
  // After the previous replay: stream order covers one on this stream, an
  // event wait one on another stream; the event then marks this one.
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (s != plan->last) {
    e = hipStreamWaitEvent(s, plan->done, 0);
    if (e != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");
  }
  e = hipGraphLaunch(plan->exec, s);
  if (e != hipSuccess) return hip_fail(e, "hipGraphLaunch");
  e = hipEventRecord(plan->done, s);
  if (e != hipSuccess) return hip_fail(e, "hipEventRecord");
  plan->last = s;
  return MUON_OK;
}

muon_status_t muon_plan_destroy(muon_plan_t plan) {
  g_last_error.clear();
  if (!plan) return MUON_OK;
  // The graph is freed once its last replay (hence every replay) has ended.
  hipError_t e0 = hipEventSynchronize(plan->done);
  hipError_t e3 = hipEventDestroy(plan->done);
  hipError_t e1 = hipGraphExecDestroy(plan->exec);
  hipError_t e2 = hipGraphDestroy(plan->graph);
  delete plan;
  if (e0 != hipSuccess) return hip_fail(e0, "hipEventSynchronize");
  if (e3 != hipSuccess) return hip_fail(e3, "hipEventDestroy");
  if (e1 != hipSuccess) return hip_fail(e1, "hipGraphExecDestroy");
  if (e2 != hipSuccess) return hip_fail(e2, "hipGraphDestroy");
  return MUON_OK;
}

muon_status_t muon_step_static(const muon_matrix_t* mats, int64_t n, const muon_hparams_t* hp, void* stream) {
  g_last_error.clear();
  return step_impl(mats, n, hp, nullptr, nullptr, 0, stream, true);
}

muon_status_t muon_step_diag(const muon_matrix_t* mats, int64_t n, const muon_hparams_t* hp,
                             muon_diag_t* diag, void* workspace, size_t workspace_bytes,
                             void* stream) {
  g_last_error.clear();
  if (!diag) return fail(MUON_ERR_INVALID_ARG, "muon: diag is NULL");
  if (reinterpret_cast<uintptr_t>(diag) & 3u) return fail(MUON_ERR_ALIGN, "muon: diag is not 4-byte aligned");
  return step_impl(mats, n, hp, diag, workspace, workspace_bytes, stream);
}

static muon_status_t ortho_items(const float* const* M, float* const* O, const int64_t* rows,
                                 const int64_t* cols, int64_t n, int32_t ns_steps, bool check_ptrs,
                                 std::vector<Item>& items) {
  if (n < 0) return fail(MUON_ERR_INVALID_ARG, "muon: n < 0");
  if (ns_steps < 0 || ns_steps > MUON_MAX_NS_STEPS)
    return fail(MUON_ERR_INVALID_ARG, "muon: ns_steps outside 0..MUON_MAX_NS_STEPS");
  if (n > 0 && (!rows || !cols)) return fail(MUON_ERR_INVALID_ARG, "muon: rows or cols is NULL");
  if (check_ptrs && n > 0 && (!M || !O)) return fail(MUON_ERR_INVALID_ARG, "muon: M or O is NULL");
  items.resize(n);
  for (int64_t i = 0; i < n; ++i) {
    Item& it = items[i];
    it.W = check_ptrs ? O[i] : nullptr;
    it.G = check_ptrs ? M[i] : nullptr;
    it.B = nullptr;
    it.rows = rows[i];
    it.cols = cols[i];
    it.lr_scale = 0.f;
    it.lr_wd = 0.f;
    it.flags = kOrthoOnly;
    if (check_ptrs) {
      if (!it.W || !it.G)
        return fail(MUON_ERR_INVALID_ARG, "muon: matrix " + std::to_string(i) + " has a NULL M or O");
      if ((reinterpret_cast<uintptr_t>(it.W) | reinterpret_cast<uintptr_t>(it.G)) & 15u)
        return fail(MUON_ERR_ALIGN, "muon: matrix " + std::to_string(i) + " M or O is not 16-byte aligned");
    }
  }
  return MUON_OK;
}

size_t muon_orthogonalize_workspace_bytes(const int64_t* rows, const int64_t* cols, int64_t n,
                                          int32_t ns_steps) {
  g_last_error.clear();
  std::vector<Item> items;
  if (ortho_items(nullptr, nullptr, rows, cols, n, ns_steps, false, items) != MUON_OK) return 0;
  if (n == 0) return 0;
  Plan plan;
  if (make_plan(items, ns_steps, plan) != MUON_OK) return 0;
  return plan.total_bytes;
}

muon_status_t muon_orthogonalize(const float* const* M, float* const* O, const int64_t* rows,
                                 const int64_t* cols, int64_t n, int32_t ns_steps, float eps,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (!isfinite(eps) || eps < 0.f) return fail(MUON_ERR_INVALID_ARG, "muon: eps must be finite and >= 0");
  std::vector<Item> items;
  muon_status_t st = ortho_items(M, O, rows, cols, n, ns_steps, true, items);
  if (st != MUON_OK) return st;
  if (n == 0) return MUON_OK;
  Plan plan;
  st = make_plan(items, ns_steps, plan);
  if (st != MUON_OK) return st;
  st = check_workspace(plan, workspace, workspace_bytes);
  if (st != MUON_OK) return st;
  std::vector<Range> rs;
  for (int64_t i = 0; i < n; ++i) {
    const uintptr_t e = static_cast<uintptr_t>(items[i].rows * items[i].cols);
    rs.push_back({reinterpret_cast<uintptr_t>(items[i].W), reinterpret_cast<uintptr_t>(items[i].W) + 4 * e, true, "O", i});
    rs.push_back({reinterpret_cast<uintptr_t>(items[i].G), reinterpret_cast<uintptr_t>(items[i].G) + 4 * e, false, "M", i});
  }
  rs.push_back({reinterpret_cast<uintptr_t>(workspace), reinterpret_cast<uintptr_t>(workspace) + plan.total_bytes, true, "workspace", -1});
  st = check_aliasing(rs);
  if (st != MUON_OK) return st;
  fill_ptrs(plan, items);
  return execute(plan, workspace, 0.f, eps, static_cast<hipStream_t>(stream));
}

muon_status_t muon_plan_query(const muon_matrix_t* mats, int64_t n, const muon_hparams_t* hp,
                              muon_plan_info_t* info, muon_matrix_plan_t* per_matrix) {
  g_last_error.clear();
  if (!info) return fail(MUON_ERR_INVALID_ARG, "muon: info is NULL");
  std::vector<Item> items;
  muon_status_t st = items_from_step(mats, n, hp, false, items);
  if (st != MUON_OK) return st;
  memset(info, 0, sizeof(*info));
  if (n == 0) return MUON_OK;
  Plan plan;
  st = make_plan(items, hp->ns_steps, plan);
  if (st != MUON_OK) return st;
  info->workspace_bytes = static_cast<int64_t>(plan.total_bytes);
  int64_t launches_per_iter = plan.tot[kTabSmallGram] > 0 ? 3 : 0;
  for (int c = 0; c < kNumCfg; ++c) {
    if (plan.tot[tab_sym(c)] > 0) {
      launches_per_iter += 2;
      info->gram_tiles += plan.tot[tab_sym(c)];
      if (info->tile == 0) info->tile = kCfgRows[c];
    }
    if (plan.tot[tab_bx(c)] > 0) {
      launches_per_iter += 1;
      info->bx_tiles += plan.tot[tab_bx(c)];
    }
  }
  info->poly_tiles = info->gram_tiles;
  // momentum, norm, prep (+ update unless every matrix fuses it); the table copy is extra
  info->launches = 3 + (plan.tot[kTabUpd] > 0 ? 1 : 0) + launches_per_iter * static_cast<int64_t>(hp->ns_steps);
  info->ew_blocks = plan.tot[kTabMom];
  if (per_matrix) {
    for (int64_t i = 0; i < n; ++i) {
      const MatDesc& d = plan.descs[i];
      muon_matrix_plan_t& p = per_matrix[i];
      p.transposed = (d.flags & kTransposed) ? 1 : 0;
      p.m = d.m;
      p.n = d.n;
      p.m_pad = d.m_pad;
      p.n_pad = d.n_pad;
      p.tile = (d.flags & kSmall) ? 0 : kCfgRows[d.sym_cfg];
      p.bx_tile_rows = (d.flags & kSmall) ? 0 : kCfgRows[d.bx_cfg];
      p.bx_tile_cols = (d.flags & kSmall) ? 0 : kCfgCols[d.bx_cfg];
      p.fused_update = (d.flags & kFusedUpd) ? 1 : 0;
      p.xcd_edges = 0;
      p.x_offset = plan.x_offset[i];
    }
    // Matrices whose work range holds the start of an XCD's range in a
    // matrix-core launch (the split of make_split, as execute uses it).
    for (int c = 0; c < kNumCfg; ++c) {
      for (int mode = 0; mode < 3; ++mode) {
        const int tab = mode == 2 ? tab_bx(c) : tab_sym(c);
        if (plan.tot[tab] == 0) continue;
        const XcdSplit sp = make_split(plan, tab, mode);
        const std::vector<int32_t>& pre = plan.pre[tab];
        for (int x = 1; x < 8; ++x) {
          const int32_t b = sp.begin[x];
          if (b >= plan.tot[tab]) continue;
          const int64_t i = std::upper_bound(pre.begin(), pre.begin() + n, b) - pre.begin() - 1;
          per_matrix[i].xcd_edges |= 1 << mode;
        }
      }
    }
  }
  return MUON_OK;
}

muon_status_t muon_profile_enable(int32_t on) {
  std::lock_guard<std::mutex> lock(g_prof_mu);
  g_prof_on = on != 0;
  return MUON_OK;
}

muon_status_t muon_profile_read(double* ms, int64_t* launches) {
  g_last_error.clear();
  if (!ms || !launches) return fail(MUON_ERR_INVALID_ARG, "muon: ms or launches is NULL");
  std::vector<PendingEv> pend;
  {
    std::lock_guard<std::mutex> lock(g_prof_mu);
    pend.swap(g_prof_pending);
  }
  for (int k = 0; k < MUON_STAGE_COUNT; ++k) {
    ms[k] = 0.0;
    launches[k] = 0;
  }
  muon_status_t st = MUON_OK;
  for (const PendingEv& p : pend) {
    float t = 0.f;
    hipError_t e = hipEventSynchronize(p.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&t, p.a, p.b);
    if (e != hipSuccess && st == MUON_OK) st = hip_fail(e, "profile read");
    ms[p.stage] += t;
    launches[p.stage] += 1;
  }
  std::lock_guard<std::mutex> lock(g_prof_mu);
  for (const PendingEv& p : pend) {
    g_prof_pool.push_back(p.a);
    g_prof_pool.push_back(p.b);
  }
  return st;
}

muon_status_t muon_qk_clip(const muon_qk_clip_matrix_t* mats, int64_t n, float tau, void* stream) {
  g_last_error.clear();
  if (!finite(tau) || !(tau > 0.f)) return fail(MUON_ERR_INVALID_ARG, "muon: tau must be finite and > 0");
  if (n < 0) return fail(MUON_ERR_INVALID_ARG, "muon: n < 0");
  if (n == 0) return MUON_OK;
  if (!mats) return fail(MUON_ERR_INVALID_ARG, "muon: mats is NULL");
  if (n > (1 << 20)) return fail(MUON_ERR_UNSUPPORTED, "muon: more than 2^20 matrices");
  std::vector<Range> rs;
  int64_t heads_total = 0;
  for (int64_t i = 0; i < n; ++i) {
    const muon_qk_clip_matrix_t& m = mats[i];
    const std::string id = "muon: QK-Clip matrix " + std::to_string(i);
    if (!m.W || !m.max_logit) return fail(MUON_ERR_INVALID_ARG, id + " has a NULL W or max_logit");
    if (m.rows < 1 || m.cols < 1 || m.head_dim < 1)
      return fail(MUON_ERR_INVALID_ARG, id + " has rows, cols or head_dim < 1");
    if (m.rows > MUON_MAX_DIM || m.cols > MUON_MAX_DIM)
      return fail(MUON_ERR_UNSUPPORTED, id + " exceeds MUON_MAX_DIM");
    if (m.rows % m.head_dim != 0) return fail(MUON_ERR_INVALID_ARG, id + ": rows is not a multiple of head_dim");
    if ((reinterpret_cast<uintptr_t>(m.W) & 15u) || (reinterpret_cast<uintptr_t>(m.max_logit) & 3u))
      return fail(MUON_ERR_ALIGN, id + ": W is not 16-byte or max_logit not 4-byte aligned");
    const int64_t heads = m.rows / m.head_dim;
    heads_total += heads;
    if (heads_total > (int64_t{1} << 31) - 1) return fail(MUON_ERR_UNSUPPORTED, "muon: too many heads");
    const uintptr_t w = reinterpret_cast<uintptr_t>(m.W), l = reinterpret_cast<uintptr_t>(m.max_logit);
    rs.push_back({w, w + 4 * static_cast<uintptr_t>(m.rows * m.cols), true, "W", i});
    rs.push_back({l, l + 4 * static_cast<uintptr_t>(heads), false, "max_logit", i});
  }
  muon_status_t st = check_aliasing(rs);
  if (st != MUON_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  for (int64_t i0 = 0; i0 < n; i0 += kClipBatch) {
    ClipBatch b;
    memset(&b, 0, sizeof(b));
    b.n = static_cast<int32_t>(std::min<int64_t>(kClipBatch, n - i0));
    b.tau = tau;
    int32_t acc = 0;
    for (int k = 0; k < b.n; ++k) {
      const muon_qk_clip_matrix_t& m = mats[i0 + k];
      b.d[k].W = m.W;
      b.d[k].max_logit = m.max_logit;
      b.d[k].head_elems = static_cast<int64_t>(m.head_dim) * m.cols;
      b.d[k].vec = (b.d[k].head_elems % 4 == 0) ? 1 : 0;
      b.prefix[k] = acc;
      acc += static_cast<int32_t>(m.rows / m.head_dim);
    }
    b.prefix[b.n] = acc;
    const hipError_t e = launch_qk_clip(b, s);
    if (e != hipSuccess) return hip_fail(e, "QK-Clip launch");
  }
  return MUON_OK;
}

muon_status_t muon_copy_probe(const void* src, void* dst, size_t bytes, int32_t variant, void* stream) {
  g_last_error.clear();
  if (!src || !dst) return fail(MUON_ERR_INVALID_ARG, "muon: src or dst is NULL");
  if (((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u) || (bytes & 15u))
    return fail(MUON_ERR_ALIGN, "muon: copy probe needs 16-byte aligned buffers and a multiple of 16 bytes");
  if (variant < 0 || variant >= MUON_COPY_PROBE_VARIANTS)
    return fail(MUON_ERR_INVALID_ARG, "muon: copy probe variant outside 0..MUON_COPY_PROBE_VARIANTS-1");
  const uintptr_t a = reinterpret_cast<uintptr_t>(src), b = reinterpret_cast<uintptr_t>(dst);
  if (bytes > 0 && a < b + bytes && b < a + bytes) return fail(MUON_ERR_ALIAS, "muon: copy probe buffers overlap");
  if (bytes == 0) return MUON_OK;
  const hipError_t e = launch_copy_probe(src, dst, static_cast<int64_t>(bytes / 16), variant,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "copy probe launch");
  return MUON_OK;
}

const char* muon_status_string(muon_status_t status) {
  switch (status) {
    case MUON_OK: return "MUON_OK";
    case MUON_ERR_INVALID_ARG: return "MUON_ERR_INVALID_ARG";
    case MUON_ERR_UNSUPPORTED: return "MUON_ERR_UNSUPPORTED";
    case MUON_ERR_WORKSPACE: return "MUON_ERR_WORKSPACE";
    case MUON_ERR_ALIAS: return "MUON_ERR_ALIAS";
    case MUON_ERR_ALIGN: return "MUON_ERR_ALIGN";
    case MUON_ERR_HIP: return "MUON_ERR_HIP";
  }
  return "MUON_ERR_UNKNOWN";
}

const char* muon_last_error(void) { return g_last_error.c_str(); }

int32_t muon_abi_version(void) { return MUON_ABI_VERSION; }

}  // extern "C"
