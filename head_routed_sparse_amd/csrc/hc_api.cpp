// Host side of the C ABI: argument validation, per-head buffer layout and ring
// bookkeeping (HeadCast Sec. 4.3), the work planner of the routed step (Sec. 4.4),
// the classifier's host reductions (Sec. 4.2 Eqs. 3-5) and kernel launches.
#include "../../include/headcast.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <array>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <map>
#include <mutex>
#include <queue>
#include <string>
#include <thread>
#include <vector>

#include "hc_internal.h"

using namespace hc;

namespace {

thread_local std::string g_last_error;

hc_status fail(hc_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

hc_status ok() {
  g_last_error.clear();
  return HC_OK;
}

#define HC_TRY(expr)                       \
  do {                                     \
    hc_status _st = (expr);                \
    if (_st != HC_OK) return _st;          \
  } while (0)

#define HC_HIP(expr)                                                                  \
  do {                                                                                \
    hipError_t _e = (expr);                                                           \
    if (_e != hipSuccess) return fail(HC_ERR_HIP, "%s: %s", #expr, hipGetErrorString(_e)); \
  } while (0)

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

size_t esize(const hc_layer_desc& d) { return d.dtype == HC_BF16 ? 2 : 4; }
int64_t tokens_per_frame(const hc_layer_desc& d) { return (int64_t)d.frame_h * d.frame_w; }
int64_t lq_of(const hc_layer_desc& d) { return (int64_t)d.chunk_frames * tokens_per_frame(d); }
int rolling_blocks(const hc_layer_desc& d) { return std::max(d.window_frames / d.chunk_frames - 2, 0); }

hc_status check_desc(const hc_layer_desc* d) {
  if (!d) return fail(HC_ERR_NULL, "desc is NULL");
  if (d->dtype != HC_BF16 && d->dtype != HC_F32) return fail(HC_ERR_DTYPE, "dtype %d unknown", d->dtype);
  if (d->num_heads < 1 || d->num_heads > kMaxEntries)
    return fail(HC_ERR_SHAPE, "num_heads %d outside 1..%d", d->num_heads, kMaxEntries);
  if (d->head_dim != 64 && d->head_dim != 128) return fail(HC_ERR_SHAPE, "head_dim %d not 64 or 128", d->head_dim);
  if (d->frame_h < 1 || d->frame_w < 1 || d->frame_h > 32767 || d->frame_w > 32767)
    return fail(HC_ERR_SHAPE, "frame %dx%d out of range", d->frame_h, d->frame_w);
  if (d->chunk_frames < 1 || d->window_frames < d->chunk_frames || d->window_frames % d->chunk_frames)
    return fail(HC_ERR_SHAPE, "window_frames %d must be a positive multiple of chunk_frames %d",
                d->window_frames, d->chunk_frames);
  if (d->grid_h < 1 || d->grid_w < 1) return fail(HC_ERR_SHAPE, "grid %dx%d must be >= 1", d->grid_h, d->grid_w);
  if (d->variant < 0 ||
      d->variant > (HC_VARIANT_DUMMY_PREVIOUS | HC_VARIANT_SPATIAL_CELLS | HC_VARIANT_SPATIAL_OWN_LAUNCH))
    return fail(HC_ERR_SHAPE, "variant %d unknown", d->variant);
  if (!(d->softmax_scale > 0.f) || !std::isfinite(d->softmax_scale))
    return fail(HC_ERR_SHAPE, "softmax_scale must be positive and finite");
  const int64_t keys = (int64_t)d->window_frames * tokens_per_frame(*d);
  if (keys >= (int64_t(1) << 30)) return fail(HC_ERR_SHAPE, "window of %lld keys too large", (long long)keys);
  // the kernels address the rows of one window tensor by 32-bit byte offsets
  const int64_t bytes = keys * d->num_heads * d->head_dim * (int64_t)esize(*d);
  if (bytes >= (int64_t(1) << 32) - (int64_t(1) << 16))
    return fail(HC_ERR_SHAPE, "window K (or V) of %lld bytes: must stay under 4 GiB", (long long)bytes);
  return HC_OK;
}

hc_status check_labels(const hc_layer_desc& d, const int32_t* labels) {
  if (!labels) return fail(HC_ERR_NULL, "labels is NULL");
  for (int h = 0; h < d.num_heads; ++h)
    if (labels[h] < HC_SINK || labels[h] > HC_GLOBAL)
      return fail(HC_ERR_LABEL, "label %d of head %d outside 0..3", labels[h], h);
  return HC_OK;
}

hc_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(HC_ERR_NULL, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % 16) return fail(HC_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return HC_OK;
}

hc_status check_hist_frames(const hc_layer_desc& d, int32_t n) {
  if (n < 0 || n > d.window_frames - d.chunk_frames || n % d.chunk_frames)
    return fail(HC_ERR_SHAPE, "n_hist_frames %d must be a multiple of %d in [0, %d]", n, d.chunk_frames,
                d.window_frames - d.chunk_frames);
  return HC_OK;
}

// gfx950 check, once per device.
std::mutex g_dev_mutex;
std::vector<int> g_dev_ok;   // -1 unknown, 0 bad, 1 good

hc_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return fail(HC_ERR_DEVICE, "no HIP device");
  std::lock_guard<std::mutex> lk(g_dev_mutex);
  if ((int)g_dev_ok.size() <= dev) g_dev_ok.resize(dev + 1, -1);
  if (g_dev_ok[dev] < 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return fail(HC_ERR_DEVICE, "device %d unreadable", dev);
    g_dev_ok[dev] = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
  }
  if (!g_dev_ok[dev]) return fail(HC_ERR_DEVICE, "device %d is not gfx950", dev);
  return HC_OK;
}

// ---------------------------------------------------------------- timing
struct TimedLaunch {
  int kind;
  hipEvent_t a, b;
};
std::mutex g_time_mutex;
bool g_timing = false;
std::vector<TimedLaunch> g_timed;

template <class F>
hipError_t timed(int kind, hipStream_t s, F&& launch) {
  bool on;
  {
    std::lock_guard<std::mutex> lk(g_time_mutex);
    on = g_timing;
  }
  if (!on) return launch();
  hipEvent_t a, b;
  hipError_t e = hipEventCreate(&a);
  if (e != hipSuccess) return e;
  if ((e = hipEventCreate(&b)) != hipSuccess) return e;
  if ((e = hipEventRecord(a, s)) != hipSuccess) return e;
  if ((e = launch()) != hipSuccess) return e;
  if ((e = hipEventRecord(b, s)) != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_time_mutex);
  g_timed.push_back({kind, a, b});
  return hipSuccess;
}

// ---------------------------------------------------------------- dense planning
struct Entry {
  int64_t hist_off;
  int32_t hist_len, cur_len, head, nsplit, split_len, slot;
  bool whole;   // never split (the current block of a Spatial head)
};

constexpr int kSlotsPerCu = 2;    // Spatial (and d = 128 dense) workgroups resident per CU
constexpr int kNumCu = 256;

// Dense workgroups resident per CU: d = 128 fills half the LDS and registers with two,
// d = 64 (a 32 KB ring, 119 registers) takes four.
int dense_slots(int head_dim) { return kNumCu * (head_dim == 64 ? 4 : kSlotsPerCu); }
// Fixed cost of one dense item (query loads, ring fill, epilogue), in key tiles: fitted
// to the measured times of two plans of the 480P-shaped layer (888 and 1443 items).
constexpr double kItemOverheadTiles = 9.0;
// The merge of key-split partials in key-tile units of the dense makespan: a dense
// workgroup takes about 1.8 us per 64-key tile (128 queries, d = 128) and the merge
// kernel reads partials at about 3.9 TB/s, so one tile of time reads about 7 MB.
constexpr double kMergeBytesPerTile = 7e6;

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// Cost (in key tiles) of one dense item: its keys, the fixed cost, and the partial of a
// split entry.
double item_cost(int len, int nsplit) { return len / (double)kKeyTile + kItemOverheadTiles + (nsplit > 1 ? 1.0 : 0.0); }

// Makespan estimate (in key tiles) of LPT list scheduling of the entries' items on
// n_slots workgroup slots; items run in order of decreasing length. Stops early, with
// a value above `cutoff`, once the makespan passes it.
double lpt_makespan(const std::vector<Entry>& es, int nqt, int n_slots, double cutoff = 1e300) {
  std::vector<std::pair<double, int64_t>> items;   // (cost, count)
  for (const Entry& e : es) {
    const int total = e.hist_len + e.cur_len;
    for (int s = 0; s < e.nsplit; ++s) {
      items.push_back({item_cost(std::min(e.split_len, total - s * e.split_len), e.nsplit), nqt});
    }
  }
  std::sort(items.begin(), items.end(), [](auto& a, auto& b) { return a.first > b.first; });
  std::priority_queue<double, std::vector<double>, std::greater<double>> slots;
  for (int i = 0; i < n_slots; ++i) slots.push(0.0);
  double makespan = 0.0;
  for (auto& it : items)
    for (int64_t c = 0; c < it.second; ++c) {
      double t = slots.top() + it.first;
      slots.pop();
      slots.push(t);
      makespan = std::max(makespan, t);
      if (makespan > cutoff) return makespan;
    }
  return makespan;
}

// Key splits of the entries: each class of equally long entries (all Global heads, all
// Sink heads, ...) is cut into k pieces of one length (a multiple of the key tile), k
// chosen for the smallest estimated time; splitting only when it pays. The search
// starts from the best length common to all classes and then improves one class at a
// time (each class: k = 1..16, kept when the makespan drops). A split entry takes one
// partial slot per piece; choices needing more than slot_budget such slots are skipped
// (< 0: no limit; no splits always fits). n_slots: dense workgroups the GPU runs at once.
// The estimate adds the merge of the pieces' fp32 partials (piece_bytes each).
void plan_splits_search(std::vector<Entry>& es, int nqt, int slot_budget, int n_slots, double piece_bytes) {
  auto apply = [](Entry& e, int len) {
    const int total = e.hist_len + e.cur_len;
    e.nsplit = e.whole ? 1 : std::max(1, ceil_div(total, len));
    e.split_len = std::max(kKeyTile, ceil_div(ceil_div(std::max(total, 1), e.nsplit), kKeyTile) * kKeyTile);
  };
  auto piece = [](int total, int k) { return ceil_div(ceil_div(std::max(total, 1), k), kKeyTile) * kKeyTile; };
  // classes: the distinct lengths of the entries that may be split
  std::vector<int> totals;
  for (const Entry& e : es)
    if (!e.whole) totals.push_back(e.hist_len + e.cur_len);
  std::sort(totals.begin(), totals.end(), std::greater<int>());
  totals.erase(std::unique(totals.begin(), totals.end()), totals.end());
  if (totals.empty() || totals[0] == 0) {
    for (Entry& e : es) apply(e, std::max(totals.empty() ? 1 : totals[0], 1));
    return;
  }
  // cost of a choice (pieces per class): estimated makespan plus the merge of the
  // pieces' partials; negative when the partial slots do not fit the budget
  std::vector<int> k(totals.size(), 1);
  double best = -1;
  auto cost = [&](const std::vector<int>& kk) {
    std::vector<Entry> trial = es;
    int slots = 0, extra = 0;
    for (Entry& e : trial) {
      if (e.whole) {
        apply(e, e.hist_len + e.cur_len);
        continue;
      }
      const int c = (int)(std::find(totals.begin(), totals.end(), e.hist_len + e.cur_len) - totals.begin());
      apply(e, piece(totals[c], kk[c]));
      if (e.nsplit > 1) slots += e.nsplit;
    }
    for (int x : kk) extra += x - 1;
    if (slot_budget >= 0 && slots > slot_budget && extra > 0) return -1.0;
    const double bias = 1.0 + 0.001 * extra;   // ties go to fewer pieces
    const double merge = slots * piece_bytes / kMergeBytesPerTile;
    return (lpt_makespan(trial, nqt, n_slots, best < 0 ? 1e300 : best / bias - merge) + merge) * bias;
  };
  // common length first (k pieces of the longest entry)
  for (int kl = 1; kl <= 16; ++kl) {
    const int len = piece(totals[0], kl);
    std::vector<int> kk(totals.size());
    for (size_t c = 0; c < totals.size(); ++c) kk[c] = std::max(1, ceil_div(totals[c], len));
    const double m = cost(kk);
    if (m >= 0 && (best < 0 || m < best)) {
      best = m;
      k = kk;
    }
  }
  // then one class at a time
  for (int round = 0; round < 3; ++round) {
    bool moved = false;
    for (size_t c = 0; c < totals.size(); ++c)
      for (int kc = 1; kc <= 16; ++kc) {
        if (kc == k[c]) continue;
        std::vector<int> kk = k;
        kk[c] = kc;
        const double m = cost(kk);
        if (m >= 0 && m < best * 0.999) {
          best = m;
          k = kk;
          moved = true;
        }
      }
    if (!moved) break;
  }
  for (Entry& e : es) {
    if (e.whole) {
      apply(e, e.hist_len + e.cur_len);
      continue;
    }
    const int c = (int)(std::find(totals.begin(), totals.end(), e.hist_len + e.cur_len) - totals.begin());
    apply(e, piece(totals[c], k[c]));
  }
}

// Planner decisions kept per input, at most this many at a time.
constexpr size_t kMemoCap = 1024;

void plan_splits(std::vector<Entry>& es, int nqt, int slot_budget, int n_slots, int64_t piece_bytes) {
  // decisions are kept per input (layers of one geometry and head mix plan alike)
  static std::mutex mu;
  static std::map<std::vector<int64_t>, std::vector<std::pair<int, int>>> memo;
  std::vector<int64_t> key{nqt, slot_budget, n_slots, piece_bytes};
  for (const Entry& e : es) key.push_back(((int64_t)(e.hist_len + e.cur_len) << 1) | (e.whole ? 1 : 0));
  {
    std::lock_guard<std::mutex> lk(mu);
    auto it = memo.find(key);
    if (it != memo.end()) {
      for (size_t i = 0; i < es.size(); ++i) {
        es[i].nsplit = it->second[i].first;
        es[i].split_len = it->second[i].second;
      }
      return;
    }
  }
  plan_splits_search(es, nqt, slot_budget, n_slots, (double)piece_bytes);
  std::vector<std::pair<int, int>> val;
  for (const Entry& e : es) val.push_back({e.nsplit, e.split_len});
  std::lock_guard<std::mutex> lk(mu);
  if (memo.size() >= kMemoCap) memo.clear();   // bounded in a long-lived process
  memo[key] = val;
}

// Spatial query tile (tile_r x tile_c positions, 24..32 of them): the shape with the
// shortest estimated Spatial kernel. A tile costs one step per 32 keys of the union of
// its positions' windows (per frame); the tiles of all heads are list-scheduled,
// longest first, on kNumCu * kSlotsPerCu workgroup slots. Ties go to the fewer steps.
// Results are kept per geometry (the search takes milliseconds).
// 32-key chunks of the window union of every position tile (tile_r x tile_c, row-major).
std::vector<int> tile_union_chunks(int fh, int fw, int gh, int gw, bool cells, int tile_r, int tile_c) {
  auto lo = [&](int pos, int g, int ext) { return cells ? cell_origin(pos, g) : win_origin(pos, g, ext); };
  auto hi = [&](int pos, int g, int ext) {
    return lo(pos, g, ext) + (cells ? cell_extent(pos, g, ext) : std::min(g, ext));
  };
  std::vector<int> chunks;
  for (int r0 = 0; r0 < fh; r0 += tile_r)
    for (int c0 = 0; c0 < fw; c0 += tile_c) {
      const int r1 = std::min(r0 + tile_r, fh) - 1, c1 = std::min(c0 + tile_c, fw) - 1;
      const int ur = hi(r1, gh, fh) - lo(r0, gh, fh), uc = hi(c1, gw, fw) - lo(c0, gw, fw);
      chunks.push_back(ceil_div((int64_t)ur * uc, kStep));
    }
  return chunks;
}

void choose_spatial_tile(int fh, int fw, int gh, int gw, bool cells, int n_heads, int* tile_r, int* tile_c) {
  static std::mutex mu;
  static std::map<std::array<int, 6>, std::pair<int, int>> memo;
  const std::array<int, 6> key{fh, fw, gh, gw, cells ? 1 : 0, n_heads};
  {
    std::lock_guard<std::mutex> lk(mu);
    auto it = memo.find(key);
    if (it != memo.end()) {
      *tile_r = it->second.first;
      *tile_c = it->second.second;
      return;
    }
  }
  double best_t = -1.0;
  int64_t best_total = 0;
  *tile_r = 4;
  *tile_c = 8;
  for (int a = 1; a <= kSpTileMax; ++a)
    for (int b = 1; a * b <= kSpTileMax; ++b) {
      if (4 * a * b < 3 * kSpTileMax) continue;   // keep >= 3/4 of the MFMA rows busy
      if (a > fh || b > fw) continue;             // (no candidate: a frame under 24 positions keeps 4 x 8)
      std::vector<int> steps = tile_union_chunks(fh, fw, gh, gw, cells, a, b);
      std::sort(steps.begin(), steps.end(), std::greater<int>());
      std::priority_queue<int64_t, std::vector<int64_t>, std::greater<int64_t>> slots;
      for (int i = 0; i < kNumCu * kSlotsPerCu; ++i) slots.push(0);
      int64_t span = 0, total = 0;
      for (int st : steps)
        for (int h = 0; h < n_heads; ++h) {
          const int64_t t = slots.top() + st;
          slots.pop();
          slots.push(t);
          span = std::max(span, t);
          total += st;
        }
      if (best_t < 0 || span < best_t || (span == best_t && total < best_total)) {
        best_t = (double)span;
        best_total = total;
        *tile_r = a;
        *tile_c = b;
      }
    }
  std::lock_guard<std::mutex> lk(mu);
  if (memo.size() >= kMemoCap) memo.clear();
  memo[key] = {*tile_r, *tile_c};
}

// Frame parts of the Spatial launch: when the tiles of all Spatial heads leave
// workgroup slots free, each tile's frames are split over that many workgroups (their
// partials are merged afterwards), shortening the chain of dependent steps. bf16 only;
// at most kMaxSpParts and one frame per part.
constexpr int kMaxSpParts = 4;
int spatial_parts(const hc_layer_desc& d, int tile_r, int tile_c, int n_sp, int n_frames) {
  if (d.dtype != HC_BF16 || n_sp == 0 || n_frames <= 1) return 1;
  const int64_t wgs = (int64_t)ceil_div(d.frame_h, tile_r) * ceil_div(d.frame_w, tile_c) * n_sp;
  const int64_t free_x = (int64_t)kNumCu * kSlotsPerCu / wgs;
  return (int)std::max<int64_t>(1, std::min<int64_t>({free_x, kMaxSpParts, n_frames}));
}

// XCD queues of one dense launch. A group is the query tiles of one key range (one split
// of one entry); its tiles read the same keys, which an XCD's L2 fetches once for all of
// them. Each class of equally long items (the groups of one split length, in logical
// order) is dealt to the 8 XCDs in 8 contiguous, equal parts: every XCD then runs the
// same mix of item lengths, longest first, on its 64 workgroup slots (the packing of a
// deal of single items), while a group spans only the XCDs its part boundaries cross.
// If some queue would need more than kXcdRuns runs, each XCD takes one contiguous block
// of items instead.
struct ItemGroup {
  int first, count;
  double cost;   // per item, in key tiles
};

void plan_xcd_queues(DenseParams& p, std::vector<ItemGroup> gs) {
  std::stable_sort(gs.begin(), gs.end(), [](const ItemGroup& a, const ItemGroup& b) { return a.cost > b.cost; });
  std::vector<XcdRun> q[kXcds];
  auto add = [&](int x, int f, int c) {
    if (c <= 0) return;
    if (!q[x].empty() && q[x].back().first + q[x].back().count == f)
      q[x].back().count += c;
    else
      q[x].push_back(XcdRun{f, c});
  };
  for (size_t c0 = 0; c0 < gs.size();) {
    size_t c1 = c0;
    int n = 0;
    while (c1 < gs.size() && gs[c1].cost == gs[c0].cost) n += gs[c1++].count;
    // items of the class in order: position t lies in group g at tile t - start(g)
    int start = 0;
    for (size_t g = c0; g < c1; ++g) {
      const int a = start, b = start + gs[g].count;
      for (int x = 0; x < kXcds; ++x) {
        const int lo = (int)((int64_t)n * x / kXcds), hi = (int)((int64_t)n * (x + 1) / kXcds);
        const int f = std::max(a, lo), e = std::min(b, hi);
        add(x, gs[g].first + (f - a), e - f);
      }
      start = b;
    }
    c0 = c1;
  }
  bool fits = true;
  for (int x = 0; x < kXcds; ++x) fits = fits && (int)q[x].size() <= kXcdRuns;
  if (!fits) {
    for (int x = 0; x < kXcds; ++x) {
      const int b0 = (int)((int64_t)p.n_items * x / kXcds), b1 = (int)((int64_t)p.n_items * (x + 1) / kXcds);
      q[x].assign(1, XcdRun{b0, b1 - b0});
    }
  }
  p.xcd_len = 0;
  for (int x = 0; x < kXcds; ++x) {
    int len = 0;
    p.xcd_nrun[x] = (int)q[x].size();
    for (size_t r = 0; r < q[x].size(); ++r) {
      p.xcd_run[x][r] = q[x][r];
      len += q[x][r].count;
    }
    p.xcd_len = std::max(p.xcd_len, len);
  }
}

// Launch parameters of dense entries (batched by kMaxEntries), longest items first.
// With base.sp.n_sp > 0 the Spatial tiles of heads sp_heads (in the order of their
// SpatialEntry list) follow the dense items of the single launch, each costing sp_cost
// key tiles in the XCD queues.
hc_status dense_launches(std::vector<Entry> es, const DenseParams& base, std::vector<DenseParams>* out,
                         const std::vector<int>& sp_heads = {}, double sp_cost = 0.0) {
  std::stable_sort(es.begin(), es.end(), [](const Entry& a, const Entry& b) { return a.split_len > b.split_len; });
  // every item must own at least one key: the kernel's step pipeline runs n >= 1 steps
  for (const Entry& e : es)
    if (e.nsplit < 1 || e.split_len < 1 || e.hist_len + e.cur_len < 1 ||
        (int64_t)(e.nsplit - 1) * e.split_len >= (int64_t)e.hist_len + e.cur_len)
      return fail(HC_ERR_STATE, "internal: dense entry of head %d has an empty key split (%d x %d over %d keys)",
                  e.head, e.nsplit, e.split_len, e.hist_len + e.cur_len);
  out->clear();
  for (size_t b0 = 0; b0 < es.size(); b0 += kMaxEntries) {
    DenseParams p = base;
    const size_t n = std::min(es.size() - b0, (size_t)kMaxEntries);
    int items = 0;
    std::vector<ItemGroup> groups;
    for (size_t i = 0; i < n; ++i) {
      const Entry& e = es[b0 + i];
      DenseEntry& d = p.e[i];
      d.hist_off = e.hist_off;
      d.hist_len = e.hist_len;
      d.cur_len = e.cur_len;
      d.head = e.head;
      d.nsplit = e.nsplit;
      d.split_len = e.split_len;
      d.slot = e.slot;
      d.item_begin = items;
      d.pad = 0;
      const int total = e.hist_len + e.cur_len;
      for (int sp = 0; sp < e.nsplit; ++sp) {
        const int len = std::min(e.split_len, total - sp * e.split_len);
        groups.push_back(ItemGroup{items + sp * base.nqt, base.nqt, len / (double)kKeyTile + kItemOverheadTiles});
      }
      items += e.nsplit * base.nqt;
    }
    p.n_entries = (int)n;
    if (base.sp.n_sp > 0) {
      if (es.size() > (size_t)kMaxEntries || (int)sp_heads.size() != base.sp.n_sp)
        return fail(HC_ERR_STATE, "internal: Spatial tiles need one dense launch");
      const int n_tiles = base.sp.g.tiles_r * base.sp.g.tiles_c * base.sp.g.n_parts;   // items per head
      p.sp.n_dense_items = items;
      for (int j = 0; j < base.sp.n_sp; ++j) {
        int ei = -1;
        for (size_t i = 0; i < n; ++i)
          if (p.e[i].head == sp_heads[j]) ei = (int)i;
        if (ei < 0) return fail(HC_ERR_STATE, "internal: Spatial head %d has no dense entry", sp_heads[j]);
        p.sp.sp_entry[j] = (int8_t)ei;
        groups.push_back(ItemGroup{items, n_tiles, sp_cost});
        items += n_tiles;
      }
    }
    p.n_items = items;
    plan_xcd_queues(p, groups);
    out->push_back(p);
  }
  return HC_OK;
}

// Launch dense entries (and, with base.sp.n_sp > 0, the Spatial tiles after them).
hc_status run_dense(const std::vector<Entry>& es, const DenseParams& base, int head_dim, int bf16, hipStream_t s,
                    const std::vector<int>& sp_heads = {}, double sp_cost = 0.0) {
  std::vector<DenseParams> ps;
  HC_TRY(dense_launches(es, base, &ps, sp_heads, sp_cost));
  for (const DenseParams& p : ps)
    HC_HIP(timed(bf16 ? K_DENSE : K_F32, s, [&] { return launch_dense(p, head_dim, bf16, s); }));
  return HC_OK;
}

}  // namespace

// ---------------------------------------------------------------- handle
// The launches of a routed call for the handle's current state (rebuilt only when some
// head's stored history length changes) and the partial slots its workspace holds.
struct Plan {
  int64_t plan_block = -1;
  std::vector<int32_t> plan_hist_len;
  std::vector<Entry> entries;
  std::vector<MergeEntry> merges;
  std::vector<SpatialEntry> spatials;
  int sp_parts = 1;                  // Spatial workgroups per tile (frame parts)
  bool fused = false;                // Spatial tiles run as the last items of the dense launch
                                     // (decided per fill state)
  int n_slots = 0;
  int max_slots = -1;                // partial slots the workspace provides
  int slot_cap = -1;                 // >= 0: at most this many (the library's scratch)
  bool ok = true;                    // false: the Spatial partials alone exceed slot_cap
};

struct hc_head_buffers {
  hc_layer_desc desc;
  std::vector<int32_t> labels;
  char* mem = nullptr;
  size_t mem_bytes = 0;
  size_t v_region = 0;               // byte offset of the V region (K region at 0)
  std::vector<int64_t> head_off;     // element offset of head rows in a region, -1 = none
  std::vector<int64_t> head_rows;    // row capacity
  int64_t next_block = 0;
  int sp_tile_r = 0, sp_tile_c = 0;  // Spatial query tile
  Plan plan;                         // calls with a caller workspace
  Plan scratch_plan;                 // the allocation-free call (slot_cap set on first use)
  bool plan_only = false;            // host-only handle (hc_plan_head_buffers)
};

namespace {

bool dummy_prev(const hc_layer_desc& d) { return (d.variant & HC_VARIANT_DUMMY_PREVIOUS) != 0; }
bool spatial_cells(const hc_layer_desc& d) { return (d.variant & HC_VARIANT_SPATIAL_CELLS) != 0; }

int64_t capacity_rows(const hc_layer_desc& d, int cls) {
  const int64_t S = tokens_per_frame(d);
  if (d.window_frames == d.chunk_frames) return 0;
  if (cls == HC_SINK) return (int64_t)d.chunk_frames * S;
  if (cls == HC_DUMMY) return dummy_prev(d) ? (int64_t)d.chunk_frames * S : 0;
  return (int64_t)(d.window_frames - d.chunk_frames) * S;
}

size_t layout(const hc_layer_desc& d, const int32_t* labels, std::vector<int64_t>* off, std::vector<int64_t>* rows) {
  size_t bytes = 0;
  for (int h = 0; h < d.num_heads; ++h) {
    const int64_t r = capacity_rows(d, labels[h]);
    if (off) off->push_back(r ? (int64_t)(bytes / esize(d)) : -1);
    if (rows) rows->push_back(r);
    bytes += align_up((size_t)r * d.head_dim * esize(d));
  }
  return bytes;   // one region (K or V)
}

// History frames currently stored for a head class, given the next block index.
int64_t stored_frames(const hc_layer_desc& d, int cls, int64_t next_block) {
  if (d.window_frames == d.chunk_frames || next_block <= 0) return 0;
  if (cls == HC_DUMMY) return dummy_prev(d) ? d.chunk_frames : 0;   // the window's latest history block
  if (cls == HC_SINK) return d.chunk_frames;
  const int64_t rolling = std::min<int64_t>(next_block - 1, rolling_blocks(d));
  return (1 + rolling) * d.chunk_frames;
}

void build_plan(hc_head_buffers* b, Plan& P) {
  const hc_layer_desc& d = b->desc;
  const int64_t S = tokens_per_frame(d);
  const int lq = (int)lq_of(d);
  const int nqt = ceil_div(lq, kDenseQ);
  auto make = [&](int64_t next_block, int slot_budget) {
    std::vector<Entry> es;
    for (int h = 0; h < d.num_heads; ++h) {
      const int cls = b->labels[h];
      Entry e{};
      e.head = h;
      e.cur_len = lq;
      e.slot = -1;
      e.hist_off = b->head_off[h] < 0 ? 0 : b->head_off[h];
      if (cls == HC_SPATIAL && spatial_cells(d)) continue;   // served whole by the cell kernel
      if (cls != HC_SPATIAL) e.hist_len = (int)(stored_frames(d, cls, next_block) * S);
      e.whole = cls == HC_SPATIAL;
      es.push_back(e);
    }
    plan_splits(es, nqt, slot_budget, dense_slots(d.head_dim), (int64_t)lq * (d.head_dim + 2) * 4);
    return es;
  };
  // the plan depends on the state only through the stored history lengths, which stop
  // changing once the window is full: steady-state appends keep the plan
  std::vector<int32_t> hist_len(d.num_heads);
  for (int h = 0; h < d.num_heads; ++h)
    hist_len[h] = (int32_t)(stored_frames(d, b->labels[h], b->next_block) * S);
  if (P.plan_block >= 0 && hist_len == P.plan_hist_len) {
    P.plan_block = b->next_block;
    return;
  }
  P.plan_hist_len = hist_len;
  // Spatial tiles and frame parts
  const bool cells = spatial_cells(d);
  int n_sp = 0;
  for (int h = 0; h < d.num_heads; ++h) n_sp += b->labels[h] == HC_SPATIAL;
  if (n_sp > 0 && b->sp_tile_r == 0)
    choose_spatial_tile(d.frame_h, d.frame_w, d.grid_h, d.grid_w, cells, n_sp, &b->sp_tile_r, &b->sp_tile_c);
  // Spatial tiles run as the last items of the dense launch (bf16, d = 128, sliding
  // windows: cells walk the current block themselves), unless the caller asks for their
  // own launch: there they fill the slots the dense items leave idle at the end, which
  // outweighs the merge of one more partial per Spatial head (480P-shaped layer 4.5%
  // faster, 720P and 1080P 0.3%)
  const bool fusable = d.dtype == HC_BF16 && d.head_dim == 128 && !cells && n_sp > 0 && n_sp <= kMaxFusedSp &&
                       d.num_heads <= kMaxEntries && !(d.variant & HC_VARIANT_SPATIAL_OWN_LAUNCH);
  // frame parts of their own launch: while the tiles leave workgroup slots free
  auto parts_at = [&](int64_t next_block) {
    const int n_all = (int)stored_frames(d, HC_SPATIAL, next_block) + (cells ? d.chunk_frames : 0);
    return n_sp > 0 ? spatial_parts(d, b->sp_tile_r, b->sp_tile_c, n_sp, n_all) : 1;
  };
  // partial slots of the Spatial heads: the current-block part (sliding windows) and,
  // with frames in parts or with the tiles in the dense launch, one per part
  auto spatial_slots = [&](bool fused, int parts) {
    return cells ? (parts > 1 ? n_sp * parts : 0) : n_sp * (fused || parts > 1 ? 1 + parts : 1);
  };
  // The workspace is sized once, for the full window in the launch form used there;
  // every other fill state (more parts never, but possibly more key splits; the own
  // launch, with one slot per Spatial head, before any history frame) plans within the
  // same slots. A capped plan (the allocation-free call) takes at most slot_cap slots:
  // fewer key splits, and no frame parts (or the own launch) when those do not fit.
  if (P.max_slots < 0) {
    const int64_t full_block = 1 + rolling_blocks(d);
    int split_slots = 0;
    for (const Entry& e : make(full_block, -1))
      if (e.nsplit > 1) split_slots += e.nsplit;
    P.max_slots = (fusable ? spatial_slots(true, 1) : spatial_slots(false, parts_at(full_block))) + split_slots;
    if (P.slot_cap >= 0) P.max_slots = std::min(P.max_slots, P.slot_cap);
  }
  P.fused = fusable && spatial_slots(true, 1) <= P.max_slots && stored_frames(d, HC_SPATIAL, b->next_block) > 0;
  P.sp_parts = P.fused ? 1 : parts_at(b->next_block);
  if (spatial_slots(P.fused, P.sp_parts) > P.max_slots) P.sp_parts = 1;
  P.ok = spatial_slots(P.fused, P.sp_parts) <= P.max_slots;
  if (!P.ok) {
    P.plan_block = -1;   // planned again (and refused again) at the next call
    return;
  }
  const int NP = P.sp_parts;
  std::vector<Entry> es = make(b->next_block, P.max_slots - spatial_slots(P.fused, NP));
  // slots: split heads and Spatial heads write fp32 partials; a Spatial head with its
  // frames in parts takes the current-block slot and one per part, merged afterwards
  int slot = 0;
  P.merges.clear();
  P.spatials.clear();
  if (cells)
    for (int h = 0; h < d.num_heads; ++h)
      if (b->labels[h] == HC_SPATIAL) {
        SpatialEntry se{};
        se.hist_off = b->head_off[h] < 0 ? 0 : b->head_off[h];
        se.head = h;
        se.cur_slot = -1;
        se.out_slot = -1;
        if (NP > 1) {
          se.out_slot = slot;
          P.merges.push_back(MergeEntry{h, slot, NP, 0});
          slot += NP;
        }
        P.spatials.push_back(se);
      }
  for (Entry& e : es) {
    const int cls = b->labels[e.head];
    if (cls == HC_SPATIAL) {   // planned whole
      e.slot = slot++;
      SpatialEntry se{};
      se.hist_off = b->head_off[e.head] < 0 ? 0 : b->head_off[e.head];
      se.head = e.head;
      se.cur_slot = e.slot;
      se.out_slot = -1;
      if (NP > 1 || P.fused) {   // partials of the history part, merged afterwards
        se.cur_slot = -1;
        se.out_slot = slot;
        P.merges.push_back(MergeEntry{e.head, e.slot, 1 + NP, 0});
        slot += NP;
      }
      P.spatials.push_back(se);
    } else if (e.nsplit > 1) {
      e.slot = slot;
      P.merges.push_back(MergeEntry{e.head, slot, e.nsplit, 0});
      slot += e.nsplit;
    }
  }
  P.entries = es;
  P.n_slots = slot;
  P.plan_block = b->next_block;
  P.max_slots = std::max(P.max_slots, slot);   // (never grows: the budget above holds)
  if (P.slot_cap >= 0 && slot > P.slot_cap) P.ok = false;
}

// Both plans of a handle follow its state (the capped one once it has been used).
void update_plans(hc_head_buffers* b) {
  build_plan(b, b->plan);
  if (b->scratch_plan.slot_cap >= 0) build_plan(b, b->scratch_plan);
}

size_t partial_bytes(int slots, int64_t lq, int head_dim) {
  return align_up((size_t)slots * lq * head_dim * 4) + align_up((size_t)slots * lq * 2 * 4);
}

}  // namespace

// ---------------------------------------------------------------- ABI
extern "C" {

const char* hc_status_string(int st) {
  switch (st) {
    case HC_OK: return "ok";
    case HC_ERR_NULL: return "null pointer";
    case HC_ERR_SHAPE: return "bad shape";
    case HC_ERR_DTYPE: return "bad dtype";
    case HC_ERR_LABEL: return "bad label";
    case HC_ERR_WORKSPACE: return "workspace too small";
    case HC_ERR_ALIGN: return "misaligned pointer";
    case HC_ERR_DEVICE: return "no gfx950 device";
    case HC_ERR_HIP: return "HIP error";
    case HC_ERR_STATE: return "bad state";
    default: return "unknown status";
  }
}

const char* hc_last_error(void) { return g_last_error.c_str(); }

hc_status hc_default_classify_params(hc_classify_params* p) {
  if (!p) return fail(HC_ERR_NULL, "params is NULL");
  p->theta_sink = p->theta_dummy = p->theta_spatial = 0.95f;
  p->theta_score = 0.755f;
  p->gamma = 5.0f;
  p->percentile = 5.0f;
  p->proxy_grid_h = p->proxy_grid_w = 0;
  p->sink_proxy_includes_current = 0;
  return ok();
}

hc_status hc_head_buffers_bytes(const hc_layer_desc* desc, const int32_t* labels, size_t* bytes) {
  HC_TRY(check_desc(desc));
  HC_TRY(check_labels(*desc, labels));
  if (!bytes) return fail(HC_ERR_NULL, "bytes is NULL");
  *bytes = 2 * layout(*desc, labels, nullptr, nullptr);
  return ok();
}

hc_status hc_build_head_buffers_at(const hc_layer_desc* desc, const int32_t* labels, const void* k_hist,
                                   const void* v_hist, int32_t n_hist_frames, int64_t next_block,
                                   void* buffer_mem, size_t buffer_bytes, hc_head_buffers** out, void* stream) {
  HC_TRY(check_desc(desc));
  HC_TRY(check_labels(*desc, labels));
  HC_TRY(check_hist_frames(*desc, n_hist_frames));
  if (!out) return fail(HC_ERR_NULL, "out is NULL");
  const hc_layer_desc& d = *desc;
  const int C = d.chunk_frames;
  const int R = rolling_blocks(d);
  if (next_block < 0) return fail(HC_ERR_SHAPE, "next_block %lld negative", (long long)next_block);
  // the window's history when block next_block is current: the sink block and the
  // min(next_block - 1, R) most recent rolling blocks
  const int64_t n_blk = (d.window_frames == C || next_block == 0) ? 0 : 1 + std::min<int64_t>(next_block - 1, R);
  if ((int64_t)n_hist_frames != n_blk * C)
    return fail(HC_ERR_SHAPE, "n_hist_frames %d does not match next_block %lld: the window then holds %lld frames",
                n_hist_frames, (long long)next_block, (long long)(n_blk * C));
  const size_t need = 2 * layout(d, labels, nullptr, nullptr);
  if (need > 0) HC_TRY(check_ptr(buffer_mem, "buffer_mem"));
  if (buffer_bytes < need) return fail(HC_ERR_WORKSPACE, "buffer_mem has %zu bytes, needs %zu", buffer_bytes, need);
  if (n_hist_frames > 0) {
    HC_TRY(check_ptr(k_hist, "k_hist"));
    HC_TRY(check_ptr(v_hist, "v_hist"));
  }
  HC_TRY(check_device());

  hc_head_buffers* b = new hc_head_buffers();
  b->desc = d;
  b->labels.assign(labels, labels + d.num_heads);
  b->mem = (char*)buffer_mem;
  b->mem_bytes = buffer_bytes;
  b->v_region = layout(d, labels, &b->head_off, &b->head_rows);
  b->next_block = next_block;

  const int64_t S = tokens_per_frame(d);
  const size_t es_ = esize(d);
  hipStream_t s = (hipStream_t)stream;
  // Logical history block i (0 = the sink block) is absolute block 0 for i = 0 and
  // next_block - n_blk + i otherwise; block b >= 1 sits at ring position 1 + (b - 1) mod R.
  // Sink heads keep block 0, Global and Spatial heads every block, a Dummy head with a
  // buffer the latest one. One copy entry per (head, block).
  std::vector<CopyEntry> copies;
  for (int h = 0; h < d.num_heads; ++h) {
    const int cls = b->labels[h];
    if (b->head_off[h] < 0) continue;
    for (int64_t i = 0; i < n_blk; ++i) {
      int64_t pos;
      if (cls == HC_SINK) {
        if (i > 0) break;
        pos = 0;
      } else if (cls == HC_DUMMY) {
        if (i != n_blk - 1) continue;
        pos = 0;
      } else {
        const int64_t blk = i == 0 ? 0 : next_block - n_blk + i;
        pos = blk == 0 ? 0 : 1 + (blk - 1) % R;
      }
      const int64_t src_row = i * C * S;
      copies.push_back(CopyEntry{((int64_t)h * d.head_dim + src_row * d.num_heads * d.head_dim) * (int64_t)es_,
                                 (b->head_off[h] + pos * C * S * d.head_dim) * (int64_t)es_});
    }
  }
  for (size_t c0 = 0; c0 < copies.size(); c0 += kMaxEntries) {
    CopyParams p{};
    p.src_k = k_hist;
    p.src_v = v_hist;
    p.dst_k = b->mem;
    p.dst_v = b->mem + b->v_region;
    p.src_stride = (int64_t)d.num_heads * d.head_dim * es_;
    p.row_bytes = d.head_dim * (int)es_;
    p.rows = (int)(C * S);
    p.n_entries = (int)std::min(copies.size() - c0, (size_t)kMaxEntries);
    for (int i = 0; i < p.n_entries; ++i) p.e[i] = copies[c0 + i];
    hipError_t e = timed(K_COPY, s, [&] { return launch_copy(p, s); });
    if (e != hipSuccess) {
      delete b;
      return fail(HC_ERR_HIP, "build copy: %s", hipGetErrorString(e));
    }
  }
  update_plans(b);
  *out = b;
  return ok();
}

hc_status hc_build_head_buffers(const hc_layer_desc* desc, const int32_t* labels, const void* k_hist,
                                const void* v_hist, int32_t n_hist_frames, void* buffer_mem,
                                size_t buffer_bytes, hc_head_buffers** out, void* stream) {
  HC_TRY(check_desc(desc));
  HC_TRY(check_hist_frames(*desc, n_hist_frames));
  return hc_build_head_buffers_at(desc, labels, k_hist, v_hist, n_hist_frames, n_hist_frames / desc->chunk_frames,
                                  buffer_mem, buffer_bytes, out, stream);
}

hc_status hc_plan_head_buffers(const hc_layer_desc* desc, const int32_t* labels, int64_t next_block,
                               hc_head_buffers** out) {
  HC_TRY(check_desc(desc));
  HC_TRY(check_labels(*desc, labels));
  if (!out) return fail(HC_ERR_NULL, "out is NULL");
  if (next_block < 0) return fail(HC_ERR_SHAPE, "next_block %lld negative", (long long)next_block);
  hc_head_buffers* b = new hc_head_buffers();
  b->desc = *desc;
  b->labels.assign(labels, labels + desc->num_heads);
  b->v_region = layout(*desc, labels, &b->head_off, &b->head_rows);
  b->next_block = next_block;
  b->plan_only = true;
  update_plans(b);
  *out = b;
  return ok();
}

hc_status hc_append_chunk(hc_head_buffers* b, const void* k_chunk, const void* v_chunk, void* stream) {
  if (!b) return fail(HC_ERR_NULL, "buffers is NULL");
  if (b->plan_only) return fail(HC_ERR_STATE, "a planning handle holds no device buffers");
  HC_TRY(check_ptr(k_chunk, "k_chunk"));
  HC_TRY(check_ptr(v_chunk, "v_chunk"));
  HC_TRY(check_device());
  const hc_layer_desc& d = b->desc;
  const int64_t blk = b->next_block;
  const int R = rolling_blocks(d);
  int pos = -1;   // block position inside the buffers
  if (d.window_frames > d.chunk_frames) pos = blk == 0 ? 0 : (R > 0 ? 1 + (int)((blk - 1) % R) : -1);
  if (pos >= 0) {
    const int64_t S = tokens_per_frame(d);
    const size_t es_ = esize(d);
    CopyParams p{};
    p.src_k = k_chunk;
    p.src_v = v_chunk;
    p.dst_k = b->mem;
    p.dst_v = b->mem + b->v_region;
    p.src_stride = (int64_t)d.num_heads * d.head_dim * es_;
    p.row_bytes = d.head_dim * (int)es_;
    p.rows = (int)(d.chunk_frames * S);
    int n = 0;
    for (int h = 0; h < d.num_heads; ++h) {
      const int cls = b->labels[h];
      if (b->head_off[h] < 0) continue;
      if (cls == HC_SINK && pos != 0) continue;
      // a Dummy buffer holds the window's latest history block: every new block while
      // rolling blocks exist, else only the sink block
      if (cls == HC_DUMMY && !(blk == 0 || R > 0)) continue;
      const int64_t at = cls == HC_DUMMY ? 0 : pos;
      p.e[n].src_off = (int64_t)h * d.head_dim * es_;
      p.e[n].dst_off = (b->head_off[h] + at * d.chunk_frames * S * d.head_dim) * (int64_t)es_;
      ++n;
    }
    p.n_entries = n;
    HC_HIP(timed(K_COPY, (hipStream_t)stream, [&] { return launch_copy(p, (hipStream_t)stream); }));
  }
  b->next_block = blk + 1;
  update_plans(b);
  return ok();
}

hc_status hc_buffers_state(const hc_head_buffers* b, int64_t* next_block) {
  if (!b || !next_block) return fail(HC_ERR_NULL, "NULL argument");
  *next_block = b->next_block;
  return ok();
}

hc_status hc_free_head_buffers(hc_head_buffers* b) {
  delete b;
  return ok();
}

hc_status hc_routed_workspace_bytes(const hc_head_buffers* b, size_t* bytes) {
  if (!b || !bytes) return fail(HC_ERR_NULL, "NULL argument");
  *bytes = partial_bytes(b->plan.max_slots, lq_of(b->desc), b->desc.head_dim);
  return ok();
}

}  // extern "C"

namespace {

hc_status check_routed_args(const hc_head_buffers* b, const void* q, const void* k_cur, const void* v_cur,
                            const void* out) {
  if (!b) return fail(HC_ERR_NULL, "buffers is NULL");
  if (b->plan_only) return fail(HC_ERR_STATE, "a planning handle holds no device buffers");
  HC_TRY(check_ptr(q, "q"));
  HC_TRY(check_ptr(k_cur, "k_cur"));
  HC_TRY(check_ptr(v_cur, "v_cur"));
  HC_TRY(check_ptr(out, "out"));
  return HC_OK;
}

// The launches of one routed call under plan P, its partial results in `workspace`
// (at least partial_bytes(P.n_slots, ...)).
// The Spatial launch geometry of a routed call (pointers and strides as in the dense
// parameters p).
void spatial_geom(const hc_head_buffers* b, const Plan& P, const DenseParams& p, SpatialGeom& g) {
  const hc_layer_desc& d = b->desc;
  g.q = p.q;
  g.k_hist = p.k_hist;
  g.v_hist = p.v_hist;
  g.out = p.out;
  g.part_o = p.part_o;
  g.part_ml = p.part_ml;
  g.hist_stride = p.hist_stride;
  g.tok_stride = p.tok_stride;
  g.lq = p.lq;
  g.frame_h = d.frame_h;
  g.frame_w = d.frame_w;
  g.chunk_frames = d.chunk_frames;
  g.n_hist_frames = (int)stored_frames(d, HC_SPATIAL, b->next_block);
  g.grid_h = d.grid_h;
  g.grid_w = d.grid_w;
  g.tile_r = b->sp_tile_r;
  g.tile_c = b->sp_tile_c;
  g.tiles_r = ceil_div(d.frame_h, g.tile_r);
  g.tiles_c = ceil_div(d.frame_w, g.tile_c);
  g.n_parts = P.sp_parts;
  g.scale_log2 = p.scale_log2;
  g.cells = spatial_cells(d) ? 1 : 0;
  g.k_cur = p.k_cur;
  g.v_cur = p.v_cur;
  g.n_entries = (int)P.spatials.size();
}

// With the Spatial tiles in the dense launch: their geometry in p.sp, the Spatial heads
// in SpatialEntry order, and one item's (frame part of a tile) cost in key tiles for the
// XCD queues (a step of 96 queries of a tile takes about 1.2 dense 128-query steps).
void fused_spatial(const hc_head_buffers* b, const Plan& P, DenseParams& p, std::vector<int>& heads, double& cost) {
  heads.clear();
  cost = 0.0;
  p.sp.n_sp = 0;
  if (!P.fused || P.spatials.empty()) return;
  spatial_geom(b, P, p, p.sp.g);
  p.sp.n_sp = (int)P.spatials.size();
  for (const SpatialEntry& se : P.spatials) heads.push_back(se.head);
  const int frames = ceil_div(p.sp.g.n_hist_frames, p.sp.g.n_parts);
  cost = 1.2 * spatial_max_chunks(p.sp.g) * frames * kStep / (double)kKeyTile + kItemOverheadTiles;
}

hc_status launch_routed(const hc_head_buffers* b, const Plan& P, const void* q, const void* k_cur,
                        const void* v_cur, void* out, void* workspace, hipStream_t s) {
  const hc_layer_desc& d = b->desc;
  const int64_t lq = lq_of(d);
  const int bf16 = d.dtype == HC_BF16;
  float* part_o = (float*)workspace;
  float* part_ml = (float*)((char*)workspace + align_up((size_t)P.n_slots * lq * d.head_dim * 4));

  DenseParams p{};
  p.q = q;
  p.k_hist = b->mem;
  p.v_hist = b->mem + b->v_region;
  p.k_cur = k_cur;
  p.v_cur = v_cur;
  p.out = out;
  p.part_o = part_o;
  p.part_ml = part_ml;
  p.hist_stride = d.head_dim;
  p.tok_stride = (int64_t)d.num_heads * d.head_dim;
  p.lq = (int)lq;
  p.nqt = ceil_div(lq, kDenseQ);
  p.scale_log2 = d.softmax_scale * 1.4426950408889634f;
  std::vector<int> sp_heads;
  double sp_cost = 0.0;
  fused_spatial(b, P, p, sp_heads, sp_cost);
  HC_TRY(run_dense(P.entries, p, d.head_dim, bf16, s, sp_heads, sp_cost));

  if (!P.spatials.empty() && !P.fused) {
    SpatialParams sp{};
    spatial_geom(b, P, p, sp);
    for (size_t i = 0; i < P.spatials.size(); ++i) sp.e[i] = P.spatials[i];
    HC_HIP(timed(bf16 ? K_SPATIAL : K_F32, s, [&] { return launch_spatial(sp, d.head_dim, bf16, s); }));
  }
  if (!P.merges.empty()) {
    MergeParams m{};
    m.part_o = part_o;
    m.part_ml = part_ml;
    m.out = out;
    m.tok_stride = p.tok_stride;
    m.lq = (int)lq;
    m.head_dim = d.head_dim;
    m.n_entries = (int)P.merges.size();
    for (size_t i = 0; i < P.merges.size(); ++i) m.e[i] = P.merges[i];
    HC_HIP(timed(K_MERGE, s, [&] { return launch_merge(m, d.head_dim, bf16, s); }));
  }
  return HC_OK;
}


}  // namespace

extern "C" {

hc_status hc_routed_attention(const hc_head_buffers* b, const void* q, const void* k_cur, const void* v_cur,
                              void* out, void* workspace, size_t ws_bytes, void* stream) {
  HC_TRY(check_routed_args(b, q, k_cur, v_cur, out));
  const size_t need = partial_bytes(b->plan.n_slots, lq_of(b->desc), b->desc.head_dim);
  if (b->plan.n_slots > 0) HC_TRY(check_ptr(workspace, "workspace"));
  if (ws_bytes < need) return fail(HC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, need);
  HC_TRY(check_device());
  HC_TRY(launch_routed(b, b->plan, q, k_cur, v_cur, out, workspace, (hipStream_t)stream));
  return ok();
}

hc_status hc_routed_attention_noalloc(hc_head_buffers* b, const void* q, const void* k_cur, const void* v_cur,
                                      void* out, void* stream) {
  HC_TRY(check_routed_args(b, q, k_cur, v_cur, out));
  HC_TRY(check_device());
  void* scratch = nullptr;
  size_t cap = 0;
  HC_HIP(noalloc_scratch(&scratch, &cap));
  const hc_layer_desc& d = b->desc;
  const int64_t lq = lq_of(d);
  Plan& P = b->scratch_plan;
  if (P.slot_cap < 0) {   // first call on this handle: plan within the scratch
    int slots = (int)(cap / ((size_t)lq * (d.head_dim + 2) * 4));
    while (slots > 0 && partial_bytes(slots, lq, d.head_dim) > cap) --slots;
    P.slot_cap = slots;
    build_plan(b, P);
  }
  if (!P.ok)
    return fail(HC_ERR_WORKSPACE, "the Spatial heads' partial results need more than the %zu-byte scratch", cap);
  if (partial_bytes(P.n_slots, lq, d.head_dim) > cap)
    return fail(HC_ERR_WORKSPACE, "internal: plan of %d slots exceeds the scratch", P.n_slots);
  HC_TRY(launch_routed(b, P, q, k_cur, v_cur, out, scratch, (hipStream_t)stream));
  return ok();
}

// ---------------------------------------------------------------- classification
namespace {

struct ClassifyLayout {
  int n_mid, slots_per_head, slots;
  size_t part_o, part_ml, stats, total;
};

ClassifyLayout classify_layout(const hc_layer_desc& d, int32_t n_hist) {
  ClassifyLayout L{};
  const int64_t lq = lq_of(d);
  // middle history frames, split into ranges of one block (rounded up to the key tile)
  const int64_t blk = (int64_t)d.chunk_frames * tokens_per_frame(d);
  const int64_t split = (blk + kKeyTile - 1) / kKeyTile * kKeyTile;
  const int64_t mid_keys = (int64_t)std::max(0, n_hist - d.chunk_frames) * tokens_per_frame(d);
  L.n_mid = (int)((mid_keys + split - 1) / split);
  L.slots_per_head = 3 + L.n_mid;
  L.slots = L.slots_per_head * d.num_heads;
  L.part_o = 0;
  L.part_ml = align_up((size_t)L.slots * lq * d.head_dim * 4);
  L.stats = L.part_ml + align_up((size_t)L.slots * lq * 2 * 4);
  L.total = L.stats + align_up((size_t)d.num_heads * lq * 4 * 4);
  return L;
}

hc_status check_params(const hc_classify_params* p) {
  if (!p) return fail(HC_ERR_NULL, "params is NULL");
  if (!(p->percentile >= 0.f && p->percentile <= 100.f)) return fail(HC_ERR_SHAPE, "percentile outside [0, 100]");
  if (p->proxy_grid_h < 0 || p->proxy_grid_w < 0) return fail(HC_ERR_SHAPE, "negative proxy grid");
  return HC_OK;
}

}  // namespace

hc_status hc_classify_workspace_bytes(const hc_layer_desc* desc, const hc_classify_params* params,
                                      int32_t n_hist_frames, size_t* bytes) {
  HC_TRY(check_desc(desc));
  HC_TRY(check_params(params));
  HC_TRY(check_hist_frames(*desc, n_hist_frames));
  if (!bytes) return fail(HC_ERR_NULL, "bytes is NULL");
  *bytes = classify_layout(*desc, n_hist_frames).total;
  return ok();
}

hc_status hc_reduce_statistics(const float* per_token, int64_t lq, int32_t head_dim, double gamma,
                               double percentile, double* out) {
  if (!per_token || !out) return fail(HC_ERR_NULL, "NULL argument");
  if (lq < 1 || head_dim < 1) return fail(HC_ERR_SHAPE, "empty statistics");
  double s0 = 0, s1 = 0, s2 = 0, se = 0;
  std::vector<double> cp(lq);
  for (int64_t t = 0; t < lq; ++t) {
    s0 += per_token[t * 4 + 0];
    s1 += per_token[t * 4 + 1];
    s2 += per_token[t * 4 + 2];
    se += per_token[t * 4 + 3];
    cp[t] = per_token[t * 4 + 2];
  }
  // linear interpolation between the order statistics i and i + 1 (selected, not sorted)
  const double pos = percentile / 100.0 * (double)(lq - 1);
  const int64_t i = std::min<int64_t>((int64_t)std::floor(pos), lq - 1);
  const double frac = pos - (double)i;
  std::nth_element(cp.begin(), cp.begin() + i, cp.end());
  const double lo = cp[i];
  const double hi = i + 1 < lq ? *std::min_element(cp.begin() + i + 1, cp.end()) : lo;
  const double pct = i + 1 < lq ? lo + frac * (hi - lo) : lo;
  const double mse = se / ((double)lq * head_dim);
  out[0] = s0 / lq;
  out[1] = s1 / lq;
  out[2] = s2 / lq;
  out[3] = pct;
  out[4] = mse;
  out[5] = pct - gamma * mse;
  return ok();
}

int32_t hc_decide(double cs, double cd, double cp, double score, const hc_classify_params* p) {
  hc_classify_params def;
  if (!p) {
    hc_default_classify_params(&def);
    p = &def;
  }
  if (cs >= (double)p->theta_sink) return HC_SINK;
  if (cd >= (double)p->theta_dummy) return HC_DUMMY;
  if (cp >= (double)p->theta_spatial && score >= (double)p->theta_score) return HC_SPATIAL;
  return HC_GLOBAL;
}

hc_status hc_classify_heads(const hc_layer_desc* desc, const hc_classify_params* params, const void* q,
                            const void* k_hist, const void* v_hist, int32_t n_hist_frames, const void* k_cur,
                            const void* v_cur, void* workspace, size_t ws_bytes, int32_t* labels_out,
                            double* stats_out, void* stream) {
  HC_TRY(check_desc(desc));
  HC_TRY(check_params(params));
  HC_TRY(check_hist_frames(*desc, n_hist_frames));
  const hc_layer_desc& d = *desc;
  if (n_hist_frames < d.chunk_frames)
    return fail(HC_ERR_STATE, "classification needs the sink block: n_hist_frames %d < %d", n_hist_frames,
                d.chunk_frames);
  HC_TRY(check_ptr(q, "q"));
  HC_TRY(check_ptr(k_hist, "k_hist"));
  HC_TRY(check_ptr(v_hist, "v_hist"));
  HC_TRY(check_ptr(k_cur, "k_cur"));
  HC_TRY(check_ptr(v_cur, "v_cur"));
  HC_TRY(check_ptr(workspace, "workspace"));
  if (!labels_out) return fail(HC_ERR_NULL, "labels_out is NULL");
  const ClassifyLayout L = classify_layout(d, n_hist_frames);
  if (ws_bytes < L.total) return fail(HC_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", ws_bytes, L.total);
  HC_TRY(check_device());

  hipStream_t s = (hipStream_t)stream;
  const int bf16 = d.dtype == HC_BF16;
  const int64_t S = tokens_per_frame(d);
  const int64_t lq = lq_of(d);
  const int H = d.num_heads, D = d.head_dim;
  float* part_o = (float*)((char*)workspace + L.part_o);
  float* part_ml = (float*)((char*)workspace + L.part_ml);
  float* stats = (float*)((char*)workspace + L.stats);

  // Dense partials per head: current block (slot 0), sink block (slot 1), and one
  // slot per middle block (slots 3..): each is one C*S-key range.
  std::vector<Entry> es;
  const int blk = (int)(d.chunk_frames * S);
  for (int h = 0; h < H; ++h) {
    const int base = h * L.slots_per_head;
    Entry cur{0, 0, blk, h, 1, blk, base};
    cur.split_len = ceil_div(blk, kKeyTile) * kKeyTile;
    Entry first{(int64_t)h * D, blk, 0, h, 1, cur.split_len, base + 1};
    es.push_back(cur);
    es.push_back(first);
    if (L.n_mid > 0) {   // every middle key, in n_mid ranges of split_len keys (the last one shorter)
      const int mid_keys = (int)((int64_t)(n_hist_frames - d.chunk_frames) * S);
      Entry mid{(int64_t)h * D + (int64_t)blk * H * D, mid_keys, 0, h, L.n_mid, cur.split_len, base + 3};
      es.push_back(mid);
    }
  }
  DenseParams p{};
  p.q = q;
  p.k_hist = k_hist;
  p.v_hist = v_hist;
  p.k_cur = k_cur;
  p.v_cur = v_cur;
  p.out = nullptr;
  p.part_o = part_o;
  p.part_ml = part_ml;
  p.hist_stride = (int64_t)H * D;
  p.tok_stride = (int64_t)H * D;
  p.lq = (int)lq;
  p.nqt = ceil_div(lq, kDenseQ);
  p.scale_log2 = d.softmax_scale * 1.4426950408889634f;
  HC_TRY(run_dense(es, p, D, bf16, s));

  // Spatial proxy: gathered history windows of every head (slot 2), partial mode.
  SpatialParams sp{};
  sp.q = q;
  sp.k_hist = k_hist;
  sp.v_hist = v_hist;
  sp.part_o = part_o;
  sp.part_ml = part_ml;
  sp.hist_stride = (int64_t)H * D;
  sp.tok_stride = (int64_t)H * D;
  sp.lq = (int)lq;
  sp.frame_h = d.frame_h;
  sp.frame_w = d.frame_w;
  sp.chunk_frames = d.chunk_frames;
  sp.n_hist_frames = n_hist_frames;
  sp.grid_h = params->proxy_grid_h > 0 ? params->proxy_grid_h : d.grid_h;
  sp.grid_w = params->proxy_grid_w > 0 ? params->proxy_grid_w : d.grid_w;
  choose_spatial_tile(d.frame_h, d.frame_w, sp.grid_h, sp.grid_w, false, H, &sp.tile_r, &sp.tile_c);
  sp.tiles_r = ceil_div(d.frame_h, sp.tile_r);
  sp.tiles_c = ceil_div(d.frame_w, sp.tile_c);
  sp.n_parts = 1;
  sp.scale_log2 = p.scale_log2;
  for (int h0 = 0; h0 < H; h0 += kMaxEntries) {
    const int n = std::min(H - h0, kMaxEntries);
    for (int i = 0; i < n; ++i) {
      const int h = h0 + i;
      sp.e[i] = SpatialEntry{(int64_t)h * D, h, -1, h * L.slots_per_head + 2, 0};
    }
    sp.n_entries = n;
    HC_HIP(timed(bf16 ? K_SPATIAL : K_F32, s, [&] { return launch_spatial(sp, D, bf16, s); }));
  }

  StatsParams st{};
  st.part_o = part_o;
  st.part_ml = part_ml;
  st.stats = stats;
  st.lq = (int)lq;
  st.num_heads = H;
  st.head_dim = D;
  st.n_mid = L.n_mid;
  st.sink_with_cur = params->sink_proxy_includes_current ? 1 : 0;
  st.slots_per_head = L.slots_per_head;
  HC_HIP(timed(K_STATS, s, [&] { return launch_stats(st, s); }));

  std::vector<float> host((size_t)H * lq * 4);
  HC_HIP(hipMemcpyAsync(host.data(), stats, host.size() * sizeof(float), hipMemcpyDeviceToHost, s));
  HC_HIP(hipStreamSynchronize(s));
  // per-head reductions (independent; inputs validated above, so they cannot fail) on
  // a few host threads
  std::vector<double> red((size_t)H * 6);
  auto reduce = [&](int h) {
    hc_reduce_statistics(host.data() + (size_t)h * lq * 4, lq, D, params->gamma, params->percentile,
                         red.data() + (size_t)h * 6);
  };
  const int n_thr = std::max(1, std::min<int>({H, 8, (int)std::thread::hardware_concurrency()}));
  std::vector<std::thread> pool;
  for (int t = 1; t < n_thr; ++t)
    pool.emplace_back([&, t] {
      for (int h = t; h < H; h += n_thr) reduce(h);
    });
  for (int h = 0; h < H; h += n_thr) reduce(h);
  for (std::thread& th : pool) th.join();
  for (int h = 0; h < H; ++h) {
    const double* o = red.data() + (size_t)h * 6;
    labels_out[h] = hc_decide(o[0], o[1], o[2], o[5], params);
    if (stats_out)
      for (int i = 0; i < 6; ++i) stats_out[h * 6 + i] = o[i];
  }
  return ok();
}

// ---------------------------------------------------------------- index exports
hc_status hc_debug_slot_table(const hc_head_buffers* b, int32_t* frames) {
  if (!b || !frames) return fail(HC_ERR_NULL, "NULL argument");
  const hc_layer_desc& d = b->desc;
  const int C = d.chunk_frames, HF = d.window_frames - C;
  const int R = rolling_blocks(d);
  for (int h = 0; h < d.num_heads; ++h) {
    int32_t* row = frames + (size_t)h * HF;
    for (int i = 0; i < HF; ++i) row[i] = -1;
    const int cls = b->labels[h];
    if (HF == 0 || b->next_block <= 0) continue;
    if (cls == HC_DUMMY) {
      if (!dummy_prev(d)) continue;
      const int64_t blk = R > 0 ? b->next_block - 1 : 0;   // the window's latest history block
      for (int i = 0; i < C; ++i) row[i] = (int32_t)(blk * C + i);
      continue;
    }
    for (int i = 0; i < C; ++i) row[i] = i;   // sink block (absolute block 0)
    if (cls == HC_SINK || R == 0) continue;
    // the latest block stored at each rolling position
    for (int64_t blk = std::max<int64_t>(1, b->next_block - R); blk < b->next_block; ++blk) {
      const int pos = 1 + (int)((blk - 1) % R);
      for (int i = 0; i < C; ++i) row[pos * C + i] = (int32_t)(blk * C + i);
    }
  }
  return ok();
}

hc_status hc_debug_head_region(const hc_head_buffers* b, int32_t head, int64_t* k_offset, int64_t* v_offset,
                               int64_t* rows) {
  if (!b || !k_offset || !v_offset || !rows) return fail(HC_ERR_NULL, "NULL argument");
  if (head < 0 || head >= b->desc.num_heads) return fail(HC_ERR_SHAPE, "head %d out of range", head);
  const size_t es_ = esize(b->desc);
  if (b->head_off[head] < 0) {
    *k_offset = *v_offset = -1;
    *rows = 0;
  } else {
    *k_offset = b->head_off[head] * (int64_t)es_;
    *v_offset = (int64_t)b->v_region + b->head_off[head] * (int64_t)es_;
    *rows = b->head_rows[head];
  }
  return ok();
}

hc_status hc_debug_gather_origins(const hc_layer_desc* desc, int32_t grid_h, int32_t grid_w, void* r0c0,
                                  void* stream) {
  HC_TRY(check_desc(desc));
  HC_TRY(check_ptr(r0c0, "r0c0"));
  if (grid_h < 1 || grid_w < 1) return fail(HC_ERR_SHAPE, "grid must be >= 1");
  HC_TRY(check_device());
  HC_HIP(launch_gather_origins(desc->frame_h, desc->frame_w, grid_h, grid_w,
                              (desc->variant & HC_VARIANT_SPATIAL_CELLS) ? 1 : 0, (int32_t*)r0c0,
                              (hipStream_t)stream));
  return ok();
}

hc_status hc_debug_routed_plan(const hc_head_buffers* b, int32_t* entries, int32_t max_entries, int32_t* n_entries,
                               int32_t* n_items) {
  if (!b || !n_entries || !n_items) return fail(HC_ERR_NULL, "NULL argument");
  std::vector<Entry> es = b->plan.entries;
  std::stable_sort(es.begin(), es.end(), [](const Entry& a, const Entry& x) { return a.split_len > x.split_len; });
  const int nqt = ceil_div(lq_of(b->desc), kDenseQ);
  int items = 0;
  for (size_t i = 0; i < es.size(); ++i) {
    if (entries && (int)i < max_entries) {
      int32_t* r = entries + i * 8;
      r[0] = es[i].head;
      r[1] = es[i].hist_len;
      r[2] = es[i].cur_len;
      r[3] = es[i].nsplit;
      r[4] = es[i].split_len;
      r[5] = es[i].slot;
      r[6] = items;
      r[7] = kDenseQ;
    }
    items += es[i].nsplit * nqt;
  }
  *n_entries = (int32_t)es.size();
  *n_items = items;
  return ok();
}

hc_status hc_debug_dense_queues(const hc_head_buffers* b, int32_t* runs, int32_t* n_runs, int32_t* queue_len) {
  if (!b || !runs || !n_runs || !queue_len) return fail(HC_ERR_NULL, "NULL argument");
  DenseParams base{};
  base.lq = (int)lq_of(b->desc);
  base.nqt = ceil_div(base.lq, kDenseQ);
  std::vector<int> sp_heads;
  double sp_cost = 0.0;
  fused_spatial(b, b->plan, base, sp_heads, sp_cost);
  std::vector<DenseParams> ps;
  HC_TRY(dense_launches(b->plan.entries, base, &ps, sp_heads, sp_cost));
  for (int x = 0; x < kXcds; ++x) n_runs[x] = 0;
  *queue_len = 0;
  if (ps.empty()) return ok();
  const DenseParams& p = ps[0];
  for (int x = 0; x < kXcds; ++x) {
    n_runs[x] = p.xcd_nrun[x];
    for (int r = 0; r < kXcdRuns; ++r) {
      runs[(x * kXcdRuns + r) * 2] = r < p.xcd_nrun[x] ? p.xcd_run[x][r].first : -1;
      runs[(x * kXcdRuns + r) * 2 + 1] = r < p.xcd_nrun[x] ? p.xcd_run[x][r].count : 0;
    }
  }
  *queue_len = p.xcd_len;
  return ok();
}

hc_status hc_debug_spatial_plan(const hc_head_buffers* b, int32_t* plan) {
  if (!b || !plan) return fail(HC_ERR_NULL, "NULL argument");
  const bool any = !b->plan.spatials.empty();
  plan[0] = any ? b->sp_tile_r : 0;
  plan[1] = any ? b->sp_tile_c : 0;
  plan[2] = any ? b->plan.sp_parts : 0;
  plan[3] = b->plan.n_slots;
  plan[4] = any && b->plan.fused ? 1 : 0;
  return ok();
}

hc_status hc_timing_enable(int32_t enable) {
  std::lock_guard<std::mutex> lk(g_time_mutex);
  g_timing = enable != 0;
  return ok();
}

hc_status hc_timing_read(double* ms_out, int64_t* counts_out) {
  if (!ms_out || !counts_out) return fail(HC_ERR_NULL, "NULL argument");
  std::vector<TimedLaunch> v;
  {
    std::lock_guard<std::mutex> lk(g_time_mutex);
    v.swap(g_timed);
  }
  for (int i = 0; i < K_NUM; ++i) {
    ms_out[i] = 0.0;
    counts_out[i] = 0;
  }
  hc_status st = HC_OK;
  for (auto& t : v) {
    float ms = 0.f;
    if (hipEventSynchronize(t.b) != hipSuccess || hipEventElapsedTime(&ms, t.a, t.b) != hipSuccess)
      st = fail(HC_ERR_HIP, "event timing failed");
    ms_out[t.kind] += ms;
    counts_out[t.kind] += 1;
    (void)hipEventDestroy(t.a);
    (void)hipEventDestroy(t.b);
  }
  return st == HC_OK ? ok() : st;
}

}  // extern "C"
