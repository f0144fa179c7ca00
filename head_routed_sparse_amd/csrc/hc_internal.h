// Internal structures shared by the host planner (hc_api.cpp) and the HIP kernels.
// Not part of the public ABI (include/headcast.h).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace hc {

constexpr int kMaxEntries = 64;   // dense work entries per launch (kernel arguments by value)
constexpr int kKeyTile = 64;      // granularity of key-range splits (a multiple of the 32-key step)
constexpr int kDenseQ = 128;      // queries per dense workgroup (query tile)
constexpr int kXcds = 8;          // XCDs; workgroup i is dispatched to XCD i % 8, in order i / 8
constexpr int kXcdRuns = 16;      // runs of consecutive items in one XCD's queue
constexpr int kSpTileMax = 32;    // positions per Spatial query tile (one 32-query MFMA block)
constexpr int kStep = 32;         // keys per pipeline step

// First row (or column) of the g-wide Spatial window around pos in a frame of `extent`
// rows (columns): the query sits at offset g/2, and the window is shifted (never cut)
// to stay inside the frame; g >= extent covers the whole frame.
__host__ __device__ __forceinline__ int win_origin(int pos, int g, int extent) {
  const int o = pos - g / 2;
  const int hi = extent - g > 0 ? extent - g : 0;
  return o < 0 ? 0 : (o > hi ? hi : o);
}

// Non-overlapping cells: origin and size of the cell holding pos (the last cell keeps
// the remainder rows / columns).
__host__ __device__ __forceinline__ int cell_origin(int pos, int cell) { return (pos / cell) * cell; }
__host__ __device__ __forceinline__ int cell_extent(int pos, int cell, int extent) {
  const int o = cell_origin(pos, cell);
  return cell < extent - o ? cell : extent - o;
}

// One dense work entry: a head's queries against one contiguous key range made of
// [history rows 0..hist_len) followed by [current-block rows 0..cur_len). The range is
// split into nsplit pieces of split_len keys; every (split, query tile) is one item.
struct DenseEntry {
  int64_t hist_off;    // element offset of history row 0 (into k_hist / v_hist)
  int32_t hist_len;    // history keys
  int32_t cur_len;     // current-block keys (0 or C*S)
  int32_t head;        // head index: column of q / k_cur / v_cur / out
  int32_t nsplit;      // key splits
  int32_t split_len;   // keys per split (multiple of kKeyTile)
  int32_t slot;        // first partial slot, or -1: write the normalised output
  int32_t item_begin;  // index of this entry's first item
  int32_t pad;
};

// Items [first, first + count) of one dense launch, run in order by one XCD.
struct XcdRun {
  int32_t first;
  int32_t count;
};

// Spatial history gather for the Spatial heads: every query (f, r, c) of the current
// block against the g x g window of every history frame; merged with the dense
// current-block partial held in cur_slot (final mode), or written as a partial.
struct SpatialEntry {
  int64_t hist_off;   // element offset of history row 0
  int32_t head;
  int32_t cur_slot;   // partial slot of the current-block part; -1 in partial mode
  int32_t out_slot;   // first partial slot to write (partial mode), -1 in final mode
  int32_t pad;
};

struct SpatialGeom {
  const void* q;
  const void* k_hist;
  const void* v_hist;
  void* out;
  float* part_o;
  float* part_ml;
  int64_t hist_stride;
  int64_t tok_stride;
  int32_t lq;
  int32_t frame_h, frame_w, chunk_frames;
  int32_t n_hist_frames;   // valid history frames (a prefix of the buffer positions)
  int32_t grid_h, grid_w;
  int32_t tile_r, tile_c;    // query tile: rows x cols of positions (tile_r * tile_c <= kSpTileMax)
  int32_t tiles_r, tiles_c;  // position tiles per frame
  int32_t n_parts;           // workgroups per tile, each over its share of the frames; with
                             // more than one, part i writes the partial of slot out_slot + i
  int32_t n_entries;
  float scale_log2;
  int32_t cells;           // 1: own non-overlapping cell in every window frame (current
                           //    block read from k_cur / v_cur), output written directly
  const void* k_cur;       // [C*S][H][D], cell mode only
  const void* v_cur;
};

struct SpatialParams : SpatialGeom {
  SpatialEntry e[kMaxEntries];
};

// Spatial tiles as the last items of a dense launch (d = 128, bf16, sliding windows):
// item n_dense_items + s is tile s % tiles, frame part s / tiles % g.n_parts, of Spatial
// head entry e[sp_entry[s / (tiles * g.n_parts)]]; part i writes the partial of slot
// e[...].slot + 1 + i, which the merge kernel joins with the current-block partial in
// e[...].slot.
constexpr int kMaxFusedSp = 16;
struct FusedSpatial {
  SpatialGeom g;           // q, out, partials and strides as in the dense parameters
  int32_t n_dense_items;   // items below are dense items
  int32_t n_sp;            // Spatial head entries (0: no Spatial items)
  int8_t sp_entry[kMaxFusedSp];
};

// Unions of up to this many 32-key chunks keep their per-chunk tables in LDS.
constexpr int kTblChunks = 8;

// 32-key chunks of the largest union of a tile's windows; rows and columns of the union
// vary independently, so the largest union is the product of the largest row and
// column extents. Host code.
inline int spatial_max_chunks(const SpatialGeom& p) {
  int ur = 0, uc = 0;
  const bool cells = p.cells != 0;
  for (int r0 = 0; r0 < p.frame_h; r0 += p.tile_r) {
    const int r1 = std::min(r0 + p.tile_r, p.frame_h) - 1;
    const int lo = cells ? cell_origin(r0, p.grid_h) : win_origin(r0, p.grid_h, p.frame_h);
    const int hi = cells ? cell_origin(r1, p.grid_h) + cell_extent(r1, p.grid_h, p.frame_h)
                         : win_origin(r1, p.grid_h, p.frame_h) + std::min(p.grid_h, p.frame_h);
    ur = std::max(ur, hi - lo);
  }
  for (int c0 = 0; c0 < p.frame_w; c0 += p.tile_c) {
    const int c1 = std::min(c0 + p.tile_c, p.frame_w) - 1;
    const int lo = cells ? cell_origin(c0, p.grid_w) : win_origin(c0, p.grid_w, p.frame_w);
    const int hi = cells ? cell_origin(c1, p.grid_w) + cell_extent(c1, p.grid_w, p.frame_w)
                         : win_origin(c1, p.grid_w, p.frame_w) + std::min(p.grid_w, p.frame_w);
    uc = std::max(uc, hi - lo);
  }
  return (ur * uc + kStep - 1) / kStep;
}

// Whether every tile's union fits the tables (kTblChunks chunks). Host code.
inline bool spatial_table(const SpatialGeom& p) { return spatial_max_chunks(p) <= kTblChunks; }

struct DenseParams {
  const void* q;         // [lq][H][D]
  const void* k_hist;    // history rows, row stride hist_stride elements
  const void* v_hist;
  const void* k_cur;     // [C*S][H][D]
  const void* v_cur;
  void* out;             // [lq][H][D], same dtype as q
  float* part_o;         // [slot][lq][D] fp32, unnormalised
  float* part_ml;        // [slot][lq][2]: running max (log2 units, scale folded) and sum
  int64_t hist_stride;   // elements between consecutive history rows
  int64_t tok_stride;    // H*D: elements between tokens of q / k_cur / v_cur / out
  int32_t lq;            // queries per head
  int32_t nqt;           // query tiles per head
  int32_t n_entries;
  int32_t n_items;
  float scale_log2;      // softmax_scale * log2(e)
  int32_t xcd_len;       // workgroups of each XCD's queue (grid = kXcds * xcd_len)
  DenseEntry e[kMaxEntries];
  int32_t xcd_nrun[kXcds];           // runs in each XCD's queue
  XcdRun xcd_run[kXcds][kXcdRuns];   // queue x = the items of its runs, in order
  FusedSpatial sp;                   // n_sp > 0: Spatial tiles after the dense items
};

// Merge of partial slots into the normalised output (split keys, Spatial merge).
struct MergeEntry {
  int32_t head;
  int32_t slot;
  int32_t nslot;
  int32_t pad;
};

struct MergeParams {
  const float* part_o;
  const float* part_ml;
  void* out;
  int64_t tok_stride;
  int32_t lq;
  int32_t n_entries;
  int32_t head_dim;
  int32_t pad;
  MergeEntry e[kMaxEntries];
};


// Row copy: `rows` rows of row_bytes from src (byte offset src_off, byte stride
// src_stride) to contiguous rows at dst byte offset dst_off. K and V move together.
struct CopyEntry {
  int64_t src_off;
  int64_t dst_off;
};

struct CopyParams {
  const void* src_k;
  const void* src_v;
  void* dst_k;
  void* dst_v;
  int64_t src_stride;
  int32_t rows;
  int32_t row_bytes;
  int32_t n_entries;
  int32_t pad;
  CopyEntry e[kMaxEntries];
};

// Classifier statistics: per (head, token) cosines of the three proxies and the
// squared error of the Spatial proxy, all against the full-window reference.
struct StatsParams {
  const float* part_o;
  const float* part_ml;
  float* stats;          // [H][lq][4]: cos_sink, cos_dummy, cos_spatial, sq_err_spatial
  int32_t lq;
  int32_t num_heads;
  int32_t head_dim;
  int32_t n_mid;         // partial slots of the middle history frames per head
  int32_t sink_with_cur; // sink proxy also sees the current block
  int32_t pad;
  // slot index of head h: cur = h*slots_per_head + 0, first = +1, spatial = +2, mid = +3..
  int32_t slots_per_head;
  int32_t pad2;
};

// Kernel ids for the optional per-kernel event timing.
enum KernelId { K_DENSE = 0, K_MERGE, K_SPATIAL, K_COPY, K_STATS, K_F32, K_NUM };

// Launchers (defined in the .hip files). Each returns the hipError_t of the launch.
hipError_t launch_dense(const DenseParams& p, int head_dim, int bf16, hipStream_t s);
hipError_t launch_merge(const MergeParams& p, int head_dim, int bf16, hipStream_t s);
hipError_t launch_spatial(const SpatialParams& p, int head_dim, int bf16, hipStream_t s);
hipError_t launch_copy(const CopyParams& p, hipStream_t s);
hipError_t launch_stats(const StatsParams& p, hipStream_t s);
hipError_t launch_gather_origins(int frame_h, int frame_w, int grid_h, int grid_w, int cells, int32_t* out,
                                 hipStream_t s);


// Device address and size of the library's own scratch array on the current device (the
// partial results of the allocation-free routed call). Looked up once per device.
hipError_t noalloc_scratch(void** ptr, size_t* bytes);

}  // namespace hc
