// Dense varlen-per-head attention for gfx950: the Sink, Dummy and Global paths, the
// current-block part of the Spatial path, and the classifier's reference and block
// proxies (HeadCast Sec. 4.4 "Head-Specific Attention"; Sec. 4.2 Eq. 2).
//
// One workgroup = 128 queries of one head against one key range: a split of the
// head's [history rows ; current-block rows]. History rows come from the compact
// per-head buffer (stride D) or, for the classifier, from the monolithic cache
// (stride H*D); current-block rows are read in place from [C*S][H][D]. Items run from
// per-XCD queues (planned on the host) that keep the query tiles of one key range on
// one XCD, so that they share the range through its L2, each queue longest first.
//
// A workgroup is four waves of 32 queries (one per SIMD, all state in VGPRs). For D=128
// two workgroups share a CU, each with its own LDS ring and barrier, so that one's
// softmax overlaps the other's MFMAs; for D=64 (119 registers, a 32 KB ring) four do,
// which the softmax needs more, with half the matrix work per score. The step pipeline
// (direct loads into an LDS ring, transposed V reads, reference-max softmax) is in
// hc_pipe.h.
//
// For d = 128 with Spatial heads on sliding windows, the routed call appends the
// Spatial path's tiles (hc_spatial_tile.h) to the launch as its last, shortest items:
// they fill the workgroup slots that the dense items leave idle at the end, and write
// fp32 partials that the merge kernel joins with the heads' current-block partials.
#include "hc_spatial_tile.h"

namespace hc {

namespace {

// This workgroup's item: position blockIdx.x / 8 of the queue of XCD blockIdx.x % 8
// (-1 past the end of the queue).
__device__ __forceinline__ int queue_item(const DenseParams& p) {
  const int xq = blockIdx.x % kXcds;
  int k = blockIdx.x / kXcds;
  for (int r = 0; r < p.xcd_nrun[xq]; ++r) {
    if (k < p.xcd_run[xq][r].count) return p.xcd_run[xq][r].first + k;
    k -= p.xcd_run[xq][r].count;
  }
  return -1;
}

// One dense item (128 queries of one head against one key split) with the LDS ring at
// `lds` (four stages).
template <int D, int QB>
__device__ __forceinline__ void dense_item(const DenseParams& p, int item, lds_char* lds) {
  constexpr int W = kDenseQ / (32 * QB);   // waves per workgroup
  using R = Ring<D, QB, W>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NS = 4;   // ring stages
  int ei = 0;
  while (ei + 1 < p.n_entries && item >= p.e[ei + 1].item_begin) ++ei;
  const DenseEntry e = p.e[ei];
  const int local = item - e.item_begin;
  const int split = local / p.nqt;
  const int qt = local - split * p.nqt;

  const int k_begin = split * e.split_len;
  const int k_end = min(e.hist_len + e.cur_len, k_begin + e.split_len);
  const int n = (k_end - k_begin + kStep - 1) / kStep;   // steps (>= 1)

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  // this wave's query blocks: B operands of S^T = K Q^T
  int q_row[QB];
  u32x4 q[QB][KS];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    q_row[b] = qt * kDenseQ + (wave * QB + b) * 32 + l32;
    const uint16_t* qp = (const uint16_t*)p.q + (int64_t)min(q_row[b], p.lq - 1) * p.tok_stride +
                         (int64_t)e.head * D + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) q[b][ks] = *(const u32x4*)(qp + ks * 16);
  }

  LaneAddr<D, QB, W> la;
  la.init(wave, lane);
  const char* kh = (const char*)p.k_hist + e.hist_off * 2;
  const char* vh = (const char*)p.v_hist + e.hist_off * 2;
  const char* kc = (const char*)p.k_cur + (int64_t)e.head * D * 2;
  const char* vc = (const char*)p.v_cur + (int64_t)e.head * D * 2;
  const int64_t hs = p.hist_stride * 2, ts = p.tok_stride * 2;   // bytes
  const int hl = e.hist_len;
  uint32_t off_h[R::kLoads], off_c[R::kLoads];   // byte offsets within a step, per segment
#pragma unroll
  for (int i = 0; i < R::kLoads; ++i) {
    off_h[i] = (uint32_t)(la.ld_row[i] * hs) + la.ld_chunk[i];
    off_c[i] = (uint32_t)(la.ld_row[i] * ts) + la.ld_chunk[i];
  }

  // direct loads of step t (keys k_begin + 32 t ...) into ring stage `stage`
  auto issue = [&](int t, int stage) {
    const int k0 = k_begin + t * kStep;
    if (k0 + kStep <= min(hl, k_end)) {   // whole step in the history segment
      const char* kb = kh + (int64_t)k0 * hs;
      const char* vb = vh + (int64_t)k0 * hs;
#pragma unroll
      for (int i = 0; i < R::kLoads; ++i) {
        dma16(kb, off_h[i], la.dst(lds, stage, wave, i, 0));
        dma16(vb, off_h[i], la.dst(lds, stage, wave, i, 1));
      }
    } else if (k0 >= hl && k0 + kStep <= k_end) {   // whole step in the current block
      const char* kb = kc + (int64_t)(k0 - hl) * ts;
      const char* vb = vc + (int64_t)(k0 - hl) * ts;
#pragma unroll
      for (int i = 0; i < R::kLoads; ++i) {
        dma16(kb, off_c[i], la.dst(lds, stage, wave, i, 0));
        dma16(vb, off_c[i], la.dst(lds, stage, wave, i, 1));
      }
    } else {   // straddles the segments or runs past the end: per-row offsets, clamped
#pragma unroll
      for (int i = 0; i < R::kLoads; ++i) {
        const int kk = min(k0 + la.ld_row[i], k_end - 1);
        const bool h = kk < hl;
        const uint32_t off = (uint32_t)(h ? (int64_t)kk * hs : (int64_t)(kk - hl) * ts) + la.ld_chunk[i];
        if (h) {   // lanes of the two segments issue in turn
          dma16(kh, off, la.dst(lds, stage, wave, i, 0));
          dma16(vh, off, la.dst(lds, stage, wave, i, 1));
        } else {
          dma16(kc, off, la.dst(lds, stage, wave, i, 0));
          dma16(vc, off, la.dst(lds, stage, wave, i, 1));
        }
      }
    }
  };
  // only the last step can be ragged
  auto mask_last = [&](f32x16 (&sc)[QB]) {
    const int valid = k_end - (k_begin + (n - 1) * kStep);
    if (valid < kStep) {
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (step_key(r, half) >= valid) sc[b][r] = -INFINITY;
    }
  };

  Block<D> blk[QB];
  init_blocks(blk);
  const float c = p.scale_log2;
  auto soft = [&](f32x16 (&sc)[QB], u32x4 (&pk)[QB][2], bool last) {
    if (last) mask_last(sc);
    softmax_step(blk, sc, c, pk);
  };
  run_steps<D, QB, W, NS, false>(n, lds, la, q, blk, true, issue, [] {}, soft);

  // outputs
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const float l_tot = sum_halves(blk[b].l);
    if (q_row[b] >= p.lq) continue;
    if (e.slot < 0) {
      uint16_t* op = (uint16_t*)p.out + (int64_t)q_row[b] * p.tok_stride + (int64_t)e.head * D;
      store_out_bf16<D>(blk[b], 1.0f / l_tot, op, half);
    } else {
      const int64_t prow = (int64_t)(e.slot + split) * p.lq + q_row[b];
      store_partial<D>(blk[b], l_tot, p.part_o + prow * D, p.part_ml + prow * 2, half);
    }
  }
}

template <int D, int QB>
__global__ __launch_bounds__(64 * (kDenseQ / (32 * QB)), kDenseQ / (32 * QB) >= 8 ? 1 : 8 / (kDenseQ / (32 * QB)))
void dense_attn_bf16(const DenseParams p) {
  constexpr int W = kDenseQ / (32 * QB);
  __shared__ __attribute__((aligned(1024))) char ring[4 * Ring<D, QB, W>::kStageBytes];
  const int item = queue_item(p);
  if (item < 0) return;
  dense_item<D, QB>(p, item, (lds_char*)ring);
}

// Dense items, then the Spatial tiles (d = 128). Both use four waves and a four-stage
// ring of the same layout; the LDS adds the Spatial tables when TABLE.
template <bool TABLE>
__global__ __launch_bounds__(256, 2) void dense_spatial_bf16(const DenseParams p) {
  static_assert(4 * Ring<128, 1, 4>::kStageBytes <= spatial_lds_bytes<128, TABLE>(), "shared ring");
  __shared__ __attribute__((aligned(1024))) char ring[spatial_lds_bytes<128, TABLE>()];
  const int item = queue_item(p);
  if (item < 0) return;
  if (item < p.sp.n_dense_items) {
    dense_item<128, 1>(p, item, (lds_char*)ring);
    return;
  }
  // item s of the Spatial items: tile s % n_tiles, frame part s / n_tiles % n_parts of
  // the head s / (n_tiles * n_parts)
  const int n_tiles = p.sp.g.tiles_r * p.sp.g.tiles_c;
  const int s = item - p.sp.n_dense_items;
  const DenseEntry d = p.e[p.sp.sp_entry[s / (n_tiles * p.sp.g.n_parts)]];
  SpatialEntry e;
  e.hist_off = d.hist_off;
  e.head = d.head;
  e.cur_slot = -1;
  e.out_slot = d.slot + 1;
  e.pad = 0;
  spatial_tile<128, TABLE>(p.sp.g, e, s % n_tiles, s / n_tiles % p.sp.g.n_parts, (lds_char*)ring);
}

}  // namespace

hipError_t launch_dense_f32(const DenseParams& p, int head_dim, hipStream_t s);

hipError_t launch_dense(const DenseParams& p, int head_dim, int bf16, hipStream_t s) {
  if (p.n_items == 0) return hipSuccess;
  if (!bf16) return launch_dense_f32(p, head_dim, s);
  // four waves of 32 queries for both head sizes
  const dim3 grid(kXcds * p.xcd_len);
  if (p.sp.n_sp > 0) {   // with the Spatial tiles (d = 128 only)
    if (head_dim != 128) return hipErrorInvalidValue;
    if (spatial_table(p.sp.g))
      hipLaunchKernelGGL((dense_spatial_bf16<true>), grid, dim3(256), 0, s, p);
    else
      hipLaunchKernelGGL((dense_spatial_bf16<false>), grid, dim3(256), 0, s, p);
  } else if (head_dim == 64)
    hipLaunchKernelGGL((dense_attn_bf16<64, 1>), grid, dim3(64 * (kDenseQ / 32)), 0, s, p);
  else
    hipLaunchKernelGGL((dense_attn_bf16<128, 1>), grid, dim3(64 * (kDenseQ / 32)), 0, s, p);
  return hipGetLastError();
}

}  // namespace hc
