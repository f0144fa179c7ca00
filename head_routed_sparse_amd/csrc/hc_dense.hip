// Dense varlen-per-head attention for gfx950: the Sink, Dummy and Global paths, the
// current-block part of the Spatial path, and the classifier's reference and block
// proxies (HeadCast Sec. 4.4 "Head-Specific Attention"; Sec. 4.2 Eq. 2).
//
// One workgroup = 4 waves = 128 queries of one head against one key range: a split of
// the head's [history rows ; current-block rows]. History rows come from the compact
// per-head buffer (stride D) or, for the classifier, from the monolithic cache
// (stride H*D); current-block rows are read in place from [C*S][H][D]. Items are
// ordered longest first and grouped per XCD so that the query tiles sharing a key
// range run on the same L2.
#include "hc_tile.h"

namespace hc {

namespace {

template <int D>
__global__ __launch_bounds__(256, 2) void dense_attn_bf16(const DenseParams p) {
  using L = AttnLds<D>;
  constexpr int KS = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * L::bufElems];

  const int item = xcd_logical(blockIdx.x, p.xcd_group);
  if (item >= p.n_items) return;
  int ei = 0;
  while (ei + 1 < p.n_entries && item >= p.e[ei + 1].item_begin) ++ei;
  const DenseEntry e = p.e[ei];
  const int local = item - e.item_begin;
  const int split = local / p.nqt;
  const int qt = local - split * p.nqt;

  const int k_begin = split * e.split_len;
  const int k_end = min(e.hist_len + e.cur_len, k_begin + e.split_len);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;

  const int q_row = qt * kDenseQ + wave * 32 + l32;
  const uint16_t* qp = (const uint16_t*)p.q + (int64_t)min(q_row, p.lq - 1) * p.tok_stride +
                       (int64_t)e.head * D;
  u32x4 qreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) qreg[ks] = *(const u32x4*)(qp + ks * 16 + half * 8);

  const uint16_t* kh = (const uint16_t*)p.k_hist + e.hist_off;
  const uint16_t* vh = (const uint16_t*)p.v_hist + e.hist_off;
  const uint16_t* kc = (const uint16_t*)p.k_cur + (int64_t)e.head * D;
  const uint16_t* vc = (const uint16_t*)p.v_cur + (int64_t)e.head * D;
  const int64_t hs = p.hist_stride, ts = p.tok_stride;
  const int hl = e.hist_len;

  AttnState<D> st;
  st.init();
  const int n_tiles = (k_end - k_begin + kKeyTile - 1) / kKeyTile;
  TileRegs<D> regs;
  auto load = [&](int k0) {
    if (k0 + kKeyTile <= min(hl, k_end)) {            // whole tile in the history segment
      load_tile_rows<D>(regs, kh + (int64_t)k0 * hs, vh + (int64_t)k0 * hs, hs, tid);
    } else if (k0 >= hl && k0 + kKeyTile <= k_end) {  // whole tile in the current block
      load_tile_rows<D>(regs, kc + (int64_t)(k0 - hl) * ts, vc + (int64_t)(k0 - hl) * ts, ts, tid);
    } else {                                           // straddles the segments or the end
      auto kp = [&](int j) {
        const int kk = min(k0 + j, k_end - 1);
        return kk < hl ? kh + (int64_t)kk * hs : kc + (int64_t)(kk - hl) * ts;
      };
      auto vp = [&](int j) {
        const int kk = min(k0 + j, k_end - 1);
        return kk < hl ? vh + (int64_t)kk * hs : vc + (int64_t)(kk - hl) * ts;
      };
      load_tile<D>(regs, kp, vp, tid);
    }
  };
  load(k_begin);
  store_tile<D>(regs, lds, tid);
  __syncthreads();

  // every tile but the last is full: one straight-line loop body
  for (int t = 0; t + 1 < n_tiles; ++t) {
    const int k0 = k_begin + t * kKeyTile;
    load(k0 + kKeyTile);
    attend_tile<D, false>(st, qreg, lds + (t & 1) * L::bufElems, p.scale_log2, l32, half,
                          [](int, int) { return true; });
    store_tile<D>(regs, lds + ((t + 1) & 1) * L::bufElems, tid);
    __syncthreads();
  }
  if (n_tiles > 0) {   // last tile, possibly ragged
    const int t = n_tiles - 1;
    const int valid = k_end - (k_begin + t * kKeyTile);
    attend_tile<D, true>(st, qreg, lds + (t & 1) * L::bufElems, p.scale_log2, l32, half,
                         [&](int kb, int r) { return score_key(kb, r, half) < valid; });
  }

  const float l_tot = sum_halves(st.l_run);
  if (q_row >= p.lq) return;
  if (e.slot < 0) {
    uint16_t* op = (uint16_t*)p.out + (int64_t)q_row * p.tok_stride + (int64_t)e.head * D;
    store_out_bf16<D>(st, 1.0f / l_tot, op, half);
  } else {
    const int64_t prow = (int64_t)(e.slot + split) * p.lq + q_row;
    store_partial<D>(st, l_tot, p.part_o + prow * D, p.part_ml + prow * 2, half);
  }
}

}  // namespace

int dense_items_grid(int n_items, int xcd_group) {
  const int span = 8 * xcd_group;
  return (n_items + span - 1) / span * span;
}

hipError_t launch_dense_f32(const DenseParams& p, int head_dim, hipStream_t s);

hipError_t launch_dense(const DenseParams& p, int head_dim, int bf16, hipStream_t s) {
  if (p.n_items == 0) return hipSuccess;
  if (!bf16) return launch_dense_f32(p, head_dim, s);
  const dim3 grid(dense_items_grid(p.n_items, p.xcd_group)), block(256);
  if (head_dim == 128)
    hipLaunchKernelGGL(dense_attn_bf16<128>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(dense_attn_bf16<64>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace hc
