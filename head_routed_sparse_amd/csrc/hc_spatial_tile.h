// Spatial path, history part: the work of one workgroup (HeadCast Sec. 3.2 "Spatial
// Pattern", Sec. 4.4 Spatial Path, with the sliding g x g neighbourhood of the Sec. 4.2
// Spatial proxy): every query (f, r, c) of the current block attends, in each history
// frame, to the g x g window whose origin is clamp(r - g/2, 0, fh - g) x
// clamp(c - g/2, 0, fw - g).
//
// A workgroup (4 waves) takes a tile of up to 32 positions (tile_r x tile_c, chosen by
// the host) of one Spatial head, one wave per chunk frame (the chunk frames at one
// position share the key set exactly; with three chunk frames the fourth wave only
// loads). It walks the union of the tile's windows in 32-key steps, chunk-outer and
// frame-inner, on the dense kernel's pipeline (hc_pipe.h): every step's rows are
// gathered whole (256 B) by 16-byte direct loads into the LDS ring. The token of every
// row a step loads, and every lane's window bits, depend only on the chunk: for unions
// of up to kTblChunks chunks the workgroup writes them to two small LDS tables once, and
// each lane reads its entries when a chunk starts (larger unions work them out there).
// The window mask is folded into the exponent's addend (-inf outside the window), which
// changes only with the chunk and the reference max. With frame parts, each of n_parts
// workgroups walks its share of the frames and stores an fp32 partial that the merge
// kernel joins. In final mode the result is merged with the dense current-block partial
// by its log-sum-exp and written as bf16; in partial mode (classifier, frame parts, tiles
// run in the dense launch) it is stored as fp32; with cells the whole key set is walked
// here.
#pragma once
#include "hc_pipe.h"

namespace hc {

// LDS bytes of one workgroup: the four-stage ring and, with TABLE, the two tables.
template <int D, bool TABLE>
constexpr int spatial_lds_bytes() {
  return 4 * Ring<D, 1, 4>::kStageBytes + (TABLE ? kTblChunks * kStep * 4 + kTblChunks * 64 * 2 : 0);
}

// One workgroup's work: position tile `tile` of Spatial head entry e, over frame part
// `part` of p.n_parts, with the LDS at `lds` (spatial_lds_bytes<D, TABLE>() bytes).
template <int D, bool TABLE>
__device__ __forceinline__ void spatial_tile(const SpatialGeom& p, const SpatialEntry e, int tile, int part,
                                             lds_char* lds) {
  constexpr int W = 4;
  using R = Ring<D, 1, W>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  constexpr int NS = 4;   // ring stages
  constexpr int kTokBytes = TABLE ? kTblChunks * kStep * 4 : 0;
  lds_char* const tok_tbl = lds + NS * R::kStageBytes;   // int32 [chunk][row of the step]
  lds_char* const bit_tbl = tok_tbl + kTokBytes;         // uint16 [chunk][lane]
  const int tr = tile / p.tiles_c, tc = tile % p.tiles_c;
  const int fh = p.frame_h, fw = p.frame_w, S = fh * fw;
  const bool cells = p.cells != 0;
  // window of a position: sliding g x g (never cut) or its own cell
  auto org_r = [&](int r) { return cells ? cell_origin(r, p.grid_h) : win_origin(r, p.grid_h, fh); };
  auto org_c = [&](int c) { return cells ? cell_origin(c, p.grid_w) : win_origin(c, p.grid_w, fw); };
  auto ext_r = [&](int r) { return cells ? cell_extent(r, p.grid_h, fh) : min(p.grid_h, fh); };
  auto ext_c = [&](int c) { return cells ? cell_extent(c, p.grid_w, fw) : min(p.grid_w, fw); };
  const int R0 = tr * p.tile_r, C0 = tc * p.tile_c;
  const int R1 = min(R0 + p.tile_r, fh) - 1, C1 = min(C0 + p.tile_c, fw) - 1;
  // union of the windows of the tile's positions (origins and ends grow with the position)
  const int ur0 = org_r(R0), ur1 = org_r(R1) + ext_r(R1);
  const int uc0 = org_c(C0), uc1 = org_c(C1) + ext_c(C1);
  const int UW = uc1 - uc0;
  const int nU = (ur1 - ur0) * UW;
  const int nchunk = (nU + kStep - 1) / kStep;
  // frames walked: this part's share of the history (and, for cells, of the current
  // block after it)
  const int nh = p.n_hist_frames;
  const int n_all = nh + (cells ? p.chunk_frames : 0);
  const int f0 = part * n_all / p.n_parts, f1 = (part + 1) * n_all / p.n_parts;
  const int n_frames = f1 - f0;
  const int n = nchunk * n_frames;   // steps

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int pr = R0 + l32 / p.tile_c, pc = C0 + l32 % p.tile_c;
  const bool pos_ok = l32 < p.tile_r * p.tile_c && pr < fh && pc < fw;

  const char* kh = (const char*)p.k_hist + e.hist_off * 2;
  const char* vh = (const char*)p.v_hist + e.hist_off * 2;
  const char* kcb = cells ? (const char*)p.k_cur + (int64_t)e.head * D * 2 : kh;
  const char* vcb = cells ? (const char*)p.v_cur + (int64_t)e.head * D * 2 : vh;
  const int64_t hs = p.hist_stride * 2, ts = p.tok_stride * 2;   // bytes

  LaneAddr<D, 1, W> la;
  la.init(wave, lane);
  // token (row * fw + col within a frame) of union index i
  auto union_tok = [&](int i) {
    i = min(i, nU - 1);
    const int q = i / UW;
    return (ur0 + q) * fw + uc0 + (i - q * UW);
  };
  // window bits of lane ln's 16 keys in union chunk cu: bit 4 a + b for key 8 a + 4 (ln / 32) + b
  auto chunk_bits = [&](int cu, int ln) {
    const int q32 = ln & 31, hf = ln >> 5;
    const int qr = R0 + q32 / p.tile_c, qc = C0 + q32 % p.tile_c;
    const int r0l = org_r(min(qr, fh - 1)), ehl = ext_r(min(qr, fh - 1));
    const int c0l = org_c(min(qc, fw - 1)), ewl = ext_c(min(qc, fw - 1));
    uint32_t b16 = 0;
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int i0 = cu * kStep + 8 * a + 4 * hf;
      int ur = i0 / UW, uc = i0 - ur * UW;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const bool in = i0 + b < nU && (unsigned)(ur0 + ur - r0l) < (unsigned)ehl &&
                        (unsigned)(uc0 + uc - c0l) < (unsigned)ewl;
        b16 |= (uint32_t)in << (4 * a + b);
        if (++uc == UW) {
          uc = 0;
          ++ur;
        }
      }
    }
    return b16;
  };
  // the per-chunk data: the token of each row a step loads, and each lane's window bits
  // (written once per workgroup; larger unions work them out when a chunk starts)
  if (TABLE) {
    for (int x = tid; x < nchunk * kStep; x += 256)
      *(__attribute__((address_space(3))) int*)(tok_tbl + 4 * x) = union_tok(x);
    for (int x = tid; x < nchunk * 64; x += 256)
      *(__attribute__((address_space(3))) uint16_t*)(bit_tbl + 2 * x) = (uint16_t)chunk_bits(x / 64, x % 64);
    __syncthreads();
  }

  for (int cf0 = 0; cf0 < p.chunk_frames; cf0 += W) {
    const int cf = cf0 + wave;
    const bool active = cf < p.chunk_frames;   // wave-uniform
    const bool q_ok = pos_ok && active;
    const int q_row = min(cf, p.chunk_frames - 1) * S + min(pr, fh - 1) * fw + min(pc, fw - 1);
    const uint16_t* qp = (const uint16_t*)p.q + (int64_t)q_row * p.tok_stride + (int64_t)e.head * D;
    u32x4 q[1][KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) q[0][ks] = *(const u32x4*)(qp + ks * 16 + half * 8);
    // wait for the query loads here: the compiler does not count the ring's direct
    // loads, and with these loads still pending it would wait at every step's score
    // MFMAs for a vector-memory count that the direct loads then also have to reach,
    // draining the ring's prefetch each step
    wait_vmcnt<0>();

    // loads: step t = chunk t / n_frames of the union in frame f0 + t % n_frames, issued
    // in order. With the tables, the byte offsets of this lane's rows within a history
    // frame are worked out once per chunk and the frame base advances one frame per
    // step; larger unions (no tables) work each step's offsets out from the tokens,
    // which keeps their register count.
    int iu = 0, ifr = 0;
    auto row_tok = [&](int i) {   // token of this lane's row i of the current chunk
      const int row = iu * kStep + la.ld_row[i];
      return TABLE ? *(const __attribute__((address_space(3))) int*)(tok_tbl + 4 * row) : union_tok(row);
    };
    uint32_t off_h[R::kLoads];                 // (tables) row byte offsets within a history frame
    int tok[R::kLoads];                        // (no tables) row tokens of the current chunk
    const int64_t frame_h = (int64_t)S * hs;   // bytes per history frame
    int64_t fb = 0;                            // (tables) byte offset of history frame f0 + ifr
    auto issue = [&](int, int stage) {
      const int fr = f0 + ifr;
      if constexpr (TABLE) {
        if (ifr == 0) {   // a new chunk: the rows of this lane, from the part's first frame
#pragma unroll
          for (int i = 0; i < R::kLoads; ++i) off_h[i] = (uint32_t)(row_tok(i) * hs) + la.ld_chunk[i];
          fb = (int64_t)f0 * frame_h;
        }
        if (!cells || fr < nh) {   // a history frame (sliding windows walk only these)
#pragma unroll
          for (int i = 0; i < R::kLoads; ++i) {
            dma16(kh + fb, off_h[i], la.dst(lds, stage, wave, i, 0));
            dma16(vh + fb, off_h[i], la.dst(lds, stage, wave, i, 1));
          }
          fb += frame_h;
        } else {   // a current-block frame (cells): token stride
          const int64_t cb = (int64_t)(fr - nh) * S * ts;
#pragma unroll
          for (int i = 0; i < R::kLoads; ++i) {
            const uint32_t off = (uint32_t)(row_tok(i) * ts) + la.ld_chunk[i];
            dma16(kcb + cb, off, la.dst(lds, stage, wave, i, 0));
            dma16(vcb + cb, off, la.dst(lds, stage, wave, i, 1));
          }
        }
      } else {
        if (ifr == 0)
#pragma unroll
          for (int i = 0; i < R::kLoads; ++i) tok[i] = row_tok(i);
        const bool cur = fr >= nh;
        const int64_t stride = cur ? ts : hs;
        const int64_t fbase = (int64_t)(cur ? fr - nh : fr) * S * stride;
        const char* kb = (cur ? kcb : kh) + fbase;
        const char* vb = (cur ? vcb : vh) + fbase;
#pragma unroll
        for (int i = 0; i < R::kLoads; ++i) {
          const uint32_t off = (uint32_t)(tok[i] * stride) + la.ld_chunk[i];
          dma16(kb, off, la.dst(lds, stage, wave, i, 0));
          dma16(vb, off, la.dst(lds, stage, wave, i, 1));
        }
      }
      if (++ifr == n_frames) {
        ifr = 0;
        ++iu;
      }
    };
    Block<D> blk[1];
    init_blocks(blk);
    const float c = p.scale_log2;
    // window of this lane's query over the keys of the current union chunk: bit r =
    // key step_key(r, half) lies in the window (and in the union). The exponent addends
    // are -m inside, -inf outside, so masking costs nothing per step; they change with
    // the chunk and with the reference max.
    int mu = 0, mf = 0;
    uint32_t bits = 0;
    float add[16];
    auto refresh = [&]() {
#pragma unroll
      for (int r = 0; r < 16; ++r) add[r] = (bits >> r) & 1u ? -blk[0].m : -INFINITY;
    };
    auto prep = [&]() {
      if (mf == 0) {   // a new chunk
        bits = TABLE ? *(const __attribute__((address_space(3))) uint16_t*)(bit_tbl + 2 * (mu * 64 + lane))
                     : chunk_bits(mu, lane);
        refresh();
      }
      if (++mf == n_frames) {
        mf = 0;
        ++mu;
      }
    };
    auto soft = [&](f32x16 (&sc)[1], u32x4 (&pk)[1][2], bool) {
      float ls = exponentiate(sc[0], [&](int r) { return add[r]; }, c, pk[0]);
      if (__builtin_amdgcn_ballot_w64(ls > kSumLimit)) {   // move the reference max
        float mx = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if ((bits >> r) & 1u) mx = __builtin_fmaxf(mx, sc[0][r]);
        move_max(blk[0], __builtin_fmaxf(blk[0].m, max_halves(mx) * c));
        refresh();
        ls = exponentiate(sc[0], [&](int r) { return add[r]; }, c, pk[0]);
      }
      blk[0].l += ls;
    };

    if (n > 0) run_steps<D, 1, W, NS, true>(n, lds, la, q, blk, active, issue, prep, soft);
    __syncthreads();   // the ring is reused by the next group of chunk frames

    const float l_tot = sum_halves(blk[0].l);
    const float m_s = blk[0].m;
    if (q_ok) {
      if (e.out_slot >= 0) {
        const int64_t prow = (int64_t)(e.out_slot + part) * p.lq + q_row;
        store_partial<D>(blk[0], l_tot, p.part_o + prow * D, p.part_ml + prow * 2, half);
      } else if (cells) {   // the whole key set was walked here: normalise and write
        uint16_t* op = (uint16_t*)p.out + (int64_t)q_row * p.tok_stride + (int64_t)e.head * D;
        store_out_bf16<D>(blk[0], 1.0f / l_tot, op, half);
      } else {
        // merge with the dense current-block partial by log-sum-exp (an empty history
        // leaves m_s at the finite stand-in and weight 0)
        const int64_t crow = (int64_t)e.cur_slot * p.lq + q_row;
        const float m_c = p.part_ml[crow * 2], l_c = p.part_ml[crow * 2 + 1];
        const float M = fmaxf(m_s, m_c);
        const float wa = fast_exp2(m_s - M);
        const float wc = fast_exp2(m_c - M);
        const float inv = 1.0f / (wa * l_tot + wc * l_c);
        const float* po = p.part_o + crow * D;
        uint16_t* op = (uint16_t*)p.out + (int64_t)q_row * p.tok_stride + (int64_t)e.head * D;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int d = db * 32 + 8 * a + 4 * half;
            const f32x4 oc = *(const f32x4*)(po + d);
            u32x2 w;
            w[0] = pack_bf16((wa * blk[0].o[db][4 * a] + wc * oc[0]) * inv,
                             (wa * blk[0].o[db][4 * a + 1] + wc * oc[1]) * inv);
            w[1] = pack_bf16((wa * blk[0].o[db][4 * a + 2] + wc * oc[2]) * inv,
                             (wa * blk[0].o[db][4 * a + 3] + wc * oc[3]) * inv);
            *(u32x2*)(op + d) = w;
          }
      }
    }
  }
}

}  // namespace hc
