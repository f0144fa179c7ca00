// Spatial path, history part (HeadCast Sec. 3.2 "Spatial Pattern", Sec. 4.4 Spatial
// Path, with the sliding g x g neighbourhood of the Sec. 4.2 Spatial proxy): every
// query (f, r, c) of the current block attends, in each history frame, to the g x g
// window whose origin is clamp(r - g/2, 0, fh - g) x clamp(c - g/2, 0, fw - g).
//
// A workgroup (4 waves) takes a tile of 4 x 8 positions of one Spatial head, one wave
// per chunk frame (the chunk frames at one position share the key set exactly). For each
// history frame it walks the union of the 32 windows in 64-key LDS tiles: K/V rows
// are gathered as whole 256-B rows (coalesced), scores come from the same MFMA tile
// step as the dense path, and keys outside a query's own window are masked.
// In final mode the result is merged with the dense current-block partial by its
// log-sum-exp and written as bf16; in partial mode (classifier) it is stored as fp32.
#include "hc_tile.h"

namespace hc {

namespace {

template <int D>
__global__ __launch_bounds__(256, 2) void spatial_attn_bf16(const SpatialParams p) {
  using L = AttnLds<D>;
  constexpr int KS = D / 16;
  __shared__ __attribute__((aligned(16))) uint16_t lds[2 * L::bufElems];

  const SpatialEntry e = p.e[blockIdx.y];
  const int tr = blockIdx.x / p.tiles_c, tc = blockIdx.x % p.tiles_c;
  const int fh = p.frame_h, fw = p.frame_w, S = fh * fw;
  const bool cells = p.cells != 0;
  // window of a position: sliding g x g (never cut) or its own cell
  auto org_r = [&](int r) { return cells ? cell_origin(r, p.grid_h) : win_origin(r, p.grid_h, fh); };
  auto org_c = [&](int c) { return cells ? cell_origin(c, p.grid_w) : win_origin(c, p.grid_w, fw); };
  auto ext_r = [&](int r) { return cells ? cell_extent(r, p.grid_h, fh) : min(p.grid_h, fh); };
  auto ext_c = [&](int c) { return cells ? cell_extent(c, p.grid_w, fw) : min(p.grid_w, fw); };
  const int R0 = tr * kSpTileR, C0 = tc * kSpTileC;
  const int R1 = min(R0 + kSpTileR, fh) - 1, C1 = min(C0 + kSpTileC, fw) - 1;
  // union of the windows of the tile's positions (origins and ends grow with the position)
  const int ur0 = org_r(R0), ur1 = org_r(R1) + ext_r(R1);
  const int uc0 = org_c(C0), uc1 = org_c(C1) + ext_c(C1);
  const int UW = uc1 - uc0;
  const int nU = (ur1 - ur0) * UW;
  const int nchunk = (nU + kKeyTile - 1) / kKeyTile;
  // frames walked: the history (and, for cells, the current block after it)
  const int n_frames = p.n_hist_frames + (cells ? p.chunk_frames : 0);
  const int n_tiles = n_frames * nchunk;

  const int tid = threadIdx.x;
  constexpr int nwave = 4;   // one wave per chunk frame; spare waves only load
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int half = lane >> 5;
  const int pr = R0 + l32 / kSpTileC, pc = C0 + l32 % kSpTileC;
  const bool pos_ok = pr < fh && pc < fw;
  const int r0q = org_r(min(pr, fh - 1)), ehq = ext_r(min(pr, fh - 1));
  const int c0q = org_c(min(pc, fw - 1)), ewq = ext_c(min(pc, fw - 1));

  const uint16_t* kh = (const uint16_t*)p.k_hist + e.hist_off;
  const uint16_t* vh = (const uint16_t*)p.v_hist + e.hist_off;
  const uint16_t* kcb = cells ? (const uint16_t*)p.k_cur + (int64_t)e.head * D : kh;
  const uint16_t* vcb = cells ? (const uint16_t*)p.v_cur + (int64_t)e.head * D : vh;
  const int64_t hs = p.hist_stride, ts = p.tok_stride;
  const int nh = p.n_hist_frames;

  TileRegs<D> regs;
  constexpr int cpr = TileRegs<D>::cpr;
  // Tiles are walked chunk-outer, frame-inner: tile t = chunk t / n_frames of the window
  // union, in frame t % n_frames. The union position of every key a thread stages, and
  // every lane's mask bits, depend only on the chunk, so they are computed once per chunk.
  int tok_k[TileRegs<D>::kChunks], tok_v[4];   // within-frame token offsets of the staged rows
  int cached_u = -1;
  auto union_tok = [&](int u, int j) {
    const int ui = min(u * kKeyTile + j, nU - 1);
    const int q = ui / UW;
    return (ur0 + q) * fw + uc0 + (ui - q * UW);
  };
  auto load = [&](int t) {
    const int u = t / n_frames, f = t - u * n_frames;
    if (u != cached_u) {
      cached_u = u;
#pragma unroll
      for (int i = 0; i < TileRegs<D>::kChunks; ++i) tok_k[i] = union_tok(u, (tid + 256 * i) / cpr);
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) tok_v[jj] = union_tok(u, 4 * (tid % 16) + jj);
    }
    const bool cur = f >= nh;
    const int64_t stride = cur ? ts : hs;
    const int64_t fbase = (int64_t)(cur ? f - nh : f) * S * stride;
    const uint16_t* kb = (cur ? kcb : kh) + fbase;
    const uint16_t* vb = (cur ? vcb : vh) + fbase;
#pragma unroll
    for (int i = 0; i < TileRegs<D>::kChunks; ++i)
      regs.k[i] = *(const u32x4*)(kb + (int64_t)tok_k[i] * stride + ((tid + 256 * i) % cpr) * 8);
#pragma unroll
    for (int i = 0; i < TileRegs<D>::vPer; ++i) {
      const int uu = tid + 256 * i;
      if (uu < TileRegs<D>::vUnits) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          regs.v[i][jj] = *(const u32x4*)(vb + (int64_t)tok_v[jj] * stride + (uu / 16) * 8);
      }
    }
  };
  // Bit kb*16 + r: key score_key(kb, r, half) of chunk u lies in this lane's window.
  auto mask_bits = [&](int u) {
    uint32_t bits = 0;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int ui0 = u * kKeyTile + score_key(kb, 4 * a, half);
        int ur = ui0 / UW, uc = ui0 - ur * UW;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const bool in = ui0 + b < nU && (unsigned)(ur0 + ur - r0q) < (unsigned)ehq &&
                          (unsigned)(uc0 + uc - c0q) < (unsigned)ewq;
          bits |= (uint32_t)in << (kb * 16 + 4 * a + b);
          if (++uc == UW) {
            uc = 0;
            ++ur;
          }
        }
      }
    return bits;
  };

  for (int cf0 = 0; cf0 < p.chunk_frames; cf0 += nwave) {
    const int cf = cf0 + wave;
    const bool q_ok = pos_ok && cf < p.chunk_frames;
    const int q_row = min(cf, p.chunk_frames - 1) * S + min(pr, fh - 1) * fw + min(pc, fw - 1);
    const uint16_t* qp = (const uint16_t*)p.q + (int64_t)q_row * p.tok_stride + (int64_t)e.head * D;
    u32x4 qreg[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) qreg[ks] = *(const u32x4*)(qp + ks * 16 + half * 8);

    AttnState<D> st;
    st.init();
    cached_u = -1;
    if (n_tiles > 0) {
      load(0);
      store_tile<D>(regs, lds, tid);
    }
    __syncthreads();
    uint32_t bits = 0;
    for (int t = 0; t < n_tiles; ++t) {
      const bool more = t + 1 < n_tiles;
      if (more) load(t + 1);
      if (t % n_frames == 0) bits = mask_bits(t / n_frames);
      attend_tile<D, true>(st, qreg, lds + (t & 1) * L::bufElems, p.scale_log2, l32, half,
                           [&](int kb, int r) { return ((bits >> (kb * 16 + r)) & 1u) != 0; });
      if (more) store_tile<D>(regs, lds + ((t + 1) & 1) * L::bufElems, tid);
      __syncthreads();
    }

    const float l_tot = sum_halves(st.l_run);
    if (q_ok) {
      if (cells) {   // the whole key set was walked here: normalise and write
        uint16_t* op = (uint16_t*)p.out + (int64_t)q_row * p.tok_stride + (int64_t)e.head * D;
        store_out_bf16<D>(st, 1.0f / l_tot, op, half);
      } else if (e.out_slot >= 0) {
        const int64_t prow = (int64_t)e.out_slot * p.lq + q_row;
        store_partial<D>(st, l_tot, p.part_o + prow * D, p.part_ml + prow * 2, half);
      } else {
        // merge with the dense current-block partial by log-sum-exp
        const int64_t crow = (int64_t)e.cur_slot * p.lq + q_row;
        const float m_c = p.part_ml[crow * 2], l_c = p.part_ml[crow * 2 + 1];
        const float M = fmaxf(st.m_run, m_c);
        const float wa = st.m_run == -INFINITY ? 0.f : fast_exp2(st.m_run - M);
        const float wc = fast_exp2(m_c - M);
        const float inv = 1.0f / (wa * l_tot + wc * l_c);
        const float* po = p.part_o + crow * D;
        uint16_t* op = (uint16_t*)p.out + (int64_t)q_row * p.tok_stride + (int64_t)e.head * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int a = 0; a < 4; ++a) {
            const int d = db * 32 + 8 * a + 4 * half;
            const f32x4 oc = *(const f32x4*)(po + d);
            u32x2 w;
            w[0] = pack_bf16((wa * st.o[db][4 * a] + wc * oc[0]) * inv,
                             (wa * st.o[db][4 * a + 1] + wc * oc[1]) * inv);
            w[1] = pack_bf16((wa * st.o[db][4 * a + 2] + wc * oc[2]) * inv,
                             (wa * st.o[db][4 * a + 3] + wc * oc[3]) * inv);
            *(u32x2*)(op + d) = w;
          }
      }
    }
  }
}

__global__ void gather_origins_kernel(int fh, int fw, int gh, int gw, int cells, int32_t* out) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= fh * fw) return;
  out[2 * t] = cells ? cell_origin(t / fw, gh) : win_origin(t / fw, gh, fh);
  out[2 * t + 1] = cells ? cell_origin(t % fw, gw) : win_origin(t % fw, gw, fw);
}

}  // namespace

hipError_t launch_spatial_f32(const SpatialParams& p, int head_dim, hipStream_t s);

hipError_t launch_spatial(const SpatialParams& p, int head_dim, int bf16, hipStream_t s) {
  if (p.n_entries == 0) return hipSuccess;
  if (!bf16) return launch_spatial_f32(p, head_dim, s);
  const dim3 grid(p.tiles_r * p.tiles_c, p.n_entries), block(256);
  if (head_dim == 128)
    hipLaunchKernelGGL(spatial_attn_bf16<128>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(spatial_attn_bf16<64>, grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_gather_origins(int frame_h, int frame_w, int grid_h, int grid_w, int cells, int32_t* out,
                                 hipStream_t s) {
  const int n = frame_h * frame_w;
  hipLaunchKernelGGL(gather_origins_kernel, dim3((n + 255) / 256), dim3(256), 0, s, frame_h, frame_w,
                     grid_h, grid_w, cells, out);
  return hipGetLastError();
}

}  // namespace hc
