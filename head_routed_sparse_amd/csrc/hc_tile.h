// The flash-attention tile step shared by the dense and Spatial kernels (bf16, gfx950).
//
// A workgroup of 256 threads stages a 64-key tile in LDS: K row-major, V transposed
// (V^T, keys permuted by vt_pos). Each wave owns 32 queries held as the B operand of
// S^T = K Q^T, so a lane carries one query's 32 scores of the tile (its wave half
// carries the other 32). The tile step updates an online softmax in fp32 and
// accumulates O^T = V^T P^T with P taken from the score registers.
#pragma once
#include "hc_internal.h"
#include "hc_mfma.h"

namespace hc {

constexpr float kRescaleSlack = 8.0f;   // log2 units the running max may lag the tile max

template <int D>
struct AttnLds {
  static constexpr int kStride = D + 8;         // bf16 per K row (16-B pad)
  static constexpr int vStride = kKeyTile + 8;  // bf16 per V^T row
  static constexpr int kElems = kKeyTile * kStride;
  static constexpr int vElems = D * vStride;
  static constexpr int bufElems = kElems + vElems;
};

template <int D>
struct TileRegs {
  static constexpr int cpr = D / 8;                        // 16-B chunks per row
  static constexpr int kChunks = kKeyTile * cpr / 256;     // K chunks per thread
  // (4 keys x 8 d) units; unit u = key group u % 16, d chunk u / 16, so that the 16 lanes
  // of one LDS write group hit 16 different bank pairs of the transposed tile
  static constexpr int vUnits = (kKeyTile / 4) * cpr;
  static constexpr int vPer = (vUnits + 255) / 256;
  u32x4 k[kChunks];
  u32x4 v[vPer][4];
};

// kptr(j), vptr(j): address of the K / V row of local key j (0..63); always valid.
template <int D, class KPtr, class VPtr>
__device__ __forceinline__ void load_tile(TileRegs<D>& t, KPtr kptr, VPtr vptr, int tid) {
  constexpr int cpr = TileRegs<D>::cpr;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kChunks; ++i) {
    const int idx = tid + 256 * i;
    t.k[i] = *(const u32x4*)(kptr(idx / cpr) + (idx % cpr) * 8);
  }
#pragma unroll
  for (int i = 0; i < TileRegs<D>::vPer; ++i) {
    const int u = tid + 256 * i;
    if (u < TileRegs<D>::vUnits) {
      const int g = u % 16, ch = u / 16;   // 16-lane groups: one d chunk, all key groups
#pragma unroll
      for (int j = 0; j < 4; ++j) t.v[i][j] = *(const u32x4*)(vptr(4 * g + j) + ch * 8);
    }
  }
}

// Fast path: the tile's 64 rows are consecutive rows base[0..63] with a fixed stride.
template <int D>
__device__ __forceinline__ void load_tile_rows(TileRegs<D>& t, const uint16_t* kbase, const uint16_t* vbase,
                                               int64_t stride, int tid) {
  constexpr int cpr = TileRegs<D>::cpr;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kChunks; ++i) {
    const int idx = tid + 256 * i;
    t.k[i] = *(const u32x4*)(kbase + (int64_t)(idx / cpr) * stride + (idx % cpr) * 8);
  }
#pragma unroll
  for (int i = 0; i < TileRegs<D>::vPer; ++i) {
    const int u = tid + 256 * i;
    if (u < TileRegs<D>::vUnits) {
      const int g = u % 16, ch = u / 16;   // 16-lane groups: one d chunk, all key groups
#pragma unroll
      for (int j = 0; j < 4; ++j) t.v[i][j] = *(const u32x4*)(vbase + (int64_t)(4 * g + j) * stride + ch * 8);
    }
  }
}

template <int D>
__device__ __forceinline__ void store_tile(const TileRegs<D>& t, uint16_t* buf, int tid) {
  using L = AttnLds<D>;
  constexpr int cpr = TileRegs<D>::cpr;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::kChunks; ++i) {
    const int idx = tid + 256 * i;
    *(u32x4*)(buf + (idx / cpr) * L::kStride + (idx % cpr) * 8) = t.k[i];
  }
  uint16_t* vt = buf + L::kElems;
#pragma unroll
  for (int i = 0; i < TileRegs<D>::vPer; ++i) {
    const int u = tid + 256 * i;
    if (u < TileRegs<D>::vUnits) {
      const int g = u % 16, ch = u / 16;   // 16-lane groups: one d chunk, all key groups
      const int pos = vt_pos(4 * g);
#pragma unroll
      for (int w = 0; w < 4; ++w) {   // dword w of each key row holds d = 2w, 2w+1
        u32x2 lo, hi;
        lo[0] = pair_lo(t.v[i][0][w], t.v[i][1][w]);
        lo[1] = pair_lo(t.v[i][2][w], t.v[i][3][w]);
        hi[0] = pair_hi(t.v[i][0][w], t.v[i][1][w]);
        hi[1] = pair_hi(t.v[i][2][w], t.v[i][3][w]);
        const int d = ch * 8 + 2 * w;
        *(u32x2*)(vt + d * L::vStride + pos) = lo;
        *(u32x2*)(vt + (d + 1) * L::vStride + pos) = hi;
      }
    }
  }
}

template <int D>
struct AttnState {
  static constexpr int DB = D / 32;
  f32x16 o[DB];
  float m_run;   // running max, log2 units with the softmax scale folded in
  float l_run;   // this lane's share of the running sum
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] = f32x16{};
    m_run = -INFINITY;
    l_run = 0.f;
  }
};

// Local key index (0..63) held in score register r of lane half `half`, block kb.
__device__ __forceinline__ int score_key(int kb, int r, int half) {
  return kb * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
}

// One tile: scores, optional mask (keep(kb, r) false -> dropped), online softmax, PV.
template <int D, bool kMasked, class Keep>
__device__ __forceinline__ void attend_tile(AttnState<D>& st, const u32x4* qreg, const uint16_t* buf,
                                            float c, int l32, int half, Keep keep) {
  using L = AttnLds<D>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = f32x16{};
    const uint16_t* krow = buf + (kb * 32 + l32) * L::kStride + half * 8;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) s[kb] = mfma32(*(const u32x4*)(krow + ks * 16), qreg[ks], s[kb]);
  }
  if (kMasked) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (!keep(kb, r)) s[kb][r] = -INFINITY;
  }
  float mx = s[0][0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[0][r]);
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[1][r]);
  mx = max_halves(mx);
  const float mt = mx * c;
  if (__builtin_amdgcn_ballot_w64(mt > st.m_run + kRescaleSlack)) {
    const float m_new = fmaxf(st.m_run, mt);
    const float f = (m_new == -INFINITY) ? 1.f : fast_exp2(st.m_run - m_new);
    st.l_run *= f;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.o[db][r] *= f;
    st.m_run = m_new;
  }
  const float m_sub = (st.m_run == -INFINITY) ? 0.f : st.m_run;
  u32x4 pb[2][2];
  float lsum = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0 = fast_exp2(__builtin_fmaf(s[kb][r], c, -m_sub));
      const float p1 = fast_exp2(__builtin_fmaf(s[kb][r + 1], c, -m_sub));
      lsum += p0 + p1;
      pb[kb][r >> 3][(r & 7) >> 1] = pack_bf16(p0, p1);
    }
  st.l_run += lsum;
  const uint16_t* vt = buf + L::kElems;
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const uint16_t* vrow = vt + (db * 32 + l32) * L::vStride + half * 8;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        st.o[db] = mfma32(*(const u32x4*)(vrow + kb * 32 + s2 * 16), pb[kb][s2], st.o[db]);
  }
}

// Write the normalised output row (bf16) of this lane's query; factor multiplies O.
template <int D>
__device__ __forceinline__ void store_out_bf16(const AttnState<D>& st, float factor, uint16_t* row,
                                               int half) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      u32x2 w;
      w[0] = pack_bf16(st.o[db][4 * a] * factor, st.o[db][4 * a + 1] * factor);
      w[1] = pack_bf16(st.o[db][4 * a + 2] * factor, st.o[db][4 * a + 3] * factor);
      *(u32x2*)(row + db * 32 + 8 * a + 4 * half) = w;
    }
}

// Write the unnormalised partial (fp32 O, running max, total sum) of this lane's query.
template <int D>
__device__ __forceinline__ void store_partial(const AttnState<D>& st, float l_tot, float* po,
                                              float* pml, int half) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      f32x4 w = {st.o[db][4 * a], st.o[db][4 * a + 1], st.o[db][4 * a + 2], st.o[db][4 * a + 3]};
      *(f32x4*)(po + db * 32 + 8 * a + 4 * half) = w;
    }
  if (half == 0) {
    pml[0] = st.m_run;
    pml[1] = l_tot;
  }
}

}  // namespace hc
