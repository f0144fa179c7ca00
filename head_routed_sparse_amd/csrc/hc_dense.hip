// Dense varlen-per-head attention for gfx950: the Sink, Dummy and Global paths, the
// current-block part of the Spatial path, and the classifier's reference and block
// proxies (HeadCast Sec. 4.4 "Head-Specific Attention"; Sec. 4.2 Eq. 2).
//
// One workgroup = 128 queries of one head against one key range: a split of the
// head's [history rows ; current-block rows]. History rows come from the compact
// per-head buffer (stride D) or, for the classifier, from the monolithic cache
// (stride H*D); current-block rows are read in place from [C*S][H][D]. Items are
// ordered longest first and grouped per XCD so that the query tiles sharing a key
// range run on the same L2.
//
// For D=128 the workgroup has four waves of 32 queries (one per SIMD, all state in
// VGPRs) and two workgroups share a CU, each with its own LDS ring and barrier, so
// that one's softmax overlaps the other's MFMAs; for D=64, two waves of two 32-query
// blocks, where each K or V fragment read from LDS feeds one MFMA per block. Keys advance in steps of 32. The
// K and V rows of a step travel from global memory straight into a ring of LDS
// stages (16-byte direct loads, no staging registers), row-major, with the 16-byte
// chunks of row r permuted (chunk c stored at c ^ swz(r)) so that the K fragment
// reads and the transposed V reads (ds_read_b64_tr_b16) hit distinct banks. Per step,
// the scores of step j+1 run on the matrix cores while the VALU exponentiates step j,
// and the PV product of step j runs while the VALU reduces the row maxima of step j+1.
#include "hc_tile.h"

namespace hc {

namespace {

constexpr int kStep = 32;     // keys per pipeline step
constexpr int kStages = 4;    // LDS ring depth (even: the score buffers alternate with it)
static_assert(kStages % 2 == 0 && kStages >= 3 + 1, "ring depth");

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

template <int D, int QB>
struct Ring {
  static constexpr int kWaves = kDenseQ / (32 * QB);       // waves per workgroup
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kCpr = D / 8;                       // 16-byte chunks per row
  static constexpr int kTileBytes = kStep * kRowBytes;     // the K (or V) rows of a step
  static constexpr int kStageBytes = 2 * kTileBytes;
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;    // rows one wave-wide 16-B load fills
  static constexpr int kLoads = kStep / kRowsPerLoad / kWaves;   // per wave and tensor
  static constexpr int kBytes = kStages * kStageBytes;
  static_assert(kLoads >= 1, "tile too small for the wave count");
  static_assert(kWaves * 32 * QB == kDenseQ, "queries per workgroup");
};

// Chunk permutation of row r (16-byte chunk c stored at c ^ chunk_swz(r)). It is a
// bijection over any 16 consecutive rows (D=128; 8 rows for D=64), so the 16 lanes of
// a K fragment read (16 rows, one chunk) hit 16 different bank groups. For D=128 the
// 32-byte pair index (chunk >> 1) it applies to rows 4i..4i+3 is {k, k^2, k^4, k^6}:
// the transposed V reads of one 32-lane half (4 rows, pairs 2db and 2db+1) then touch
// 8 distinct 32-byte bank groups.
template <int D>
__device__ __forceinline__ int chunk_swz(int r) {
  if (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  constexpr int h = D / 16;
  return ((r & (h - 1)) << 1) | ((r / h) & 1);
}

// Wait until at most N vector memory loads of this wave are in flight (s_waitcnt
// immediate: vmcnt low 4 bits at [3:0], high 2 at [15:14]; expcnt and lgkmcnt at
// their maxima, i.e. not waited on).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// One wave-wide 16-byte direct load from global memory into LDS: lane i copies the 16
// bytes at base + voff (its own offset) to LDS address lds_dst + 16 i. Written out
// rather than left to the compiler, which cannot tell the ring stages apart and would
// wait for every direct load in flight before any LDS read; the loads are waited for
// explicitly (s_waitcnt vmcnt) before the barrier that publishes a stage.
// M0 is written here and nowhere else in this kernel (the compiler reserves it and
// would warn about the clobber).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const void* base, uint32_t voff, uint32_t lds_dst) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(lds_dst), "v"(voff), "s"(base) : "m0");
}
#pragma clang diagnostic pop

// Online softmax state of one 32-query block (per lane: its query; the lane halves
// hold different keys of the same queries).
template <int D>
struct Block {
  f32x16 o[D / 32];
  float m;   // reference max, log2 units with the scale folded in
  float l;   // this lane's share of the running sum
};

// Until the first step has set it, m holds this finite stand-in for minus infinity:
// every finite score then exponentiates to +inf and forces the first rescale, while
// masked scores (-inf) still give exactly 0 (no inf - inf).
constexpr float kNoMax = -1e30f;
// The reference max only moves when a step's probabilities would exceed this sum per
// lane (2^64): p stays far inside the fp32 and bf16 ranges, and precision does not
// depend on the scale, so no per-step row maximum is needed.
constexpr float kSumLimit = 18446744073709551616.0f;

// Row max of a step's scores across both lane halves.
__device__ __forceinline__ float step_max(const f32x16& s) {
  float m = __builtin_fmaxf(__builtin_fmaxf(s[0], s[1]), s[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) m = __builtin_fmaxf(__builtin_fmaxf(m, s[r]), s[r + 1]);
  m = __builtin_fmaxf(m, s[15]);
  return max_halves(m);
}

// p = exp2(s c - m) packed to bf16 pairs (register r of the scores = element r of the
// B operand of the PV product); returns this lane's sum of the same rounded p.
__device__ __forceinline__ float exponentiate(const f32x16& s, float m, float c, u32x4 (&pk)[2]) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  float ls = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p0 = fast_exp2(__builtin_fmaf(s[2 * e], c, -m));
    const float p1 = fast_exp2(__builtin_fmaf(s[2 * e + 1], c, -m));
    const uint32_t w = pack_bf16(p0, p1);
    pk[e >> 2][e & 3] = w;
    ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, ls, false);
  }
  return ls;
}

// Softmax of one step for every block: exponentiate against the reference max; in
// the rare step where some lane's sum passes kSumLimit (always the first step), move
// the reference max to the step's row max, rescale O and l, and exponentiate again.
template <int D, int QB>
__device__ __forceinline__ void softmax_step(Block<D> (&blk)[QB], const f32x16 (&sc)[QB], float c,
                                             u32x4 (&pk)[QB][2]) {
  float ls[QB];
  bool over = false;
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    ls[b] = exponentiate(sc[b], blk[b].m, c, pk[b]);
    over |= ls[b] > kSumLimit;
  }
  if (__builtin_amdgcn_ballot_w64(over)) {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      const float m_new = __builtin_fmaxf(blk[b].m, step_max(sc[b]) * c);
      const float f = fast_exp2(blk[b].m - m_new);
      blk[b].l *= f;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) blk[b].o[db][r] *= f;
      blk[b].m = m_new;
      ls[b] = exponentiate(sc[b], m_new, c, pk[b]);
    }
  }
#pragma unroll
  for (int b = 0; b < QB; ++b) blk[b].l += ls[b];
}

template <int D, int QB>
__global__ __launch_bounds__(64 * (kDenseQ / (32 * QB)), kDenseQ / (32 * QB) >= 8 ? 1 : 8 / (kDenseQ / (32 * QB)))
void dense_attn_bf16(const DenseParams p) {
  using R = Ring<D, QB>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  __shared__ __attribute__((aligned(1024))) char ring[R::kBytes];
  lds_char* const lds = (lds_char*)ring;

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

  // per-lane LDS addresses (relative to a stage) of the K fragments and the
  // transposed V fragments; s2 (keys 16..31 of the step) adds 16 rows
  uint32_t kaddr[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    kaddr[ks] = l32 * R::kRowBytes + (((2 * ks + half) ^ chunk_swz<D>(l32)) << 4);
  uint32_t vaddr[DB][2];
  {
    const int j16 = lane & 15, grp = lane >> 4, h = grp >> 1, g = grp & 1;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int row = 8 * x + 4 * h + j16 / 4;
        const int c = 4 * db + 2 * g + (j16 % 4) / 2;
        vaddr[db][x] = R::kTileBytes + row * R::kRowBytes + ((c ^ chunk_swz<D>(row)) << 4) + (j16 % 2) * 8;
      }
  }

  // direct loads: this lane's row within the step and its chunk's byte offset
  int ld_row[R::kLoads];
  uint32_t ld_chunk[R::kLoads];
#pragma unroll
  for (int i = 0; i < R::kLoads; ++i) {
    const int gi = wave * R::kLoads + i;
    ld_row[i] = gi * R::kRowsPerLoad + lane / R::kCpr;
    ld_chunk[i] = (uint32_t)(((lane % R::kCpr) ^ chunk_swz<D>(ld_row[i])) << 4);
  }
  const char* kh = (const char*)p.k_hist + e.hist_off * 2;
  const char* vh = (const char*)p.v_hist + e.hist_off * 2;
  const char* kc = (const char*)p.k_cur + (int64_t)e.head * D * 2;
  const char* vc = (const char*)p.v_cur + (int64_t)e.head * D * 2;
  const int64_t hs = p.hist_stride * 2, ts = p.tok_stride * 2;   // bytes
  const int hl = e.hist_len;
  uint32_t off_h[R::kLoads], off_c[R::kLoads];   // byte offsets within a step, per segment
#pragma unroll
  for (int i = 0; i < R::kLoads; ++i) {
    off_h[i] = (uint32_t)(ld_row[i] * hs) + ld_chunk[i];
    off_c[i] = (uint32_t)(ld_row[i] * ts) + ld_chunk[i];
  }

  // direct loads of step t into ring stage `stage`
  auto issue = [&](int t, int stage) {
    const int k0 = k_begin + t * kStep;
    const uint32_t dst = (uint32_t)(uintptr_t)(lds + stage * R::kStageBytes) + wave * R::kLoads * 1024;
    if (k0 + kStep <= min(hl, k_end)) {   // whole step in the history segment
      const char* kb = kh + (int64_t)k0 * hs;
      const char* vb = vh + (int64_t)k0 * hs;
#pragma unroll
      for (int i = 0; i < R::kLoads; ++i) {
        dma16(kb, off_h[i], dst + i * 1024);
        dma16(vb, off_h[i], dst + R::kTileBytes + i * 1024);
      }
    } else if (k0 >= hl && k0 + kStep <= k_end) {   // whole step in the current block
      const char* kb = kc + (int64_t)(k0 - hl) * ts;
      const char* vb = vc + (int64_t)(k0 - hl) * ts;
#pragma unroll
      for (int i = 0; i < R::kLoads; ++i) {
        dma16(kb, off_c[i], dst + i * 1024);
        dma16(vb, off_c[i], dst + R::kTileBytes + i * 1024);
      }
    } else {   // straddles the segments or runs past the end: per-row offsets, clamped
#pragma unroll
      for (int i = 0; i < R::kLoads; ++i) {
        const int kk = min(k0 + ld_row[i], k_end - 1);
        const bool h = kk < hl;
        const uint32_t off = (uint32_t)(h ? (int64_t)kk * hs : (int64_t)(kk - hl) * ts) + ld_chunk[i];
        if (h) {   // lanes of the two segments issue in turn
          dma16(kh, off, dst + i * 1024);
          dma16(vh, off, dst + R::kTileBytes + i * 1024);
        } else {
          dma16(kc, off, dst + i * 1024);
          dma16(vc, off, dst + R::kTileBytes + i * 1024);
        }
      }
    }
  };

  // S^T of a step for every block (each K fragment read once, used QB times)
  auto scores = [&](f32x16 (&sc)[QB], int stage) {
    const lds_char* base = lds + stage * R::kStageBytes;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 kf = *(const __attribute__((address_space(3))) u32x4*)(base + kaddr[ks]);
#pragma unroll
      for (int b = 0; b < QB; ++b) sc[b] = mfma32(kf, q[b][ks], ks == 0 ? f32x16{} : sc[b]);
    }
  };
  Block<D> blk[QB];
  // O^T += V^T P^T of a step for every block (each V^T fragment read once, used QB times)
  auto pv = [&](const u32x4 (&pk)[QB][2], int stage) {
    const lds_char* base = lds + stage * R::kStageBytes;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(base + vaddr[db][0] + s2 * 16 * R::kRowBytes));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(base + vaddr[db][1] + s2 * 16 * R::kRowBytes));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 vf = {l2[0], l2[1], h2[0], h2[1]};
#pragma unroll
        for (int b = 0; b < QB; ++b) blk[b].o[db] = mfma32(vf, pk[b][s2], blk[b].o[db]);
      }
  };

#pragma unroll
  for (int b = 0; b < QB; ++b) {
#pragma unroll
    for (int db = 0; db < DB; ++db) blk[b].o[db] = f32x16{};
    blk[b].m = kNoMax;
    blk[b].l = 0.f;
  }
  const float c = p.scale_log2;

  // Step t sits on ring stage (t - r0) mod 4 with r0 = (n - 1) mod 4: the first r0
  // steps run with run-time stage offsets, the other n - 1 - r0 (a multiple of 4) in
  // groups of four with the offsets folded into the LDS instructions, and the last
  // step lands on stage 0.
  static_assert(kStages == 4, "the step groups below walk four stages");
  const int r0 = (n - 1) & 3;

  // prologue: steps 0 .. kStages-2 in flight, scores and row maxima of step 0
#pragma unroll
  for (int t = 0; t < kStages - 1; ++t)
    if (t < n) issue(t, (t - r0) & 3);
  if (n >= kStages - 1)
    wait_vmcnt<2 * R::kLoads * (kStages - 2)>();
  else
    wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  f32x16 s0[QB], s1[QB];   // scores of two consecutive steps
  scores(s0, (0 - r0) & 3);

  // step j on stage `stage` (scores in sc): loads of step j+kStages-1, scores of
  // step j+1 (into sn) beside the softmax of step j, then PV of step j
  auto step = [&](f32x16 (&sc)[QB], f32x16 (&sn)[QB], int stage, int j) {
    if (j + kStages - 2 < n)
      wait_vmcnt<2 * R::kLoads * (kStages - 3)>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    if (j + kStages - 1 < n) issue(j + kStages - 1, (stage + kStages - 1) & 3);
    scores(sn, (stage + 1) & 3);
    u32x4 pk[QB][2];
    softmax_step(blk, sc, c, pk);
    // issue in order: alternate each score MFMA with the exponentials that fit under
    // it, and read K fragments kAhead MFMA groups ahead of their use
    constexpr int kAhead = 3;
    constexpr int kVq = 6;
    __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);
#pragma unroll
    for (int i = 0; i < KS; ++i) {
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kVq, 0);
      }
      if (i + kAhead < KS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    pv(pk, stage);
  };

  int j = 0;
  for (; j < r0; ++j) {
    step(s0, s1, (j - r0) & 3, j);
#pragma unroll
    for (int b = 0; b < QB; ++b) s0[b] = s1[b];
  }
  for (; j + 1 < n; j += 4) {
    step(s0, s1, 0, j);
    step(s1, s0, 1, j + 1);
    step(s0, s1, 2, j + 2);
    step(s1, s0, 3, j + 3);
  }

  // last step (stage 0, scores in s0): masked when ragged
  {
    const int valid = k_end - (k_begin + j * kStep);
    if (valid < kStep) {
#pragma unroll
      for (int b = 0; b < QB; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (8 * (r >> 2) + 4 * half + (r & 3) >= valid) s0[b][r] = -INFINITY;
    }
    u32x4 pk[QB][2];
    softmax_step(blk, s0, c, pk);
    pv(pk, 0);
  }

  // outputs
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const float l_tot = sum_halves(blk[b].l);
    if (q_row[b] >= p.lq) continue;
    AttnState<D> st;
#pragma unroll
    for (int db = 0; db < DB; ++db) st.o[db] = blk[b].o[db];
    st.m_run = blk[b].m;
    if (e.slot < 0) {
      uint16_t* op = (uint16_t*)p.out + (int64_t)q_row[b] * p.tok_stride + (int64_t)e.head * D;
      store_out_bf16<D>(st, 1.0f / l_tot, op, half);
    } else {
      const int64_t prow = (int64_t)(e.slot + split) * p.lq + q_row[b];
      store_partial<D>(st, l_tot, p.part_o + prow * D, p.part_ml + prow * 2, half);
    }
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
  // D=128: four waves of 32 queries; D=64: two waves of 64 queries
  const dim3 grid(dense_items_grid(p.n_items, p.xcd_group));
  if (head_dim == 64)
    hipLaunchKernelGGL((dense_attn_bf16<64, 2>), grid, dim3(64 * Ring<64, 2>::kWaves), 0, s, p);
  else
    hipLaunchKernelGGL((dense_attn_bf16<128, 1>), grid, dim3(64 * Ring<128, 1>::kWaves), 0, s, p);
  return hipGetLastError();
}

}  // namespace hc
