// The pipelined attention step shared by the dense and Spatial kernels (bf16, gfx950).
//
// Keys advance in steps of 32. The K and V rows of a step travel from global memory
// straight into a ring of LDS stages (16-byte direct loads, no staging registers),
// row-major, with the 16-byte chunks of row r permuted (chunk c stored at
// c ^ chunk_swz(r)) so that the K fragment reads and the transposed V reads
// (ds_read_b64_tr_b16) hit distinct banks. Each wave holds QB blocks of 32 queries as
// the B operand of S^T = K Q^T (a lane carries one query's 16 scores of the step) and
// accumulates O^T += V^T P^T with P taken from the score registers. Per step, the
// scores of step j+1 run on the matrix cores while the VALU exponentiates step j.
#pragma once
#include "hc_internal.h"
#include "hc_mfma.h"

namespace hc {


typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) char lds_char;

// Step-tile geometry for head dim D, QB query blocks per wave and W waves per workgroup
// (an LDS ring of NS stages takes NS * kStageBytes).
template <int D, int QB, int W>
struct Ring {
  static constexpr int kWaves = W;
  static constexpr int kRowBytes = 2 * D;
  static constexpr int kCpr = D / 8;                       // 16-byte chunks per row
  static constexpr int kTileBytes = kStep * kRowBytes;     // the K (or V) rows of a step
  static constexpr int kStageBytes = 2 * kTileBytes;
  static constexpr int kRowsPerLoad = 1024 / kRowBytes;    // rows one wave-wide 16-B load fills
  static constexpr int kLoads = kStep / kRowsPerLoad / W;  // per wave and tensor
  static_assert(kLoads >= 1 && kLoads * kRowsPerLoad * W == kStep, "step tile and wave count");
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
// explicitly (s_waitcnt vmcnt) before the barrier that publishes a stage. M0 is
// written here and nowhere else in these kernels (the compiler reserves it and would
// warn about the clobber).
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

template <int D, int QB>
__device__ __forceinline__ void init_blocks(Block<D> (&blk)[QB]) {
#pragma unroll
  for (int b = 0; b < QB; ++b) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) blk[b].o[db] = f32x16{};
    blk[b].m = kNoMax;
    blk[b].l = 0.f;
  }
}

// Row max of a step's scores across both lane halves.
__device__ __forceinline__ float step_max(const f32x16& s) {
  float m = __builtin_fmaxf(__builtin_fmaxf(s[0], s[1]), s[2]);
#pragma unroll
  for (int r = 3; r < 15; r += 2) m = __builtin_fmaxf(__builtin_fmaxf(m, s[r]), s[r + 1]);
  m = __builtin_fmaxf(m, s[15]);
  return max_halves(m);
}

// p = exp2(s c + add(r)) packed to bf16 pairs (register r of the scores = element r of
// the B operand of the PV product); returns this lane's sum of the same rounded p. The
// addend is -m, or -inf for a key the query does not see (p = 0 exactly).
template <class Add>
__device__ __forceinline__ float exponentiate(const f32x16& s, Add&& add, float c, u32x4 (&pk)[2]) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  float ls = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p0 = fast_exp2(__builtin_fmaf(s[2 * e], c, add(2 * e)));
    const float p1 = fast_exp2(__builtin_fmaf(s[2 * e + 1], c, add(2 * e + 1)));
    const uint32_t w = pack_bf16(p0, p1);
    pk[e >> 2][e & 3] = w;
    ls = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w), one, ls, false);
  }
  return ls;
}

// Move the reference max of a block to m_new (>= m): rescale O and l.
template <int D>
__device__ __forceinline__ void move_max(Block<D>& b, float m_new) {
  const float f = fast_exp2(b.m - m_new);
  b.l *= f;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) b.o[db][r] *= f;
  b.m = m_new;
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
    const float neg_m = -blk[b].m;
    ls[b] = exponentiate(sc[b], [&](int) { return neg_m; }, c, pk[b]);
    over |= ls[b] > kSumLimit;
  }
  if (__builtin_amdgcn_ballot_w64(over)) {
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      move_max(blk[b], __builtin_fmaxf(blk[b].m, step_max(sc[b]) * c));
      const float neg_m = -blk[b].m;
      ls[b] = exponentiate(sc[b], [&](int) { return neg_m; }, c, pk[b]);
    }
  }
#pragma unroll
  for (int b = 0; b < QB; ++b) blk[b].l += ls[b];
}

// Write the normalised output row (bf16) of this lane's query; factor multiplies O.
// Register r of o[db] holds dimension db*32 + 8*(r/4) + 4*half + r%4.
template <int D>
__device__ __forceinline__ void store_out_bf16(const Block<D>& b, float factor, uint16_t* row, int half) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      u32x2 w;
      w[0] = pack_bf16(b.o[db][4 * a] * factor, b.o[db][4 * a + 1] * factor);
      w[1] = pack_bf16(b.o[db][4 * a + 2] * factor, b.o[db][4 * a + 3] * factor);
      *(u32x2*)(row + db * 32 + 8 * a + 4 * half) = w;
    }
}

// Write the unnormalised partial (fp32 O, reference max, total sum) of this lane's query.
template <int D>
__device__ __forceinline__ void store_partial(const Block<D>& b, float l_tot, float* po, float* pml, int half) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      f32x4 w = {b.o[db][4 * a], b.o[db][4 * a + 1], b.o[db][4 * a + 2], b.o[db][4 * a + 3]};
      *(f32x4*)(po + db * 32 + 8 * a + 4 * half) = w;
    }
  if (half == 0) {
    pml[0] = b.m;
    pml[1] = l_tot;
  }
}

// Local key (0..31) of score register r in lane half `half`.
__device__ __forceinline__ int step_key(int r, int half) { return 8 * (r >> 2) + 4 * half + (r & 3); }

// Per-lane addresses: LDS offsets (relative to a stage) of the K fragments and of the
// transposed V fragments (s2 = keys 16..31 of the step adds 16 rows), and for the
// direct loads the lane's rows within a step and its chunk's byte offset in a row.
template <int D, int QB, int W>
struct LaneAddr {
  using R = Ring<D, QB, W>;
  uint32_t k[D / 16];
  uint32_t v[D / 32][2];
  int ld_row[R::kLoads];
  uint32_t ld_chunk[R::kLoads];
  __device__ __forceinline__ void init(int wave, int lane) {
    const int l32 = lane & 31, half = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) k[ks] = l32 * R::kRowBytes + (((2 * ks + half) ^ chunk_swz<D>(l32)) << 4);
    const int j16 = lane & 15, grp = lane >> 4, h = grp >> 1, g = grp & 1;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        const int row = 8 * x + 4 * h + j16 / 4;
        const int c = 4 * db + 2 * g + (j16 % 4) / 2;
        v[db][x] = R::kTileBytes + row * R::kRowBytes + ((c ^ chunk_swz<D>(row)) << 4) + (j16 % 2) * 8;
      }
#pragma unroll
    for (int i = 0; i < R::kLoads; ++i) {
      const int gi = wave * R::kLoads + i;
      ld_row[i] = gi * R::kRowsPerLoad + lane / R::kCpr;
      ld_chunk[i] = (uint32_t)(((lane % R::kCpr) ^ chunk_swz<D>(ld_row[i])) << 4);
    }
  }
  // LDS destination of this wave's load i of tensor `which` (0 = K, 1 = V) in a stage.
  __device__ __forceinline__ uint32_t dst(const lds_char* lds, int stage, int wave, int i, int which) const {
    return (uint32_t)(uintptr_t)(lds + stage * R::kStageBytes) + which * R::kTileBytes +
           (wave * R::kLoads + i) * 1024;
  }
};

// The step pipeline over n >= 1 steps of 32 keys for W waves of QB query blocks.
//   issue(t, stage): start the direct loads of step t into ring stage `stage` (called
//                    once for t = 0, 1, 2, ... in order);
//   prep():          get ready for the softmax of the next step (may branch; called once
//                    per step, in order, before the score MFMAs issued beside it);
//   soft(sc, pk, last): the softmax of that step: fold its scores sc into the blocks'
//                    running max and sum and write the bf16 probabilities to pk (last is
//                    true for the final step only).
// The ring has NS stages (3 or 4); loads run NS - 1 steps ahead. With G = lcm(2, NS)
// (the score buffers alternate every step), step t sits on ring stage (t - r0) mod NS
// with r0 = (n - 1) mod G: the first r0 steps run with run-time stage offsets, the other
// n - 1 - r0 (a multiple of G) in groups of G with the offsets folded into the LDS
// instructions, and the last step lands on stage 0 with its scores in the first buffer.
//   active:          false for a wave with no queries of its own: it still issues its
//                    share of the loads and meets every barrier, but skips the math.
//   kEarlyV:         read the step's V^T fragments right after the barrier (their stage
//                    stays put for the whole step); otherwise after the score MFMAs and
//                    the softmax, before the step's loads go out, so that the reads land
//                    while the load addresses are worked out and the PV MFMAs then issue
//                    back to back. Early reads hold 32 more registers over the score
//                    phase (they pay in the Spatial kernel, the later ones in the dense).
template <int D, int QB, int W, int NS, bool kEarlyV, class Issue, class Prep, class Soft>
__device__ __forceinline__ void run_steps(int n, lds_char* lds, const LaneAddr<D, QB, W>& la,
                                          const u32x4 (&q)[QB][D / 16], Block<D> (&blk)[QB], bool active,
                                          Issue&& issue, Prep&& prep, Soft&& soft) {
  using R = Ring<D, QB, W>;
  constexpr int KS = D / 16;
  constexpr int DB = D / 32;
  static_assert(NS == 3 || NS == 4, "ring depth");
  constexpr int G = NS % 2 == 0 ? NS : 2 * NS;   // steps per group

  // S^T of a step for every block (each K fragment read once, used QB times)
  auto scores = [&](f32x16 (&sc)[QB], int stage) {
    const lds_char* base = lds + stage * R::kStageBytes;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const u32x4 kf = *(const __attribute__((address_space(3))) u32x4*)(base + la.k[ks]);
#pragma unroll
      for (int b = 0; b < QB; ++b) sc[b] = mfma32(kf, q[b][ks], ks == 0 ? f32x16{} : sc[b]);
    }
  };
  // O^T += V^T P^T of a step for every block (each V^T fragment read once, used QB times)
  // V^T fragments of a step
  auto read_v = [&](u32x4 (&vf)[2][DB], int stage) {
    const lds_char* base = lds + stage * R::kStageBytes;
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(base + la.v[db][0] + s2 * 16 * R::kRowBytes));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(base + la.v[db][1] + s2 * 16 * R::kRowBytes));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        vf[s2][db] = u32x4{l2[0], l2[1], h2[0], h2[1]};
      }
  };
  // O^T += V^T P^T of a step for every block (each V^T fragment used QB times)
  auto pv = [&](const u32x4 (&pk)[QB][2], const u32x4 (&vf)[2][DB]) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int b = 0; b < QB; ++b) blk[b].o[db] = mfma32(vf[s2][db], pk[b][s2], blk[b].o[db]);
  };

  const int r0 = (n - 1) % G;
  auto stage_of = [&](int t) { return (t - r0 + G) % NS; };   // t >= 0 > -G
  // prologue: steps 0 .. NS-2 in flight, scores of step 0
#pragma unroll
  for (int t = 0; t < NS - 1; ++t)
    if (t < n) issue(t, stage_of(t));
  if (n >= NS - 1)
    wait_vmcnt<2 * R::kLoads * (NS - 2)>();
  else
    wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  f32x16 s0[QB], s1[QB];   // scores of two consecutive steps
  if (active) scores(s0, stage_of(0));

  // step j on stage `stage` (scores in sc): scores of step j+1 (into sn) beside the
  // softmax of step j, the loads of step j+NS-1, then PV of step j
  auto step = [&](f32x16 (&sc)[QB], f32x16 (&sn)[QB], int stage, int j) {
    if (j + NS - 2 < n)
      wait_vmcnt<2 * R::kLoads * (NS - 3)>();
    else
      wait_vmcnt<0>();
    __builtin_amdgcn_s_barrier();
    // the loads of step j+NS-1 go out just before the PV product (below): issued right
    // after the barrier, the eight waves of a CU queue on the texture path together
    if (!active) {
      if (j + NS - 1 < n) issue(j + NS - 1, (stage + NS - 1) % NS);
      return;
    }
    prep();
    scores(sn, (stage + 1) % NS);
    u32x4 vf[2][DB] = {};
    if (kEarlyV) read_v(vf, stage);
    u32x4 pk[QB][2];
    soft(sc, pk, false);
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
    if (!kEarlyV) read_v(vf, stage);
    if (j + NS - 1 < n) issue(j + NS - 1, (stage + NS - 1) % NS);
    // raised wave priority over the PV product: the SIMD's other wave, which is then
    // most likely in its softmax, yields issue slots to these MFMAs
    __builtin_amdgcn_s_setprio(1);
    pv(pk, vf);
    __builtin_amdgcn_s_setprio(0);
  };

  int j = 0;
  for (; j < r0; ++j) {
    step(s0, s1, stage_of(j), j);
#pragma unroll
    for (int b = 0; b < QB; ++b) s0[b] = s1[b];
  }
  for (; j + 1 < n; j += G) {
    step(s0, s1, 0, j);
    step(s1, s0, 1 % NS, j + 1);
    step(s0, s1, 2 % NS, j + 2);
    step(s1, s0, 3 % NS, j + 3);
    if (G == 6) {
      step(s0, s1, 4 % NS, j + 4);
      step(s1, s0, 5 % NS, j + 5);
    }
  }
  // last step (stage 0, scores in s0)
  if (!active) return;
  prep();
  u32x4 vf[2][DB] = {};
  if (kEarlyV) read_v(vf, 0);
  u32x4 pk[QB][2];
  soft(s0, pk, true);
  if (!kEarlyV) read_v(vf, 0);
  pv(pk, vf);
}

}  // namespace hc
