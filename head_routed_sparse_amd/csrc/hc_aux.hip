// Supporting kernels: log-sum-exp merge of key-split partials, the per-head buffer
// copy (HeadCast Sec. 4.3 "Heterogeneous Cache Management": build and rolling append),
// the classifier's per-token statistics (Sec. 4.2 Eqs. 2-4), and the fp32 variants of
// the dense and Spatial paths used when the inputs are fp32.
#include <mutex>
#include <vector>

#include "../../include/headcast.h"
#include "hc_internal.h"
#include "hc_mfma.h"

namespace hc {

namespace {

// Normalised mix of partial slots [slot, slot + n) of query row q at dims d..d+3.
__device__ __forceinline__ f32x4 mix_slots(const float* po, const float* pml, int64_t lq, int D,
                                           int slot, int n, int q, int d, float* l_out) {
  float M = -INFINITY;
  for (int i = 0; i < n; ++i) M = fmaxf(M, pml[((slot + i) * lq + q) * 2]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int i = 0; i < n; ++i) {
    const int64_t row = (slot + i) * lq + q;
    const float m = pml[row * 2];
    const float w = m == -INFINITY ? 0.f : fast_exp2(m - M);
    L += w * pml[row * 2 + 1];
    const f32x4 o = *(const f32x4*)(po + row * D + d);
    acc += w * o;
  }
  if (l_out) *l_out = L;
  return acc * (1.0f / L);
}

// The same mix for at most N slots, with every load issued before the first use (one
// memory round trip instead of one for the maxima and one for the rest).
template <int N>
__device__ __forceinline__ f32x4 mix_few_slots(const float* po, const float* pml, int64_t lq, int D,
                                               int slot, int n, int q, int d) {
  float m[N], l[N];
  f32x4 v[N];
#pragma unroll
  for (int i = 0; i < N; ++i) {   // slots past n load the last slot again, with weight 0
    const int64_t row = (slot + min(i, n - 1)) * lq + q;
    const float2 ml = *(const float2*)(pml + row * 2);
    m[i] = i < n ? ml.x : -INFINITY;
    l[i] = ml.y;
    v[i] = *(const f32x4*)(po + row * D + d);
  }
  float M = m[0];
#pragma unroll
  for (int i = 1; i < N; ++i) M = fmaxf(M, m[i]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float w = m[i] == -INFINITY ? 0.f : fast_exp2(m[i] - M);
    L += w * l[i];
    acc += w * v[i];
  }
  return acc * (1.0f / L);
}

template <bool kBf16>
__global__ __launch_bounds__(256) void merge_kernel(const MergeParams p) {
  const MergeEntry e = p.e[blockIdx.y];
  const int D = p.head_dim;
  const int tpq = D / 4;
  const int q = blockIdx.x * (256 / tpq) + threadIdx.x / tpq;
  const int d = (threadIdx.x % tpq) * 4;
  if (q >= p.lq) return;
  const f32x4 o = e.nslot <= 4   ? mix_few_slots<4>(p.part_o, p.part_ml, p.lq, D, e.slot, e.nslot, q, d)
                 : e.nslot <= 8  ? mix_few_slots<8>(p.part_o, p.part_ml, p.lq, D, e.slot, e.nslot, q, d)
                 : e.nslot <= 16 ? mix_few_slots<16>(p.part_o, p.part_ml, p.lq, D, e.slot, e.nslot, q, d)
                                 : mix_slots(p.part_o, p.part_ml, p.lq, D, e.slot, e.nslot, q, d, nullptr);
  const int64_t off = (int64_t)q * p.tok_stride + (int64_t)e.head * D + d;
  if (kBf16) {
    u32x2 w = {pack_bf16(o[0], o[1]), pack_bf16(o[2], o[3])};
    *(u32x2*)((uint16_t*)p.out + off) = w;
  } else {
    *(f32x4*)((float*)p.out + off) = o;
  }
}

__global__ __launch_bounds__(256) void copy_rows_kernel(const CopyParams p) {
  const CopyEntry e = p.e[blockIdx.y];
  const int cpr = p.row_bytes / 16;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (int64_t)p.rows * cpr) return;
  const int64_t row = idx / cpr;
  const int ch = (int)(idx % cpr);
  const int64_t src = e.src_off + row * p.src_stride + ch * 16;
  const int64_t dst = e.dst_off + row * p.row_bytes + ch * 16;
  *(u32x4*)((char*)p.dst_k + dst) = *(const u32x4*)((const char*)p.src_k + src);
  *(u32x4*)((char*)p.dst_v + dst) = *(const u32x4*)((const char*)p.src_v + src);
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

// One wave per (head, token): rebuild the normalised reference and proxy outputs from
// the partial slots and reduce the dot products the cosines and the MSE need.
__global__ __launch_bounds__(256) void stats_kernel(const StatsParams p) {
  const int h = blockIdx.y;
  const int q = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (q >= p.lq) return;
  const int D = p.head_dim;
  const int base = h * p.slots_per_head;
  float dot_s = 0, nn_s = 0, dot_d = 0, nn_d = 0, dot_p = 0, nn_p = 0, nn_r = 0, se = 0;
  for (int d = lane * 4; d < D; d += 256) {
    // reference: current block + sink block + middle frames (base, base+1, base+3..)
    float M = -INFINITY;
    const int nref = 2 + p.n_mid;
    for (int i = 0; i < nref; ++i) {
      const int slot = i < 2 ? base + i : base + 1 + i;
      M = fmaxf(M, p.part_ml[((int64_t)slot * p.lq + q) * 2]);
    }
    f32x4 ref = {0.f, 0.f, 0.f, 0.f};
    float L = 0.f;
    for (int i = 0; i < nref; ++i) {
      const int slot = i < 2 ? base + i : base + 1 + i;
      const int64_t row = (int64_t)slot * p.lq + q;
      const float m = p.part_ml[row * 2];
      const float w = m == -INFINITY ? 0.f : fast_exp2(m - M);
      L += w * p.part_ml[row * 2 + 1];
      ref += w * *(const f32x4*)(p.part_o + row * D + d);
    }
    ref *= 1.0f / L;
    const f32x4 dum = mix_slots(p.part_o, p.part_ml, p.lq, D, base, 1, q, d, nullptr);
    const f32x4 snk = p.sink_with_cur ? mix_slots(p.part_o, p.part_ml, p.lq, D, base, 2, q, d, nullptr)
                                      : mix_slots(p.part_o, p.part_ml, p.lq, D, base + 1, 1, q, d, nullptr);
    // spatial proxy: current block (slot base) + gathered history (slot base + 2)
    float Ms = fmaxf(p.part_ml[((int64_t)base * p.lq + q) * 2], p.part_ml[((int64_t)(base + 2) * p.lq + q) * 2]);
    f32x4 sp = {0.f, 0.f, 0.f, 0.f};
    float Ls = 0.f;
    for (int i = 0; i < 2; ++i) {
      const int64_t row = (int64_t)(base + 2 * i) * p.lq + q;
      const float m = p.part_ml[row * 2];
      const float w = m == -INFINITY ? 0.f : fast_exp2(m - Ms);
      Ls += w * p.part_ml[row * 2 + 1];
      sp += w * *(const f32x4*)(p.part_o + row * D + d);
    }
    sp *= 1.0f / Ls;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      nn_r += ref[j] * ref[j];
      dot_s += snk[j] * ref[j];
      nn_s += snk[j] * snk[j];
      dot_d += dum[j] * ref[j];
      nn_d += dum[j] * dum[j];
      dot_p += sp[j] * ref[j];
      nn_p += sp[j] * sp[j];
      const float df = sp[j] - ref[j];
      se += df * df;
    }
  }
  dot_s = wave_sum(dot_s);
  nn_s = wave_sum(nn_s);
  dot_d = wave_sum(dot_d);
  nn_d = wave_sum(nn_d);
  dot_p = wave_sum(dot_p);
  nn_p = wave_sum(nn_p);
  nn_r = wave_sum(nn_r);
  se = wave_sum(se);
  if (lane == 0) {
    const float nr = sqrtf(nn_r);
    float* out = p.stats + ((int64_t)h * p.lq + q) * 4;
    out[0] = dot_s / fmaxf(sqrtf(nn_s) * nr, 1e-8f);
    out[1] = dot_d / fmaxf(sqrtf(nn_d) * nr, 1e-8f);
    out[2] = dot_p / fmaxf(sqrtf(nn_p) * nr, 1e-8f);
    out[3] = se;
  }
}

// ---------------------------------------------------------------- fp32 inputs
// One thread per query, exact online softmax in fp32; same item enumeration and
// output conventions as the bf16 kernels (the output is fp32).
template <int D>
__global__ __launch_bounds__(kDenseQ) void dense_attn_f32(const DenseParams p) {
  const int item = blockIdx.x;
  if (item >= p.n_items) return;
  int ei = 0;
  while (ei + 1 < p.n_entries && item >= p.e[ei + 1].item_begin) ++ei;
  const DenseEntry e = p.e[ei];
  const int local = item - e.item_begin;
  const int split = local / p.nqt;
  const int qt = local - split * p.nqt;
  const int k_begin = split * e.split_len;
  const int k_end = min(e.hist_len + e.cur_len, k_begin + e.split_len);
  const int q_row = qt * kDenseQ + threadIdx.x;
  if (q_row >= p.lq) return;
  const float* qp = (const float*)p.q + (int64_t)q_row * p.tok_stride + (int64_t)e.head * D;
  float qv[D], o[D];
  for (int d = 0; d < D; ++d) {
    qv[d] = qp[d];
    o[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int kk = k_begin; kk < k_end; ++kk) {
    const float* kr;
    const float* vr;
    if (kk < e.hist_len) {
      kr = (const float*)p.k_hist + e.hist_off + (int64_t)kk * p.hist_stride;
      vr = (const float*)p.v_hist + e.hist_off + (int64_t)kk * p.hist_stride;
    } else {
      kr = (const float*)p.k_cur + (int64_t)(kk - e.hist_len) * p.tok_stride + (int64_t)e.head * D;
      vr = (const float*)p.v_cur + (int64_t)(kk - e.hist_len) * p.tok_stride + (int64_t)e.head * D;
    }
    float s = 0.f;
    for (int d = 0; d < D; ++d) s += qv[d] * kr[d];
    s *= p.scale_log2;
    const float mn = fmaxf(m, s);
    const float f = exp2f(m - mn);
    const float w = exp2f(s - mn);
    l = l * f + w;
    for (int d = 0; d < D; ++d) o[d] = o[d] * f + w * vr[d];
    m = mn;
  }
  if (e.slot < 0) {
    float* op = (float*)p.out + (int64_t)q_row * p.tok_stride + (int64_t)e.head * D;
    for (int d = 0; d < D; ++d) op[d] = o[d] / l;
  } else {
    const int64_t prow = (int64_t)(e.slot + split) * p.lq + q_row;
    for (int d = 0; d < D; ++d) p.part_o[prow * D + d] = o[d];
    p.part_ml[prow * 2] = m;
    p.part_ml[prow * 2 + 1] = l;
  }
}

template <int D>
__global__ __launch_bounds__(64) void spatial_attn_f32(const SpatialParams p) {
  const SpatialEntry e = p.e[blockIdx.y];
  const int fh = p.frame_h, fw = p.frame_w, S = fh * fw;
  const int pos = blockIdx.x * 64 + threadIdx.x;
  if (pos >= S) return;
  const int r = pos / fw, c = pos % fw;
  const bool cells = p.cells != 0;
  const int r0 = cells ? cell_origin(r, p.grid_h) : win_origin(r, p.grid_h, fh);
  const int c0 = cells ? cell_origin(c, p.grid_w) : win_origin(c, p.grid_w, fw);
  const int eh = cells ? cell_extent(r, p.grid_h, fh) : min(p.grid_h, fh);
  const int ew = cells ? cell_extent(c, p.grid_w, fw) : min(p.grid_w, fw);
  const int n_frames = p.n_hist_frames + (cells ? p.chunk_frames : 0);
  for (int cf = 0; cf < p.chunk_frames; ++cf) {
    const int q_row = cf * S + pos;
    const float* qp = (const float*)p.q + (int64_t)q_row * p.tok_stride + (int64_t)e.head * D;
    float qv[D], o[D];
    for (int d = 0; d < D; ++d) {
      qv[d] = qp[d];
      o[d] = 0.f;
    }
    float m = -INFINITY, l = 0.f;
    for (int f = 0; f < n_frames; ++f)
      for (int kr = r0; kr < r0 + eh; ++kr)
        for (int kc = c0; kc < c0 + ew; ++kc) {
          const float* kp;
          const float* vp;
          if (f < p.n_hist_frames) {
            const int64_t row = (int64_t)f * S + kr * fw + kc;
            kp = (const float*)p.k_hist + e.hist_off + row * p.hist_stride;
            vp = (const float*)p.v_hist + e.hist_off + row * p.hist_stride;
          } else {
            const int64_t tok = (int64_t)(f - p.n_hist_frames) * S + kr * fw + kc;
            kp = (const float*)p.k_cur + tok * p.tok_stride + (int64_t)e.head * D;
            vp = (const float*)p.v_cur + tok * p.tok_stride + (int64_t)e.head * D;
          }
          float s = 0.f;
          for (int d = 0; d < D; ++d) s += qv[d] * kp[d];
          s *= p.scale_log2;
          const float mn = fmaxf(m, s);
          const float fct = exp2f(m - mn);
          const float w = exp2f(s - mn);
          l = l * fct + w;
          for (int d = 0; d < D; ++d) o[d] = o[d] * fct + w * vp[d];
          m = mn;
        }
    float* op = (float*)p.out + (int64_t)q_row * p.tok_stride + (int64_t)e.head * D;
    if (cells) {
      for (int d = 0; d < D; ++d) op[d] = o[d] / l;
    } else if (e.out_slot >= 0) {
      const int64_t prow = (int64_t)e.out_slot * p.lq + q_row;
      for (int d = 0; d < D; ++d) p.part_o[prow * D + d] = o[d];
      p.part_ml[prow * 2] = m;
      p.part_ml[prow * 2 + 1] = l;
    } else {
      const int64_t crow = (int64_t)e.cur_slot * p.lq + q_row;
      const float m_c = p.part_ml[crow * 2], l_c = p.part_ml[crow * 2 + 1];
      const float M = fmaxf(m, m_c);
      const float wa = m == -INFINITY ? 0.f : exp2f(m - M);
      const float wc = exp2f(m_c - M);
      const float inv = 1.0f / (wa * l + wc * l_c);
      for (int d = 0; d < D; ++d) op[d] = (wa * o[d] + wc * p.part_o[crow * D + d]) * inv;
    }
  }
}

}  // namespace

// Partial results of the allocation-free routed call: one array per device, alive until
// the process ends. Host code never uses the array's name as an address: each device's
// copy is found with hipGetSymbolAddress (with that device current) and kept per device.
static __device__ __align__(256) char scratch[HC_NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static std::vector<void*> addr;   // by device id
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(mu);
  if ((int)addr.size() <= dev) addr.resize(dev + 1, nullptr);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = sizeof(scratch);
  return hipSuccess;
}

hipError_t launch_merge(const MergeParams& p, int head_dim, int bf16, hipStream_t s) {
  if (p.n_entries == 0) return hipSuccess;
  const int qpb = 256 / (head_dim / 4);
  const dim3 grid((p.lq + qpb - 1) / qpb, p.n_entries);
  if (bf16)
    hipLaunchKernelGGL(merge_kernel<true>, grid, dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(merge_kernel<false>, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_copy(const CopyParams& p, hipStream_t s) {
  if (p.n_entries == 0 || p.rows == 0) return hipSuccess;
  const int64_t n = (int64_t)p.rows * (p.row_bytes / 16);
  const dim3 grid((unsigned)((n + 255) / 256), p.n_entries);
  hipLaunchKernelGGL(copy_rows_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_stats(const StatsParams& p, hipStream_t s) {
  const dim3 grid((p.lq + 3) / 4, p.num_heads);
  hipLaunchKernelGGL(stats_kernel, grid, dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_dense_f32(const DenseParams& p, int head_dim, hipStream_t s) {
  const dim3 grid(p.n_items), block(kDenseQ);
  if (head_dim == 128)
    hipLaunchKernelGGL(dense_attn_f32<128>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(dense_attn_f32<64>, grid, block, 0, s, p);
  return hipGetLastError();
}

hipError_t launch_spatial_f32(const SpatialParams& p, int head_dim, hipStream_t s) {
  const int S = p.frame_h * p.frame_w;
  const dim3 grid((S + 63) / 64, p.n_entries), block(64);
  if (head_dim == 128)
    hipLaunchKernelGGL(spatial_attn_f32<128>, grid, block, 0, s, p);
  else
    hipLaunchKernelGGL(spatial_attn_f32<64>, grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace hc
