// The Spatial path's own launch (HeadCast Sec. 4.4 Spatial Path): one workgroup per
// (Spatial head, position tile, frame part); the work of a workgroup is in
// hc_spatial_tile.h. With sliding windows and d = 128 the routed call usually runs the
// same tiles as the last items of its dense launch instead (hc_dense.hip).
#include "hc_spatial_tile.h"

namespace hc {

namespace {

template <int D, bool TABLE>
__global__ __launch_bounds__(256, 2) void spatial_attn_bf16(const SpatialParams p) {
  __shared__ __attribute__((aligned(1024))) char ring[spatial_lds_bytes<D, TABLE>()];
  // the tiles of one XCD are neighbours (same head, same frames), so the L2 keeps the
  // window rows they share
  const int n_tiles = p.tiles_r * p.tiles_c;
  const int lid = xcd_block(blockIdx.x, n_tiles * p.n_parts * p.n_entries);
  spatial_tile<D, TABLE>(p, p.e[lid / (n_tiles * p.n_parts)], lid % n_tiles, (lid / n_tiles) % p.n_parts,
                         (lds_char*)ring);
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
  const dim3 grid(p.tiles_r * p.tiles_c * p.n_parts * p.n_entries), block(256);
  const bool table = spatial_table(p);
  if (head_dim == 128) {
    if (table)
      hipLaunchKernelGGL((spatial_attn_bf16<128, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((spatial_attn_bf16<128, false>), grid, block, 0, s, p);
  } else {
    if (table)
      hipLaunchKernelGGL((spatial_attn_bf16<64, true>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((spatial_attn_bf16<64, false>), grid, block, 0, s, p);
  }
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
