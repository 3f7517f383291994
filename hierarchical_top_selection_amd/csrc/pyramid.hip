// pyramid.hip - mean-pooled key pyramid (Method steps, first step; Core method
// eq. 10-15 of "Block Sparse Attention with Log-Linear Complexity").
//
// HBM-bound: the keys are read once (coalesced, one column per thread, rows in
// key order) and the float32 summaries written once.  One workgroup owns 8
// consecutive leaves and finishes their subtree (levels 2-4) in LDS; a second
// launch with one workgroup per (b, kvh) builds the levels above.
#include "kernels.h"
#include "pyramid_dev.h"

namespace pisa {

constexpr int kLeavesPerBlock = 8;   // subtree of levels 1..4 per workgroup
constexpr int kInBlockLevels = 4;

template <typename T, int D>
__global__ __launch_bounds__(256) void pyramid_leaves_kernel(PyramidArgs a) {
  __shared__ float tile[kLeavesPerBlock][D];
  const int bh = blockIdx.y;
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const T* kbase = reinterpret_cast<const T*>(a.k) + b * a.k_sb + kvh * a.k_sh;
  float* pyr = a.pyr + (int64_t)bh * a.lv.nodes * D;
  const int leaf0 = blockIdx.x * kLeavesPerBlock;
  const int m1 = a.lv.size[0];

  for (int item = threadIdx.x; item < kLeavesPerBlock * D; item += blockDim.x) {
    const int li = item / D, c = item % D;
    const int leaf = leaf0 + li;
    float v = 0.f;
    if (leaf < m1) {
      const int64_t first = (int64_t)leaf * kLeaf;
      const int cnt = (int)min((int64_t)kLeaf, (int64_t)a.n - first);
      v = leaf_mean_column(kbase, a.k_st, first, cnt, c);
      pyr[(a.lv.offset[0] + leaf) * D + c] = v;
    }
    tile[li][c] = v;
  }
  __syncthreads();

  // Levels 2..4 of this subtree: level l holds kLeavesPerBlock >> (l-1) local nodes.
  for (int level = 2; level <= kInBlockLevels && level <= a.lv.count; ++level) {
    const int nodes = kLeavesPerBlock >> (level - 1);
    const int base = blockIdx.x * nodes;              // first global node index at this level
    const int child_size = a.lv.size[level - 2];
    float out[2] = {0.f, 0.f};
    // each thread produces up to two (node, column) values, read before any write
    for (int r = 0; r < 2; ++r) {
      const int item = threadIdx.x + r * blockDim.x;
      if (item < nodes * D) {
        const int p = item / D, c = item % D;
        const int gp = base + p;
        const bool has2 = 2 * gp + 1 < child_size;
        out[r] = node_mean(tile[2 * p][c], tile[2 * p + 1][c], has2);
      }
    }
    __syncthreads();
    for (int r = 0; r < 2; ++r) {
      const int item = threadIdx.x + r * blockDim.x;
      if (item < nodes * D) {
        const int p = item / D, c = item % D;
        const int gp = base + p;
        tile[p][c] = out[r];
        if (gp < a.lv.size[level - 1]) pyr[(a.lv.offset[level - 1] + gp) * D + c] = out[r];
      }
    }
    __syncthreads();
  }
}

template <int D>
__global__ __launch_bounds__(1024) void pyramid_top_kernel(PyramidArgs a) {
  const int bh = blockIdx.x;
  float* pyr = a.pyr + (int64_t)bh * a.lv.nodes * D;
  for (int level = kInBlockLevels + 1; level <= a.lv.count; ++level) {
    const int nodes = a.lv.size[level - 1];
    const int child_size = a.lv.size[level - 2];
    const float* child = pyr + a.lv.offset[level - 2] * D;
    float* dst = pyr + a.lv.offset[level - 1] * D;
#pragma unroll 4
    for (int item = threadIdx.x; item < nodes * D; item += blockDim.x) {
      const int p = item / D, c = item % D;
      const bool has2 = 2 * p + 1 < child_size;
      const float c0 = child[(2 * p) * D + c];
      const float c1 = has2 ? child[(2 * p + 1) * D + c] : 0.f;
      dst[p * D + c] = node_mean(c0, c1, has2);
    }
    __syncthreads();
  }
}

template <typename T, int D>
hipError_t launch_pyramid_t(const PyramidArgs& a, hipStream_t s) {
  dim3 grid(ceil_div(a.lv.size[0], kLeavesPerBlock), a.batch * a.n_kv_heads);
  hipLaunchKernelGGL((pyramid_leaves_kernel<T, D>), grid, dim3(256), 0, s, a);
  hipError_t e = launched(s);
  if (e != hipSuccess) return e;
  if (a.lv.count > kInBlockLevels) {
    hipLaunchKernelGGL((pyramid_top_kernel<D>), dim3(a.batch * a.n_kv_heads), dim3(1024), 0, s, a);
    e = launched(s);
  }
  return e;
}

hipError_t launch_pyramid(const PyramidArgs& a, hipStream_t s) {
  if (a.bf16) return a.head_dim == 64 ? launch_pyramid_t<__bf16, 64>(a, s) : launch_pyramid_t<__bf16, 128>(a, s);
  return a.head_dim == 64 ? launch_pyramid_t<float, 64>(a, s) : launch_pyramid_t<float, 128>(a, s);
}

}  // namespace pisa
