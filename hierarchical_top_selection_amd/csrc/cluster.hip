// cluster.hip - inverse index for Stage 2 (Method steps, Stage 2 of "Block Sparse
// Attention with Log-Linear Complexity"): the queries that must score the same
// leaf are grouped so the leaf's 64 keys are loaded once and reused.
//
// One workgroup per (b, kvh, window of tokens) runs a counting sort of the
// window's (token, slot) leaf candidates by leaf id entirely in LDS:
// histogram -> exclusive scan -> scatter.  Output per window: the pairs grouped
// by leaf (packed t << 6 | slot, stored in the window's own slot range), the
// M1 + 1 leaf offsets, and the list of work items {leaf, first pair | count << 20},
// each covering at most kPairsPerItem pairs of one leaf.  The order of pairs inside
// one leaf is not fixed (LDS atomics); every pair's score is computed
// independently, so results do not depend on it.
#include "kernels.h"

namespace pisa {

constexpr int kClusterThreads = 1024;

__global__ __launch_bounds__(kClusterThreads) void cluster_kernel(ClusterArgs a) {
  extern __shared__ int lds[];
  const int M = a.n_leaves;
  int* cnt = lds;                  // M counters, then cursors
  int* wave_sum = lds + M;         // 2 x kClusterThreads / 64 entries
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = blockDim.x / 64;
  const int w = blockIdx.x, bh = blockIdx.y;
  const int t0 = w * a.window;
  const int t1 = min(a.n, t0 + a.window);
  const int items = (t1 - t0) * a.width;
  const int32_t* cand = a.cand + ((int64_t)bh * a.n + t0) * a.width;
  int32_t* pairs = a.pairs + ((int64_t)bh * a.n + t0) * a.width;
  const int64_t wid = (int64_t)bh * a.n_windows + w;
  int32_t* off = a.leaf_off + wid * (M + 1);
  int2* work = a.items + wid * a.item_cap;

  for (int i = tid; i < M; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  for (int i = tid; i < items; i += blockDim.x) {
    const int leaf = cand[i];
    if (leaf >= 0) atomicAdd(&cnt[leaf], 1);
  }
  __syncthreads();

  // exclusive scans of the pair counts and of the item counts ceil(count / P);
  // each thread owns a contiguous run of leaves
  const int per = (M + blockDim.x - 1) / blockDim.x;
  const int lo = min(M, tid * per), hi = min(M, lo + per);
  int local_p = 0, local_i = 0;
  for (int i = lo; i < hi; ++i) {
    local_p += cnt[i];
    local_i += (cnt[i] + kPairsPerItem - 1) / kPairsPerItem;
  }
  int incl_p = local_p, incl_i = local_i;
  for (int o = 1; o < 64; o <<= 1) {
    const int vp = __shfl_up(incl_p, o, 64);
    const int vi = __shfl_up(incl_i, o, 64);
    if (lane >= o) { incl_p += vp; incl_i += vi; }
  }
  if (lane == 63) { wave_sum[wave] = incl_p; wave_sum[nw + wave] = incl_i; }
  __syncthreads();
  if (wave == 0) {
    const int vp = lane < nw ? wave_sum[lane] : 0;
    const int vi = lane < nw ? wave_sum[nw + lane] : 0;
    int ip = vp, ii = vi;
    for (int o = 1; o < 64; o <<= 1) {
      const int xp = __shfl_up(ip, o, 64);
      const int xi = __shfl_up(ii, o, 64);
      if (lane >= o) { ip += xp; ii += xi; }
    }
    if (lane < nw) { wave_sum[lane] = ip - vp; wave_sum[nw + lane] = ii - vi; }
  }
  __syncthreads();
  int run_p = incl_p - local_p + wave_sum[wave];
  int run_i = incl_i - local_i + wave_sum[nw + wave];
  for (int i = lo; i < hi; ++i) {
    const int c = cnt[i];
    cnt[i] = run_p;
    off[i] = run_p;
    const int nchunks = (c + kPairsPerItem - 1) / kPairsPerItem;
    for (int ch = 0; ch < nchunks; ++ch) {
      const int first = run_p + ch * kPairsPerItem;
      work[run_i + ch] = make_int2(i, first | (min(kPairsPerItem, c - ch * kPairsPerItem) << 20));
    }
    run_p += c;
    run_i += nchunks;
  }
  if (tid == blockDim.x - 1) {
    off[M] = run_p;
    a.n_items[wid] = run_i;
  }
  __syncthreads();

  for (int i = tid; i < items; i += blockDim.x) {
    const int leaf = cand[i];
    if (leaf >= 0) {
      const int pos = atomicAdd(&cnt[leaf], 1);
      pairs[pos] = ((t0 + i / a.width) << 6) | (i % a.width);
    }
  }
}

hipError_t launch_cluster(const ClusterArgs& a, hipStream_t s) {
  const size_t lds = (size_t)(a.n_leaves + 2 * kClusterThreads / 64) * sizeof(int);
  dim3 grid(a.n_windows, a.batch * a.n_kv_heads);
  hipLaunchKernelGGL(cluster_kernel, grid, dim3(kClusterThreads), lds, s, a);
  return launched(s);
}

}  // namespace pisa
