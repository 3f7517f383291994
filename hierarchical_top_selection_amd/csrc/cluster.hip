// cluster.hip - inverse index for Stage 2 (Method steps, Stage 2 of "Block Sparse
// Attention with Log-Linear Complexity"): the queries that must score the same
// leaf are grouped so the leaf's 64 keys are loaded once and reused.
//
// One workgroup per (b, kvh, window of tokens) runs a counting sort of the
// window's (token, slot) leaf candidates by leaf id entirely in LDS:
// histogram -> exclusive scan -> scatter.  Output per window: the pairs grouped
// by leaf (packed t << 6 | slot, stored in the window's own slot range) and the
// M1 + 1 leaf offsets.  The order of pairs inside one leaf is not fixed (LDS
// atomics); every pair's score is computed independently, so results do not
// depend on it.  Windows keep each leaf kernel's query rows cache-resident.
#include "kernels.h"

namespace pisa {

constexpr int kClusterThreads = 1024;

__global__ __launch_bounds__(kClusterThreads) void cluster_kernel(ClusterArgs a) {
  extern __shared__ int lds[];
  const int M = a.n_leaves;
  int* cnt = lds;                  // M counters, then cursors
  int* wave_sum = lds + M;         // kClusterThreads / 64 entries
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int w = blockIdx.x, bh = blockIdx.y;
  const int t0 = w * a.window;
  const int t1 = min(a.n, t0 + a.window);
  const int items = (t1 - t0) * a.width;
  const int32_t* cand = a.cand + ((int64_t)bh * a.n + t0) * a.width;
  int32_t* pairs = a.pairs + ((int64_t)bh * a.n + t0) * a.width;
  int32_t* off = a.leaf_off + ((int64_t)bh * a.n_windows + w) * (M + 1);

  for (int i = tid; i < M; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  for (int i = tid; i < items; i += blockDim.x) {
    const int leaf = cand[i];
    if (leaf >= 0) atomicAdd(&cnt[leaf], 1);
  }
  __syncthreads();

  // exclusive scan: each thread owns a contiguous run of counters
  const int per = (M + blockDim.x - 1) / blockDim.x;
  const int lo = min(M, tid * per), hi = min(M, lo + per);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += cnt[i];
  int incl = local;
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int nw = blockDim.x / 64;
    int v = lane < nw ? wave_sum[lane] : 0;
    int inc = v;
    for (int o = 1; o < 64; o <<= 1) {
      const int x = __shfl_up(inc, o, 64);
      if (lane >= o) inc += x;
    }
    if (lane < nw) wave_sum[lane] = inc - v;
  }
  __syncthreads();
  int run = incl - local + wave_sum[wave];
  for (int i = lo; i < hi; ++i) {
    const int c = cnt[i];
    cnt[i] = run;
    off[i] = run;
    run += c;
  }
  if (tid == blockDim.x - 1) off[M] = run;
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
  const size_t lds = (size_t)(a.n_leaves + kClusterThreads / 64) * sizeof(int);
  dim3 grid(a.n_windows, a.batch * a.n_kv_heads);
  hipLaunchKernelGGL(cluster_kernel, grid, dim3(kClusterThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace pisa
