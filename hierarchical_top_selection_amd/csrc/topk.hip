// topk.hip - final top-K over the exact leaf scores (Method steps, Stage 2's separate
// top-K kernel of "Block Sparse Attention with Log-Linear Complexity").
//
// One wave per (b, kvh, token); lane i owns candidate slot i (2K <= 64).  A
// candidate survives when fewer than K valid candidates beat it by (score
// descending, leaf index ascending); survivors are written in ascending leaf
// order and the rest of the K slots get -1.
#include "kernels.h"

namespace pisa {

__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.n) return;
  const int64_t row = (int64_t)blockIdx.y * a.n + t;
  int c = -1;
  float u = kNegInf;
  if (lane < a.width) {
    c = a.cand[row * a.width + lane];
    if (c >= 0) u = a.leaf_u[row * a.width + lane];
  }
  const int n_valid = __popcll(__ballot(c >= 0));
  bool keep = c >= 0;
  if (n_valid > a.top_k) {
    int rank = 0;
    for (int j = 0; j < a.width; ++j) {
      const float uj = __shfl(u, j, 64);
      const int cj = __shfl(c, j, 64);
      rank += (cj >= 0) && (uj > u || (uj == u && cj < c));
    }
    keep = keep && rank < a.top_k;
  }
  const uint64_t kept = __ballot(keep);
  const int m = __popcll(kept);
  int pos = 0;
  for (int j = 0; j < a.width; ++j) {
    const int cj = __shfl(c, j, 64);
    pos += (int)((kept >> j) & 1ull) & (cj < c);
  }
  int32_t* sel = a.sel + row * a.top_k;
  float* sel_u = a.sel_u ? a.sel_u + row * a.top_k : nullptr;
  if (keep) {
    sel[pos] = c;
    if (sel_u) sel_u[pos] = u;
  }
  if (lane >= m && lane < a.top_k) {
    sel[lane] = -1;
    if (sel_u) sel_u[lane] = kNegInf;
  }
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  dim3 grid(ceil_div(a.n, 4), a.batch * a.n_kv_heads);
  hipLaunchKernelGGL(topk_kernel, grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pisa
