// topk.hip - final top-K over the exact leaf scores (Method steps, Stage 2's separate
// top-K kernel of "Block Sparse Attention with Log-Linear Complexity").
//
// One wave per (b, kvh, token); lane i owns candidate slot i (2K <= 64).  The
// K best candidates by (score descending, leaf index ascending) survive, found
// with a ballot search for the K-th score; survivors are written in ascending
// leaf order and the rest of the K slots get -1.
#include "kernels.h"

namespace pisa {

__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.n) return;
  const int64_t row = (int64_t)blockIdx.y * a.n + t;
  int c = -1;
  float u = kNegInf;
  if (lane < a.width) {
    c = a.cand[row * a.width + lane];
    if (c >= 0) u = a.leaf_u[row * a.width + lane];
  }
  // The leaf candidates of a row are the lowest slots, in ascending leaf order (routing expands its
  // survivors in order and only the last one can lose its second child), so slot order is index
  // order: ties go to the lower slot, and a survivor's output position is the number of survivors
  // in lower slots.
  const int n_valid = __popcll(__ballot(c >= 0));
  const bool best = n_valid > a.top_k ? keep_top_k(score_key(u, c >= 0), a.top_k) : true;   // uniform branch
  const bool keep = c >= 0 && best;
  const uint64_t kept = __ballot(keep);
  const int m = __popcll(kept);
  const int pos = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(kept >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)kept, 0u));
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
  return launched(s);
}

}  // namespace pisa
