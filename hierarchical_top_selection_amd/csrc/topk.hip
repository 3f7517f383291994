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
  const int n_valid = __popcll(__ballot(c >= 0));
  bool keep = c >= 0;
  if (n_valid > a.top_k) {
    // rank by (score descending, leaf ascending) as one 64-bit key: the score's bits made
    // order-preserving above the complemented leaf index; empty slots are 0, below every
    // candidate.  Lane j's key is read into scalar registers.
    const uint32_t ubits = __builtin_bit_cast(uint32_t, u + 0.f);          // -0 compares as +0
    const uint32_t khi = c >= 0 ? ((ubits & 0x80000000u) ? ~ubits : (ubits | 0x80000000u)) : 0u;
    const uint32_t klo = c >= 0 ? 0xffffffffu - (uint32_t)c : 0u;
    const uint64_t key = ((uint64_t)khi << 32) | klo;
    int rank = 0;
    for (int j = 0; j < a.width; ++j) {
      const uint64_t kj = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(khi, j) << 32) |
                          (uint64_t)(uint32_t)__builtin_amdgcn_readlane(klo, j);
      rank += (int)(kj > key);
    }
    keep = keep && rank < a.top_k;
  }
  const uint64_t kept = __ballot(keep);
  const int m = __popcll(kept);
  int pos = 0;                                          // kept candidates with a lower leaf index
  for (int j = 0; j < a.width; ++j) {
    const int cj = __builtin_amdgcn_readlane(c, j);
    pos += (int)(((kept >> j) & 1ull) != 0 && cj < c);
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
  return launched(s);
}

}  // namespace pisa
