// topk.hip - final top-K over the exact leaf scores (Method steps, Stage 2's separate
// top-K kernel of "Block Sparse Attention with Log-Linear Complexity").
//
// Lane i of a row owns candidate slot i.  With 2K <= 32 a wave takes two rows (tokens t and
// t + 1 of one (b, kvh)), one per 32-lane half, and runs both rows' searches side by side;
// otherwise (2K <= 64) one row.  The K best candidates by (score descending, leaf index
// ascending) survive, found with a ballot search for the K-th score; survivors are written in
// ascending leaf order and the rest of the K slots get -1.
#include "kernels.h"

namespace pisa {

namespace {

// keep_top_k on each 32-lane half of the wave separately: the K-th largest key of each half as the
// largest threshold that at least k lanes of the half reach, every lane above it kept and the lowest
// lanes equal to it filling the places that remain.
__device__ inline bool keep_top_k_halves(uint32_t khi, int k, int lane) {
  uint32_t thr_lo = 0, thr_hi = 0;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t trial_lo = thr_lo | (1u << bit), trial_hi = thr_hi | (1u << bit);
    const uint64_t reach = __ballot(khi >= (lane < 32 ? trial_lo : trial_hi));
    if (__popc((uint32_t)reach) >= k) thr_lo = trial_lo;
    if (__popc((uint32_t)(reach >> 32)) >= k) thr_hi = trial_hi;
  }
  const uint32_t thr = lane < 32 ? thr_lo : thr_hi;
  const uint64_t ties = __ballot(khi == thr), above = __ballot(khi > thr);
  const uint32_t ties_lo = (uint32_t)ties, ties_hi = (uint32_t)(ties >> 32);
  const int need = k - __popc(lane < 32 ? (uint32_t)above : (uint32_t)(above >> 32));
  // ties in lower lanes of the same half
  const int before = (int)__builtin_amdgcn_mbcnt_hi(ties_hi, __builtin_amdgcn_mbcnt_lo(ties_lo, 0u)) -
                     (lane < 32 ? 0 : __popc(ties_lo));
  return khi > thr || (khi == thr && before < need);
}

}  // namespace

__global__ __launch_bounds__(256) void topk_kernel(TopkArgs a) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const bool two = a.width <= 32;                     // wave-uniform: two rows per wave
  const int half = two ? lane >> 5 : 0;
  const int slot = two ? lane & 31 : lane;
  const int t0 = (blockIdx.x * 4 + wave) * (two ? 2 : 1);
  if (t0 >= a.n) return;
  const int t = t0 + half;
  const bool row_ok = t < a.n;                        // the second row of the last wave may be past n
  const int64_t row = (int64_t)blockIdx.y * a.n + t;
  int c = -1;
  float u = kNegInf;
  if (row_ok && slot < a.width) {
    c = a.cand[row * a.width + slot];
    if (c >= 0) u = a.leaf_u[row * a.width + slot];
  }
  // The leaf candidates of a row are the lowest slots, in ascending leaf order (routing expands its
  // survivors in order and only the last one can lose its second child), so slot order is index
  // order: ties go to the lower slot, and a survivor's output position is the number of survivors
  // in lower slots of its row.
  const uint64_t valid = __ballot(c >= 0);
  bool best;
  if (two) {
    const int n_valid = __popc(half ? (uint32_t)(valid >> 32) : (uint32_t)valid);
    const bool any_full = __popc((uint32_t)valid) > a.top_k || __popc((uint32_t)(valid >> 32)) > a.top_k;
    best = true;
    if (any_full) {                                     // uniform branch; both halves search
      const bool kth = keep_top_k_halves(score_key(u, c >= 0), a.top_k, lane);
      best = n_valid > a.top_k ? kth : true;
    }
  } else {
    const int n_valid = __popcll(valid);
    best = n_valid > a.top_k ? keep_top_k(score_key(u, c >= 0), a.top_k) : true;   // uniform branch
  }
  const bool keep = c >= 0 && best;
  const uint64_t kept = __ballot(keep);
  const uint32_t kept_lo = (uint32_t)kept, kept_hi = (uint32_t)(kept >> 32);
  const int m = two ? __popc(half ? kept_hi : kept_lo) : __popcll(kept);
  const int pos = (int)__builtin_amdgcn_mbcnt_hi(kept_hi, __builtin_amdgcn_mbcnt_lo(kept_lo, 0u)) -
                  (half ? __popc(kept_lo) : 0);
  if (!row_ok) return;
  int32_t* sel = a.sel + row * a.top_k;
  float* sel_u = a.sel_u ? a.sel_u + row * a.top_k : nullptr;
  if (keep) {
    sel[pos] = c;
    if (sel_u) sel_u[pos] = u;
  }
  if (slot >= m && slot < a.top_k) {
    sel[slot] = -1;
    if (sel_u) sel_u[slot] = kNegInf;
  }
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  const int rows_per_block = a.width <= 32 ? 8 : 4;
  dim3 grid(ceil_div(a.n, rows_per_block), a.batch * a.n_kv_heads);
  hipLaunchKernelGGL(topk_kernel, grid, dim3(256), 0, s, a);
  return launched(s);
}

}  // namespace pisa
