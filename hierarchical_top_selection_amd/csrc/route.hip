// route.hip - Stage 1 of hierarchical selection: top-down routing through the
// pyramid levels above the leaves (Core method eq. 16-21; Method steps eq. 22 of
// "Block Sparse Attention with Log-Linear Complexity").
//
// One wave routes one (b, kvh, token).  The candidates' children are gathered 16
// at a time as the rows of an MFMA A tile and the group's G query heads are the
// columns of the B tile (columns >= G are zero), so one MFMA pass yields the
// logits of every head against 16 children, and a candidate's two children land
// in the same lane.  Candidate lists never leave registers: lane
// i owns candidate i, a level keeps K of them by exact rank (score descending,
// node index ascending) and the survivors expand into the next list with a
// ballot/bit-select compaction.  The leaf candidates (at most 2K per token) are
// the only output.
//
// Scores need full single precision (near-ties between candidates are common),
// so the summaries stay float32 and the products run on v_mfma_f32_16x16x4_f32
// (bf16 queries are widened exactly).  The kernel is bound by gathering summary
// rows (8 KB per 16-child tile), so each tile's rows are requested one tile
// ahead.  (Splitting each summary into three bf16 terms would cut the MFMA
// cycles fivefold but gathers 1.5x the bytes, and measured slower.)  The LSE of
// a candidate's two children is evaluated in base 2 as max + log2(1 + 2^-|diff|)
// on pre-scaled logits.
#include "kernels.h"

namespace pisa {

template <typename T, int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void route_kernel(RouteArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.n) return;
  const int bh = blockIdx.y;
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int g = lane >> 4, col = lane & 15;
  const int width = 2 * a.top_k;
  const float c2 = a.scale * 1.4426950408889634f;       // logits in base-2 units

  FragF32<D> qf;
  if (col < a.group) {
    const T* qrow = reinterpret_cast<const T*>(a.q) + b * a.q_sb + (int64_t)t * a.q_st +
                    (int64_t)(kvh * a.group + col) * a.q_sh;
    qf.load(qrow, g);
  } else {
    qf.zero();
  }
  const float* pyr = a.pyr + (int64_t)bh * a.lv.nodes * D;

  int cand = lane == 0 ? 0 : -1;                       // A^(L) = {root}
  for (int level = a.lv.count; level >= 2; --level) {
    const uint64_t valid = __ballot(cand >= 0);
    const int n_valid = __popcll(valid);
    const int child_size = a.lv.size[level - 2];
    const int64_t child_off = a.lv.offset[level - 2];
    bool keep = cand >= 0;
    if (n_valid > a.top_k) {
      const int span = 64 - __clzll(valid);            // highest occupied lane + 1
      const int tiles = (2 * span + 15) / 16;
      // child of tile nt owned by this lane's row index: candidate slot/2, child slot&1.  Rows of
      // invalid children load a clamped row and are masked.
      auto child_of = [&](int nt, bool& ok) {
        const int slot = 16 * nt + col;
        const int parent = __shfl(cand, slot >> 1, 64);
        const int child = 2 * parent + (slot & 1);
        ok = parent >= 0 && child < child_size && node_first_key(level - 1, child) <= t;
        return ok ? child : 0;
      };
      float u = kNegInf;                               // score of candidate `lane` (base 2)
      bool ok_n;
      int child_n = child_of(0, ok_n);
      FragF32<D> kf_n;
      kf_n.load(pyr + (child_off + child_n) * D, g);
      for (int nt = 0; nt < tiles; ++nt) {
        const FragF32<D> kf = kf_n;
        // validity of the children this lane holds results for: rows 4g .. 4g+3 of the tile
        const uint64_t okmask = __ballot(ok_n);
        if (nt + 1 < tiles) {                          // next tile's rows in flight during this one
          child_n = child_of(nt + 1, ok_n);
          kf_n.load(pyr + (child_off + child_n) * D, g);
        }
        // S^T tile: rows = 16 children, columns = heads; lane (g, col) gets children 4g + i of head col
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma(kf, qf, acc);
        float pair_score[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {                  // candidate 8 nt + 2g + h: children rows 4g + 2h, +1
          const int r0 = 4 * g + 2 * h;
          const float z0 = ((okmask >> r0) & 1) ? acc[2 * h] * c2 : kNegInf;
          const float z1 = ((okmask >> (r0 + 1)) & 1) ? acc[2 * h + 1] * c2 : kNegInf;
          const float m = fmaxf(z0, z1);
          const float sc = m == kNegInf ? kNegInf
                                        : m + __builtin_amdgcn_logf(1.f + __builtin_amdgcn_exp2f(fminf(z0, z1) - m));
          pair_score[h] = row_sum_to_last(col < a.group ? sc : 0.f);   // sum over the group's heads
        }
        // lane 16 g + 15 holds candidates 8 nt + 2 g and 8 nt + 2 g + 1
        const int src = 16 * ((lane & 7) >> 1) + 15;
        const float s0 = __shfl(pair_score[0], src, 64);
        const float s1 = __shfl(pair_score[1], src, 64);
        if ((lane >> 3) == nt) u = (lane & 1) ? s1 : s0;
      }
      int rank = 0;
      for (int j = 0; j < span; ++j) {
        const float uj = __shfl(u, j, 64);
        const int cj = __shfl(cand, j, 64);
        rank += (cj >= 0) && (uj > u || (uj == u && cj < cand));
      }
      keep = cand >= 0 && rank < a.top_k;
    }
    // expand the survivors into their causally valid children
    const uint64_t kept = __ballot(keep);
    const int m = __popcll(kept);
    const int p = lane >> 1;
    const int src = nth_set_bit(kept, p < m ? p : 0);
    const int parent = __shfl(cand, src, 64);
    const int child = 2 * parent + (lane & 1);
    cand = (p < m && child < child_size && node_first_key(level - 1, child) <= t) ? child : -1;
  }
  if (lane < width) a.cand[((int64_t)bh * a.n + t) * width + lane] = cand;
}

template <typename T, int D>
hipError_t launch_route_t(const RouteArgs& a, hipStream_t s) {
  dim3 grid(ceil_div(a.n, 4), a.batch * a.n_kv_heads);
  hipLaunchKernelGGL((route_kernel<T, D>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.bf16) return a.head_dim == 64 ? launch_route_t<__bf16, 64>(a, s) : launch_route_t<__bf16, 128>(a, s);
  return a.head_dim == 64 ? launch_route_t<float, 64>(a, s) : launch_route_t<float, 128>(a, s);
}

}  // namespace pisa
