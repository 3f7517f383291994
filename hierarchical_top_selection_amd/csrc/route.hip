// route.hip - Stage 1 of hierarchical selection: top-down routing through the
// pyramid levels above the leaves (Core method eq. 16-21; Method steps eq. 22 of
// "Block Sparse Attention with Log-Linear Complexity").
//
// One wave routes one (b, kvh, token).  The G query heads of the group are the
// 16 rows of an fp32 MFMA A tile (rows >= G are zero); the candidates' children
// are gathered 16 at a time as the B tile, so one MFMA pass yields the logits of
// every head against 16 children.  Candidate lists never leave registers: lane
// i owns candidate i, a level keeps K of them by exact rank (score descending,
// node index ascending) and the survivors expand into the next list with a
// ballot/bit-select compaction.  The leaf candidates (at most 2K per token) are
// the only output.  The pyramid is float32 and the products are fp32 MFMA, so
// the scores carry full single precision.
#include "kernels.h"

namespace pisa {

template <typename T, int D>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.n) return;
  const int bh = blockIdx.y;
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int g = lane >> 4, col = lane & 15;
  const int width = 2 * a.top_k;

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
    const float* child_base = pyr + a.lv.offset[level - 2] * D;
    bool keep = cand >= 0;
    if (n_valid > a.top_k) {
      const int span = 64 - __clzll(valid);            // highest occupied lane + 1
      const int tiles = (2 * span + 15) / 16;
      float u = kNegInf;                               // score of candidate `lane`
      for (int nt = 0; nt < tiles; ++nt) {
        const int slot = 16 * nt + col;                // child slot: candidate slot/2, child slot&1
        const int parent = __shfl(cand, slot >> 1, 64);
        const int child = 2 * parent + (slot & 1);
        const bool ok = parent >= 0 && child < child_size && node_first_key(level - 1, child) <= t;
        FragF32<D> kf;
        if (ok) kf.load(child_base + (int64_t)child * D, g); else kf.zero();
        floatx4 acc = {0.f, 0.f, 0.f, 0.f};
        acc = mma(qf, kf, acc);
        // rows 4g+i are heads, column col is this child; pair children 2c, 2c+1 are lanes col, col^1
        float head_sum = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float z = ok ? acc[i] * a.scale : kNegInf;
          const float zp = __shfl_xor(z, 1, 64);
          const float m = fmaxf(z, zp);
          const float s = m == kNegInf ? kNegInf : m + logf(expf(z - m) + expf(zp - m));
          if (4 * g + i < a.group) head_sum += s;
        }
        head_sum += __shfl_xor(head_sum, 16, 64);
        head_sum += __shfl_xor(head_sum, 32, 64);
        // lane 2c of any group now holds candidate 8 nt + c's score
        const float got = __shfl(head_sum, 2 * (lane & 7), 64);
        if ((lane >> 3) == nt) u = got;
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
