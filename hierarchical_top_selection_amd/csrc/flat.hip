// flat.hip - single-level block selection of the block-sparse framework (Prerequisites:
// block sparse attention and top-K block selection; grouped-query attention) of "Block
// Sparse Attention with Log-Linear Complexity": every causally valid leaf j of a query
// token t is scored by q . k_bar_j / sqrt(d) against the leaf's mean key, the group's
// heads share the selection by summing their scores, and K leaves are kept by (score
// descending, index ascending).  This is the O(N^2 / C) scan that the hierarchical
// routing replaces; it is built as the baseline that routing is measured against.
//
// The head sum is linear, so sum_h q_h . k_bar = (sum_h q_h) . k_bar: the scores of a
// 16-token group against a 16-leaf tile are one fp32 S^T = K_bar Q_sum^T MFMA tile
// (v_mfma_f32_16x16x4_f32).  Two packing passes write the summed queries and the leaf
// means in MFMA fragment order (whole-line loads).  One wave owns 16 tokens: lane
// (g, col) receives leaves 16 T + 4 g + i of token col, keeps a running top-K over that
// quarter of the leaves, and the four quarters are merged at the end.
#include "kernels.h"

namespace pisa {

namespace {

constexpr int kFlatMaxK = 16;

// (u, j) ranks before (u2, j2): higher score, then lower index.
__device__ inline bool flat_better(float u, int j, float u2, int j2) { return u > u2 || (u == u2 && j < j2); }

}  // namespace

// Summed query heads of each 16-token group in fragment order: piece m of group grp holds, in
// lane (g, col), elements 16 m + 4 g .. + 3 of token 16 grp + col (zero past n).
template <typename T, int D>
__global__ __launch_bounds__(256) void flat_qsum_kernel(FlatArgs a) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;     // (bh, grp, m, lane)
  const int groups = ceil_div(a.n, 16);
  const int64_t per_bh = (int64_t)groups * (D / 16) * 64;
  if (e >= (int64_t)a.batch * a.n_kv_heads * per_bh) return;
  const int bh = (int)(e / per_bh);
  const int64_t r = e % per_bh;
  const int lane = (int)(r % 64), m = (int)((r / 64) % (D / 16));
  const int grp = (int)(r / (64 * (D / 16)));
  const int g = lane >> 4, col = lane & 15;
  const int t = 16 * grp + col;
  float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
  if (t < a.n) {
    const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
    const T* row = reinterpret_cast<const T*>(a.q) + b * a.q_sb + (int64_t)t * a.q_st +
                   (int64_t)kvh * a.group * a.q_sh + 16 * m + 4 * g;
    for (int h = 0; h < a.group; ++h) {                                // heads in order
      const float4 v = load4(row + (int64_t)h * a.q_sh);
      s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
    }
  }
  a.qsum[e] = s;
}

// Leaf means of level 1 in 16-leaf tiles, same fragment order (zero past M_1).
template <int D>
__global__ __launch_bounds__(256) void flat_kpack_kernel(FlatArgs a) {
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;     // (bh, tile, m, lane)
  const int m1 = ceil_div(a.n, kLeaf);
  const int tiles = ceil_div(m1, 16);
  const int64_t per_bh = (int64_t)tiles * (D / 16) * 64;
  if (e >= (int64_t)a.batch * a.n_kv_heads * per_bh) return;
  const int bh = (int)(e / per_bh);
  const int64_t r = e % per_bh;
  const int lane = (int)(r % 64), m = (int)((r / 64) % (D / 16));
  const int tile = (int)(r / (64 * (D / 16)));
  const int g = lane >> 4, col = lane & 15;
  const int j = 16 * tile + col;
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  if (j < m1) v = load4(a.pyr + ((int64_t)bh * a.nodes + j) * D + 16 * m + 4 * g);
  a.kpack[e] = v;
}

template <int D>
__global__ __launch_bounds__(256) void flat_select_kernel(FlatArgs a) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int grp = blockIdx.x * 4 + wave;                               // 16-token group
  const int t0 = 16 * grp;
  if (t0 >= a.n) return;
  const int bh = blockIdx.y;
  const int g = lane >> 4, col = lane & 15;
  const int m1 = ceil_div(a.n, kLeaf);
  const int jmax = t0 / kLeaf;                     // the same for the group's 16 tokens (16 | 64)
  const int tiles_bh = ceil_div(m1, 16);
  const int K = a.top_k;

  FragF32<D> qf;                                   // B: columns = the group's tokens
  const float4* qp = a.qsum + ((int64_t)bh * ceil_div(a.n, 16) + grp) * (D / 16) * 64 + lane;
#pragma unroll
  for (int m = 0; m < D / 16; ++m) qf.v[m] = qp[m * 64];
  const float4* kp = a.kpack + (int64_t)bh * tiles_bh * (D / 16) * 64 + lane;

  // running top-K of this lane's quarter of the leaves (entries >= K stay empty)
  float lu[kFlatMaxK];
  int lj[kFlatMaxK];
#pragma unroll
  for (int e = 0; e < kFlatMaxK; ++e) { lu[e] = kNegInf; lj[e] = 0x7fffffff; }
  float wu = kNegInf;                              // the worst kept entry
  int wj = 0x7fffffff, wpos = 0;
  auto insert = [&](float u, int j) {
#pragma unroll
    for (int e = 0; e < kFlatMaxK; ++e)
      if (e == wpos) { lu[e] = u; lj[e] = j; }
    wu = lu[0]; wj = lj[0]; wpos = 0;
#pragma unroll
    for (int e = 1; e < kFlatMaxK; ++e)
      if (e < K && flat_better(wu, wj, lu[e], lj[e])) { wu = lu[e]; wj = lj[e]; wpos = e; }
  };

  const int ntiles = jmax / 16 + 1;
  FragF32<D> kf;
#pragma unroll
  for (int m = 0; m < D / 16; ++m) kf.v[m] = kp[m * 64];
  for (int tile = 0; tile < ntiles; ++tile) {
    const FragF32<D> cur = kf;
    if (tile + 1 < ntiles) {                       // next tile in flight while this one is ranked
#pragma unroll
      for (int m = 0; m < D / 16; ++m) kf.v[m] = kp[((tile + 1) * (D / 16) + m) * 64];
    }
    const floatx4 acc = mma(cur, qf, floatx4{0.f, 0.f, 0.f, 0.f});
    // acc[i]: leaf 16 tile + 4 g + i against token t0 + col
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 16 * tile + 4 * g + i;
      const float u = acc[i] * a.scale;
      if (j <= jmax && flat_better(u, j, wu, wj)) insert(u, j);
    }
  }

  // merge the four quarters of each token into lane group 0
#pragma unroll
  for (int src = 1; src < 4; ++src) {
#pragma unroll
    for (int e = 0; e < kFlatMaxK; ++e) {
      const float u = __shfl(lu[e], col + 16 * src, 64);
      const int j = __shfl(lj[e], col + 16 * src, 64);
      if (g == 0 && e < K && j != 0x7fffffff && flat_better(u, j, wu, wj)) insert(u, j);
    }
  }
  // ascending leaf order (odd-even transposition over the fixed register slots)
#pragma unroll
  for (int pass = 0; pass < kFlatMaxK; ++pass)
#pragma unroll
    for (int e = pass & 1; e + 1 < kFlatMaxK; e += 2)
      if (lj[e] > lj[e + 1]) {
        const float tu = lu[e]; lu[e] = lu[e + 1]; lu[e + 1] = tu;
        const int tj = lj[e]; lj[e] = lj[e + 1]; lj[e + 1] = tj;
      }
  const int t = t0 + col;
  if (g == 0 && t < a.n) {
    int32_t* out = a.sel + ((int64_t)bh * a.n + t) * K;
    float* out_u = a.sel_u ? a.sel_u + ((int64_t)bh * a.n + t) * K : nullptr;
#pragma unroll
    for (int e = 0; e < kFlatMaxK; ++e)
      if (e < K) {
        const bool ok = lj[e] != 0x7fffffff;
        out[e] = ok ? lj[e] : -1;
        if (out_u) out_u[e] = ok ? lu[e] : kNegInf;
      }
  }
}

template <typename T, int D>
hipError_t launch_flat_t(const FlatArgs& a, hipStream_t s) {
  const int64_t bhs = (int64_t)a.batch * a.n_kv_heads;
  const int64_t q_threads = bhs * ceil_div(a.n, 16) * (D / 16) * 64;
  hipLaunchKernelGGL((flat_qsum_kernel<T, D>), dim3((unsigned)((q_threads + 255) / 256)), dim3(256), 0, s, a);
  hipError_t e = launched(s);
  if (e != hipSuccess) return e;
  const int64_t k_threads = bhs * ceil_div(ceil_div(a.n, kLeaf), 16) * (D / 16) * 64;
  hipLaunchKernelGGL((flat_kpack_kernel<D>), dim3((unsigned)((k_threads + 255) / 256)), dim3(256), 0, s, a);
  if ((e = launched(s)) != hipSuccess) return e;
  hipLaunchKernelGGL((flat_select_kernel<D>), dim3(ceil_div(ceil_div(a.n, 16), 4), (unsigned)bhs), dim3(256), 0, s, a);
  return launched(s);
}

hipError_t launch_flat(const FlatArgs& a, hipStream_t s) {
  if (a.bf16) return a.head_dim == 64 ? launch_flat_t<__bf16, 64>(a, s) : launch_flat_t<__bf16, 128>(a, s);
  return a.head_dim == 64 ? launch_flat_t<float, 64>(a, s) : launch_flat_t<float, 128>(a, s);
}

}  // namespace pisa
