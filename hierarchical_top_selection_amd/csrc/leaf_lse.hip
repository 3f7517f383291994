// leaf_lse.hip - Stage 2 of hierarchical selection: exact leaf scores (Method steps,
// Stage 2; Core method eq. 21 at the leaf level; Method steps eq. 22 head sum of
// "Block Sparse Attention with Log-Linear Complexity").
//
// Leaf-major: a wave takes one work item (one leaf of one token window, at most
// kPairsPerItem queries).  The leaf's 64 keys are loaded once into MFMA A
// fragments held in registers (bf16: 64 VGPRs at d = 128) and reused by every
// query of the item; each query streams in only its G head rows (the B tile),
// prefetched three queries ahead.  The product is kept transposed, S^T = K Q^T
// (keys on rows, heads on columns), so a lane owns 16 keys of one head: the
// per-head max and sum over the 64 keys are in-lane plus two cross-group
// shuffles, and exp2/log2 run on pre-scaled logits.  The group's head sum is a
// 16-lane reduction; lane 0 writes the pair's score.  bf16 inputs use
// v_mfma_f32_16x16x32_bf16 (exact products, fp32 sums); fp32 inputs
// v_mfma_f32_16x16x4_f32.
#include "kernels.h"

namespace pisa {

// Blocks are mapped to windows XCD by XCD: workgroup L runs on XCD L % 8, and XCD x
// walks windows x, x + 8, x + 16, ... so one window's query rows stay in one L2.
constexpr int kXcds = 8;

template <typename T, int D>
__device__ inline void leaf_pair(const typename RawFrag<T, D>::type (&kf)[4], const typename RawFrag<T, D>::type& qf,
                                 int packed, const LeafArgs& a, int64_t leaf_first, bool edge_leaf, float c2,
                                 bool head_ok, int g, int lane, float* uout) {
  const int t = packed >> 6, slot = packed & 63;
  floatx4 acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    acc[mt] = mma(kf[mt], qf, acc[mt]);
  }
  // acc[mt][r]: key leaf_first + 16 mt + 4 g + r against head column col
  if (leaf_first + kLeaf - 1 > t || edge_leaf) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t key = leaf_first + 16 * mt + 4 * g + r;
        if (key > t || key >= a.n) acc[mt][r] = kNegInf;
      }
  }
  float m = kNegInf;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) m = fmaxf(m, acc[mt][r]);
  m = wave_max_xor(m, 16);
  m = wave_max_xor(m, 32);
  const float mc = m * c2;
  float s = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) s += __builtin_amdgcn_exp2f(fmaf(acc[mt][r], c2, -mc));   // arguments <= 0
  s = wave_add_xor(s, 16);
  s = wave_add_xor(s, 32);
  // natural-log LSE of this head: (m c2 + log2 s) ln 2
  float u = head_ok ? (mc + __builtin_amdgcn_logf(s)) * 0.6931471805599453f : 0.f;   // s >= 1: no denormal fix-up needed
  u = wave_add_xor(u, 1);
  u = wave_add_xor(u, 2);
  u = wave_add_xor(u, 4);
  u = wave_add_xor(u, 8);
  if (lane == 0) uout[(int64_t)t * a.width + slot] = u;
}

template <typename T, int D>
__global__ __launch_bounds__(256) void leaf_lse_kernel(LeafArgs a) {
  typedef typename RawFrag<T, D>::type Frag;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int blocks_per_window = ceil_div(a.item_cap, 4);
  const int xcd = blockIdx.x % kXcds, slot_id = blockIdx.x / kXcds;
  const int64_t wid = (int64_t)kXcds * (slot_id / blocks_per_window) + xcd;   // bh * n_windows + w
  if (wid >= (int64_t)a.batch * a.n_kv_heads * a.n_windows) return;
  const int item = (slot_id % blocks_per_window) * 4 + wave;
  if (item >= a.n_items[wid]) return;
  const int bh = (int)(wid / a.n_windows), w = (int)(wid % a.n_windows);
  const int code = a.items[wid * a.item_cap + item];
  const int leaf = code & 0xffff, chunk = code >> 16;
  const int32_t* off = a.leaf_off + wid * (a.n_leaves + 1);
  const int p0 = off[leaf] + chunk * kPairsPerItem;
  const int np = min(kPairsPerItem, off[leaf + 1] - p0);
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int g = lane >> 4, col = lane & 15;

  const T* kbase = reinterpret_cast<const T*>(a.k) + b * a.k_sb + kvh * a.k_sh;
  const int64_t leaf_first = (int64_t)leaf * kLeaf;
  Frag kf[4];                                          // rows past the end are clamped, then masked
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) kf[mt].load(kbase + min(leaf_first + 16 * mt + col, (int64_t)a.n - 1) * a.k_st, g);
  const int32_t* pairs = a.pairs + ((int64_t)bh * a.n + (int64_t)w * a.window) * a.width;
  const int my_pair = lane < np ? pairs[p0 + lane] : 0;
  const T* qbase = reinterpret_cast<const T*>(a.q) + b * a.q_sb + (int64_t)(kvh * a.group + col) * a.q_sh;
  float* uout = a.leaf_u + (int64_t)bh * a.n * a.width;
  const float c2 = a.scale * 1.4426950408889634f;      // logits in base-2 units
  const bool head_ok = col < a.group;
  const bool edge_leaf = leaf_first + kLeaf > a.n;     // last, partial leaf

  // query rows of pair i, prefetched three pairs ahead through a ring of four fragments
  auto load_q = [&](Frag& f, int i) {
    if (i < np) {
      const int t = __shfl(my_pair, i, 64) >> 6;
      if (head_ok) f.load(qbase + (int64_t)t * a.q_st, g); else f.zero();
    }
  };
  Frag q0, q1, q2, q3;
  load_q(q0, 0);
  load_q(q1, 1);
  load_q(q2, 2);
  for (int i = 0; i < np; i += 4) {
    load_q(q3, i + 3);
    leaf_pair<T, D>(kf, q0, __shfl(my_pair, i, 64), a, leaf_first, edge_leaf, c2, head_ok, g, lane, uout);
    if (i + 1 >= np) break;
    load_q(q0, i + 4);
    leaf_pair<T, D>(kf, q1, __shfl(my_pair, i + 1, 64), a, leaf_first, edge_leaf, c2, head_ok, g, lane, uout);
    if (i + 2 >= np) break;
    load_q(q1, i + 5);
    leaf_pair<T, D>(kf, q2, __shfl(my_pair, i + 2, 64), a, leaf_first, edge_leaf, c2, head_ok, g, lane, uout);
    if (i + 3 >= np) break;
    load_q(q2, i + 6);
    leaf_pair<T, D>(kf, q3, __shfl(my_pair, i + 3, 64), a, leaf_first, edge_leaf, c2, head_ok, g, lane, uout);
  }
}

template <typename T, int D>
hipError_t launch_leaf_t(const LeafArgs& a, hipStream_t s) {
  const int64_t windows = (int64_t)a.batch * a.n_kv_heads * a.n_windows;
  const int64_t blocks = kXcds * ((windows + kXcds - 1) / kXcds) * ceil_div(a.item_cap, 4);
  hipLaunchKernelGGL((leaf_lse_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_leaf_lse(const LeafArgs& a, hipStream_t s) {
  if (a.bf16) return a.head_dim == 64 ? launch_leaf_t<__bf16, 64>(a, s) : launch_leaf_t<__bf16, 128>(a, s);
  return a.head_dim == 64 ? launch_leaf_t<float, 64>(a, s) : launch_leaf_t<float, 128>(a, s);
}

}  // namespace pisa
