// leaf_lse.hip - Stage 2 of hierarchical selection: exact leaf scores (Method steps,
// Stage 2; Core method eq. 21 at the leaf level; Method steps eq. 22 head sum of
// "Block Sparse Attention with Log-Linear Complexity").
//
// Leaf-major: a wave owns one leaf of one token window.  The leaf's 64 keys are
// loaded once into MFMA B fragments held in registers (bf16: 64 VGPRs at
// d = 128) and reused by every query of the window that has the leaf as a
// candidate; each such query streams in only its G head rows (the A tile).
// Per pair: 16 x 64 logits, per-head LSE over the keys at positions <= t, and
// the sum over the group's heads, written to the pair's (token, slot).
// bf16 inputs use v_mfma_f32_16x16x32_bf16 (exact products, fp32 sums); fp32
// inputs use v_mfma_f32_16x16x4_f32.
#include "kernels.h"

namespace pisa {

template <typename T, int D>
__global__ __launch_bounds__(256) void leaf_lse_kernel(LeafArgs a) {
  typedef typename RawFrag<T, D>::type Frag;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int leaf = blockIdx.x * 4 + wave;
  const int w = blockIdx.y, bh = blockIdx.z;
  if (leaf >= a.n_leaves) return;
  const int32_t* off = a.leaf_off + ((int64_t)bh * a.n_windows + w) * (a.n_leaves + 1);
  const int p0 = off[leaf], p1 = off[leaf + 1];
  if (p0 >= p1) return;
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int g = lane >> 4, col = lane & 15;

  const T* kbase = reinterpret_cast<const T*>(a.k) + b * a.k_sb + kvh * a.k_sh;
  Frag kf[4];
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int64_t key = (int64_t)leaf * kLeaf + 16 * nt + col;
    if (key < a.n) kf[nt].load(kbase + key * a.k_st, g); else kf[nt].zero();
  }
  const int32_t* pairs = a.pairs + ((int64_t)bh * a.n + (int64_t)w * a.window) * a.width;
  const T* qbase = reinterpret_cast<const T*>(a.q) + b * a.q_sb + (int64_t)(kvh * a.group + col) * a.q_sh;
  float* uout = a.leaf_u + (int64_t)bh * a.n * a.width;
  const int64_t leaf_first = (int64_t)leaf * kLeaf;

  for (int p = p0; p < p1; ++p) {
    const int packed = pairs[p];
    const int t = packed >> 6, slot = packed & 63;
    Frag qf;
    if (col < a.group) qf.load(qbase + (int64_t)t * a.q_st, g); else qf.zero();
    floatx4 acc[4];
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      acc[nt] = floatx4{0.f, 0.f, 0.f, 0.f};
      acc[nt] = mma(qf, kf[nt], acc[nt]);
    }
    // acc[nt][i]: head 4g+i against key leaf_first + 16 nt + col
    float u = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float z[4];
      float m = kNegInf;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int64_t key = leaf_first + 16 * nt + col;
        z[nt] = (key <= t && key < a.n) ? acc[nt][i] * a.scale : kNegInf;
        m = fmaxf(m, z[nt]);
      }
      m = wave_max_xor(m, 1); m = wave_max_xor(m, 2); m = wave_max_xor(m, 4); m = wave_max_xor(m, 8);
      float s = 0.f;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) s += expf(z[nt] - m);
      s = wave_add_xor(s, 1); s = wave_add_xor(s, 2); s = wave_add_xor(s, 4); s = wave_add_xor(s, 8);
      if (4 * g + i < a.group) u += m + logf(s);
    }
    u = wave_add_xor(u, 16);
    u = wave_add_xor(u, 32);
    if (lane == 0) uout[(int64_t)t * a.width + slot] = u;
  }
}

template <typename T, int D>
hipError_t launch_leaf_t(const LeafArgs& a, hipStream_t s) {
  dim3 grid(ceil_div(a.n_leaves, 4), a.n_windows, a.batch * a.n_kv_heads);
  hipLaunchKernelGGL((leaf_lse_kernel<T, D>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_leaf_lse(const LeafArgs& a, hipStream_t s) {
  if (a.bf16) return a.head_dim == 64 ? launch_leaf_t<__bf16, 64>(a, s) : launch_leaf_t<__bf16, 128>(a, s);
  return a.head_dim == 64 ? launch_leaf_t<float, 64>(a, s) : launch_leaf_t<float, 128>(a, s);
}

}  // namespace pisa
