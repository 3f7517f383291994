// pack.hip - packed 64-key blocks of bf16 K and V (the leaf blocks of "Block Sparse
// Attention with Log-Linear Complexity", Prerequisites: block sparse attention).
//
// The Stage-2 leaf scoring and the block-sparse attention gather whole 64-key
// blocks into MFMA fragments.  Loaded straight from the [B][N][H][d] tensors, one
// fragment load touches 16 rows x 64 bytes, i.e. 16 half-used cache lines, and the
// vector L1 serves such loads at about a third of the rate of loads that cover whole
// lines.  One pass over K (and V) rewrites every block so that each fragment is a
// contiguous 1 KB run in lane order (layout documented with PackArgs).
#include "kernels.h"

namespace pisa {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// One workgroup per (block j, b * Hkv + kvh): the block's rows are staged in LDS, then
// every thread writes whole 16-byte pieces.
template <int D>
__global__ __launch_bounds__(256) void pack_blocks_kernel(PackArgs a) {
  constexpr int kRowPad = D + 8;                  // bf16 elements per staged row
  __shared__ __align__(16) __bf16 ks[kLeaf][kRowPad];
  __shared__ __align__(16) __bf16 vs[kLeaf][kRowPad];
  const int j = blockIdx.x, bh = blockIdx.y;
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const bool with_v = a.v != nullptr;
  const __bf16* kbase = reinterpret_cast<const __bf16*>(a.k) + b * a.k_sb + kvh * a.k_sh;
  const __bf16* vbase = reinterpret_cast<const __bf16*>(a.v) + b * a.v_sb + kvh * a.v_sh;
  const int64_t first = (int64_t)j * kLeaf;
  for (int e = threadIdx.x; e < kLeaf * D / 8; e += blockDim.x) {
    const int r = e / (D / 8), c8 = e % (D / 8);
    const int64_t key = first + r;
    const bool in = key < a.n;
    const u32x4 zero = {0u, 0u, 0u, 0u};         // native vector type: stays in registers
    *reinterpret_cast<u32x4*>(&ks[r][8 * c8]) = in ? *reinterpret_cast<const u32x4*>(kbase + key * a.k_st + 8 * c8) : zero;
    if (with_v)
      *reinterpret_cast<u32x4*>(&vs[r][8 * c8]) = in ? *reinterpret_cast<const u32x4*>(vbase + key * a.v_st + 8 * c8) : zero;
  }
  __syncthreads();
  const int m1 = ceil_div(a.n, kLeaf);
  const int64_t blk = ((int64_t)bh * m1 + j) * (kLeaf * D / 8);
  for (int e = threadIdx.x; e < kLeaf * D / 8; e += blockDim.x) {
    const int piece = e / 64, l = e % 64;
    const int g = l >> 4, col = l & 15;
    // K piece (mt, s)
    const int mt = piece / (D / 32), s = piece % (D / 32);
    a.kpack[blk + e] = *reinterpret_cast<const bf16x8*>(&ks[perm_key(mt, col)][32 * s + 8 * g]);
    if (with_v) {
      // V piece (kb, dt)
      const int kb = piece / (D / 16), dt = piece % (D / 16);
      bf16x8 out;
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = vs[32 * kb + 8 * g + i][16 * dt + col];
      a.vpack[blk + e] = out;
    }
  }
}

hipError_t launch_pack(const PackArgs& a, hipStream_t s) {
  const dim3 grid(ceil_div(a.n, kLeaf), a.batch * a.n_kv_heads);
  if (a.head_dim == 64)
    hipLaunchKernelGGL(pack_blocks_kernel<64>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(pack_blocks_kernel<128>, grid, dim3(256), 0, s, a);
  return launched(s);
}

}  // namespace pisa
