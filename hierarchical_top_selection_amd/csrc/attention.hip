// attention.hip - causal attention over the raw K/V of the selected leaf blocks
// (Prerequisites, block sparse attention; Method steps, fourth step of "Block
// Sparse Attention with Log-Linear Complexity").
//
// One wave per (b, kvh, token): the group's G <= 16 query heads are the 16
// columns of every MFMA.  Per selected block the wave forms S^T = K_j Q^T
// (keys on rows, heads on columns, K rows streamed from HBM straight into A
// fragments), updates an online softmax per head column, and accumulates
// O^T += V_j^T P^T.  Keeping S transposed makes P^T's B fragment exactly the
// lane's own accumulator values; only V has to be read transposed, which the
// wave does from a private, bank-padded LDS stage (32 keys at a time for bf16,
// 16 for fp32).  bf16 inputs run on v_mfma_f32_16x16x32_bf16 with P rounded to
// bf16 for the PV product; fp32 inputs on v_mfma_f32_16x16x4_f32.
#include <type_traits>

#include "kernels.h"

namespace pisa {

template <typename T, typename TO, int D>
__global__ __launch_bounds__(256) void attention_kernel(AttnArgs a) {
  typedef typename RawFrag<T, D>::type Frag;
  constexpr bool kBF = std::is_same<T, __bf16>::value;
  constexpr int kChunk = kBF ? 32 : 16;     // keys staged per LDS round
  constexpr int kPad = kBF ? 8 : 4;         // row padding (elements): conflict-free transposed reads
  constexpr int kVec = 16 / sizeof(T);      // elements per 16-byte load
  constexpr int kRowVecs = D / kVec;
  __shared__ __align__(16) T vstage[4][kChunk][D + kPad];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.n) return;
  const int bh = blockIdx.y;
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int g = lane >> 4, col = lane & 15;
  T (*vs)[D + kPad] = vstage[wave];

  const int head = kvh * a.group + col;
  Frag qf;
  if (col < a.group) qf.load(reinterpret_cast<const T*>(a.q) + b * a.q_sb + (int64_t)t * a.q_st + (int64_t)head * a.q_sh, g);
  else qf.zero();
  const T* kbase = reinterpret_cast<const T*>(a.k) + b * a.k_sb + kvh * a.k_sh;
  const T* vbase = reinterpret_cast<const T*>(a.v) + b * a.v_sb + kvh * a.v_sh;
  const int32_t* sel = a.sel + ((int64_t)bh * a.n + t) * a.top_k;

  floatx4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  for (int s = 0; s < a.top_k; ++s) {
    const int j = sel[s];
    if (j < 0) continue;
    const int64_t first = (int64_t)j * kLeaf;
    floatx4 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      const int64_t key = first + 16 * mt + col;
      Frag kf;
      if (key < a.n) kf.load(kbase + key * a.k_st, g); else kf.zero();
      acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      acc[mt] = mma(kf, qf, acc[mt]);
    }
    // acc[mt][i]: key first + 16 mt + 4 g + i against head column col
    float tile_max = kNegInf;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t key = first + 16 * mt + 4 * g + i;
        const float z = (key <= t && key < a.n) ? acc[mt][i] * a.scale : kNegInf;
        acc[mt][i] = z;
        tile_max = fmaxf(tile_max, z);
      }
    tile_max = wave_max_xor(tile_max, 16);
    tile_max = wave_max_xor(tile_max, 32);
    if (tile_max == kNegInf) continue;   // block holds no key <= t (masking is per key, so wave-uniform)
    const float m_new = fmaxf(m_run, tile_max);
    const float alpha = expf(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = expf(acc[mt][i] - m_new);
        acc[mt][i] = p;
        psum += p;
      }
    psum = wave_add_xor(psum, 16);
    psum = wave_add_xor(psum, 32);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;

#pragma unroll
    for (int ch = 0; ch < kLeaf / kChunk; ++ch) {
      for (int e = lane; e < kChunk * kRowVecs; e += 64) {
        const int r = e / kRowVecs, cv = e % kRowVecs;
        const int64_t key = first + ch * kChunk + r;
        uint4 val = make_uint4(0u, 0u, 0u, 0u);
        if (key < a.n) val = *reinterpret_cast<const uint4*>(vbase + key * a.v_st + cv * kVec);
        *reinterpret_cast<uint4*>(&vs[r][cv * kVec]) = val;
      }
      wave_lds_sync();
      if constexpr (kBF) {
        // k-index j of lane group g: keys 4g+j (j < 4) and 16+4g+j-4 (j >= 4) of this chunk
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pb[i] = (__bf16)acc[2 * ch][i];
          pb[4 + i] = (__bf16)acc[2 * ch + 1][i];
        }
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          bf16x8 av;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            av[i] = vs[4 * g + i][16 * dt + col];
            av[4 + i] = vs[16 + 4 * g + i][16 * dt + col];
          }
          o[dt] = mfma_bf16(av, pb, o[dt]);
        }
      } else {
        // chunk = key tile ch; k-step i: lane group g supplies key 4g+i
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[dt] = mfma_f32(to_f32(vs[4 * g + i][16 * dt + col]), acc[ch][i], o[dt]);
      }
      wave_lds_sync();
    }
  }

  if (col < a.group) {
    const float inv = 1.f / l_run;
    TO* orow = reinterpret_cast<TO*>(a.o) + b * a.o_sb + (int64_t)t * a.o_st + (int64_t)head * a.o_sh;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) orow[16 * dt + 4 * g + i] = from_f32<TO>(o[dt][i] * inv);
    if (a.row_lse && g == 0) {
      const int hq = a.n_kv_heads * a.group;
      a.row_lse[((int64_t)b * hq + head) * a.n + t] = m_run + logf(l_run);
    }
  }
}

template <typename T, typename TO, int D>
hipError_t launch_attention_t(const AttnArgs& a, hipStream_t s) {
  dim3 grid(ceil_div(a.n, 4), a.batch * a.n_kv_heads);
  hipLaunchKernelGGL((attention_kernel<T, TO, D>), grid, dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, typename TO>
hipError_t launch_attention_o(const AttnArgs& a, hipStream_t s) {
  return a.head_dim == 64 ? launch_attention_t<T, TO, 64>(a, s) : launch_attention_t<T, TO, 128>(a, s);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  if (a.bf16) return a.out_bf16 ? launch_attention_o<__bf16, __bf16>(a, s) : launch_attention_o<__bf16, float>(a, s);
  return a.out_bf16 ? launch_attention_o<float, __bf16>(a, s) : launch_attention_o<float, float>(a, s);
}

}  // namespace pisa
