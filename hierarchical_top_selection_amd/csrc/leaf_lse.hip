// leaf_lse.hip - Stage 2 of hierarchical selection: exact leaf scores (Method steps,
// Stage 2; Core method eq. 21 at the leaf level; Method steps eq. 22 head sum of
// "Block Sparse Attention with Log-Linear Complexity").
//
// Leaf-major: a wave walks a few work items (each one leaf of one token window,
// at most kPairsPerItem queries).  The leaf's 64 keys are loaded once into MFMA
// A fragments held in registers (bf16: 64 VGPRs at d = 128) and reused by every
// query of the item; each query streams in only its G head rows (the B tile).
// bf16 inputs read both from packed copies (K blocks with keys in perm_key order,
// query groups; pack.hip) so every fragment load is one contiguous run.  The product is kept transposed, S^T = K Q^T
// (keys on rows, heads on columns), so a lane owns 16 keys of one head: the
// per-head max and sum over the 64 keys are in-lane plus two cross-group
// shuffles, and exp2/log2 run on pre-scaled logits.  The group's head sum is a
// 16-lane reduction; one lane writes the pair's score.  The mean and mean + var/2 score
// variants (PISA-1 / PISA-2) reduce the same logits to their mean and variance instead.  bf16 inputs use
// v_mfma_f32_16x16x32_bf16 (exact products, fp32 sums); fp32 inputs
// v_mfma_f32_16x16x4_f32.
#include "kernels.h"

namespace pisa {

// Blocks are mapped to windows XCD by XCD: workgroup L runs on XCD L % 8, and XCD x
// walks windows x, x + 8, x + 16, ... so one window's query rows stay in one L2.
constexpr int kXcds = 8;

constexpr int kItemsPerWave = 4;

template <typename T, int D>
__device__ inline void leaf_pair(const typename RawFrag<T, D>::type (&kf)[4], const typename RawFrag<T, D>::type& qf,
                                 int packed, const LeafArgs& a, int start, int last, float c2, bool head_ok,
                                 int g, int lane, float* uout) {
  const int t = packed >> 6, slot = packed & 63;
  floatx4 acc[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) {
    acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
    acc[mt] = mma(kf[mt], qf, acc[mt]);
  }
  // acc[mt][r]: key start + key_off(mt, r) against head column col (packed bf16 blocks hold
  // keys in perm_key order, fp32 keys are in order).  Keys past min(t, n - 1) are left out;
  // `last` is n - 1 - start capped at 63.
  auto key_off = [&](int mt, int r) {
    return sizeof(T) == 2 ? 32 * (mt >> 1) + 8 * g + 4 * (mt & 1) + r : 16 * mt + 4 * g + r;
  };
  const int lim = min(t - start, last);
  float head;                                           // this head's score, natural units
  if (a.score == 0) {                                   // LSE
    if (lim < kLeaf - 1) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (key_off(mt, r) > lim) acc[mt][r] = kNegInf;
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
    // natural-log LSE: (m c2 + log2 s) ln 2; s >= 1, so the raw log2 needs no fix-up
    head = (mc + __builtin_amdgcn_logf(s)) * 0.6931471805599453f;
  } else {                                              // mean, or mean + var / 2, of the valid logits
    const float cnt = (float)(min(lim, kLeaf - 1) + 1);
    float s1 = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) s1 += key_off(mt, r) <= lim ? acc[mt][r] : 0.f;
    s1 = wave_add_xor(s1, 16);
    s1 = wave_add_xor(s1, 32);
    const float mean = s1 / cnt;                        // of the raw dot products
    head = mean * a.scale;
    if (a.score == 2) {
      float s2 = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float dv = (acc[mt][r] - mean) * a.scale;
          s2 += key_off(mt, r) <= lim ? dv * dv : 0.f;
        }
      s2 = wave_add_xor(s2, 16);
      s2 = wave_add_xor(s2, 32);
      head += 0.5f * s2 / cnt;
    }
  }
  const float u = row_sum_to_last(head_ok ? head : 0.f);
  if (lane == 15) uout[(int64_t)t * a.width + slot] = u;   // the group's head sum (row 0)
}

// Each wave walks kItemsPerWave consecutive items of one window.  The next item's
// record and query list are fetched one item ahead, the query rows one query ahead
// (across item boundaries), and consecutive items of the same leaf keep their keys.
// fp32 keys at d = 128 need 128 VGPRs of fragments: no occupancy target there.
template <typename T, int D, int kWaves = (sizeof(T) == 4 && D == 128) ? 1 : 3>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWaves))) void leaf_lse_kernel(LeafArgs a) {
  typedef typename RawFrag<T, D>::type Frag;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int blocks_per_window = ceil_div(a.item_cap, 4 * kItemsPerWave);
  const int xcd = blockIdx.x % kXcds, slot_id = blockIdx.x / kXcds;
  const int64_t wid = (int64_t)kXcds * (slot_id / blocks_per_window) + xcd;   // bh * n_windows + w
  if (wid >= (int64_t)a.batch * a.n_kv_heads * a.n_windows) return;
  const int it0 = ((slot_id % blocks_per_window) * 4 + wave) * kItemsPerWave;
  const int it_end = min(it0 + kItemsPerWave, a.n_items[wid]);
  if (it0 >= it_end) return;
  const int bh = (int)(wid / a.n_windows), w = (int)(wid % a.n_windows);
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int g = lane >> 4, col = lane & 15;
  const int2* items = a.items + wid * a.item_cap;
  const int32_t* pairs = a.pairs + ((int64_t)bh * a.n + (int64_t)w * a.window) * a.width;
  const T* kbase = reinterpret_cast<const T*>(a.k) + b * a.k_sb + kvh * a.k_sh;
  const T* qbase = reinterpret_cast<const T*>(a.q) + b * a.q_sb + (int64_t)(kvh * a.group + col) * a.q_sh;
  float* uout = a.leaf_u + (int64_t)bh * a.n * a.width;
  const float c2 = a.scale * 1.4426950408889634f;      // logits in base-2 units
  const bool head_ok = col < a.group;

  auto item_pairs = [&](int2 rec) {
    const int np = rec.y >> 20, p0 = rec.y & 0xfffff;
    return lane < np ? pairs[p0 + lane] : 0;
  };
  const int64_t qp_token = (int64_t)a.group * D / 8;                  // packed query pieces per token
  const bf16x8* qpack = a.qpack + (int64_t)bh * a.n * qp_token + g * a.group + col;
  auto load_q = [&](Frag& f, int packed) {
    if (!head_ok) {
      f.zero();
    } else if constexpr (sizeof(T) == 2) {
      const bf16x8* p = qpack + (int64_t)(packed >> 6) * qp_token;
#pragma unroll
      for (int s = 0; s < D / 32; ++s) f.v[s] = p[4 * s * a.group];
    } else {
      f.load(qbase + (int64_t)(packed >> 6) * a.q_st, g);
    }
  };

  int2 rec = items[it0];
  int2 rec_n = it0 + 1 < it_end ? items[it0 + 1] : make_int2(-1, 0);
  int pr = item_pairs(rec);
  int pr_n = it0 + 1 < it_end ? item_pairs(rec_n) : 0;
  Frag kf[4];
  int cur_leaf = -1;
  Frag q0, q1;
  load_q(q0, __builtin_amdgcn_readfirstlane(pr));
  for (int it = it0; it < it_end; ++it) {
    const int leaf = rec.x, np = rec.y >> 20;
    const int2 rec_nn = it + 2 < it_end ? items[it + 2] : make_int2(-1, 0);
    if (leaf != cur_leaf) {                            // rows past the end are zero or clamped, then masked
      if constexpr (sizeof(T) == 2) {
        const bf16x8* blk = a.kpack + ((int64_t)bh * a.n_leaves + leaf) * (kLeaf * D / 8) + lane;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int s = 0; s < D / 32; ++s) kf[mt].v[s] = blk[(mt * (D / 32) + s) * 64];
      } else {
        const int64_t first = (int64_t)leaf * kLeaf;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) kf[mt].load(kbase + min(first + 16 * mt + col, (int64_t)a.n - 1) * a.k_st, g);
      }
      cur_leaf = leaf;
    }
    const int start = leaf * kLeaf;
    const int last = min(kLeaf - 1, a.n - 1 - start);   // last key of this leaf, relative to its start
    for (int i = 0; i < np; ++i) {
      // rows of the following query (this item's next, or the next item's first)
      const bool in_item = i + 1 < np;
      const bool have_next = in_item || it + 1 < it_end;
      // lane broadcasts of the uniform pair index: scalar reads, no LDS round trip
      const int nxt = in_item ? __builtin_amdgcn_readlane(pr, i + 1) : __builtin_amdgcn_readfirstlane(pr_n);
      if (have_next) load_q(q1, nxt);
      leaf_pair<T, D>(kf, q0, __builtin_amdgcn_readlane(pr, i), a, start, last, c2, head_ok, g, lane, uout);
      q0 = q1;
    }
    if (it + 1 < it_end) {
      rec = rec_n;
      pr = pr_n;
      rec_n = rec_nn;
      pr_n = it + 2 < it_end ? item_pairs(rec_n) : 0;
    }
  }
}

template <typename T, int D>
hipError_t launch_leaf_t(const LeafArgs& a, hipStream_t s) {
  const int64_t windows = (int64_t)a.batch * a.n_kv_heads * a.n_windows;
  const int64_t blocks = kXcds * ((windows + kXcds - 1) / kXcds) * ceil_div(a.item_cap, 4 * kItemsPerWave);
  hipLaunchKernelGGL((leaf_lse_kernel<T, D>), dim3((unsigned)blocks), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_leaf_lse(const LeafArgs& a, hipStream_t s) {
  if (a.bf16) return a.head_dim == 64 ? launch_leaf_t<__bf16, 64>(a, s) : launch_leaf_t<__bf16, 128>(a, s);
  return a.head_dim == 64 ? launch_leaf_t<float, 64>(a, s) : launch_leaf_t<float, 128>(a, s);
}

}  // namespace pisa
