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
// per-head sum over the 64 keys (and the maximum, where the sum needs a shift) is
// in-lane plus two row-swap permutes across the lane groups, and exp2/log2 run on
// pre-scaled logits.  The group's head sum is a
// 16-lane reduction; one lane writes the pair's score.  The mean and mean + var/2 score
// variants (PISA-1 / PISA-2) reduce the same logits to their mean and variance instead; the
// score is a template parameter, so each instantiation carries only its own reduction.  bf16 inputs use
// v_mfma_f32_16x16x32_bf16 (exact products, fp32 sums); fp32 inputs
// v_mfma_f32_16x16x4_f32.
#include "kernels.h"

namespace pisa {

// Blocks are mapped to windows XCD by XCD: workgroup L runs on XCD L % 8 (kXcds), and XCD x
// walks windows x, x + 8, x + 16, ... so one window's query rows stay in one L2.

constexpr int kItemsPerWave = 2;
// a wave's pairs fit two registers per lane, and its items the four-way picks below
static_assert(kItemsPerWave <= 4 && kItemsPerWave * kPairsPerItem <= 128, "wave pair stream too long");

template <typename T, int D, int kScore>
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
  if constexpr (kScore == 0) {                          // LSE
    if (lim < kLeaf - 1) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (key_off(mt, r) > lim) acc[mt][r] = kNegInf;
    }
    // First with no shift: s = sum of 2^(x c2).  When every head's s lies in [2^-60, 2^60], its
    // largest term lies in [2^-66, 2^60]: no term overflowed, the terms that underflowed (below
    // 2^-126) are below 2^-60 of the largest, and log2 s is the base-2 LSE to the rounding of the max-shifted form
    // (whose shift m c2 is rounded the same way as x c2 here).  Otherwise the whole wave redoes the
    // pair with the maximum subtracted first.
    float s = __builtin_amdgcn_exp2f(acc[0][0] * c2);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (mt + r > 0) s += __builtin_amdgcn_exp2f(acc[mt][r] * c2);
    s = rows_sum(s);
    float mc = 0.f;
    if (__ballot(!(s >= 0x1p-60f && s <= 0x1p60f))) {   // wave-uniform
      float m = kNegInf;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, acc[mt][r]);
      m = rows_max(m);
      mc = m * c2;
      s = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) s += __builtin_amdgcn_exp2f(fmaf(acc[mt][r], c2, -mc));   // arguments <= 0
      s = rows_sum(s);
    }
    // natural-log LSE: (m c2 + log2 s) ln 2; s >= 2^-60 (>= 1 after the shift), so the raw log2
    // needs no fix-up for denormals
    head = (mc + __builtin_amdgcn_logf(s)) * 0.6931471805599453f;
  } else {                                              // mean, or mean + var / 2, of the valid logits
    const float cnt = (float)(min(lim, kLeaf - 1) + 1);
    float s1 = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) s1 += key_off(mt, r) <= lim ? acc[mt][r] : 0.f;
    s1 = rows_sum(s1);
    const float mean = s1 / cnt;                        // of the raw dot products
    head = mean * a.scale;
    if constexpr (kScore == 2) {
      float s2 = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float dv = (acc[mt][r] - mean) * a.scale;
          s2 += key_off(mt, r) <= lim ? dv * dv : 0.f;
        }
      s2 = rows_sum(s2);
      head += 0.5f * s2 / cnt;
    }
  }
  const float u = row_sum_to_last(head_ok ? head : 0.f);
  if (lane == 15) uout[(int64_t)t * a.width + slot] = u;   // the group's head sum (row 0)
}

// Each wave walks kItemsPerWave consecutive items of one window as one stream of pairs:
// the query rows are fetched kAhead pairs ahead (across item boundaries), and consecutive
// items of the same leaf keep their keys.  Two pairs ahead at three waves per SIMD suits the
// longer windows of long sequences, whose query rows come from beyond the L2 more often; one
// pair ahead at four waves per SIMD (128 VGPRs) the 512-token windows, whose rows mostly hit
// it (measured: 2.46 -> 2.34 ms at 32K, 3.37 -> 3.49 ms at 256K).
// fp32 keys at d = 128 need 128 VGPRs of fragments: no occupancy target there.
template <typename T, int D, int kScore, int kAhead,
          int kWaves = (sizeof(T) == 4 && D == 128) ? 1 : (kAhead == 2 ? 3 : 4)>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWaves))) void leaf_lse_kernel(LeafArgs a) {
  typedef typename RawFrag<T, D>::type Frag;
  const int lane = threadIdx.x & 63, wave = wave_id();
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
  float* uout = a.leaf_u + (int64_t)bh * a.n * a.width;
  const float c2 = a.scale * 1.4426950408889634f;      // logits in base-2 units
  const bool head_ok = col < a.group;

  const int64_t qp_token = (int64_t)a.group * D / 8;                  // packed query pieces per token
  // Lanes of head columns >= G read column 0's rows instead (finite values; those columns never
  // reach the head sum), so every query load is unconditional and the compiler's wait counts
  // stay exact across the look-ahead below.
  const int qcol = head_ok ? col : 0;
  const bf16x8* qpack = a.qpack + (int64_t)bh * a.n * qp_token + g * a.group + qcol;
  const T* qbase = reinterpret_cast<const T*>(a.q) + b * a.q_sb + (int64_t)(kvh * a.group + qcol) * a.q_sh;
  auto load_q = [&](Frag& f, int packed) {
    if constexpr (sizeof(T) == 2) {
      const bf16x8* p = qpack + (int64_t)(packed >> 6) * qp_token;
#pragma unroll
      for (int s = 0; s < D / 32; ++s) f.v[s] = p[4 * s * a.group];
    } else {
      f.load(qbase + (int64_t)(packed >> 6) * a.q_st, g);
    }
  };

  // The wave's items (at most kItemsPerWave, each 1..kPairsPerItem pairs) as one flat stream of
  // pairs: item j's record in lane j, its pairs at flat positions [off_j, off_j + count_j); lane l
  // holds the pairs at flat positions l and l + 64.
  const int nit = it_end - it0;
  const int2 myrec = lane < nit ? items[it0 + lane] : make_int2(0, 0);
  const int cnt0 = __builtin_amdgcn_readlane(myrec.y >> 20, 0), cnt1 = __builtin_amdgcn_readlane(myrec.y >> 20, 1);
  const int cnt2 = __builtin_amdgcn_readlane(myrec.y >> 20, 2), cnt3 = __builtin_amdgcn_readlane(myrec.y >> 20, 3);
  const int off1 = cnt0, off2 = off1 + cnt1, off3 = off2 + cnt2;
  const int total = __builtin_amdgcn_readfirstlane(off3 + cnt3);
  auto pick = [](int j, int v0, int v1, int v2, int v3) { return j == 0 ? v0 : j == 1 ? v1 : j == 2 ? v2 : v3; };
  const int p00 = __builtin_amdgcn_readlane(myrec.y & 0xfffff, 0), p01 = __builtin_amdgcn_readlane(myrec.y & 0xfffff, 1);
  const int p02 = __builtin_amdgcn_readlane(myrec.y & 0xfffff, 2), p03 = __builtin_amdgcn_readlane(myrec.y & 0xfffff, 3);
  auto flat_pair = [&](int f) {
    if (f >= total) return 0;
    const int j = (f >= off1) + (f >= off2) + (f >= off3);
    return pairs[pick(j, p00, p01, p02, p03) + f - pick(j, 0, off1, off2, off3)];
  };
  const int fl0 = flat_pair(lane), fl1 = flat_pair(lane + 64);
  auto pair_at = [&](int f) {                          // f is wave-uniform: a scalar read
    return f < 64 ? __builtin_amdgcn_readlane(fl0, f) : __builtin_amdgcn_readlane(fl1, f - 64);
  };
  const int leaf0 = __builtin_amdgcn_readlane(myrec.x, 0), leaf1 = __builtin_amdgcn_readlane(myrec.x, 1);
  const int leaf2 = __builtin_amdgcn_readlane(myrec.x, 2), leaf3 = __builtin_amdgcn_readlane(myrec.x, 3);

  Frag kf[4];
  int cur_leaf = -1, start = 0, last = 0;
  int next_item = 0, next_start = 0;                   // the next item to enter and its first flat position
  // Query rows are fetched two pairs ahead through a ring of three fragments (static slots, so
  // the ring stays in registers).  At an item boundary the keys are requested before the
  // look-ahead query, so the wait for them does not include it.
  auto step = [&](int f, Frag& cur, Frag& fill) {
    if (f == next_start) {
      const int leaf = __builtin_amdgcn_readfirstlane(pick(next_item, leaf0, leaf1, leaf2, leaf3));
      if (leaf != cur_leaf) {                          // rows past the end are zero or clamped, then masked
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
      start = leaf * kLeaf;
      last = min(kLeaf - 1, a.n - 1 - start);          // last key of this leaf, relative to its start
      ++next_item;
      next_start = __builtin_amdgcn_readfirstlane(next_item < nit ? pick(next_item, 0, off1, off2, off3) : total);
    }
    load_q(fill, pair_at(min(f + kAhead, total - 1)));   // past the end: a repeat, never used
    leaf_pair<T, D, kScore>(kf, cur, pair_at(f), a, start, last, c2, head_ok, g, lane, uout);
  };
  if constexpr (kAhead == 2) {
    Frag qa, qb, qc;
    load_q(qa, pair_at(0));
    load_q(qb, pair_at(min(1, total - 1)));
    for (int f = 0; f < total; f += 3) {
      step(f, qa, qc);
      if (f + 1 < total) step(f + 1, qb, qa);
      if (f + 2 < total) step(f + 2, qc, qb);
    }
  } else {
    Frag qa, qb;
    load_q(qa, pair_at(0));
    for (int f = 0; f < total; f += 2) {
      step(f, qa, qb);
      if (f + 1 < total) step(f + 1, qb, qa);
    }
  }
}

template <typename T, int D, int kAhead>
void launch_leaf_score(const LeafArgs& a, dim3 grid, hipStream_t s) {
  if (a.score == 1)
    hipLaunchKernelGGL((leaf_lse_kernel<T, D, 1, kAhead>), grid, dim3(256), 0, s, a);
  else if (a.score == 2)
    hipLaunchKernelGGL((leaf_lse_kernel<T, D, 2, kAhead>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((leaf_lse_kernel<T, D, 0, kAhead>), grid, dim3(256), 0, s, a);
}

template <typename T, int D>
hipError_t launch_leaf_t(const LeafArgs& a, hipStream_t s) {
  const int64_t windows = (int64_t)a.batch * a.n_kv_heads * a.n_windows;
  const int64_t blocks = kXcds * ((windows + kXcds - 1) / kXcds) * ceil_div(a.item_cap, 4 * kItemsPerWave);
  const dim3 grid((unsigned)blocks);
  if (a.window > 512)
    launch_leaf_score<T, D, 2>(a, grid, s);
  else
    launch_leaf_score<T, D, 1>(a, grid, s);
  return launched(s);
}

hipError_t launch_leaf_lse(const LeafArgs& a, hipStream_t s) {
  if (a.bf16) return a.head_dim == 64 ? launch_leaf_t<__bf16, 64>(a, s) : launch_leaf_t<__bf16, 128>(a, s);
  return a.head_dim == 64 ? launch_leaf_t<float, 64>(a, s) : launch_leaf_t<float, 128>(a, s);
}

}  // namespace pisa
