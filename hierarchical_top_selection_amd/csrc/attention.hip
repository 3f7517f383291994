// attention.hip - causal attention over the raw K/V of the selected leaf blocks
// (Prerequisites, block sparse attention; Method steps, fourth step of "Block
// Sparse Attention with Log-Linear Complexity").
//
// One wave per (b, kvh, token): the group's G <= 16 query heads are the 16
// columns of every MFMA.  Per selected block the wave forms S^T = K_j Q^T
// (keys on rows, heads on columns, K rows loaded straight into A fragments),
// updates an online softmax per head column (base-2 exponentials on pre-scaled
// logits), and accumulates O^T += V_j^T P^T.  Keeping S transposed makes P^T's
// B fragment exactly the lane's own accumulator values.
//
// The kernel is bound by gathering K/V blocks from memory.  The bf16 path reads
// K and V from packed blocks (one cheap pass over K and V, pack.hip): every MFMA
// fragment, including V^T's and the K rows in the permuted key order that makes
// P^T a lane's own values, is one contiguous 1 KB load straight into registers --
// no LDS at all.  It is software-pipelined one block ahead: as soon as the S^T
// MFMAs have consumed K_j (and the PV MFMAs V_j), the registers are refilled for
// block j+1, so the gather latency overlaps the softmax and MFMA work.  fp32
// inputs take a plain path that stages V through LDS, on v_mfma_f32_16x16x4_f32.
//
// With a float32 output the bf16 path runs in two passes, the even block ids and
// then the odd ones.  The first pass leaves its online-softmax state (o not yet
// normalised in the output row, the running max and sum per head in the
// workspace) and the second resumes from it.  The softmax is order-free, so this
// only changes the order of the fp32 sums.  Each pass gathers from half of the
// blocks, so the hot blocks take half the L2 and more of the other reads hit it.
#include "kernels.h"

namespace pisa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

template <typename TO>
__device__ inline void store4(TO* p, float a, float b, float c, float d);
template <>
__device__ inline void store4<float>(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
template <>
__device__ inline void store4<__bf16>(__bf16* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}

// Online-softmax update of one 64-key block held as acc[mt][r] (key 16 mt + 4 g + r,
// head column of this lane): replaces acc by P (fp32) and returns the rescale factor
// of the running output.  m_run is kept in base-2 units of the scaled logits.
__device__ inline float softmax_block(floatx4 (&acc)[4], float c2, bool mask, int64_t first, int g, int64_t t,
                                      int n, float& m_run, float& l_run) {
  if (mask) {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t key = first + 16 * mt + 4 * g + r;
        if (key > t || key >= n) acc[mt][r] = kNegInf;
      }
  }
  float tmax = kNegInf;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, acc[mt][r]);
  tmax = rows_max(tmax);
  const float m_new = fmaxf(m_run, tmax * c2);
  const float m_use = m_new == kNegInf ? 0.f : m_new;
  const float alpha = exp2f(m_run - m_use);
  float psum = 0.f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = exp2f(fmaf(acc[mt][r], c2, -m_use));
      acc[mt][r] = p;
      psum += p;
    }
  psum = rows_sum(psum);
  l_run = l_run * alpha + psum;
  m_run = m_new;
  return alpha;
}

template <typename TO>
__device__ inline void finish_row(const AttnArgs& a, const floatx4* o, int nd16, float m_run, float l_run, int b,
                                  int64_t t, int head, int g) {
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  TO* orow = reinterpret_cast<TO*>(a.o) + b * a.o_sb + t * a.o_st + (int64_t)head * a.o_sh;
  for (int dt = 0; dt < nd16; ++dt)
    store4<TO>(orow + 16 * dt + 4 * g, o[dt][0] * inv, o[dt][1] * inv, o[dt][2] * inv, o[dt][3] * inv);
  if (a.row_lse && g == 0) {
    const int hq = a.n_kv_heads * a.group;
    a.row_lse[((int64_t)b * hq + head) * a.n + t] = (m_run + log2f(l_run)) * kLn2;
  }
}

}  // namespace

// ----------------------------------------------------------------------------- bf16, pipelined
template <typename TO, int D>
__global__ __launch_bounds__(256, 2) void attention_bf16_kernel(AttnArgs a) {
  typedef FragBF16<D> Frag;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int bh = blockIdx.y;
  int t;
  if (a.ord.order && order_sorted(a.ord.stats)) {
    // the pass's sorted order (order.hip), cut into kXcds contiguous slices: XCD x walks the x-th
    // slice in time order (the grid's x size is a multiple of kXcds)
    const int slice = gridDim.x / kXcds;
    const int pos = ((blockIdx.x % kXcds) * slice + blockIdx.x / kXcds) * 4 + wave;
    if (pos >= a.n) return;
    t = __builtin_amdgcn_readfirstlane(a.ord.order[((int64_t)a.pass * a.ord.bh + bh) * a.n + pos]);
  } else {
    t = blockIdx.x * 4 + wave;
    if (t >= a.n) return;
  }
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int g = lane >> 4, col = lane & 15;
  const int m1 = ceil_div(a.n, kLeaf);

  const int head = kvh * a.group + col;
  Frag qf;
  if (col < a.group)
    qf.load(reinterpret_cast<const __bf16*>(a.q) + b * a.q_sb + (int64_t)t * a.q_st + (int64_t)head * a.q_sh, g);
  else
    qf.zero();
  const bf16x8* kpack = a.kpack + (int64_t)bh * m1 * (kLeaf * D / 8);
  const bf16x8* vpack = a.vpack + (int64_t)bh * m1 * (kLeaf * D / 8);
  const int my_sel = lane < a.top_k ? a.sel[((int64_t)bh * a.n + t) * a.top_k + lane] : -1;
  // The key set is the union of the listed blocks cut to positions <= t: an entry takes part if
  // 0 <= j <= t / 64 (so j < ceil(n / 64) and every gather below stays inside the packed blocks)
  // and no lower slot of the row lists the same id.  With several passes this one takes the
  // blocks j % n_passes == pass.
  bool use = my_sel >= 0 && my_sel <= t / kLeaf;
  for (int i = 0; i < a.top_k; ++i) use = use && !(i < lane && __builtin_amdgcn_readlane(my_sel, i) == my_sel);
  const uint64_t valid = __ballot(use && (a.n_passes == 1 || my_sel % a.n_passes == a.pass));
  const int nsel = __popcll(valid);
  const float c2 = a.scale * kLog2e;

  Frag kf[4];                 // A fragments of S^T = K Q^T, rows in perm_key order
  bf16x8 vf[2][D / 16];       // A fragments of O^T = V^T P^T: [key half][value column tile]
  // keys past the end of the sequence are zero in the packed blocks; their logits are masked
  auto load_k = [&](int leaf) {
    const bf16x8* blk = kpack + (int64_t)leaf * (kLeaf * D / 8) + lane;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int s = 0; s < D / 32; ++s) kf[mt].v[s] = blk[(mt * (D / 32) + s) * 64];
  };
  auto load_v = [&](int leaf) {
    const bf16x8* blk = vpack + (int64_t)leaf * (kLeaf * D / 8) + lane;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) vf[kb][dt] = blk[(kb * (D / 16) + dt) * 64];
  };

  floatx4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;
  // with several passes (float32 output only): this head's output row, which carries o between the
  // passes, and its (m, l) pair
  const bool multi = a.n_passes > 1;
  float* orow = multi ? reinterpret_cast<float*>(a.o) + b * a.o_sb + (int64_t)t * a.o_st + (int64_t)head * a.o_sh
                      : nullptr;
  float* ml = multi ? a.part_ml + (((int64_t)bh * a.n + t) * a.group + col) * 2 : nullptr;
  if (a.pass > 0 && col < a.group) {                   // resume the previous pass's online softmax
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const float4 x = *reinterpret_cast<const float4*>(orow + 16 * dt + 4 * g);
      o[dt] = floatx4{x.x, x.y, x.z, x.w};
    }
    m_run = ml[0];
    l_run = ml[1];
  }

  uint64_t rest = valid;
  int leaf = 0;
  if (rest) {
    leaf = __builtin_amdgcn_readfirstlane(__shfl(my_sel, __builtin_ctzll(rest), 64));
    rest &= rest - 1;
    load_k(leaf);
    load_v(leaf);
  }
  for (int done = 0; done < nsel; ++done) {
    const bool more = rest != 0;
    const int leaf_n = more ? __builtin_amdgcn_readfirstlane(__shfl(my_sel, __builtin_ctzll(rest), 64)) : 0;
    rest &= rest - 1;
    const int64_t first = (int64_t)leaf * kLeaf;

    floatx4 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      acc[mt] = floatx4{0.f, 0.f, 0.f, 0.f};
      acc[mt] = mma(kf[mt], qf, acc[mt]);
    }
    if (more) load_k(leaf_n);                          // K of the next block into the freed fragments

    // acc[mt][r]: key first + perm_key(mt, 4 g + r) against head column col.  Only a block that
    // reaches past t needs a mask; t < n, so that also masks keys past the end.  The key offset
    // 32 (mt / 2) + 8 g + 4 (mt % 2) + r is compared with t - first - 8 g in 32 bits.
    if (first + kLeaf - 1 > t) {
      const int lim = t - (int)first - 8 * g;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (32 * (mt >> 1) + 4 * (mt & 1) + r > lim) acc[mt][r] = kNegInf;
    }
    float tmax = kNegInf;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) tmax = fmaxf(tmax, acc[mt][r]);
    tmax = rows_max(tmax);
    const float m_new = fmaxf(m_run, tmax * c2);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);   // arguments <= 0: no range fix-up needed
    float psum = 0.f;
    bf16x8 pb[2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(fmaf(acc[mt][r], c2, -m_use));
        psum += p;
        pb[mt >> 1][4 * (mt & 1) + r] = (__bf16)p;      // k-index 4 h + r of key half kb = mt / 2
      }
    psum = rows_sum(psum);
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      o[dt] *= alpha;
      o[dt] = mfma_bf16(vf[0][dt], pb[0], o[dt]);
      o[dt] = mfma_bf16(vf[1][dt], pb[1], o[dt]);
    }
    if (more) load_v(leaf_n);                          // V^T of the next block into the freed fragments
    leaf = leaf_n;
  }
  if (col < a.group) {
    if (a.pass + 1 < a.n_passes) {                     // hand the state to the next pass
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) store4<float>(orow + 16 * dt + 4 * g, o[dt][0], o[dt][1], o[dt][2], o[dt][3]);
      if (g == 0) {
        ml[0] = m_run;
        ml[1] = l_run;
      }
    } else {
      finish_row<TO>(a, o, D / 16, m_run, l_run, b, t, head, g);
    }
  }
}

// ----------------------------------------------------------------------------- fp32, plain
template <typename TO, int D>
__global__ __launch_bounds__(256) void attention_f32_kernel(AttnArgs a) {
  typedef FragF32<D> Frag;
  constexpr int kChunk = 16;                    // keys staged per LDS round (one key tile)
  constexpr int kPad = 4;
  constexpr int kRowVecs = D / 4;
  __shared__ __align__(16) float vstage[4][kChunk][D + kPad];

  const int lane = threadIdx.x & 63, wave = wave_id();
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.n) return;
  const int bh = blockIdx.y;
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int g = lane >> 4, col = lane & 15;
  float (*vs)[D + kPad] = vstage[wave];

  const int head = kvh * a.group + col;
  Frag qf;
  if (col < a.group)
    qf.load(reinterpret_cast<const float*>(a.q) + b * a.q_sb + (int64_t)t * a.q_st + (int64_t)head * a.q_sh, g);
  else
    qf.zero();
  const float* kbase = reinterpret_cast<const float*>(a.k) + b * a.k_sb + kvh * a.k_sh;
  const float* vbase = reinterpret_cast<const float*>(a.v) + b * a.v_sb + kvh * a.v_sh;
  const int32_t* sel = a.sel + ((int64_t)bh * a.n + t) * a.top_k;
  const float c2 = a.scale * kLog2e;

  floatx4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  for (int s = 0; s < a.top_k; ++s) {
    const int j = sel[s];
    // union of the listed blocks cut to positions <= t: skip -1, blocks past t and repeats
    if (j < 0 || j > t / kLeaf) continue;
    bool repeat = false;
    for (int s2 = 0; s2 < s; ++s2) repeat = repeat || sel[s2] == j;
    if (repeat) continue;
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
    const bool mask = first + kLeaf - 1 > t || first + kLeaf > a.n;
    const float alpha = softmax_block(acc, c2, mask, first, g, t, a.n, m_run, l_run);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] *= alpha;
#pragma unroll
    for (int ch = 0; ch < kLeaf / kChunk; ++ch) {
      for (int e = lane; e < kChunk * kRowVecs; e += 64) {
        const int r = e / kRowVecs, cv = e % kRowVecs;
        const int64_t key = first + ch * kChunk + r;
        float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
        if (key < a.n) val = *reinterpret_cast<const float4*>(vbase + key * a.v_st + cv * 4);
        *reinterpret_cast<float4*>(&vs[r][cv * 4]) = val;
      }
      wave_lds_sync();
      // chunk = key tile ch; k-step r: lane group g supplies key 4g + r
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) o[dt] = mfma_f32(vs[4 * g + r][16 * dt + col], acc[ch][r], o[dt]);
      wave_lds_sync();
    }
  }
  if (col < a.group) finish_row<TO>(a, o, D / 16, m_run, l_run, b, t, head, g);
}

template <typename TO, int D>
hipError_t launch_attention_t(const AttnArgs& a, hipStream_t s) {
  dim3 grid(ceil_div(a.n, 4), a.batch * a.n_kv_heads);
  if (a.bf16) {
    PackArgs p;
    p.k = a.k; p.k_sb = a.k_sb; p.k_st = a.k_st; p.k_sh = a.k_sh;
    p.v = a.v; p.v_sb = a.v_sb; p.v_st = a.v_st; p.v_sh = a.v_sh;
    p.kpack = a.kpack; p.vpack = a.vpack;
    p.batch = a.batch; p.n_kv_heads = a.n_kv_heads; p.head_dim = D; p.n = a.n;
    hipError_t e = launch_pack(p, s);
    if (e != hipSuccess) return e;
    dim3 grid_bf16 = grid;
    if (a.ord.order) {
      if ((e = launch_order(a.ord, s)) != hipSuccess) return e;
      grid_bf16.x = kXcds * ceil_div(grid.x, kXcds);
    }
    for (int pass = 0; pass < a.n_passes; ++pass) {
      AttnArgs ap = a;
      ap.pass = pass;
      hipLaunchKernelGGL((attention_bf16_kernel<TO, D>), grid_bf16, dim3(256), 0, s, ap);
      if ((e = launched(s)) != hipSuccess) return e;
    }
    return hipSuccess;
  }
  hipLaunchKernelGGL((attention_f32_kernel<TO, D>), grid, dim3(256), 0, s, a);
  return launched(s);
}

template <typename TO>
hipError_t launch_attention_o(const AttnArgs& a, hipStream_t s) {
  return a.head_dim == 64 ? launch_attention_t<TO, 64>(a, s) : launch_attention_t<TO, 128>(a, s);
}

hipError_t launch_attention(const AttnArgs& a, hipStream_t s) {
  return a.out_bf16 ? launch_attention_o<__bf16>(a, s) : launch_attention_o<float>(a, s);
}

}  // namespace pisa
