// attention_bwd.hip - gradients of the block-sparse attention of "Block Sparse Attention
// with Log-Linear Complexity" (Prerequisites, block sparse attention; Method steps,
// fourth step) with the selected sets held fixed.  The page calls the method trainable but
// states no gradient; the selection is piecewise constant in q and k, so only the
// attention over the selected keys is differentiated.  For token t, head h and key r of
// its selected blocks (r <= t), with P = softmax(scale q . k_r) and upstream dO:
//   dV_r += P_r dO,  dP_r = dO . v_r,  Delta = dO . O,  dS_r = P_r (dP_r - Delta),
//   dq = scale sum_r dS_r k_r,  dk_r += scale dS_r q.
//
// Two passes over the (token, block) pairs, both bf16 MFMA with fp32 accumulation:
//
// * dq, query-major: one wave per (b, kvh, token), the group's heads as the 16 MFMA
//   columns, exactly the shape of the forward kernel.  Per selected block it forms
//   S^T = K Q^T and dP^T = V dO^T from packed key-major rows, rescales with the saved row
//   LSE (no online softmax: P is final), and accumulates dq^T += K^T dS^T with the lane's own
//   dS^T values as the B fragment.  K^T comes from the K rows already in registers: an MFMA
//   against a 0/1 selector puts the keys on the result rows, in the order dS^T uses.
// * dk and dv, key-major: a deterministic inverse of the selection lists each block's
//   tokens in ascending order (a stable counting sort: per-chunk occurrence ranks, a
//   per-block scan over chunks, one scan over blocks, a scatter).  A work item is up to
//   512 tokens of one block; its four waves own 16 keys each, copy the tokens' records
//   (bf16 query and output-gradient rows and row statistics, written once per token by a
//   packing pass) into LDS, double-buffered, form S = Q K^T and dP = dO V^T
//   with the heads as rows, and accumulate dv^T += dO^T P and dk^T += Q^T dS on the
//   16x16x16 MFMA, whose contraction runs over the 16 head rows; dO^T and Q^T come from
//   the row fragments by selector MFMAs.  Items write partial
//   sums; a last pass adds each block's partials in item order.  No atomics anywhere, so
//   repeated calls give identical bits.
#include <type_traits>

#include "attention_bwd.h"

namespace pisa {

namespace {

constexpr float kLog2e = 1.4426950408889634f;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ inline floatx4 mfma_k16(bf16x4 a, bf16x4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// Eight consecutive gradient elements as bf16 (p 16-byte aligned for bf16, 32-byte for f32).
__device__ inline bf16x8 load8_bf16(const __bf16* p) { return *reinterpret_cast<const bf16x8*>(p); }
__device__ inline bf16x8 load8_bf16(const float* p) {
  const float4 x = *reinterpret_cast<const float4*>(p), y = *reinterpret_cast<const float4*>(p + 4);
  bf16x8 r;
  r[0] = (__bf16)x.x; r[1] = (__bf16)x.y; r[2] = (__bf16)x.z; r[3] = (__bf16)x.w;
  r[4] = (__bf16)y.x; r[5] = (__bf16)y.y; r[6] = (__bf16)y.z; r[7] = (__bf16)y.w;
  return r;
}

// f(std::integral_constant<int, i>) for i = 0 .. N - 1, unrolled at compile time.
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (N > 0) {
    static_for<N - 1>(f);
    f(std::integral_constant<int, N - 1>{});
  }
}

// Lane < K holds slot `lane` of the token's selection; true for entries that take part:
// a block j with 0 <= j <= t / 64 not listed in an earlier slot.  Called by the whole wave.
__device__ inline bool slot_in_use(int j, int lane, int K, int t) {
  bool ok = lane < K && j >= 0 && j <= t / kLeaf;
  for (int e = 0; e < K; ++e) {
    const int je = __shfl(j, e, 64);
    if (e < lane && je == j) ok = false;
  }
  return ok;
}

}  // namespace

// ----------------------------------------------------------------------------- token records
// One record per (b, kvh, token) (see BwdArgs): the group's query rows and upstream-gradient
// rows in bf16 (dO rounded to nearest-even), and per head (row LSE * log2 e, Delta = dO . O)
// with Delta taken from the unrounded dO; +inf / 0 for the padding heads h >= G, which makes
// their probabilities exactly zero.  One thread per 16-byte piece; a row's pieces are
// adjacent lanes, which reduce Delta among themselves.
template <typename TD, int D>
__global__ __launch_bounds__(256) void bwd_tokens_kernel(BwdArgs a) {
  constexpr int kPieces = D / 8;                     // 16-byte pieces per row
  constexpr int64_t kRec = bwd_record_bytes(D);
  const int t = blockIdx.x;                          // one token per workgroup of 16 * D / 8 threads
  const int h = threadIdx.x / kPieces, p = threadIdx.x % kPieces;
  const int bh = blockIdx.y, b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  bf16x8 qv, dv;
#pragma unroll
  for (int e = 0; e < 8; ++e) { qv[e] = (__bf16)0.f; dv[e] = (__bf16)0.f; }
  float dot = 0.f;
  if (t < a.n && h < a.group) {
    const int head = kvh * a.group + h;
    qv = *reinterpret_cast<const bf16x8*>(reinterpret_cast<const __bf16*>(a.q) + b * a.q_sb +
                                          (int64_t)t * a.q_st + (int64_t)head * a.q_sh + 8 * p);
    const TD* dp = reinterpret_cast<const TD*>(a.dout) + b * a.do_sb + (int64_t)t * a.do_st +
                   (int64_t)head * a.do_sh + 8 * p;
    const TD* op = reinterpret_cast<const TD*>(a.o) + b * a.o_sb + (int64_t)t * a.o_st + (int64_t)head * a.o_sh +
                   8 * p;
    const float4 d0 = load4(dp), d1 = load4(dp + 4), o0 = load4(op), o1 = load4(op + 4);
    dot = d0.x * o0.x + d0.y * o0.y + d0.z * o0.z + d0.w * o0.w + d1.x * o1.x + d1.y * o1.y + d1.z * o1.z +
          d1.w * o1.w;
    dv[0] = (__bf16)d0.x; dv[1] = (__bf16)d0.y; dv[2] = (__bf16)d0.z; dv[3] = (__bf16)d0.w;
    dv[4] = (__bf16)d1.x; dv[5] = (__bf16)d1.y; dv[6] = (__bf16)d1.z; dv[7] = (__bf16)d1.w;
  }
#pragma unroll
  for (int m = 1; m < kPieces; m <<= 1) dot += __shfl_xor(dot, m, 64);     // the row's kPieces lanes
  if (t < a.n) {
    char* rec = a.tok + ((int64_t)bh * a.n + t) * kRec;
    *reinterpret_cast<bf16x8*>(rec + (h * D + 8 * p) * 2) = qv;
    *reinterpret_cast<bf16x8*>(rec + bwd_row_bytes(D) + (h * D + 8 * p) * 2) = dv;
    if (p == 0) {
      float2 st = make_float2(__builtin_huge_valf(), 0.f);
      if (h < a.group) {
        const int hq = a.n_kv_heads * a.group;
        st = make_float2(a.row_lse[((int64_t)b * hq + kvh * a.group + h) * a.n + t] * kLog2e, dot);
      }
      *reinterpret_cast<float2*>(rec + bwd_stats_offset(D) + 8 * h) = st;
    }
  }
}

// ----------------------------------------------------------------------------- inverse index
// Chunk c of 256 tokens of (b, kvh): rank[t][s] = how many earlier tokens of the chunk list
// the block of slot s (-1 for slots not in use); hist[c][j] = the chunk's count of block j.
// Counting runs in token order in one wave, so ranks are deterministic.
__global__ __launch_bounds__(256) void bwd_rank_kernel(BwdArgs a, int chunks) {
  extern __shared__ int32_t lds[];
  const int c = blockIdx.x, bh = blockIdx.y;
  const int K = a.top_k;
  const int t0 = c * kBwdChunk;
  const int nt = min(kBwdChunk, a.n - t0);
  const int jn = (t0 + nt - 1) / kLeaf + 1;              // blocks this chunk's tokens may list
  int32_t* sl = lds;
  int32_t* cnt = lds + kBwdChunk * K;
  const int32_t* src = a.sel + ((int64_t)bh * a.n + t0) * K;
  for (int i = threadIdx.x; i < nt * K; i += blockDim.x) sl[i] = src[i];
  for (int i = threadIdx.x; i < jn; i += blockDim.x) cnt[i] = 0;
  __syncthreads();
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    for (int i = 0; i < nt; ++i) {
      const int t = t0 + i;
      const int j = lane < K ? sl[i * K + lane] : -1;
      const bool ok = slot_in_use(j, lane, K, t);
      int r = -1;
      if (ok) {                                           // distinct blocks: no two lanes collide
        r = cnt[j];
        cnt[j] = r + 1;
      }
      if (lane < K) a.rank[((int64_t)bh * a.n + t) * K + lane] = r;
    }
  }
  __syncthreads();
  const int m1 = ceil_div(a.n, kLeaf);
  int32_t* h = a.hist + ((int64_t)bh * chunks + c) * m1;
  for (int i = threadIdx.x; i < jn; i += blockDim.x) h[i] = cnt[i];
}

// Per block e = bh * M1 + j: hist[c][j] becomes the exclusive prefix over chunks (tokens of
// earlier chunks listing j) and seg_len[e] the total.  Chunks before 64 j / 256 cannot list j.
__global__ __launch_bounds__(256) void bwd_colscan_kernel(BwdArgs a, int chunks) {
  const int m1 = ceil_div(a.n, kLeaf);
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)a.batch * a.n_kv_heads * m1) return;
  const int bh = (int)(e / m1), j = (int)(e % m1);
  int32_t run = 0;
  for (int c = j * kLeaf / kBwdChunk; c < chunks; ++c) {
    int32_t* p = a.hist + ((int64_t)bh * chunks + c) * m1 + j;
    const int32_t x = *p;
    *p = run;
    run += x;
  }
  a.seg_len[e] = run;
}

// One workgroup: seg_base = exclusive prefix of seg_len, item_base = exclusive prefix of the
// items per block (ceil(seg_len / 512)), n_items = their total.
__global__ __launch_bounds__(1024) void bwd_scan_kernel(BwdArgs a, int64_t blocks) {
  __shared__ int32_t s_len[1024], s_items[1024];
  const int tid = threadIdx.x;
  const int64_t per = (blocks + 1023) / 1024;
  const int64_t lo = min(blocks, (int64_t)tid * per), hi = min(blocks, lo + per);
  int32_t sl = 0, si = 0;
  for (int64_t e = lo; e < hi; ++e) {
    const int32_t len = a.seg_len[e];
    sl += len;
    si += (len + kBwdItem - 1) / kBwdItem;
  }
  s_len[tid] = sl;
  s_items[tid] = si;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {              // inclusive scan of the 1024 sums
    const int32_t x = tid >= off ? s_len[tid - off] : 0, y = tid >= off ? s_items[tid - off] : 0;
    __syncthreads();
    s_len[tid] += x;
    s_items[tid] += y;
    __syncthreads();
  }
  int32_t bl = tid ? s_len[tid - 1] : 0, bi = tid ? s_items[tid - 1] : 0;
  for (int64_t e = lo; e < hi; ++e) {
    const int32_t len = a.seg_len[e];
    a.seg_base[e] = bl;
    a.item_base[e] = bi;
    bl += len;
    bi += (len + kBwdItem - 1) / kBwdItem;
  }
  if (tid == 1023) a.n_items[0] = s_items[1023];
}

// Work items of block e: (e, 512 i) for i < ceil(seg_len / 512).
__global__ __launch_bounds__(256) void bwd_items_kernel(BwdArgs a) {
  const int m1 = ceil_div(a.n, kLeaf);
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= (int64_t)a.batch * a.n_kv_heads * m1) return;
  const int32_t len = a.seg_len[e], first = a.item_base[e];
  for (int i = 0; i * kBwdItem < len; ++i) a.items[first + i] = make_int2((int)e, i * kBwdItem);
}

// list[seg_base[e] + hist[c(t)][j] + rank] = t for every slot in use: tokens ascending per block.
__global__ __launch_bounds__(256) void bwd_scatter_kernel(BwdArgs a, int chunks) {
  const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (bh, t)
  if (x >= (int64_t)a.batch * a.n_kv_heads * a.n) return;
  const int bh = (int)(x / a.n), t = (int)(x % a.n);
  const int m1 = ceil_div(a.n, kLeaf);
  const int c = t / kBwdChunk;
  for (int s = 0; s < a.top_k; ++s) {
    const int32_t r = a.rank[x * a.top_k + s];
    if (r < 0) continue;
    const int j = a.sel[x * a.top_k + s];
    const int64_t e = (int64_t)bh * m1 + j;
    a.list[a.seg_base[e] + a.hist[((int64_t)bh * chunks + c) * m1 + j] + r] = t;
  }
}

// ----------------------------------------------------------------------------- dq (query-major)
template <typename TD, int D>
__global__ __launch_bounds__(256, 2) void attn_bwd_dq_kernel(BwdArgs a) {
  typedef FragBF16<D> Frag;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.n) return;
  const int bh = blockIdx.y;
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int g = lane >> 4, col = lane & 15;
  const int m1 = ceil_div(a.n, kLeaf);
  const int head = kvh * a.group + col;

  Frag qf, df;                                         // B fragments: head col, d k-slices
  if (col < a.group) {
    qf.load(reinterpret_cast<const __bf16*>(a.q) + b * a.q_sb + (int64_t)t * a.q_st + (int64_t)head * a.q_sh, g);
    const TD* drow = reinterpret_cast<const TD*>(a.dout) + b * a.do_sb + (int64_t)t * a.do_st +
                     (int64_t)head * a.do_sh;
#pragma unroll
    for (int s = 0; s < D / 32; ++s) df.v[s] = load8_bf16(drow + 32 * s + 8 * g);
  } else {
    qf.zero();
    df.zero();
  }
  const float2 st = *reinterpret_cast<const float2*>(a.tok + ((int64_t)bh * a.n + t) * bwd_record_bytes(D) +
                                                     bwd_stats_offset(D) + 8 * col);
  const float c2 = a.scale * kLog2e;

  const int64_t blk = (int64_t)bh * m1 * (kLeaf * D / 8);
  const bf16x8* krow = a.kpack + blk + lane;
  const bf16x8* vrow = a.vrows + blk + lane;
  // 0/1 selector B fragments: for half h of a 32-wide k-step, column c picks k = 16 h + c, so an
  // MFMA of a K-row fragment with sel[h] yields those 16 key columns with the keys on the result
  // rows: K transposed, exactly (products with 1 and 0, fp32 sums).
  bf16x8 sel[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[h][e] = (__bf16)(8 * g + e == 16 * h + col ? 1.f : 0.f);
  const int my_sel = lane < a.top_k ? a.sel[((int64_t)bh * a.n + t) * a.top_k + lane] : -1;
  uint64_t rest = __ballot(slot_in_use(my_sel, lane, a.top_k, t));
  const int nsel = __popcll(rest);

  floatx4 dq[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) dq[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // K one block ahead: the next block's K is requested half by half, as soon as the dq products have
  // read each half of this block's K.
  Frag kf[4];
  auto load_k = [&](int leaf, int m0) {
    const int64_t off = (int64_t)leaf * (kLeaf * D / 8);
#pragma unroll
    for (int mt = m0; mt < m0 + 2; ++mt)
#pragma unroll
      for (int s = 0; s < D / 32; ++s) kf[mt].v[s] = krow[off + (mt * (D / 32) + s) * 64];
  };
  int leaf = 0;
  if (rest) {
    leaf = __builtin_amdgcn_readfirstlane(__shfl(my_sel, __builtin_ctzll(rest), 64));
    rest &= rest - 1;
    load_k(leaf, 0);
    load_k(leaf, 2);
  }
  for (int done = 0; done < nsel; ++done) {
    const bool more = rest != 0;
    const int leaf_n = more ? __builtin_amdgcn_readfirstlane(__shfl(my_sel, __builtin_ctzll(rest), 64)) : 0;
    rest &= rest - 1;
    const int64_t first = (int64_t)leaf * kLeaf;
    const int64_t off = (int64_t)leaf * (kLeaf * D / 8);
    floatx4 s_acc[4], p_acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      Frag vf;
#pragma unroll
      for (int s = 0; s < D / 32; ++s) vf.v[s] = vrow[off + (mt * (D / 32) + s) * 64];
      s_acc[mt] = mma(kf[mt], qf, floatx4{0.f, 0.f, 0.f, 0.f});
      p_acc[mt] = mma(vf, df, floatx4{0.f, 0.f, 0.f, 0.f});
    }
    // s_acc[mt][r]: key first + perm_key(mt, 4 g + r) = first + 32 (mt / 2) + 8 g + 4 (mt % 2) + r
    const bool edge = first + kLeaf - 1 > t;
    const int lim = (int)(t - first) - 8 * g;
    bf16x8 db[2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const bool masked = edge && 32 * (mt >> 1) + 4 * (mt & 1) + r > lim;
        const float p = masked ? 0.f : __builtin_amdgcn_exp2f(fmaf(s_acc[mt][r], c2, -st.x));
        db[mt >> 1][4 * (mt & 1) + r] = (__bf16)(p * (p_acc[mt][r] - st.y));
      }
    // dq^T += K^T dS^T.  The A fragment of key half kb and d tile dt holds, in lane (g, col), element
    // e: K[first + perm_key(2 kb + e / 4, 4 g + e % 4)][16 dt + col], the key order of db[kb].  Each
    // dq[dt] still takes key half 0, then key half 1.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const floatx4 lo = mfma_bf16(kf[2 * kb].v[dt >> 1], sel[dt & 1], floatx4{0.f, 0.f, 0.f, 0.f});
        const floatx4 hi = mfma_bf16(kf[2 * kb + 1].v[dt >> 1], sel[dt & 1], floatx4{0.f, 0.f, 0.f, 0.f});
        bf16x8 kt;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          kt[r] = (__bf16)lo[r];
          kt[4 + r] = (__bf16)hi[r];
        }
        dq[dt] = mfma_bf16(kt, db[kb], dq[dt]);
      }
      if (more) load_k(leaf_n, 2 * kb);
    }
    leaf = leaf_n;
  }
  if (col < a.group) {
    float* out = a.dq + b * a.dq_sb + (int64_t)t * a.dq_st + (int64_t)head * a.dq_sh;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      *reinterpret_cast<float4*>(out + 16 * dt + 4 * g) =
          make_float4(dq[dt][0] * a.scale, dq[dt][1] * a.scale, dq[dt][2] * a.scale, dq[dt][3] * a.scale);
  }
}

// ----------------------------------------------------------------------------- dk, dv (key-major)
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_dkv_kernel(BwdArgs a) {
  constexpr int kTok = 4;                               // tokens per round
  constexpr int kRow = D + 8;                           // padded LDS row (bf16 elements)
  constexpr int kRec = bwd_record_bytes(D);
  constexpr int kPieces = kRec / 16;                    // 16-byte pieces per record
  constexpr int kPer = (kTok * kPieces + 255) / 256;    // pieces per thread per round
  constexpr int kRowPieces = D / 8;
  struct Tok {
    __bf16 q[16][kRow];
    __bf16 dout[16][kRow];
    float2 st[16];
  };
  __shared__ __align__(16) Tok s_tok[2][kTok];
  __shared__ int s_list[kBwdItem];                      // the item's tokens

  const int item = blockIdx.x;
  if (item >= a.n_items[0]) return;       // uniform over the workgroup
  const int2 it = a.items[item];
  const int m1 = ceil_div(a.n, kLeaf);
  const int e = it.x, start = it.y;
  const int bh = e / m1, j = e % m1;
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int len = min(kBwdItem, a.seg_len[e] - start);
  const int32_t* toks = a.list + a.seg_base[e] + start;
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int g = lane >> 4, col = lane & 15;
  const int key = j * kLeaf + 16 * wave + col;          // this lane's key column
  const char* records = a.tok + (int64_t)bh * a.n * kRec;
  for (int i = threadIdx.x; i < len; i += blockDim.x) s_list[i] = toks[i];
  __syncthreads();

  // Round r stages tokens [kTok r, kTok r + kTok) of the item: piece c of a record goes to row
  // c / (D / 8) of q (c < 16 D / 8), of dO, or to the statistics.
  u32x4 stage[kPer];                                    // a native vector type: kept in registers
  auto fetch = [&](int base) __attribute__((always_inline)) {   // base < len
    // unconditional loads (a piece past the round re-reads a valid one and is not stored): a
    // guarded load would be waited for where its branch joins
    const int last = min(kTok, len - base) - 1;
    static_for<kPer>([&](auto I) {
      const int x = threadIdx.x + 256 * I();
      const int tb = min(x / kPieces, last), c = x % kPieces;
      stage[I()] = reinterpret_cast<const u32x4*>(records + (int64_t)s_list[base + tb] * kRec)[c];
    });
  };
  auto store = [&](int buf, int base) __attribute__((always_inline)) {
    // piece c: row c / (d / 8) of q (rows 0-15) or dO (rows 16-31), or the statistics
    static_for<kPer>([&](auto I) {
      const int x = threadIdx.x + 256 * I();
      const int tb = x / kPieces, c = x % kPieces;
      const int off = c < 32 * kRowPieces ? (c / kRowPieces) * kRow * 2 + 16 * (c % kRowPieces)
                                          : 64 * kRow + 16 * (c - 32 * kRowPieces);
      if (x < kTok * kPieces && base + tb < len)
        *reinterpret_cast<u32x4*>(reinterpret_cast<char*>(&s_tok[buf][tb]) + off) = stage[I()];
    });
  };

  FragBF16<D> kb, vb;                                   // B fragments: key col, d k-slices
  if (key < a.n) {
    kb.load(reinterpret_cast<const __bf16*>(a.k) + b * a.k_sb + (int64_t)key * a.k_st + (int64_t)kvh * a.k_sh, g);
    vb.load(reinterpret_cast<const __bf16*>(a.v) + b * a.v_sb + (int64_t)key * a.v_st + (int64_t)kvh * a.v_sh, g);
  } else {
    kb.zero();
    vb.zero();
  }
  floatx4 dk[D / 16], dv[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    dk[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
    dv[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  const float c2 = a.scale * kLog2e;
  bf16x8 sel[2];                                        // 0/1 selectors, as in the dq pass
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) sel[h][e] = (__bf16)(8 * g + e == 16 * h + col ? 1.f : 0.f);

  // Round r's records are fetched into registers two rounds ahead and stored to LDS at the start
  // of round r - 1, so the loads stay in flight during a whole round of compute; the registers
  // carry them across the loop, which also keeps the compiler from sinking the loads.
  fetch(0);
  store(0, 0);
  if (kTok < len) fetch(kTok);
  __syncthreads();
  for (int base = 0, buf = 0; base < len; base += kTok, buf ^= 1) {
    if (base + kTok < len) store(buf ^ 1, base + kTok);      // that buffer was last read a round ago
    if (base + 2 * kTok < len) fetch(base + 2 * kTok);
    const int nt = min(kTok, len - base);
    for (int tb = 0; tb < nt; ++tb) {
      const Tok& tk = s_tok[buf][tb];
      const int t = s_list[base + tb];
      FragBF16<D> qa, da;                               // A fragments: head col, d k-slices
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        qa.v[s] = *reinterpret_cast<const bf16x8*>(&tk.q[col][32 * s + 8 * g]);
        da.v[s] = *reinterpret_cast<const bf16x8*>(&tk.dout[col][32 * s + 8 * g]);
      }
      const floatx4 sacc = mma(qa, kb, floatx4{0.f, 0.f, 0.f, 0.f});    // [head 4 g + r][key col]
      const floatx4 pacc = mma(da, vb, floatx4{0.f, 0.f, 0.f, 0.f});
      bf16x4 pb, db;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float2 sr = tk.st[4 * g + r];
        const float p = key > t ? 0.f : __builtin_amdgcn_exp2f(fmaf(sacc[r], c2, -sr.x));
        pb[r] = (__bf16)p;
        db[r] = (__bf16)(p * (pacc[r] - sr.y));
      }
      // A fragments of d tile dt (lane (g, col): heads 4 g + r of d column 16 dt + col) from the row
      // fragments by a selector MFMA, which puts the heads on the result rows
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const floatx4 tdo = mfma_bf16(da.v[dt >> 1], sel[dt & 1], floatx4{0.f, 0.f, 0.f, 0.f});
        const floatx4 tq = mfma_bf16(qa.v[dt >> 1], sel[dt & 1], floatx4{0.f, 0.f, 0.f, 0.f});
        bf16x4 doa, qta;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          doa[r] = (__bf16)tdo[r];
          qta[r] = (__bf16)tq[r];
        }
        dv[dt] = mfma_k16(doa, pb, dv[dt]);                // [d 16 dt + 4 g + r][key col]
        dk[dt] = mfma_k16(qta, db, dk[dt]);
      }
    }
    __syncthreads();
  }
  float* pk = a.partial + (int64_t)item * 2 * kLeaf * D;
  float* pv = pk + kLeaf * D;
  const int kr = 16 * wave + col;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) {
    *reinterpret_cast<float4*>(pk + kr * D + 16 * dt + 4 * g) = make_float4(dk[dt][0], dk[dt][1], dk[dt][2], dk[dt][3]);
    *reinterpret_cast<float4*>(pv + kr * D + 16 * dt + 4 * g) = make_float4(dv[dt][0], dv[dt][1], dv[dt][2], dv[dt][3]);
  }
}

// dk, dv of every key: the block's item partials added in item order (zero for blocks that
// no token selected), dk scaled once.
template <int D>
__global__ __launch_bounds__(256) void attn_bwd_finish_kernel(BwdArgs a) {
  const int m1 = ceil_div(a.n, kLeaf);
  const int64_t x = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;   // (e, key row, 4-column group)
  if (x >= (int64_t)a.batch * a.n_kv_heads * m1 * kLeaf * (D / 4)) return;
  const int d4 = (int)(x % (D / 4));
  const int kr = (int)((x / (D / 4)) % kLeaf);
  const int64_t e = x / ((D / 4) * kLeaf);
  const int bh = (int)(e / m1), j = (int)(e % m1);
  const int64_t key = (int64_t)j * kLeaf + kr;
  if (key >= a.n) return;
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int items = (a.seg_len[e] + kBwdItem - 1) / kBwdItem;
  const int64_t first = a.item_base[e];
  float4 sk = make_float4(0.f, 0.f, 0.f, 0.f), sv = sk;
  for (int i = 0; i < items; ++i) {
    const float* pk = a.partial + (first + i) * 2 * kLeaf * D + kr * D + 4 * d4;
    const float4 xk = *reinterpret_cast<const float4*>(pk);
    const float4 xv = *reinterpret_cast<const float4*>(pk + kLeaf * D);
    sk.x += xk.x; sk.y += xk.y; sk.z += xk.z; sk.w += xk.w;
    sv.x += xv.x; sv.y += xv.y; sv.z += xv.z; sv.w += xv.w;
  }
  float* ok = a.dk + b * a.dk_sb + key * a.dk_st + (int64_t)kvh * a.dk_sh + 4 * d4;
  float* ov = a.dv + b * a.dv_sb + key * a.dv_st + (int64_t)kvh * a.dv_sh + 4 * d4;
  *reinterpret_cast<float4*>(ok) = make_float4(sk.x * a.scale, sk.y * a.scale, sk.z * a.scale, sk.w * a.scale);
  *reinterpret_cast<float4*>(ov) = sv;
}

// ----------------------------------------------------------------------------- launcher
template <typename TD, int D>
hipError_t launch_attention_bwd_t(const BwdArgs& a, hipStream_t s) {
  const int bhs = a.batch * a.n_kv_heads;
  const int m1 = ceil_div(a.n, kLeaf);
  const int chunks = ceil_div(a.n, kBwdChunk);
  const int64_t blocks = (int64_t)bhs * m1;
  hipError_t e;

  PackArgs p;                                           // K rows
  p.k = a.k; p.k_sb = a.k_sb; p.k_st = a.k_st; p.k_sh = a.k_sh;
  p.v = nullptr; p.v_sb = p.v_st = p.v_sh = 0;
  p.kpack = a.kpack; p.vpack = nullptr;
  p.batch = a.batch; p.n_kv_heads = a.n_kv_heads; p.head_dim = D; p.n = a.n;
  if ((e = launch_pack(p, s)) != hipSuccess) return e;
  p.k = a.v; p.k_sb = a.v_sb; p.k_st = a.v_st; p.k_sh = a.v_sh;      // V rows in the same key order
  p.kpack = a.vrows;
  if ((e = launch_pack(p, s)) != hipSuccess) return e;

  const dim3 tok_grid(ceil_div(a.n, 4), bhs);
  const int rec_threads = 16 * (D / 8);                     // one token's pieces
  hipLaunchKernelGGL((bwd_tokens_kernel<TD, D>), dim3((unsigned)a.n, bhs), dim3(rec_threads), 0, s, a);
  if ((e = launched(s)) != hipSuccess) return e;
  const size_t rank_lds = (size_t)(kBwdChunk * a.top_k + m1) * sizeof(int32_t);
  hipLaunchKernelGGL(bwd_rank_kernel, dim3(chunks, bhs), dim3(256), rank_lds, s, a, chunks);
  if ((e = launched(s)) != hipSuccess) return e;
  const unsigned blk_grid = (unsigned)((blocks + 255) / 256);
  hipLaunchKernelGGL(bwd_colscan_kernel, dim3(blk_grid), dim3(256), 0, s, a, chunks);
  if ((e = launched(s)) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_scan_kernel, dim3(1), dim3(1024), 0, s, a, blocks);
  if ((e = launched(s)) != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_items_kernel, dim3(blk_grid), dim3(256), 0, s, a);
  if ((e = launched(s)) != hipSuccess) return e;
  const int64_t rows = (int64_t)bhs * a.n;
  hipLaunchKernelGGL(bwd_scatter_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, a, chunks);
  if ((e = launched(s)) != hipSuccess) return e;

  hipLaunchKernelGGL((attn_bwd_dq_kernel<TD, D>), tok_grid, dim3(256), 0, s, a);
  if ((e = launched(s)) != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dkv_kernel<D>), dim3((unsigned)a.max_items), dim3(256), 0, s, a);
  if ((e = launched(s)) != hipSuccess) return e;
  const int64_t fin = blocks * kLeaf * (D / 4);
  hipLaunchKernelGGL((attn_bwd_finish_kernel<D>), dim3((unsigned)((fin + 255) / 256)), dim3(256), 0, s, a);
  return launched(s);
}

template <typename TD>
hipError_t launch_attention_bwd_d(const BwdArgs& a, hipStream_t s) {
  return a.head_dim == 64 ? launch_attention_bwd_t<TD, 64>(a, s) : launch_attention_bwd_t<TD, 128>(a, s);
}

hipError_t launch_attention_bwd(const BwdArgs& a, hipStream_t s) {
  return a.grad_bf16 ? launch_attention_bwd_d<__bf16>(a, s) : launch_attention_bwd_d<float>(a, s);
}

}  // namespace pisa
