// decode.hip - one decode step (Method steps, third step of "Block Sparse Attention
// with Log-Linear Complexity"): append the new key/value, refresh the new token's
// leaf mean and its ancestor path, then a single fused pass that walks every
// level down to exact leaf scores, keeps K leaves and attends over them.
//
// One multi-wave workgroup per (b, kvh) does the whole step: first the update,
// one thread per column with the same pooling functions as the prefill build (so
// the pyramid stays bit-identical to a rebuild), then the routing levels (serial),
// with the work inside each level, the candidate leaves and the attended blocks
// spread over the waves (see the kernel's comment).
#include "kernels.h"
#include "pyramid_dev.h"

namespace pisa {

// Update of unit bh by threads c < D (one per column): append the new key and value at n_ctx,
// recompute the new token's leaf mean and its ancestor path with the pooling of the prefill build,
// so the pyramid stays bit-identical to a rebuild.
template <typename T, int D>
__device__ inline void decode_update_unit(const DecodeArgs& a, int bh, int c) {
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int64_t pos = a.n_ctx;
  T* kc = reinterpret_cast<T*>(a.k_cache) + b * a.kc_sb + kvh * a.kc_sh;
  T* vc = reinterpret_cast<T*>(a.v_cache) + b * a.vc_sb + kvh * a.vc_sh;
  const T* kn = reinterpret_cast<const T*>(a.k_new) + b * a.kn_sb + kvh * a.kn_sh;
  const T* vn = reinterpret_cast<const T*>(a.v_new) + b * a.vn_sb + kvh * a.vn_sh;
  kc[pos * a.kc_st + c] = kn[c];
  vc[pos * a.vc_st + c] = vn[c];

  float* pyr = a.pyr + (int64_t)bh * a.lv.nodes * D;
  const int leaf = (int)(pos / kLeaf);
  const int64_t first = (int64_t)leaf * kLeaf;
  float val = leaf_mean_column(kc, a.kc_st, first, (int)(pos - first + 1), c);  // reads this thread's own write
  pyr[(a.lv.offset[0] + leaf) * D + c] = val;
  // The siblings along the path do not change: load them for every level first, then
  // recompute the path bottom-up (level l's node is the parent of the level l - 1 path node).
  float sib[kMaxLevels];
  int idx = leaf;
#pragma unroll
  for (int l = 2; l <= kMaxLevels; ++l) {
    if (l <= a.lv.count) {
      const int s = idx ^ 1;
      sib[l - 2] = s < a.lv.size[l - 2] ? pyr[(a.lv.offset[l - 2] + s) * D + c] : 0.f;
      idx >>= 1;
    }
  }
  idx = leaf;
#pragma unroll
  for (int l = 2; l <= kMaxLevels; ++l) {
    if (l <= a.lv.count) {
      const int p = idx >> 1;
      const bool has2 = 2 * p + 1 < a.lv.size[l - 2];
      const float c0 = (idx & 1) ? sib[l - 2] : val;
      const float c1 = (idx & 1) ? val : sib[l - 2];
      val = node_mean(c0, c1, has2);
      pyr[(a.lv.offset[l - 1] + p) * D + c] = val;
      idx = p;
    }
  }
}

// ----------------------------------------------------------------------------- fused route + attend
// One workgroup of kDecodeWaves waves per (b, kvh).  Every phase spreads its work over the waves:
//  * routing, level by level from the root: the candidates' children are scored 16 at a time as the
//    rows of an S^T = (children) Q^T MFMA tile (fp32 summaries, v_mfma_f32_16x16x4_f32), one tile per
//    wave; a candidate's two children sit in the same lane, so its per-head LSE is in-lane and the
//    head sum a DPP row reduction; wave 0 keeps K by (score descending, index ascending) and expands;
//  * leaf scoring: one candidate leaf per wave, S^T over its 64 raw keys on the input type's MFMA;
//    the logits (base-2 units) are staged in LDS and reused by the attention, so the selected keys
//    are read from HBM once; every level scores with the configured candidate score (LSE, or the
//    mean / mean + var/2 variants);
//  * attention: softmax statistics per head over the selected leaves' staged logits, then P V with
//    one selected block per wave, 16 value rows in flight at a time, and a fixed-order sum of the
//    per-wave partial outputs.
constexpr int kDecodeWaves = 8;

// LDS carve-up of the fused kernel (4-byte words).
struct DecodeLds {
  int zl, part, us, hstat, ints;
  size_t bytes;
  __host__ __device__ DecodeLds(int G, int width, int D) {
    zl = 0;                                   // width * 64 * G staged leaf logits, then probabilities
    part = zl + width * kLeaf * G;            // kDecodeWaves * G * D partial outputs
    us = part + kDecodeWaves * G * D;         // 64 candidate scores
    hstat = us + 64;                          // per-head max and 1 / sum
    ints = hstat + 2 * G;                     // cand[64], selv[64], sels[64], misc[4]
    bytes = (size_t)(ints + 3 * 64 + 4) * 4;
  }
};

// Wave 0: keep flag of slot `lane` (candidate ci): when more than K are valid, the K best by
// (score descending, index ascending), else every valid one.  The valid slots are the lowest ones
// and hold ascending indices (each expansion keeps the parents' slot order and only the last
// parent can lose its second child), as keep_top_k needs.
__device__ inline bool decode_keep(int ci, const float* us, int nvalid, int K, int lane) {
  const bool best = nvalid > K ? keep_top_k(score_key(us[lane], ci >= 0), K) : true;   // uniform branch
  return ci >= 0 && best;
}

template <typename T, typename TO, int D, int G>
__global__ __launch_bounds__(kDecodeWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) void decode_fused_kernel(
    DecodeArgs a) {
  typedef typename RawFrag<T, D>::type Frag;
  extern __shared__ __align__(16) float smem[];
  const int width = 2 * a.top_k, K = a.top_k;
  const DecodeLds L(G, width, D);
  float* zl = smem + L.zl;
  float* part = smem + L.part;
  float* us = smem + L.us;
  float* hstat = smem + L.hstat;
  int* cand = reinterpret_cast<int*>(smem + L.ints);
  int* selv = cand + 64;               // selected leaf ids, ascending
  int* sels = selv + 64;               // their candidate slots
  int* misc = sels + 64;               // [0] slots, [1] valid, [2] selected

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, col = lane & 15;
  const int bh = blockIdx.x;
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int t = a.n_ctx;               // query position: every stored key is valid
  const float c2 = a.scale * 1.4426950408889634f;   // logits in base-2 units
  const bool head_ok = col < G;
  const T* qrow = reinterpret_cast<const T*>(a.q) + b * a.q_sb + (int64_t)(kvh * G + (head_ok ? col : 0)) * a.q_sh;
  const float* pyr = a.pyr + (int64_t)bh * a.lv.nodes * D;

  // ---- update of this unit (its rows and nodes only), then routing in the same workgroup: the
  // barrier makes the new key, value and path visible to every wave (one CU, one L1)
  if (tid < D) decode_update_unit<T, D>(a, bh, tid);
  if (tid < 64) cand[tid] = tid == 0 ? 0 : -1;  // A^(L) = {root}
  if (tid == 0) { misc[0] = 1; misc[1] = 1; }
  __syncthreads();

  // ---- routing, levels L .. 2
  FragF32<D> qf;
  if (head_ok) qf.load(qrow, g); else qf.zero();
  for (int level = a.lv.count; level >= 2; --level) {
    const int nslots = misc[0], nvalid = misc[1];
    const int child_size = a.lv.size[level - 2];
    const float* child_base = pyr + a.lv.offset[level - 2] * D;
    if (nvalid > K) {
      const int tiles = (2 * nslots + 15) / 16;
      for (int nt = wave; nt < tiles; nt += kDecodeWaves) {
        const int slot = 16 * nt + col;
        const int parent = cand[slot >> 1];
        const int child = 2 * parent + (slot & 1);
        const bool ok = parent >= 0 && child < child_size;
        FragF32<D> kf;
        kf.load(child_base + (int64_t)(ok ? child : 0) * D, g);
        const uint64_t okmask = __ballot(ok);
        const floatx4 acc = mma(kf, qf, floatx4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int h = 0; h < 2; ++h) {                   // candidate 8 nt + 2 g + h: rows 4 g + 2 h, +1
          const int r0 = 4 * g + 2 * h;
          const float sc = pair_score(acc[2 * h], acc[2 * h + 1], (okmask >> r0) & 1, (okmask >> (r0 + 1)) & 1,
                                      a.score, a.scale, c2);
          const float u = row_sum_to_last(head_ok ? sc : 0.f);
          if (col == 15) us[8 * nt + 2 * g + h] = u;
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      const int ci = lane < nslots ? cand[lane] : -1;
      const bool kp = decode_keep(ci, us, nvalid, K, lane);
      const uint64_t kept = __ballot(kp);
      const int m = __popcll(kept);
      const int p = lane >> 1;
      const int parent = __shfl(ci, nth_set_bit(kept, p < m ? p : 0), 64);
      const int child = 2 * parent + (lane & 1);
      const int nc = (p < m && child < child_size) ? child : -1;
      cand[lane] = nc;
      const int nv = __popcll(__ballot(nc >= 0));
      if (lane == 0) { misc[0] = 2 * m; misc[1] = nv; }
    }
    __syncthreads();
  }

  // ---- leaf level: exact logits of every candidate leaf over its raw keys <= t
  const int nslots = misc[0], nvalid = misc[1];
  Frag qr;
  if (head_ok) qr.load(qrow, g); else qr.zero();
  const T* kbase = reinterpret_cast<const T*>(a.k_cache) + b * a.kc_sb + kvh * a.kc_sh;
  for (int slot = wave; slot < nslots; slot += kDecodeWaves) {
    const int leaf = cand[slot];
    if (leaf < 0) continue;                             // wave-uniform
    const int first = leaf * kLeaf;
    floatx4 acc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {                    // rows past t are clamped to t, then masked
      Frag kf;
      kf.load(kbase + (int64_t)min(first + 16 * mt + col, t) * a.kc_st, g);
      acc[mt] = mma(kf, qr, floatx4{0.f, 0.f, 0.f, 0.f});
    }
    // acc[mt][r]: key first + 16 mt + 4 g + r, head col; the attention reuses the staged logits
    float head;                                         // this head's leaf score
    if (a.score == 0) {                                 // LSE, base-2 units
      float m = kNegInf;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 16 * mt + 4 * g + r;
          const float z = first + key <= t ? acc[mt][r] * c2 : kNegInf;
          if (head_ok) zl[(slot * kLeaf + key) * G + col] = z;
          acc[mt][r] = z;
          m = fmaxf(m, z);
        }
      m = rows_max(m);
      float sum = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) sum += __builtin_amdgcn_exp2f(acc[mt][r] - m);   // key t is valid: m finite
      sum = rows_sum(sum);
      head = m + __builtin_amdgcn_logf(sum);
    } else {                                            // mean, or mean + var / 2, natural units
      const float cnt = (float)min(kLeaf, t - first + 1);
      float s1 = 0.f;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 16 * mt + 4 * g + r;
          const bool ok = first + key <= t;
          if (head_ok) zl[(slot * kLeaf + key) * G + col] = ok ? acc[mt][r] * c2 : kNegInf;
          s1 += ok ? acc[mt][r] : 0.f;
        }
      s1 = rows_sum(s1);
      const float mean = s1 / cnt;
      head = mean * a.scale;
      if (a.score == 2) {
        float s2 = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float dv = (acc[mt][r] - mean) * a.scale;
            s2 += first + 16 * mt + 4 * g + r <= t ? dv * dv : 0.f;
          }
        s2 = rows_sum(s2);
        head += 0.5f * s2 / cnt;
      }
    }
    const float u = row_sum_to_last(head_ok ? head : 0.f);
    if (lane == 15) us[slot] = u;
  }
  __syncthreads();
  if (wave == 0) {
    const int ci = lane < nslots ? cand[lane] : -1;
    const bool kp = decode_keep(ci, us, nvalid, K, lane);
    const int c = kp ? ci : 0x7fffffff;
    int pos = 0;                                        // ascending leaf order among the kept
    for (int j = 0; j < 64; ++j) pos += __builtin_amdgcn_readlane(c, j) < c;
    if (kp) { selv[pos] = c; sels[pos] = lane; }
    const int ns = __popcll(__ballot(kp));               // the whole wave votes, outside the lane-0 store
    if (lane == 0) misc[2] = ns;
  }
  __syncthreads();

  // ---- softmax over the selected leaves' keys, per head
  const int nsel = misc[2];
  const int nkeys = nsel * kLeaf;
  for (int h = wave; h < G; h += kDecodeWaves) {
    float m = kNegInf;
    for (int e = lane; e < nkeys; e += 64) m = fmaxf(m, zl[(sels[e / kLeaf] * kLeaf + e % kLeaf) * G + h]);
    for (int o = 1; o < 64; o <<= 1) m = wave_max_xor(m, o);
    float s = 0.f;
    for (int e = lane; e < nkeys; e += 64) s += __builtin_amdgcn_exp2f(zl[(sels[e / kLeaf] * kLeaf + e % kLeaf) * G + h] - m);
    for (int o = 1; o < 64; o <<= 1) s = wave_add_xor(s, o);
    if (lane == 0) { hstat[h] = m; hstat[G + h] = 1.f / s; }
  }
  __syncthreads();
  for (int e = tid; e < nkeys * G; e += blockDim.x) {
    const int h = e % G, kk = e / G;
    float* z = &zl[(sels[kk / kLeaf] * kLeaf + kk % kLeaf) * G + h];
    *z = __builtin_amdgcn_exp2f(*z - hstat[h]) * hstat[G + h];
  }
  __syncthreads();

  // ---- P V: one selected block per wave, 16 of its value rows in flight at a time (more rows, or
  // a register cap for more waves per SIMD, measured slower)
  constexpr int kCols = D / 64;                         // value columns per lane
  constexpr int kRows = 8;
  float accv[G][kCols];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < kCols; ++c) accv[h][c] = 0.f;
  const T* vbase = reinterpret_cast<const T*>(a.v_cache) + b * a.vc_sb + kvh * a.vc_sh + lane * kCols;
  // This wave's blocks j = wave, wave + 8, ... walked as one stream of 16-row chunks; the next
  // chunk's value rows are requested before the current chunk's products (two buffers).  The
  // products run chunk by chunk and row by row, so the order of the sums is the plain one.
  constexpr int kChunks = kLeaf / kRows;
  const int n_chunks = (nsel > wave ? (nsel - wave + kDecodeWaves - 1) / kDecodeWaves : 0) * kChunks;
  auto load_chunk = [&](int ci, T (&buf)[kRows][kCols]) {
    const int first = selv[wave + (ci / kChunks) * kDecodeWaves] * kLeaf + (ci % kChunks) * kRows;
#pragma unroll
    for (int i = 0; i < kRows; ++i)                     // keys past t: clamped row, probability 0
#pragma unroll
      for (int c = 0; c < kCols; ++c) buf[i][c] = vbase[(int64_t)min(first + i, t) * a.vc_st + c];
  };
  auto fma_chunk = [&](int ci, const T (&buf)[kRows][kCols]) {
    const int slot = sels[wave + (ci / kChunks) * kDecodeWaves];
    const int r0 = (ci % kChunks) * kRows;
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const float* p = &zl[(slot * kLeaf + r0 + i) * G];
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int c = 0; c < kCols; ++c) accv[h][c] = fmaf(p[h], to_f32(buf[i][c]), accv[h][c]);
    }
  };
  T vb0[kRows][kCols], vb1[kRows][kCols];
  if (n_chunks > 0) load_chunk(0, vb0);
  for (int ci = 0; ci < n_chunks; ci += 2) {            // n_chunks is a multiple of kChunks (even)
    load_chunk(ci + 1, vb1);
    fma_chunk(ci, vb0);
    if (ci + 2 < n_chunks) load_chunk(ci + 2, vb0);
    fma_chunk(ci + 1, vb1);
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < kCols; ++c) part[(wave * G + h) * D + lane * kCols + c] = accv[h][c];
  __syncthreads();
  TO* obase = reinterpret_cast<TO*>(a.o) + b * a.o_sb + (int64_t)kvh * G * a.o_sh;
  for (int e = tid; e < G * D; e += blockDim.x) {
    const int h = e / D, c = e % D;
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) v += part[(w * G + h) * D + c];
    obase[h * a.o_sh + c] = from_f32<TO>(v);
  }
  if (a.sel_out && tid < K) a.sel_out[(int64_t)bh * K + tid] = tid < nsel ? selv[tid] : -1;
}

size_t decode_lds_bytes(int group, int width, int head_dim) {
  return DecodeLds(group, width, head_dim).bytes;
}

template <typename T, int D, int G>
hipError_t launch_decode_fused(const DecodeArgs& a, hipStream_t s) {
  const size_t lds = decode_lds_bytes(G, 2 * a.top_k, D);
  auto kern = a.out_bf16 ? decode_fused_kernel<T, __bf16, D, G> : decode_fused_kernel<T, float, D, G>;
  if (lds > 64 * 1024) {
    hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(a.batch * a.n_kv_heads), dim3(kDecodeWaves * 64), lds, s, a);
  return launched(s);
}

template <typename T, int D>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  switch (a.group) {
    case 1: return launch_decode_fused<T, D, 1>(a, s);
    case 2: return launch_decode_fused<T, D, 2>(a, s);
    case 4: return launch_decode_fused<T, D, 4>(a, s);
    case 8: return launch_decode_fused<T, D, 8>(a, s);
    default: return launch_decode_fused<T, D, 16>(a, s);
  }
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.bf16) return a.head_dim == 64 ? launch_decode_t<__bf16, 64>(a, s) : launch_decode_t<__bf16, 128>(a, s);
  return a.head_dim == 64 ? launch_decode_t<float, 64>(a, s) : launch_decode_t<float, 128>(a, s);
}

}  // namespace pisa
