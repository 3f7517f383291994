// decode.hip - one decode step (Method steps, third step of "Block Sparse Attention
// with Log-Linear Complexity"): append the new key/value, refresh the new token's
// leaf mean and its ancestor path, then a single fused pass that walks every
// level down to exact leaf scores, keeps K leaves and attends over them.
//
// The update runs one workgroup per (b, kvh) with one thread per column and the
// same pooling functions as the prefill build, so the pyramid stays
// bit-identical to a rebuild.  The fused kernel is one workgroup per (b, kvh):
// levels are serial, candidates parallel; the leaf logits of every candidate
// leaf are staged in LDS and reused by the attention of the selected leaves, so
// selected keys are read from HBM once.  Decode is HBM-bound, so it uses fp32
// FMA on the VALU (G is a template parameter to keep the head accumulators in
// registers).
#include "kernels.h"
#include "pyramid_dev.h"

namespace pisa {

template <typename T, int D>
__global__ __launch_bounds__(128) void decode_update_kernel(DecodeArgs a) {
  const int bh = blockIdx.x;
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int c = threadIdx.x;                      // blockDim.x == D
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
  int idx = leaf;
  for (int level = 2; level <= a.lv.count; ++level) {
    const int p = idx >> 1;
    const int child_size = a.lv.size[level - 2];
    const float* ch = pyr + a.lv.offset[level - 2] * D;
    const bool has2 = 2 * p + 1 < child_size;
    const float c0 = (2 * p == idx) ? val : ch[(int64_t)(2 * p) * D + c];
    const float c1 = has2 ? ((2 * p + 1 == idx) ? val : ch[(int64_t)(2 * p + 1) * D + c]) : 0.f;
    val = node_mean(c0, c1, has2);
    pyr[(a.lv.offset[level - 1] + p) * D + c] = val;
    idx = p;
  }
}

// LDS carve-up of the fused kernel (floats unless noted).
struct DecodeLds {
  int qs, zc, zl, part, ints;
  size_t bytes;
  __host__ __device__ DecodeLds(int G, int width, int D) {
    qs = 0;                          // G * D query rows
    zc = qs + G * D;                 // 128 child slots * G logits
    zl = zc + 128 * G;               // width * 64 * G leaf logits, then probabilities
    part = zl + width * 64 * G;      // 4 waves * G * D partial outputs
    ints = part + 4 * G * D;         // int scratch: 6 * 64 + 8
    bytes = (size_t)(ints + 6 * 64 + 8) * 4;
  }
};

template <typename T, typename TO, int D, int G>
__global__ __launch_bounds__(256) void decode_fused_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) float smem[];
  const int width = 2 * a.top_k, K = a.top_k;
  const DecodeLds L(G, width, D);
  float* qs = smem + L.qs;
  float* zc = smem + L.zc;
  float* zl = smem + L.zl;
  float* part = smem + L.part;
  int* cand = reinterpret_cast<int*>(smem + L.ints);
  int* cand2 = cand + 64;
  float* us = reinterpret_cast<float*>(cand2 + 64);
  int* keep = reinterpret_cast<int*>(us + 64);
  int* selv = keep + 64;               // selected leaf ids, ascending
  int* sels = selv + 64;               // their candidate slots
  int* misc = sels + 64;               // [0] slots, [1] valid, [2] selected
  float* hstat = zc;                   // per-head max and 1/sum, reused after routing

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int bh = blockIdx.x;
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int64_t t = a.n_ctx;           // query position: every stored key is valid
  const T* qsrc = reinterpret_cast<const T*>(a.q) + b * a.q_sb + (int64_t)kvh * G * a.q_sh;
  for (int e = tid; e < G * D; e += blockDim.x) qs[e] = to_f32(qsrc[(e / D) * a.q_sh + e % D]);
  if (tid == 0) { cand[0] = 0; misc[0] = 1; misc[1] = 1; }
  __syncthreads();
  const float* pyr = a.pyr + (int64_t)bh * a.lv.nodes * D;

  for (int level = a.lv.count; level >= 2; --level) {
    const int nslots = misc[0], nvalid = misc[1];
    const int child_size = a.lv.size[level - 2];
    const float* child_base = pyr + a.lv.offset[level - 2] * D;
    if (nvalid > K) {
      for (int e = tid; e < 2 * nslots * G; e += blockDim.x) {
        const int slot = e / G, h = e % G;
        const int parent = cand[slot >> 1];
        const int child = 2 * parent + (slot & 1);
        float z = kNegInf;
        if (parent >= 0 && child < child_size) {
          const float* row = child_base + (int64_t)child * D;
          const float* qh = qs + h * D;
          float acc = 0.f;
          for (int c = 0; c < D; c += 4) {
            const float4 r = *reinterpret_cast<const float4*>(row + c);
            acc = fmaf(r.x, qh[c], acc);
            acc = fmaf(r.y, qh[c + 1], acc);
            acc = fmaf(r.z, qh[c + 2], acc);
            acc = fmaf(r.w, qh[c + 3], acc);
          }
          z = acc * a.scale;
        }
        zc[slot * G + h] = z;
      }
      __syncthreads();
      for (int i = tid; i < nslots; i += blockDim.x) {
        float u = kNegInf;
        if (cand[i] >= 0) {
          u = 0.f;
          for (int h = 0; h < G; ++h) {
            const float z0 = zc[(2 * i) * G + h], z1 = zc[(2 * i + 1) * G + h];
            const float m = fmaxf(z0, z1);
            u += m + logf(expf(z0 - m) + expf(z1 - m));
          }
        }
        us[i] = u;
      }
      __syncthreads();
      for (int i = tid; i < nslots; i += blockDim.x) {
        const int ci = cand[i];
        int rank = 0;
        if (ci >= 0)
          for (int j = 0; j < nslots; ++j) {
            const int cj = cand[j];
            rank += (cj >= 0) && (us[j] > us[i] || (us[j] == us[i] && cj < ci));
          }
        keep[i] = ci >= 0 && rank < K;
      }
    } else {
      for (int i = tid; i < nslots; i += blockDim.x) keep[i] = cand[i] >= 0;
    }
    __syncthreads();
    if (wave == 0) {
      const bool kp = lane < nslots && keep[lane];
      const uint64_t km = __ballot(kp);
      const int pos = __popcll(km & ((1ull << lane) - 1ull));
      if (kp) {
        const int parent = cand[lane];
        cand2[2 * pos] = 2 * parent < child_size ? 2 * parent : -1;
        cand2[2 * pos + 1] = 2 * parent + 1 < child_size ? 2 * parent + 1 : -1;
      }
      wave_lds_sync();
      const int m2 = 2 * __popcll(km);
      const int v = lane < m2 ? cand2[lane] : -1;
      cand[lane] = v;
      const int nv = __popcll(__ballot(v >= 0));
      if (lane == 0) { misc[0] = m2; misc[1] = nv; }
    }
    __syncthreads();
  }

  // leaf level: exact logits of every candidate leaf, staged for the attention
  const int nslots = misc[0], nvalid = misc[1];
  const T* kbase = reinterpret_cast<const T*>(a.k_cache) + b * a.kc_sb + kvh * a.kc_sh;
  for (int e = tid; e < nslots * kLeaf; e += blockDim.x) {
    const int slot = e / kLeaf, r = e % kLeaf;
    const int leaf = cand[slot];
    const int64_t key = (int64_t)leaf * kLeaf + r;
    float acc[G];
#pragma unroll
    for (int h = 0; h < G; ++h) acc[h] = kNegInf;
    if (leaf >= 0 && key <= t) {
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] = 0.f;
      const T* krow = kbase + key * a.kc_st;
      for (int c = 0; c < D; c += 4) {
        const float4 kk = load4(krow + c);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float* qh = qs + h * D + c;
          acc[h] = fmaf(kk.x, qh[0], acc[h]);
          acc[h] = fmaf(kk.y, qh[1], acc[h]);
          acc[h] = fmaf(kk.z, qh[2], acc[h]);
          acc[h] = fmaf(kk.w, qh[3], acc[h]);
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) acc[h] *= a.scale;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) zl[(slot * kLeaf + r) * G + h] = acc[h];
  }
  __syncthreads();
  if (nvalid > K) {
    for (int i = tid; i < nslots; i += blockDim.x) {
      float u = kNegInf;
      if (cand[i] >= 0) {
        u = 0.f;
        for (int h = 0; h < G; ++h) {
          float m = kNegInf;
          for (int r = 0; r < kLeaf; ++r) m = fmaxf(m, zl[(i * kLeaf + r) * G + h]);
          float s = 0.f;
          for (int r = 0; r < kLeaf; ++r) s += expf(zl[(i * kLeaf + r) * G + h] - m);
          u += m + logf(s);
        }
      }
      us[i] = u;
    }
    __syncthreads();
    for (int i = tid; i < nslots; i += blockDim.x) {
      const int ci = cand[i];
      int rank = 0;
      if (ci >= 0)
        for (int j = 0; j < nslots; ++j) {
          const int cj = cand[j];
          rank += (cj >= 0) && (us[j] > us[i] || (us[j] == us[i] && cj < ci));
        }
      keep[i] = ci >= 0 && rank < K;
    }
  } else {
    for (int i = tid; i < nslots; i += blockDim.x) keep[i] = cand[i] >= 0;
  }
  __syncthreads();
  if (wave == 0) {
    const bool kp = lane < nslots && keep[lane];
    const int c = kp ? cand[lane] : 0x7fffffff;
    int pos = 0;
    for (int j = 0; j < 64; ++j) {
      const int cj = __shfl(c, j, 64);
      const bool kj = __shfl((int)kp, j, 64) != 0;
      pos += kj && cj < c;
    }
    if (kp) { selv[pos] = c; sels[pos] = lane; }
    const int ns = __popcll(__ballot(kp));
    if (lane == 0) misc[2] = ns;
  }
  __syncthreads();

  // attention over the selected leaves: per-head softmax statistics, then P in place
  const int nsel = misc[2];
  const int nkeys = nsel * kLeaf;
  for (int h = wave; h < G; h += 4) {
    float m = kNegInf;
    for (int e = lane; e < nkeys; e += 64) m = fmaxf(m, zl[(sels[e / kLeaf] * kLeaf + e % kLeaf) * G + h]);
    for (int o = 1; o < 64; o <<= 1) m = wave_max_xor(m, o);
    float s = 0.f;
    for (int e = lane; e < nkeys; e += 64) s += expf(zl[(sels[e / kLeaf] * kLeaf + e % kLeaf) * G + h] - m);
    for (int o = 1; o < 64; o <<= 1) s = wave_add_xor(s, o);
    if (lane == 0) { hstat[h] = m; hstat[G + h] = 1.f / s; }
  }
  __syncthreads();
  for (int e = tid; e < nkeys * G; e += blockDim.x) {
    const int h = e % G, kk = e / G;
    float* z = &zl[(sels[kk / kLeaf] * kLeaf + kk % kLeaf) * G + h];
    *z = expf(*z - hstat[h]) * hstat[G + h];
  }
  __syncthreads();

  constexpr int kCols = D / 64;        // value columns per lane
  float accv[G][kCols];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < kCols; ++c) accv[h][c] = 0.f;
  const T* vbase = reinterpret_cast<const T*>(a.v_cache) + b * a.vc_sb + kvh * a.vc_sh;
  for (int kk = wave; kk < nkeys; kk += 4) {
    const int slot = sels[kk / kLeaf];
    const int64_t key = (int64_t)cand[slot] * kLeaf + kk % kLeaf;
    if (key > t) continue;
    const T* vrow = vbase + key * a.vc_st + lane * kCols;
    float vv[kCols];
#pragma unroll
    for (int c = 0; c < kCols; ++c) vv[c] = to_f32(vrow[c]);
    const float* p = &zl[(slot * kLeaf + kk % kLeaf) * G];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int c = 0; c < kCols; ++c) accv[h][c] = fmaf(p[h], vv[c], accv[h][c]);
  }
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int c = 0; c < kCols; ++c) part[(wave * G + h) * D + lane * kCols + c] = accv[h][c];
  __syncthreads();
  TO* obase = reinterpret_cast<TO*>(a.o) + b * a.o_sb + (int64_t)kvh * G * a.o_sh;
  for (int e = tid; e < G * D; e += blockDim.x) {
    const int h = e / D, c = e % D;
    const float v = ((part[(0 * G + h) * D + c] + part[(1 * G + h) * D + c]) + part[(2 * G + h) * D + c]) +
                    part[(3 * G + h) * D + c];
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
  hipLaunchKernelGGL(kern, dim3(a.batch * a.n_kv_heads), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((decode_update_kernel<T, D>), dim3(a.batch * a.n_kv_heads), dim3(D), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
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
