// order.hip - the order in which the attention passes visit tokens (Method steps, fourth step
// of "Block Sparse Attention with Log-Linear Complexity": attention over the selected leaf blocks).
//
// The attention kernel gathers the K and V of every selected block from memory, one wave per
// token, so its speed is set by how many of those gathers hit the L2.  Two orders are possible:
//  * the natural one, tokens in position order: consecutive tokens run on one workgroup and close
//    in time, so blocks they share stay in the L2;
//  * a selection-aware one: a pass's tokens sorted by the smallest block of the pass that is not
//    hot (hot: selected more than 4 * 64 * K times, i.e. four times the average count), and the
//    sorted order cut into eight contiguous slices, one per XCD.  Tokens that share a cold block
//    then run on the same XCD at about the same time, so the block stays in that XCD's L2.
// Which one wins depends on the selections: where consecutive tokens already share many blocks
// the natural order keeps that sharing, and sorting by one block per token destroys it.  The
// kernels below measure it on the device: the share of each token's blocks that the previous token
// also lists, over the whole call.  Below a quarter (order_sorted), the attention takes the sorted
// order, otherwise the natural one.  Which order runs changes no output bit: every token's row is
// computed by one wave from its own selection.
//
// Kernels, all on the caller's stream: clear the counters; the adjacent-token share (on every 64th
// token); count block selections (per (b, kvh), an LDS histogram per 1024 tokens flushed with
// atomics); key every token per pass and count the keys per chunk of kOrderChunk tokens; the
// prefix of each key's counts over the chunks, then of the key totals; scatter the tokens to their
// positions, a stable counting sort (ties in position order).  When the share says natural, all
// but the first two exit at once.
#include <algorithm>

#include "kernels.h"

namespace pisa {

namespace {

constexpr int kOrderThreads = 1024;         // one token per thread, a chunk of 1024 tokens per workgroup
constexpr int kOrderMaxK = 32;
constexpr int kOrderSample = 64;            // the share is measured on every 64th token

__device__ inline bool valid_entry(int j, int t) { return j >= 0 && j <= t / kLeaf; }

// Row t of (b, kvh) in registers (slots past K hold -1).
__device__ inline void load_row(const OrderArgs& a, int bh, int t, int (&r)[kOrderMaxK]) {
  const int32_t* row = a.sel + ((int64_t)bh * a.n + t) * a.top_k;
#pragma unroll
  for (int i = 0; i < kOrderMaxK; ++i) r[i] = i < a.top_k ? row[i] : -1;
}

__global__ __launch_bounds__(256) void order_clear_kernel(OrderArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < (int64_t)a.bh * a.m1) a.hist[i] = 0;
  if (i < 2) a.stats[i] = 0ull;
}

// The adjacent-token share, on every kOrderSample-th token t: for every valid entry of row t,
// whether row t - 1 lists the same block among its valid entries.  A workgroup takes 8 sampled
// tokens, 32 threads (slots) each; row t - 1 is staged in LDS.
__global__ __launch_bounds__(256) void order_share_kernel(OrderArgs a) {
  __shared__ int prev_row[8][kOrderMaxK];
  __shared__ unsigned long long red[2][256 / 64];
  const int bh = blockIdx.y;
  const int tok = threadIdx.x / kOrderMaxK, slot = threadIdx.x % kOrderMaxK;
  const int64_t t = ((int64_t)blockIdx.x * 8 + tok) * kOrderSample + 1;
  const bool live = t < a.n && slot < a.top_k;
  const int32_t* row = a.sel + ((int64_t)bh * a.n + (live ? t : 1)) * a.top_k;
  const int pj = live ? row[slot - a.top_k] : -1;               // row t - 1
  prev_row[tok][slot] = valid_entry(pj, (int)t - 1) ? pj : -1;
  __syncthreads();
  unsigned entries = 0, overlap = 0;
  const int j = live ? row[slot] : -1;
  if (live && valid_entry(j, (int)t)) {
    entries = 1;
    bool hit = false;
#pragma unroll
    for (int k = 0; k < kOrderMaxK; ++k) hit = hit || prev_row[tok][k] == j;
    overlap = hit;
  }
  unsigned long long e = entries, o = overlap;
  for (int off = 32; off > 0; off >>= 1) {
    e += __shfl_xor(e, off, 64);
    o += __shfl_xor(o, off, 64);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) { red[0][wave] = e; red[1][wave] = o; }
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long se = 0, so = 0;
    for (int w = 0; w < 256 / 64; ++w) { se += red[0][w]; so += red[1][w]; }
    if (se) {
      atomicAdd(&a.stats[0], se);
      atomicAdd(&a.stats[1], so);
    }
  }
}

// Block selection counts per (b, kvh), through an LDS histogram per chunk of tokens.
__global__ __launch_bounds__(kOrderThreads) void order_hist_kernel(OrderArgs a) {
  if (!order_sorted(a.stats)) return;
  extern __shared__ int lds_hist[];         // m1 counters
  const int bh = blockIdx.y;
  const int t = blockIdx.x * kOrderThreads + threadIdx.x;
  for (int i = threadIdx.x; i < a.m1; i += blockDim.x) lds_hist[i] = 0;
  __syncthreads();
  if (t < a.n) {
    int r[kOrderMaxK];
    load_row(a, bh, t, r);
#pragma unroll
    for (int i = 0; i < kOrderMaxK; ++i)
      if (valid_entry(r[i], t)) atomicAdd(&lds_hist[r[i]], 1);
  }
  __syncthreads();
  int32_t* hist = a.hist + (int64_t)bh * a.m1;
  for (int i = threadIdx.x; i < a.m1; i += blockDim.x)
    if (lds_hist[i]) atomicAdd(&hist[i], lds_hist[i]);
}

// Key of every token in every pass: its smallest valid block j with j % n_passes == p that is not
// hot, or m1 when the pass has none; stored, and counted per (pass, b, kvh, chunk of kOrderChunk
// tokens) through an LDS histogram.  The chunk's counts go to the key-major matrix
// keycnt[p][bh][key][chunk], every entry written.
__global__ __launch_bounds__(kOrderThreads) void order_keys_kernel(OrderArgs a) {
  if (!order_sorted(a.stats)) return;
  extern __shared__ int lds_cnt[];
  const int bh = blockIdx.y, chunk = blockIdx.x;
  const int nb = a.n_passes * (a.m1 + 1);
  for (int i = threadIdx.x; i < nb; i += blockDim.x) lds_cnt[i] = 0;
  __syncthreads();
  const int32_t* hist = a.hist + (int64_t)bh * a.m1;
  for (int r = 0; r < kOrderChunk / kOrderThreads; ++r) {
    const int t = chunk * kOrderChunk + r * kOrderThreads + threadIdx.x;
    if (t >= a.n) break;
    int row[kOrderMaxK];
    load_row(a, bh, t, row);
    int cold[kOrderMaxK];                   // the valid entries that are not hot, else m1
#pragma unroll
    for (int i = 0; i < kOrderMaxK; ++i)
      cold[i] = valid_entry(row[i], t) && hist[row[i]] <= a.hot_cut ? row[i] : a.m1;
    for (int p = 0; p < a.n_passes; ++p) {
      int key = a.m1;
#pragma unroll
      for (int i = 0; i < kOrderMaxK; ++i)
        if (cold[i] < a.m1 && cold[i] % a.n_passes == p) key = min(key, cold[i]);
      a.keys[((int64_t)p * a.bh + bh) * a.n + t] = key;
      atomicAdd(&lds_cnt[p * (a.m1 + 1) + key], 1);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nb; i += blockDim.x) {
    const int p = i / (a.m1 + 1), key = i % (a.m1 + 1);
    a.keycnt[(((int64_t)p * a.bh + bh) * (a.m1 + 1) + key) * a.n_chunks + chunk] = lds_cnt[i];
  }
}

// Per (pass, b, kvh) and key, one thread: the exclusive prefix of the key's counts over the chunks,
// in place, and the key's total.
__global__ __launch_bounds__(256) void order_prefix_kernel(OrderArgs a) {
  if (!order_sorted(a.stats)) return;
  const int64_t seg = blockIdx.y;
  const int key = blockIdx.x * blockDim.x + threadIdx.x;
  if (key > a.m1) return;
  int32_t* cnt = a.keycnt + (seg * (a.m1 + 1) + key) * a.n_chunks;
  int run = 0;
  for (int c0 = 0; c0 < a.n_chunks; c0 += 16) {
    int v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = c0 + i < a.n_chunks ? cnt[c0 + i] : 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (c0 + i < a.n_chunks) cnt[c0 + i] = run;
      run += v[i];
    }
  }
  a.keytot[seg * (a.m1 + 1) + key] = run;
}

// Per (pass, b, kvh): exclusive scan of the m1 + 1 key totals, in place (the first position of each
// key in the pass's order).
__global__ __launch_bounds__(1024) void order_keyscan_kernel(OrderArgs a) {
  if (!order_sorted(a.stats)) return;
  __shared__ int wave_sum[1024 / 64];
  int32_t* cnt = a.keytot + (int64_t)blockIdx.x * (a.m1 + 1);
  const int nb = a.m1 + 1;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = blockDim.x / 64;
  const int per = (nb + blockDim.x - 1) / blockDim.x;
  const int lo = min(nb, tid * per), hi = min(nb, lo + per);
  int local = 0;
  for (int i = lo; i < hi; ++i) local += cnt[i];
  int incl = local;
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const int v = lane < nw ? wave_sum[lane] : 0;
    int sum = v;
    for (int o = 1; o < 64; o <<= 1) {
      const int x = __shfl_up(sum, o, 64);
      if (lane >= o) sum += x;
    }
    if (lane < nw) wave_sum[lane] = sum - v;
  }
  __syncthreads();
  int run = incl - local + wave_sum[wave];
  for (int i = lo; i < hi; ++i) {
    const int c = cnt[i];
    cnt[i] = run;
    run += c;
  }
}

// Every token to its position in each pass's order: one wave per (chunk, b, kvh, pass) walks the
// chunk's tokens in position order, 64 at a time.  A token's position is the first position of its
// key, plus the chunk's offset within the key, plus the number of the chunk's earlier tokens with
// the same key: those of earlier steps are counted in LDS, those of the same step by matching the
// key bits across the wave with ballots.  Keys and bases are fetched 16 steps at a time.
__global__ __launch_bounds__(64) void order_scatter_kernel(OrderArgs a) {
  if (!order_sorted(a.stats)) return;
  extern __shared__ int lds_seen[];         // m1 + 1 counters
  const int bh = blockIdx.y, chunk = blockIdx.x, p = blockIdx.z;
  const int lane = threadIdx.x;
  const int key_bits = 32 - __builtin_clz((unsigned)a.m1);   // keys are 0 .. m1
  const uint64_t below = (1ull << lane) - 1ull;
  const int64_t seg = (int64_t)p * a.bh + bh;
  for (int i = lane; i <= a.m1; i += 64) lds_seen[i] = 0;
  wave_lds_sync();
  const int32_t* keys = a.keys + seg * a.n;
  const int32_t* local = a.keycnt + seg * (int64_t)(a.m1 + 1) * a.n_chunks + chunk;
  const int32_t* start = a.keytot + seg * (int64_t)(a.m1 + 1);
  int32_t* order = a.order + seg * a.n;
  const int t0 = chunk * kOrderChunk;
  for (int s0 = 0; s0 < kOrderChunk / 64 && t0 + s0 * 64 < a.n; s0 += 16) {
    int key[16], base[16];
    // unconditional loads from clamped indices, the values selected afterwards: loads under a
    // branch make the compiler wait for every load in flight where the paths merge
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = t0 + (s0 + i) * 64 + lane;
      const int k = keys[min(t, a.n - 1)];
      key[i] = t < a.n ? k : -1;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int kk = max(key[i], 0);
      const int b0 = start[kk] + local[(int64_t)kk * a.n_chunks];
      base[i] = key[i] >= 0 ? b0 : 0;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int t = t0 + (s0 + i) * 64 + lane;
      const bool live = key[i] >= 0;
      uint64_t same = __ballot(live);
      for (int b = 0; b < key_bits; ++b) {
        const uint64_t ones = __ballot(live && ((key[i] >> b) & 1));
        same &= ((key[i] >> b) & 1) ? ones : ~ones;
      }
      const int rank = __popcll(same & below), count = __popcll(same);
      const int seen = live ? lds_seen[key[i]] : 0;
      if (live) order[base[i] + seen + rank] = t;
      wave_lds_sync();
      if (live && rank == count - 1) lds_seen[key[i]] = seen + count;
      wave_lds_sync();
    }
  }
}

}  // namespace

size_t order_hist_lds_bytes(int m1) { return (size_t)m1 * sizeof(int); }
size_t order_keys_lds_bytes(int m1, int n_passes) { return (size_t)n_passes * (m1 + 1) * sizeof(int); }

hipError_t launch_order(const OrderArgs& a, hipStream_t s) {
  if (a.top_k > kOrderMaxK) return hipErrorInvalidValue;
  const int64_t clear = std::max<int64_t>((int64_t)a.bh * a.m1, 2);
  hipLaunchKernelGGL(order_clear_kernel, dim3((unsigned)((clear + 255) / 256)), dim3(256), 0, s, a);
  hipError_t e = launched(s);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(order_share_kernel, dim3(ceil_div(ceil_div(a.n, kOrderSample), 8), a.bh), dim3(256), 0, s, a);
  if ((e = launched(s)) != hipSuccess) return e;
  const size_t lds_hist = order_hist_lds_bytes(a.m1), lds_keys = order_keys_lds_bytes(a.m1, a.n_passes),
               lds_seen = order_hist_lds_bytes(a.m1 + 1);
  const void* kernels[3] = {(const void*)order_hist_kernel, (const void*)order_keys_kernel,
                            (const void*)order_scatter_kernel};
  const size_t lds[3] = {lds_hist, lds_keys, lds_seen};
  for (int i = 0; i < 3; ++i)
    if (lds[i] > 64 * 1024 &&
        (e = hipFuncSetAttribute(kernels[i], hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds[i])) != hipSuccess)
      return e;
  hipLaunchKernelGGL(order_hist_kernel, dim3(ceil_div(a.n, kOrderThreads), a.bh), dim3(kOrderThreads), lds_hist, s, a);
  if ((e = launched(s)) != hipSuccess) return e;
  const dim3 chunks(a.n_chunks, a.bh);
  hipLaunchKernelGGL(order_keys_kernel, chunks, dim3(kOrderThreads), lds_keys, s, a);
  if ((e = launched(s)) != hipSuccess) return e;
  hipLaunchKernelGGL(order_prefix_kernel, dim3(ceil_div(a.m1 + 1, 256), a.n_passes * a.bh), dim3(256), 0, s, a);
  if ((e = launched(s)) != hipSuccess) return e;
  hipLaunchKernelGGL(order_keyscan_kernel, dim3(a.n_passes * a.bh), dim3(1024), 0, s, a);
  if ((e = launched(s)) != hipSuccess) return e;
  hipLaunchKernelGGL(order_scatter_kernel, dim3(a.n_chunks, a.bh, a.n_passes), dim3(64), lds_seen, s, a);
  return launched(s);
}

}  // namespace pisa
