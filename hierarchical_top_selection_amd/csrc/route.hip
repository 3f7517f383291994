// route.hip - Stage 1 of hierarchical selection: top-down routing through the
// pyramid levels above the leaves (Core method eq. 16-21; Method steps eq. 22 of
// "Block Sparse Attention with Log-Linear Complexity").
//
// One wave routes one (b, kvh, token).  The candidates' children are gathered 16
// at a time as the rows of an MFMA A tile and the group's G query heads are the
// columns of the B tile (columns >= G are zero), so one MFMA pass yields the
// logits of every head against 16 children, and a candidate's two children land
// in the same lane.  Candidate lists never leave registers: lane
// i owns candidate i, a level keeps K of them by exact rank (score descending,
// node index ascending) and the survivors expand into the next list with a
// ballot/bit-select compaction.  The leaf candidates (at most 2K per token) are
// the output, and for bf16 inputs the query rows it loads are also stored in the
// leaf stage's packed query layout.
//
// Scores need close to single precision (near-ties between candidates are
// common).  fp32 queries use fp32 summaries on v_mfma_f32_16x16x4_f32.  For
// bf16 queries each fp32 summary x is split once into hi = bf16(x) and lo =
// f16((x - hi) 2^10) (the remainder's 8 + 11 bits leave a relative error of
// about 2^-20 per element), and q . x = q . hi + 2^-10 q . lo runs on the
// 16-cycle bf16 and f16 16x16x32 MFMAs: 8 instead of 32 fp32 MFMAs per tile,
// from the same 4 bytes per element.  q . hi uses the bf16 query as it is.  The
// remainder product takes the query in f16, which holds a bf16 value exactly
// for 2^-14 <= |q| <= 65504; smaller values become f16 subnormals (absolute
// error <= 2^-25, so at most 2^-35 |lo| per element after the 2^-10 factor) and
// larger ones are clamped to 65504 (an error of at most 2^-10 |lo| (|q| - 65504)
// per element, reached only by queries far outside any trained model's range).  The kernel
// gathers summary rows (8 KB per 16-child tile), so each tile's rows are
// requested one tile ahead.  The LSE of a candidate's two children is evaluated
// in base 2 as max + log2(1 + 2^-|diff|) on pre-scaled logits; the mean and mean + var/2 score
// variants (PISA-1 / PISA-2) from the same two logits in natural units.
#include "kernels.h"

namespace pisa {

// ----------------------------------------------------------------------------- operands
// Query operands (B tile columns) and summary tiles (A tile rows) of one precision.
template <typename T, int D> struct RouteOps;

// Tile::load(a, rows, li, child, g): row `child` of pyramid level li + 1 for lane group g.
template <int D> struct RouteOps<float, D> {         // fp32 summaries, fp32 MFMA
  typedef float Row;
  struct Q { FragF32<D> f; };
  struct Tile {
    FragF32<D> f;
    __device__ inline void load(const RouteArgs& a, const Row* rows, int li, int child, int g) {
      f.load(rows + (a.lv.offset[li] + child) * D, g);
    }
  };
  __device__ static inline void load_q(Q& q, const float* row, int g) { q.f.load(row, g); }
  __device__ static inline void zero_q(Q& q) { q.f.zero(); }
  __device__ static inline const Row* rows(const RouteArgs& a, int bh) { return a.pyr + (int64_t)bh * a.lv.nodes * D; }
  __device__ static inline floatx4 dot(const Tile& t, const Q& q) {
    return mma(t.f, q.f, floatx4{0.f, 0.f, 0.f, 0.f});
  }
};

template <int D> struct RouteOps<__bf16, D> {        // bf16 high part + f16 remainder
  typedef uint16_t Row;
  struct Q { FragBF16<D> h; FragF16<D> l; };
  struct Tile {
    FragBF16<D> h;
    FragF16<D> l;
    // tile rows 2 i, 2 i + 1 are the two children of one candidate, so each fragment
    // load covers whole 128-byte lines of the pair blocks
    __device__ inline void load(const RouteArgs& a, const Row* rows, int li, int child, int g) {
      // uniform level base plus a 32-bit per-lane offset (a level's pair blocks span far less than 4 GB)
      const Row* r = rows + a.pair_off[li] * (4 * D) + (uint32_t)((child >> 1) * (4 * D) + 32 * (child & 1) + 8 * g);
#pragma unroll
      for (int s = 0; s < D / 32; ++s) {
        h.v[s] = *reinterpret_cast<const bf16x8*>(r + 64 * s);
        l.v[s] = *reinterpret_cast<const f16x8*>(r + 64 * (D / 32 + s));
      }
    }
  };
  // the remainder product's f16 copy of the query: exact for 2^-14 <= |q| <= 65504, subnormal
  // below (absolute error <= 2^-25), clamped above
  __device__ static inline void load_q(Q& q, const __bf16* row, int g) {
    q.h.load(row, g);
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) q.l.v[s][j] = (_Float16)fminf(fmaxf((float)q.h.v[s][j], -65504.f), 65504.f);
  }
  __device__ static inline void zero_q(Q& q) {
    q.h.zero();
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) q.l.v[s][j] = (_Float16)0.f;
  }
  __device__ static inline const Row* rows(const RouteArgs& a, int bh) { return a.split + (int64_t)bh * a.pairs * (4 * D); }
  __device__ static inline floatx4 dot(const Tile& t, const Q& q) {
    const floatx4 hi = mma(t.h, q.h, floatx4{0.f, 0.f, 0.f, 0.f});
    const floatx4 lo = mma(t.l, q.l, floatx4{0.f, 0.f, 0.f, 0.f});
    return hi + lo * 0.0009765625f;                   // 2^-10
  }
};

// Fills the pair blocks of the split layout (RouteArgs): one thread per 16-byte piece q of a
// block, q = 8 line + 4 c + g with elements [32 s + 8 g, +8) of node 2p + c (zero past the
// level's end).  hi = bf16(x) to nearest; the remainder x - hi is exact in fp32, is scaled by
// 2^10 and rounded to the nearest f16 after clamping to its range.
// For the routing pre-filter it also writes the float16 copy x16 = f16(x) (clamped to the f16
// range; plane-0 threads write the piece of their eight elements) and, per node, the bounds R and
// X of route_prefilter_kernel from five sums of squares over the node's d elements: plane-0
// threads add xi = x - x16, hi and x16, plane-1 threads rho = (x - hi) - lo 2^-10 (the remainder's
// own rounding) and lo 2^-10.  The kPieces threads of a block are one aligned group of lanes, so
// the per-node sums are xor reductions within it.
template <int D>
__global__ __launch_bounds__(256) void split_summaries_kernel(RouteArgs a) {
  constexpr int kPieces = D / 2;                      // 16-byte pieces per pair block
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t blk = e / kPieces;                    // bh * pairs + pair
  if (blk >= (int64_t)a.batch * a.n_kv_heads * a.pairs) return;
  const int q = (int)(e % kPieces);
  const int bh = (int)(blk / a.pairs);
  const int64_t pr = blk % a.pairs;
  int li = 0;
  while (li + 1 < a.lv.count && pr >= a.pair_off[li + 1]) ++li;
  const int c = (q >> 2) & 1;
  const int64_t node = 2 * (pr - a.pair_off[li]) + c;
  const int line = q >> 3, g = q & 3;
  const int plane = line / (D / 32), s = line % (D / 32);
  uint4 out = make_uint4(0u, 0u, 0u, 0u), out16 = make_uint4(0u, 0u, 0u, 0u);
  float sq[5] = {0.f, 0.f, 0.f, 0.f, 0.f};            // xi, hi, x16 (plane 0) | rho, lo (plane 1)
  if (node < a.lv.size[li]) {
    const float* src = a.pyr + ((int64_t)bh * a.lv.nodes + a.lv.offset[li] + node) * D + 32 * s + 8 * g;
    const float4 x0 = *reinterpret_cast<const float4*>(src);
    const float4 x1 = *reinterpret_cast<const float4*>(src + 4);
    const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
    bf16x8 hi;
    f16x8 lo, x16;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      hi[j] = (__bf16)x[j];
      const float r = (x[j] - (float)hi[j]) * 1024.f;
      lo[j] = (_Float16)fminf(fmaxf(r, -65504.f), 65504.f);
      x16[j] = (_Float16)fminf(fmaxf(x[j], -65504.f), 65504.f);
      if (plane == 0) {
        const float xi = x[j] - (float)x16[j], h = (float)hi[j], y = (float)x16[j];
        sq[0] = fmaf(xi, xi, sq[0]);
        sq[1] = fmaf(h, h, sq[1]);
        sq[2] = fmaf(y, y, sq[2]);
      } else {
        const float l = (float)lo[j] * 0.0009765625f;  // 2^-10, exact
        const float rho = (x[j] - (float)hi[j]) - l;
        sq[3] = fmaf(rho, rho, sq[3]);
        sq[4] = fmaf(l, l, sq[4]);
      }
    }
    out = plane == 0 ? __builtin_bit_cast(uint4, hi) : __builtin_bit_cast(uint4, lo);
    out16 = __builtin_bit_cast(uint4, x16);
  }
  *reinterpret_cast<uint4*>(a.split + e * 8) = out;
  if (plane == 0) *reinterpret_cast<uint4*>(a.split16 + (blk * (kPieces / 2) + q) * 8) = out16;
  float n0[5], n1[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    n0[i] = c == 0 ? sq[i] : 0.f;
    n1[i] = c == 1 ? sq[i] : 0.f;
  }
#pragma unroll
  for (int off = 1; off < kPieces; off <<= 1)
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      n0[i] += __shfl_xor(n0[i], off, 64);
      n1[i] += __shfl_xor(n1[i], off, 64);
    }
  if (q == 0) {
    // a sum of d squares rounds by less than 2^-17 relative and sqrt by an ulp: 2^-15 covers both
    float* bnd = a.bounds + blk * 4;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const float* n = k == 0 ? n0 : n1;
      const float xi = __builtin_sqrtf(n[0]), hn = __builtin_sqrtf(n[1]), x16n = __builtin_sqrtf(n[2]);
      const float rho = __builtin_sqrtf(n[3]), lon = __builtin_sqrtf(n[4]);
      bnd[2 * k] = (rho + xi) * 1.0000306f + 0x1p-15f * 1.01f * (hn + lon + x16n) + 0x1p-60f;   // R
      bnd[2 * k + 1] = (lon + x16n) * 1.0000306f + 0x1p-60f;                                  // X
    }
  }
}

// The levels from the root down keep every causally valid node while there are at most K of them.
// Returns the first level with more than K valid nodes (1 if none: the valid leaves are then the
// candidates) and that level's valid count: its candidates are nodes 0 .. count - 1, in the order
// the expansions above it would list them.
__device__ inline int first_scored_level(const RouteArgs& a, int t, int& n_valid) {
  int level = a.lv.count;
  for (;;) {
    n_valid = (int)min((int64_t)a.lv.size[level - 1], ((int64_t)t >> (level - 1)) / kLeaf + 1);
    if (level == 1 || n_valid > a.top_k) return level;
    --level;
  }
}

// ----------------------------------------------------------------------------- routing
// kScore: the candidate score (pisa_score), fixed per instantiation so only its code is live.
template <typename T, int D, int kScore>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void route_kernel(RouteArgs a) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.n) return;
  const int bh = blockIdx.y;
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int g = lane >> 4, col = lane & 15;
  const int width = 2 * a.top_k;
  const float c2 = a.scale * 1.4426950408889634f;       // logits in base-2 units

  typedef RouteOps<T, D> Ops;
  typename Ops::Q qf;
  if (col < a.group) {
    const T* qrow = reinterpret_cast<const T*>(a.q) + b * a.q_sb + (int64_t)t * a.q_st +
                    (int64_t)(kvh * a.group + col) * a.q_sh;
    Ops::load_q(qf, qrow, g);
    if constexpr (sizeof(T) == 2) {
      if (a.qpack) {                                   // the leaf stage's packed copy of this query group
        bf16x8* dst = a.qpack + ((int64_t)bh * a.n + t) * (a.group * D / 8) + g * a.group + col;
#pragma unroll
        for (int s = 0; s < D / 32; ++s) dst[4 * s * a.group] = qf.h.v[s];
      }
    }
  } else {
    Ops::zero_q(qf);
  }
  const typename Ops::Row* rows = Ops::rows(a, bh);

  int n_first;
  const int first = first_scored_level(a, t, n_first);
  int cand = lane < n_first ? lane : -1;              // every valid node of the first scored level
  for (int level = first; level >= 2; --level) {
    const uint64_t valid = __ballot(cand >= 0);
    const int n_valid = __popcll(valid);
    const int child_size = a.lv.size[level - 2];
    bool keep = cand >= 0;
    if (n_valid > a.top_k) {
      const int span = 64 - __clzll(valid);            // highest occupied lane + 1
      // an even tile count, so the double-buffered loop below has no conditional half; a padding
      // tile only scores empty candidate lanes, whose keys are 0
      const int tiles = (((2 * span + 15) / 16) + 1) & ~1;
      // child of tile nt owned by this lane's row index: candidate slot/2, child slot&1.  Rows of
      // invalid children load a clamped row and are masked.
      auto child_of = [&](int nt, bool& ok) {
        const int slot = 16 * nt + col;
        const int parent = __shfl(cand, slot >> 1, 64);
        const int child = 2 * parent + (slot & 1);
        ok = parent >= 0 && child < child_size && node_first_key(level - 1, child) <= t;
        return ok ? child : 0;
      };
      float u = kNegInf;                               // score of candidate `lane` (base 2)
      // Tiles are double-buffered without copies: tile nt computes from `cur` while tile nt + 1's
      // rows are requested into `nxt` (the last tile requests its own rows again, so every load
      // is unconditional).  The compiler may still sink those loads below the products to save
      // registers; pinning them with a scheduling barrier measured slower (3.2 -> 3.85 ms at
      // N = 262144), so they are left to it.
      auto do_tile = [&](int nt, typename Ops::Tile& cur, typename Ops::Tile& nxt, bool& ok_cur) {
        // rows 4g .. 4g+3 of the tile hold this lane's results: bits 4g .. 4g+3 of the ballot.  A
        // candidate's first child is valid whenever the candidate is (its first key is the
        // candidate's own), so only the second child of each pair is tested; padding candidates
        // score finite garbage and never rank (their key is 0).
        const uint32_t rows_ok = (uint32_t)__ballot(ok_cur) >> (4 * g);
        bool ok_n;
        const int child_n = child_of(min(nt + 1, tiles - 1), ok_n);
        nxt.load(a, rows, level - 2, child_n, g);
        ok_cur = ok_n;
        // S^T tile: rows = 16 children, columns = heads; lane (g, col) gets children 4g + i of head col
        const floatx4 acc = Ops::dot(cur, qf);
        float pscore[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {                  // candidate 8 nt + 2g + h: children rows 4g + 2h, +1
          const float sc = pair_score(acc[2 * h], acc[2 * h + 1], true, (rows_ok >> (2 * h + 1)) & 1u,
                                      kScore, a.scale, c2);
          pscore[h] = row_sum_to_last(col < a.group ? sc : 0.f);   // sum over the group's heads
        }
        // lane 16 g + 15 holds candidates 8 nt + 2 g and 8 nt + 2 g + 1
        const int src = 16 * ((lane & 7) >> 1) + 15;
        const float s0 = __shfl(pscore[0], src, 64);
        const float s1 = __shfl(pscore[1], src, 64);
        if ((lane >> 3) == nt) u = (lane & 1) ? s1 : s0;
      };
      bool ok_t;
      typename Ops::Tile ta, tb;
      ta.load(a, rows, level - 2, child_of(0, ok_t), g);
      for (int nt = 0; nt < tiles; nt += 2) {
        do_tile(nt, ta, tb, ok_t);
        do_tile(nt + 1, tb, ta, ok_t);
      }
      // exact rank among the candidates by (score descending, index ascending), as one 64-bit key:
      // the score's bits made order-preserving above the complemented index; empty lanes are 0,
      // below every candidate.  Lane j's key is read into scalar registers.
      const uint32_t ubits = __builtin_bit_cast(uint32_t, u + 0.f);          // -0 compares as +0
      const uint32_t khi = cand >= 0 ? ((ubits & 0x80000000u) ? ~ubits : (ubits | 0x80000000u)) : 0u;
      const uint32_t klo = cand >= 0 ? 0xffffffffu - (uint32_t)cand : 0u;
      const uint64_t key = ((uint64_t)khi << 32) | klo;
      // lanes past `span` hold key 0 and never count, so the loop runs to a multiple of 4
      auto key_of = [&](int j) {
        return ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(khi, j) << 32) |
               (uint64_t)(uint32_t)__builtin_amdgcn_readlane(klo, j);
      };
      int r0 = 0, r1 = 0, r2 = 0, r3 = 0;
      for (int j = 0; j < span; j += 4) {
        r0 += (int)(key_of(j) > key);
        r1 += (int)(key_of(j + 1) > key);
        r2 += (int)(key_of(j + 2) > key);
        r3 += (int)(key_of(j + 3) > key);
      }
      const int rank = r0 + r1 + r2 + r3;
      keep = cand >= 0 && rank < a.top_k;
    }
    // expand the survivors into their causally valid children
    const uint64_t kept = __ballot(keep);
    const int m = __popcll(kept);
    const int p = lane >> 1;
    const int src = nth_set_bit(kept, p < m ? p : 0);
    const int parent = __shfl(cand, src, 64);
    const int child = 2 * parent + (lane & 1);
    cand = (p < m && child < child_size && node_first_key(level - 1, child) <= t) ? child : -1;
  }
  if (lane < width) a.cand[((int64_t)bh * a.n + t) * width + lane] = cand;
}

// ----------------------------------------------------------------------------- routing with a pre-filter
// bf16 inputs, every score.  Each scored level first scores its candidates from a float16 copy of the
// summaries (half the bytes of the split rows, half the products) and bounds, per candidate, how
// far route_kernel's score from the split rows can lie from that estimate.  Only candidates whose
// interval straddles the K-th place are scored again from the split rows, with route_kernel's
// arithmetic, so the kept set is route_kernel's:
//  * per child and head, with q the bf16 query, q_lo its f16 copy (eps = q - q_lo), x the node,
//    hi, lo its split parts, rho = (x - hi) - lo 2^-10, x16 = f16(x), xi = x - x16, and g = 2^-15
//    a bound on the relative error of a float32 sum of d <= 128 products (132 additions at most,
//    each off by 2^-23 even when truncating):
//      |y_split - q.x| <= |q| (|rho| + g (|hi| + |lo 2^-10|)) + |eps| |lo 2^-10| + 2^-24 |y_split|,
//      |y_16 - q.x| <= |q| (|xi| + g |x16|) + |eps| |x16|   (Cauchy-Schwarz, Euclidean norms),
//    so |y_split - y_16| <= |q| R + |eps| X (1 + g) + 2^-24 |y_split| with the per-node bounds
//    R = |rho| + |xi| + g (|hi| + |lo 2^-10| + |x16|) and X = |lo 2^-10| + |x16| of
//    split_summaries_kernel (rounded up), and the query norms rounded up here;
//  * the pair LSE moves by at most its larger logit change (its gradient is a probability vector)
//    and the head sum by the sum over heads.  R and X are the same for every head, so the sum over
//    heads only needs QN = sum |q_h| and QD = sum |eps_h| of the token, and a candidate lane bounds
//    its score from the (R, X) of its two children alone.  The rounding differences of the logit
//    scaling, the exp2/log2 evaluation and the head sum are at most 2^-20 (|z0| + |z1| + 1) per
//    head, with |z_i| <= c2 (|q_h| + |eps_h|) X_i (1 + g);
//  * the mean of two logits (PISA-1) also moves by at most the larger change; the added half variance
//    (PISA-2) h^2 / 2 with h = (a - b) / 2 by at most |h| |dh| + dh^2 / 2 with |dh| <= scale max_i |dy_i|,
//    which needs the sums over heads of |q_h| |h_h| and |eps_h| |h_h| per candidate (two more head
//    sums in the tile loop), and its rounding 2^-21 h^2 per head more, h^2 <= (scale (|q_h| +
//    |eps_h|) (X0 + X1) / 2)^2;
//  * with L = u - E and U = u + E around the estimate u: a candidate whose L exceeds the (K+1)-th
//    largest U is in the split score's top K, one whose U is below the K-th largest L is not, and the
//    rest are scored again and fill the remaining places by (score, then lower index).  Should the
//    bounds ever leave a count that cannot be right, every candidate of the level is scored again.

// The largest threshold that at least k lanes' keys reach (the k-th largest key), one ballot per bit.
__device__ inline uint32_t kth_key(uint32_t key, int k) {
  uint32_t thr = 0;
#pragma unroll
  for (int bit = 31; bit >= 0; --bit) {
    const uint32_t trial = thr | (1u << bit);
    if (__popcll(__ballot(key >= trial)) >= k) thr = trial;
  }
  return thr;
}

template <int D>
struct F16Tile {                                     // the float16 copy of 16 child rows
  FragF16<D> f;
  __device__ inline void load(const RouteArgs& a, const uint16_t* rows16, int li, int child, int g) {
    const uint16_t* r = rows16 + a.pair_off[li] * (2 * D) + (uint32_t)((child >> 1) * (2 * D) + 32 * (child & 1) + 8 * g);
#pragma unroll
    for (int s = 0; s < D / 32; ++s) f.v[s] = *reinterpret_cast<const f16x8*>(r + 64 * s);
  }
};

template <int D, int kScore>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void route_prefilter_kernel(RouteArgs a) {
  const int lane = threadIdx.x & 63, wave = wave_id();
  const int t = blockIdx.x * 4 + wave;
  if (t >= a.n) return;
  const int bh = blockIdx.y;
  const int b = bh / a.n_kv_heads, kvh = bh % a.n_kv_heads;
  const int g = lane >> 4, col = lane & 15;
  const int width = 2 * a.top_k, K = a.top_k;
  const float c2 = a.scale * 1.4426950408889634f;       // logits in base-2 units
  const bool head_ok = col < a.group;

  typedef RouteOps<__bf16, D> Ops;
  typename Ops::Q qf;
  float qsq = 0.f, qdsq = 0.f;                         // this lane's parts of |q|^2 and |q - q_lo|^2
  if (head_ok) {
    const __bf16* qrow = reinterpret_cast<const __bf16*>(a.q) + b * a.q_sb + (int64_t)t * a.q_st +
                         (int64_t)(kvh * a.group + col) * a.q_sh;
    Ops::load_q(qf, qrow, g);
    if (a.qpack) {                                     // the leaf stage's packed copy of this query group
      bf16x8* dst = a.qpack + ((int64_t)bh * a.n + t) * (a.group * D / 8) + g * a.group + col;
#pragma unroll
      for (int s = 0; s < D / 32; ++s) dst[4 * s * a.group] = qf.h.v[s];
    }
#pragma unroll
    for (int s = 0; s < D / 32; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float x = (float)qf.h.v[s][j], dx = x - (float)qf.l.v[s][j];
        qsq = fmaf(x, x, qsq);
        qdsq = fmaf(dx, dx, qdsq);
      }
  } else {
    Ops::zero_q(qf);
  }
  qsq += __shfl_xor(qsq, 16, 64);
  qsq += __shfl_xor(qsq, 32, 64);
  qdsq += __shfl_xor(qdsq, 16, 64);
  qdsq += __shfl_xor(qdsq, 32, 64);
  // |q|_2 and |q - q_lo|_2 of this lane's head, rounded up (sum and sqrt rounding below 2^-16)
  const float qn = __builtin_sqrtf(qsq) * 1.0000153f + 0x1p-60f;
  const float qd = __builtin_sqrtf(qdsq) * 1.0000153f + 0x1p-60f;
  // QN = sum over the group's heads of |q_h|, QD of |eps_h| (sums of positive terms, rounded up)
  const float qn_sum = row_sum_to_last(head_ok ? qn : 0.f), qd_sum = row_sum_to_last(head_ok ? qd : 0.f);
  const float QN = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, qn_sum), 15)) * 1.000001f;
  const float QD = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, qd_sum), 15)) * 1.000001f;
  const float cs = kScore == 0 ? c2 : a.scale;        // score units per logit: base 2 (LSE) or natural
  float Q2 = 0.f;                                      // mean + var / 2: sum over heads of (|q_h| + |eps_h|)^2
  if constexpr (kScore == 2) {
    const float q2_sum = row_sum_to_last(head_ok ? (qn + qd) * (qn + qd) : 0.f);
    Q2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, q2_sum), 15)) * 1.000001f;
  }
  const uint16_t* rows = a.split + (int64_t)bh * a.pairs * (4 * D);
  const uint16_t* rows16 = a.split16 + (int64_t)bh * a.pairs * (2 * D);
  const float4* bounds = reinterpret_cast<const float4*>(a.bounds) + (int64_t)bh * a.pairs;

  int n_first;
  const int first = first_scored_level(a, t, n_first);
  int cand = lane < n_first ? lane : -1;              // every valid node of the first scored level
  for (int level = first; level >= 2; --level) {
    const uint64_t valid = __ballot(cand >= 0);
    const int n_valid = __popcll(valid);
    const int child_size = a.lv.size[level - 2];
    bool keep = cand >= 0;
    auto child_ok = [&](int parent, int child) {
      return parent >= 0 && child < child_size && node_first_key(level - 1, child) <= t;
    };
    if (n_valid > K) {
      const int span = 64 - __clzll(valid);
      const int tiles = (((2 * span + 15) / 16) + 1) & ~1;
      auto child_of = [&](int nt, bool& ok) {
        const int slot = 16 * nt + col;
        const int parent = __shfl(cand, slot >> 1, 64);
        const int child = 2 * parent + (slot & 1);
        ok = child_ok(parent, child);
        return ok ? child : 0;
      };
      // (R0, X0, R1, X1) of this lane's candidate's two children, for its bound after the tiles
      const float4 b4 = bounds[a.pair_off[level - 2] + (cand >= 0 ? cand : 0)];
      float u = kNegInf;                               // estimate of candidate `lane`
      float hq = 0.f, he = 0.f;                        // mean + var / 2: sums over heads of |q_h| |h_h|, |eps_h| |h_h|
      auto do_tile = [&](int nt, F16Tile<D>& cur, F16Tile<D>& nxt, bool& ok_cur) {
        const uint32_t rows_ok = (uint32_t)__ballot(ok_cur) >> (4 * g);
        bool ok_n;
        const int child_n = child_of(min(nt + 1, tiles - 1), ok_n);
        nxt.load(a, rows16, level - 2, child_n, g);
        ok_cur = ok_n;
        const floatx4 acc = mma(cur.f, qf.l, floatx4{0.f, 0.f, 0.f, 0.f});
        float ps[2], pq[2], pe[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool ok1 = (rows_ok >> (2 * h + 1)) & 1u;
          const float sc = pair_score(acc[2 * h], acc[2 * h + 1], true, ok1, kScore, a.scale, c2);
          ps[h] = row_sum_to_last(head_ok ? sc : 0.f);
          if constexpr (kScore == 2) {
            const float hh = head_ok && ok1 ? 0.5f * fabsf(acc[2 * h] - acc[2 * h + 1]) * a.scale : 0.f;
            pq[h] = row_sum_to_last(qn * hh);
            pe[h] = row_sum_to_last(qd * hh);
          }
        }
        const int src = 16 * ((lane & 7) >> 1) + 15;
        const float s0 = __shfl(ps[0], src, 64), s1 = __shfl(ps[1], src, 64);
        if ((lane >> 3) == nt) u = (lane & 1) ? s1 : s0;
        if constexpr (kScore == 2) {
          const float q0 = __shfl(pq[0], src, 64), q1 = __shfl(pq[1], src, 64);
          const float e0 = __shfl(pe[0], src, 64), e1 = __shfl(pe[1], src, 64);
          if ((lane >> 3) == nt) {
            hq = (lane & 1) ? q1 : q0;
            he = (lane & 1) ? e1 : e0;
          }
        }
      };
      bool ok_t;
      F16Tile<D> ta, tb;
      ta.load(a, rows16, level - 2, child_of(0, ok_t), g);
      for (int nt = 0; nt < tiles; nt += 2) {
        do_tile(nt, ta, tb, ok_t);
        do_tile(nt + 1, tb, ta, ok_t);
      }
      // E: the sum over heads of c2 max_i (|q_h| R_i + |eps_h| X_i (1 + 2^-15) + 2^-24 |y_i|) (1 + 2^-23),
      // with |y_i| <= (|q_h| + |eps_h|) X_i (1 + g), plus the rounding slack 2^-20 (|z0| + |z1| + 1)
      // per head, here doubled
      // (c2 in base-2 units for the LSE, the scale for the mean variants; the mean of two logits moves by
      // at most their larger change, like the LSE)
      const float rmax = fmaxf(b4.x, b4.z), xmax = fmaxf(b4.y, b4.w);
      const float dsum = rmax * QN + xmax * (QD * 1.0001f + 0x1p-23f * (QN + QD));
      float E = cs * 1.001f * dsum + 0x1p-19f * (cs * (QN + QD) * (b4.y + b4.w) * 1.001f + (float)a.group) + 0x1p-40f;
      if constexpr (kScore == 2) {
        // sum over heads of |h| |dh| <= scale (R_max hq + X_max (1 + 2^-13) he + 2^-23 (X0 + X1) (hq + he)),
        // of dh^2 / 2 <= (scale dsum)^2 / 2; the rounding of h^2 / 2
        const float sx = a.scale * (b4.y + b4.w);
        E += a.scale * 1.001f * (rmax * hq + xmax * 1.0002f * he + 0x1p-23f * (b4.y + b4.w) * (hq + he)) +
             0.5f * (cs * 1.001f * dsum) * (cs * 1.001f * dsum) + 0x1p-19f * 0.25f * sx * sx * Q2;
      }
      // the interval [u - E', u + E'] holds route_kernel's score (E' also covers rounding here)
      const bool vc = cand >= 0;
      const float Ep = E * 1.0000003f + 0x1p-20f * fabsf(u) + 0x1p-40f;
      const uint32_t kl = score_key(u - Ep, vc), ku = score_key(u + Ep, vc);
      const uint32_t tl = kth_key(kl, K), tu = kth_key(ku, K + 1);
      const bool in = vc && kl > tu;                   // in the top K whatever the full scores
      const bool undecided = vc && !in && !(ku < tl);
      const int n_in = __popcll(__ballot(in));
      const uint64_t und = __ballot(undecided);
      if (!(und == 0 && n_in == K)) {                  // wave-uniform
        const bool redo_all = und == 0 || n_in > K;
        const bool again = redo_all ? vc : undecided;
        const uint64_t am = __ballot(again);
        const int places = redo_all ? K : K - n_in;
        keep = redo_all ? false : in;
        if (places > 0) {
          // the candidates to score again, compacted into lanes 0 .. n_again - 1
          const int n_again = __popcll(am);
          const int src_lane = nth_set_bit(am, lane < n_again ? lane : 0);
          const int cs = __shfl(cand, src_lane, 64);
          const int rc = lane < n_again ? cs : -1;
          float ur = kNegInf;
          const int rtiles = (2 * n_again + 15) / 16;
          for (int nt = 0; nt < rtiles; ++nt) {
            const int slot = 16 * nt + col;
            const int parent = __shfl(rc, slot >> 1, 64);
            const int child = 2 * parent + (slot & 1);
            const bool ok = child_ok(parent, child);
            typename Ops::Tile tile;
            tile.load(a, rows, level - 2, ok ? child : 0, g);
            const uint32_t rows_ok = (uint32_t)__ballot(ok) >> (4 * g);
            const floatx4 acc = Ops::dot(tile, qf);
            float pscore[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const float sc = pair_score(acc[2 * h], acc[2 * h + 1], true, (rows_ok >> (2 * h + 1)) & 1u, kScore,
                                          a.scale, c2);
              pscore[h] = row_sum_to_last(head_ok ? sc : 0.f);
            }
            const int src = 16 * ((lane & 7) >> 1) + 15;
            const float s0 = __shfl(pscore[0], src, 64), s1 = __shfl(pscore[1], src, 64);
            if ((lane >> 3) == nt) ur = (lane & 1) ? s1 : s0;
          }
          // back to the candidates' lanes: candidate lane i is entry mbcnt(am below i)
          const int j = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(am >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)am, 0u));
          const float ux = __shfl(ur, again ? j : 0, 64);
          const bool best = keep_top_k(score_key(ux, again), places);   // the whole wave votes
          keep = keep || (again && best);
        }
      } else {
        keep = in;
      }
    }
    // expand the survivors into their causally valid children
    const uint64_t kept = __ballot(keep);
    const int m = __popcll(kept);
    const int p = lane >> 1;
    const int src = nth_set_bit(kept, p < m ? p : 0);
    const int parent = __shfl(cand, src, 64);
    const int child = 2 * parent + (lane & 1);
    cand = (p < m && child < child_size && node_first_key(level - 1, child) <= t) ? child : -1;
  }
  if (lane < width) a.cand[((int64_t)bh * a.n + t) * width + lane] = cand;
}

template <typename T, int D>
hipError_t launch_route_t(const RouteArgs& a, hipStream_t s) {
  dim3 grid(ceil_div(a.n, 4), a.batch * a.n_kv_heads);
  if constexpr (sizeof(T) == 2) {
    if (a.prefilter) {
      if (a.score == 1)
        hipLaunchKernelGGL((route_prefilter_kernel<D, 1>), grid, dim3(256), 0, s, a);
      else if (a.score == 2)
        hipLaunchKernelGGL((route_prefilter_kernel<D, 2>), grid, dim3(256), 0, s, a);
      else
        hipLaunchKernelGGL((route_prefilter_kernel<D, 0>), grid, dim3(256), 0, s, a);
      return launched(s);
    }
  }
  if (a.score == 1)
    hipLaunchKernelGGL((route_kernel<T, D, 1>), grid, dim3(256), 0, s, a);
  else if (a.score == 2)
    hipLaunchKernelGGL((route_kernel<T, D, 2>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((route_kernel<T, D, 0>), grid, dim3(256), 0, s, a);
  return launched(s);
}

hipError_t launch_split_summaries(const RouteArgs& a, hipStream_t s) {
  const int64_t threads = (int64_t)a.batch * a.n_kv_heads * a.pairs * (a.head_dim / 2);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (a.head_dim == 64)
    hipLaunchKernelGGL(split_summaries_kernel<64>, dim3(blocks), dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(split_summaries_kernel<128>, dim3(blocks), dim3(256), 0, s, a);
  return launched(s);
}

hipError_t launch_route(const RouteArgs& a, hipStream_t s) {
  if (a.bf16) return a.head_dim == 64 ? launch_route_t<__bf16, 64>(a, s) : launch_route_t<__bf16, 128>(a, s);
  return a.head_dim == 64 ? launch_route_t<float, 64>(a, s) : launch_route_t<float, 128>(a, s);
}

}  // namespace pisa
