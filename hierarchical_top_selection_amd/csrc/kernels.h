// kernels.h - host-visible argument blocks and launchers of the gfx950 kernels.
// Strides are in elements; every launcher enqueues on the given stream and
// returns the launch status (nothing is synchronised).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pisa_device.h"

namespace pisa {

struct PyramidArgs {
  const void* k;
  int64_t k_sb, k_st, k_sh;
  float* pyr;
  int batch, n_kv_heads, head_dim, n;
  bool bf16;
  Levels lv;          // sizes for length n, offsets for the capacity layout
};

struct RouteArgs {
  const void* q;
  int64_t q_sb, q_st, q_sh;
  const float* pyr;
  // bf16 inputs: split summaries (bf16 high part, f16 remainder scaled by 2^10) by child
  // pairs: nodes 2p, 2p + 1 of a level form a block of 8 d bytes at pair_off[level - 1] + p
  // (per b * Hkv: `pairs` blocks).  Line (plane, s), plane 0 = high / 1 = remainder, s < d / 32,
  // is 128 bytes: elements [32 s, 32 s + 32) of node 2p, then of node 2p + 1.
  uint16_t* split;
  // bf16 inputs, for the routing pre-filter: a float16 copy of the summaries, one plane of the
  // same pair-block layout (2 d elements per block: line s holds elements [32 s, 32 s + 32) of node
  // 2p, then of node 2p + 1), and per node two bounds (R, X) at ((b * Hkv * pairs + pair) * 2 +
  // (node & 1)) * 2 (split_summaries_kernel writes both; route.hip states what they bound)
  uint16_t* split16;
  float* bounds;
  int64_t pair_off[kMaxLevels];
  int64_t pairs;
  int32_t* cand;      // [B*Hkv][N][2K] leaf candidates, -1 padded
  // bf16 inputs: packed query groups, written on the way (or null).  The G heads of (b, kvh) at
  // token t occupy G d / 8 sixteen-byte pieces at ((b * Hkv + kvh) * N + t) * G d / 8; piece
  // (s, g, col), s < d / 32, g < 4, col < G, at (4 s + g) * G + col holds elements
  // [32 s + 8 g, +8) of head kvh * G + col, so the MFMA B fragment of a query (lane 16 g + col)
  // is one contiguous run.
  bf16x8* qpack;
  int batch, n_kv_heads, group, head_dim, n, top_k;
  int score;          // 0 LSE, 1 mean, 2 mean + var / 2 (pisa_score)
  float scale;
  bool bf16;
  bool prefilter;     // bf16 routing: score from the float16 copy first (route_prefilter_kernel)
  Levels lv;
};

// Stage-2 work is cut into items of at most kPairsPerItem (token, slot) pairs of one
// leaf in one window, so a leaf that many queries share is spread over many waves.
constexpr int kPairsPerItem = 16;

struct ClusterArgs {
  const int32_t* cand;   // [B*Hkv][N][2K]
  int32_t* pairs;        // [B*Hkv][N][2K] packed (t << 6 | slot), grouped by leaf per window
  int32_t* leaf_off;     // [B*Hkv][n_windows][M1 + 1]
  int2* items;           // [B*Hkv][n_windows][item_cap] {leaf, first pair | count << 20}
  int32_t* n_items;      // [B*Hkv][n_windows]
  int batch, n_kv_heads, n, width, n_leaves, window, n_windows, item_cap;
};

struct LeafArgs {
  const void* q;
  int64_t q_sb, q_st, q_sh;
  const void* k;
  int64_t k_sb, k_st, k_sh;
  const int32_t* pairs;
  const int32_t* leaf_off;
  const int2* items;
  const int32_t* n_items;
  float* leaf_u;         // [B*Hkv][N][2K]
  const bf16x8* kpack;   // bf16 inputs: packed K blocks (PackArgs layout)
  const bf16x8* qpack;   // bf16 inputs: packed query groups (RouteArgs::qpack layout)
  int batch, n_kv_heads, group, head_dim, n, width, n_leaves, window, n_windows, item_cap;
  int score;             // 0 LSE, 1 mean, 2 mean + var / 2 (pisa_score)
  float scale;
  bool bf16;
};

struct TopkArgs {
  const int32_t* cand;
  const float* leaf_u;
  int32_t* sel;          // [B*Hkv][N][K]
  float* sel_u;          // optional
  int batch, n_kv_heads, n, width, top_k;
};

// Token order of the attention passes (order.hip): workspace arrays; order == nullptr means the
// natural order.
struct OrderArgs {
  const int32_t* sel;           // [bh][n][top_k] selections
  int32_t* hist;                // [bh][m1] block selection counts
  int32_t* keycnt;              // [n_passes][bh][m1 + 1][n_chunks] key counts per chunk, then their prefix
  int32_t* keytot;              // [n_passes][bh][m1 + 1] key totals, then the first position of each key
  int32_t* keys;                // [n_passes][bh][n] each token's key in each pass
  unsigned long long* stats;    // [0] valid entries, [1] of them also listed by the previous token
  int32_t* order;               // [n_passes][bh][n] tokens in each pass's visiting order
  int bh, n, m1, top_k, n_passes;
  int n_chunks;                 // chunks of kOrderChunk tokens
  int hot_cut;                  // a block selected more often than this is hot
};

// The attention takes the sorted order when the selections' blocks are listed by the previous
// token less than a quarter of the time (stats: valid entries, entries also in the previous row).
__device__ inline bool order_sorted(const unsigned long long* stats) {
  const unsigned long long entries = stats[0], overlap = stats[1];
  return entries > 0 && overlap * 4 < entries;
}

// Tokens per chunk of the order's stable counting sort (order.hip).
constexpr int kOrderChunk = 4096;

// Workgroup L of a launch runs on XCD L % kXcds.
constexpr int kXcds = 8;

struct AttnArgs {
  const void* q;
  int64_t q_sb, q_st, q_sh;
  const void* k;
  int64_t k_sb, k_st, k_sh;
  const void* v;
  int64_t v_sb, v_st, v_sh;
  const int32_t* sel;
  void* o;
  int64_t o_sb, o_st, o_sh;
  float* row_lse;        // optional [B][Hq][N]
  bf16x8* kpack;         // bf16 inputs: packed K blocks (see PackArgs), workspace
  bf16x8* vpack;         // bf16 inputs: packed V blocks, workspace
  // Passes over the selected blocks (bf16 inputs, float32 output): pass p takes the blocks j with
  // j % n_passes == p.  A pass before the last leaves its online-softmax state in the output
  // rows (o not yet normalised) and in part_ml ([B*Hkv][N][G] pairs (m in base-2 units, l),
  // workspace); the next pass resumes from it.
  int pass, n_passes;
  float* part_ml;
  // bf16 inputs: the visiting order of each pass's tokens and the statistics that choose between
  // it and the natural order (ord.order == nullptr: natural order, no order kernels)
  OrderArgs ord;
  int batch, n_kv_heads, group, head_dim, n, top_k;
  float scale;
  bool bf16;             // element type of q, k, v
  bool out_bf16;         // element type of o
};


// Packed 64-key blocks for bf16 K and V: every MFMA fragment of a block is one contiguous
// 1 KB run in lane order (lane l = 16 g + col holds 16 bytes), so a fragment load reads whole
// cache lines.  Block j of (b, kvh) occupies 64 d / 8 sixteen-byte pieces at
// ((b * Hkv + kvh) * M1 + j) * 8 d.
//   K piece (mt, s), mt < 4, s < d / 32, at (mt * d / 32 + s) * 64 + l: elements
//     [32 s + 8 g, +8) of key 64 j + perm_key(mt, col).
//   V piece (kb, dt), kb < 2, dt < d / 16, at (kb * d / 16 + dt) * 64 + l: column
//     16 dt + col of keys 64 j + 32 kb + 8 g + i, i < 8.
// Keys at or past n are zero.
struct PackArgs {
  const void* k;
  int64_t k_sb, k_st, k_sh;
  const void* v;            // may be null: K only
  int64_t v_sb, v_st, v_sh;
  bf16x8* kpack;
  bf16x8* vpack;
  int batch, n_kv_heads, head_dim, n;
};


// Key order inside a packed K block: M-tile mt = 2 kb + h, row m holds key
// 32 kb + 8 (m / 4) + 4 h + m % 4.  In an S^T = K Q^T result lane group g of tiles (2 kb, 2 kb + 1)
// then owns keys 32 kb + 8 g + 0..7, which is exactly the k-slice that the lane supplies to the
// P V product of key half kb.
__host__ __device__ inline int perm_key(int mt, int m) { return 32 * (mt >> 1) + 8 * (m >> 2) + 4 * (mt & 1) + (m & 3); }

// Single-level (flat) selection: summed query groups and leaf means in MFMA fragment order.
struct FlatArgs {
  const void* q;
  int64_t q_sb, q_st, q_sh;
  const float* pyr;         // pyramid built with capacity n (leaf level first)
  int64_t nodes;            // pyramid nodes per (b, kvh)
  float4* qsum;             // workspace: [B*Hkv][ceil(n/16)][d/16][64] summed heads, fp32
  float4* kpack;            // workspace: [B*Hkv][ceil(M1/16)][d/16][64] leaf means, fp32
  int32_t* sel;             // [B*Hkv][n][K] ascending, -1 padded
  float* sel_u;             // optional scores
  int batch, n_kv_heads, group, head_dim, n, top_k;
  float scale;
  bool bf16;
};

struct DecodeArgs {
  const void* q;            // [B][Hq][d]
  int64_t q_sb, q_sh;
  const void* k_new;
  int64_t kn_sb, kn_sh;
  const void* v_new;
  int64_t vn_sb, vn_sh;
  void* k_cache;
  int64_t kc_sb, kc_st, kc_sh;
  void* v_cache;
  int64_t vc_sb, vc_st, vc_sh;
  float* pyr;
  int32_t* sel_out;         // optional [B][Hkv][K]
  void* o;                  // [B][Hq][d]
  int64_t o_sb, o_sh;
  int batch, n_kv_heads, group, head_dim, top_k, n_ctx;
  int score;                // 0 LSE, 1 mean, 2 mean + var / 2 (pisa_score)
  float scale;
  bool bf16;                // element type of q, k/v (new and cached)
  bool out_bf16;            // element type of o
  Levels lv;                // sizes for length n_ctx + 1, capacity offsets
};

// Status of the kernel just enqueued on s.  When it launched and the calling thread has stage
// events pending (pisa_stage_events), the next of them is recorded on s, so a caller can time
// every kernel of an entry point on the stream it runs on.
hipError_t launched(hipStream_t s);

hipError_t launch_pyramid(const PyramidArgs& a, hipStream_t s);
hipError_t launch_pack(const PackArgs& a, hipStream_t s);
hipError_t launch_route(const RouteArgs& a, hipStream_t s);
// bf16 inputs: fills a.split from a.pyr.
hipError_t launch_split_summaries(const RouteArgs& a, hipStream_t s);
hipError_t launch_cluster(const ClusterArgs& a, hipStream_t s);
hipError_t launch_leaf_lse(const LeafArgs& a, hipStream_t s);
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
hipError_t launch_attention(const AttnArgs& a, hipStream_t s);
// Fills a.order and a.stats for the attention passes (counters cleared first).
hipError_t launch_order(const OrderArgs& a, hipStream_t s);
size_t order_hist_lds_bytes(int m1);
size_t order_keys_lds_bytes(int m1, int n_passes);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_flat(const FlatArgs& a, hipStream_t s);

// LDS bytes of the fused decode kernel for (group, 2K, d).
size_t decode_lds_bytes(int group, int width, int head_dim);

}  // namespace pisa
