// attention_bwd.h - arguments and workspace geometry of the attention gradients (see
// attention_bwd.hip and pisa_sparse_attn_bwd in pisa.h).
#pragma once

#include "kernels.h"

namespace pisa {

// Gradients of the block-sparse attention with the selections held fixed (bf16 q, k, v).
//   tok     [B*Hkv][N] token records of bwd_record_bytes(d) bytes: the group's queries and
//           upstream gradients as bf16 rows [16][d] (heads past G zero) and per head
//           (row LSE * log2 e, Delta = dO . O) as float2 [16] (+inf / 0 past G): everything
//           the key-major pass stages for a token, one contiguous copy
//   rank    [B*Hkv][N][K] int32: occurrence of (t, slot)'s block among earlier tokens of its chunk
//   hist    [B*Hkv][chunks][M1] int32: per-chunk block counts, then their exclusive prefix per block
//   seg_len, seg_base, item_base [B*Hkv*M1] int32: tokens selecting each block, their list offset,
//           and the first work item of the block
//   list    [sum of seg_len] int32: tokens of each block, ascending
//   items   [max_items] int2: (block e = bh * M1 + j, first list entry of the item within the block)
//   partial [max_items][2][64][d] float32: the item's dK and dV contributions
struct BwdArgs {
  const void* q;
  int64_t q_sb, q_st, q_sh;
  const void* k;
  int64_t k_sb, k_st, k_sh;
  const void* v;
  int64_t v_sb, v_st, v_sh;
  const int32_t* sel;
  const void* o;
  int64_t o_sb, o_st, o_sh;
  const void* dout;
  int64_t do_sb, do_st, do_sh;
  const float* row_lse;  // [B][Hq][N]
  float* dq;
  int64_t dq_sb, dq_st, dq_sh;
  float* dk;
  int64_t dk_sb, dk_st, dk_sh;
  float* dv;
  int64_t dv_sb, dv_st, dv_sh;
  // workspace
  bf16x8* kpack;         // K rows (attention K layout)
  bf16x8* vrows;         // V rows in the K layout
  char* tok;
  int32_t* rank;
  int32_t* hist;
  int32_t* seg_len;
  int32_t* seg_base;
  int32_t* item_base;
  int32_t* list;
  int2* items;
  int32_t* n_items;      // one int: items in use
  float* partial;
  int64_t max_items;
  int batch, n_kv_heads, group, head_dim, n, top_k;
  float scale;
  bool grad_bf16;        // element type of o and dout
};

// Token record geometry (bytes): rows of q, rows of dO, the statistics.
__host__ __device__ constexpr int bwd_row_bytes(int d) { return 16 * d * 2; }
__host__ __device__ constexpr int bwd_stats_offset(int d) { return 2 * bwd_row_bytes(d); }
__host__ __device__ constexpr int bwd_record_bytes(int d) { return bwd_stats_offset(d) + 16 * 8; }

constexpr int kBwdChunk = 256;      // tokens per ranking chunk
constexpr int kBwdItem = 512;       // tokens per key-major work item
constexpr int kBwdMaxLeaves = 8192;   // ranking LDS: 256 K + M1 int32 <= 64 KB

hipError_t launch_attention_bwd(const BwdArgs& a, hipStream_t s);

}  // namespace pisa
