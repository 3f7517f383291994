// api.hip - the C ABI declared in include/pisa.h: host-side validation, pyramid
// geometry, workspace carving and kernel launch order.  Nothing here allocates
// or synchronises; every call enqueues on the caller's stream.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "attention_bwd.h"
#include "kernels.h"
#include "pisa.h"

namespace {

using pisa::Levels;

thread_local int g_last_hip_error = 0;

// Stage events handed over by pisa_stage_events, consumed by the calling thread's next entry
// point: one is recorded on its stream after each kernel it launches.
thread_local void* const* g_stage_events = nullptr;
thread_local int g_stage_left = 0;

// Clears the pending stage events when an entry point returns, whether or not it launched.
struct StageScope {
  ~StageScope() {
    g_stage_events = nullptr;
    g_stage_left = 0;
  }
};

constexpr int kMaxSeqSelect = 1000000;     // leaf counters of one window must fit in LDS
constexpr int kMaxSeq = (1 << 25) - 1;     // packed (token << 6 | slot) fits int32
// Tokens per Stage-2 clustering window: a window's query rows and the key blocks its
// items stream share the L2; measured best at 512 tokens up to 64K and 2048 above (with
// items of at most 16 pairs; 1024 and 4096 are slower at 256K, 1024 at 32K).
int window_tokens(int seq_len) { return seq_len <= 65536 ? 512 : 2048; }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

bool aligned16(const void* p) { return p && ((uintptr_t)p & 15u) == 0; }

// Level sizes for length n laid out for `capacity` keys (capacity >= n >= 1).
Levels make_levels(int n, int capacity) {
  Levels lv;
  memset(&lv, 0, sizeof(lv));
  int m = (capacity + pisa::kLeaf - 1) / pisa::kLeaf;
  int64_t off = 0;
  int level = 0;
  while (true) {
    lv.offset[level] = off;
    off += m;
    ++level;
    if (m == 1) break;
    m = (m + 1) / 2;
  }
  lv.nodes = off;
  int cur = (n + pisa::kLeaf - 1) / pisa::kLeaf;
  int count = 0;
  while (true) {
    lv.size[count++] = cur;
    if (cur == 1) break;
    cur = (cur + 1) / 2;
  }
  lv.count = count;
  return lv;
}

// Split-summary pair blocks of the levels of `lv`: offsets per level and the total.
int64_t split_pairs(const Levels& lv, int64_t* pair_off) {
  int64_t off = 0;
  for (int l = 0; l < lv.count; ++l) {
    if (pair_off) pair_off[l] = off;
    off += (lv.size[l] + 1) / 2;
  }
  return off;
}

pisa_status check_cfg(const pisa_cfg* c) {
  if (!c) return PISA_ERR_INVALID_ARG;
  if (c->batch < 1 || c->seq_len < 1 || c->n_q_heads < 1 || c->n_kv_heads < 1 || c->top_k < 1)
    return PISA_ERR_INVALID_ARG;
  if (c->n_q_heads % c->n_kv_heads != 0) return PISA_ERR_INVALID_ARG;
  if (c->dtype != PISA_F32 && c->dtype != PISA_BF16) return PISA_ERR_INVALID_ARG;
  if (c->score != PISA_SCORE_LSE && c->score != PISA_SCORE_MEAN && c->score != PISA_SCORE_MEAN_VAR)
    return PISA_ERR_INVALID_ARG;
  const int G = c->n_q_heads / c->n_kv_heads;
  if (c->block != pisa::kLeaf || c->fanout != pisa::kFanout) return PISA_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return PISA_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return PISA_ERR_UNSUPPORTED;
  if (c->top_k > 32) return PISA_ERR_UNSUPPORTED;
  if (c->seq_len > kMaxSeq) return PISA_ERR_UNSUPPORTED;
  return PISA_OK;
}

pisa_status check_tensor(const void* ptr, int64_t sb, int64_t st, int64_t sh) {
  if (!aligned16(ptr)) return PISA_ERR_INVALID_ARG;
  if (sb < 0 || st < 0 || sh < 0 || (sb % 8) || (st % 8) || (sh % 8)) return PISA_ERR_INVALID_ARG;
  return PISA_OK;
}

float resolve_scale(const pisa_cfg* c) {
  return c->scale > 0.f ? c->scale : 1.0f / sqrtf((float)c->head_dim);
}

pisa_status hip_status(hipError_t e) {
  if (e == hipSuccess) return PISA_OK;
  g_last_hip_error = (int)e;
  return PISA_ERR_HIP;
}

struct SelectWorkspace {
  size_t cand, leaf_u, pairs, leaf_off, items, n_items, split, split16, bounds, kpack, qpack, total;
  int n_windows, item_cap;
};

SelectWorkspace select_layout(const pisa_cfg* c) {
  SelectWorkspace w;
  const int64_t bh = (int64_t)c->batch * c->n_kv_heads;
  const int64_t slots = bh * c->seq_len * 2 * c->top_k;
  const int m1 = (c->seq_len + pisa::kLeaf - 1) / pisa::kLeaf;
  const int window = window_tokens(c->seq_len);
  w.n_windows = (c->seq_len + window - 1) / window;
  w.cand = 0;
  w.leaf_u = align256(w.cand + slots * 4);
  w.pairs = align256(w.leaf_u + slots * 4);
  w.leaf_off = align256(w.pairs + slots * 4);
  // items per window: sum over leaves of ceil(count / P) <= window pairs / P + distinct leaves
  const int64_t window_pairs = (int64_t)window * 2 * c->top_k;
  w.item_cap = (int)((window_pairs + pisa::kPairsPerItem - 1) / pisa::kPairsPerItem +
                     (m1 < window_pairs ? m1 : window_pairs));
  w.items = align256(w.leaf_off + (size_t)bh * w.n_windows * (m1 + 1) * 4);
  w.n_items = align256(w.items + (size_t)bh * w.n_windows * w.item_cap * 8);
  w.split = align256(w.n_items + (size_t)bh * w.n_windows * 4);
  // bf16 inputs: split summaries for routing (4 bytes per pyramid element), packed K
  // blocks and packed query groups for the leaf scores
  const bool bf16 = c->dtype == PISA_BF16;
  const int64_t split_blocks = bf16 ? bh * split_pairs(make_levels(c->seq_len, c->seq_len), nullptr) : 0;
  const size_t split_bytes = (size_t)split_blocks * c->head_dim * 8;
  const size_t kpack_bytes = bf16 ? (size_t)bh * m1 * pisa::kLeaf * c->head_dim * 2 : 0;
  const size_t qpack_bytes = bf16 ? (size_t)bh * c->seq_len * c->n_q_heads / c->n_kv_heads * c->head_dim * 2 : 0;
  w.split16 = align256(w.split + split_bytes);        // the float16 copy: half the split bytes
  w.bounds = align256(w.split16 + split_bytes / 2);   // (R, X) per node: four floats per block
  w.kpack = align256(w.bounds + (size_t)split_blocks * 16);
  w.qpack = align256(w.kpack + kpack_bytes);
  w.total = align256(w.qpack + qpack_bytes);
  return w;
}

struct BwdWorkspace {
  size_t kpack, vrows, tok, rank, hist, seg_len, seg_base, item_base, list, items, n_items, partial, total;
  int64_t max_items;
};

// Backward workspace: packed K rows and V rows, the token records, the inverse index of
// the selections and the per-item dK / dV partial sums (see BwdArgs).
BwdWorkspace bwd_layout(const pisa_cfg* c) {
  BwdWorkspace w;
  const int64_t bh = (int64_t)c->batch * c->n_kv_heads;
  const int64_t m1 = (c->seq_len + pisa::kLeaf - 1) / pisa::kLeaf;
  const int64_t chunks = (c->seq_len + pisa::kBwdChunk - 1) / pisa::kBwdChunk;
  const int64_t slots = bh * c->seq_len * c->top_k;
  const size_t pack = (size_t)bh * m1 * pisa::kLeaf * c->head_dim * 2;
  w.max_items = slots / pisa::kBwdItem + bh * m1;         // sum over blocks of ceil(len / 512)
  w.kpack = 0;
  w.vrows = align256(w.kpack + pack);
  w.tok = align256(w.vrows + pack);
  w.rank = align256(w.tok + (size_t)bh * c->seq_len * pisa::bwd_record_bytes(c->head_dim));
  w.hist = align256(w.rank + (size_t)slots * 4);
  w.seg_len = align256(w.hist + (size_t)bh * chunks * m1 * 4);
  w.seg_base = align256(w.seg_len + (size_t)bh * m1 * 4);
  w.item_base = align256(w.seg_base + (size_t)bh * m1 * 4);
  w.list = align256(w.item_base + (size_t)bh * m1 * 4);
  w.items = align256(w.list + (size_t)slots * 4);
  w.n_items = align256(w.items + (size_t)w.max_items * 8);
  w.partial = align256(w.n_items + 4);
  w.total = align256(w.partial + (size_t)w.max_items * 2 * pisa::kLeaf * c->head_dim * 4);
  return w;
}

pisa_status check_bwd_cfg(const pisa_cfg* c) {
  pisa_status st = check_cfg(c);
  if (st != PISA_OK) return st;
  if (c->dtype != PISA_BF16) return PISA_ERR_UNSUPPORTED;
  if ((c->seq_len + pisa::kLeaf - 1) / pisa::kLeaf > pisa::kBwdMaxLeaves) return PISA_ERR_UNSUPPORTED;
  if ((int64_t)c->batch * c->n_kv_heads * c->seq_len * c->top_k > INT32_MAX) return PISA_ERR_UNSUPPORTED;
  return PISA_OK;
}

constexpr int kAttnPasses = 2;
constexpr int kOrderMaxLeaves = 16384;       // the order kernels keep per-leaf counters in LDS

// Attention workspace (bf16 inputs): packed K blocks, packed V blocks, the (m, l) pair of every
// (b, kvh, token, head) carried between the two passes of a float32-output call, and, up to
// kOrderMaxLeaves leaf blocks, the arrays of the passes' token order (OrderArgs): block counts,
// key counts per chunk of kOrderChunk tokens, key totals, two 64-bit statistics, the tokens' keys and
// the order itself (sizes 0 beyond that).
struct AttnWorkspace {
  size_t kpack, vpack, part_ml, hist, keycnt, keytot, stats, keys, order, total;
};

AttnWorkspace attn_layout(const pisa_cfg* c) {
  AttnWorkspace w;
  const int64_t m1 = (c->seq_len + pisa::kLeaf - 1) / pisa::kLeaf;
  const int64_t bh = (int64_t)c->batch * c->n_kv_heads;
  const size_t pack = align256((size_t)bh * m1 * pisa::kLeaf * c->head_dim * 2);
  w.kpack = 0;
  w.vpack = pack;
  w.part_ml = 2 * pack;
  w.hist = w.part_ml + align256((size_t)c->batch * c->n_q_heads * c->seq_len * 2 * sizeof(float));
  const bool ordered = m1 <= kOrderMaxLeaves;
  w.keycnt = w.hist + (ordered ? align256((size_t)bh * m1 * 4) : 0);
  const int64_t chunks = (c->seq_len + pisa::kOrderChunk - 1) / pisa::kOrderChunk;
  w.keytot = w.keycnt + (ordered ? align256((size_t)kAttnPasses * bh * (m1 + 1) * chunks * 4) : 0);
  w.stats = w.keytot + (ordered ? align256((size_t)kAttnPasses * bh * (m1 + 1) * 4) : 0);
  w.keys = w.stats + (ordered ? 256 : 0);
  w.order = w.keys + (ordered ? align256((size_t)kAttnPasses * bh * c->seq_len * 4) : 0);
  w.total = w.order + (ordered ? align256((size_t)kAttnPasses * bh * c->seq_len * 4) : 0);
  if (!ordered) w.hist = w.keycnt = w.keytot = w.stats = w.keys = w.order = 0;
  return w;
}

// Whether the attention workspace holds the token-order arrays.
bool attn_has_order(const pisa_cfg* c) { return attn_layout(c).order != 0; }

// Passes of a bf16-input attention call: the blocks are split into even and odd ids when the
// output is float32 (the output rows carry the state between them).  Each pass's gathers then
// touch half of the blocks, so more of their reads hit the L2 (0.55 against 0.48 at N = 262144): the
// call takes 8.6 ms against 9.4 ms in one pass there, and 4.9 against 5.7 ms at N = 32768.

}  // namespace

namespace pisa {

// PISA_ROUTE_EXACT set to a value other than "0" in the environment at the first selection call:
// bf16 LSE routing scores every candidate from the full split rows (route_kernel) instead of
// pre-filtering with the high parts; the selections are the same either way.  Read once.
static bool route_exact() {
  static const bool on = [] {
    const char* v = getenv("PISA_ROUTE_EXACT");
    return v && v[0] && strcmp(v, "0") != 0;
  }();
  return on;
}

// Debug mode: with PISA_SYNC_LAUNCHES set to a value other than "0" in the environment when the
// library first launches, every launch waits for its stream, so a kernel's fault or error is
// reported by the entry point and the kernel that caused it (not by a later call).  Read once.
static bool sync_launches() {
  static const bool on = [] {
    const char* v = getenv("PISA_SYNC_LAUNCHES");
    return v && v[0] && strcmp(v, "0") != 0;
  }();
  return on;
}

hipError_t launched(hipStream_t s) {
  hipError_t e = hipGetLastError();
  if (e == hipSuccess && sync_launches()) e = hipStreamSynchronize(s);
  if (e != hipSuccess || g_stage_left <= 0) return e;
  e = hipEventRecord(static_cast<hipEvent_t>(*g_stage_events), s);
  ++g_stage_events;
  --g_stage_left;
  return e;
}

}  // namespace pisa

extern "C" {

pisa_status pisa_stage_events(void* const* events, int32_t count) {
  g_stage_events = nullptr;
  g_stage_left = 0;
  if (count < 0 || (count > 0 && !events)) return PISA_ERR_INVALID_ARG;
  for (int32_t i = 0; i < count; ++i)
    if (!events[i]) return PISA_ERR_INVALID_ARG;
  g_stage_events = events;
  g_stage_left = count;
  return PISA_OK;
}

int pisa_abi_version(void) { return PISA_ABI_VERSION; }

const char* pisa_status_string(int32_t s) {
  switch (s) {
    case PISA_OK: return "ok";
    case PISA_ERR_INVALID_ARG: return "invalid argument";
    case PISA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PISA_ERR_WORKSPACE: return "workspace missing or too small";
    case PISA_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int pisa_last_hip_error(void) { return g_last_hip_error; }

int64_t pisa_pyramid_nodes(int32_t capacity) {
  if (capacity < 1) return 0;
  return make_levels(1, capacity).nodes;
}

size_t pisa_pyramid_bytes(const pisa_cfg* cfg, int32_t capacity) {
  if (check_cfg(cfg) != PISA_OK || capacity < 1) return 0;
  return (size_t)cfg->batch * cfg->n_kv_heads * pisa_pyramid_nodes(capacity) * cfg->head_dim * sizeof(float);
}

pisa_status pisa_build_pyramid(const pisa_cfg* cfg, pisa_tensor k, int32_t n, int32_t capacity, float* pyr,
                               void* stream) {
  StageScope stages;
  pisa_status st = check_cfg(cfg);
  if (st != PISA_OK) return st;
  if (n < 1 || capacity < n || capacity > kMaxSeq) return PISA_ERR_INVALID_ARG;
  if ((st = check_tensor(k.ptr, k.stride_b, k.stride_t, k.stride_h)) != PISA_OK) return st;
  if (!aligned16(pyr)) return PISA_ERR_INVALID_ARG;
  pisa::PyramidArgs a;
  a.k = k.ptr; a.k_sb = k.stride_b; a.k_st = k.stride_t; a.k_sh = k.stride_h;
  a.pyr = pyr;
  a.batch = cfg->batch; a.n_kv_heads = cfg->n_kv_heads; a.head_dim = cfg->head_dim; a.n = n;
  a.bf16 = cfg->dtype == PISA_BF16;
  a.lv = make_levels(n, capacity);
  return hip_status(pisa::launch_pyramid(a, (hipStream_t)stream));
}

size_t pisa_select_workspace_bytes(const pisa_cfg* cfg) {
  if (check_cfg(cfg) != PISA_OK) return 0;
  return select_layout(cfg).total;
}

pisa_status pisa_select_blocks(const pisa_cfg* cfg, pisa_tensor q, pisa_tensor k, const float* pyr, int32_t* sel,
                               float* sel_u, void* ws, size_t ws_bytes, void* stream) {
  StageScope stages;
  pisa_status st = check_cfg(cfg);
  if (st != PISA_OK) return st;
  if (cfg->seq_len > kMaxSeqSelect) return PISA_ERR_UNSUPPORTED;
  if ((st = check_tensor(q.ptr, q.stride_b, q.stride_t, q.stride_h)) != PISA_OK) return st;
  if ((st = check_tensor(k.ptr, k.stride_b, k.stride_t, k.stride_h)) != PISA_OK) return st;
  if (!aligned16(pyr) || !sel) return PISA_ERR_INVALID_ARG;
  const SelectWorkspace w = select_layout(cfg);
  if (!ws || ws_bytes < w.total || ((uintptr_t)ws & 255u)) return PISA_ERR_WORKSPACE;
  char* base = static_cast<char*>(ws);
  int32_t* cand = reinterpret_cast<int32_t*>(base + w.cand);
  float* leaf_u = reinterpret_cast<float*>(base + w.leaf_u);
  int32_t* pairs = reinterpret_cast<int32_t*>(base + w.pairs);
  int32_t* leaf_off = reinterpret_cast<int32_t*>(base + w.leaf_off);
  int2* items = reinterpret_cast<int2*>(base + w.items);
  int32_t* n_items = reinterpret_cast<int32_t*>(base + w.n_items);
  const int N = cfg->seq_len, G = cfg->n_q_heads / cfg->n_kv_heads, width = 2 * cfg->top_k;
  const int m1 = (N + pisa::kLeaf - 1) / pisa::kLeaf;
  const bool bf16 = cfg->dtype == PISA_BF16;
  const float scale = resolve_scale(cfg);
  hipStream_t s = (hipStream_t)stream;

  pisa::RouteArgs r;
  r.q = q.ptr; r.q_sb = q.stride_b; r.q_st = q.stride_t; r.q_sh = q.stride_h;
  r.pyr = pyr; r.cand = cand;
  r.batch = cfg->batch; r.n_kv_heads = cfg->n_kv_heads; r.group = G; r.head_dim = cfg->head_dim;
  r.n = N; r.top_k = cfg->top_k; r.scale = scale; r.bf16 = bf16; r.score = cfg->score;
  r.lv = make_levels(N, N);
  r.split = bf16 ? reinterpret_cast<uint16_t*>(base + w.split) : nullptr;
  r.split16 = bf16 ? reinterpret_cast<uint16_t*>(base + w.split16) : nullptr;
  r.bounds = bf16 ? reinterpret_cast<float*>(base + w.bounds) : nullptr;
  r.prefilter = bf16 && !pisa::route_exact();
  r.pairs = split_pairs(r.lv, r.pair_off);
  pisa::bf16x8* kpack = reinterpret_cast<pisa::bf16x8*>(base + w.kpack);
  pisa::bf16x8* qpack = reinterpret_cast<pisa::bf16x8*>(base + w.qpack);
  r.qpack = bf16 ? qpack : nullptr;                   // routing writes the packed query groups
  if (bf16 && (st = hip_status(pisa::launch_split_summaries(r, s))) != PISA_OK) return st;
  if ((st = hip_status(pisa::launch_route(r, s))) != PISA_OK) return st;

  pisa::ClusterArgs c;
  c.cand = cand; c.pairs = pairs; c.leaf_off = leaf_off;
  c.batch = cfg->batch; c.n_kv_heads = cfg->n_kv_heads; c.n = N; c.width = width;
  c.n_leaves = m1; c.window = window_tokens(N); c.n_windows = w.n_windows;
  c.items = items; c.n_items = n_items; c.item_cap = w.item_cap;
  if ((st = hip_status(pisa::launch_cluster(c, s))) != PISA_OK) return st;

  if (bf16) {
    pisa::PackArgs p;
    p.k = k.ptr; p.k_sb = k.stride_b; p.k_st = k.stride_t; p.k_sh = k.stride_h;
    p.v = nullptr; p.v_sb = p.v_st = p.v_sh = 0;
    p.kpack = kpack; p.vpack = nullptr;
    p.batch = cfg->batch; p.n_kv_heads = cfg->n_kv_heads; p.head_dim = cfg->head_dim; p.n = N;
    if ((st = hip_status(pisa::launch_pack(p, s))) != PISA_OK) return st;
  }

  pisa::LeafArgs l;
  l.q = q.ptr; l.q_sb = q.stride_b; l.q_st = q.stride_t; l.q_sh = q.stride_h;
  l.k = k.ptr; l.k_sb = k.stride_b; l.k_st = k.stride_t; l.k_sh = k.stride_h;
  l.pairs = pairs; l.leaf_off = leaf_off; l.leaf_u = leaf_u;
  l.batch = cfg->batch; l.n_kv_heads = cfg->n_kv_heads; l.group = G; l.head_dim = cfg->head_dim;
  l.n = N; l.width = width; l.n_leaves = m1; l.window = window_tokens(N); l.n_windows = w.n_windows;
  l.items = items; l.n_items = n_items; l.item_cap = w.item_cap;
  l.scale = scale; l.bf16 = bf16; l.score = cfg->score;
  l.kpack = kpack; l.qpack = qpack;
  if ((st = hip_status(pisa::launch_leaf_lse(l, s))) != PISA_OK) return st;

  pisa::TopkArgs t;
  t.cand = cand; t.leaf_u = leaf_u; t.sel = sel; t.sel_u = sel_u;
  t.batch = cfg->batch; t.n_kv_heads = cfg->n_kv_heads; t.n = N; t.width = width; t.top_k = cfg->top_k;
  return hip_status(pisa::launch_topk(t, s));
}

size_t pisa_flat_workspace_bytes(const pisa_cfg* cfg) {
  if (check_cfg(cfg) != PISA_OK) return 0;
  const size_t bh = (size_t)cfg->batch * cfg->n_kv_heads;
  const size_t groups = (cfg->seq_len + 15) / 16;
  const size_t tiles = ((cfg->seq_len + pisa::kLeaf - 1) / pisa::kLeaf + 15) / 16;
  return align256(bh * groups * 16 * cfg->head_dim * 4) + align256(bh * tiles * 16 * cfg->head_dim * 4);
}

pisa_status pisa_select_flat(const pisa_cfg* cfg, pisa_tensor q, const float* pyr, int32_t* sel, float* sel_u,
                             void* ws, size_t ws_bytes, void* stream) {
  StageScope stages;
  pisa_status st = check_cfg(cfg);
  if (st != PISA_OK) return st;
  if (cfg->top_k > 16) return PISA_ERR_UNSUPPORTED;
  if ((st = check_tensor(q.ptr, q.stride_b, q.stride_t, q.stride_h)) != PISA_OK) return st;
  if (!aligned16(pyr) || !sel) return PISA_ERR_INVALID_ARG;
  const size_t need = pisa_flat_workspace_bytes(cfg);
  if (!ws || ws_bytes < need || ((uintptr_t)ws & 255u)) return PISA_ERR_WORKSPACE;
  const size_t bh = (size_t)cfg->batch * cfg->n_kv_heads;
  const size_t groups = (cfg->seq_len + 15) / 16;
  pisa::FlatArgs a;
  a.q = q.ptr; a.q_sb = q.stride_b; a.q_st = q.stride_t; a.q_sh = q.stride_h;
  a.pyr = pyr; a.nodes = make_levels(cfg->seq_len, cfg->seq_len).nodes;
  a.qsum = static_cast<float4*>(ws);
  a.kpack = reinterpret_cast<float4*>(static_cast<char*>(ws) + align256(bh * groups * 16 * cfg->head_dim * 4));
  a.sel = sel; a.sel_u = sel_u;
  a.batch = cfg->batch; a.n_kv_heads = cfg->n_kv_heads; a.group = cfg->n_q_heads / cfg->n_kv_heads;
  a.head_dim = cfg->head_dim; a.n = cfg->seq_len; a.top_k = cfg->top_k;
  a.scale = resolve_scale(cfg); a.bf16 = cfg->dtype == PISA_BF16;
  return hip_status(pisa::launch_flat(a, (hipStream_t)stream));
}

size_t pisa_attn_workspace_bytes(const pisa_cfg* cfg) {
  if (check_cfg(cfg) != PISA_OK) return 0;
  if (cfg->dtype != PISA_BF16) return 0;
  return attn_layout(cfg).total;
}

}  // extern "C"

namespace {

// Forward attention with the workspace the caller (or the fixed device array) provides.
pisa_status attn_fwd(const pisa_cfg* cfg, pisa_tensor q, pisa_tensor k, pisa_tensor v, const int32_t* sel,
                     pisa_tensor_mut o, int32_t o_dtype, float* row_lse, void* ws, size_t ws_bytes,
                     void* stream) {
  pisa_status st = check_cfg(cfg);
  if (st != PISA_OK) return st;
  const size_t need = pisa_attn_workspace_bytes(cfg);
  if (need && (!ws || ws_bytes < need || ((uintptr_t)ws & 255u))) return PISA_ERR_WORKSPACE;
  if (o_dtype != PISA_F32 && o_dtype != PISA_BF16) return PISA_ERR_INVALID_ARG;
  if ((st = check_tensor(q.ptr, q.stride_b, q.stride_t, q.stride_h)) != PISA_OK) return st;
  if ((st = check_tensor(k.ptr, k.stride_b, k.stride_t, k.stride_h)) != PISA_OK) return st;
  if ((st = check_tensor(v.ptr, v.stride_b, v.stride_t, v.stride_h)) != PISA_OK) return st;
  if ((st = check_tensor(o.ptr, o.stride_b, o.stride_t, o.stride_h)) != PISA_OK) return st;
  if (!sel) return PISA_ERR_INVALID_ARG;
  pisa::AttnArgs a;
  a.q = q.ptr; a.q_sb = q.stride_b; a.q_st = q.stride_t; a.q_sh = q.stride_h;
  a.k = k.ptr; a.k_sb = k.stride_b; a.k_st = k.stride_t; a.k_sh = k.stride_h;
  a.v = v.ptr; a.v_sb = v.stride_b; a.v_st = v.stride_t; a.v_sh = v.stride_h;
  a.sel = sel;
  a.o = o.ptr; a.o_sb = o.stride_b; a.o_st = o.stride_t; a.o_sh = o.stride_h;
  a.row_lse = row_lse;
  const bool out_bf16 = o_dtype == PISA_BF16;
  if (need) {
    const AttnWorkspace w = attn_layout(cfg);
    char* base = static_cast<char*>(ws);
    a.kpack = reinterpret_cast<pisa::bf16x8*>(base + w.kpack);
    a.vpack = reinterpret_cast<pisa::bf16x8*>(base + w.vpack);
    a.part_ml = reinterpret_cast<float*>(base + w.part_ml);
  } else {
    a.kpack = a.vpack = nullptr;
    a.part_ml = nullptr;
  }
  a.pass = 0;
  a.n_passes = (need && !out_bf16) ? kAttnPasses : 1;
  a.ord = pisa::OrderArgs{};
  if (need && attn_has_order(cfg)) {
    const AttnWorkspace w = attn_layout(cfg);
    char* base = static_cast<char*>(ws);
    a.ord.sel = sel;
    a.ord.hist = reinterpret_cast<int32_t*>(base + w.hist);
    a.ord.keycnt = reinterpret_cast<int32_t*>(base + w.keycnt);
    a.ord.keytot = reinterpret_cast<int32_t*>(base + w.keytot);
    a.ord.stats = reinterpret_cast<unsigned long long*>(base + w.stats);
    a.ord.keys = reinterpret_cast<int32_t*>(base + w.keys);
    a.ord.order = reinterpret_cast<int32_t*>(base + w.order);
    a.ord.bh = cfg->batch * cfg->n_kv_heads;
    a.ord.n = cfg->seq_len;
    a.ord.m1 = (cfg->seq_len + pisa::kLeaf - 1) / pisa::kLeaf;
    a.ord.top_k = cfg->top_k;
    a.ord.n_passes = a.n_passes;
    a.ord.n_chunks = (cfg->seq_len + pisa::kOrderChunk - 1) / pisa::kOrderChunk;
    a.ord.hot_cut = 4 * pisa::kLeaf * cfg->top_k;
  }
  a.batch = cfg->batch; a.n_kv_heads = cfg->n_kv_heads; a.group = cfg->n_q_heads / cfg->n_kv_heads;
  a.head_dim = cfg->head_dim; a.n = cfg->seq_len; a.top_k = cfg->top_k;
  a.scale = resolve_scale(cfg); a.bf16 = cfg->dtype == PISA_BF16; a.out_bf16 = out_bf16;
  return hip_status(pisa::launch_attention(a, (hipStream_t)stream));
}

// The allocation-free forward's workspace: one fixed array per GPU, held until the process ends.
// Host code never passes `scratch` itself (in host code its name stands for a host-side stand-in):
// its device address, queried once per device, is what the kernels get.
constexpr int kMaxDevices = 64;
static_assert(PISA_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[PISA_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's array (null with the HIP error recorded on failure).
void* scratch_on_current_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    g_last_hip_error = e != hipSuccess ? (int)e : (int)hipErrorInvalidDevice;
    return nullptr;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      g_last_hip_error = e != hipSuccess ? (int)e : (int)hipErrorInvalidSymbol;
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

pisa_status pisa_sparse_attn_fwd(const pisa_cfg* cfg, pisa_tensor q, pisa_tensor k, pisa_tensor v,
                                 const int32_t* sel, pisa_tensor_mut o, int32_t o_dtype, float* row_lse,
                                 void* ws, size_t ws_bytes, void* stream) {
  StageScope stages;
  return attn_fwd(cfg, q, k, v, sel, o, o_dtype, row_lse, ws, ws_bytes, stream);
}

pisa_status pisa_sparse_attn_fwd_noalloc(const pisa_cfg* cfg, pisa_tensor q, pisa_tensor k, pisa_tensor v,
                                         const int32_t* sel, pisa_tensor_mut o, int32_t o_dtype,
                                         float* row_lse, void* stream) {
  StageScope stages;
  pisa_status st = check_cfg(cfg);
  if (st != PISA_OK) return st;
  const size_t need = pisa_attn_workspace_bytes(cfg);
  if (need > PISA_NOALLOC_SCRATCH_BYTES) return PISA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (need && !(ws = scratch_on_current_device())) return PISA_ERR_HIP;
  return attn_fwd(cfg, q, k, v, sel, o, o_dtype, row_lse, ws, need ? PISA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

size_t pisa_attn_bwd_workspace_bytes(const pisa_cfg* cfg) {
  if (check_bwd_cfg(cfg) != PISA_OK) return 0;
  return bwd_layout(cfg).total;
}

pisa_status pisa_sparse_attn_bwd(const pisa_cfg* cfg, pisa_tensor q, pisa_tensor k, pisa_tensor v,
                                 const int32_t* sel, pisa_tensor o, pisa_tensor dout, int32_t grad_dtype,
                                 const float* row_lse, pisa_tensor_mut dq, pisa_tensor_mut dk, pisa_tensor_mut dv,
                                 void* ws, size_t ws_bytes, void* stream) {
  StageScope stages;
  pisa_status st = check_bwd_cfg(cfg);
  if (st != PISA_OK) return st;
  const BwdWorkspace w = bwd_layout(cfg);
  if (!ws || ws_bytes < w.total || ((uintptr_t)ws & 255u)) return PISA_ERR_WORKSPACE;
  if (grad_dtype != PISA_F32 && grad_dtype != PISA_BF16) return PISA_ERR_INVALID_ARG;
  if ((st = check_tensor(q.ptr, q.stride_b, q.stride_t, q.stride_h)) != PISA_OK) return st;
  if ((st = check_tensor(k.ptr, k.stride_b, k.stride_t, k.stride_h)) != PISA_OK) return st;
  if ((st = check_tensor(v.ptr, v.stride_b, v.stride_t, v.stride_h)) != PISA_OK) return st;
  if ((st = check_tensor(o.ptr, o.stride_b, o.stride_t, o.stride_h)) != PISA_OK) return st;
  if ((st = check_tensor(dout.ptr, dout.stride_b, dout.stride_t, dout.stride_h)) != PISA_OK) return st;
  if ((st = check_tensor(dq.ptr, dq.stride_b, dq.stride_t, dq.stride_h)) != PISA_OK) return st;
  if ((st = check_tensor(dk.ptr, dk.stride_b, dk.stride_t, dk.stride_h)) != PISA_OK) return st;
  if ((st = check_tensor(dv.ptr, dv.stride_b, dv.stride_t, dv.stride_h)) != PISA_OK) return st;
  if (!sel || !row_lse) return PISA_ERR_INVALID_ARG;
  char* base = static_cast<char*>(ws);
  pisa::BwdArgs a;
  a.q = q.ptr; a.q_sb = q.stride_b; a.q_st = q.stride_t; a.q_sh = q.stride_h;
  a.k = k.ptr; a.k_sb = k.stride_b; a.k_st = k.stride_t; a.k_sh = k.stride_h;
  a.v = v.ptr; a.v_sb = v.stride_b; a.v_st = v.stride_t; a.v_sh = v.stride_h;
  a.sel = sel;
  a.o = o.ptr; a.o_sb = o.stride_b; a.o_st = o.stride_t; a.o_sh = o.stride_h;
  a.dout = dout.ptr; a.do_sb = dout.stride_b; a.do_st = dout.stride_t; a.do_sh = dout.stride_h;
  a.row_lse = row_lse;
  a.dq = static_cast<float*>(dq.ptr); a.dq_sb = dq.stride_b; a.dq_st = dq.stride_t; a.dq_sh = dq.stride_h;
  a.dk = static_cast<float*>(dk.ptr); a.dk_sb = dk.stride_b; a.dk_st = dk.stride_t; a.dk_sh = dk.stride_h;
  a.dv = static_cast<float*>(dv.ptr); a.dv_sb = dv.stride_b; a.dv_st = dv.stride_t; a.dv_sh = dv.stride_h;
  a.kpack = reinterpret_cast<pisa::bf16x8*>(base + w.kpack);
  a.vrows = reinterpret_cast<pisa::bf16x8*>(base + w.vrows);
  a.tok = base + w.tok;
  a.rank = reinterpret_cast<int32_t*>(base + w.rank);
  a.hist = reinterpret_cast<int32_t*>(base + w.hist);
  a.seg_len = reinterpret_cast<int32_t*>(base + w.seg_len);
  a.seg_base = reinterpret_cast<int32_t*>(base + w.seg_base);
  a.item_base = reinterpret_cast<int32_t*>(base + w.item_base);
  a.list = reinterpret_cast<int32_t*>(base + w.list);
  a.items = reinterpret_cast<int2*>(base + w.items);
  a.n_items = reinterpret_cast<int32_t*>(base + w.n_items);
  a.partial = reinterpret_cast<float*>(base + w.partial);
  a.max_items = w.max_items;
  a.batch = cfg->batch; a.n_kv_heads = cfg->n_kv_heads; a.group = cfg->n_q_heads / cfg->n_kv_heads;
  a.head_dim = cfg->head_dim; a.n = cfg->seq_len; a.top_k = cfg->top_k;
  a.scale = resolve_scale(cfg); a.grad_bf16 = grad_dtype == PISA_BF16;
  return hip_status(pisa::launch_attention_bwd(a, (hipStream_t)stream));
}

pisa_status pisa_decode_step(const pisa_cfg* cfg, int32_t n_ctx, pisa_tensor q, pisa_tensor k_new,
                             pisa_tensor v_new, pisa_tensor_mut k_cache, pisa_tensor_mut v_cache, float* pyr,
                             int32_t* sel_out, pisa_tensor_mut o, int32_t o_dtype, void* stream) {
  StageScope stages;
  pisa_status st = check_cfg(cfg);
  if (st != PISA_OK) return st;
  if (o_dtype != PISA_F32 && o_dtype != PISA_BF16) return PISA_ERR_INVALID_ARG;
  const int G = cfg->n_q_heads / cfg->n_kv_heads;
  if (n_ctx < 0 || n_ctx + 1 > cfg->seq_len) return PISA_ERR_INVALID_ARG;
  if (G * 2 * cfg->top_k > 256) return PISA_ERR_UNSUPPORTED;
  if ((st = check_tensor(q.ptr, q.stride_b, 0, q.stride_h)) != PISA_OK) return st;
  if ((st = check_tensor(k_new.ptr, k_new.stride_b, 0, k_new.stride_h)) != PISA_OK) return st;
  if ((st = check_tensor(v_new.ptr, v_new.stride_b, 0, v_new.stride_h)) != PISA_OK) return st;
  if ((st = check_tensor(k_cache.ptr, k_cache.stride_b, k_cache.stride_t, k_cache.stride_h)) != PISA_OK) return st;
  if ((st = check_tensor(v_cache.ptr, v_cache.stride_b, v_cache.stride_t, v_cache.stride_h)) != PISA_OK) return st;
  if ((st = check_tensor(o.ptr, o.stride_b, 0, o.stride_h)) != PISA_OK) return st;
  if (!aligned16(pyr)) return PISA_ERR_INVALID_ARG;
  pisa::DecodeArgs a;
  a.q = q.ptr; a.q_sb = q.stride_b; a.q_sh = q.stride_h;
  a.k_new = k_new.ptr; a.kn_sb = k_new.stride_b; a.kn_sh = k_new.stride_h;
  a.v_new = v_new.ptr; a.vn_sb = v_new.stride_b; a.vn_sh = v_new.stride_h;
  a.k_cache = k_cache.ptr; a.kc_sb = k_cache.stride_b; a.kc_st = k_cache.stride_t; a.kc_sh = k_cache.stride_h;
  a.v_cache = v_cache.ptr; a.vc_sb = v_cache.stride_b; a.vc_st = v_cache.stride_t; a.vc_sh = v_cache.stride_h;
  a.pyr = pyr; a.sel_out = sel_out;
  a.o = o.ptr; a.o_sb = o.stride_b; a.o_sh = o.stride_h;
  a.batch = cfg->batch; a.n_kv_heads = cfg->n_kv_heads; a.group = G; a.head_dim = cfg->head_dim;
  a.top_k = cfg->top_k; a.n_ctx = n_ctx; a.scale = resolve_scale(cfg); a.bf16 = cfg->dtype == PISA_BF16;
  a.score = cfg->score;
  a.out_bf16 = o_dtype == PISA_BF16;
  a.lv = make_levels(n_ctx + 1, cfg->seq_len);
  return hip_status(pisa::launch_decode(a, (hipStream_t)stream));
}

}  // extern "C"
