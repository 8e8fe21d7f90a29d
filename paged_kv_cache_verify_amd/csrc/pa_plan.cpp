// Host side of the C ABI: validation, the work plan, scratch, launches.
//
// The plan follows the prior art's split between a host-built work plan with
// its own cached scratch and an allocation-free call (ATOM #2843, review
// thread on run_pa_decode: feasibility is checked right after the call's
// arguments are known and before any plan or scratch is built; the call then
// uses its plan's scratch and allocates none). Refusals name the limit they
// hit and never fall back to another path (same page, vLLM bridge section:
// fail loudly rather than compute a wrong answer).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/pa_verify.h"
#include "pa_internal.h"

using namespace pav;

namespace {

// Host-side record of one sequence while the plan is built.
struct SeqInfo {
  int32_t ctx_len;   // L
  int32_t q_len;     // q (0: padded slot)
  int32_t q_off;     // first query row of this sequence in q/out
  int32_t lo;        // first key any row may see (window), else 0
  int32_t window;    // W, 0 = none
  int32_t n_parts;   // work items per KV head
  int32_t piece;     // keys per work item (the last one may be shorter)
  int32_t slot_base; // partial slot of (kv head 0, part 0) when n_parts > 1
  int32_t rblocks;   // row blocks (work items per key piece)
  int32_t rper;      // rows per row block (the last may have fewer)
  double cost;       // relative time per key of one of this sequence's items
};

}  // namespace

struct pa_plan_s {
  int device = -1;
  int cus = 0;  // compute units of the device the plan was built for
  pa_shape shape{};
  std::vector<SeqInfo> seqs;
  std::vector<WorkItem> items;
  int64_t kv_bytes = 0;
  int64_t scratch_bytes = 0;
  int32_t partition_tokens = 0;
  int32_t rows_stride = 0;
  int64_t n_slots = 0;
  std::vector<ReduceItem> red;  // split (sequence, KV head) pairs
  int32_t max_parts = 0;        // most partials of any split pair
  int32_t occ = 1;              // partition workgroups per CU (2 when items exceed one round)
  int32_t ntmax = 1;            // row tiles of the largest item (selects the kernel layout)
  std::vector<int32_t> tokens;  // [T][2]: sequence, position of each new token
  std::vector<int32_t> seq_rows;  // [B][2]: first verify row, verify rows (q)
  WorkItem* d_items = nullptr;
  int32_t* d_tokens = nullptr;
  int32_t* d_seq_rows = nullptr;
  float* d_verdict_val = nullptr;  // [T][kVerdictSlices] argmax partials
  int32_t* d_verdict_idx = nullptr;
  ReduceItem* d_red = nullptr;
  float* d_part_o = nullptr;
  float* d_part_ml = nullptr;
  // Two-level merge (some pair has more than 512 partials): the first level
  // folds chunks of at most ceil(n / 32) partials into first-level slots,
  // and `red` then lists each pair's first-level slots.
  std::vector<ReduceItem> red1;
  int64_t l1_slots = 0;
  ReduceItem* d_red1 = nullptr;
  float* d_l1_o = nullptr;
  float* d_l1_ml = nullptr;
  // Fused call: merge nodes (a tree per split pair and row block), their
  // arrival counters (zeroed once here, reset by each node's last arriver;
  // two more after them for the persistent grid's work list) and the tree
  // slots the inner nodes write.
  std::vector<MergeNode> nodes;
  int64_t tree_slots = 0;
  MergeNode* d_nodes = nullptr;
  int32_t* d_counters = nullptr;
  float* d_tree_o = nullptr;
  float* d_tree_ml = nullptr;
  hipEvent_t ev_before = nullptr;
  hipEvent_t ev_after = nullptr;
  unsigned long long* stamps = nullptr;  // pa_set_workgroup_stamps
};

namespace {

thread_local std::string g_last_error;

constexpr int kItemFields = 7;  // int32 per row of pa_plan_items

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pa_status hip_fail(hipError_t e, const char* what) {
  return fail(e == hipErrorOutOfMemory ? PA_E_NOMEM : PA_E_HIP, "%s: %s", what,
              hipGetErrorString(e));
}

void release_device(pa_plan_s* p) {
  if (p->device < 0) return;
  int cur = 0;
  bool have = hipGetDevice(&cur) == hipSuccess;
  if (have && cur != p->device) (void)hipSetDevice(p->device);
  if (p->d_items) (void)hipFree(p->d_items);
  if (p->d_red) (void)hipFree(p->d_red);
  if (p->d_part_o) (void)hipFree(p->d_part_o);
  if (p->d_part_ml) (void)hipFree(p->d_part_ml);
  if (p->d_red1) (void)hipFree(p->d_red1);
  if (p->d_l1_o) (void)hipFree(p->d_l1_o);
  if (p->d_l1_ml) (void)hipFree(p->d_l1_ml);
  if (p->d_tokens) (void)hipFree(p->d_tokens);
  if (p->d_seq_rows) (void)hipFree(p->d_seq_rows);
  if (p->d_verdict_val) (void)hipFree(p->d_verdict_val);
  if (p->d_verdict_idx) (void)hipFree(p->d_verdict_idx);
  if (p->d_nodes) (void)hipFree(p->d_nodes);
  if (p->d_counters) (void)hipFree(p->d_counters);
  if (p->d_tree_o) (void)hipFree(p->d_tree_o);
  if (p->d_tree_ml) (void)hipFree(p->d_tree_ml);
  p->d_nodes = nullptr;
  p->d_counters = nullptr;
  p->d_tree_o = nullptr;
  p->d_tree_ml = nullptr;
  p->d_items = nullptr;
  p->d_tokens = nullptr;
  p->d_seq_rows = nullptr;
  p->d_verdict_val = nullptr;
  p->d_verdict_idx = nullptr;
  p->d_red = nullptr;
  p->d_part_o = nullptr;
  p->d_part_ml = nullptr;
  p->d_red1 = nullptr;
  p->d_l1_o = nullptr;
  p->d_l1_ml = nullptr;
  if (have && cur != p->device) (void)hipSetDevice(cur);
}

// Every check a call can fail, before anything is allocated.
pa_status validate(const pa_shape* s, const int32_t* ctx, const int32_t* ql, const int32_t* win,
                   int device) {
  if (!s) return fail(PA_E_INVALID, "shape is NULL");
  if (!ctx || !ql) return fail(PA_E_INVALID, "context_lens and query_lens are required");
  if (device < -1) return fail(PA_E_INVALID, "device %d is not a device ordinal or -1", device);
  if (s->num_seqs < 1) return fail(PA_E_INVALID, "num_seqs %d < 1", s->num_seqs);
  if (s->num_q_heads < 1 || s->num_kv_heads < 1)
    return fail(PA_E_INVALID, "head counts must be >= 1 (Hq %d, Hkv %d)", s->num_q_heads,
                s->num_kv_heads);
  if (s->num_q_heads % s->num_kv_heads != 0)
    return fail(PA_E_INVALID, "num_q_heads %d is not a multiple of num_kv_heads %d",
                s->num_q_heads, s->num_kv_heads);
  if (s->block_size != kBlock)
    return fail(PA_E_UNSUPPORTED, "block_size %d: only 16-token blocks are served", s->block_size);
  if (s->head_dim != 64 && s->head_dim != 128 && s->head_dim != 256)
    return fail(PA_E_UNSUPPORTED, "head_dim %d: only 64, 128 and 256 are served", s->head_dim);
  if (s->head_dim == 256 && s->kv_dtype != PA_FP8_E4M3)
    return fail(PA_E_UNSUPPORTED, "head_dim 256 is served for FP8 e4m3 KV only");
  if (s->q_dtype != PA_BF16) return fail(PA_E_UNSUPPORTED, "q_dtype must be bf16");
  if (s->kv_dtype != PA_BF16 && s->kv_dtype != PA_FP8_E4M3)
    return fail(PA_E_UNSUPPORTED, "kv_dtype must be bf16 or fp8 e4m3");
  if (s->out_dtype != PA_BF16 && s->out_dtype != PA_FP32)
    return fail(PA_E_UNSUPPORTED, "out_dtype must be bf16 or fp32");
  if (!(std::isfinite(s->softmax_scale) && s->softmax_scale > 0.f))
    return fail(PA_E_INVALID, "softmax_scale must be finite and > 0");
  if (s->num_blocks < 1) return fail(PA_E_INVALID, "num_blocks %d < 1", s->num_blocks);
  if (s->max_blocks_per_seq < 1)
    return fail(PA_E_INVALID, "max_blocks_per_seq %d < 1", s->max_blocks_per_seq);
  if (s->partition_tokens < 0 || s->partition_tokens % kBlock != 0)
    return fail(PA_E_INVALID, "partition_tokens %d must be 0 or a positive multiple of 16",
                s->partition_tokens);
  if (s->partition_tokens > kMaxItemKeys)
    return fail(PA_E_UNSUPPORTED, "partition_tokens %d exceeds the %d keys a work item spans",
                s->partition_tokens, kMaxItemKeys);
  if (s->sinks_mode < 0 || s->sinks_mode > 2)
    return fail(PA_E_INVALID, "sinks_mode %d is not 0, 1 or 2", s->sinks_mode);
  if (s->lengths_are_bounds != 0 && s->lengths_are_bounds != 1)
    return fail(PA_E_INVALID, "lengths_are_bounds %d is not 0 or 1", s->lengths_are_bounds);
  const int G = s->num_q_heads / s->num_kv_heads;
  int64_t total_q = 0;
  for (int b = 0; b < s->num_seqs; ++b) {
    const int L = ctx[b], q = ql[b];
    if (q < 0) return fail(PA_E_INVALID, "query_lens[%d] = %d < 0", b, q);
    if (q > kMaxQuery)
      return fail(PA_E_UNSUPPORTED, "query_lens[%d] = %d exceeds the verify limit of %d", b, q,
                  kMaxQuery);
    if (L < q)
      return fail(PA_E_INVALID, "context_lens[%d] = %d is smaller than its query length %d", b,
                  L, q);
    if (L > kMaxContext)
      return fail(PA_E_UNSUPPORTED, "context_lens[%d] = %d exceeds the 1 Mi-token limit", b, L);
    if ((L + kBlock - 1) / kBlock > s->max_blocks_per_seq)
      return fail(PA_E_INVALID, "context_lens[%d] = %d needs %d blocks > max_blocks_per_seq %d",
                  b, L, (L + kBlock - 1) / kBlock, s->max_blocks_per_seq);
    if ((int64_t)(L + kBlock - 1) / kBlock > s->num_blocks)
      return fail(PA_E_INVALID, "context_lens[%d] = %d needs more blocks than the pool holds", b,
                  L);
    if (win && win[b] < 0) return fail(PA_E_INVALID, "window[%d] = %d < 0", b, win[b]);
    if (q * G > kMaxRows)
      return fail(PA_E_UNSUPPORTED,
                  "sequence %d packs %d x %d = %d rows per KV head; at most %d are served", b,
                  q, G, q * G, kMaxRows);
    total_q += q;
  }
  if (total_q * s->num_q_heads * (int64_t)s->head_dim > ((int64_t)1 << 40))
    return fail(PA_E_UNSUPPORTED, "query tensor too large");
  return PA_OK;
}

// Relative time per key of an item with `rows` packed rows. bf16 KV is
// bound by its bytes (1). With FP8 KV a chunk costs a fixed part (its
// streaming, the softmax's bookkeeping, the ring's barriers) plus a part
// that grows with the busiest SIMD's compute waves per chunk, c, which
// depends on the item's row tiles and the workgroup layout (head dim 128:
// four groups of three tile waves, c = tiles / 4, for plans of at most 48
// rows; head dims 64 and 256: two rotated groups, 1/2 for up to two tiles,
// else 1). The slope 4/3 fits measured partition times of items with two
// and three row tiles (about 0.5 and 0.6 us per chunk). Head dim 128 above
// 48 rows runs three groups of four tile waves, where c = 0.22 tiles + 0.11
// fits the measured times per key of a mixed batch's items of 1 to 4 tiles
// (10.2, 11.1, 14.1 and 15.4 ns).
double item_cost(const pa_shape& s, int rows, int ntmax) {
  if (s.kv_dtype != PA_FP8_E4M3) return 1.0;
  const int tiles = (rows + 15) / 16;
  double c;
  if (s.head_dim == 128 && ntmax <= 3) c = 0.25 * tiles;
  else if (s.head_dim == 128) c = 0.22 * tiles + 0.11;
  else c = tiles <= 2 ? 0.5 : 1.0;
  return 1.0 + (4.0 / 3.0) * c;
}

// Keys per item of a sequence for a cost-weighted item size P: a multiple
// of 32, within [lo_keys, kMaxItemKeys].
int64_t keys_for(double P, double cost, int64_t lo_keys) {
  const int64_t k = ((int64_t)(P / cost) / kChunk) * kChunk;
  return std::min<int64_t>(kMaxItemKeys, std::max<int64_t>(lo_keys, k));
}

// Work items of a cost-weighted item size P for every active sequence,
// counted over all KV heads and row blocks.
int64_t count_items(const std::vector<SeqInfo>& seqs, int Hkv, double P, int64_t lo_keys) {
  int64_t n = 0;
  for (const SeqInfo& si : seqs) {
    if (si.q_len == 0) continue;
    const int64_t span = si.ctx_len - (si.lo / kBlock) * kBlock;
    const int64_t piece = keys_for(P, si.cost, lo_keys);
    n += (int64_t)Hkv * si.rblocks * ((span + piece - 1) / piece);
  }
  return n;
}

// Item size, in cost-weighted keys, when the caller leaves the choice to the
// plan. One workgroup runs per CU, so the plan looks for the smallest size
// whose items fit one round on the device; the workgroups then start
// together and each runs for about the same time (a sequence whose items
// cost less per key gets more keys per item). When no size up to the item
// limit fits one round, items of about a third of a round's share keep the
// rounds' tails short.
double auto_piece(const std::vector<SeqInfo>& seqs, int Hkv, int cus, int64_t& lo_keys) {
  double total = 0.0, max_cost = 1.0;
  for (const SeqInfo& si : seqs)
    if (si.q_len > 0) {
      total += (double)Hkv * si.rblocks * (si.ctx_len - (si.lo / kBlock) * kBlock) * si.cost;
      max_cost = std::max(max_cost, si.cost);
    }
  lo_keys = kChunk;
  if (total == 0.0) return kChunk;
  const double p_max = (double)kMaxItemKeys * max_cost;
  if (count_items(seqs, Hkv, p_max, lo_keys) <= cus) {
    double lo = total / cus / 2, hi = p_max;
    for (int it = 0; it < 40; ++it) {  // the smallest size that fits one round
      const double mid = 0.5 * (lo + hi);
      if (count_items(seqs, Hkv, mid, lo_keys) <= cus) hi = mid;
      else lo = mid;
    }
    return hi;
  }
  lo_keys = 512;
  return total / (3.0 * cus);
}

// The merge of one split pair's n partials in the fused call: nodes of at
// most kFusedFanIn inputs, level by level until one node remains. Level-0
// nodes take partials first + j * stride (j < count); a node of a higher
// level takes the tree slots [first, first + count) (numbered from the
// pair's first) that its children write, out_slot being a child's.
//
// Workgroups go to the XCDs in turn (item i to XCD i mod 8), and a node is
// merged by its last arriving item, most often its last dispatched one. A
// leaf of 16 consecutive items would always end on the same XCD, which then
// carries every merge; so the leaves of each run of 8 x 16 partials take
// every L-th partial (L the run's leaves): a leaf's items share an XCD, and
// the run's leaves spread over the eight.
struct TreeNode {
  int32_t first, count, stride, level;
  int32_t out_slot;  // -1 at the root
  int32_t parent;    // index in the tree, -1 at the root
};

void merge_tree(int32_t n, std::vector<TreeNode>& t, std::vector<int32_t>& leaf, int32_t& slots) {
  t.clear();
  leaf.assign(n, 0);
  slots = 0;
  if (n <= kFusedFanIn) {
    t.push_back({0, n, 1, 0, -1, -1});
  } else {
    constexpr int32_t kRun = 8 * kFusedFanIn;
    for (int32_t b0 = 0; b0 < n; b0 += kRun) {
      const int32_t r = std::min(kRun, n - b0), L = (r + kFusedFanIn - 1) / kFusedFanIn;
      for (int32_t j = 0; j < L; ++j) {
        for (int32_t x = b0 + j; x < b0 + r; x += L) leaf[x] = (int32_t)t.size();
        t.push_back({b0 + j, (r - j + L - 1) / L, L, 0, -1, -1});
      }
    }
  }
  int32_t k = (int32_t)t.size(), lb = 0, level = 0;
  while (k > 1) {
    const int32_t base = slots;
    for (int32_t j = 0; j < k; ++j) t[lb + j].out_slot = base + j;
    slots += k;
    const int32_t k2 = (k + kFusedFanIn - 1) / kFusedFanIn, nb = (int32_t)t.size();
    ++level;
    for (int32_t j = 0; j < k2; ++j) {
      const int32_t a = (int32_t)((int64_t)j * k / k2), e = (int32_t)((int64_t)(j + 1) * k / k2);
      for (int32_t x = a; x < e; ++x) t[lb + x].parent = nb + j;
      t.push_back({base + a, e - a, 1, level, -1, -1});
    }
    lb = nb;
    k = k2;
  }
}

}  // namespace

extern "C" {

const char* pa_last_error(void) { return g_last_error.c_str(); }

pa_status pa_plan(const pa_shape* shape, const int32_t* context_lens, const int32_t* query_lens,
                  const int32_t* window, int device, pa_plan_t** out) {
  if (!out) return fail(PA_E_INVALID, "out is NULL");
  *out = nullptr;
  pa_status st = validate(shape, context_lens, query_lens, window, device);
  if (st != PA_OK) return st;

  const pa_shape& s = *shape;
  const int B = s.num_seqs, Hkv = s.num_kv_heads, G = s.num_q_heads / s.num_kv_heads;
  const int esz = s.kv_dtype == PA_FP8_E4M3 ? 1 : 2;
  const int64_t tok_bytes = 2LL * s.head_dim * esz + (s.kv_dtype == PA_FP8_E4M3 ? 8 : 0);

  // Work items are sized for the device's CU count (256 on MI355X, assumed
  // for a host-only plan).
  int cus = 256;
  if (device >= 0) {
    hipError_t e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(multiprocessor count)");
    if (cus < 1) cus = 1;
  }

  pa_plan_s* p = new (std::nothrow) pa_plan_s();
  if (!p) return fail(PA_E_NOMEM, "host allocation of the plan failed");
  p->shape = s;
  p->device = device;
  p->cus = cus;

  try {
    p->seqs.resize(B);
    int64_t total_keys = 0;
    int32_t q_off = 0, rows_stride = 0;
    for (int b = 0; b < B; ++b) {
      SeqInfo& si = p->seqs[b];
      si.ctx_len = context_lens[b];
      si.q_len = query_lens[b];
      si.q_off = q_off;
      si.window = window ? window[b] : 0;
      si.lo = 0;
      // With lengths that are upper bounds, a shorter length moves a window
      // earlier: the items then cover a windowed sequence from key 0.
      if (si.q_len > 0 && si.window > 0 && !s.lengths_are_bounds)
        si.lo = std::max(0, si.ctx_len - si.q_len - si.window + 1);
      si.n_parts = 0;
      si.piece = 0;
      si.slot_base = -1;
      si.rblocks = 0;
      si.rper = 0;
      p->seq_rows.push_back(q_off);
      p->seq_rows.push_back(si.q_len);
      q_off += si.q_len;
      for (int i = 0; i < si.q_len; ++i) {
        p->tokens.push_back(b);
        p->tokens.push_back(si.ctx_len - si.q_len + i);
      }
      if (si.q_len > 0) {
        total_keys += (int64_t)Hkv * (si.ctx_len - si.lo);
        rows_stride = std::max(rows_stride, si.q_len * G);
      }
    }
    p->rows_stride = rows_stride;
    p->kv_bytes = total_keys * tok_bytes;

    // Row blocks: a workgroup carries at most item_rows packed rows, so a
    // sequence with more is split into ceil(rows / item_rows) blocks of
    // about equal size (whole 16-row tiles), each a work item of its own
    // over the same keys. They share the key piece's partial slot, each
    // writing its own rows of it.
    const int item_rows = s.head_dim == 256 ? kItemRows256 : kItemRows;
    int max_item_rows = 0;
    for (SeqInfo& si : p->seqs) {
      if (si.q_len == 0) continue;
      const int rows = si.q_len * G;
      si.rblocks = (rows + item_rows - 1) / item_rows;
      si.rper = (((rows + si.rblocks - 1) / si.rblocks) + 15) / 16 * 16;
      si.rper = std::min(si.rper, rows);
      max_item_rows = std::max(max_item_rows, si.rper);
    }
    p->ntmax = (max_item_rows + 15) / 16;
    // Cut [a, L) of every active sequence, a = lo rounded down to a page,
    // into pieces of one size per sequence (a multiple of 16 keys, so every
    // cut falls on a page boundary), the same for every KV head. A caller's
    // partition_tokens is that size for every sequence; otherwise each
    // sequence is cut into as few equal pieces of at most the plan's item
    // size as will do.
    const int ntmax = p->ntmax;
    for (SeqInfo& si : p->seqs) si.cost = item_cost(s, si.rper, ntmax);
    int64_t lo_keys = kChunk;
    const double weighted = s.partition_tokens > 0 ? 0.0 : auto_piece(p->seqs, Hkv, cus, lo_keys);
    int64_t slots = 0;
    int32_t largest = 0;
    for (int b = 0; b < B; ++b) {
      SeqInfo& si = p->seqs[b];
      if (si.q_len == 0) continue;
      const int a = (si.lo / kBlock) * kBlock;
      const int span = si.ctx_len - a;
      const int64_t limit = s.partition_tokens > 0 ? s.partition_tokens
                                                   : keys_for(weighted, si.cost, lo_keys);
      si.n_parts = (int32_t)((span + limit - 1) / limit);
      if (s.partition_tokens > 0) {
        si.piece = (int32_t)limit;
      } else {
        const int per = (span + si.n_parts - 1) / si.n_parts;
        si.piece = std::min<int32_t>((int32_t)limit, ((per + kBlock - 1) / kBlock) * kBlock);
        si.n_parts = (span + si.piece - 1) / si.piece;
      }
      largest = std::max(largest, std::min(si.piece, span));
      if (si.n_parts > 1) {
        si.slot_base = (int32_t)slots;
        slots += (int64_t)Hkv * si.n_parts;
      }
      std::vector<TreeNode> tree;
      std::vector<int32_t> leaf;
      int32_t tslots = 0;
      if (si.n_parts > 1) merge_tree(si.n_parts, tree, leaf, tslots);
      for (int g = 0; g < Hkv; ++g) {
        // The fused call's nodes of this pair: tree node t of row block rb
        // is node nbase + t * rblocks + rb; the pair's tree slots start at
        // tbase (shared by the row blocks, whose rows are disjoint).
        const int64_t nbase = (int64_t)p->nodes.size(), tbase = p->tree_slots;
        const int32_t pslot = (int32_t)(si.slot_base + (int64_t)g * si.n_parts);
        for (const TreeNode& tn : tree) {
          for (int rb = 0; rb < si.rblocks; ++rb) {
            MergeNode m{};
            m.seq = b;
            m.kv_head = g;
            m.q_len = si.q_len;
            m.q_off = si.q_off;
            m.row0 = rb * si.rper;
            m.nrows = std::min(si.rper, si.q_len * G - m.row0);
            m.from_tree = tn.level > 0;
            m.slot_base = (int32_t)(tn.level > 0 ? tbase + tn.first : pslot + tn.first);
            m.n_parts = tn.count;
            m.slot_stride = tn.stride;
            m.out_slot = tn.out_slot >= 0 ? (int32_t)(tbase + tn.out_slot) : -1;
            m.parent = tn.parent >= 0 ? (int32_t)(nbase + (int64_t)tn.parent * si.rblocks + rb)
                                      : -1;
            p->nodes.push_back(m);
          }
        }
        p->tree_slots += tslots;
        for (int k = 0; k < si.n_parts; ++k) {
          for (int rb = 0; rb < si.rblocks; ++rb) {
            WorkItem it{};
            it.seq = b;
            it.kv_head = g;
            it.key_begin = std::max(si.lo, a + k * si.piece);
            it.key_end = std::min(si.ctx_len, a + (k + 1) * si.piece);
            it.slot =
                si.n_parts > 1 ? (int32_t)(si.slot_base + (int64_t)g * si.n_parts + k) : -1;
            it.ctx_len = si.ctx_len;
            it.q_len = si.q_len;
            it.q_off = si.q_off;
            it.window = si.window;
            it.row0 = rb * si.rper;
            it.nrows = std::min(si.rper, si.q_len * G - it.row0);
            it.node = si.n_parts > 1 ? (int32_t)(nbase + (int64_t)leaf[k] * si.rblocks + rb) : -1;
            p->items.push_back(it);
          }
        }
        if (si.n_parts > 1) {
          ReduceItem r{};
          r.seq = b;
          r.kv_head = g;
          r.slot_base = (int32_t)(si.slot_base + (int64_t)g * si.n_parts);
          r.n_parts = si.n_parts;
          r.q_len = si.q_len;
          r.q_off = si.q_off;
          p->red.push_back(r);
          p->max_parts = std::max(p->max_parts, si.n_parts);
        }
      }
    }
    p->partition_tokens = s.partition_tokens > 0 ? s.partition_tokens : largest;
    // More items than one round of one workgroup per CU: with bf16 KV two
    // smaller workgroups share each CU, so one streams while the other
    // starts or finishes an item (FP8 items are bound by compute and keep
    // one workgroup per CU).
    p->occ = ((int64_t)p->items.size() > cus && s.kv_dtype == PA_BF16) ? 2 : 1;
    for (const WorkItem& it : p->items) {
      // A workgroup keeps the page ids of at most kMaxItemChunks chunks.
      const int span = it.key_end - (it.key_begin / kBlock) * kBlock;
      if ((span + kChunk - 1) / kChunk > kMaxItemChunks) {
        delete p;
        return fail(PA_E_UNSUPPORTED, "a work item spans more than %d keys", kMaxItemKeys);
      }
    }
    if (p->items.size() >= (size_t)INT32_MAX || slots >= (int64_t)INT32_MAX ||
        p->nodes.size() >= (size_t)INT32_MAX || p->tree_slots >= (int64_t)INT32_MAX ||
        (int64_t)p->red.size() * rows_stride * 4 >= (int64_t)INT32_MAX) {
      delete p;
      return fail(PA_E_UNSUPPORTED, "the work list exceeds a 1-D grid");
    }
    // Longest items first, by estimated time (keys x the sequence's cost per
    // key), so that with more items than one round the short ones fill in
    // last. (By keys alone, the FP8 items of many rows, fewer keys but the
    // highest cost per key, ran in the last round of a mixed batch and set
    // its end.)
    const std::vector<SeqInfo>& sq = p->seqs;
    std::stable_sort(p->items.begin(), p->items.end(),
                     [&sq](const WorkItem& x, const WorkItem& y) {
                       return (x.key_end - x.key_begin) * sq[x.seq].cost >
                              (y.key_end - y.key_begin) * sq[y.seq].cost;
                     });
    p->n_slots = slots;
    // With more than 512 partials in some pair, the pairs are merged in two
    // levels: chunks of C = ceil(n / 32) consecutive partials fold into at
    // most 32 first-level partials, which the usual merge then combines.
    // One level with thousands of partials per row is bound by its 128-byte
    // reads 24 KiB apart, where chunks read whole rows of consecutive
    // partials: at 2,048 partials per pair (512-key items over 1 Mi keys)
    // the call measured 3.2 us faster, while at 128 (8,192-key items) the
    // second launch made it 3.9 us slower.
    if (p->max_parts > 512) {
      int32_t max2 = 0;
      for (ReduceItem& r : p->red) {
        const int32_t n = r.n_parts, C = (n + 31) / 32, nch = (n + C - 1) / C;
        for (int32_t c = 0; c < nch; ++c) {
          ReduceItem r1 = r;
          r1.slot_base = r.slot_base + c * C;
          r1.n_parts = std::min(C, n - c * C);
          r1.out_slot = (int32_t)(p->l1_slots + c);
          p->red1.push_back(r1);
        }
        r.slot_base = (int32_t)p->l1_slots;
        r.n_parts = nch;
        p->l1_slots += nch;
        max2 = std::max(max2, nch);
      }
      p->max_parts = max2;
      if ((int64_t)p->red1.size() * rows_stride >= (int64_t)INT32_MAX) {
        delete p;
        return fail(PA_E_UNSUPPORTED, "the first-level merge list exceeds a 1-D grid");
      }
    }
    p->scratch_bytes =
        (slots + p->l1_slots + p->tree_slots) * rows_stride * ((int64_t)s.head_dim + 2) * 4;
  } catch (const std::bad_alloc&) {
    delete p;
    return fail(PA_E_NOMEM, "host allocation of the work list failed");
  }

  if (device < 0) {
    *out = p;
    return PA_OK;
  }

  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e, "hipGetDevice");
  }
  if (cur != device && (e = hipSetDevice(device)) != hipSuccess) {
    delete p;
    return hip_fail(e, "hipSetDevice");
  }
  auto upload = [&](void** dst, const void* src, size_t bytes) -> hipError_t {
    if (bytes == 0) return hipSuccess;
    hipError_t r = hipMalloc(dst, bytes);
    if (r != hipSuccess) return r;
    return hipMemcpy(*dst, src, bytes, hipMemcpyHostToDevice);
  };
  e = upload((void**)&p->d_items, p->items.data(), p->items.size() * sizeof(WorkItem));
  if (e == hipSuccess)
    e = upload((void**)&p->d_red, p->red.data(), p->red.size() * sizeof(ReduceItem));
  if (e == hipSuccess)
    e = upload((void**)&p->d_red1, p->red1.data(), p->red1.size() * sizeof(ReduceItem));
  if (e == hipSuccess)
    e = upload((void**)&p->d_tokens, p->tokens.data(), p->tokens.size() * sizeof(int32_t));
  if (e == hipSuccess)
    e = upload((void**)&p->d_seq_rows, p->seq_rows.data(), p->seq_rows.size() * sizeof(int32_t));
  const size_t n_verdict = p->tokens.size() / 2 * kVerdictSlices;
  if (e == hipSuccess && n_verdict > 0) {
    e = hipMalloc((void**)&p->d_verdict_val, n_verdict * sizeof(float));
    if (e == hipSuccess) e = hipMalloc((void**)&p->d_verdict_idx, n_verdict * sizeof(int32_t));
  }
  if (e == hipSuccess && p->n_slots > 0) {
    e = hipMalloc((void**)&p->d_part_o,
                  (size_t)p->n_slots * p->rows_stride * s.head_dim * sizeof(float));
    if (e == hipSuccess)
      e = hipMalloc((void**)&p->d_part_ml, (size_t)p->n_slots * p->rows_stride * 2 * sizeof(float));
  }
  if (e == hipSuccess && p->l1_slots > 0) {
    e = hipMalloc((void**)&p->d_l1_o,
                  (size_t)p->l1_slots * p->rows_stride * s.head_dim * sizeof(float));
    if (e == hipSuccess)
      e = hipMalloc((void**)&p->d_l1_ml, (size_t)p->l1_slots * p->rows_stride * 2 * sizeof(float));
  }
  if (e == hipSuccess)
    e = upload((void**)&p->d_nodes, p->nodes.data(), p->nodes.size() * sizeof(MergeNode));
  if (e == hipSuccess) {
    const size_t nc = (p->nodes.size() + 2) * sizeof(int32_t);
    e = hipMalloc((void**)&p->d_counters, nc);
    // The counters are zero before the plan is returned.
    if (e == hipSuccess) e = hipMemset(p->d_counters, 0, nc);
    if (e == hipSuccess) e = hipStreamSynchronize(nullptr);
  }
  if (e == hipSuccess && p->tree_slots > 0) {
    e = hipMalloc((void**)&p->d_tree_o,
                  (size_t)p->tree_slots * p->rows_stride * s.head_dim * sizeof(float));
    if (e == hipSuccess)
      e = hipMalloc((void**)&p->d_tree_ml,
                    (size_t)p->tree_slots * p->rows_stride * 2 * sizeof(float));
  }
  if (cur != device) (void)hipSetDevice(cur);
  if (e != hipSuccess) {
    release_device(p);
    delete p;
    return hip_fail(e, "allocating the plan's device memory");
  }
  *out = p;
  return PA_OK;
}

namespace {

// Device buffers one call uses: the plan's own, or the zero-allocation
// call's carve-up of the library's static scratch.
struct CallBufs {
  const WorkItem* items;
  const ReduceItem* red;
  const ReduceItem* red1;
  float* part_o;
  float* part_ml;
  float* l1_o;
  float* l1_ml;
};

// The fused call's buffers (the plan's own).
struct FusedBufs {
  const MergeNode* nodes;
  int32_t* counters;
  float* tree_o;
  float* tree_ml;
};

// The argument checks every attention call makes before it launches.
pa_status check_call(const pa_plan_t* plan, const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_table, const float* k_scales, const float* v_scales,
                     const float* sinks, void* out) {
  const pa_shape& s = plan->shape;
  const bool fp8 = s.kv_dtype == PA_FP8_E4M3;
  if (!q || !k_pool || !v_pool || !block_table || !out)
    return fail(PA_E_INVALID, "q, k_pool, v_pool, block_table and out are required");
  if (fp8 && (!k_scales || !v_scales))
    return fail(PA_E_INVALID, "FP8 KV needs k_scales and v_scales");
  if (!fp8 && (k_scales || v_scales))
    return fail(PA_E_INVALID, "bf16 KV takes no scales");
  if (s.sinks_mode != 0 && !sinks) return fail(PA_E_INVALID, "sinks_mode %d needs sinks",
                                               s.sinks_mode);
  if (s.sinks_mode == 0 && sinks) return fail(PA_E_INVALID, "sinks given with sinks_mode 0");
  return PA_OK;
}

// Enqueue the partition kernel and the reduce (one or two launches), or
// (fused non-null) the fused partition kernel alone.
pa_status launch_call(const pa_plan_t* plan, const CallBufs& d, const int32_t* dev_ctx,
                      const void* q, const void* k_pool, const void* v_pool,
                      const int32_t* block_table, const float* k_scales, const float* v_scales,
                      const float* sinks, void* out, hipStream_t st,
                      const FusedBufs* fused = nullptr) {
  const pa_shape& s = plan->shape;
  const bool fp8 = s.kv_dtype == PA_FP8_E4M3;
  KernelArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.sinks = sinks;
  a.out = out;
  a.part_o = d.part_o;
  a.part_ml = d.part_ml;
  a.items = d.items;
  a.red = d.red;
  a.num_q_heads = s.num_q_heads;
  a.num_kv_heads = s.num_kv_heads;
  a.group = s.num_q_heads / s.num_kv_heads;
  a.max_blocks = s.max_blocks_per_seq;
  a.rows_stride = plan->rows_stride;
  a.sinks_mode = s.sinks_mode;
  a.out_fp32 = s.out_dtype == PA_FP32;
  a.scale_log2 = s.softmax_scale * kLog2e;
  a.dev_ctx = dev_ctx;
  a.stamps = plan->stamps;

  hipError_t e;
  if (fused) {
    a.nodes = fused->nodes;
    a.counters = fused->counters;
    a.tree_o = fused->tree_o;
    a.tree_ml = fused->tree_ml;
    a.n_items = (int32_t)plan->items.size();
    a.grid = plan->cus * plan->occ;
    a.work = fused->counters + plan->nodes.size();
    e = launch_partition(a, (int)plan->items.size(), s.head_dim, fp8, plan->ntmax, plan->occ, st,
                         plan->ev_before, plan->ev_after, true);
    if (e != hipSuccess) return hip_fail(e, "fused partition kernel launch");
    return PA_OK;
  }
  e = launch_partition(a, (int)plan->items.size(), s.head_dim, fp8, plan->ntmax, plan->occ, st,
                       plan->ev_before, plan->ev_after);
  if (e != hipSuccess) return hip_fail(e, "partition kernel launch");
  if (!plan->red1.empty()) {
    // Two-level merge: chunks of the partials into first-level partials,
    // then the pairs' merge over those.
    a.red = d.red1;
    a.l1_o = d.l1_o;
    a.l1_ml = d.l1_ml;
    e = launch_reduce_stage1(a, (int)plan->red1.size(), s.head_dim, plan->rows_stride, st);
    if (e != hipSuccess) return hip_fail(e, "first-level reduce kernel launch");
    a.red = d.red;
    a.part_o = d.l1_o;
    a.part_ml = d.l1_ml;
  }
  e = launch_reduce(a, (int)plan->red.size(), s.head_dim, plan->rows_stride, plan->max_parts, st);
  if (e != hipSuccess) return hip_fail(e, "reduce kernel launch");
  return PA_OK;
}

pa_status decode(const pa_plan_t* plan, const int32_t* dev_ctx, const void* q, const void* k_pool,
                 const void* v_pool, const int32_t* block_table, const float* k_scales,
                 const float* v_scales, const float* sinks, void* out, void* stream,
                 bool fused = false) {
  if (!plan) return fail(PA_E_INVALID, "plan is NULL");
  if (plan->device < 0) return fail(PA_E_INVALID, "a host-only plan cannot run");
  if (plan->items.empty()) return PA_OK;  // every sequence is a padded slot
  pa_status st = check_call(plan, q, k_pool, v_pool, block_table, k_scales, v_scales, sinks, out);
  if (st != PA_OK) return st;
  const CallBufs d{plan->d_items, plan->d_red,  plan->d_red1, plan->d_part_o,
                   plan->d_part_ml, plan->d_l1_o, plan->d_l1_ml};
  const FusedBufs f{plan->d_nodes, plan->d_counters, plan->d_tree_o, plan->d_tree_ml};
  return launch_call(plan, d, dev_ctx, q, k_pool, v_pool, block_table, k_scales, v_scales, sinks,
                     out, static_cast<hipStream_t>(stream), fused ? &f : nullptr);
}

// Device lengths need bounds for windowed plans (see pa_decode_verify_dev).
pa_status check_dev_lengths(const pa_plan_t* plan) {
  if (!plan->shape.lengths_are_bounds)
    for (const SeqInfo& si : plan->seqs)
      if (si.q_len > 0 && si.window > 0)
        return fail(PA_E_INVALID,
                    "a windowed plan read with device lengths must be built with "
                    "lengths_are_bounds = 1");
  return PA_OK;
}

// Byte offsets of one zero-allocation call's buffers in the static scratch
// (each 256-byte aligned); `total` is what the call needs.
struct StaticLayout {
  size_t items, red, red1, part_o, part_ml, l1_o, l1_ml, total;
};

StaticLayout static_layout(const pa_plan_t* p) {
  auto up = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t D = (size_t)p->shape.head_dim, R = (size_t)p->rows_stride;
  StaticLayout L{};
  size_t o = 0;
  L.items = o; o += up(p->items.size() * sizeof(WorkItem));
  L.red = o; o += up(p->red.size() * sizeof(ReduceItem));
  L.red1 = o; o += up(p->red1.size() * sizeof(ReduceItem));
  L.part_o = o; o += up((size_t)p->n_slots * R * D * sizeof(float));
  L.part_ml = o; o += up((size_t)p->n_slots * R * 2 * sizeof(float));
  L.l1_o = o; o += up((size_t)p->l1_slots * R * D * sizeof(float));
  L.l1_ml = o; o += up((size_t)p->l1_slots * R * 2 * sizeof(float));
  L.total = o;
  return L;
}

}  // namespace

pa_status pa_decode_verify(const pa_plan_t* plan, const void* q, const void* k_pool,
                           const void* v_pool, const int32_t* block_table, const float* k_scales,
                           const float* v_scales, const float* sinks, void* out, void* stream) {
  return decode(plan, nullptr, q, k_pool, v_pool, block_table, k_scales, v_scales, sinks, out,
                stream);
}

pa_status pa_decode_verify_dev(const pa_plan_t* plan, const int32_t* context_lens_dev,
                               const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_table, const float* k_scales,
                               const float* v_scales, const float* sinks, void* out,
                               void* stream) {
  if (!plan) return fail(PA_E_INVALID, "plan is NULL");
  if (!context_lens_dev) return fail(PA_E_INVALID, "context_lens_dev is required");
  pa_status st = check_dev_lengths(plan);
  if (st != PA_OK) return st;
  return decode(plan, context_lens_dev, q, k_pool, v_pool, block_table, k_scales, v_scales, sinks,
                out, stream);
}

pa_status pa_decode_verify_fused(const pa_plan_t* plan, const int32_t* context_lens_dev,
                                 const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* block_table, const float* k_scales,
                                 const float* v_scales, const float* sinks, void* out,
                                 void* stream) {
  if (!plan) return fail(PA_E_INVALID, "plan is NULL");
  if (context_lens_dev) {
    pa_status st = check_dev_lengths(plan);
    if (st != PA_OK) return st;
  }
  return decode(plan, context_lens_dev, q, k_pool, v_pool, block_table, k_scales, v_scales, sinks,
                out, stream, true);
}

pa_status pa_decode_verify_noalloc(const pa_plan_t* plan, const void* q, const void* k_pool,
                                   const void* v_pool, const int32_t* block_table,
                                   const float* k_scales, const float* v_scales,
                                   const float* sinks, void* out, void* stream) {
  if (!plan) return fail(PA_E_INVALID, "plan is NULL");
  if (plan->items.empty()) return PA_OK;  // every sequence is a padded slot
  pa_status st = check_call(plan, q, k_pool, v_pool, block_table, k_scales, v_scales, sinks, out);
  if (st != PA_OK) return st;
  const StaticLayout L = static_layout(plan);
  if (L.total > kNoAllocScratchBytes)
    return fail(PA_E_UNSUPPORTED,
                "the call needs %zu bytes of work list and partials; the static scratch of the "
                "zero-allocation call holds %zu (use pa_decode_verify, or larger work items)",
                L.total, (size_t)kNoAllocScratchBytes);
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (plan->device >= 0 && plan->device != dev)
    return fail(PA_E_INVALID, "the plan was built for device %d, the current device is %d",
                plan->device, dev);
  unsigned char* base = nullptr;
  e = noalloc_scratch(dev, reinterpret_cast<void**>(&base));
  if (e != hipSuccess) return hip_fail(e, "locating the static scratch");
  hipStream_t hs = static_cast<hipStream_t>(stream);
  // The work lists go in ahead of the kernels on the same stream.
  auto put = [&](size_t off, const void* src, size_t bytes) -> hipError_t {
    if (bytes == 0) return hipSuccess;
    return hipMemcpyAsync(base + off, src, bytes, hipMemcpyHostToDevice, hs);
  };
  e = put(L.items, plan->items.data(), plan->items.size() * sizeof(WorkItem));
  if (e == hipSuccess) e = put(L.red, plan->red.data(), plan->red.size() * sizeof(ReduceItem));
  if (e == hipSuccess) e = put(L.red1, plan->red1.data(), plan->red1.size() * sizeof(ReduceItem));
  if (e != hipSuccess) return hip_fail(e, "copying the work list into the static scratch");
  const CallBufs d{reinterpret_cast<const WorkItem*>(base + L.items),
                   reinterpret_cast<const ReduceItem*>(base + L.red),
                   reinterpret_cast<const ReduceItem*>(base + L.red1),
                   reinterpret_cast<float*>(base + L.part_o),
                   reinterpret_cast<float*>(base + L.part_ml),
                   reinterpret_cast<float*>(base + L.l1_o),
                   reinterpret_cast<float*>(base + L.l1_ml)};
  return launch_call(plan, d, nullptr, q, k_pool, v_pool, block_table, k_scales, v_scales, sinks,
                     out, hs);
}

pa_status pa_stream_floor(const pa_plan_t* plan, const void* k_pool, const void* v_pool,
                          const int32_t* block_table, const float* k_scales,
                          const float* v_scales, void* stream) {
  if (!plan) return fail(PA_E_INVALID, "plan is NULL");
  if (plan->device < 0) return fail(PA_E_INVALID, "a host-only plan cannot run");
  const pa_shape& s = plan->shape;
  const bool fp8 = s.kv_dtype == PA_FP8_E4M3;
  if (plan->items.empty()) return PA_OK;
  if (!k_pool || !v_pool || !block_table)
    return fail(PA_E_INVALID, "k_pool, v_pool and block_table are required");
  if (fp8 != (k_scales && v_scales))
    return fail(PA_E_INVALID, "scales are required exactly for FP8 KV");
  KernelArgs a{};
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.block_table = block_table;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.items = plan->d_items;
  a.num_kv_heads = s.num_kv_heads;
  a.max_blocks = s.max_blocks_per_seq;
  const hipError_t e = launch_stream_floor(a, (int)plan->items.size(), s.head_dim, fp8,
                                           static_cast<hipStream_t>(stream), plan->ev_before,
                                           plan->ev_after);
  if (e != hipSuccess) return hip_fail(e, "stream floor kernel launch");
  return PA_OK;
}

pa_status pa_kv_append(const pa_plan_t* plan, const void* k_new, const void* v_new,
                       const int32_t* block_table, void* k_pool, void* v_pool,
                       float* k_scales, float* v_scales, void* stream) {
  if (!plan) return fail(PA_E_INVALID, "plan is NULL");
  const pa_shape& s = plan->shape;
  const bool fp8 = s.kv_dtype == PA_FP8_E4M3;
  // The append kernel has one instance per served (head dim, KV dtype):
  // 64 and 128 with either KV dtype, 256 with FP8 KV (what validate()
  // accepts). Anything else is refused here, never run on another instance.
  if (!((s.head_dim == 64 || s.head_dim == 128) || (s.head_dim == 256 && fp8)))
    return fail(PA_E_UNSUPPORTED, "no KV append for head_dim %d with %s KV", s.head_dim,
                fp8 ? "FP8" : "bf16");
  // The new tokens' positions come from the plan's lengths; on a plan built
  // on upper bounds those are not the lengths a device-length call reads.
  if (s.lengths_are_bounds)
    return fail(PA_E_INVALID,
                "a plan built on upper bounds (lengths_are_bounds = 1) has no new-token "
                "positions: plan the append with the step's actual lengths");
  if (plan->device < 0) return fail(PA_E_INVALID, "a host-only plan cannot run");
  if (plan->tokens.empty()) return PA_OK;  // no sequence brings a new token
  if (!k_new || !v_new || !block_table || !k_pool || !v_pool)
    return fail(PA_E_INVALID, "k_new, v_new, block_table, k_pool and v_pool are required");
  if (fp8 && (!k_scales || !v_scales))
    return fail(PA_E_INVALID, "FP8 KV needs k_scales and v_scales");
  if (!fp8 && (k_scales || v_scales)) return fail(PA_E_INVALID, "bf16 KV takes no scales");
  // Each lane moves D / 64 values: 8 bytes of bf16 input at head dim 256.
  const uintptr_t align = s.head_dim == 256 ? 8 : 4;
  if ((reinterpret_cast<uintptr_t>(k_new) | reinterpret_cast<uintptr_t>(v_new) |
       reinterpret_cast<uintptr_t>(k_pool) | reinterpret_cast<uintptr_t>(v_pool)) & (align - 1))
    return fail(PA_E_INVALID, "k_new, v_new, k_pool and v_pool must be %d-byte aligned",
                (int)align);

  AppendArgs a{};
  a.k_new = static_cast<const uint16_t*>(k_new);
  a.v_new = static_cast<const uint16_t*>(v_new);
  a.block_table = block_table;
  a.tokens = plan->d_tokens;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_scales = k_scales;
  a.v_scales = v_scales;
  a.num_tokens = (int32_t)(plan->tokens.size() / 2);
  a.num_kv_heads = s.num_kv_heads;
  a.max_blocks = s.max_blocks_per_seq;
  a.num_blocks = s.num_blocks;
  hipError_t e = launch_append(a, s.head_dim, fp8, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append kernel launch");
  return PA_OK;
}

pa_status pa_verify_greedy(const pa_plan_t* plan, const void* logits, pa_dtype logits_dtype,
                           int32_t vocab, int64_t row_stride, const int32_t* input_ids,
                           int32_t* out_ids, int32_t* accepted, int32_t* next_ids, void* stream) {
  if (!plan) return fail(PA_E_INVALID, "plan is NULL");
  if (plan->device < 0) return fail(PA_E_INVALID, "a host-only plan cannot run");
  if (logits_dtype != PA_BF16 && logits_dtype != PA_FP32)
    return fail(PA_E_UNSUPPORTED, "logits must be bf16 or fp32");
  if (vocab < 1) return fail(PA_E_INVALID, "vocab %d < 1", vocab);
  if (row_stride < vocab)
    return fail(PA_E_INVALID, "row_stride %lld is smaller than vocab %d", (long long)row_stride,
                vocab);
  const int esz = logits_dtype == PA_BF16 ? 2 : 4;
  if ((row_stride * esz) % 16 != 0)
    return fail(PA_E_INVALID, "a logits row must span a multiple of 16 bytes (row_stride %lld)",
                (long long)row_stride);
  if (plan->tokens.empty()) return PA_OK;  // every sequence is a padded slot
  if (!logits || !input_ids || !out_ids || !accepted || !next_ids)
    return fail(PA_E_INVALID, "logits, input_ids, out_ids, accepted and next_ids are required");
  if (reinterpret_cast<uintptr_t>(logits) % 16 != 0)
    return fail(PA_E_INVALID, "logits must be 16-byte aligned");

  VerdictArgs a{};
  a.logits = logits;
  a.row_stride = row_stride;
  a.vocab = vocab;
  const int64_t per = ((int64_t)vocab + kVerdictSlices - 1) / kVerdictSlices;
  a.slice = (int32_t)(((per + 7) / 8) * 8);
  a.logits_bf16 = logits_dtype == PA_BF16;
  a.num_tokens = (int32_t)(plan->tokens.size() / 2);
  a.num_seqs = plan->shape.num_seqs;
  a.seq_rows = plan->d_seq_rows;
  a.input_ids = input_ids;
  a.part_val = plan->d_verdict_val;
  a.part_idx = plan->d_verdict_idx;
  a.out_ids = out_ids;
  a.accepted = accepted;
  a.next_ids = next_ids;
  hipError_t e = launch_verdict(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "verdict kernel launch");
  return PA_OK;
}

void pa_free(pa_plan_t* plan) {
  if (!plan) return;
  release_device(plan);
  delete plan;
}

pa_status pa_plan_info(const pa_plan_t* plan, int64_t* kv_bytes, int64_t* scratch_bytes,
                       int32_t* work_items, int32_t* partition_tokens) {
  if (!plan) return fail(PA_E_INVALID, "plan is NULL");
  if (kv_bytes) *kv_bytes = plan->kv_bytes;
  if (scratch_bytes) *scratch_bytes = plan->scratch_bytes;
  if (work_items) *work_items = (int32_t)plan->items.size();
  if (partition_tokens) *partition_tokens = plan->partition_tokens;
  return PA_OK;
}

pa_status pa_plan_items(const pa_plan_t* plan, int32_t* items, int32_t capacity) {
  if (!plan) return fail(PA_E_INVALID, "plan is NULL");
  if (capacity > 0 && !items) return fail(PA_E_INVALID, "items is NULL");
  const int32_t n = std::min<int32_t>(capacity, (int32_t)plan->items.size());
  for (int32_t i = 0; i < n; ++i) {
    const WorkItem& it = plan->items[i];
    int32_t* r = items + (int64_t)kItemFields * i;
    r[0] = it.seq;
    r[1] = it.kv_head;
    r[2] = it.key_begin;
    r[3] = it.key_end;
    r[4] = it.slot;
    r[5] = it.row0;
    r[6] = it.nrows;
  }
  return PA_OK;
}

pa_status pa_set_workgroup_stamps(pa_plan_t* plan, void* stamps, int64_t capacity) {
  if (!plan) return fail(PA_E_INVALID, "plan is NULL");
  const int64_t need = (int64_t)kStampsPerItem * (int64_t)plan->items.size();
  if (stamps && capacity < need)
    return fail(PA_E_INVALID, "the stamps buffer holds %lld entries; the plan's %zu work items "
                "need %lld", (long long)capacity, plan->items.size(), (long long)need);
  plan->stamps = static_cast<unsigned long long*>(stamps);
  return PA_OK;
}

pa_status pa_set_partition_events(pa_plan_t* plan, void* before, void* after) {
  if (!plan) return fail(PA_E_INVALID, "plan is NULL");
  if ((before == nullptr) != (after == nullptr))
    return fail(PA_E_INVALID, "give both events or neither");
  plan->ev_before = static_cast<hipEvent_t>(before);
  plan->ev_after = static_cast<hipEvent_t>(after);
  return PA_OK;
}

}  // extern "C"
