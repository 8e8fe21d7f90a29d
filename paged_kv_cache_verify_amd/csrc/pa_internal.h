// Internal declarations shared by the host planner (pa_plan.cpp) and the
// gfx950 kernels (pa_kernels.hip). Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pav {

constexpr int kBlock = 16;      // tokens per KV block
constexpr int kChunk = 32;      // tokens a wave consumes per iteration (two blocks)
constexpr int kMaxRows = 128;      // q x G packed rows per KV head
// Rows one partition workgroup carries: 4 MFMA row tiles, 3 at head_dim 256.
// A sequence with more rows is split into row blocks of at most this many,
// each a work item of its own over the same keys.
constexpr int kItemRows = 64;
constexpr int kItemRows256 = 48;
constexpr int kMaxQuery = 8;
constexpr int kMaxContext = 1 << 20;
// Keys a work item spans from its page-aligned start; the workgroup keeps
// the page ids of its (at most 256) chunks in LDS.
constexpr int kMaxItemKeys = 8192;
constexpr int kMaxItemChunks = kMaxItemKeys / kChunk;
constexpr float kLog2e = 1.4426950408889634f;

// One workgroup's share of the work: the keys [key_begin, key_end) of one
// (sequence, KV head), all its q x G rows.
struct WorkItem {
  int32_t seq;
  int32_t kv_head;
  int32_t key_begin;
  int32_t key_end;
  // slot < 0: the item covers all of the pair's visible keys and writes the
  // output itself; otherwise it writes partial `slot`, which the reduce
  // kernel merges with the pair's other partials.
  int32_t slot;
  // the sequence's fields, repeated here so one load brings everything
  int32_t ctx_len;
  int32_t q_len;
  int32_t q_off;
  int32_t window;
  // the item's packed rows: [row0, row0 + nrows) of the q x G rows
  int32_t row0;
  int32_t nrows;
  // fused call: the merge node this item's partial arrives at (-1 when
  // slot < 0)
  int32_t node;
  int32_t pad[4];
};

// Fan-in of a merge node in the fused call: a split pair with at most this
// many partials is merged in one node, more go through a tree of nodes.
constexpr int kFusedFanIn = 16;

// One merge of the fused call (single launch, no reduce kernel): n_parts
// partials, slots slot_base + j * slot_stride (j < n_parts) of the partition
// partials (from_tree 0) or of the tree slots (1), rows [row0, row0 + nrows)
// of (seq, kv_head). The workgroup whose arrival brings the node's counter
// to n_parts merges them: into the output (parent < 0), or into tree slot
// out_slot, after which it arrives at node `parent`.
struct MergeNode {
  int32_t seq;
  int32_t kv_head;
  int32_t q_len;
  int32_t q_off;
  int32_t row0;
  int32_t nrows;
  int32_t slot_base;
  int32_t n_parts;
  int32_t from_tree;
  int32_t out_slot;
  int32_t parent;
  int32_t slot_stride;
  int32_t pad[4];
};

// A split (sequence, KV head) whose partials [slot_base, slot_base +
// n_parts) the reduce kernel merges.
struct ReduceItem {
  int32_t seq;
  int32_t kv_head;
  int32_t slot_base;
  int32_t n_parts;
  int32_t q_len;
  int32_t q_off;
  // first level of a two-level merge: the first-level slot this chunk of
  // the pair's partials merges into (unused otherwise)
  int32_t out_slot;
  int32_t pad;
};

struct KernelArgs {
  const uint16_t* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const float* k_scales;
  const float* v_scales;
  const float* sinks;
  void* out;
  float* part_o;     // [slots][rows_stride][D]
  float* part_ml;    // [slots][rows_stride][2]: max (log2 units), sum
  const WorkItem* items;
  const ReduceItem* red;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t max_blocks;
  int32_t rows_stride;
  int32_t sinks_mode;
  int32_t out_fp32;
  float scale_log2;  // softmax scale x log2(e)
  // Device context lengths [B] read at run time (the plan's lengths are
  // then upper bounds), or null: the plan's own lengths.
  const int32_t* dev_ctx;
  // First-level scratch of the two-level merge (pairs with more than 32
  // partials): [chunks][rows_stride][D] and [chunks][rows_stride][2].
  float* l1_o;
  float* l1_ml;
  // Fused call (null otherwise): merge nodes, one arrival counter per node
  // (zero between calls: the last arriver resets it), and the tree slots
  // [slots][rows_stride][D] and [slots][rows_stride][2].
  const MergeNode* nodes;
  int32_t* counters;
  float* tree_o;
  float* tree_ml;
  // Fused call's persistent grid: the work list's length, the grid (at most
  // the device's resident workgroups) and two counters, zero between calls
  // (the next item to take; the workgroups done).
  int32_t n_items;
  int32_t grid;
  int32_t* work;
  // Optional per-workgroup stamps of the partition kernel (null: none):
  // kStampsPerItem uint64 per work item, see pa_set_workgroup_stamps.
  unsigned long long* stamps;
};
constexpr int kStampsPerItem = 8;

// The new tokens of a verify step, for the paged KV append kernel.
struct AppendArgs {
  const uint16_t* k_new;       // [T][Hkv][D] bf16
  const uint16_t* v_new;
  const int32_t* block_table;  // [B][max_blocks]
  const int32_t* tokens;       // [T][2]: sequence, position of new token t
  void* k_pool;                // [num_blocks][Hkv][16][D] bf16 or e4m3
  void* v_pool;
  float* k_scales;             // [num_blocks][Hkv][16] (FP8 only)
  float* v_scales;
  int32_t num_tokens;
  int32_t num_kv_heads;
  int32_t max_blocks;
  int32_t num_blocks;
};

// The greedy verify verdict.
constexpr int kVerdictSlices = 32;  // workgroups per verify row in the argmax pass
struct VerdictArgs {
  const void* logits;        // [T][row_stride], bf16 or fp32
  int64_t row_stride;        // elements
  int32_t vocab;
  int32_t slice;             // vocabulary entries per slice (a multiple of 8)
  int32_t logits_bf16;
  int32_t num_tokens;        // T
  int32_t num_seqs;          // B
  const int32_t* seq_rows;   // [B][2]: first verify row, verify rows (q)
  const int32_t* input_ids;  // [T]
  float* part_val;           // [T][kVerdictSlices]
  int32_t* part_idx;         // [T][kVerdictSlices]
  int32_t* out_ids;          // [T]
  int32_t* accepted;         // [B]
  int32_t* next_ids;         // [B]
};

hipError_t launch_verdict(const VerdictArgs& a, hipStream_t stream);

// ntmax: row tiles of 16 the kernel is built for (ceil(max q x G / 16));
// items with fewer rows skip the missing tiles. occ: workgroups meant to
// share a CU, 1 (items fit one round) or 2 (more items than CUs, bf16 KV
// only).
// ev_start, ev_stop: optional timing events taken by the launch itself.
// fused: the single-launch variant, whose split items merge their pair's
// partials themselves (a.nodes, a.counters, a.tree_o, a.tree_ml set).
hipError_t launch_partition(const KernelArgs& a, int n_items, int head_dim, bool fp8, int ntmax,
                            int occ, hipStream_t stream, hipEvent_t ev_start = nullptr,
                            hipEvent_t ev_stop = nullptr, bool fused = false);
// rows_stride: the most rows any reduce item has; max_parts: the most
// partials any reduce item merges (picks the reduce kernel's shape).
hipError_t launch_reduce(const KernelArgs& a, int n_red, int head_dim, int rows_stride,
                         int max_parts, hipStream_t stream);
// First level of the two-level merge: a.red lists n_chunks chunks of a
// pair's partials (ReduceItem::out_slot: the first-level slot written).
hipError_t launch_reduce_stage1(const KernelArgs& a, int n_chunks, int head_dim, int rows_stride,
                                hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, int head_dim, bool fp8, hipStream_t stream);
// The streaming-floor measurement kernel over a plan's work items (timing
// events as for launch_partition).
hipError_t launch_stream_floor(const KernelArgs& a, int n_items, int head_dim, bool fp8,
                               hipStream_t stream, hipEvent_t ev_start = nullptr,
                               hipEvent_t ev_stop = nullptr);

// The zero-allocation attention call's scratch: a file-scope device array of
// this many bytes (pa_noalloc.hip), one copy per device the library runs on.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
// Its device address on `device` (which must be the current device), looked
// up once per device and cached.
hipError_t noalloc_scratch(int device, void** ptr);

}  // namespace pav
