// Internal declarations shared by the host planner (pa_plan.cpp) and the
// gfx950 kernels (pa_kernels.hip). Not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pav {

constexpr int kBlock = 16;      // tokens per KV block
constexpr int kChunk = 32;      // tokens one wave consumes per iteration (two blocks)
constexpr int kWaves = 4;       // waves per workgroup; each takes every 4th chunk
constexpr int kThreads = 64 * kWaves;
constexpr int kMaxRows = 64;    // q x G packed rows per KV head (4 MFMA row tiles)
constexpr int kMaxQuery = 8;
constexpr int kMaxContext = 1 << 20;
// Keys per work item: each wave keeps the page ids of its (at most 64)
// chunks in one register, one chunk per lane.
constexpr int kMaxItemKeys = 64 * kWaves * kChunk;  // 8192
constexpr float kLog2e = 1.4426950408889634f;

// One workgroup's share of the work: the keys [key_begin, key_end) of one
// (sequence, KV head). slot < 0 means the item covers all of the pair's
// visible keys and writes the final output itself.
struct WorkItem {
  int32_t seq;
  int32_t kv_head;
  int32_t key_begin;
  int32_t key_end;
  int32_t slot;
  // the sequence's fields, repeated here so one load brings everything
  int32_t ctx_len;
  int32_t q_len;
  int32_t q_off;
  int32_t window;
  int32_t pad[7];
};

struct SeqInfo {
  int32_t ctx_len;   // L
  int32_t q_len;     // q (0: padded slot)
  int32_t q_off;     // first query row of this sequence in q/out
  int32_t lo;        // first key any row may see (window), else 0
  int32_t window;    // W, 0 = none
  int32_t n_parts;   // work items per KV head
  int32_t slot_base; // partial slot of (kv head 0, part 0) when n_parts > 1
  int32_t pad;
};

// A (sequence, KV head) whose partials the reduce kernel merges.
struct ReduceItem {
  int32_t seq;
  int32_t kv_head;
  int32_t slot_base;
  int32_t n_parts;
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
  float* part_o;   // [slots][rows_stride][D]
  float* part_ml;  // [slots][rows_stride][2]: running max (log2 units), sum
  const WorkItem* items;
  const SeqInfo* seqs;
  const ReduceItem* red;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t max_blocks;
  int32_t rows_stride;
  int32_t sinks_mode;
  int32_t out_fp32;
  float scale_log2;  // softmax scale x log2(e)
};

hipError_t launch_partition(const KernelArgs& a, int n_items, int head_dim, bool fp8,
                            hipStream_t stream);
hipError_t launch_reduce(const KernelArgs& a, int n_red, int head_dim, hipStream_t stream);

}  // namespace pav
