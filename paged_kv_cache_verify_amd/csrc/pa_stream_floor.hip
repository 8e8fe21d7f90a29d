// Streaming floor of a plan: a kernel that reads exactly the KV bytes the
// plan's partition kernel reads (every work item's pages of K and V, and
// the FP8 scales), through the same block table, with the same 1 KiB
// direct global-to-LDS loads and nontemporal policy, one workgroup per work
// item, and computes nothing. Its duration is the time this call size and
// page pattern allow for the bytes alone: the floor the partition kernel's
// streaming is measured against. (It is a measurement kernel; no result of
// the attention depends on it.)
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pav {
namespace {

constexpr int kFloorWaves = 8;      // waves per workgroup
constexpr int kFloorInFlight = 48;  // loads a wave keeps in flight (vmcnt)

#define PAV_FLOOR_LDS __attribute__((address_space(3))) void

// Wave w of NW streams the contiguous share [n w / NW, n (w + 1) / NW) of
// the item's n 16-token pages: for each, the K page (D x esz x 16 bytes, in
// 1 KiB loads of 16 bytes per lane), the V page, and for FP8 the page's
// 64-byte K and V scale rows. The page ids come first, 64 per vector load
// (lane j: page j of the batch), so no page waits on a scalar load of its
// id. Every load lands in the wave's own 1 KiB of LDS, which nothing reads;
// a wave keeps at most kFloorInFlight loads in flight. (Measured on the
// MTP-5 bf16 workload: 1 to 16 waves and 12 to 48 loads in flight per wave
// all stream within 3% of one another, so the floor does not depend on
// this choice.)
template <int ROWB, bool FP8>
__global__ __launch_bounds__(64 * kFloorWaves) void pa_stream_floor_kernel(KernelArgs A) {
  __shared__ __attribute__((aligned(1024))) unsigned char sink[kFloorWaves][1024];
  constexpr int BLKB = kBlock * ROWB;  // bytes per (page, KV head)
  constexpr int LD = BLKB / 1024;      // 1 KiB loads per page of K (or V)
  const WorkItem it = A.items[blockIdx.x];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tv0 = it.key_begin, tv1 = it.key_end;
  if (tv1 <= tv0) return;
  const int p0 = tv0 / kBlock, n = (tv1 + kBlock - 1) / kBlock - p0;
  const int q0 = p0 + n * w / kFloorWaves, q1 = p0 + n * (w + 1) / kFloorWaves;
  const int32_t* bt = A.block_table + (int64_t)it.seq * A.max_blocks;
  unsigned char* dst = sink[w];
  for (int b0 = q0; b0 < q1; b0 += 64) {
    const int cnt = min(64, q1 - b0);
    int pid = 0;
    if (lane < cnt) pid = bt[b0 + lane];
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): the page ids are in
    for (int j = 0; j < cnt; ++j) {
      const int page = __builtin_amdgcn_readlane(pid, j);
      const int64_t base = ((int64_t)page * A.num_kv_heads + it.kv_head) * BLKB;
      const char* k = static_cast<const char*>(A.k_pool) + base + lane * 16;
      const char* v = static_cast<const char*>(A.v_pool) + base + lane * 16;
#pragma unroll
      for (int u = 0; u < LD; ++u) {
        __builtin_amdgcn_global_load_lds(k + u * 1024, (PAV_FLOOR_LDS*)dst, 16, 0, 2);
        __builtin_amdgcn_global_load_lds(v + u * 1024, (PAV_FLOOR_LDS*)dst, 16, 0, 2);
      }
      if constexpr (FP8) {  // lanes 0..15: K scales, 16..31: V scales of the page
        const int64_t so = ((int64_t)page * A.num_kv_heads + it.kv_head) * kBlock + (lane & 15);
        const float* s = (lane < 16 ? A.k_scales : A.v_scales) + so;
        if (lane < 32) __builtin_amdgcn_global_load_lds(s, (PAV_FLOOR_LDS*)dst, 4, 0, 2);
      }
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kFloorInFlight) : "memory");
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace

template <int ROWB, bool FP8>
static void launch_floor_one(const KernelArgs& a, int n_items, hipStream_t stream,
                             hipEvent_t ev_start, hipEvent_t ev_stop) {
  const dim3 grid(n_items), block(64 * kFloorWaves);
  if (ev_start && ev_stop)
    hipExtLaunchKernelGGL((pa_stream_floor_kernel<ROWB, FP8>), grid, block, 0, stream, ev_start,
                          ev_stop, 0, a);
  else
    hipLaunchKernelGGL((pa_stream_floor_kernel<ROWB, FP8>), grid, block, 0, stream, a);
}

hipError_t launch_stream_floor(const KernelArgs& a, int n_items, int head_dim, bool fp8,
                               hipStream_t stream, hipEvent_t ev_start, hipEvent_t ev_stop) {
  if (n_items <= 0) return hipSuccess;
  // Template argument: bytes per token row of a page (D x element size).
  const hipEvent_t e0 = ev_start, e1 = ev_stop;
  if (fp8 && head_dim == 256) launch_floor_one<256, true>(a, n_items, stream, e0, e1);
  else if (fp8 && head_dim == 128) launch_floor_one<128, true>(a, n_items, stream, e0, e1);
  else if (fp8 && head_dim == 64) launch_floor_one<64, true>(a, n_items, stream, e0, e1);
  else if (!fp8 && head_dim == 128) launch_floor_one<256, false>(a, n_items, stream, e0, e1);
  else if (!fp8 && head_dim == 64) launch_floor_one<128, false>(a, n_items, stream, e0, e1);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace pav
