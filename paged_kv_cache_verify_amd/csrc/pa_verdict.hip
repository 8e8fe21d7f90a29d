// gfx950 kernels for the greedy verify verdict: the step after the target's
// head in a verify round. For every verify row the target's argmax over the
// vocabulary, then per sequence the number of leading draft tokens the
// target agrees with and the next token.
//
// Two launches. The argmax pass splits each row's vocabulary into
// kVerdictSlices slices, one 256-thread workgroup each (enough workgroups to
// fill the chip at a few dozen rows); every thread scans its 16-byte vectors
// in index order, keeping the first largest value, then the workgroup
// reduces (value, index) pairs, lower index first among equal values. The
// verdict pass (one workgroup per sequence) merges a row's slices the same
// way and applies the acceptance rule.
//
// Source: ATOM #3091 ("High-interactivity monokernel decode for
// DeepSeek-V4.1-Flash on MI355X"): the verify head produces the step's ids
// and verdict in one launch for greedy rows (Engine hooks), and the next
// step's input is taken from the output ids at the verdict's accepted count
// (the review rounds on the head-served verify).
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pav {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// (v, i) replaces (bv, bi) when it is larger, or equal with a lower index.
__device__ __forceinline__ void better(float v, int i, float& bv, int& bi) {
  if (v > bv || (v == bv && i < bi)) {
    bv = v;
    bi = i;
  }
}

// Wave-wide argmax of (bv, bi) pairs; every lane ends with the result.
__device__ __forceinline__ void wave_argmax(float& bv, int& bi) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    const float ov = __shfl_xor(bv, m, 64);
    const int oi = __shfl_xor(bi, m, 64);
    better(ov, oi, bv, bi);
  }
}

constexpr int kThreads = 256;
constexpr int kNoIndex = 0x7FFFFFFF;  // no value above -inf seen

__global__ __launch_bounds__(kThreads) void verdict_argmax_kernel(VerdictArgs A) {
  const int row = blockIdx.x / kVerdictSlices;
  const int s = blockIdx.x % kVerdictSlices;
  const int lo = s * A.slice;
  const int hi = min(A.vocab, lo + A.slice);
  float bv = -INFINITY;
  int bi = kNoIndex;
  if (A.logits_bf16) {
    const uint16_t* base = static_cast<const uint16_t*>(A.logits) + (int64_t)row * A.row_stride;
    // 8 values per 16-byte vector; thread k takes vectors k, k + 256, ...
    for (int v0 = lo + 8 * (int)threadIdx.x; v0 < hi; v0 += 8 * kThreads) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(base + v0);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t b16 = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        const float x = __uint_as_float(b16 << 16);
        if (v0 + e < hi && x > bv) {
          bv = x;
          bi = v0 + e;
        }
      }
    }
  } else {
    const float* base = static_cast<const float*>(A.logits) + (int64_t)row * A.row_stride;
    for (int v0 = lo + 4 * (int)threadIdx.x; v0 < hi; v0 += 4 * kThreads) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(base + v0);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = __uint_as_float(w[e]);
        if (v0 + e < hi && x > bv) {
          bv = x;
          bi = v0 + e;
        }
      }
    }
  }
  wave_argmax(bv, bi);
  __shared__ float sv[kThreads / 64];
  __shared__ int si[kThreads / 64];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) {
    sv[w] = bv;
    si[w] = bi;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int k = 1; k < kThreads / 64; ++k) better(sv[k], si[k], bv, bi);
    A.part_val[(int64_t)row * kVerdictSlices + s] = bv;
    A.part_idx[(int64_t)row * kVerdictSlices + s] = bi;
  }
}

// One workgroup of 256 threads per sequence: thread (i, s) = (tid / 32,
// tid % 32) merges slice s of verify row i (q <= 8 rows).
__global__ __launch_bounds__(kThreads) void verdict_accept_kernel(VerdictArgs A) {
  const int b = blockIdx.x;
  const int t0 = A.seq_rows[2 * b], q = A.seq_rows[2 * b + 1];
  if (q == 0) return;  // a padded slot writes nothing
  const int i = threadIdx.x >> 5, s = threadIdx.x & 31;
  float bv = -INFINITY;
  int bi = kNoIndex;
  if (i < q) {
    bv = A.part_val[(int64_t)(t0 + i) * kVerdictSlices + s];
    bi = A.part_idx[(int64_t)(t0 + i) * kVerdictSlices + s];
  }
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) {  // within the 32 lanes of row i
    const float ov = __shfl_xor(bv, m, 32);
    const int oi = __shfl_xor(bi, m, 32);
    better(ov, oi, bv, bi);
  }
  __shared__ int a[kMaxQuery];
  if (i < q && s == 0) {
    const int id = bi == kNoIndex ? 0 : bi;
    a[i] = id;
    A.out_ids[t0 + i] = id;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int n = 0;
    while (n < q - 1 && A.input_ids[t0 + 1 + n] == a[n]) ++n;
    A.accepted[b] = n;
    A.next_ids[b] = a[n];
  }
}

}  // namespace

hipError_t launch_verdict(const VerdictArgs& a, hipStream_t stream) {
  if (a.num_tokens <= 0) return hipSuccess;
  hipLaunchKernelGGL(verdict_argmax_kernel, dim3((unsigned)a.num_tokens * kVerdictSlices),
                     dim3(kThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(verdict_accept_kernel, dim3((unsigned)a.num_seqs), dim3(kThreads), 0, stream,
                     a);
  return hipGetLastError();
}

}  // namespace pav
