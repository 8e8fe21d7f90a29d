// gfx950 kernel for the paged KV append: the step of a verify step that
// stores its new tokens' K and V rows into their 16-token pages before the
// attention kernels read them.
//
// One wave per stored row (one token, one KV head, K or V): the wave loads
// the D bf16 values (D / 64 per lane: one, two or four), and either copies
// them bit for bit (bf16 pool) or quantises them to e4m3 with the row's own fp32 scale,
// scale = amax / 448 (the e4m3 maximum), code = nearest e4m3 value to
// x / scale, ties to the even code. The amax is a wave reduction; lane 0
// writes the scale.
//
// Sources: ATOM #3091 ("High-interactivity monokernel decode for
// DeepSeek-V4.1-Flash on MI355X", Summary: stores into the 16-token pages
// happen only for live rows, so padded requests store nothing); ATOM #2843
// ("keep MTP-5 decode on FlyDSL pa_decode past the gluon query-length
// limit", Motivation: FP8 KV with one fp32 scale per token and KV head).
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pav {
namespace {

constexpr int kAppendRowsPerBlock = 4;  // waves per workgroup

// e4m3 code (bias 7, largest finite 448, no infinities) of v with
// |v| <= 448: round to nearest, ties to the even code.
__device__ inline uint32_t e4m3_rne(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fabsf(v);
  uint32_t code;
  if (a < 0.015625f) {
    // Below 2^-6 the codes 0..8 are the multiples of 2^-9 (code 8 is 2^-6,
    // the first normal): scaling by 2^9 is exact and rint rounds to even.
    code = (uint32_t)__builtin_rintf(a * 512.0f);
  } else {
    // Keep 3 of fp32's 23 mantissa bits, rounding to nearest even on the 20
    // dropped ones (a carry moves into the exponent), then rebias 127 -> 7.
    const uint32_t b = __float_as_uint(a);
    const uint32_t r = b + 0x7FFFFu + ((b >> 20) & 1u);
    code = (r >> 20) - (120u << 3);
  }
  return sign | code;
}

template <int D, bool FP8>
__global__ __launch_bounds__(64 * kAppendRowsPerBlock) void pa_append_kernel(AppendArgs A) {
  constexpr int E = D / 64;  // values per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * kAppendRowsPerBlock + (threadIdx.x >> 6);
  const int64_t rows = (int64_t)A.num_tokens * A.num_kv_heads;  // per tensor (K or V)
  if (row >= 2 * rows) return;
  const bool is_v = row >= rows;
  const int64_t r = is_v ? row - rows : row;  // t * Hkv + g
  const int t = (int)(r / A.num_kv_heads), g = (int)(r % A.num_kv_heads);
  const int seq = A.tokens[2 * t], pos = A.tokens[2 * t + 1];
  const int page = A.block_table[(int64_t)seq * A.max_blocks + pos / kBlock];
  if (page < 0 || page >= A.num_blocks) return;  // never store outside the pool
  const int64_t dst = ((int64_t)page * A.num_kv_heads + g) * kBlock + pos % kBlock;
  const uint16_t* src = (is_v ? A.v_new : A.k_new) + r * D + lane * E;

  // E bf16 values, the first in the low half of word 0.
  uint32_t bits[(E + 1) / 2];
  if constexpr (E == 4) {
    const uint2 v = *reinterpret_cast<const uint2*>(src);
    bits[0] = v.x;
    bits[1] = v.y;
  } else if constexpr (E == 2) {
    bits[0] = *reinterpret_cast<const uint32_t*>(src);
  } else {
    bits[0] = *src;
  }

  if constexpr (!FP8) {
    uint16_t* out = static_cast<uint16_t*>(is_v ? A.v_pool : A.k_pool) + dst * D + lane * E;
    if constexpr (E == 4) *reinterpret_cast<uint2*>(out) = make_uint2(bits[0], bits[1]);
    else if constexpr (E == 2) *reinterpret_cast<uint32_t*>(out) = bits[0];
    else *out = (uint16_t)bits[0];
  } else {
    float x[E];
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      x[e] = __uint_as_float(((bits[e / 2] >> (16 * (e % 2))) & 0xFFFFu) << 16);
      amax = fmaxf(amax, fabsf(x[e]));
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
    const float scale = amax > 0.f ? amax / 448.0f : 1.0f;
    uint32_t codes = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float y = fminf(fmaxf(x[e] / scale, -448.0f), 448.0f);
      codes |= e4m3_rne(y) << (8 * e);
    }
    uint8_t* out = static_cast<uint8_t*>(is_v ? A.v_pool : A.k_pool) + dst * D + lane * E;
    if constexpr (E == 4) *reinterpret_cast<uint32_t*>(out) = codes;
    else if constexpr (E == 2) *reinterpret_cast<uint16_t*>(out) = (uint16_t)codes;
    else *out = (uint8_t)codes;
    if (lane == 0) (is_v ? A.v_scales : A.k_scales)[dst] = scale;
  }
}

}  // namespace

hipError_t launch_append(const AppendArgs& a, int head_dim, bool fp8, hipStream_t stream) {
  const int64_t rows = 2LL * a.num_tokens * a.num_kv_heads;
  if (rows <= 0) return hipSuccess;
  const dim3 grid((unsigned)((rows + kAppendRowsPerBlock - 1) / kAppendRowsPerBlock));
  const dim3 block(64 * kAppendRowsPerBlock);
  // One instance per head dim the attention serves (head 256 with FP8 KV
  // only); any other combination is refused here, before a launch.
  if (head_dim == 256) {
    if (!fp8) return hipErrorInvalidValue;
    hipLaunchKernelGGL((pa_append_kernel<256, true>), grid, block, 0, stream, a);
  } else if (head_dim == 128) {
    if (fp8) hipLaunchKernelGGL((pa_append_kernel<128, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((pa_append_kernel<128, false>), grid, block, 0, stream, a);
  } else if (head_dim == 64) {
    if (fp8) hipLaunchKernelGGL((pa_append_kernel<64, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((pa_append_kernel<64, false>), grid, block, 0, stream, a);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pav
