// gfx950 kernels for paged verify attention.
//
// Partition kernel: one workgroup (4 waves) per work item = the keys
// [key_begin, key_end) of one (sequence, KV head). Every wave takes every
// 4th 32-token chunk (two 16-token pages) of the item and keeps its own
// online-softmax state for all q x G packed rows of the KV head; the four
// states are merged in LDS at the end. Per chunk a wave
//   1. reads the two page ids from the block table (wave-uniform),
//   2. loads K straight from HBM into MFMA A-operand registers (token on M,
//      16 contiguous bytes per lane) and V in token-major 1 KiB slabs,
//      both one chunk ahead of use,
//   3. computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16 (FP8 codes are
//      first converted exactly to bf16 in registers; the per-token K scale
//      multiplies the scores),
//   4. masks (causal within the query, window, key range) by selecting -inf,
//   5. runs the online softmax in the exp2 domain (row max over 16-lane
//      groups via cross-lane exchange),
//   6. writes V transposed-on-read into a wave-private, XOR-swizzled LDS
//      tile (invalid tokens zeroed), gathers the V^T A-operand, and
//      accumulates O^T += V^T P^T, the P^T B-operand coming straight from the
//      S^T accumulator registers (the per-token V scale folded into P).
// The log-sum-exp reduce kernel merges the partial (O, m, l) of split pairs.
//
// Sources: ATOM #2843 ("keep MTP-5 decode on FlyDSL pa_decode past the gluon
// query-length limit", Motivation and Follow-up in aiter: rows = query length
// x GQA group, per-token FP8 KV scales, a partition kernel and a reducer);
// ATOM #3091 (Summary: 16-token pages through a block table, stores masked
// by row liveness).
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pav {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));

template <int D, bool FP8>
struct Cfg {
  static constexpr int KS = D / 32;                 // QK contraction steps of 32
  static constexpr int MT = D / 16;                 // PV output tiles along D
  static constexpr int ESZ = FP8 ? 1 : 2;           // bytes per KV element
  static constexpr int ROWB = D * ESZ;              // bytes per token in a page
  static constexpr int BLKB = kBlock * ROWB;        // bytes per (page, KV head)
  static constexpr int KLD = FP8 ? KS / 2 : KS;     // 16-byte K loads per page per lane
  static constexpr int VLD = (2 * BLKB) / 1024;     // 16-byte V loads per chunk per lane
  static_assert(BLKB >= 1024, "a 1 KiB V slab must stay inside one page");
  static_assert(FP8 ? (KS % 2 == 0) : true, "FP8 loads cover two contraction steps");
};

// Element offset of the 8 contraction values a lane holds for QK step s.
// bf16: lane group c holds d = 32 s + 8 c .. +8 (64 contiguous bytes per
// token across the 4 lane groups). FP8: one 16-byte load covers steps
// 2u and 2u+1, d = 64 u + 16 c + 8 (s & 1) .. +8. Q uses the same map, so the
// contraction order is a permutation of d that both operands share.
template <int D, bool FP8>
__device__ __forceinline__ int qk_dmap(int s, int c) {
  return FP8 ? 64 * (s >> 1) + 16 * c + 8 * (s & 1) : 32 * s + 8 * c;
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}

// Eight e4m3 codes (two dwords) -> eight bf16, exactly (every e4m3 value is
// a bf16 value); gfx950 conversion with a unit scale.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16(uint32_t w0, uint32_t w1) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w0, 1.0f, true);
  bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, false);
  bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w1, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ float xlane_max4(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float xlane_sum4(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// LDS V tile of one wave: [32 tokens][D] elements (bf16, or FP8 codes),
// token-major, stored in 16-byte chunks whose position within a token row is
// XOR-swizzled by the token, so that the transposing reads below (16 lanes
// of a group reading 4 tokens x 32 bytes for bf16, 8 tokens x 16 bytes for
// FP8) hit distinct banks.
template <int D, bool FP8>
__device__ __forceinline__ int vswz(int t) {
  if constexpr (FP8) {
    return D == 128 ? ((t & 3) | (((t >> 4) & 1) << 2)) : (((t & 3) >> 1) | (((t >> 4) & 1) << 1));
  } else {
    return D == 128 ? (2 * (t & 3) + 8 * ((t >> 2) & 1)) : 2 * (t & 3);
  }
}

// Byte offset of 16-byte chunk `chunk` of token t in the tile.
template <int D, bool FP8>
__device__ __forceinline__ int vtile_chunk(int t, int chunk) {
  constexpr int ROWB = D * (FP8 ? 1 : 2);
  return t * ROWB + ((chunk ^ vswz<D, FP8>(t)) << 4);
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
#define PAV_LDS __attribute__((address_space(3)))

// ds_read_b64_tr_b16: within each 16-lane group, lane 4r + k names the 8
// bytes at (row r, columns 4k..4k+3) of a 4 x 16 tile of 16-bit values, and
// lane i receives column i (rows 0..3).
__device__ __forceinline__ s16x4 lds_tr16(const unsigned char* base, int off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((PAV_LDS s16x4*)(base + off));
}
// ds_read_b64_tr_b8: lane 2r + k names the 8 bytes at (row r, columns
// 8k..8k+7) of an 8 x 16 tile of bytes; lane i receives column i (rows 0..7).
__device__ __forceinline__ i32x2 lds_tr8(const unsigned char* base, int off) {
  return __builtin_amdgcn_ds_read_tr8_b64_v2i32((PAV_LDS i32x2*)(base + off));
}

template <int D, bool FP8>
struct ChunkRegs {
  u32x4 k[2][Cfg<D, FP8>::KLD];
  u32x4 v[Cfg<D, FP8>::VLD];
  f32x4 ks[2];
  f32x4 vs[2];
};

struct Smem {
  // The V tiles (4 x 32 x D, at most 32 KiB) alias the merge buffers.
  float buf[kWaves][kMaxRows][128];
  float2 ml[kWaves][kMaxRows];
};

struct PageIds {
  int a, b;
};

__device__ __forceinline__ PageIds page_ids(const int32_t* bt, int tok0, int tv1) {
  const int pg = tok0 >> 4;
  PageIds p;
  p.a = bt[pg];
  p.b = (tok0 + kBlock < tv1) ? bt[pg + 1] : p.a;  // never read past the last page
  return p;
}

template <int D, bool FP8>
__device__ __forceinline__ void load_k(ChunkRegs<D, FP8>& R, const KernelArgs& A, PageIds pid,
                                       int g, int lane) {
  using C = Cfg<D, FP8>;
  const int n = lane & 15, c = lane >> 4;
  const char* kp = static_cast<const char*>(A.k_pool);
  const int64_t baseA = ((int64_t)pid.a * A.num_kv_heads + g) * C::BLKB;
  const int64_t baseB = ((int64_t)pid.b * A.num_kv_heads + g) * C::BLKB;
#pragma unroll
  for (int u = 0; u < C::KLD; ++u) {
    const int off = n * C::ROWB + 64 * u + 16 * c;
    R.k[0][u] = *reinterpret_cast<const u32x4*>(kp + baseA + off);
    R.k[1][u] = *reinterpret_cast<const u32x4*>(kp + baseB + off);
  }
  if constexpr (FP8) {
    const int64_t sA = ((int64_t)pid.a * A.num_kv_heads + g) * kBlock + 4 * c;
    const int64_t sB = ((int64_t)pid.b * A.num_kv_heads + g) * kBlock + 4 * c;
    R.ks[0] = *reinterpret_cast<const f32x4*>(A.k_scales + sA);
    R.ks[1] = *reinterpret_cast<const f32x4*>(A.k_scales + sB);
  }
}

template <int D, bool FP8>
__device__ __forceinline__ void load_v(ChunkRegs<D, FP8>& R, const KernelArgs& A, PageIds pid,
                                       int g, int lane) {
  using C = Cfg<D, FP8>;
  const int c = lane >> 4;
  const char* vp = static_cast<const char*>(A.v_pool);
  const int64_t baseA = ((int64_t)pid.a * A.num_kv_heads + g) * C::BLKB;
  const int64_t baseB = ((int64_t)pid.b * A.num_kv_heads + g) * C::BLKB;
#pragma unroll
  for (int u = 0; u < C::VLD; ++u) {
    const int o = u * 1024;
    const int64_t base = (o / C::BLKB) ? baseB : baseA;
    R.v[u] = *reinterpret_cast<const u32x4*>(vp + base + (o % C::BLKB) + lane * 16);
  }
  if constexpr (FP8) {
    const int64_t sA = ((int64_t)pid.a * A.num_kv_heads + g) * kBlock + 4 * c;
    const int64_t sB = ((int64_t)pid.b * A.num_kv_heads + g) * kBlock + 4 * c;
    R.vs[0] = *reinterpret_cast<const f32x4*>(A.v_scales + sA);
    R.vs[1] = *reinterpret_cast<const f32x4*>(A.v_scales + sB);
  }
}

template <int D, bool FP8, int NT>
struct WaveState {
  bf16x8 q[NT][Cfg<D, FP8>::KS];
  f32x4 o[Cfg<D, FP8>::MT][NT];
  float m[NT];   // reference max per row (log2 units); p <= 2^kRescale
  float l[NT];   // this lane's share of the row sum
  int prow[NT];  // absolute position of the lane's row (row = 16 nt + lane % 16)
};

// The reference max only moves when a chunk's max exceeds it by more than
// this many log2 units; until then probabilities stay below 2^8, and the
// accumulators are rescaled rarely. The result is the same up to rounding:
// O, l and m always refer to one common reference.
constexpr float kRescale = 8.0f;

// One 32-token chunk: QK, the next chunk's loads, mask, online softmax, PV.
template <int D, bool FP8, int NT>
__device__ __forceinline__ void process_chunk(WaveState<D, FP8, NT>& S, ChunkRegs<D, FP8>& R,
                                              unsigned char* vt, const KernelArgs& A,
                                              const int32_t* bt, int g, int tok0, int next_tok0,
                                              int tv0, int tv1, int L, int q, int W, int lane) {
  using C = Cfg<D, FP8>;
  const int n = lane & 15, c = lane >> 4;
  const float scale_log2 = A.scale_log2;

  // ---- S^T = K Q^T: tokens of each page on M, packed rows on N.
  f32x4 sc[2][NT];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    bf16x8 kop[C::KS];
#pragma unroll
    for (int u = 0; u < C::KLD; ++u) {
      if constexpr (FP8) {
        kop[2 * u] = fp8x8_to_bf16(R.k[bb][u][0], R.k[bb][u][1]);
        kop[2 * u + 1] = fp8x8_to_bf16(R.k[bb][u][2], R.k[bb][u][3]);
      } else {
        kop[u] = __builtin_bit_cast(bf16x8, R.k[bb][u]);
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < C::KS; ++s) acc = mfma_bf16(kop[s], S.q[nt][s], acc);
      sc[bb][nt] = acc;
    }
  }
  if constexpr (FP8) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb)
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) sc[bb][nt] *= R.ks[bb];
  }
  // K registers are free: start the next chunk's K loads.
  const bool has_next = next_tok0 >= 0;
  PageIds nxt{0, 0};
  if (has_next) {
    nxt = page_ids(bt, next_tok0, tv1);
    load_k<D, FP8>(R, A, nxt, g, lane);
  }

  // Chunks wholly inside every row's visible range skip the mask.
  const bool fast = (tok0 >= tv0) && (tok0 + kChunk <= tv1) && (tok0 + kChunk - 1 <= L - q) &&
                    (W == 0 || tok0 > L - 1 - W);

  // ---- V: registers -> swizzled LDS tile (invalid tokens zeroed).
  f32x4 vs[2];
  if constexpr (FP8) {
    vs[0] = R.vs[0];
    vs[1] = R.vs[1];
  }
#pragma unroll
  for (int u = 0; u < C::VLD; ++u) {
    const int o = u * 1024 + lane * 16;
    const int bb = o / C::BLKB;
    const int ob = o % C::BLKB;
    const int t = 16 * bb + ob / C::ROWB;  // token within the chunk
    const int ch = (ob % C::ROWB) >> 4;    // 16-byte chunk within the token row
    const int j = tok0 + t;
    u32x4 val = R.v[u];
    if (!fast && !((j >= tv0) && (j < tv1))) val = u32x4{0, 0, 0, 0};
    *reinterpret_cast<u32x4*>(vt + vtile_chunk<D, FP8>(t, ch)) = val;
  }
  // V registers are free: start the next chunk's V loads.
  if (has_next) load_v<D, FP8>(R, A, nxt, g, lane);

  if (!fast) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = tok0 + 16 * bb + 4 * c + i;
        const bool tok_ok = (j >= tv0) && (j < tv1);
        if constexpr (FP8) vs[bb][i] = tok_ok ? vs[bb][i] : 0.f;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          const int p = S.prow[nt];
          const bool vis = tok_ok && (j <= p) && (W == 0 || j > p - W);
          sc[bb][nt][i] = vis ? sc[bb][nt][i] : -INFINITY;
        }
      }
    }
  }

  // ---- Online softmax in the exp2 domain (x = s * sigma * log2 e).
  float mx[NT];
  bool grow = false;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float v = fmaxf(fmaxf(fmaxf(sc[0][nt][0], sc[0][nt][1]), fmaxf(sc[0][nt][2], sc[0][nt][3])),
                    fmaxf(fmaxf(sc[1][nt][0], sc[1][nt][1]), fmaxf(sc[1][nt][2], sc[1][nt][3])));
    mx[nt] = xlane_max4(v) * scale_log2;
    grow |= mx[nt] > S.m[nt] + kRescale;
  }
  if (__any(grow)) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float mnew = fmaxf(S.m[nt], mx[nt]);
      const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(S.m[nt] - mnew);
      S.m[nt] = mnew;
      S.l[nt] *= alpha;
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt) S.o[mt][nt] *= alpha;
    }
  }
  // P enters the PV product as two bf16 terms, hi = bf16(p) and
  // lo = bf16(p - hi), so its rounding error (about 2^-17 relative) stays far
  // below the output's own bf16 rounding even when one key dominates a row.
  bf16x8 pop_hi[NT], pop_lo[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float msafe = (S.m[nt] == -INFINITY) ? 0.f : S.m[nt];
    float ps = 0.f;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = fast_exp2(__builtin_fmaf(sc[bb][nt][i], scale_log2, -msafe));
        ps += p;
        const float pw = FP8 ? p * vs[bb][i] : p;
        const __bf16 hi = (__bf16)pw;
        pop_hi[nt][4 * bb + i] = hi;
        pop_lo[nt][4 * bb + i] = (__bf16)(pw - (float)hi);
      }
    }
    S.l[nt] += ps;
  }

  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  // ---- O^T[d][row] += V^T[d][token] P^T[token][row]. The contraction index
  // (lane group c, element e) is token 16 (e / 4) + 4 c + e % 4 for both
  // operands: that is where the S^T accumulator left P.
  const int i16 = lane & 15;
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) {
    bf16x8 vop;
    if constexpr (FP8) {
      const int r = i16 >> 1, k = i16 & 1;
      const int t = 16 * (r >> 2) + 4 * c + (r & 3);
      const i32x2 codes = lds_tr8(vt, vtile_chunk<D, FP8>(t, mt) + 8 * k);
      vop = fp8x8_to_bf16((uint32_t)codes[0], (uint32_t)codes[1]);
    } else {
      const int r = i16 >> 2, k = i16 & 3;
      const int t0 = 4 * c + r;
      const int ch = 2 * mt + (k >> 1);
      const s16x4 lo = lds_tr16(vt, vtile_chunk<D, FP8>(t0, ch) + 8 * (k & 1));
      const s16x4 hi = lds_tr16(vt, vtile_chunk<D, FP8>(t0 + 16, ch) + 8 * (k & 1));
      vop = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      S.o[mt][nt] = mfma_bf16(vop, pop_hi[nt], S.o[mt][nt]);
      S.o[mt][nt] = mfma_bf16(vop, pop_lo[nt], S.o[mt][nt]);
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  (void)n;
}

template <int D, bool FP8, int NT>
__device__ __forceinline__ void run_item(const KernelArgs& A, const WorkItem& it,
                                         const SeqInfo& si, Smem& sm) {
  using C = Cfg<D, FP8>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int n = lane & 15, c = lane >> 4;
  const int b = it.seq, g = it.kv_head;
  const int G = A.group, Hq = A.num_q_heads;
  const int L = si.ctx_len, q = si.q_len, W = si.window;
  const int rows = q * G;
  const int tv0 = it.key_begin, tv1 = it.key_end;

  WaveState<D, FP8, NT> S;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = 16 * nt + n;
    const bool live = row < rows;
    const int rr = live ? row : rows - 1;  // padding rows mirror the last real row
    const int i = rr / G, hh = rr % G;
    S.prow[nt] = L - q + i;
    S.m[nt] = -INFINITY;
    S.l[nt] = 0.f;
    const uint16_t* qp = A.q + ((int64_t)(si.q_off + i) * Hq + g * G + hh) * D;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      u32x4 v = {0, 0, 0, 0};
      if (live) v = *reinterpret_cast<const u32x4*>(qp + qk_dmap<D, FP8>(s, c));
      S.q[nt][s] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) S.o[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  unsigned char* vt = reinterpret_cast<unsigned char*>(&sm.buf[0][0][0]) +
                      w * (kChunk * D * (FP8 ? 1 : 2));
  const int32_t* bt = A.block_table + (int64_t)b * A.max_blocks;
  const int tokbase = (tv0 >> 4) << 4;
  const int nch = (tv1 - tokbase + kChunk - 1) / kChunk;

  // One chunk of look-ahead: the next chunk's K is requested as soon as the
  // current K has been consumed by the MFMAs, its V once the current V sits
  // in LDS.
  ChunkRegs<D, FP8> R;
  if (w < nch) {
    const PageIds pid = page_ids(bt, tokbase + w * kChunk, tv1);
    load_k<D, FP8>(R, A, pid, g, lane);
    load_v<D, FP8>(R, A, pid, g, lane);
  }
  for (int ci = w; ci < nch; ci += kWaves) {
    const int next = ci + kWaves < nch ? tokbase + (ci + kWaves) * kChunk : -1;
    process_chunk<D, FP8, NT>(S, R, vt, A, bt, g, tokbase + ci * kChunk, next, tv0, tv1, L, q, W,
                              lane);
  }

  // ---- Merge the four waves' states.
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) S.l[nt] = xlane_sum4(S.l[nt]);
  __syncthreads();  // every wave is done with its V tile (aliases buf)
  if (c == 0) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) sm.ml[w][16 * nt + n] = make_float2(S.m[nt], S.l[nt]);
  }
  __syncthreads();
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int row = 16 * nt + n;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, sm.ml[v][row].x);
    const float f = (S.m[nt] == -INFINITY) ? 0.f : fast_exp2(S.m[nt] - M);
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
      *reinterpret_cast<f32x4*>(&sm.buf[w][row][16 * mt + 4 * c]) = S.o[mt][nt] * f;
  }
  __syncthreads();

  // ---- Epilogue: all 256 threads, 4 consecutive d per thread.
  constexpr int D4 = D / 4;
  for (int e = tid; e < rows * D4; e += kThreads) {
    const int row = e / D4;
    const int d = (e % D4) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) M = fmaxf(M, sm.ml[v][row].x);
    float Ls = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float2 ml = sm.ml[v][row];
      Ls += (ml.x == -INFINITY) ? 0.f : ml.y * fast_exp2(ml.x - M);
    }
    f32x4 acc = *reinterpret_cast<const f32x4*>(&sm.buf[0][row][d]);
#pragma unroll
    for (int v = 1; v < kWaves; ++v) acc += *reinterpret_cast<const f32x4*>(&sm.buf[v][row][d]);
    const int i = row / G, hh = row % G;
    const int h = g * G + hh;
    if (it.slot < 0) {
      float zs = -INFINITY;
      if (A.sinks_mode == 1) zs = A.sinks[h] * kLog2e;
      else if (A.sinks_mode == 2) zs = A.sinks[(int64_t)b * Hq + h] * kLog2e;
      const float Mx = fmaxf(M, zs);
      const float a = fast_exp2(M - Mx);
      const float den = Ls * a + ((zs == -INFINITY) ? 0.f : fast_exp2(zs - Mx));
      acc *= a / den;
      const int64_t oi = ((int64_t)(si.q_off + i) * Hq + h) * D + d;
      if (A.out_fp32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(A.out) + oi) = acc;
      } else {
        bf16x2 p0 = {(__bf16)acc[0], (__bf16)acc[1]};
        bf16x2 p1 = {(__bf16)acc[2], (__bf16)acc[3]};
        uint2 pk = make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
        *reinterpret_cast<uint2*>(static_cast<__bf16*>(A.out) + oi) = pk;
      }
    } else {
      const int64_t pr = (int64_t)it.slot * A.rows_stride + row;
      *reinterpret_cast<f32x4*>(A.part_o + pr * D + d) = acc;
      if (d == 0) *reinterpret_cast<float2*>(A.part_ml + pr * 2) = make_float2(M, Ls);
    }
  }
}

template <int D, bool FP8>
__global__ __launch_bounds__(kThreads, 1) void pa_partition_kernel(KernelArgs A) {
  __shared__ Smem sm;
  const WorkItem it = A.items[blockIdx.x];
  const SeqInfo si = A.seqs[it.seq];
  const int rows = si.q_len * A.group;
  switch ((rows + 15) >> 4) {
    case 1: run_item<D, FP8, 1>(A, it, si, sm); break;
    case 2: run_item<D, FP8, 2>(A, it, si, sm); break;
    case 3: run_item<D, FP8, 3>(A, it, si, sm); break;
    default: run_item<D, FP8, 4>(A, it, si, sm); break;
  }
}

// Log-sum-exp merge of the partials of one (sequence, KV head):
//   M = max(max_k m_k, z), Z = sum_k l_k 2^(m_k - M) + 2^(z - M),
//   out = sum_k 2^(m_k - M) O_k / Z       (all in log2 units).
// Grid: one workgroup per (reduce item, group of rows); D/4 threads per row.
template <int D>
__global__ __launch_bounds__(256) void pa_reduce_kernel(KernelArgs A) {
  constexpr int TPR = D / 4;
  constexpr int RPW = 256 / TPR;
  constexpr int GROUPS = (kMaxRows + RPW - 1) / RPW;
  const ReduceItem ri = A.red[blockIdx.x / GROUPS];
  const int rg = blockIdx.x % GROUPS;
  const SeqInfo si = A.seqs[ri.seq];
  const int G = A.group, Hq = A.num_q_heads;
  const int rows = si.q_len * G;
  const int row = rg * RPW + threadIdx.x / TPR;
  if (row >= rows) return;
  const int d = (threadIdx.x % TPR) * 4;
  const int i = row / G, hh = row % G;
  const int h = ri.kv_head * G + hh;
  float M = -INFINITY;
  for (int k = 0; k < ri.n_parts; ++k) {
    const int64_t pr = (int64_t)(ri.slot_base + k) * A.rows_stride + row;
    M = fmaxf(M, A.part_ml[pr * 2]);
  }
  float zs = -INFINITY;
  if (A.sinks_mode == 1) zs = A.sinks[h] * kLog2e;
  else if (A.sinks_mode == 2) zs = A.sinks[(int64_t)ri.seq * Hq + h] * kLog2e;
  const float Mx = fmaxf(M, zs);
  float Z = (zs == -INFINITY) ? 0.f : fast_exp2(zs - Mx);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < ri.n_parts; ++k) {
    const int64_t pr = (int64_t)(ri.slot_base + k) * A.rows_stride + row;
    const float2 ml = *reinterpret_cast<const float2*>(A.part_ml + pr * 2);
    if (ml.x == -INFINITY) continue;  // a partition no key of which this row sees
    const float wk = fast_exp2(ml.x - Mx);
    Z += ml.y * wk;
    acc += *reinterpret_cast<const f32x4*>(A.part_o + pr * D + d) * wk;
  }
  acc *= 1.0f / Z;
  const int64_t oi = ((int64_t)(si.q_off + i) * Hq + h) * D + d;
  if (A.out_fp32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(A.out) + oi) = acc;
  } else {
    bf16x2 p0 = {(__bf16)acc[0], (__bf16)acc[1]};
    bf16x2 p1 = {(__bf16)acc[2], (__bf16)acc[3]};
    uint2 pk = make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
    *reinterpret_cast<uint2*>(static_cast<__bf16*>(A.out) + oi) = pk;
  }
}

hipError_t launch_partition(const KernelArgs& a, int n_items, int head_dim, bool fp8,
                            hipStream_t stream) {
  if (n_items <= 0) return hipSuccess;
  dim3 grid(n_items), block(kThreads);
  if (head_dim == 128) {
    if (fp8) hipLaunchKernelGGL((pa_partition_kernel<128, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((pa_partition_kernel<128, false>), grid, block, 0, stream, a);
  } else {
    if (fp8) hipLaunchKernelGGL((pa_partition_kernel<64, true>), grid, block, 0, stream, a);
    else hipLaunchKernelGGL((pa_partition_kernel<64, false>), grid, block, 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_reduce(const KernelArgs& a, int n_red, int head_dim, hipStream_t stream) {
  if (n_red <= 0) return hipSuccess;
  dim3 block(256);
  if (head_dim == 128) {
    constexpr int groups = kMaxRows / (256 / 32);
    hipLaunchKernelGGL((pa_reduce_kernel<128>), dim3(n_red * groups), block, 0, stream, a);
  } else {
    constexpr int groups = kMaxRows / (256 / 16);
    hipLaunchKernelGGL((pa_reduce_kernel<64>), dim3(n_red * groups), block, 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pav
