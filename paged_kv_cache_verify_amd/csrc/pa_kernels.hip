// gfx950 kernels for paged verify attention.
//
// Partition kernel: one workgroup of ten waves per work item (and per CU)
// = the keys [key_begin, key_end) of one (sequence, KV head), all q x G
// packed rows of that KV head. The waves form two token groups of five:
// group 0 takes the item's even 32-token chunks (two 16-token pages), group
// 1 the odd ones, each through an LDS ring of its own that the group's
// loader wave fills by direct global-to-LDS loads (K in MFMA A-operand
// order, V into an XOR-swizzled token-major tile); one workgroup barrier per
// step recycles a stage in both rings. Within a group, compute wave r owns
// row tile r (16 rows) and, per chunk,
//   1. computes S^T = K Q^T with v_mfma_f32_16x16x32_bf16, tokens on the M
//      index (FP8 codes are converted exactly to bf16 by the group's compute
//      waves one step ahead, and the per-token K scale multiplies the
//      scores),
//   2. masks (causal within the query, window, key range) by selecting -inf,
//   3. runs an online softmax in the exp2 domain whose reference max only
//      moves when a chunk beats it by 2^8 (rare rescaling),
//   4. accumulates O^T += V^T P^T: V^T comes from ds_read_b64_tr_b16 on
//      the (bf16 or converted) tile, P^T straight from the S^T accumulator
//      registers as a bf16 hi+lo pair (the per-token V scale folded in).
// At the end the two groups' states of each tile merge through LDS and the
// workgroup writes the output, or this item's partial, which the reduce
// kernel merges with the other partials of a split (sequence, KV head) by
// log-sum-exp.
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

// Reductions over the four lanes l, l^16, l^32, l^48 (the MFMA's four lane
// groups holding one row). v_permlane16_swap / v_permlane32_swap exchange
// rows of two registers; applied to two copies of v they leave the pair
// (v[l], v[l^16]) resp. (v[l], v[l^32]) in the two registers. Issued from asm
// on two distinct copies: the compiler folds the builtin's two results into
// one when both inputs are the same value. s_nop 1 covers the VALU-write to
// permlane-read hazard.
__device__ __forceinline__ void swap16(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32(float& a, float& b) {
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}

__device__ __forceinline__ float xlane_max4(float v) {
  float a = v, b = v;
  swap16(a, b);
  float c = fmaxf(a, b), d = c;
  swap32(c, d);
  return fmaxf(c, d);
}

__device__ __forceinline__ float xlane_sum4(float v) {
  float a = v, b = v;
  swap16(a, b);
  float c = a + b, d = c;
  swap32(c, d);
  return c + d;
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

// Transposing LDS reads (issued from asm below):
// ds_read_b64_tr_b16: within each 16-lane group, lane 4r + k names the 8
// bytes at (row r, columns 4k..4k+3) of a 4 x 16 tile of 16-bit values, and
// lane i receives column i (rows 0..3).
// ds_read_b64_tr_b8: lane 2r + k names the 8 bytes at (row r, columns
// 8k..8k+7) of an 8 x 16 tile of bytes; lane i receives column i (rows 0..7).

// ---------------------------------------------------------------------------
// The LDS rings: one per token group.
// ---------------------------------------------------------------------------

constexpr int kGroups = 2;                 // token groups per workgroup
constexpr int kTileWaves = 4;              // compute waves per group (one per row tile)
constexpr int kGroupWaves = kTileWaves + 1;  // ... and the group's loader
constexpr int kWaves = kGroups * kGroupWaves;
constexpr int kThreads = 64 * kWaves;
// LDS per group (the workgroup holds most of a CU's 160 KiB): 64 KiB for
// bf16; 76 KiB for FP8, whose ring also holds two bf16 copies of chunks.
template <bool FP8>
constexpr int kGroupRingBytes = (FP8 ? 76 : 64) * 1024;

template <int D, bool FP8>
struct Ring {
  using C = Cfg<D, FP8>;
  using CB = Cfg<D, false>;                      // bf16 layout the compute reads
  static constexpr int KB = 2 * C::KLD * 1024;   // K of two pages, operand order
  static constexpr int VB = C::VLD * 1024;       // V tile of two pages
  static constexpr int SB = FP8 ? 256 : 0;       // K and V scales of two pages
  static constexpr int STAGE = KB + VB + SB;
  // FP8: chunks converted to bf16 once per group (K in operand order, then
  // the V tile in the bf16 swizzle), two copies: the one computed on and the
  // one being converted for the next step.
  static constexpr int KB16 = 2 * CB::KLD * 1024;
  static constexpr int COPY = KB16 + CB::VLD * 1024;
  static constexpr int BUF = FP8 ? 2 * COPY : 0;
  static constexpr int R0 = (kGroupRingBytes<FP8> - BUF) / STAGE;
  static constexpr int R = R0 < 8 ? R0 : 8;      // stages per group
  // Loads per chunk, all issued by the group's loader wave: 1 KiB ones of
  // K and V, and (FP8) one of the scales.
  static constexpr int T = 2 * C::KLD + C::VLD + (FP8 ? 1 : 0);
  static_assert(R >= (FP8 ? 4 : 3), "the ring needs enough stages to keep loads in flight");
  // Loads the loader may still have in flight when its group starts on a
  // step: bf16 needs the step's chunk, so the next R - 2 chunks may be
  // pending; FP8 converts one chunk ahead, so it needs the next chunk too
  // and R - 3 may be pending. WAIT0: before the first FP8 conversion.
  static constexpr int WAIT = (R - (FP8 ? 3 : 2)) * T;
  static constexpr int WAIT0 = (R - 2) * T;
  static_assert(WAIT0 <= 63, "vmcnt holds at most 63");
  static constexpr int RING = R * STAGE + BUF;   // bytes per group
};

template <int D, bool FP8>
struct Smem {
  unsigned char ring[kGroups][Ring<D, FP8>::RING];
  int32_t pages[2 * kMaxItemChunks];  // page ids of each chunk's two pages
};

#define PAV_LDS_VOID __attribute__((address_space(3))) void

// Direct global-to-LDS loads: every lane moves `size` bytes from its own
// address to lds_dst + size * lane (lds_dst is wave-uniform). The KV is read
// once per call, so the loads carry the nontemporal bit (cache policy 2):
// on MI355X that raises the streaming rate of random 4 KiB pages by about a
// tenth over the default policy.
constexpr int kNonTemporal = 2;
__device__ __forceinline__ void dma16(const void* src, unsigned char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (PAV_LDS_VOID*)lds_dst, 16, 0, kNonTemporal);
}
__device__ __forceinline__ void dma4(const void* src, unsigned char* lds_dst) {
  __builtin_amdgcn_global_load_lds(src, (PAV_LDS_VOID*)lds_dst, 4, 0, kNonTemporal);
}

// Wait until at most N of this wave's vector-memory operations are pending.
// The compiler does not order direct-to-LDS loads before the LDS reads of
// their data, so the ring's waits are explicit; the memory clobber keeps
// later LDS reads below the wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier for the ring: this wave's LDS reads and writes are done
// (lgkmcnt 0) before it arrives. Unlike __syncthreads() it does not drain
// vector-memory operations, so the loads of later stages stay in flight;
// each wave has already waited for its own loads of the stage it needs.
__device__ __forceinline__ void ring_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Page ids of chunk k's two pages, read from asm: the compiler would
// otherwise drain the ring's in-flight loads before an LDS read it cannot
// tell apart from their destinations.
__device__ __forceinline__ void chunk_pages(uint32_t pages_addr, int k, int& pa, int& pb) {
  i32x2 pp;
  asm volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)"
               : "=v"(pp)
               : "v"(pages_addr + 8 * k)
               : "memory");
  pa = __builtin_amdgcn_readfirstlane(pp[0]);
  pb = __builtin_amdgcn_readfirstlane(pp[1]);
}

// All loads of one chunk into stage `sb` of the group's ring, issued by the
// group's loader wave: K of the chunk's two pages (KLD loads of 1 KiB per
// page, in MFMA operand order: lane l of load u sits at byte 1024 u + 16 l
// and is what lane l of the MFMA reads back), V of the two pages into the
// swizzled tile (lane l fetches whichever source chunk belongs at its tile
// position), and the FP8 scales. The lane's offsets are derived on every
// call (the empty asm hides that they never change), rather than held in
// registers across the loop.
template <int D, bool FP8>
__device__ __forceinline__ void issue_chunk(const KernelArgs& A, unsigned char* sb, int pa,
                                            int pb, int g, int lane) {
  using C = Cfg<D, FP8>;
  using RG = Ring<D, FP8>;
  int ln = lane;
  asm volatile("" : "+v"(ln));
  const uint32_t koff = (ln & 15) * C::ROWB + 16 * (ln >> 4);
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int page = half ? pb : pa;
    const char* src = static_cast<const char*>(A.k_pool) +
                      ((int64_t)page * A.num_kv_heads + g) * C::BLKB;
    unsigned char* dst = sb + half * C::KLD * 1024;
#pragma unroll
    for (int u = 0; u < C::KLD; ++u) dma16(src + (koff + 64 * u), dst + u * 1024);
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int page = half ? pb : pa;
    const char* src = static_cast<const char*>(A.v_pool) +
                      ((int64_t)page * A.num_kv_heads + g) * C::BLKB;
    unsigned char* dst = sb + RG::KB + half * (C::BLKB);
#pragma unroll
    for (int u = 0; u < C::VLD / 2; ++u) {
      const int pos = u * 1024 + ln * 16;  // byte position in this page's half of the tile
      const int tp = pos / C::ROWB;        // token within the page
      const int t = 16 * half + tp;        // token within the chunk (sets the swizzle)
      const int ch = ((pos % C::ROWB) >> 4) ^ vswz<D, FP8>(t);  // its source chunk
      dma16(src + (uint32_t)(tp * C::ROWB + ch * 16), dst + u * 1024);
    }
  }
  if constexpr (FP8) {  // scales: [K page A][K page B][V page A][V page B] x 16 tokens
    const int which = ln >> 4, tok = ln & 15;
    const int pgs = (which & 1) ? pb : pa;
    const float* src2 = ((which < 2) ? A.k_scales : A.v_scales) +
                        ((int64_t)pgs * A.num_kv_heads + g) * kBlock + tok;
    dma4(src2, sb + RG::KB + RG::VB);
  }
}

// ---------------------------------------------------------------------------
// V^T operands for one chunk: all transposing LDS reads of the stage in one
// asm block that ends with lgkmcnt(0). (The compiler treats the transposing
// read intrinsics as possibly aliasing any in-flight direct-to-LDS load and
// would drain every outstanding load before them; the ring's own waits have
// already made the stage's data visible.) lane_off[mt] is the lane's byte
// address of the first read of output tile mt; the bf16 reads of tokens
// 16..31 sit 16 token rows further.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

#define PAV_TR16_PAIR(i, off) "ds_read_b64_tr_b16 %" #i ", %[a" #off "]\n\t"

__device__ __forceinline__ void vt_reads_bf16_d128(s16x4 (&r)[16], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:4096\n\t"
      "ds_read_b64_tr_b16 %2, %17\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:4096\n\t"
      "ds_read_b64_tr_b16 %4, %18\n\t"
      "ds_read_b64_tr_b16 %5, %18 offset:4096\n\t"
      "ds_read_b64_tr_b16 %6, %19\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:4096\n\t"
      "ds_read_b64_tr_b16 %8, %20\n\t"
      "ds_read_b64_tr_b16 %9, %20 offset:4096\n\t"
      "ds_read_b64_tr_b16 %10, %21\n\t"
      "ds_read_b64_tr_b16 %11, %21 offset:4096\n\t"
      "ds_read_b64_tr_b16 %12, %22\n\t"
      "ds_read_b64_tr_b16 %13, %22 offset:4096\n\t"
      "ds_read_b64_tr_b16 %14, %23\n\t"
      "ds_read_b64_tr_b16 %15, %23 offset:4096\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
        "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

__device__ __forceinline__ void vt_reads_bf16_d64(s16x4 (&r)[8], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b64_tr_b16 %0, %8\n\t"
      "ds_read_b64_tr_b16 %1, %8 offset:2048\n\t"
      "ds_read_b64_tr_b16 %2, %9\n\t"
      "ds_read_b64_tr_b16 %3, %9 offset:2048\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %10 offset:2048\n\t"
      "ds_read_b64_tr_b16 %6, %11\n\t"
      "ds_read_b64_tr_b16 %7, %11 offset:2048\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}

template <int D, bool FP8>
struct WaveState {
  bf16x8 q[Cfg<D, FP8>::KS];
  f32x4 o[Cfg<D, FP8>::MT];
  float m;   // reference max of the lane's row (log2 units); p <= 2^kRescale
  float l;   // this lane's share of the row sum
  int prow;  // absolute position of the lane's row
};

// The reference max only moves when a chunk's max exceeds it by more than
// this many log2 units; until then probabilities stay below 2^8 and the
// accumulators are not rescaled. O, l and m always share one reference.
constexpr float kRescale = 8.0f;

// One chunk for the wave's 16-row tile. kv holds the chunk in the bf16
// layout (K of the two pages in operand order, then the V tile); for FP8
// it is the group's converted copy and scl the stage's K and V scales.
template <int D, bool FP8>
__device__ __forceinline__ void compute_chunk(WaveState<D, FP8>& S, const unsigned char* kv,
                                              const unsigned char* scl, int tok0, int tv0,
                                              int tv1, int L, int q, int W, float scale_log2,
                                              int lane) {
  using C = Cfg<D, FP8>;
  using CB = Cfg<D, false>;
  using RG = Ring<D, FP8>;
  const int c = lane >> 4;
  const int i16 = lane & 15;

  // ---- LDS reads of the chunk: K operands, then every V^T operand (one
  // asm block whose lgkmcnt(0) also covers the K reads), so both latencies
  // overlap.
  u32x4 kr[2][CB::KLD];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb)
#pragma unroll
    for (int u = 0; u < CB::KLD; ++u)
      kr[bb][u] = *reinterpret_cast<const u32x4*>(kv + (bb * CB::KLD + u) * 1024 + lane * 16);
  f32x4 ksc[2], vs[2];
  if constexpr (FP8) {
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      ksc[bb] = *reinterpret_cast<const f32x4*>(scl + (bb * 16 + 4 * c) * 4);
      vs[bb] = *reinterpret_cast<const f32x4*>(scl + 128 + (bb * 16 + 4 * c) * 4);
    }
  }
  const uint32_t vt = lds_addr(kv + RG::KB16);
  uint32_t va[C::MT];
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) {
    const int r = i16 >> 2, k = i16 & 3;
    va[mt] = vt + vtile_chunk<D, false>(4 * c + r, 2 * mt + (k >> 1)) + 8 * (k & 1);
  }
  bf16x8 vops[C::MT];
  {
    s16x4 rd[2 * C::MT];
    if constexpr (D == 128) vt_reads_bf16_d128(rd, va);
    else vt_reads_bf16_d64(rd, va);
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
      vops[mt] = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(rd[2 * mt], rd[2 * mt + 1], 0, 1, 2, 3, 4, 5, 6, 7));
  }

  // ---- S^T = K Q^T: the two pages' tokens on M, the tile's rows on N.
  f32x4 sc[2];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < CB::KLD; ++u) acc = mfma_bf16(__builtin_bit_cast(bf16x8, kr[bb][u]), S.q[u], acc);
    sc[bb] = FP8 ? acc * ksc[bb] : acc;
  }

  // ---- Masks, only for chunks not wholly inside every row's visible range:
  // scores of invisible keys become -inf; V^T entries (and FP8 V scales) of
  // tokens outside the item's valid range become 0, since their pool slots
  // may hold anything, NaN included.
  const bool fast = (tok0 >= tv0) && (tok0 + kChunk <= tv1) && (tok0 + kChunk - 1 <= L - q) &&
                    (W == 0 || tok0 > L - 1 - W);
  if (!fast) {
    // A real branch: the compiler would otherwise turn the selects into
    // straight-line code that every chunk pays for.
    asm volatile("");
    const int p = S.prow;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = tok0 + 16 * bb + 4 * c + i;
        const bool ok = (j >= tv0) && (j < tv1);
        const bool vis = ok && (j <= p) && (W == 0 || j > p - W);
        sc[bb][i] = vis ? sc[bb][i] : -INFINITY;
        if constexpr (FP8) vs[bb][i] = ok ? vs[bb][i] : 0.f;
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
          vops[mt][4 * bb + i] = ok ? vops[mt][4 * bb + i] : (__bf16)0.f;
      }
    }
  }

  // ---- Online softmax in the exp2 domain (x = s * sigma * log2 e).
  float mx = fmaxf(fmaxf(fmaxf(sc[0][0], sc[0][1]), fmaxf(sc[0][2], sc[0][3])),
                   fmaxf(fmaxf(sc[1][0], sc[1][1]), fmaxf(sc[1][2], sc[1][3])));
  mx = xlane_max4(mx) * scale_log2;
  if (__any(mx > S.m + kRescale)) {
    asm volatile("");  // a real branch (rescaling is rare)
    const float mnew = fmaxf(S.m, mx);
    const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(S.m - mnew);
    S.m = mnew;
    S.l *= alpha;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) S.o[mt] *= alpha;
  }
  // P enters the PV product as two bf16 terms, hi = bf16(p) and
  // lo = bf16(p - hi), so its rounding error (about 2^-17 relative) stays far
  // below the output's own bf16 rounding even when one key dominates a row.
  const float msafe = (S.m == -INFINITY) ? 0.f : S.m;
  bf16x8 p_hi, p_lo;
  float ps = 0.f;
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = fast_exp2(__builtin_fmaf(sc[bb][i], scale_log2, -msafe));
      ps += p;
      const float pw = FP8 ? p * vs[bb][i] : p;
      const __bf16 hi = (__bf16)pw;
      p_hi[4 * bb + i] = hi;
      p_lo[4 * bb + i] = (__bf16)(pw - (float)hi);
    }
  }
  S.l += ps;

  // ---- O^T[d][row] += V^T[d][token] P^T[token][row]. The contraction index
  // (lane group c, element e) is token 16 (e / 4) + 4 c + e % 4 for both
  // operands: that is where the S^T accumulator left P.
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) {
    S.o[mt] = mfma_bf16(vops[mt], p_hi, S.o[mt]);
    S.o[mt] = mfma_bf16(vops[mt], p_lo, S.o[mt]);
  }
}

// FP8: the group's four waves convert the chunk in stage `st` to bf16 in
// the group's buffer `buf`, exactly, each a quarter of it. K: wave r takes
// 1 KiB block r of the stage (16 codes per lane = contraction steps 2u and
// 2u + 1 of one token, which land in bf16 blocks 2u and 2u + 1). V: lane l
// of wave r takes 16-byte chunk 64 r + l of the FP8 tile (16 columns of one
// token), which lands as two bf16 chunks in the bf16 swizzle. LDS reads and
// writes are issued from asm, so that the compiler does not hold them back
// for the ring's in-flight loads.
template <int D>
__device__ __forceinline__ void convert_chunk(const unsigned char* st, unsigned char* buf, int r,
                                              int lane) {
  using C8 = Cfg<D, true>;
  using CB = Cfg<D, false>;
  using RG = Ring<D, true>;
  constexpr int KBLK = 2 * C8::KLD;   // FP8 K blocks per chunk (4 for D 128, 2 for D 64)
  constexpr int VCH = kChunk * D / 16; // FP8 V chunks of 16 bytes (256 / 128)
  u32x4 kw = {0, 0, 0, 0}, vw = {0, 0, 0, 0};
  const bool kdo = r < KBLK;
  const int x = r * 64 + lane;
  const bool vdo = x < VCH;
  const int t = x / (D / 16), j = x % (D / 16);
  const uint32_t ksrc = lds_addr(st + r * 1024 + lane * 16);
  const uint32_t vsrc = lds_addr(st + RG::KB + t * C8::ROWB + ((j ^ vswz<D, true>(t)) << 4));
  if (kdo) asm volatile("ds_read_b128 %0, %1" : "=v"(kw) : "v"(ksrc) : "memory");
  if (vdo) asm volatile("ds_read_b128 %0, %1" : "=v"(vw) : "v"(vsrc) : "memory");
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(kw), "+v"(vw) :: "memory");
  if (kdo) {
    const int bb = r / C8::KLD, u = r % C8::KLD;
    const bf16x8 lo = fp8x8_to_bf16(kw[0], kw[1]), hi = fp8x8_to_bf16(kw[2], kw[3]);
    const uint32_t d0 = lds_addr(buf + (bb * CB::KLD + 2 * u) * 1024 + lane * 16);
    asm volatile("ds_write_b128 %0, %1\n\tds_write_b128 %0, %2 offset:1024"
                 :: "v"(d0), "v"(lo), "v"(hi) : "memory");
  }
  if (vdo) {
    const bf16x8 lo = fp8x8_to_bf16(vw[0], vw[1]), hi = fp8x8_to_bf16(vw[2], vw[3]);
    unsigned char* vb = buf + RG::KB16;
    const uint32_t d0 = lds_addr(vb + vtile_chunk<D, false>(t, 2 * j));
    const uint32_t d1 = lds_addr(vb + vtile_chunk<D, false>(t, 2 * j + 1));
    asm volatile("ds_write_b128 %0, %2\n\tds_write_b128 %1, %3"
                 :: "v"(d0), "v"(d1), "v"(lo), "v"(hi) : "memory");
  }
}

template <int D, bool FP8>
__device__ __forceinline__ void store_out(const KernelArgs& A, int64_t idx, f32x4 v) {
  if (A.out_fp32) {
    *reinterpret_cast<f32x4*>(static_cast<float*>(A.out) + idx) = v;
  } else {
    bf16x2 p0 = {(__bf16)v[0], (__bf16)v[1]};
    bf16x2 p1 = {(__bf16)v[2], (__bf16)v[3]};
    uint2 pk = make_uint2(__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1));
    *reinterpret_cast<uint2*>(static_cast<__bf16*>(A.out) + idx) = pk;
  }
}

__device__ __forceinline__ float sink_log2(const KernelArgs& A, int b, int h) {
  if (A.sinks_mode == 1) return A.sinks[h] * kLog2e;
  if (A.sinks_mode == 2) return A.sinks[(int64_t)b * A.num_q_heads + h] * kLog2e;
  return -INFINITY;
}

template <int D, bool FP8>
__global__ __launch_bounds__(kThreads, 1) void pa_partition_kernel(KernelArgs A) {
  using C = Cfg<D, FP8>;
  using RG = Ring<D, FP8>;
  __shared__ Smem<D, FP8> sm;
  const WorkItem it = A.items[blockIdx.x];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int gp = w / kGroupWaves, r = w % kGroupWaves;     // token group, row tile
  const bool loader = r == kTileWaves;                      // the group's loader
  const int n = lane & 15, c = lane >> 4;
  const int b = it.seq, g = it.kv_head;
  const int G = A.group, Hq = A.num_q_heads;
  const int L = it.ctx_len, q = it.q_len, W = it.window;
  const int rows = q * G;
  const int nt = (rows + 15) >> 4;  // row tiles; waves r >= nt do not compute
  const bool active = r < nt;
  const int tv0 = it.key_begin, tv1 = it.key_end;
  const int tokbase = (tv0 >> 4) << 4;
  const int nch = (tv1 - tokbase + kChunk - 1) / kChunk;  // <= kMaxItemChunks
  const int nst = (nch + kGroups - 1) / kGroups;           // steps: one chunk per group

  // Page ids of every chunk (a page past the item's end repeats the
  // chunk's first page, whose slots the masks then exclude).
  const int32_t* bt = A.block_table + (int64_t)b * A.max_blocks;
  for (int i = tid; i < 2 * nch; i += kThreads) {
    const int k = i >> 1, which = i & 1;
    const int tok0 = tokbase + k * kChunk;
    const int pg = (tok0 >> 4) + which;
    sm.pages[i] = bt[(which == 0 || tok0 + kBlock < tv1) ? pg : pg - 1];
  }

  // The wave's row tile: row = 16 r + lane % 16 (padding rows mirror the
  // last real row and carry a zero query).
  WaveState<D, FP8> S;
  {
    const int row = 16 * r + n;
    const bool live = active && row < rows;
    const int rr = live ? row : rows - 1;
    const int i = rr / G, hh = rr % G;
    S.prow = L - q + i;
    S.m = -INFINITY;
    S.l = 0.f;
    const uint16_t* qp = A.q + ((int64_t)(it.q_off + i) * Hq + g * G + hh) * D;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      u32x4 v = {0, 0, 0, 0};
      if (live) v = *reinterpret_cast<const u32x4*>(qp + qk_dmap<D, FP8>(s, c));
      S.q[s] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) S.o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // Finish the query and table loads here, with a wait the compiler sees:
  // otherwise it waits for the query inside the chunk loop, where vmcnt(0)
  // would also drain the ring's loads on every chunk.
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt unbounded
  __syncthreads();  // page ids visible to every wave
  const uint32_t pages_addr = lds_addr(sm.pages);
  unsigned char* ring = sm.ring[gp];

  // Chunk of this wave's group at step k: gp + 2 k. The loader fills the
  // first R - 1 stages; then per step: the loader waits for its loads of
  // the step's chunk, the barrier (every group's chunk has landed and every
  // wave is done with the stage about to be refilled), the loader refills
  // that stage while the compute waves work. Compute waves never issue or
  // wait for ring loads, so they never stall behind the load queue.
  if (loader) {
    for (int k = 0; k < RG::R - 1 && gp + kGroups * k < nch; ++k) {
      int pa, pb;
      chunk_pages(pages_addr, gp + kGroups * k, pa, pb);
      issue_chunk<D, FP8>(A, ring + k * RG::STAGE, pa, pb, g, lane);
    }
  }
  unsigned char* cbuf = ring + RG::R * RG::STAGE;  // FP8: bf16 copies [2][COPY]
  if constexpr (FP8) {
    // The first chunk's copy, before the loop: wait for its stage (the next
    // R - 2 stages may be pending), barrier, convert.
    if (loader) {
      if (gp + kGroups * (RG::R - 2) < nch) wait_vm<RG::WAIT0>();
      else wait_vm<0>();
    }
    ring_barrier();
    if (gp < nch) convert_chunk<D>(ring, cbuf, r, lane);
  }
  for (int k = 0; k < nst; ++k) {
    const int ck = gp + kGroups * k;
    if (loader) {
      // bf16: this step's chunk has landed; FP8: the next one too (it is
      // converted during this step).
      if (gp + kGroups * (k + RG::R - 2) < nch) wait_vm<RG::WAIT>();
      else wait_vm<0>();
    }
    ring_barrier();
    const int cn = gp + kGroups * (k + RG::R - 1);
    if (loader && cn < nch) {
      int pa, pb;
      chunk_pages(pages_addr, cn, pa, pb);
      issue_chunk<D, FP8>(A, ring + ((k + RG::R - 1) % RG::R) * RG::STAGE, pa, pb, g, lane);
    }
    const unsigned char* st = ring + (k % RG::R) * RG::STAGE;
    if constexpr (FP8) {
      // Convert the next chunk into the other copy (whose last reader, the
      // previous step's compute, finished before the barrier above), then
      // compute on this step's copy (converted during the previous step).
      if (ck + kGroups < nch)
        convert_chunk<D>(ring + ((k + 1) % RG::R) * RG::STAGE, cbuf + ((k + 1) & 1) * RG::COPY,
                         r, lane);
      if (active && ck < nch)
        compute_chunk<D, FP8>(S, cbuf + (k & 1) * RG::COPY, st + RG::KB + RG::VB,
                              tokbase + ck * kChunk, tv0, tv1, L, q, W, A.scale_log2, lane);
    } else {
      if (active && ck < nch)
        compute_chunk<D, FP8>(S, st, nullptr, tokbase + ck * kChunk, tv0, tv1, L, q, W,
                              A.scale_log2, lane);
    }
  }

  // ---- Merge the groups: group 1's waves hand (m, l, O) of their tile to
  // group 0's through LDS (the rings are free once every wave is past the
  // barrier; every wave's loads have completed, its last wait was vmcnt(0)).
  S.l = xlane_sum4(S.l);
  __syncthreads();
  f32x4* xo = reinterpret_cast<f32x4*>(&sm.ring[0][0]);       // [tile][mt][lane]
  float* xm = reinterpret_cast<float*>(&sm.ring[0][0]) + kGroupWaves * C::MT * 64 * 4;  // [tile][lane][m, l]
  if (gp == 1 && active) {
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) xo[(r * C::MT + mt) * 64 + lane] = S.o[mt];
    xm[(r * 64 + lane) * 2] = S.m;
    xm[(r * 64 + lane) * 2 + 1] = S.l;
  }
  __syncthreads();
  if (gp == 1 || !active) return;
  {
    const float m1 = xm[(r * 64 + lane) * 2], l1 = xm[(r * 64 + lane) * 2 + 1];
    const float M = fmaxf(S.m, m1);
    const float a0 = (S.m == -INFINITY) ? 0.f : fast_exp2(S.m - M);
    const float a1 = (m1 == -INFINITY) ? 0.f : fast_exp2(m1 - M);
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) S.o[mt] = S.o[mt] * a0 + xo[(r * C::MT + mt) * 64 + lane] * a1;
    S.l = S.l * a0 + l1 * a1;
    S.m = M;
  }

  // ---- Epilogue: the wave writes its rows (lane: row n, d = 16 mt + 4 c + i).
  const int row = 16 * r + n;
  if (row >= rows) return;
  const int i = row / G, hh = row % G;
  const int h = g * G + hh;
  if (it.slot < 0) {
    const float zs = sink_log2(A, b, h);
    const float Mx = fmaxf(S.m, zs);
    const float a = fast_exp2(S.m - Mx);
    const float den = S.l * a + ((zs == -INFINITY) ? 0.f : fast_exp2(zs - Mx));
    const float rs = a / den;
    const int64_t ob = ((int64_t)(it.q_off + i) * Hq + h) * D + 4 * c;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) store_out<D, FP8>(A, ob + 16 * mt, S.o[mt] * rs);
  } else {
    const int64_t pr = (int64_t)it.slot * A.rows_stride + row;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
      *reinterpret_cast<f32x4*>(A.part_o + pr * D + 16 * mt + 4 * c) = S.o[mt];
    if (c == 0) *reinterpret_cast<float2*>(A.part_ml + pr * 2) = make_float2(S.m, S.l);
  }
}

// Log-sum-exp merge of the partials of one split (sequence, KV head):
//   M = max(max_k m_k, z), Z = sum_k l_k 2^(m_k - M) + 2^(z - M),
//   out = sum_k 2^(m_k - M) O_k / Z       (all in log2 units).
// Grid: (reduce item, row, D / (4 COLS) column blocks); COLS x PARTS
// threads = COLS column lanes (4 values each) x PARTS partition lanes. Each
// thread folds its partials in one pass with a running maximum; the
// partition lanes then combine through LDS in a fixed order. Two shapes:
// few partials per pair (all columns of a row in one workgroup of 128
// threads) and many (a quarter of the columns, 32 partition lanes).
template <int D, int COLS, int PARTS>
__global__ __launch_bounds__(COLS * PARTS) void pa_reduce_kernel(KernelArgs A) {
  constexpr int DSPLIT = D / 4 / COLS;
  __shared__ float s_m[PARTS][COLS];
  __shared__ float s_z[PARTS][COLS];
  __shared__ f32x4 s_o[PARTS][COLS];
  const int bid = blockIdx.x;
  const int ds = bid % DSPLIT;
  const int row = (bid / DSPLIT) % A.rows_stride;
  const ReduceItem ri = A.red[bid / (DSPLIT * A.rows_stride)];
  const int G = A.group, Hq = A.num_q_heads;
  const int rows = ri.q_len * G;
  if (row >= rows) return;  // uniform over the workgroup
  const int dl = threadIdx.x % COLS, pl = threadIdx.x / COLS;
  const int d = (ds * COLS + dl) * 4;
  const int n = ri.n_parts;
  const float* ml = A.part_ml + ((int64_t)ri.slot_base * A.rows_stride + row) * 2;
  const float* po = A.part_o + ((int64_t)ri.slot_base * A.rows_stride + row) * D + d;
  const int64_t mstride = (int64_t)A.rows_stride * 2;
  const int64_t ostride = (int64_t)A.rows_stride * D;

  // Batches of U partials: all loads of a batch are in flight together,
  // then they are folded in order.
  constexpr int U = 4;
  float M = -INFINITY, z = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = pl; k0 < n; k0 += PARTS * U) {
    float2 v[U];
    f32x4 o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + u * PARTS;
      v[u] = make_float2(-INFINITY, 0.f);
      o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (k < n) {
        v[u] = *reinterpret_cast<const float2*>(ml + k * mstride);
        o[u] = *reinterpret_cast<const f32x4*>(po + k * ostride);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // m = -inf: no key of that item is visible to the row (or no item).
      const float Mn = fmaxf(M, v[u].x);
      const float a = (M == -INFINITY) ? 0.f : fast_exp2(M - Mn);
      const float wk = (v[u].x == -INFINITY) ? 0.f : fast_exp2(v[u].x - Mn);
      acc = acc * a + o[u] * wk;
      z = z * a + v[u].y * wk;
      M = Mn;
    }
  }
  s_m[pl][dl] = M;
  s_z[pl][dl] = z;
  s_o[pl][dl] = acc;
  __syncthreads();
  if (pl != 0) return;
  const int i = row / G, hh = row % G;
  const int h = ri.kv_head * G + hh;
  const float zs = sink_log2(A, ri.seq, h);
  float Mx = zs;
#pragma unroll
  for (int j = 0; j < PARTS; ++j) Mx = fmaxf(Mx, s_m[j][dl]);
  float Z = (zs == -INFINITY) ? 0.f : fast_exp2(zs - Mx);
  f32x4 tot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < PARTS; ++j) {
    const float mj = s_m[j][dl];
    const float wj = (mj == -INFINITY) ? 0.f : fast_exp2(mj - Mx);
    Z += s_z[j][dl] * wj;
    tot += s_o[j][dl] * wj;
  }
  store_out<D, false>(A, ((int64_t)(ri.q_off + i) * Hq + h) * D + d, tot * (1.0f / Z));
}

hipError_t launch_partition(const KernelArgs& a, int n_items, int head_dim, bool fp8, int ntmax,
                            hipStream_t stream) {
  if (n_items <= 0) return hipSuccess;
  if (ntmax < 1 || ntmax > kGroupWaves) return hipErrorInvalidValue;
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

hipError_t launch_reduce(const KernelArgs& a, int n_red, int head_dim, int rows_stride,
                         int max_parts, hipStream_t stream) {
  if (n_red <= 0) return hipSuccess;
  const unsigned items = (unsigned)n_red * rows_stride;
  if (max_parts <= 32) {  // one workgroup per row: 32 (D 128) or 16 column lanes x 4 or 8
    if (head_dim == 128)
      hipLaunchKernelGGL((pa_reduce_kernel<128, 32, 4>), dim3(items), dim3(128), 0, stream, a);
    else
      hipLaunchKernelGGL((pa_reduce_kernel<64, 16, 8>), dim3(items), dim3(128), 0, stream, a);
  } else {  // 8 column lanes x 32 partition lanes per quarter (or half) of a row
    if (head_dim == 128)
      hipLaunchKernelGGL((pa_reduce_kernel<128, 8, 32>), dim3(items * 4), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((pa_reduce_kernel<64, 8, 32>), dim3(items * 2), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace pav
