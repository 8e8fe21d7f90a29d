// gfx950 kernels for paged verify attention.
//
// Partition kernel: one workgroup per work item (one or two per CU, by
// layout; the single-launch call runs a persistent grid that takes the items
// in turn) = the keys [key_begin, key_end) of one (sequence, KV head), the
// item's packed rows of that KV head. The waves form NG token groups (1 to
// 4, by layout): group g takes the item's 32-token chunks (two 16-token
// pages) g, g + NG, ..., each through an LDS ring of its own that the group's
// loader wave fills by direct global-to-LDS loads (K as token rows with a
// 16-byte chunk swizzle, V into an XOR-swizzled token-major tile); one
// workgroup barrier per step recycles a stage in every ring. Within a group,
// compute wave r owns row tile r (16 rows) and, per chunk,
//   1. computes S^T = K Q^T, tokens on the M index: bf16 K with
//      v_mfma_f32_16x16x32_bf16; FP8 K codes as stored with the e4m3 MFMA
//      (v_mfma_f32_16x16x128_f8f6f4) against the query split once into two
//      e4m3 terms, the per-token K scale multiplying the scores,
//   2. masks (causal within the query, window, key range) by selecting -inf
//      on boundary chunks,
//   3. runs an online softmax in the exp2 domain whose reference max only
//      moves when a chunk beats it by 2^8 (rare rescaling),
//   4. accumulates O^T += V^T P^T: bf16 V^T from ds_read_b64_tr_b16 with
//      P^T straight from the S^T accumulator registers as a bf16 hi+lo pair;
//      FP8 V codes from ds_read_b64_tr_b8, converted exactly to fp16 in
//      registers, against P w in fp16 (the per-token V scale folded in).
// At the end the groups' states of each tile merge through LDS and the
// workgroup writes the output, or this item's partial, which the reduce
// kernel merges with the other partials of a split (sequence, KV head) by
// log-sum-exp.
//
// Sources: ATOM #2843 ("keep MTP-5 decode on FlyDSL pa_decode past the gluon
// query-length limit", Motivation and Follow-up in aiter: rows = query length
// x GQA group, per-token FP8 KV scales, a partition kernel and a reducer);
// ATOM #3091 (Summary: 16-token pages through a block table, stores masked
// by row liveness).
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "pa_internal.h"

namespace pav {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

template <int D, bool FP8>
struct Cfg {
  static constexpr int KS = D / 32;                 // bf16 QK contraction steps of 32
  static constexpr int KS8 = D >= 128 ? D / 128 : 1;  // FP8 QK steps of 128 (D 64: half used)
  static constexpr int MT = D / 16;                 // PV output tiles along D
  static constexpr int ESZ = FP8 ? 1 : 2;           // bytes per KV element
  static constexpr int ROWB = D * ESZ;              // bytes per token in a page
  static constexpr int BLKB = kBlock * ROWB;        // bytes per (page, KV head)
  static constexpr int KLD = BLKB / 1024;           // 1 KiB K loads per page
  static constexpr int VLD = (2 * BLKB) / 1024;     // 1 KiB V loads per chunk
  static_assert(BLKB >= 1024, "a 1 KiB slab must stay inside one page");
};


// bf16 QK: lane group c holds d = 32 s + 8 c .. +8 of contraction step s
// (64 contiguous bytes per token across the 4 lane groups); Q uses the same
// map.
__device__ __forceinline__ int qk_dmap(int s, int c) { return 32 * s + 8 * c; }

// FP8 QK runs on v_mfma_f32_16x16x128_f8f6f4 with the codes as they are:
// lane l holds 32 codes of token (or query row) l % 16 at d = 128 ks +
// 32 (l / 16) + j, j = 0..31, for both operands (at D 64 lane groups 2 and 3
// hold zeros).

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

// The same eight codes -> eight fp16 values, exactly (e4m3's range and
// precision fit inside fp16's).
__device__ __forceinline__ f16x8 fp8x8_to_f16(uint32_t w0, uint32_t w1) {
  const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, false);
  const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w0, 1.0f, true);
  const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, false);
  const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w1, 1.0f, true);
  return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
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

// max(a, b) in one instruction (see max3 below: the operands are never NaN
// where these are used, so the quieting fmaxf adds is not needed).
__device__ __forceinline__ float max2(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}

__device__ __forceinline__ float xlane_max4(float v) {
  float a = v, b = v;
  swap16(a, b);
  float c = max2(a, b), d = c;
  swap32(c, d);
  return max2(c, d);
}

__device__ __forceinline__ float xlane_sum4(float v) {
  float a = v, b = v;
  swap16(a, b);
  float c = a + b, d = c;
  swap32(c, d);
  return c + d;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max(a, b, c) in one instruction. (fmaxf would first quiet possible
// signalling NaNs with an extra instruction per operand; the operands here
// are scores and scales, never NaN where they are used.)
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float max8(const f32x4 (&x)[2]) {
  return max3(max3(x[0][0], x[0][1], x[0][2]), max3(x[0][3], x[1][0], x[1][1]),
              max2(x[1][2], x[1][3]));
}

// LDS V tile of one wave: [32 tokens][D] elements (bf16, or FP8 codes),
// token-major, stored in 16-byte chunks whose position within a token row is
// XOR-swizzled by the token, so that the transposing reads below (16 lanes
// of a group reading 4 tokens x 32 bytes for bf16, 8 tokens x 16 bytes for
// FP8) hit distinct banks.
template <int D, bool FP8>
__device__ __forceinline__ int vswz(int t) {
  if constexpr (FP8) {
    if constexpr (D == 64) return ((t & 3) >> 1) | (((t >> 4) & 1) << 1);
    else if constexpr (D == 128) return (t & 3) | (((t >> 4) & 1) << 2);
    else return (t & 3) | (((t >> 4) & 1) << 2) | (((t >> 2) & 1) << 3);
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

// LDS K tile of one page: its 16 token rows of ROWB bytes, token-major as in
// the pool, with the 16-byte chunks of row t XOR-swizzled by kswz(t). The
// direct-to-LDS loads then fetch whole token rows (every 1 KiB load covers
// full cache lines: a load of 16 rows x 64 bytes, the MFMA operand order,
// streamed at about 80% of the rate of whole rows), and the operand reads,
// in which 16 lanes read one chunk index of 16 consecutive rows, hit
// distinct banks: the swizzle spreads those rows over all sixteen 16-byte
// slots of a 256-byte bank window.
template <int D, bool FP8>
__device__ __forceinline__ int kswz(int t) {
  constexpr int ROWB = D * (FP8 ? 1 : 2);
  constexpr int RPW = 256 / ROWB;  // token rows per 256-byte bank window
  constexpr int CPR = ROWB / 16;   // 16-byte chunks per row
  return (t / RPW) % CPR;
}
template <int D, bool FP8>
__device__ __forceinline__ int ktile_chunk(int t, int chunk) {
  constexpr int ROWB = D * (FP8 ? 1 : 2);
  return t * ROWB + ((chunk ^ kswz<D, FP8>(t)) << 4);
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

// A workgroup's layout: NG token groups of TW row-tile waves and one
// loader each. Two groups of four tile waves serve up to 64 rows (three at
// D 256, up to 48 rows); FP8 at D 128 uses four groups of three for plans of
// at most 48 rows and three groups of four above, so that every SIMD hosts
// three compute waves (fifteen waves of at most 128 registers fill a SIMD's
// 512; the two-group layout, two compute waves per SIMD, measured 4-5%
// slower on a mixed FP8 batch).
//
// OCC is the number of workgroups meant to share a CU. One (OCC 1) holds
// most of the CU's 160 KiB of LDS; that suits a plan whose items fit one
// round. When there are more items than CUs, two smaller workgroups (OCC 2,
// at most 80 KiB each) share a CU, so that one streams while the other is
// in its prologue or epilogue. (FP8 KV keeps one: its items are bound by
// compute per SIMD, and the role rotation below only spreads the compute
// waves over the SIMDs within one workgroup; two one-group workgroups
// measured 6% slower on a mixed FP8 batch.)
template <int NG, int TW, int NL>
constexpr int kThreads = 64 * NG * (TW + NL);
// Ring bytes per group.
template <int NG, int OCC>
constexpr int kGroupRingBytes = OCC == 2 ? 72 * 1024 / NG : (NG == 2 ? 76 * 1024 : 38 * 1024);

// One ring stage: a 32-token chunk.
template <int D, bool FP8>
struct Ring {
  using C = Cfg<D, FP8>;
  static constexpr int KB = 2 * C::KLD * 1024;   // K tiles of two pages (swizzled rows)
  static constexpr int VB = C::VLD * 1024;       // V tile of two pages
  static constexpr int SB = FP8 ? 256 : 0;       // K and V scales of two pages
  static constexpr int STAGE = KB + VB + SB;
  // Loads per chunk: 1 KiB ones of K and V, and (FP8) one of the scales.
  // Load j of a chunk is issued by the group's issuer j mod P (below).
  static constexpr int T = 2 * C::KLD + C::VLD + (FP8 ? 1 : 0);
  static_assert(STAGE % 256 == 0 && KB % 256 == 0, "stage addresses keep their low 8 bits zero");
};

// A group's ring of R stages.
template <int D, bool FP8, int NG, int OCC>
struct RingN : Ring<D, FP8> {
  using S = Ring<D, FP8>;
  static constexpr int R0 = kGroupRingBytes<NG, OCC> / S::STAGE;
  // Stages per group, at most four: the loader issues R - 1 chunks in the
  // prologue, and with eight stages (FP8 at D 128, more than 48 rows) that
  // early burst measured ~10 us slower over a multi-round call than four.
  static constexpr int R = R0 < 4 ? R0 : 4;
  static_assert(R >= 3, "the ring needs enough stages to keep loads in flight");
  static_assert((R - 2) * S::T <= 63, "vmcnt holds at most 63");
  static constexpr int RING = R * S::STAGE;      // bytes per group
};

// The loads of one chunk that issuer i of a group's P issuers makes (load j
// goes to issuer j mod P): T / P, one more for the first T mod P issuers.
template <int T, int P>
struct Share {
  static constexpr int LO = T / P;
  static constexpr int HI = LO + (T % P ? 1 : 0);
  static constexpr int NHI = T % P;  // issuers with HI loads
};

// The ring starts 1 KiB aligned, and stages are multiples of 256 bytes: the
// FP8 V reads rely on the low 8 bits of a stage's address being zero.
template <int D, bool FP8, int NG, int TW, int OCC>
struct Smem {
  alignas(1024) unsigned char ring[NG][RingN<D, FP8, NG, OCC>::RING];
  int32_t pages[2 * kMaxItemChunks];  // page ids of each chunk's two pages
  int32_t next_item;                  // single-launch call: the workgroup's next item
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

// Issuer `ii` of P's loads of one chunk into stage `sb` of the group's ring
// (load j when j mod P == ii): K of the chunk's two pages (KLD loads of
// 1 KiB per page) into their swizzled K tiles and V of the two pages into
// the swizzled V tile (in both, lane l fetches whichever source chunk
// belongs at its tile position, so every load reads whole token rows), and
// the FP8 scales. `ii` is wave-uniform,
// so the selection is a scalar branch per load. The lane's offsets are
// derived on every call (the empty asm hides that they never change),
// rather than held in registers across the loop.
template <int D, bool FP8, int P>
__device__ __forceinline__ void issue_chunk(const KernelArgs& A, unsigned char* sb, int pa,
                                            int pb, int g, int lane, int ii) {
  using C = Cfg<D, FP8>;
  using RG = Ring<D, FP8>;
  int ln = lane;
  asm volatile("" : "+v"(ln));
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int page = half ? pb : pa;
    const char* src = static_cast<const char*>(A.k_pool) +
                      ((int64_t)page * A.num_kv_heads + g) * C::BLKB;
    unsigned char* dst = sb + half * C::BLKB;
#pragma unroll
    for (int u = 0; u < C::KLD; ++u) {
      if ((half * C::KLD + u) % P != ii) continue;
      const int pos = u * 1024 + ln * 16;  // byte position in this page's K tile
      const int tp = pos / C::ROWB;        // its token row
      const int ch = ((pos % C::ROWB) >> 4) ^ kswz<D, FP8>(tp);  // its source chunk
      dma16(src + (uint32_t)(tp * C::ROWB + ch * 16), dst + u * 1024);
    }
  }
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int page = half ? pb : pa;
    const char* src = static_cast<const char*>(A.v_pool) +
                      ((int64_t)page * A.num_kv_heads + g) * C::BLKB;
    unsigned char* dst = sb + RG::KB + half * (C::BLKB);
#pragma unroll
    for (int u = 0; u < C::VLD / 2; ++u) {
      if ((2 * C::KLD + half * (C::VLD / 2) + u) % P != ii) continue;
      const int pos = u * 1024 + ln * 16;  // byte position in this page's half of the tile
      const int tp = pos / C::ROWB;        // token within the page
      const int t = 16 * half + tp;        // token within the chunk (sets the swizzle)
      const int ch = ((pos % C::ROWB) >> 4) ^ vswz<D, FP8>(t);  // its source chunk
      dma16(src + (uint32_t)(tp * C::ROWB + ch * 16), dst + u * 1024);
    }
  }
  if constexpr (FP8) {  // scales: [K page A][K page B][V page A][V page B] x 16 tokens
    if ((2 * C::KLD + C::VLD) % P == ii) {
      const int which = ln >> 4, tok = ln & 15;
      const int pgs = (which & 1) ? pb : pa;
      const float* src2 = ((which < 2) ? A.k_scales : A.v_scales) +
                          ((int64_t)pgs * A.num_kv_heads + g) * kBlock + tok;
      dma4(src2, sb + RG::KB + RG::VB);
    }
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

// Query operands of the lane's row: bf16 (the bf16 MFMA's B operand), or for
// FP8 KV two e4m3 terms, Q = qs (hi + lo), in the FP8 MFMA's B layout.
template <int D, bool FP8>
struct QOps {
  bf16x8 q[Cfg<D, FP8>::KS];
};
template <int D>
struct QOps<D, true> {
  i32x8 hi[Cfg<D, true>::KS8];
  i32x8 lo[Cfg<D, true>::KS8];
  float qs;  // the row's power-of-two scale
};

template <int D, bool FP8>
struct WaveState {
  QOps<D, FP8> Q;
  f32x4 o[Cfg<D, FP8>::MT];
  float m;   // reference max of the lane's row (log2 units); p <= 2^kRescale
  float l;   // this lane's share of the row sum
  int prow;  // absolute position of the lane's row
};

// The reference max only moves when a chunk's max exceeds it by more than
// this many log2 units; until then probabilities stay below 2^8 and the
// accumulators are not rescaled. O, l and m always share one reference.
constexpr float kRescale = 8.0f;

// True when every key of the chunk lies in the item's range and is visible
// to every row of the item (no masks needed).
__device__ __forceinline__ bool chunk_interior(int tok0, int tv0, int tv1, int L, int q, int W) {
  return (tok0 >= tv0) && (tok0 + kChunk <= tv1) && (tok0 + kChunk - 1 <= L - q) &&
         (W == 0 || tok0 > L - 1 - W);
}

// Token of score element (bb, i) in lane group c: tok0 + 16 bb + 4 c + i.
// Scores of keys the lane's row may not see become -inf (a select: the
// pool slots of tokens outside the item's range may hold anything, NaN
// included).
template <int D, bool FP8>
__device__ __forceinline__ void mask_scores(const WaveState<D, FP8>& S, f32x4 (&sc)[2], int tok0,
                                            int tv0, int tv1, int W, int c) {
  const int p = S.prow;
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = tok0 + 16 * bb + 4 * c + i;
      const bool vis = (j >= tv0) && (j < tv1) && (j <= p) && (W == 0 || j > p - W);
      sc[bb][i] = vis ? sc[bb][i] : -INFINITY;
    }
  }
}

// Online softmax over one chunk in the exp2 domain (x = s * sigma * log2 e).
// The state (m, l, O) keeps l = sum 2^(x - m) and O = sum 2^(x - m) V over
// the keys so far, for a reference m that moves only when a chunk's largest x
// exceeds m + kShift + kRescale (then m = that x - kShift, and O and l are
// rescaled), so probabilities stay below 2^(kShift + kRescale). FP8 KV keeps
// kShift = 6: its P enters an fp16 product, and the shift keeps small
// probabilities clear of fp16's subnormal range. Adds the chunk's
// probabilities to l and returns p w per score element, w the token's V scale
// (FP8) or 1.
//
// FP8: `extra` (log2 units, per lane) raises the lane's largest x for that
// test by the log2 bound of its V scales minus one, so the bounds hold for
// p w rather than p: p w stays below 2^15 whatever the scales are.
template <bool FP8>
constexpr float kShift = FP8 ? 6.0f : 0.0f;

// Whether any row must move its reference, and then (in mx) the chunk's
// largest x per row, plus `extra`.
template <int D, bool FP8>
__device__ __forceinline__ bool needs_rescale(const WaveState<D, FP8>& S, const f32x4 (&sc)[2],
                                              float scale_log2, float extra, float& mx) {
  // Some row must move exactly when some lane's own largest x exceeds the
  // threshold (scale_log2 > 0, and the row's reference is the same on its
  // four lanes), so the maximum across the row's lanes is only taken on
  // that rare path.
  mx = max8(sc) * scale_log2 + extra;
  const bool move = __any(mx > S.m + (kShift<FP8> + kRescale));
  if (move) mx = xlane_max4(mx);
  return move;
}

template <int D, bool FP8>
__device__ __forceinline__ void rescale(WaveState<D, FP8>& S, float mx) {
  using C = Cfg<D, FP8>;
  const float mnew = fmaxf(S.m, mx - kShift<FP8>);
  const float alpha = (mnew == -INFINITY) ? 1.f : fast_exp2(S.m - mnew);
  S.m = mnew;
  S.l *= alpha;
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) S.o[mt] *= alpha;
}

// The chunk's probabilities for the current reference: adds them to l and
// returns p w per score element.
template <int D, bool FP8>
__device__ __forceinline__ void chunk_probs(WaveState<D, FP8>& S, const f32x4 (&sc)[2],
                                            const f32x4 (&vs)[2], float scale_log2,
                                            float (&pw)[8]) {
  const float msafe = (S.m == -INFINITY) ? 0.f : S.m;
  float p[8];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      p[4 * bb + i] = fast_exp2(__builtin_fmaf(sc[bb][i], scale_log2, -msafe));
      pw[4 * bb + i] = FP8 ? p[4 * bb + i] * vs[bb][i] : p[4 * bb + i];
    }
  }
  S.l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
}

template <int D, bool FP8>
__device__ __forceinline__ void softmax_p(WaveState<D, FP8>& S, const f32x4 (&sc)[2],
                                          const f32x4 (&vs)[2], float scale_log2, float (&pw)[8],
                                          float extra = 0.f) {
  float mx;
  if (needs_rescale(S, sc, scale_log2, extra, mx)) {
    asm volatile("");  // a real branch (rescaling is rare)
    rescale(S, mx);
  }
  chunk_probs(S, sc, vs, scale_log2, pw);
}

// P^T as two bf16 terms, hi = bf16(p w) and lo = bf16(p w - hi): its
// rounding error (about 2^-17 relative) stays far below the output's own
// bf16 rounding even when one key dominates a row.
__device__ __forceinline__ void split_bf16(const float (&pw)[8], bf16x8& p_hi, bf16x8& p_lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 hi = (__bf16)pw[e];
    p_hi[e] = hi;
    p_lo[e] = (__bf16)(pw[e] - (float)hi);
  }
}

// O^T[d][row] += V^T[d][token] P^T[token][row] for output tile mt. The
// contraction index (lane group c, element e) is token 16 (e / 4) + 4 c +
// e % 4 for both operands: that is where the S^T accumulator left P.
__device__ __forceinline__ f32x4 pv_tile(bf16x8 v, bf16x8 p_hi, bf16x8 p_lo, f32x4 o) {
  o = mfma_bf16(v, p_hi, o);
  return mfma_bf16(v, p_lo, o);
}

// One chunk for the wave's 16-row tile, bf16 KV: kv is the ring stage (the
// K tiles of the two pages as swizzled token rows, then the V tile).
template <int D>
__device__ __forceinline__ void compute_chunk(WaveState<D, false>& S, const unsigned char* kv,
                                              int tok0, int tv0, int tv1, int L, int q, int W,
                                              float scale_log2, int lane) {
  using C = Cfg<D, false>;
  using RG = Ring<D, false>;
  const int c = lane >> 4;
  const int i16 = lane & 15;

  // ---- LDS reads of the chunk: K operands, then every V^T operand (one
  // asm block whose lgkmcnt(0) also covers the K reads), so both latencies
  // overlap.
  // Contraction step u of token row i16 is chunk 4 u + c of its K tile row.
  u32x4 kr[2][C::KLD];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb)
#pragma unroll
    for (int u = 0; u < C::KLD; ++u)
      kr[bb][u] = *reinterpret_cast<const u32x4*>(kv + bb * C::BLKB +
                                                  ktile_chunk<D, false>(i16, 4 * u + c));
  const uint32_t vt = lds_addr(kv + RG::KB);
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
    for (int u = 0; u < C::KLD; ++u)
      acc = mfma_bf16(__builtin_bit_cast(bf16x8, kr[bb][u]), S.Q.q[u], acc);
    sc[bb] = acc;
  }
  if (!chunk_interior(tok0, tv0, tv1, L, q, W)) {
    // A real branch: the compiler would otherwise turn the selects into
    // straight-line code that every chunk pays for.
    asm volatile("");
    mask_scores<D, false>(S, sc, tok0, tv0, tv1, W, c);
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = tok0 + 16 * bb + 4 * c + i;
        const bool ok = (j >= tv0) && (j < tv1);  // V of other tokens may be NaN
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
          vops[mt][4 * bb + i] = ok ? vops[mt][4 * bb + i] : (__bf16)0.f;
      }
    }
  }
  const f32x4 vs[2] = {};
  float pw[8];
  softmax_p<D, false>(S, sc, vs, scale_log2, pw);
  bf16x8 p_hi, p_lo;
  split_bf16(pw, p_hi, p_lo);
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) S.o[mt] = pv_tile(vops[mt], p_hi, p_lo, S.o[mt]);
}

// V^T operands of one FP8 chunk: ds_read_b64_tr_b8 gives lane i of a
// 16-lane group column i of an 8 x 16 byte tile whose row r the lanes 2r,
// 2r + 1 address; the group's rows are its 8 tokens 16 (r / 4) + 4 c + r % 4,
// the contraction order of P^T. One asm block, ending with lgkmcnt(0).
template <int N>
__device__ __forceinline__ void vt_reads_b8(i32x2 (&r)[N], const uint32_t (&a)[N]);

template <>
__device__ __forceinline__ void vt_reads_b8<4>(i32x2 (&r)[4], const uint32_t (&a)[4]) {
  asm volatile(
      "ds_read_b64_tr_b8 %0, %4\n\t"
      "ds_read_b64_tr_b8 %1, %5\n\t"
      "ds_read_b64_tr_b8 %2, %6\n\t"
      "ds_read_b64_tr_b8 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
}

template <>
__device__ __forceinline__ void vt_reads_b8<8>(i32x2 (&r)[8], const uint32_t (&a)[8]) {
  asm volatile(
      "ds_read_b64_tr_b8 %0, %8\n\t"
      "ds_read_b64_tr_b8 %1, %9\n\t"
      "ds_read_b64_tr_b8 %2, %10\n\t"
      "ds_read_b64_tr_b8 %3, %11\n\t"
      "ds_read_b64_tr_b8 %4, %12\n\t"
      "ds_read_b64_tr_b8 %5, %13\n\t"
      "ds_read_b64_tr_b8 %6, %14\n\t"
      "ds_read_b64_tr_b8 %7, %15\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
}

template <>
__device__ __forceinline__ void vt_reads_b8<16>(i32x2 (&r)[16], const uint32_t (&a)[16]) {
  asm volatile(
      "ds_read_b64_tr_b8 %0, %16\n\t"
      "ds_read_b64_tr_b8 %1, %17\n\t"
      "ds_read_b64_tr_b8 %2, %18\n\t"
      "ds_read_b64_tr_b8 %3, %19\n\t"
      "ds_read_b64_tr_b8 %4, %20\n\t"
      "ds_read_b64_tr_b8 %5, %21\n\t"
      "ds_read_b64_tr_b8 %6, %22\n\t"
      "ds_read_b64_tr_b8 %7, %23\n\t"
      "ds_read_b64_tr_b8 %8, %24\n\t"
      "ds_read_b64_tr_b8 %9, %25\n\t"
      "ds_read_b64_tr_b8 %10, %26\n\t"
      "ds_read_b64_tr_b8 %11, %27\n\t"
      "ds_read_b64_tr_b8 %12, %28\n\t"
      "ds_read_b64_tr_b8 %13, %29\n\t"
      "ds_read_b64_tr_b8 %14, %30\n\t"
      "ds_read_b64_tr_b8 %15, %31\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]),
        "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]),
        "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7]),
        "v"(a[8]), "v"(a[9]), "v"(a[10]), "v"(a[11]), "v"(a[12]), "v"(a[13]), "v"(a[14]),
        "v"(a[15])
      : "memory");
}

// The FP8 MFMA: S^T (16 tokens x 16 rows) += K codes x query codes over 128
// values of d, both e4m3, unscaled.
__device__ __forceinline__ f32x4 mfma_fp8(i32x8 a, i32x8 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, acc, 0, 0, 0, 0, 0, 0);
}

// One chunk of FP8 KV for the wave's 16-row tile between its two phases:
// the scores (masked, in score units), the V scales, the V code columns and
// the chunk's largest x per row.
template <int D>
struct Fp8Chunk {
  f32x4 sc[2];
  f32x4 vs[2];
  i32x2 vcode[Cfg<D, true>::MT];
  float mx;
  int tok0;
  bool interior;
};

// Phase 1 of an FP8 chunk, straight from the ring stage st (K codes in the
// FP8 MFMA's operand order, the V code tile, then the K and V scales):
// S^T = K Q^T on the codes, once with each query term, times the per-token
// K scale (the row's query scale is folded into scale_log2, which the
// caller passes per row); masks; the V code columns (transposing byte
// reads, issued while the QK products run). Returns whether a row's
// reference must move before the chunk's probabilities are taken.
// The lane's byte offset in the V code tile for the transposing reads of
// output tile 0: lanes 2r, 2r + 1 of a group address token 16 (r / 4) +
// 4 c + r % 4 (the P^T order), bytes 8 k of the tile's 16-byte chunk.
template <int D>
__device__ __forceinline__ uint32_t vcode_lane_off(int lane) {
  const int rr = (lane & 15) >> 1, k = lane & 1;
  const int t = 16 * (rr >> 2) + 4 * (lane >> 4) + (rr & 3);
  return t * Cfg<D, true>::ROWB + (vswz<D, true>(t) << 4) + 8 * k;
}

// ASM_TR: the V code columns are read by one asm block (ending in
// lgkmcnt(0)) issued with the K reads, ahead of the QK products. Tile waves
// that also issue ring loads need it: the compiler drains every outstanding
// direct-to-LDS load (vmcnt(0)) before the transposing-read builtin.
// Otherwise the builtin lets the compiler spread the reads over the QK
// products.
template <int D, bool ASM_TR>
__device__ __forceinline__ bool chunk_scores(const WaveState<D, true>& S, Fp8Chunk<D>& X,
                                             const unsigned char* st, int tok0, int tv0, int tv1,
                                             int L, int q, int W, float scale_log2, int lane,
                                             uint32_t voff) {
  using C = Cfg<D, true>;
  using RG = Ring<D, true>;
  const int c = lane >> 4;
  const int i16 = lane & 15;
  const unsigned char* scl = st + RG::KB + RG::VB;
  X.tok0 = tok0;

  // ---- S^T = K Q^T: the K operands of both pages, then the products.
  i32x8 kop[2][C::KS8];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
    for (int ks = 0; ks < C::KS8; ++ks) {
      // Token row i16's codes d = 128 ks + 32 c .. +32: chunks 8 ks + 2 c
      // and the next one of its K tile row (D 64: lane groups 2 and 3 carry
      // zeros).
      const int ch = 8 * ks + 2 * (D >= 128 ? c : (c & 1));
      const unsigned char* kt = st + bb * C::BLKB;
      u32x4 x0 = *reinterpret_cast<const u32x4*>(kt + ktile_chunk<D, true>(i16, ch));
      u32x4 x1 = *reinterpret_cast<const u32x4*>(kt + ktile_chunk<D, true>(i16, ch + 1));
      if constexpr (D < 128) {
        if (c >= 2) x0 = x1 = u32x4{0, 0, 0, 0};
      }
      kop[bb][ks] = i32x8{(int)x0[0], (int)x0[1], (int)x0[2], (int)x0[3],
                          (int)x1[0], (int)x1[1], (int)x1[2], (int)x1[3]};
    }
  }
  if constexpr (ASM_TR) {
    // The V code columns, in one asm block whose lgkmcnt(0) also covers the
    // K reads above (voff: vcode_lane_off; see below for the addresses).
    uint32_t vo = voff;
    asm volatile("" : "+v"(vo));  // keep the per-tile addresses out of the loop
    const uint32_t vbase = lds_addr(st + RG::KB) + vo;
    uint32_t va[C::MT];
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) va[mt] = vbase ^ (uint32_t)(mt << 4);
    vt_reads_b8<C::MT>(X.vcode, va);
  }
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < C::KS8; ++ks) {
      acc = mfma_fp8(kop[bb][ks], S.Q.hi[ks], acc);
      acc = mfma_fp8(kop[bb][ks], S.Q.lo[ks], acc);
    }
    X.sc[bb] = acc;
  }
  f32x4 ksc[2];
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    ksc[bb] = *reinterpret_cast<const f32x4*>(scl + (bb * 16 + 4 * c) * 4);
    X.vs[bb] = *reinterpret_cast<const f32x4*>(scl + 128 + (bb * 16 + 4 * c) * 4);
  }

  // ---- V code columns (voff: vcode_lane_off), bytes 16 mt + 8 k of the
  // lane's token. The stage and the token row are 256-byte and ROWB aligned
  // and the swizzle only touches the 16-byte chunk bits, so tile mt's
  // address is a fixed XOR of one base. (The compute waves issue no
  // direct-to-LDS loads, so the compiler's own waits around these reads
  // cost nothing.)
  if constexpr (!ASM_TR) {
    uint32_t vo = voff;
    asm volatile("" : "+v"(vo));  // keep the per-tile addresses out of the loop
    const uint32_t vbase = lds_addr(st + RG::KB) + vo;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt)
      X.vcode[mt] = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
          (__attribute__((address_space(3))) i32x2*)(uintptr_t)(vbase ^ (uint32_t)(mt << 4)));
  }

  // (The row's query scale rides in scale_log2: the caller passes
  // sigma log2(e) times it.)
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) X.sc[bb] = X.sc[bb] * ksc[bb];
  X.interior = chunk_interior(tok0, tv0, tv1, L, q, W);
  if (!X.interior) {
    asm volatile("");  // a real branch
    mask_scores<D, true>(S, X.sc, tok0, tv0, tv1, W, c);
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = tok0 + 16 * bb + 4 * c + i;
        X.vs[bb][i] = ((j >= tv0) && (j < tv1)) ? X.vs[bb][i] : 0.f;  // NaN scales of other slots
      }
    }
  }
  // p w enters an fp16 product, so the reference is kept for p w rather
  // than for p: each lane raises its chunk maximum of x by e - 1, where
  // 2^(e-1) <= its largest V scale < 2^e (e from the exponent, at least
  // -63). After a rescale a row's largest p w is then within [2^6, 2^7], and
  // no chunk reaches 2^15 before the next one, whatever the magnitude of the
  // scales: V scales far below 1 keep p w clear of fp16's subnormal range,
  // and large ones of its overflow. (p itself stays below 2^78, l below
  // 2^98 over 1 Mi keys: far inside fp32.)
  const float vmax = max8(X.vs);
  const float extra = (float)(max(__builtin_amdgcn_frexp_expf(vmax), -63) - 1);
  return needs_rescale(S, X.sc, scale_log2, extra, X.mx);
}

// Phase 2 of an FP8 chunk: probabilities for the current reference, the V
// code mask and O^T += V^T P^T in fp16 (V codes convert exactly, p w
// (< 2^15) rounds to 11 bits: a relative error of at most 2^-12), one
// product per output tile.
template <int D>
__device__ __forceinline__ void chunk_finish(WaveState<D, true>& S, Fp8Chunk<D>& X, int tv0,
                                             int tv1, float scale_log2, int lane) {
  using C = Cfg<D, true>;
  const int c = lane >> 4;
  float pw[8];
  chunk_probs<D, true>(S, X.sc, X.vs, scale_log2, pw);
  if (!X.interior) {
    asm volatile("");
    // Codes of tokens outside the item's range become 0 (byte e of a
    // column is token 16 (e / 4) + 4 c + e % 4).
    uint32_t keep[2];
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      keep[bb] = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = X.tok0 + 16 * bb + 4 * c + i;
        keep[bb] |= ((j >= tv0) && (j < tv1)) ? (0xFFu << (8 * i)) : 0u;
      }
    }
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) {
      X.vcode[mt][0] &= (int)keep[0];
      X.vcode[mt][1] &= (int)keep[1];
    }
  }
  f16x8 p16;
#pragma unroll
  for (int e = 0; e < 8; ++e) p16[e] = (_Float16)pw[e];
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt)
    S.o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
        fp8x8_to_f16((uint32_t)X.vcode[mt][0], (uint32_t)X.vcode[mt][1]), p16, S.o[mt], 0, 0, 0);
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

// ---- The fused call: split items merge their pair's partials themselves.
//
// Partials and tree slots are written and read with device-scope buffer
// accesses (sc1: the mapping of relaxed device-scope atomic stores and
// loads on gfx950): the stores write through the XCD's L2, and the loads are
// not served from another XCD's stale lines. A workgroup waits until its
// stores have completed before its one atomic arrival at the node, so the
// workgroup whose arrival completes the node's count finds every partial
// at the point of coherence. No L2 write-back or invalidation is needed (a
// device-scope fence per workgroup writes back the XCD's whole L2 and cost
// more than the separate reduce kernel).
constexpr int kScopeDevice = 16;  // buffer access cache bits: sc1

// A raw buffer over [base, base + bytes): offsets are 32-bit and accesses
// past the end read zeros and write nothing.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t dev_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ void st_dev(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, kScopeDevice);
}
__device__ __forceinline__ void st_dev(__amdgpu_buffer_rsrc_t r, uint32_t off, float2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, off, 0, kScopeDevice);
}
__device__ __forceinline__ f32x4 ld_dev4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kScopeDevice));
}
__device__ __forceinline__ float2 ld_dev2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(float2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kScopeDevice));
}

// Optional stamps per work item (the device's 100 MHz real-time clock),
// taken by thread 0 of the workgroup running it when the caller attached a
// buffer: slot 0 the item's start, 1 every wave past its chunk loop, 2 the
// outputs issued (or, for a split item of the fused call, its partial's
// stores complete), 3 the arrival counted, 4 + l the merge of tree level l
// done (l < 3; last arrivers only), 7 the XCC id (high half) and HW_ID
// register (low half).
__device__ __forceinline__ void stamp(const KernelArgs& A, int item, int slot) {
  if (A.stamps && threadIdx.x == 0)
    A.stamps[(size_t)item * kStampsPerItem + slot] = __builtin_amdgcn_s_memrealtime();
}

// Arrival of a workgroup whose partial (or tree slot) is written, at merge
// node `node`; every thread of the workgroup calls it (NT threads). The last
// arriver resets the node's counter and folds the node's partials, row by
// row in index order, into the output or into its tree slot, and then
// arrives at the parent node. s_flag: one int of LDS no wave still uses.
// (One workgroup folds a node: with device-scope loads it pulls about
// 60 GB/s, 16 partials of 48 rows at D 128 in about 7 us, where the
// separate reduce kernel spreads every pair's merge over the device.)
template <int D, int NT>
__device__ void fused_arrive(const KernelArgs& A, int item, int node, int* s_flag) {
  constexpr int COLS = D / 4;
  constexpr int U = 8;  // partials in flight per thread
  const int tid = threadIdx.x;
  for (int lev = 0;; ++lev) {
    wait_vm<0>();  // this wave's stores are complete at device scope
    __syncthreads();
    if (lev == 0) stamp(A, item, 2);
    if (tid == 0) {
      const int need = A.nodes[node].n_parts;
      const int old =
          __hip_atomic_fetch_add(A.counters + node, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const int last = old == need - 1;
      // Every arrival of this call is counted: zero for the next call.
      if (last)
        __hip_atomic_store(A.counters + node, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      *s_flag = last;
    }
    if (lev == 0) stamp(A, item, 3);
    __syncthreads();
    if (!*s_flag) return;  // uniform over the workgroup
    const MergeNode nd = A.nodes[node];
    const int64_t RS = A.rows_stride;
    const float* so = nd.from_tree ? A.tree_o : A.part_o;
    const float* sm = nd.from_tree ? A.tree_ml : A.part_ml;
    const uint32_t ostride = (uint32_t)(RS * D * 4), mstride = (uint32_t)(RS * 8);
    const int n = nd.n_parts;
    const uint32_t span = (uint32_t)((n - 1) * nd.slot_stride + 1);  // slots the node spans
    const __amdgpu_buffer_rsrc_t ro = dev_rsrc(so + nd.slot_base * RS * D, ostride * span);
    const __amdgpu_buffer_rsrc_t rm = dev_rsrc(sm + nd.slot_base * RS * 2, mstride * span);
    const uint32_t ps = ostride * nd.slot_stride, pm = mstride * nd.slot_stride;
    for (int t = tid; t < nd.nrows * COLS; t += NT) {
      const int row = nd.row0 + t / COLS;  // packed row of the sequence
      const int d = (t % COLS) * 4;
      const uint32_t oo = (uint32_t)(row * D + d) * 4, om = (uint32_t)row * 8;
      float M = -INFINITY, z = 0.f;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      for (int k0 = 0; k0 < n; k0 += U) {
        float2 v[U];
        f32x4 o[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          v[u] = make_float2(-INFINITY, 0.f);
          o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
          if (k0 + u < n) {
            v[u] = ld_dev2(rm, om + (k0 + u) * pm);
            o[u] = ld_dev4(ro, oo + (k0 + u) * ps);
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          // m = -inf: no key of that partial is visible to the row.
          const float Mn = fmaxf(M, v[u].x);
          const float a = (M == -INFINITY) ? 0.f : fast_exp2(M - Mn);
          const float wk = (v[u].x == -INFINITY) ? 0.f : fast_exp2(v[u].x - Mn);
          acc = acc * a + o[u] * wk;
          z = z * a + v[u].y * wk;
          M = Mn;
        }
      }
      if (nd.parent >= 0) {
        // A tree slot, in the partition kernel's partial format.
        const __amdgpu_buffer_rsrc_t wo = dev_rsrc(A.tree_o + nd.out_slot * RS * D, ostride);
        st_dev(wo, oo, acc);
        if (d == 0)
          st_dev(dev_rsrc(A.tree_ml + nd.out_slot * RS * 2, mstride), om, make_float2(M, z));
      } else {
        const int i = row / A.group, hh = row % A.group;
        const int h = nd.kv_head * A.group + hh;
        const float zs = sink_log2(A, nd.seq, h);
        const float Mx = fmaxf(M, zs);
        const float a = (M == -INFINITY) ? 0.f : fast_exp2(M - Mx);
        const float Z = z * a + ((zs == -INFINITY) ? 0.f : fast_exp2(zs - Mx));
        store_out<D, false>(A, ((int64_t)(nd.q_off + i) * A.num_q_heads + h) * D + d,
                            acc * (a / Z));
      }
    }
    if (lev < 3) stamp(A, item, 4 + lev);
    if (nd.parent < 0) return;
    node = nd.parent;
  }
}

// The lane's query values for the FP8 MFMA: the 32 values d = 128 ks +
// 32 c + j of its row (zeros past D), as two e4m3 terms of the row scaled by
// a power of two, Q = qs (hi + lo). With the row's largest |value| scaled
// into [128, 256), hi keeps the top 4 significant bits and the exact
// residual fits lo's 4 bits for every value within 2^-9 of the row's
// largest (bf16 values carry 8 significant bits), so the two terms
// reproduce Q exactly there and to within 2^-17 of the row's largest
// value below that.
template <int D>
__device__ __forceinline__ void load_query_fp8(QOps<D, true>& Q, const uint16_t* qp, bool live,
                                               int c) {
  using C = Cfg<D, true>;
  u32x4 raw[C::KS8][4];
  float amax = 0.f;
#pragma unroll
  for (int ks = 0; ks < C::KS8; ++ks) {
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int d = 128 * ks + 32 * c + 8 * v;
      raw[ks][v] = u32x4{0, 0, 0, 0};
      if (live && d < D) raw[ks][v] = *reinterpret_cast<const u32x4*>(qp + d);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        amax = fmaxf(amax, fabsf(__uint_as_float(raw[ks][v][e] << 16)));
        amax = fmaxf(amax, fabsf(__uint_as_float(raw[ks][v][e] & 0xFFFF0000u)));
      }
    }
  }
  amax = xlane_max4(amax);
  // 2^e <= amax < 2^(e+1); a zero (or subnormal) row keeps e >= -100.
  int e = (int)((__float_as_uint(amax) >> 23) & 0xFF) - 127;
  e = e < -100 ? -100 : e;
  const float inv = __uint_as_float((uint32_t)(127 + 7 - e) << 23);  // 2^(7 - e)
  Q.qs = __uint_as_float((uint32_t)(127 - 7 + e) << 23);             // 2^(e - 7)
  // hi and lo come from the hardware conversion (v_cvt_pk_fp8_f32, nearest
  // even; |y| < 2^8 stays far from e4m3's overflow), the residual y - hi
  // from converting hi back: both exact in fp32.
#pragma unroll
  for (int ks = 0; ks < C::KS8; ++ks) {
    uint32_t hw[8], lw[8];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {  // dwords 2v, 2v + 1: four values each
        float y[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const uint32_t w = raw[ks][v][2 * h + (b >> 1)];
          y[b] = __uint_as_float((b & 1) ? (w & 0xFFFF0000u) : (w << 16)) * inv;
        }
        int hb = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
        hb = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], hb, true);
        const f32x2 h01 = __builtin_amdgcn_cvt_pk_f32_fp8(hb, false);
        const f32x2 h23 = __builtin_amdgcn_cvt_pk_f32_fp8(hb, true);
        int lb = __builtin_amdgcn_cvt_pk_fp8_f32(y[0] - h01[0], y[1] - h01[1], 0, false);
        lb = __builtin_amdgcn_cvt_pk_fp8_f32(y[2] - h23[0], y[3] - h23[1], lb, true);
        hw[2 * v + h] = (uint32_t)hb;
        lw[2 * v + h] = (uint32_t)lb;
      }
    }
    Q.hi[ks] = i32x8{(int)hw[0], (int)hw[1], (int)hw[2], (int)hw[3],
                     (int)hw[4], (int)hw[5], (int)hw[6], (int)hw[7]};
    Q.lo[ks] = i32x8{(int)lw[0], (int)lw[1], (int)lw[2], (int)lw[3],
                     (int)lw[4], (int)lw[5], (int)lw[6], (int)lw[7]};
  }
}

// Rotation of the roles in the second of two token groups: it puts that
// group's tile 0 on SIMD 2 (wave w runs on SIMD w mod 4), so that the two
// groups' first tiles use different SIMDs.
constexpr int rot2(int GW) {
  const int slot0 = (((2 - GW) % 4) + 4) % 4;  // group 1's slot on SIMD 2
  return (GW - slot0) % GW;
}

// NL: loader waves per token group. CL: whether the tile waves also issue a
// share of their group's ring loads (then P = NL + TW issuers per group,
// else P = NL).
// One work item, by the whole workgroup: item `idx` of the list. FUSED:
// the item of the single-launch call, which also fetches the index of the
// workgroup's next item (sm.next_item, set by thread 0 at the end).
template <int D, bool FP8, int NG, int TW, int NL, int OCC, bool CL, bool FUSED>
__device__ __forceinline__ void partition_item(const KernelArgs& A,
                                               Smem<D, FP8, NG, TW, OCC>& sm, int idx) {
  using C = Cfg<D, FP8>;
  using RG = RingN<D, FP8, NG, OCC>;
  constexpr int GW = TW + NL;            // waves per group
  constexpr int P = NL + (CL ? TW : 0);  // load issuers per group
  using SH = Share<RG::T, P>;
  stamp(A, idx, 0);
  const WorkItem it = A.items[idx];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  // Token group gp, role r (row tile r < TW, or loader r - TW). The roles
  // rotate by group so that the tile waves spread over the SIMDs (wave w
  // runs on SIMD w mod 4): with four groups of three tile waves and a loader
  // every SIMD hosts three tile waves and one loader; with two groups the
  // second group's tiles 0 and 1 sit on the two SIMDs the first group's
  // tiles 0 and 1 do not use, so items of up to two tiles run one compute
  // wave per SIMD. Three groups of five waves need no rotation: group gp's
  // four tile waves sit on four distinct SIMDs starting at SIMD gp, so
  // every SIMD hosts three of the twelve.
  constexpr int kRot = NG == 4 ? 1 : (NG == 2 ? rot2(GW) : 0);
  const int gp = w / GW, slot = w % GW;
  const int r = (slot + gp * kRot) % GW;
  const bool loader = r >= TW;
  // Ring-load issuer index within the group: loaders first, then (CL) the
  // tile waves.
  const int ii = loader ? r - TW : NL + r;
  const bool issuer = loader || CL;
  const int n = lane & 15, c = lane >> 4;
  const int b = it.seq, g = it.kv_head;
  const int G = A.group, Hq = A.num_q_heads;
  const int q = it.q_len, W = it.window;
  int L = it.ctx_len;
  int tv0 = it.key_begin, tv1 = it.key_end;
  if (A.dev_ctx) {
    // Lengths read at run time (the plan was built on upper bounds, which
    // its items cover): clamp to [q, bound], then clip the item's keys to
    // what this length makes visible. An item may end up empty.
    L = min(max(A.dev_ctx[b], q), L);
    const int lo = W > 0 ? max(0, L - q - W + 1) : 0;
    tv0 = max(tv0, lo);
    tv1 = min(tv1, L);
  }
  // The item's packed rows: [row0, row0 + rows) of the sequence's q x G
  // (a sequence with more rows than a workgroup carries is split into row
  // blocks, each its own item over the same keys).
  const int row0 = it.row0;
  const int rows = it.nrows;
  const int nt = (rows + 15) >> 4;  // row tiles; waves r >= nt do not compute
  const bool active = r < nt;
  const int tokbase = (tv0 >> 4) << 4;
  // <= kMaxItemChunks: [tv0, tv1) lies inside the planned item
  const int nch = tv1 > tv0 ? (tv1 - tokbase + kChunk - 1) / kChunk : 0;
  const int nst = (nch + NG - 1) / NG;  // steps: one chunk per group

  // Page ids of every chunk (a page past the item's end repeats the
  // chunk's first page, whose slots the masks then exclude).
  const int32_t* bt = A.block_table + (int64_t)b * A.max_blocks;
  // The loaders start their group's first R - 1 chunks at once (loader i of
  // NL issues load j of each when j mod NL == i) while the other waves fill
  // the page table and load the query. One vector load brings every page id
  // those chunks need: lane j < 2 (R - 1) reads chunk j / 2's page j % 2
  // (the chunk's first page where its second lies past the item). (Scalar
  // loads of the same entries came back up to 2.5 us later than vector
  // loads, and held the later groups' loaders back.)
  if (loader) {
    int pid = 0;
    {
      const int k = lane >> 1, which = lane & 1;
      const int ck = gp + NG * k;
      if (lane < 2 * (RG::R - 1) && ck < nch) {
        const int tok0 = tokbase + ck * kChunk;
        const int pg = (tok0 >> 4) + which;
        pid = bt[(which == 0 || tok0 + kBlock < tv1) ? pg : pg - 1];
      }
    }
    // The wait is the loader's only one here (no chunk is in flight yet);
    // with it explicit, the compiler adds none between the chunks' loads.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt unbounded
    int pa[RG::R - 1], pb[RG::R - 1];
#pragma unroll
    for (int k = 0; k < RG::R - 1; ++k) {
      pa[k] = __builtin_amdgcn_readlane(pid, 2 * k);
      pb[k] = __builtin_amdgcn_readlane(pid, 2 * k + 1);
    }
#pragma unroll
    for (int k = 0; k < RG::R - 1; ++k)
      if (gp + NG * k < nch)
        issue_chunk<D, FP8, NL>(A, sm.ring[gp] + k * RG::STAGE, pa[k], pb[k], g, lane, r - TW);
  }
  constexpr int kFillThreads = NG * TW * 64;
  const int fill_tid = (gp * TW + (loader ? 0 : r)) * 64 + lane;
  for (int i = fill_tid; !loader && i < 2 * nch; i += kFillThreads) {
    const int k = i >> 1, which = i & 1;
    const int tok0 = tokbase + k * kChunk;
    const int pg = (tok0 >> 4) + which;
    sm.pages[i] = bt[(which == 0 || tok0 + kBlock < tv1) ? pg : pg - 1];
  }

  // The wave's row tile: item row 16 r + lane % 16, packed row row0 + that
  // (padding rows mirror the item's last row and carry a zero query).
  WaveState<D, FP8> S;
  S.m = -INFINITY;
  S.l = 0.f;
#pragma unroll
  for (int mt = 0; mt < C::MT; ++mt) S.o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  // The loader skips the query (a wave-uniform branch): on a path shared
  // with the query loads it would also execute their vmcnt(0) and wait for
  // its ring's first chunks before the barrier below.
  if (!loader) {
    const int row = 16 * r + n;
    const bool live = active && row < rows;
    const int rr = row0 + (live ? row : rows - 1);
    const int i = rr / G, hh = rr % G;
    S.prow = L - q + i;
    const uint16_t* qp = A.q + ((int64_t)(it.q_off + i) * Hq + g * G + hh) * D;
    if constexpr (!FP8) {
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        u32x4 v = {0, 0, 0, 0};
        if (live) v = *reinterpret_cast<const u32x4*>(qp + qk_dmap(s, c));
        S.Q.q[s] = __builtin_bit_cast(bf16x8, v);
      }
    } else {
      load_query_fp8<D>(S.Q, qp, live, c);
    }
    // Finish the query and table loads here, with a wait the compiler sees:
    // otherwise it waits for the query inside the chunk loop.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), expcnt and lgkmcnt unbounded
  }
  ring_barrier();  // the page table is visible to every wave
  // The single-launch call's next item for this workgroup, fetched now so
  // that the round trip overlaps the item (the query loads above are done;
  // no other wait of this wave covers vector memory until the epilogue).
  int next_item = 0;
  if constexpr (FUSED) {
    if (tid == 0)
      next_item = (int)gridDim.x +
                  __hip_atomic_fetch_add(A.work, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  const uint32_t pages_addr = lds_addr(sm.pages);
  unsigned char* ring = sm.ring[gp];

  // Chunk of this wave's group at step k: gp + NG k. The loaders filled the
  // first R - 1 stages above; then per step: every issuer waits for its
  // loads of the step's chunk, the barrier (every group's chunk has landed
  // and every wave is done with the stage about to be refilled), the
  // issuers refill that stage (issuer ii of P making load j when j mod P ==
  // ii) while the tile waves work.
  //
  // The waits are per issuer: after the step's chunk, an issuer has made at
  // most its share of each of the next R - 2 chunks (the loaders' share of a
  // prologue chunk is larger, so the wait is then stricter than needed,
  // never looser); waiting until no more than R - 2 shares are pending
  // therefore covers its part of the step's chunk.
  auto step_begin = [&](int k) __attribute__((always_inline)) {
    if (issuer) {
      if (gp + NG * (k + RG::R - 2) < nch) {
        if (ii < SH::NHI) wait_vm<(RG::R - 2) * SH::HI>();
        else wait_vm<(RG::R - 2) * SH::LO>();
      } else {
        wait_vm<0>();
      }
    }
    ring_barrier();
    const int cn = gp + NG * (k + RG::R - 1);
    if (issuer && cn < nch) {
      int pa, pb;
      chunk_pages(pages_addr, cn, pa, pb);
      issue_chunk<D, FP8, P>(A, ring + ((k + RG::R - 1) % RG::R) * RG::STAGE, pa, pb, g, lane,
                             ii);
    }
  };
  if constexpr (!FP8) {
    for (int k = 0; k < nst; ++k) {
      const int ck = gp + NG * k;
      step_begin(k);
      if (active && ck < nch)
        compute_chunk<D>(S, ring + (k % RG::R) * RG::STAGE, tokbase + ck * kChunk, tv0, tv1, L,
                         q, W, A.scale_log2, lane);
    }
  } else {
    // The inner loop runs chunks whose rows keep their softmax reference;
    // a chunk that must move it leaves the loop, is finished after the
    // rescale, and the loop resumes at the next step. (With the rescale
    // inside the loop the compiler moves the accumulators between
    // registers on every chunk.)
    Fp8Chunk<D> X;
    const float sl = A.scale_log2 * S.Q.qs;  // per row: the query scale folded in
    const uint32_t voff = vcode_lane_off<D>(lane);
    int k = 0;
    for (;;) {
      bool moved = false;
      for (; k < nst; ++k) {
        const int ck = gp + NG * k;
        step_begin(k);
        if (active && ck < nch) {
          if (chunk_scores<D, CL>(S, X, ring + (k % RG::R) * RG::STAGE, tokbase + ck * kChunk,
                                  tv0, tv1, L, q, W, sl, lane, voff)) {
            moved = true;
            break;
          }
          chunk_finish<D>(S, X, tv0, tv1, sl, lane);
        }
      }
      if (!moved) break;
      rescale(S, X.mx);
      chunk_finish<D>(S, X, tv0, tv1, sl, lane);
      ++k;
    }
  }

  // ---- Merge the groups: the waves of groups 1..NG-1 hand (m, l, O) of
  // their tile to group 0's through LDS, which merges them in group order
  // (the rings are free once every wave is past the barrier; every wave's
  // loads have completed, its last wait was vmcnt(0)).
  S.l = xlane_sum4(S.l);
  __syncthreads();
  stamp(A, idx, 1);
  if (A.stamps && tid == 0)
    A.stamps[(size_t)idx * kStampsPerItem + 7] =
        ((unsigned long long)__builtin_amdgcn_s_getreg(0xF814) << 32) |  // XCC_ID
        (unsigned)__builtin_amdgcn_s_getreg(0xF804);                      // HW_ID
  constexpr int kXo = TW * C::MT * 64;                              // f32x4 per group
  f32x4* xo = reinterpret_cast<f32x4*>(&sm.ring[0][0]);           // [group-1][tile][mt][lane]
  float* xm = reinterpret_cast<float*>(xo + (NG - 1) * kXo);       // [group-1][tile][lane][m, l]
  static_assert((NG - 1) * (kXo * 16 + TW * 64 * 8) <= NG * RG::RING, "merge fits the rings");
  if (gp > 0 && active) {
    f32x4* o = xo + (gp - 1) * kXo;
    float* ml = xm + ((gp - 1) * TW + r) * 128;
#pragma unroll
    for (int mt = 0; mt < C::MT; ++mt) o[(r * C::MT + mt) * 64 + lane] = S.o[mt];
    ml[lane * 2] = S.m;
    ml[lane * 2 + 1] = S.l;
  }
  __syncthreads();
  const bool writer = gp == 0 && active;
  if constexpr (!FUSED) {
    if (!writer) return;
  }
  if (writer) {
#pragma unroll
    for (int j = 0; j < NG - 1; ++j) {
      const f32x4* o = xo + j * kXo;
      const float* ml = xm + (j * TW + r) * 128;
      const float m1 = ml[lane * 2], l1 = ml[lane * 2 + 1];
      const float M = fmaxf(S.m, m1);
      const float a0 = (S.m == -INFINITY) ? 0.f : fast_exp2(S.m - M);
      const float a1 = (m1 == -INFINITY) ? 0.f : fast_exp2(m1 - M);
#pragma unroll
      for (int mt = 0; mt < C::MT; ++mt)
        S.o[mt] = S.o[mt] * a0 + o[(r * C::MT + mt) * 64 + lane] * a1;
      S.l = S.l * a0 + l1 * a1;
      S.m = M;
    }

    // ---- Epilogue: the wave writes its rows (lane: row n, d = 16 mt +
    // 4 c + i).
    const int row = 16 * r + n;
    if (row < rows) {
      const int arow = row0 + row;  // packed row within the sequence's q x G
      const int i = arow / G, hh = arow % G;
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
      } else if constexpr (FUSED) {
        // Device-scope stores: the node's last arriver may run on another XCD.
        const int64_t RS = A.rows_stride;
        const __amdgpu_buffer_rsrc_t wo =
            dev_rsrc(A.part_o + it.slot * RS * D, (uint32_t)(RS * D * 4));
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
          st_dev(wo, (uint32_t)(arow * D + 16 * mt + 4 * c) * 4, S.o[mt]);
        if (c == 0)
          st_dev(dev_rsrc(A.part_ml + it.slot * RS * 2, (uint32_t)(RS * 8)), (uint32_t)arow * 8,
                 make_float2(S.m, S.l));
      } else {
        // Partials go out with nontemporal stores: the reduce kernel reads
        // them once, and lines kept out of the L2 make the kernel's final
        // write-back shorter (the partition kernel measured 1.5 us faster on
        // the MTP-5 workload).
        const int64_t pr = (int64_t)it.slot * A.rows_stride + arow;
#pragma unroll
        for (int mt = 0; mt < C::MT; ++mt)
          __builtin_nontemporal_store(
              S.o[mt], reinterpret_cast<f32x4*>(A.part_o + pr * D + 16 * mt + 4 * c));
        if (c == 0) {
          __builtin_nontemporal_store(S.m, A.part_ml + pr * 2);
          __builtin_nontemporal_store(S.l, A.part_ml + pr * 2 + 1);
        }
      }
    }
  }
  if (!FUSED || it.slot < 0) stamp(A, idx, 2);
  if constexpr (FUSED) {
    // Every wave of the workgroup takes part in the arrival (the pages
    // table is no longer read: its first entry holds the arrival's flag).
    if (it.slot >= 0) fused_arrive<D, kThreads<NG, TW, NL>>(A, idx, it.node, &sm.pages[0]);
    if (tid == 0) sm.next_item = next_item;
  }
}

// The partition kernel. Two-launch call: one workgroup per work item.
// Single-launch call (FUSED): a persistent grid of at most the device's
// resident workgroups; workgroup w runs item w, then the items it takes in
// turn from the counter A.work[0] (item gridDim.x + the count), until the
// list is exhausted. No workgroup waits for another, so the grid need not
// all be resident. Each workgroup ends by adding one to A.work[1]; the
// last one resets both counters, as every workgroup has then made its last
// fetch, so the next call (or graph replay) starts from zero.
template <int D, bool FP8, int NG, int TW, int NL, int OCC, bool CL, bool FUSED>
__global__ __launch_bounds__((kThreads<NG, TW, NL>), 1) void pa_partition_kernel(KernelArgs A) {
  using SM = Smem<D, FP8, NG, TW, OCC>;
  static_assert(OCC == 1 || sizeof(SM) <= 80 * 1024, "two workgroups share a CU's LDS");
  __shared__ SM sm;
  if constexpr (!FUSED) {
    partition_item<D, FP8, NG, TW, NL, OCC, CL, false>(A, sm, blockIdx.x);
  } else {
    int idx = blockIdx.x;
    while (idx < A.n_items) {  // uniform over the workgroup
      partition_item<D, FP8, NG, TW, NL, OCC, CL, true>(A, sm, idx);
      // Every wave is done with the item's LDS (and reads the next index)
      // before the next item's loads and page table overwrite it.
      __syncthreads();
      idx = sm.next_item;
    }
    if (threadIdx.x == 0) {
      const int done =
          __hip_atomic_fetch_add(A.work + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (done == (int)gridDim.x - 1) {
        __hip_atomic_store(A.work, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(A.work + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
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
template <int D, int COLS, int PARTS, int U>
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
  // then they are folded in order (PARTS x U covers the few-partials shape
  // in one batch).
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

// The same merge for pairs with few partials (at most 32): one thread per
// (row, four columns) folds every partial of its row in index order, with
// the loads of up to U partials in flight at once; a workgroup covers RB
// consecutive rows of one pair across all D columns, so each wave reads
// whole rows of a partial (contiguous 512-byte runs at D 128) and no thread
// waits on another. Grid: (reduce item, block of RB rows). For many split
// pairs this launches a fraction of the workgroups of one per row (16,384
// on a mixed batch of 256 split pairs with a 64-row stride, where the merge
// was mostly latency).
//
// STAGE1: the first level of the two-level merge (plans with more than 512
// partials in some pair). The item is then one chunk of a pair's partials
// (slot_base, n_parts), and the thread writes the chunk's merged partial
// (O relative to its maximum, the maximum, the sum: the partition kernel's
// format) to slot out_slot of the first-level scratch instead of the
// output.
template <int D, int RB, int U, bool STAGE1>
__global__ __launch_bounds__(RB * D / 4) void pa_reduce_rows_kernel(KernelArgs A) {
  constexpr int COLS = D / 4;
  const int nblk = (A.rows_stride + RB - 1) / RB;
  const ReduceItem ri = A.red[blockIdx.x / nblk];
  const int row = (blockIdx.x % nblk) * RB + (int)threadIdx.x / COLS;
  const int G = A.group, Hq = A.num_q_heads;
  if (row >= ri.q_len * G) return;  // no barrier follows
  const int d = ((int)threadIdx.x % COLS) * 4;
  const int n = ri.n_parts;
  const float* ml = A.part_ml + ((int64_t)ri.slot_base * A.rows_stride + row) * 2;
  const float* po = A.part_o + ((int64_t)ri.slot_base * A.rows_stride + row) * D + d;
  const int64_t mstride = (int64_t)A.rows_stride * 2;
  const int64_t ostride = (int64_t)A.rows_stride * D;

  float M = -INFINITY, z = 0.f;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < n; k0 += U) {
    float2 v[U];
    f32x4 o[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = k0 + u;
      v[u] = make_float2(-INFINITY, 0.f);
      o[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (k < n) {
        v[u] = *reinterpret_cast<const float2*>(ml + k * mstride);
        o[u] = *reinterpret_cast<const f32x4*>(po + k * ostride);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // m = -inf: no key of that item is visible to the row.
      const float Mn = fmaxf(M, v[u].x);
      const float a = (M == -INFINITY) ? 0.f : fast_exp2(M - Mn);
      const float wk = (v[u].x == -INFINITY) ? 0.f : fast_exp2(v[u].x - Mn);
      acc = acc * a + o[u] * wk;
      z = z * a + v[u].y * wk;
      M = Mn;
    }
  }
  if constexpr (STAGE1) {
    const int64_t pr = (int64_t)ri.out_slot * A.rows_stride + row;
    *reinterpret_cast<f32x4*>(A.l1_o + pr * D + d) = acc;
    if (d == 0) *reinterpret_cast<float2*>(A.l1_ml + pr * 2) = make_float2(M, z);
    return;
  }
  const int i = row / G, hh = row % G;
  const int h = ri.kv_head * G + hh;
  const float zs = sink_log2(A, ri.seq, h);
  const float Mx = fmaxf(M, zs);
  const float a = (M == -INFINITY) ? 0.f : fast_exp2(M - Mx);
  const float Z = z * a + ((zs == -INFINITY) ? 0.f : fast_exp2(zs - Mx));
  store_out<D, false>(A, ((int64_t)(ri.q_off + i) * Hq + h) * D + d, acc * (a / Z));
}

// One template instance per (head dim, KV dtype, layout, occupancy). With
// timing events the launch carries them itself (hipExtLaunchKernelGGL), so
// they take the kernel's own start and end timestamps, as a kernel trace
// does, rather than those of marker packets around its dispatch.
template <int D, bool FP8, int NG, int TW, int NL, int OCC, bool CL, bool FUSED>
static void launch_fx(const KernelArgs& a, int n_items, hipStream_t stream, hipEvent_t ev_start,
                      hipEvent_t ev_stop) {
  // The single-launch call's persistent grid: at most the resident
  // workgroups (a.grid, from the plan), at most the items.
  if (FUSED) n_items = n_items < a.grid ? n_items : a.grid;
  if (ev_start && ev_stop)
    hipExtLaunchKernelGGL((pa_partition_kernel<D, FP8, NG, TW, NL, OCC, CL, FUSED>),
                          dim3(n_items), dim3(kThreads<NG, TW, NL>), 0, stream, ev_start, ev_stop,
                          0, a);
  else
    hipLaunchKernelGGL((pa_partition_kernel<D, FP8, NG, TW, NL, OCC, CL, FUSED>), dim3(n_items),
                       dim3(kThreads<NG, TW, NL>), 0, stream, a);
}
template <int D, bool FP8, int NG, int TW, int NL, int OCC, bool CL>
static void launch_one(const KernelArgs& a, int n_items, hipStream_t stream, hipEvent_t ev_start,
                       hipEvent_t ev_stop, bool fused) {
  if (fused)
    launch_fx<D, FP8, NG, TW, NL, OCC, CL, true>(a, n_items, stream, ev_start, ev_stop);
  else
    launch_fx<D, FP8, NG, TW, NL, OCC, CL, false>(a, n_items, stream, ev_start, ev_stop);
}

hipError_t launch_partition(const KernelArgs& a, int n_items, int head_dim, bool fp8, int ntmax,
                            int occ, hipStream_t stream, hipEvent_t ev_start,
                            hipEvent_t ev_stop, bool fused) {
  if (n_items <= 0) return hipSuccess;
  if (ntmax < 1 || (occ != 1 && occ != 2)) return hipErrorInvalidValue;
  if (head_dim == 256) {  // FP8 KV only, at most 48 rows; one workgroup per CU
    if (!fp8 || ntmax > 3) return hipErrorInvalidValue;
    launch_one<256, true, 2, 3, 1, 1, false>(a, n_items, stream, ev_start, ev_stop, fused);
    return hipGetLastError();
  }
  if (ntmax > 4) return hipErrorInvalidValue;
  if (fp8 && occ != 1) return hipErrorInvalidValue;  // FP8 runs one workgroup per CU
  const hipEvent_t e0 = ev_start, e1 = ev_stop;
  if (head_dim == 128) {
    if (fp8 && ntmax <= 3)
      launch_one<128, true, 4, 3, 1, 1, false>(a, n_items, stream, e0, e1, fused);
    else if (fp8) launch_one<128, true, 3, 4, 1, 1, false>(a, n_items, stream, e0, e1, fused);
    else if (occ == 1)
      launch_one<128, false, 2, 4, 1, 1, false>(a, n_items, stream, e0, e1, fused);
    else if (ntmax <= 3)
      launch_one<128, false, 1, 3, 1, 2, false>(a, n_items, stream, e0, e1, fused);
    else launch_one<128, false, 1, 4, 1, 2, false>(a, n_items, stream, e0, e1, fused);
  } else {
    if (fp8) launch_one<64, true, 2, 4, 1, 1, false>(a, n_items, stream, e0, e1, fused);
    else if (occ == 1)
      launch_one<64, false, 2, 4, 1, 1, false>(a, n_items, stream, e0, e1, fused);
    else if (ntmax <= 3)
      launch_one<64, false, 1, 3, 1, 2, false>(a, n_items, stream, e0, e1, fused);
    else launch_one<64, false, 1, 4, 1, 2, false>(a, n_items, stream, e0, e1, fused);
  }
  return hipGetLastError();
}

hipError_t launch_reduce_stage1(const KernelArgs& a, int n_chunks, int head_dim, int rows_stride,
                                hipStream_t stream) {
  if (n_chunks <= 0) return hipSuccess;
  const unsigned blocks =
      (unsigned)n_chunks * ((rows_stride + 1024 / head_dim - 1) / (1024 / head_dim));
  if (head_dim == 256)
    hipLaunchKernelGGL((pa_reduce_rows_kernel<256, 4, 16, true>),
                       dim3(blocks), dim3(256), 0, stream, a);
  else if (head_dim == 128)
    hipLaunchKernelGGL((pa_reduce_rows_kernel<128, 8, 16, true>),
                       dim3(blocks), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((pa_reduce_rows_kernel<64, 16, 16, true>),
                       dim3(blocks), dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_reduce(const KernelArgs& a, int n_red, int head_dim, int rows_stride,
                         int max_parts, hipStream_t stream) {
  if (n_red <= 0) return hipSuccess;
  const unsigned items = (unsigned)n_red * rows_stride;
  if (max_parts <= 32 && items >= 2048) {
    // Many split pairs: 256 threads = RB rows x D / 4 column lanes, 16
    // partials in flight per thread. (With few pairs, e.g. 16 pairs of 48
    // rows, this makes too few workgroups to pull the partials quickly,
    // and the one-row shape below with its partition lanes is faster.)
    const unsigned rb = 1024 / head_dim;  // rows per workgroup
    const unsigned blocks = (unsigned)n_red * ((rows_stride + rb - 1) / rb);
    if (head_dim == 256)
      hipLaunchKernelGGL((pa_reduce_rows_kernel<256, 4, 16, false>),
                         dim3(blocks), dim3(256), 0, stream, a);
    else if (head_dim == 128)
      hipLaunchKernelGGL((pa_reduce_rows_kernel<128, 8, 16, false>),
                         dim3(blocks), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((pa_reduce_rows_kernel<64, 16, 16, false>),
                         dim3(blocks), dim3(256), 0, stream, a);
  } else if (max_parts <= 32) {
    // One row: 32 (D 128, 256) or 16 column lanes x 4 or 8 partition lanes.
    if (head_dim == 256)  // half a row per workgroup
      hipLaunchKernelGGL((pa_reduce_kernel<256, 32, 4, 8>), dim3(items * 2), dim3(128), 0, stream,
                         a);
    else if (head_dim == 128)
      hipLaunchKernelGGL((pa_reduce_kernel<128, 32, 4, 8>), dim3(items), dim3(128), 0, stream, a);
    else
      hipLaunchKernelGGL((pa_reduce_kernel<64, 16, 8, 4>), dim3(items), dim3(128), 0, stream, a);
  } else {  // 8 column lanes x 32 partition lanes per eighth, quarter or half of a row
    if (head_dim == 256)
      hipLaunchKernelGGL((pa_reduce_kernel<256, 8, 32, 4>), dim3(items * 8), dim3(256), 0, stream,
                         a);
    else if (head_dim == 128)
      hipLaunchKernelGGL((pa_reduce_kernel<128, 8, 32, 4>), dim3(items * 4), dim3(256), 0, stream,
                         a);
    else
      hipLaunchKernelGGL((pa_reduce_kernel<64, 8, 32, 4>), dim3(items * 2), dim3(256), 0, stream,
                         a);
  }
  return hipGetLastError();
}

}  // namespace pav
