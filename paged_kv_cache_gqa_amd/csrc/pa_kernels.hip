// pa_kernels.hip -- gfx950 (MI355X, CDNA4) kernels for causal GQA attention over a
// paged KV cache: planner, persistent P/D/V attention kernel, log-sum-exp merge,
// page-walk gather and content validation.
//
// What is computed: XY-Serve verdict page, pith_extraction.key_machinery (the
// attention primitive is matmul-softmax-matmul over a tile of query rows and a
// K/V length) and core_discovery (prefill, decode and verify rows in one batch
// over a PagedAttention-style block cache; tiles the causal mask empties are
// skipped; FlashAttention-style tiling).  Grouped-query attention: query heads
// h of one group read K/V head h / (Hq/Hkv) ("Understanding Inference Scaling
// for LLMs" review, Reference graph [4]).
//
// Design for CDNA4 (what differs from the Ascend design on the XY-Serve page):
//  * A chunk is 32 keys = two 16-slot pages.  QK^T runs as S^T = K . Q^T on
//    v_mfma_f32_16x16x32_bf16 (16 keys x 16 query rows per MFMA, D in steps of
//    32) and PV as O^T = V^T . P^T (16 d x 16 rows, 32 keys per MFMA).  K pages
//    are [slot][D], V pages are stored [D][slot] so the key axis that PV reduces
//    over is contiguous; nothing is transposed on chip.
//  * QK MFMA half h takes its 16 key rows from page h of the chunk.  After the
//    C-layout write-back lane (row n, quad q) holds the scores of keys
//    4q..4q+3 of both pages; those 8 values are exactly the lane's B operand of
//    the PV MFMA (element j = key 16*(j/4) + 4q + j%4), so softmax needs no
//    cross-lane data movement beyond two lane swaps for the row statistics.
//  * Rows are (window token, head in group) pairs, so the G query heads that
//    share a K/V head -- and all tokens of a verify window or prefill block --
//    read each K/V byte once.
//  * One persistent launch of (#CU x workgroups per CU) workgroups walks a
//    work list laid on one cost axis cut into equal grains (stream-K style); a
//    grain can span several units and split a unit's keys, in which case it
//    writes partial (o, lse) rows that the merge kernel combines.  Split points
//    depend only on the batch shape, so results are bitwise reproducible.
//  * Decode/verify units (<= 32 rows) let the 4 waves take alternate chunks and
//    merge in LDS.  Each wave keeps one chunk in flight: V straight to
//    registers, K (bf16) by global->LDS DMA into the wave's own slot.  Prefill
//    units (<= 64 rows; <= 128 in the kernel for prefill-heavy bf16 batches)
//    give each wave 16 (32) rows; the 4 waves DMA the 4 page blocks of a chunk
//    into a ring of LDS slots shared by all of them (XOR-swizzled rows, so the
//    MFMA fragment reads are conflict-free).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pa_internal.h"

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

__device__ __forceinline__ u32x4_t ld16(const char* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// Read-only kernel inputs (plan, block table, lengths) are read through the
// constant address space: the attention kernel never writes them, and uniform
// reads then become scalar loads that do not wait behind in-flight K/V loads.
template <typename T>
using cptr = const __attribute__((address_space(4))) T*;
template <typename T>
__device__ __forceinline__ cptr<T> ro(const T* p) { return (cptr<T>)p; }


__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ f32x4_t as_f32x4(u32x4_t v) { return __builtin_bit_cast(f32x4_t, v); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  // one v_cvt_pk_bf16_f32 (round to nearest even): a in the low half, b in the high half
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Maxima of scores and running maxima (never NaN, -inf for masked keys): NaN-propagating maxima,
// which gfx950 does in one v_maximum3_f32 for up to three operands.  fmaxf would first quiet
// possible signalling NaNs in every operand the compiler cannot prove canonical -- MFMA results
// and cross-lane moves -- at one extra instruction per operand.
__device__ __forceinline__ float max2(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max3(float a, float b, float c) { return max2(max2(a, b), c); }

// Reductions over the 4 lanes (one per quad) that hold the same query row: a
// butterfly over lane ^ 32 and lane ^ 16 with the gfx950 permlane swaps.
__device__ __forceinline__ float quad_max(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = max2(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max2(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float quad_sum(float v) {
  auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Inclusive sum of one int64 per lane over a wave (lane l gets lanes 0..l) in DPP moves: shifts by
// 1, 2, 4, 8 within each 16-lane row (lanes shifted in from outside the row read 0), then lane 15
// broadcast into rows 1 and 3 and lane 31 into rows 2 and 3 -- the classic GCN wave scan, without
// the LDS round trips of ds_bpermute shuffles.  The 64-bit value moves as two 32-bit halves.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ int64_t dpp_add64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_update_dpp(0u, uint32_t(uint64_t(x)), kCtrl, kRowMask, 0xF, true);
  const uint32_t hi = __builtin_amdgcn_update_dpp(0u, uint32_t(uint64_t(x) >> 32), kCtrl, kRowMask, 0xF, true);
  return x + int64_t((uint64_t(hi) << 32) | lo);
}
__device__ __forceinline__ int64_t wave_incl_scan64(int64_t x) {
  x = dpp_add64<0x111, 0xF>(x);  // row_shr:1
  x = dpp_add64<0x112, 0xF>(x);  // row_shr:2
  x = dpp_add64<0x114, 0xF>(x);  // row_shr:4
  x = dpp_add64<0x118, 0xF>(x);  // row_shr:8
  x = dpp_add64<0x142, 0xA>(x);  // row_bcast:15 into rows 1, 3
  x = dpp_add64<0x143, 0xC>(x);  // row_bcast:31 into rows 2, 3
  return x;
}

// The running maximum that P is scaled against is only moved when a row's new
// maximum exceeds it by more than this many powers of two; in between, P may
// reach 2^kLazy (exact for the sums, same relative precision for bf16 P).
constexpr float kLazy = 8.0f;

// Chunk-relative key of element j (0..7) of the P operand held by a lane of quad q:
// QK half j/4 read page j/4, and the C layout gives the lane MFMA rows 4q..4q+3.
__device__ __forceinline__ int p_key(int j, int quad) { return 16 * (j >> 2) + 4 * quad + (j & 3); }

__device__ __forceinline__ uint2 ld8(const char* p) { return *reinterpret_cast<const uint2*>(p); }

// LDS reads that follow a global->LDS DMA still in flight.  The compiler treats every LDS read as
// possibly aliasing every DMA in flight (all LDS is one object to it) and would wait for all of
// them; these reads are written as inline asm that completes its own reads (s_waitcnt lgkmcnt(0)
// inside the block), and the DMA data they need is waited for explicitly (vmcnt + barrier).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return uint32_t(uintptr_t((const __attribute__((address_space(3))) char*)p));
}
__device__ __forceinline__ void lds_read4_b128(const uint32_t (&a)[4], u32x4_t& r0, u32x4_t& r1, u32x4_t& r2,
                                               u32x4_t& r3) {
  asm volatile(
      "ds_read_b128 %0, %4\n"
      "ds_read_b128 %1, %5\n"
      "ds_read_b128 %2, %6\n"
      "ds_read_b128 %3, %7\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
}
__device__ __forceinline__ void lds_read2_b128(uint32_t a0, uint32_t a1, u32x4_t& r0, u32x4_t& r1) {
  asm volatile(
      "ds_read_b128 %0, %2\n"
      "ds_read_b128 %1, %3\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1)
      : "v"(a0), "v"(a1));
}
__device__ __forceinline__ void lds_read4_b64(const uint32_t (&a)[4], u32x2_t& r0, u32x2_t& r1, u32x2_t& r2,
                                              u32x2_t& r3) {
  asm volatile(
      "ds_read_b64 %0, %4\n"
      "ds_read_b64 %1, %5\n"
      "ds_read_b64 %2, %6\n"
      "ds_read_b64 %3, %7\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
}
__device__ __forceinline__ void lds_read4_b32(const uint32_t (&a)[4], uint32_t& r0, uint32_t& r1, uint32_t& r2,
                                              uint32_t& r3) {
  asm volatile(
      "ds_read_b32 %0, %4\n"
      "ds_read_b32 %1, %5\n"
      "ds_read_b32 %2, %6\n"
      "ds_read_b32 %3, %7\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]));
}
// Four 16-byte reads at a[i] + kOff (kOff an immediate byte offset below 64 KiB).
template <int kOff>
__device__ __forceinline__ void lds_read4_b128_at(const uint32_t (&a)[4], u32x4_t& r0, u32x4_t& r1, u32x4_t& r2,
                                                  u32x4_t& r3) {
  static_assert(kOff >= 0 && kOff < 65536, "ds offset field");
  asm volatile(
      "ds_read_b128 %0, %4 offset:%8\n"
      "ds_read_b128 %1, %5 offset:%8\n"
      "ds_read_b128 %2, %6 offset:%8\n"
      "ds_read_b128 %3, %7 offset:%8\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r0), "=&v"(r1), "=&v"(r2), "=&v"(r3)
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "i"(kOff));
}
// 16-byte LDS write that the compiler does not order behind DMAs in flight (the data it writes
// does not overlap any DMA target; LDS operations of one wave execute in issue order).
__device__ __forceinline__ void lds_write_b128(uint32_t a, u32x4_t v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_write_b64(uint32_t a, u32x2_t v) {
  asm volatile("ds_write_b64 %0, %1" ::"v"(a), "v"(v) : "memory");
}
// N 16-byte reads (N even), in blocks of four and two.
template <int N>
__device__ __forceinline__ void lds_read_b128(const uint32_t (&a)[N], u32x4_t (&r)[N]) {
  static_assert(N % 2 == 0, "even count");
#pragma unroll
  for (int i = 0; i + 4 <= N; i += 4) {
    const uint32_t b[4] = {a[i], a[i + 1], a[i + 2], a[i + 3]};
    lds_read4_b128(b, r[i], r[i + 1], r[i + 2], r[i + 3]);
  }
  if constexpr (N % 4 == 2) lds_read2_b128(a[N - 2], a[N - 1], r[N - 2], r[N - 1]);
}

// ---------------------------------------------------------------------------
// Element types.  A "fragment" is the 16 bytes one lane feeds to one MFMA
// operand slot (bf16: 8 values; fp32: 4 values).
// ---------------------------------------------------------------------------

// V fragments of a bf16 chunk in the LDS ring (head dim D): 2 * D / 16 8-byte reads from one base
// address, pages at byte 2 * 32 D and 3 * 32 D of the slot, tile t at + 512 t.
#define PA_V8(P, B, T) "ds_read_b64 %" #P ", %" #B " offset:" #T "\n"
template <int D>
__device__ __forceinline__ void lds_read_v_imm(uint32_t base, u32x4_t* vf);
template <>
__device__ __forceinline__ void lds_read_v_imm<128>(uint32_t base, u32x4_t* vf) {
  u32x2_t x[16];
  asm volatile(PA_V8(0, 16, 8192) PA_V8(1, 16, 12288) PA_V8(2, 16, 8704) PA_V8(3, 16, 12800)
               PA_V8(4, 16, 9216) PA_V8(5, 16, 13312) PA_V8(6, 16, 9728) PA_V8(7, 16, 13824)
               PA_V8(8, 16, 10240) PA_V8(9, 16, 14336) PA_V8(10, 16, 10752) PA_V8(11, 16, 14848)
               PA_V8(12, 16, 11264) PA_V8(13, 16, 15360) PA_V8(14, 16, 11776) PA_V8(15, 16, 15872)
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]),
                 "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]), "=&v"(x[12]), "=&v"(x[13]),
                 "=&v"(x[14]), "=&v"(x[15])
               : "v"(base));
#pragma unroll
  for (int t = 0; t < 8; ++t) vf[t] = u32x4_t{x[2 * t][0], x[2 * t][1], x[2 * t + 1][0], x[2 * t + 1][1]};
}
template <>
__device__ __forceinline__ void lds_read_v_imm<64>(uint32_t base, u32x4_t* vf) {
  u32x2_t x[8];
  asm volatile(PA_V8(0, 8, 4096) PA_V8(1, 8, 6144) PA_V8(2, 8, 4608) PA_V8(3, 8, 6656)
               PA_V8(4, 8, 5120) PA_V8(5, 8, 7168) PA_V8(6, 8, 5632) PA_V8(7, 8, 7680) "s_waitcnt lgkmcnt(0)"
               : "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]),
                 "=&v"(x[7])
               : "v"(base));
#pragma unroll
  for (int t = 0; t < 4; ++t) vf[t] = u32x4_t{x[2 * t][0], x[2 * t][1], x[2 * t + 1][0], x[2 * t + 1][1]};
}

// K fragments of chunk slot `ks` and V fragments of slot `vs` of the row-split ring (bf16 pages) in
// one LDS round trip: K page 0 rows at the four swizzled column addresses ka[kk] (page 1 at
// +kBlk), V^T rows from one per-lane base with immediate offsets (pages at 2 and 3 kBlk, tile t at
// +512 t).
#define PA_K16(P, A, O) "ds_read_b128 %" #P ", %" #A " offset:" #O "\n"
template <int D>
__device__ __forceinline__ void lds_read_kv_imm(const uint32_t (&ka)[D / 32], uint32_t vbase, u32x4_t* kf, u32x4_t* vf);
template <>
__device__ __forceinline__ void lds_read_kv_imm<128>(const uint32_t (&ka)[4], uint32_t vbase, u32x4_t* kf, u32x4_t* vf) {
  u32x2_t x[16];
  asm volatile(PA_K16(0, 24, 0) PA_K16(1, 25, 0) PA_K16(2, 26, 0) PA_K16(3, 27, 0)
               PA_K16(4, 24, 4096) PA_K16(5, 25, 4096) PA_K16(6, 26, 4096) PA_K16(7, 27, 4096)
               PA_V8(8, 28, 8192) PA_V8(9, 28, 12288) PA_V8(10, 28, 8704) PA_V8(11, 28, 12800)
               PA_V8(12, 28, 9216) PA_V8(13, 28, 13312) PA_V8(14, 28, 9728) PA_V8(15, 28, 13824)
               PA_V8(16, 28, 10240) PA_V8(17, 28, 14336) PA_V8(18, 28, 10752) PA_V8(19, 28, 14848)
               PA_V8(20, 28, 11264) PA_V8(21, 28, 15360) PA_V8(22, 28, 11776) PA_V8(23, 28, 15872)
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3]), "=&v"(kf[4]), "=&v"(kf[5]), "=&v"(kf[6]),
                 "=&v"(kf[7]), "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]), "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]),
                 "=&v"(x[6]), "=&v"(x[7]), "=&v"(x[8]), "=&v"(x[9]), "=&v"(x[10]), "=&v"(x[11]), "=&v"(x[12]),
                 "=&v"(x[13]), "=&v"(x[14]), "=&v"(x[15])
               : "v"(ka[0]), "v"(ka[1]), "v"(ka[2]), "v"(ka[3]), "v"(vbase));
#pragma unroll
  for (int t = 0; t < 8; ++t) vf[t] = u32x4_t{x[2 * t][0], x[2 * t][1], x[2 * t + 1][0], x[2 * t + 1][1]};
}
template <>
__device__ __forceinline__ void lds_read_kv_imm<64>(const uint32_t (&ka)[2], uint32_t vbase, u32x4_t* kf, u32x4_t* vf) {
  u32x2_t x[8];
  asm volatile(PA_K16(0, 12, 0) PA_K16(1, 13, 0) PA_K16(2, 12, 2048) PA_K16(3, 13, 2048)
               PA_V8(4, 14, 4096) PA_V8(5, 14, 6144) PA_V8(6, 14, 4608) PA_V8(7, 14, 6656)
               PA_V8(8, 14, 5120) PA_V8(9, 14, 7168) PA_V8(10, 14, 5632) PA_V8(11, 14, 7680)
               "s_waitcnt lgkmcnt(0)"
               : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3]), "=&v"(x[0]), "=&v"(x[1]), "=&v"(x[2]),
                 "=&v"(x[3]), "=&v"(x[4]), "=&v"(x[5]), "=&v"(x[6]), "=&v"(x[7])
               : "v"(ka[0]), "v"(ka[1]), "v"(vbase));
#pragma unroll
  for (int t = 0; t < 4; ++t) vf[t] = u32x4_t{x[2 * t][0], x[2 * t][1], x[2 * t + 1][0], x[2 * t + 1][1]};
}
#undef PA_K16
#undef PA_V8

template <int D_>
struct Bf16 {
  static constexpr int D = D_;
  static constexpr int kEb = 2;
  static constexpr int kQF = D / 32;        // Q fragments per 16-row tile
  static constexpr int kKF = 2 * (D / 32);  // K fragments per chunk (2 pages x D/32)
  static constexpr int kVF = D / 16;        // V fragments per chunk (one per 16-wide d tile)
  static constexpr int kNF = kKF + kVF;
  static constexpr int kTiles = D / 16;
  static constexpr bool kBf16 = true;
  static constexpr int kVLoads = 2 * kVF;  // global load instructions per chunk of V (two pages per tile)
  static constexpr int kEbKV = kEb;        // bytes per K/V pool element
  static constexpr bool kScaled = false;   // per-(page, head) K/V scales
  static constexpr bool kPrior = false;  // final outputs fold in a result over other keys (WithPrior)
  static constexpr int kRowTiles = 1;  // 16-row tiles of each wave in a row-split unit
  static constexpr int kRowGeom = row_geom(kCostRowSplit, kRowTiles);  // the planner's row-split geometry
  using VRaw = u32x4_t;                    // a V fragment as loaded

  __device__ static int q_off(int f, int quad) { return (32 * f + 8 * quad) * kEb; }
  // lane offsets within a (page, head) block: K row = lane%16, d = 8*quad (+32*kk)
  __device__ static uint32_t k_lane(int lane) { return uint32_t(((lane & 15) * D + 8 * (lane >> 4)) * kEb); }
  // V^T row d = lane%16 (+16*t), slots 4*quad .. 4*quad+3
  __device__ static uint32_t v_lane(int lane) { return uint32_t(((lane & 15) * kPage + 4 * (lane >> 4)) * kEb); }
  // fragment f: page and byte offset (K: f = page*(D/32) + kk; V: f = kKF + t, two 8-byte halves)
  __device__ static u32x4_t load_frag(const char* k0, const char* k1, const char* v0, const char* v1, uint32_t kl,
                                      uint32_t vl, int f) {
    if (f < kKF) return ld16((f < D / 32 ? k0 : k1) + kl + (f % (D / 32)) * 32 * kEb);
    const int t = f - kKF;
    const uint2 a = ld8(v0 + vl + t * 16 * kPage * kEb);
    const uint2 b = ld8(v1 + vl + t * 16 * kPage * kEb);
    return u32x4_t{a.x, a.y, b.x, b.y};
  }
  __device__ static VRaw load_v_raw(const char* v0, const char* v1, uint32_t vl, int g) {
    return load_frag(nullptr, nullptr, v0, v1, 0u, vl, kKF + g);
  }
  __device__ static u32x4_t v_convert(const VRaw& r) { return r; }
  // acc0: the accumulators' start value (zero, or minus the rows' score offsets)
  __device__ static f32x4_t qk(const u32x4_t* kf, int h, const u32x4_t* qf,
                               f32x4_t acc0 = f32x4_t{0.f, 0.f, 0.f, 0.f}) {
    f32x4_t acc = acc0;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[h * (D / 32) + kk]), as_bf16x8(qf[kk]), acc, 0, 0, 0);
    return acc;
  }
  // zero V elements whose chunk-relative key is >= n_valid
  __device__ static void sanitize_v(u32x4_t* vf, int quad, int n_valid) {
    uint32_t keep[4];
#pragma unroll
    for (int w = 0; w < 4; ++w)
      keep[w] = (p_key(2 * w, quad) < n_valid ? 0x0000FFFFu : 0u) | (p_key(2 * w + 1, quad) < n_valid ? 0xFFFF0000u : 0u);
#pragma unroll
    for (int t = 0; t < kVF; ++t)
#pragma unroll
      for (int w = 0; w < 4; ++w) vf[t][w] &= keep[w];
  }
  struct PFrag { u32x4_t v; };
  __device__ static PFrag make_p(const float (&p)[8]) {
    PFrag r;
    r.v[0] = pack_bf16x2(p[0], p[1]);
    r.v[1] = pack_bf16x2(p[2], p[3]);
    r.v[2] = pack_bf16x2(p[4], p[5]);
    r.v[3] = pack_bf16x2(p[6], p[7]);
    return r;
  }
  __device__ static f32x4_t pv(const u32x4_t* vf, int t, const PFrag& p, f32x4_t acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vf[t]), as_bf16x8(p.v), acc, 0, 0, 0);
  }
  // K and V fragments of a chunk held in LDS (block images of Ring<Bf16<D>>: K page 0, K page 1,
  // V page 0, V page 1, rows XOR-swizzled by 16-byte column)
  template <class RG>
  __device__ static void lds_read_k(const char* slot, int lane, u32x4_t (&kf)[kKF]) {
    const int m = lane & 15, quad = lane >> 4;
    if constexpr (D == 128) {
      // page 1's block sits kBlk bytes after page 0's: the same four addresses, an immediate offset
      uint32_t a[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) a[kk] = lds_addr(slot + m * RG::kPitchK + RG::swz_k(m, 4 * kk + quad) * 16);
      lds_read4_b128_at<0>(a, kf[0], kf[1], kf[2], kf[3]);
      lds_read4_b128_at<RG::kBlk>(a, kf[4], kf[5], kf[6], kf[7]);
    } else {
      uint32_t a[kKF];
#pragma unroll
      for (int f = 0; f < kKF; ++f) {
        const int h = f / (D / 32), kk = f % (D / 32);
        a[f] = lds_addr(slot + h * RG::kBlk + m * RG::kPitchK + RG::swz_k(m, 4 * kk + quad) * 16);
      }
      lds_read_b128<kKF>(a, kf);
    }
  }
  template <class RG>
  __device__ static void lds_read_v(const char* slot, int lane, u32x4_t (&vf)[kVF]) {
    const int m = lane & 15, quad = lane >> 4;
    if constexpr (RG::kPitchV == 32 && RG::kBlk == 32 * D) {
      // V^T row d = 16 t + m sits at d * 32 bytes with the same swizzled column for every t, so
      // the 2 * kVF addresses are one per-lane base plus immediate offsets (page 0 at 2 * kBlk,
      // page 1 at 3 * kBlk, tile t at + 512 t), all read under one wait.
      const uint32_t base = lds_addr(slot + m * RG::kPitchV + RG::swz_v(m, quad >> 1) * 16 + 8 * (quad & 1));
      lds_read_v_imm<D>(base, vf);
      return;
    }
#pragma unroll
    for (int t0 = 0; t0 < kVF; t0 += 2) {
      uint32_t a[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int d = 16 * (t0 + i) + m;
        const int off = d * RG::kPitchV + RG::swz_v(d, quad >> 1) * 16 + 8 * (quad & 1);
        a[2 * i] = lds_addr(slot + 2 * RG::kBlk + off);
        a[2 * i + 1] = lds_addr(slot + 3 * RG::kBlk + off);
      }
      u32x2_t x0, x1, x2, x3;
      lds_read4_b64(a, x0, x1, x2, x3);
      vf[t0] = u32x4_t{x0[0], x0[1], x1[0], x1[1]};
      vf[t0 + 1] = u32x4_t{x2[0], x2[1], x3[0], x3[1]};
    }
  }
  // K of ring slot `ks` and V of slot `vs` in one LDS round trip where the geometry allows it
  template <class RG>
  __device__ static void lds_read_kv(const char* ks, const char* vs, int lane, u32x4_t (&kf)[kKF],
                                     u32x4_t (&vf)[kVF]) {
    if constexpr (RG::kPitchV == 32 && RG::kBlk == 32 * D) {
      const int m = lane & 15, quad = lane >> 4;
      uint32_t ka[D / 32];
#pragma unroll
      for (int kk = 0; kk < D / 32; ++kk) ka[kk] = lds_addr(ks + m * RG::kPitchK + RG::swz_k(m, 4 * kk + quad) * 16);
      const uint32_t vbase = lds_addr(vs + m * RG::kPitchV + RG::swz_v(m, quad >> 1) * 16 + 8 * (quad & 1));
      lds_read_kv_imm<D>(ka, vbase, kf, vf);
    } else {
      lds_read_k<RG>(ks, lane, kf);
      lds_read_v<RG>(vs, lane, vf);
    }
  }
  __device__ static void store_out(char* dst, f32x4_t o) {  // 4 consecutive d
    uint2 v;
    v.x = pack_bf16x2(o[0], o[1]);
    v.y = pack_bf16x2(o[2], o[3]);
    *reinterpret_cast<uint2*>(dst) = v;
  }
};

// bf16 pages with 128-row row-split units (two 16-row tiles per wave), for batches with a lot of
// prefill work; a 128-row chunk step weighs twice a 64-row one on the cost axis.
template <int D_>
struct Bf16Tall : Bf16<D_> {
  static constexpr int kRowTiles = 2;
  static constexpr int kRowGeom = row_geom(2 * kCostRowSplit, kRowTiles);
};

template <int D_>
struct F32 {
  static constexpr int D = D_;
  static constexpr int kEb = 4;
  static constexpr int kQF = D / 16;
  static constexpr int kKF = 2 * (D / 16);
  static constexpr int kVF = 2 * (D / 16);  // per d tile: page 0 keys 4q..4q+3, page 1 keys 4q..4q+3
  static constexpr int kNF = kKF + kVF;
  static constexpr int kTiles = D / 16;
  static constexpr bool kBf16 = false;
  static constexpr int kVLoads = kVF;
  static constexpr int kEbKV = kEb;
  static constexpr bool kScaled = false;
  static constexpr bool kPrior = false;
  static constexpr int kRowTiles = 1;
  static constexpr int kRowGeom = row_geom(kCostRowSplit, kRowTiles);
  using VRaw = u32x4_t;

  __device__ static int q_off(int f, int quad) { return (16 * f + 4 * quad) * kEb; }
  __device__ static uint32_t k_lane(int lane) { return uint32_t(((lane & 15) * D + 4 * (lane >> 4)) * kEb); }
  __device__ static uint32_t v_lane(int lane) { return uint32_t(((lane & 15) * kPage + 4 * (lane >> 4)) * kEb); }
  __device__ static u32x4_t load_frag(const char* k0, const char* k1, const char* v0, const char* v1, uint32_t kl,
                                      uint32_t vl, int f) {
    if (f < kKF) return ld16((f < D / 16 ? k0 : k1) + kl + (f % (D / 16)) * 16 * kEb);
    const int g = f - kKF;
    return ld16(((g & 1) ? v1 : v0) + vl + (g >> 1) * 16 * kPage * kEb);
  }
  __device__ static VRaw load_v_raw(const char* v0, const char* v1, uint32_t vl, int g) {
    return load_frag(nullptr, nullptr, v0, v1, 0u, vl, kKF + g);
  }
  __device__ static u32x4_t v_convert(const VRaw& r) { return r; }
  __device__ static f32x4_t qk(const u32x4_t* kf, int h, const u32x4_t* qf) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int jj = 0; jj < D / 16; ++jj) {
      const f32x4_t a = as_f32x4(kf[h * (D / 16) + jj]);
      const f32x4_t b = as_f32x4(qf[jj]);
#pragma unroll
      for (int c = 0; c < 4; ++c) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a[c], b[c], acc, 0, 0, 0);
    }
    return acc;
  }
  __device__ static void sanitize_v(u32x4_t* vf, int quad, int n_valid) {
#pragma unroll
    for (int f = 0; f < kVF; ++f)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        if (p_key(4 * (f & 1) + c, quad) >= n_valid) vf[f][c] = 0u;
  }
  struct PFrag { float p[8]; };
  __device__ static PFrag make_p(const float (&p)[8]) {
    PFrag r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r.p[j] = p[j];
    return r;
  }
  __device__ static f32x4_t pv(const u32x4_t* vf, int t, const PFrag& p, f32x4_t acc) {
#pragma unroll
    for (int j = 0; j < 8; ++j)
      acc = __builtin_amdgcn_mfma_f32_16x16x4f32(as_f32x4(vf[2 * t + (j >> 2)])[j & 3], p.p[j], acc, 0, 0, 0);
    return acc;
  }
  template <class RG>
  __device__ static void lds_read_k(const char* slot, int lane, u32x4_t (&kf)[kKF]) {
    const int m = lane & 15, quad = lane >> 4;
    uint32_t a[kKF];
#pragma unroll
    for (int f = 0; f < kKF; ++f) {
      const int h = f / (D / 16), jj = f % (D / 16);
      a[f] = lds_addr(slot + h * RG::kBlk + m * RG::kPitchK + RG::swz_k(m, 4 * jj + quad) * 16);
    }
    lds_read_b128<kKF>(a, kf);
  }
  template <class RG>
  __device__ static void lds_read_v(const char* slot, int lane, u32x4_t (&vf)[kVF]) {
    const int m = lane & 15, quad = lane >> 4;
    uint32_t a[kVF];
#pragma unroll
    for (int g = 0; g < kVF; ++g) {
      const int t = g >> 1, h = g & 1;
      const int d = 16 * t + m;
      a[g] = lds_addr(slot + (2 + h) * RG::kBlk + d * RG::kPitchV + RG::swz_v(d, quad) * 16);
    }
    lds_read_b128<kVF>(a, vf);
  }
  template <class RG>
  __device__ static void lds_read_kv(const char* ks, const char* vs, int lane, u32x4_t (&kf)[kKF],
                                     u32x4_t (&vf)[kVF]) {
    lds_read_k<RG>(ks, lane, kf);
    lds_read_v<RG>(vs, lane, vf);
  }
  __device__ static void store_out(char* dst, f32x4_t o) { *reinterpret_cast<f32x4_t*>(dst) = o; }
};

// OCP FP8 E4M3 -> bf16, four values (exact: every E4M3 value is a bf16 value), two per
// v_cvt_scalef32_pk_bf16_fp8 with scale 1.  A probe over all 256 codes on MI355X gave the same bits
// as v_cvt_pk_f32_fp8 followed by v_cvt_pk_bf16_f32 (NaN codes: NaN both ways), in half the
// instructions.
__device__ __forceinline__ uint2 fp8x4_to_bf16x4(uint32_t x) {
  const auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);  // bytes 0, 1
  const auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true);   // bytes 2, 3
  return uint2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
}
__device__ __forceinline__ u32x4_t fp8x8_to_bf16x8(u32x2_t x) {
  const uint2 lo = fp8x4_to_bf16x4(x[0]), hi = fp8x4_to_bf16x4(x[1]);
  return u32x4_t{lo.x, lo.y, hi.x, hi.y};
}
__device__ __forceinline__ uint32_t ld4(const char* p) { return *reinterpret_cast<const uint32_t*>(p); }

// FP8 KV pages: K/V pools hold OCP FP8 E4M3 codes with one fp32 scale per (page, kv head) for K
// and for V; q and out are bf16.  Fragments are converted to bf16 (exactly) and go through the
// bf16 MFMAs; the K scale multiplies a page's scores, the V scale its P values.
template <int D_>
struct Fp8Kv {
  static constexpr int D = D_;
  static constexpr int kEb = 2;    // q, out: bf16
  static constexpr int kEbKV = 1;  // pools: one byte per element
  static constexpr int kQF = D / 32;
  static constexpr int kKF = 2 * (D / 32);
  static constexpr int kVF = D / 16;
  static constexpr int kNF = kKF + kVF;
  static constexpr int kTiles = D / 16;
  static constexpr bool kBf16 = true;
  static constexpr bool kScaled = true;
  static constexpr bool kPrior = false;
  static constexpr int kRowTiles = 1;
  static constexpr int kRowGeom = row_geom(kCostRowSplitFp8, kRowTiles);
  using VRaw = u32x2_t;  // 4 codes of page 0 (keys 4q..4q+3), 4 codes of page 1

  __device__ static int q_off(int f, int quad) { return (32 * f + 8 * quad) * kEb; }
  __device__ static uint32_t k_lane(int lane) { return uint32_t((lane & 15) * D + 8 * (lane >> 4)); }
  __device__ static uint32_t v_lane(int lane) { return uint32_t((lane & 15) * kPage + 4 * (lane >> 4)); }
  __device__ static u32x4_t v_convert(const VRaw& r) {
    const uint2 a = fp8x4_to_bf16x4(r[0]), b = fp8x4_to_bf16x4(r[1]);
    return u32x4_t{a.x, a.y, b.x, b.y};
  }
  // K comes through LDS only (the register path is not instantiated for this trait)
  __device__ static u32x4_t load_frag(const char*, const char*, const char*, const char*, uint32_t, uint32_t, int) {
    return u32x4_t{0u, 0u, 0u, 0u};
  }
  __device__ static f32x4_t qk(const u32x4_t* kf, int h, const u32x4_t* qf) { return Bf16<D>::qk(kf, h, qf); }
  __device__ static void sanitize_v(u32x4_t* vf, int quad, int n_valid) { Bf16<D>::sanitize_v(vf, quad, n_valid); }
  using PFrag = typename Bf16<D>::PFrag;
  __device__ static PFrag make_p(const float (&p)[8]) { return Bf16<D>::make_p(p); }
  __device__ static f32x4_t pv(const u32x4_t* vf, int t, const PFrag& p, f32x4_t acc) { return Bf16<D>::pv(vf, t, p, acc); }
  // fragments from the LDS block images of Ring<Fp8Kv<D>> (K rows of D bytes, XOR-swizzled by 16-byte
  // column; V^T rows of 16 bytes = one column per d)
  template <class RG>
  __device__ static void lds_read_k(const char* slot, int lane, u32x4_t (&kf)[kKF]) {
    const int m = lane & 15, quad = lane >> 4;
#pragma unroll
    for (int f0 = 0; f0 < kKF; f0 += 4) {
      uint32_t a[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int f = f0 + i, h = f / (D / 32), kk = f % (D / 32);
        a[i] = lds_addr(slot + h * RG::kBlk + m * RG::kPitchK + RG::swz_k(m, 2 * kk + (quad >> 1)) * 16 +
                        8 * (quad & 1));
      }
      u32x2_t x[4];
      lds_read4_b64(a, x[0], x[1], x[2], x[3]);
#pragma unroll
      for (int i = 0; i < 4; ++i) kf[f0 + i] = fp8x8_to_bf16x8(x[i]);
    }
  }
  template <class RG>
  __device__ static void lds_read_v(const char* slot, int lane, u32x4_t (&vf)[kVF]) {
    const int m = lane & 15, quad = lane >> 4;
#pragma unroll
    for (int t0 = 0; t0 < kVF; t0 += 2) {
      uint32_t a[4];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int d = 16 * (t0 + i) + m;
        a[2 * i] = lds_addr(slot + 2 * RG::kBlk + d * RG::kPitchV + 4 * quad);
        a[2 * i + 1] = lds_addr(slot + 3 * RG::kBlk + d * RG::kPitchV + 4 * quad);
      }
      uint32_t x0, x1, x2, x3;
      lds_read4_b32(a, x0, x1, x2, x3);
      vf[t0] = v_convert(VRaw{x0, x1});
      vf[t0 + 1] = v_convert(VRaw{x2, x3});
    }
  }
  template <class RG>
  __device__ static void lds_read_kv(const char* ks, const char* vs, int lane, u32x4_t (&kf)[kKF],
                                     u32x4_t (&vf)[kVF]) {
    lds_read_k<RG>(ks, lane, kf);
    lds_read_v<RG>(vs, lane, vf);
  }
  __device__ static void store_out(char* dst, f32x4_t o) { Bf16<D>::store_out(dst, o); }
};

// FP8 pages with 128-row row-split units, as Bf16Tall.  Their chunk weighs as much as a 64-row FP8
// chunk (8; measured on MI355X, 4 x 2048-token windows + 128 decodes, 32/8 heads: weight 4 / 8 / 16
// / 32 took 889 / 742 / 838 / 1398 us): widening K and V to bf16 costs the same for either height.
template <int D_>
struct Fp8KvTall : Fp8Kv<D_> {
  static constexpr int kRowTiles = 2;
  static constexpr int kRowGeom = row_geom(kCostRowSplitFp8, kRowTiles);
};

// A trait whose final outputs fold in a result over other keys of the same rows (AttnArgs::prior_o /
// prior_lse, log-sum-exp weights): the suffix pass of shared-prefix attention finishes its rows with
// the prefix pass's results this way instead of a separate merge launch.
template <class B>
struct WithPrior : B {
  static constexpr bool kPrior = true;
};

// (o, lse) over some keys of row `orow` and the prior result over the others -> the result over both.
// A side that saw no key (lse = -inf) has weight 0.
__device__ __forceinline__ void fold_prior(const float* prior_o, const float* prior_lse, int64_t orow, int D, int d,
                                           f32x4_t& o, float& lse) {
  const float lp = prior_lse[orow];
  if (lp == -INFINITY) return;
  const f32x4_t op = *reinterpret_cast<const f32x4_t*>(prior_o + orow * D + d);
  if (lse == -INFINITY) {
    o = op;
    lse = lp;
    return;
  }
  const float m = fmaxf(lse, lp);
  const float ws = fast_exp2((lse - m) * kLog2e), wp = fast_exp2((lp - m) * kLog2e);
  const float inv = 1.f / (ws + wp);
  o = (o * ws + op * wp) * inv;
  lse = m + fast_log2(ws + wp) * kLn2;
}

// ---------------------------------------------------------------------------
// Per-lane online-softmax state for RT tiles of 16 query rows.
// Lane (row n = lane%16, quad q) holds O^T[d = 16t + 4q + e][n] for every tile t.
// ---------------------------------------------------------------------------
template <class TR, int RT>
struct State {
  f32x4_t o[RT][TR::kTiles];
  float m[RT];  // running max of base-2 scores (identical in the 4 lanes of a row)
  float l[RT];  // this lane's share of the running sum of 2^(x - m)
};

template <class TR, int RT>
__device__ __forceinline__ void state_init(State<TR, RT>& st) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    st.m[rt] = -INFINITY;
    st.l[rt] = 0.f;
#pragma unroll
    for (int t = 0; t < TR::kTiles; ++t) st.o[rt][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
}

// Page bases of one chunk: K and V blocks of (page, kv head) for its two pages
// (page 1 aliases page 0 when the chunk's second page is past the sequence end).
struct ChunkPages {
  const char* k0;
  const char* k1;
  const char* v0;
  const char* v1;
};

// Physical pages of chunk c (scalar loads of the block table; page b = page a past the end).
struct PageIds {
  int a, b;
};
// The block-table loads of chunk c (every lane loads the same two entries) ...
__device__ __forceinline__ PageIds page_ids_load(cptr<int32_t> bt_row, int c, int n_seq) {
  // both loads unconditional (no wait at a branch join); the second index is clamped to the
  // sequence's last page, so it never reads past the pages the sequence owns: for a chunk that
  // holds keys (c * 32 < n_seq) it is 2c + 1 when that page starts before n_seq, else 2c (a
  // minimum, which stays in scalar registers)
  const int ib = min(2 * c + 1, (n_seq - 1) / kPage);
  return PageIds{bt_row[2 * c], bt_row[ib]};
}
// ... and their values as wave-uniform page ids (waits for the loads).
__device__ __forceinline__ PageIds uniform_ids(PageIds p) {
  return PageIds{__builtin_amdgcn_readfirstlane(p.a), __builtin_amdgcn_readfirstlane(p.b)};
}
__device__ __forceinline__ PageIds page_ids(cptr<int32_t> bt_row, int c, int n_seq) {
  return uniform_ids(page_ids_load(bt_row, c, n_seq));
}

template <class TR>
__device__ __forceinline__ ChunkPages pages_of(const AttnArgs& A, int kvh, PageIds p) {
  const int64_t blk = int64_t(kPage) * TR::D * TR::kEbKV;  // bytes of one (page, head) block
  const int64_t hkv = A.plan.num_kv_heads;
  ChunkPages cp;
  cp.k0 = static_cast<const char*>(A.k_pool) + (int64_t(p.a) * hkv + kvh) * blk;
  cp.k1 = static_cast<const char*>(A.k_pool) + (int64_t(p.b) * hkv + kvh) * blk;
  cp.v0 = static_cast<const char*>(A.v_pool) + (int64_t(p.a) * hkv + kvh) * blk;
  cp.v1 = static_cast<const char*>(A.v_pool) + (int64_t(p.b) * hkv + kvh) * blk;
  return cp;
}

template <class TR>
__device__ __forceinline__ ChunkPages chunk_pages(const AttnArgs& A, cptr<int32_t> bt_row, int kvh, int c,
                                                  int n_seq) {
  return pages_of<TR>(A, kvh, page_ids(bt_row, c, n_seq));
}

template <class TR>
__device__ __forceinline__ u32x4_t frag(const ChunkPages& cp, uint32_t kl, uint32_t vl, int f) {
  return TR::load_frag(cp.k0, cp.k1, cp.v0, cp.v1, kl, vl, f);
}

template <class TR>
__device__ __forceinline__ void load_k(const ChunkPages& cp, uint32_t kl, uint32_t vl, u32x4_t (&kf)[TR::kKF]) {
#pragma unroll
  for (int f = 0; f < TR::kKF; ++f) kf[f] = frag<TR>(cp, kl, vl, f);
}
template <class TR>
__device__ __forceinline__ void load_v(const ChunkPages& cp, uint32_t vl, typename TR::VRaw (&vr)[TR::kVF]) {
#pragma unroll
  for (int f = 0; f < TR::kVF; ++f) vr[f] = TR::load_v_raw(cp.v0, cp.v1, vl, f);
}

// Per-(page, kv head) scales of one chunk (FP8 pages): lane l loads (k0, k1, v0, v1)[l & 3], the
// K and V scales of the chunk's two pages; read_scales broadcasts them once the load has landed.
struct ChunkScale {
  float k0, k1, v0, v1;
};
template <class TR>
__device__ __forceinline__ float load_scale_lane(const AttnArgs& A, int kvh, PageIds p, int lane) {
  if constexpr (!TR::kScaled) {
    return 0.f;
  } else {
    const int sel = lane & 3;
    const float* base = (sel & 2) ? A.v_scale : A.k_scale;
    return base[int64_t((sel & 1) ? p.b : p.a) * A.plan.num_kv_heads + kvh];
  }
}
template <class TR>
__device__ __forceinline__ ChunkScale read_scales(float v) {
  ChunkScale c{1.f, 1.f, 1.f, 1.f};
  if constexpr (TR::kScaled) {
    c.k0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    c.k1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 1));
    c.v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 2));
    c.v1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 3));
  }
  return c;
}

// Tree-structured verify windows: per row tile, the lane's row mask (bit k: window token k
// visible; all ones for rows of windows longer than 64 tokens) and the first window key.
template <int RT>
struct TreeMask {
  uint64_t m[RT];
  int win0;
};

// Masked keys of one row tile's 8 scores of a chunk (key0: the chunk's first key) set to -inf:
// keys past the row's position p_row, and with kTree window keys whose bit is clear in the row's
// tree mask.
template <int RT, bool kTree>
__device__ __forceinline__ void mask_scores(float (&x)[8], int p_row, int key0, const TreeMask<RT>& tm, int rt,
                                            int quad) {
  const int lim = p_row - key0;  // element j visible iff its key <= lim
  // tree rows: a window key k (>= 0) is visible only where bit k of the row's mask is set.
  // Written branch-free (bitwise & | on the conditions, the bit index clamped to 0..63): a
  // short-circuit form compiled to divergent branches that lost the score of visible keys.
  const uint32_t m_lo = uint32_t(tm.m[rt]), m_hi = uint32_t(tm.m[rt] >> 32);
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    bool vis = p_key(j, quad) <= lim;
    if constexpr (kTree) {
      const int k = key0 + p_key(j, quad) - tm.win0;  // window token index of the key
      const uint32_t kc = uint32_t(min(max(k, 0), 63));
      const uint32_t bit = ((kc < 32 ? m_lo : m_hi) >> (kc & 31)) & 1u;
      vis = vis & ((k < 0) | (bit != 0u));
    }
    x[j] = vis ? x[j] : -INFINITY;
  }
}

// Softmax of NC chunks in two phases.
//
// Phase 1 (softmax_prep): the raw scores s[j] (QK^T results of chunk j; half h holds the keys of
// page h) of every row tile, with the K scale applied and masked keys set to -inf, into x; and the
// running maxima moved where a score exceeds them by more than 2^kLazy.  The common path tests each
// lane's own scores only: a row's maximum exceeds the threshold iff one of the four lanes holding
// the row sees a score above it, so the cross-lane maximum (two lane swaps) is taken only on the
// rare path that moves a maximum.  The results are the same as with the row maximum taken first.
// kTree: keys of the window are also masked by the rows' tree masks.
template <class TR, int RT, int NC, bool kTree>
__device__ __forceinline__ void softmax_prep(State<TR, RT>& st, const f32x4_t (&s)[NC][RT][2], const int (&key0)[NC],
                                             const int (&p_row)[RT], const TreeMask<RT>& tm,
                                             const ChunkScale (&cs)[NC], const bool (&mask)[NC], float sl2, int lane,
                                             float (&x)[NC][RT][8]) {
  const int quad = lane >> 4;
  bool over = false;
  float lm[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {  // raw scores q.k; the positive factor scale*log2(e) is applied inside exp2
        x[c][rt][e] = s[c][rt][0][e];
        x[c][rt][4 + e] = s[c][rt][1][e];
      }
      if constexpr (TR::kScaled) {  // the K scale of each page multiplies its keys' scores
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          x[c][rt][e] *= cs[c].k0;
          x[c][rt][4 + e] *= cs[c].k1;
        }
      }
      if (mask[c]) mask_scores<RT, kTree>(x[c][rt], p_row[rt], key0[c], tm, rt, quad);
      const float cm = max3(max3(x[c][rt][0], x[c][rt][1], x[c][rt][2]), max3(x[c][rt][3], x[c][rt][4], x[c][rt][5]),
                            max2(x[c][rt][6], x[c][rt][7]));
      lm[rt] = c == 0 ? cm : max2(lm[rt], cm);
    }
    over |= lm[rt] * sl2 > st.m[rt] + kLazy;  // -inf * sl2 = -inf never passes (sl2 > 0)
  }
  if (__any(over)) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float mx = quad_max(lm[rt]);
      const float mx2 = mx == -INFINITY ? -INFINITY : mx * sl2;  // row maximum in the base-2 domain
      if (__any(mx2 > st.m[rt] + kLazy)) {
        const float m_new = max2(st.m[rt], mx2);
        const float alpha = fast_exp2(st.m[rt] - (m_new == -INFINITY ? 0.f : m_new));
        st.l[rt] *= alpha;
#pragma unroll
        for (int t = 0; t < TR::kTiles; ++t) st.o[rt][t] *= alpha;
        st.m[rt] = m_new;
      }
    }
  }
}

// Phase 2 (softmax_exp): P = 2^(x * sl2 - m) against the running maxima, its sum into l, and the
// P operands of the PV MFMAs (FP8 pages: P times the V scale of its page; l takes the unscaled P).
template <class TR, int RT, int NC>
__device__ __forceinline__ void softmax_exp(State<TR, RT>& st, const float (&x)[NC][RT][8],
                                            const ChunkScale (&cs)[NC], float sl2,
                                            typename TR::PFrag (&pf)[NC][RT]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float neg_m = st.m[rt] == -INFINITY ? 0.f : -st.m[rt];
    float sum = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        p[j] = fast_exp2(__builtin_fmaf(x[c][rt][j], sl2, neg_m));
        sum += p[j];
      }
      if constexpr (TR::kScaled) {  // the V scale of each page multiplies its P values (the sum l does not)
        float pv[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pv[j] = p[j] * cs[c].v0;
          pv[4 + j] = p[4 + j] * cs[c].v1;
        }
        pf[c][rt] = TR::make_p(pv);
      } else {
        pf[c][rt] = TR::make_p(p);
      }
    }
    st.l[rt] += sum;
  }
}

// The same softmax with each row's running maximum folded into the QK products (bf16 row-split
// units).  A row keeps its offset o in raw score units (q.k, before the factor sl2): the QK
// accumulation starts from -o, so the MFMA results are q.k - o, and the row's running maximum in
// the base-2 domain is m = o * sl2 (o = 0 and m = -inf before the row's first visible key).  The
// lazy-rescale test then compares the MFMA results with a per-row threshold in raw units
// (kLazy / sl2, or -inf while m is -inf) without arithmetic on them, and P = 2^((q.k - o) * sl2).
// Where m moves, the chunk's results are re-based by the offset's change; that is the rare path.
template <int RT>
struct ScoreBase {
  f32x4_t neg[RT];  // -o in all four elements: the QK accumulators' start value
  float thr[RT];    // a result above this moves the row's maximum
};

template <int RT>
__device__ __forceinline__ void score_base_init(ScoreBase<RT>& sb) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    sb.neg[rt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    sb.thr[rt] = -INFINITY;
  }
}

// thr_lazy: kLazy / sl2, the raw-unit threshold once a row has a finite maximum
template <class TR, int RT, int NC, bool kTree>
__device__ __forceinline__ void softmax_prep_based(State<TR, RT>& st, ScoreBase<RT>& sb,
                                                   const f32x4_t (&s)[NC][RT][2], const int (&key0)[NC],
                                                   const int (&p_row)[RT], const TreeMask<RT>& tm,
                                                   const bool (&mask)[NC], float sl2, float thr_lazy, int lane,
                                                   float (&x)[NC][RT][8]) {
  const int quad = lane >> 4;
  bool over = false;
  float lm[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int c = 0; c < NC; ++c) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[c][rt][e] = s[c][rt][0][e];
        x[c][rt][4 + e] = s[c][rt][1][e];
      }
      if (mask[c]) mask_scores<RT, kTree>(x[c][rt], p_row[rt], key0[c], tm, rt, quad);
      const float cm = max3(max3(x[c][rt][0], x[c][rt][1], x[c][rt][2]), max3(x[c][rt][3], x[c][rt][4], x[c][rt][5]),
                            max2(x[c][rt][6], x[c][rt][7]));
      lm[rt] = c == 0 ? cm : max2(lm[rt], cm);
    }
    over |= lm[rt] > sb.thr[rt];  // -inf never passes
  }
  if (__any(over)) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float mx = quad_max(lm[rt]);  // the row's largest result against its offset
      if (__any(mx > sb.thr[rt])) {
        const float o = -sb.neg[rt][0];
        // the new offset: the row's largest raw score where that exceeds the old maximum
        const bool moves = mx > 0.f || st.m[rt] == -INFINITY;
        const float o_new = mx == -INFINITY ? o : (moves ? mx + o : o);
        const float m_new = mx == -INFINITY && st.m[rt] == -INFINITY ? -INFINITY : o_new * sl2;
        const float alpha = fast_exp2(st.m[rt] - (m_new == -INFINITY ? 0.f : m_new));
        st.l[rt] *= alpha;
#pragma unroll
        for (int t = 0; t < TR::kTiles; ++t) st.o[rt][t] *= alpha;
        st.m[rt] = m_new;
        const float d = o - o_new;
#pragma unroll
        for (int c = 0; c < NC; ++c)
#pragma unroll
          for (int j = 0; j < 8; ++j) x[c][rt][j] += d;
        sb.neg[rt] = f32x4_t{-o_new, -o_new, -o_new, -o_new};
        sb.thr[rt] = m_new == -INFINITY ? -INFINITY : thr_lazy;
      }
    }
  }
}

template <class TR, int RT, int NC>
__device__ __forceinline__ void softmax_exp_based(State<TR, RT>& st, const float (&x)[NC][RT][8], float sl2,
                                                  typename TR::PFrag (&pf)[NC][RT]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float sum;
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) p[j] = fast_exp2(x[c][rt][j] * sl2);
      // a pairwise sum of the chunk's 8 values (no add of a zero start value)
      const float cs = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
      sum = c == 0 ? cs : sum + cs;
      pf[c][rt] = TR::make_p(p);
    }
    st.l[rt] += sum;
  }
}

// QK^T of one chunk for every row tile: s[rt][h] = scores of page h's keys for row tile rt.
// `getq(rt, qf)` fills the Q fragments of row tile rt (from registers or LDS).
template <class TR, int RT, class GetQ>
__device__ __forceinline__ void qk_chunk(GetQ getq, const u32x4_t (&kf)[TR::kKF], f32x4_t (&s)[RT][2]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    u32x4_t qf[TR::kQF];
    getq(rt, qf);
    s[rt][0] = TR::qk(kf, 0, qf);
    s[rt][1] = TR::qk(kf, 1, qf);
  }
}

// Scores of one chunk for every row tile, masked, folded into the online softmax: the P operands,
// with O rescaled by 2^(m_old - m_new) where a running maximum moved.
template <class TR, int RT, bool kTree, class GetQ>
__device__ __forceinline__ void softmax_chunk(State<TR, RT>& st, GetQ getq, const u32x4_t (&kf)[TR::kKF], int key0,
                                              const int (&p_row)[RT], const TreeMask<RT>& tm, const ChunkScale& cs,
                                              bool mask, float sl2, int lane, typename TR::PFrag (&pf)[RT]) {
  f32x4_t s[1][RT][2];
  qk_chunk<TR, RT>(getq, kf, s[0]);
  float x[1][RT][8];
  const int k0[1] = {key0};
  const ChunkScale c1[1] = {cs};
  const bool m1[1] = {mask};
  softmax_prep<TR, RT, 1, kTree>(st, s, k0, p_row, tm, c1, m1, sl2, lane, x);
  typename TR::PFrag p1[1][RT];
  softmax_exp<TR, RT, 1>(st, x, c1, sl2, p1);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) pf[rt] = p1[0][rt];
}

template <class TR, int RT>
__device__ __forceinline__ void pv_chunk(State<TR, RT>& st, const u32x4_t (&vf)[TR::kVF],
                                         const typename TR::PFrag (&pf)[RT]) {
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
    for (int t = 0; t < TR::kTiles; ++t) st.o[rt][t] = TR::pv(vf, t, pf[rt], st.o[rt][t]);
  }
}

// Where the rows of one unit go.
// One sequence's units: n keys, qn query tokens from row q0, G query heads per kv head.
struct SeqUnits {
  int n, qn, rows, nb;
  int q0;            // row of q / out of the sequence's first query token
  bool split;        // one key-split unit per kv head
  bool full;         // every row sees all n keys
  int64_t per_head;  // cost of one kv head's units
};

struct RowInfo {
  int tok;    // global query token (row of q / out), valid rows only
  int head;   // query head
  int p;      // last visible key (-1 for rows beyond the unit)
  bool valid;
};

__device__ __forceinline__ RowInfo row_info(const AttnArgs& A, const pa_plan_unit& U, int r, int n_seq, int q0,
                                            int qn) {
  RowInfo ri;
  ri.valid = r < U.n_rows;
  const int rr = U.row0 + (ri.valid ? r : 0);
  const int t = rr / A.plan.group;
  const int hh = rr - t * A.plan.group;
  ri.tok = q0 + t;
  ri.head = U.kv_head * A.plan.group + hh;
  ri.p = ri.valid ? (A.plan.full_rows ? n_seq - 1 : n_seq - qn + t) : -1;
  return ri;
}

// The tree masks of a unit's row tiles (rows of windows longer than 64 tokens: all ones) and the
// first key from which chunks need masking: the window start for a tree window, else the first
// row's diagonal.
template <int RT, bool kTree>
__device__ __forceinline__ int tree_setup(const AttnArgs& A, const RowInfo (&ri)[RT], int n_seq, int qn, int min_p,
                                          TreeMask<RT>& tm) {
  tm.win0 = n_seq - qn;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    tm.m[rt] = (kTree && qn <= 64 && ri[rt].valid) ? A.tree_mask[ri[rt].tok] : ~uint64_t(0);
    // The loads complete here, before the unit's first DMA: the waits for the DMAs count the loads
    // issued after them, and a mask load moved past a DMA would throw that count off.
    if constexpr (kTree) asm volatile("" ::"v"(tm.m[rt]));
  }
  return (kTree && qn <= 64) ? tm.win0 : min_p + 1;
}

// Q fragment of one row; for a negative scale the signs are flipped (exact), so that the
// factor applied to q.k is always |scale| * log2(e) > 0; for scale 0 the fragment is cleared
// (every score is then exactly 0) and the factor is 1.
template <class TR>
__device__ __forceinline__ u32x4_t load_q_frag(const AttnArgs& A, const RowInfo& ri, int f, int quad) {
  const char* base = static_cast<const char*>(A.q) + (int64_t(ri.tok) * A.num_q_heads + ri.head) * TR::D * TR::kEb;
  return ri.valid ? ((ld16(base + TR::q_off(f, quad)) & A.q_keep) ^ A.q_sign) : u32x4_t{0u, 0u, 0u, 0u};
}

// Final (normalised) output of one row tile's 4 d values at tile t (part < 0), or
// the same values as partial row r of partial position `part` (slot * 2 + 0/1).
// Partial results travel between workgroups of one launch that may sit on different XCDs (each
// with its own L2).  They are written and read with agent-coherent (sc1) buffer accesses, so no
// L2-wide write-back or invalidate is needed to hand them over.
constexpr int kCoherent = 16;  // cache-policy bits: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t flat_rsrc(const float* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(base), 0, 0x7fffffff, 0x00020000);
}
__device__ __forceinline__ void store_coherent(const float* base, uint32_t off, f32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), flat_rsrc(base), off, 0, kCoherent);
}
__device__ __forceinline__ void store_coherent(const float* base, uint32_t off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), flat_rsrc(base), off, 0, kCoherent);
}
__device__ __forceinline__ f32x4_t load_coherent4(const float* base, uint32_t off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(flat_rsrc(base), off, 0, kCoherent));
}
__device__ __forceinline__ float load_coherent(const float* base, uint32_t off) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(flat_rsrc(base), off, 0, kCoherent));
}

template <class TR>
__device__ __forceinline__ void emit(const AttnArgs& A, const RowInfo& ri, int r, int part, int t, int quad,
                                     f32x4_t o, float lse_nat, bool write_lse) {
  if (!ri.valid) return;
  const int d = 16 * t + 4 * quad;
  if (part < 0) {
    const int64_t elem = (int64_t(ri.tok) * A.num_q_heads + ri.head) * TR::D + d;
    if constexpr (TR::kPrior) fold_prior(A.prior_o, A.prior_lse, int64_t(ri.tok) * A.num_q_heads + ri.head, TR::D, d, o, lse_nat);
    if (A.out_f32) *reinterpret_cast<f32x4_t*>(A.out_f32 + elem) = o;  // cascade pass: fp32 result
    else TR::store_out(static_cast<char*>(A.out) + elem * TR::kEb, o);
    if (write_lse) A.lse[int64_t(ri.tok) * A.num_q_heads + ri.head] = lse_nat;
  } else {
    const uint32_t prow = uint32_t(part) * kPartRows + r;
    store_coherent(A.part_o, (prow * TR::D + d) * 4, o);
    if (write_lse) store_coherent(A.part_lse, prow * 4, lse_nat);
  }
}

// Geometry of the LDS ring that row-split units stream chunks through.  A
// chunk is four (page, head) blocks -- K page 0, K page 1, V page 0, V page 1 --
// copied by global->LDS DMA (wave w copies block w, 1 KiB per instruction).
// Each block's LDS image is a permutation of its 16-byte columns (XOR swizzle
// by row) so that the fragment reads are free of bank conflicts.
template <class TR>
struct Ring {
  static constexpr int kBlk = kPage * TR::D * TR::kEbKV;  // bytes of one (page, head) block
  static constexpr int kChunk = 4 * kBlk;
  static constexpr int kNB = 65536 / kChunk > 4 ? 4 : (65536 / kChunk < 2 ? 2 : 65536 / kChunk);  // ring slots
  static constexpr int kInstr = kBlk / 1024;  // DMA instructions per wave per chunk
  static constexpr int kPitchK = TR::D * TR::kEbKV;  // K row (slot) pitch
  static constexpr int kNCk = kPitchK / 16;
  static constexpr int kPitchV = kPage * TR::kEbKV;  // V^T row (d) pitch: 16, 32 or 64 bytes
  static constexpr int kNCv = kPitchV / 16;          // 1, 2 or 4 columns
  static constexpr int kShV = kNCv == 4 ? 2 : 3;     // rows per 256 bytes = 1 << kShV (swizzle period)
  static constexpr int kBytes = kNB * kChunk;
  // swizzled column of global column c in row r
  __device__ static int swz_k(int r, int c) { return c ^ (r & (kNCk - 1)); }
  __device__ static int swz_v(int r, int c) { return c ^ ((r >> kShV) & (kNCv - 1)); }
};

// LDS: the row-split ring and the key-split Q slices / cross-wave merge buffer share one region.
template <class TR>
struct Smem {
  static constexpr int kMergeBytes = kWaves * 2 * TR::kTiles * 64 * 16;
  static constexpr int kBytes = Ring<TR>::kBytes > kMergeBytes ? Ring<TR>::kBytes : kMergeBytes;
  u32x4_t buf[kBytes / 16];
  float stat[kWaves][2][2][16];  // [wave][row tile][m | l][row]
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Global->LDS DMA of 16 bytes per lane from one (page, head) block: lane l writes LDS bytes
// [dst + 16 l, +16) from block byte `off`.  The MUBUF form (buffer_load ... lds) is used rather
// than the FLAT-global one: the compiler's wait analysis treats a FLAT instruction that touches
// two address spaces as completing out of order and then drains every load with vmcnt(0) at the
// next wait for a register load; with MUBUF its waits for the V register loads stay exact.
// The descriptor covers exactly one block (`bytes`), so an offset past it would read zeros.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_rsrc(const char* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), 0, int(bytes), 0x00020000);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t off, char* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, off, 0, 0, 0);
}

// s_waitcnt vmcnt(0) lgkmcnt(0): every load of this wave has landed.
// A compiler barrier for memory operations: loads, stores and DMAs are issued in program order
// across it.  The waits below count instructions in flight, so wherever they stand for a
// particular load having landed, the order of issue they count on is fixed with these.
__device__ __forceinline__ void issue_order() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ void wait_all_loads() {
  issue_order();
  __builtin_amdgcn_s_waitcnt(0x0070);
  issue_order();
}

// s_waitcnt vmcnt(N), leaving LDS / scalar loads (lgkmcnt) and expcnt unwaited.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  issue_order();
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
  issue_order();
}

// s_waitcnt lgkmcnt(0): this wave's LDS accesses written as inline asm are done; global loads and
// DMAs in flight are not waited for.
__device__ __forceinline__ void wait_lds() {
  issue_order();
  __builtin_amdgcn_s_waitcnt(0xC07F);
  issue_order();
}

// Workgroup barrier that orders LDS accesses for the compiler without waiting on global memory.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// Key-split unit (decode / verify, <= 32 rows): wave w takes chunks i0+w, i0+w+4, ...
// ---------------------------------------------------------------------------
template <class TR, int RT, bool kTree>
__device__ void run_keysplit(const AttnArgs& A, const pa_plan_unit& U, const SeqUnits& sq, int i0, int i1, int part,
                             Smem<TR>& sm) {
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));  // lane-derived values are recomputed per unit, not held across the unit loop
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int quad = lane >> 4;
  const int s = U.seq;
  const int n_seq = sq.n, q0 = sq.q0, qn = sq.qn;
  const cptr<int32_t> bt_row = ro(A.block_table) + int64_t(s) * A.max_pages +
                               (A.key_base ? ro(A.key_base)[s] / kPage : 0);

  RowInfo ri[RT];
  int p_row[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    ri[rt] = row_info(A, U, 16 * rt + (lane & 15), n_seq, q0, qn);
    p_row[rt] = ri[rt].p;
  }
  const int min_p = A.plan.full_rows ? n_seq - 1 : n_seq - qn + U.row0 / A.plan.group;  // first row's last key
  TreeMask<RT> tm;
  const int mask_from = tree_setup<RT, kTree>(A, ri, n_seq, qn, min_p, tm);

  // Q fragments live in this wave's slice of LDS (re-read every chunk; keeps VGPRs for K/V in flight).
  // Order of issue at a unit start: Q loads, then the first chunk's K/V loads, then the LDS copy of Q,
  // so the Q and K/V latencies overlap.
  u32x4_t* qlds = sm.buf + w * (RT * TR::kQF * 64);
  u32x4_t qtmp[RT][TR::kQF];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int f = 0; f < TR::kQF; ++f) qtmp[rt][f] = load_q_frag<TR>(A, ri[rt], f, quad);
  auto getq = [&](int rt, u32x4_t (&qf)[TR::kQF]) {
#pragma unroll
    for (int f = 0; f < TR::kQF; ++f) qf[f] = qlds[(rt * TR::kQF + f) * 64 + lane];
  };
  State<TR, RT> st;
  state_init(st);

  // A wave keeps one chunk (16 KiB for bf16, D = 128) of K/V in flight: measured on MI355X, two
  // chunks per wave streamed slower than one.  For bf16 the K half of a chunk travels by
  // global->LDS DMA into this wave's 2-page slot (contiguous 1 KiB per instruction; K fragments
  // read directly from the pool touch 16 rows x 64 B per instruction, which streams ~10% slower
  // at this occupancy) and V goes straight to registers (512 contiguous bytes per instruction).
  // FP8 pages move K and V by DMA into a 4-page slot: read straight from the pool, a V fragment
  // is 4 bytes per lane (16 instructions of 256 B per chunk against 4 DMA instructions of 1 KiB).
  // Every load is issued unconditionally: past the wave's last chunk it re-reads the chunk it has
  // (an L2 hit), so the number of loads in flight is the same on every path and the waits --
  // the compiler's for V, the explicit one for the K DMA -- are exact.
  using RG = Ring<TR>;
  constexpr bool kKviaLds = TR::kBf16;  // fp32 pages: K fragments straight to registers
  constexpr bool kVviaLds = TR::kScaled;  // FP8 pages: V by DMA too
  constexpr int kSlotBlocks = kVviaLds ? 4 : 2;  // (page, head) blocks of a wave's slot
  constexpr int kQRegion = kWaves * 2 * TR::kQF * 64;  // u32x4 slots of the Q slices (2 row tiles)
  static_assert(!kKviaLds || (kQRegion * 16 + kWaves * kSlotBlocks * RG::kBlk <= Smem<TR>::kBytes), "LDS budget");
  char* kslot = reinterpret_cast<char*>(sm.buf + kQRegion) + w * kSlotBlocks * RG::kBlk;
  const uint32_t kl = TR::k_lane(lane), vl = TR::v_lane(lane);
  auto dma_k = [&](char* slot, const ChunkPages& cp) {
    constexpr int kPer = RG::kBlk / 1024;  // DMA instructions per page
    const __amdgpu_buffer_rsrc_t r0 = block_rsrc(cp.k0, RG::kBlk), r1 = block_rsrc(cp.k1, RG::kBlk);
#pragma unroll
    for (int i = 0; i < 2 * kPer; ++i) {
      const int o = (i % kPer) * 1024 + 16 * lane;
      const int r = o / RG::kPitchK, cc = (o % RG::kPitchK) / 16;
      dma16(i < kPer ? r0 : r1, uint32_t(r * RG::kPitchK + RG::swz_k(r, cc) * 16),
            slot + (i / kPer) * RG::kBlk + (i % kPer) * 1024);
    }
  };
  const int c = i0 + w;
  u32x4_t kf[TR::kKF];
  const int mine = i1 > c ? (i1 - c + kWaves - 1) / kWaves : 0;  // chunks of this wave
  if constexpr (kVviaLds) {
    // FP8 pages: the slot holds K page 0, K page 1, V page 0, V page 1 (V^T rows of 16 codes, no
    // swizzle).  Each step waits for everything in flight (its chunk's scales, K and V), reads the
    // K and V fragments, then issues the next chunk's scales, K and V: they land during the whole
    // step's compute, with no count to keep.
    auto dma_v = [&](const ChunkPages& cp) {
      constexpr int kPer = RG::kBlk / 1024;
      const __amdgpu_buffer_rsrc_t r0 = block_rsrc(cp.v0, RG::kBlk), r1 = block_rsrc(cp.v1, RG::kBlk);
#pragma unroll
      for (int i = 0; i < 2 * kPer; ++i) {
        const int o = (i % kPer) * 1024 + 16 * lane;
        const int r = o / RG::kPitchV, cc = (o % RG::kPitchV) / 16;
        dma16(i < kPer ? r0 : r1, uint32_t(r * RG::kPitchV + RG::swz_v(r, cc) * 16),
              kslot + (2 + i / kPer) * RG::kBlk + (i % kPer) * 1024);
      }
    };
    // lane (m, quad), fragment t: the 4 codes of keys 4 quad .. 4 quad + 3 of both pages at d = 16 t + m
    auto read_v_raw = [&](typename TR::VRaw (&vr)[TR::kVF]) {
      const int m = lane & 15;
#pragma unroll
      for (int t0 = 0; t0 < TR::kVF; t0 += 2) {
        uint32_t a[4];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int d = 16 * (t0 + i) + m;
          a[2 * i] = lds_addr(kslot + 2 * RG::kBlk + d * RG::kPitchV + 4 * quad);
          a[2 * i + 1] = lds_addr(kslot + 3 * RG::kBlk + d * RG::kPitchV + 4 * quad);
        }
        uint32_t x0, x1, x2, x3;
        lds_read4_b32(a, x0, x1, x2, x3);
        vr[t0] = typename TR::VRaw{x0, x1};
        vr[t0 + 1] = typename TR::VRaw{x2, x3};
      }
    };
    PageIds cp_ids = page_ids(bt_row, c < i1 ? c : i0, n_seq);
    ChunkPages cp = pages_of<TR>(A, U.kv_head, cp_ids);
    float scl_cur = load_scale_lane<TR>(A, U.kv_head, cp_ids, lane);
    dma_k(kslot, cp);
    dma_v(cp);
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int f = 0; f < TR::kQF; ++f) lds_write_b128(lds_addr(qlds + (rt * TR::kQF + f) * 64 + lane), qtmp[rt][f]);
    PageIds nx = page_ids(bt_row, min(c + kWaves, i1 - 1), n_seq);
    auto getq_asm = [&](int rt, u32x4_t (&qf)[TR::kQF]) {
      uint32_t a[TR::kQF];
#pragma unroll
      for (int f = 0; f < TR::kQF; ++f) a[f] = lds_addr(qlds + (rt * TR::kQF + f) * 64 + lane);
      lds_read_b128<TR::kQF>(a, qf);
    };
    for (int j = 0; j < mine; ++j) {
      const int cc = c + j * kWaves;
      const int key0 = cc * kChunkKeys;
      const int cn = cc + kWaves;
      if (cn < i1) {
        cp_ids = nx;
        cp = pages_of<TR>(A, U.kv_head, nx);
      }
      wait_all_loads();  // this chunk's scales, K and V have landed (nothing else is in flight)
      TR::template lds_read_k<RG>(kslot, lane, kf);
      typename TR::VRaw vr[TR::kVF];
      read_v_raw(vr);  // both reads complete in place before the slot is refilled
      asm volatile("" ::: "memory");
      const float scl_nxt = load_scale_lane<TR>(A, U.kv_head, cp_ids, lane);
      dma_k(kslot, cp);
      dma_v(cp);
      typename TR::PFrag pf[RT];
      softmax_chunk<TR, RT, kTree>(st, getq_asm, kf, key0, p_row, tm, read_scales<TR>(scl_cur),
                                   key0 + kChunkKeys - 1 >= mask_from, A.scale_log2, lane, pf);
      asm volatile("" ::: "memory");
      scl_cur = scl_nxt;
      nx = page_ids(bt_row, min(cn + kWaves, i1 - 1), n_seq);
      u32x4_t vf[TR::kVF];
#pragma unroll
      for (int f = 0; f < TR::kVF; ++f) vf[f] = TR::v_convert(vr[f]);
      if (key0 + kChunkKeys > n_seq) TR::sanitize_v(vf, quad, n_seq - key0);  // the sequence's last chunk
      pv_chunk<TR, RT>(st, vf, pf);
    }
  } else {
  typename TR::VRaw vr[TR::kVF];
  PageIds cp_ids = page_ids(bt_row, c < i1 ? c : i0, n_seq);
  ChunkPages cp = pages_of<TR>(A, U.kv_head, cp_ids);
  // FP8 pages: each chunk's scales are loaded just before its K DMA (so only V follows the DMA)
  float scl_cur = load_scale_lane<TR>(A, U.kv_head, cp_ids, lane);
  if constexpr (kKviaLds) dma_k(kslot, cp);
  else load_k<TR>(cp, kl, vl, kf);
  issue_order();  // V after the K DMA: the loop's first wait for it counts on that order
  load_v<TR>(cp, vl, vr);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int f = 0; f < TR::kQF; ++f) {
      if constexpr (kKviaLds) lds_write_b128(lds_addr(qlds + (rt * TR::kQF + f) * 64 + lane), qtmp[rt][f]);
      else qlds[(rt * TR::kQF + f) * 64 + lane] = qtmp[rt][f];
    }

  // The loop body has a single path.  A step past the wave's last chunk is a dummy: all its keys
  // are masked and its V is zeroed, so it adds nothing.
  // Page ids are loaded one iteration before their DMA is issued, after the iteration's last LDS
  // read (those reads wait for every LDS and scalar load in flight).
  PageIds nx = page_ids(bt_row, min(c + kWaves, i1 - 1), n_seq);
  for (int j = 0; j < mine; ++j) {
    const int cc = c + j * kWaves;
    const int key0 = cc * kChunkKeys;
    const int cn = cc + kWaves;
    if (cn < i1) {
      cp_ids = nx;
      cp = pages_of<TR>(A, U.kv_head, nx);
    }
    typename TR::PFrag pf[RT];
    float scl_nxt = 0.f;
    if constexpr (kKviaLds) {
      wait_vmcnt<TR::kVLoads>();  // the K DMA of this chunk has landed (only V was issued after it)
      asm volatile("" ::: "memory");
      TR::template lds_read_k<RG>(kslot, lane, kf);  // completes before the slot is refilled
      asm volatile("" ::: "memory");
      scl_nxt = load_scale_lane<TR>(A, U.kv_head, cp_ids, lane);
      dma_k(kslot, cp);
      auto getq_asm = [&](int rt, u32x4_t (&qf)[TR::kQF]) {  // Q reads behind the DMA just issued
        uint32_t a[TR::kQF];
#pragma unroll
        for (int f = 0; f < TR::kQF; ++f) a[f] = lds_addr(qlds + (rt * TR::kQF + f) * 64 + lane);
        lds_read_b128<TR::kQF>(a, qf);
      };
      softmax_chunk<TR, RT, kTree>(st, getq_asm, kf, key0, p_row, tm, read_scales<TR>(scl_cur),
                                   key0 + kChunkKeys - 1 >= mask_from, A.scale_log2, lane, pf);
      asm volatile("" ::: "memory");
    } else {
      asm volatile("" ::: "memory");  // keep the Q reads inside the loop
      softmax_chunk<TR, RT, kTree>(st, getq, kf, key0, p_row, tm, read_scales<TR>(scl_cur),
                                   key0 + kChunkKeys - 1 >= mask_from, A.scale_log2, lane, pf);
      scl_nxt = load_scale_lane<TR>(A, U.kv_head, cp_ids, lane);
      load_k<TR>(cp, kl, vl, kf);
    }
    scl_cur = scl_nxt;
    nx = page_ids(bt_row, min(cn + kWaves, i1 - 1), n_seq);
    u32x4_t vf[TR::kVF];
#pragma unroll
    for (int f = 0; f < TR::kVF; ++f) vf[f] = TR::v_convert(vr[f]);
    if (key0 + kChunkKeys > n_seq) TR::sanitize_v(vf, quad, n_seq - key0);  // the sequence's last chunk
    pv_chunk<TR, RT>(st, vf, pf);
    load_v<TR>(cp, vl, vr);
  }
  }
  if constexpr (kKviaLds) wait_all_loads();  // the last (unused) DMA has landed before LDS is reused
  __syncthreads();  // every wave is done with its Q slice before the merge buffer overwrites it

  // merge the 4 waves' states through LDS
  f32x4_t* obuf = reinterpret_cast<f32x4_t*>(sm.buf);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const float l = quad_sum(st.l[rt]);
    if (quad == 0) {
      sm.stat[w][rt][0][lane] = st.m[rt];
      sm.stat[w][rt][1][lane] = l;
    }
#pragma unroll
    for (int t = 0; t < TR::kTiles; ++t) obuf[((w * 2 + rt) * TR::kTiles + t) * 64 + lane] = st.o[rt][t];
  }
  __syncthreads();
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    const int n = lane & 15;
    float mw[kWaves], M = -INFINITY;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      mw[i] = sm.stat[i][rt][0][n];
      M = fmaxf(M, mw[i]);
    }
    float sc[kWaves], L = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      sc[i] = mw[i] == -INFINITY ? 0.f : fast_exp2(mw[i] - M);
      L += sm.stat[i][rt][1][n] * sc[i];
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    const float lse_nat = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
    for (int t = w; t < TR::kTiles; t += kWaves) {
      f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < kWaves; ++i) o += obuf[((i * 2 + rt) * TR::kTiles + t) * 64 + lane] * sc[i];
      emit<TR>(A, ri[rt], 16 * rt + n, part, t, quad, o * inv, lse_nat, t == 0 && quad == 0);
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Row-split unit (prefill, <= 64 x kRowTiles rows): wave w owns rows [16 RT w, 16 RT (w + 1)).
// The workgroup streams chunks through an LDS ring with global->LDS DMA; every wave issues 1/4 of
// each chunk.  A step covers NP chunks (64 keys with one row tile per wave; 32 for fp32 pages at
// D = 128, whose chunks fill half the ring each, and with two row tiles, whose registers hold one
// chunk) under one barrier and one softmax pass, and the ring holds at least two steps: the next
// step's chunks land while this one is computed.
// ---------------------------------------------------------------------------
template <class TR, bool kTree>
__device__ void run_rowsplit(const AttnArgs& A, const pa_plan_unit& U, const SeqUnits& sq, int i0, int i1, int part,
                             Smem<TR>& sm) {
  using RG = Ring<TR>;
  constexpr int RT = TR::kRowTiles;
  constexpr int kWaveRows = 16 * RT;  // rows of each wave
  // chunks per step: two with one row tile per wave; one with two (their registers hold one chunk)
  constexpr int NP = RT == 1 ? RG::kNB / 2 : 1;
  static_assert(RG::kNB == 4 || RG::kNB == 2, "ring of two steps");
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));  // lane-derived values are recomputed per unit, not held across the unit loop
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int quad = lane >> 4;
  // wave-uniform values in scalar registers (the chunk loop's index and address arithmetic stays scalar)
  const int s = __builtin_amdgcn_readfirstlane(U.seq);
  const int n_seq = __builtin_amdgcn_readfirstlane(sq.n), q0 = sq.q0, qn = __builtin_amdgcn_readfirstlane(sq.qn);
  i0 = __builtin_amdgcn_readfirstlane(i0);
  i1 = __builtin_amdgcn_readfirstlane(i1);
  const int kvh = __builtin_amdgcn_readfirstlane(U.kv_head);
  const cptr<int32_t> bt_row = ro(A.block_table) + int64_t(s) * A.max_pages +
                               (A.key_base ? ro(A.key_base)[s] / kPage : 0);
  const bool active = kWaveRows * w < U.n_rows;

  RowInfo ri[RT];
  int p_row[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    ri[rt] = row_info(A, U, kWaveRows * w + 16 * rt + (lane & 15), n_seq, q0, qn);
    p_row[rt] = ri[rt].p;
  }
  const int min_p = A.plan.full_rows ? n_seq - 1 : n_seq - qn + (U.row0 + kWaveRows * w) / A.plan.group;
  TreeMask<RT> tm;
  const int mask_from = tree_setup<RT, kTree>(A, ri, n_seq, qn, min_p, tm);

  // Unit start: the page ids of the first two steps are loaded before Q, so that the first step's
  // DMAs wait for one round trip only and Q arrives behind them.
  PageIds ids0[RG::kNB];
#pragma unroll
  for (int j = 0; j < RG::kNB; ++j) ids0[j] = page_ids_load(bt_row, min(i0 + j, i1 - 1), n_seq);
  u32x4_t qreg[RT][TR::kQF];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int f = 0; f < TR::kQF; ++f) qreg[rt][f] = load_q_frag<TR>(A, ri[rt], f, quad);
  auto getq = [&](int rt, u32x4_t (&qf)[TR::kQF]) {
#pragma unroll
    for (int f = 0; f < TR::kQF; ++f) qf[f] = qreg[rt][f];
  };
  State<TR, RT> st;
  state_init(st);
  // bf16 pages: the running maxima folded into the QK products
  constexpr bool kBased = TR::kBf16 && !TR::kScaled;
  ScoreBase<RT> sb;
  score_base_init(sb);
  const float thr_lazy = kLazy / A.scale_log2;

  // Wave w copies the (page, kv head) block of K page 0, K page 1, V page 0 or V page 1 (w = 0..3):
  // its pool and head offset are fixed for the unit, the page changes per chunk.  Lane `lane` of DMA
  // instruction i fills LDS bytes [i*1024 + 16*lane, +16) of the block image (row r, swizzled column).
  char* ring = reinterpret_cast<char*>(sm.buf);
  const char* wave_pool = static_cast<const char*>(w < 2 ? A.k_pool : A.v_pool) + int64_t(kvh) * RG::kBlk;
  const int64_t page_stride = int64_t(A.plan.num_kv_heads) * RG::kBlk;
  uint32_t src[RG::kInstr];  // this lane's source offset within the block, per DMA instruction
#pragma unroll
  for (int i = 0; i < RG::kInstr; ++i) {
    const int o = i * 1024 + 16 * lane;
    if (w < 2) {
      const int r = o / RG::kPitchK, cc = (o % RG::kPitchK) / 16;
      src[i] = uint32_t(r * RG::kPitchK + RG::swz_k(r, cc) * 16);
    } else {
      const int r = o / RG::kPitchV, cc = (o % RG::kPitchV) / 16;
      src[i] = uint32_t(r * RG::kPitchV + RG::swz_v(r, cc) * 16);
    }
  }
  // FP8 pages: every wave loads a chunk's scales just before its DMAs (lane l: scale (l & 3) of it)
  auto issue = [&](PageIds ids, char* slot) -> float {
    const float sc = load_scale_lane<TR>(A, kvh, ids, lane);
    const int pg = (w & 1) ? ids.b : ids.a;
    const __amdgpu_buffer_rsrc_t rs = block_rsrc(wave_pool + int64_t(pg) * page_stride, RG::kBlk);
    char* dst = slot + w * RG::kBlk;
#pragma unroll
    for (int i = 0; i < RG::kInstr; ++i) dma16(rs, src[i], dst + i * 1024);
    return sc;
  };
  auto slot_of_chunk = [&](int c) { return ring + ((c - i0) & (RG::kNB - 1)) * RG::kChunk; };

  // prologue: the first step's chunks; the page ids of the second step are already loaded
  float scl[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) scl[j] = i0 + j < i1 ? issue(uniform_ids(ids0[j]), slot_of_chunk(i0 + j)) : 0.f;
  PageIds nx[NP];
#pragma unroll
  for (int j = 0; j < NP; ++j) nx[j] = uniform_ids(ids0[NP + j]);

  for (int c = i0; c < i1; c += NP) {
    wait_vmcnt<0>();  // this wave's share of the step's chunks has landed (nothing was issued after them)
    lds_barrier();    // ... every wave's share; every wave is done with the previous step's slots
    float scl_new[NP];
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      const int cn = c + NP + j;
      scl_new[j] = cn < i1 ? issue(nx[j], slot_of_chunk(cn)) : 0.f;
    }
    if (active) {
      // chunk j of the step: c + j, or (past the unit's end) a copy of chunk c whose keys are all
      // masked, so that it adds exactly nothing
      int key0[NP];
      bool msk[NP];
      ChunkScale cs[NP];
      f32x4_t sc[NP][RT][2];
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const bool real = c + j < i1;
        const int cj = real ? c + j : c;
        u32x4_t kf[TR::kKF];
        TR::template lds_read_k<RG>(slot_of_chunk(cj), lane, kf);
        // matrix work at a raised wave priority: of the two waves sharing a SIMD, the one ready to
        // issue MFMAs goes first while the other runs its softmax (tile 1-3% faster on three boxes)
        __builtin_amdgcn_s_setprio(1);
        if constexpr (kBased) {
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) {
            sc[j][rt][0] = TR::qk(kf, 0, qreg[rt], sb.neg[rt]);
            sc[j][rt][1] = TR::qk(kf, 1, qreg[rt], sb.neg[rt]);
          }
        } else {
          qk_chunk<TR, RT>(getq, kf, sc[j]);
        }
        __builtin_amdgcn_s_setprio(0);
        key0[j] = real ? cj * kChunkKeys : (1 << 29);
        msk[j] = !real || cj * kChunkKeys + kChunkKeys - 1 >= mask_from;
        cs[j] = read_scales<TR>(scl[j]);
      }
      float x[NP][RT][8];
      typename TR::PFrag pf[NP][RT];
      if constexpr (kBased) {
        softmax_prep_based<TR, RT, NP, kTree>(st, sb, sc, key0, p_row, tm, msk, A.scale_log2, thr_lazy, lane, x);
        softmax_exp_based<TR, RT, NP>(st, x, A.scale_log2, pf);
      } else {
        softmax_prep<TR, RT, NP, kTree>(st, sc, key0, p_row, tm, cs, msk, A.scale_log2, lane, x);
        softmax_exp<TR, RT, NP>(st, x, cs, A.scale_log2, pf);
      }
      // V after the scores, so that K and V fragments of the step are not live together
      u32x4_t vf[NP][TR::kVF];
#pragma unroll
      for (int j = 0; j < NP; ++j) TR::template lds_read_v<RG>(slot_of_chunk(c + j < i1 ? c + j : c), lane, vf[j]);
      asm volatile("" ::: "memory");
      // page ids of the step after next, after the step's last LDS read
#pragma unroll
      for (int j = 0; j < NP; ++j) nx[j] = page_ids_load(bt_row, min(c + 2 * NP + j, i1 - 1), n_seq);
#pragma unroll
      for (int j = 0; j < NP; ++j) {
        const int cj = c + j < i1 ? c + j : c;
        if (cj * kChunkKeys + kChunkKeys > n_seq) TR::sanitize_v(vf[j], quad, n_seq - cj * kChunkKeys);
      }
      // tile by tile, the step's chunks back to back into one accumulator (chunk by chunk, the
      // compiler wrote the second chunk's results beside the accumulators and copied them back)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int t = 0; t < TR::kTiles; ++t)
#pragma unroll
          for (int j = 0; j < NP; ++j) st.o[rt][t] = TR::pv(vf[j], t, pf[j][rt], st.o[rt][t]);
      __builtin_amdgcn_s_setprio(0);
    } else {
#pragma unroll
      for (int j = 0; j < NP; ++j) nx[j] = page_ids_load(bt_row, min(c + 2 * NP + j, i1 - 1), n_seq);
    }
#pragma unroll
    for (int j = 0; j < NP; ++j) {
      nx[j] = uniform_ids(nx[j]);
      scl[j] = scl_new[j];
    }
  }
  wait_all_loads();  // nothing of this unit left in flight
  lds_barrier();     // every wave is done with the ring before it is reused

  if (active) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float l = quad_sum(st.l[rt]);
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const float lse_nat = l > 0.f ? (st.m[rt] + fast_log2(l)) * kLn2 : -INFINITY;
#pragma unroll
      for (int t = 0; t < TR::kTiles; ++t)
        emit<TR>(A, ri[rt], kWaveRows * w + 16 * rt + (lane & 15), part, t, quad, st.o[rt][t] * inv, lse_nat,
                 t == 0 && quad == 0);
    }
  }
}

// slot_of(c): the slot whose slice [floor(k*C/S), floor((k+1)*C/S)) holds cost c
__device__ __forceinline__ int64_t slot_of(int64_t c, int64_t S, int64_t C) { return ((c + 1) * S - 1) / C; }
__device__ __forceinline__ int64_t slice_begin(int64_t k, int64_t S, int64_t C) { return k * C / S; }

// ---------------------------------------------------------------------------
// The plan.  Sequence s contributes Hkv groups of nb units (nb = 1 when its
// q_len * G rows fit one key-split unit, else ceil(rows / R) row blocks of R rows, R set by the
// kernel's row geometry);
// units are ordered (sequence, kv head, row block) on one cost axis.  Only the
// per-sequence cost prefix is stored; units are rebuilt from it on the fly.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// keys visible to the last row of row block rb (R rows per block) of a sequence (n keys, qn
// tokens, G heads; with full rows every row sees all n keys)
template <int R>
__device__ __forceinline__ int block_keys(int n, int qn, int G, int rb, bool full) {
  if (full) return n;
  const int rows = qn * G;
  const int last = (min(R * (rb + 1), rows) - 1) / G;
  return n - qn + last + 1;
}

// sum over i in [0, n) of floor((a * i + b) / m), for m > 0 and a * n + b + 2 * m < 2^32: split
// off the whole parts of a / m and b / m, then count the remaining lattice points under the line
// from the other axis (the Euclid-like reduction of floor sums; O(log m) rounds).
__device__ __forceinline__ int64_t floor_sum(uint32_t n, uint32_t m, uint32_t a, uint32_t b) {
  int64_t s = 0;
  while (n > 0) {
    if (a >= m) {
      s += int64_t(n) * int64_t(n - 1) / 2 * int64_t(a / m);
      a %= m;
    }
    if (b >= m) {
      s += int64_t(n) * int64_t(b / m);
      b %= m;
    }
    const uint32_t y = a * n + b;
    if (y < m) break;
    n = y / m;
    b = y % m;
    const uint32_t t = m;
    m = a;
    a = t;
  }
  return s;
}

// Chunks of row blocks 0 .. r-1 of a sequence, r < nb (none of them the last block).  With
// R rows per block, block rb's last row is token floor((R rb + R - 1) / G), so it sees
// keys(rb) = c + floor((R rb + R - 1) / G) keys, c = n - qn + 1, and ceil(keys / 32) =
// floor((R rb + G (c + 31) + R - 1) / (32 G)) (a floor of a floor is one floor of the product).
// That numerator's constant B splits into 32 G h + b with h = floor((c + 31 + floor((R - 1) / G))
// / 32) and 0 <= b < 32 G, which leaves a floor sum over rb with small coefficients.
template <int R>
__device__ __forceinline__ int64_t block_chunks_before(int n, int qn, int G, bool full, int r) {
  if (full) return int64_t(r) * ceil_div(n, kChunkKeys);
  const int x = n - qn + kChunkKeys;  // c + 31
  const int h = (x + (R - 1) / G) / kChunkKeys;
  const int b = G * (x - kChunkKeys * h) + R - 1;
  return int64_t(r) * h + floor_sum(uint32_t(r), uint32_t(kChunkKeys * G), R, uint32_t(b));
}

template <int kRg = kRgDefault>
__device__ SeqUnits seq_units(int n, int q0, int qn, int G, bool full) {
  SeqUnits q;
  q.n = n;
  q.q0 = q0;
  q.qn = qn;
  q.full = full;
  q.rows = qn > 0 ? qn * G : 0;
  q.split = q.rows <= kSplitRows;
  if (qn <= 0) {
    q.nb = 0;
    q.per_head = 0;
  } else if (q.split) {
    q.nb = 1;
    q.per_head = unit_start_cost(true, q.rows) + int64_t(ceil_div(n, kChunkKeys)) * kCostKeySplit;
  } else {
    q.nb = ceil_div(q.rows, rg_rows(kRg));
    // the last block's last row is the window's last token: it sees all n keys
    const int64_t ch = block_chunks_before<rg_rows(kRg)>(n, qn, G, full, q.nb - 1) + ceil_div(n, kChunkKeys);
    q.per_head = int64_t(q.nb) * kCostStartRow + ch * rg_weight(kRg);
  }
  return q;
}

// A unit occupies [cost0, cost0 + start + n_chunks * weight) on the cost axis (start: its fixed
// start cost); chunk i starts at cost0 + start + i * weight.
__device__ __forceinline__ int64_t unit_cost(const pa_plan_unit& U) {
  return unit_start_cost(U.kind == 0, U.n_rows) + int64_t(U.n_chunks) * U.cost_weight;
}
__device__ __forceinline__ int64_t chunk_start(const pa_plan_unit& U, int i) {
  return U.cost0 + unit_start_cost(U.kind == 0, U.n_rows) + int64_t(i) * U.cost_weight;
}

// Cost from the start of a kv head's row blocks to the start of block rb (rb < nb).
template <int kRg>
__device__ __forceinline__ int64_t block_start(const SeqUnits& q, int G, int rb) {
  return int64_t(rb) * kCostStartRow + block_chunks_before<rg_rows(kRg)>(q.n, q.qn, G, q.full, rb) * rg_weight(kRg);
}

template <int kRg>
__device__ pa_plan_unit make_unit(int s, const SeqUnits& q, int G, int g, int rb, int64_t cost0) {
  pa_plan_unit U;
  U.seq = s;
  U.kv_head = g;
  constexpr int R = rg_rows(kRg);
  U.row0 = q.split ? 0 : rb * R;
  U.n_rows = q.split ? q.rows : min(R, q.rows - rb * R);
  U.n_keys = q.split ? q.n : block_keys<R>(q.n, q.qn, G, rb, q.full);
  U.n_chunks = ceil_div(U.n_keys, kChunkKeys);
  U.kind = q.split ? 0 : 1;
  U.cost_weight = q.split ? kCostKeySplit : rg_weight(kRg);
  U.cost0 = cost0;
  U.first_slot = 0;
  U.n_pieces = 0;
  return U;
}

// Cursor over the units of the plan, in cost order.
struct UnitCursor {
  int s, g, rb;
  int64_t seq_base;  // cost at which sequence s starts
  SeqUnits q;
  pa_plan_unit U;
};

template <int kRg, class P>
__device__ void cursor_load_seq(UnitCursor& cu, const PlanView& v, P seq_lens, P qsl) {
  const int q0 = qsl[cu.s];
  cu.q = seq_units<kRg>(seq_lens[cu.s], q0, qsl[cu.s + 1] - q0, v.group, v.full_rows != 0);
}

// Position the cursor on the unit of sequence s (n keys, queries q0 .. q0 + qn - 1, starting at
// cost seq_base) whose cost range holds c.
template <int kRg>
__device__ void cursor_place(UnitCursor& cu, const PlanView& v, int s, int64_t seq_base, int n, int q0, int qn,
                             int64_t c) {
  cu.s = s;
  cu.seq_base = seq_base;
  cu.q = seq_units<kRg>(n, q0, qn, v.group, v.full_rows != 0);
  const int64_t off = c - cu.seq_base;
  cu.g = int(off / cu.q.per_head);
  int64_t acc = cu.seq_base + int64_t(cu.g) * cu.q.per_head;
  cu.rb = 0;
  if (!cu.q.split) {
    // the last row block whose start cost is <= c; start costs rise with rb
    int lo = 0, hi = cu.q.nb - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (acc + block_start<kRg>(cu.q, v.group, mid) <= c) lo = mid; else hi = mid - 1;
    }
    cu.rb = lo;
    acc += block_start<kRg>(cu.q, v.group, lo);
  }
  cu.U = make_unit<kRg>(cu.s, cu.q, v.group, cu.g, cu.rb, acc);
}

// cursor_place done by all 64 lanes of a wave together (every lane gets the same cursor): the
// row block is found by lanes evaluating 64 block starts at once and a ballot of which ones lie
// at or below c.  Up to 64 blocks: lane r takes block r's chunk count and a wave scan of the
// counts gives every start; more blocks: lanes evaluate floor-sum starts of 64 candidates per
// round (two rounds for up to 4096) -- instead of a serial binary search of floor sums.
template <int kRg>
__device__ void cursor_place_wave(UnitCursor& cu, const PlanView& v, int s, int64_t seq_base, int n, int q0, int qn,
                                  int64_t c, int lane) {
  cu.s = s;
  cu.seq_base = seq_base;
  cu.q = seq_units<kRg>(n, q0, qn, v.group, v.full_rows != 0);
  const int64_t off = c - cu.seq_base;
  cu.g = int(off / cu.q.per_head);
  int64_t acc = cu.seq_base + int64_t(cu.g) * cu.q.per_head;
  cu.rb = 0;
  if (!cu.q.split && cu.q.nb <= 64) {
    // one block per lane: its chunk count, and a wave scan of the counts gives every block's start
    const int64_t ch =
        lane < cu.q.nb ? ceil_div(block_keys<rg_rows(kRg)>(n, qn, v.group, lane, cu.q.full), kChunkKeys) : 0;
    const int64_t start = int64_t(lane) * kCostStartRow + (wave_incl_scan64(ch) - ch) * rg_weight(kRg);
    const uint64_t below = __ballot(lane < cu.q.nb && acc + start <= c);  // a prefix of the lanes
    const int rb = 63 - __builtin_clzll(below);
    cu.rb = rb;
    const uint64_t st = uint64_t(start);
    acc += int64_t((uint64_t(uint32_t(__builtin_amdgcn_readlane(int(uint32_t(st >> 32)), rb))) << 32) |
                   uint32_t(__builtin_amdgcn_readlane(int(uint32_t(st)), rb)));
  } else if (!cu.q.split) {
    int lo = 0, hi = cu.q.nb - 1;  // the block holding c lies in [lo, hi]; block lo starts at or below c
    while (lo < hi) {
      const int step = (hi - lo + 64) / 64;  // candidates lo, lo + step, ... cover [lo, hi]
      const int r = min(lo + lane * step, hi);
      const uint64_t below = __ballot(acc + block_start<kRg>(cu.q, v.group, r) <= c);  // a prefix of the lanes
      const int last = 63 - __builtin_clzll(below);
      const int r_last = min(lo + last * step, hi);
      hi = min(r_last + step - 1, hi);
      lo = r_last;
      if (step == 1) break;
    }
    cu.rb = lo;
    acc += block_start<kRg>(cu.q, v.group, lo);
  }
  cu.U = make_unit<kRg>(cu.s, cu.q, v.group, cu.g, cu.rb, acc);
}

// Position the cursor on the unit whose cost range holds c (0 <= c < total).
template <int kRg = kRgDefault, class P, class Q>
__device__ void cursor_find(UnitCursor& cu, const PlanView& v, P seq_lens, P qsl, Q seq_cost, int64_t c) {
  int lo = 0, hi = v.num_seqs - 1;  // last s with seq_cost[s] <= c
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (seq_cost[mid] <= c) lo = mid; else hi = mid - 1;
  }
  const int q0 = qsl[lo];
  cursor_place<kRg>(cu, v, lo, seq_cost[lo], seq_lens[lo], q0, qsl[lo + 1] - q0, c);
}

__device__ __forceinline__ SlotStart slot_from_cursor(const UnitCursor& cu, int64_t c0, int64_t c1) {
  SlotStart r;
  r.c0 = c0;
  r.c1 = c1;
  r.seq_base = cu.seq_base;
  r.unit_cost0 = cu.U.cost0;
  r.s = cu.s;
  r.g = cu.g;
  r.rb = cu.rb;
  r.n = cu.q.n;
  r.qn = cu.q.qn;
  r.q0 = cu.q.q0;
  r.pad[0] = r.pad[1] = 0;
  return r;
}

// Position the cursor as the planner recorded for one slot.
template <int kRg = kRgDefault>
__device__ __forceinline__ void cursor_from_slot(UnitCursor& cu, const PlanView& v, const SlotStart& st) {
  cu.s = st.s;
  cu.g = st.g;
  cu.rb = st.rb;
  cu.seq_base = st.seq_base;
  cu.q = seq_units<kRg>(st.n, st.q0, st.qn, v.group, v.full_rows != 0);
  cu.U = make_unit<kRg>(st.s, cu.q, v.group, st.g, st.rb, st.unit_cost0);
}

__device__ __forceinline__ SlotStart load_slot(cptr<SlotStart> p) {
  SlotStart r;
  r.c0 = p->c0;
  r.c1 = p->c1;
  r.seq_base = p->seq_base;
  r.unit_cost0 = p->unit_cost0;
  r.s = p->s;
  r.g = p->g;
  r.rb = p->rb;
  r.n = p->n;
  r.qn = p->qn;
  r.q0 = p->q0;
  return r;
}

// Advance to the next unit; returns false past the last one.
template <int kRg = kRgDefault, class P>
__device__ bool cursor_next(UnitCursor& cu, const PlanView& v, P seq_lens, P qsl) {
  const int64_t next_cost = cu.U.cost0 + unit_cost(cu.U);
  if (++cu.rb >= cu.q.nb) {
    cu.rb = 0;
    if (++cu.g >= v.num_kv_heads) {
      cu.g = 0;
      do {
        cu.seq_base += int64_t(v.num_kv_heads) * cu.q.per_head;
        if (++cu.s >= v.num_seqs) return false;
        cursor_load_seq<kRg>(cu, v, seq_lens, qsl);
      } while (cu.q.nb == 0);
    }
  }
  cu.U = make_unit<kRg>(cu.s, cu.q, v.group, cu.g, cu.rb, next_cost);
  return true;
}

// Log-sum-exp merge of the n_pieces partial results of a split unit (piece j sits in grain
// first + j: position 1 -- the grain's last unit -- for j = 0, position 0 after) into out / lse.
// All kThreads threads of the workgroup take part.  A thread takes kInFlight of its rows at a time
// and loads kPieces pieces of them together before folding them in, in piece order.
// Results over other keys folded into a merge's final rows (read only when TR::kPrior).
struct Prior {
  const float* o;
  const float* lse;
};

template <class TR, int kInFlight, int kPieces>
__device__ void merge_unit_stream(const float* part_o, const float* part_lse, void* out, float* out_f32, float* lse,
                           cptr<int32_t> qsl, int num_q_heads, int group, const pa_plan_unit& U, int64_t first,
                           int n_pieces, Prior pr = {nullptr, nullptr}) {
  constexpr int kLanesPerRow = TR::D / 4;
  constexpr int kRowsPerPass = kThreads / kLanesPerRow;
  const int q0 = qsl[U.seq];
  const int d4 = threadIdx.x % kLanesPerRow;
  for (int r0 = threadIdx.x / kLanesPerRow; r0 < U.n_rows; r0 += kInFlight * kRowsPerPass) {
    float M[kInFlight], L[kInFlight];
    f32x4_t O[kInFlight];
#pragma unroll
    for (int i = 0; i < kInFlight; ++i) {
      M[i] = -INFINITY;
      L[i] = 0.f;
      O[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    }
    for (int j0 = 0; j0 < n_pieces; j0 += kPieces) {
      float lj[kPieces][kInFlight];
      f32x4_t oj[kPieces][kInFlight];
#pragma unroll
      for (int p = 0; p < kPieces; ++p) {
        const int j = j0 + p;
        const uint32_t pbase = uint32_t((2 * (first + j) + (j == 0 ? 1 : 0)) * kPartRows);
#pragma unroll
        for (int i = 0; i < kInFlight; ++i) {
          const int r = r0 + i * kRowsPerPass;
          lj[p][i] = -INFINITY;
          if (j < n_pieces && r < U.n_rows) {
            lj[p][i] = load_coherent(part_lse, (pbase + r) * 4);
            oj[p][i] = load_coherent4(part_o, ((pbase + r) * TR::D + 4 * d4) * 4);
          }
        }
      }
#pragma unroll
      for (int p = 0; p < kPieces; ++p)
#pragma unroll
        for (int i = 0; i < kInFlight; ++i) {
          if (lj[p][i] != -INFINITY) {  // a piece that saw no key of this row adds nothing
            const float m_new = fmaxf(M[i], lj[p][i]);
            const float a_old = fast_exp2((M[i] - m_new) * kLog2e);
            const float a_new = fast_exp2((lj[p][i] - m_new) * kLog2e);
            L[i] = L[i] * a_old + a_new;
            O[i] = O[i] * a_old + oj[p][i] * a_new;
            M[i] = m_new;
          }
        }
    }
#pragma unroll
    for (int i = 0; i < kInFlight; ++i) {
      const int r = r0 + i * kRowsPerPass;
      if (r >= U.n_rows) continue;
      const int rr = U.row0 + r;
      const int tk = rr / group;
      const int head = U.kv_head * group + (rr - tk * group);
      const int64_t orow = int64_t(q0 + tk) * num_q_heads + head;
      // a row that saw no key at all (possible under a tree mask) gets out = 0, lse = -inf
      f32x4_t res = O[i] * (L[i] > 0.f ? 1.f / L[i] : 0.f);
      float lse_v = L[i] > 0.f ? M[i] + fast_log2(L[i]) * kLn2 : -INFINITY;
      if constexpr (TR::kPrior) fold_prior(pr.o, pr.lse, orow, TR::D, 4 * d4, res, lse_v);
      if (out_f32) *reinterpret_cast<f32x4_t*>(out_f32 + orow * TR::D + 4 * d4) = res;
      else TR::store_out(static_cast<char*>(out) + (orow * TR::D + 4 * d4) * TR::kEb, res);
      if (d4 == 0) lse[orow] = lse_v;
    }
  }
}

// Pieces a unit merge takes in one pass (more go through merge_unit_stream).
constexpr int kMergeFastPieces = 8;

// Log-sum-exp merge of a split unit's n_pieces partial results (piece j sits in grain first + j:
// position 1 for j = 0, position 0 after) into out / lse, with every load of a stage in flight
// at once: first one thread per row loads the row's n_pieces lse values and puts the pieces'
// weights exp(lse_j - lse) in LDS (wbuf, kMergeFastPieces * kPartRows floats) and writes the
// merged lse; then every thread folds kP pieces of all its rows per round trip.  All kThreads
// threads take part.
template <class TR>
__device__ void merge_unit(const float* part_o, const float* part_lse, void* out, float* out_f32, float* lse,
                           cptr<int32_t> qsl, int num_q_heads, int group, const pa_plan_unit& U, int64_t first,
                           int n_pieces, float* wbuf, Prior pr = {nullptr, nullptr}) {
  // key-split units (<= 32 rows) take one round trip for up to 4 pieces in the streaming form
  if (n_pieces > kMergeFastPieces || U.n_rows <= kSplitRows) {
    merge_unit_stream<TR, 4, 4>(part_o, part_lse, out, out_f32, lse, qsl, num_q_heads, group, U, first, n_pieces, pr);
    return;
  }
  const int q0 = qsl[U.seq];
  auto pbase = [&](int j) { return uint32_t((2 * (first + j) + (j == 0 ? 1 : 0)) * kPartRows); };
  auto out_row = [&](int r) {
    const int rr = U.row0 + r;
    const int tk = rr / group;
    return int64_t(q0 + tk) * num_q_heads + U.kv_head * group + (rr - tk * group);
  };
  constexpr int kLanesPerRow = TR::D / 4;
  constexpr int kRowsPerPass = kThreads / kLanesPerRow;
  constexpr int kMergeRows = 64;                   // rows folded per pass (a 128-row unit takes two)
  constexpr int kRows = kMergeRows / kRowsPerPass;  // rows of each thread per pass
  constexpr int kP = 16 / kRows;                   // pieces per round trip
  const int d4 = threadIdx.x % kLanesPerRow, r0 = threadIdx.x / kLanesPerRow;
  f32x4_t oj[kP][kRows];
  auto load_pieces = [&](int j0, int rbase) {
#pragma unroll
    for (int p = 0; p < kP; ++p)
#pragma unroll
      for (int i = 0; i < kRows; ++i) {
        const int r = rbase + r0 + i * kRowsPerPass;
        oj[p][i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        if (j0 + p < n_pieces && r < U.n_rows)
          oj[p][i] = load_coherent4(part_o, ((pbase(j0 + p) + r) * TR::D + 4 * d4) * 4);
      }
  };
  // the first pieces' o rows are loaded before the lse round trip, so the two latencies overlap
  load_pieces(0, 0);
  for (int r = threadIdx.x; r < U.n_rows; r += kThreads) {
    float lj[kMergeFastPieces];
#pragma unroll
    for (int j = 0; j < kMergeFastPieces; ++j)
      lj[j] = j < n_pieces ? load_coherent(part_lse, (pbase(j) + r) * 4) : -INFINITY;
    float M = -INFINITY;
#pragma unroll
    for (int j = 0; j < kMergeFastPieces; ++j) M = fmaxf(M, lj[j]);
    float e[kMergeFastPieces], L = 0.f;
#pragma unroll
    for (int j = 0; j < kMergeFastPieces; ++j) {  // a piece that saw no key of this row adds nothing
      e[j] = lj[j] == -INFINITY ? 0.f : fast_exp2((lj[j] - M) * kLog2e);
      L += e[j];
    }
    // a row that saw no key at all (possible under a tree mask) gets out = 0, lse = -inf
    float inv = L > 0.f ? 1.f / L : 0.f;
    float lse_v = L > 0.f ? M + fast_log2(L) * kLn2 : -INFINITY;
    if constexpr (TR::kPrior) {  // the pieces' weights scaled by the unit's share against the prior result
      const float lp = pr.lse[out_row(r)];
      float wp = 0.f;
      if (lp != -INFINITY) {
        if (lse_v == -INFINITY) {
          wp = 1.f;
          lse_v = lp;
        } else {
          const float m = fmaxf(lse_v, lp);
          const float ws = fast_exp2((lse_v - m) * kLog2e), wq = fast_exp2((lp - m) * kLog2e);
          const float t = 1.f / (ws + wq);
          inv *= ws * t;
          wp = wq * t;
          lse_v = m + fast_log2(ws + wq) * kLn2;
        }
      }
      wbuf[kMergeFastPieces * kPartRows + r] = wp;
    }
#pragma unroll
    for (int j = 0; j < kMergeFastPieces; ++j)
      if (j < n_pieces) wbuf[j * kPartRows + r] = e[j] * inv;
    lse[out_row(r)] = lse_v;
  }
  wait_lds();
  lds_barrier();  // wbuf written (a full __syncthreads would also wait for the o loads in flight)
  for (int rbase = 0; rbase < U.n_rows; rbase += kMergeRows) {
    f32x4_t acc[kRows];
#pragma unroll
    for (int i = 0; i < kRows; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    for (int j0 = 0; j0 < n_pieces; j0 += kP) {
      if (j0 > 0 || rbase > 0) load_pieces(j0, rbase);
#pragma unroll
      for (int p = 0; p < kP; ++p)
#pragma unroll
        for (int i = 0; i < kRows; ++i) {
          const int r = rbase + r0 + i * kRowsPerPass;
          if (j0 + p < n_pieces && r < U.n_rows) acc[i] += oj[p][i] * wbuf[(j0 + p) * kPartRows + r];
        }
    }
#pragma unroll
    for (int i = 0; i < kRows; ++i) {
      const int r = rbase + r0 + i * kRowsPerPass;
      if (r >= U.n_rows) continue;
      const int64_t orow = out_row(r);
      if constexpr (TR::kPrior)
        acc[i] += *reinterpret_cast<const f32x4_t*>(pr.o + orow * TR::D + 4 * d4) * wbuf[kMergeFastPieces * kPartRows + r];
      if (out_f32) *reinterpret_cast<f32x4_t*>(out_f32 + orow * TR::D + 4 * d4) = acc[i];
      else TR::store_out(static_cast<char*>(out) + (orow * TR::D + 4 * d4) * TR::kEb, acc[i]);
    }
  }
  __syncthreads();  // wbuf is read by every thread before the caller reuses LDS
}

// Grains holding the first and the last chunk of a unit.
__device__ __forceinline__ int64_t first_grain(const pa_plan_unit& U, int64_t S, int64_t C) {
  return slot_of(chunk_start(U, 0), S, C);
}
__device__ __forceinline__ int64_t last_grain(const pa_plan_unit& U, int64_t S, int64_t C) {
  return slot_of(chunk_start(U, U.n_chunks - 1), S, C);
}

// Single launch: after writing its piece of a split unit, the workgroup counts itself in; the
// one that completes the count merges every piece and re-zeroes the counter for the next call.
// The pieces are agent-coherent stores that have completed (vmcnt(0)) before the count, and the
// merging workgroup reads them with agent-coherent loads issued after it saw the count.
template <class TR>
__device__ void arrive_and_merge(const AttnArgs& A, const pa_plan_unit& U, int64_t S, int64_t C, int* flag,
                                 float* wbuf) {
  const int64_t first = first_grain(U, S, C);
  const int n_pieces = int(last_grain(U, S, C) - first + 1);
  wait_all_loads();  // this wave's partial stores are done
  __syncthreads();
  if (threadIdx.x == 0) {
    const int done = __hip_atomic_fetch_add(A.arrive + first, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *flag = done == n_pieces - 1;
  }
  __syncthreads();
  const bool last = *flag;
  __syncthreads();  // flag read by every thread before it is reused
  if (!last) return;
  merge_unit<TR>(A.part_o, A.part_lse, A.out, A.out_f32, A.lse, ro(A.plan.qsl), A.num_q_heads, A.plan.group, U,
                 first, n_pieces, wbuf, Prior{A.prior_o, A.prior_lse});
  if (threadIdx.x == 0) __hip_atomic_store(A.arrive + first, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The chunks [i0, i1) of a unit that lie in the grain [c0, c1), and where their result goes:
// part < 0 -- the whole unit, final output; else the partial position (grain * 2 + 0 for the piece
// the grain starts inside, + 1 for the one it ends inside).
struct Piece {
  int i0, i1, part;
};
__device__ __forceinline__ Piece piece_of(const pa_plan_unit& U, int64_t c0, int64_t c1, int grain) {
  // chunk weights are powers of two: ceil divisions by them are shifts (a 64-bit division is a long
  // emulated sequence, measured at ~0.7 us per unit start on MI355X)
  const int64_t w = U.cost_weight;
  const int sh = __builtin_ctz(uint32_t(U.cost_weight));
  const int64_t cs = chunk_start(U, 0);
  Piece p;
  p.i0 = int(c0 > cs ? (c0 - cs + w - 1) >> sh : 0);
  const int64_t e = c1 > cs ? (c1 - cs + w - 1) >> sh : 0;
  p.i1 = int(e < U.n_chunks ? e : U.n_chunks);
  // a grain holds at most two pieces of split units: the one it starts inside (position 0)
  // and the one it ends inside (position 1)
  p.part = (p.i0 > 0 || p.i1 < U.n_chunks) ? 2 * grain + (cs < c0 ? 0 : 1) : -1;
  return p;
}

// Key-split units of RT row tiles (bf16 pages, K by DMA) run back to back: the cursor's unit and
// the units after it in the grain while they are of that kind.  In a wave's last step of a unit,
// its one load in flight is already its first chunk of the next unit (page ids loaded at the unit
// start), and for one row tile the next unit's Q is in registers by then too, so the unit's end --
// the cross-wave merge and the output -- overlaps those loads instead of adding two dependent
// round trips (page ids, then K/V) to every unit start.  The merge goes through the Q slices only
// (the K slots may be receiving a DMA), one row tile at a time, with LDS accesses that do not wait
// for global loads.  Leaves the cursor on the last unit it ran.
template <class TR, int RT>
__device__ void run_keysplit_stream(const AttnArgs& A, UnitCursor& cu, Piece p, int64_t c0, int64_t c1, int grain,
                                    Smem<TR>& sm) {
  using RG = Ring<TR>;
  static_assert(TR::kBf16, "bf16 pages with K by DMA");
  constexpr bool kPreQ = RT == 1;  // two row tiles of Q held across a unit would spill
  const PlanView& v = A.plan;
  const cptr<int32_t> seq_lens = ro(v.seq_lens);
  const cptr<int32_t> qsl = ro(v.qsl);
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int quad = lane >> 4;
  const int n = lane & 15;
  constexpr int kQRegion = kWaves * 2 * TR::kQF * 64;  // u32x4 slots of the Q slices
  static_assert(kWaves * TR::kTiles * 64 <= kQRegion, "one row tile's merge buffer inside the Q slices");
  static_assert(kQRegion * 16 + kWaves * 2 * RG::kBlk <= Smem<TR>::kBytes, "LDS budget");
  u32x4_t* qlds = sm.buf + w * (RT * TR::kQF * 64);
  char* kslot = reinterpret_cast<char*>(sm.buf + kQRegion) + w * 2 * RG::kBlk;
  f32x4_t* obuf = reinterpret_cast<f32x4_t*>(sm.buf);
  float* stat = &sm.stat[0][0][0][0];  // (m, l) of wave i, row r at 2 * (16 i + r)
  const uint32_t vl = TR::v_lane(lane);
  auto dma_k = [&](const ChunkPages& cp) {
    constexpr int kPer = RG::kBlk / 1024;  // DMA instructions per page
    const __amdgpu_buffer_rsrc_t r0 = block_rsrc(cp.k0, RG::kBlk), r1 = block_rsrc(cp.k1, RG::kBlk);
#pragma unroll
    for (int i = 0; i < 2 * kPer; ++i) {
      const int o = (i % kPer) * 1024 + 16 * lane;
      const int r = o / RG::kPitchK, cc = (o % RG::kPitchK) / 16;
      dma16(i < kPer ? r0 : r1, uint32_t(r * RG::kPitchK + RG::swz_k(r, cc) * 16),
            kslot + (i / kPer) * RG::kBlk + (i % kPer) * 1024);
    }
  };
  auto bt_of = [&](int s) {
    return ro(A.block_table) + int64_t(s) * A.max_pages + (A.key_base ? ro(A.key_base)[s] / kPage : 0);
  };
  auto same_kind = [&](const pa_plan_unit& N) {
    return N.kind == 0 && (RT == 1 ? N.n_rows <= 16 : N.n_rows > 16);
  };
  typename TR::VRaw vr[TR::kVF];
  u32x4_t qnext[kPreQ ? TR::kQF : 1];  // Q of the next unit, loaded during this one
  bool pre = false;  // this wave's first load (and Q, for one row tile) of the unit were issued before
  for (;;) {
    const pa_plan_unit& U = cu.U;
    const int n_seq = cu.q.n, qn = cu.q.qn;
    const cptr<int32_t> bt_row = bt_of(U.seq);
    RowInfo ri[RT];
    int p_row[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      ri[rt] = row_info(A, U, 16 * rt + n, n_seq, cu.q.q0, qn);
      p_row[rt] = ri[rt].p;
    }
    u32x4_t qtmp[RT][TR::kQF];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int f = 0; f < TR::kQF; ++f) {
        if constexpr (kPreQ) qtmp[rt][f] = pre ? qnext[f] : load_q_frag<TR>(A, ri[rt], f, quad);
        else qtmp[rt][f] = load_q_frag<TR>(A, ri[rt], f, quad);
      }
    // Does the stream go on?  Only the next unit's kv head, this wave's first page ids in it and
    // (one row tile) its Q rows are kept; the cursor is advanced again after the unit.
    bool nxt;
    int nkvh = 0;
    PageIds held{0, 0};
    RowInfo rnext{0, 0, -1, false};
    {
      UnitCursor nc = cu;
      nxt = cursor_next<TR::kRowGeom>(nc, v, seq_lens, qsl) && nc.U.cost0 < c1 && same_kind(nc.U);
      if (nxt) {
        const Piece np = piece_of(nc.U, c0, c1, grain);
        nxt = np.i0 < np.i1;
        if (nxt) {
          held = page_ids_load(bt_of(nc.U.seq), np.i0 + w < np.i1 ? np.i0 + w : np.i0, nc.q.n);
          if constexpr (kPreQ) rnext = row_info(A, nc.U, n, nc.q.n, nc.q.q0, nc.q.qn);
        }
        nkvh = nc.U.kv_head;
      }
    }
    // The next unit's Q is loaded in this unit's first step, after the wait for its first chunk
    // (so that wait does not also cover it) and before the next DMA (so the next wait does not).
    auto load_qnext = [&] {
      if constexpr (kPreQ) {
        if (nxt) {
#pragma unroll
          for (int f = 0; f < TR::kQF; ++f) qnext[f] = load_q_frag<TR>(A, rnext, f, quad);
        }
      }
    };
    const int c = p.i0 + w;
    const int mine = p.i1 > c ? (p.i1 - c + kWaves - 1) / kWaves : 0;  // chunks of this wave
    TreeMask<RT> tm;
    tm.win0 = 0;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) tm.m[rt] = ~uint64_t(0);
    const int min_p = v.full_rows ? n_seq - 1 : n_seq - qn + U.row0 / v.group;  // first row's last key
    if (!pre) {
      const ChunkPages cp = pages_of<TR>(A, U.kv_head, page_ids(bt_row, c < p.i1 ? c : p.i0, n_seq));
      dma_k(cp);
      issue_order();  // V after the K DMA: the loop's first wait for it counts on that order
      load_v<TR>(cp, vl, vr);
    }
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int f = 0; f < TR::kQF; ++f) lds_write_b128(lds_addr(qlds + (rt * TR::kQF + f) * 64 + lane), qtmp[rt][f]);
    // the next unit's page ids: waited for here only on the stream's first unit (issued after
    // this unit's Q); later they were issued one unit ahead
    const PageIds nid = uniform_ids(held);
    State<TR, RT> st;
    state_init(st);
    if (mine == 0) load_qnext();
    if (mine == 0 && nxt) {
      // no chunk of this unit for this wave: its load in flight is a dummy; replace it by its first
      // chunk of the next unit once the dummy's DMA into the slot has landed
      wait_all_loads();
      const ChunkPages cp = pages_of<TR>(A, nkvh, nid);
      dma_k(cp);
      issue_order();
      load_v<TR>(cp, vl, vr);
    }
    PageIds nx = page_ids(bt_row, min(c + kWaves, p.i1 - 1), n_seq);
    for (int j = 0; j < mine; ++j) {
      const int cc = c + j * kWaves;
      const int key0 = cc * kChunkKeys;
      const int cn = cc + kWaves;
      // the wave's next load: its next chunk, else its first chunk of the next unit, else a dummy
      // (the pool's first page: an L2 hit) that keeps one load in flight on every path
      const ChunkPages ncp = pages_of<TR>(A, cn < p.i1 ? U.kv_head : nkvh,
                                          cn < p.i1 ? nx : (nxt ? nid : PageIds{0, 0}));
      typename TR::PFrag pf[RT];
      u32x4_t kf[TR::kKF];
      wait_vmcnt<TR::kVLoads>();  // the K DMA of this chunk has landed (only V was issued after it)
      asm volatile("" ::: "memory");
      TR::template lds_read_k<RG>(kslot, lane, kf);  // completes before the slot is refilled
      asm volatile("" ::: "memory");
      if (j == 0) load_qnext();
      dma_k(ncp);
      auto getq_asm = [&](int rt, u32x4_t (&qf)[TR::kQF]) {
        uint32_t a[TR::kQF];
#pragma unroll
        for (int f = 0; f < TR::kQF; ++f) a[f] = lds_addr(qlds + (rt * TR::kQF + f) * 64 + lane);
        lds_read_b128<TR::kQF>(a, qf);
      };
      softmax_chunk<TR, RT, false>(st, getq_asm, kf, key0, p_row, tm, ChunkScale{1.f, 1.f, 1.f, 1.f},
                                   key0 + kChunkKeys - 1 > min_p, A.scale_log2, lane, pf);
      asm volatile("" ::: "memory");
      nx = page_ids(bt_row, min(cn + kWaves, p.i1 - 1), n_seq);
      u32x4_t vf[TR::kVF];
#pragma unroll
      for (int f = 0; f < TR::kVF; ++f) vf[f] = TR::v_convert(vr[f]);
      if (key0 + kChunkKeys > n_seq) TR::sanitize_v(vf, quad, n_seq - key0);  // the sequence's last chunk
      pv_chunk<TR, RT>(st, vf, pf);
      load_v<TR>(ncp, vl, vr);
    }
    if (!nxt) wait_all_loads();  // the stream ends: nothing of it left in flight
    wait_lds();
    lds_barrier();  // every wave is done with its Q slice before the merge buffer overwrites it

    // merge the 4 waves' states through LDS, one row tile at a time
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const float l = quad_sum(st.l[rt]);
      if (quad == 0)
        lds_write_b64(lds_addr(stat + 2 * (16 * w + n)), u32x2_t{__float_as_uint(st.m[rt]), __float_as_uint(l)});
#pragma unroll
      for (int t = 0; t < TR::kTiles; ++t)
        lds_write_b128(lds_addr(obuf + (w * TR::kTiles + t) * 64 + lane), __builtin_bit_cast(u32x4_t, st.o[rt][t]));
      wait_lds();
      lds_barrier();
      uint32_t a[kWaves];
#pragma unroll
      for (int i = 0; i < kWaves; ++i) a[i] = lds_addr(stat + 2 * (16 * i + n));
      u32x2_t ml[kWaves];
      lds_read4_b64(a, ml[0], ml[1], ml[2], ml[3]);
      float M = -INFINITY;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) M = fmaxf(M, __uint_as_float(ml[i][0]));
      float sc[kWaves], L = 0.f;
#pragma unroll
      for (int i = 0; i < kWaves; ++i) {
        const float mw = __uint_as_float(ml[i][0]);
        sc[i] = mw == -INFINITY ? 0.f : fast_exp2(mw - M);
        L += __uint_as_float(ml[i][1]) * sc[i];
      }
      const float inv = L > 0.f ? 1.f / L : 0.f;
      const float lse_nat = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
      for (int t = w; t < TR::kTiles; t += kWaves) {
#pragma unroll
        for (int i = 0; i < kWaves; ++i) a[i] = lds_addr(obuf + (i * TR::kTiles + t) * 64 + lane);
        u32x4_t x[kWaves];
        lds_read4_b128(a, x[0], x[1], x[2], x[3]);
        f32x4_t o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int i = 0; i < kWaves; ++i) o += as_f32x4(x[i]) * sc[i];
        emit<TR>(A, ri[rt], 16 * rt + n, p.part, t, quad, o * inv, lse_nat, t == 0 && quad == 0);
      }
      lds_barrier();  // the merge reads are done (each waited in place) before the region is rewritten
    }
    if (!nxt) return;
    cursor_next<TR::kRowGeom>(cu, v, seq_lens, qsl);
    p = piece_of(cu.U, c0, c1, grain);
    pre = true;
  }
}

// One grain: the chunks whose start cost lies in [st.c0, st.c1), unit by unit.  kFused: the
// single-launch kernel (S grains over total cost C; split units are merged here), else the staged
// kernel (split units are left as partial results for the merge kernel).
template <class TR, bool kFused, bool kTree>
__device__ __forceinline__ void run_grain(const AttnArgs& A, int grain, const SlotStart& st, int64_t S, int64_t C, Smem<TR>& sm,
                          int* flag) {
  const PlanView& v = A.plan;
  const int64_t c0 = st.c0, c1 = st.c1;
  if (c0 >= c1) return;
  const cptr<int32_t> seq_lens = ro(v.seq_lens);
  const cptr<int32_t> qsl = ro(v.qsl);
  UnitCursor cu;
  cursor_from_slot<TR::kRowGeom>(cu, v, st);
  do {
    const pa_plan_unit& U = cu.U;
    if (U.cost0 >= c1) break;
    const Piece pc = piece_of(U, c0, c1, grain);
    const int i0 = pc.i0, i1 = pc.i1, part = pc.part;
    if (i0 < i1) {
      bool streamed = false;
      if constexpr (TR::kBf16 && !TR::kScaled && !kTree) {
        // a stream never holds the piece the grain starts inside (its arrival would wait for the
        // next unit's loads); the one it ends inside can only be the stream's last unit
        // (units of two row tiles streamed ~1% slower: their Q cannot be held across a unit)
        if (U.kind == 0 && U.n_rows <= 16 && (part < 0 || (part & 1))) {
          run_keysplit_stream<TR, 1>(A, cu, pc, c0, c1, grain, sm);  // moves the cursor to its last unit
          streamed = true;
        }
      }
      if (!streamed) {
        if (U.kind == 0) {
          if (U.n_rows <= 16) run_keysplit<TR, 1, kTree>(A, U, cu.q, i0, i1, part, sm);
          else run_keysplit<TR, 2, kTree>(A, U, cu.q, i0, i1, part, sm);
        } else {
          run_rowsplit<TR, kTree>(A, U, cu.q, i0, i1, part, sm);
        }
      }
      if constexpr (kFused) {  // cu.U: the unit just run (the stream's last one)
        if ((streamed ? piece_of(cu.U, c0, c1, grain).part : part) >= 0)
          arrive_and_merge<TR>(A, cu.U, S, C, flag, reinterpret_cast<float*>(sm.buf));
      }
    }
  } while (cursor_next<TR::kRowGeom>(cu, v, seq_lens, qsl));
}

// Staged path: workgroup b runs grain b, b + grid, ... of the plan in the workspace.
template <class TR>
__global__ __launch_bounds__(kThreads, 2) void attention_kernel(AttnArgs A) {
  __shared__ Smem<TR> sm;
  const int64_t S = ro(A.plan.hdr)->n_slots;
  for (int64_t g = blockIdx.x; g < S; g += gridDim.x)
    run_grain<TR, false, false>(A, int(g), load_slot(ro(A.plan.slots) + g), 0, 0, sm, nullptr);
}

// Sums and scans of one int64 per thread over the kThreads threads of a workgroup.
__device__ __forceinline__ int64_t wg_sum(int64_t x, int64_t* red) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  x = wave_incl_scan64(x);
  if (lane == 63) red[wid] = x;
  __syncthreads();
  int64_t t = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) t += red[i];
  __syncthreads();
  return t;
}
// Both sums of two int64 per thread, with one exchange through LDS (red: 2 * kWaves slots).
__device__ __forceinline__ void wg_sum2(int64_t x, int64_t y, int64_t* red, int64_t& sx, int64_t& sy) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  x = wave_incl_scan64(x);
  y = wave_incl_scan64(y);
  if (lane == 63) {
    red[wid] = x;
    red[kWaves + wid] = y;
  }
  __syncthreads();
  sx = sy = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    sx += red[i];
    sy += red[kWaves + i];
  }
  __syncthreads();
}
// Exclusive scan of x and the sums of x and y over the workgroup, with one exchange through LDS
// (red: 2 * kWaves slots).
__device__ __forceinline__ int64_t wg_scan_sum(int64_t x, int64_t y, int64_t* red, int64_t& sx, int64_t& sy) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t incl = wave_incl_scan64(x);
  y = wave_incl_scan64(y);
  if (lane == 63) {
    red[wid] = incl;
    red[kWaves + wid] = y;
  }
  __syncthreads();
  int64_t before = 0;
  sx = sy = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    if (i < wid) before += red[i];
    sx += red[i];
    sy += red[kWaves + i];
  }
  __syncthreads();
  return incl - x + before;
}
__device__ __forceinline__ int64_t wg_exclusive_scan(int64_t x, int64_t* red, int64_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t incl = wave_incl_scan64(x);
  if (lane == 63) red[wid] = incl;
  __syncthreads();
  int64_t before = 0, all = 0;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    if (i < wid) before += red[i];
    all += red[i];
  }
  __syncthreads();
  *total = all;
  return incl - x + before;
}

struct PreLds {
  int64_t red[2 * kWaves];
  int64_t hold_base;  // the sequence holding the grain start: its first cost, index, lengths
  int32_t hold_s, hold_n, hold_q0, hold_qn;
  SlotStart st;
  int flag;
};

// Cost of the kPer sequences of this thread in the block of kThreads * kPer at `base`
// (c), and the part of their sum that is row-split work (returned).
template <int kPer, int kRg>
__device__ __forceinline__ int64_t block_seq_costs(const PlanView& v, cptr<int32_t> sl, cptr<int32_t> qsl, int base,
                                                   int64_t (&c)[kPer], int (&n)[kPer], int (&q0)[kPer],
                                                   int (&qn)[kPer]) {
  int64_t row = 0;
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    const int s = base + threadIdx.x * kPer + e;
    n[e] = q0[e] = qn[e] = 0;
    c[e] = 0;
    if (s < v.num_seqs) {
      n[e] = sl[s];
      q0[e] = qsl[s];
      qn[e] = qsl[s + 1] - q0[e];
      const SeqUnits q = seq_units<kRg>(n[e], q0[e], qn[e], v.group, v.full_rows != 0);
      c[e] = int64_t(v.num_kv_heads) * q.per_head;
      if (!q.split) row += c[e];
    }
  }
  return row;
}

// Workgroups that run grains out of a launch of `grid`: a batch without row-split work (decode,
// verify) uses one workgroup per CU, the first of each CU's two (workgroups b and b + grid / 2
// share a CU).  Two workgroups on a CU are not served alike -- the older streams about 1.4x as
// fast -- so with two per CU the younger ones end well after the older (measured on MI355X: the
// llama3-8b decode batch 2.5% faster with one).  Staged and single launch cut grains alike.
__host__ __device__ __forceinline__ int decode_grid(int grid, int64_t row_cost) {
  return row_cost == 0 && grid % 16 == 0 ? grid / 2 : grid;
}

// Grain run by workgroup b of a grid of `grid` (S <= grid grains; S or more means none).
// Workgroups are dealt to the 8 XCDs (each with its own L2) round-robin, so workgroup b runs on
// XCD b % 8; grains adjacent on the cost axis -- the units of one sequence, which read the same
// K/V pages, and the pieces of one split unit -- go to one XCD: with n = ceil(S / 8), XCD x runs
// grains x * n .. x * n + n - 1.  Any placement is correct (grains are independent and pieces are
// exchanged coherently); this one keeps a sequence's pages in one L2.
constexpr int kXcds = 8;
__device__ __forceinline__ int64_t grain_of_block(int b, int grid, int64_t S) {
  if (grid % kXcds != 0) return b;
  const int64_t n = (S + kXcds - 1) / kXcds, j = b / kXcds;
  return j < n ? int64_t(b % kXcds) * n + j : S;
}

// The single launch's plan, in every workgroup: the total cost C and the grain count S from
// seq_lens and query_start_loc (the same numbers the staged planner writes), then -- for this
// workgroup's grain, found with a workgroup-wide scan of the per-sequence costs -- the grain's
// start in pl.st.  Each thread takes kPer sequences per pass of kThreads * kPer (one when the
// batch fits one pass, so that no thread computes several sequences' costs in a row).  Returns
// the grain index; S or more means the workgroup has none.
template <int kPer, bool kSolo, int kRg>
__device__ __forceinline__ int64_t plan_grain(const PlanView& v, PreLds& pl, int64_t& S, int64_t& C) {
  const cptr<int32_t> sl = ro(v.seq_lens), qsl = ro(v.qsl);
  constexpr int kBlock = kThreads * kPer;
  int64_t c[kPer];
  int n[kPer], q0[kPer], qn[kPer];
  const int64_t row0 = block_seq_costs<kPer, kRg>(v, sl, qsl, 0, c, n, q0, qn);  // kept for the search below
  C = 0;
  int64_t Cr = 0;
  // one block of sequences: the totals and this block's prefix come from one exchange
  const bool one = v.num_seqs <= kBlock;
  int64_t pre0 = 0;
  if (one) {
    int64_t x = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) x += c[e];
    pre0 = wg_scan_sum(x, row0, pl.red, C, Cr);
  }
  for (int base = 0; !one && base < v.num_seqs; base += kBlock) {
    int64_t c2[kPer];
    int n2[kPer], q02[kPer], qn2[kPer];
    const int64_t row = base > 0 ? block_seq_costs<kPer, kRg>(v, sl, qsl, base, c2, n2, q02, qn2) : row0;
    int64_t x = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) x += base > 0 ? c2[e] : c[e];
    int64_t sx, sy;
    wg_sum2(x, row, pl.red, sx, sy);
    C += sx;
    Cr += sy;
  }
  const int grid = kSolo ? decode_grid(int(gridDim.x), Cr) : int(gridDim.x);
  if (int(blockIdx.x) >= grid) {
    S = 0;
    return 0;
  }
  S = grain_count(C - Cr, Cr, grid, rg_weight(kRg));
  const int64_t k = grain_of_block(int(blockIdx.x), grid, S);
  if (k >= S) return k;
  const int64_t c0 = slice_begin(k, S, C), c1 = slice_begin(k + 1, S, C);
  int64_t carry = 0;
  for (int base = 0; base < v.num_seqs; base += kBlock) {
    if (base > 0) block_seq_costs<kPer, kRg>(v, sl, qsl, base, c, n, q0, qn);
    int64_t x = 0;
#pragma unroll
    for (int e = 0; e < kPer; ++e) x += c[e];
    int64_t tot = C;
    int64_t pre = one ? pre0 : carry + wg_exclusive_scan(x, pl.red, &tot);
    if (c0 >= pre && c0 < pre + x) {  // exactly one thread holds the sequence of cost c0
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        if (c0 >= pre && c0 < pre + c[e]) {
          pl.hold_base = pre;
          pl.hold_s = base + int(threadIdx.x) * kPer + e;
          pl.hold_n = n[e];
          pl.hold_q0 = q0[e];
          pl.hold_qn = qn[e];
        }
        pre += c[e];
      }
    }
    carry += tot;
    if (c0 < carry) break;  // uniform: every thread holds the same carry
  }
  __syncthreads();
  if (threadIdx.x < 64) {  // wave 0 places the cursor
    UnitCursor cu;
    cursor_place_wave<kRg>(cu, v, pl.hold_s, pl.hold_base, pl.hold_n, pl.hold_q0, pl.hold_qn, c0, int(threadIdx.x));
    if (threadIdx.x == 0) pl.st = slot_from_cursor(cu, c0, c1);
  }
  __syncthreads();
  return k;
}

// Single launch: every workgroup plans (plan_grain), then runs its grain and merges the split
// units it completes.
template <class TR, bool kTree>
__global__ __launch_bounds__(kThreads, 2) void attention_fused_kernel(AttnArgs A) {
  __shared__ Smem<TR> sm;
  __shared__ PreLds pl;
  int64_t S, C;
  constexpr bool kSolo = !TR::kScaled;  // FP8 pages stream faster with both workgroups of a CU
  const int64_t k = A.plan.num_seqs <= kThreads ? plan_grain<1, kSolo, TR::kRowGeom>(A.plan, pl, S, C)
                                                : plan_grain<4, kSolo, TR::kRowGeom>(A.plan, pl, S, C);
  if (k >= S) return;
  const SlotStart st = pl.st;
  run_grain<TR, true, kTree>(A, int(k), st, S, C, sm, &pl.flag);
}

// ---------------------------------------------------------------------------
// Planner: one workgroup writes the per-sequence cost prefix and the header.
// ---------------------------------------------------------------------------
constexpr int kScanThreads = 1024;

// Exclusive scan of one int64 per thread over the workgroup; *total gets the sum.
__device__ int64_t block_exclusive_scan(int64_t x, int64_t* wave_tot, int64_t* total) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  constexpr int kNW = kScanThreads / 64;
  const int64_t incl = wave_incl_scan64(x);
  if (lane == 63) wave_tot[wid] = incl;
  __syncthreads();
  if (wid == 0) {
    const int64_t t = wave_incl_scan64(lane < kNW ? wave_tot[lane] : 0);
    if (lane < kNW) wave_tot[lane] = t;
  }
  __syncthreads();
  const int64_t excl = incl - x + (wid > 0 ? wave_tot[wid - 1] : 0);
  *total = wave_tot[kNW - 1];
  __syncthreads();
  return excl;
}

constexpr int kPlanLdsSeqs = 4096;  // sequences whose cost prefix the planner keeps in LDS

__global__ __launch_bounds__(kScanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int64_t wave_tot[kScanThreads / 64];
  __shared__ int64_t lds_cost[kPlanLdsSeqs + 1];
  int64_t carry = 0, units = 0, row_cost = 0;
  for (int base = 0; base < a.num_seqs; base += kScanThreads) {
    const int s = base + threadIdx.x;
    int64_t cost = 0, nu = 0;
    bool split = true;
    if (s < a.num_seqs) {
      const SeqUnits q = seq_units(a.seq_lens[s], 0, a.qsl[s + 1] - a.qsl[s], a.group, a.full_rows != 0);
      cost = int64_t(a.num_kv_heads) * q.per_head;
      nu = int64_t(a.num_kv_heads) * q.nb;
      split = q.split;
    }
    int64_t tot, tot_u, tot_r;
    const int64_t ex = block_exclusive_scan(cost, wave_tot, &tot);
    block_exclusive_scan(nu, wave_tot, &tot_u);
    block_exclusive_scan(split ? 0 : cost, wave_tot, &tot_r);
    row_cost += tot_r;
    if (s < a.num_seqs) {
      a.seq_cost[s] = carry + ex;
      if (s < kPlanLdsSeqs) lds_cost[s] = carry + ex;
    }
    carry += tot;
    units += tot_u;
  }
  const int64_t C = carry;
  const int64_t S = grain_count(C - row_cost, row_cost, decode_grid(a.grid, row_cost));
  if (threadIdx.x == 0) {
    a.seq_cost[a.num_seqs] = C;
    a.hdr->n_units = int32_t(units);
    a.hdr->n_slots = int32_t(S);
    a.hdr->grid = a.grid;
    a.hdr->num_seqs = a.num_seqs;
    a.hdr->total_cost = C;
    a.hdr->reserved = 0;
  }
  for (int k = threadIdx.x; k < a.grid; k += kScanThreads) a.arrive[k] = 0;  // for a single launch
  __syncthreads();  // seq_cost (global and LDS) complete
  // where every slot starts: one binary search per slot
  PlanView v;
  v.seq_lens = a.seq_lens;
  v.qsl = a.qsl;
  v.hdr = a.hdr;
  v.seq_cost = a.seq_cost;
  v.slots = a.slots;
  v.num_seqs = a.num_seqs;
  v.num_kv_heads = a.num_kv_heads;
  v.group = a.group;
  v.full_rows = a.full_rows;
  for (int k = threadIdx.x; k < S; k += kScanThreads) {
    SlotStart r;
    r.c0 = slice_begin(k, S, C);
    r.c1 = slice_begin(k + 1, S, C);
    UnitCursor cu;
    if (a.num_seqs <= kPlanLdsSeqs) cursor_find(cu, v, a.seq_lens, a.qsl, lds_cost, r.c0);
    else cursor_find(cu, v, a.seq_lens, a.qsl, a.seq_cost, r.c0);
    a.slots[k] = slot_from_cursor(cu, r.c0, r.c1);
  }
}

// Plan inspection: one thread walks every unit in cost order (tests and debugging only).
__global__ void plan_units_kernel(PlanView v, pa_plan_unit* out, int64_t max_units) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  const int64_t C = v.hdr->total_cost, S = v.hdr->n_slots;
  if (C <= 0) return;
  UnitCursor cu;
  cursor_find(cu, v, v.seq_lens, v.qsl, v.seq_cost, 0);
  int64_t i = 0;
  do {
    pa_plan_unit U = cu.U;
    const int64_t first = slot_of(chunk_start(U, 0), S, C);
    const int64_t last = slot_of(chunk_start(U, U.n_chunks - 1), S, C);
    U.first_slot = int32_t(first);
    U.n_pieces = int32_t(last - first + 1);
    if (i < max_units) out[i] = U;
    ++i;
  } while (cursor_next(cu, v, v.seq_lens, v.qsl));
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of split units.  Workgroup k looks at slice boundary k; the
// unit that boundary cuts is merged by the workgroup of its first boundary.
// ---------------------------------------------------------------------------
template <class TR>
__device__ __forceinline__ void merge_row(const float* o_parts, const float* lse_parts, int64_t stride_rows,
                                          int n_parts, int d4, float* lse_out_val, f32x4_t* o_out) {
  float M = -INFINITY;
  for (int j = 0; j < n_parts; ++j) M = fmaxf(M, lse_parts[j * stride_rows]);
  float sum = 0.f;
  if (M != -INFINITY)
    for (int j = 0; j < n_parts; ++j) sum += fast_exp2((lse_parts[j * stride_rows] - M) * kLog2e);
  const float lse = M == -INFINITY ? -INFINITY : M + fast_log2(sum) * kLn2;
  f32x4_t o = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < n_parts; ++j) {
    const float lj = lse_parts[j * stride_rows];
    if (lj == -INFINITY) continue;
    const float wgt = fast_exp2((lj - lse) * kLog2e);
    o += wgt * *reinterpret_cast<const f32x4_t*>(o_parts + j * stride_rows * TR::D + 4 * d4);
  }
  *lse_out_val = lse;
  *o_out = o;
}

template <class TR>
__global__ __launch_bounds__(kThreads) void merge_planned_kernel(MergeArgs a) {
  const PlanView& v = a.plan;
  const int64_t S = ro(v.hdr)->n_slots, C = ro(v.hdr)->total_cost;
  const int k = blockIdx.x;
  if (k == 0 || k >= S) return;
  UnitCursor cu;
  cursor_from_slot(cu, v, load_slot(ro(v.slots) + k));  // the unit holding the first cost of grain k
  const pa_plan_unit& U = cu.U;
  const int64_t first = first_grain(U, S, C);
  const int64_t last = last_grain(U, S, C);
  if (first != k - 1 || last < k) return;  // boundary k does not open this unit's split
  __shared__ float wbuf[kMergeFastPieces * kPartRows];
  merge_unit<TR>(a.part_o, a.part_lse, a.out, nullptr, a.lse, ro(v.qsl), a.num_q_heads, v.group, U, first,
                 int(last - first + 1), wbuf);
}

// Stand-alone merge: rows of n_parts partial results (o_parts [P][rows][D], lse_parts [P][rows]).
template <class TR>
__global__ __launch_bounds__(kThreads) void merge_kernel(int n_parts, int64_t rows, const float* o_parts,
                                                         const float* lse_parts, void* out, float* lse_out) {
  constexpr int kLanesPerRow = TR::D / 4;
  const int64_t gid = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t r = gid / kLanesPerRow;
  const int d4 = int(gid % kLanesPerRow);
  if (r >= rows) return;
  float lse;
  f32x4_t o;
  merge_row<TR>(o_parts + r * TR::D, lse_parts + r, rows, n_parts, d4, &lse, &o);
  TR::store_out(static_cast<char*>(out) + (r * TR::D + 4 * d4) * TR::kEb, o);
  if (d4 == 0) lse_out[r] = lse;
}

// ---------------------------------------------------------------------------
// Paged KV append: the K/V rows of the new tokens go to positions n - q .. n - 1 of their
// sequence (the window's own keys for the attention call).  Workgroup (s, g, z) writes pages
// first + kAppendPages*z ... of sequence s, K/V head g.  K rows are copied as 16-byte vectors.
// V rows of a page are staged in LDS ([slot][D], padded rows) and written back transposed: a full
// page's [D][16] block as whole 16-byte vectors, a partial page slot by slot.
// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(256) void append_kv_kernel(AppendArgs a) {
  constexpr int kPerVec = 16 / sizeof(E);            // elements per 16-byte vector
  constexpr int kPitch = 128 + 16 / sizeof(E);        // LDS row pitch in elements (D <= 128, 16-byte pad)
  __shared__ __align__(16) E tile[kPage * kPitch];
  const int s = blockIdx.x, g = blockIdx.y;
  const int n = a.seq_lens[s];
  const int q0 = a.qsl[s];
  const int qn = a.qsl[s + 1] - q0;
  if (qn <= 0) return;
  const int p0 = n - qn;  // position of the first new token
  const int jl = (n - 1) / kPage;
  const int D = a.head_dim, Hkv = a.num_kv_heads;
  const int vpr = D / kPerVec;  // 16-byte vectors per row
  const int32_t* bt = a.block_table + int64_t(s) * a.max_pages;
  const E* kn = static_cast<const E*>(a.k_new);
  const E* vn = static_cast<const E*>(a.v_new);
  E* kp = static_cast<E*>(a.k_pool);
  E* vp = static_cast<E*>(a.v_pool);
  for (int j0 = p0 / kPage + int(blockIdx.z) * kAppendPages; j0 <= jl; j0 += int(gridDim.z) * kAppendPages)
  for (int j = j0; j <= min(jl, j0 + kAppendPages - 1); ++j) {
    const int lo = max(p0, j * kPage) - j * kPage, hi = min(n, (j + 1) * kPage) - j * kPage;  // slots [lo, hi)
    const int w = hi - lo;
    const int64_t blk = (int64_t(bt[j]) * Hkv + g) * D * kPage;  // (page, head) block, in elements
    for (int idx = threadIdx.x; idx < w * vpr; idx += blockDim.x) {
      const int it = idx / vpr, c = idx - it * vpr;
      const int t = lo + it;
      const int64_t row = (int64_t(q0 + j * kPage + t - p0) * Hkv + g) * D + c * kPerVec;  // new-token row
      *reinterpret_cast<u32x4_t*>(kp + blk + int64_t(t) * D + c * kPerVec) =
          *reinterpret_cast<const u32x4_t*>(kn + row);
      *reinterpret_cast<u32x4_t*>(tile + t * kPitch + c * kPerVec) = *reinterpret_cast<const u32x4_t*>(vn + row);
    }
    __syncthreads();
    if (w == kPage) {
      for (int idx = threadIdx.x; idx < D * (kPage / kPerVec); idx += blockDim.x) {
        const int d = idx / (kPage / kPerVec), t0 = (idx - d * (kPage / kPerVec)) * kPerVec;
        E e[kPerVec];
#pragma unroll
        for (int k = 0; k < kPerVec; ++k) e[k] = tile[(t0 + k) * kPitch + d];
        *reinterpret_cast<u32x4_t*>(vp + blk + int64_t(d) * kPage + t0) = __builtin_bit_cast(u32x4_t, e);
      }
    } else {
      for (int e = threadIdx.x; e < D * w; e += blockDim.x) {
        const int d = e / w, t = lo + (e - d * w);
        vp[blk + int64_t(d) * kPage + t] = tile[t * kPitch + d];
      }
    }
    __syncthreads();  // the tile is reused for the next page
  }
}

// ---------------------------------------------------------------------------
// Page-walk gather: dense[g][j][d] = pool element of key j of sequence seq.
// ---------------------------------------------------------------------------
template <typename E>
__global__ void gather_kernel(int which, int Hkv, int D, int max_pages, const E* pool, const int32_t* block_table,
                              const int32_t* seq_lens, int seq, int n_keys, E* dense) {
  const int64_t total = int64_t(Hkv) * n_keys * D;
  const int n_seq = seq_lens[seq];
  const int32_t* bt = block_table + int64_t(seq) * max_pages;
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < total; i += int64_t(gridDim.x) * blockDim.x) {
    const int d = int(i % D);
    const int j = int((i / D) % n_keys);
    const int g = int(i / (int64_t(D) * n_keys));
    if (j >= n_seq) {
      dense[i] = E(0);
      continue;
    }
    const int64_t pg = bt[j / kPage];
    const int slot = j % kPage;
    const int64_t src = which == 0 ? ((pg * Hkv + g) * kPage + slot) * D + d : ((pg * Hkv + g) * D + d) * kPage + slot;
    dense[i] = pool[src];
  }
}

// ---------------------------------------------------------------------------
// Content validation: sets *flag to 1 on the first inconsistency found.
// ---------------------------------------------------------------------------
__global__ void validate_kernel(int B, int T, int NP, int max_pages, int max_len, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* qsl, int32_t* flag) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s == 0 && (qsl[0] != 0 || qsl[B] != T)) atomicOr(flag, 1);
  if (s >= B) return;
  const int n = seq_lens[s];
  const int qn = qsl[s + 1] - qsl[s];
  if (qn < 0 || n < 0 || qn > n || n > max_len) {
    atomicOr(flag, 1);
    return;
  }
  const int pages = (n + kPage - 1) / kPage;
  if (pages > max_pages) {
    atomicOr(flag, 1);
    return;
  }
  for (int j = 0; j < pages; ++j) {
    const int pg = block_table[int64_t(s) * max_pages + j];
    if (pg < 0 || pg >= NP) {
      atomicOr(flag, 1);
      return;
    }
  }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

int launch_plan(const PlanArgs& a, void* stream) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kScanThreads), 0, as_stream(stream), a);
  return int(hipGetLastError());
}

int launch_plan_units(const PlanView& v, pa_plan_unit* units, int64_t max_units, void* stream) {
  hipLaunchKernelGGL(plan_units_kernel, dim3(1), dim3(64), 0, as_stream(stream), v, units, max_units);
  return int(hipGetLastError());
}

template <class TR>
static int launch_attn_t(const AttnArgs& a, int grid, void* stream) {
  hipLaunchKernelGGL(attention_kernel<TR>, dim3(grid), dim3(kThreads), 0, as_stream(stream), a);
  return int(hipGetLastError());
}

int launch_attention(const AttnArgs& a, int dtype, int D, int grid, void* stream) {
  if (dtype == PA_BF16) return D == 128 ? launch_attn_t<Bf16<128>>(a, grid, stream) : launch_attn_t<Bf16<64>>(a, grid, stream);
  return D == 128 ? launch_attn_t<F32<128>>(a, grid, stream) : launch_attn_t<F32<64>>(a, grid, stream);
}

template <class TR>
static int launch_fused_t(const AttnArgs& a, int grid, void* stream) {
  if (a.tree_mask)
    hipLaunchKernelGGL((attention_fused_kernel<TR, true>), dim3(grid), dim3(kThreads), 0, as_stream(stream), a);
  else
    hipLaunchKernelGGL((attention_fused_kernel<TR, false>), dim3(grid), dim3(kThreads), 0, as_stream(stream), a);
  return int(hipGetLastError());
}

int launch_attention_fused(const AttnArgs& a, int dtype, int D, int grid, void* stream, bool tall) {
  if (a.prior_lse) {  // causal masks only (the shared-prefix suffix pass)
    if (dtype == PA_BF16 && D == 128 && tall)
      hipLaunchKernelGGL((attention_fused_kernel<WithPrior<Bf16Tall<128>>, false>), dim3(grid), dim3(kThreads), 0,
                         as_stream(stream), a);
    else if (dtype == PA_BF16 && D == 128)
      hipLaunchKernelGGL((attention_fused_kernel<WithPrior<Bf16<128>>, false>), dim3(grid), dim3(kThreads), 0,
                         as_stream(stream), a);
    else if (dtype == PA_BF16)
      hipLaunchKernelGGL((attention_fused_kernel<WithPrior<Bf16<64>>, false>), dim3(grid), dim3(kThreads), 0,
                         as_stream(stream), a);
    else if (D == 128)
      hipLaunchKernelGGL((attention_fused_kernel<WithPrior<F32<128>>, false>), dim3(grid), dim3(kThreads), 0,
                         as_stream(stream), a);
    else
      hipLaunchKernelGGL((attention_fused_kernel<WithPrior<F32<64>>, false>), dim3(grid), dim3(kThreads), 0,
                         as_stream(stream), a);
    return int(hipGetLastError());
  }
  if (dtype == PA_BF16 && D == 128 && tall && !a.tree_mask) {
    hipLaunchKernelGGL((attention_fused_kernel<Bf16Tall<128>, false>), dim3(grid), dim3(kThreads), 0,
                       as_stream(stream), a);
    return int(hipGetLastError());
  }
  if (dtype == PA_BF16) return D == 128 ? launch_fused_t<Bf16<128>>(a, grid, stream) : launch_fused_t<Bf16<64>>(a, grid, stream);
  return D == 128 ? launch_fused_t<F32<128>>(a, grid, stream) : launch_fused_t<F32<64>>(a, grid, stream);
}

int launch_attention_fp8kv(const AttnArgs& a, int D, int grid, void* stream, bool tall) {
  if (D == 128 && tall)
    hipLaunchKernelGGL((attention_fused_kernel<Fp8KvTall<128>, false>), dim3(grid), dim3(kThreads), 0,
                       as_stream(stream), a);
  else if (D == 128)
    hipLaunchKernelGGL((attention_fused_kernel<Fp8Kv<128>, false>), dim3(grid), dim3(kThreads), 0,
                       as_stream(stream), a);
  else
    hipLaunchKernelGGL((attention_fused_kernel<Fp8Kv<64>, false>), dim3(grid), dim3(kThreads), 0,
                       as_stream(stream), a);
  return int(hipGetLastError());
}

// The staged and the single-launch kernels (with and without tree masks) run on the same grid (the
// smallest occupancy), so all cut the batch into the same grains and the staged and single-launch
// paths give bitwise identical results.
template <class TR>
static int blocks_per_cu_t() {
  int n = 0, m = 0, t = 0, h = 1 << 20;
  void (*staged)(AttnArgs) = attention_kernel<TR>;
  void (*fused)(AttnArgs) = attention_fused_kernel<TR, false>;
  void (*tree)(AttnArgs) = attention_fused_kernel<TR, true>;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(staged), kThreads, 0) !=
          hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&m, reinterpret_cast<const void*>(fused), kThreads, 0) !=
          hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&t, reinterpret_cast<const void*>(tree), kThreads, 0) !=
          hipSuccess)
    return -1;
  if constexpr (std::is_same<TR, Bf16<128>>::value) {  // the 128-row-block kernel shares the grid
    void (*tall)(AttnArgs) = attention_fused_kernel<Bf16Tall<128>, false>;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&h, reinterpret_cast<const void*>(tall), kThreads, 0) !=
        hipSuccess)
      return -1;
  }
  n = n < m ? n : m;
  n = n < h ? n : h;
  return n < t ? n : t;
}

__global__ void fill_zero_kernel(uint32_t* p, int64_t words) {
  for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < words; i += int64_t(gridDim.x) * blockDim.x)
    p[i] = 0u;
}

int launch_fill_zero(void* p, size_t bytes, void* stream) {
  const int64_t words = int64_t(bytes / 4);
  if (words == 0) return 0;
  int64_t grid = (words + 255) / 256;
  if (grid > 1024) grid = 1024;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(unsigned(grid)), dim3(256), 0, as_stream(stream),
                     static_cast<uint32_t*>(p), words);
  return int(hipGetLastError());
}

// Streaming read of one contiguous slice per workgroup (16-byte loads, four in flight per thread
// per pass), folded to one XOR word per workgroup.
__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4_t* __restrict__ buf, int64_t per,
                                                          uint32_t* sink) {
  const u32x4_t* b = buf + per * blockIdx.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (int64_t i = threadIdx.x; i < per; i += 4 * 256) {
    const u32x4_t z = {0u, 0u, 0u, 0u};
    const u32x4_t x0 = b[i];
    const u32x4_t x1 = i + 256 < per ? b[i + 256] : z;
    const u32x4_t x2 = i + 512 < per ? b[i + 512] : z;
    const u32x4_t x3 = i + 768 < per ? b[i + 768] : z;
    acc ^= x0 ^ x1 ^ x2 ^ x3;
  }
  uint32_t r = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) r ^= uint32_t(__shfl_xor(int(r), o));
  __shared__ uint32_t wx[4];
  if ((threadIdx.x & 63) == 0) wx[threadIdx.x >> 6] = r;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = wx[0] ^ wx[1] ^ wx[2] ^ wx[3];
}

int launch_read_stream(const void* buf, size_t bytes, int grid, uint32_t* sink, void* stream) {
  hipLaunchKernelGGL(read_stream_kernel, dim3(unsigned(grid)), dim3(256), 0, as_stream(stream),
                     static_cast<const u32x4_t*>(buf), int64_t(bytes / 16 / size_t(grid)), sink);
  return int(hipGetLastError());
}

template <class TR>
static int fp8_blocks_per_cu_t() {
  int n = 0;
  void (*fn)(AttnArgs) = attention_fused_kernel<TR, false>;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(fn), kThreads, 0) != hipSuccess)
    return -1;
  return n;
}

// bf16 descriptors also cover FP8 pages (bf16 q / out): their grid is the smaller of the two occupancies
int attention_blocks_per_cu(int dtype, int D) {
  if (dtype == PA_BF16) {
    const int a = D == 128 ? blocks_per_cu_t<Bf16<128>>() : blocks_per_cu_t<Bf16<64>>();
    const int b = D == 128 ? fp8_blocks_per_cu_t<Fp8Kv<128>>() : fp8_blocks_per_cu_t<Fp8Kv<64>>();
    const int c = D == 128 ? fp8_blocks_per_cu_t<Fp8KvTall<128>>() : b;
    if (a < 0 || b < 0 || c < 0) return -1;
    const int m = a < b ? a : b;
    return m < c ? m : c;
  }
  return D == 128 ? blocks_per_cu_t<F32<128>>() : blocks_per_cu_t<F32<64>>();
}

template <class TR>
static int launch_merge_planned_t(const MergeArgs& a, int grid, void* stream) {
  hipLaunchKernelGGL(merge_planned_kernel<TR>, dim3(grid), dim3(kThreads), 0, as_stream(stream), a);
  return int(hipGetLastError());
}

int launch_merge_planned(const MergeArgs& a, int dtype, int D, int grid, void* stream) {
  if (dtype == PA_BF16)
    return D == 128 ? launch_merge_planned_t<Bf16<128>>(a, grid, stream) : launch_merge_planned_t<Bf16<64>>(a, grid, stream);
  return D == 128 ? launch_merge_planned_t<F32<128>>(a, grid, stream) : launch_merge_planned_t<F32<64>>(a, grid, stream);
}

template <class TR>
static int launch_merge_t(int n_parts, int64_t rows, const float* o, const float* l, void* out, float* lse,
                          void* stream) {
  const int64_t threads = rows * (TR::D / 4);
  const int64_t grid = (threads + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(merge_kernel<TR>, dim3(unsigned(grid)), dim3(kThreads), 0, as_stream(stream), n_parts, rows, o,
                     l, out, lse);
  return int(hipGetLastError());
}

int launch_merge(int n_parts, int64_t rows, int D, const float* o_parts, const float* lse_parts, int out_dtype,
                 void* out, float* lse, void* stream) {
  if (rows == 0) return 0;
  if (out_dtype == PA_BF16)
    return D == 128 ? launch_merge_t<Bf16<128>>(n_parts, rows, o_parts, lse_parts, out, lse, stream)
                    : launch_merge_t<Bf16<64>>(n_parts, rows, o_parts, lse_parts, out, lse, stream);
  return D == 128 ? launch_merge_t<F32<128>>(n_parts, rows, o_parts, lse_parts, out, lse, stream)
                  : launch_merge_t<F32<64>>(n_parts, rows, o_parts, lse_parts, out, lse, stream);
}

int launch_gather(int which, int dtype, int Hkv, int D, int max_pages, const void* pool, const int32_t* block_table,
                  const int32_t* seq_lens, int seq, int n_keys, void* dense, void* stream) {
  const int64_t total = int64_t(Hkv) * n_keys * D;
  if (total == 0) return 0;
  int64_t grid = (total + 255) / 256;
  if (grid > 4096) grid = 4096;
  if (dtype == PA_BF16)
    hipLaunchKernelGGL(gather_kernel<uint16_t>, dim3(unsigned(grid)), dim3(256), 0, as_stream(stream), which, Hkv, D,
                       max_pages, static_cast<const uint16_t*>(pool), block_table, seq_lens, seq, n_keys,
                       static_cast<uint16_t*>(dense));
  else
    hipLaunchKernelGGL(gather_kernel<uint32_t>, dim3(unsigned(grid)), dim3(256), 0, as_stream(stream), which, Hkv, D,
                       max_pages, static_cast<const uint32_t*>(pool), block_table, seq_lens, seq, n_keys,
                       static_cast<uint32_t*>(dense));
  return int(hipGetLastError());
}

int launch_append_kv(const AppendArgs& a, int dtype, int num_seqs, int num_q_tokens, void* stream) {
  if (num_seqs == 0) return 0;
  // a sequence's new tokens touch at most ceil(T_q / 16) + 1 pages
  const int max_pages = (num_q_tokens + kPage - 1) / kPage + 1;
  // page groups per (sequence, head): enough for the longest possible window, but no more than keeps
  // the grid near 4096 workgroups (most windows are short; the kernel strides over the rest)
  int groups = (max_pages + kAppendPages - 1) / kAppendPages;
  const int64_t base = int64_t(num_seqs) * a.num_kv_heads;
  const int cap = int(base >= 4096 ? 1 : 4096 / base);
  if (groups > cap) groups = cap;
  if (groups > 65535) groups = 65535;
  const dim3 grid(unsigned(num_seqs), unsigned(a.num_kv_heads), unsigned(groups));
  if (dtype == PA_BF16)
    hipLaunchKernelGGL(append_kv_kernel<uint16_t>, grid, dim3(256), 0, as_stream(stream), a);
  else
    hipLaunchKernelGGL(append_kv_kernel<uint32_t>, grid, dim3(256), 0, as_stream(stream), a);
  return int(hipGetLastError());
}

// ---------------------------------------------------------------------------
// Shared-prefix batches: derive the two passes of the cascade.  Group g (sequences
// group_start[g] .. group_start[g+1]-1, contiguous, whose block tables agree on their first
// prefix_len[g] / 16 entries) becomes one sequence of the prefix pass: prefix_len[g] keys (the
// first member's pages) and all the group's query tokens, every row seeing every key.  Every
// sequence of the suffix pass keeps its queries and sees its keys from prefix_len onwards.
// ---------------------------------------------------------------------------
// Every output element has its own thread (grid-strided): the groups' prefix windows, their
// block-table rows (one entry per thread), each sequence's suffix length and key base (its group
// found by a binary search of group_start), and the prefix pass's zeroed results.
__global__ void prefix_prep_kernel(PrefixPrep a) {
  const int64_t tid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t nthreads = int64_t(gridDim.x) * blockDim.x;
  const cptr<int32_t> gs = ro(a.group_start), pl = ro(a.prefix_len);
  for (int64_t g = tid; g < a.num_groups; g += nthreads) {
    a.pre_seq_lens[g] = pl[g];
    a.pre_qsl[g] = a.qsl[gs[g]];
    if (g == a.num_groups - 1) a.pre_qsl[a.num_groups] = a.qsl[gs[a.num_groups]];
  }
  const int64_t bt_entries = int64_t(a.num_groups) * a.max_pages;
  for (int64_t i = tid; i < bt_entries; i += nthreads) {
    const int g = int(i / a.max_pages), j = int(i - int64_t(g) * a.max_pages);
    a.pre_bt[i] = j < pl[g] / kPage ? a.block_table[int64_t(gs[g]) * a.max_pages + j] : -1;
  }
  for (int64_t s = tid; s < a.num_seqs; s += nthreads) {
    int lo = 0, hi = a.num_groups - 1;  // the last g with group_start[g] <= s
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (gs[mid] <= s) lo = mid;
      else hi = mid - 1;
    }
    const int P = pl[lo];
    a.suf_seq_lens[s] = a.seq_lens[s] - P;
    a.key_base[s] = P;
  }
  // rows of a group without a shared prefix are never written by the prefix pass: they count as
  // having seen no key there
  for (int64_t i = tid; i < a.rows; i += nthreads) a.pre_lse[i] = -INFINITY;
  for (int64_t i = tid; i < a.rows * a.head_dim; i += nthreads) a.pre_o[i] = 0.f;
}

int launch_prefix_prep(const PrefixPrep& a, void* stream) {
  int64_t work = a.rows * a.head_dim;
  if (work < int64_t(a.num_groups) * a.max_pages) work = int64_t(a.num_groups) * a.max_pages;
  if (work < a.num_seqs) work = a.num_seqs;
  int64_t grid = (work + 255) / 256;
  if (grid > 2048) grid = 2048;
  if (grid < 1) grid = 1;
  hipLaunchKernelGGL(prefix_prep_kernel, dim3(unsigned(grid)), dim3(256), 0, as_stream(stream), a);
  return int(hipGetLastError());
}

int launch_validate(const pa_desc& d, const int32_t* block_table, const int32_t* seq_lens, const int32_t* qsl,
                    int32_t* flag, void* stream) {
  const int grid = d.num_seqs > 0 ? (d.num_seqs + 255) / 256 : 1;
  // a sequence may not exceed the stated max_seq_len, or (none stated) its block-table row
  const int max_len = d.max_seq_len > 0 ? d.max_seq_len : d.max_pages_per_seq * kPage;
  hipLaunchKernelGGL(validate_kernel, dim3(grid), dim3(256), 0, as_stream(stream), d.num_seqs, d.num_q_tokens,
                     d.num_pages, d.max_pages_per_seq, max_len, block_table, seq_lens, qsl, flag);
  return int(hipGetLastError());
}

}  // namespace pa
