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
//    32) and PV as O^T = V^T . P^T (16 d x 16 rows, 32 keys per MFMA).  Every
//    MFMA operand is one 16-byte load per lane straight from the pool: K pages
//    are [slot][D], V pages are stored [D][slot] so the key axis that PV reduces
//    over is contiguous.  Nothing is transposed in LDS.
//  * QK MFMA half h takes its 16 key rows from page h of the chunk, so every
//    load of a chunk is (uniform page base) + (one 32-bit lane offset) +
//    (immediate).  After the C-layout write-back lane (row n, quad q) holds the
//    scores of keys 4q..4q+3 of both pages; those 8 values are exactly the
//    lane's B operand of the PV MFMA (element j = key 16*(j/4) + 4q + j%4), so
//    softmax needs no cross-lane data movement beyond two xor-shuffles for the
//    row maximum.
//  * Rows are (window token, head in group) pairs, so the G query heads that
//    share a K/V head -- and all tokens of a verify window or prefill block --
//    read each K/V byte once.
//  * One persistent launch of (#CU x workgroups per CU) workgroups walks a
//    work list on one cost axis cut into equal slices (stream-K style); a
//    workgroup's slice can span several units and split a unit's keys, in
//    which case it writes partial (o, lse) rows that the merge kernel combines.
//    Decode/verify units (<= 32 rows) let the 4 waves take alternate chunks
//    and merge in LDS; prefill units (<= 128 rows) give each wave 32 rows and
//    stage each chunk once in LDS for all 4 waves.
//  * Workgroup k runs on XCD k % 8; slots are renumbered so that consecutive
//    slices (which share K/V pages of one sequence) sit on one XCD's L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

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

__device__ __forceinline__ pa_plan_unit load_unit(cptr<pa_plan_unit> p) {
  pa_plan_unit u;
  u.seq = p->seq;
  u.kv_head = p->kv_head;
  u.row0 = p->row0;
  u.n_rows = p->n_rows;
  u.n_keys = p->n_keys;
  u.n_chunks = p->n_chunks;
  u.kind = p->kind;
  u.cost_weight = p->cost_weight;
  u.cost0 = p->cost0;
  u.piece_base = p->piece_base;
  u.n_pieces = p->n_pieces;
  return u;
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ f32x4_t as_f32x4(u32x4_t v) { return __builtin_bit_cast(f32x4_t, v); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  __bf16 x = (__bf16)a, y = (__bf16)b;  // v_cvt_pk_bf16_f32, round to nearest even
  return uint32_t(__builtin_bit_cast(uint16_t, x)) | (uint32_t(__builtin_bit_cast(uint16_t, y)) << 16);
}

// Chunk-relative key of element j (0..7) of the P operand held by a lane of quad q:
// QK half j/4 read page j/4, and the C layout gives the lane MFMA rows 4q..4q+3.
__device__ __forceinline__ int p_key(int j, int quad) { return 16 * (j >> 2) + 4 * quad + (j & 3); }

__device__ __forceinline__ uint2 ld8(const char* p) { return *reinterpret_cast<const uint2*>(p); }

// ---------------------------------------------------------------------------
// Element types.  A "fragment" is the 16 bytes one lane feeds to one MFMA
// operand slot (bf16: 8 values; fp32: 4 values).
// ---------------------------------------------------------------------------

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
  __device__ static f32x4_t qk(const u32x4_t* kf, int h, const u32x4_t* qf) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
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
  __device__ static void store_out(char* dst, f32x4_t o) {  // 4 consecutive d
    uint2 v;
    v.x = pack_bf16x2(o[0], o[1]);
    v.y = pack_bf16x2(o[2], o[3]);
    *reinterpret_cast<uint2*>(dst) = v;
  }
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

  __device__ static int q_off(int f, int quad) { return (16 * f + 4 * quad) * kEb; }
  __device__ static uint32_t k_lane(int lane) { return uint32_t(((lane & 15) * D + 4 * (lane >> 4)) * kEb); }
  __device__ static uint32_t v_lane(int lane) { return uint32_t(((lane & 15) * kPage + 4 * (lane >> 4)) * kEb); }
  __device__ static u32x4_t load_frag(const char* k0, const char* k1, const char* v0, const char* v1, uint32_t kl,
                                      uint32_t vl, int f) {
    if (f < kKF) return ld16((f < D / 16 ? k0 : k1) + kl + (f % (D / 16)) * 16 * kEb);
    const int g = f - kKF;
    return ld16(((g & 1) ? v1 : v0) + vl + (g >> 1) * 16 * kPage * kEb);
  }
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
  __device__ static void store_out(char* dst, f32x4_t o) { *reinterpret_cast<f32x4_t*>(dst) = o; }
};

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

template <class TR>
__device__ __forceinline__ ChunkPages chunk_pages(const AttnArgs& A, cptr<int32_t> bt_row, int kvh, int c,
                                                  int n_seq) {
  const int key0 = c * kChunkKeys;
  const int pa = __builtin_amdgcn_readfirstlane(bt_row[2 * c]);
  const int pb = key0 + kPage < n_seq ? __builtin_amdgcn_readfirstlane(bt_row[2 * c + 1]) : pa;
  const int64_t blk = int64_t(kPage) * TR::D * TR::kEb;  // bytes of one (page, head) block
  const int64_t hkv = A.num_kv_heads;
  ChunkPages cp;
  cp.k0 = static_cast<const char*>(A.k_pool) + (int64_t(pa) * hkv + kvh) * blk;
  cp.k1 = static_cast<const char*>(A.k_pool) + (int64_t(pb) * hkv + kvh) * blk;
  cp.v0 = static_cast<const char*>(A.v_pool) + (int64_t(pa) * hkv + kvh) * blk;
  cp.v1 = static_cast<const char*>(A.v_pool) + (int64_t(pb) * hkv + kvh) * blk;
  return cp;
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
__device__ __forceinline__ void load_v(const ChunkPages& cp, uint32_t kl, uint32_t vl, u32x4_t (&vf)[TR::kVF]) {
#pragma unroll
  for (int f = 0; f < TR::kVF; ++f) vf[f] = frag<TR>(cp, kl, vl, TR::kKF + f);
}

// Scores of one chunk for every row tile, masked, folded into the online softmax.
// Returns the P operands; rescales O by exp2(m_old - m_new).
// `getq(rt, qf)` fills the Q fragments of row tile rt (from registers or LDS).
template <class TR, int RT, class GetQ>
__device__ __forceinline__ void softmax_chunk(State<TR, RT>& st, GetQ getq, const u32x4_t (&kf)[TR::kKF], int key0,
                                              const int (&p_row)[RT], bool mask, float sl2, int lane,
                                              typename TR::PFrag (&pf)[RT]) {
  const int quad = lane >> 4;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    u32x4_t qf[TR::kQF];
    getq(rt, qf);
    const f32x4_t s0 = TR::qk(kf, 0, qf);
    const f32x4_t s1 = TR::qk(kf, 1, qf);
    float x[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[e] = s0[e] * sl2;
      x[4 + e] = s1[e] * sl2;
    }
    if (mask) {
      const int lim = p_row[rt] - key0;  // element j visible iff its key <= lim
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = p_key(j, quad) <= lim ? x[j] : -INFINITY;
    }
    float mx = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) mx = fmaxf(mx, x[j]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(st.m[rt], mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(st.m[rt] - m_use);
    float p[8];
    float sum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = fast_exp2(x[j] - m_use);
      sum += p[j];
    }
    st.l[rt] = st.l[rt] * alpha + sum;
    st.m[rt] = m_new;
#pragma unroll
    for (int t = 0; t < TR::kTiles; ++t) st.o[rt][t] *= alpha;
    pf[rt] = TR::make_p(p);
  }
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
  const int t = rr / A.group;
  const int hh = rr - t * A.group;
  ri.tok = q0 + t;
  ri.head = U.kv_head * A.group + hh;
  ri.p = ri.valid ? n_seq - qn + t : -1;
  return ri;
}

template <class TR>
__device__ __forceinline__ u32x4_t load_q_frag(const AttnArgs& A, const RowInfo& ri, int f, int quad) {
  const char* base = static_cast<const char*>(A.q) + (int64_t(ri.tok) * A.num_q_heads + ri.head) * TR::D * TR::kEb;
  return ri.valid ? ld16(base + TR::q_off(f, quad)) : u32x4_t{0u, 0u, 0u, 0u};
}

// Final (normalised) output of one row tile's 4 d values at tile t, or a partial row.
template <class TR>
__device__ __forceinline__ void emit(const AttnArgs& A, const pa_plan_unit& U, const RowInfo& ri, int r, int piece,
                                     int t, int quad, f32x4_t o, float lse_nat, bool write_lse) {
  if (!ri.valid) return;
  const int d = 16 * t + 4 * quad;
  if (U.n_pieces <= 1) {
    char* dst = static_cast<char*>(A.out) + ((int64_t(ri.tok) * A.num_q_heads + ri.head) * TR::D + d) * TR::kEb;
    TR::store_out(dst, o);
    if (write_lse) A.lse[int64_t(ri.tok) * A.num_q_heads + ri.head] = lse_nat;
  } else {
    const int64_t prow = int64_t(U.piece_base) + int64_t(piece) * U.n_rows + r;
    *reinterpret_cast<f32x4_t*>(A.part_o + prow * TR::D + d) = o;
    if (write_lse) A.part_lse[prow] = lse_nat;
  }
}

// LDS: staging for row-split units (2 buffers x kNF fragments x 64 lanes) and
// the cross-wave merge of key-split units (4 waves x 2 row tiles x kTiles).
template <class TR>
struct Smem {
  static constexpr int kStage = 2 * TR::kNF * 64;            // u32x4 slots
  static constexpr int kMerge = kWaves * 2 * TR::kTiles * 64;  // f32x4 slots
  static constexpr int kSlots = kStage > kMerge ? kStage : kMerge;
  u32x4_t buf[kSlots];
  float stat[kWaves][2][2][16];  // [wave][row tile][m | l][row]
};

// ---------------------------------------------------------------------------
// Key-split unit (decode / verify, <= 32 rows): wave w takes chunks i0+w, i0+w+4, ...
// ---------------------------------------------------------------------------
template <class TR, int RT>
__device__ void run_keysplit(const AttnArgs& A, const pa_plan_unit& U, int i0, int i1, int piece, Smem<TR>& sm) {
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int quad = lane >> 4;
  const int s = U.seq;
  const int n_seq = ro(A.seq_lens)[s];
  const int q0 = ro(A.qsl)[s];
  const int qn = ro(A.qsl)[s + 1] - q0;
  const cptr<int32_t> bt_row = ro(A.block_table) + int64_t(s) * A.max_pages;

  RowInfo ri[RT];
  int p_row[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    ri[rt] = row_info(A, U, 16 * rt + (lane & 15), n_seq, q0, qn);
    p_row[rt] = ri[rt].p;
  }
  const int min_p = n_seq - qn + U.row0 / A.group;  // first row's last visible key

  // Q fragments live in this wave's slice of LDS (re-read every chunk; keeps VGPRs for K/V in flight)
  u32x4_t* qlds = sm.buf + w * (RT * TR::kQF * 64);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int f = 0; f < TR::kQF; ++f) qlds[(rt * TR::kQF + f) * 64 + lane] = load_q_frag<TR>(A, ri[rt], f, quad);
  auto getq = [&](int rt, u32x4_t (&qf)[TR::kQF]) {
#pragma unroll
    for (int f = 0; f < TR::kQF; ++f) qf[f] = qlds[(rt * TR::kQF + f) * 64 + lane];
  };
  State<TR, RT> st;
  state_init(st);

  const uint32_t kl = TR::k_lane(lane), vl = TR::v_lane(lane);
  int c = i0 + w;
  u32x4_t kf[TR::kKF];
  u32x4_t vf[TR::kVF];
  if (c < i1) {
    const ChunkPages cp = chunk_pages<TR>(A, bt_row, U.kv_head, c, n_seq);
    load_k<TR>(cp, kl, vl, kf);
    load_v<TR>(cp, kl, vl, vf);
  }
  for (; c < i1; c += kWaves) {
    const int key0 = c * kChunkKeys;
    const int cn = c + kWaves;
    ChunkPages cpn;
    if (cn < i1) cpn = chunk_pages<TR>(A, bt_row, U.kv_head, cn, n_seq);
    asm volatile("" ::: "memory");  // keep the Q reads inside the loop
    typename TR::PFrag pf[RT];
    softmax_chunk<TR, RT>(st, getq, kf, key0, p_row, key0 + kChunkKeys - 1 > min_p, A.scale_log2, lane, pf);
    if (cn < i1) load_k<TR>(cpn, kl, vl, kf);
    if (key0 + kChunkKeys > n_seq) TR::sanitize_v(vf, quad, n_seq - key0);
    pv_chunk<TR, RT>(st, vf, pf);
    if (cn < i1) load_v<TR>(cpn, kl, vl, vf);
  }
  __syncthreads();  // every wave is done with its Q slice before the merge buffer overwrites it

  // merge the 4 waves' states through LDS
  f32x4_t* obuf = reinterpret_cast<f32x4_t*>(sm.buf);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    float l = st.l[rt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
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
      emit<TR>(A, U, ri[rt], 16 * rt + n, piece, t, quad, o * inv, lse_nat, t == 0 && quad == 0);
    }
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------
// Row-split unit (prefill, <= 128 rows): wave w owns rows [32w, 32w+32); the
// workgroup stages each chunk once in LDS (double-buffered) for all 4 waves.
// ---------------------------------------------------------------------------
template <class TR>
__device__ void run_rowsplit(const AttnArgs& A, const pa_plan_unit& U, int i0, int i1, int piece, Smem<TR>& sm) {
  constexpr int RT = 2;
  constexpr int kPer = (TR::kNF + kWaves - 1) / kWaves;  // fragments each thread stages per chunk
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int quad = lane >> 4;
  const int s = U.seq;
  const int n_seq = ro(A.seq_lens)[s];
  const int q0 = ro(A.qsl)[s];
  const int qn = ro(A.qsl)[s + 1] - q0;
  const cptr<int32_t> bt_row = ro(A.block_table) + int64_t(s) * A.max_pages;
  const bool active = 32 * w < U.n_rows;

  RowInfo ri[RT];
  int p_row[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    ri[rt] = row_info(A, U, 32 * w + 16 * rt + (lane & 15), n_seq, q0, qn);
    p_row[rt] = ri[rt].p;
  }
  const int min_p = n_seq - qn + (U.row0 + 32 * w) / A.group;

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

  const uint32_t kl = TR::k_lane(lane), vl = TR::v_lane(lane);
  u32x4_t stage[kPer];
  auto fetch = [&](int c) {
    const ChunkPages cp = chunk_pages<TR>(A, bt_row, U.kv_head, c, n_seq);
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int f = w + kWaves * j;
      if (f < TR::kNF) stage[j] = frag<TR>(cp, kl, vl, f);
    }
  };
  auto deposit = [&](int b) {
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int f = w + kWaves * j;
      if (f < TR::kNF) sm.buf[(b * TR::kNF + f) * 64 + lane] = stage[j];
    }
  };

  fetch(i0);
  deposit(0);
  __syncthreads();
  for (int c = i0; c < i1; ++c) {
    const int b = (c - i0) & 1;
    const int key0 = c * kChunkKeys;
    if (c + 1 < i1) fetch(c + 1);
    if (active) {
      u32x4_t kf[TR::kKF];
#pragma unroll
      for (int f = 0; f < TR::kKF; ++f) kf[f] = sm.buf[(b * TR::kNF + f) * 64 + lane];
      typename TR::PFrag pf[RT];
      softmax_chunk<TR, RT>(st, getq, kf, key0, p_row, key0 + kChunkKeys - 1 > min_p, A.scale_log2, lane, pf);
      u32x4_t vf[TR::kVF];
#pragma unroll
      for (int f = 0; f < TR::kVF; ++f) vf[f] = sm.buf[(b * TR::kNF + TR::kKF + f) * 64 + lane];
      if (key0 + kChunkKeys > n_seq) TR::sanitize_v(vf, quad, n_seq - key0);
      pv_chunk<TR, RT>(st, vf, pf);
    }
    if (c + 1 < i1) deposit(b ^ 1);
    __syncthreads();
  }

  if (active) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      float l = st.l[rt];
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const float lse_nat = l > 0.f ? (st.m[rt] + fast_log2(l)) * kLn2 : -INFINITY;
#pragma unroll
      for (int t = 0; t < TR::kTiles; ++t)
        emit<TR>(A, U, ri[rt], 32 * w + 16 * rt + (lane & 15), piece, t, quad, st.o[rt][t] * inv, lse_nat,
                 t == 0 && quad == 0);
    }
  }
}

// slot_of(c): the slot whose slice [floor(k*C/S), floor((k+1)*C/S)) holds cost c
__device__ __forceinline__ int64_t slot_of(int64_t c, int64_t S, int64_t C) { return ((c + 1) * S - 1) / C; }
__device__ __forceinline__ int64_t slice_begin(int64_t k, int64_t S, int64_t C) { return k * C / S; }

// Renumber workgroups so that consecutive slots run on one XCD (workgroup b runs on XCD b % 8).
__device__ __forceinline__ int xcd_slot(int b, int S) {
  const int x = b & 7, k = b >> 3;
  const int per = S >> 3, rem = S & 7;
  return x * per + (x < rem ? x : rem) + k;
}

template <class TR>
__global__ __launch_bounds__(kThreads, 2) void attention_kernel(AttnArgs A) {
  __shared__ Smem<TR> sm;
  const cptr<pa_plan_header> hdr = ro(A.hdr);
  const cptr<pa_plan_unit> units = ro(A.units);
  const int S = hdr->n_slots;
  if (int(blockIdx.x) >= S) return;
  const int slot = xcd_slot(blockIdx.x, S);
  const int64_t C = hdr->total_cost;
  const int n_units = hdr->n_units;
  const int64_t c0 = slice_begin(slot, S, C);
  const int64_t c1 = slice_begin(slot + 1, S, C);
  if (c0 >= c1) return;
  // last unit whose cost0 <= c0
  int lo = 0, hi = n_units - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (units[mid].cost0 <= c0) lo = mid; else hi = mid - 1;
  }
  for (int u = lo; u < n_units; ++u) {
    const pa_plan_unit U = load_unit(units + u);
    if (U.cost0 >= c1) break;
    const int64_t w = U.cost_weight;
    const int i0 = int(c0 > U.cost0 ? (c0 - U.cost0 + w - 1) / w : 0);
    const int64_t e = (c1 - U.cost0 + w - 1) / w;
    const int i1 = int(e < U.n_chunks ? e : U.n_chunks);
    if (i0 >= i1) continue;
    const int piece = int(slot - slot_of(U.cost0, S, C));
    if (U.kind == 0) {
      if (U.n_rows <= 16) run_keysplit<TR, 1>(A, U, i0, i1, piece, sm);
      else run_keysplit<TR, 2>(A, U, i0, i1, piece, sm);
    } else {
      run_rowsplit<TR>(A, U, i0, i1, piece, sm);
    }
  }
}

// ---------------------------------------------------------------------------
// Planner: one workgroup of 1024 threads.
// ---------------------------------------------------------------------------
struct SeqShape {
  int units;
  int64_t cost;
};

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

// keys visible to the last row of row block rb of a sequence (n keys, qn tokens, G heads)
__device__ __forceinline__ int block_keys(int n, int qn, int G, int rb) {
  const int rows = qn * G;
  const int last = (min(kBlockRows * (rb + 1), rows) - 1) / G;
  return n - qn + last + 1;
}

__device__ SeqShape seq_shape(int n, int qn, int G, int Hkv) {
  SeqShape r{0, 0};
  if (qn <= 0) return r;
  const int rows = qn * G;
  if (rows <= kSplitRows) {
    r.units = Hkv;
    r.cost = int64_t(Hkv) * ceil_div(n, kChunkKeys) * kCostKeySplit;
  } else {
    const int nb = ceil_div(rows, kBlockRows);
    int64_t ch = 0;
    for (int rb = 0; rb < nb; ++rb) ch += ceil_div(block_keys(n, qn, G, rb), kChunkKeys);
    r.units = Hkv * nb;
    r.cost = int64_t(Hkv) * ch * kCostRowSplit;
  }
  return r;
}

// Inclusive block scan of one int64 per thread (kPlanThreads threads).
__device__ int64_t block_scan(int64_t v, int64_t* tmp) {
  const int t = threadIdx.x;
  tmp[t] = v;
  __syncthreads();
  for (int off = 1; off < kPlanThreads; off <<= 1) {
    const int64_t add = t >= off ? tmp[t - off] : 0;
    __syncthreads();
    tmp[t] += add;
    __syncthreads();
  }
  const int64_t r = tmp[t];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int64_t tmp[kPlanThreads];
  __shared__ int64_t tot_cost_s, tot_units_s;
  const int t = threadIdx.x;
  const int B = a.num_seqs;
  // phase 1: per-sequence unit counts and costs, exclusive prefixes
  int64_t carry_c = 0, carry_u = 0;
  for (int base = 0; base < B; base += kPlanThreads) {
    const int s = base + t;
    SeqShape sh{0, 0};
    if (s < B) sh = seq_shape(a.seq_lens[s], a.qsl[s + 1] - a.qsl[s], a.group, a.num_kv_heads);
    const int64_t ic = block_scan(sh.cost, tmp);
    const int64_t tc = tmp[kPlanThreads - 1 < B - base ? kPlanThreads - 1 : B - base - 1];
    __syncthreads();
    const int64_t iu = block_scan(sh.units, tmp);
    const int64_t tu = tmp[kPlanThreads - 1 < B - base ? kPlanThreads - 1 : B - base - 1];
    __syncthreads();
    if (s < B) {
      a.seq_cost[s] = carry_c + ic - sh.cost;
      a.seq_unit[s] = int32_t(carry_u + iu - sh.units);
    }
    carry_c += tc;
    carry_u += tu;
  }
  if (t == 0) {
    tot_cost_s = carry_c;
    tot_units_s = carry_u;
  }
  __syncthreads();
  // Capacity guard: the workspace is sized from the descriptor; inconsistent
  // seq_lens / query_start_loc contents could ask for more units -- plan nothing.
  if (tot_units_s > a.max_units) {
    if (t == 0) {
      a.hdr->n_units = 0;
      a.hdr->n_split = 0;
      a.hdr->n_slots = 0;
      a.hdr->grid = a.grid;
      a.hdr->total_cost = 0;
      a.hdr->partial_rows = 0;
    }
    return;
  }
  const int64_t C = tot_cost_s;
  const int n_units = int(tot_units_s);
  int64_t S = C / kCostMax;  // every slice at least one chunk of the heaviest kind wide
  if (S > a.grid) S = a.grid;
  if (S < 1 && C > 0) S = 1;
  // phase 2: write units
  for (int s = t; s < B; s += kPlanThreads) {
    const int n = a.seq_lens[s];
    const int qn = a.qsl[s + 1] - a.qsl[s];
    if (qn <= 0) continue;
    const int G = a.group;
    const int rows = qn * G;
    int64_t cost = a.seq_cost[s];
    int u = a.seq_unit[s];
    const bool split = rows <= kSplitRows;
    const int nb = split ? 1 : ceil_div(rows, kBlockRows);
    for (int g = 0; g < a.num_kv_heads; ++g) {
      for (int rb = 0; rb < nb; ++rb) {
        pa_plan_unit U;
        U.seq = s;
        U.kv_head = g;
        U.row0 = split ? 0 : rb * kBlockRows;
        U.n_rows = split ? rows : min(kBlockRows, rows - rb * kBlockRows);
        U.n_keys = split ? n : block_keys(n, qn, G, rb);
        U.n_chunks = ceil_div(U.n_keys, kChunkKeys);
        U.kind = split ? 0 : 1;
        U.cost_weight = split ? kCostKeySplit : kCostRowSplit;
        U.cost0 = cost;
        const int64_t last = cost + int64_t(U.n_chunks - 1) * U.cost_weight;
        U.n_pieces = int(((last + 1) * S - 1) / C - ((cost + 1) * S - 1) / C + 1);
        U.piece_base = 0;
        cost += int64_t(U.n_chunks) * U.cost_weight;
        a.units[u++] = U;
      }
    }
  }
  __syncthreads();
  // phase 3: partial-row storage and the list of split units
  int64_t carry_r = 0, carry_s = 0;
  for (int base = 0; base < n_units; base += kPlanThreads) {
    const int u = base + t;
    int64_t rows = 0, flag = 0;
    if (u < n_units) {
      const pa_plan_unit& U = a.units[u];
      if (U.n_pieces > 1) {
        rows = int64_t(U.n_pieces) * U.n_rows;
        flag = 1;
      }
    }
    const int last_t = kPlanThreads - 1 < n_units - base ? kPlanThreads - 1 : n_units - base - 1;
    const int64_t ir = block_scan(rows, tmp);
    const int64_t tr = tmp[last_t];
    __syncthreads();
    const int64_t is = block_scan(flag, tmp);
    const int64_t ts = tmp[last_t];
    __syncthreads();
    if (u < n_units) {
      a.units[u].piece_base = int32_t(carry_r + ir - rows);
      if (flag) a.split[carry_s + is - 1] = u;
    }
    carry_r += tr;
    carry_s += ts;
  }
  if (t == 0) {
    const bool fits = carry_r <= a.max_partial_rows;  // holds by construction; guards the workspace
    a.hdr->n_units = fits ? n_units : 0;
    a.hdr->n_split = fits ? int32_t(carry_s) : 0;
    a.hdr->n_slots = fits ? int32_t(S) : 0;
    a.hdr->grid = a.grid;
    a.hdr->total_cost = C;
    a.hdr->partial_rows = carry_r;
  }
}

// ---------------------------------------------------------------------------
// Log-sum-exp merge of partial rows: one workgroup per split unit (grid-stride).
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
  constexpr int kLanesPerRow = TR::D / 4;
  constexpr int kRowsPerPass = kThreads / kLanesPerRow;
  const int n_split = a.hdr->n_split;
  const int d4 = threadIdx.x % kLanesPerRow;
  for (int i = blockIdx.x; i < n_split; i += gridDim.x) {
    const pa_plan_unit U = a.units[a.split[i]];
    const int q0 = a.qsl[U.seq];
    for (int r = threadIdx.x / kLanesPerRow; r < U.n_rows; r += kRowsPerPass) {
      const int64_t prow = int64_t(U.piece_base) + r;
      float lse;
      f32x4_t o;
      merge_row<TR>(a.part_o + prow * TR::D, a.part_lse + prow, U.n_rows, U.n_pieces, d4, &lse, &o);
      const int rr = U.row0 + r;
      const int tk = rr / a.group;
      const int head = U.kv_head * a.group + (rr - tk * a.group);
      const int64_t orow = int64_t(q0 + tk) * a.num_q_heads + head;
      TR::store_out(static_cast<char*>(a.out) + (orow * TR::D + 4 * d4) * TR::kEb, o);
      if (d4 == 0) a.lse[orow] = lse;
    }
  }
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
__global__ void validate_kernel(int B, int T, int NP, int max_pages, const int32_t* block_table,
                                const int32_t* seq_lens, const int32_t* qsl, int32_t* flag) {
  const int s = blockIdx.x * blockDim.x + threadIdx.x;
  if (s == 0 && (qsl[0] != 0 || qsl[B] != T)) atomicOr(flag, 1);
  if (s >= B) return;
  const int n = seq_lens[s];
  const int qn = qsl[s + 1] - qsl[s];
  if (qn < 0 || n < 0 || qn > n) {
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
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, as_stream(stream), a);
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
static int blocks_per_cu_t() {
  int n = 0;
  void (*fn)(AttnArgs) = attention_kernel<TR>;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, reinterpret_cast<const void*>(fn), kThreads, 0) != hipSuccess)
    return -1;
  return n;
}

int attention_blocks_per_cu(int dtype, int D) {
  if (dtype == PA_BF16) return D == 128 ? blocks_per_cu_t<Bf16<128>>() : blocks_per_cu_t<Bf16<64>>();
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

int launch_validate(const pa_desc& d, const int32_t* block_table, const int32_t* seq_lens, const int32_t* qsl,
                    int32_t* flag, void* stream) {
  const int grid = d.num_seqs > 0 ? (d.num_seqs + 255) / 256 : 1;
  hipLaunchKernelGGL(validate_kernel, dim3(grid), dim3(256), 0, as_stream(stream), d.num_seqs, d.num_q_tokens,
                     d.num_pages, d.max_pages_per_seq, block_table, seq_lens, qsl, flag);
  return int(hipGetLastError());
}

}  // namespace pa
