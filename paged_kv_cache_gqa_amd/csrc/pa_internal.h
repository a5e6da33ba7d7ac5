// pa_internal.h -- constants, kernel argument blocks and the workspace layout
// shared by the host API (pa_api.cpp) and the gfx950 kernels (pa_kernels.hip).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pa.h"

namespace pa {

constexpr int kPage = PA_PAGE_SIZE;  // token slots per page
constexpr int kChunkKeys = 32;       // keys per chunk = two pages = one 16x16x32 MFMA K-step of PV
constexpr int kWaves = 4;            // waves per workgroup
constexpr int kThreads = 64 * kWaves;
constexpr int kSplitRows = 32;       // a unit with <= 32 rows splits its chunks across the 4 waves
// Row-split units are blocks of 4 waves x 16 kRowTiles rows.  The staged path and most batches use
// one row tile per wave (64-row blocks): twice the units of two row tiles means half the pieces
// per split unit, so half the partial results written and merged (config-3-sized prefill: 31.8
// against 38.8 us with 128-row blocks).  Batches with a lot of prefill work run a kernel with two
// row tiles per wave (128-row blocks: twice the MFMA work per K/V byte read from LDS and per
// chunk's DMA, page-table and loop instructions; the long prefill tile 344 -> 279 us).
constexpr int kBlockRows = 64;      // rows of a staged-path row block
constexpr int kMaxBlockRows = 128;  // rows of the largest row block of any kernel
// The row-split geometry of a kernel, one template integer for the planner: the cost weight of a
// row-split chunk (low byte) and the row tiles per wave (a block has 64 x tiles rows).
constexpr int row_geom(int weight, int tiles) { return weight | (tiles << 8); }
constexpr int rg_weight(int rg) { return rg & 255; }
constexpr int rg_rows(int rg) { return 64 * (rg >> 8); }
constexpr int kPlanThreads = 1024;

// Cost weights per 32-key chunk on the planner's balancing axis, fitted to
// measured wall time on MI355X (mixed prefill + decode batch): a chunk of a
// row-split unit (prefill: up to 64 rows of MFMA work on one chunk staged in
// LDS) takes about as long as a chunk of a key-split unit (decode / verify:
// one wave streams 8 KiB of K and 8 KiB of V from HBM for a few rows).  A chunk of a 128-row
// unit weighs twice as much (8: of 4, 8 and 16 the fastest on prefill-heavy mixed batches).
constexpr int kCostKeySplit = 4;
constexpr int kCostRowSplit = 4;
constexpr int kRgDefault = row_geom(kCostRowSplit, 1);  // the staged planner's geometry
// FP8 pages change the ratio: a key-split chunk moves half the bytes, while a row-split chunk also
// widens its K and V fragments to bf16 before the MFMAs.  Fitted on MI355X (the mixed prefill +
// decode batch with FP8 pages, µs per launch, three runs each on one machine): row-split weight
// 6: 68.8, 7: 65.7, 8: 65.0, 9: 65.3, 10: 66.5, 11: 67.7 (with the two-instruction widening of
// codes to bf16 the optimum was 10; 4, bf16's weight, took 90.9).
constexpr int kCostRowSplitFp8 = 8;
static_assert((kCostKeySplit & (kCostKeySplit - 1)) == 0 && (kCostRowSplit & (kCostRowSplit - 1)) == 0 &&
                  (kCostRowSplitFp8 & (kCostRowSplitFp8 - 1)) == 0,
              "chunk weights are powers of two (the kernels divide by them with shifts)");
// Fixed cost charged at the start of every unit (row and page-table loads, the
// pipeline fill, the cross-wave merge and the output), so that grains that start
// many units get fewer chunks.  Fitted on MI355X (bench.py, configurations 2-5):
// a key-split unit of one row tile (decode; units stream back to back) and a
// 64-row block cost about 8 chunks more than their chunks, a key-split unit of
// two row tiles (verify) about 12.
constexpr int kCostStartKs1 = 32;
constexpr int kCostStartKs2 = 48;
constexpr int kCostStartRow = 32;
inline __host__ __device__ int unit_start_cost(bool key_split, int rows) {
  return key_split ? (rows <= 16 ? kCostStartKs1 : kCostStartKs2) : kCostStartRow;
}

// The cost axis is cut into S equal grains, one per workgroup (measured on
// MI355X: more, smaller grains per workgroup only added merge work), with
//   S = min(grid, Ck / kCostKeySplit + Cr / (kRowGrainChunks * rw))
// for Ck, Cr the total cost of key-split and of row-split units (rw: the row-split chunk weight of
// the page format): decode work
// may be cut down to one chunk per grain (its partial results are a few rows),
// prefill work no finer than kRowGrainChunks chunks per grain (a piece of a
// 128-row unit leaves 64 KiB of partial state to merge).  Grain boundaries --
// and so every split of a unit's keys and its partial-result slots -- depend
// only on the batch shape and the grid.
// No grain is shorter than a row-split chunk's weight rw (>= kCostKeySplit): S <= (Ck + Cr) / rw.
// A shorter grain could lie between two chunk starts of a unit and so hold an empty piece of it,
// which never arrives at the unit's merge (with rw = 8, FP8 pages or 128-row blocks, the first
// term alone allows grains of ~4 in small batches of mostly decode work).
constexpr int kRowGrainChunks = 8;
inline __host__ __device__ int64_t grain_count(int64_t ck, int64_t cr, int grid, int rw = kCostRowSplit) {
  int64_t s = ck / kCostKeySplit + cr / (int64_t(kRowGrainChunks) * rw);
  if (cr > 0 && s > (ck + cr) / rw) s = (ck + cr) / rw;
  if (s > grid) s = grid;
  if (s < 1 && ck + cr > 0) s = 1;
  return s;
}

// Where grain k starts: its cost range and the unit holding cost c0, as written by the planner.
struct SlotStart {
  int64_t c0, c1;
  int64_t seq_base;    // cost at which sequence s starts
  int64_t unit_cost0;  // cost at which unit (s, g, rb) starts
  int32_t s, g, rb;
  int32_t n, qn;       // seq_lens[s], query count of s
  int32_t q0;          // query_start_loc[s]
  int32_t pad[2];
};

// Arguments shared by the kernels that walk the plan.
struct PlanView {
  const int32_t* seq_lens;
  const int32_t* qsl;
  const pa_plan_header* hdr;
  const int64_t* seq_cost;  // [B+1]: cost at which sequence s's units start; seq_cost[B] = total
  const SlotStart* slots;   // [max grains]
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t group;      // Hq / Hkv
  int32_t full_rows;  // 1: every row of a sequence sees all its keys (no causal limit)
};

struct AttnArgs {
  PlanView plan;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  void* out;
  float* lse;
  float* part_o;    // [grains][2][128][D]: per grain, the piece of its first and of its last unit
  float* part_lse;  // [grains][2][128]
  const uint64_t* tree_mask;  // [T_q] per-row window masks, or null for the causal rule
  const float* k_scale;       // [NP][Hkv] FP8 pages: scale of each (page, kv head), else null
  const float* v_scale;
  const int32_t* key_base;    // [B] or null: sequence s's keys start at key key_base[s] (a multiple of 16)
                              // of its block-table row; seq_lens then count keys from there
  float* out_f32;             // [T_q][Hq][D] or null: final results go here in fp32 instead of to out
  const float* prior_o;       // [T_q][Hq][D] and [T_q][Hq] fp32, read by kernels of a trait with kPrior only:
  const float* prior_lse;     // each row's result over other keys, folded into its final output (log-sum-exp)
  int32_t* arrive;  // [grains]: pieces of the split unit whose first piece is in grain k that have
                    // finished (single-launch path; zero between calls)
  int32_t num_q_heads;
  int32_t max_pages;
  float scale_log2;  // |scale| * log2(e): scores live in the base-2 domain
  uint32_t q_sign;   // xor applied to Q's bits: the sign bits when scale < 0, else 0
  uint32_t q_keep;   // and applied to Q's bits first: 0 when scale == 0 (every score 0), else all ones
};

struct PlanArgs {
  const int32_t* seq_lens;
  const int32_t* qsl;
  pa_plan_header* hdr;
  int64_t* seq_cost;
  SlotStart* slots;
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t group;
  int32_t grid;  // workgroups of the persistent attention launch
  int32_t* arrive;  // zeroed for a following single-launch call
  int32_t full_rows;
};

struct MergeArgs {
  PlanView plan;
  const float* part_o;
  const float* part_lse;
  void* out;
  float* lse;
  int32_t num_q_heads;
};

struct AppendArgs {
  const void* k_new;  // [T_q][Hkv][D]
  const void* v_new;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* qsl;
  void* k_pool;
  void* v_pool;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t max_pages;
};

struct PrefixPrep {
  const int32_t* group_start;  // [G+1]
  const int32_t* prefix_len;   // [G]
  const int32_t* seq_lens;
  const int32_t* qsl;
  const int32_t* block_table;
  int32_t* pre_seq_lens;  // [G]
  int32_t* pre_qsl;       // [G+1]
  int32_t* pre_bt;        // [G][max_pages]
  int32_t* suf_seq_lens;  // [B]
  int32_t* key_base;      // [B]
  float* pre_o;           // [rows][D]
  float* pre_lse;         // [rows]
  int64_t rows;           // T_q * Hq
  int32_t num_seqs;       // B = group_start[num_groups]
  int32_t num_groups;
  int32_t max_pages;
  int32_t head_dim;
};

// Workspace: [header | arrival counters | per-sequence cost prefix | grain starts | partial lse |
// partial o | unit list (plan inspection only)], every region 256-byte aligned.  The arrival
// counters must be zero before a single-launch call; every call leaves them zero.
struct WsLayout {
  size_t header, arrive, seq_cost, slots, part_lse, part_o, units, total;
  int64_t partial_rows, max_units;
};

constexpr size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Rows of one partial position: the largest unit.
constexpr int kPartRows = kMaxBlockRows;

// grid: workgroups of the attention launch for d; max_grid: the largest such grid of any dtype /
// head dim on the device (the arrival counters sit at a fixed offset with a fixed size, so one
// workspace serves every descriptor it is large enough for).
inline WsLayout ws_layout(const pa_desc& d, int grid, int max_grid) {
  WsLayout L{};
  const int64_t B = d.num_seqs > 0 ? d.num_seqs : 0;
  const int64_t T = d.num_q_tokens > 0 ? d.num_q_tokens : 0;
  const int64_t G = d.num_kv_heads > 0 ? d.num_q_heads / d.num_kv_heads : 1;
  // staged-plan units per sequence = Hkv * (1 if q_len*G <= 32 else ceil(q_len*G/64))
  L.max_units = int64_t(d.num_kv_heads) * (B + (T * G + kBlockRows - 1) / kBlockRows);
  const int64_t grains = grid;
  L.partial_rows = grains * 2 * kPartRows;
  size_t off = 0;
  L.header = off;   off += align256(sizeof(pa_plan_header));
  L.arrive = off;   off += align256(sizeof(int32_t) * size_t(max_grid > 0 ? max_grid : 1));
  L.seq_cost = off; off += align256(sizeof(int64_t) * size_t(B + 1));
  L.slots = off;    off += align256(sizeof(SlotStart) * size_t(grains > 0 ? grains : 1));
  L.part_lse = off; off += align256(sizeof(float) * size_t(L.partial_rows));
  L.part_o = off;   off += align256(sizeof(float) * size_t(L.partial_rows) * size_t(d.head_dim));
  L.units = off;    off += align256(sizeof(pa_plan_unit) * size_t(L.max_units > 0 ? L.max_units : 1));
  L.total = off;
  return L;
}

}  // namespace pa

// Launchers implemented in pa_kernels.hip (return hipError_t as int).
namespace pa {
int launch_plan(const PlanArgs& a, void* stream);
int launch_attention(const AttnArgs& a, int dtype, int head_dim, int grid, void* stream);
// single launch: in-kernel planning of each grain and merge of split units by their last piece
// tall: bf16 at head dim 128 without tree masks runs the kernel with 128-row row blocks
int launch_attention_fused(const AttnArgs& a, int dtype, int head_dim, int grid, void* stream, bool tall = false);
// single launch over FP8 E4M3 pages (bf16 q / out; a.k_scale, a.v_scale set)
int launch_attention_fp8kv(const AttnArgs& a, int head_dim, int grid, void* stream, bool tall = false);
int launch_fill_zero(void* p, size_t bytes, void* stream);
int launch_read_stream(const void* buf, size_t bytes, int grid, uint32_t* sink, void* stream);
int launch_merge_planned(const MergeArgs& a, int dtype, int head_dim, int grid, void* stream);
int launch_plan_units(const PlanView& v, pa_plan_unit* units, int64_t max_units, void* stream);
int launch_gather(int which, int dtype, int Hkv, int D, int max_pages, const void* pool,
                  const int32_t* block_table, const int32_t* seq_lens, int seq, int n_keys, void* dense,
                  void* stream);
int launch_merge(int n_parts, int64_t rows, int D, const float* o_parts, const float* lse_parts,
                 int out_dtype, void* out, float* lse, void* stream);
// pages of one sequence per workgroup of the append kernel
constexpr int kAppendPages = 2;
int launch_append_kv(const AppendArgs& a, int dtype, int num_seqs, int num_q_tokens, void* stream);
int launch_prefix_prep(const PrefixPrep& a, void* stream);
int launch_validate(const pa_desc& d, const int32_t* block_table, const int32_t* seq_lens,
                    const int32_t* qsl, int32_t* flag, void* stream);
// Workgroups per CU the attention kernel can hold (occupancy query), or < 0 on error.
int attention_blocks_per_cu(int dtype, int head_dim);
// Host side (pa_api.cpp): the single launch's grid for d on the current device, and its arguments
// with the partial results and arrival counters at the given device addresses.
pa_status attention_grid(const pa_desc& d, int* grid);
// whether the single launch runs 128-row row blocks for d on a grid of `grid` workgroups
bool tall_blocks(const pa_desc& d, int grid);
AttnArgs single_launch_args(const pa_desc& d, const void* q, const void* k, const void* v, const int32_t* bt,
                            const int32_t* sl, const int32_t* qsl, void* out, float* lse, float* part_o,
                            float* part_lse, int32_t* arrive);
}  // namespace pa
