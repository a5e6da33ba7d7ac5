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
constexpr int kBlockRows = 128;      // a larger unit is cut into blocks of 4 waves x 32 rows
constexpr int kPlanThreads = 1024;

// Cost weights per 32-key chunk on the planner's balancing axis.  A chunk of a
// key-split unit (decode / verify: one wave streams 8 KiB of K and 8 KiB of V
// from HBM) costs more wall time than a chunk of a row-split unit (prefill: the
// workgroup reads the chunk once and four waves spend MFMA time on it).
constexpr int kCostKeySplit = 4;
constexpr int kCostRowSplit = 1;
constexpr int kCostMax = kCostKeySplit > kCostRowSplit ? kCostKeySplit : kCostRowSplit;

struct AttnArgs {
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* qsl;
  void* out;
  float* lse;
  const pa_plan_header* hdr;
  const pa_plan_unit* units;
  float* part_o;    // [partial rows][D]
  float* part_lse;  // [partial rows]
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;  // Hq / Hkv
  int32_t max_pages;
  float scale_log2;  // scale * log2(e): scores live in the base-2 domain
};

struct PlanArgs {
  const int32_t* seq_lens;
  const int32_t* qsl;
  pa_plan_header* hdr;
  pa_plan_unit* units;
  int32_t* split;      // indices of units with n_pieces > 1
  int64_t* seq_cost;   // per-sequence exclusive cost prefix (scratch)
  int32_t* seq_unit;   // per-sequence exclusive unit prefix (scratch)
  int32_t num_seqs;
  int32_t num_kv_heads;
  int32_t group;
  int32_t grid;        // workgroups of the persistent attention launch
  int64_t max_units;         // capacity of `units` / `split`
  int64_t max_partial_rows;  // capacity of the partial-result arrays
};

struct MergeArgs {
  const int32_t* qsl;
  const pa_plan_header* hdr;
  const pa_plan_unit* units;
  const int32_t* split;
  const float* part_o;
  const float* part_lse;
  void* out;
  float* lse;
  int32_t num_q_heads;
  int32_t group;
};

// Workspace: [header | seq scratch | units | split list | partial lse | partial o],
// every region 256-byte aligned.
struct WsLayout {
  size_t header, seq_cost, seq_unit, units, split, part_lse, part_o, total;
  int64_t max_units, max_partial_rows;
};

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

inline WsLayout ws_layout(const pa_desc& d, int grid) {
  WsLayout L{};
  const int64_t B = d.num_seqs > 0 ? d.num_seqs : 0;
  const int64_t T = d.num_q_tokens > 0 ? d.num_q_tokens : 0;
  const int64_t G = d.num_kv_heads > 0 ? d.num_q_heads / d.num_kv_heads : 1;
  // units per sequence = Hkv * (1 if q_len*G <= 32 else ceil(q_len*G/128))
  L.max_units = int64_t(d.num_kv_heads) * (B + (T * G + kBlockRows - 1) / kBlockRows);
  // every (row, head) once, plus one extra piece of <= 128 rows per slot boundary
  L.max_partial_rows = T * d.num_q_heads + int64_t(grid) * kBlockRows;
  size_t off = 0;
  L.header = off;   off += align256(sizeof(pa_plan_header));
  L.seq_cost = off; off += align256(sizeof(int64_t) * size_t(B + 1));
  L.seq_unit = off; off += align256(sizeof(int32_t) * size_t(B + 1));
  L.units = off;    off += align256(sizeof(pa_plan_unit) * size_t(L.max_units > 0 ? L.max_units : 1));
  L.split = off;    off += align256(sizeof(int32_t) * size_t(L.max_units > 0 ? L.max_units : 1));
  L.part_lse = off; off += align256(sizeof(float) * size_t(L.max_partial_rows));
  L.part_o = off;   off += align256(sizeof(float) * size_t(L.max_partial_rows) * size_t(d.head_dim));
  L.total = off;
  return L;
}

}  // namespace pa

// Launchers implemented in pa_kernels.hip (return hipError_t as int).
namespace pa {
int launch_plan(const PlanArgs& a, void* stream);
int launch_attention(const AttnArgs& a, int dtype, int head_dim, int grid, void* stream);
int launch_merge_planned(const MergeArgs& a, int dtype, int head_dim, int grid, void* stream);
int launch_gather(int which, int dtype, int Hkv, int D, int max_pages, const void* pool,
                  const int32_t* block_table, const int32_t* seq_lens, int seq, int n_keys, void* dense,
                  void* stream);
int launch_merge(int n_parts, int64_t rows, int D, const float* o_parts, const float* lse_parts,
                 int out_dtype, void* out, float* lse, void* stream);
int launch_validate(const pa_desc& d, const int32_t* block_table, const int32_t* seq_lens,
                    const int32_t* qsl, int32_t* flag, void* stream);
// Workgroups per CU the attention kernel can hold (occupancy query), or < 0 on error.
int attention_blocks_per_cu(int dtype, int head_dim);
}  // namespace pa
