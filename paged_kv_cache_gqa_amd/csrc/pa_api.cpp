// pa_api.cpp -- host side of the C ABI declared in include/pa.h: descriptor
// checks, workspace sizing, and the launches of the gfx950 kernels.
#include <hip/hip_runtime.h>

#include <cfloat>
#include <cmath>
#include <cstring>
#include <atomic>
#include <mutex>

#include "pa_internal.h"

namespace {

using pa::WsLayout;

struct DeviceInfo {
  std::atomic<bool> ready{false};
  int cus = 0;
  int blocks_per_cu[2][2] = {{0, 0}, {0, 0}};  // [dtype][D == 128]
  int max_grid = 0;                             // largest grid over dtypes and head dims
};

constexpr int kMaxDevices = 64;
std::mutex g_mu;
DeviceInfo g_dev[kMaxDevices];

// Compute units of the current device and how many attention workgroups each holds.
pa_status device_grid(const pa_desc& d, int* grid, int* max_grid = nullptr) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  DeviceInfo& info = g_dev[dev];
  if (info.ready.load(std::memory_order_acquire)) {
    *grid = info.cus * info.blocks_per_cu[d.dtype == PA_BF16 ? 1 : 0][d.head_dim == 128 ? 1 : 0];
    if (max_grid) *max_grid = info.max_grid;
    return PA_OK;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!info.ready.load(std::memory_order_relaxed)) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return PA_ERR_HIP;
    for (int dt = 0; dt < 2; ++dt)
      for (int big = 0; big < 2; ++big) {
        const int n = pa::attention_blocks_per_cu(dt, big ? 128 : 64);
        if (n <= 0) return PA_ERR_HIP;
        info.blocks_per_cu[dt][big] = n;
        if (cus * n > info.max_grid) info.max_grid = cus * n;
      }
    info.cus = cus;
    info.ready.store(true, std::memory_order_release);
  }
  *grid = info.cus * info.blocks_per_cu[d.dtype == PA_BF16 ? 1 : 0][d.head_dim == 128 ? 1 : 0];
  if (max_grid) *max_grid = info.max_grid;
  return PA_OK;
}

struct Ws {
  WsLayout L;
  pa_plan_header* hdr;
  int32_t* arrive;
  int64_t* seq_cost;
  pa::SlotStart* slots;
  float* part_lse;
  float* part_o;
  pa_plan_unit* units;
};

Ws carve(void* base, const WsLayout& L) {
  char* b = static_cast<char*>(base);
  Ws w;
  w.L = L;
  w.hdr = reinterpret_cast<pa_plan_header*>(b + L.header);
  w.arrive = reinterpret_cast<int32_t*>(b + L.arrive);
  w.seq_cost = reinterpret_cast<int64_t*>(b + L.seq_cost);
  w.slots = reinterpret_cast<pa::SlotStart*>(b + L.slots);
  w.part_lse = reinterpret_cast<float*>(b + L.part_lse);
  w.part_o = reinterpret_cast<float*>(b + L.part_o);
  w.units = reinterpret_cast<pa_plan_unit*>(b + L.units);
  return w;
}

// Descriptor + workspace checks shared by the staged entry points.
pa_status prepare(const pa_desc* desc, void* workspace, size_t workspace_bytes, int* grid, Ws* ws) {
  if (!desc) return PA_ERR_NULL_POINTER;
  const pa_status st = pa_check_desc(desc);
  if (st != PA_OK) return st;
  if (!workspace) return PA_ERR_NULL_POINTER;
  if (reinterpret_cast<uintptr_t>(workspace) & 255) return PA_ERR_BAD_SHAPE;
  int max_grid = 0;
  const pa_status gs = device_grid(*desc, grid, &max_grid);
  if (gs != PA_OK) return gs;
  const WsLayout L = pa::ws_layout(*desc, *grid, max_grid);
  if (workspace_bytes < L.total) return PA_ERR_WORKSPACE_TOO_SMALL;
  *ws = carve(workspace, L);
  return PA_OK;
}

pa::PlanView plan_view(const pa_desc& d, const int32_t* seq_lens, const int32_t* qsl, const Ws& ws) {
  pa::PlanView v;
  v.seq_lens = seq_lens;
  v.qsl = qsl;
  v.hdr = ws.hdr;
  v.seq_cost = ws.seq_cost;
  v.slots = ws.slots;
  v.num_seqs = d.num_seqs;
  v.num_kv_heads = d.num_kv_heads;
  v.group = d.num_q_heads / d.num_kv_heads;
  v.full_rows = 0;
  return v;
}

pa::AttnArgs attn_args(const pa_desc& d, const void* q, const void* k, const void* v, const int32_t* bt,
                       const int32_t* sl, const int32_t* qsl, void* out, float* lse, const Ws& ws) {
  pa::AttnArgs a = pa::single_launch_args(d, q, k, v, bt, sl, qsl, out, lse, ws.part_o, ws.part_lse, ws.arrive);
  a.plan = plan_view(d, sl, qsl, ws);
  return a;
}

}  // namespace

namespace pa {

pa_status attention_grid(const pa_desc& d, int* grid) { return device_grid(d, grid); }

// 128-row row blocks for bf16 batches at head dim 128 with at least one 64-row block of query rows
// per workgroup of the grid (T_q x Hq >= 64 x grid): with that much prefill work, twice the MFMA
// work per K/V byte read from LDS outweighs the extra pieces of the longer units (measured on
// MI355X: long prefill tile 344 -> 279 us, 4 x 1024-token windows 62 -> 58 us; configuration 3's
// prefill, 272 blocks of 64 rows on a 512-workgroup grid, 31.8 -> 38.8 us with 128-row blocks).
bool tall_blocks(const pa_desc& d, int grid) {
  return d.dtype == PA_BF16 && d.head_dim == 128 &&
         int64_t(d.num_q_tokens) * d.num_q_heads >= int64_t(kBlockRows) * grid;
}

AttnArgs single_launch_args(const pa_desc& d, const void* q, const void* k, const void* v, const int32_t* bt,
                            const int32_t* sl, const int32_t* qsl, void* out, float* lse, float* part_o,
                            float* part_lse, int32_t* arrive) {
  AttnArgs a;
  a.plan.seq_lens = sl;
  a.plan.qsl = qsl;
  a.plan.hdr = nullptr;  // the single launch plans in-kernel: no stored plan
  a.plan.seq_cost = nullptr;
  a.plan.slots = nullptr;
  a.plan.num_seqs = d.num_seqs;
  a.plan.num_kv_heads = d.num_kv_heads;
  a.plan.group = d.num_q_heads / d.num_kv_heads;
  a.plan.full_rows = 0;
  a.q = q;
  a.k_pool = k;
  a.v_pool = v;
  a.block_table = bt;
  a.out = out;
  a.lse = lse;
  a.part_o = part_o;
  a.part_lse = part_lse;
  a.tree_mask = nullptr;
  a.k_scale = nullptr;
  a.v_scale = nullptr;
  a.key_base = nullptr;
  a.out_f32 = nullptr;
  a.prior_o = nullptr;
  a.prior_lse = nullptr;
  a.arrive = arrive;
  a.num_q_heads = d.num_q_heads;
  a.max_pages = d.max_pages_per_seq;
  // Scores are taken in the base-2 domain with the positive factor |scale| * log2(e); a negative
  // scale flips Q's sign bits instead.  scale == 0 makes every score 0: Q is cleared (q_keep = 0)
  // and the factor set to 1, so that masked keys (-inf) never meet a zero factor (-inf * 0 = NaN).
  // A factor below the smallest normal float counts as 0: the kernels' fp32 arithmetic flushes it
  // to zero, and scores that small are 0 to fp32 precision anyway (their exponentials round to 1).
  const float f = std::fabs(d.scale) * 1.44269504088896340736f;
  const bool zero = !(f >= FLT_MIN);
  a.scale_log2 = zero ? 1.f : f;
  a.q_sign = !zero && d.scale < 0.f ? (d.dtype == PA_BF16 ? 0x80008000u : 0x80000000u) : 0u;
  a.q_keep = zero ? 0u : 0xFFFFFFFFu;
  return a;
}

}  // namespace pa

extern "C" {

int pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_status_str(pa_status s) { return pa_status_string(s); }

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL_POINTER: return "PA_ERR_NULL_POINTER: a required pointer is NULL";
    case PA_ERR_BAD_SHAPE: return "PA_ERR_BAD_SHAPE: inconsistent sizes in the descriptor";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: head_dim must be 64 or 128, page_size 16, dtype f32 or bf16";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "PA_ERR_WORKSPACE_TOO_SMALL: workspace smaller than pa_workspace_size";
    case PA_ERR_HIP: return "PA_ERR_HIP: a HIP runtime call or kernel launch failed";
    case PA_ERR_INVALID_CONTENT: return "PA_ERR_INVALID_CONTENT: seq_lens / query_start_loc / block_table inconsistent";
  }
  return "unknown pa_status";
}

pa_status pa_check_desc(const pa_desc* d) {
  if (!d) return PA_ERR_NULL_POINTER;
  if (d->num_seqs < 0 || d->num_q_tokens < 0 || d->num_q_heads < 1 || d->num_kv_heads < 1) return PA_ERR_BAD_SHAPE;
  if (d->num_q_heads % d->num_kv_heads != 0) return PA_ERR_BAD_SHAPE;
  if (d->num_pages < 1 || d->max_pages_per_seq < 1) return PA_ERR_BAD_SHAPE;
  if (d->max_seq_len < 0 || int64_t(d->max_seq_len) > int64_t(d->max_pages_per_seq) * PA_PAGE_SIZE)
    return PA_ERR_BAD_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (d->page_size != PA_PAGE_SIZE) return PA_ERR_UNSUPPORTED;
  if (d->dtype != PA_F32 && d->dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (!std::isfinite(d->scale)) return PA_ERR_BAD_SHAPE;
  // row and offset arithmetic in the kernels is 32-bit per sequence / 64-bit for addresses
  if (int64_t(d->num_q_tokens) * d->num_q_heads > (int64_t(1) << 31) - 1) return PA_ERR_BAD_SHAPE;
  if (int64_t(d->max_pages_per_seq) * PA_PAGE_SIZE > (int64_t(1) << 30)) return PA_ERR_BAD_SHAPE;
  return PA_OK;
}

pa_status pa_workspace_size(const pa_desc* desc, size_t* bytes) {
  if (!desc || !bytes) return PA_ERR_NULL_POINTER;
  const pa_status st = pa_check_desc(desc);
  if (st != PA_OK) return st;
  int grid = 0, max_grid = 0;
  const pa_status gs = device_grid(*desc, &grid, &max_grid);
  if (gs != PA_OK) return gs;
  *bytes = pa::ws_layout(*desc, grid, max_grid).total;
  return PA_OK;
}

size_t pa_workspace_bytes(const pa_desc* desc) {
  size_t n = 0;
  return pa_workspace_size(desc, &n) == PA_OK ? n : 0;
}

pa_status pa_plan(const pa_desc* desc, const int32_t* seq_lens, const int32_t* qsl, void* workspace,
                  size_t workspace_bytes, void* stream) {
  int grid = 0;
  Ws ws;
  const pa_status st = prepare(desc, workspace, workspace_bytes, &grid, &ws);
  if (st != PA_OK) return st;
  if (desc->num_seqs > 0 && (!seq_lens || !qsl)) return PA_ERR_NULL_POINTER;
  pa::PlanArgs a;
  a.seq_lens = seq_lens;
  a.qsl = qsl;
  a.hdr = ws.hdr;
  a.seq_cost = ws.seq_cost;
  a.slots = ws.slots;
  a.arrive = ws.arrive;
  a.full_rows = 0;
  a.num_seqs = desc->num_seqs;
  a.num_kv_heads = desc->num_kv_heads;
  a.group = desc->num_q_heads / desc->num_kv_heads;
  a.grid = grid;
  return pa::launch_plan(a, stream) == 0 ? PA_OK : PA_ERR_HIP;
}

pa_status pa_attention_planned(const pa_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_table, const int32_t* seq_lens, const int32_t* qsl, void* out,
                               float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  int grid = 0;
  Ws ws;
  const pa_status st = prepare(desc, workspace, workspace_bytes, &grid, &ws);
  if (st != PA_OK) return st;
  if (desc->num_q_tokens == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !qsl || !out || !lse) return PA_ERR_NULL_POINTER;
  const pa::AttnArgs a = attn_args(*desc, q, k_pool, v_pool, block_table, seq_lens, qsl, out, lse, ws);
  return pa::launch_attention(a, desc->dtype, desc->head_dim, grid, stream) == 0 ? PA_OK : PA_ERR_HIP;
}

pa_status pa_merge_planned(const pa_desc* desc, const int32_t* seq_lens, const int32_t* qsl, void* out, float* lse,
                           void* workspace, size_t workspace_bytes, void* stream) {
  int grid = 0;
  Ws ws;
  const pa_status st = prepare(desc, workspace, workspace_bytes, &grid, &ws);
  if (st != PA_OK) return st;
  if (desc->num_q_tokens == 0) return PA_OK;
  if (!seq_lens || !qsl || !out || !lse) return PA_ERR_NULL_POINTER;
  pa::MergeArgs m;
  m.plan = plan_view(*desc, seq_lens, qsl, ws);
  m.part_o = ws.part_o;
  m.part_lse = ws.part_lse;
  m.out = out;
  m.lse = lse;
  m.num_q_heads = desc->num_q_heads;
  // one workgroup per grain boundary
  return pa::launch_merge_planned(m, desc->dtype, desc->head_dim, grid, stream) == 0 ? PA_OK : PA_ERR_HIP;
}

namespace {
pa_status single_launch(const pa_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_table, const int32_t* seq_lens, const int32_t* qsl,
                        const uint64_t* tree_mask, void* out, float* lse, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!desc) return PA_ERR_NULL_POINTER;
  const pa_status st = pa_check_desc(desc);
  if (st != PA_OK) return st;
  if (desc->num_q_tokens == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !qsl || !out || !lse || !workspace)
    return PA_ERR_NULL_POINTER;
  int grid = 0;
  Ws ws;
  const pa_status ps = prepare(desc, workspace, workspace_bytes, &grid, &ws);
  if (ps != PA_OK) return ps;
  pa::AttnArgs a = attn_args(*desc, q, k_pool, v_pool, block_table, seq_lens, qsl, out, lse, ws);
  a.tree_mask = tree_mask;
  return pa::launch_attention_fused(a, desc->dtype, desc->head_dim, grid, stream, pa::tall_blocks(*desc, grid)) == 0
             ? PA_OK
             : PA_ERR_HIP;
}
}  // namespace

pa_status pa_attention(const pa_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_table, const int32_t* seq_lens, const int32_t* qsl, void* out, float* lse,
                       void* workspace, size_t workspace_bytes, void* stream) {
  return single_launch(desc, q, k_pool, v_pool, block_table, seq_lens, qsl, nullptr, out, lse, workspace,
                       workspace_bytes, stream);
}

namespace {
// Shared-prefix batches: after the attention workspace come the two passes' derived arrays and
// their fp32 results (part 0: prefix pass, part 1: suffix pass).
struct PrefixWs {
  int32_t *pre_seq_lens, *pre_qsl, *pre_bt, *suf_seq_lens, *key_base;
  float *part_lse, *part_o;
  size_t total;
};
PrefixWs prefix_layout(const pa_desc& d, int G, size_t base, void* ws) {
  const size_t B = size_t(d.num_seqs), rows = size_t(d.num_q_tokens) * size_t(d.num_q_heads);
  size_t off = base;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += pa::align256(bytes > 0 ? bytes : 1);
    return static_cast<char*>(ws) + o;
  };
  PrefixWs p;
  p.pre_seq_lens = reinterpret_cast<int32_t*>(take(4 * size_t(G)));
  p.pre_qsl = reinterpret_cast<int32_t*>(take(4 * (size_t(G) + 1)));
  p.pre_bt = reinterpret_cast<int32_t*>(take(4 * size_t(G) * size_t(d.max_pages_per_seq)));
  p.suf_seq_lens = reinterpret_cast<int32_t*>(take(4 * B));
  p.key_base = reinterpret_cast<int32_t*>(take(4 * B));
  p.part_lse = reinterpret_cast<float*>(take(4 * 2 * rows));
  p.part_o = reinterpret_cast<float*>(take(4 * 2 * rows * size_t(d.head_dim)));
  p.total = off;
  return p;
}
}  // namespace

pa_status pa_shared_prefix_workspace_size(const pa_desc* desc, int32_t num_groups, size_t* bytes) {
  if (!desc || !bytes) return PA_ERR_NULL_POINTER;
  size_t base = 0;
  const pa_status st = pa_workspace_size(desc, &base);
  if (st != PA_OK) return st;
  if (num_groups < 0 || num_groups > desc->num_seqs) return PA_ERR_BAD_SHAPE;
  *bytes = prefix_layout(*desc, num_groups, base, nullptr).total;
  return PA_OK;
}

pa_status pa_attention_shared_prefix(const pa_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* block_table, const int32_t* seq_lens, const int32_t* qsl,
                                     int32_t num_groups, const int32_t* group_start, const int32_t* prefix_len,
                                     void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (!desc) return PA_ERR_NULL_POINTER;
  const pa_status st = pa_check_desc(desc);
  if (st != PA_OK) return st;
  if (desc->num_q_tokens == 0) return PA_OK;
  if (num_groups < 1 || num_groups > desc->num_seqs) return PA_ERR_BAD_SHAPE;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !qsl || !group_start || !prefix_len || !out ||
      !lse || !workspace)
    return PA_ERR_NULL_POINTER;
  int grid = 0;
  Ws ws;
  const pa_status ps = prepare(desc, workspace, workspace_bytes, &grid, &ws);
  if (ps != PA_OK) return ps;
  const PrefixWs pw = prefix_layout(*desc, num_groups, ws.L.total, workspace);
  if (workspace_bytes < pw.total) return PA_ERR_WORKSPACE_TOO_SMALL;
  const int64_t rows = int64_t(desc->num_q_tokens) * desc->num_q_heads;
  pa::PrefixPrep pp;
  pp.group_start = group_start;
  pp.prefix_len = prefix_len;
  pp.seq_lens = seq_lens;
  pp.qsl = qsl;
  pp.block_table = block_table;
  pp.pre_seq_lens = pw.pre_seq_lens;
  pp.pre_qsl = pw.pre_qsl;
  pp.pre_bt = pw.pre_bt;
  pp.suf_seq_lens = pw.suf_seq_lens;
  pp.key_base = pw.key_base;
  pp.pre_o = pw.part_o;
  pp.pre_lse = pw.part_lse;
  pp.rows = rows;
  pp.num_seqs = desc->num_seqs;
  pp.num_groups = num_groups;
  pp.max_pages = desc->max_pages_per_seq;
  pp.head_dim = desc->head_dim;
  if (pa::launch_prefix_prep(pp, stream) != 0) return PA_ERR_HIP;
  // prefix pass: one sequence per group, every row sees the whole shared prefix
  pa_desc dp = *desc;
  dp.num_seqs = num_groups;
  pa::AttnArgs a = attn_args(dp, q, k_pool, v_pool, pw.pre_bt, pw.pre_seq_lens, pw.pre_qsl, out, pw.part_lse, ws);
  a.plan.full_rows = 1;
  a.out_f32 = pw.part_o;
  if (pa::launch_attention_fused(a, desc->dtype, desc->head_dim, grid, stream, pa::tall_blocks(dp, grid)) != 0)
    return PA_ERR_HIP;
  // suffix pass: every sequence from the end of its prefix on, causal as usual; each row's final
  // output folds in the prefix pass's result for it (log-sum-exp weights), so no merge launch follows
  pa::AttnArgs b = attn_args(*desc, q, k_pool, v_pool, block_table, pw.suf_seq_lens, qsl, out, lse, ws);
  b.key_base = pw.key_base;
  b.prior_o = pw.part_o;
  b.prior_lse = pw.part_lse;
  return pa::launch_attention_fused(b, desc->dtype, desc->head_dim, grid, stream, pa::tall_blocks(*desc, grid)) == 0
             ? PA_OK
             : PA_ERR_HIP;
}

pa_status pa_attention_fp8kv(const pa_desc* desc, const void* q, const uint8_t* k_pool, const uint8_t* v_pool,
                             const float* k_scale, const float* v_scale, const int32_t* block_table,
                             const int32_t* seq_lens, const int32_t* qsl, void* out, float* lse, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!desc) return PA_ERR_NULL_POINTER;
  const pa_status st = pa_check_desc(desc);
  if (st != PA_OK) return st;
  if (desc->dtype != PA_BF16) return PA_ERR_UNSUPPORTED;  // q and out are bf16
  if (desc->num_q_tokens == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !k_scale || !v_scale || !block_table || !seq_lens || !qsl || !out || !lse ||
      !workspace)
    return PA_ERR_NULL_POINTER;
  int grid = 0;
  Ws ws;
  const pa_status ps = prepare(desc, workspace, workspace_bytes, &grid, &ws);
  if (ps != PA_OK) return ps;
  pa::AttnArgs a = attn_args(*desc, q, k_pool, v_pool, block_table, seq_lens, qsl, out, lse, ws);
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  return pa::launch_attention_fp8kv(a, desc->head_dim, grid, stream, pa::tall_blocks(*desc, grid)) == 0 ? PA_OK
                                                                                                      : PA_ERR_HIP;
}

pa_status pa_attention_tree(const pa_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, const int32_t* seq_lens, const int32_t* qsl,
                            const uint64_t* tree_mask, void* out, float* lse, void* workspace, size_t workspace_bytes,
                            void* stream) {
  if (desc && desc->num_q_tokens > 0 && !tree_mask) return PA_ERR_NULL_POINTER;
  return single_launch(desc, q, k_pool, v_pool, block_table, seq_lens, qsl, tree_mask, out, lse, workspace,
                       workspace_bytes, stream);
}

pa_status pa_workspace_init(const pa_desc* desc, void* workspace, size_t workspace_bytes, void* stream) {
  int grid = 0;
  Ws ws;
  const pa_status st = prepare(desc, workspace, workspace_bytes, &grid, &ws);
  if (st != PA_OK) return st;
  return pa::launch_fill_zero(ws.arrive, ws.L.seq_cost - ws.L.arrive, stream) == 0 ? PA_OK : PA_ERR_HIP;
}

pa_status pa_plan_read(const pa_desc* desc, const int32_t* seq_lens, const int32_t* qsl, void* workspace,
                       size_t workspace_bytes, pa_plan_header* header, pa_plan_unit* units, int32_t max_units,
                       void* stream) {
  int grid = 0;
  Ws ws;
  if (!header) return PA_ERR_NULL_POINTER;
  if (max_units > 0 && !units) return PA_ERR_NULL_POINTER;
  const pa_status st = prepare(desc, workspace, workspace_bytes, &grid, &ws);
  if (st != PA_OK) return st;
  if (desc->num_seqs > 0 && (!seq_lens || !qsl)) return PA_ERR_NULL_POINTER;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(header, ws.hdr, sizeof(pa_plan_header), hipMemcpyDeviceToHost, s) != hipSuccess) return PA_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return PA_ERR_HIP;
  const int64_t cap = ws.L.max_units;
  int64_t n = header->n_units < max_units ? header->n_units : max_units;
  if (n > cap) n = cap;
  if (n > 0) {
    if (pa::launch_plan_units(plan_view(*desc, seq_lens, qsl, ws), ws.units, cap, stream) != 0) return PA_ERR_HIP;
    if (hipMemcpyAsync(units, ws.units, sizeof(pa_plan_unit) * size_t(n), hipMemcpyDeviceToHost, s) != hipSuccess)
      return PA_ERR_HIP;
    if (hipStreamSynchronize(s) != hipSuccess) return PA_ERR_HIP;
  }
  return PA_OK;
}

pa_status pa_gather_kv(const pa_desc* desc, int32_t which, const void* pool, const int32_t* block_table,
                       const int32_t* seq_lens, int32_t seq, int32_t n_keys, void* dense_out, void* stream) {
  if (!desc) return PA_ERR_NULL_POINTER;
  const pa_status st = pa_check_desc(desc);
  if (st != PA_OK) return st;
  if (which != 0 && which != 1) return PA_ERR_BAD_SHAPE;
  if (seq < 0 || seq >= desc->num_seqs || n_keys < 0 || n_keys > desc->max_pages_per_seq * PA_PAGE_SIZE)
    return PA_ERR_BAD_SHAPE;
  if (n_keys == 0) return PA_OK;
  if (!pool || !block_table || !seq_lens || !dense_out) return PA_ERR_NULL_POINTER;
  return pa::launch_gather(which, desc->dtype, desc->num_kv_heads, desc->head_dim, desc->max_pages_per_seq, pool,
                           block_table, seq_lens, seq, n_keys, dense_out, stream) == 0
             ? PA_OK
             : PA_ERR_HIP;
}

pa_status pa_merge(int32_t n_parts, int64_t rows, int32_t head_dim, const float* o_parts, const float* lse_parts,
                   int32_t out_dtype, void* out, float* lse, void* stream) {
  if (n_parts < 1 || rows < 0) return PA_ERR_BAD_SHAPE;
  if (head_dim != 64 && head_dim != 128) return PA_ERR_UNSUPPORTED;
  if (out_dtype != PA_F32 && out_dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (rows == 0) return PA_OK;
  if (!o_parts || !lse_parts || !out || !lse) return PA_ERR_NULL_POINTER;
  return pa::launch_merge(n_parts, rows, head_dim, o_parts, lse_parts, out_dtype, out, lse, stream) == 0 ? PA_OK
                                                                                                        : PA_ERR_HIP;
}

pa_status pa_append_kv(const pa_desc* desc, const void* k_new, const void* v_new, const int32_t* block_table,
                       const int32_t* seq_lens, const int32_t* qsl, void* k_pool, void* v_pool, void* stream) {
  if (!desc) return PA_ERR_NULL_POINTER;
  const pa_status st = pa_check_desc(desc);
  if (st != PA_OK) return st;
  if (desc->num_seqs == 0 || desc->num_q_tokens == 0) return PA_OK;
  if (!k_new || !v_new || !block_table || !seq_lens || !qsl || !k_pool || !v_pool) return PA_ERR_NULL_POINTER;
  if (desc->num_kv_heads > 65535) return PA_ERR_BAD_SHAPE;  // grid y
  pa::AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.qsl = qsl;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.num_kv_heads = desc->num_kv_heads;
  a.head_dim = desc->head_dim;
  a.max_pages = desc->max_pages_per_seq;
  return pa::launch_append_kv(a, desc->dtype, desc->num_seqs, desc->num_q_tokens, stream) == 0 ? PA_OK : PA_ERR_HIP;
}

pa_status pa_validate(const pa_desc* desc, const int32_t* block_table, const int32_t* seq_lens, const int32_t* qsl,
                      void* workspace, size_t workspace_bytes, void* stream) {
  if (!desc) return PA_ERR_NULL_POINTER;
  const pa_status st = pa_check_desc(desc);
  if (st != PA_OK) return st;
  if (!workspace || !qsl || (desc->num_seqs > 0 && (!block_table || !seq_lens))) return PA_ERR_NULL_POINTER;
  if (workspace_bytes < 256) return PA_ERR_WORKSPACE_TOO_SMALL;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int32_t* flag = static_cast<int32_t*>(workspace);
  if (pa::launch_fill_zero(flag, sizeof(int32_t), stream) != 0) return PA_ERR_HIP;
  if (pa::launch_validate(*desc, block_table, seq_lens, qsl, flag, stream) != 0) return PA_ERR_HIP;
  int32_t host = 0;
  if (hipMemcpyAsync(&host, flag, sizeof(int32_t), hipMemcpyDeviceToHost, s) != hipSuccess) return PA_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return PA_ERR_HIP;
  return host ? PA_ERR_INVALID_CONTENT : PA_OK;
}

pa_status pa_read_stream(const void* buf, size_t bytes, int32_t grid, uint32_t* sink, void* stream) {
  if (!buf || !sink) return PA_ERR_NULL_POINTER;
  if (grid < 1 || grid > 65535 || bytes == 0 || bytes % (size_t(16) * size_t(grid)) != 0) return PA_ERR_BAD_SHAPE;
  return pa::launch_read_stream(buf, bytes, grid, sink, stream) == 0 ? PA_OK : PA_ERR_HIP;
}

}  // extern "C"
