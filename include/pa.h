/*
 * pa.h -- C ABI of the MI355X (gfx950) paged-KV grouped-query attention library.
 *
 * One call computes causal grouped-query attention for a mixed batch of
 * prefill chunks, decode steps and speculative-verify windows whose keys and
 * values sit in fixed-size pages addressed through a block table, and returns
 * the output and the per-row log-sum-exp.
 *
 * Sources for what is computed:
 *   - XY-Serve verdict page, pith_extraction.key_machinery: the attention
 *     primitive is a tile of the matmul-softmax-matmul pattern over a set of
 *     query rows and a K/V length.
 *   - same page, core_discovery: prefill, decode and verify tokens are batched
 *     together; K/V live in a PagedAttention-style block cache; tiles that the
 *     causal mask makes empty are skipped.
 *   - same page, forward_implications: one kernel with row-wise mask control
 *     serves all three kinds of rows.
 *   - "Understanding Inference Scaling for LLMs" review, Reference graph [4]:
 *     grouped-query attention (a group of query heads shares one K/V head).
 *
 * For sequence s with n_s = seq_lens[s] keys and q_s = query_start_loc[s+1] -
 * query_start_loc[s] query tokens, window row i (query token
 * r = query_start_loc[s] + i) sits at absolute position p = n_s - q_s + i and
 * sees keys 0..p (bottom-right causal alignment; the new tokens' own K/V are
 * already in the pool).  Query head h reads K/V head h / (Hq / Hkv).
 *     out[r][h][:] = sum_j softmax_j(scale * q[r][h].k_j) v_j
 *     lse[r][h]    = ln sum_j exp(scale * q[r][h].k_j)          (natural log)
 *
 * Memory layout (all device memory, row-major, no padding):
 *   q            [T_q][Hq][D]          dtype      T_q = query_start_loc[B]
 *   k_pool       [NP][Hkv][16][D]      dtype      a page holds 16 token slots
 *   v_pool       [NP][Hkv][D][16]      dtype      the same pages with slots innermost
 *   block_table  [B][max_pages_per_seq] int32     physical page of logical page j of
 *                                                 sequence s; entries >= ceil(n_s/16)
 *                                                 are never read (pad with -1)
 *   seq_lens     [B]                   int32      keys per sequence (new tokens included)
 *   query_start_loc [B+1]              int32      0 = qsl[0] <= qsl[1] <= ... = T_q
 *   out          [T_q][Hq][D]          dtype
 *   lse          [T_q][Hq]             float32
 * Slots beyond n_s in a sequence's last page and pages no sequence uses may
 * hold any bits (NaN included); they never reach the result.
 *
 * Ownership and streams: the caller allocates and owns every buffer; the
 * library never allocates or frees device memory on these calls and keeps no
 * state between calls.  Work is enqueued on `stream` (a hipStream_t; NULL is
 * the default stream) and the call returns without waiting, except
 * pa_validate, which synchronizes.  Two calls that share a workspace must be
 * ordered on one stream.
 *
 * Errors: descriptor and pointer checks run on the host before anything is
 * enqueued and return a pa_status; a failed launch returns PA_ERR_HIP.  The
 * contents of seq_lens, query_start_loc and block_table are not checked on the
 * attention path (q_len > seq_len or a page id outside [0, NP) is undefined
 * behaviour there); pa_validate checks them.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 2
#define PA_PAGE_SIZE 16

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL_POINTER = 1,       /* a required pointer is NULL */
  PA_ERR_BAD_SHAPE = 2,          /* negative size, Hq % Hkv != 0, ... */
  PA_ERR_UNSUPPORTED = 3,        /* head_dim not 64/128, page_size not 16, unknown dtype */
  PA_ERR_WORKSPACE_TOO_SMALL = 4,
  PA_ERR_HIP = 5,                /* a HIP runtime call or kernel launch failed */
  PA_ERR_INVALID_CONTENT = 6     /* pa_validate found bad seq_lens / query_start_loc / block_table */
} pa_status;

typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/* Shapes of one batch.  All fields are host values. */
typedef struct pa_desc {
  int32_t num_seqs;          /* B >= 0 */
  int32_t num_q_tokens;      /* T_q >= 0; must equal query_start_loc[B] */
  int32_t num_q_heads;       /* Hq >= 1 */
  int32_t num_kv_heads;      /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;          /* D: 64 or 128 */
  int32_t page_size;         /* must be PA_PAGE_SIZE (16) */
  int32_t num_pages;         /* NP >= 1: pages in each pool */
  int32_t max_pages_per_seq; /* block_table row stride, >= ceil(max n_s / 16) */
  int32_t max_seq_len;       /* host upper bound on every seq_lens[s], 0 <= max_seq_len <=
                                max_pages_per_seq * 16; 0 = not stated (the bound is then
                                max_pages_per_seq * 16).  Neither the workspace nor the plan
                                depends on it: the single launch derives its work list on the
                                device from seq_lens.  pa_validate reports a longer sequence. */
  int32_t dtype;             /* pa_dtype of q, k_pool, v_pool and out */
  float scale;               /* multiplies q.k before the softmax; any finite value.  0, and
                                magnitudes whose |scale| * log2(e) is below FLT_MIN, give every
                                score exactly 0 (uniform weights over the visible keys) */
} pa_desc;

/* PA_ABI_VERSION of the loaded library. */
int pa_abi_version(void);

/* Static, human-readable name of a status code (never NULL).  pa_status_str is the same
 * function under a second name. */
const char* pa_status_string(pa_status status);
const char* pa_status_str(pa_status status);

/* Host-only check of a descriptor (no HIP call): PA_OK, PA_ERR_BAD_SHAPE or PA_ERR_UNSUPPORTED. */
pa_status pa_check_desc(const pa_desc* desc);

/*
 * Bytes of device workspace pa_attention needs for `desc` on the current HIP
 * device (per workgroup of the persistent launch: an arrival counter and room
 * for two partial results of up to 128 rows; the staged plan).  The size
 * depends only on the descriptor and on the device's compute-unit count.
 * Writes *bytes; returns PA_ERR_NULL_POINTER, a descriptor error or PA_ERR_HIP.
 *
 * Workspace state: the arrival counters must be zero when pa_attention starts.
 * Zero them once after allocating the workspace (pa_workspace_init, or a zero
 * fill of the whole buffer); every pa_attention call leaves them zero, and so
 * does pa_plan.  A workspace sized for a larger descriptor serves smaller ones.
 */
pa_status pa_workspace_size(const pa_desc* desc, size_t* bytes);

/* The same size as a return value: pa_workspace_size's *bytes, or 0 when pa_workspace_size
 * would return an error (NULL or bad descriptor, no HIP device). */
size_t pa_workspace_bytes(const pa_desc* desc);

/*
 * Zero the workspace's arrival counters (enqueues one small fill kernel on
 * `stream`; no hipMemset, so it may be captured in a HIP graph).  Same checks
 * as pa_attention on desc / workspace / workspace_bytes.
 */
pa_status pa_workspace_init(const pa_desc* desc, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Causal GQA attention over the paged cache for a mixed prefill / decode /
 * verify batch (the formula and layouts above), as ONE kernel launch on
 * `stream`: every workgroup of the persistent launch derives the work list
 * from seq_lens and query_start_loc (units of (sequence, kv head, row block)
 * laid on one cost axis cut into equal grains), runs its grain -- decode and
 * verify rows split keys across waves, prefill rows share K/V chunks through
 * LDS -- and the workgroup that finishes the last piece of a unit whose keys
 * were split across grains merges the pieces by log-sum-exp.  `workspace` must
 * hold at least pa_workspace_size bytes, be 256-byte aligned and have zero
 * arrival counters (see pa_workspace_size).  T_q == 0 enqueues nothing.
 * Row blocks have 64 rows, or 128 for bf16 batches at head_dim 128 with
 * T_q * Hq >= 64 * (the launch's workgroups) -- a lot of prefill work, where
 * longer blocks double the MFMA work per K/V byte staged in LDS.  Results are
 * bitwise reproducible for a given batch shape and device, and bitwise equal
 * to those of the staged path below whenever the single launch uses 64-row
 * blocks (the staged path always does).
 *
 * Ordering the in-launch merge relies on (gfx950): a piece's partial results
 * are stored with device scope (written through the XCD's L2 to the
 * device-coherent level) and have completed (s_waitcnt vmcnt(0)) before its
 * workgroup increments the unit's arrival counter, a relaxed atomic at agent
 * scope; the workgroup that reads the completing count then loads the pieces
 * with device scope (missing the non-coherent L2).  No L2-wide write-back or
 * invalidate is issued.  Two calls that share one workspace must not overlap.
 */
pa_status pa_attention(const pa_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_table, const int32_t* seq_lens,
                       const int32_t* query_start_loc, void* out, float* lse, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * pa_attention without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid allocation.  Same computation, kernel, grid and result (bitwise) as
 * pa_attention; the caller passes inputs and outputs only.  The arrival
 * counters and partial results live in a static device array of the library
 * (64.3 MiB on each GPU it runs on, held until the process ends), sized for an
 * attention grid of at most 512 workgroups (MI355X: 256 compute units x 2) and
 * D <= 128; a device whose grid is larger gets PA_ERR_WORKSPACE_TOO_SMALL.  The
 * batch size is not limited.  The first call on a device looks the array up and
 * enqueues one fill kernel on `stream` that zeroes its counters; every call
 * leaves them zero.  Nothing is allocated or freed.  All calls on one GPU share
 * its array: calls that overlap on one GPU (on different streams, or from
 * several threads) race and give undefined results -- order them on one stream.
 */
pa_status pa_attention_noalloc(const pa_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                               const int32_t* block_table, const int32_t* seq_lens,
                               const int32_t* query_start_loc, void* out, float* lse, void* stream);

/*
 * pa_attention for batches whose sequences share prompt prefixes (the
 * prefix-reuse attention of the XY-Serve verdict page, load_bearing_attack
 * and pith_inferences: shared prefix pages; the result is identical to
 * pa_attention's, up to rounding).  Sequences group_start[g] ..
 * group_start[g+1]-1 form group g (groups are contiguous runs of sequences,
 * group_start[0] = 0, group_start[num_groups] = B; a sequence alone is a
 * group of one).  The first prefix_len[g] keys of every member are the same
 * physical pages: prefix_len[g] is a multiple of 16 (0 allowed), every member
 * has prefix_len[g] <= seq_len - q_len (its query window lies after the
 * prefix) and the same first prefix_len[g] / 16 block-table entries; breaking
 * these is undefined behaviour.  The shared pages are read once per group and
 * KV head (all the group's query rows form MFMA tiles over them), each
 * sequence's remaining keys once; the second pass folds the first pass's
 * result for each row into its output by log-sum-exp.  group_start [num_groups+1] and prefix_len [num_groups] are
 * int32 device arrays.  Workspace: pa_shared_prefix_workspace_size bytes,
 * 256-byte aligned, zero arrival counters as for pa_attention (it begins with
 * the pa_attention workspace).  Enqueues three kernels; 1 <= num_groups <= B.
 */
pa_status pa_shared_prefix_workspace_size(const pa_desc* desc, int32_t num_groups, size_t* bytes);
pa_status pa_attention_shared_prefix(const pa_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                                     const int32_t* block_table, const int32_t* seq_lens,
                                     const int32_t* query_start_loc, int32_t num_groups, const int32_t* group_start,
                                     const int32_t* prefix_len, void* out, float* lse, void* workspace,
                                     size_t workspace_bytes, void* stream);

/*
 * pa_attention over FP8 KV pages (a quantized KV cache, as listed among the
 * serving optimizations in the "Arctic Inference with Shift Parallelism"
 * review; MI355X decodes OCP FP8 natively).  k_pool / v_pool hold OCP FP8 E4M3
 * codes, one byte per element, in the layouts above; k_scale / v_scale
 * [NP][Hkv] float32 (device memory) hold one scale per (page, kv head): key j
 * of sequence s is E4M3(k_pool[pg][g][t][:]) * k_scale[pg][g], and V likewise.
 * q and out are bf16 (desc->dtype must be PA_BF16, else PA_ERR_UNSUPPORTED);
 * lse as for pa_attention.  The codes are converted to bf16 exactly and go
 * through the bf16 MFMAs; the K scale multiplies a page's scores and the V
 * scale its softmax weights before those are rounded to bf16.  Same single
 * launch, workspace (sized by pa_workspace_size for the bf16 descriptor) and
 * errors as pa_attention.  The grains are cut as in pa_plan's description
 * except that a chunk of a row-split unit weighs 8 instead of 4 (its K and V
 * are widened to bf16 on the way to the MFMAs, while a decode chunk moves half
 * the bytes), so that pa_plan does not describe this call's grains.  Row
 * blocks follow pa_attention's rule (128 rows at head_dim 128 when T_q * Hq
 * >= 64 * the launch's workgroups; a 128-row chunk also weighs 8).
 */
pa_status pa_attention_fp8kv(const pa_desc* desc, const void* q, const uint8_t* k_pool, const uint8_t* v_pool,
                             const float* k_scale, const float* v_scale, const int32_t* block_table,
                             const int32_t* seq_lens, const int32_t* query_start_loc, void* out, float* lse,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_attention for batches whose verify windows are draft-token trees
 * (speculative decoding with a token tree: XY-Serve verdict page,
 * referee_report "significance" and the desk-editor letter on verifying token
 * trees).  tree_mask [T_q] uint64 (device memory, read only): for a sequence
 * whose window has q <= 64 tokens, window row i sees every context key
 * (positions < n - q), and window token k (position n - q + k) only where bit
 * k of tree_mask[query_start_loc[s] + i] is set; keys past the row's own
 * position n - q + i stay hidden whatever its bits say.  Rows of windows
 * longer than 64 tokens follow the causal rule and their entries are
 * ignored.  The causal rule is the mask with bits 0..i set.  A row that sees
 * no key gets out = 0 and lse = -inf.  Same launch, workspace and errors as
 * pa_attention; tree_mask may not be NULL when T_q > 0.
 */
pa_status pa_attention_tree(const pa_desc* desc, const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_table, const int32_t* seq_lens, const int32_t* query_start_loc,
                            const uint64_t* tree_mask, void* out, float* lse, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * The same computation in three stages, for callers that inspect, time or
 * reuse them.  pa_plan writes the plan into the workspace (it reads only
 * seq_lens and query_start_loc; a plan stays valid while those and desc are
 * unchanged) and zeroes the arrival counters.  pa_attention_planned runs the
 * attention kernel on a planned workspace: unsplit rows get their final
 * out/lse, split rows leave partial results in the workspace.
 * pa_merge_planned combines those partials into out/lse.  The three together
 * give bitwise the result of pa_attention.
 */
pa_status pa_plan(const pa_desc* desc, const int32_t* seq_lens, const int32_t* query_start_loc,
                  void* workspace, size_t workspace_bytes, void* stream);
pa_status pa_attention_planned(const pa_desc* desc, const void* q, const void* k_pool,
                               const void* v_pool, const int32_t* block_table,
                               const int32_t* seq_lens, const int32_t* query_start_loc, void* out,
                               float* lse, void* workspace, size_t workspace_bytes, void* stream);
pa_status pa_merge_planned(const pa_desc* desc, const int32_t* seq_lens, const int32_t* query_start_loc,
                           void* out, float* lse, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Plan inspection (debug / tests).  The planner (pa_plan) writes only the
 * per-sequence cost prefix; work units are derived from it on the fly.  Unit
 * u covers query rows [row0, row0 + n_rows) of sequence `seq` for K/V head
 * `kv_head` (row index = window token * (Hq/Hkv) + head within the group)
 * against keys [0, n_keys), cut into ceil(n_keys / 32) chunks of 32 keys.
 * Units lie on one cost axis in (sequence, kv head, row block) order (cost0 =
 * prefix of the unit costs; a unit costs a fixed start cost -- 48 for kind 0
 * with more than 16 rows, else 32 -- plus
 * n_chunks * cost_weight, and its chunk i starts at cost0 + start + i *
 * cost_weight); grain k -- run by one workgroup of the
 * persistent launch -- takes the chunks whose start lies in
 * [floor(k*C/S), floor((k+1)*C/S)), C = total_cost, S = n_slots.  kind 0:
 * rows <= 32, the four waves of a workgroup split the chunks; kind 1:
 * rows <= 64, each wave takes 16 rows and the chunks are shared.  n_pieces > 1 means the unit's chunks fall into slots
 * first_slot .. first_slot + n_pieces - 1 and their partial results are merged.
 */
typedef struct pa_plan_unit {
  int32_t seq, kv_head, row0, n_rows;
  int32_t n_keys, n_chunks, kind, cost_weight;
  int64_t cost0;
  int32_t first_slot, n_pieces;
} pa_plan_unit;

typedef struct pa_plan_header {
  int32_t n_units, n_slots, grid, num_seqs;
  int64_t total_cost, reserved;
} pa_plan_header;

/*
 * Enumerate the plan held in `workspace` (after pa_plan) and copy it to host
 * memory: *header, and the first min(n_units, max_units) units into `units`
 * (host memory; may be NULL when max_units is 0).  Synchronizes `stream`.
 */
pa_status pa_plan_read(const pa_desc* desc, const int32_t* seq_lens, const int32_t* query_start_loc,
                       void* workspace, size_t workspace_bytes, pa_plan_header* header, pa_plan_unit* units,
                       int32_t max_units, void* stream);

/*
 * Gather keys [0, n_keys) of sequence `seq` from one pool into dense
 * [Hkv][n_keys][D] (element bits copied unchanged), walking the block table.
 * which = 0 reads a K pool ([NP][Hkv][16][D]), which = 1 a V pool
 * ([NP][Hkv][D][16]).  Keys at or beyond seq_lens[seq] are written as zero bits.
 */
pa_status pa_gather_kv(const pa_desc* desc, int32_t which, const void* pool, const int32_t* block_table,
                       const int32_t* seq_lens, int32_t seq, int32_t n_keys, void* dense_out,
                       void* stream);

/*
 * Log-sum-exp merge of attention results over disjoint key sets (for keys
 * split across launches or devices):
 *     lse[r] = ln sum_i exp(lse_parts[i][r]),
 *     out[r][:] = sum_i exp(lse_parts[i][r] - lse[r]) * o_parts[i][r][:]
 * o_parts [n_parts][rows][D] float32, lse_parts [n_parts][rows] float32 (a
 * part with lse = -inf saw no key and contributes nothing), out [rows][D] in
 * out_dtype (pa_dtype), lse [rows] float32.  D: 64 or 128.
 */
pa_status pa_merge(int32_t n_parts, int64_t rows, int32_t head_dim, const float* o_parts,
                   const float* lse_parts, int32_t out_dtype, void* out, float* lse, void* stream);

/*
 * Paged KV append -- the step before attention in a decode or chunked-prefill
 * loop: write the K and V rows of the batch's new tokens into their pages.
 * New token i of sequence s (row query_start_loc[s] + i of k_new / v_new)
 * goes to position p = seq_lens[s] - q_s + i, i.e. page
 * block_table[s][p / 16], slot p % 16 -- the positions pa_attention reads as
 * the window's own keys (seq_lens count the new tokens).  Sources: XY-Serve
 * verdict page, core_discovery (K/V kept in a PagedAttention-style block
 * cache that each step extends).
 *   k_new, v_new   [T_q][Hkv][D]  desc->dtype, device memory, read only
 *   k_pool, v_pool as above; only the (page, head, slot) rows of new tokens
 *                  are written, element bits copied unchanged
 * desc->num_q_heads and desc->scale are not used.  Two new tokens that map
 * to the same slot is undefined behaviour (sequences that share pages must
 * not append into a shared page); pa_validate checks the block-table range.
 * Enqueued on `stream`; no workspace.
 */
pa_status pa_append_kv(const pa_desc* desc, const void* k_new, const void* v_new, const int32_t* block_table,
                       const int32_t* seq_lens, const int32_t* query_start_loc, void* k_pool, void* v_pool,
                       void* stream);

/*
 * Check the batch contents on the device: query_start_loc starts at 0, is
 * non-decreasing and ends at T_q; 0 <= q_len <= seq_len; ceil(seq_len/16) <=
 * max_pages_per_seq; seq_len <= max_seq_len when that is stated; every
 * block-table entry a sequence reads lies in [0, num_pages).  Uses the first 256 bytes of `workspace` and synchronizes
 * `stream`.  Returns PA_OK or PA_ERR_INVALID_CONTENT.
 */
pa_status pa_validate(const pa_desc* desc, const int32_t* block_table, const int32_t* seq_lens,
                      const int32_t* query_start_loc, void* workspace, size_t workspace_bytes,
                      void* stream);

/*
 * Diagnostics: the device's streaming-read rate, the practical ceiling for the
 * memory-bound (decode) paths.  Reads `bytes` of device memory at `buf` with
 * 16-byte loads, workgroup g taking the contiguous slice [g * bytes / grid,
 * (g + 1) * bytes / grid), and writes the XOR of the slice's 32-bit words to
 * sink[g] (device memory, `grid` words), so that the reads cannot be skipped
 * and the caller can check them.  `bytes` must be a positive multiple of
 * 16 * grid and 1 <= grid <= 65535, else PA_ERR_BAD_SHAPE.  Asynchronous on
 * `stream`.
 */
pa_status pa_read_stream(const void* buf, size_t bytes, int32_t grid, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
