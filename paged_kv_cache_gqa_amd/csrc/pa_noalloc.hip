// pa_noalloc.hip -- pa_attention_noalloc: the single-launch attention call with its scratch
// (arrival counters and partial results of key-split units) in a static device array instead of
// a caller workspace, for callers that cannot allocate device memory.
//
// The single launch needs, per workgroup of its grid, one arrival counter and room for two
// partial results of up to kPartRows rows of D <= 128 floats (and their log-sum-exp); nothing in
// it depends on the batch size, so one array of fixed size serves every batch.  Each GPU holds its
// own copy of the array for the life of the process; its device address is looked up once per
// device with hipGetSymbolAddress, and only that address is handed to kernels and fills.
#include <hip/hip_runtime.h>

#include <mutex>

#include "pa_internal.h"

namespace {

// Largest attention grid the scratch serves: 256 compute units x 2 workgroups (MI355X).  With
// partial results of up to 128 rows of D <= 128 floats that is 64.3 MiB per device.
constexpr int kScratchGrid = 512;
constexpr int kScratchMaxD = 128;
constexpr size_t kArriveBytes = pa::align256(sizeof(int32_t) * kScratchGrid);
constexpr size_t kPartLseBytes = pa::align256(sizeof(float) * size_t(kScratchGrid) * 2 * pa::kPartRows);
constexpr size_t kPartOBytes = sizeof(float) * size_t(kScratchGrid) * 2 * pa::kPartRows * kScratchMaxD;
constexpr size_t kScratchBytes = kArriveBytes + kPartLseBytes + kPartOBytes;

// Zero-initialised at load; the single launch leaves every arrival counter zero when it ends.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};  // device address of `scratch` on each device (null: not set up)

// The scratch's device address on the current device.  The first call on a device looks it up
// (with that device current) and zeroes the arrival counters with a fill kernel on `stream`.
pa_status scratch_on_device(void* stream, char** base) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return PA_ERR_HIP;
    if (pa::launch_fill_zero(p, kArriveBytes, stream) != 0) return PA_ERR_HIP;
    g_scratch[dev] = p;
  }
  *base = static_cast<char*>(g_scratch[dev]);
  return PA_OK;
}

}  // namespace

extern "C" pa_status pa_attention_noalloc(const pa_desc* desc, const void* q, const void* k_pool,
                                          const void* v_pool, const int32_t* block_table, const int32_t* seq_lens,
                                          const int32_t* query_start_loc, void* out, float* lse, void* stream) {
  if (!desc) return PA_ERR_NULL_POINTER;
  const pa_status st = pa_check_desc(desc);
  if (st != PA_OK) return st;
  if (desc->num_q_tokens == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_table || !seq_lens || !query_start_loc || !out || !lse)
    return PA_ERR_NULL_POINTER;
  int grid = 0;
  const pa_status gs = pa::attention_grid(*desc, &grid);
  if (gs != PA_OK) return gs;
  if (grid > kScratchGrid || desc->head_dim > kScratchMaxD) return PA_ERR_WORKSPACE_TOO_SMALL;
  char* base = nullptr;
  const pa_status ss = scratch_on_device(stream, &base);
  if (ss != PA_OK) return ss;
  int32_t* arrive = reinterpret_cast<int32_t*>(base);
  float* part_lse = reinterpret_cast<float*>(base + kArriveBytes);
  float* part_o = reinterpret_cast<float*>(base + kArriveBytes + kPartLseBytes);
  const pa::AttnArgs a = pa::single_launch_args(*desc, q, k_pool, v_pool, block_table, seq_lens, query_start_loc,
                                                out, lse, part_o, part_lse, arrive);
  return pa::launch_attention_fused(a, desc->dtype, desc->head_dim, grid, stream, pa::tall_blocks(*desc, grid)) == 0
             ? PA_OK
             : PA_ERR_HIP;
}
