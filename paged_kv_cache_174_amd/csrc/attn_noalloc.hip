// pkv_paged_attn for callers that cannot allocate device memory (code under
// HIP graph capture, serving loops that forbid hipMalloc): the split-key
// partial results go to a scratch array that the library's code object
// brings with it, instead of a caller-provided workspace.
//
// The array is a file-scope __device__ variable, so every device the library
// runs on holds its own copy for the life of the process.  In host code its
// name only stands for the variable; the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current
// and kept here.  Kernels only ever receive that address.

#include <mutex>

#include "pkv_internal.hpp"

namespace pkv {
namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(PKV_NOALLOC_SCRATCH_BYTES);
static_assert(kScratchBytes % 256 == 0, "the scratch holds whole 256-byte lines");

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// Device address of the current device's copy of `scratch`.
int scratch_address(void** out) {
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess)
    return fail(PKV_EHIP, "hipGetDevice failed: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(PKV_EUNSUPPORTED, "device %d: the static scratch is kept for devices 0..%d", dev,
                kMaxScratchDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(PKV_EHIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

extern "C" int pkv_paged_attn_noalloc(const void* q, int32_t q_dtype, int64_t num_q_tokens, int32_t num_q_heads,
                                      const pkv_pools* pools, const int32_t* block_table, int32_t table_width,
                                      const int32_t* query_start_loc, const int32_t* seq_lens, int32_t num_seqs,
                                      int32_t max_query_len, int32_t max_seq_len, const int32_t* segments,
                                      const int32_t* segment_start_loc, const int32_t* seq_order,
                                      const int32_t* host_seq_lens, float softmax_scale, void* out, void* stream) {
  using pkv::fail;
  if (!pools) return fail(PKV_EINVAL, "pools is NULL");
  // The workspace pkv_paged_attn would like for these sizes; with at least
  // that much it plans exactly the splits it plans with that much.
  const size_t need = pkv_paged_attn_workspace_size(num_q_tokens, num_q_heads, pools->num_kv_heads, pools->head_dim,
                                                    num_seqs, max_query_len, max_seq_len);
  if (need > pkv::kScratchBytes)
    return fail(PKV_ERANGE,
                "these sizes need %zu bytes of split scratch, more than the %zu the library holds per device; "
                "call pkv_paged_attn with a workspace instead",
                need, pkv::kScratchBytes);
  void* ws = nullptr;
  if (int rc = pkv::scratch_address(&ws)) return rc;
  return pkv_paged_attn(q, q_dtype, num_q_tokens, num_q_heads, pools, block_table, table_width, query_start_loc,
                        seq_lens, num_seqs, max_query_len, max_seq_len, segments, segment_start_loc, seq_order,
                        host_seq_lens, softmax_scale, out, ws, pkv::kScratchBytes, stream);
}
