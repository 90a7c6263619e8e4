// ts_mha_api.hip -- the C ABI declared in include/ts_mha.h: host-side argument
// validation, device capability check, error text, and the pair count used by
// the throughput metric.  All arithmetic of the operations runs in the kernels
// of prefill_fwd.hip and decode_fwd.hip.
#include "ts_mha.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <mutex>
#include <vector>

#include "decode_fwd.h"
#include "prefill_fwd.h"

namespace {

constexpr int kMaxDevices = 64;

// Per-device answer to "is this a gfx950?": 0 unknown, 1 yes, 2 no; and its
// number of compute units.
int g_arch_state[kMaxDevices];
int g_cu_count[kMaxDevices];
constexpr int kDefaultCUs = 256;  // MI355X, when the device was not queried (test hook)
std::mutex g_arch_mutex;

thread_local char g_launch_msg[256] = "";

// Scratch of ts_mha_decode_with_kvcache_noalloc: the per-chunk partial results
// of split sequences, in a device array of the library itself instead of a
// caller's workspace.  Each device the library runs on holds its own copy
// until the process ends.  In host code `scratch` is only a stand-in for the
// symbol: its device address, per device, comes from hipGetSymbolAddress on
// the first call on that device and is kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[TS_MHA_NOALLOC_SCRATCH_BYTES];
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mutex;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_device(int* cus = nullptr) {
  if (cus) *cus = kDefaultCUs;
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) {
    (void)hipGetLastError();
    return TS_MHA_ERR_NO_DEVICE;
  }
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return TS_MHA_ERR_NO_DEVICE;
  }
  // Test hook: pretend the device reports this architecture name.
  const char* forced = getenv("TS_MHA_TEST_ARCH");
  if (forced && forced[0]) return strncmp(forced, "gfx950", 6) == 0 ? TS_MHA_OK : TS_MHA_ERR_ARCH;
  if (dev >= kMaxDevices) return TS_MHA_ERR_ARCH;
  std::lock_guard<std::mutex> lock(g_arch_mutex);
  if (g_arch_state[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return TS_MHA_ERR_NO_DEVICE;
    }
    g_arch_state[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_cu_count[dev] = prop.multiProcessorCount;
  }
  if (cus && g_cu_count[dev] > 0) *cus = g_cu_count[dev];
  return g_arch_state[dev] == 1 ? TS_MHA_OK : TS_MHA_ERR_ARCH;
}

// Debug mode: read cu_seqlens back and check it against the documented contract.
int validate_seqlens(const int32_t* cu, int32_t n_seqs, int32_t max_seqlen, hipStream_t stream) {
  std::vector<int32_t> h((size_t)n_seqs + 1);
  if (hipMemcpyAsync(h.data(), cu, sizeof(int32_t) * h.size(), hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    snprintf(g_launch_msg, sizeof g_launch_msg, "%s", hipGetErrorString(hipGetLastError()));
    return TS_MHA_ERR_LAUNCH;
  }
  if (h[0] != 0) return TS_MHA_ERR_SEQLENS;
  for (int32_t b = 0; b < n_seqs; ++b) {
    const int64_t len = (int64_t)h[b + 1] - h[b];
    if (len < 0 || len > max_seqlen) return TS_MHA_ERR_SEQLENS;
  }
  return TS_MHA_OK;
}

// Debug mode for the cache calls: read seqlens_k and the block table back and
// check them against the documented contract.
int validate_cache(const int32_t* seqlens_k, const int32_t* block_table, int32_t n_seqs,
                   int32_t n_pages, int32_t page_size, int32_t pages_per_seq, int32_t max_seqlen_k,
                   hipStream_t stream) {
  std::vector<int32_t> lens((size_t)n_seqs);
  std::vector<int32_t> table((size_t)n_seqs * pages_per_seq);
  if (hipMemcpyAsync(lens.data(), seqlens_k, sizeof(int32_t) * lens.size(), hipMemcpyDeviceToHost,
                     stream) != hipSuccess ||
      hipMemcpyAsync(table.data(), block_table, sizeof(int32_t) * table.size(), hipMemcpyDeviceToHost,
                     stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    snprintf(g_launch_msg, sizeof g_launch_msg, "%s", hipGetErrorString(hipGetLastError()));
    return TS_MHA_ERR_LAUNCH;
  }
  for (int32_t b = 0; b < n_seqs; ++b) {
    if (lens[b] < 0 || lens[b] > max_seqlen_k) return TS_MHA_ERR_SEQLENS;
    const int64_t need = ((int64_t)lens[b] + page_size - 1) / page_size;
    for (int64_t i = 0; i < need; ++i) {
      const int32_t pg = table[(size_t)b * pages_per_seq + i];
      if (pg < 0 || pg >= n_pages) return TS_MHA_ERR_PAGES;
    }
  }
  return TS_MHA_OK;
}

// Debug mode for the prefill with a cache: every sequence has at least as many
// cached keys as new rows.
int validate_rows_fit(const int32_t* cu_seqlens_q, const int32_t* seqlens_k, int32_t n_seqs,
                      hipStream_t stream) {
  std::vector<int32_t> cu((size_t)n_seqs + 1), lens((size_t)n_seqs);
  if (hipMemcpyAsync(cu.data(), cu_seqlens_q, sizeof(int32_t) * cu.size(), hipMemcpyDeviceToHost, stream) !=
          hipSuccess ||
      hipMemcpyAsync(lens.data(), seqlens_k, sizeof(int32_t) * lens.size(), hipMemcpyDeviceToHost, stream) !=
          hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess) {
    snprintf(g_launch_msg, sizeof g_launch_msg, "%s", hipGetErrorString(hipGetLastError()));
    return TS_MHA_ERR_LAUNCH;
  }
  for (int32_t b = 0; b < n_seqs; ++b)
    if (cu[b + 1] - cu[b] > lens[b]) return TS_MHA_ERR_SEQLENS;
  return TS_MHA_OK;
}

bool is_pow2(int32_t x) { return x > 0 && (x & (x - 1)) == 0; }

// Checks shared by the cache calls; TS_MHA_OK when the shapes are acceptable.
int check_cache_shapes(int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, float softmax_scale,
                       int32_t n_seqs, int32_t n_pages, int32_t page_size, int32_t pages_per_seq,
                       int32_t max_seqlen_k) {
  if (n_q_heads <= 0 || n_kv_heads <= 0 || n_seqs < 0 || max_seqlen_k < 0) return TS_MHA_ERR_BAD_SHAPE;
  if (n_q_heads % n_kv_heads != 0) return TS_MHA_ERR_BAD_SHAPE;
  if (n_pages <= 0 || pages_per_seq <= 0 || !is_pow2(page_size) || page_size < 16) return TS_MHA_ERR_BAD_SHAPE;
  if ((int64_t)page_size * n_kv_heads * head_dim * 2 > 0x7fff0000LL) return TS_MHA_ERR_BAD_SHAPE;
  if (max_seqlen_k > (1 << 30) || (int64_t)max_seqlen_k > (int64_t)pages_per_seq * page_size)
    return TS_MHA_ERR_BAD_SHAPE;
  const int32_t G = n_q_heads / n_kv_heads;
  if (head_dim != 64 && head_dim != 128) return TS_MHA_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return TS_MHA_ERR_UNSUPPORTED;
  if (!isfinite(softmax_scale) || !(softmax_scale > 0.f)) return TS_MHA_ERR_BAD_SCALE;
  return TS_MHA_OK;
}

tsmha::DecodeArgs decode_args(int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim, int32_t window,
                              int32_t n_seqs, int32_t max_seqlen_k) {
  tsmha::DecodeArgs a{};
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.head_dim = head_dim;
  a.window = window;
  a.n_seqs = n_seqs;
  a.max_seqlen_k = max_seqlen_k;
  return a;
}

}  // namespace

extern "C" int ts_mha_prefill(const void* q, const void* k, const void* v, const float* sinks,
                              const int32_t* cu_seqlens, int32_t n_q_heads, int32_t n_kv_heads,
                              int32_t head_dim, int32_t window, float softmax_scale, void* out,
                              int32_t n_seqs, int32_t max_seqlen, void* stream) {
  if (!q || !k || !v || !cu_seqlens || !out) return TS_MHA_ERR_NULL_ARG;
  if (n_q_heads <= 0 || n_kv_heads <= 0 || n_seqs < 0 || max_seqlen < 0) return TS_MHA_ERR_BAD_SHAPE;
  if (n_q_heads % n_kv_heads != 0) return TS_MHA_ERR_BAD_SHAPE;
  const int32_t G = n_q_heads / n_kv_heads;
  if (head_dim != 64 && head_dim != 128) return TS_MHA_ERR_UNSUPPORTED;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16) return TS_MHA_ERR_UNSUPPORTED;
  if (!isfinite(softmax_scale) || !(softmax_scale > 0.f)) return TS_MHA_ERR_BAD_SCALE;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(sinks, 4) || !aligned(cu_seqlens, 4))
    return TS_MHA_ERR_ALIGN;

  tsmha::PrefillArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.sinks = sinks;
  a.cu_seqlens = cu_seqlens;
  a.out = out;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.window = window;
  a.softmax_scale = softmax_scale;
  a.n_seqs = n_seqs;
  a.max_seqlen = max_seqlen;
  // head_dim 64 has two kernels: the 256-row work-groups of prefill_fwd.hip,
  // and the 128-row ones of prefill_fwd_narrow.hip, which take over when the
  // former would give no compute unit more than two work-groups (short or few
  // sequences): twice as many work-groups, each half as long, then fill the
  // GPU.  head_dim 128 always uses the 128-row form.  TS_MHA_PREFILL_KERNEL =
  // wide | narrow forces one of the head_dim 64 kernels (tests, measurement).
  const int64_t wide = head_dim == 64 ? tsmha::prefill_grid_size(a) : -1;
  const int64_t narrow = tsmha::prefill_grid_size_narrow(a, head_dim);
  if ((head_dim == 64 ? wide : narrow) < 0) return TS_MHA_ERR_BAD_SHAPE;

  int cus = 0;
  const int dev_rc = check_device(&cus);
  if (dev_rc != TS_MHA_OK) return dev_rc;
  bool use_narrow = true;
  if (head_dim == 64) {
    const char* kname = getenv("TS_MHA_PREFILL_KERNEL");
    if (kname && strcmp(kname, "wide") == 0) use_narrow = false;
    else if (kname && strcmp(kname, "narrow") == 0) use_narrow = narrow >= 0;
    else use_narrow = narrow >= 0 && wide <= 2 * (int64_t)cus;
  }
  const int64_t grid = use_narrow ? narrow : wide;

  hipStream_t st = static_cast<hipStream_t>(stream);
  const char* dbg = getenv("TS_MHA_VALIDATE");
  if (dbg && dbg[0] == '1' && n_seqs > 0) {
    const int rc = validate_seqlens(cu_seqlens, n_seqs, max_seqlen, st);
    if (rc != TS_MHA_OK) return rc;
  }
  if (grid == 0) return TS_MHA_OK;

  const hipError_t err = use_narrow ? tsmha::launch_prefill_narrow(a, head_dim, st) : tsmha::launch_prefill(a, st);
  if (err != hipSuccess) {
    snprintf(g_launch_msg, sizeof g_launch_msg, "%s", hipGetErrorString(err));
    return TS_MHA_ERR_LAUNCH;
  }
  return TS_MHA_OK;
}

extern "C" int ts_mha_prefill_with_kvcache(const void* q, const void* k_cache, const void* v_cache,
                                           const float* sinks, const int32_t* cu_seqlens_q,
                                           const int32_t* seqlens_k, const int32_t* block_table,
                                           int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                                           int32_t window, float softmax_scale, void* out, int32_t n_seqs,
                                           int32_t n_pages, int32_t page_size, int32_t pages_per_seq,
                                           int32_t max_seqlen_q, int32_t max_seqlen_k, void* stream) {
  if (!q || !k_cache || !v_cache || !cu_seqlens_q || !seqlens_k || !block_table || !out)
    return TS_MHA_ERR_NULL_ARG;
  int rc = check_cache_shapes(n_q_heads, n_kv_heads, head_dim, softmax_scale, n_seqs, n_pages, page_size,
                              pages_per_seq, max_seqlen_k);
  if (rc != TS_MHA_OK) return rc;
  if (max_seqlen_q < 0 || max_seqlen_q > max_seqlen_k) return TS_MHA_ERR_BAD_SHAPE;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(sinks, 4) || !aligned(cu_seqlens_q, 4) || !aligned(seqlens_k, 4) || !aligned(block_table, 4))
    return TS_MHA_ERR_ALIGN;

  tsmha::PrefillArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.sinks = sinks;
  a.cu_seqlens = cu_seqlens_q;
  a.out = out;
  a.n_q_heads = n_q_heads;
  a.n_kv_heads = n_kv_heads;
  a.window = window;
  a.softmax_scale = softmax_scale;
  a.n_seqs = n_seqs;
  a.max_seqlen = max_seqlen_q;
  a.seqlens_k = seqlens_k;
  a.block_table = block_table;
  a.n_pages = n_pages;
  a.page_size = page_size;
  a.pages_per_seq = pages_per_seq;
  // head_dim 64: the 256-row kernel's paged form; head_dim 128: the 128-row kernel's
  const int64_t grid = head_dim == 64 ? tsmha::prefill_grid_size(a) : tsmha::prefill_grid_size_narrow(a, head_dim);
  if (grid < 0) return TS_MHA_ERR_BAD_SHAPE;

  rc = check_device();
  if (rc != TS_MHA_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  const char* dbg = getenv("TS_MHA_VALIDATE");
  if (dbg && dbg[0] == '1' && n_seqs > 0) {
    rc = validate_seqlens(cu_seqlens_q, n_seqs, max_seqlen_q, st);
    if (rc == TS_MHA_OK)
      rc = validate_cache(seqlens_k, block_table, n_seqs, n_pages, page_size, pages_per_seq, max_seqlen_k, st);
    if (rc == TS_MHA_OK) rc = validate_rows_fit(cu_seqlens_q, seqlens_k, n_seqs, st);
    if (rc != TS_MHA_OK) return rc;
  }
  if (grid == 0) return TS_MHA_OK;
  const hipError_t err = head_dim == 64 ? tsmha::launch_prefill(a, st) : tsmha::launch_prefill_narrow(a, head_dim, st);
  if (err != hipSuccess) {
    snprintf(g_launch_msg, sizeof g_launch_msg, "%s", hipGetErrorString(err));
    return TS_MHA_ERR_LAUNCH;
  }
  return TS_MHA_OK;
}

extern "C" int64_t ts_mha_decode_workspace_size(int32_t n_seqs, int32_t n_q_heads, int32_t n_kv_heads,
                                                int32_t head_dim, int32_t window, int32_t max_seqlen_k) {
  const int rc = check_cache_shapes(n_q_heads, n_kv_heads, head_dim, 1.f, n_seqs, 1, 16,
                                    (max_seqlen_k + 15) / 16 + 1, max_seqlen_k);
  if (rc != TS_MHA_OK) return rc;
  const tsmha::DecodePlan plan = tsmha::decode_plan(decode_args(n_q_heads, n_kv_heads, head_dim, window, n_seqs, max_seqlen_k));
  if (plan.n_splits < 0) return TS_MHA_ERR_BAD_SHAPE;
  return plan.workspace_bytes;
}

namespace {

// This device's copy of `scratch`, looked up on the device's first call.
int scratch_for_current_device(void** ptr) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return TS_MHA_ERR_NO_DEVICE;
  }
  if (dev >= kMaxDevices) return TS_MHA_ERR_ARCH;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess || !p) {
      snprintf(g_launch_msg, sizeof g_launch_msg, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(err));
      (void)hipGetLastError();
      return TS_MHA_ERR_LAUNCH;
    }
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return TS_MHA_OK;
}

// Both decode entry points: the caller's workspace, or (noalloc) the library's scratch.
int decode_call(const void* q, const void* k_cache, const void* v_cache, const float* sinks,
                const int32_t* seqlens_k, const int32_t* block_table, int32_t n_q_heads,
                int32_t n_kv_heads, int32_t head_dim, int32_t window, float softmax_scale, void* out,
                int32_t n_seqs, int32_t n_pages, int32_t page_size, int32_t pages_per_seq,
                int32_t max_seqlen_k, void* workspace, int64_t workspace_bytes, bool noalloc,
                void* stream) {
  if (!q || !k_cache || !v_cache || !seqlens_k || !block_table || !out) return TS_MHA_ERR_NULL_ARG;
  int rc = check_cache_shapes(n_q_heads, n_kv_heads, head_dim, softmax_scale, n_seqs, n_pages, page_size,
                              pages_per_seq, max_seqlen_k);
  if (rc != TS_MHA_OK) return rc;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) ||
      !aligned(sinks, 4) || !aligned(seqlens_k, 4) || !aligned(block_table, 4) || !aligned(workspace, 256))
    return TS_MHA_ERR_ALIGN;
  tsmha::DecodeArgs a = decode_args(n_q_heads, n_kv_heads, head_dim, window, n_seqs, max_seqlen_k);
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.sinks = sinks;
  a.seqlens_k = seqlens_k;
  a.block_table = block_table;
  a.out = out;
  a.softmax_scale = softmax_scale;
  a.n_pages = n_pages;
  a.page_size = page_size;
  a.pages_per_seq = pages_per_seq;
  const tsmha::DecodePlan plan = tsmha::decode_plan(a);
  if (plan.n_splits < 0) return TS_MHA_ERR_BAD_SHAPE;
  if (noalloc) {
    if (plan.workspace_bytes > TS_MHA_NOALLOC_SCRATCH_BYTES) return TS_MHA_ERR_WORKSPACE;
  } else if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes)) {
    return TS_MHA_ERR_WORKSPACE;
  }

  rc = check_device();
  if (rc != TS_MHA_OK) return rc;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (noalloc) {
    rc = scratch_for_current_device(&workspace);
    if (rc != TS_MHA_OK) return rc;
  } else {
    const char* dbg = getenv("TS_MHA_VALIDATE");
    if (dbg && dbg[0] == '1' && n_seqs > 0) {
      rc = validate_cache(seqlens_k, block_table, n_seqs, n_pages, page_size, pages_per_seq, max_seqlen_k, st);
      if (rc != TS_MHA_OK) return rc;
    }
  }
  if (n_seqs == 0) return TS_MHA_OK;
  const hipError_t err = tsmha::launch_decode(a, plan, workspace, st);
  if (err != hipSuccess) {
    snprintf(g_launch_msg, sizeof g_launch_msg, "%s", hipGetErrorString(err));
    return TS_MHA_ERR_LAUNCH;
  }
  return TS_MHA_OK;
}

}  // namespace

extern "C" int ts_mha_decode_with_kvcache(const void* q, const void* k_cache, const void* v_cache,
                                          const float* sinks, const int32_t* seqlens_k,
                                          const int32_t* block_table, int32_t n_q_heads,
                                          int32_t n_kv_heads, int32_t head_dim, int32_t window,
                                          float softmax_scale, void* out, int32_t n_seqs,
                                          int32_t n_pages, int32_t page_size, int32_t pages_per_seq,
                                          int32_t max_seqlen_k, void* workspace,
                                          int64_t workspace_bytes, void* stream) {
  return decode_call(q, k_cache, v_cache, sinks, seqlens_k, block_table, n_q_heads, n_kv_heads, head_dim,
                     window, softmax_scale, out, n_seqs, n_pages, page_size, pages_per_seq, max_seqlen_k,
                     workspace, workspace_bytes, false, stream);
}

extern "C" int ts_mha_decode_with_kvcache_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                                  const float* sinks, const int32_t* seqlens_k,
                                                  const int32_t* block_table, int32_t n_q_heads,
                                                  int32_t n_kv_heads, int32_t head_dim, int32_t window,
                                                  float softmax_scale, void* out, int32_t n_seqs,
                                                  int32_t n_pages, int32_t page_size,
                                                  int32_t pages_per_seq, int32_t max_seqlen_k,
                                                  void* stream) {
  return decode_call(q, k_cache, v_cache, sinks, seqlens_k, block_table, n_q_heads, n_kv_heads, head_dim,
                     window, softmax_scale, out, n_seqs, n_pages, page_size, pages_per_seq, max_seqlen_k,
                     nullptr, 0, true, stream);
}

extern "C" const char* ts_mha_strerror(int code) {
  switch (code) {
    case TS_MHA_OK: return "success";
    case TS_MHA_ERR_NULL_ARG: return "a required pointer argument is NULL";
    case TS_MHA_ERR_BAD_SHAPE:
      return "bad shape: heads must be > 0 with n_q_heads a multiple of n_kv_heads, n_seqs and "
             "max_seqlen must be >= 0, the launch grid must fit; for the cache calls page_size a power "
             "of two >= 16, n_pages and pages_per_seq > 0, max_seqlen_k <= pages_per_seq * page_size";
    case TS_MHA_ERR_UNSUPPORTED:
      return "unsupported configuration: head_dim must be 64 or 128 and n_q_heads / n_kv_heads one of "
             "1, 2, 4, 8, 16";
    case TS_MHA_ERR_BAD_SCALE: return "softmax_scale must be finite and > 0";
    case TS_MHA_ERR_ALIGN:
      return "misaligned pointer: q, k, v (or the caches), out need 16-byte alignment, sinks, "
             "cu_seqlens, seqlens_k and block_table 4-byte, the workspace 256-byte";
    case TS_MHA_ERR_NO_DEVICE: return "no HIP device is available";
    case TS_MHA_ERR_ARCH: return "the current HIP device is not a gfx950 (MI355X-class) GPU";
    case TS_MHA_ERR_LAUNCH: {
      static thread_local char msg[320];
      snprintf(msg, sizeof msg, "HIP launch failed: %s", g_launch_msg);
      return msg;
    }
    case TS_MHA_ERR_SEQLENS:
      return "sequence lengths violate their contract (cu_seqlens: cu[0] == 0, non-decreasing, lengths <= "
             "max_seqlen; seqlens_k: 0 <= length <= max_seqlen_k)";
    case TS_MHA_ERR_WORKSPACE:
      return "workspace missing or smaller than ts_mha_decode_workspace_size reports (noalloc decode: the "
             "call needs more than the library's TS_MHA_NOALLOC_SCRATCH_BYTES of scratch)";
    case TS_MHA_ERR_PAGES: return "a block-table entry a sequence needs is outside [0, n_pages)";
    default: return "unknown error";
  }
}

extern "C" int64_t ts_mha_unmasked_pairs(const int32_t* cu_seqlens_host, int32_t n_seqs, int32_t window) {
  if (!cu_seqlens_host || n_seqs < 0) return -1;
  int64_t total = 0;
  for (int32_t b = 0; b < n_seqs; ++b) {
    const int64_t L = (int64_t)cu_seqlens_host[b + 1] - cu_seqlens_host[b];
    if (L < 0) return -1;
    if (window > 0 && window < L) {
      const int64_t W = window;
      total += W * (W + 1) / 2 + (L - W) * W;
    } else {
      total += L * (L + 1) / 2;
    }
  }
  return total;
}
