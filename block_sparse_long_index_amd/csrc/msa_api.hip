// Host side of the C ABI declared in include/msa.h: argument validation,
// workspace layout, query-chunk loops and kernel launches.  No device memory
// is allocated here and nothing synchronises the stream.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <vector>

#include "msa.h"
#include "msa_common.h"

namespace msa {
hipError_t launch_index_select_prefill(const void*, const void*, const int32_t*, const int32_t*,
                                       KvMap, int, int, int, int, int, int32_t*, float*, hipStream_t);
hipError_t launch_index_score_decode(const void*, const void*, const int32_t*, const int32_t*, KvMap,
                                     int, int, int, int, int, int, int, float*, long long,
                                     hipStream_t);
hipError_t launch_topk_select(const float*, long long, int, int, int, const int32_t*, const int32_t*,
                              int, int, int, int32_t*, float*, hipStream_t);
size_t lists_workspace_bytes(int batch, int G, int nqt_max, int nb_max);
int list_tile_rows();
hipError_t launch_build_lists(const int32_t*, const int32_t*, const int32_t*, int, int, int, int,
                              int, int32_t*, int32_t*, void*, hipStream_t);
hipError_t launch_attend_blocks(int, int, bool, const void*, const void*, const void*, MainFp8,
                                const int32_t*, const int32_t*, KvMap, int, int, int, int, int,
                                const int32_t*, const int32_t*, int, int, int, float, void*, float2*,
                                hipStream_t);
hipError_t launch_attend_decode(int, int, const void*, const void*, const void*, MainFp8,
                                const int32_t*, const int32_t*, KvMap, int, int, int, int, int,
                                const int32_t*, int, int, float, float*, float2*, hipStream_t);
hipError_t launch_main_quantize_fp8(int, const void*, const void*, const void*, const int32_t*, KvMap,
                                    int, int, int, long long, void*, uint8_t*, void*, uint8_t*,
                                    void*, uint8_t*, hipStream_t);
hipError_t launch_main_quantize_q8kv4(int, const void*, const void*, const void*, const int32_t*,
                                      KvMap, int, int, int, long long, void*, uint8_t*, void*,
                                      uint8_t*, void*, uint8_t*, hipStream_t);
hipError_t launch_merge(int, bool, const void*, const float2*, const int32_t*, int, int, int, int,
                        int, void*, float*, hipStream_t);
int fp8_max_blocks_per_sequence();
int fp8_prefill_rows_per_wg();
int prefill_rows_per_wg();
hipError_t launch_block_mass(int, const float2*, const int32_t*, int, int, int, int, float*,
                             hipStream_t);
hipError_t launch_index_kl(int, const void*, const void*, const int32_t*, const int32_t*, KvMap, int,
                           int, int, int, const int32_t*, const float*, const float*, float*,
                           float*, hipStream_t);
hipError_t launch_index_project(const void*, const void*, const void*, int, int, int, int,
                                const int32_t*, const int32_t*, KvMap, int, void*, void*, void*,
                                size_t, hipStream_t);
size_t project_workspace_bytes(int, int);
size_t project_workspace_required(int, int);
hipError_t launch_hbm_stream(const void*, long long, int, void*, void*, int, hipStream_t);
hipError_t launch_quantize_index_fp8(int, const void*, const void*, const int32_t*, KvMap, int, int,
                                     long long, void*, uint8_t*, void*, uint8_t*, hipStream_t);
hipError_t launch_index_select_prefill_fp8(const void*, const uint8_t*, const void*, const uint8_t*,
                                           bool, const int32_t*, const int32_t*, KvMap, int, int,
                                           int, int, int, int, int32_t*, float*, hipStream_t);
hipError_t launch_index_score_decode_fp8(const void*, const uint8_t*, const void*, const uint8_t*,
                                         bool, const int32_t*, const int32_t*, KvMap, int, int, int,
                                         int, int, int, int, float*, long long, hipStream_t);
hipError_t launch_quantize_index_q8k4(int, const void*, const void*, const int32_t*, KvMap, int, int,
                                      long long, void*, uint8_t*, void*, uint8_t*, hipStream_t);
}  // namespace msa

namespace {

thread_local std::string g_last_error;

constexpr size_t kDefaultChunkBytes = (size_t)72 << 30;   // workspace cap when q_chunk == 0
constexpr int kMaxNbLds = 12288;                          // per-sequence blocks the LDS lists hold
constexpr int kMaxBatch = 65535;                            // a grid dimension's limit
constexpr int kDecodeRowsMax = 128;                       // (query, group) rows per sequence, decode path
constexpr int kDecodeAttendMaxQ = 8;                      // queries per sequence, per-(query, slot) attend

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

msa_status_t fail(msa_status_t s, const char* msg) {
  g_last_error = msg;
  return s;
}

struct Derived {
  int G, Hq, D, DI, hpg, top_k;
  int nb_max, nqt_max;
  bool decode_path;
  bool compact;     // compact Main-Branch partials (lists path only)
  float scale;
  long long total_q;
  msa::KvMap kv;   // where key rows live (contiguous or paged)
};

msa_status_t check_dims(const msa_dims_t* d, Derived* out) {
  if (!d) return fail(MSA_ERR_NULL_ARG, "dims is NULL");
  if (d->batch < 1) return fail(MSA_ERR_BAD_DIMS, "batch must be >= 1");
  if (d->batch > kMaxBatch) return fail(MSA_ERR_UNSUPPORTED, "batch must be <= 65535 (sequences index a grid dimension)");
  if (d->num_q_heads < 1 || d->num_kv_heads < 1) return fail(MSA_ERR_BAD_DIMS, "head counts must be >= 1");
  if (d->num_q_heads % d->num_kv_heads) return fail(MSA_ERR_BAD_DIMS, "num_q_heads % num_kv_heads != 0");
  // grid limits: some kernels put the KV head in a grid dimension of at most
  // 65535; the list builder runs one 256-lane workgroup per (sequence, group)
  // along x, whose lane count must stay below 2^32
  if (d->num_kv_heads > kMaxBatch) return fail(MSA_ERR_UNSUPPORTED, "num_kv_heads must be <= 65535");
  if ((long long)d->batch * d->num_kv_heads >= (1ll << 24))
    return fail(MSA_ERR_UNSUPPORTED, "batch * num_kv_heads must be < 2^24");
  int hpg = d->num_q_heads / d->num_kv_heads;
  if (hpg > 32 || (hpg & (hpg - 1))) return fail(MSA_ERR_UNSUPPORTED, "heads per group must be a power of two <= 32");
  if (d->head_dim != 64 && d->head_dim != 128) return fail(MSA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (d->index_dim != 32 && d->index_dim != 64 && d->index_dim != 128)
    return fail(MSA_ERR_UNSUPPORTED, "index_dim must be 32, 64 or 128");
  if (d->block_size != MSA_BLOCK_SIZE) return fail(MSA_ERR_UNSUPPORTED, "block_size must be 128");
  if (d->top_k < 1 || d->top_k > MSA_MAX_TOP_K) return fail(MSA_ERR_BAD_DIMS, "top_k must be in 1..32");
  if (!(d->softmax_scale >= 0.f) || isinf(d->softmax_scale)) return fail(MSA_ERR_BAD_DIMS, "softmax_scale must be finite and >= 0");
  if (d->total_q < 0 || d->total_k < 0) return fail(MSA_ERR_BAD_DIMS, "negative totals");
  if (d->total_q >= ((long long)1 << 26)) return fail(MSA_ERR_UNSUPPORTED, "total_q must be < 2^26");
  if (d->total_k >= ((long long)1 << 31)) return fail(MSA_ERR_UNSUPPORTED, "total_k must be < 2^31");
  if (d->total_q > d->total_k) return fail(MSA_ERR_BAD_DIMS, "total_q > total_k (each sequence needs Lq <= Lk)");
  if (d->max_q_len < 0 || d->max_k_len < 0 || d->max_q_len > d->max_k_len)
    return fail(MSA_ERR_BAD_DIMS, "need 0 <= max_q_len <= max_k_len");
  if (d->max_q_len > d->total_q || d->max_k_len > d->total_k)
    return fail(MSA_ERR_BAD_DIMS, "max lengths exceed totals");
  if (d->q_chunk < 0) return fail(MSA_ERR_BAD_DIMS, "q_chunk must be >= 0");
  if (d->flags & ~MSA_FLAG_COMPACT_PARTIALS) return fail(MSA_ERR_BAD_DIMS, "unknown bits in flags");
  if (d->kv_pages < 0) return fail(MSA_ERR_BAD_DIMS, "kv_pages must be >= 0");
  if (d->kv_pages > 0) {
    if (!d->block_table) return fail(MSA_ERR_NULL_ARG, "block_table is NULL (paged key cache)");
    if ((long long)d->max_blocks_per_seq * MSA_BLOCK_SIZE < d->max_k_len)
      return fail(MSA_ERR_BAD_DIMS, "max_blocks_per_seq below ceil(max_k_len / 128)");
    if ((long long)d->kv_pages * MSA_BLOCK_SIZE != d->total_k)
      return fail(MSA_ERR_BAD_DIMS, "paged key cache: total_k must equal 128 * kv_pages");
    if ((long long)d->batch * d->max_blocks_per_seq >= ((long long)1 << 31))
      return fail(MSA_ERR_UNSUPPORTED, "block table too large");
  } else if (d->block_table || d->max_blocks_per_seq) {
    return fail(MSA_ERR_BAD_DIMS, "block_table / max_blocks_per_seq are for a paged cache (kv_pages > 0)");
  }
  out->G = d->num_kv_heads;
  out->Hq = d->num_q_heads;
  out->D = d->head_dim;
  out->DI = d->index_dim;
  out->hpg = hpg;
  out->top_k = d->top_k;
  out->nb_max = (d->max_k_len + MSA_BLOCK_SIZE - 1) / MSA_BLOCK_SIZE;
  out->nqt_max = (d->max_q_len + msa::list_tile_rows() - 1) / msa::list_tile_rows();
  if (out->nb_max + msa::list_tile_rows() * d->top_k > kMaxNbLds + 4096)
    return fail(MSA_ERR_UNSUPPORTED, "max_k_len too long for the on-chip list builder");
  if ((long long)d->batch * out->G * out->nb_max >= ((long long)1 << 30))
    return fail(MSA_ERR_UNSUPPORTED, "batch * num_kv_heads * blocks too large");
  // decode-shaped steps (a few new tokens per sequence): split-scan index kernels
  out->decode_path = (long long)d->max_q_len * out->G <= kDecodeRowsMax;
  out->compact = (d->flags & MSA_FLAG_COMPACT_PARTIALS) && d->max_q_len > kDecodeAttendMaxQ;
  out->scale = d->softmax_scale > 0.f ? d->softmax_scale : 1.f / sqrtf((float)d->head_dim);
  out->total_q = d->total_q;
  out->kv.table = d->kv_pages > 0 ? d->block_table : nullptr;
  out->kv.max_blocks = d->kv_pages > 0 ? d->max_blocks_per_seq : 0;
  out->kv.pages = d->kv_pages;
  return MSA_OK;
}

// Rows per pass: an explicit q_chunk is used as given; a byte cap is turned
// into equal passes (rounded up to 128 rows) so no pass is a small tail.
long long round_chunk(long long rows, long long total, bool exact) {
  if (rows >= total) return total;
  if (rows < 1) rows = 1;
  if (exact) return rows;
  long long passes = (total + rows - 1) / rows;
  long long even = (total + passes - 1) / passes;
  long long r128 = (even + 127) / 128 * 128;
  return r128 <= rows ? r128 : even;
}

// rows per pass of msa_index_select and the bytes of its score buffer
long long select_chunk(const msa_dims_t* d, const Derived& x) {
  long long per_row = (long long)x.G * x.nb_max * 4;
  long long rows = d->q_chunk > 0 ? d->q_chunk : (long long)(kDefaultChunkBytes / (per_row ? per_row : 1));
  return round_chunk(rows, x.total_q, d->q_chunk > 0);
}

// bytes of one partial row's acc values: fp32, or fp16 when compact
long long acc_bytes(const Derived& x) { return (long long)x.D * (x.compact ? 2 : 4); }

long long attend_chunk(const msa_dims_t* d, const Derived& x) {
  long long per_row = (long long)x.Hq * x.top_k * (acc_bytes(x) + 8);
  long long rows = d->q_chunk > 0 ? d->q_chunk : (long long)(kDefaultChunkBytes / per_row);
  // partial rows are indexed with int32
  long long cap = (((long long)1 << 31) - 1) / ((long long)x.Hq * x.top_k);
  if (rows > cap) rows = cap;
  return round_chunk(rows, x.total_q, d->q_chunk > 0 && d->q_chunk <= cap);
}

// the prefill path selects inside its scoring kernel and needs no workspace;
// the decode path keeps a block-score buffer for its wide top-k
size_t ws_select(const msa_dims_t* d, const Derived& x) {
  if (!x.decode_path) return 256;
  long long c = select_chunk(d, x);
  return align256((size_t)c * x.G * x.nb_max * 4) + 256;
}
size_t ws_lists(const msa_dims_t* d, const Derived& x) {
  return msa::lists_workspace_bytes(d->batch, x.G, x.nqt_max, x.nb_max) + 256;
}
// partial rows of one pass plus one spare row that padding lanes write to
size_t attend_rows(const msa_dims_t* d, const Derived& x) {
  return (size_t)attend_chunk(d, x) * x.Hq * x.top_k + 1;
}
size_t ws_attend(const msa_dims_t* d, const Derived& x) {
  size_t rows = attend_rows(d, x);
  return align256(rows * acc_bytes(x)) + align256(rows * 8) + 256;
}

size_t ws_project(const Derived& x) {
  // fp32 tiles of the slices of K: always for few-token steps, and up to a few
  // thousand tokens when the large-tile kernel would not fill the GPU (0 above)
  if (x.total_q > (1ll << 30)) return 0;
  return msa::project_workspace_bytes((int)x.total_q, (x.G + 1) * x.DI);
}

size_t ws_project_required(const Derived& x) {
  // the part a call cannot do without (the few-token path's slices)
  if (x.total_q > (1ll << 30)) return 0;
  return msa::project_workspace_required((int)x.total_q, (x.G + 1) * x.DI);
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// --- opt-in per-launch timing: each launcher call is bracketed by two hipEvents
// recorded on the launch stream; msa_profile_collect() waits for them.
enum KernelId { K_INDEX_PREFILL, K_INDEX_DECODE, K_TOPK, K_LISTS, K_ATTEND, K_MERGE,
                K_QUANT_FP8, K_INDEX_PREFILL_FP8, K_INDEX_DECODE_FP8, K_PROJECT, K_MASS,
                K_INDEX_KL, K_QUANT_MAIN_FP8, K_QUANT_Q8K4, K_INDEX_PREFILL_Q8K4,
                K_INDEX_DECODE_Q8K4, K_QUANT_MAIN_Q8KV4 };
const char* const kKernelNames[MSA_PROFILE_KERNELS] = {
    "index_select_prefill", "index_score_decode", "topk_select",
    "build_lists", "attend_blocks", "merge_partials",
    "quantize_index_fp8", "index_select_prefill_fp8", "index_score_decode_fp8",
    "index_project", "block_mass", "index_kl", "quantize_main_fp8", "quantize_index_q8k4",
    "index_select_prefill_q8k4", "index_score_decode_q8k4", "quantize_main_q8kv4"};

std::atomic<bool> g_prof_on{false};
std::mutex g_prof_mu;
struct ProfRec { int kid; hipEvent_t a, b; };
std::vector<ProfRec> g_prof_pending;
std::vector<hipEvent_t> g_event_pool;

hipEvent_t pool_get() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

struct ProfScope {
  int kid;
  hipStream_t st;
  hipEvent_t a = nullptr, b = nullptr;
  ProfScope(int k, hipStream_t s) : kid(k), st(s) {
    if (!g_prof_on.load(std::memory_order_relaxed)) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    a = pool_get();
    b = pool_get();
    if (a && b) (void)hipEventRecord(a, st);
  }
  ~ProfScope() {
    if (!a || !b) return;
    (void)hipEventRecord(b, st);
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_prof_pending.push_back({kid, a, b});
  }
};

msa_status_t hip_fail(hipError_t e) {
  g_last_error = std::string("HIP: ") + hipGetErrorString(e);
  return MSA_ERR_HIP;
}

// MSA_DEBUG_SYNC (environment, read at every call; any value but "" or "0"):
// a debugging aid that blocks the host.  Each call first validates its
// cu_seqlens on the host, and every kernel stage is followed by a wait on the
// call's stream and an error check that names the stage.  Not for use under
// graph capture (it synchronises the stream).
bool debug_sync_on() {
  const char* v = getenv("MSA_DEBUG_SYNC");
  return v && v[0] && strcmp(v, "0") != 0;
}

// status of a stage whose launch returned e
msa_status_t launched(hipError_t e, hipStream_t st, int kid) {
  if (e != hipSuccess) return hip_fail(e);
  if (!debug_sync_on()) return MSA_OK;
  e = hipStreamSynchronize(st);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) {
    g_last_error = std::string("MSA_DEBUG_SYNC: after stage ") + kKernelNames[kid] + ": " +
                   hipGetErrorString(e);
    return MSA_ERR_HIP;
  }
  return MSA_OK;
}

// MSA_DEBUG_SYNC: cu_seqlens_q / cu_seqlens_k (either may be NULL) must start
// at 0, not decrease, end at total_q / total_k (total_k: contiguous caches
// only) and agree with max_q_len / max_k_len and Lq_b <= Lk_b.
msa_status_t debug_check_seqlens(const msa_dims_t* d, const int32_t* cu_q, const int32_t* cu_k,
                                 hipStream_t st) {
  if (!debug_sync_on()) return MSA_OK;
  const int n = d->batch + 1;
  std::vector<int32_t> q(n, 0), k(n, 0);
  hipError_t e = hipStreamSynchronize(st);
  if (e == hipSuccess && cu_q) e = hipMemcpy(q.data(), cu_q, n * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e == hipSuccess && cu_k) e = hipMemcpy(k.data(), cu_k, n * sizeof(int32_t), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return hip_fail(e);
  for (int b = 0; b + 1 < n; ++b) {
    const long long lq = (long long)q[b + 1] - q[b], lk = (long long)k[b + 1] - k[b];
    if ((cu_q && (lq < 0 || lq > d->max_q_len)) || (cu_k && (lk < 0 || lk > d->max_k_len)) ||
        (cu_q && cu_k && lq > lk))
      return fail(MSA_ERR_BAD_DIMS, "MSA_DEBUG_SYNC: cu_seqlens do not match the dims");
  }
  if ((cu_q && (q[0] != 0 || q[n - 1] != d->total_q)) ||
      (cu_k && (k[0] != 0 || (d->kv_pages == 0 && k[n - 1] != d->total_k))))
    return fail(MSA_ERR_BAD_DIMS, "MSA_DEBUG_SYNC: cu_seqlens do not start at 0 or end at the totals");
  return MSA_OK;
}

}  // namespace

// Scratch of msa_attend_noalloc (the Main Branch's partials), for callers that
// cannot allocate.  Each GPU the library runs on holds its own copy for the
// life of the process.  Host code never passes `scratch` itself to a kernel
// (on the host it names a stand-in, not device memory): it uses the device
// address resolved by scratch_address() for the device of the call's stream.
static __device__ __align__(256) uint8_t scratch[MSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device `stream` belongs to (the current
// device for the NULL stream), looked up once per device with that device
// current and kept.
msa_status_t scratch_address(hipStream_t stream, void** out) {
  int cur = -1, dev = -1;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return hip_fail(e);
  dev = cur;
  if (stream) {
    e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return hip_fail(e);
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(MSA_ERR_UNSUPPORTED, "device ordinal above 63");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    hipError_t e2 = dev != cur ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return hip_fail(e);
    if (e2 != hipSuccess) return hip_fail(e2);
    if (!p || ((uintptr_t)p & 255u)) return fail(MSA_ERR_HIP, "scratch address missing or misaligned");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

}  // namespace

extern "C" {

int32_t msa_abi_version(void) { return MSA_ABI_VERSION; }

const char* msa_last_error(void) { return g_last_error.c_str(); }

const char* msa_status_string(msa_status_t s_in) {
  // a C caller may pass any int: read it as one (loading an out-of-range value
  // as this C++ enum would be undefined)
  int s;
  memcpy(&s, &s_in, sizeof s);
  switch (s) {
    case MSA_OK: return "MSA_OK";
    case MSA_ERR_NULL_ARG: return "MSA_ERR_NULL_ARG: a required pointer is NULL";
    case MSA_ERR_BAD_DIMS: return "MSA_ERR_BAD_DIMS: inconsistent or out-of-range sizes";
    case MSA_ERR_UNSUPPORTED: return "MSA_ERR_UNSUPPORTED: size not implemented by this build";
    case MSA_ERR_ALIGNMENT: return "MSA_ERR_ALIGNMENT: tensor pointer not 16-byte aligned";
    case MSA_ERR_WORKSPACE_TOO_SMALL: return "MSA_ERR_WORKSPACE_TOO_SMALL: workspace below msa_workspace_size()";
    case MSA_ERR_HIP: return "MSA_ERR_HIP: a HIP call failed";
  }
  return "MSA_ERR_UNKNOWN";
}

msa_status_t msa_workspace_size(const msa_dims_t* dims, msa_op_t op_in, size_t* bytes) {
  Derived x;
  msa_status_t s = check_dims(dims, &x);
  if (s != MSA_OK) return s;
  if (!bytes) return fail(MSA_ERR_NULL_ARG, "bytes is NULL");
  int op;   // any int from a C caller (see msa_status_string)
  memcpy(&op, &op_in, sizeof op);
  switch (op) {
    case MSA_OP_INDEX_SELECT: *bytes = ws_select(dims, x); return MSA_OK;
    case MSA_OP_BUILD_LISTS: *bytes = ws_lists(dims, x); return MSA_OK;
    case MSA_OP_ATTEND: *bytes = ws_attend(dims, x); return MSA_OK;
    case MSA_OP_INDEX_PROJECT: *bytes = ws_project(x); return MSA_OK;
  }
  return fail(MSA_ERR_BAD_DIMS, "unknown op");
}

msa_status_t msa_index_select(const msa_dims_t* dims, const void* q_idx, const void* k_idx,
                              const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                              int32_t* sel, float* sel_score, void* workspace,
                              size_t workspace_bytes, void* stream) {
  Derived x;
  msa_status_t s = check_dims(dims, &x);
  if (s != MSA_OK) return s;
  if (x.total_q == 0) return MSA_OK;   // no queries: nothing to select
  // a prefill workgroup scores whole queries: all G of their (query, group) rows
  if (!x.decode_path && x.G > msa::prefill_rows_per_wg())
    return fail(MSA_ERR_UNSUPPORTED, "num_kv_heads must be <= 512 when max_q_len * num_kv_heads > 128");
  if (!q_idx || !k_idx || !cu_seqlens_q || !cu_seqlens_k || !sel || !workspace)
    return fail(MSA_ERR_NULL_ARG, "a required pointer is NULL");
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(sel) || !aligned16(workspace) ||
      (sel_score && !aligned16(sel_score)))
    return fail(MSA_ERR_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  if (workspace_bytes < ws_select(dims, x))
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "index_select workspace too small");
  hipStream_t st = (hipStream_t)stream;
  if (msa_status_t v = debug_check_seqlens(dims, cu_seqlens_q, cu_seqlens_k, st); v != MSA_OK) return v;
  if (!x.decode_path) {
    ProfScope ps(K_INDEX_PREFILL, st);
    hipError_t e = msa::launch_index_select_prefill(q_idx, k_idx, cu_seqlens_q, cu_seqlens_k, x.kv,
                                                    dims->batch, x.G, x.DI, dims->max_q_len,
                                                    x.top_k, sel, sel_score, st);
    return launched(e, st, K_INDEX_PREFILL);
  }
  float* S = (float*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
  const long long chunk = select_chunk(dims, x);
  for (long long r0 = 0; r0 < x.total_q; r0 += chunk) {
    const int a = (int)r0, z = (int)std::min<long long>(x.total_q, r0 + chunk);
    const long long ld = (long long)(z - a) * x.G;
    hipError_t e;
    {
      ProfScope ps(K_INDEX_DECODE, st);
      e = msa::launch_index_score_decode(q_idx, k_idx, cu_seqlens_q, cu_seqlens_k, x.kv, dims->batch, x.G,
                                         x.DI, x.nb_max, dims->max_q_len * x.G, a, z, S, ld, st);
    }
    if (msa_status_t ls = launched(e, st, K_INDEX_DECODE); ls != MSA_OK) return ls;
    ProfScope ps(K_TOPK, st);
    e = msa::launch_topk_select(S, ld, x.nb_max, a, z, cu_seqlens_q, cu_seqlens_k, dims->batch, x.G, x.top_k,
                                sel, sel_score, st);
    if (msa_status_t ls = launched(e, st, K_TOPK); ls != MSA_OK) return ls;
  }
  return MSA_OK;
}

msa_status_t msa_index_project(const msa_dims_t* dims, int32_t model_dim, const void* x,
                               const void* w_q, const void* w_k, const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k, void* q_idx, void* k_idx,
                               void* workspace, size_t workspace_bytes, void* stream) {
  Derived x_;
  msa_status_t s = check_dims(dims, &x_);
  if (s != MSA_OK) return s;
  if (model_dim < 64 || model_dim % 64 || model_dim > 65536)
    return fail(MSA_ERR_UNSUPPORTED, "model_dim must be a multiple of 64 in 64..65536");
  if (x_.total_q == 0) return MSA_OK;   // no new tokens
  if (!x || !w_q || !w_k || !cu_seqlens_q || !cu_seqlens_k || !q_idx || !k_idx)
    return fail(MSA_ERR_NULL_ARG, "a required pointer is NULL");
  const size_t need = ws_project_required(x_);
  if (need && !workspace) return fail(MSA_ERR_NULL_ARG, "a required pointer is NULL");
  if (!aligned16(x) || !aligned16(w_q) || !aligned16(w_k) || !aligned16(q_idx) ||
      !aligned16(k_idx) || (workspace && !aligned16(workspace)))
    return fail(MSA_ERR_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  if (workspace_bytes < need)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "index_project workspace too small");
  hipStream_t st = (hipStream_t)stream;
  if (msa_status_t v = debug_check_seqlens(dims, cu_seqlens_q, cu_seqlens_k, st); v != MSA_OK) return v;
  ProfScope ps(K_PROJECT, st);
  hipError_t e = msa::launch_index_project(x, w_q, w_k, model_dim, x_.G, x_.DI, (int)x_.total_q,
                                           cu_seqlens_q, cu_seqlens_k, x_.kv, dims->batch, q_idx,
                                           k_idx, workspace, workspace ? workspace_bytes : 0, st);
  return launched(e, st, K_PROJECT);
}

msa_status_t msa_index_quantize_fp8(const msa_dims_t* dims, const void* q_idx, const void* k_idx,
                                    const int32_t* cu_seqlens_k, void* q_idx8, uint8_t* q_exp,
                                    void* k_idx8, uint8_t* k_exp, void* stream) {
  Derived x;
  msa_status_t s = check_dims(dims, &x);
  if (s != MSA_OK) return s;
  // either side may be left out (NULL input): e.g. a decode step quantises its
  // new queries against a key cache quantised when it was written
  const bool has_q = x.total_q > 0 && q_idx, has_k = dims->total_k > 0 && k_idx;
  if ((has_q && (!q_idx8 || !q_exp)) || (has_k && (!k_idx8 || !k_exp || !cu_seqlens_k)))
    return fail(MSA_ERR_NULL_ARG, "a required pointer is NULL");
  if ((has_q && (!aligned16(q_idx) || !aligned16(q_idx8))) ||
      (has_k && (!aligned16(k_idx) || !aligned16(k_idx8))))
    return fail(MSA_ERR_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  if (!has_q && !has_k) return MSA_OK;
  hipStream_t st = (hipStream_t)stream;
  ProfScope ps(K_QUANT_FP8, st);
  hipError_t e = msa::launch_quantize_index_fp8(x.DI, q_idx, k_idx, cu_seqlens_k, x.kv, dims->batch,
                                                has_k ? x.nb_max : 0,
                                                has_q ? x.total_q * x.G : 0, q_idx8, q_exp, k_idx8,
                                                k_exp, st);
  return launched(e, st, K_QUANT_FP8);
}

namespace {

// The Index Branch on 8-bit query codes against 8-bit (k4 = false) or 4-bit
// (k4 = true) key codes; both share the selection kernels' organisation.
msa_status_t select_q8(const msa_dims_t* dims, const void* q_idx8, const uint8_t* q_exp,
                       const void* k_codes, const uint8_t* k_exp, bool k4,
                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int32_t* sel,
                       float* sel_score, void* workspace, size_t workspace_bytes, void* stream) {
  Derived x;
  msa_status_t s = check_dims(dims, &x);
  if (s != MSA_OK) return s;
  if (!k4 && x.nb_max > msa::fp8_max_blocks_per_sequence())
    return fail(MSA_ERR_UNSUPPORTED, "max_k_len too long for the fp8 index kernels (16384 blocks)");
  if (x.total_q == 0) return MSA_OK;
  if (!x.decode_path && x.G > msa::fp8_prefill_rows_per_wg())
    return fail(MSA_ERR_UNSUPPORTED, "num_kv_heads must be <= 256 when max_q_len * num_kv_heads > 128");
  if (!q_idx8 || !q_exp || !k_codes || !k_exp || !cu_seqlens_q || !cu_seqlens_k || !sel || !workspace)
    return fail(MSA_ERR_NULL_ARG, "a required pointer is NULL");
  if (!aligned16(q_idx8) || !aligned16(k_codes) || !aligned16(sel) || !aligned16(workspace) ||
      (sel_score && !aligned16(sel_score)) || (k4 && !aligned16(k_exp)))
    return fail(MSA_ERR_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  if (workspace_bytes < ws_select(dims, x))
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "index_select workspace too small");
  hipStream_t st = (hipStream_t)stream;
  if (msa_status_t v = debug_check_seqlens(dims, cu_seqlens_q, cu_seqlens_k, st); v != MSA_OK) return v;
  if (!x.decode_path) {
    ProfScope ps(k4 ? K_INDEX_PREFILL_Q8K4 : K_INDEX_PREFILL_FP8, st);
    hipError_t e = msa::launch_index_select_prefill_fp8(q_idx8, q_exp, k_codes, k_exp, k4,
                                                        cu_seqlens_q, cu_seqlens_k, x.kv,
                                                        dims->batch, x.G, x.DI, x.nb_max,
                                                        dims->max_q_len, x.top_k, sel, sel_score, st);
    return launched(e, st, k4 ? K_INDEX_PREFILL_Q8K4 : K_INDEX_PREFILL_FP8);
  }
  float* S = (float*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
  const long long chunk = select_chunk(dims, x);
  for (long long r0 = 0; r0 < x.total_q; r0 += chunk) {
    const int a = (int)r0, z = (int)std::min<long long>(x.total_q, r0 + chunk);
    const long long ld = (long long)(z - a) * x.G;
    hipError_t e;
    {
      ProfScope ps(k4 ? K_INDEX_DECODE_Q8K4 : K_INDEX_DECODE_FP8, st);
      e = msa::launch_index_score_decode_fp8(q_idx8, q_exp, k_codes, k_exp, k4, cu_seqlens_q,
                                             cu_seqlens_k, x.kv, dims->batch, x.G, x.DI, x.nb_max,
                                             dims->max_q_len * x.G, a, z, S, ld, st);
    }
    if (msa_status_t ls = launched(e, st, k4 ? K_INDEX_DECODE_Q8K4 : K_INDEX_DECODE_FP8); ls != MSA_OK) return ls;
    ProfScope ps(K_TOPK, st);
    e = msa::launch_topk_select(S, ld, x.nb_max, a, z, cu_seqlens_q, cu_seqlens_k, dims->batch, x.G, x.top_k,
                                sel, sel_score, st);
    if (msa_status_t ls = launched(e, st, K_TOPK); ls != MSA_OK) return ls;
  }
  return MSA_OK;
}

}  // namespace

msa_status_t msa_index_select_fp8(const msa_dims_t* dims, const void* q_idx8, const uint8_t* q_exp,
                                  const void* k_idx8, const uint8_t* k_exp,
                                  const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                  int32_t* sel, float* sel_score, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  return select_q8(dims, q_idx8, q_exp, k_idx8, k_exp, false, cu_seqlens_q, cu_seqlens_k, sel,
                   sel_score, workspace, workspace_bytes, stream);
}

msa_status_t msa_index_quantize_q8k4(const msa_dims_t* dims, const void* q_idx, const void* k_idx,
                                     const int32_t* cu_seqlens_k, void* q_idx8, uint8_t* q_exp,
                                     void* k_idx4, uint8_t* k_exp4, void* stream) {
  Derived x;
  msa_status_t s = check_dims(dims, &x);
  if (s != MSA_OK) return s;
  const bool has_q = x.total_q > 0 && q_idx, has_k = dims->total_k > 0 && k_idx;
  if ((has_q && (!q_idx8 || !q_exp)) || (has_k && (!k_idx4 || !k_exp4 || !cu_seqlens_k)))
    return fail(MSA_ERR_NULL_ARG, "a required pointer is NULL");
  if ((has_q && (!aligned16(q_idx) || !aligned16(q_idx8))) ||
      (has_k && (!aligned16(k_idx) || !aligned16(k_idx4) || !aligned16(k_exp4))))
    return fail(MSA_ERR_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  if (!has_q && !has_k) return MSA_OK;
  hipStream_t st = (hipStream_t)stream;
  ProfScope ps(K_QUANT_Q8K4, st);
  hipError_t e = msa::launch_quantize_index_q8k4(x.DI, q_idx, k_idx, cu_seqlens_k, x.kv, dims->batch,
                                                 has_k ? x.nb_max : 0,
                                                 has_q ? x.total_q * x.G : 0, q_idx8, q_exp, k_idx4,
                                                 k_exp4, st);
  return launched(e, st, K_QUANT_Q8K4);
}

msa_status_t msa_index_select_q8k4(const msa_dims_t* dims, const void* q_idx8, const uint8_t* q_exp,
                                   const void* k_idx4, const uint8_t* k_exp4,
                                   const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                   int32_t* sel, float* sel_score, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  return select_q8(dims, q_idx8, q_exp, k_idx4, k_exp4, true, cu_seqlens_q, cu_seqlens_k, sel,
                   sel_score, workspace, workspace_bytes, stream);
}

msa_status_t msa_build_block_query_lists(const msa_dims_t* dims, const int32_t* sel,
                                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                         int32_t* block_offsets, int32_t* block_entries,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  Derived x;
  msa_status_t s = check_dims(dims, &x);
  if (s != MSA_OK) return s;
  // with no queries the offsets are still written (all zero); sel/entries are not touched
  if (!cu_seqlens_q || !cu_seqlens_k || !block_offsets || !workspace ||
      (x.total_q > 0 && (!sel || !block_entries)))
    return fail(MSA_ERR_NULL_ARG, "a required pointer is NULL");
  if (!aligned16(sel) || !aligned16(block_offsets) || !aligned16(block_entries) || !aligned16(workspace))
    return fail(MSA_ERR_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  if (workspace_bytes < ws_lists(dims, x))
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "build_lists workspace too small");
  if (msa_status_t v = debug_check_seqlens(dims, cu_seqlens_q, cu_seqlens_k, (hipStream_t)stream); v != MSA_OK)
    return v;
  void* ws = (void*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
  ProfScope ps(K_LISTS, (hipStream_t)stream);
  hipError_t e = msa::launch_build_lists(sel, cu_seqlens_q, cu_seqlens_k, dims->batch, x.G, x.top_k,
                                         x.nqt_max, x.nb_max, block_offsets, block_entries, ws,
                                         (hipStream_t)stream);
  return launched(e, (hipStream_t)stream, K_LISTS);
}

// decode-shaped steps attend per (query, slot) from the selection alone
static bool reads_lists(const msa_dims_t* d) { return d->max_q_len > kDecodeAttendMaxQ; }

int32_t msa_attend_reads_lists(const msa_dims_t* dims) {
  Derived x;
  msa_status_t s = check_dims(dims, &x);
  if (s != MSA_OK) return -(int32_t)s;
  return reads_lists(dims) ? 1 : 0;
}

int64_t msa_attend_pass_rows(const msa_dims_t* dims) {
  Derived x;
  msa_status_t s = check_dims(dims, &x);
  if (s != MSA_OK) return -(int64_t)s;
  return attend_chunk(dims, x);
}

static msa_status_t attend_impl(const msa_dims_t* dims, const void* q, const void* k,
                                const void* v, msa::MainFp8 f8, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_k, const int32_t* sel,
                                const int32_t* block_offsets, const int32_t* block_entries,
                                void* out, float* lse, float* block_mass, void* workspace,
                                size_t workspace_bytes, void* stream) {
  Derived x;
  msa_status_t s = check_dims(dims, &x);
  if (s != MSA_OK) return s;
  if (x.total_q == 0) return MSA_OK;   // no queries: no output
  const bool lists = reads_lists(dims);
  if (!q || !k || !v || !cu_seqlens_q || !cu_seqlens_k || !sel || !out || !workspace ||
      (lists && (!block_offsets || !block_entries)) ||
      (f8.qe != nullptr) != (f8.ke != nullptr) || (f8.qe != nullptr) != (f8.ve != nullptr))
    return fail(MSA_ERR_NULL_ARG, "a required pointer is NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(sel) || !aligned16(out) ||
      !aligned16(workspace) || (lists && (!aligned16(block_offsets) || !aligned16(block_entries))) ||
      (lse && !aligned16(lse)) || (f8.kv4 && (!aligned16(f8.ke) || !aligned16(f8.ve))))
    return fail(MSA_ERR_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  if (workspace_bytes < ws_attend(dims, x))
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL, "attend workspace too small");
  hipStream_t st = (hipStream_t)stream;
  if (msa_status_t dv = debug_check_seqlens(dims, cu_seqlens_q, cu_seqlens_k, st); dv != MSA_OK) return dv;
  const long long chunk = attend_chunk(dims, x);
  char* base = (char*)(((uintptr_t)workspace + 255) & ~(uintptr_t)255);
  void* part_acc = base;
  float2* part_ml = (float2*)(base + align256(attend_rows(dims, x) * acc_bytes(x)));
  const float scale_log2 = x.scale * 1.44269504088896340736f;
  for (long long r0 = 0; r0 < x.total_q; r0 += chunk) {
    const int a = (int)r0, z = (int)std::min<long long>(x.total_q, r0 + chunk);
    hipError_t e;
    {
      ProfScope ps(K_ATTEND, st);
      if (!lists)
        // a few queries per sequence: each selected block is hit by few queries;
        // one workgroup per (group, slot, query) reads it straight from the selection
        e = msa::launch_attend_decode(x.D, x.hpg, q, k, v, f8, cu_seqlens_q, cu_seqlens_k, x.kv,
                                      dims->batch, x.G, x.Hq, x.top_k, x.nb_max, sel, a, z,
                                      scale_log2, (float*)part_acc, part_ml, st);
      else
        e = msa::launch_attend_blocks(x.D, x.hpg, x.compact, q, k, v, f8, cu_seqlens_q, cu_seqlens_k, x.kv,
                                      dims->batch, x.G, x.Hq, x.top_k, x.nb_max, block_offsets,
                                      block_entries, a, z, (int)x.total_q, scale_log2, part_acc,
                                      part_ml, st);
    }
    if (msa_status_t ls = launched(e, st, K_ATTEND); ls != MSA_OK) return ls;
    {
      ProfScope ps(K_MERGE, st);
      e = msa::launch_merge(x.D, x.compact, part_acc, part_ml, sel, a, z, x.Hq, x.G, x.top_k, out,
                            lse, st);
    }
    if (msa_status_t ls = launched(e, st, K_MERGE); ls != MSA_OK) return ls;
    if (block_mass) {
      ProfScope ps(K_MASS, st);
      e = msa::launch_block_mass(x.hpg, part_ml, sel, a, z, x.G, x.top_k, block_mass, st);
      if (msa_status_t ls = launched(e, st, K_MASS); ls != MSA_OK) return ls;
    }
  }
  return MSA_OK;
}

msa_status_t msa_attend(const msa_dims_t* dims, const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        const int32_t* sel, const int32_t* block_offsets,
                        const int32_t* block_entries, void* out, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream) {
  return attend_impl(dims, q, k, v, msa::MainFp8{nullptr, nullptr, nullptr}, cu_seqlens_q,
                     cu_seqlens_k, sel, block_offsets, block_entries, out, lse, nullptr, workspace,
                     workspace_bytes, stream);
}

msa_status_t msa_attend_noalloc(const msa_dims_t* dims, const void* q, const void* k,
                                const void* v, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_k, const int32_t* sel,
                                const int32_t* block_offsets, const int32_t* block_entries,
                                void* out, float* lse, void* stream) {
  Derived x;
  msa_status_t s = check_dims(dims, &x);
  if (s != MSA_OK) return s;
  if (ws_attend(dims, x) > (size_t)MSA_NOALLOC_SCRATCH_BYTES)
    return fail(MSA_ERR_WORKSPACE_TOO_SMALL,
                "msa_attend_noalloc: the partials of one pass exceed the library's "
                "MSA_NOALLOC_SCRATCH_BYTES scratch; set dims->q_chunk so that "
                "msa_workspace_size(dims, MSA_OP_ATTEND) <= MSA_NOALLOC_SCRATCH_BYTES");
  if (x.total_q == 0) return MSA_OK;
  void* ws = nullptr;
  s = scratch_address((hipStream_t)stream, &ws);
  if (s != MSA_OK) return s;
  return attend_impl(dims, q, k, v, msa::MainFp8{nullptr, nullptr, nullptr}, cu_seqlens_q,
                     cu_seqlens_k, sel, block_offsets, block_entries, out, lse, nullptr, ws,
                     (size_t)MSA_NOALLOC_SCRATCH_BYTES, stream);
}

msa_status_t msa_attend_fp8(const msa_dims_t* dims, const void* q8, const uint8_t* q_exp,
                            const void* k8, const uint8_t* k_exp, const void* v8,
                            const uint8_t* v_exp, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, const int32_t* sel,
                            const int32_t* block_offsets, const int32_t* block_entries, void* out,
                            float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (dims && dims->total_q > 0 && (!q_exp || !k_exp || !v_exp))
    return fail(MSA_ERR_NULL_ARG, "a required pointer is NULL");
  return attend_impl(dims, q8, k8, v8, msa::MainFp8{q_exp, k_exp, v_exp}, cu_seqlens_q,
                     cu_seqlens_k, sel, block_offsets, block_entries, out, lse, nullptr, workspace,
                     workspace_bytes, stream);
}

msa_status_t msa_attend_q8kv4(const msa_dims_t* dims, const void* q8, const uint8_t* q_exp,
                              const void* k4, const uint8_t* k_exp4, const void* v4,
                              const uint8_t* v_exp4, const int32_t* cu_seqlens_q,
                              const int32_t* cu_seqlens_k, const int32_t* sel,
                              const int32_t* block_offsets, const int32_t* block_entries, void* out,
                              float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (dims && dims->total_q > 0 && (!q_exp || !k_exp4 || !v_exp4))
    return fail(MSA_ERR_NULL_ARG, "a required pointer is NULL");
  return attend_impl(dims, q8, k4, v4, msa::MainFp8{q_exp, k_exp4, v_exp4, 1}, cu_seqlens_q,
                     cu_seqlens_k, sel, block_offsets, block_entries, out, lse, nullptr, workspace,
                     workspace_bytes, stream);
}

msa_status_t msa_main_quantize_fp8(const msa_dims_t* dims, const void* q, const void* k,
                                   const void* v, const int32_t* cu_seqlens_k, void* q8,
                                   uint8_t* q_exp, void* k8, uint8_t* k_exp, void* v8,
                                   uint8_t* v_exp, void* stream) {
  Derived x;
  msa_status_t s = check_dims(dims, &x);
  if (s != MSA_OK) return s;
  // any of q, k, v may be left out (NULL input): a decode step quantises its new
  // queries against a key/value cache quantised when it was written
  const bool has_q = x.total_q > 0 && q, has_kv = dims->total_k > 0;
  const bool has_k = has_kv && k, has_v = has_kv && v;
  if ((has_q && (!q8 || !q_exp)) || ((has_k || has_v) && !cu_seqlens_k) ||
      (has_k && (!k8 || !k_exp)) || (has_v && (!v8 || !v_exp)))
    return fail(MSA_ERR_NULL_ARG, "a required pointer is NULL");
  if ((has_q && (!aligned16(q) || !aligned16(q8))) || (has_k && (!aligned16(k) || !aligned16(k8))) ||
      (has_v && (!aligned16(v) || !aligned16(v8))))
    return fail(MSA_ERR_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  if (!has_q && !has_k && !has_v) return MSA_OK;
  hipStream_t st = (hipStream_t)stream;
  ProfScope ps(K_QUANT_MAIN_FP8, st);
  hipError_t e = msa::launch_main_quantize_fp8(
      x.D, has_q ? q : nullptr, has_k ? k : nullptr, has_v ? v : nullptr, cu_seqlens_k, x.kv,
      dims->batch, x.G, x.nb_max, has_q ? x.total_q * x.Hq : 0, q8, q_exp, k8, k_exp, v8, v_exp, st);
  return launched(e, st, K_QUANT_MAIN_FP8);
}

msa_status_t msa_main_quantize_q8kv4(const msa_dims_t* dims, const void* q, const void* k,
                                     const void* v, const int32_t* cu_seqlens_k, void* q8,
                                     uint8_t* q_exp, void* k4, uint8_t* k_exp4, void* v4,
                                     uint8_t* v_exp4, void* stream) {
  Derived x;
  msa_status_t s = check_dims(dims, &x);
  if (s != MSA_OK) return s;
  const bool has_q = x.total_q > 0 && q, has_kv = dims->total_k > 0;
  const bool has_k = has_kv && k, has_v = has_kv && v;
  if ((has_q && (!q8 || !q_exp)) || ((has_k || has_v) && !cu_seqlens_k) ||
      (has_k && (!k4 || !k_exp4)) || (has_v && (!v4 || !v_exp4)))
    return fail(MSA_ERR_NULL_ARG, "a required pointer is NULL");
  if ((has_q && (!aligned16(q) || !aligned16(q8))) ||
      (has_k && (!aligned16(k) || !aligned16(k4) || !aligned16(k_exp4))) ||
      (has_v && (!aligned16(v) || !aligned16(v4) || !aligned16(v_exp4))))
    return fail(MSA_ERR_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  if (!has_q && !has_k && !has_v) return MSA_OK;
  hipStream_t st = (hipStream_t)stream;
  ProfScope ps(K_QUANT_MAIN_Q8KV4, st);
  hipError_t e = msa::launch_main_quantize_q8kv4(
      x.D, has_q ? q : nullptr, has_k ? k : nullptr, has_v ? v : nullptr, cu_seqlens_k, x.kv,
      dims->batch, x.G, x.nb_max, has_q ? x.total_q * x.Hq : 0, q8, q_exp, k4, k_exp4, v4, v_exp4,
      st);
  return launched(e, st, K_QUANT_MAIN_Q8KV4);
}

msa_status_t msa_attend_with_mass(const msa_dims_t* dims, const void* q, const void* k,
                                  const void* v, const int32_t* cu_seqlens_q,
                                  const int32_t* cu_seqlens_k, const int32_t* sel,
                                  const int32_t* block_offsets, const int32_t* block_entries,
                                  void* out, float* lse, float* block_mass, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (dims && (dims->flags & MSA_FLAG_COMPACT_PARTIALS))
    return fail(MSA_ERR_UNSUPPORTED, "block masses need fp32 partials (MSA_FLAG_COMPACT_PARTIALS)");
  if (dims && dims->total_q > 0 && !block_mass)
    return fail(MSA_ERR_NULL_ARG, "block_mass is NULL");
  if (block_mass && !aligned16(block_mass))
    return fail(MSA_ERR_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  return attend_impl(dims, q, k, v, msa::MainFp8{nullptr, nullptr, nullptr}, cu_seqlens_q,
                     cu_seqlens_k, sel, block_offsets, block_entries, out, lse, block_mass,
                     workspace, workspace_bytes, stream);
}

msa_status_t msa_index_kl(const msa_dims_t* dims, const void* q_idx, const void* k_idx,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          const int32_t* sel, const float* sel_score, const float* block_mass,
                          float* log_q, float* kl, void* stream) {
  Derived x;
  msa_status_t s = check_dims(dims, &x);
  if (s != MSA_OK) return s;
  if (x.total_q == 0) return MSA_OK;
  if (!q_idx || !k_idx || !cu_seqlens_q || !cu_seqlens_k || !sel || !sel_score || !block_mass || !kl)
    return fail(MSA_ERR_NULL_ARG, "a required pointer is NULL");
  if (!aligned16(q_idx) || !aligned16(k_idx) || !aligned16(sel) || !aligned16(sel_score) ||
      !aligned16(block_mass) || !aligned16(kl) || (log_q && !aligned16(log_q)))
    return fail(MSA_ERR_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  hipStream_t st = (hipStream_t)stream;
  if (msa_status_t v = debug_check_seqlens(dims, cu_seqlens_q, cu_seqlens_k, st); v != MSA_OK) return v;
  ProfScope ps(K_INDEX_KL, st);
  hipError_t e = msa::launch_index_kl(x.DI, q_idx, k_idx, cu_seqlens_q, cu_seqlens_k, x.kv, dims->batch,
                                      x.G, x.top_k, dims->max_q_len, sel, sel_score, block_mass,
                                      log_q, kl, st);
  return launched(e, st, K_INDEX_KL);
}

msa_status_t msa_hbm_stream(const void* src, size_t read_bytes, int32_t ratio, void* dst,
                            void* sink, void* stream) {
  if (!src || !sink || (ratio > 0 && !dst)) return fail(MSA_ERR_NULL_ARG, "a required pointer is NULL");
  if (ratio < 0 || ratio > 4) return fail(MSA_ERR_BAD_DIMS, "ratio must be in 0..4");
  if (read_bytes == 0 || read_bytes % 16) return fail(MSA_ERR_BAD_DIMS, "read_bytes must be a positive multiple of 16");
  if (!aligned16(src) || !aligned16(sink) || (ratio > 0 && !aligned16(dst)))
    return fail(MSA_ERR_ALIGNMENT, "tensor pointers must be 16-byte aligned");
  const long long units = (long long)(read_bytes / 16);
  const long long wgs = (units + 255) / 256;
  const int grid = (int)std::min<long long>(wgs, MSA_HBM_STREAM_MAX_WORKGROUPS);
  hipError_t e = msa::launch_hbm_stream(src, units, ratio, dst, sink, grid, (hipStream_t)stream);
  return e == hipSuccess ? MSA_OK : hip_fail(e);
}

msa_status_t msa_profile_enable(int32_t enable) {
  g_prof_on.store(enable != 0);
  return MSA_OK;
}

msa_status_t msa_profile_collect(float* total_ms, int32_t* launches) {
  if (!total_ms || !launches) return fail(MSA_ERR_NULL_ARG, "profile output is NULL");
  for (int i = 0; i < MSA_PROFILE_KERNELS; ++i) {
    total_ms[i] = 0.f;
    launches[i] = 0;
  }
  std::vector<ProfRec> recs;
  {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    recs.swap(g_prof_pending);
  }
  msa_status_t st = MSA_OK;
  for (const ProfRec& r : recs) {
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
    if (e != hipSuccess) {
      st = hip_fail(e);
    } else {
      total_ms[r.kid] += ms;
      launches[r.kid] += 1;
    }
  }
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (const ProfRec& r : recs) {
    g_event_pool.push_back(r.a);
    g_event_pool.push_back(r.b);
  }
  return st;
}

const char* msa_profile_kernel_name(int32_t id) {
  return (id >= 0 && id < MSA_PROFILE_KERNELS) ? kKernelNames[id] : "";
}

}  // extern "C"
