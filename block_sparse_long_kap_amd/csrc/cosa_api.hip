// Host side of the C ABI declared in include/cosa.h: argument validation,
// sizing and kernel launches.  No allocation and no synchronisation; the
// state kept between calls is a thread-local text for the last error and,
// per device, the address of the static workspace of the no-allocation
// proxy entry point.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>

#include <mutex>

#include "cosa.h"
#include "cosa_internal.h"

#define COSA_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

thread_local char g_last_error[256] = "";

cosa_status fail(cosa_status st, const char* msg) {
  snprintf(g_last_error, sizeof(g_last_error), "%s", msg);
  return st;
}
cosa_status ok() {
  g_last_error[0] = '\0';
  return COSA_OK;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool budget_to_ppm(float budget, int32_t* ppm) {
  if (!(budget > 0.f) || !(budget <= 1.f)) return false;
  const double v = floor((double)budget * 1e6 + 0.5);
  *ppm = (int32_t)(v < 1.0 ? 1.0 : v);
  return true;
}

int64_t budget_count(int64_t n, int32_t ppm) {
  if (n <= 0) return 0;
  int64_t k = (n * ppm + 999999) / 1000000;
  if (k < 1) k = 1;
  if (k > n) k = n;
  return k;
}

cosa_status validate(const cosa_problem* p) {
  if (p == nullptr) return fail(COSA_ERR_INVALID_ARG, "problem is null");
  if (p->batch < 1) return fail(COSA_ERR_INVALID_ARG, "batch must be >= 1");
  if (p->num_kv_heads < 1 || p->num_q_heads < 1 || p->num_q_heads % p->num_kv_heads != 0)
    return fail(COSA_ERR_INVALID_ARG, "num_q_heads must be a positive multiple of num_kv_heads");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(COSA_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (p->q_block != 64 && p->q_block != 128)
    return fail(COSA_ERR_UNSUPPORTED, "q_block must be 64 or 128");
  if (p->page_size != cosa::kPage) return fail(COSA_ERR_UNSUPPORTED, "page_size must be 64");
  if (p->kv_block != p->page_size && p->kv_block != 2 * p->page_size)
    return fail(COSA_ERR_UNSUPPORTED, "kv_block must be page_size or 2 * page_size");
  if (p->max_seqlen < 1 || p->max_seqlen > (1 << 20))
    return fail(COSA_ERR_INVALID_ARG, "max_seqlen must lie in [1, 2^20]");
  if (p->max_pages_per_seq <
      ceil_div(p->max_seqlen, p->kv_block) * (p->kv_block / p->page_size))
    return fail(COSA_ERR_INVALID_ARG,
                "max_pages_per_seq < ceil(max_seqlen / kv_block) * (kv_block / page_size)");
  if (p->num_pages < 1) return fail(COSA_ERR_INVALID_ARG, "num_pages must be >= 1");
  if (p->total_q < 0 || p->total_q > (int64_t)p->batch * p->max_seqlen)
    return fail(COSA_ERR_INVALID_ARG, "total_q must lie in [0, batch * max_seqlen]");
  if (!(p->softmax_scale > 0.f) || !isfinite(p->softmax_scale))
    return fail(COSA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (p->cu_seqlens == nullptr || p->page_table == nullptr)
    return fail(COSA_ERR_INVALID_ARG, "cu_seqlens and page_table must be non-null");
  const int64_t grid = (int64_t)p->batch * p->num_q_heads * ceil_div(p->max_seqlen, p->q_block);
  if (grid > 0x7FFFFFFFLL) return fail(COSA_ERR_UNSUPPORTED, "too many query tiles");
  return ok();
}

cosa_status hip_status(hipError_t e) {
  if (e == hipSuccess) return ok();
  return fail(COSA_ERR_HIP, hipGetErrorString(e));
}

int32_t xcd_groups(const cosa_problem* p) {
  const int64_t groups = (int64_t)p->batch * p->num_kv_heads;
  return (groups % 8 == 0 && groups <= 0x7FFFFFFF) ? (int32_t)groups : 0;
}

void fill_attn(cosa::AttnParams& a, const cosa_problem* p, const void* q, const void* k_pool,
               const void* v_pool, void* out, float* lse) {
  a.q = static_cast<const uint16_t*>(q);
  a.k_pool = static_cast<const uint16_t*>(k_pool);
  a.v_pool = static_cast<const uint16_t*>(v_pool);
  a.out = static_cast<uint16_t*>(out);
  a.lse = lse;
  a.cu_seqlens = p->cu_seqlens;
  a.page_table = p->page_table;
  a.ordered_blocks = nullptr;
  a.ordered_pages = nullptr;
  a.counts = nullptr;
  a.skip_record = nullptr;
  a.row_stats = nullptr;
  a.mask_heads = p->num_q_heads;
  a.ppb = p->kv_block / p->page_size;
  a.block_mask = nullptr;
  a.mask_words = 0;
  a.capacity = 0;
  a.total_q = p->total_q;
  a.batch = p->batch;
  a.hq = p->num_q_heads;
  a.hkv = p->num_kv_heads;
  a.max_pages = p->max_pages_per_seq;
  a.nqb = (int32_t)ceil_div(p->max_seqlen, p->q_block);
  a.xcd_groups = xcd_groups(p);
  {
    const int64_t units = (int64_t)p->batch * p->num_kv_heads * a.nqb;
    a.xcd_units = units % 8 == 0 ? (int32_t)units : 0;
  }
#ifndef COSA_TILE_ORDER
#define COSA_TILE_ORDER cosa::kOrderGroupXcd
#endif
  a.order = COSA_TILE_ORDER;
  a.group_begin = 0;
  a.group_count = 0;
  if (a.order == cosa::kOrderXcdGroup && a.xcd_groups == 0) a.order = cosa::kOrderLevel;
  if (a.order == cosa::kOrderGroupXcd && a.xcd_units == 0) a.order = cosa::kOrderGroupMajor;
  a.scale_log2 = p->softmax_scale * 1.4426950408889634f;
  a.skip_mode = cosa::kSkipOff;
  a.tau_log2 = 0.f;
  a.log2_delta = 0.f;
}

}  // namespace

COSA_EXPORT int32_t cosa_abi_version(void) { return COSA_ABI_VERSION; }

COSA_EXPORT const char* cosa_status_string(cosa_status s) {
  switch (s) {
    case COSA_OK: return "COSA_OK";
    case COSA_ERR_INVALID_ARG: return "COSA_ERR_INVALID_ARG";
    case COSA_ERR_UNSUPPORTED: return "COSA_ERR_UNSUPPORTED";
    case COSA_ERR_WORKSPACE: return "COSA_ERR_WORKSPACE";
    case COSA_ERR_HIP: return "COSA_ERR_HIP";
  }
  return "COSA_ERR_UNKNOWN";
}

COSA_EXPORT const char* cosa_last_error(void) { return g_last_error; }

COSA_EXPORT cosa_status cosa_validate_problem(const cosa_problem* p) { return validate(p); }

COSA_EXPORT int64_t cosa_num_q_tiles(const cosa_problem* p) {
  const cosa_status st = validate(p);
  if (st != COSA_OK) return st;
  return ceil_div(p->max_seqlen, p->q_block);
}

COSA_EXPORT int64_t cosa_mask_capacity(const cosa_problem* p, float budget) {
  const cosa_status st = validate(p);
  if (st != COSA_OK) return st;
  int32_t ppm;
  if (!budget_to_ppm(budget, &ppm)) return fail(COSA_ERR_INVALID_ARG, "budget must lie in (0, 1]");
  return budget_count(ceil_div(p->max_seqlen, p->kv_block), ppm);
}

COSA_EXPORT size_t cosa_kap_workspace_size(const cosa_problem* p) {
  if (validate(p) != COSA_OK) return 0;
  const int64_t n_max = ceil_div(p->max_seqlen, p->kv_block);
  // pooled keys as a bf16 hi plane and a bf16 lo plane, blocks padded to a
  // multiple of 32
  const int64_t n_pad = ceil_div(n_max, 32) * 32;
  return (size_t)2 * p->batch * p->num_kv_heads * p->head_dim * n_pad * sizeof(uint16_t);
}

COSA_EXPORT cosa_status cosa_check_page_table_host(const cosa_problem* p,
                                                   const int32_t* cu_host,
                                                   const int32_t* table_host) {
  cosa_status st = validate(p);
  if (st != COSA_OK) return st;
  if (cu_host == nullptr || table_host == nullptr)
    return fail(COSA_ERR_INVALID_ARG, "host arrays must be non-null");
  if (cu_host[0] != 0) return fail(COSA_ERR_INVALID_ARG, "cu_seqlens[0] must be 0");
  for (int b = 0; b < p->batch; ++b) {
    const int64_t len = (int64_t)cu_host[b + 1] - cu_host[b];
    if (len < 0) return fail(COSA_ERR_INVALID_ARG, "cu_seqlens must be non-decreasing");
    if (len > p->max_seqlen) return fail(COSA_ERR_INVALID_ARG, "a sequence exceeds max_seqlen");
    const int64_t pages = ceil_div(len, p->page_size);
    for (int64_t j = 0; j < pages; ++j) {
      const int32_t pg = table_host[(int64_t)b * p->max_pages_per_seq + j];
      if (pg < 0 || pg >= p->num_pages)
        return fail(COSA_ERR_INVALID_ARG, "page id out of [0, num_pages)");
    }
  }
  if (cu_host[p->batch] != p->total_q)
    return fail(COSA_ERR_INVALID_ARG, "cu_seqlens[batch] != total_q");
  return ok();
}

namespace {

// Validates the proxy's arguments and fills its kernel parameters
// (check_workspace false: the caller supplies the workspace afterwards).
cosa_status build_kap(cosa::KapParams& k, const cosa_problem* p, const void* q, const void* k_pool,
                      float budget, uint64_t top_p_fx, bool shared, int32_t* ordered_blocks,
                      int32_t* ordered_pages, int32_t* counts, int32_t* hrm_counts, float* debug_w,
                      uint8_t* debug_hrm, int64_t capacity, void* workspace,
                      size_t workspace_bytes, bool check_workspace = true) {
  cosa_status st = validate(p);
  if (st != COSA_OK) return st;
  if (q == nullptr || k_pool == nullptr || ordered_blocks == nullptr ||
      ordered_pages == nullptr || counts == nullptr)
    return fail(COSA_ERR_INVALID_ARG, "q, k_pool, ordered_blocks, ordered_pages, counts required");
  int32_t ppm;
  if (!budget_to_ppm(budget, &ppm)) return fail(COSA_ERR_INVALID_ARG, "budget must lie in (0, 1]");
  const int64_t n_max = ceil_div(p->max_seqlen, p->kv_block);
  if (n_max > cosa::kMaxCandidates)
    return fail(COSA_ERR_UNSUPPORTED, "the proxy handles at most 2048 key blocks per sequence");
  if (capacity < budget_count(n_max, ppm))
    return fail(COSA_ERR_INVALID_ARG, "capacity < cosa_mask_capacity(problem, budget)");
  const size_t need = cosa_kap_workspace_size(p);
  if (check_workspace && (workspace == nullptr || workspace_bytes < need))
    return fail(COSA_ERR_WORKSPACE, "workspace null or smaller than cosa_kap_workspace_size()");
  k.q = static_cast<const uint16_t*>(q);
  k.k_pool = static_cast<const uint16_t*>(k_pool);
  k.cu_seqlens = p->cu_seqlens;
  k.page_table = p->page_table;
  k.kbar = static_cast<uint16_t*>(workspace);
  k.ordered_blocks = ordered_blocks;
  k.ordered_pages = ordered_pages;
  k.counts = counts;
  k.hrm_counts = hrm_counts;
  k.debug_w = debug_w;
  k.debug_hrm = debug_hrm;
  k.capacity = capacity;
  k.batch = p->batch;
  k.hq = p->num_q_heads;
  k.hkv = p->num_kv_heads;
  k.max_pages = p->max_pages_per_seq;
  k.nqb = (int32_t)ceil_div(p->max_seqlen, p->q_block);
  k.n_max = (int32_t)n_max;
  k.kv_block = p->kv_block;
  k.ppb = p->kv_block / p->page_size;
  k.beta_ppm = ppm;
  k.scale = p->softmax_scale;
  k.top_p_fx = top_p_fx;
  k.group_begin = 0;
  k.group_count = 0;
  k.shared_heads = 0;
  if (shared) {
    const int hg = p->num_q_heads / p->num_kv_heads;
    // one KV head per query head: the shared mask is the per-head mask
    if (hg > 1) {
      if (hg * (p->q_block / cosa::kProxyRows) > 32 || (hg & (hg - 1)) != 0)
        return fail(COSA_ERR_UNSUPPORTED,
                    "shared masks need (q_heads / kv_heads) * (q_block / 16) <= 32, a power of 2");
      k.shared_heads = hg;
    }
  }
  return COSA_OK;
}

cosa_status proxy_mask(const cosa_problem* p, const void* q, const void* k_pool, float budget,
                       uint64_t top_p_fx, bool shared, int32_t* ordered_blocks, int32_t* ordered_pages,
                       int32_t* counts, int32_t* hrm_counts, float* debug_w, uint8_t* debug_hrm,
                       int64_t capacity, void* workspace, size_t workspace_bytes, void* stream) {
  cosa::KapParams k;
  const cosa_status st =
      build_kap(k, p, q, k_pool, budget, top_p_fx, shared, ordered_blocks, ordered_pages, counts,
                hrm_counts, debug_w, debug_hrm, capacity, workspace, workspace_bytes);
  if (st != COSA_OK) return st;
  return hip_status(cosa::launch_kap(k, p->head_dim, p->q_block, (hipStream_t)stream));
}

}  // namespace

COSA_EXPORT cosa_status cosa_proxy_ordered_mask(const cosa_problem* p, const void* q,
                                                const void* k_pool, float budget,
                                                int32_t* ordered_blocks, int32_t* ordered_pages,
                                                int32_t* counts, int32_t* hrm_counts,
                                                float* debug_w, uint8_t* debug_hrm,
                                                int64_t capacity, void* workspace,
                                                size_t workspace_bytes, void* stream) {
  return proxy_mask(p, q, k_pool, budget, 0, false, ordered_blocks, ordered_pages, counts,
                    hrm_counts, debug_w, debug_hrm, capacity, workspace, workspace_bytes, stream);
}

namespace {

// Workspace of cosa_proxy_ordered_mask_no_alloc(), for callers that cannot
// allocate device memory: a file-scope device array, one copy per GPU the
// library runs on, held until the process ends.  On the host its name is a
// stand-in, not a device address: host code only ever uses the address that
// hipGetSymbolAddress returns for the device, looked up once per device on
// its first call.
static __device__ __align__(256) unsigned char scratch[COSA_NO_ALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

// The device address of `scratch` on the device that runs `stream` (the
// current device for the null stream).
cosa_status scratch_address(hipStream_t stream, void** addr) {
  int dev = -1;
  hipError_t e = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(COSA_ERR_HIP, hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(COSA_ERR_UNSUPPORTED, "device ordinal beyond 63");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_addr[dev] == nullptr) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* ptr = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (e == hipSuccess) e = back;
    }
    if (e != hipSuccess) return fail(COSA_ERR_HIP, hipGetErrorString(e));
    if (ptr == nullptr) return fail(COSA_ERR_HIP, "hipGetSymbolAddress returned null");
    g_scratch_addr[dev] = ptr;
  }
  *addr = g_scratch_addr[dev];
  return COSA_OK;
}

}  // namespace

COSA_EXPORT cosa_status cosa_proxy_ordered_mask_no_alloc(
    const cosa_problem* p, const void* q, const void* k_pool, float budget,
    int32_t* ordered_blocks, int32_t* ordered_pages, int32_t* counts, int32_t* hrm_counts,
    float* debug_w, uint8_t* debug_hrm, int64_t capacity, void* stream) {
  cosa::KapParams k;
  cosa_status st = build_kap(k, p, q, k_pool, budget, 0, false, ordered_blocks, ordered_pages,
                             counts, hrm_counts, debug_w, debug_hrm, capacity, nullptr, 0,
                             /*check_workspace=*/false);
  if (st != COSA_OK) return st;
  if (cosa_kap_workspace_size(p) > (size_t)COSA_NO_ALLOC_SCRATCH_BYTES)
    return fail(COSA_ERR_WORKSPACE,
                "the problem needs more than COSA_NO_ALLOC_SCRATCH_BYTES of workspace "
                "(cosa_kap_workspace_size); use cosa_proxy_ordered_mask with a workspace");
  void* ws = nullptr;
  st = scratch_address((hipStream_t)stream, &ws);
  if (st != COSA_OK) return st;
  k.kbar = static_cast<uint16_t*>(ws);
  return hip_status(cosa::launch_kap(k, p->head_dim, p->q_block, (hipStream_t)stream));
}

COSA_EXPORT cosa_status cosa_proxy_ordered_mask_shared_kv(
    const cosa_problem* p, const void* q, const void* k_pool, float top_p, float budget,
    int32_t* ordered_blocks, int32_t* ordered_pages, int32_t* counts, int32_t* hrm_counts,
    float* debug_w, uint8_t* debug_hrm, int64_t capacity, void* workspace,
    size_t workspace_bytes, void* stream) {
  if (!(top_p > 0.f) || !(top_p <= 1.f)) return fail(COSA_ERR_INVALID_ARG, "top_p must lie in (0, 1]");
  const uint64_t fx = top_p >= 1.f ? 0ull : (uint64_t)floor((double)top_p * 281474976710656.0);
  return proxy_mask(p, q, k_pool, budget, top_p >= 1.f ? 0ull : (fx < 1 ? 1 : fx), true,
                    ordered_blocks, ordered_pages, counts, hrm_counts, debug_w, debug_hrm,
                    capacity, workspace, workspace_bytes, stream);
}

COSA_EXPORT cosa_status cosa_proxy_ordered_mask_top_p(
    const cosa_problem* p, const void* q, const void* k_pool, float top_p, float budget,
    int32_t* ordered_blocks, int32_t* ordered_pages, int32_t* counts, int32_t* hrm_counts,
    float* debug_w, uint8_t* debug_hrm, int64_t capacity, void* workspace,
    size_t workspace_bytes, void* stream) {
  if (!(top_p > 0.f) || !(top_p <= 1.f)) return fail(COSA_ERR_INVALID_ARG, "top_p must lie in (0, 1]");
  // p * 2^48 rounded down (exact in double); p = 1 keeps every candidate
  const uint64_t fx = top_p >= 1.f ? ~0ull : (uint64_t)floor((double)top_p * 281474976710656.0);
  return proxy_mask(p, q, k_pool, budget, fx < 1 ? 1 : fx, false, ordered_blocks, ordered_pages,
                    counts, hrm_counts, debug_w, debug_hrm, capacity, workspace, workspace_bytes,
                    stream);
}

COSA_EXPORT cosa_status cosa_osk_prefill(const cosa_problem* p, const void* q, const void* k_pool,
                                         const void* v_pool, const int32_t* ordered_blocks,
                                         const int32_t* ordered_pages, const int32_t* counts,
                                         int64_t capacity, float skip_tau, void* out, float* lse,
                                         uint8_t* skip_record, int32_t* row_stats, void* stream) {
  cosa_status st = validate(p);
  if (st != COSA_OK) return st;
  if (q == nullptr || k_pool == nullptr || v_pool == nullptr || out == nullptr ||
      ordered_blocks == nullptr || ordered_pages == nullptr || counts == nullptr)
    return fail(COSA_ERR_INVALID_ARG, "q, k_pool, v_pool, out and the mask arrays are required");
  if (capacity < 1) return fail(COSA_ERR_INVALID_ARG, "capacity must be >= 1");
  if (isnan(skip_tau)) return fail(COSA_ERR_INVALID_ARG, "skip_tau is NaN");
  cosa::AttnParams a;
  fill_attn(a, p, q, k_pool, v_pool, out, lse);
  a.ordered_blocks = ordered_blocks;
  a.ordered_pages = ordered_pages;
  a.counts = counts;
  a.skip_record = skip_record;
  a.row_stats = row_stats;
  a.capacity = capacity;
  if (skip_tau >= 0.f) {
    a.skip_mode = cosa::kSkipTau;
    a.tau_log2 = skip_tau * 1.4426950408889634f;
  }
  return hip_status(
      cosa::launch_attention(a, p->head_dim, p->q_block, cosa::kModeOrdered, (hipStream_t)stream));
}

COSA_EXPORT cosa_status cosa_sparse_prefill(
    const cosa_problem* p, const void* q, const void* k_pool, const void* v_pool, float budget,
    float skip_tau, int32_t* ordered_blocks, int32_t* ordered_pages, int32_t* counts,
    int32_t* hrm_counts, int64_t capacity, void* workspace, size_t workspace_bytes, void* out,
    float* lse, uint8_t* skip_record, int32_t* row_stats, void* stream, void* aux_stream) {
  cosa::KapParams k;
  cosa_status st = build_kap(k, p, q, k_pool, budget, 0, false, ordered_blocks, ordered_pages,
                             counts, hrm_counts, nullptr, nullptr, capacity, workspace,
                             workspace_bytes);
  if (st != COSA_OK) return st;
  if (v_pool == nullptr || out == nullptr)
    return fail(COSA_ERR_INVALID_ARG, "v_pool and out are required");
  if (isnan(skip_tau)) return fail(COSA_ERR_INVALID_ARG, "skip_tau is NaN");
  if (aux_stream != nullptr && aux_stream == stream)
    return fail(COSA_ERR_INVALID_ARG, "aux_stream must differ from stream");
  cosa::AttnParams a;
  fill_attn(a, p, q, k_pool, v_pool, out, lse);
  a.ordered_blocks = ordered_blocks;
  a.ordered_pages = ordered_pages;
  a.counts = counts;
  a.skip_record = skip_record;
  a.row_stats = row_stats;
  a.capacity = capacity;
  a.order = cosa::kOrderGroupMajor;   // group ranges need a group-major order
  if (skip_tau >= 0.f) {
    a.skip_mode = cosa::kSkipTau;
    a.tau_log2 = skip_tau * 1.4426950408889634f;
  }
  const hipStream_t s0 = (hipStream_t)stream;
  const hipStream_t s1 = (hipStream_t)aux_stream;
  hipError_t e = cosa::launch_kap(k, p->head_dim, p->q_block, s0, cosa::kKapPool);
  if (e != hipSuccess) return hip_status(e);
  // (sequence, KV head) groups in at most 8 chunks: the proxy of chunk c+1
  // runs while the kernel of chunk c does.  Each chunk's kernel spans at
  // least kChunkWorkgroups workgroups (sixteen rounds of two per CU), or the
  // launch gaps, the stream hand-offs and the tail of every launch cost more
  // than the hidden proxy time wins: shorter inputs take fewer, larger
  // chunks, down to one on the caller's stream.
  constexpr int64_t kChunkWorkgroups = 8192;
  const int n_groups = p->batch * p->num_kv_heads;
  const int64_t wg_per_group = (int64_t)(p->num_q_heads / p->num_kv_heads) * a.nqb;
  int chunk = (n_groups + 7) / 8;
  const int64_t need = (kChunkWorkgroups + wg_per_group - 1) / wg_per_group;
  if (need > chunk) chunk = need < n_groups ? (int)need : n_groups;
  const bool overlap = s1 != nullptr && chunk < n_groups;
  hipEvent_t ev[9] = {};
  int n_ev = 0;
  auto cleanup = [&]() {
    for (int x = 0; x < n_ev; ++x) (void)hipEventDestroy(ev[x]);
  };
  bool used_aux = false;
  for (int g0 = 0; g0 < n_groups; g0 += chunk) {
    const int cnt = n_groups - g0 < chunk ? n_groups - g0 : chunk;
    k.group_begin = a.group_begin = g0;
    k.group_count = a.group_count = cnt;
    // the heads of a tile on one XCD when the chunk's tiles split evenly
    a.order = (int64_t)cnt * a.nqb % 8 == 0 ? cosa::kOrderGroupXcd : cosa::kOrderGroupMajor;
    e = cosa::launch_kap(k, p->head_dim, p->q_block, s0, cosa::kKapSelect);
    if (e != hipSuccess) break;
    hipStream_t s_attn = s0;
    if (overlap) {
      e = hipEventCreateWithFlags(&ev[n_ev], hipEventDisableTiming);
      if (e != hipSuccess) break;
      ++n_ev;
      e = hipEventRecord(ev[n_ev - 1], s0);
      if (e == hipSuccess) e = hipStreamWaitEvent(s1, ev[n_ev - 1], 0);
      if (e != hipSuccess) break;
      s_attn = s1;
      used_aux = true;
    }
    e = cosa::launch_attention(a, p->head_dim, p->q_block, cosa::kModeOrdered, s_attn);
    if (e != hipSuccess) break;
  }
  if (used_aux) {
    // the caller's stream continues after the last kernel on aux_stream (also
    // after an error, so that nothing of this call is left unordered)
    hipError_t ej = hipEventCreateWithFlags(&ev[n_ev], hipEventDisableTiming);
    if (ej == hipSuccess) {
      ++n_ev;
      ej = hipEventRecord(ev[n_ev - 1], s1);
      if (ej == hipSuccess) ej = hipStreamWaitEvent(s0, ev[n_ev - 1], 0);
    }
    if (e == hipSuccess) e = ej;
  }
  cleanup();
  return hip_status(e);
}

COSA_EXPORT cosa_status cosa_osk_prefill_shared_kv(
    const cosa_problem* p, const void* q, const void* k_pool, const void* v_pool,
    const int32_t* ordered_blocks, const int32_t* ordered_pages, const int32_t* counts,
    int64_t capacity, float skip_tau, void* out, float* lse, uint8_t* skip_record,
    int32_t* row_stats, void* stream) {
  cosa_status st = validate(p);
  if (st != COSA_OK) return st;
  if (q == nullptr || k_pool == nullptr || v_pool == nullptr || out == nullptr ||
      ordered_blocks == nullptr || ordered_pages == nullptr || counts == nullptr)
    return fail(COSA_ERR_INVALID_ARG, "q, k_pool, v_pool, out and the mask arrays are required");
  if (capacity < 1) return fail(COSA_ERR_INVALID_ARG, "capacity must be >= 1");
  if (isnan(skip_tau)) return fail(COSA_ERR_INVALID_ARG, "skip_tau is NaN");
  cosa::AttnParams a;
  fill_attn(a, p, q, k_pool, v_pool, out, lse);
  a.ordered_blocks = ordered_blocks;
  a.ordered_pages = ordered_pages;
  a.counts = counts;
  a.skip_record = skip_record;
  a.row_stats = row_stats;
  a.capacity = capacity;
  a.mask_heads = p->num_kv_heads;
  // the heads that share a mask visit the same pages: run them side by side
  // on one XCD so that those pages are fetched into its L2 once
  if (a.xcd_units != 0) a.order = cosa::kOrderGroupXcd;
  if (skip_tau >= 0.f) {
    a.skip_mode = cosa::kSkipTau;
    a.tau_log2 = skip_tau * 1.4426950408889634f;
  }
  return hip_status(
      cosa::launch_attention(a, p->head_dim, p->q_block, cosa::kModeOrdered, (hipStream_t)stream));
}

COSA_EXPORT cosa_status cosa_osk_prefill_delta(const cosa_problem* p, const void* q,
                                               const void* k_pool, const void* v_pool,
                                               const int32_t* ordered_blocks,
                                               const int32_t* ordered_pages, const int32_t* counts,
                                               int64_t capacity, float skip_delta, void* out,
                                               float* lse, uint8_t* skip_record,
                                               int32_t* row_stats, void* stream) {
  cosa_status st = validate(p);
  if (st != COSA_OK) return st;
  if (q == nullptr || k_pool == nullptr || v_pool == nullptr || out == nullptr ||
      ordered_blocks == nullptr || ordered_pages == nullptr || counts == nullptr)
    return fail(COSA_ERR_INVALID_ARG, "q, k_pool, v_pool, out and the mask arrays are required");
  if (capacity < 1) return fail(COSA_ERR_INVALID_ARG, "capacity must be >= 1");
  if (isnan(skip_delta) || isinf(skip_delta))
    return fail(COSA_ERR_INVALID_ARG, "skip_delta must be finite");
  cosa::AttnParams a;
  fill_attn(a, p, q, k_pool, v_pool, out, lse);
  a.ordered_blocks = ordered_blocks;
  a.ordered_pages = ordered_pages;
  a.counts = counts;
  a.skip_record = skip_record;
  a.row_stats = row_stats;
  a.capacity = capacity;
  if (skip_delta > 0.f) {
    a.skip_mode = cosa::kSkipDelta;
    a.log2_delta = (float)log2((double)skip_delta);
  }
  return hip_status(
      cosa::launch_attention(a, p->head_dim, p->q_block, cosa::kModeOrdered, (hipStream_t)stream));
}

COSA_EXPORT cosa_status cosa_dense_prefill(const cosa_problem* p, const void* q,
                                           const void* k_pool, const void* v_pool, void* out,
                                           float* lse, void* stream) {
  cosa_status st = validate(p);
  if (st != COSA_OK) return st;
  if (q == nullptr || k_pool == nullptr || v_pool == nullptr || out == nullptr)
    return fail(COSA_ERR_INVALID_ARG, "q, k_pool, v_pool and out are required");
  cosa::AttnParams a;
  fill_attn(a, p, q, k_pool, v_pool, out, lse);
  return hip_status(
      cosa::launch_attention(a, p->head_dim, p->q_block, cosa::kModeDense, (hipStream_t)stream));
}

COSA_EXPORT cosa_status cosa_block_mask_prefill(const cosa_problem* p, const void* q,
                                                const void* k_pool, const void* v_pool,
                                                const uint32_t* block_mask, int64_t mask_words,
                                                void* out, float* lse, void* stream) {
  cosa_status st = validate(p);
  if (st != COSA_OK) return st;
  if (q == nullptr || k_pool == nullptr || v_pool == nullptr || out == nullptr ||
      block_mask == nullptr)
    return fail(COSA_ERR_INVALID_ARG, "q, k_pool, v_pool, block_mask and out are required");
  if (p->kv_block != p->page_size)
    return fail(COSA_ERR_UNSUPPORTED, "logical mask skipping needs kv_block == page_size");
  if (mask_words < ceil_div(ceil_div(p->max_seqlen, p->kv_block), 32))
    return fail(COSA_ERR_INVALID_ARG, "mask_words < ceil(ceil(max_seqlen / kv_block) / 32)");
  cosa::AttnParams a;
  fill_attn(a, p, q, k_pool, v_pool, out, lse);
  a.block_mask = block_mask;
  a.mask_words = mask_words;
  return hip_status(
      cosa::launch_attention(a, p->head_dim, p->q_block, cosa::kModeLogical, (hipStream_t)stream));
}
