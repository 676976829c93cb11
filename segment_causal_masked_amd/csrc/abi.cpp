// C ABI of the library: argument checks, plan upload, cache bookkeeping and
// kernel launches.  Every entry point returns a status and records a
// thread-local error text; nothing throws across the boundary.
#include <hip/hip_runtime.h>

#include <cmath>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"
#include "nomas_attn.h"
#include "plan.h"
#include "status.h"

namespace {

thread_local std::string t_err;

nomas_status fail(nomas_status s, const std::string& what) {
  t_err = what;
  return s;
}

nomas_status ok() {
  t_err.clear();
  return NOMAS_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Environment switches, read once per process:
//   NOMAS_TRACE=1         one line of plan statistics on stderr per plan;
//   NOMAS_DEBUG_CHECKS=1  every plan's tables are checked against their
//                         invariants, and every call waits for its kernels and
//                         reports a failed one as NOMAS_ERR_HIP (slow: for
//                         debugging only; not usable under graph capture).
bool env_flag(const char* name) {
  const char* v = std::getenv(name);
  return v && *v && std::strcmp(v, "0") != 0;
}
bool trace_on() {
  static const bool on = env_flag("NOMAS_TRACE");
  return on;
}
bool debug_checks() {
  static const bool on = env_flag("NOMAS_DEBUG_CHECKS");
  return on;
}

}  // namespace

namespace nomas {
nomas_status set_error(nomas_status s, const std::string& what) { return fail(s, what); }
nomas_status clear_error() { return ok(); }
}  // namespace nomas

struct nomas_kvcache {
  int32_t heads = 0, head_dim = 0;
  int64_t capacity = 0, len = 0;
  void* k = nullptr;
  void* v = nullptr;
  std::vector<nomas_segment> segs;  // committed segments, in append order
};

struct nomas_kvcache_int8 {
  int32_t heads = 0;
  int64_t capacity = 0, len = 0;
  void *k_codes = nullptr, *v_codes = nullptr, *k_exp = nullptr, *v_exp = nullptr;
  std::vector<nomas_segment> segs;  // committed segments, in append order
};

struct nomas_plan {
  nomas::HostPlan host;
  bool has_cache = false;
  std::vector<nomas_segment> cache_segs;  // the cache contents the plan was built for
  bool on_device = false;
  int device = -1;
  void* dmem = nullptr;
  const nomas::QDescDev* d_qdesc = nullptr;
  const nomas::KDescDev* d_kdesc = nullptr;
  const int32_t *d_csr_ptr = nullptr, *d_csr_idx = nullptr;
  const int32_t *d_csc_ptr = nullptr, *d_csc_idx = nullptr;
  const int32_t* d_wg_ptr = nullptr;
  const int4 *d_pieces = nullptr, *d_combine = nullptr;
  const int32_t *d_pair_ptr = nullptr, *d_pair_idx = nullptr;
  const int32_t *d_kpair_ptr = nullptr, *d_kpair_idx = nullptr;
  const int32_t* d_unit_shift = nullptr;
  const int32_t *d_sp_ptr = nullptr, *d_sp_keep = nullptr, *d_video_tile = nullptr;
};

namespace {

nomas_status check_layout_ptr(const nomas_layout* l, const char* name) {
  if (!l) return fail(NOMAS_ERR_INVALID_ARGUMENT, std::string(name) + " layout is NULL");
  if (l->n_segments < 0) return fail(NOMAS_ERR_INVALID_ARGUMENT, std::string(name) + ": n_segments < 0");
  if (l->n_segments > 0 && !l->segments)
    return fail(NOMAS_ERR_INVALID_ARGUMENT, std::string(name) + ": segments is NULL");
  return NOMAS_OK;
}

std::vector<nomas_segment> to_vec(const nomas_layout* l) {
  return std::vector<nomas_segment>(l->segments, l->segments + l->n_segments);
}

nomas_status hip_fail(hipError_t e, const char* where) {
  return fail(NOMAS_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

// Under NOMAS_DEBUG_CHECKS: wait for the work just enqueued and report a
// kernel that failed, naming the call.
nomas_status debug_sync(void* stream, const char* where) {
  if (!debug_checks()) return NOMAS_OK;
  hipError_t e = hipStreamSynchronize(static_cast<hipStream_t>(stream));
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess) return fail(NOMAS_ERR_HIP, std::string(where) + " (NOMAS_DEBUG_CHECKS): " +
                                                      hipGetErrorString(e));
  return NOMAS_OK;
}

// A plan encodes the layout only: it is valid for any cache of its head count
// that holds exactly the segments it was built for (same identities and
// records, same order), whichever cache object that is.
size_t fwd_workspace_bytes(const nomas::HostPlan& h);  // defined with the forward

bool plan_matches_cache(const nomas_plan* p, const nomas_kvcache* c) {
  if (!p->has_cache) return c == nullptr;
  if (!c || c->heads != p->host.heads || c->segs.size() != p->cache_segs.size()) return false;
  for (size_t i = 0; i < c->segs.size(); ++i)
    if (!nomas::same_segment(c->segs[i], p->cache_segs[i])) return false;
  return true;
}

nomas_status check_stride(int64_t stride, int32_t heads, const char* name) {
  if (stride < (int64_t)heads * NOMAS_HEAD_DIM)
    return fail(NOMAS_ERR_INVALID_ARGUMENT, std::string(name) + " stride < heads * 128");
  if (stride % 8 != 0) return fail(NOMAS_ERR_ALIGNMENT, std::string(name) + " stride not a multiple of 8");
  // the kernels form a block's per-lane offsets (up to 63 rows) in 32 bits
  if (stride > (int64_t(1) << 24))
    return fail(NOMAS_ERR_INVALID_ARGUMENT, std::string(name) + " stride above 2^24 elements");
  return NOMAS_OK;
}

// Row and head strides of the new-token K / V (and dK / dV) rows from the
// caller's kv_stride: token-major [n][H][128] (kv_stride = the token stride)
// or, for plans built with NOMAS_PLAN_KV_HEAD_MAJOR, head-major [H][n][128]
// (kv_stride = the head stride, at least n rows).
nomas_status kv_strides(const nomas::HostPlan& h, int64_t kv_stride, int64_t n_rows, int64_t* row,
                        int64_t* head) {
  if (!h.kv_head_major) {
    nomas_status s = check_stride(kv_stride, h.heads, "kv");
    *row = kv_stride;
    *head = NOMAS_HEAD_DIM;
    return s;
  }
  if (kv_stride < n_rows * NOMAS_HEAD_DIM)
    return fail(NOMAS_ERR_INVALID_ARGUMENT, "kv head stride < rows * 128 (head-major keys)");
  if (kv_stride % 8 != 0) return fail(NOMAS_ERR_ALIGNMENT, "kv head stride not a multiple of 8");
  *row = NOMAS_HEAD_DIM;
  *head = kv_stride;
  return NOMAS_OK;
}

nomas_status check_dev_ptr(const void* p, bool needed, const char* name) {
  if (!needed) return NOMAS_OK;
  if (!p) return fail(NOMAS_ERR_INVALID_ARGUMENT, std::string(name) + " is NULL");
  if (!aligned16(p)) return fail(NOMAS_ERR_ALIGNMENT, std::string(name) + " not 16-byte aligned");
  return NOMAS_OK;
}

nomas_status check_device(const nomas_plan* p) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != p->device) return fail(NOMAS_ERR_INVALID_ARGUMENT, "plan was built on another device");
  return NOMAS_OK;
}

}  // namespace

extern "C" {

nomas_status nomas_action_latent_window(int64_t first, int64_t end, int64_t n_pixel_frames,
                                        int32_t* lo, int32_t* hi) {
  if (!lo || !hi) return fail(NOMAS_ERR_INVALID_ARGUMENT, "NULL output");
  if (first < 0 || end <= first || end > n_pixel_frames)
    return fail(NOMAS_ERR_INVALID_ARGUMENT, "need 0 <= first < end <= n_pixel_frames");
  if (n_pixel_frames > (int64_t(1) << 33)) return fail(NOMAS_ERR_INVALID_ARGUMENT, "n_pixel_frames too large");
  const int64_t n_latent = (n_pixel_frames - 1) / 4 + 1;  // Eq. 1
  // pixel frame t sits in latent frame ceil(t / 4): 0 -> 0, 4i - 3 .. 4i -> i
  const int64_t a = std::min((first + 3) / 4, n_latent);
  const int64_t b = std::min((end - 1 + 3) / 4 + 1, n_latent);
  *lo = int32_t(a);
  *hi = int32_t(std::max(a, b));
  return ok();
}

const char* nomas_status_string(nomas_status s) {
  switch (s) {
    case NOMAS_OK: return "ok";
    case NOMAS_ERR_INVALID_ARGUMENT: return "invalid argument";
    case NOMAS_ERR_LAYOUT: return "malformed layout";
    case NOMAS_ERR_UNSUPPORTED: return "unsupported";
    case NOMAS_ERR_CAPACITY: return "cache capacity exceeded";
    case NOMAS_ERR_STALE_PLAN: return "stale plan (cache changed)";
    case NOMAS_ERR_ALIGNMENT: return "misaligned pointer or stride";
    case NOMAS_ERR_HIP: return "HIP error";
    default: return "unknown status";
  }
}

const char* nomas_last_error(void) { return t_err.c_str(); }

// ---------------------------------------------------------------------------
// plans
// ---------------------------------------------------------------------------

nomas_status nomas_attn_plan(const nomas_layout* q, const nomas_layout* kv_new,
                             const nomas_kvcache* cache, const nomas_plan_opts* opts,
                             nomas_plan** out) {
  if (!out) return fail(NOMAS_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  if (!opts) return fail(NOMAS_ERR_INVALID_ARGUMENT, "opts is NULL");
  nomas_status s;
  if ((s = check_layout_ptr(q, "query")) != NOMAS_OK) return s;
  if ((s = check_layout_ptr(kv_new, "kv_new")) != NOMAS_OK) return s;
  if (cache && cache->heads != opts->num_heads)
    return fail(NOMAS_ERR_INVALID_ARGUMENT, "cache heads differ from opts.num_heads");

  const auto t_start = std::chrono::steady_clock::now();
  nomas_plan* p = new (std::nothrow) nomas_plan();
  if (!p) return fail(NOMAS_ERR_INVALID_ARGUMENT, "out of host memory");
  std::string err;
  std::vector<nomas_segment> cached;
  if (cache) cached = cache->segs;
  try {
    s = nomas::build_host_plan(to_vec(q), cached, to_vec(kv_new), *opts, &p->host, &err);
  } catch (const std::bad_alloc&) {
    s = NOMAS_ERR_INVALID_ARGUMENT;
    err = "out of host memory while building the plan";
  }
  if (s != NOMAS_OK) {
    delete p;
    return fail(s, err);
  }
  if (cache) {
    p->has_cache = true;
    p->cache_segs = cache->segs;
  }
  int groups = 256 * nomas::attn_fwd_groups_per_cu();  // host-only plans: MI355X's 256 CUs
  if (!(opts->flags & NOMAS_PLAN_HOST_ONLY)) {
    hipError_t e = hipGetDevice(&p->device);
    int cus = 0;
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, p->device);
    if (e != hipSuccess) {
      delete p;
      return hip_fail(e, "device query");
    }
    groups = cus * nomas::attn_fwd_groups_per_cu();
    // set-up of the allocation-free forward on this device: its scratch
    // address, resolved once per device while the device is current
    void* scratch = nullptr;
    e = nomas::noalloc_scratch(p->device, &scratch);
    if (e != hipSuccess) {
      delete p;
      return hip_fail(e, "device scratch address");
    }
  }
  nomas::build_fwd_schedule(&p->host, groups);
  if (!p->has_cache) nomas::build_bwd_schedule(&p->host);
  if (debug_checks()) {
    const std::string bad = nomas::validate_host_plan(p->host);
    if (!bad.empty()) {
      delete p;
      return fail(NOMAS_ERR_INVALID_ARGUMENT, "internal " + bad);
    }
  }
  if (!(opts->flags & NOMAS_PLAN_HOST_ONLY)) {
    const nomas::HostPlan& h = p->host;
    struct Part { const void* src; size_t bytes; size_t off; };
    Part parts[] = {{h.qdesc.data(), h.qdesc.size() * sizeof(nomas::QDesc), 0},
                    {h.kdesc.data(), h.kdesc.size() * sizeof(nomas::KDesc), 0},
                    {h.csr_ptr.data(), h.csr_ptr.size() * 4, 0},
                    {h.csr_idx.data(), h.csr_idx.size() * 4, 0},
                    {h.csc_ptr.data(), h.csc_ptr.size() * 4, 0},
                    {h.csc_idx.data(), h.csc_idx.size() * 4, 0},
                    {h.wg_ptr.data(), h.wg_ptr.size() * 4, 0},
                    {h.pieces.data(), h.pieces.size() * sizeof(nomas::Piece), 0},
                    {h.combine.data(), h.combine.size() * sizeof(nomas::CombineItem), 0},
                    {h.pair_ptr.data(), h.pair_ptr.size() * 4, 0},
                    {h.pair_idx.data(), h.pair_idx.size() * 4, 0},
                    {h.kpair_ptr.data(), h.kpair_ptr.size() * 4, 0},
                    {h.kpair_idx.data(), h.kpair_idx.size() * 4, 0},
                    {h.unit_shift.data(), h.unit_shift.size() * 4, 0},
                    {h.sp_ptr.data(), h.sp_ptr.size() * 4, 0},
                    {h.sp_keep.data(), h.sp_keep.size() * 4, 0},
                    {h.video_tile.data(), h.video_tile.size() * 4, 0}};
    size_t total = 0;
    for (Part& part : parts) {
      part.off = total;
      total += (part.bytes + 16 + 255) & ~size_t(255);  // >= 16 B slack, 256-B aligned
    }
    hipError_t e = hipMalloc(&p->dmem, total);
    if (e != hipSuccess) {
      delete p;
      return hip_fail(e, "plan upload");
    }
    std::vector<char> staging(total, 0);
    for (const Part& part : parts)
      if (part.bytes) std::memcpy(staging.data() + part.off, part.src, part.bytes);
    e = hipMemcpy(p->dmem, staging.data(), total, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      (void)hipFree(p->dmem);
      delete p;
      return hip_fail(e, "plan upload");
    }
    char* base = static_cast<char*>(p->dmem);
    p->d_qdesc = reinterpret_cast<const nomas::QDescDev*>(base + parts[0].off);
    p->d_kdesc = reinterpret_cast<const nomas::KDescDev*>(base + parts[1].off);
    p->d_csr_ptr = reinterpret_cast<const int32_t*>(base + parts[2].off);
    p->d_csr_idx = reinterpret_cast<const int32_t*>(base + parts[3].off);
    p->d_csc_ptr = reinterpret_cast<const int32_t*>(base + parts[4].off);
    p->d_csc_idx = reinterpret_cast<const int32_t*>(base + parts[5].off);
    p->d_wg_ptr = reinterpret_cast<const int32_t*>(base + parts[6].off);
    p->d_pieces = reinterpret_cast<const int4*>(base + parts[7].off);
    p->d_combine = reinterpret_cast<const int4*>(base + parts[8].off);
    p->d_pair_ptr = reinterpret_cast<const int32_t*>(base + parts[9].off);
    p->d_pair_idx = reinterpret_cast<const int32_t*>(base + parts[10].off);
    p->d_kpair_ptr = reinterpret_cast<const int32_t*>(base + parts[11].off);
    p->d_kpair_idx = reinterpret_cast<const int32_t*>(base + parts[12].off);
    p->d_unit_shift = reinterpret_cast<const int32_t*>(base + parts[13].off);
    p->d_sp_ptr = reinterpret_cast<const int32_t*>(base + parts[14].off);
    p->d_sp_keep = reinterpret_cast<const int32_t*>(base + parts[15].off);
    p->d_video_tile = reinterpret_cast<const int32_t*>(base + parts[16].off);
    p->on_device = true;
  }
  if (trace_on()) {
    const nomas::HostPlan& h = p->host;
    const double ms =
        std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - t_start).count();
    std::fprintf(stderr,
                 "nomas_attn_plan: queries %lld keys %lld (cached %lld) heads %d mode %d window %d "
                 "keep %d%% | tiles %lldx%lld: full %lld partial %lld empty %lld | A %lld "
                 "executed/A %.4f | units %lld pieces %zu merges %zu slots %d | fwd workspace %zu B "
                 "| %s | %.2f ms\n",
                 (long long)h.nq, (long long)h.nk, (long long)h.n_cached, h.heads, h.mode, h.window,
                 h.keep_percent, (long long)h.nqt, (long long)h.nkt, (long long)h.n_full,
                 (long long)h.n_partial, (long long)h.n_empty, (long long)h.unmasked_pairs,
                 h.unmasked_pairs ? (double)h.executed_pairs / (double)h.unmasked_pairs : 0.0,
                 (long long)(int64_t(h.heads) * h.n_pairs), h.pieces.size(), h.combine.size(), h.n_slots,
                 fwd_workspace_bytes(h), p->on_device ? "device" : "host only", ms);
  }
  *out = p;
  return ok();
}

nomas_status nomas_plan_get_info(const nomas_plan* p, nomas_plan_info* info) {
  if (!p || !info) return fail(NOMAS_ERR_INVALID_ARGUMENT, "NULL argument");
  const nomas::HostPlan& h = p->host;
  info->n_queries = h.nq;
  info->n_keys = h.nk;
  info->n_cached_keys = h.n_cached;
  info->n_q_tiles = h.nqt;
  info->n_k_tiles = h.nkt;
  info->n_empty_tiles = h.n_empty;
  info->n_full_tiles = h.n_full;
  info->n_partial_tiles = h.n_partial;
  info->unmasked_pairs = h.unmasked_pairs;
  info->executed_pairs = h.executed_pairs;
  info->effective_flop = 4.0 * h.head_dim * h.heads * (double)h.unmasked_pairs;
  info->block_q = h.bq;
  info->block_k = h.bk;
  info->num_heads = h.heads;
  info->text_query_mode = h.mode;
  info->sparse_list_entries = h.sp_total;
  info->video_keep_percent = h.keep_percent;
  info->window_segments = h.window;
  return ok();
}

nomas_status nomas_plan_export_classes(const nomas_plan* p, uint8_t* buf, size_t n) {
  if (!p || !buf) return fail(NOMAS_ERR_INVALID_ARGUMENT, "NULL argument");
  if (n < p->host.classes.size()) return fail(NOMAS_ERR_INVALID_ARGUMENT, "buffer too small");
  std::memcpy(buf, p->host.classes.data(), p->host.classes.size());
  return ok();
}

nomas_status nomas_plan_destroy(nomas_plan* p) {
  if (!p) return ok();
  if (p->dmem) (void)hipFree(p->dmem);
  delete p;
  return ok();
}

// ---------------------------------------------------------------------------
// forward
// ---------------------------------------------------------------------------

}  // extern "C"

namespace {

// Forward workspace: [sparse plans: kept lists [H][sp_total] int32 | key sums
// [H][nkt][128] fp32 | query sums [H][n_pairs][128] fp32 | (lists longer than
// 4096 entries) sort keys [H][pair_total] uint64] [partial slots], each part
// 256-byte aligned.
struct FwdWorkspace {
  size_t lists = 0, k_sum = 0, q_sum = 0, keys = 0, partial = 0, claim = 0, total = 0;
  bool has_keys = false;
};

FwdWorkspace fwd_workspace(const nomas::HostPlan& h) {
  auto al = [](size_t b) { return (b + 255) & ~size_t(255); };
  FwdWorkspace w;
  size_t at = 0;
  if (h.keep_percent > 0) {
    w.lists = at;
    at += al(size_t(h.heads) * size_t(h.sp_total) * 4);
    w.k_sum = at;
    at += al(size_t(h.heads) * size_t(h.nkt) * 128 * 4);
    w.q_sum = at;
    at += al(size_t(h.heads) * size_t(h.n_pairs) * 128 * 4);
    // sort keys of the pair lists ranked by radix select (longer than a
    // workgroup's LDS sort holds)
    for (int64_t u = 0; u < h.n_pairs && !w.has_keys; ++u)
      w.has_keys = h.pair_ptr[size_t(u + 1)] - h.pair_ptr[size_t(u)] > nomas::SELECT_SORT_ENTRIES;
    if (w.has_keys) {
      w.keys = at;
      at += al(size_t(h.heads) * size_t(h.pair_ptr.back()) * 8);
    }
  }
  w.partial = at;
  at += (size_t)h.n_slots * nomas::attn_fwd_slot_bytes();
  if (h.n_chunks > 0) {  // the tail chunks' claim counter
    w.claim = at;
    at += 256;
  }
  w.total = at;
  return w;
}

size_t fwd_workspace_bytes(const nomas::HostPlan& h) { return fwd_workspace(h).total; }

}  // namespace

extern "C" {

nomas_status nomas_attn_fwd_workspace_size(const nomas_plan* p, size_t* bytes) {
  if (!p || !bytes) return fail(NOMAS_ERR_INVALID_ARGUMENT, "NULL argument");
  *bytes = fwd_workspace(p->host).total;
  return ok();
}

}  // extern "C"

namespace {

nomas_status check_fwd_plan(const nomas_plan* p, const nomas_kvcache* cache) {
  if (!p) return fail(NOMAS_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!p->on_device) return fail(NOMAS_ERR_INVALID_ARGUMENT, "host-only plan cannot run");
  if (!plan_matches_cache(p, cache))
    return fail(p->has_cache && cache ? NOMAS_ERR_STALE_PLAN : NOMAS_ERR_INVALID_ARGUMENT,
                p->has_cache && cache ? "cache changed since the plan was built"
                                      : "cache argument does not match the plan");
  return NOMAS_OK;
}

// The forward of a checked plan over `workspace` (device memory of at least
// the plan's workspace size): argument checks and launches, no allocation.
nomas_status fwd_impl(const nomas_plan* p, const nomas_kvcache* cache, const void* q,
                      int64_t q_stride, const void* k_new, const void* v_new, int64_t kv_stride,
                      void* o, int64_t o_stride, float* lse, float scale, void* workspace,
                      size_t workspace_bytes, void* hip_stream) {
  const nomas::HostPlan& h = p->host;
  const bool has_new = h.nk > h.n_cached;
  nomas_status s;
  if ((s = check_dev_ptr(q, h.nq > 0, "q")) || (s = check_dev_ptr(o, h.nq > 0, "o")) ||
      (s = check_dev_ptr(k_new, has_new, "k_new")) || (s = check_dev_ptr(v_new, has_new, "v_new")))
    return s;
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u)) return fail(NOMAS_ERR_ALIGNMENT, "lse misaligned");
  if ((s = check_stride(q_stride, h.heads, "q")) || (s = check_stride(o_stride, h.heads, "o")))
    return s;
  int64_t kv_row = NOMAS_HEAD_DIM, kv_head = NOMAS_HEAD_DIM;
  if (has_new && (s = kv_strides(h, kv_stride, h.nk - h.n_cached, &kv_row, &kv_head))) return s;
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(NOMAS_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
  const FwdWorkspace ws = fwd_workspace(h);
  size_t need = ws.total;
  if (need && (!workspace || workspace_bytes < need))
    return fail(NOMAS_ERR_INVALID_ARGUMENT, "workspace missing or smaller than nomas_attn_fwd_workspace_size");
  if ((s = check_dev_ptr(workspace, need > 0, "workspace"))) return s;
  if ((s = check_device(p))) return s;
  char* wsb = static_cast<char*>(workspace);
  if (h.keep_percent > 0 && h.nq > 0) {
    nomas::SelParams sp{};
    sp.q = static_cast<const uint16_t*>(q);
    sp.k_cache = cache ? static_cast<const uint16_t*>(cache->k) : nullptr;
    sp.k_new = static_cast<const uint16_t*>(k_new);
    sp.pair_ptr = p->d_pair_ptr;
    sp.pair_idx = p->d_pair_idx;
    sp.sp_ptr = p->d_sp_ptr;
    sp.sp_keep = p->d_sp_keep;
    sp.video_tile = p->d_video_tile;
    sp.k_sum = reinterpret_cast<float*>(wsb + ws.k_sum);
    sp.q_sum = reinterpret_cast<float*>(wsb + ws.q_sum);
    sp.lists = reinterpret_cast<int32_t*>(wsb + ws.lists);
    sp.keys = ws.has_keys ? reinterpret_cast<uint64_t*>(wsb + ws.keys) : nullptr;
    sp.pair_total = h.pair_ptr.back();
    sp.q_stride = q_stride;
    sp.kv_stride = kv_row;
    sp.kv_head_stride = kv_head;
    sp.cache_cap = cache ? cache->capacity : 0;
    sp.sp_total = h.sp_total;
    sp.nq = (int32_t)h.nq;
    sp.nk = (int32_t)h.nk;
    sp.n_cached = (int32_t)h.n_cached;
    sp.heads = h.heads;
    sp.nkt = (int32_t)h.nkt;
    sp.n_pairs = (int32_t)h.n_pairs;
    hipError_t e = nomas::launch_select(sp, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return hip_fail(e, "video-block selection launch");
  }

  nomas::FwdParams fp{};
  fp.q = static_cast<const uint16_t*>(q);
  fp.k_cache = cache ? static_cast<const uint16_t*>(cache->k) : nullptr;
  fp.v_cache = cache ? static_cast<const uint16_t*>(cache->v) : nullptr;
  fp.k_new = static_cast<const uint16_t*>(k_new);
  fp.v_new = static_cast<const uint16_t*>(v_new);
  fp.o = static_cast<uint16_t*>(o);
  fp.lse = lse;
  fp.qdesc = p->d_qdesc;
  fp.kdesc = p->d_kdesc;
  if (h.keep_percent > 0) {  // per-head lists chosen by the selection above
    fp.csr_ptr = p->d_sp_ptr;
    fp.csr_idx = reinterpret_cast<const int32_t*>(wsb + ws.lists);
    fp.list_head_stride = h.sp_total;
  } else {
    fp.csr_ptr = p->d_pair_ptr;
    fp.csr_idx = p->d_pair_idx;
    fp.list_head_stride = 0;
  }
  fp.n_pairs = (int32_t)h.n_pairs;
  fp.wg_ptr = p->d_wg_ptr;
  fp.pieces = p->d_pieces;
  fp.combine = p->d_combine;
  fp.chunks = p->d_pieces + h.wg_ptr.back();
  fp.n_chunks = h.n_chunks;
  fp.claim = h.n_chunks > 0 ? reinterpret_cast<uint32_t*>(wsb + ws.claim) : nullptr;
  fp.unit_shift = p->d_unit_shift;
  fp.partial = reinterpret_cast<float*>(wsb + ws.partial);
  fp.groups = h.fwd_groups;
  fp.n_combine = (int32_t)h.combine.size();
  fp.q_stride = q_stride;
  fp.kv_stride = kv_row;
  fp.kv_head_stride = kv_head;
  fp.o_stride = o_stride;
  fp.cache_cap = cache ? cache->capacity : 0;
  fp.nq = (int32_t)h.nq;
  fp.nk = (int32_t)h.nk;
  fp.n_cached = (int32_t)h.n_cached;
  fp.heads = h.heads;
  fp.nqt = (int32_t)h.nqt;
  fp.nkt = (int32_t)h.nkt;
  fp.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e = nomas::launch_attn_fwd(fp, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "attn_fwd launch");
  return ok();
}

}  // namespace

extern "C" {

nomas_status nomas_attn_fwd(const nomas_plan* p, const nomas_kvcache* cache, const void* q,
                            int64_t q_stride, const void* k_new, const void* v_new,
                            int64_t kv_stride, void* o, int64_t o_stride, float* lse,
                            float scale, void* workspace, size_t workspace_bytes,
                            void* hip_stream) {
  nomas_status s = check_fwd_plan(p, cache);
  if (s != NOMAS_OK) return s;
  return fwd_impl(p, cache, q, q_stride, k_new, v_new, kv_stride, o, o_stride, lse, scale,
                  workspace, workspace_bytes, hip_stream);
}

nomas_status nomas_attn_fwd_noalloc(const nomas_plan* p, const nomas_kvcache* cache,
                                    const void* q, int64_t q_stride, const void* k_new,
                                    const void* v_new, int64_t kv_stride, void* o,
                                    int64_t o_stride, float* lse, float scale, void* hip_stream) {
  nomas_status s = check_fwd_plan(p, cache);
  if (s != NOMAS_OK) return s;
  const size_t need = fwd_workspace(p->host).total;
  if (need > nomas::NOALLOC_SCRATCH_BYTES)
    return fail(NOMAS_ERR_UNSUPPORTED,
                "plan needs " + std::to_string(need) + " bytes of forward workspace; "
                "nomas_attn_fwd_noalloc holds at most " +
                    std::to_string(nomas::NOALLOC_SCRATCH_BYTES) + " (use nomas_attn_fwd)");
  if ((s = check_device(p))) return s;
  void* scratch = nullptr;
  hipError_t e = nomas::noalloc_scratch(p->device, &scratch);
  if (e != hipSuccess) return hip_fail(e, "device scratch address");
  return fwd_impl(p, cache, q, q_stride, k_new, v_new, kv_stride, o, o_stride, lse, scale,
                  need ? scratch : nullptr, need ? nomas::NOALLOC_SCRATCH_BYTES : 0, hip_stream);
}

// ---------------------------------------------------------------------------
// backward
// ---------------------------------------------------------------------------

nomas_status nomas_attn_bwd_workspace_size(const nomas_plan* p, size_t* bytes) {
  if (!p || !bytes) return fail(NOMAS_ERR_INVALID_ARGUMENT, "NULL argument");
  // -delta and -lse * log2(e) per (head, query row of the padded q-tiles),
  // then the two kernels' work-queue counters
  *bytes = 2 * (size_t)p->host.heads * (size_t)p->host.nqt * 128 * sizeof(float) + 256;
  return ok();
}

nomas_status nomas_attn_bwd(const nomas_plan* p, const void* q, const void* k, const void* v,
                            const void* o, const void* d_o, const float* lse, int64_t q_stride,
                            int64_t kv_stride, void* dq, void* dk, void* dv, float scale,
                            void* workspace, size_t workspace_bytes, void* hip_stream) {
  if (!p) return fail(NOMAS_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!p->on_device) return fail(NOMAS_ERR_INVALID_ARGUMENT, "host-only plan cannot run");
  if (p->has_cache) return fail(NOMAS_ERR_INVALID_ARGUMENT, "backward needs a plan without a cache");
  if (p->host.keep_percent > 0) return fail(NOMAS_ERR_UNSUPPORTED, "backward of a video-block sparse plan");
  const nomas::HostPlan& h = p->host;
  const bool hq = h.nq > 0, hk = h.nk > 0;
  nomas_status s;
  if ((s = check_dev_ptr(q, hq, "q")) || (s = check_dev_ptr(o, hq, "o")) ||
      (s = check_dev_ptr(d_o, hq, "d_o")) || (s = check_dev_ptr(dq, hq, "dq")) ||
      (s = check_dev_ptr(k, hk, "k")) || (s = check_dev_ptr(v, hk, "v")) ||
      (s = check_dev_ptr(dk, hk, "dk")) || (s = check_dev_ptr(dv, hk, "dv")) ||
      (s = check_dev_ptr(lse, hq, "lse")))
    return s;
  int64_t kv_row = NOMAS_HEAD_DIM, kv_head = NOMAS_HEAD_DIM;
  if ((s = check_stride(q_stride, h.heads, "q")) || (hk && (s = kv_strides(h, kv_stride, h.nk, &kv_row, &kv_head))))
    return s;
  size_t need = 0;
  nomas_attn_bwd_workspace_size(p, &need);
  if (need && (!workspace || workspace_bytes < need))
    return fail(NOMAS_ERR_INVALID_ARGUMENT, "workspace missing or too small");
  if ((s = check_dev_ptr(workspace, need > 0, "workspace"))) return s;
  if (!(scale > 0.f) || !std::isfinite(scale)) return fail(NOMAS_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
  if ((s = check_device(p))) return s;

  nomas::BwdParams bp{};
  bp.q = static_cast<const uint16_t*>(q);
  bp.k = static_cast<const uint16_t*>(k);
  bp.v = static_cast<const uint16_t*>(v);
  bp.o = static_cast<const uint16_t*>(o);
  bp.d_o = static_cast<const uint16_t*>(d_o);
  bp.lse = lse;
  bp.dq = static_cast<uint16_t*>(dq);
  bp.dk = static_cast<uint16_t*>(dk);
  bp.dv = static_cast<uint16_t*>(dv);
  bp.ndelta = static_cast<float*>(workspace);
  bp.nlse2 = bp.ndelta + (size_t)h.heads * (size_t)h.nqt * 128;
  bp.claim = reinterpret_cast<uint32_t*>(bp.nlse2 + (size_t)h.heads * (size_t)h.nqt * 128);
  bp.groups = std::max<int32_t>(1, h.fwd_groups);
  bp.qdesc = p->d_qdesc;
  bp.kdesc = p->d_kdesc;
  bp.pair_ptr = p->d_pair_ptr;
  bp.pair_idx = p->d_pair_idx;
  bp.kpair_ptr = p->d_kpair_ptr;
  bp.kpair_idx = p->d_kpair_idx;
  bp.q_stride = q_stride;
  bp.kv_stride = kv_row;
  bp.kv_head_stride = kv_head;
  bp.nq = (int32_t)h.nq;
  bp.nk = (int32_t)h.nk;
  bp.heads = h.heads;
  bp.nqt = (int32_t)h.nqt;
  bp.nkt = (int32_t)h.nkt;
  bp.n_pairs = (int32_t)h.n_pairs;
  bp.n_kpairs = (int32_t)h.n_kpairs;
  bp.grad_f32 = h.grad_f32 ? 1 : 0;
  bp.scale = scale;
  bp.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e = nomas::launch_attn_bwd(bp, static_cast<hipStream_t>(hip_stream));
  if (e == hipErrorNotSupported) return fail(NOMAS_ERR_UNSUPPORTED, "backward kernels not built");
  if (e != hipSuccess) return hip_fail(e, "attn_bwd launch");
  return ok();
}

// ---------------------------------------------------------------------------
// KV cache
// ---------------------------------------------------------------------------

nomas_status nomas_kvcache_create(int32_t heads, int32_t head_dim, int64_t capacity, void* k_buf,
                                  void* v_buf, nomas_kvcache** out) {
  if (!out) return fail(NOMAS_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  if (heads < 1) return fail(NOMAS_ERR_INVALID_ARGUMENT, "heads must be >= 1");
  if (head_dim != NOMAS_HEAD_DIM) return fail(NOMAS_ERR_UNSUPPORTED, "head_dim must be 128");
  if (capacity < 0 || capacity > (int64_t(1) << 30)) return fail(NOMAS_ERR_INVALID_ARGUMENT, "capacity out of range");
  nomas_status s;
  if ((s = check_dev_ptr(k_buf, capacity > 0, "k_buf")) || (s = check_dev_ptr(v_buf, capacity > 0, "v_buf")))
    return s;
  nomas_kvcache* c = new (std::nothrow) nomas_kvcache();
  if (!c) return fail(NOMAS_ERR_INVALID_ARGUMENT, "out of host memory");
  c->heads = heads;
  c->head_dim = head_dim;
  c->capacity = capacity;
  c->k = k_buf;
  c->v = v_buf;
  *out = c;
  return ok();
}

nomas_status nomas_kvcache_append(nomas_kvcache* c, const nomas_segment* seg, const void* k_new,
                                  const void* v_new, int64_t kv_stride, void* hip_stream) {
  if (!c || !seg) return fail(NOMAS_ERR_INVALID_ARGUMENT, "NULL argument");
  std::string e = nomas::check_segment(*seg);
  if (!e.empty()) return fail(NOMAS_ERR_LAYOUT, e);
  for (const auto& s : c->segs)
    if (s.video == seg->video && s.index == seg->index)
      return fail(NOMAS_ERR_LAYOUT, "segment already in the cache");
  const int64_t n = nomas::segment_cached_tokens(*seg);  // video + head rows, the first ones
  if (c->len + n > c->capacity) return fail(NOMAS_ERR_CAPACITY, "append would exceed the cache capacity");
  nomas_status s;
  if ((s = check_dev_ptr(k_new, true, "k_new")) || (s = check_dev_ptr(v_new, true, "v_new"))) return s;
  if ((s = check_stride(kv_stride, c->heads, "kv"))) return s;
  nomas::AppendParams ap{};
  ap.k_src = static_cast<const uint16_t*>(k_new);
  ap.v_src = static_cast<const uint16_t*>(v_new);
  ap.k_dst = static_cast<uint16_t*>(c->k);
  ap.v_dst = static_cast<uint16_t*>(c->v);
  ap.src_stride = kv_stride;
  ap.cap = c->capacity;
  ap.dst_offset = c->len;
  ap.tokens = (int32_t)n;
  ap.heads = c->heads;
  hipError_t he = nomas::launch_kvcache_append(ap, static_cast<hipStream_t>(hip_stream));
  if (he != hipSuccess) return hip_fail(he, "kvcache_append launch");
  c->segs.push_back(*seg);
  c->len += n;
  return ok();
}

}  // extern "C"

namespace {

// Records of segments whose rows are already in a cache's buffers: checked
// like appends (records, duplicates, capacity) before anything is recorded.
template <typename Cache>
nomas_status adopt_segments(Cache* c, const nomas_segment* segs, int32_t n) {
  if (!c) return fail(NOMAS_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (n < 0 || (n > 0 && !segs)) return fail(NOMAS_ERR_INVALID_ARGUMENT, "bad segment array");
  if (!c->segs.empty()) return fail(NOMAS_ERR_INVALID_ARGUMENT, "cache already holds segments");
  int64_t len = 0;
  for (int32_t i = 0; i < n; ++i) {
    std::string e = nomas::check_segment(segs[i]);
    if (!e.empty()) return fail(NOMAS_ERR_LAYOUT, "segment " + std::to_string(i) + ": " + e);
    for (int32_t j = 0; j < i; ++j)
      if (segs[j].video == segs[i].video && segs[j].index == segs[i].index)
        return fail(NOMAS_ERR_LAYOUT, "segment listed twice");
    len += nomas::segment_cached_tokens(segs[i]);
  }
  if (len > c->capacity) return fail(NOMAS_ERR_CAPACITY, "segments exceed the cache capacity");
  c->segs.assign(segs, segs + n);
  c->len = len;
  return ok();
}

}  // namespace

extern "C" {

nomas_status nomas_kvcache_adopt(nomas_kvcache* c, const nomas_segment* segs, int32_t n_segments) {
  return adopt_segments(c, segs, n_segments);
}

nomas_status nomas_kvcache_int8_adopt(nomas_kvcache_int8* c, const nomas_segment* segs,
                                      int32_t n_segments) {
  return adopt_segments(c, segs, n_segments);
}

nomas_status nomas_kvcache_truncate(nomas_kvcache* c, int32_t n_segments) {
  if (!c) return fail(NOMAS_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (n_segments < 0 || n_segments > (int32_t)c->segs.size())
    return fail(NOMAS_ERR_INVALID_ARGUMENT, "n_segments out of range");
  c->segs.resize((size_t)n_segments);
  int64_t len = 0;
  for (const auto& s : c->segs) len += nomas::segment_cached_tokens(s);
  c->len = len;
  return ok();
}

nomas_status nomas_kvcache_reset(nomas_kvcache* c) { return nomas_kvcache_truncate(c, 0); }

nomas_status nomas_kvcache_len(const nomas_kvcache* c, int64_t* n_tokens, int32_t* n_segments) {
  if (!c) return fail(NOMAS_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (n_tokens) *n_tokens = c->len;
  if (n_segments) *n_segments = (int32_t)c->segs.size();
  return ok();
}

nomas_status nomas_kvcache_destroy(nomas_kvcache* c) {
  delete c;
  return ok();
}

// ---------------------------------------------------------------------------
// INT8 KV cache
// ---------------------------------------------------------------------------

nomas_status nomas_kvcache_int8_create(int32_t heads, int32_t head_dim, int64_t capacity,
                                       void* k_codes, void* v_codes, void* k_exp, void* v_exp,
                                       nomas_kvcache_int8** out) {
  if (!out) return fail(NOMAS_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  if (heads < 1) return fail(NOMAS_ERR_INVALID_ARGUMENT, "heads must be >= 1");
  if (head_dim != NOMAS_HEAD_DIM) return fail(NOMAS_ERR_UNSUPPORTED, "head_dim must be 128");
  if (capacity < 0 || capacity > (int64_t(1) << 30)) return fail(NOMAS_ERR_INVALID_ARGUMENT, "capacity out of range");
  nomas_status s;
  const bool need = capacity > 0;
  if ((s = check_dev_ptr(k_codes, need, "k_codes")) || (s = check_dev_ptr(v_codes, need, "v_codes")) ||
      (s = check_dev_ptr(k_exp, need, "k_exp")) || (s = check_dev_ptr(v_exp, need, "v_exp")))
    return s;
  nomas_kvcache_int8* c = new (std::nothrow) nomas_kvcache_int8();
  if (!c) return fail(NOMAS_ERR_INVALID_ARGUMENT, "out of host memory");
  c->heads = heads;
  c->capacity = capacity;
  c->k_codes = k_codes;
  c->v_codes = v_codes;
  c->k_exp = k_exp;
  c->v_exp = v_exp;
  *out = c;
  return ok();
}

nomas_status nomas_kvcache_int8_append(nomas_kvcache_int8* c, const nomas_segment* seg,
                                       const void* k_new, const void* v_new, int64_t kv_stride,
                                       void* hip_stream) {
  if (!c || !seg) return fail(NOMAS_ERR_INVALID_ARGUMENT, "NULL argument");
  std::string e = nomas::check_segment(*seg);
  if (!e.empty()) return fail(NOMAS_ERR_LAYOUT, e);
  for (const auto& s : c->segs)
    if (s.video == seg->video && s.index == seg->index)
      return fail(NOMAS_ERR_LAYOUT, "segment already in the cache");
  const int64_t n = nomas::segment_cached_tokens(*seg);  // video + head rows, the first ones
  if (c->len + n > c->capacity) return fail(NOMAS_ERR_CAPACITY, "append would exceed the cache capacity");
  nomas_status s;
  if ((s = check_dev_ptr(k_new, true, "k_new")) || (s = check_dev_ptr(v_new, true, "v_new"))) return s;
  if ((s = check_stride(kv_stride, c->heads, "kv"))) return s;
  nomas::Int8AppendParams ap{};
  ap.k_src = static_cast<const uint16_t*>(k_new);
  ap.v_src = static_cast<const uint16_t*>(v_new);
  ap.k_codes = static_cast<int8_t*>(c->k_codes);
  ap.v_codes = static_cast<int8_t*>(c->v_codes);
  ap.k_exp = static_cast<int8_t*>(c->k_exp);
  ap.v_exp = static_cast<int8_t*>(c->v_exp);
  ap.src_stride = kv_stride;
  ap.cap = c->capacity;
  ap.dst_offset = c->len;
  ap.tokens = (int32_t)n;
  ap.heads = c->heads;
  hipError_t he = nomas::launch_kvcache_int8_append(ap, static_cast<hipStream_t>(hip_stream));
  if (he != hipSuccess) return hip_fail(he, "kvcache_int8_append launch");
  c->segs.push_back(*seg);
  c->len += n;
  return ok();
}

nomas_status nomas_kvcache_int8_expand(const nomas_kvcache_int8* c, nomas_kvcache* dst,
                                       void* hip_stream) {
  if (!c || !dst) return fail(NOMAS_ERR_INVALID_ARGUMENT, "NULL argument");
  if (dst->heads != c->heads) return fail(NOMAS_ERR_INVALID_ARGUMENT, "caches differ in head count");
  if (c->len > dst->capacity) return fail(NOMAS_ERR_CAPACITY, "destination cache too small");
  nomas::Int8ExpandParams xp{};
  xp.k_codes = static_cast<const int8_t*>(c->k_codes);
  xp.v_codes = static_cast<const int8_t*>(c->v_codes);
  xp.k_exp = static_cast<const int8_t*>(c->k_exp);
  xp.v_exp = static_cast<const int8_t*>(c->v_exp);
  xp.k_dst = static_cast<uint16_t*>(dst->k);
  xp.v_dst = static_cast<uint16_t*>(dst->v);
  xp.src_cap = c->capacity;
  xp.dst_cap = dst->capacity;
  xp.rows = c->len;
  xp.heads = c->heads;
  hipError_t he = nomas::launch_kvcache_int8_expand(xp, static_cast<hipStream_t>(hip_stream));
  if (he != hipSuccess) return hip_fail(he, "kvcache_int8_expand launch");
  dst->segs = c->segs;
  dst->len = c->len;
  return ok();
}

nomas_status nomas_kvcache_int8_truncate(nomas_kvcache_int8* c, int32_t n_segments) {
  if (!c) return fail(NOMAS_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (n_segments < 0 || n_segments > (int32_t)c->segs.size())
    return fail(NOMAS_ERR_INVALID_ARGUMENT, "n_segments out of range");
  c->segs.resize((size_t)n_segments);
  int64_t len = 0;
  for (const auto& s : c->segs) len += nomas::segment_cached_tokens(s);
  c->len = len;
  return ok();
}

nomas_status nomas_kvcache_int8_len(const nomas_kvcache_int8* c, int64_t* n_tokens,
                                    int32_t* n_segments) {
  if (!c) return fail(NOMAS_ERR_INVALID_ARGUMENT, "cache is NULL");
  if (n_tokens) *n_tokens = c->len;
  if (n_segments) *n_segments = (int32_t)c->segs.size();
  return ok();
}

nomas_status nomas_kvcache_int8_destroy(nomas_kvcache_int8* c) {
  delete c;
  return ok();
}

}  // extern "C"
