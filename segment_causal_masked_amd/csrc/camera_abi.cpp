// C ABI of the camera cross-attention: plan (per-token camera-token ranges),
// info / export, and the forward launch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kernels.h"
#include "nomas_attn.h"
#include "plan.h"
#include "status.h"

struct nomas_camera_plan {
  int32_t heads = 0, radius = 0;
  int64_t nq = 0, n_video = 0, n_cam = 0, pairs = 0, n_groups = 0;
  std::vector<int32_t> ranges;   // [nq][2]: first, end camera token
  std::vector<int32_t> granges;  // [n_groups][2]: union over CAM_GROUP query tokens
  int device = -1, cus = 256;
  void* dmem = nullptr;
  const int2* d_qrange = nullptr;
  const int2* d_grange = nullptr;
};

namespace {

using nomas::clear_error;
using nomas::set_error;

nomas_status hip_fail(hipError_t e, const char* where) {
  return set_error(NOMAS_ERR_HIP, std::string(where) + ": " + hipGetErrorString(e));
}

// Camera tokens: n_frames per segment, in layout order.  A video token of
// latent frame f in a segment whose camera tokens start at c sees
// [c + max(0, f - r), c + min(F, f + r + 1)) (r < 0: [c, c + F)); every other
// token sees none.
nomas_status build_ranges(const nomas_layout* q, nomas_camera_plan* p) {
  int64_t cam = 0;
  for (int32_t i = 0; i < q->n_segments; ++i) {
    const nomas_segment& s = q->segments[i];
    const std::string e = nomas::check_segment(s);
    if (!e.empty()) return set_error(NOMAS_ERR_LAYOUT, "segment " + std::to_string(i) + ": " + e);
    const int64_t F = s.n_frames, T = s.tokens_per_frame;
    if (cam + F > INT32_MAX || p->nq + nomas::segment_tokens(s) > INT32_MAX)
      return set_error(NOMAS_ERR_UNSUPPORTED, "more than 2^31 - 1 tokens or camera tokens");
    for (int64_t f = 0; f < F; ++f) {
      const int64_t lo = cam + (p->radius < 0 ? 0 : std::max<int64_t>(0, f - p->radius));
      const int64_t hi = cam + (p->radius < 0 ? F : std::min<int64_t>(F, f + p->radius + 1));
      for (int64_t t = 0; t < T; ++t) {
        p->ranges.push_back((int32_t)lo);
        p->ranges.push_back((int32_t)hi);
      }
      p->pairs += T * (hi - lo);
    }
    p->n_video += F * T;
    const int64_t rest = nomas::segment_tokens(s) - F * T;
    p->ranges.insert(p->ranges.end(), size_t(2 * rest), 0);
    p->nq += F * T + rest;
    cam += F;
  }
  p->n_cam = cam;
  const int64_t G = nomas::CAM_GROUP;
  p->n_groups = (p->nq + G - 1) / G;
  p->granges.assign(size_t(2 * p->n_groups), 0);
  for (int64_t b = 0; b < p->n_groups; ++b) {
    int32_t lo = INT32_MAX, hi = INT32_MIN;
    for (int64_t t = G * b; t < std::min(p->nq, G * b + G); ++t) {
      const int32_t a = p->ranges[size_t(2 * t)], z = p->ranges[size_t(2 * t + 1)];
      if (z > a) {
        lo = std::min(lo, a);
        hi = std::max(hi, z);
      }
    }
    if (hi > lo) {
      p->granges[size_t(2 * b)] = lo;
      p->granges[size_t(2 * b + 1)] = hi;
    }
  }
  return NOMAS_OK;
}

}  // namespace

extern "C" {

nomas_status nomas_camera_attn_plan(const nomas_layout* q, int32_t num_heads, int32_t radius_frames,
                               int32_t flags, nomas_camera_plan** out) {
  if (!out) return set_error(NOMAS_ERR_INVALID_ARGUMENT, "out is NULL");
  *out = nullptr;
  if (!q) return set_error(NOMAS_ERR_INVALID_ARGUMENT, "query layout is NULL");
  if (q->n_segments < 0 || (q->n_segments > 0 && !q->segments))
    return set_error(NOMAS_ERR_INVALID_ARGUMENT, "query layout: bad n_segments or NULL segments");
  if (num_heads < 1) return set_error(NOMAS_ERR_INVALID_ARGUMENT, "num_heads < 1");
  if (flags & ~NOMAS_PLAN_HOST_ONLY) return set_error(NOMAS_ERR_INVALID_ARGUMENT, "unknown flags");
  nomas_camera_plan* p = new (std::nothrow) nomas_camera_plan();
  if (!p) return set_error(NOMAS_ERR_INVALID_ARGUMENT, "out of host memory");
  p->heads = num_heads;
  p->radius = radius_frames < 0 ? -1 : radius_frames;
  nomas_status s;
  try {
    s = build_ranges(q, p);
  } catch (const std::bad_alloc&) {
    s = set_error(NOMAS_ERR_INVALID_ARGUMENT, "out of host memory while building the plan");
  }
  if (s != NOMAS_OK) {
    delete p;
    return s;
  }
  if (!(flags & NOMAS_PLAN_HOST_ONLY)) {
    hipError_t e = hipGetDevice(&p->device);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&p->cus, hipDeviceAttributeMultiprocessorCount, p->device);
    if (e != hipSuccess) {
      delete p;
      return hip_fail(e, "device query");
    }
    // query ranges padded to whole groups (empty), then the group ranges
    const size_t qbytes = size_t(p->n_groups) * nomas::CAM_GROUP * sizeof(int2);
    const size_t boff = (qbytes + 255) & ~size_t(255);
    const size_t total = boff + std::max<size_t>(16, size_t(p->n_groups) * sizeof(int2));
    std::vector<char> staging(total, 0);
    if (!p->ranges.empty()) std::memcpy(staging.data(), p->ranges.data(), p->ranges.size() * 4);
    if (!p->granges.empty()) std::memcpy(staging.data() + boff, p->granges.data(), p->granges.size() * 4);
    e = hipMalloc(&p->dmem, total);
    if (e == hipSuccess) e = hipMemcpy(p->dmem, staging.data(), total, hipMemcpyHostToDevice);
    if (e != hipSuccess) {
      if (p->dmem) (void)hipFree(p->dmem);
      delete p;
      return hip_fail(e, "camera plan upload");
    }
    p->d_qrange = reinterpret_cast<const int2*>(p->dmem);
    p->d_grange = reinterpret_cast<const int2*>(static_cast<char*>(p->dmem) + boff);
  }
  *out = p;
  return clear_error();
}

nomas_status nomas_camera_plan_get_info(const nomas_camera_plan* p, nomas_camera_plan_info* info) {
  if (!p || !info) return set_error(NOMAS_ERR_INVALID_ARGUMENT, "NULL argument");
  info->n_queries = p->nq;
  info->n_video_queries = p->n_video;
  info->n_camera_tokens = p->n_cam;
  info->visible_pairs = p->pairs;
  info->effective_flop = 4.0 * NOMAS_HEAD_DIM * p->heads * (double)p->pairs;
  info->algorithmic_bytes = 2.0 * NOMAS_HEAD_DIM * p->heads * (2.0 * (double)p->nq + 2.0 * (double)p->n_cam);
  info->num_heads = p->heads;
  info->radius_frames = p->radius;
  return clear_error();
}

nomas_status nomas_camera_plan_export_ranges(const nomas_camera_plan* p, int32_t* buf, size_t n) {
  if (!p || !buf) return set_error(NOMAS_ERR_INVALID_ARGUMENT, "NULL argument");
  if (n < p->ranges.size()) return set_error(NOMAS_ERR_INVALID_ARGUMENT, "buffer too small");
  if (!p->ranges.empty()) std::memcpy(buf, p->ranges.data(), p->ranges.size() * 4);
  return clear_error();
}

nomas_status nomas_camera_plan_destroy(nomas_camera_plan* p) {
  if (!p) return clear_error();
  if (p->dmem) (void)hipFree(p->dmem);
  delete p;
  return clear_error();
}

nomas_status nomas_camera_attn_fwd(const nomas_camera_plan* p, const void* q, int64_t q_stride,
                                   const void* k_cam, const void* v_cam, int64_t cam_stride,
                                   void* o, int64_t o_stride, float scale, void* hip_stream) {
  if (!p) return set_error(NOMAS_ERR_INVALID_ARGUMENT, "plan is NULL");
  if (!p->dmem) return set_error(NOMAS_ERR_INVALID_ARGUMENT, "host-only plan");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev != p->device) return set_error(NOMAS_ERR_INVALID_ARGUMENT, "plan was built on another device");
  if (p->nq == 0) return clear_error();
  const int64_t row = (int64_t)p->heads * NOMAS_HEAD_DIM;
  struct S { int64_t v; const char* name; bool needed; };
  for (const S& st : {S{q_stride, "q", true}, S{o_stride, "o", true}, S{cam_stride, "camera", p->n_cam > 0}}) {
    if (!st.needed) continue;
    if (st.v < row) return set_error(NOMAS_ERR_INVALID_ARGUMENT, std::string(st.name) + " stride < heads * 128");
    if (st.v % 8 != 0) return set_error(NOMAS_ERR_ALIGNMENT, std::string(st.name) + " stride not a multiple of 8");
    if (st.v > (int64_t(1) << 24))
      return set_error(NOMAS_ERR_INVALID_ARGUMENT, std::string(st.name) + " stride above 2^24 elements");
  }
  struct Ptr { const void* v; const char* name; bool needed; };
  for (const Ptr& pt : {Ptr{q, "q", true}, Ptr{o, "o", true}, Ptr{k_cam, "k_cam", p->n_cam > 0},
                        Ptr{v_cam, "v_cam", p->n_cam > 0}}) {
    if (!pt.needed) continue;
    if (!pt.v) return set_error(NOMAS_ERR_INVALID_ARGUMENT, std::string(pt.name) + " is NULL");
    if (reinterpret_cast<uintptr_t>(pt.v) & 15u)
      return set_error(NOMAS_ERR_ALIGNMENT, std::string(pt.name) + " not 16-byte aligned");
  }
  if (!(scale > 0.f) || !std::isfinite(scale)) return set_error(NOMAS_ERR_INVALID_ARGUMENT, "scale must be finite and > 0");
  nomas::CamParams cp{};
  cp.q = static_cast<const uint16_t*>(q);
  cp.kc = static_cast<const uint16_t*>(k_cam);
  cp.vc = static_cast<const uint16_t*>(v_cam);
  cp.o = static_cast<uint16_t*>(o);
  cp.qrange = p->d_qrange;
  cp.grange = p->d_grange;
  cp.q_stride = q_stride;
  cp.cam_stride = cam_stride;
  cp.o_stride = o_stride;
  cp.nq = (int32_t)p->nq;
  cp.heads = p->heads;
  cp.n_groups = (int32_t)p->n_groups;
  cp.scale_log2 = scale * 1.4426950408889634f;
  e = nomas::launch_camera_attn(cp, p->cus, static_cast<hipStream_t>(hip_stream));
  if (e != hipSuccess) return hip_fail(e, "camera_attn_kernel launch");
  return clear_error();
}

}  // extern "C"
