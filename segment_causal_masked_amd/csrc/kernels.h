// Internal interface between the C ABI (abi.cpp) and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace nomas {

struct QDescDev {
  int32_t seg, lo;
  uint32_t amask;
  int32_t pad_;
};
struct KDescDev {
  int32_t seg;
  uint32_t bits;
};

struct FwdParams {
  const uint16_t* q;       // [nq][H][128] bf16, stride q_stride
  const uint16_t* k_cache; // [H][cap][128] bf16 (or null)
  const uint16_t* v_cache;
  const uint16_t* k_new;   // new-token rows: row r of head h at r * kv_stride + h * kv_head_stride
  const uint16_t* v_new;
  uint16_t* o;             // [nq][H][128] bf16, stride o_stride
  float* lse;              // [H][nq] or null
  const QDescDev* qdesc;   // nqt*128 entries
  const KDescDev* kdesc;   // nkt*64 entries
  const int32_t* csr_ptr;  // per q-tile pair: n_pairs+1
  const int32_t* csr_idx;  // (k_tile << 4) | flags (see plan.h)
  const int32_t* wg_ptr;   // groups+1: pieces of each persistent workgroup
  const int4* pieces;      // {unit, entry_begin, entry_end, slot or -1}
  const int4* combine;     // {unit, first_slot, n_pieces, 0}
  const int4* chunks;      // tail pieces, claimed in turn through *claim (or none)
  uint32_t* claim;         // workspace: the next chunk to hand out (zeroed per call)
  const int32_t* unit_shift;  // per unit: entries visited in order (j + shift) mod n
  int64_t list_head_stride;    // lists per head (sparse plans), else 0: unit (h, u')
                               // walks csr_idx + h * list_head_stride + csr_ptr[u']
  float* partial;          // workspace: n_slots * attn_fwd_slot_bytes()
  int64_t q_stride, kv_stride, kv_head_stride, o_stride, cache_cap;
  int32_t nq, nk, n_cached, heads, nqt, nkt;
  int32_t groups, n_combine, n_pairs, n_chunks;
  float scale_log2;        // softmax scale * log2(e)
};

hipError_t launch_attn_fwd(const FwdParams& p, hipStream_t stream);

// Fixed device scratch of the allocation-free forward (noalloc.hip): its
// address on `device` (which must be the current device on the first call for
// it), resolved once per device.
constexpr size_t NOALLOC_SCRATCH_BYTES = size_t(64) << 20;
hipError_t noalloc_scratch(int device, void** ptr);

// Video-block selection of sparse plans (select.hip): per (head, query-tile
// pair) the kept key-tile list, written to `lists`.
struct SelParams {
  const uint16_t* q;        // [nq][H][128] bf16, stride q_stride
  const uint16_t* k_cache;  // [H][cap][128] bf16 (or null)
  const uint16_t* k_new;    // new-token rows, as in FwdParams
  const int32_t* pair_ptr;  // dense merged lists per pair (n_pairs + 1)
  const int32_t* pair_idx;  // (k_tile << 4) | flags
  const int32_t* sp_ptr;    // sparse list prefix per pair (n_pairs + 1)
  const int32_t* sp_keep;   // video entries kept per pair
  const int32_t* video_tile;  // per key tile: 1 = every key a video token
  float* k_sum;             // workspace [H][nkt][128]
  float* q_sum;             // workspace [H][n_pairs][128]
  int32_t* lists;           // workspace [H][sp_total]
  uint64_t* keys;           // workspace [H][pair_total] (null unless some pair list
                            // is longer than SELECT_SORT_ENTRIES): sort keys of long lists
  int64_t q_stride, kv_stride, kv_head_stride, cache_cap, sp_total, pair_total;
  int32_t nq, nk, n_cached, heads, nkt, n_pairs;
};
// Pair lists up to this length are ranked by a bitonic sort in LDS; longer
// ones by a radix select over keys kept in the workspace.
constexpr int SELECT_SORT_ENTRIES = 4096;
hipError_t launch_select(const SelParams& p, hipStream_t stream);
size_t attn_fwd_slot_bytes();
int attn_fwd_groups_per_cu();  // persistent forward workgroups per CU

struct AppendParams {
  const uint16_t* k_src;   // [T][H][128], stride src_stride
  const uint16_t* v_src;
  uint16_t* k_dst;         // [H][cap][128]
  uint16_t* v_dst;
  int64_t src_stride, cap, dst_offset;
  int32_t tokens, heads;
};

hipError_t launch_kvcache_append(const AppendParams& p, hipStream_t stream);

// INT8 cache (kvcache.hip): per (head, token) row, 128 int8 codes and one
// int8 exponent e, value = code * 2^e.
struct Int8AppendParams {
  const uint16_t* k_src;   // [T][H][128] bf16, stride src_stride
  const uint16_t* v_src;
  int8_t* k_codes;         // [H][cap][128]
  int8_t* v_codes;
  int8_t* k_exp;           // [H][cap]
  int8_t* v_exp;
  int64_t src_stride, cap, dst_offset;
  int32_t tokens, heads;
};
hipError_t launch_kvcache_int8_append(const Int8AppendParams& p, hipStream_t stream);

struct Int8ExpandParams {
  const int8_t *k_codes, *v_codes, *k_exp, *v_exp;  // [H][src_cap][128], [H][src_cap]
  uint16_t *k_dst, *v_dst;                          // bf16 [H][dst_cap][128]
  int64_t src_cap, dst_cap, rows;                   // rows [0, rows) of every head
  int32_t heads;
};
hipError_t launch_kvcache_int8_expand(const Int8ExpandParams& p, hipStream_t stream);

struct BwdParams {
  const uint16_t *q, *k, *v, *o, *d_o;  // bf16; q, o, d_o: [T][H][128], token stride q_stride
  const float* lse;        // [H][nq], natural log (from the forward)
  uint16_t *dq, *dk, *dv;  // outputs, same layouts (element strides) as q / k / v;
                           // fp32 elements when grad_f32 != 0, else bf16
  float* ndelta;           // workspace [H][nqt*128]: -rowsum(dO * O)
  float* nlse2;            // workspace [H][nqt*128]: -lse * log2(e), 0 where -inf or padding
  uint32_t* claim;         // workspace: 8 + 8 work-queue counters of the dK/dV and dQ
                           // kernels, zeroed by the row-statistics kernel
  const QDescDev* qdesc;   // nqt*128 entries
  const KDescDev* kdesc;   // nkt*64 entries
  const int32_t *pair_ptr, *pair_idx;    // per q-tile pair: the forward's key-tile lists
  const int32_t *kpair_ptr, *kpair_idx;  // per key-tile pair: (q_tile << 4) | flags
  int64_t q_stride, kv_stride, kv_head_stride;  // k, v, dk, dv: row r of head h at
                                                // r * kv_stride + h * kv_head_stride
  int32_t nq, nk, heads, nqt, nkt, n_pairs, n_kpairs;
  int32_t groups;          // persistent workgroups of the dK/dV and dQ kernels (one per CU)
  int32_t grad_f32;
  float scale, scale_log2;
};

hipError_t launch_attn_bwd(const BwdParams& p, hipStream_t stream);

// Camera cross-attention (camera.hip): query token t sees the camera tokens
// [qrange[t].x, qrange[t].y); a workgroup computes groups of CAM_GROUP
// consecutive query tokens of one head, each over the union grange[group] of
// its tokens' ranges; `cus` (compute units) sizes the grid.
constexpr int CAM_GROUP = 128;
struct CamParams {
  const uint16_t* q;       // [nq][H][128] bf16, stride q_stride
  const uint16_t* kc;      // [n_cam][H][128] bf16, stride cam_stride
  const uint16_t* vc;
  uint16_t* o;             // [nq][H][128] bf16, stride o_stride
  const int2* qrange;      // n_groups * CAM_GROUP entries (tail: empty ranges)
  const int2* grange;      // n_groups entries
  int64_t q_stride, cam_stride, o_stride;
  int32_t nq, heads, n_groups;
  float scale_log2;        // softmax scale * log2(e)
};

hipError_t launch_camera_attn(const CamParams& p, int cus, hipStream_t stream);

}  // namespace nomas
