// Video-block selection for sparse forward plans (gfx950).
//
// "Summary (Overview)", Inference: after the first two denoising steps only a
// quarter of the video blocks are retained.  The pages do not say how blocks
// are chosen; the reading implemented here (and stated in the ABI header):
// per (head h, query-tile pair u), among the key tiles of u's list whose keys
// are all video tokens, keep the ceil(P% of them) with the highest block score
//     s(h, u, t) = sum_d qsum[d] * ksum[d],
//     qsum[d] = sum of Q[q, h, d] over the 256 query rows of u,
//     ksum[d] = sum of K[k, h, d] over the 64 key rows of tile t,
// (the sum of u's logits over tile t, up to the softmax scale); ties go to
// the lower key tile.  Tiles holding any head, tail or padding key are always
// kept.  The kept entries, in list order, form u's list for head h.
//
// s is evaluated in fp32 in a fixed order, so the lists are deterministic:
// every add and product rounded separately (this file is built without
// floating-point contraction), a row sum taken in groups of 16 consecutive
// rows -- each group summed in ascending row order, then the group sums added
// in ascending group order, every sum starting from +0.0, rows past the end
// entering as +0.0 -- and the dot over ascending d.  The ranking then differs
// from the exact one only between tiles whose exact scores are closer than
// the rounding error of that evaluation.
//
// Two launches: the key-tile and query-pair sums, then one workgroup per
// (pair, head) that scores, ranks (a bitonic sort in LDS, or for lists of
// more than 4096 entries a radix select over keys in the workspace) and
// compacts the list.
#include "kernels.h"

namespace nomas {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

constexpr int GROUP = 16;  // rows per partial sum

// Sum of `rows` rows (ascending, in groups of 16) of 128 dims for one block:
// thread t adds dims 8 (t % 16) .. +7 over rows 16 (t / 16) .. +15 of its
// group, then threads 0..127 add the group sums of their dim in group order.
// row_ptr(r) gives the 8 bf16 of row r at dims 8 (t % 16), or null (absent).
template <int ROWS, typename RowPtr>
__device__ __forceinline__ void block_row_sum(RowPtr row_ptr, float* out, float* part) {
  constexpr int NG = ROWS / GROUP;
  const int t = (int)threadIdx.x;
  if (t < 16 * NG) {
    const int dg = t & 15, g = t >> 4;
    uint4 x[GROUP];
#pragma unroll
    for (int r = 0; r < GROUP; ++r) {
      const uint16_t* src = row_ptr(GROUP * g + r, dg);
      x[r] = src ? *reinterpret_cast<const uint4*>(src) : uint4{0u, 0u, 0u, 0u};
    }
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < GROUP; ++r) {
      const uint32_t w[4] = {x[r].x, x[r].y, x[r].z, x[r].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] = acc[2 * j] + __uint_as_float(w[j] << 16);
        acc[2 * j + 1] = acc[2 * j + 1] + __uint_as_float(w[j] & 0xffff0000u);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) part[g * 128 + 8 * dg + j] = acc[j];
  }
  __syncthreads();
  if (t < 128) {
    float s = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) s = s + part[g * 128 + t];
    out[t] = s;
  }
}

// One launch for both kinds of sums, one workgroup per (item, head): items
// 0 .. nkt - 1 are key tiles (ksum of every video key tile), the rest
// query-tile pairs (qsum).  The branch is uniform per workgroup.
__global__ __launch_bounds__(256) void select_sums_kernel(SelParams p) {
  const int item = (int)blockIdx.x, h = (int)blockIdx.y;
  __shared__ float part[(256 / GROUP) * 128];
  if (item < p.nkt) {
    const int kt = item;
    if (!p.video_tile[kt]) return;
    auto row = [&](int r, int dg) -> const uint16_t* {
      const int key = kt * 64 + r;
      if (key >= p.nk) return nullptr;
      return (key < p.n_cached ? p.k_cache + ((int64_t)h * p.cache_cap + key) * 128
                               : p.k_new + (int64_t)(key - p.n_cached) * p.kv_stride + (int64_t)h * p.kv_head_stride) +
             8 * dg;
    };
    block_row_sum<64>(row, p.k_sum + ((int64_t)h * p.nkt + kt) * 128, part);
  } else {
    const int u = item - p.nkt;
    auto row = [&](int r, int dg) -> const uint16_t* {
      const int q = u * 256 + r;
      if (q >= p.nq) return nullptr;
      return p.q + (int64_t)q * p.q_stride + (int64_t)h * 128 + 8 * dg;
    };
    block_row_sum<256>(row, p.q_sum + ((int64_t)h * p.n_pairs + u) * 128, part);
  }
}

// fp32 -> uint32 with the same order (negative values reversed)
__device__ __forceinline__ uint32_t order_key(float s) {
  const uint32_t b = __float_as_uint(s);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

// Sort key of list entry i (a key tile of the pair's list): (score order <<
// 32) | ~i, larger = better score, the lower index first among equal scores;
// 0 for an entry that is not a video tile (always kept, never ranked).
// Real keys are never 0: order_key of any float is nonzero except for one
// NaN pattern, and ~i is nonzero for i < 2^32 - 1.
__device__ __forceinline__ uint64_t entry_key(const SelParams& p, const float* qs, int h, int e0,
                                              int i) {
  const int kt = p.pair_idx[e0 + i] >> 4;
  if (!p.video_tile[kt]) return 0;
  const float* ks = p.k_sum + ((int64_t)h * p.nkt + kt) * 128;
  float s = 0.f;
  // product and sum rounded separately (this file is built without
  // floating-point contraction), ascending d; loads in batches of 32
  for (int d0 = 0; d0 < 128; d0 += 32) {
    float kv[32];
#pragma unroll
    for (int d = 0; d < 32; ++d) kv[d] = ks[d0 + d];
#pragma unroll
    for (int d = 0; d < 32; ++d) s = s + qs[d0 + d] * kv[d];
  }
  return ((uint64_t)order_key(s) << 32) | (uint64_t)(~(uint32_t)i);
}

// Write the kept entries of a pair's list, in list order, given each
// entry's keep flag: thread t handles entries [c0, c1), an exclusive prefix
// sum of the per-thread counts (inclusive scan inside each wave, then the
// totals of the waves before) gives its output position.
template <typename Keep>
__device__ __forceinline__ void compact_list(const SelParams& p, int u, int h, int e0, int n,
                                             Keep keep, int* wave_tot) {
  const int tid = (int)threadIdx.x;
  const int per = (n + 255) / 256;
  const int c0 = min(n, tid * per), c1 = min(n, c0 + per);
  int c = 0;
  for (int i = c0; i < c1; ++i) c += keep(i);
  const int lane = tid & 63;
  int incl = c;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int v = __shfl_up(incl, d);
    if (lane >= d) incl += v;
  }
  if (lane == 63) wave_tot[tid >> 6] = incl;
  __syncthreads();
  int before = incl - c;
  for (int w = 0; w < (tid >> 6); ++w) before += wave_tot[w];
  int32_t* out = p.lists + (int64_t)h * p.sp_total + p.sp_ptr[u] + before;
  for (int i = c0; i < c1; ++i)
    if (keep(i)) *out++ = p.pair_idx[e0 + i];
}

// A list longer than SELECT_SORT_ENTRIES: keys go to the workspace, and the
// k-th largest key is found by a radix select, 8 bits per pass from the top
// (a histogram of the next digit over the keys that match the digits chosen
// so far; keys are unique, so after 8 passes the prefix is that key); then
// the video entries with a key at or above it are kept.  Every loop is
// bounded by n or by the 8 passes.
__device__ void select_long_list(const SelParams& p, const float* qs, int u, int h, int e0, int n,
                                 int* wave_tot) {
  __shared__ unsigned hist[256];
  __shared__ uint64_t s_prefix;
  __shared__ int s_remain;
  const int tid = (int)threadIdx.x;
  uint64_t* kb = p.keys + (int64_t)h * p.pair_total + e0;
  for (int i = tid; i < n; i += 256) kb[i] = entry_key(p, qs, h, e0, i);
  __syncthreads();  // the workgroup's global writes are visible to it after the barrier
  const int k = p.sp_keep[u];
  uint64_t prefix = 0, mask = 0;
  int remain = k;
  for (int shift = 56; k > 0 && shift >= 0; shift -= 8) {
    hist[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += 256) {
      const uint64_t key = kb[i];
      if (key != 0 && (key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      int cum = 0, b = 255;
      for (; b > 0; --b) {
        if (cum + (int)hist[b] >= remain) break;
        cum += (int)hist[b];
      }
      s_prefix = prefix | ((uint64_t)b << shift);
      s_remain = remain - cum;
    }
    __syncthreads();
    prefix = s_prefix;
    remain = s_remain;
    mask |= (uint64_t)0xFF << shift;
  }
  const uint64_t threshold = prefix;
  compact_list(p, u, h, e0, n,
               [&](int i) {
                 const uint64_t key = kb[i];
                 return key == 0 || (k > 0 && key >= threshold);
               },
               wave_tot);
}

__global__ __launch_bounds__(256) void select_lists_kernel(SelParams p) {
  const int u = (int)blockIdx.x, h = (int)blockIdx.y, tid = (int)threadIdx.x;
  __shared__ float qs[128];
  __shared__ uint64_t keys[SELECT_SORT_ENTRIES];
  __shared__ uint8_t keep[SELECT_SORT_ENTRIES];
  __shared__ int wave_tot[4];
  const int e0 = p.pair_ptr[u], n = p.pair_ptr[u + 1] - e0;
  if (tid < 128) qs[tid] = p.q_sum[((int64_t)h * p.n_pairs + u) * 128 + tid];
  __syncthreads();
  if (n > SELECT_SORT_ENTRIES) {  // uniform: the whole workgroup
    select_long_list(p, qs, u, h, e0, n, wave_tot);
    return;
  }
  int npow = 1;
  while (npow < n) npow <<= 1;
  // sort keys: (score order << 32) | ~index, descending = best score first,
  // lower index first among equal scores; entries that are not video tiles
  // (and the padding up to a power of two) get 0 and sort last
  for (int i = tid; i < npow; i += 256) {
    const uint64_t key = i < n ? entry_key(p, qs, h, e0, i) : 0;
    keys[i] = key;
    keep[i] = i < n && key == 0;  // not a video tile: always kept
  }
  __syncthreads();
  for (int size = 2; size <= npow; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < npow; i += 256) {
        const int j = i ^ stride;
        if (j > i) {
          const uint64_t a = keys[i], b = keys[j];
          const bool first_half_desc = (i & size) == 0;
          if (first_half_desc ? (a < b) : (a > b)) {
            keys[i] = b;
            keys[j] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  const int k = p.sp_keep[u];
  for (int r = tid; r < k; r += 256) keep[~(uint32_t)(keys[r] & 0xffffffffu)] = 1;
  __syncthreads();
  compact_list(p, u, h, e0, n, [&](int i) { return (int)keep[i]; }, wave_tot);
}

}  // namespace

hipError_t launch_select(const SelParams& p, hipStream_t stream) {
  if (p.n_pairs == 0) return hipSuccess;
  hipLaunchKernelGGL(select_sums_kernel, dim3((unsigned)(p.nkt + p.n_pairs), (unsigned)p.heads),
                     dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_lists_kernel, dim3((unsigned)p.n_pairs, (unsigned)p.heads), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace nomas
