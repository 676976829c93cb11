// KV-cache append for gfx950: commit one segment's keys and values to the
// permanent, growing cache ("Tencent's Hy-Nomas Steers a 60-Second Video World
// ...", section "One World, Generated Segment by Segment").
//
// Source rows are token-major [T][H][128] (the projection's layout), the cache
// is head-major [H][cap][128] so that a head's keys are one contiguous run for
// the attention kernel's tile loads.  Pure copy, HBM-bound: each thread moves
// 16 bytes; a 16-thread group moves one (token, head) row of 256 bytes, so
// reads are fully coalesced along the token's H*128 elements and writes are
// 256-byte runs.
#include "kernels.h"

namespace nomas {
namespace {

__global__ __launch_bounds__(256) void kvcache_append_kernel(AppendParams p) {
  const uint16_t* src = blockIdx.y == 0 ? p.k_src : p.v_src;
  uint16_t* dst = blockIdx.y == 0 ? p.k_dst : p.v_dst;
  const int64_t total = (int64_t)p.tokens * p.heads * 16;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i & 15);
    const int64_t row = i >> 4;          // token * heads + head
    const int h = (int)(row % p.heads);
    const int64_t t = row / p.heads;
    const uint4 v = *reinterpret_cast<const uint4*>(src + t * p.src_stride + (int64_t)h * 128 + 8 * c);
    *reinterpret_cast<uint4*>(dst + ((int64_t)h * p.cap + p.dst_offset + t) * 128 + 8 * c) = v;
  }
}

}  // namespace

hipError_t launch_kvcache_append(const AppendParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.tokens * p.heads * 16;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  dim3 grid((unsigned)blocks, 2), block(256);
  hipLaunchKernelGGL(kvcache_append_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace nomas
