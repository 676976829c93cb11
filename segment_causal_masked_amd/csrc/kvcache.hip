// KV-cache append (bf16 and INT8) and INT8 expansion for gfx950: commit one
// segment's keys and values to the permanent, growing cache ("Tencent's Hy-Nomas Steers a 60-Second Video World
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

// fp32 holding a value with at most 8 significant bits -> its bf16 pattern
// (the truncation is exact there)
__device__ __forceinline__ uint16_t f2bf_exact(float x) { return (uint16_t)(__float_as_uint(x) >> 16); }

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

// INT8 rows ("Summary (Overview)", Inference: INT8 KV-cache quantization).
// A (head, token) row of 128 values x is stored as int8 codes
// q = round-half-even(x / 2^e) and one int8 exponent e, the smallest with
// max |x| <= 127 * 2^e (0 for a zero row, at least -127): q * 2^e is exact in
// bf16.  Sixteen lanes per row, eight values each; the row maximum by a
// 16-lane exchange.  frexp, ldexp and rint are exact, so the codes do not
// depend on any rounding choice.
__global__ __launch_bounds__(256) void kvcache_int8_append_kernel(Int8AppendParams p) {
  const bool is_v = blockIdx.y != 0;
  const uint16_t* src = is_v ? p.v_src : p.k_src;
  int8_t* codes = is_v ? p.v_codes : p.k_codes;
  int8_t* exps = is_v ? p.v_exp : p.k_exp;
  const int64_t total = (int64_t)p.tokens * p.heads * 16;
  // whole 16-lane groups stay together: total is a multiple of 16 and so is
  // the stride of the loop
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i & 15);
    const int64_t row = i >> 4;  // token * heads + head
    const int h = (int)(row % p.heads);
    const int64_t t = row / p.heads;
    const uint4 v = *reinterpret_cast<const uint4*>(src + t * p.src_stride + (int64_t)h * 128 + 8 * c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[2 * j] = __uint_as_float(w[j] << 16);
      x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(x[j]));
#pragma unroll
    for (int o = 8; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    int k;
    const float m = frexpf(amax, &k);  // amax = m 2^k, m in [0.5, 1)
    int e = k - 7;                     // amax / 2^e = 128 m in [64, 128)
    if (128.f * m > 127.f) ++e;
    if (amax == 0.f) e = 0;
    e = max(e, -127);
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int q = (int)rintf(ldexpf(x[j], -e));
      packed[j >> 2] |= (uint32_t)(q & 0xff) << (8 * (j & 3));
    }
    const int64_t dst_row = (int64_t)h * p.cap + p.dst_offset + t;
    *reinterpret_cast<uint2*>(codes + dst_row * 128 + 8 * c) = uint2{packed[0], packed[1]};
    if (c == 0) exps[dst_row] = (int8_t)e;
  }
}

// Rows [0, rows) of every head back to bf16 (exact): 16 lanes per row.
__global__ __launch_bounds__(256) void kvcache_int8_expand_kernel(Int8ExpandParams p) {
  const bool is_v = blockIdx.y != 0;
  const int8_t* codes = is_v ? p.v_codes : p.k_codes;
  const int8_t* exps = is_v ? p.v_exp : p.k_exp;
  uint16_t* dst = is_v ? p.v_dst : p.k_dst;
  const int64_t total = p.rows * p.heads * 16;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int c = (int)(i & 15);
    const int64_t row = i >> 4;  // head * rows + token: each head's rows are contiguous
    const int h = (int)(row / p.rows);
    const int64_t t = row - (int64_t)h * p.rows;
    const int64_t src_row = (int64_t)h * p.src_cap + t;
    const uint2 q = *reinterpret_cast<const uint2*>(codes + src_row * 128 + 8 * c);
    const int e = exps[src_row];
    const uint32_t b[2] = {q.x, q.y};
    uint32_t out[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int q0 = (int)(int8_t)(b[j >> 1] >> (16 * (j & 1)));
      const int q1 = (int)(int8_t)(b[j >> 1] >> (16 * (j & 1) + 8));
      out[j] = (uint32_t)f2bf_exact(ldexpf((float)q0, e)) | ((uint32_t)f2bf_exact(ldexpf((float)q1, e)) << 16);
    }
    *reinterpret_cast<uint4*>(dst + ((int64_t)h * p.dst_cap + t) * 128 + 8 * c) = uint4{out[0], out[1], out[2], out[3]};
  }
}

}  // namespace

hipError_t launch_kvcache_int8_append(const Int8AppendParams& p, hipStream_t stream) {
  const int64_t total = (int64_t)p.tokens * p.heads * 16;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(kvcache_int8_append_kernel, dim3((unsigned)blocks, 2), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_kvcache_int8_expand(const Int8ExpandParams& p, hipStream_t stream) {
  const int64_t total = p.rows * p.heads * 16;
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 16384) blocks = 16384;
  hipLaunchKernelGGL(kvcache_int8_expand_kernel, dim3((unsigned)blocks, 2), dim3(256), 0, stream, p);
  return hipGetLastError();
}

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
