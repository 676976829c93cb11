// Device helpers shared by the attention kernels (gfx950): bf16 MFMA operand
// types, the mask predicate on per-token descriptors, direct HBM -> LDS
// loads with explicit waits, and the swizzled LDS tile layout with its
// 8-wave K/V tile loader.
//
// LDS tile layout (R rows x 16 chunks of 16 bytes, R a multiple of 16; 64 for
// K / V tiles): chunk c of row r sits at
//   (c / 4) * (64 R) + r * 64 + 16 * ((c % 4) ^ ((r / 4) % 4)).
// Each 16-lane phase of the K reads (16 rows, one chunk) and each 32-lane
// phase of the V transpose reads (4 rows x 4 chunks x 8 bytes) covers all 64
// banks exactly once, and every per-step address is an immediate offset from
// two per-lane bases.  A 1 KB block (16 rows x one 4-chunk group) is filled
// by a single direct HBM -> LDS load (global_load_lds_dwordx4).
#pragma once

#include "kernels.h"

namespace nomas {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef const __attribute__((address_space(4))) int32_t* const_i32p;
typedef __attribute__((address_space(3))) i16x4* lds_i16x4p;

constexpr int D = 128;
constexpr int BK = 64;
constexpr int TILE_BYTES = BK * D * 2;  // 16 KB: one 64-row K or V tile

// MFMA output row i (of 32) -> key offset inside a 32-key block.
__device__ __forceinline__ int kmap(int i) {
  const int g = i >> 3, q = (i >> 2) & 1, r = i & 3;
  return 16 * (g >> 1) + 8 * q + 4 * (g & 1) + r;
}

// Branch-free (bitwise, not short-circuit), so that masking compiles to
// compares and selects on the score registers in place.
__device__ __forceinline__ bool visible(const QDescDev& q, int kseg, uint32_t kbits) {
  const bool in_range = (kseg >= q.lo) & (kseg <= q.seg);
  const bool tail_ok = (kseg == q.seg) & ((q.amask & kbits) != 0u);
  return in_range & ((kbits == 0u) | tail_ok);
}

__device__ __forceinline__ uint16_t f2bf(float x) {
  __bf16 b = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// 16-byte direct load HBM -> LDS (global_load_lds_dwordx4): lane i's 16 bytes
// land at lds + 16 * i.  Issued through inline asm so that the compiler does
// not track it: its alias analysis for in-flight LDS DMA is conservative and
// would drain every prefetch at the next LDS read or fence.  The instruction
// writes no VGPR (only LDS), so nothing the compiler sees can be overwritten
// late; completion of a stage is ensured explicitly with s_waitcnt vmcnt
// before the barrier that publishes it.  Waits the compiler inserts for its
// own loads stay correct (only stricter): vector memory ops complete in order.
__device__ __forceinline__ void dma16(const void* gsrc, const void* lds_dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)((const __attribute__((address_space(3))) char*)lds_dst));
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(m0) : "memory");
}

// The same load with a uniform base address in SGPRs and a 32-bit per-lane
// byte offset: one VGPR per lane instead of a 64-bit pointer, which matters
// in kernels at the edge of their register budget.  (No immediate offset:
// the instruction's offset field moves the LDS destination as well.)
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, const void* lds_dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)((const __attribute__((address_space(3))) char*)lds_dst));
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}

// LDS byte address of a __shared__ object.  Taken once, from the object
// itself, so that staging code carries 32-bit LDS addresses in SGPRs instead
// of 64-bit generic pointers (and their null checks) for every stage buffer.
__device__ __forceinline__ uint32_t lds_addr(const void* shared_obj) {
  return (uint32_t)(uintptr_t)((const __attribute__((address_space(3))) char*)shared_obj);
}

// dma16 / dma16_s with the LDS destination given as an LDS byte address.
__device__ __forceinline__ void dma16(const void* gsrc, uint32_t lds) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(m0) : "memory");
}
__device__ __forceinline__ void dma16_s(const void* sbase, uint32_t voff, uint32_t lds) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0) : "memory");
}

// Workgroup barrier ordering LDS accesses only (no wait on global memory).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt vmcnt(N) (expcnt, lgkmcnt untouched): N in [0, 63].
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Everything the tile loads need, copied out of the kernel arguments.
// Wave w fills LDS blocks (chunk group w / 4 + 2 i, rows 16 (w % 4) ..+15) of
// a tile for i = 0, 1.  Lane l fetches row 16 (w % 4) + l / 4 and chunk
// 4 (w / 4 + 2 i) + ((l % 4) ^ ((l / 16) % 4)): its offset inside a tile is
// constant up to the scalar 32 (w / 4 + 2 i).
struct LoadCtx {
  const uint16_t *k_cache_h, *v_cache_h;  // head h's rows in the cache
  const uint16_t *k_new_h, *v_new_h;      // head h's column in the new-token rows
  int64_t kv_stride;                      // new-token stride (elements)
  int32_t nk, n_cached;
  int32_t lane_row, lane_chunk;           // this lane's row / chunk inside a block
  uint32_t lane_cache, lane_new;          // byte offsets of (lane_row, lane_chunk) from a
                                          // block's first row (cache / new-token rows)
};

// dst: LDS byte address of the half-tile (K or V) buffer.
__device__ __forceinline__ void issue_half(const LoadCtx& c, const uint16_t* cache_h,
                                           const uint16_t* new_h, uint32_t dst, int kt, int w) {
  const int k0 = kt * BK;
  const int gq = w >> 2;
  const uint32_t d = dst + 4096u * gq + 1024u * (w & 3);
  // Whole blocks of cache or new-token rows: a uniform base (SGPRs) plus the
  // lane's loop-invariant byte offset, so no per-lane address arithmetic.
  if (k0 + BK <= c.n_cached) {
    const uint16_t* sb = cache_h + (int64_t)k0 * D + 32 * gq;
    dma16_s(sb, c.lane_cache, d);
    dma16_s(sb + 64, c.lane_cache, d + 8192);
  } else if (k0 >= c.n_cached && k0 + BK <= c.nk) {
    const uint16_t* sb = new_h + (int64_t)(k0 - c.n_cached) * c.kv_stride + 32 * gq;
    dma16_s(sb, c.lane_new, d);
    dma16_s(sb + 64, c.lane_new, d + 8192);
  } else {  // straddles the cache / new boundary or runs past the last key
    int key = k0 + c.lane_row;
    key = key < c.nk ? key : c.nk - 1;  // any valid row: masked later
    const uint16_t* src = (key < c.n_cached ? cache_h + (int64_t)key * D
                                            : new_h + (int64_t)(key - c.n_cached) * c.kv_stride) +
                          8 * c.lane_chunk + 32 * gq;
    dma16(src, d);
    dma16(src + 64, d + 8192);
  }
}

}  // namespace
}  // namespace nomas
