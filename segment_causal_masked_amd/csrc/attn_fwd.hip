// Forward kernel of action-aware causal attention for gfx950 (CDNA4).
//
// Computes O = softmax(scale * Q K^T + M) V with M = -inf on hidden pairs
// (the mask of "Summary (Overview)", Model Architecture: Segment-wise and
// Action-Aware Causal Attention), flash-style over the tile map: only the
// non-empty 64-key tiles of a 128-query tile are visited; FULL tiles run
// unmasked, PARTIAL (or ragged) tiles evaluate the per-token descriptors.
// Online softmax keeps a running max and sum per query in fp32, so the result
// equals the plain softmax up to rounding.
//
// Scheduling (persistent, stream-K style): the host cuts the (unit, key tile)
// iterations, unit = head * n_q_tiles + q_tile, into equal contiguous ranges,
// one per workgroup (one workgroup of four waves per CU).  A unit split between ranges is
// computed in pieces whose un-normalised (O, max, sum) go to a workspace and
// are merged by attn_fwd_combine_kernel.  Workgroup ids are remapped so that
// the workgroups of one XCD take consecutive ranges, i.e. the q-tiles of the
// same heads, which then share that XCD's L2 for their K/V.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, fp32 accumulate), per wave of
// 32 queries (4 waves per workgroup, 128 queries, one wave per SIMD so each
// wave has the whole register file for the software pipeline below):
//   S^T (64 keys x 32 queries) = K_tile * Q^T   -- K from LDS, Q in registers
//   O^T (128 dims x 32 queries) += V^T * P^T    -- V^T from LDS, P^T in regs
// One query per lane column: row max / row sum are in-lane over 32 keys plus
// one exchange between half-waves, and the rescale factor is a per-lane
// scalar.  Key rows of the S^T MFMA are permuted (kmap) so that each half-wave
// holds 8 consecutive keys per 16-key step, which is the B-operand layout of
// the P^T V^T product: P never leaves registers.  V^T operands come straight
// from the row-major V tile with the LDS transpose read (ds_read_b64_tr_b16).
//
// The reference max is only raised when a tile's max exceeds it by more than
// RESCALE_SLACK (log2 units); until then exp2 arguments stay <= RESCALE_SLACK,
// P <= 2^RESCALE_SLACK, and the O rescale (64 multiplies per lane) is skipped.
// O / l does not depend on the reference max, so this changes rounding only.
//
// Staging: K and V tiles are copied HBM -> LDS by direct 16-byte loads
// (global_load_lds_dwordx4), double buffered, one barrier per tile.  LDS rows
// are 256 bytes with the 16-byte chunks XOR-swizzled by swz(row) so that both
// the K reads (8 rows x 16 B per cycle) and the transpose reads of V (4 rows x
// 32 B per 16 lanes) hit distinct banks.
#include "kernels.h"

namespace nomas {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef const __attribute__((address_space(4))) int32_t* const_i32p;
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int D = 128;
constexpr int BQ = 128;
constexpr int BK = 64;
constexpr int NWAVES = 4;    // one wave per SIMD, one workgroup per CU
constexpr int NQB = 1;       // 32-query blocks per wave
constexpr int NTHREADS = 64 * NWAVES;
constexpr int TILE_BYTES = BK * D * 2;  // 16 KB: one K or V tile
constexpr float RESCALE_SLACK = 8.0f;
// per partial piece: for each of the 128 threads and 2 query blocks, 64 O + m + l
constexpr int SLOT_FLOATS = NTHREADS * NQB * 66;

// MFMA output row i (of 32) -> key offset inside a 32-key block.
__device__ __forceinline__ int kmap(int i) {
  const int g = i >> 3, q = (i >> 2) & 1, r = i & 3;
  return 16 * (g >> 1) + 8 * q + 4 * (g & 1) + r;
}

// 16-byte chunk swizzle of LDS row `row` (see the header comment).
__device__ __forceinline__ int swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }

__device__ __forceinline__ bool visible(const QDescDev& q, int kseg, uint32_t kbits) {
  return kseg >= q.lo && kseg <= q.seg &&
         (kbits == 0u || (kseg == q.seg && (q.amask & kbits) != 0u));
}

__device__ __forceinline__ uint16_t f2bf(float x) {
  __bf16 b = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// 16-byte direct load HBM -> LDS (global_load_lds_dwordx4): each lane's 16
// bytes land at lds + 16 * lane.  Issued through inline asm so that the
// compiler does not track it: its alias analysis for in-flight LDS DMA is
// conservative and would drain every prefetch at the next LDS read or fence.
// The instruction writes no VGPR (only LDS), so nothing the compiler sees can
// be overwritten late; completion of a stage is ensured explicitly with
// s_waitcnt vmcnt(N) before the barrier that publishes it.  Waits the
// compiler inserts for its own loads stay correct (only stricter), because
// vector memory operations complete in issue order.
__device__ __forceinline__ void dma16(const void* gsrc, const void* lds_dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane(
      (unsigned)(uintptr_t)((const __attribute__((address_space(3))) char*)lds_dst));
  asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gsrc), "{m0}"(m0) : "memory");
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

// Everything the tile loads need, copied out of the kernel arguments so that
// it lives in registers.
struct LoadCtx {
  const uint16_t *k_cache_h, *v_cache_h;  // head h's rows in the cache
  const uint16_t *k_new_h, *v_new_h;      // head h's column in the new-token rows
  int64_t kv_stride;                      // new-token stride (elements)
  int32_t nk, n_cached;
  int32_t lane_cache, lane_new;           // per-lane element offsets (row r0 + chunk)
};

// Direct loads of one 16 KB tile (K or V) of key tile kt: wave w issues 4
// loads, load i covering rows 16 i + 4 w .. +3 (1 KB of LDS at block 4 i + w).
// Every row this lane fetches has the same chunk swizzle (row & 3 = lane / 16,
// (row >> 2) & 3 = w), so in the fast path (tile in one source, not ragged)
// an address is a scalar tile base plus the lane's constant offset.
__device__ __forceinline__ void issue_half(const LoadCtx& c, const uint16_t* cache_h,
                                           const uint16_t* new_h, char* dst, int kt, int w,
                                           int lane) {
  const int k0 = kt * BK;
  static_assert(NWAVES == 4, "lane-constant swizzle needs 4 waves");
  if (k0 + BK <= c.n_cached) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma16(cache_h + (int64_t)(k0 + 16 * i) * D + c.lane_cache, dst + (4 * i + w) * 1024);
  } else if (k0 >= c.n_cached && k0 + BK <= c.nk) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      dma16(new_h + (int64_t)(k0 - c.n_cached + 16 * i) * c.kv_stride + c.lane_new,
            dst + (4 * i + w) * 1024);
  } else {  // straddles the cache / new boundary or runs past the last key
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 16 * i + 4 * w + (lane >> 4);
      const int ch = (lane & 15) ^ swz(row);
      int key = k0 + row;
      key = key < c.nk ? key : c.nk - 1;  // any valid row: masked later
      const uint16_t* src = key < c.n_cached ? cache_h + (int64_t)key * D + 8 * ch
                                             : new_h + (int64_t)(key - c.n_cached) * c.kv_stride + 8 * ch;
      dma16(src, dst + (4 * i + w) * 1024);
    }
  }
}

struct WaveState {
  bf16x8 qf[NQB][8];    // Q fragments: query jq of block qi, dims [16 s + 8 hh, +8)
  f32x16 acc[NQB][4];   // O^T, dims 32 db + 8 (ri / 4) + 4 hh + ri % 4
  float m_run[NQB];     // reference max, log2 domain (same in both half-waves)
  float l_run[NQB];     // this half-wave's share of the running sum
  QDescDev qd[NQB];
  int k_off[2], k_swz[2];
};

// S^T = K Q^T for one 64-key tile and both query blocks (independent of the
// softmax in flight): each K fragment feeds two MFMAs.
__device__ __forceinline__ void qk_tile(const WaveState& ws, const char* kbase, int hh,
                                        f32x16 (*s)[2]) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int qi = 0; qi < NQB; ++qi) s[qi][kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int c = (2 * ks + hh) ^ ws.k_swz[kb];
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kbase + ws.k_off[kb] + 16 * c);
#pragma unroll
      for (int qi = 0; qi < NQB; ++qi)
        s[qi][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, ws.qf[qi][ks], s[qi][kb], 0, 0, 0);
    }
  }
}

// Mask and online softmax of one query block's S^T (in place -> P^T bf16).
__device__ __forceinline__ void softmax_block(WaveState& ws, int qi, f32x16* s, bf16x8* pf,
                                              const KDescDev* kd, bool masked, float scale_log2,
                                              int hh) {
  // register ri of block kb holds key 32 kb + 16 (ri / 8) + 8 hh + ri % 8
  if (masked) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ri = 0; ri < 16; ++ri) {
        const KDescDev d = kd[32 * kb + 16 * (ri >> 3) + 8 * hh + (ri & 7)];
        const bool vis = visible(ws.qd[qi], d.seg, d.bits);
        s[kb][ri] = vis ? s[kb][ri] : -INFINITY;
      }
  }
  // this half-wave's max over its 32 keys (tree)
  float t[11];
#pragma unroll
  for (int j = 0; j < 5; ++j) t[j] = fmaxf(fmaxf(s[0][3 * j], s[0][3 * j + 1]), s[0][3 * j + 2]);
#pragma unroll
  for (int j = 0; j < 5; ++j) t[5 + j] = fmaxf(fmaxf(s[1][3 * j], s[1][3 * j + 1]), s[1][3 * j + 2]);
  t[10] = fmaxf(s[0][15], s[1][15]);
  float mx = fmaxf(fmaxf(fmaxf(t[0], t[1]), fmaxf(t[2], t[3])),
                   fmaxf(fmaxf(t[4], t[5]), fmaxf(t[6], t[7])));
  mx = fmaxf(mx, fmaxf(fmaxf(t[8], t[9]), t[10]));
  const float m_half = mx * scale_log2;
  // Raise the reference max only when a row's tile max exceeds it by more than
  // RESCALE_SLACK; the decision is per row (both halves agree after the
  // exchange), the branch only skips work no row of the wave needs.
  if (__builtin_amdgcn_ballot_w64(m_half > ws.m_run[qi] + RESCALE_SLACK)) {
    const float m_row = fmaxf(m_half, __shfl_xor(m_half, 32));
    const bool raise = m_row > ws.m_run[qi] + RESCALE_SLACK;
    const float m_new = raise ? m_row : ws.m_run[qi];
    const float alpha = __builtin_amdgcn_exp2f(ws.m_run[qi] - (m_new == -INFINITY ? 0.f : m_new));
    ws.m_run[qi] = m_new;
    ws.l_run[qi] *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int ri = 0; ri < 16; ++ri) ws.acc[qi][db][ri] *= alpha;
  }
  const float m_use = ws.m_run[qi] == -INFINITY ? 0.f : ws.m_run[qi];
  float lsum[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      bf16x8 v;
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const float pe = __builtin_amdgcn_exp2f(
            __builtin_fmaf(s[kb][8 * half + e8], scale_log2, -m_use));
        lsum[e8 & 3] += pe;
        v[e8] = (__bf16)pe;
      }
      pf[2 * kb + half] = v;
    }
  ws.l_run[qi] += (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
}

// O^T += V^T P^T for both query blocks: each V^T fragment feeds two MFMAs.
__device__ __forceinline__ void pv_tile(WaveState& ws, const bf16x8 (*pf)[4], const char* vbase,
                                        int hh, int lane) {
  const int g16 = lane >> 4, i16 = lane & 15;
  const int tr_j = i16 >> 2, tr_c4 = i16 & 3;  // transpose read: row j, 4-dim chunk c4
#pragma unroll
  for (int step = 0; step < 4; ++step) {
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      // keys 16 step + 8 hh + {0..3 | 4..7}, dims 32 db + 16 (g16 & 1) + 4 tr_c4 + {0..3}
      const int c = 4 * db + 2 * (g16 & 1) + (tr_c4 >> 1);
      const int row0 = 16 * step + 8 * hh + tr_j;
      const int row1 = row0 + 4;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vbase + row0 * 256 + 16 * (c ^ swz(row0)) + 8 * (tr_c4 & 1)));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) i16x4*)(vbase + row1 * 256 + 16 * (c ^ swz(row1)) + 8 * (tr_c4 & 1)));
      const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int qi = 0; qi < NQB; ++qi)
        ws.acc[qi][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qi][step], ws.acc[qi][db], 0, 0, 0);
    }
  }
}

// Normalise and store one lane's query row (O in bf16, LSE in natural log);
// dims 32 db + 8 g + 4 hh + {0..3} for the blocks db in [db0, db0 + ndb).
__device__ __forceinline__ void store_row(const FwdParams& p, const f32x16* acc, int db0, int ndb,
                                          float m_run, float l_tot, int h, int qrow, int hh,
                                          bool write_lse) {
  if (qrow >= p.nq) return;
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* dst = p.o + (int64_t)qrow * p.o_stride + (int64_t)h * D;
  for (int j = 0; j < ndb; ++j) {
    const int db = db0 + j;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * db + 8 * g + 4 * hh;
      uint2 pk;
      pk.x = (uint32_t)f2bf(acc[j][4 * g + 0] * inv) | ((uint32_t)f2bf(acc[j][4 * g + 1] * inv) << 16);
      pk.y = (uint32_t)f2bf(acc[j][4 * g + 2] * inv) | ((uint32_t)f2bf(acc[j][4 * g + 3] * inv) << 16);
      *reinterpret_cast<uint2*>(dst + d0) = pk;
    }
  }
  if (p.lse && write_lse && hh == 0)
    p.lse[(int64_t)h * p.nq + qrow] =
        l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
}

// Software pipeline over the tiles of a piece.  Iteration t computes S^T of
// tile t on the MFMA units while the softmax of tile t - 1 runs on the VALU,
// then O^T += V^T P^T of tile t - 1; so the stage buffer of iteration t holds
// K of tile t and V (+ key descriptors) of tile t - 1.  NSTAGE buffers let the
// loads of iteration t + NSTAGE - 1 be issued at iteration t, hiding the
// latency of the HBM / last-level-cache reads behind NSTAGE - 1 iterations.
// Every iteration issues the same loads (missing tiles are replaced by a valid
// tile that is never read), so the number of loads still in flight after
// iteration t's is known exactly and the wait can be precise.
constexpr int NSTAGE = 4;
constexpr int LOADS_PER_ITER = 8;  // 4 (K) + 4 (V) per wave; wave 0 adds 1 (descriptors)

__global__ __launch_bounds__(NTHREADS, 1) void attn_fwd_kernel(FwdParams p) {
  // Stage buffers as distinct LDS objects, so that reads of one are known not
  // to alias the direct loads in flight into the others.
  __shared__ __attribute__((aligned(1024))) char sbuf0[2 * TILE_BYTES];  // K | V
  __shared__ __attribute__((aligned(1024))) char sbuf1[2 * TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sbuf2[2 * TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sbuf3[2 * TILE_BYTES];
  __shared__ __attribute__((aligned(16))) KDescDev skd0[BK];
  __shared__ __attribute__((aligned(16))) KDescDev skd1[BK];
  __shared__ __attribute__((aligned(16))) KDescDev skd2[BK];
  __shared__ __attribute__((aligned(16))) KDescDev skd3[BK];
  static_assert(NSTAGE == 4, "the unrolled loop below names four stage buffers");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int jq = lane & 31;   // query column of this lane
  const int hh = lane >> 5;   // half-wave

  // logical workgroup: XCD-major (dispatch places workgroup b on XCD b % 8)
  const int G = (int)gridDim.x;
  const int g = (G & 7) ? (int)blockIdx.x : (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3);

  const const_i32p csr_ptr = (const_i32p)p.csr_ptr;
  const const_i32p csr_idx = (const_i32p)p.csr_idx;
  const const_i32p pieces = (const_i32p)p.pieces;  // 4 ints per piece
  const int pc0 = ((const_i32p)p.wg_ptr)[g], pc1 = ((const_i32p)p.wg_ptr)[g + 1];
  const float scale_log2 = p.scale_log2;

  WaveState ws;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = 32 * kb + kmap(jq);
    ws.k_off[kb] = row * 256;
    ws.k_swz[kb] = swz(row);
  }
  LoadCtx lc;
  lc.kv_stride = p.kv_stride;
  lc.nk = p.nk;
  lc.n_cached = p.n_cached;
  {
    const int r0 = 4 * w + (lane >> 4);     // rows 16 i + r0: swz(row) = swz(r0)
    const int ch = (lane & 15) ^ swz(r0);
    lc.lane_cache = r0 * D + 8 * ch;
    lc.lane_new = (int)(r0 * p.kv_stride) + 8 * ch;
  }

  for (int pc = pc0; pc < pc1; ++pc) {
    const int unit = pieces[4 * pc];
    const int e_begin = pieces[4 * pc + 1], e_end = pieces[4 * pc + 2], slot = pieces[4 * pc + 3];
    const int h = unit / p.nqt;
    const int qt = unit - h * p.nqt;
    const const_i32p ent = csr_idx + csr_ptr[qt] + e_begin;
    const int n_ent = e_end - e_begin;
    const int last = n_ent - 1;
    lc.k_cache_h = p.k_cache + (int64_t)h * p.cache_cap * D;
    lc.v_cache_h = p.v_cache + (int64_t)h * p.cache_cap * D;
    lc.k_new_h = p.k_new + (int64_t)h * D;
    lc.v_new_h = p.v_new + (int64_t)h * D;

#pragma unroll
    for (int qi = 0; qi < NQB; ++qi) {
      const int qrow = qt * BQ + (NQB * w + qi) * 32 + jq;
      if (qrow < p.nq) {
        const uint16_t* src = p.q + (int64_t)qrow * p.q_stride + (int64_t)h * D + 8 * hh;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) ws.qf[qi][s8] = *reinterpret_cast<const bf16x8*>(src + 16 * s8);
      } else {
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) ws.qf[qi][s8] = bf16x8{};
      }
      ws.qd[qi] = p.qdesc[qrow];  // padded to whole tiles
#pragma unroll
      for (int db = 0; db < 4; ++db) ws.acc[qi][db] = f32x16{};
      ws.m_run[qi] = -INFINITY;
      ws.l_run[qi] = 0.f;
    }

    // Q and the query descriptors must have arrived before the tile loop:
    // otherwise the compiler's own waits for them, placed inside the loop,
    // would also drain the tile prefetches issued below.
    wait_vm_all();

    // loads of iteration i into stage buffer i % NSTAGE: K_i and V_{i-1}
    // (K_{n-1} stands in for K_n, V_0 for V_{-1})
    auto issue_iter = [&](int i, char* buf, KDescDev* kd) {
      const int kt_k = ent[i < n_ent ? i : last] >> 1;
      const int kt_v = ent[i > 0 ? i - 1 : 0] >> 1;
      issue_half(lc, lc.k_cache_h, lc.k_new_h, buf, kt_k, w, lane);
      issue_half(lc, lc.v_cache_h, lc.v_new_h, buf + TILE_BYTES, kt_v, w, lane);
      if (w == 0 && lane < 32) dma16(p.kdesc + kt_v * BK + 2 * lane, kd);
    };
    if (n_ent > 0) {
      issue_iter(0, sbuf0, skd0);
      if (1 <= n_ent) issue_iter(1, sbuf1, skd1);
      if (2 <= n_ent) issue_iter(2, sbuf2, skd2);
    }

    f32x16 sa[NQB][2], sb[NQB][2];  // S^T of the tile in flight / the one being consumed
    // cbuf/ckd: this iteration's stage; nbuf/nkd: the stage refilled for
    // iteration t + NSTAGE - 1 (the one iteration t - 1 just released)
    auto body = [&](int t, char* cbuf, KDescDev* ckd, char* nbuf, KDescDev* nkd,
                    f32x16 (*s_new)[2], f32x16 (*s_old)[2]) {
      // own loads of iteration t complete: those of t+1 .. min(t+NSTAGE-2, n) may fly
      const int ahead = (n_ent < t + NSTAGE - 2 ? n_ent : t + NSTAGE - 2) - t;
      if (w == 0) {
        if (ahead >= 2) wait_vm<2 * (LOADS_PER_ITER + 1)>();
        else if (ahead == 1) wait_vm<LOADS_PER_ITER + 1>();
        else wait_vm<0>();
      } else {
        if (ahead >= 2) wait_vm<2 * LOADS_PER_ITER>();
        else if (ahead == 1) wait_vm<LOADS_PER_ITER>();
        else wait_vm<0>();
      }
      lds_barrier();  // iteration t's stage landed for all waves; t-1 is done with its buffer
      if (t + NSTAGE - 1 <= n_ent) issue_iter(t + NSTAGE - 1, nbuf, nkd);
      if (t < n_ent) qk_tile(ws, cbuf, hh, s_new);
      if (t > 0) {
        bf16x8 pf[NQB][4];
        const bool masked = ent[t - 1] & 1;
#pragma unroll
        for (int qi = 0; qi < NQB; ++qi)
          softmax_block(ws, qi, s_old[qi], pf[qi], ckd, masked, scale_log2, hh);
        pv_tile(ws, pf, cbuf + TILE_BYTES, hh, lane);
      }
    };
    for (int t = 0; t <= n_ent; t += NSTAGE) {
      body(t, sbuf0, skd0, sbuf3, skd3, sa, sb);
      if (t + 1 <= n_ent) body(t + 1, sbuf1, skd1, sbuf0, skd0, sb, sa);
      if (t + 2 <= n_ent) body(t + 2, sbuf2, skd2, sbuf1, skd1, sa, sb);
      if (t + 3 <= n_ent) body(t + 3, sbuf3, skd3, sbuf2, skd2, sb, sa);
    }

#pragma unroll
    for (int qi = 0; qi < NQB; ++qi) {
      const int qrow = qt * BQ + (NQB * w + qi) * 32 + jq;
      if (slot < 0) {
        const float l_tot = ws.l_run[qi] + __shfl_xor(ws.l_run[qi], 32);
        store_row(p, ws.acc[qi], 0, 4, ws.m_run[qi], l_tot, h, qrow, hh, true);
      } else {  // partial piece: un-normalised state, thread-native layout
        float* dst = p.partial + (int64_t)slot * SLOT_FLOATS + qi * 66 * NTHREADS + tid;
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int ri = 0; ri < 16; ++ri) dst[(16 * db + ri) * NTHREADS] = ws.acc[qi][db][ri];
        dst[64 * NTHREADS] = ws.m_run[qi];
        dst[65 * NTHREADS] = ws.l_run[qi];
      }
    }
    wait_vm_all();    // stores and stray loads retired before the next piece's accounting
    __syncthreads();  // the stage buffers are reused by the next piece
  }
}

// Merge the pieces of split units: O = sum_k 2^(m_k - m) O_k / sum_k 2^(m_k - m) l_k.
// Workgroup (item, db) handles dims 32 db .. 32 db + 31 of one split unit's
// 128 rows; thread T covers query block T / 64 (= 2 * wave + qi of the
// forward) and lane T % 64.
__global__ __launch_bounds__(256) void attn_fwd_combine_kernel(FwdParams p) {
  const const_i32p cmb = (const_i32p)p.combine + 4 * (blockIdx.x >> 2);
  const int db = blockIdx.x & 3;
  const int unit = cmb[0], first = cmb[1], n = cmb[2];
  const int h = unit / p.nqt;
  const int qt = unit - h * p.nqt;
  const int T = threadIdx.x;
  const int vb = T >> 6, lane = T & 63;
  const int wave = vb / NQB, qi = vb % NQB;
  const int qrow = qt * BQ + vb * 32 + (lane & 31);
  const int hh = lane >> 5;
  const float* base = p.partial + (int64_t)first * SLOT_FLOATS + qi * 66 * NTHREADS + wave * 64 + lane;
  float m = -INFINITY;
  for (int k = 0; k < n; ++k) m = fmaxf(m, base[(int64_t)k * SLOT_FLOATS + 64 * NTHREADS]);
  const float mu = m == -INFINITY ? 0.f : m;
  f32x16 acc[1] = {f32x16{}};
  float l = 0.f;
  for (int k = 0; k < n; ++k) {
    const float* src = base + (int64_t)k * SLOT_FLOATS;
    const float a = __builtin_amdgcn_exp2f(src[64 * NTHREADS] - mu);
    l += a * src[65 * NTHREADS];
#pragma unroll
    for (int ri = 0; ri < 16; ++ri) acc[0][ri] += a * src[(16 * db + ri) * NTHREADS];
  }
  const float l_tot = l + __shfl_xor(l, 32);
  store_row(p, acc, db, 1, m, l_tot, h, qrow, hh, db == 0);
}

}  // namespace

size_t attn_fwd_slot_bytes() { return (size_t)SLOT_FLOATS * sizeof(float); }
int attn_fwd_groups_per_cu() { return 1; }

hipError_t launch_attn_fwd(const FwdParams& p, hipStream_t stream) {
  if (p.nq == 0) return hipSuccess;
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)p.groups), dim3(NTHREADS), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_combine == 0) return e;
  hipLaunchKernelGGL(attn_fwd_combine_kernel, dim3((unsigned)(4 * p.n_combine)), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace nomas
