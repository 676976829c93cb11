// Backward kernels of action-aware causal attention for gfx950 (CDNA4).
//
// Gradients of O = softmax(scale Q K^T + M) V (M = -inf on pairs the
// segment-causal / action-window mask hides; "Model Architecture",
// Segment-wise and Action-Aware Causal Attention) for an upstream dO, with P
// recomputed from the forward's log-sum-exp:
//   P = exp(scale S - lse),  dV = P^T dO,  dP = dO V^T,
//   delta = rowsum(dO * O),  dS = P * (dP - delta),
//   dQ = scale dS K,  dK = scale dS^T Q.
// Both gradient kernels form P the same way, from the scores of Q and K as
// given (bf16 products, fp32 accumulation) scaled by scale * log2(e) in fp32:
// P = exp2(s * scale * log2(e) - lse * log2(e)).  The forward rounds
// Q * scale * log2(e) to bf16 before its products, so its lse differs from
// the exact one by a softmax-weighted mean of those rounding shifts; the rows
// of this P then sum to exp(-(that difference)) instead of 1, a relative
// error bounded per row by the forward's LSE bound, and smaller than forming
// P from the forward's rounded scores would leave against exact gradients.
// Three launches on one stream:
//   1. bwd_rowstats_kernel: -delta and -lse * log2(e) per (head, query);
//   2. bwd_dkdv_kernel: one workgroup per pair of 64-key tiles of a head
//      (eight waves, two per SIMD: four key groups of 32 keys x two halves of
//      each q-tile), looping over the q-tiles that see those keys (the union
//      of the two key tiles' column lists); 128-query tiles of Q, dO and the
//      row statistics are staged in LDS, double buffered; dK and dV
//      accumulate in registers and the two halves are summed at the end.
//      The grid has 1/16 more workgroups than units; each claims one unit
//      from the work queues below and the surplus ones find none and exit
//      (a loop over claimed units would hold more registers than the 256
//      this kernel already uses, and it measured slower);
//   3. bwd_dq_kernel: one workgroup per pair of 128-query tiles (eight waves,
//      32 queries each) looping over the forward's key-tile lists, with K / V
//      tiles staged as in the forward; dQ accumulates in registers.  One
//      persistent workgroup per CU loops over units claimed from the work
//      queues.
// Only FULL / PARTIAL tiles are visited and the per-element mask is applied on
// PARTIAL (or ragged) tiles only, as in the forward.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, fp32 accumulate):
//   dK/dV wave (32 keys), per 32-query block b of a q-tile:
//     S  (32 q x 32 k) = Q_b K^T     A: Q rows from LDS, B: K in registers
//     dP (32 q x 32 k) = dO_b V^T    A: dO rows from LDS, B: V in registers
//     dV^T (128 x 32 k) += dO_b^T P  A: dO^T (LDS transpose read), B: P
//     dK^T (128 x 32 k) += Q_b^T dS  A: Q^T (LDS transpose read), B: dS
//   The query rows of the first two products are permuted (kmap) so that P
//   and dS come out of the accumulators already in B-operand order.
//   dQ wave (32 queries), per 64-key tile:
//     S^T = K Q^T, dP^T = V dO^T     A: K / V rows from LDS, B: Q / dO regs
//     dQ^T (128 x 32 q) += K^T dS^T  A: K^T (LDS transpose read), B: dS^T
// Both reuse the forward's swizzled LDS tile layout (tile_common.h); the
// 128-row Q / dO tiles of the dK/dV kernel use the same layout with R = 128.
#include "tile_common.h"

namespace nomas {
namespace {

constexpr float LOG2E = 1.4426950408889634f;

// Work queues of the dK/dV and dQ kernels.  Workgroup b is dispatched to XCD
// b % 8; the n_units units form n_q queues of consecutive units
// ([q n / n_q, (q + 1) n / n_q)), one per XCD when the grid is a multiple of
// 8.  A workgroup takes units from its own XCD's queue, so that each XCD works
// through neighbouring tiles of one head, whose Q / dO or K / V tiles then
// meet in its L2, and once that queue is drained from the others in turn:
// the XCDs do not run at quite the same speed, and a fixed share per XCD
// would leave the faster ones idle at the end.  Thread 0 claims (one atomic
// add on the queue's counter; the counters are zeroed per call by the
// row-statistics kernel) and broadcasts the unit through LDS; -1 when every
// queue is drained.  `tried` (thread 0's) counts the queues found empty.  A
// loop of claims alternates between two slots: a unit without entries has no
// barrier of its own, so a wave may still be about to read one claim's slot
// when thread 0 writes the next claim; the claim after that waits at the
// barrier for every wave.
__device__ __forceinline__ int claim_unit(uint32_t* ctr, int n_units, int& tried, int* slot) {
  const int n_q = (gridDim.x & 7) ? 1 : 8;
  if (threadIdx.x == 0) {
    const int own = (int)(blockIdx.x & (unsigned)(n_q - 1));
    int got = -1;
    while (tried < n_q) {
      const int q = (own + tried) & (n_q - 1);
      const int b = (int)(((int64_t)q * n_units) / n_q), e = (int)(((int64_t)(q + 1) * n_units) / n_q);
      const int i = (int)atomicAdd(ctr + q, 1u);
      if (b + i < e) {
        got = b + i;
        break;
      }
      ++tried;
    }
    *slot = got;
  }
  lds_barrier();
  return __builtin_amdgcn_readfirstlane(*slot);
}

// ---------------------------------------------------------------------------
// 1. row statistics
// ---------------------------------------------------------------------------

// 16 lanes per (head, query row) over rows 0 .. nqt * 128 - 1; rows past nq
// (and rows that see no key, lse = -inf) get delta = 0 and nlse2 = 0: they are
// masked wherever they occur, so only finiteness matters there.
__global__ __launch_bounds__(256) void bwd_rowstats_kernel(BwdParams p) {
  const int64_t rows = (int64_t)p.nqt * 128;
  const int64_t item = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 4;
  const int sub = threadIdx.x & 15;
  if (blockIdx.x == 0 && threadIdx.x < 16) p.claim[threadIdx.x] = 0u;  // the queues start empty-handed
  if (item >= rows * p.heads) return;  // whole 16-lane groups leave together
  const int h = (int)(item / rows);
  const int i = (int)(item - (int64_t)h * rows);
  float acc = 0.f;
  if (i < p.nq) {
    const int64_t off = (int64_t)i * p.q_stride + (int64_t)h * D + 8 * sub;
    const uint4 a = *reinterpret_cast<const uint4*>(p.o + off);
    const uint4 b = *reinterpret_cast<const uint4*>(p.d_o + off);
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc += __uint_as_float(av[j] << 16) * __uint_as_float(bv[j] << 16);
      acc += __uint_as_float(av[j] & 0xffff0000u) * __uint_as_float(bv[j] & 0xffff0000u);
    }
  }
  acc += __shfl_xor(acc, 8);
  acc += __shfl_xor(acc, 4);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 1);
  if (sub == 0) {
    p.ndelta[item] = -acc;
    const float l = i < p.nq ? p.lse[(int64_t)h * p.nq + i] : -INFINITY;
    p.nlse2[item] = l == -INFINITY ? 0.f : -l * LOG2E;
  }
}

// ---------------------------------------------------------------------------
// 2. dK, dV
// ---------------------------------------------------------------------------

constexpr int KV_WAVES = 8;
constexpr int KV_THREADS = 64 * KV_WAVES;
constexpr int QT_ROWS = 128;
constexpr int QTILE_BYTES = QT_ROWS * D * 2;         // 32 KB: a 128-row Q or dO tile
constexpr int GRP128 = QT_ROWS * 64;                 // chunk-group stride of such a tile
constexpr int STAT_OFF = 2 * QTILE_BYTES;            // -lse2[128] | -delta[128]
constexpr int QD_OFF = STAT_OFF + 2 * QT_ROWS * 4;   // qdesc[128]
constexpr int KV_STAGE_BYTES = QD_OFF + QT_ROWS * 16;
static_assert(KV_STAGE_BYTES >= 4 * 64 * 64 * 4, "a stage holds one dV or dK half for the final sum");

// Stage q-tile qt of head h: Q and dO rows (rows past nq read row nq - 1:
// masked), -lse2 / delta, query descriptors.  Wave w fills row group w of both
// tiles (4 + 4 loads); wave 0 also the statistics, wave 1 the descriptors.
__device__ __forceinline__ void kv_issue_stage(const BwdParams& p, int h, int qt, char* stg,
                                               int w, int lane) {
  const int qt0 = __builtin_amdgcn_readfirstlane(qt * QT_ROWS);
  // statistics and descriptors first: a value the compiler reloads from
  // scratch here then waits only for loads that have already landed, not for
  // the Q / dO rows of this stage
  const int64_t srow = (int64_t)h * p.nqt * QT_ROWS + qt0;
  if (w == 0) {  // lanes 0..31: -lse2, lanes 32..63: -delta (each 32 x 16 B)
    if (lane < 32) dma16_s(p.nlse2 + srow, 16u * lane, stg + STAT_OFF);
    else dma16_s(p.ndelta + srow, 16u * (lane - 32), stg + STAT_OFF);
  } else if (w == 1) {
    const QDescDev* src = p.qdesc + qt0;
    dma16_s(src, 16u * lane, stg + QD_OFF);
    dma16_s(src + 64, 16u * lane, stg + QD_OFF + 1024);
  }
  // uniform row base (the q-tile's first row, head h) in SGPRs plus a 32-bit
  // per-lane byte offset: row 16 w + lane / 4 of the tile (clamped to nq - 1),
  // chunk (lane % 4) ^ ((lane / 16) % 4) of each 4-chunk group
  const int64_t base = (int64_t)qt0 * p.q_stride + (int64_t)h * D;
  const int r = min(16 * w + (lane >> 2), p.nq - 1 - qt0);
  // (the lane's chunk is recomputed here from a lane id the compiler cannot
  // hoist: kept across the loop it is one more value to spill, and its
  // reload from scratch would wait for the loads just issued)
  int ln;
  asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(ln));
  const uint32_t voff = (uint32_t)(r * (int)p.q_stride + 8 * ((ln & 3) ^ ((ln >> 4) & 3))) * 2u;
  const uint16_t* qb = p.q + base;
  const uint16_t* ob = p.d_o + base;
#pragma unroll
  for (int cg = 0; cg < 4; ++cg) {  // chunk group cg: 32 elements further along the row
    dma16_s(qb + 32 * cg, voff, stg + cg * GRP128 + w * 1024);
    dma16_s(ob + 32 * cg, voff, stg + QTILE_BYTES + cg * GRP128 + w * 1024);
  }
}

struct KvWave {
  bf16x8 kf[8];   // K row of this lane's key, dims [16 s + 8 hh, +8)
  bf16x8 vf[8];   // V row, same layout
  f32x16 dv[4];   // dV^T, dims 32 db + 8 (ri / 4) + 4 hh + ri % 4
  f32x16 dk[4];   // dK^T (unscaled)
  int kseg;
  uint32_t kbits;
};

// Visibility of this wave's 64 queries of the staged q-tile (query blocks
// 2 qh, 2 qh + 1) for this lane's key, in score-register order: bit 16 bb + i
// <-> query 32 (2 qh + bb) + 16 (i / 8) + 8 hh + i % 8.  PARTIAL tiles only.
__device__ __forceinline__ uint32_t kv_vis_bits(const char* stg, int kseg, uint32_t kbits, int hh,
                                                int qh) {
  uint32_t v = 0;
#pragma unroll 4
  for (int j = 0; j < 32; ++j) {
    const int ql = 32 * (2 * qh + (j >> 4)) + 16 * ((j >> 3) & 1) + 8 * hh + (j & 7);
    const QDescDev qd = *reinterpret_cast<const QDescDev*>(stg + QD_OFF + 16 * ql);
    v |= (uint32_t)visible(qd, kseg, kbits) << j;
  }
  return v;
}

// This wave's half of a staged q-tile (query blocks 2 qh, 2 qh + 1) against
// its 32 keys; vis = all ones on FULL tiles.
// bases: this lane's {row-read base for even / odd 16-dim steps (Q / dO rows),
// transpose-read base for rows +0 / +4}, kept in LDS rather than registers
// (the wave is at its register limit; a spilled base would be reloaded from
// scratch memory, and that wait would also drain the next stage's loads).
__device__ __forceinline__ void kv_qtile(KvWave& st, const char* stg, const int4* bases, bool masked,
                                         uint32_t vis, float scale_log2, int hh, int qh) {
  const char* qtile = stg;
  const char* dotile = stg + QTILE_BYTES;
  const int4 lb = *bases;
  const int rbase[2] = {lb.x, lb.y}, tbase[2] = {lb.z, lb.w};
#pragma unroll
  for (int bb = 0; bb < 2; ++bb) {
    const int b = 2 * qh + bb;
    // register i holds query 32 b + 16 (i / 8) + 8 hh + i % 8.  The score
    // chain starts from zero (no register set-up: the first product takes a
    // constant accumulator); hidden pairs get -inf after it, so P = 0
    // (uniform branch: FULL tiles skip the selects).  Q and K enter unscaled
    // and the fp32 score is scaled once (the P of the dQ kernel, formed the
    // same way).  The dP chain starts from -delta of those queries and ends
    // at dP - delta.
    f32x16 s = f32x16{}, dp;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int q0 = 32 * b + 16 * (g >> 1) + 8 * hh + 4 * (g & 1);
      const float4 nd = *reinterpret_cast<const float4*>(stg + STAT_OFF + 512 + 4 * q0);
      dp[4 * g] = nd.x;
      dp[4 * g + 1] = nd.y;
      dp[4 * g + 2] = nd.z;
      dp[4 * g + 3] = nd.w;
    }
    // the S / dP chains run at raised priority (as the forward's S^T block);
    // their A operands (Q, dO rows) are read one MFMA ahead, so that each
    // read's latency hides under the previous product instead of stalling it
    // (two ahead pushes the wave past its registers: K rows spill into the loop)
    __builtin_amdgcn_s_setprio(1);
    auto afrag = [&](int i) {  // i = 2 ks + (0: Q row, 1: dO row)
      const int ks = i >> 1;
      const int off = rbase[ks & 1] + 2048 * b + GRP128 * (ks >> 1);
      return *reinterpret_cast<const bf16x8*>(((i & 1) ? dotile : qtile) + off);
    };
    bf16x8 fa = afrag(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bf16x8 fn = afrag(i + 1 < 16 ? i + 1 : i);
      if (i & 1) dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, st.vf[i >> 1], dp, 0, 0, 0);
      else s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa, st.kf[i >> 1], s, 0, 0, 0);
      fa = fn;
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // the first read
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // read i + 1
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // product i
    }
    __builtin_amdgcn_s_setprio(0);
    if (masked) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[i] = ((vis >> (16 * bb + i)) & 1u) ? s[i] : -INFINITY;
    }
    bf16x8 pb[2], dsb[2];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int q0 = 32 * b + 16 * (g >> 1) + 8 * hh + 4 * (g & 1);
      const float4 nl = *reinterpret_cast<const float4*>(stg + STAT_OFF + 4 * q0);
      const float nl2[4] = {nl.x, nl.y, nl.z, nl.w};
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 4 * g + r;
        const float pv = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], scale_log2, nl2[r]));
        pb[i >> 3][i & 7] = (__bf16)pv;
        dsb[i >> 3][i & 7] = (__bf16)(pv * dp[i]);
      }
    }
#pragma unroll
    for (int half = 0; half < 2; ++half) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int off = GRP128 * db + 1024 * (2 * b + half);
        const i16x4 dlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4p)(dotile + off + tbase[0]));
        const i16x4 dhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4p)(dotile + off + tbase[1]));
        const i16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4p)(qtile + off + tbase[0]));
        const i16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4p)(qtile + off + tbase[1]));
        const bf16x8 at = __builtin_bit_cast(bf16x8, __builtin_shufflevector(dlo, dhi, 0, 1, 2, 3, 4, 5, 6, 7));
        const bf16x8 qt = __builtin_bit_cast(bf16x8, __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7));
        st.dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(at, pb[half], st.dv[db], 0, 0, 0);
        st.dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qt, dsb[half], st.dk[db], 0, 0, 0);
      }
    }
  }
}

// One lane's gradient row (dims 32 db + 8 g + 4 hh + {0..3}) times mul, as
// bf16 (RNE) or fp32 elements of row `row` (element offset) of dst.
template <bool F32>
__device__ __forceinline__ void store_grad_row(void* dst, int64_t row, const f32x16* acc, float mul,
                                               int hh) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t d0 = row + 32 * db + 8 * g + 4 * hh;
      const float a0 = acc[db][4 * g + 0] * mul, a1 = acc[db][4 * g + 1] * mul;
      const float a2 = acc[db][4 * g + 2] * mul, a3 = acc[db][4 * g + 3] * mul;
      if (F32) {
        *reinterpret_cast<float4*>(static_cast<float*>(dst) + d0) = float4{a0, a1, a2, a3};
      } else {
        uint2 pk;
        pk.x = (uint32_t)f2bf(a0) | ((uint32_t)f2bf(a1) << 16);
        pk.y = (uint32_t)f2bf(a2) | ((uint32_t)f2bf(a3) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(dst) + d0) = pk;
      }
    }
}

// Eight waves, two per SIMD: wave w takes the 32 keys of key group w % 4
// (64-key tile 2 u + (w % 4) / 2, half (w % 4) % 2) against query blocks
// 2 (w / 4), 2 (w / 4) + 1 of every staged q-tile; the two waves of a key
// group (one per SIMD pair... w and w + 4) add their dK / dV through LDS at
// the end.
__global__ __launch_bounds__(KV_THREADS, 1) void bwd_dkdv_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) char stg0[KV_STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char stg1[KV_STAGE_BYTES];
  __shared__ int4 lane_bases[KV_THREADS];  // per-lane LDS read bases (see kv_qtile)
  __shared__ int s_unit;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jq = lane & 31, hh = lane >> 5;
  const int kg = w & 3, qh = w >> 2;
  int tried = 0;
  const int unit = claim_unit(p.claim, p.heads * p.n_kpairs, tried, &s_unit);  // h * n_kpairs + u
  if (unit < 0) return;
  const int h = unit / p.n_kpairs;
  const int u = unit - h * p.n_kpairs;
  const int sub = kg >> 1;                     // which key tile of the pair
  const int key = (2 * u + sub) * BK + 32 * (kg & 1) + jq;
  const float scale_log2 = p.scale_log2;

  KvWave st;
  {
    const int kr = key < p.nk ? key : p.nk - 1;  // rows past nk: computed, never stored
    const int64_t row = (int64_t)kr * p.kv_stride + (int64_t)h * p.kv_head_stride + 8 * hh;
    const uint16_t* ks = p.k + row;
    const uint16_t* vs = p.v + row;
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      st.kf[s8] = *reinterpret_cast<const bf16x8*>(ks + 16 * s8);
      st.vf[s8] = *reinterpret_cast<const bf16x8*>(vs + 16 * s8);
    }
    // the second key tile of the last pair may not exist (its entries are
    // all EMPTY for these waves)
    const KDescDev kd = 2 * u + sub < p.nkt ? p.kdesc[(2 * u + sub) * BK + 32 * (kg & 1) + jq]
                                            : KDescDev{-1, 0u};
    st.kseg = kd.seg;
    st.kbits = kd.bits;
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      st.dv[db] = f32x16{};
      st.dk[db] = f32x16{};
    }
    const int rrow = kmap(jq), rsw = (rrow >> 2) & 3;
    const int tr_j = (lane & 15) >> 2, tr_c4 = lane & 3;
    const int x = 2 * ((lane >> 4) & 1) + (tr_c4 >> 1);
    lane_bases[tid] = int4{rrow * 64 + 16 * (hh ^ rsw), rrow * 64 + 16 * ((2 + hh) ^ rsw),
                           (8 * hh + tr_j) * 64 + 16 * (x ^ (2 * hh)) + 8 * (tr_c4 & 1),
                           (8 * hh + tr_j + 4) * 64 + 16 * (x ^ (2 * hh + 1)) + 8 * (tr_c4 & 1)};
  }

  const const_i32p ent = (const_i32p)p.kpair_idx + ((const_i32p)p.kpair_ptr)[u];
  const int n_ent = ((const_i32p)p.kpair_ptr)[u + 1] - ((const_i32p)p.kpair_ptr)[u];
  wait_vm_all();  // K / V rows in registers before the stage loads start

  auto compute = [&](int t, const char* stg) __attribute__((always_inline)) {
    const int e = ent[t];
    if ((e >> (2 + sub)) & 1) return;  // no visible pair for this key tile
    const bool masked = (e >> sub) & 1;
    const uint32_t vis = masked ? kv_vis_bits(stg, st.kseg, st.kbits, hh, qh) : ~0u;
    kv_qtile(st, stg, lane_bases + tid, masked, vis, scale_log2, hh, qh);
  };
  if (n_ent > 0) kv_issue_stage(p, h, ent[0] >> 4, stg0, w, lane);
  for (int t = 0; t < n_ent; t += 2) {
    wait_vm_all();   // this wave's loads of tile t
    lds_barrier();   // everyone's; tile t - 1 (other stage) fully consumed
    if (t + 1 < n_ent) kv_issue_stage(p, h, ent[t + 1] >> 4, stg1, w, lane);
    compute(t, stg0);
    if (t + 1 < n_ent) {
      wait_vm_all();
      lds_barrier();
      if (t + 2 < n_ent) kv_issue_stage(p, h, ent[t + 2] >> 4, stg0, w, lane);
      compute(t + 1, stg1);
    }
  }

  // dK, dV of a key group = the sum of its two waves' halves: the upper waves
  // hand theirs over through the (now idle) stage buffers.
  lds_barrier();
  float* xv = reinterpret_cast<float*>(stg0) + kg * 4096 + lane;
  float* xk = reinterpret_cast<float*>(stg1) + kg * 4096 + lane;
  if (qh == 1) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int ri = 0; ri < 16; ++ri) {
        xv[(16 * db + ri) * 64] = st.dv[db][ri];
        xk[(16 * db + ri) * 64] = st.dk[db][ri];
      }
  }
  lds_barrier();
  if (qh == 0) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int ri = 0; ri < 16; ++ri) {
        st.dv[db][ri] += xv[(16 * db + ri) * 64];
        st.dk[db][ri] += xk[(16 * db + ri) * 64];
      }
    if (key < p.nk) {
      const int64_t off = (int64_t)key * p.kv_stride + (int64_t)h * p.kv_head_stride;
      if (p.grad_f32) {
        store_grad_row<true>(p.dv, off, st.dv, 1.f, hh);
        store_grad_row<true>(p.dk, off, st.dk, p.scale, hh);
      } else {
        store_grad_row<false>(p.dv, off, st.dv, 1.f, hh);
        store_grad_row<false>(p.dk, off, st.dk, p.scale, hh);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// 3. dQ
// ---------------------------------------------------------------------------

constexpr int Q_WAVES = 8;
constexpr int Q_THREADS = 64 * Q_WAVES;
constexpr int Q_STAGE_BYTES = 2 * TILE_BYTES;  // K | V of one 64-key tile

struct QWave {
  bf16x8 qf[8];    // Q row of this lane's query, dims [16 s + 8 hh, +8)
  bf16x8 dof[8];   // dO row, same layout
  f32x16 acc[4];   // dQ^T (unscaled), dims 32 db + 8 (ri / 4) + 4 hh + ri % 4
  f32x16 negdelta;  // -delta in every register: the dP chains start from it
  float nlse2;      // -lse * log2(e) of this lane's query
  QDescDev qd;
  int kbase[2];    // K / V row-read base for even / odd 16-dim steps
  int tbase[2];    // K transpose-read base for rows +0 / +4
};

// Visibility of this lane's query against the 32 keys it holds scores for in
// a 64-key tile: bit 16 kb + ri <-> key 32 kb + 16 (ri / 8) + 8 hh + ri % 8.
// Computed before the products, while few registers are live.
__device__ __forceinline__ uint32_t dq_vis_bits(const QDescDev& qd, const KDescDev* kd, int hh) {
  uint32_t v = 0;
#pragma unroll 4
  for (int j = 0; j < 32; ++j) {
    const KDescDev d = kd[32 * (j >> 4) + 16 * ((j >> 3) & 1) + 8 * hh + (j & 7)];
    v |= (uint32_t)visible(qd, d.seg, d.bits) << j;
  }
  return v;
}

// P = exp2(s * scale * log2(e) - lse2) from the fp32 score of Q and K as
// given, as the dK/dV kernel forms it.
__device__ __forceinline__ void dq_tile(QWave& st, const char* ktile, const char* vtile, bool masked,
                                        uint32_t vis, float scale_log2, int hh) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    // S^T and dP^T for keys 32 kb + (0..31): two chains, interleaved, with the
    // K / V row fragments read two MFMA pairs ahead
    f32x16 s, dp;  // chains start from 0 / -delta
    auto rd = [&](const char* t, int ks) {
      return *reinterpret_cast<const bf16x8*>(t + st.kbase[ks & 1] + 2048 * kb + 4096 * (ks >> 1));
    };
    bf16x8 fk[2], fv[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      fk[i] = rd(ktile, i);
      fv[i] = rd(vtile, i);
    }
    __builtin_amdgcn_s_setprio(1);  // as the forward's S^T block
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fk[ks & 1], st.qf[ks], ks == 0 ? f32x16{} : s, 0, 0, 0);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fv[ks & 1], st.dof[ks], ks == 0 ? st.negdelta : dp, 0, 0, 0);
      if (ks + 2 < 8) {
        fk[ks & 1] = rd(ktile, ks + 2);
        fv[ks & 1] = rd(vtile, ks + 2);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);
#pragma unroll
    for (int i = 0; i < 6; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
    __builtin_amdgcn_s_setprio(0);

    // register ri holds key 32 kb + 16 (ri / 8) + 8 hh + ri % 8
    float pv[16];
#pragma unroll
    for (int ri = 0; ri < 16; ++ri) pv[ri] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[ri], scale_log2, st.nlse2));
    if (masked) {  // uniform: PARTIAL (or ragged) tiles only
#pragma unroll
      for (int ri = 0; ri < 16; ++ri) pv[ri] = ((vis >> (16 * kb + ri)) & 1u) ? pv[ri] : 0.f;
    }
    bf16x8 dsb[2];
#pragma unroll
    for (int ri = 0; ri < 16; ++ri) dsb[ri >> 3][ri & 7] = (__bf16)(pv[ri] * dp[ri]);

    // dQ^T += K^T dS^T over the two 16-key steps of this half
    auto tr = [&](int i) {  // i = 4 half + db
      const char* a = ktile + 4096 * (i & 3) + 1024 * (2 * kb + (i >> 2));
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4p)(a + st.tbase[0]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4p)(a + st.tbase[1]));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    bf16x8 ft[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) ft[i] = tr(i);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      st.acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ft[i & 1], dsb[i >> 2], st.acc[i & 3], 0, 0, 0);
      if (i + 2 < 8) ft[i & 1] = tr(i + 2);
    }
  }
}

__global__ __launch_bounds__(Q_THREADS, 1) void bwd_dq_kernel(BwdParams p) {
  __shared__ __attribute__((aligned(1024))) char sbuf0[Q_STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sbuf1[Q_STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sbuf2[Q_STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sbuf3[Q_STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) KDescDev skd0[BK];
  __shared__ __attribute__((aligned(16))) KDescDev skd1[BK];
  __shared__ __attribute__((aligned(16))) KDescDev skd2[BK];
  __shared__ __attribute__((aligned(16))) KDescDev skd3[BK];
  // LDS byte addresses of the stage buffers, for the staging loads
  const uint32_t lb0 = lds_addr(sbuf0), lb1 = lds_addr(sbuf1), lb2 = lds_addr(sbuf2), lb3 = lds_addr(sbuf3);
  const uint32_t lk0 = lds_addr(skd0), lk1 = lds_addr(skd1), lk2 = lds_addr(skd2), lk3 = lds_addr(skd3);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jq = lane & 31, hh = lane >> 5;
  const int half = w >> 2;  // which q-tile of the pair
  __shared__ int s_unit[2];

  // persistent: one unit (h * n_pairs + pair) per claim until the queues run dry
  const int n_units = p.heads * p.n_pairs;
  int tried = 0;
  for (int it = 0;; ++it) {
    const int unit = claim_unit(p.claim + 8, n_units, tried, &s_unit[it & 1]);
    if (unit < 0) break;
    const int h = unit / p.n_pairs;
    const int pr = unit - h * p.n_pairs;
    const int qrow = pr * 256 + w * 32 + jq;
    const float scale_log2 = p.scale_log2;

    QWave st;
    float nl2, nd;  // -lse2 and -delta of this lane's query
    {
      const int qr = qrow < p.nq ? qrow : p.nq - 1;  // rows past nq: computed, never stored
      const int64_t off = (int64_t)qr * p.q_stride + (int64_t)h * D + 8 * hh;
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) {
        st.qf[s8] = *reinterpret_cast<const bf16x8*>(p.q + off + 16 * s8);
        st.dof[s8] = *reinterpret_cast<const bf16x8*>(p.d_o + off + 16 * s8);
      }
      const bool in_tiles = qrow < p.nqt * QT_ROWS;
      const int64_t srow = (int64_t)h * p.nqt * QT_ROWS + qrow;
      nl2 = in_tiles ? p.nlse2[srow] : 0.f;
      nd = in_tiles ? p.ndelta[srow] : 0.f;
      st.qd = in_tiles ? p.qdesc[qrow] : QDescDev{-1, 0, 0u, 0};
#pragma unroll
      for (int db = 0; db < 4; ++db) st.acc[db] = f32x16{};
      const int krow = kmap(jq), ksw = (krow >> 2) & 3;
#pragma unroll
      for (int e = 0; e < 2; ++e) st.kbase[e] = krow * 64 + 16 * ((2 * e + hh) ^ ksw);
      const int tr_j = (lane & 15) >> 2, tr_c4 = lane & 3;
      const int x = 2 * ((lane >> 4) & 1) + (tr_c4 >> 1);
#pragma unroll
      for (int r = 0; r < 2; ++r)
        st.tbase[r] = (8 * hh + tr_j + 4 * r) * 64 + 16 * (x ^ (2 * hh + r)) + 8 * (tr_c4 & 1);
    }

    LoadCtx lc;
    lc.kv_stride = p.kv_stride;
    lc.nk = p.nk;
    lc.n_cached = 0;
    lc.lane_row = 16 * (w & 3) + (lane >> 2);
    lc.lane_chunk = (lane & 3) ^ ((lane >> 4) & 3);
    lc.lane_cache = (uint32_t)(lc.lane_row * D + 8 * lc.lane_chunk) * 2u;
    lc.lane_new = (uint32_t)((int)(lc.lane_row * p.kv_stride) + 8 * lc.lane_chunk) * 2u;
    lc.k_cache_h = p.k;  // unused: no cached keys
    lc.v_cache_h = p.v;
    lc.k_new_h = p.k + (int64_t)h * p.kv_head_stride;
    lc.v_new_h = p.v + (int64_t)h * p.kv_head_stride;

    const const_i32p ent = (const_i32p)p.pair_idx + ((const_i32p)p.pair_ptr)[pr];
    const int n_ent = ((const_i32p)p.pair_ptr)[pr + 1] - ((const_i32p)p.pair_ptr)[pr];
    wait_vm_all();  // rows and statistics in registers before the tile loads start
    st.nlse2 = nl2;
#pragma unroll
    for (int ri = 0; ri < 16; ++ri) st.negdelta[ri] = nd;

    // (always_inline: otherwise the wave state would be passed through scratch)
    auto issue_tile = [&](int kt, uint32_t buf, uint32_t kd) __attribute__((always_inline)) {
      issue_half(lc, lc.k_cache_h, lc.k_new_h, buf, kt, w);
      issue_half(lc, lc.v_cache_h, lc.v_new_h, buf + TILE_BYTES, kt, w);
      if (w == 0 && lane < 32) dma16_s(p.kdesc + kt * BK, 16u * lane, kd);
    };
    auto tile = [&](int here, const char* cbuf, const KDescDev* ckd) __attribute__((always_inline)) {
      if ((here >> (2 + half)) & 1) return;  // EMPTY for this wave's q-tile
      // one code path for FULL and PARTIAL tiles (a second variant would push
      // the wave past its 256 registers); the per-element mask sits behind a
      // uniform branch that FULL tiles skip
      const bool masked = (here >> half) & 1;
      const uint32_t vis = masked ? dq_vis_bits(st.qd, ckd, hh) : ~0u;
      dq_tile(st, cbuf, cbuf + TILE_BYTES, masked, vis, scale_log2, hh);
    };
    // four stages used as two pairs, one barrier per pair (as in the forward)
    auto pair = [&](int t, const char* b0, const KDescDev* k0, const char* b1, const KDescDev* k1,
                    uint32_t n0, uint32_t nk0, uint32_t n1, uint32_t nk1) __attribute__((always_inline)) {
      const int last = n_ent - 1;
      const int e0 = ent[t], e1 = ent[min(t + 1, last)];
      int e2 = ent[min(t + 2, last)], e3 = ent[min(t + 3, last)];
      // (pin the loads here: otherwise they are rematerialised after the barrier)
      asm volatile("" : "+s"(e2), "+s"(e3));
      wait_vm_all();
      lds_barrier();
      if (t + 2 < n_ent) issue_tile(e2 >> 4, n0, nk0);
      if (t + 3 < n_ent) issue_tile(e3 >> 4, n1, nk1);
      tile(e0, b0, k0);
      if (t + 1 < n_ent) tile(e1, b1, k1);
    };
    if (n_ent > 0) issue_tile(ent[0] >> 4, lb0, lk0);
    if (n_ent > 1) issue_tile(ent[1] >> 4, lb1, lk1);
    for (int t = 0; t < n_ent; t += 4) {
      pair(t, sbuf0, skd0, sbuf1, skd1, lb2, lk2, lb3, lk3);
      if (t + 2 < n_ent) pair(t + 2, sbuf2, skd2, sbuf3, skd3, lb0, lk0, lb1, lk1);
    }

    if (qrow < p.nq) {
      // a row that sees no key (padding) may have been computed unmasked on
      // tiles no other row needs a mask for: its gradient is zero
      if (st.qd.seg < 0) {
#pragma unroll
        for (int db = 0; db < 4; ++db) st.acc[db] = f32x16{};
      }
      const int64_t off = (int64_t)qrow * p.q_stride + (int64_t)h * D;
      if (p.grad_f32) store_grad_row<true>(p.dq, off, st.acc, p.scale, hh);
      else store_grad_row<false>(p.dq, off, st.acc, p.scale, hh);
    }
    // (the next claim's barrier ends every wave's reads of the stage buffers
    // before the next unit's loads refill them)
  }
}

}  // namespace

hipError_t launch_attn_bwd(const BwdParams& p, hipStream_t stream) {
  if (p.heads <= 0) return hipSuccess;
  const int64_t items = (int64_t)p.heads * p.nqt * QT_ROWS * 16;
  {  // at least one block: it also zeroes the work-queue counters
    hipLaunchKernelGGL(bwd_rowstats_kernel, dim3((unsigned)std::max<int64_t>(1, (items + 255) / 256)),
                       dim3(256), 0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.nk > 0 && p.n_kpairs > 0) {
    const int units = p.heads * p.n_kpairs;
    // a surplus of 1/16: workgroups that a faster XCD runs after its own
    // queue is drained take units from the others
    hipLaunchKernelGGL(bwd_dkdv_kernel, dim3((unsigned)(8 * ((units + units / 16 + 7) / 8))), dim3(KV_THREADS),
                       0, stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (p.nq > 0 && p.n_pairs > 0) {
    const int units = p.heads * p.n_pairs;
    hipLaunchKernelGGL(bwd_dq_kernel, dim3((unsigned)std::min(units, p.groups)), dim3(Q_THREADS), 0,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace nomas
