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
// Scheduling (persistent, stream-K style): a unit is a pair of consecutive
// 128-query tiles of one head (256 queries, one per lane column of the eight
// waves of a workgroup, two waves per SIMD); its key tiles are the union of the
// pair's tile lists, with per-q-tile EMPTY / mask flags.  The host cuts the
// (unit, key tile) iterations into ranges of equal estimated cost, one per
// workgroup (one per CU).  Each K/V tile fetched serves 256 queries, and the 130 KB of
// LDS hold four tile stages used as two pairs: a pair of tiles is computed
// while the next pair loads, with one barrier per pair.  A unit
// split between ranges is
// computed in pieces whose un-normalised (O, max, sum) go to a workspace and
// are merged by attn_fwd_combine_kernel.  Workgroup ids are remapped so that
// the workgroups of one XCD take consecutive ranges, i.e. the q-tiles of the
// same heads, which then share that XCD's L2 for their K/V.  A video-block
// sparse plan gives every head its own key-tile lists (chosen on the device
// before this kernel); the schedule is the same, only the list base moves.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, fp32 accumulate), per wave of
// 32 queries:
//   S^T (64 keys x 32 queries) = K_tile * Q^T   -- K from LDS, Q in registers
//   O^T (128 dims x 32 queries) += V^T * P^T    -- V^T from LDS, P^T in regs
// One query per lane column: row max / row sum are in-lane over 32 keys, and
// the rescale factor is a per-lane scalar.  Key rows of the S^T MFMA are
// permuted (kmap) so that each half-wave holds 8 consecutive keys per 16-key
// step, which is the B-operand layout of the P^T V^T product: P never leaves
// registers.  V^T operands come straight from the V tile with the LDS
// transpose read (ds_read_b64_tr_b16).
//
// The reference max is not recomputed per tile.  P is formed against the
// row's current reference, which is set to an exact tile max; only when a
// half-wave's sum of P exceeds RESCALE_SUM (a score far above the reference,
// or a row that has not seen a visible key yet) does the wave take the exact
// path: row max over the tile (half-wave exchange), O and the sum rescaled,
// P formed again.  O / l does not depend on the reference, so this changes
// rounding only, and P stays <= RESCALE_SUM, far from fp32 / bf16 limits.
//
// LDS tiles use the swizzled layout of tile_common.h (64 rows per K or V tile).
#include "tile_common.h"

namespace nomas {
namespace {

constexpr int NWAVES = 8;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int UNIT_ROWS = 32 * NWAVES;  // 256 queries: a pair of 128-query tiles
constexpr int NSTAGE = 4;
constexpr int LOADS_PER_TILE = 4;       // per wave: 2 K + 2 V blocks (wave 0: + descriptors)
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
// A half-wave's sum of P over its 32 keys above this value sends the wave to
// the exact path (new reference = the row max); below it every P <= 2^16.
constexpr float RESCALE_SUM = 65536.0f;
// per partial piece, for each thread: its 64 O values divided by the piece's
// row sum, as 32 bf16 pairs, then the piece's reference max and row sum (fp32)
constexpr int SLOT_WORDS = NTHREADS * 34;

struct WaveState {
  bf16x8 qf[8];     // Q fragment, pre-scaled: query jq, dims [16 s + 8 hh, +8) of Q * scale * log2(e)
  f32x16 acc[4];    // O^T, dims 32 db + 8 (ri / 4) + 4 hh + ri % 4
  f32x16 negref;    // -reference in every register: the score chains start from it
  float m_run;      // reference max, log2 domain (same in both half-waves)
  float l_run;      // this half-wave's share of the running sum
  QDescDev qd;
  int kbase[2];     // K read base for even / odd 16-dim steps
  int vbase[2];     // V transpose-read base for key rows +0 / +4
};

// One 64-key tile for one wave: S^T, mask, online softmax, O^T += V^T P^T.
// With Q pre-scaled by scale * log2(e) and the score chains started from
// -reference, the accumulators hold x = s * scale * log2(e) - ref directly:
// P = exp2(x) needs no multiply-add per score.
__device__ __forceinline__ void tile_step(WaveState& ws, const char* ktile, const char* vtile,
                                          const KDescDev* kd, bool masked, int hh) {
  // S^T for keys 32 kb + (0..31): two independent accumulation chains,
  // interleaved, with the K fragments read four MFMAs ahead.
  f32x16 s[2];
  auto kfrag = [&](int i) {  // i = 2 ks + kb: row 32 kb + kmap(jq), chunk 2 ks + hh
    const int kb = i & 1, ks = i >> 1;
    return *reinterpret_cast<const bf16x8*>(ktile + ws.kbase[ks & 1] + 2048 * kb + 4096 * (ks >> 1));
  };
  bf16x8 kf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) kf[i] = kfrag(i);
  // A wave issuing its S^T block runs at raised priority, so that the other
  // wave of the SIMD fills the gaps with its softmax instead of competing.
  // (The P.V block runs at normal priority: raising it there too is slower.)
  __builtin_amdgcn_s_setprio(1);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[i & 3], ws.qf[i >> 1], i < 2 ? ws.negref : s[i & 1],
                                                       0, 0, 0);
    if (i + 4 < 16) kf[i & 3] = kfrag(i + 4);
  }
  // keep that order: the scheduler would otherwise sink each read next to
  // its MFMA and expose the LDS latency sixteen times
  __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);  // 4 LDS reads
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // 1 LDS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  __builtin_amdgcn_s_setprio(0);

  // the first V^T fragments of O^T += V^T P^T, read now so that their
  // latency hides under the softmax
  auto vfrag = [&](int i) {  // i = 4 step + db: keys 16 step + 8 hh + (0..7), dims 32 db + ..
    const char* a = vtile + 4096 * (i & 3) + 1024 * (i >> 2);
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4p)(a + ws.vbase[0]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4p)(a + ws.vbase[1]));
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  };
  bf16x8 vf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) vf[i] = vfrag(i);
  // register ri of block kb holds key 32 kb + 16 (ri / 8) + 8 hh + ri % 8
  if (masked) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ri = 0; ri < 16; ++ri) {
        const KDescDev d = kd[32 * kb + 16 * (ri >> 3) + 8 * hh + (ri & 7)];
        s[kb][ri] = visible(ws.qd, d.seg, d.bits) ? s[kb][ri] : -INFINITY;
      }
  }
  // P = exp2(x + d) in fp32, x = s * scale * log2(e) - ref as the chains left
  // it and d = 0 (the common path) or old minus new reference, summed in fp32
  // (four chains) and rounded to bf16 as the P.V operand.
  bf16x8 pf[4];  // P^T operand for step (kb, half) = 2 kb + half
  float l_half;  // this half-wave's sum over its 32 keys
  auto probs = [&](bool shift, float d) {
    float lsum[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8 v;
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) {
          const float x = s[kb][8 * half + e8];
          const float pe = __builtin_amdgcn_exp2f(shift ? x + d : x);
          lsum[e8 & 3] = (kb | half | (e8 >> 2)) ? lsum[e8 & 3] + pe : pe;
          v[e8] = (__bf16)pe;
        }
        pf[2 * kb + half] = v;
      }
    l_half = (lsum[0] + lsum[1]) + (lsum[2] + lsum[3]);
  };
  // Common path: no max at all.  P is formed against the current reference
  // (0 while the row has seen no visible key); a row needs a new reference
  // only if it has none yet or a half's sum exceeds RESCALE_SUM (a score far
  // above the reference, or an overflow).  Then the wave computes the row
  // maxima, and each such row -- only those, so a row's result depends on its
  // own scores alone -- takes max(reference, row max), rescales O and its sum
  // and forms P again (rows keeping their reference recompute the same P).
  probs(false, 0.f);
  const bool need_half = ws.m_run == -INFINITY || !(l_half <= RESCALE_SUM);
  if (__builtin_amdgcn_ballot_w64(need_half)) {
    const float ref_old = ws.m_run == -INFINITY ? 0.f : ws.m_run;
    float t[12];
#pragma unroll
    for (int j = 0; j < 5; ++j) t[j] = fmaxf(fmaxf(s[0][3 * j], s[0][3 * j + 1]), s[0][3 * j + 2]);
#pragma unroll
    for (int j = 0; j < 5; ++j) t[5 + j] = fmaxf(fmaxf(s[1][3 * j], s[1][3 * j + 1]), s[1][3 * j + 2]);
    t[10] = s[0][15];
    t[11] = s[1][15];
    const float u0 = fmaxf(fmaxf(t[0], t[1]), t[2]), u1 = fmaxf(fmaxf(t[3], t[4]), t[5]);
    const float u2 = fmaxf(fmaxf(t[6], t[7]), t[8]), u3 = fmaxf(fmaxf(t[9], t[10]), t[11]);
    const float m_half = fmaxf(fmaxf(fmaxf(u0, u1), u2), u3) + ref_old;
    const float m_row = fmaxf(m_half, __shfl_xor(m_half, 32));
    const bool need_row = need_half || __shfl_xor((int)need_half, 32);
    const float m_new = need_row ? fmaxf(ws.m_run, m_row) : ws.m_run;
    const float alpha = m_new == ws.m_run ? 1.f : __builtin_amdgcn_exp2f(ws.m_run - m_new);
    ws.m_run = m_new;
    ws.l_run *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db) ws.acc[db] *= alpha;
    const float ref_new = m_new == -INFINITY ? 0.f : m_new;
    probs(true, ref_old - ref_new);  // 0 for rows that keep their reference
#pragma unroll
    for (int ri = 0; ri < 16; ++ri) ws.negref[ri] = -ref_new;
  }
  ws.l_run += l_half;

#pragma unroll
  for (int i = 0; i < 16; ++i) {
    ws.acc[i & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i & 3], pf[i >> 2], ws.acc[i & 3], 0, 0, 0);
    if (i + 4 < 16) vf[i & 3] = vfrag(i + 4);
  }
#pragma unroll
  for (int i = 0; i < 12; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 1 MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // the two reads of a fragment
  }
  __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);
  __builtin_amdgcn_s_setprio(0);
}

// Normalise and store one lane's query row (O in bf16, LSE in natural log);
// dims 32 db + 8 g + 4 hh + {0..3} for the blocks db in [db0, db0 + ndb).
__device__ __forceinline__ void store_row(const FwdParams& p, const f32x16* acc, int db0, int ndb,
                                          float m_run, float l_tot, int h, int qrow, int hh,
                                          bool write_lse) {
  if (qrow >= p.nq) return;
  // a row with a zero sum sees no key: exact zeros, whatever its accumulator
  // holds (a padding row may have been computed unmasked)
  const bool dead = !(l_tot > 0.f);
  const float inv = dead ? 0.f : 1.f / l_tot;
  uint16_t* dst = p.o + (int64_t)qrow * p.o_stride + (int64_t)h * D;
  for (int j = 0; j < ndb; ++j) {
    const int db = db0 + j;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = 32 * db + 8 * g + 4 * hh;
      uint2 pk;
      pk.x = (uint32_t)f2bf(acc[j][4 * g + 0] * inv) | ((uint32_t)f2bf(acc[j][4 * g + 1] * inv) << 16);
      pk.y = (uint32_t)f2bf(acc[j][4 * g + 2] * inv) | ((uint32_t)f2bf(acc[j][4 * g + 3] * inv) << 16);
      if (dead) pk = uint2{0u, 0u};
      *reinterpret_cast<uint2*>(dst + d0) = pk;
    }
  }
  if (p.lse && write_lse && hh == 0)
    p.lse[(int64_t)h * p.nq + qrow] =
        l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
}

__global__ __launch_bounds__(NTHREADS, 1) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_fwd_kernel(FwdParams p) {
  // Four stage buffers (K | V of one tile) and their key descriptors, as
  // distinct LDS objects.
  __shared__ __attribute__((aligned(1024))) char sbuf0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sbuf1[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sbuf2[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sbuf3[STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) KDescDev skd0[BK];
  __shared__ __attribute__((aligned(16))) KDescDev skd1[BK];
  __shared__ __attribute__((aligned(16))) KDescDev skd2[BK];
  __shared__ __attribute__((aligned(16))) KDescDev skd3[BK];
  // LDS byte addresses of the stage buffers, for the staging loads
  const uint32_t lb0 = lds_addr(sbuf0), lb1 = lds_addr(sbuf1), lb2 = lds_addr(sbuf2), lb3 = lds_addr(sbuf3);
  const uint32_t lk0 = lds_addr(skd0), lk1 = lds_addr(skd1), lk2 = lds_addr(skd2), lk3 = lds_addr(skd3);
  static_assert(NSTAGE == 4, "the unrolled loop below names four stage buffers");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int jq = lane & 31;   // query column of this lane
  const int hh = lane >> 5;   // half-wave
  const int half = w >> 2;    // which q-tile of the pair this wave serves

  // logical workgroup: XCD-major (dispatch places workgroup b on XCD b % 8)
  const int G = (int)gridDim.x;
  const int g = (G & 7) ? (int)blockIdx.x : (int)(blockIdx.x & 7) * (G >> 3) + (int)(blockIdx.x >> 3);

  const const_i32p unit_ptr = (const_i32p)p.csr_ptr;   // merged lists per q-tile pair
  const const_i32p unit_idx = (const_i32p)p.csr_idx;
  const const_i32p pieces = (const_i32p)p.pieces;     // 4 ints per piece
  const int pc0 = ((const_i32p)p.wg_ptr)[g], pc1 = ((const_i32p)p.wg_ptr)[g + 1];
  const float scale_log2 = p.scale_log2;

  WaveState ws;
  {
    const int krow = kmap(jq);             // + 32 kb
    const int ksw = (krow >> 2) & 3;
#pragma unroll
    for (int e = 0; e < 2; ++e) ws.kbase[e] = krow * 64 + 16 * ((2 * e + hh) ^ ksw);
    const int tr_j = (lane & 15) >> 2, tr_c4 = lane & 3;
    const int x = 2 * ((lane >> 4) & 1) + (tr_c4 >> 1);
#pragma unroll
    for (int r = 0; r < 2; ++r)
      ws.vbase[r] = (8 * hh + tr_j + 4 * r) * 64 + 16 * (x ^ (2 * hh + r)) + 8 * (tr_c4 & 1);
  }
  LoadCtx lc;
  lc.kv_stride = p.kv_stride;
  lc.nk = p.nk;
  lc.n_cached = p.n_cached;
  lc.lane_row = 16 * (w & 3) + (lane >> 2);
  lc.lane_chunk = (lane & 3) ^ ((lane >> 4) & 3);
  lc.lane_cache = (uint32_t)(lc.lane_row * D + 8 * lc.lane_chunk) * 2u;
  lc.lane_new = (uint32_t)((int)(lc.lane_row * p.kv_stride) + 8 * lc.lane_chunk) * 2u;

  // The workgroup's own pieces, then (long calls) tail chunks claimed in turn
  // from the per-call counter until none is left.
  __shared__ int s_claim;
  const const_i32p chunk_list = (const_i32p)p.chunks;
  for (int pc = pc0;; ++pc) {
    const_i32p src;
    if (pc < pc1) {
      src = pieces + 4 * pc;
    } else {
      if (p.n_chunks == 0) break;
      if (tid == 0) s_claim = (int)atomicAdd(p.claim, 1u);
      lds_barrier();
      const int c = __builtin_amdgcn_readfirstlane(s_claim);
      if (c >= p.n_chunks) break;
      src = chunk_list + 4 * c;
    }
    const int unit = src[0];
    const int e_begin = src[1], e_end = src[2], slot = src[3];
    const int h = unit / p.n_pairs;
    const int pr = unit - h * p.n_pairs;
    const int qrow = pr * UNIT_ROWS + w * 32 + jq;
    // entries in the unit's rotated order: tile t of this piece is list entry
    // (e_begin + t + shift) mod n_unit
    const const_i32p ulist = unit_idx + p.list_head_stride * h + unit_ptr[pr];
    const int n_unit = unit_ptr[pr + 1] - unit_ptr[pr];
    const int rot = e_begin + ((const_i32p)p.unit_shift)[unit];
    auto ent_at = [&](int t) {
      const int j = rot + t;
      return ulist[j >= n_unit ? j - n_unit : j];
    };
    const int n_ent = e_end - e_begin;
    lc.k_cache_h = p.k_cache + (int64_t)h * p.cache_cap * D;
    lc.v_cache_h = p.v_cache + (int64_t)h * p.cache_cap * D;
    lc.k_new_h = p.k_new + (int64_t)h * p.kv_head_stride;
    lc.v_new_h = p.v_new + (int64_t)h * p.kv_head_stride;

    if (qrow < p.nq) {
      const uint16_t* src = p.q + (int64_t)qrow * p.q_stride + (int64_t)h * D + 8 * hh;
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) ws.qf[s8] = *reinterpret_cast<const bf16x8*>(src + 16 * s8);
    } else {
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) ws.qf[s8] = bf16x8{};
    }
    // the query descriptors are padded to whole 128-query tiles; a missing
    // second tile of the last pair reads the padding of the first tile's end
    ws.qd = qrow < p.nqt * 128 ? p.qdesc[qrow] : QDescDev{-1, 0, 0u, 0};
#pragma unroll
    for (int db = 0; db < 4; ++db) ws.acc[db] = f32x16{};
    ws.m_run = -INFINITY;
    ws.l_run = 0.f;
    ws.negref = f32x16{};  // reference 0 until the row has one
    // Q and the query descriptors must have arrived before the tile loop:
    // otherwise the compiler's own waits for them, placed inside the loop,
    // would also drain the tile prefetches issued below.
    wait_vm_all();
    // Q * scale * log2(e), rounded to bf16 (one more rounding of Q, relative
    // 2^-9, for no multiply per score in the tile loop)
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8)
#pragma unroll
      for (int e = 0; e < 8; ++e) ws.qf[s8][e] = (__bf16)((float)ws.qf[s8][e] * scale_log2);

    auto issue_tile = [&](int kt, uint32_t buf, uint32_t kd) {
      issue_half(lc, lc.k_cache_h, lc.k_new_h, buf, kt, w);
      issue_half(lc, lc.v_cache_h, lc.v_new_h, buf + TILE_BYTES, kt, w);
      if (w == 0 && lane < 32) dma16_s(p.kdesc + kt * BK, 16u * lane, kd);
    };
    if (n_ent > 0) issue_tile(ent_at(0) >> 4, lb0, lk0);
    if (n_ent > 1) issue_tile(ent_at(1) >> 4, lb1, lk1);

    // Tiles go in pairs: iteration j computes tiles 2j, 2j+1 (buffers of one
    // half of the ring) after issuing tiles 2j+2, 2j+3 into the other half,
    // which the barrier has just released; one barrier per two tiles.
    auto tile = [&](int here, const char* cbuf, const KDescDev* ckd) {
      if (!((here >> (2 + half)) & 1))  // not EMPTY for this wave's q-tile
        tile_step(ws, cbuf, cbuf + TILE_BYTES, ckd, (here >> half) & 1, hh);
    };
    auto pair = [&](int t, const char* b0, const KDescDev* k0, const char* b1, const KDescDev* k1,
                    uint32_t n0, uint32_t nk0, uint32_t n1, uint32_t nk1) {
      // the four entries this pair needs, read before the barrier (their
      // scalar-load latency then overlaps the wait instead of following it)
      const int last = n_ent - 1;
      const int e0 = ent_at(t), e1 = ent_at(min(t + 1, last));
      int e2 = ent_at(min(t + 2, last)), e3 = ent_at(min(t + 3, last));
      // (pin the loads here: otherwise they are rematerialised after the barrier)
      asm volatile("" : "+s"(e2), "+s"(e3));
      wait_vm_all();  // this wave's loads of tiles t, t+1 (the only ones in flight)
      lds_barrier();  // ... and every other wave's; tiles t-2, t-1 fully consumed
      if (t + 2 < n_ent) issue_tile(e2 >> 4, n0, nk0);
      if (t + 3 < n_ent) issue_tile(e3 >> 4, n1, nk1);
      tile(e0, b0, k0);
      if (t + 1 < n_ent) tile(e1, b1, k1);
    };
    for (int t = 0; t < n_ent; t += 4) {
      pair(t, sbuf0, skd0, sbuf1, skd1, lb2, lk2, lb3, lk3);
      if (t + 2 < n_ent) pair(t + 2, sbuf2, skd2, sbuf3, skd3, lb0, lk0, lb1, lk1);
    }

    // Rows that see no key (padding) may have been computed unmasked on tiles
    // that need no mask for any other row: a zero sum makes them O = 0,
    // LSE = -inf, here and through the merge.
    const float l_sum = ws.l_run + __shfl_xor(ws.l_run, 32);
    const float l_tot = ws.qd.seg < 0 ? 0.f : l_sum;
    if (slot < 0) {
      store_row(p, ws.acc, 0, 4, ws.m_run, l_tot, h, qrow, hh, true);
    } else {  // partial piece: O / l (bf16) and (m, l), thread-native layout
      // (a zero sum: zeros and m = -inf, so the merge gives it no weight)
      const bool dead = !(l_tot > 0.f);
      const float inv = dead ? 0.f : 1.f / l_tot;
      uint32_t* dst = reinterpret_cast<uint32_t*>(p.partial) + (int64_t)slot * SLOT_WORDS + tid;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t v = (uint32_t)f2bf(ws.acc[db][2 * j] * inv) |
                             ((uint32_t)f2bf(ws.acc[db][2 * j + 1] * inv) << 16);
          dst[(8 * db + j) * NTHREADS] = dead ? 0u : v;
        }
      reinterpret_cast<float*>(dst)[32 * NTHREADS] = dead ? -INFINITY : ws.m_run;
      reinterpret_cast<float*>(dst)[33 * NTHREADS] = l_tot;
    }
    wait_vm_all();  // stores retired before the next piece's load accounting
    lds_barrier();  // the stage buffers are reused by the next piece
  }
}

// Merge the pieces of split units: with a_k = 2^(m_k - m), m = max_k m_k,
// O = sum_k a_k l_k (O_k / l_k) / sum_k a_k l_k.  Workgroup (item, db, r)
// handles dims 32 db .. 32 db + 31 of rows 128 r .. 128 r + 127 of one split
// unit; thread T mirrors forward thread 256 r + T.
__global__ __launch_bounds__(256) void attn_fwd_combine_kernel(FwdParams p) {
  const const_i32p cmb = (const_i32p)p.combine + 4 * (blockIdx.x >> 3);
  const int db = (blockIdx.x >> 1) & 3, r = blockIdx.x & 1;
  const int unit = cmb[0], first = cmb[1], n = cmb[2];
  const int h = unit / p.n_pairs;
  const int pr = unit - h * p.n_pairs;
  const int T = 256 * r + (int)threadIdx.x;
  const int lane = T & 63;
  const int qrow = pr * UNIT_ROWS + (T >> 6) * 32 + (lane & 31);
  const int hh = lane >> 5;
  const uint32_t* base = reinterpret_cast<const uint32_t*>(p.partial) + (int64_t)first * SLOT_WORDS + T;
  float m = -INFINITY;
  for (int k = 0; k < n; ++k)
    m = fmaxf(m, __uint_as_float(base[(int64_t)k * SLOT_WORDS + 32 * NTHREADS]));
  const float mu = m == -INFINITY ? 0.f : m;
  f32x16 acc[1] = {f32x16{}};
  float l = 0.f;
  for (int k = 0; k < n; ++k) {
    const uint32_t* src = base + (int64_t)k * SLOT_WORDS;
    const float wk = __builtin_amdgcn_exp2f(__uint_as_float(src[32 * NTHREADS]) - mu) *
                     __uint_as_float(src[33 * NTHREADS]);
    l += wk;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t v = src[(8 * db + j) * NTHREADS];
      acc[0][2 * j] += wk * __uint_as_float(v << 16);
      acc[0][2 * j + 1] += wk * __uint_as_float(v & 0xffff0000u);
    }
  }
  store_row(p, acc, db, 1, m, l, h, qrow, hh, db == 0);
}

// Reset of the tail-chunk counter before a call (a kernel rather than a
// memset, so that graph capture records a kernel node).
__global__ __launch_bounds__(64) void attn_fwd_claim_reset_kernel(uint32_t* claim) {
  if (threadIdx.x == 0) claim[threadIdx.x] = 0u;
}

}  // namespace

size_t attn_fwd_slot_bytes() { return (size_t)SLOT_WORDS * sizeof(uint32_t); }
int attn_fwd_groups_per_cu() { return 1; }

hipError_t launch_attn_fwd(const FwdParams& p, hipStream_t stream) {
  if (p.nq == 0) return hipSuccess;
  if (p.n_chunks > 0) {  // the tail chunks are handed out from zero in every call
    hipLaunchKernelGGL(attn_fwd_claim_reset_kernel, dim3(1), dim3(64), 0, stream, p.claim);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(attn_fwd_kernel, dim3((unsigned)p.groups), dim3(NTHREADS), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.n_combine == 0) return e;
  hipLaunchKernelGGL(attn_fwd_combine_kernel, dim3((unsigned)(8 * p.n_combine)), dim3(256), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace nomas
