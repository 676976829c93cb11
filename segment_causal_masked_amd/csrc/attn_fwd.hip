// Forward kernel of action-aware causal attention for gfx950 (CDNA4).
//
// Computes O = softmax(scale * Q K^T + M) V with M = -inf on hidden pairs
// (the mask of "Summary (Overview)", Model Architecture: Segment-wise and
// Action-Aware Causal Attention), flash-style: a workgroup owns a 128-query
// tile of one head and walks only the non-empty 64-key tiles of its row of the
// tile map; FULL tiles run unmasked, PARTIAL (or ragged) tiles evaluate the
// per-token descriptors.  Online softmax keeps a running max and sum per query
// in fp32, so the result equals the plain softmax up to rounding.
//
// Work split inside the workgroup (8 waves, two per SIMD): wave w owns the 32
// queries 32*(w%4).. of the tile and key group w/4.  Tiles are consumed in
// pairs: group 0 takes the first tile of a pair, group 1 the second, so each
// K/V byte in LDS is read by four waves instead of eight.  The two groups'
// (O, max, sum) are merged at the end.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, fp32 accumulate), per wave:
//   S^T (64 keys x 32 queries) = K_tile * Q^T   -- K from LDS, Q in registers
//   O^T (128 dims x 32 queries) += V^T * P^T    -- V^T from LDS, P^T in regs
// One query per lane column: row max / row sum are in-lane over 32 keys plus
// one exchange between half-waves, and the rescale factor is a per-lane
// scalar.  Key rows of the S^T MFMA are permuted (kmap) so that each half-wave
// holds 8 consecutive keys per 16-key step, which is the B-operand layout of
// the P^T V^T product: P never leaves registers.  V^T operands come straight
// from the row-major V tile with the LDS transpose read (ds_read_b64_tr_b16).
//
// Staging: K and V tiles are copied HBM -> LDS by direct 16-byte loads
// (global_load_lds_dwordx4), double buffered, one barrier per tile pair.  LDS
// rows are 256 bytes with the 16-byte chunks XOR-swizzled by swz(row) so that
// both the K reads (8 rows x 16 B per cycle) and the transpose reads of V
// (4 rows x 32 B per 16 lanes) hit distinct banks.
#include "kernels.h"

namespace nomas {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int D = 128;
constexpr int BQ = 128;
constexpr int BK = 64;
constexpr int NWAVES = 8;
constexpr int TILE_BYTES = BK * D * 2;          // 16 KB: one K or V tile
constexpr int STAGE_BYTES = 4 * TILE_BYTES;     // K,V of two tiles

// MFMA output row i (of 32) -> key offset inside a 32-key block.
__device__ __forceinline__ int kmap(int i) {
  const int g = i >> 3, q = (i >> 2) & 1, r = i & 3;
  return 16 * (g >> 1) + 8 * q + 4 * (g & 1) + r;
}

// 16-byte chunk swizzle of LDS row `row` (see the header comment).
__device__ __forceinline__ int swz(int row) { return 2 * (row & 3) + ((row >> 3) & 1); }

__device__ __forceinline__ bool visible(const QDescDev& q, int kseg, uint32_t kbits) {
  return kseg >= q.lo && kseg <= q.seg &&
         (kbits == 0u || (kseg == q.seg && (q.amask & kbits) != 0u));
}

__device__ __forceinline__ uint16_t f2bf(float x) {
  __bf16 b = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}

__device__ __forceinline__ void wait_vm_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }  // vmcnt(0)

// Everything the stage loads need, copied out of the kernel arguments so that
// it lives in scalar registers.
struct LoadCtx {
  const uint16_t *k_cache, *v_cache, *k_new, *v_new;
  const KDescDev* kdesc;
  int64_t hc, hn, kv_stride;  // head offsets (cache, new row) and new-token stride
  int32_t nk, n_cached;
};

// Issue the direct loads of one stage: K and V of key tiles kt0, kt1 (kt1 may
// repeat kt0 when the pair is incomplete) and their key descriptors.  Block
// i (1 KB) of wave w covers tile i/4, K (i/2 even) or V, rows 4*(8*(i&1)+w)..+3.
__device__ __forceinline__ void issue_stage(const LoadCtx c, char* buf, KDescDev* kd_buf,
                                            int kt0, int kt1, int w, int lane) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int t = i >> 2, kv = (i >> 1) & 1, rb = 8 * (i & 1) + w;
    const int row = 4 * rb + (lane >> 4);
    const int ch = (lane & 15) ^ swz(row);  // logical chunk this lane fetches
    int key = (t ? kt1 : kt0) * BK + row;
    key = key < c.nk ? key : c.nk - 1;      // ragged tail: any valid row, masked later
    const bool cached = key < c.n_cached;
    const int64_t off = cached ? c.hc + (int64_t)key * D
                               : c.hn + (int64_t)(key - c.n_cached) * c.kv_stride;
    const uint16_t* base = cached ? (kv ? c.v_cache : c.k_cache) : (kv ? c.v_new : c.k_new);
    __builtin_amdgcn_global_load_lds(base + off + 8 * ch,
                                     LDS_PTR(buf + (2 * t + kv) * TILE_BYTES + rb * 1024), 16, 0, 0);
  }
  if (w == 0) {  // lanes 0..31: tile 0 descriptors, 32..63: tile 1 (2 per lane)
    const int kt = (lane >> 5) ? kt1 : kt0;
    __builtin_amdgcn_global_load_lds(c.kdesc + kt * BK + 2 * (lane & 31), LDS_PTR(kd_buf), 16, 0, 0);
  }
}

struct WaveState {
  bf16x8 qf[8];       // Q fragment: query jq, dims [16 s + 8 hh, +8)
  f32x16 acc[4];      // O^T, dims 32 db + 8 (ri / 4) + 4 hh + ri % 4
  float m_run;        // running max, log2 domain
  float l_run;        // this half-wave's share of the running sum
  QDescDev qd;
  int k_off[2], k_swz[2];
};

// One 64-key tile for one wave: S^T, mask, online softmax, O^T += V^T P^T.
__device__ __forceinline__ void tile_step(WaveState& ws, const char* kbase, const char* vbase,
                                          const KDescDev* kd, bool masked, float scale_log2,
                                          int hh, int lane) {
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    s[kb] = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const int c = (2 * ks + hh) ^ ws.k_swz[kb];
      const bf16x8 kf = *reinterpret_cast<const bf16x8*>(kbase + ws.k_off[kb] + 16 * c);
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, ws.qf[ks], s[kb], 0, 0, 0);
    }
  }
  // register ri of block kb holds key 32 kb + 16 (ri / 8) + 8 hh + ri % 8
  if (masked) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ri = 0; ri < 16; ++ri) {
        const KDescDev d = kd[32 * kb + 16 * (ri >> 3) + 8 * hh + (ri & 7)];
        const bool vis = visible(ws.qd, d.seg, d.bits);
        s[kb][ri] = vis ? s[kb][ri] : -INFINITY;
      }
  }

  float mx = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int ri = 0; ri < 16; ++ri) mx = fmaxf(mx, s[kb][ri]);
  mx = fmaxf(mx, __shfl_xor(mx, 32));
  const float m_new = fmaxf(ws.m_run, mx * scale_log2);
  const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
  const float alpha = __builtin_amdgcn_exp2f(ws.m_run - m_use);
  ws.m_run = m_new;
  ws.l_run *= alpha;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int ri = 0; ri < 16; ++ri) ws.acc[db][ri] *= alpha;

  bf16x8 pf[4];  // P^T operand for step (kb, half) = 2 kb + half
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      bf16x8 v;
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        const float pe = __builtin_amdgcn_exp2f(
            __builtin_fmaf(s[kb][8 * half + e8], scale_log2, -m_use));
        ws.l_run += pe;
        v[e8] = (__bf16)pe;
      }
      pf[2 * kb + half] = v;
    }

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
      ws.acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[step], ws.acc[db], 0, 0, 0);
    }
  }
}

__global__ __launch_bounds__(512, 1) void attn_fwd_kernel(FwdParams p) {
  // Two stage buffers as distinct LDS objects, so that reads of one are known
  // not to alias the direct loads in flight into the other.
  __shared__ __attribute__((aligned(1024))) char sbuf0[STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sbuf1[STAGE_BYTES];
  __shared__ __attribute__((aligned(16))) KDescDev skd0[2 * BK];
  __shared__ __attribute__((aligned(16))) KDescDev skd1[2 * BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int qb = w & 3;       // query block of this wave
  const int kg = w >> 2;      // key group of this wave
  const int jq = lane & 31;   // query column of this lane
  const int hh = lane >> 5;   // half-wave

  // XCD-aware unit order: consecutive workgroups of one XCD take consecutive
  // (head-major) units, so the q-tiles of a head share that XCD's L2.
  const int n_units = p.heads * p.nqt;
  const int per_xcd = (n_units + 7) >> 3;
  const int unit = (int)(blockIdx.x & 7) * per_xcd + (int)(blockIdx.x >> 3);
  if (unit >= n_units) return;
  const int h = unit / p.nqt;
  const int qt = unit - h * p.nqt;
  const int qrow = qt * BQ + qb * 32 + jq;

  // the tile list is read with scalar loads (constant address space)
  typedef const __attribute__((address_space(4))) int32_t* const_i32p;
  const const_i32p csr_ptr = (const_i32p)p.csr_ptr;
  const int e0 = csr_ptr[qt], e1 = csr_ptr[qt + 1];
  const int n_ent = e1 - e0;
  const int n_stage = (n_ent + 1) >> 1;
  const const_i32p ent = (const_i32p)p.csr_idx + e0;
  const int last = n_ent - 1;
  auto entry = [=](int e) { return ent[e < last ? e : last]; };
  const float scale_log2 = p.scale_log2;
  LoadCtx lc;
  lc.k_cache = p.k_cache;
  lc.v_cache = p.v_cache;
  lc.k_new = p.k_new;
  lc.v_new = p.v_new;
  lc.kdesc = p.kdesc;
  lc.hc = (int64_t)h * p.cache_cap * D;
  lc.hn = (int64_t)h * D;
  lc.kv_stride = p.kv_stride;
  lc.nk = p.nk;
  lc.n_cached = p.n_cached;

  // CSR entries run one stage ahead of the loads they drive
  int cur0 = 0, cur1 = 0, nxt0 = 0, nxt1 = 0;
  if (n_stage > 0) {
    cur0 = entry(0);
    cur1 = entry(1);
    nxt0 = entry(2);
    nxt1 = entry(3);
    issue_stage(lc, sbuf0, skd0, cur0 >> 1, cur1 >> 1, w, lane);
  }

  WaveState ws;
  if (qrow < p.nq) {
    const uint16_t* src = p.q + (int64_t)qrow * p.q_stride + (int64_t)h * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < 8; ++s) ws.qf[s] = *reinterpret_cast<const bf16x8*>(src + 16 * s);
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) ws.qf[s] = bf16x8{};
  }
  ws.qd = p.qdesc[qrow];  // padded to whole tiles
#pragma unroll
  for (int db = 0; db < 4; ++db) ws.acc[db] = f32x16{};
  ws.m_run = -INFINITY;
  ws.l_run = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const int row = 32 * kb + kmap(jq);
    ws.k_off[kb] = row * 256;
    ws.k_swz[kb] = swz(row);
  }

  // stage st computes from buffer st & 1 while stage st + 1 loads into the other
  auto body = [&](int st, const char* cbuf, const KDescDev* ckd, char* nbuf, KDescDev* nkd) {
    wait_vm_all();
    __syncthreads();  // stage st landed for every wave; stage st-1 fully consumed
    const int a0 = cur0, a1 = cur1;
    if (st + 1 < n_stage) {
      issue_stage(lc, nbuf, nkd, nxt0 >> 1, nxt1 >> 1, w, lane);
      cur0 = nxt0;
      cur1 = nxt1;
      nxt0 = entry(2 * st + 4);
      nxt1 = entry(2 * st + 5);
    }
    if (2 * st + kg < n_ent) {
      const int a = kg ? a1 : a0;
      tile_step(ws, cbuf + (2 * kg) * TILE_BYTES, cbuf + (2 * kg + 1) * TILE_BYTES,
                ckd + kg * BK, a & 1, scale_log2, hh, lane);
    }
  };
  for (int st = 0; st < n_stage; st += 2) {
    body(st, sbuf0, skd0, sbuf1, skd1);
    if (st + 1 < n_stage) body(st + 1, sbuf1, skd1, sbuf0, skd0);
  }

  // ---- merge key group 1 into group 0 ------------------------------------------
  wait_vm_all();
  __syncthreads();  // all compute done; the stage buffers are free
  float* xf = reinterpret_cast<float*>(qb < 2 ? sbuf0 : sbuf1) + (qb & 1) * (66 * 64);
  if (kg == 1) {
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int ri = 0; ri < 16; ++ri) xf[(16 * db + ri) * 64 + lane] = ws.acc[db][ri];
    xf[64 * 64 + lane] = ws.m_run;
    xf[65 * 64 + lane] = ws.l_run;
  }
  __syncthreads();
  if (kg == 1) return;
  {
    const float m1 = xf[64 * 64 + lane], l1 = xf[65 * 64 + lane];
    const float m = fmaxf(ws.m_run, m1);
    const float mu = (m == -INFINITY) ? 0.f : m;
    const float a0 = __builtin_amdgcn_exp2f(ws.m_run - mu), a1 = __builtin_amdgcn_exp2f(m1 - mu);
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int ri = 0; ri < 16; ++ri)
        ws.acc[db][ri] = ws.acc[db][ri] * a0 + xf[(16 * db + ri) * 64 + lane] * a1;
    ws.l_run = ws.l_run * a0 + l1 * a1;
    ws.m_run = m;
  }

  // ---- epilogue ---------------------------------------------------------------
  const float l_tot = ws.l_run + __shfl_xor(ws.l_run, 32);
  if (qrow < p.nq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* dst = p.o + (int64_t)qrow * p.o_stride + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hh;
        uint2 pk;
        pk.x = (uint32_t)f2bf(ws.acc[db][4 * g + 0] * inv) | ((uint32_t)f2bf(ws.acc[db][4 * g + 1] * inv) << 16);
        pk.y = (uint32_t)f2bf(ws.acc[db][4 * g + 2] * inv) | ((uint32_t)f2bf(ws.acc[db][4 * g + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(dst + d0) = pk;
      }
    if (p.lse && hh == 0) {
      // natural-log LSE = (m_log2 + log2 l) * ln 2
      p.lse[(int64_t)h * p.nq + qrow] =
          l_tot > 0.f ? (ws.m_run + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd(const FwdParams& p, hipStream_t stream) {
  if (p.nq == 0) return hipSuccess;
  const int n_units = p.nqt * p.heads;
  const int per_xcd = (n_units + 7) / 8;
  dim3 grid((unsigned)(per_xcd * 8)), block(64 * NWAVES);
  hipLaunchKernelGGL(attn_fwd_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace nomas
