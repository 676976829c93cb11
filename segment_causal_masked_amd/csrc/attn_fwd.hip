// Forward kernel of action-aware causal attention for gfx950 (CDNA4).
//
// Computes O = softmax(scale * Q K^T + M) V with M = -inf on hidden pairs
// (the mask of "Summary (Overview)", Model Architecture: Segment-wise and
// Action-Aware Causal Attention), flash-style: one workgroup owns a 128-query
// tile of one head and walks only the non-empty 64-key tiles of its row of the
// tile map; FULL tiles run unmasked, PARTIAL (or ragged) tiles evaluate the
// per-token descriptors.  Online softmax keeps a running max and sum per query
// in fp32, so the result equals the plain softmax up to rounding.
//
// MFMA formulation (v_mfma_f32_32x32x16_bf16, fp32 accumulate), per wave of
// 32 queries:
//   S^T (64 keys x 32 queries) = K_tile * Q^T   -- K from LDS, Q in registers
//   O^T (128 dims x 32 queries) += V^T * P^T    -- V^T from LDS, P^T in regs
// Computing the transposes puts one query per lane column, so row max / row
// sum of the softmax are in-lane over 32 keys plus one exchange between the
// two half-waves, and the rescale factor is a per-lane scalar.  Key rows of
// the S^T MFMA are permuted (kmap) so that each half-wave ends up holding 8
// consecutive keys per 16-key step, which is exactly the B operand layout of
// the P^T V^T product: P never leaves registers.
#include "kernels.h"

namespace nomas {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int D = 128;
constexpr int BQ = 128;
constexpr int BK = 64;
constexpr int KS = D + 8;   // LDS row stride of K (elements): 272 B rows
constexpr int VS = BK + 8;  // LDS row stride of V^T (elements): 144 B rows

// MFMA output row i (of 32) -> key offset inside a 32-key block.
__device__ __forceinline__ int kmap(int i) {
  const int g = i >> 3, q = (i >> 2) & 1, r = i & 3;
  return 16 * (g >> 1) + 8 * q + 4 * (g & 1) + r;
}

__device__ __forceinline__ bool visible(const QDescDev& q, int kseg, uint32_t kbits) {
  return kseg >= q.lo && kseg <= q.seg &&
         (kbits == 0u || (kseg == q.seg && (q.amask & kbits) != 0u));
}

__device__ __forceinline__ uint16_t f2bf(float x) {
  __bf16 b = (__bf16)x;  // round to nearest even
  return __builtin_bit_cast(uint16_t, b);
}

__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(FwdParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[BK * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sVt[D * VS];
  __shared__ KDescDev sKd[BK];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int jq = lane & 31;   // query column of this lane
  const int hh = lane >> 5;   // half-wave

  const int unit = blockIdx.x;
  const int h = unit % p.heads;
  const int qt = unit / p.heads;
  const int qrow = qt * BQ + w * 32 + jq;

  // Q fragment: query qrow, dims [16 s + 8 hh, +8) for s = 0..7.
  bf16x8 qf[8];
  if (qrow < p.nq) {
    const uint16_t* src = p.q + (int64_t)qrow * p.q_stride + (int64_t)h * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = *reinterpret_cast<const bf16x8*>(src + 16 * s);
  } else {
#pragma unroll
    for (int s = 0; s < 8; ++s) qf[s] = bf16x8{};
  }
  const QDescDev qd = p.qdesc[qrow];  // padded to whole tiles

  f32x16 acc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY;  // running max, log2 domain
  float l_run = 0.f;        // this half-wave's share of the running sum

  const int e0 = p.csr_ptr[qt], e1 = p.csr_ptr[qt + 1];
  for (int e = e0; e < e1; ++e) {
    const int ent = p.csr_idx[e];
    const int kt = ent >> 1;
    const bool masked = ent & 1;

    __syncthreads();  // previous tile fully consumed
    // ---- stage K (row-major) and V^T into LDS --------------------------------
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      const int idx = pass * 256 + tid;
      const int row = idx >> 4, c = idx & 15;
      const int key = kt * BK + row;
      uint4 kv = make_uint4(0, 0, 0, 0), vv = make_uint4(0, 0, 0, 0);
      if (key < p.nk) {
        const uint16_t *ks, *vs;
        if (key < p.n_cached) {
          const int64_t off = ((int64_t)h * p.cache_cap + key) * D + 8 * c;
          ks = p.k_cache + off;
          vs = p.v_cache + off;
        } else {
          const int64_t off = (int64_t)(key - p.n_cached) * p.kv_stride + (int64_t)h * D + 8 * c;
          ks = p.k_new + off;
          vs = p.v_new + off;
        }
        kv = *reinterpret_cast<const uint4*>(ks);
        vv = *reinterpret_cast<const uint4*>(vs);
      }
      *reinterpret_cast<uint4*>(sK + row * KS + 8 * c) = kv;
      const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sVt[(8 * c + 2 * j) * VS + row] = (uint16_t)(vw[j] & 0xffffu);
        sVt[(8 * c + 2 * j + 1) * VS + row] = (uint16_t)(vw[j] >> 16);
      }
    }
    if (masked && tid < BK) sKd[tid] = p.kdesc[kt * BK + tid];
    __syncthreads();

    // ---- S^T = K Q^T for the wave's 32 queries ------------------------------
    f32x16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = f32x16{};
      const uint16_t* krow = sK + (32 * kb + kmap(jq)) * KS + 8 * hh;
#pragma unroll
      for (int st = 0; st < 8; ++st) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(krow + 16 * st);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[st], s[kb], 0, 0, 0);
      }
    }
    // register ri of block kb holds key 32 kb + 16 (ri / 8) + 8 hh + ri % 8
    if (masked) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int ri = 0; ri < 16; ++ri) {
          const KDescDev kd = sKd[32 * kb + 16 * (ri >> 3) + 8 * hh + (ri & 7)];
          if (!visible(qd, kd.seg, kd.bits)) s[kb][ri] = -INFINITY;
        }
    }

    // ---- online softmax -------------------------------------------------------
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ri = 0; ri < 16; ++ri) mx = fmaxf(mx, s[kb][ri]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * p.scale_log2);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int ri = 0; ri < 16; ++ri) acc[db][ri] *= alpha;

    bf16x8 pf[4];  // P^T operand for step (kb, half) = 2 kb + half
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        bf16x8 v;
#pragma unroll
        for (int e8 = 0; e8 < 8; ++e8) {
          const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][8 * half + e8], p.scale_log2, -m_use));
          l_run += pe;
          v[e8] = (__bf16)pe;
        }
        pf[2 * kb + half] = v;
      }

    // ---- O^T += V^T P^T ---------------------------------------------------------
#pragma unroll
    for (int step = 0; step < 4; ++step) {
      const int koff = 16 * step + 8 * hh;  // keys of this half-wave's 8 k-slots
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(sVt + (32 * db + jq) * VS + koff);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[step], acc[db], 0, 0, 0);
      }
    }
  }

  // ---- epilogue ---------------------------------------------------------------
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (qrow < p.nq) {
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    uint16_t* dst = p.o + (int64_t)qrow * p.o_stride + (int64_t)h * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = 32 * db + 8 * g + 4 * hh;
        uint2 pk;
        pk.x = (uint32_t)f2bf(acc[db][4 * g + 0] * inv) | ((uint32_t)f2bf(acc[db][4 * g + 1] * inv) << 16);
        pk.y = (uint32_t)f2bf(acc[db][4 * g + 2] * inv) | ((uint32_t)f2bf(acc[db][4 * g + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(dst + d0) = pk;
      }
    if (p.lse && hh == 0) {
      // natural-log LSE = (m_log2 + log2 l) * ln 2
      p.lse[(int64_t)h * p.nq + qrow] =
          l_tot > 0.f ? (m_run + __log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_attn_fwd(const FwdParams& p, hipStream_t stream) {
  if (p.nq == 0) return hipSuccess;
  dim3 grid((unsigned)(p.nqt * p.heads)), block(256);
  hipLaunchKernelGGL(attn_fwd_kernel, grid, block, 0, stream, p);
  return hipGetLastError();
}

}  // namespace nomas
