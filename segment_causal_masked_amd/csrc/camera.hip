// Camera cross-attention for gfx950 (CDNA4).
//
// "Summary (Overview)", Model Architecture, Camera-Trajectory Conditioning
// (Eq. 3): the video tokens are the queries of a cross-attention whose keys
// and values are camera tokens, one per latent frame (each stands for a group
// of four frames).  Per head, O = softmax(scale * Q K_c^T + M_c) V_c, where
// query token t sees the camera tokens of the range the plan gives it (its
// own segment's, within a frame radius); a row that sees none is written as
// zeros.
//
// The work is HBM-bound: each query row is read once and its output written
// once, against a few dozen camera keys at most, so the kernel is shaped for
// coalesced row traffic and many waves in flight: one wave per (32 query
// tokens, head), four heads per workgroup (1 KB of every query row per
// workgroup).  The two products still run on MFMA (v_mfma_f32_32x32x16_bf16),
// in the orientation of the forward attention kernel:
//   S^T (32 camera keys x 32 queries) = K_c Q^T  -- K_c rows from L2, Q in registers
//   O^T (128 dims x 32 queries)     += V_c^T P^T -- V_c^T by LDS transpose reads
// so that each lane holds one query's scores (softmax in-lane plus one
// half-wave exchange) and P stays in registers as the second product's
// operand (split into two bf16 parts, see below).  Camera keys are taken 32 at a time with a running max and sum, so
// any number of camera tokens per query works.
#include "tile_common.h"

namespace nomas {
namespace {

constexpr int CAM_WAVES = 4;
constexpr int CAM_KEYS = 32;                       // camera keys per chunk
constexpr int CAM_TILE_BYTES = CAM_KEYS * D * 2;   // 8 KB: one V_c chunk
constexpr int CAM_GRP = CAM_KEYS * 64;             // chunk-group stride of that tile

__global__ __launch_bounds__(64 * CAM_WAVES) void camera_attn_kernel(CamParams p) {
  // one V_c chunk per wave, in the swizzled tile layout of tile_common.h
  // (32 rows): chunk c of row r at (c / 4) * 2048 + 64 r + 16 ((c % 4) ^ ((r / 4) % 4))
  __shared__ __attribute__((aligned(1024))) char vtiles[CAM_WAVES * CAM_TILE_BYTES];
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int h = (int)blockIdx.y * CAM_WAVES + w;
  if (h >= p.heads) return;  // whole waves; no workgroup barrier below
  const int jq = lane & 31, hh = lane >> 5;
  const int blk = (int)blockIdx.x;
  const int qrow = blk * 32 + jq;
  char* vtile = vtiles + w * CAM_TILE_BYTES;
  const float scale_log2 = p.scale_log2;

  const int2 br = p.brange[blk];   // union of the block's ranges (empty: x == y)
  const int2 qr = p.qrange[qrow];  // this lane's query (n_blocks * 32 entries)
  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  float m_run = -INFINITY;  // log2 domain, same in both half-waves
  float l_run = 0.f;        // this half-wave's share of the sum
  if (br.y > br.x) {
    bf16x8 qf[8];
    if (qrow < p.nq) {
      const uint16_t* src = p.q + (int64_t)qrow * p.q_stride + (int64_t)h * D + 8 * hh;
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) qf[s8] = *reinterpret_cast<const bf16x8*>(src + 16 * s8);
    } else {
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) qf[s8] = bf16x8{};
    }
    int vbase[2];  // V^T transpose-read bases for key rows +0 / +4
    {
      const int tr_j = (lane & 15) >> 2, tr_c4 = lane & 3;
      const int x = 2 * ((lane >> 4) & 1) + (tr_c4 >> 1);
#pragma unroll
      for (int r = 0; r < 2; ++r)
        vbase[r] = (8 * hh + tr_j + 4 * r) * 64 + 16 * (x ^ (2 * hh + r)) + 8 * (tr_c4 & 1);
    }
    for (int c0 = br.x; c0 < br.y; c0 += CAM_KEYS) {
      // K_c as the A operand: row i of the product is key c0 + kmap(i), so
      // register ri of the result holds key c0 + 16 (ri / 8) + 8 hh + ri % 8
      bf16x8 kf[8];
      const int kr = c0 + kmap(jq);
      if (kr < br.y) {
        const uint16_t* src = p.kc + (int64_t)kr * p.cam_stride + (int64_t)h * D + 8 * hh;
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) kf[s8] = *reinterpret_cast<const bf16x8*>(src + 16 * s8);
      } else {
#pragma unroll
        for (int s8 = 0; s8 < 8; ++s8) kf[s8] = bf16x8{};
      }
      // V_c chunk into this wave's LDS tile: 32 rows x 16 chunks of 16 B,
      // 16 lanes per row (256 contiguous bytes); rows past the range are 0
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int idx = 64 * j + lane, r = idx >> 4, c = idx & 15;
        uint4 val = uint4{0u, 0u, 0u, 0u};
        if (c0 + r < br.y)
          val = *reinterpret_cast<const uint4*>(p.vc + (int64_t)(c0 + r) * p.cam_stride +
                                                (int64_t)h * D + 8 * c);
        *reinterpret_cast<uint4*>(vtile + (c >> 2) * CAM_GRP + 64 * r + 16 * ((c & 3) ^ ((r >> 2) & 3))) = val;
      }
      f32x16 s = f32x16{};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ks], qf[ks], s, 0, 0, 0);
      float mx = -INFINITY;
#pragma unroll
      for (int ri = 0; ri < 16; ++ri) {
        const int key = c0 + 16 * (ri >> 3) + 8 * hh + (ri & 7);
        const bool vis = (key >= qr.x) & (key < qr.y);
        s[ri] = vis ? s[ri] * scale_log2 : -INFINITY;
        mx = fmaxf(mx, s[ri]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run, mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;  // no visible key yet: P = 0
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db) acc[db] *= alpha;
      // P as the sum of two bf16 parts (hi = P rounded, lo = the rest rounded):
      // with a few keys per query the outputs are close to single V rows, and
      // one bf16 rounding of P would add an error comparable to the output's
      // own rounding; two products keep P to about 16 bits, at no cost that
      // shows in a memory-bound kernel
      bf16x8 pf[2], pl[2];
      float ls = 0.f;
#pragma unroll
      for (int ri = 0; ri < 16; ++ri) {
        const float pe = __builtin_amdgcn_exp2f(s[ri] - m_use);
        ls += pe;
        const __bf16 ph = (__bf16)pe;
        pf[ri >> 3][ri & 7] = ph;
        pl[ri >> 3][ri & 7] = (__bf16)(pe - (float)ph);
      }
      l_run += ls;
      // O^T += V^T P^T over the two 16-key steps (the LDS writes above are this
      // wave's own and complete in order before these reads)
#pragma unroll
      for (int step = 0; step < 2; ++step)
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const char* a = vtile + CAM_GRP * db + 1024 * step;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4p)(a + vbase[0]));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4p)(a + vbase[1]));
          const bf16x8 vf = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pl[step], acc[db], 0, 0, 0);
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[step], acc[db], 0, 0, 0);
        }
    }
  }
  if (qrow >= p.nq) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  uint16_t* dst = p.o + (int64_t)qrow * p.o_stride + (int64_t)h * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      uint2 pk;
      pk.x = (uint32_t)f2bf(acc[db][4 * g + 0] * inv) | ((uint32_t)f2bf(acc[db][4 * g + 1] * inv) << 16);
      pk.y = (uint32_t)f2bf(acc[db][4 * g + 2] * inv) | ((uint32_t)f2bf(acc[db][4 * g + 3] * inv) << 16);
      *reinterpret_cast<uint2*>(dst + 32 * db + 8 * g + 4 * hh) = pk;
    }
}

}  // namespace

hipError_t launch_camera_attn(const CamParams& p, hipStream_t stream) {
  if (p.n_blocks <= 0 || p.heads <= 0) return hipSuccess;
  hipLaunchKernelGGL(camera_attn_kernel, dim3((unsigned)p.n_blocks, (unsigned)((p.heads + CAM_WAVES - 1) / CAM_WAVES)),
                     dim3(64 * CAM_WAVES), 0, stream, p);
  return hipGetLastError();
}

}  // namespace nomas
