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
// once, against a few dozen camera keys at most.  A workgroup (four waves of
// 32 query tokens) works through groups of 128 consecutive tokens of one
// head, the groups grp, grp + G, grp + 2 G, ... (G = gridDim.y, sized to two
// workgroups per CU), and fetches the next group's Q rows while it computes
// the current one.  The heads of a token group are neighbouring workgroups,
// so the 4 KB rows of Q and O are read and written whole at about the same
// time.  All traffic moves whole rows: Q and the camera K / V rows arrive by
// direct HBM -> LDS loads (global_load_lds_dwordx4), O leaves through LDS,
// four 256-byte head rows per store instruction.  The products run on MFMA
// (v_mfma_f32_32x32x16_bf16) in the orientation of the forward attention:
//   S^T (32 camera keys x 32 queries) = K_c Q^T  -- both from LDS
//   O^T (128 dims x 32 queries)     += V_c^T P^T -- V_c^T by LDS transpose reads
// so that each lane holds one query's scores (softmax in-lane plus one
// half-wave exchange) and P stays in registers as the second product's
// operand (split into two bf16 parts, see below).  Camera keys are taken 32
// at a time with a running max and sum, so any number of camera tokens per
// query works.
#include "tile_common.h"

namespace nomas {
namespace {

constexpr int CAM_WAVES = CAM_GROUP / 32;
constexpr int CAM_KEYS = 32;                       // camera keys per chunk
constexpr int CAM_TILE_BYTES = CAM_KEYS * D * 2;   // 8 KB: 32 rows of one head
constexpr int CAM_GRP = CAM_KEYS * 64;             // chunk-group stride of the V tile
constexpr int CAM_Q_LOADS = 8;                     // direct loads per wave for its 32 Q rows

// Row tiles (Q, O, K_c: 32 rows x 16 chunks of 16 B): chunk c of row r in
// 16-byte slot 16 r + (c ^ (r % 16)).  A 16-lane phase reading one chunk of
// 16 rows distinct mod 16, or one whole row, covers the 64 banks once.
__device__ __forceinline__ int slot_off(int r, int c) { return 16 * (16 * r + (c ^ (r & 15))); }

// The camera range of group grp (uniform), by scalar loads: a vector load
// here would make the compiler wait for every load in flight.
__device__ __forceinline__ int2 group_range(const CamParams& p, int grp) {
  const const_i32p g = (const_i32p)p.grange;
  const int i = __builtin_amdgcn_readfirstlane(2 * grp);
  return int2{g[i], g[i + 1]};
}

// s_waitcnt vmcnt(N), ordered against the compiler's LDS accesses: the direct
// loads are issued through inline asm, so their completion must be waited
// for explicitly before the LDS they fill is read.
template <int N>
__device__ __forceinline__ void wait_vm_mem() {
  static_assert(N >= 0 && N < 16, "vmcnt range used here");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// This wave's 32 Q rows of a group into its row tile: load j moves rows
// 4 j .. 4 j + 3 whole (lane l: row 4 j + l / 16, chunk (l % 16) ^ (row % 16),
// which lands in slot 16 row + l % 16).  Rows past nq read row nq - 1
// (computed, never stored).
__device__ __forceinline__ void issue_q(const CamParams& p, int q0, int h, char* rt, int lane) {
#pragma unroll
  for (int j = 0; j < CAM_Q_LOADS; ++j) {
    const int r = 4 * j + (lane >> 4), c = (lane & 15) ^ (r & 15);
    const int row = min(q0 + r, p.nq - 1);
    dma16(p.q + (int64_t)row * p.q_stride + (int64_t)h * D + 8 * c, rt + 1024 * j);
  }
}

// Camera rows c0 .. c0 + 31 of K (row-tile layout) and V (transpose-read
// layout) of head h; wave w moves two 1 KB blocks of each.  Rows past the
// range read its last row: finite values whose scores are masked (P = 0).
__device__ __forceinline__ void issue_kv(const CamParams& p, int c0, int c_end, int h, char* ktile,
                                         char* vtile, int w, int lane) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int j = 2 * w + i;  // K: rows 4 j .. 4 j + 3
    const int r = 4 * j + (lane >> 4), c = (lane & 15) ^ (r & 15);
    const int row = min(c0 + r, c_end - 1);
    dma16(p.kc + (int64_t)row * p.cam_stride + (int64_t)h * D + 8 * c, ktile + 1024 * j);
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int b = 2 * w + i, cg = b >> 1, rb = b & 1;  // V: chunks 4 cg .. +3 of rows 16 rb .. +15
    const int r = 16 * rb + (lane >> 2), c = 4 * cg + ((lane & 3) ^ ((r >> 2) & 3));
    const int row = min(c0 + r, c_end - 1);
    dma16(p.vc + (int64_t)row * p.cam_stride + (int64_t)h * D + 8 * c, vtile + CAM_GRP * cg + 1024 * rb);
  }
}

__global__ __launch_bounds__(64 * CAM_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2))) void camera_attn_kernel(CamParams p) {
  __shared__ __attribute__((aligned(1024))) char ktile[CAM_TILE_BYTES];
  // V_c chunk in the transpose-read layout of tile_common.h (32 rows): chunk c
  // of row r at (c / 4) * 2048 + 64 r + 16 ((c % 4) ^ ((r / 4) % 4))
  __shared__ __attribute__((aligned(1024))) char vtile[CAM_TILE_BYTES];
  // per wave, two row tiles: the current group's Q (then O) and the next Q
  __shared__ __attribute__((aligned(1024))) char rtiles[2 * CAM_WAVES * CAM_TILE_BYTES];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int h = (int)blockIdx.x;
  const int G = (int)gridDim.y;
  const int jq = lane & 31, hh = lane >> 5;
  const int krow = kmap(jq);
  const float scale_log2 = p.scale_log2;
  int vbase[2];  // V^T transpose-read bases for key rows +0 / +4
  {
    const int tr_j = (lane & 15) >> 2, tr_c4 = lane & 3;
    const int x = 2 * ((lane >> 4) & 1) + (tr_c4 >> 1);
#pragma unroll
    for (int r = 0; r < 2; ++r)
      vbase[r] = (8 * hh + tr_j + 4 * r) * 64 + 16 * (x ^ (2 * hh + r)) + 8 * (tr_c4 & 1);
  }

  int grp = (int)blockIdx.y;
  // the ranges of the group's tokens are read one group ahead, before that
  // group's Q loads are issued, so that the waits below cover them
  int2 qr_next = p.qrange[grp * CAM_GROUP + 32 * w + jq];
  issue_q(p, grp * CAM_GROUP + 32 * w, h, rtiles + w * CAM_TILE_BYTES, lane);
  for (int it = 0; grp < p.n_groups; ++it, grp += G) {
    char* rt = rtiles + ((it & 1) * CAM_WAVES + w) * CAM_TILE_BYTES;
    const int q0 = grp * CAM_GROUP + 32 * w;  // this wave's first query token
    const int2 gr = group_range(p, grp);            // union of the group's ranges (empty: x == y)
    const int2 qr = qr_next;                  // this lane's query
    // the previous group released the K / V tiles at its closing barrier
    if (gr.y > gr.x) issue_kv(p, gr.x, gr.y, h, ktile, vtile, w, lane);
    const int nxt = grp + G;
    if (nxt < p.n_groups) {
      qr_next = p.qrange[nxt * CAM_GROUP + 32 * w + jq];
      issue_q(p, nxt * CAM_GROUP + 32 * w, h, rtiles + (((it + 1) & 1) * CAM_WAVES + w) * CAM_TILE_BYTES, lane);
      wait_vm_mem<CAM_Q_LOADS + 1>();  // all but the next group's range load and Q rows
    } else {
      wait_vm_mem<0>();
    }
    __syncthreads();  // every wave's part of the K / V chunk

    f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
    float m_run = -INFINITY;  // log2 domain, same in both half-waves
    float l_run = 0.f;        // this half-wave's share of the sum
    if (gr.y > gr.x) {        // uniform over the workgroup
      bf16x8 qf[8];  // B operand: query jq, dims 16 s + 8 hh .. + 7
#pragma unroll
      for (int s8 = 0; s8 < 8; ++s8) qf[s8] = *reinterpret_cast<const bf16x8*>(rt + slot_off(jq, 2 * s8 + hh));
      for (int c0 = gr.x; c0 < gr.y; c0 += CAM_KEYS) {
        if (c0 != gr.x) {  // a further chunk (more than 32 camera tokens in the group)
          __syncthreads();
          issue_kv(p, c0, gr.y, h, ktile, vtile, w, lane);
          wait_vm_mem<0>();
          __syncthreads();
        }
        // S^T: row i of the product is key c0 + kmap(i), so register ri of the
        // result holds key c0 + 16 (ri / 8) + 8 hh + ri % 8
        f32x16 s = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 8; ++ks) {
          const bf16x8 kf = *reinterpret_cast<const bf16x8*>(ktile + slot_off(krow, 2 * ks + hh));
          s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s, 0, 0, 0);
        }
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
        // P as the sum of two bf16 parts (hi = P rounded, lo = the rest
        // rounded): with a few keys per query the outputs are close to single
        // V rows, and one bf16 rounding of P would add an error comparable to
        // the output's own rounding; two products keep P to about 16 bits, at
        // no cost that shows in a memory-bound kernel
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
        // O^T += V^T P^T over the two 16-key steps
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
    // O = acc / l in bf16 (0 for rows that see no camera token), staged in
    // this wave's row tile (its Q rows are no longer read), then stored four
    // whole rows per instruction.  LDS accesses of one wave complete in order.
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {  // dims 32 db + 8 g + 4 hh .. + 3: chunk 4 db + g, half hh
        uint2 pk;
        pk.x = (uint32_t)f2bf(acc[db][4 * g + 0] * inv) | ((uint32_t)f2bf(acc[db][4 * g + 1] * inv) << 16);
        pk.y = (uint32_t)f2bf(acc[db][4 * g + 2] * inv) | ((uint32_t)f2bf(acc[db][4 * g + 3] * inv) << 16);
        *reinterpret_cast<uint2*>(rt + slot_off(jq, 4 * db + g) + 8 * hh) = pk;
      }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = 4 * j + (lane >> 4), c = lane & 15;
      const uint4 v = *reinterpret_cast<const uint4*>(rt + slot_off(r, c));
      if (q0 + r < p.nq) *reinterpret_cast<uint4*>(p.o + (int64_t)(q0 + r) * p.o_stride + (int64_t)h * D + 8 * c) = v;
    }
    __syncthreads();  // the K / V tiles are free for the next group
  }
}

}  // namespace

int camera_attn_groups_per_cu() { return 2; }

hipError_t launch_camera_attn(const CamParams& p, int cus, hipStream_t stream) {
  if (p.n_groups <= 0 || p.heads <= 0) return hipSuccess;
  const int per_head = std::max(1, camera_attn_groups_per_cu() * cus / p.heads);
  const int gy = std::min(p.n_groups, per_head);
  hipLaunchKernelGGL(camera_attn_kernel, dim3((unsigned)p.heads, (unsigned)gy), dim3(64 * CAM_WAVES), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace nomas
