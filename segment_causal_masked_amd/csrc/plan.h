// Host-side plan core: layout validation, per-token descriptors, tile classes,
// CSR/CSC lists of non-empty tiles and the unmasked-pair count A.
// Plain C++17, no HIP: it builds and runs on any host.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "nomas_attn.h"

namespace nomas {

// Per-token descriptors the kernels read (layout shared with the device code).
//   query: seg   internal ordinal of the query's segment, -1 for padding
//          lo    ordinal of the first segment of the query's video
//          amask bit k set = the query sees tail a_k of its own segment
//   key:   seg   ordinal of the key's segment, -1 for padding
//          bits  (1 << k) for a token of tail a_k, 0 for video / head tokens
// visible(q, k) = lo_q <= seg_k <= seg_q
//                 && (bits_k == 0 || (seg_k == seg_q && (amask_q & bits_k)))
// Ordinals number the distinct (video, index) pairs in lexicographic order, so
// "same video and index_k <= index_q" is the ordinal range [lo_q, seg_q].
struct QDesc {
  int32_t seg, lo;
  uint32_t amask;
  int32_t pad_;
};
struct KDesc {
  int32_t seg;
  uint32_t bits;
};

inline bool visible(const QDesc& q, const KDesc& k) {
  return k.seg >= q.lo && k.seg <= q.seg &&
         (k.bits == 0u || (k.seg == q.seg && (q.amask & k.bits) != 0u));
}

// Forward work schedule.  A forward unit is a pair of consecutive query tiles
// (q-tiles 2 u' and 2 u' + 1) of one head: unit = head * n_pairs + u'.  Its
// entries are the union of the two q-tiles' non-empty key tiles, each entry
// = (k_tile << 4) | flags: bit 0 / 1 = the first / second q-tile needs the
// per-element mask there, bit 2 / 3 = the tile is EMPTY for the first /
// second q-tile (its waves skip it).  The (unit, entry) iterations are cut
// into ranges of equal estimated cost, one or (training packs, in phases of
// one head and video per XCD) several per persistent workgroup; a unit cut
// by a range boundary becomes several pieces whose partial results are
// merged afterwards.
struct Piece {
  int32_t unit, e_begin, e_end, slot;  // slot = partial-result slot, -1 = final
};
struct CombineItem {
  int32_t unit, first_slot, n_pieces, pad_;
};

// CSR/CSC entry: (tile << 1) | needs_mask, needs_mask = PARTIAL class or a
// ragged last key tile (columns past the end must be masked).
struct HostPlan {
  int32_t heads = 0, head_dim = 0, bq = 0, bk = 0, mode = 0;
  int64_t nq = 0, nk = 0, n_cached = 0;
  int64_t nqt = 0, nkt = 0;
  std::vector<QDesc> qdesc;   // nqt * bq entries (tail padded with seg = -1)
  std::vector<KDesc> kdesc;   // nkt * bk entries (tail padded with seg = -1)
  std::vector<uint8_t> classes;  // nqt * nkt, NOMAS_TILE_*
  std::vector<int32_t> csr_ptr, csr_idx;  // per q-tile
  // per CSR entry: 1 if some query of the tile that sees any key at all (a
  // live row: not padding) misses a key of the tile, or the key tile is
  // ragged -- the per-element mask the forward and dQ kernels need.  Rows
  // that see no key are computed unmasked there and written as zeros.
  std::vector<uint8_t> csr_live_mask;
  std::vector<int32_t> csc_ptr, csc_idx;  // per k-tile
  int64_t n_empty = 0, n_full = 0, n_partial = 0;
  int64_t unmasked_pairs = 0, executed_pairs = 0;
  // forward schedule (build_fwd_schedule)
  int64_t n_pairs = 0;                // ceil(nqt / 2)
  std::vector<int32_t> pair_ptr, pair_idx;  // merged entry lists per q-tile pair
  int32_t fwd_groups = 0;
  std::vector<int32_t> wg_ptr;        // fwd_groups + 1
  std::vector<Piece> pieces;          // per workgroup (wg_ptr), then the n_chunks
  int32_t n_chunks = 0;               // tail chunks any workgroup claims in turn
  std::vector<CombineItem> combine;
  int32_t n_slots = 0;
  // per unit: its entries are visited in the rotated order
  // (j + unit_shift) mod n for j = 0 .. n - 1; pieces are ranges of j
  std::vector<int32_t> unit_shift;
  // video-block sparsity (keep_percent > 0): per key tile, 1 if every key in
  // it is a video token; per pair, the prefix of its sparse list lengths
  // (non-video entries + ceil(keep_percent% of its video entries)); the
  // lists themselves are chosen on the device per head.
  int32_t keep_percent = 0, window = 0;
  bool grad_f32 = false;  // nomas_attn_bwd writes fp32 gradients (NOMAS_PLAN_GRAD_F32)
  bool kv_head_major = false;  // new-token K / V (and dK / dV) are [H][n][128]
  std::vector<int32_t> video_tile;
  std::vector<int32_t> sp_ptr, sp_keep;
  int64_t sp_total = 0;
  // backward schedule (build_bwd_schedule): per pair of key tiles (2 u,
  // 2 u + 1) the union of their non-empty q-tiles, entry = (q_tile << 4) |
  // flags with bit 0 / 1 = mask for the first / second key tile (PARTIAL,
  // ragged key tile or ragged last q-tile), bit 2 / 3 = EMPTY for it
  int64_t n_kpairs = 0;
  std::vector<int32_t> kpair_ptr, kpair_idx;
};

// Cut the forward iterations into ranges of equal estimated cost for `groups`
// persistent workgroups.
void build_fwd_schedule(HostPlan* p, int32_t groups);

// Merged per-key-tile-pair lists for the dK / dV kernel.
void build_bwd_schedule(HostPlan* p);

// Identity of a cache's committed segments (used for stale-plan checks).
struct CacheState {
  int32_t n_segments = 0;
  uint64_t last_serial = 0;
};

// Validate one record; returns "" or a description of the problem.
std::string check_segment(const nomas_segment& s);
int64_t segment_tokens(const nomas_segment& s);
// Same identity (video, index) and the same record (sizes, action tails).
bool same_segment(const nomas_segment& a, const nomas_segment& b);
// Tokens of a segment that a KV cache keeps: its video and head tokens (the
// first ones).  Action tails are visible only inside their own segment and
// padding to nobody, so no later query can see them.
int64_t segment_cached_tokens(const nomas_segment& s);

// Invariants of a built plan (lists vs the class map, schedule coverage,
// slots); "" if they hold, else the first violation.
std::string validate_host_plan(const HostPlan& p);

// Build the host plan.  keys = cached ++ kv_new.  Returns NOMAS_OK or an
// error status with *err filled.
nomas_status build_host_plan(const std::vector<nomas_segment>& q,
                             const std::vector<nomas_segment>& cached,
                             const std::vector<nomas_segment>& kv_new,
                             const nomas_plan_opts& opts, HostPlan* out,
                             std::string* err);

}  // namespace nomas
