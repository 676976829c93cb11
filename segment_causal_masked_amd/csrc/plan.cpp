// Host-side plan core (no HIP).  See plan.h for the descriptor encoding.
//
// The rules encoded here are the visibility rules of action-aware causal
// attention: "Summary (Overview)" page, Model Architecture (Segment-wise
// Causal Attention; Action-Aware Causal Attention, Figure 6b), the onedev.kr
// review, section "무엇과 다른가", and packing of independent videos
// ("Summary (Overview)", Training Infrastructure).  Text-query readings
// R / K / H as documented in nomas_attn.h.
#include "plan.h"

#include <cmath>

#include <algorithm>
#include <climits>
#include <map>
#include <tuple>
#include <utility>

namespace nomas {

int64_t segment_tokens(const nomas_segment& s) {
  int64_t n = int64_t(s.n_frames) * s.tokens_per_frame + s.n_head + s.n_pad;
  for (int a = 0; a < s.n_actions && a < NOMAS_MAX_ACTIONS; ++a) n += s.actions[a].n_tokens;
  return n;
}

int64_t segment_cached_tokens(const nomas_segment& s) {
  return int64_t(s.n_frames) * s.tokens_per_frame + s.n_head;
}

std::string check_segment(const nomas_segment& s) {
  char buf[256];
  auto fail = [&](const char* what) {
    snprintf(buf, sizeof buf, "segment (video %d, index %d): %s", s.video, s.index, what);
    return std::string(buf);
  };
  if (s.video < 0 || s.index < 0) return fail("video and index must be >= 0");
  if (s.n_frames < 0 || s.tokens_per_frame < 0 || s.n_head < 0 || s.n_pad < 0)
    return fail("negative token count");
  if (s.n_actions < 0 || s.n_actions > NOMAS_MAX_ACTIONS)
    return fail("n_actions must be in [0, 32]");
  if (int64_t(s.n_frames) * s.tokens_per_frame > (int64_t(1) << 30))
    return fail("too many video tokens");
  for (int a = 0; a < s.n_actions; ++a) {
    const nomas_action& x = s.actions[a];
    if (x.n_tokens < 1) return fail("action with no tokens");
    if (!(0 <= x.frame_lo && x.frame_lo < x.frame_hi && x.frame_hi <= s.n_frames))
      return fail("action window must satisfy 0 <= lo < hi <= n_frames");
  }
  if (segment_tokens(s) < 1) return fail("empty segment");
  return "";
}

static bool same_record(const nomas_segment& a, const nomas_segment& b) {
  if (a.n_frames != b.n_frames || a.tokens_per_frame != b.tokens_per_frame ||
      a.n_head != b.n_head || a.n_actions != b.n_actions || a.n_pad != b.n_pad)
    return false;
  for (int i = 0; i < a.n_actions; ++i)
    if (a.actions[i].n_tokens != b.actions[i].n_tokens ||
        a.actions[i].frame_lo != b.actions[i].frame_lo ||
        a.actions[i].frame_hi != b.actions[i].frame_hi)
      return false;
  return true;
}

bool same_segment(const nomas_segment& a, const nomas_segment& b) {
  return a.video == b.video && a.index == b.index && same_record(a, b);
}

namespace {

using Ident = std::pair<int32_t, int32_t>;  // (video, index)

struct Run {
  int64_t start, len;
  int32_t d0, d1, d2;  // descriptor fields
};

// Query-side action mask of a video token at frame f.
uint32_t window_mask(const nomas_segment& s, int32_t f) {
  uint32_t m = 0;
  for (int a = 0; a < s.n_actions; ++a)
    if (s.actions[a].frame_lo <= f && f < s.actions[a].frame_hi) m |= (1u << a);
  return m;
}

uint32_t all_tails(const nomas_segment& s) {
  return s.n_actions >= 32 ? 0xffffffffu : ((1u << s.n_actions) - 1u);
}

// Runs of identical query descriptors for one segment, appended to out.
void q_runs(const nomas_segment& s, int32_t ord, int32_t lo, int mode, int64_t* pos,
            std::vector<Run>* out) {
  auto push = [&](int64_t n, int32_t seg, int32_t l, uint32_t m) {
    if (n <= 0) return;
    if (!out->empty()) {
      Run& r = out->back();
      if (r.start + r.len == *pos && r.d0 == seg && r.d1 == l && uint32_t(r.d2) == m) {
        r.len += n;
        *pos += n;
        return;
      }
    }
    out->push_back(Run{*pos, n, seg, l, int32_t(m)});
    *pos += n;
  };
  for (int32_t f = 0; f < s.n_frames; ++f) push(s.tokens_per_frame, ord, lo, window_mask(s, f));
  push(s.n_head, ord, lo, mode == NOMAS_TEXT_QUERY_H ? all_tails(s) : 0u);
  for (int a = 0; a < s.n_actions; ++a)
    push(s.actions[a].n_tokens, ord, lo, mode == NOMAS_TEXT_QUERY_K ? 0u : (1u << a));
  push(s.n_pad, -1, 0, 0u);
}

// cached: the segment as a KV cache holds it (video and head tokens only)
void k_runs(const nomas_segment& s, int32_t ord, int64_t* pos, std::vector<Run>* out,
            bool cached) {
  auto push = [&](int64_t n, int32_t seg, uint32_t bits) {
    if (n <= 0) return;
    if (!out->empty()) {
      Run& r = out->back();
      if (r.start + r.len == *pos && r.d0 == seg && uint32_t(r.d1) == bits) {
        r.len += n;
        *pos += n;
        return;
      }
    }
    out->push_back(Run{*pos, n, seg, int32_t(bits), 0});
    *pos += n;
  };
  push(int64_t(s.n_frames) * s.tokens_per_frame + s.n_head, ord, 0u);
  if (cached) return;
  for (int a = 0; a < s.n_actions; ++a) push(s.actions[a].n_tokens, ord, 1u << a);
  push(s.n_pad, -1, 0u);
}

inline QDesc qd_of(const Run& r) { return QDesc{r.d0, r.d1, uint32_t(r.d2), 0}; }
inline KDesc kd_of(const Run& r) { return KDesc{r.d0, uint32_t(r.d1)}; }

// For each tile [t*b, min(n,(t+1)*b)), the range [first, last] of runs it overlaps.
std::vector<std::pair<int32_t, int32_t>> tile_runs(const std::vector<Run>& runs, int64_t n,
                                                   int64_t b, int64_t ntiles) {
  std::vector<std::pair<int32_t, int32_t>> out(ntiles);
  size_t r = 0;
  for (int64_t t = 0; t < ntiles; ++t) {
    int64_t a = t * b, e = std::min(n, a + b);
    while (r < runs.size() && runs[r].start + runs[r].len <= a) ++r;
    size_t last = r;
    while (last + 1 < runs.size() && runs[last + 1].start < e) ++last;
    out[t] = {int32_t(r), int32_t(last)};
  }
  return out;
}

}  // namespace

nomas_status build_host_plan(const std::vector<nomas_segment>& q,
                             const std::vector<nomas_segment>& cached,
                             const std::vector<nomas_segment>& kv_new,
                             const nomas_plan_opts& opts, HostPlan* out, std::string* err) {
  HostPlan& p = *out;
  if (opts.num_heads < 1) { *err = "num_heads must be >= 1"; return NOMAS_ERR_INVALID_ARGUMENT; }
  if (opts.head_dim != NOMAS_HEAD_DIM) { *err = "head_dim must be 128"; return NOMAS_ERR_UNSUPPORTED; }
  if (opts.text_query_mode < 0 || opts.text_query_mode > 2) {
    *err = "text_query_mode must be R (0), K (1) or H (2)";
    return NOMAS_ERR_INVALID_ARGUMENT;
  }
  if (opts.flags & ~int32_t(NOMAS_PLAN_HOST_ONLY | NOMAS_PLAN_GRAD_F32 | NOMAS_PLAN_KV_HEAD_MAJOR)) { *err = "unknown plan flag"; return NOMAS_ERR_INVALID_ARGUMENT; }
  if (opts.window_segments < 0) { *err = "window_segments must be >= 0"; return NOMAS_ERR_INVALID_ARGUMENT; }
  if (opts.video_keep_percent < 0 || opts.video_keep_percent > 100) {
    *err = "video_keep_percent must be in [0, 100]";
    return NOMAS_ERR_INVALID_ARGUMENT;
  }
  p.keep_percent = opts.video_keep_percent;
  p.grad_f32 = (opts.flags & NOMAS_PLAN_GRAD_F32) != 0;
  p.kv_head_major = (opts.flags & NOMAS_PLAN_KV_HEAD_MAJOR) != 0;
  p.window = opts.window_segments;
  p.bq = opts.block_q ? opts.block_q : 128;
  p.bk = opts.block_k ? opts.block_k : 64;
  const bool host_only = opts.flags & NOMAS_PLAN_HOST_ONLY;
  if (p.bq < 1 || p.bk < 1 || p.bq > 4096 || p.bk > 4096) { *err = "block sizes must be in [1, 4096]"; return NOMAS_ERR_INVALID_ARGUMENT; }
  if (!host_only && (p.bq != 128 || p.bk != 64)) {
    *err = "device plans support block_q = 128, block_k = 64";
    return NOMAS_ERR_UNSUPPORTED;
  }
  p.heads = opts.num_heads;
  p.head_dim = opts.head_dim;
  p.mode = opts.text_query_mode;

  // ---- validate records, identities --------------------------------------
  std::map<Ident, const nomas_segment*> seen_q, seen_k;
  for (const auto& s : q) {
    std::string e = check_segment(s);
    if (!e.empty()) { *err = "query layout: " + e; return NOMAS_ERR_LAYOUT; }
    if (!seen_q.emplace(Ident{s.video, s.index}, &s).second) {
      *err = "query layout names a segment twice";
      return NOMAS_ERR_LAYOUT;
    }
  }
  for (const auto* lst : {&cached, &kv_new}) {
    for (const auto& s : *lst) {
      std::string e = check_segment(s);
      if (!e.empty()) { *err = "key layout: " + e; return NOMAS_ERR_LAYOUT; }
      if (!seen_k.emplace(Ident{s.video, s.index}, &s).second) {
        *err = "key layout (cache + new) names a segment twice";
        return NOMAS_ERR_LAYOUT;
      }
    }
  }
  for (const auto& kv : seen_q) {
    auto it = seen_k.find(kv.first);
    if (it != seen_k.end() && !same_record(*kv.second, *it->second)) {
      *err = "a segment appears in the query and key layouts with different records";
      return NOMAS_ERR_LAYOUT;
    }
  }

  // ---- ordinals ------------------------------------------------------------
  std::map<Ident, int32_t> ord;
  for (const auto& kv : seen_q) ord[kv.first] = 0;
  for (const auto& kv : seen_k) ord[kv.first] = 0;
  std::map<int32_t, int32_t> first_of_video;
  int32_t next = 0;
  for (auto& kv : ord) {
    kv.second = next;
    first_of_video.emplace(kv.first.first, next);  // first in sorted order
    ++next;
  }

  // ---- runs ------------------------------------------------------------------
  std::vector<Run> qr, kr;
  int64_t pos = 0;
  for (const auto& s : q) {
    int32_t o = ord[{s.video, s.index}];
    // first visible ordinal: the video's first segment, or with a window of W
    // segments the first segment whose index is at least s.index - W + 1
    // (ordinals follow (video, index) order, so that is a lower bound)
    int32_t lo = first_of_video[s.video];
    if (opts.window_segments > 0) {
      const int64_t first_index = int64_t(s.index) - opts.window_segments + 1;
      if (first_index > INT32_MIN) {
        auto it = ord.lower_bound(Ident{s.video, int32_t(first_index)});
        lo = std::max(lo, it->second);  // never past s itself, which is in ord
      }
    }
    q_runs(s, o, lo, p.mode, &pos, &qr);
  }
  p.nq = pos;
  pos = 0;
  for (const auto& s : cached) k_runs(s, ord[{s.video, s.index}], &pos, &kr, true);
  p.n_cached = pos;
  for (const auto& s : kv_new) k_runs(s, ord[{s.video, s.index}], &pos, &kr, false);
  p.nk = pos;
  if (p.nq > (int64_t(1) << 30) || p.nk > (int64_t(1) << 30)) {
    *err = "more than 2^30 query or key tokens";
    return NOMAS_ERR_INVALID_ARGUMENT;
  }
  p.nqt = (p.nq + p.bq - 1) / p.bq;
  p.nkt = (p.nk + p.bk - 1) / p.bk;
  if (p.nqt * p.nkt > (int64_t(1) << 31)) { *err = "tile map too large"; return NOMAS_ERR_INVALID_ARGUMENT; }

  // ---- descriptors (padded to whole tiles with never-visible entries) --------
  p.qdesc.assign(size_t(p.nqt * p.bq), QDesc{-1, 0, 0u, 0});
  for (const Run& r : qr)
    std::fill(p.qdesc.begin() + r.start, p.qdesc.begin() + r.start + r.len, qd_of(r));
  p.kdesc.assign(size_t(p.nkt * p.bk), KDesc{-1, 0u});
  for (const Run& r : kr)
    std::fill(p.kdesc.begin() + r.start, p.kdesc.begin() + r.start + r.len, kd_of(r));

  // ---- video key tiles (every key a video token) ----------------------------
  {
    std::vector<uint8_t> is_video(size_t(p.nk), 0);
    int64_t at = 0;
    auto mark = [&](const nomas_segment& s, bool cached) {
      const int64_t nv = int64_t(s.n_frames) * s.tokens_per_frame;
      std::fill(is_video.begin() + at, is_video.begin() + at + nv, uint8_t(1));
      int64_t rest = s.n_head;
      if (!cached) {
        for (int a = 0; a < s.n_actions; ++a) rest += s.actions[a].n_tokens;
        rest += s.n_pad;
      }
      at += nv + rest;
    };
    for (const auto& s : cached) mark(s, true);
    for (const auto& s : kv_new) mark(s, false);
    p.video_tile.assign(size_t(p.nkt), 0);
    for (int64_t j = 0; j < p.nkt; ++j) {
      const int64_t a = j * p.bk, e = std::min(p.nk, a + p.bk);
      p.video_tile[size_t(j)] = std::all_of(is_video.begin() + a, is_video.begin() + e,
                                            [](uint8_t v) { return v != 0; });
    }
  }

  // ---- A = visible pairs, from run pairs -------------------------------------
  int64_t A = 0;
  for (const Run& a : qr)
    for (const Run& b : kr)
      if (visible(qd_of(a), kd_of(b))) A += a.len * b.len;
  p.unmasked_pairs = A;

  // ---- tile classes ------------------------------------------------------------
  auto qt_runs = tile_runs(qr, p.nq, p.bq, p.nqt);
  auto kt_runs = tile_runs(kr, p.nk, p.bk, p.nkt);
  p.classes.assign(size_t(p.nqt * p.nkt), uint8_t(NOMAS_TILE_EMPTY));
  p.csr_ptr.assign(size_t(p.nqt + 1), 0);
  std::vector<int32_t> col_count(size_t(p.nkt), 0);
  p.n_empty = p.n_full = p.n_partial = 0;
  p.executed_pairs = 0;
  for (int64_t i = 0; i < p.nqt; ++i) {
    const int64_t rows = std::min(p.nq, (i + 1) * p.bq) - i * p.bq;
    for (int64_t j = 0; j < p.nkt; ++j) {
      bool any = false, all = true, live_all = true;
      for (int32_t a = qt_runs[i].first; a <= qt_runs[i].second && (live_all || !any); ++a) {
        QDesc qd = qd_of(qr[a]);
        const bool live = qd.seg >= 0;  // padding rows see no key
        for (int32_t b = kt_runs[j].first; b <= kt_runs[j].second; ++b) {
          bool v = visible(qd, kd_of(kr[b]));
          any |= v;
          all &= v;
          live_all &= v || !live;
          if (any && !live_all) break;
        }
      }
      uint8_t c = !any ? NOMAS_TILE_EMPTY : (all ? NOMAS_TILE_FULL : NOMAS_TILE_PARTIAL);
      p.classes[size_t(i * p.nkt + j)] = c;
      if (c == NOMAS_TILE_EMPTY) { ++p.n_empty; continue; }
      (c == NOMAS_TILE_FULL ? p.n_full : p.n_partial) += 1;
      const int64_t cols = std::min(p.nk, (j + 1) * p.bk) - j * p.bk;
      p.executed_pairs += rows * cols;
      const bool ragged_k = (j + 1) * p.bk > p.nk;
      p.csr_idx.push_back(int32_t((j << 1) | ((c == NOMAS_TILE_PARTIAL || ragged_k) ? 1 : 0)));
      p.csr_live_mask.push_back(uint8_t((c == NOMAS_TILE_PARTIAL && !live_all) || ragged_k));
      col_count[size_t(j)]++;
    }
    p.csr_ptr[size_t(i + 1)] = int32_t(p.csr_idx.size());
  }
  // CSC: per key tile, the query tiles that see it (ascending).
  p.csc_ptr.assign(size_t(p.nkt + 1), 0);
  for (int64_t j = 0; j < p.nkt; ++j) p.csc_ptr[size_t(j + 1)] = p.csc_ptr[size_t(j)] + col_count[size_t(j)];
  p.csc_idx.assign(p.csr_idx.size(), 0);
  std::vector<int32_t> fill(p.csc_ptr.begin(), p.csc_ptr.end() - 1);
  for (int64_t i = 0; i < p.nqt; ++i)
    for (int32_t e = p.csr_ptr[size_t(i)]; e < p.csr_ptr[size_t(i + 1)]; ++e) {
      int32_t j = p.csr_idx[size_t(e)] >> 1, m = p.csr_idx[size_t(e)] & 1;
      p.csc_idx[size_t(fill[size_t(j)]++)] = int32_t((i << 1) | m);
    }
  return NOMAS_OK;
}

void build_fwd_schedule(HostPlan* pp, int32_t groups) {
  HostPlan& p = *pp;
  // merged entry lists of q-tile pairs
  p.n_pairs = (p.nqt + 1) / 2;
  p.pair_ptr.assign(size_t(p.n_pairs + 1), 0);
  p.pair_idx.clear();
  for (int64_t u = 0; u < p.n_pairs; ++u) {
    const int64_t qa = 2 * u, qb = 2 * u + 1;
    int32_t ia = p.csr_ptr[size_t(qa)], ea = p.csr_ptr[size_t(qa + 1)];
    int32_t ib = qb < p.nqt ? p.csr_ptr[size_t(qb)] : 0, eb = qb < p.nqt ? p.csr_ptr[size_t(qb + 1)] : 0;
    while (ia < ea || ib < eb) {
      const int32_t ka = ia < ea ? (p.csr_idx[size_t(ia)] >> 1) : INT32_MAX;
      const int32_t kb = ib < eb ? (p.csr_idx[size_t(ib)] >> 1) : INT32_MAX;
      const int32_t kt = std::min(ka, kb);
      int32_t flags = 0;
      if (ka == kt) flags |= p.csr_live_mask[size_t(ia++)];
      else flags |= 4;  // EMPTY for the first q-tile
      if (kb == kt) flags |= p.csr_live_mask[size_t(ib++)] << 1;
      else flags |= 8;  // EMPTY for the second q-tile (or it does not exist)
      p.pair_idx.push_back((kt << 4) | flags);
    }
    p.pair_ptr[size_t(u + 1)] = int32_t(p.pair_idx.size());
  }

  // sparse lists: per pair, non-video entries + ceil(keep% of the video ones)
  p.sp_ptr.clear();
  p.sp_keep.clear();
  p.sp_total = 0;
  if (p.keep_percent > 0) {
    p.sp_ptr.assign(size_t(p.n_pairs + 1), 0);
    p.sp_keep.assign(size_t(p.n_pairs), 0);
    for (int64_t u = 0; u < p.n_pairs; ++u) {
      int32_t nv = 0;
      for (int32_t e = p.pair_ptr[size_t(u)]; e < p.pair_ptr[size_t(u + 1)]; ++e)
        nv += p.video_tile[size_t(p.pair_idx[size_t(e)] >> 4)];
      const int32_t n = p.pair_ptr[size_t(u + 1)] - p.pair_ptr[size_t(u)];
      const int32_t keep = int32_t((int64_t(nv) * p.keep_percent + 99) / 100);
      p.sp_keep[size_t(u)] = keep;
      p.sp_ptr[size_t(u + 1)] = p.sp_ptr[size_t(u)] + (n - nv) + keep;
    }
    p.sp_total = p.sp_ptr.back();
  }
  // the lists the forward walks: the merged pair lists, or the sparse ones
  const std::vector<int32_t>& lptr = p.keep_percent > 0 ? p.sp_ptr : p.pair_ptr;

  const int64_t n_units = int64_t(p.heads) * p.n_pairs;
  const int64_t row_total = lptr.back();
  const int64_t total = int64_t(p.heads) * row_total;
  groups = std::max<int32_t>(1, groups);
  p.fwd_groups = groups;
  p.pieces.clear();
  p.combine.clear();
  p.n_slots = 0;
  auto unit_len = [&](int64_t u) {
    const int64_t pr = u % p.n_pairs;
    return int64_t(lptr[size_t(pr + 1)] - lptr[size_t(pr)]);
  };
  auto unit_start = [&](int64_t u) { return (u / p.n_pairs) * row_total + lptr[size_t(u % p.n_pairs)]; };

  // Each workgroup takes a list of ranges of the (unit, entry) iterations, in
  // unit order.  Plain schedule: `groups` contiguous ranges of equal cost
  // (below), one per workgroup; the workgroups of an XCD (consecutive ids:
  // the kernel maps hardware workgroup b to b % 8 * (groups / 8) + b / 8)
  // then hold consecutive ranges.  Phased schedule, for plans whose units
  // fall into large groups with disjoint keys (the (head, video) groups of a
  // training pack): the iterations are first cut into one share of equal
  // cost per XCD, each share into phases -- runs of units of one (head,
  // video) -- and every phase into one range of equal cost per workgroup of
  // the XCD, so that at any time all workgroups of an XCD stream the same
  // video's keys of one head (one working set per L2) instead of as many as
  // they hold ranges.
  const int32_t n_xcd = groups % 8 == 0 ? 8 : 1, per_xcd = groups / n_xcd;
  std::vector<int64_t> group_key(size_t(n_units), 0);  // (head, video of the pair's first query)
  {
    int64_t key = -1;
    for (int64_t u = 0; u < n_units; ++u) {
      const int64_t pr = u % p.n_pairs;
      int32_t video = -1;
      for (int64_t r = 2 * pr * p.bq; r < std::min<int64_t>(2 * (pr + 1) * p.bq, p.nqt * p.bq); ++r)
        if (p.qdesc[size_t(r)].seg >= 0) {
          video = p.qdesc[size_t(r)].lo;
          break;
        }
      // a pair of padding only joins the group before it
      if (video >= 0 || key < 0 || key / (int64_t(1) << 31) != u / p.n_pairs)
        key = (u / p.n_pairs) * (int64_t(1) << 31) + std::max(video, 0);
      group_key[size_t(u)] = key;
    }
  }
  bool phased = n_xcd > 1 && total > 0;
  for (int64_t u = 0, run = 0; phased && u < n_units; ++u) {  // every group large enough
    run = (u > 0 && group_key[size_t(u)] == group_key[size_t(u - 1)]) ? run + 1 : 1;
    const bool last = u + 1 == n_units || group_key[size_t(u + 1)] != group_key[size_t(u)];
    if (last && run < 2 * int64_t(per_xcd)) phased = false;
  }
  // Cuts are placed at equal estimated cost rather than equal iteration
  // counts: a unit's entries cost 1 + MASKED_COST times the fraction of them
  // that evaluate the per-element mask, and every unit a workgroup starts
  // costs PIECE_COST more (its Q rows, pipeline fill and epilogue), both in
  // units of one 64-key tile; measured on the training pack's forward, where
  // equal iteration ranges left the workgroups holding many short units or
  // the masked ones up to 30% behind the others.
  constexpr double PIECE_COST = 4.0, MASKED_COST = 1.0;
  // (A sparse list keeps every non-video tile, where the masked entries
  // mostly are, so its masked count is estimated by the dense list's; at
  // 100% kept the two plans get the same cuts.)
  std::vector<double> w_unit(size_t(n_units), 1.0), c_start(size_t(n_units) + 1, 0.0);
  {
    std::vector<double> w_pair(size_t(p.n_pairs), 1.0);
    for (int64_t pr = 0; pr < p.n_pairs; ++pr) {
      const int32_t e0 = p.pair_ptr[size_t(pr)], e1 = p.pair_ptr[size_t(pr + 1)];
      const int64_t n = lptr[size_t(pr + 1)] - lptr[size_t(pr)];
      int64_t masked = 0;
      for (int32_t e = e0; e < e1; ++e) masked += (p.pair_idx[size_t(e)] & 3) != 0;
      if (n > 0) w_pair[size_t(pr)] = 1.0 + MASKED_COST * std::min(1.0, double(masked) / double(n));
    }
    for (int64_t u = 0; u < n_units; ++u) w_unit[size_t(u)] = w_pair[size_t(u % p.n_pairs)];
  }
  for (int64_t u = 0; u < n_units; ++u)
    c_start[size_t(u + 1)] = c_start[size_t(u)] + (unit_len(u) ? PIECE_COST : 0.0) +
                             double(unit_len(u)) * w_unit[size_t(u)];
  // cost of the iterations before global iteration i, and the iteration at
  // which a given cost is reached
  auto cost_at = [&](int64_t i) {
    int64_t lo = 0, hi = n_units - 1;  // last unit starting at or before i
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) / 2;
      if (unit_start(mid) <= i) lo = mid; else hi = mid - 1;
    }
    const int64_t j = std::max<int64_t>(0, std::min(i - unit_start(lo), unit_len(lo)));
    return c_start[size_t(lo)] + (j > 0 ? PIECE_COST : 0.0) + double(j) * w_unit[size_t(lo)];
  };
  auto iter_at = [&](double c) -> int64_t {
    if (c <= 0.0) return 0;
    if (c >= c_start.back()) return total;
    int64_t lo = 0, hi = n_units - 1;  // last unit whose start cost is <= c
    while (lo < hi) {
      const int64_t mid = (lo + hi + 1) / 2;
      if (c_start[size_t(mid)] <= c) lo = mid; else hi = mid - 1;
    }
    const int64_t u = lo, n = unit_len(u);
    const double in = c - c_start[size_t(u)] - (n ? PIECE_COST : 0.0);
    const int64_t j = in <= 0.0 ? 0 : std::min<int64_t>(n, int64_t(std::llround(in / w_unit[size_t(u)])));
    return unit_start(u) + j;
  };
  // Dynamic tail (below), for calls long enough to pay for it.
  constexpr double TAIL_FRACTION = 0.05;
  constexpr int64_t TAIL_CHUNK = 64, TAIL_MIN_WORK = 1024;
  const bool dyn_tail = total / groups >= TAIL_MIN_WORK;
  // Shares per XCD: the odd-numbered XCDs of the chip run about 3% slower
  // than the even ones (per-workgroup timestamps on several machines; the
  // slowness stays with the physical XCD when the work is handed out in the
  // reverse XCD order), so without a dynamic tail to even them out their
  // workgroups get a slightly smaller share of the cost (480p call -1.1%;
  // with the tail, or with the phased schedule, skewed shares were slower).
  constexpr double XCD_SKEW = 0.015;
  const double skew = n_xcd == 8 && !phased && !dyn_tail ? XCD_SKEW : 0.0;
  std::vector<double> xcd_at(size_t(n_xcd) + 1, 0.0);  // cumulative share, as a fraction
  for (int32_t x = 0; x < n_xcd; ++x)
    xcd_at[size_t(x + 1)] = xcd_at[size_t(x)] + 1.0 + (x % 2 ? -skew : skew);
  for (auto& f : xcd_at) f /= xcd_at.back();
  std::vector<std::vector<std::pair<int64_t, int64_t>>> ranges(static_cast<size_t>(groups));
  if (!phased) {
    const double T = c_start.back();
    auto at = [&](int64_t g) {  // cumulative share of workgroups 0 .. g - 1
      const int64_t x = g / per_xcd, i = g - x * per_xcd;
      return x >= n_xcd ? 1.0 : xcd_at[size_t(x)] + (xcd_at[size_t(x + 1)] - xcd_at[size_t(x)]) * double(i) / per_xcd;
    };
    for (int64_t g = 0; g < groups; ++g)
      ranges[size_t(g)].push_back({iter_at(T * at(g)), iter_at(T * at(g + 1))});
  } else {
    const double T = c_start.back();
    int64_t u = 0;
    for (int32_t x = 0; x < n_xcd; ++x) {
      const int64_t s0 = iter_at(T * xcd_at[size_t(x)]), s1 = iter_at(T * xcd_at[size_t(x + 1)]);
      int64_t a = s0;
      while (a < s1) {
        while (u < n_units && unit_start(u) + unit_len(u) <= a) ++u;
        // the phase: from a to the end of u's group (or of the share)
        int64_t v = u;
        while (v + 1 < n_units && group_key[size_t(v + 1)] == group_key[size_t(u)]) ++v;
        const int64_t b = std::min(s1, unit_start(v) + unit_len(v));
        const double ca = cost_at(a), cb = cost_at(b);
        int64_t prev = a;
        for (int32_t i = 0; i < per_xcd; ++i) {
          const int64_t next = i + 1 == per_xcd ? b : std::min(b, std::max(prev, iter_at(ca + (cb - ca) * (i + 1) / per_xcd)));
          ranges[size_t(x * per_xcd + i)].push_back({prev, next});
          prev = next;
        }
        a = b;
      }
    }
  }

  std::vector<int64_t> ustart(size_t(n_units) + 1, 0);
  for (int64_t u = 0; u < n_units; ++u) ustart[size_t(u)] = unit_start(u);
  ustart[size_t(n_units)] = total;
  auto unit_at = [&](int64_t i) {  // the unit holding iteration i
    return int64_t(std::upper_bound(ustart.begin(), ustart.end() - 1, i) - ustart.begin()) - 1;
  };

  // Dynamic tail: the last TAIL_FRACTION of every workgroup's work is cut
  // from the end of its last range into chunks of at most TAIL_CHUNK entries
  // of one unit, which the workgroups claim in turn (an atomic counter per
  // call) once their own ranges are done -- so that the workgroups that run
  // faster (the XCDs of one chip differ by a few percent, and so do
  // workgroups that share their key tiles in L2 with more or fewer others)
  // take over the others' ends.  Chunks are listed position by position
  // across the workgroups, so that the first claims take the first chunk of
  // every pool.
  std::vector<std::vector<std::pair<int64_t, int64_t>>> pool(static_cast<size_t>(groups));
  if (dyn_tail) {
    for (int64_t g = 0; g < groups; ++g) {
      auto& rs = ranges[size_t(g)];
      if (rs.empty()) continue;
      int64_t work = 0;
      for (const auto& rg : rs) work += rg.second - rg.first;
      auto& last = rs.back();
      const int64_t take = std::min(last.second - last.first, int64_t(TAIL_FRACTION * double(work)));
      const int64_t end = last.second;
      last.second -= take;
      for (int64_t i = last.second; i < end;) {
        const int64_t u = unit_at(i);
        const int64_t stop = std::min({end, ustart[size_t(u)] + unit_len(u), i + TAIL_CHUNK});
        if (stop <= i) break;  // (a zero-length unit cannot hold an iteration)
        pool[size_t(g)].push_back({i, stop});
        i = stop;
      }
    }
  }

  // pieces: the units each range overlaps; a workgroup's time tau counts the
  // iterations it has done before a piece
  std::vector<std::vector<Piece>> per(static_cast<size_t>(groups));
  std::vector<std::vector<int64_t>> tau(static_cast<size_t>(groups));
  std::vector<int32_t> n_pc(size_t(n_units), 0);
  for (int64_t g = 0; g < groups; ++g) {
    int64_t done = 0;
    for (const auto& rg : ranges[size_t(g)]) {
      if (rg.first >= rg.second) continue;
      int64_t u = int64_t(std::upper_bound(ustart.begin(), ustart.end() - 1, rg.first) - ustart.begin()) - 1;
      for (; u < n_units && ustart[size_t(u)] < rg.second; ++u) {
        const int64_t n = unit_len(u), st = ustart[size_t(u)];
        const int64_t a = std::max(rg.first, st), b = std::min(rg.second, st + n);
        if (a >= b) continue;
        per[size_t(g)].push_back(Piece{int32_t(u), int32_t(a - st), int32_t(b - st), -1});
        tau[size_t(g)].push_back(done + (a - rg.first));
        ++n_pc[size_t(u)];
      }
      done += rg.second - rg.first;
    }
  }
  // units with nothing visible still owe zeros / -inf to their rows: the
  // workgroup whose range holds their position (or the last) writes them
  for (int64_t u = 0; u < n_units; ++u) {
    if (unit_len(u) != 0) continue;
    const int64_t pos = std::min(ustart[size_t(u)], std::max<int64_t>(total - 1, 0));
    int64_t owner = groups - 1;
    for (int64_t g = 0; g < groups && owner == groups - 1; ++g)
      for (const auto& rg : ranges[size_t(g)])
        if (rg.first <= pos && pos < rg.second) {
          owner = g;
          break;
        }
    per[size_t(owner)].push_back(Piece{int32_t(u), 0, 0, -1});
    tau[size_t(owner)].push_back(0);
    ++n_pc[size_t(u)];
  }
  std::vector<Piece> chunks;
  for (size_t pos = 0;; ++pos) {
    bool any = false;
    for (int64_t g = 0; g < groups; ++g) {
      if (pos >= pool[size_t(g)].size()) continue;
      any = true;
      const auto& c = pool[size_t(g)][pos];
      const int64_t u = unit_at(c.first), st = ustart[size_t(u)];
      chunks.push_back(Piece{int32_t(u), int32_t(c.first - st), int32_t(c.second - st), -1});
      ++n_pc[size_t(u)];
    }
    if (!any) break;
  }
  // slots and merge items for split units (slots of a unit are consecutive)
  std::vector<int32_t> first_slot(size_t(n_units), -1), next_slot(size_t(n_units), 0);
  for (int64_t u = 0; u < n_units; ++u)
    if (n_pc[size_t(u)] > 1) {
      first_slot[size_t(u)] = p.n_slots;
      p.combine.push_back(CombineItem{int32_t(u), p.n_slots, n_pc[size_t(u)], 0});
      p.n_slots += n_pc[size_t(u)];
    }
  // Rotation: the largest piece of each unit is aligned so that at time tau
  // of its workgroup it visits entry tau mod n.  Workgroups of an XCD that
  // work on units of equal length then stream the same key tiles at about
  // the same time and share them in that XCD's L2.
  p.unit_shift.assign(size_t(n_units), 0);
  std::vector<int64_t> best_len(size_t(n_units), -1);
  for (int64_t g = 0; g < groups; ++g)
    for (size_t i = 0; i < per[size_t(g)].size(); ++i) {
      Piece& pc = per[size_t(g)][i];
      const int64_t u = pc.unit, n = unit_len(u);
      if (first_slot[size_t(u)] >= 0) pc.slot = first_slot[size_t(u)] + next_slot[size_t(u)]++;
      if (n == 0) continue;
      if (pc.e_end - pc.e_begin > best_len[size_t(u)]) {
        best_len[size_t(u)] = pc.e_end - pc.e_begin;
        // local index j of this piece runs at time tau + (j - e_begin)
        const int64_t shift = ((tau[size_t(g)][i] - pc.e_begin) % n + n) % n;
        p.unit_shift[size_t(u)] = int32_t(shift);
      }
    }
  for (Piece& pc : chunks)
    if (first_slot[size_t(pc.unit)] >= 0) pc.slot = first_slot[size_t(pc.unit)] + next_slot[size_t(pc.unit)]++;
  p.wg_ptr.assign(size_t(groups) + 1, 0);
  for (int32_t g = 0; g < groups; ++g) {
    p.pieces.insert(p.pieces.end(), per[size_t(g)].begin(), per[size_t(g)].end());
    p.wg_ptr[size_t(g) + 1] = int32_t(p.pieces.size());
  }
  p.n_chunks = int32_t(chunks.size());
  p.pieces.insert(p.pieces.end(), chunks.begin(), chunks.end());
}

void build_bwd_schedule(HostPlan* pp) {
  HostPlan& p = *pp;
  // merged CSC lists of k-tile pairs (2 u, 2 u + 1); a ragged last q-tile is
  // masked too, since its rows past the end must not reach dK / dV
  const bool ragged_q = p.nq % p.bq != 0;
  p.n_kpairs = (p.nkt + 1) / 2;
  p.kpair_ptr.assign(size_t(p.n_kpairs + 1), 0);
  p.kpair_idx.clear();
  for (int64_t u = 0; u < p.n_kpairs; ++u) {
    const int64_t ka = 2 * u, kb = 2 * u + 1;
    int32_t ia = p.csc_ptr[size_t(ka)], ea = p.csc_ptr[size_t(ka + 1)];
    int32_t ib = kb < p.nkt ? p.csc_ptr[size_t(kb)] : 0, eb = kb < p.nkt ? p.csc_ptr[size_t(kb + 1)] : 0;
    while (ia < ea || ib < eb) {
      const int32_t qa = ia < ea ? (p.csc_idx[size_t(ia)] >> 1) : INT32_MAX;
      const int32_t qb = ib < eb ? (p.csc_idx[size_t(ib)] >> 1) : INT32_MAX;
      const int32_t qt = std::min(qa, qb);
      const int32_t rq = (ragged_q && qt == p.nqt - 1) ? 1 : 0;
      int32_t flags = 0;
      if (qa == qt) flags |= (p.csc_idx[size_t(ia++)] & 1) | rq;
      else flags |= 4;  // EMPTY for the first k-tile
      if (qb == qt) flags |= ((p.csc_idx[size_t(ib++)] & 1) | rq) << 1;
      else flags |= 8;  // EMPTY for the second k-tile (or it does not exist)
      p.kpair_idx.push_back((qt << 4) | flags);
    }
    p.kpair_ptr[size_t(u + 1)] = int32_t(p.kpair_idx.size());
  }
}

}  // namespace nomas

namespace nomas {

// Consistency of a built plan's tables: the invariants the kernels rely on
// (indices in range, lists sorted and matching the class map, every unit's
// iterations covered exactly once by its pieces, slots and merge items
// consistent).  Returns "" or the first violation.
std::string validate_host_plan(const HostPlan& p) {
  auto bad = [](const std::string& what) { return "plan check: " + what; };
  if (int64_t(p.qdesc.size()) != p.nqt * p.bq || int64_t(p.kdesc.size()) != p.nkt * p.bk)
    return bad("descriptor array sizes");
  if (int64_t(p.classes.size()) != p.nqt * p.nkt) return bad("class map size");
  if (p.nqt != (p.nq + p.bq - 1) / p.bq || p.nkt != (p.nk + p.bk - 1) / p.bk) return bad("tile counts");
  int64_t cnt[3] = {0, 0, 0};
  for (uint8_t c : p.classes) {
    if (c > 2) return bad("class value");
    ++cnt[c];
  }
  if (cnt[NOMAS_TILE_EMPTY] != p.n_empty || cnt[NOMAS_TILE_FULL] != p.n_full ||
      cnt[NOMAS_TILE_PARTIAL] != p.n_partial)
    return bad("class counts");
  if (p.unmasked_pairs < 0 || p.unmasked_pairs > p.executed_pairs || p.executed_pairs > p.nq * p.nk)
    return bad("pair counts");
  // CSR (per q-tile) and CSC (per k-tile): ascending non-empty tiles
  auto check_lists = [&](const std::vector<int32_t>& ptr, const std::vector<int32_t>& idx, int64_t rows,
                         int64_t cols, bool by_row) -> std::string {
    if (int64_t(ptr.size()) != rows + 1 || ptr[0] != 0 || ptr.back() != int32_t(idx.size()))
      return bad(by_row ? "CSR pointers" : "CSC pointers");
    for (int64_t r = 0; r < rows; ++r) {
      if (ptr[size_t(r + 1)] < ptr[size_t(r)]) return bad("list pointers not monotone");
      int64_t n_nonempty = 0;
      for (int64_t c = 0; c < cols; ++c) {
        const uint8_t cl = by_row ? p.classes[size_t(r * p.nkt + c)] : p.classes[size_t(c * p.nkt + r)];
        n_nonempty += cl != NOMAS_TILE_EMPTY;
      }
      if (ptr[size_t(r + 1)] - ptr[size_t(r)] != n_nonempty) return bad("list length vs class map");
      int32_t prev = -1;
      for (int32_t e = ptr[size_t(r)]; e < ptr[size_t(r + 1)]; ++e) {
        const int32_t t = idx[size_t(e)] >> 1;
        if (t <= prev || t >= cols) return bad("list entry out of order or range");
        const uint8_t cl = by_row ? p.classes[size_t(r * p.nkt + t)] : p.classes[size_t(t * p.nkt + r)];
        if (cl == NOMAS_TILE_EMPTY) return bad("list holds an EMPTY tile");
        if (cl == NOMAS_TILE_PARTIAL && !(idx[size_t(e)] & 1)) return bad("PARTIAL tile without mask flag");
        prev = t;
      }
    }
    return "";
  };
  std::string e = check_lists(p.csr_ptr, p.csr_idx, p.nqt, p.nkt, true);
  if (!e.empty()) return e;
  e = check_lists(p.csc_ptr, p.csc_idx, p.nkt, p.nqt, false);
  if (!e.empty()) return e;
  if (p.pair_ptr.empty()) return "";  // no forward schedule
  // merged pair lists
  if (p.n_pairs != (p.nqt + 1) / 2 || int64_t(p.pair_ptr.size()) != p.n_pairs + 1)
    return bad("pair pointers");
  for (int64_t u = 0; u < p.n_pairs; ++u) {
    int32_t prev = -1;
    for (int32_t i = p.pair_ptr[size_t(u)]; i < p.pair_ptr[size_t(u + 1)]; ++i) {
      const int32_t v = p.pair_idx[size_t(i)], t = v >> 4;
      if (t <= prev || t >= p.nkt) return bad("pair entry out of order or range");
      for (int half = 0; half < 2; ++half) {
        const int64_t qt = 2 * u + half;
        const bool empty = qt >= p.nqt || p.classes[size_t(qt * p.nkt + t)] == NOMAS_TILE_EMPTY;
        if (empty != bool((v >> (2 + half)) & 1)) return bad("pair EMPTY flag vs class map");
        if (!empty && p.classes[size_t(qt * p.nkt + t)] == NOMAS_TILE_PARTIAL && !((v >> half) & 1)) {
          // allowed only if the tile's hidden pairs all belong to rows that
          // see no key at all (computed unmasked, written as zeros)
          for (int64_t r = qt * p.bq; r < std::min(p.nq, (qt + 1) * p.bq); ++r) {
            const QDesc& qd = p.qdesc[size_t(r)];
            if (qd.seg < 0) continue;
            for (int64_t k = t * p.bk; k < (t + 1) * p.bk; ++k)
              if (k >= p.nk || !visible(qd, p.kdesc[size_t(k)])) return bad("pair mask flag vs class map");
          }
        }
      }
      prev = t;
    }
  }
  const std::vector<int32_t>& lptr = p.keep_percent > 0 ? p.sp_ptr : p.pair_ptr;
  if (int64_t(lptr.size()) != p.n_pairs + 1) return bad("list pointers of the schedule");
  // pieces: every unit's entries [0, n) covered exactly once; slots and merges
  const int64_t n_units = int64_t(p.heads) * p.n_pairs;
  // (the pieces past the last workgroup's are the claimed tail chunks)
  if (int64_t(p.wg_ptr.size()) != int64_t(p.fwd_groups) + 1 || p.wg_ptr[0] != 0 || p.n_chunks < 0 ||
      int64_t(p.wg_ptr.back()) + p.n_chunks != int64_t(p.pieces.size()))
    return bad("workgroup pointers");
  for (int32_t g = 0; g < p.fwd_groups; ++g)
    if (p.wg_ptr[size_t(g + 1)] < p.wg_ptr[size_t(g)]) return bad("workgroup pointers not monotone");
  std::vector<int64_t> covered(size_t(n_units), 0);
  std::vector<int32_t> n_pieces(size_t(n_units), 0), n_slotted(size_t(n_units), 0);
  std::vector<uint8_t> slot_used(size_t(std::max<int32_t>(p.n_slots, 0)), 0);
  for (const Piece& pc : p.pieces) {
    if (pc.unit < 0 || pc.unit >= n_units) return bad("piece unit out of range");
    const int64_t pr = pc.unit % p.n_pairs;
    const int32_t n = lptr[size_t(pr + 1)] - lptr[size_t(pr)];
    if (pc.e_begin < 0 || pc.e_begin > pc.e_end || pc.e_end > n) return bad("piece range");
    covered[size_t(pc.unit)] += pc.e_end - pc.e_begin;
    ++n_pieces[size_t(pc.unit)];
    if (pc.slot >= 0) {
      if (pc.slot >= p.n_slots || slot_used[size_t(pc.slot)]) return bad("piece slot");
      slot_used[size_t(pc.slot)] = 1;
      ++n_slotted[size_t(pc.unit)];
    }
  }
  for (int64_t u = 0; u < n_units; ++u) {
    const int64_t pr = u % p.n_pairs;
    const int32_t n = lptr[size_t(pr + 1)] - lptr[size_t(pr)];
    if (covered[size_t(u)] != n || n_pieces[size_t(u)] < 1) return bad("unit not covered exactly once");
    if ((n_pieces[size_t(u)] > 1) != (n_slotted[size_t(u)] == n_pieces[size_t(u)]) ||
        (n_pieces[size_t(u)] == 1 && n_slotted[size_t(u)] != 0))
      return bad("split unit without slots, or slot on a whole unit");
    if (int64_t(p.unit_shift.size()) != n_units || p.unit_shift[size_t(u)] < 0 ||
        (n > 0 && p.unit_shift[size_t(u)] >= n))
      return bad("unit rotation");
  }
  int64_t merged = 0;
  for (const CombineItem& c : p.combine) {
    if (c.unit < 0 || c.unit >= n_units || c.n_pieces != n_pieces[size_t(c.unit)] || c.n_pieces < 2 ||
        c.first_slot < 0 || c.first_slot + c.n_pieces > p.n_slots)
      return bad("merge item");
    merged += c.n_pieces;
  }
  if (merged != p.n_slots) return bad("merge items vs slots");
  return "";
}

}  // namespace nomas
