// Host-side plan core (no HIP).  See plan.h for the descriptor encoding.
//
// The rules encoded here are the visibility rules of action-aware causal
// attention: "Summary (Overview)" page, Model Architecture (Segment-wise
// Causal Attention; Action-Aware Causal Attention, Figure 6b), the onedev.kr
// review, section "무엇과 다른가", and packing of independent videos
// ("Summary (Overview)", Training Infrastructure).  Text-query readings
// R / K / H as documented in nomas_attn.h.
#include "plan.h"

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
  if (opts.flags & ~int32_t(NOMAS_PLAN_HOST_ONLY)) { *err = "unknown plan flag"; return NOMAS_ERR_INVALID_ARGUMENT; }
  if (opts.window_segments < 0) { *err = "window_segments must be >= 0"; return NOMAS_ERR_INVALID_ARGUMENT; }
  if (opts.video_keep_percent < 0 || opts.video_keep_percent > 100) {
    *err = "video_keep_percent must be in [0, 100]";
    return NOMAS_ERR_INVALID_ARGUMENT;
  }
  p.keep_percent = opts.video_keep_percent;
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
      bool any = false, all = true;
      for (int32_t a = qt_runs[i].first; a <= qt_runs[i].second && (all || !any); ++a) {
        QDesc qd = qd_of(qr[a]);
        for (int32_t b = kt_runs[j].first; b <= kt_runs[j].second; ++b) {
          bool v = visible(qd, kd_of(kr[b]));
          any |= v;
          all &= v;
          if (any && !all) break;
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
      if (ka == kt) flags |= (p.csr_idx[size_t(ia++)] & 1);
      else flags |= 4;  // EMPTY for the first q-tile
      if (kb == kt) flags |= (p.csr_idx[size_t(ib++)] & 1) << 1;
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
  std::vector<std::vector<Piece>> per(static_cast<size_t>(groups));
  auto bound = [&](int64_t g) { return (total * g) / groups; };
  auto group_of = [&](int64_t it) {  // the range holding iteration `it`
    int64_t g = (it * groups) / std::max<int64_t>(total, 1);
    while (g + 1 < groups && bound(g + 1) <= it) ++g;
    while (g > 0 && bound(g) > it) --g;
    return std::min<int64_t>(g, groups - 1);
  };
  for (int64_t u = 0; u < n_units; ++u) {
    const int64_t h = u / p.n_pairs, pr = u % p.n_pairs;
    const int64_t n = lptr[size_t(pr + 1)] - lptr[size_t(pr)];
    const int64_t start = h * row_total + lptr[size_t(pr)];
    if (n == 0) {  // nothing visible: still owes zeros / -inf to its rows
      per[size_t(group_of(std::min(start, std::max<int64_t>(total - 1, 0))))].push_back(
          Piece{int32_t(u), 0, 0, -1});
      continue;
    }
    const int64_t g0 = group_of(start), g1 = group_of(start + n - 1);
    for (int64_t g = g0; g <= g1; ++g) {
      const int64_t a = std::max(bound(g), start), b = std::min(bound(g + 1), start + n);
      if (a >= b) continue;
      per[size_t(g)].push_back(Piece{int32_t(u), int32_t(a - start), int32_t(b - start), -1});
    }
    int32_t made = 0;
    for (int64_t g = g0; g <= g1; ++g)
      if (!per[size_t(g)].empty() && per[size_t(g)].back().unit == int32_t(u)) ++made;
    if (made > 1) {
      const int32_t first_slot = p.n_slots;
      for (int64_t g = g0; g <= g1; ++g)
        if (!per[size_t(g)].empty() && per[size_t(g)].back().unit == int32_t(u))
          per[size_t(g)].back().slot = p.n_slots++;
      p.combine.push_back(CombineItem{int32_t(u), first_slot, made, 0});
    }
  }
  // Rotation: the largest piece of each unit is aligned so that at time tau of
  // its workgroup's range (tiles already done by that workgroup) it visits
  // entry tau mod n.  The workgroups of an XCD (consecutive ranges, the same
  // heads) then stream the same key tiles at about the same time and share
  // them in that XCD's L2, instead of each walking its own offset.
  p.unit_shift.assign(size_t(n_units), 0);
  for (int64_t u = 0; u < n_units; ++u) {
    const int64_t h = u / p.n_pairs, pr = u % p.n_pairs;
    const int64_t n = lptr[size_t(pr + 1)] - lptr[size_t(pr)];
    if (n == 0) continue;
    const int64_t start = h * row_total + lptr[size_t(pr)];
    const int64_t g0 = group_of(start), g1 = group_of(start + n - 1);
    int64_t best_g = g0, best_len = -1;
    for (int64_t g = g0; g <= g1; ++g) {
      const int64_t a = std::max(bound(g), start), b = std::min(bound(g + 1), start + n);
      if (b - a > best_len) best_len = b - a, best_g = g;
    }
    // at local index j the workgroup has done (start + j - bound(best_g)) tiles
    const int64_t shift = (start - bound(best_g)) % n;
    p.unit_shift[size_t(u)] = int32_t((shift + n) % n);
  }
  p.wg_ptr.assign(size_t(groups) + 1, 0);
  for (int32_t g = 0; g < groups; ++g) {
    p.pieces.insert(p.pieces.end(), per[size_t(g)].begin(), per[size_t(g)].end());
    p.wg_ptr[size_t(g) + 1] = int32_t(p.pieces.size());
  }
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
