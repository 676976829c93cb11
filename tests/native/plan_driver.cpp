// Host driver of the plan core for sanitizer builds (AddressSanitizer and
// UndefinedBehaviorSanitizer, built with g++ on the CPU; no HIP).  Reads plan
// cases from stdin and, for each, builds the host plan, the forward schedule
// (256 workgroups) and, for plans without a cache, the backward schedule,
// then checks the plan's invariants.  Prints one line per case:
//   "ok <A> <pieces> <merges>"  or  "status <code> <message>"
// and exits with 1 if an invariant check fails.
//
// Input, whitespace separated:
//   P heads mode window keep_percent     start a case
//   Q|C|N video index n_frames tokens_per_frame n_head n_pad n_actions
//         (n_tokens frame_lo frame_hi) x n_actions
//                                        a query / cached / new-key segment
//   E                                    build and check the case
//   X                                    build the case, plant one mistake at
//                                        a time in copies of the plan and
//                                        print "caught <k> <of>"
#include <cstdio>
#include <iostream>
#include <string>
#include <vector>

#include "plan.h"

int main() {
  std::string tag;
  nomas_plan_opts opts{};
  std::vector<nomas_segment> q, cached, kv;
  int failures = 0;
  while (std::cin >> tag) {
    if (tag == "P") {
      opts = nomas_plan_opts{};
      std::cin >> opts.num_heads >> opts.text_query_mode >> opts.window_segments >> opts.video_keep_percent;
      opts.head_dim = NOMAS_HEAD_DIM;
      q.clear();
      cached.clear();
      kv.clear();
    } else if (tag == "Q" || tag == "C" || tag == "N") {
      nomas_segment s{};
      std::cin >> s.video >> s.index >> s.n_frames >> s.tokens_per_frame >> s.n_head >> s.n_pad >>
          s.n_actions;
      for (int a = 0; a < s.n_actions; ++a) {
        nomas_action act{};
        std::cin >> act.n_tokens >> act.frame_lo >> act.frame_hi;
        if (a < NOMAS_MAX_ACTIONS) s.actions[a] = act;
      }
      (tag == "Q" ? q : tag == "C" ? cached : kv).push_back(s);
    } else if (tag == "E") {
      nomas::HostPlan plan;
      std::string err;
      const nomas_status st = nomas::build_host_plan(q, cached, kv, opts, &plan, &err);
      if (st != NOMAS_OK) {
        std::printf("status %d %s\n", st, err.c_str());
        continue;
      }
      // other device sizes too: a CU count that is a multiple of the 8 XCDs
      // but not 256, and one that is not (per-XCD shares, phases and the
      // tail depend on it); the printed line is the 256-workgroup plan's
      std::string bad;
      for (const int32_t groups : {120, 250, 256}) {
        nomas::build_fwd_schedule(&plan, groups);
        if (cached.empty()) nomas::build_bwd_schedule(&plan);
        bad = nomas::validate_host_plan(plan);
        if (!bad.empty()) {
          bad += " (" + std::to_string(groups) + " workgroups)";
          break;
        }
      }
      if (!bad.empty()) {
        std::printf("invalid %s\n", bad.c_str());
        ++failures;
        continue;
      }
      std::printf("ok %lld %zu %zu\n", (long long)plan.unmasked_pairs, plan.pieces.size(),
                  plan.combine.size());
    } else if (tag == "X") {
      nomas::HostPlan plan;
      std::string err;
      if (nomas::build_host_plan(q, cached, kv, opts, &plan, &err) != NOMAS_OK) {
        std::printf("status build\n");
        continue;
      }
      nomas::build_fwd_schedule(&plan, 256);
      std::vector<nomas::HostPlan> bad(7, plan);
      bad[0].pieces.pop_back();                          // a unit's tail left uncovered
      bad[0].wg_ptr.back() -= 1;
      std::swap(bad[1].csr_idx[0], bad[1].csr_idx[1]);   // list out of order
      bad[2].classes[0] = NOMAS_TILE_EMPTY;              // list holds an EMPTY tile
      bad[2].n_empty += 1;
      bad[2].n_full -= plan.classes[0] == NOMAS_TILE_FULL;
      bad[2].n_partial -= plan.classes[0] == NOMAS_TILE_PARTIAL;
      bad[3].pieces[0].e_end += 1;                       // a piece past its list
      bad[4].combine.clear();                            // split units never merged
      bad[5].unit_shift[0] = 1 << 30;                    // rotation out of range
      // the mask bit of the first entry whose q-tile has a row that sees
      // keys but misses one of this tile's, cleared
      for (size_t e = 0, qt = 0; e < plan.csr_idx.size(); ++e) {
        while (plan.csr_ptr[qt + 1] <= int32_t(e)) ++qt;
        if (!plan.csr_live_mask[e] || plan.classes[qt * plan.nkt + (plan.csr_idx[e] >> 1)] != NOMAS_TILE_PARTIAL)
          continue;
        const int32_t kt = plan.csr_idx[e] >> 1, u = int32_t(qt / 2), bit = 1 << (qt % 2);
        for (int32_t i = plan.pair_ptr[u]; i < plan.pair_ptr[u + 1]; ++i)
          if ((plan.pair_idx[i] >> 4) == kt) bad[6].pair_idx[i] &= ~bit;
        break;
      }
      int caught = 0;
      for (const auto& b : bad) caught += !nomas::validate_host_plan(b).empty();
      std::printf("caught %d %zu\n", caught, bad.size());
    } else {
      std::fprintf(stderr, "unknown tag %s\n", tag.c_str());
      return 2;
    }
  }
  return failures ? 1 : 0;
}
