// Co-activation-aware expert placement: host code.
//
// Cobalt page, English abstract: a two-stage layout planner periodically
// co-locates experts that are often activated together, then adjusts the
// layout inside each node every step to rebalance the workload. Zyphra
// correlated expert placement page, English abstract: experts often selected
// together go to the same GPU, so a once-per-GPU dispatcher sends fewer rows.
// The pages give no algorithm; this file implements the plainest reading:
//
//  Stage 1 (co-location, E/G experts per rank). For g = 0..G-1: seed the
//  group with the heaviest unassigned expert, then repeatedly add the
//  unassigned expert with the largest co-activation weight to the group's
//  members. Then up to `swap_passes` passes over all pairs (a < b) in
//  different groups swap the two whenever that raises the total
//  within-group weight; a pass without a swap ends the refinement.
//
//  Stage 2 (per-node rebalance). Ranks [n*rpn, (n+1)*rpn) form node n. Within
//  a node, repeatedly take its most and least loaded ranks and apply the
//  expert swap between them that most lowers the larger of their two loads
//  (ties: the swap that keeps the most co-activation weight), as long as it
//  lowers it at all. Experts never leave their node, so node-level
//  co-location is kept.
//
// Ties everywhere go to the lower expert or rank index, so the result is a
// deterministic function of the inputs. Weights: c(a, b) = coact[a][b] +
// coact[b][a] for a != b (the histogram is symmetric; this also accepts a
// one-sided one), c(a, a) = 0.
#include <moe.h>

#include <cstdint>
#include <vector>

#define MOE_EXPORT extern "C" __attribute__((visibility("default")))

namespace {

struct Plan {
  int E, G;
  std::vector<int64_t> c;    // E x E symmetric weights, zero diagonal
  std::vector<int> grp;      // expert -> rank
  std::vector<int64_t> S;    // S[e * G + g] = sum of c(e, m) over members m of g
  std::vector<int64_t> load;

  int64_t w(int a, int b) const { return c[(size_t)a * E + b]; }

  void build_sums() {
    S.assign((size_t)E * G, 0);
    for (int e = 0; e < E; ++e)
      for (int m = 0; m < E; ++m) S[(size_t)e * G + grp[m]] += w(e, m);
  }
  // change of the total within-group weight if a and b (in different groups) swap
  int64_t swap_gain(int a, int b) const {
    const int A = grp[a], B = grp[b];
    return (S[(size_t)a * G + B] - w(a, b)) + (S[(size_t)b * G + A] - w(b, a)) -
           S[(size_t)a * G + A] - S[(size_t)b * G + B];
  }
  void do_swap(int a, int b) {
    const int A = grp[a], B = grp[b];
    for (int e = 0; e < E; ++e) {
      const int64_t d = w(e, b) - w(e, a);
      S[(size_t)e * G + A] += d;
      S[(size_t)e * G + B] -= d;
    }
    grp[a] = B;
    grp[b] = A;
  }
};

void stage1(Plan& p, int swap_passes) {
  const int E = p.E, G = p.G, cap = E / G;
  p.grp.assign(E, -1);
  std::vector<int64_t> score(E);
  for (int g = 0; g < G; ++g) {
    int seed = -1;
    for (int e = 0; e < E; ++e)
      if (p.grp[e] < 0 && (seed < 0 || p.load[e] > p.load[seed])) seed = e;
    p.grp[seed] = g;
    for (int u = 0; u < E; ++u) score[u] = p.w(u, seed);
    for (int n = 1; n < cap; ++n) {
      int best = -1;
      for (int u = 0; u < E; ++u) {
        if (p.grp[u] >= 0) continue;
        if (best < 0 || score[u] > score[best] ||
            (score[u] == score[best] && p.load[u] > p.load[best]))
          best = u;
      }
      p.grp[best] = g;
      for (int u = 0; u < E; ++u) score[u] += p.w(u, best);
    }
  }
  p.build_sums();
  for (int pass = 0; pass < swap_passes; ++pass) {
    bool swapped = false;
    for (int a = 0; a < E; ++a)
      for (int b = a + 1; b < E; ++b)
        if (p.grp[a] != p.grp[b] && p.swap_gain(a, b) > 0) {
          p.do_swap(a, b);
          swapped = true;
        }
    if (!swapped) break;
  }
}

void stage2(Plan& p, int rpn) {
  const int E = p.E, G = p.G;
  std::vector<int64_t> L(G, 0);
  for (int e = 0; e < E; ++e) L[p.grp[e]] += p.load[e];
  for (int n0 = 0; n0 < G; n0 += rpn) {
    for (;;) {
      int h = n0, l = n0;
      for (int r = n0 + 1; r < n0 + rpn; ++r) {
        if (L[r] > L[h]) h = r;
        if (L[r] < L[l]) l = r;
      }
      if (L[h] == L[l]) break;
      int ba = -1, bb = -1;
      int64_t bmax = 0, bgain = 0;
      for (int a = 0; a < E; ++a) {
        if (p.grp[a] != h) continue;
        for (int b = 0; b < E; ++b) {
          if (p.grp[b] != l) continue;
          const int64_t d = p.load[a] - p.load[b];
          if (d <= 0) continue;
          const int64_t nm = L[h] - d > L[l] + d ? L[h] - d : L[l] + d;
          if (nm >= L[h]) continue;
          const int64_t gain = p.swap_gain(a, b);
          if (ba < 0 || nm < bmax || (nm == bmax && gain > bgain)) {
            ba = a;
            bb = b;
            bmax = nm;
            bgain = gain;
          }
        }
      }
      if (ba < 0) break;
      const int64_t d = p.load[ba] - p.load[bb];
      L[h] -= d;
      L[l] += d;
      p.do_swap(ba, bb);
    }
  }
}

}  // namespace

MOE_EXPORT moe_status moe_plan_placement(const int64_t* coact, const int64_t* load, int32_t E,
                                         int32_t G, int32_t ranks_per_node, int32_t swap_passes,
                                         int32_t* place) {
  if (!coact || !load || !place || E < 1 || G < 1 || ranks_per_node < 1 || swap_passes < 0)
    return MOE_ERR_ARG;
  if (E % G != 0 || G % ranks_per_node != 0) return MOE_ERR_ARG;
  if (E > 256 || G > 32) return MOE_ERR_UNSUPPORTED;
  for (int e = 0; e < E; ++e)
    if (load[e] < 0) return MOE_ERR_ARG;
  Plan p;
  p.E = E;
  p.G = G;
  p.load.assign(load, load + E);
  p.c.assign((size_t)E * E, 0);
  for (int a = 0; a < E; ++a)
    for (int b = 0; b < E; ++b) {
      if (a == b) continue;
      const int64_t x = coact[(size_t)a * E + b], y = coact[(size_t)b * E + a];
      if (x < 0 || y < 0) return MOE_ERR_ARG;
      p.c[(size_t)a * E + b] = x + y;
    }
  stage1(p, swap_passes);
  if (ranks_per_node > 1) stage2(p, ranks_per_node);
  for (int e = 0; e < E; ++e) place[e] = p.grp[e];
  return MOE_OK;
}
