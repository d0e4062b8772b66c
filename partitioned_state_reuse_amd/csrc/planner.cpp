// Host-side group planner (DiTango technical summary, "Methodology §1, Anchor-Guided
// Selection Planner"): anchor steps, error model e = w * accumulated delta, online
// prediction of delta from the local state, and per-group selection.  The contract is in
// include/dit_attn.h; ties are fully ordered, so exactly one selection is correct.
#include <math.h>
#include <stdlib.h>

#include <algorithm>
#include <map>
#include <new>
#include <vector>

#include "dit_attn.h"

struct dit_planner {
  int n_qb = 0, P = 0, G = 0, anchor_every = 0, K = 0, mode = 0;
  std::vector<int32_t> go;          // group offsets [G+1]
  std::vector<int32_t> local;       // [n_qb]
  std::vector<double> w;            // [n_qb * G] group importance
  std::vector<int> last;            // [n_qb * G] step of the last recompute, -1 = never
  std::vector<std::map<int, double>> delta;  // per block: step -> observed delta

  bool is_anchor(int step) const {
    if (mode == DIT_PLAN_ANCHOR) return true;
    if (mode == DIT_PLAN_DISTANCE) return false;
    return anchor_every > 0 && step % anchor_every == 0;
  }
  int group_of(int p) const {
    for (int g = 0; g < G; ++g)
      if (go[g] <= p && p < go[g + 1]) return g;
    return -1;
  }
  int distance(int g, int lp) const {
    int d = abs(go[g] - lp);
    for (int p = go[g]; p < go[g + 1]; ++p) d = std::min(d, abs(p - lp));
    return d;
  }
  // delta_i(tau) if observed before `step`; else the latest observation before tau; else 1.
  double dhat(int i, int tau, int step) const {
    const auto &m = delta[i];
    if (tau < step) {
      auto it = m.find(tau);
      if (it != m.end()) return it->second;
    }
    auto it = m.lower_bound(tau);  // first observation at >= tau
    if (it == m.begin()) return 1.0;
    --it;
    return it->second;
  }
  double score(int i, int g, int step) const {
    double acc = 0.0;
    for (int tau = last[i * G + g] + 1; tau <= step; ++tau) acc += dhat(i, tau, step);
    return w[i * G + g] * acc;
  }
};

extern "C" {

int dit_planner_create(int n_qb, int P, const int32_t *group_offsets, int G, const int32_t *local_part,
                       int anchor_every, int recompute_groups, int mode, dit_planner **out) {
  if (!group_offsets || !local_part || !out) return DIT_ERR_NULL;
  if (n_qb < 1 || n_qb > DIT_MAX_BLOCKS || P < 1 || P > DIT_MAX_PARTITIONS || G < 1 || G > P)
    return DIT_ERR_SHAPE;
  if (group_offsets[0] != 0 || group_offsets[G] != P) return DIT_ERR_OFFSETS;
  for (int g = 0; g < G; ++g)
    if (group_offsets[g + 1] <= group_offsets[g]) return DIT_ERR_OFFSETS;
  for (int i = 0; i < n_qb; ++i)
    if (local_part[i] < 0 || local_part[i] >= P) return DIT_ERR_MASK;
  if (mode != DIT_PLAN_WDELTA && mode != DIT_PLAN_DISTANCE && mode != DIT_PLAN_ANCHOR)
    return DIT_ERR_UNSUPPORTED;
  if (recompute_groups < 1 || recompute_groups > G) return DIT_ERR_SHAPE;
  if (mode == DIT_PLAN_WDELTA && anchor_every < 1) return DIT_ERR_SHAPE;
  dit_planner *pl = new (std::nothrow) dit_planner;
  if (!pl) return DIT_ERR_INTERNAL;
  try {
    pl->n_qb = n_qb;
    pl->P = P;
    pl->G = G;
    pl->anchor_every = anchor_every;
    pl->K = recompute_groups;
    pl->mode = mode;
    pl->go.assign(group_offsets, group_offsets + G + 1);
    pl->local.assign(local_part, local_part + n_qb);
    pl->w.assign((size_t)n_qb * G, 0.0);
    pl->last.assign((size_t)n_qb * G, -1);
    pl->delta.resize(n_qb);
  } catch (...) {
    delete pl;
    return DIT_ERR_INTERNAL;
  }
  *out = pl;
  return DIT_OK;
}

int dit_planner_next(dit_planner *pl, int step, uint8_t *mask_out, int32_t *groups_out) {
  if (!pl || !mask_out) return DIT_ERR_NULL;
  if (step < 0) return DIT_ERR_SHAPE;
  try {
    const int G = pl->G;
    const bool anchor = pl->is_anchor(step);
    std::fill(mask_out, mask_out + (size_t)pl->n_qb * pl->P, (uint8_t)0);
    if (groups_out) std::fill(groups_out, groups_out + (size_t)pl->n_qb * G, -1);
    std::vector<int> others;
    std::vector<double> e(G);
    std::vector<int> dist(G);
    for (int i = 0; i < pl->n_qb; ++i) {
      const int lg = pl->group_of(pl->local[i]);
      others.clear();
      for (int g = 0; g < G; ++g) {
        dist[g] = pl->distance(g, pl->local[i]);
        if (g != lg) others.push_back(g);
      }
      int take = (int)others.size();
      if (!anchor) {
        take = std::min(take, pl->K - 1);
        if (pl->mode == DIT_PLAN_WDELTA) {
          for (int g = 0; g < G; ++g) e[g] = pl->score(i, g, step);
          std::stable_sort(others.begin(), others.end(), [&](int a, int b) {
            if (e[a] != e[b]) return e[a] > e[b];
            if (dist[a] != dist[b]) return dist[a] < dist[b];
            return a < b;
          });
        } else {
          std::stable_sort(others.begin(), others.end(), [&](int a, int b) {
            if (dist[a] != dist[b]) return dist[a] < dist[b];
            return a < b;
          });
        }
      }
      std::vector<int> chosen;
      chosen.push_back(lg);
      for (int j = 0; j < take; ++j) chosen.push_back(others[j]);
      for (size_t j = 0; j < chosen.size(); ++j) {
        const int g = chosen[j];
        for (int p = pl->go[g]; p < pl->go[g + 1]; ++p) mask_out[(size_t)i * pl->P + p] = 1;
        pl->last[(size_t)i * G + g] = step;
        if (groups_out) groups_out[(size_t)i * G + j] = g;
      }
    }
    return DIT_OK;
  } catch (...) {
    return DIT_ERR_INTERNAL;
  }
}

int dit_planner_observe(dit_planner *pl, int step, const float *importance, const float *delta) {
  if (!pl) return DIT_ERR_NULL;
  try {
    if (importance) {
      for (int i = 0; i < pl->n_qb; ++i)
        for (int g = 0; g < pl->G; ++g) {
          double acc = 0.0;
          for (int p = pl->go[g]; p < pl->go[g + 1]; ++p) acc += (double)importance[(size_t)i * pl->P + p];
          pl->w[(size_t)i * pl->G + g] = acc;
        }
    }
    if (delta) {
      for (int i = 0; i < pl->n_qb; ++i)
        if (isfinite(delta[i])) pl->delta[i][step] = (double)delta[i];
    }
    return DIT_OK;
  } catch (...) {
    return DIT_ERR_INTERNAL;
  }
}

int dit_planner_scores(const dit_planner *pl, int step, double *scores_out) {
  if (!pl || !scores_out) return DIT_ERR_NULL;
  try {
    for (int i = 0; i < pl->n_qb; ++i)
      for (int g = 0; g < pl->G; ++g) scores_out[(size_t)i * pl->G + g] = pl->score(i, g, step);
    return DIT_OK;
  } catch (...) {
    return DIT_ERR_INTERNAL;
  }
}

void dit_planner_destroy(dit_planner *pl) { delete pl; }

}  // extern "C"
