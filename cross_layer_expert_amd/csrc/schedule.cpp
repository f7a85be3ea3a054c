// Host implementation of Schedule(S, m) of EasyBalance's Algorithm 1
// ("EasyBalance: Cross-Layer Load Balancing in Distributed MoE Inference",
// §4.2 for the minimum RunSet size m, §5.2 for MaxUtil, CumUtil and DiffPeak).
//
// Utilisation of a combined workload W is U = sum_d W_d / (D * max_d W_d)
// (Eq. (3) restricted to one step).  D is common to every candidate, so two
// candidates compare by cross-multiplying (sum, max) pairs exactly; an
// all-zero workload has U = 0.
#include <stdint.h>
#include <string.h>

#include <vector>

#include "cle.h"

namespace {

struct Util {
  int64_t num;  // sum_d W_d
  int64_t den;  // max_d W_d (1 with num 0 when the workload is all zero)
};

Util util_of(const int64_t* W, int D) {
  int64_t s = 0, mx = 0;
  for (int d = 0; d < D; ++d) {
    s += W[d];
    if (W[d] > mx) mx = W[d];
  }
  if (mx == 0) return {0, 1};
  return {s, mx};
}

// a > b ?
bool util_gt(Util a, Util b) {
  return static_cast<__int128>(a.num) * b.den > static_cast<__int128>(b.num) * a.den;
}
bool util_eq(Util a, Util b) {
  return static_cast<__int128>(a.num) * b.den == static_cast<__int128>(b.num) * a.den;
}

int peak_group(const int32_t* w, int D) {
  int best = 0;
  for (int d = 1; d < D; ++d)
    if (w[d] > w[best]) best = d;
  return best;
}

// Add the lowest-id ready candidates not yet chosen until |R| >= m.
uint64_t pad_to_m(uint64_t chosen, uint64_t ready, int m) {
  for (int j = 0; j < 64 && __builtin_popcountll(chosen) < m; ++j) {
    uint64_t b = 1ull << j;
    if ((ready & b) && !(chosen & b)) chosen |= b;
  }
  return chosen;
}

uint64_t cumutil(const int32_t* w, int n, int D, uint64_t ready, int m) {
  std::vector<int64_t> W(D, 0), T(D);
  uint64_t chosen = 0;
  bool first = true;
  for (int j = 0; j < n; ++j) {
    if (!(ready >> j & 1)) continue;
    const int32_t* wj = w + static_cast<int64_t>(j) * D;
    if (first) {
      for (int d = 0; d < D; ++d) W[d] = wj[d];
      chosen |= 1ull << j;
      first = false;
      continue;
    }
    for (int d = 0; d < D; ++d) T[d] = W[d] + wj[d];
    if (util_gt(util_of(T.data(), D), util_of(W.data(), D))) {
      W.swap(T);
      chosen |= 1ull << j;
    }
  }
  return pad_to_m(chosen, ready, m);
}

uint64_t diffpeak(const int32_t* w, int n, int D, uint64_t ready, int m) {
  std::vector<char> taken(D, 0);
  uint64_t chosen = 0;
  for (int j = 0; j < n; ++j) {
    if (!(ready >> j & 1)) continue;
    int p = peak_group(w + static_cast<int64_t>(j) * D, D);
    if (chosen == 0 || !taken[p]) {
      chosen |= 1ull << j;
      taken[p] = 1;
    }
  }
  return pad_to_m(chosen, ready, m);
}

// Exhaustive search over the subsets of the pool with |R| >= m, visited in
// Gray-code order so that each step adds or removes one member.
uint64_t maxutil(const int32_t* w, int D, uint64_t ready, int m) {
  int ids[64];
  int p = 0;
  for (int j = 0; j < 64; ++j)
    if (ready >> j & 1) ids[p++] = j;
  std::vector<int64_t> W(D, 0);
  uint64_t best = 0;
  Util best_u{0, 1};
  int best_size = -1;
  uint64_t cur = 0;  // over pool positions
  uint64_t cur_ids = 0;
  const uint64_t count = 1ull << p;
  for (uint64_t i = 1; i < count; ++i) {
    int bit = __builtin_ctzll(i);
    const int32_t* wj = w + static_cast<int64_t>(ids[bit]) * D;
    if (cur >> bit & 1) {
      for (int d = 0; d < D; ++d) W[d] -= wj[d];
    } else {
      for (int d = 0; d < D; ++d) W[d] += wj[d];
    }
    cur ^= 1ull << bit;
    cur_ids ^= 1ull << ids[bit];
    int size = __builtin_popcountll(cur);
    if (size < m) continue;
    Util u = util_of(W.data(), D);
    bool take;
    if (best_size < 0 || util_gt(u, best_u)) {
      take = true;
    } else if (!util_eq(u, best_u)) {
      take = false;
    } else if (size != best_size) {
      take = size > best_size;
    } else {
      // same U and size: the lexicographically smaller sorted id tuple wins,
      // i.e. the set owning the lowest id of the symmetric difference
      uint64_t diff = cur_ids ^ best;
      take = (cur_ids >> __builtin_ctzll(diff)) & 1;
    }
    if (take) {
      best = cur_ids;
      best_u = u;
      best_size = size;
    }
  }
  return best;
}

}  // namespace

extern "C" cle_status cle_schedule_step(const int32_t* w, int32_t n, int32_t D, uint64_t ready_mask,
                                        int32_t m, int32_t policy, uint64_t* runset_mask) {
  if (!w || !runset_mask) return CLE_EINVAL;
  if (n < 1 || n > CLE_MAX_MICROBATCHES || D < 1) return CLE_EINVAL;
  if (m < 1 || m > n) return CLE_EINVAL;
  if (ready_mask == 0) return CLE_EINVAL;
  if (n < 64 && (ready_mask >> n) != 0) return CLE_EINVAL;
  for (int64_t i = 0; i < static_cast<int64_t>(n) * D; ++i)
    if (w[i] < 0) return CLE_EINVAL;
  const int pool = __builtin_popcountll(ready_mask);
  uint64_t r = 0;
  switch (policy) {
    case CLE_POLICY_B0_ALONE:
      r = ready_mask & (~ready_mask + 1);
      break;
    case CLE_POLICY_B1_LOCKSTEP:
      r = ready_mask;
      break;
    case CLE_POLICY_CUMUTIL:
      r = pool < m ? ready_mask : cumutil(w, n, D, ready_mask, m);
      break;
    case CLE_POLICY_MAXUTIL:
      if (pool <= m) {  // S itself is the only subset with |R| >= m
        r = ready_mask;
      } else {
        if (pool > CLE_MAX_MAXUTIL_POOL) return CLE_EUNSUPPORTED;
        r = maxutil(w, D, ready_mask, m);
      }
      break;
    case CLE_POLICY_DIFFPEAK:
      r = pool < m ? ready_mask : diffpeak(w, n, D, ready_mask, m);
      break;
    default:
      return CLE_EINVAL;
  }
  *runset_mask = r;
  return CLE_OK;
}
