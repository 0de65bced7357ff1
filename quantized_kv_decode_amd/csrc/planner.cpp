// The offline planner: one storage option per cell, chosen exactly.
//
// "Loop-Aware KV Cache Compression for Serving Looped Transformers": the planner takes the
// per-cell damage profile and budgets for damage and storage and minimises the bytes read per
// decode step (section 1; section 3, "System Design"; section 3.1, "Allocation"); a plan's
// damage is the sum of its cells' single-cell damages (section 2.4); a shared cell stores
// nothing and reads the final loop's pages at its layer (section 3.2); the problem is a
// knapsack the paper solves exactly (Appendix, "Layer-only allocation").
//
// Why a dynamic program over three counters is exact: a cell's stored bytes depend only on
// the bits it stores and its read bytes only on the bits it reads. So a plan's storage is a
// function of (cells storing INT4, cells storing INT2) and its reads of (cells reading INT4);
// every other difference between plans is damage. Layer by layer, the program keeps for each
// reachable (n4s, n2s, n4r) the least damage of a partial plan, and a layer's choices are
// enumerated whole (the final loop's option decides what its reusing cells read). At the end
// the feasible state with the fewest read bytes wins (ties: least damage, then least storage).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>
#include <limits>
#include <new>
#include <vector>

#include "loopkv.h"
#include "loopkv_internal.h"

using namespace loopkv;

namespace {

constexpr int kMaxLoops = 5;      // 2 * 3^4 = 162 choices per layer fit a uint8 back-pointer
constexpr int kMaxCells = 256;
constexpr int kOptInt4 = 0, kOptInt2 = 1, kOptReuse = 2;

struct LayerChoice {
  int a, b, c;        // cells of the layer storing INT4, storing INT2, reading INT4
  double dmg;
  int id;             // index among the layer's enumerated choices
};

// Option of loop t in choice `id`: the final loop's option is id / 3^(T-1) (INT4 or INT2);
// earlier loop t's is digit t of id % 3^(T-1) in base 3.
int option_of(int id, int t, int T) {
  int p = 1;
  for (int i = 0; i < T - 1; ++i) p *= 3;
  if (t == T - 1) return id / p;
  int r = id % p;
  for (int i = 0; i < t; ++i) r /= 3;
  return r % 3;
}

uint8_t plan_code(int opt) {
  return opt == kOptInt4 ? LOOPKV_INT4 : opt == kOptInt2 ? LOOPKV_INT2 : LOOPKV_REUSE;
}

// Dense index of (a, b, c) with every counter in [0, n].
inline size_t idx(int a, int b, int c, int n) {
  return ((size_t)a * (n + 1) + b) * (n + 1) + c;
}

loopkv_status plan_solve(const loopkv_shape* shape, const double* damage,
                         const loopkv_plan_budget* budget, uint8_t* plan_out,
                         loopkv_plan_cost* cost_out) {
  if (!damage || !budget || !plan_out) return LOOPKV_EINVAL;
  loopkv_status st = check_shape(shape);
  if (st != LOOPKV_OK) return st;
  const int T = shape->num_loops, L = shape->num_layers;
  if (T > kMaxLoops || T * L > kMaxCells) return LOOPKV_ENOTSUP;
  const double h = budget->hot_fraction;
  if (!(h >= 0.0 && h <= 1.0) || std::isnan(budget->max_damage) ||
      std::isnan(budget->max_stored_bytes))
    return LOOPKV_EINVAL;
  for (int t = 0; t < T; ++t)
    for (int l = 0; l < L; ++l)
      for (int o = 0; o < 3; ++o)
        if (!(o == kOptReuse && t == T - 1) && !std::isfinite(damage[((size_t)t * L + l) * 3 + o]))
          return LOOPKV_EINVAL;

  // Byte model per token over the heads.
  const int H = shape->num_kv_heads, D = shape->head_dim, nvg = shape->head_dim / shape->v_group;
  const double s4 = H * token_head_bytes(4, D, nvg, true);
  const double s2 = H * token_head_bytes(2, D, nvg, true);
  const double r4 = H * (token_head_bytes(4, D, nvg, false) + h * (D / 4.0));
  const double r2 = s2;

  // Every whole-layer choice, reduced to the cheapest one per counter delta.
  int n_choice = 2;
  for (int i = 0; i < T - 1; ++i) n_choice *= 3;
  std::vector<std::vector<LayerChoice>> choices(L);
  for (int l = 0; l < L; ++l) {
    std::vector<LayerChoice> best;
    for (int id = 0; id < n_choice; ++id) {
      const int fin = option_of(id, T - 1, T);
      LayerChoice ch{0, 0, 0, 0.0, id};
      for (int t = 0; t < T; ++t) {
        const int o = option_of(id, t, T);
        ch.dmg += damage[((size_t)t * L + l) * 3 + o];
        if (o == kOptInt4) { ++ch.a; ++ch.c; }
        else if (o == kOptInt2) ++ch.b;
        else if (fin == kOptInt4) ++ch.c;   // reuses the final loop's INT4 pages
      }
      bool merged = false;
      for (LayerChoice& b : best)
        if (b.a == ch.a && b.b == ch.b && b.c == ch.c) {
          if (ch.dmg < b.dmg) b = ch;
          merged = true;
          break;
        }
      if (!merged) best.push_back(ch);
    }
    choices[l] = best;
  }

  const double inf = std::numeric_limits<double>::infinity();
  std::vector<double> cur(1, 0.0), nxt;
  std::vector<std::vector<uint8_t>> back(L);
  for (int l = 0; l < L; ++l) {
    const int np = T * l, n = T * (l + 1);
    nxt.assign((size_t)(n + 1) * (n + 1) * (n + 1), inf);
    back[l].assign(nxt.size(), 0);
    for (int a = 0; a <= np; ++a)
      for (int b = 0; a + b <= np; ++b)
        for (int c = a; c + b <= np; ++c) {
          const double v = cur[idx(a, b, c, np)];
          if (v == inf) continue;
          for (const LayerChoice& ch : choices[l]) {
            const size_t j = idx(a + ch.a, b + ch.b, c + ch.c, n);
            const double nv = v + ch.dmg;
            if (nv < nxt[j]) {
              nxt[j] = nv;
              back[l][j] = (uint8_t)ch.id;
            }
          }
        }
    cur.swap(nxt);
  }

  // The feasible final state with the fewest read bytes, then least damage, then least storage.
  const int N = T * L;
  const bool dmg_budget = budget->max_damage >= 0.0;
  const bool sto_budget = budget->max_stored_bytes > 0.0;
  int ba = -1, bb = -1, bc = -1;
  double b_read = inf, b_dmg = inf, b_sto = inf;
  for (int a = 0; a <= N; ++a)
    for (int b = 0; a + b <= N; ++b)
      for (int c = a; c + b <= N; ++c) {
        const double v = cur[idx(a, b, c, N)];
        if (v == inf) continue;
        const double sto = a * s4 + b * s2;
        if (dmg_budget && v > budget->max_damage) continue;
        if (sto_budget && sto > budget->max_stored_bytes) continue;
        const double rd = c * r4 + (N - c) * r2;
        if (rd < b_read || (rd == b_read && (v < b_dmg || (v == b_dmg && sto < b_sto)))) {
          ba = a; bb = b; bc = c;
          b_read = rd; b_dmg = v; b_sto = sto;
        }
      }
  if (ba < 0) return LOOPKV_EINFEASIBLE;

  // Walk the back-pointers from the chosen state to layer 0.
  std::vector<uint8_t> plan((size_t)N);
  int a = ba, b = bb, c = bc;
  for (int l = L - 1; l >= 0; --l) {
    const int n = T * (l + 1);
    const int id = back[l][idx(a, b, c, n)];
    const int fin = option_of(id, T - 1, T);
    for (int t = 0; t < T; ++t) {
      const int o = option_of(id, t, T);
      plan[(size_t)t * L + l] = plan_code(o);
      if (o == kOptInt4) { --a; --c; }
      else if (o == kOptInt2) --b;
      else if (fin == kOptInt4) --c;
    }
  }
  std::memcpy(plan_out, plan.data(), plan.size());
  if (cost_out) {
    cost_out->damage = b_dmg;
    cost_out->stored_bytes_per_token = b_sto;
    cost_out->read_bytes_per_token = b_read;
  }
  return LOOPKV_OK;
}

}  // namespace

// No exception crosses the C ABI: a failed host allocation is reported as insufficient capacity.
extern "C" loopkv_status loopkv_plan_solve(const loopkv_shape* shape, const double* damage,
                                           const loopkv_plan_budget* budget, uint8_t* plan_out,
                                           loopkv_plan_cost* cost_out) {
  try {
    return plan_solve(shape, damage, budget, plan_out, cost_out);
  } catch (const std::bad_alloc&) {
    return LOOPKV_ECAPACITY;
  }
}
