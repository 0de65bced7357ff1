// Host-side code of libloopkv under AddressSanitizer: the byte model and arena layout
// (loopkv_cache_bytes), the planner (loopkv_plan_solve) and the argument checks of
// loopkv_plan_load that return before any device call, over random shapes, plans and budgets.
// The kernel launchers are stubs: nothing here launches. Built and run by test_host_asan.py.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>
#include "loopkv.h"
#include "loopkv_internal.h"
namespace loopkv {
hipError_t launch_append(const Geom&, const CellDesc*, const CellDesc&, const uint16_t*, const uint16_t*, int, int,
                         const int32_t*, const int32_t*, const int32_t*, int, hipStream_t) { return hipErrorUnknown; }
hipError_t launch_decode(const Geom&, const CellDesc&, const DecodeCall&, hipStream_t) { return hipErrorUnknown; }
void* static_workspace(int, hipStream_t) { return nullptr; }
}
int main() {
  std::mt19937_64 rng(7);
  int bad = 0;
  for (int it = 0; it < 400; ++it) {
    loopkv_shape s{};
    s.num_loops = 1 + rng() % 5; s.num_layers = 1 + rng() % 12; s.num_kv_heads = 1 + rng() % 20;
    s.num_q_heads = s.num_kv_heads; s.head_dim = 128; s.page_tokens = rng() % 2 ? 16 : 32;
    s.v_group = 32 << (rng() % 3); s.max_batch = 1 + rng() % 64; s.max_pages_per_seq = 1 + rng() % 512;
    s.tail_tokens = 64 + 32 * (rng() % 8); s.max_splits = 1 + rng() % 8; s.num_pages = 1 + rng() % 4096;
    s.sink_tokens = rng() % 2 ? 32 : 0; s.window_tokens = 0;
    const int cells = s.num_loops * s.num_layers;
    std::vector<uint8_t> plan(cells);
    for (int t = 0; t < s.num_loops; ++t)
      for (int l = 0; l < s.num_layers; ++l) {
        int c = rng() % 3; plan[t * s.num_layers + l] = c == 0 ? 4 : c == 1 ? 2 : (t == s.num_loops - 1 ? 4 : 0);
      }
    loopkv_bytes b{};
    if (loopkv_cache_bytes(&s, plan.data(), &b) != LOOPKV_OK) ++bad;
    // damage table and the planner
    std::vector<double> d((size_t)cells * 3);
    for (auto& x : d) x = std::uniform_real_distribution<double>(0.001, 1.0)(rng);
    loopkv_plan_budget bud{it % 3 == 0 ? -1.0 : 2.0 * cells * 0.3, it % 2 ? 0.0 : b.stored_bytes_per_token * 0.7, 0.2};
    std::vector<uint8_t> out(cells);
    loopkv_plan_cost cost{};
    loopkv_status st = loopkv_plan_solve(&s, d.data(), &bud, out.data(), &cost);
    if (st != LOOPKV_OK && st != LOOPKV_EINFEASIBLE) ++bad;
    // validation paths of plan_load that return before any device call
    loopkv_plan h = nullptr;
    if (loopkv_plan_load(&s, plan.data(), nullptr, 0, nullptr, &h) != LOOPKV_EINVAL) ++bad;
    plan[(s.num_loops - 1) * s.num_layers] = 0;   // REUSE in the final loop
    if (loopkv_cache_bytes(&s, plan.data(), &b) != LOOPKV_EPLAN) ++bad;
  }
  for (int st = 0; st < 8; ++st) (void)loopkv_status_string((loopkv_status)st);
  std::printf("asan harness: %d unexpected statuses\n", bad);
  return bad != 0;
}
