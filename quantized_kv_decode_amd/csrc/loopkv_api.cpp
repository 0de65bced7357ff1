// Host side of libloopkv: argument validation, the byte model, arena carving, per-cell
// descriptors and kernel launches. See include/loopkv.h for the contract of each entry point.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <memory>
#include <new>
#include <vector>

#include "loopkv.h"
#include "loopkv_internal.h"

using namespace loopkv;

struct loopkv_plan_s {
  loopkv_shape shape;
  std::vector<uint8_t> plan;
  std::vector<CellDesc> desc;     // host copy of the device descriptors
  CellDesc* desc_dev = nullptr;
  uint32_t* err_dev = nullptr;
  float* partials_dev = nullptr;
  int32_t* merge_dev = nullptr;   // split counters of the in-launch merge
  int device = 0;
  int cus = 0;                    // compute units of that device
};

namespace loopkv {

loopkv_status check_shape(const loopkv_shape* s) {
  if (!s) return LOOPKV_EINVAL;
  if (s->num_layers < 1 || s->num_loops < 1 || s->num_kv_heads < 1 || s->num_kv_heads > 1024 ||
      s->max_batch < 1 || s->max_pages_per_seq < 1 || s->num_pages < 1 || s->max_splits < 1 ||
      s->reserved != 0)
    return LOOPKV_EINVAL;
  if (s->tail_tokens < 32 || s->tail_tokens > 1024 || s->tail_tokens % 32 != 0)
    return LOOPKV_EINVAL;
  if (s->sink_tokens != 0 && s->sink_tokens != kGroup) return LOOPKV_EINVAL;
  if (s->window_tokens < 0 || s->window_tokens % kGroup != 0) return LOOPKV_EINVAL;
  // the ring holds the window, the partial group behind it, and one group of lag between a
  // reusing cell and its source
  if (s->window_tokens > 0 && s->tail_tokens < s->window_tokens + 2 * kGroup) return LOOPKV_EINVAL;
  if (s->num_q_heads != s->num_kv_heads) return LOOPKV_ENOTSUP;
  if (s->head_dim != kHeadDim) return LOOPKV_ENOTSUP;
  if (s->page_tokens != 16 && s->page_tokens != 32) return LOOPKV_ENOTSUP;
  if (s->v_group != 32 && s->v_group != 64 && s->v_group != 128) return LOOPKV_ENOTSUP;
  if ((int64_t)s->max_pages_per_seq * s->page_tokens > (1 << 26)) return LOOPKV_EINVAL;
  if (s->num_pages > ((int64_t)1 << 40)) return LOOPKV_EINVAL;
  if ((int64_t)s->num_layers * s->num_loops > 65536) return LOOPKV_EINVAL;
  return LOOPKV_OK;
}

// Algorithmic bytes of one (token, head) stored at `bits`: key codes, the token's share of
// its key group's fp16 (s, z), value codes or planes, value (s, z).
double token_head_bytes(int bits, int D, int nvg, bool with_lo) {
  double b = D * bits / 8.0 + 4.0 * D / kGroup + D / 4.0 + 4.0 * nvg;
  if (bits == 4 && with_lo) b += D / 4.0;
  return b;
}

}  // namespace loopkv

namespace {

constexpr uint64_t kAlign = 256;

uint64_t align_up(uint64_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Multiplies with an overflow check; returns false on overflow.
bool mul_ok(uint64_t a, uint64_t b, uint64_t* r) {
  if (a != 0 && b > UINT64_MAX / a) return false;
  *r = a * b;
  return true;
}

loopkv_status check_plan(const loopkv_shape* s, const uint8_t* plan) {
  if (!plan) return LOOPKV_EINVAL;
  const int T = s->num_loops, L = s->num_layers;
  for (int t = 0; t < T; ++t)
    for (int l = 0; l < L; ++l) {
      const uint8_t c = plan[t * L + l];
      if (c != LOOPKV_REUSE && c != LOOPKV_INT2 && c != LOOPKV_INT4) return LOOPKV_EPLAN;
      if (c == LOOPKV_REUSE && t == T - 1) return LOOPKV_EPLAN;
    }
  return LOOPKV_OK;
}

struct ArenaPlan {
  uint64_t desc_off, counters_off, err_off, merge_off, partials_off, tails_off, sinks_off, pools_off, total;
  uint64_t tail_bytes_per_cell;  // one of K or V
  uint64_t sink_bytes_per_cell;  // one of K or V
  std::vector<uint64_t> pool_off;  // per cell; UINT64_MAX for REUSE
  uint64_t pool_bytes;
  loopkv_bytes bytes;
};

loopkv_status plan_arena(const loopkv_shape* s, const uint8_t* plan, ArenaPlan* a) {
  const int T = s->num_loops, L = s->num_layers, H = s->num_kv_heads, D = s->head_dim;
  const int nvg = D / s->v_group;
  const uint64_t cells = (uint64_t)T * L;
  uint64_t off = 0, x;
  a->desc_off = off;
  off = align_up(off + cells * sizeof(CellDesc));
  a->counters_off = off;
  off = align_up(off + cells * (uint64_t)s->max_batch * sizeof(int32_t));
  a->err_off = off;
  off = align_up(off + sizeof(uint32_t));
  a->merge_off = off;
  off = align_up(off + (uint64_t)s->max_batch * H * sizeof(int32_t));
  const uint64_t meta = off;
  a->partials_off = off;
  if (!mul_ok((uint64_t)s->max_batch * H, (uint64_t)s->max_splits * (D + 2) * 4, &x))
    return LOOPKV_EINVAL;
  const uint64_t ws = align_up(x);
  off += ws;
  a->tails_off = off;
  if (!mul_ok((uint64_t)s->max_batch * s->tail_tokens, (uint64_t)H * D * 2, &x))
    return LOOPKV_EINVAL;
  a->tail_bytes_per_cell = align_up(x);
  uint64_t tails;
  if (!mul_ok(cells * 2, a->tail_bytes_per_cell, &tails)) return LOOPKV_EINVAL;
  off += tails;
  a->sinks_off = off;
  if (!mul_ok((uint64_t)s->max_batch * s->sink_tokens, (uint64_t)H * D * 2, &x))
    return LOOPKV_EINVAL;
  a->sink_bytes_per_cell = align_up(x);
  uint64_t sinks;
  if (!mul_ok(cells * 2, a->sink_bytes_per_cell, &sinks)) return LOOPKV_EINVAL;
  off += sinks;
  a->pools_off = off;
  a->pool_off.assign(cells, UINT64_MAX);
  uint64_t pools = 0;
  double stored = 0, read_hi = 0, read_all = 0;
  for (int t = 0; t < T; ++t)
    for (int l = 0; l < L; ++l) {
      const int c = plan[t * L + l];
      const int src_bits = c == LOOPKV_REUSE ? plan[(T - 1) * L + l] : c;
      read_hi += H * token_head_bytes(src_bits, D, nvg, false);
      read_all += H * token_head_bytes(src_bits, D, nvg, true);
      if (c == LOOPKV_REUSE) continue;
      stored += H * token_head_bytes(c, D, nvg, true);
      const uint64_t page = (uint64_t)H * head_layout(c, s->page_tokens, D, nvg).total;
      uint64_t pb;
      if (!mul_ok(page, (uint64_t)s->num_pages, &pb)) return LOOPKV_EINVAL;
      a->pool_off[(uint64_t)t * L + l] = off;
      off = align_up(off + pb);
      pools += align_up(pb);
    }
  a->pool_bytes = pools;
  a->total = off;
  a->bytes.arena_bytes = off;
  a->bytes.pool_bytes = pools;
  a->bytes.tail_bytes = tails;
  a->bytes.sink_bytes = sinks;
  a->bytes.meta_bytes = meta;
  a->bytes.workspace_bytes = ws;
  a->bytes.stored_bytes_per_token = stored;
  a->bytes.read_bytes_per_token_hi_only = read_hi;
  a->bytes.read_bytes_per_token_all_hot = read_all;
  return LOOPKV_OK;
}

Geom make_geom(const loopkv_plan_s* p) {
  Geom g;
  const loopkv_shape& s = p->shape;
  g.H = s.num_kv_heads;
  g.D = s.head_dim;
  g.P = s.page_tokens;
  g.v_group = s.v_group;
  g.nvg = s.head_dim / s.v_group;
  g.tail = s.tail_tokens;
  g.sink = s.sink_tokens;
  g.window = s.window_tokens;
  g.max_ctx = s.max_pages_per_seq * s.page_tokens;
  g.max_splits = s.max_splits;
  g.num_pages = s.num_pages;
  g.err = p->err_dev;
  g.cus = p->cus;
  return g;
}

// The split used for split_tokens = LOOPKV_SPLIT_AUTO. Enough splits that the (request, head)
// rows fill every compute unit with a four-row workgroup (rows * splits >= 4 * CUs), but splits of
// at least kAutoMinSplit tokens: a split restarts its running maximum at the seed, so short
// splits fetch more low planes, and each split workgroup pays a fixed prologue and merge. At
// most 64 splits per row (section 3.4: up to 64 far blocks per decode row) and max_splits.
constexpr int64_t kAutoRowsPerCu = 4;
constexpr int64_t kAutoMinSplit = 1024;

int32_t auto_split(const loopkv_plan_s* p, int32_t batch, int64_t ctx) {
  const int64_t rows = (int64_t)batch * p->shape.num_kv_heads;
  const int64_t cus = std::max(p->cus, 1);
  int64_t n = (kAutoRowsPerCu * cus + rows - 1) / rows;
  n = std::min<int64_t>(n, std::min<int64_t>(64, p->shape.max_splits));
  n = std::min<int64_t>(n, ctx / kAutoMinSplit);
  if (n <= 1) return 0;
  const int64_t st = (ctx + n - 1) / n;
  return (int32_t)((st + kGroup - 1) / kGroup * kGroup);
}

int64_t decode_ctx(const loopkv_plan_s* p, int32_t pt_stride) {
  return std::min<int64_t>((int64_t)p->shape.max_pages_per_seq * p->shape.page_tokens,
                           (int64_t)pt_stride * p->shape.page_tokens);
}

bool cell_ok(const loopkv_plan_s* p, int32_t layer, int32_t loop) {
  return p && layer >= 0 && layer < p->shape.num_layers && loop >= 0 && loop < p->shape.num_loops;
}

}  // namespace

extern "C" {

const char* loopkv_status_string(loopkv_status st) {
  switch (st) {
    case LOOPKV_OK: return "ok";
    case LOOPKV_EINVAL: return "invalid argument";
    case LOOPKV_EPLAN: return "invalid plan";
    case LOOPKV_ENOTSUP: return "unsupported shape";
    case LOOPKV_ECAPACITY: return "insufficient capacity";
    case LOOPKV_EHIP: return "HIP runtime error";
    case LOOPKV_EINFEASIBLE: return "no plan meets the budgets";
  }
  return "unknown status";
}

// Host allocations that fail inside an entry point are reported as insufficient capacity; no
// exception crosses the C ABI.
loopkv_status loopkv_cache_bytes(const loopkv_shape* shape, const uint8_t* plan,
                                 loopkv_bytes* out) try {
  if (!out) return LOOPKV_EINVAL;
  loopkv_status st = check_shape(shape);
  if (st != LOOPKV_OK) return st;
  st = check_plan(shape, plan);
  if (st != LOOPKV_OK) return st;
  ArenaPlan a;
  st = plan_arena(shape, plan, &a);
  if (st != LOOPKV_OK) return st;
  *out = a.bytes;
  return LOOPKV_OK;
} catch (const std::bad_alloc&) {
  return LOOPKV_ECAPACITY;
}

loopkv_status loopkv_plan_load(const loopkv_shape* shape, const uint8_t* plan, void* arena_dev,
                               uint64_t arena_bytes, void* stream, loopkv_plan* out) try {
  if (!out) return LOOPKV_EINVAL;
  *out = nullptr;
  loopkv_status st = check_shape(shape);
  if (st != LOOPKV_OK) return st;
  st = check_plan(shape, plan);
  if (st != LOOPKV_OK) return st;
  if (!arena_dev || reinterpret_cast<uintptr_t>(arena_dev) % kAlign != 0) return LOOPKV_EINVAL;
  ArenaPlan a;
  st = plan_arena(shape, plan, &a);
  if (st != LOOPKV_OK) return st;
  if (arena_bytes < a.total) return LOOPKV_ECAPACITY;

  std::unique_ptr<loopkv_plan_s> p(new loopkv_plan_s);
  p->shape = *shape;
  const int T = shape->num_loops, L = shape->num_layers, H = shape->num_kv_heads;
  const int nvg = shape->head_dim / shape->v_group;
  p->plan.assign(plan, plan + (size_t)T * L);
  uint8_t* base = static_cast<uint8_t*>(arena_dev);
  p->desc_dev = reinterpret_cast<CellDesc*>(base + a.desc_off);
  p->err_dev = reinterpret_cast<uint32_t*>(base + a.err_off);
  p->partials_dev = reinterpret_cast<float*>(base + a.partials_off);
  p->merge_dev = reinterpret_cast<int32_t*>(base + a.merge_off);
  int32_t* counters = reinterpret_cast<int32_t*>(base + a.counters_off);
  p->desc.resize((size_t)T * L);
  for (int t = 0; t < T; ++t)
    for (int l = 0; l < L; ++l) {
      const size_t i = (size_t)t * L + l;
      const size_t src = plan[i] == LOOPKV_REUSE ? (size_t)(T - 1) * L + l : i;
      const int src_bits = plan[src];
      CellDesc d;
      std::memset(&d, 0, sizeof(d));
      d.code = plan[i];
      d.read_bits = src_bits;
      d.own_bits = plan[i];
      d.gated = src_bits == LOOPKV_INT4;
      d.read_pool = base + a.pool_off[src];
      d.own_pool = plan[i] == LOOPKV_REUSE ? nullptr : base + a.pool_off[i];
      d.read_page_bytes = (int64_t)H * head_layout(src_bits, shape->page_tokens, shape->head_dim, nvg).total;
      d.own_page_bytes = plan[i] == LOOPKV_REUSE ? 0 : d.read_page_bytes;
      d.tail_k = reinterpret_cast<uint16_t*>(base + a.tails_off + (2 * i) * a.tail_bytes_per_cell);
      d.tail_v = reinterpret_cast<uint16_t*>(base + a.tails_off + (2 * i + 1) * a.tail_bytes_per_cell);
      if (shape->sink_tokens > 0) {
        d.sink_k = reinterpret_cast<uint16_t*>(base + a.sinks_off + (2 * i) * a.sink_bytes_per_cell);
        d.sink_v = reinterpret_cast<uint16_t*>(base + a.sinks_off + (2 * i + 1) * a.sink_bytes_per_cell);
      }
      d.src_qgroups = counters + src * shape->max_batch;
      d.own_qgroups = counters + i * shape->max_batch;
      p->desc[i] = d;
    }
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipGetDevice(&p->device);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&p->cus, hipDeviceAttributeMultiprocessorCount, p->device);
  if (e == hipSuccess)
    e = hipMemcpyAsync(p->desc_dev, p->desc.data(), p->desc.size() * sizeof(CellDesc),
                       hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemsetAsync(counters, 0, (size_t)T * L * shape->max_batch * sizeof(int32_t), s);
  if (e == hipSuccess) e = hipMemsetAsync(p->err_dev, 0, sizeof(uint32_t), s);
  if (e == hipSuccess)
    e = hipMemsetAsync(p->merge_dev, 0, (size_t)shape->max_batch * H * sizeof(int32_t), s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return LOOPKV_EHIP;
  if (!static_workspace(p->device, s)) return LOOPKV_EHIP;
  *out = p.release();
  return LOOPKV_OK;
} catch (const std::bad_alloc&) {
  return LOOPKV_ECAPACITY;
}

loopkv_status loopkv_plan_free(loopkv_plan plan) {
  delete plan;
  return LOOPKV_OK;
}

loopkv_status loopkv_auto_split(loopkv_plan p, int32_t batch, int32_t page_table_stride,
                                int32_t* split_tokens) {
  if (!p || !split_tokens || batch < 1 || batch > p->shape.max_batch || page_table_stride < 1)
    return LOOPKV_EINVAL;
  *split_tokens = auto_split(p, batch, decode_ctx(p, page_table_stride));
  return LOOPKV_OK;
}

loopkv_status loopkv_get_cell_info(loopkv_plan p, int32_t layer, int32_t loop,
                                   loopkv_cell_info* out) {
  if (!cell_ok(p, layer, loop) || !out) return LOOPKV_EINVAL;
  const CellDesc& d = p->desc[(size_t)loop * p->shape.num_layers + layer];
  out->code = d.code;
  out->read_bits = d.read_bits;
  out->gated = d.gated;
  out->head_block_bytes = (int32_t)(d.read_page_bytes / p->shape.num_kv_heads);
  out->page_bytes = d.read_page_bytes;
  out->read_pool_dev = d.read_pool;
  out->own_pool_dev = d.own_pool;
  out->tail_k_dev = d.tail_k;
  out->tail_v_dev = d.tail_v;
  out->qgroups_dev = d.own_qgroups;
  out->sink_k_dev = d.sink_k;
  out->sink_v_dev = d.sink_v;
  return LOOPKV_OK;
}

loopkv_status loopkv_device_errors(loopkv_plan p, void* stream, uint32_t* flags) {
  if (!p || !flags) return LOOPKV_EINVAL;
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint32_t v = 0;
  hipError_t e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemcpy(&v, p->err_dev, sizeof(v), hipMemcpyDeviceToHost);
  if (e == hipSuccess) e = hipMemset(p->err_dev, 0, sizeof(uint32_t));
  if (e != hipSuccess) return LOOPKV_EHIP;
  *flags = v;
  return LOOPKV_OK;
}

loopkv_status loopkv_quantize_append(loopkv_plan p, int32_t layer, int32_t loop,
                                     const void* k_new, const void* v_new, int32_t batch,
                                     int32_t n_new, const int32_t* n_new_dev,
                                     const int32_t* seq_lens, const int32_t* page_table,
                                     int32_t pt_stride, void* stream) {
  if (!cell_ok(p, layer, loop)) return LOOPKV_EINVAL;
  if (!k_new || !v_new || !seq_lens || !page_table) return LOOPKV_EINVAL;
  if (((uintptr_t)k_new | (uintptr_t)v_new) % 16 != 0) return LOOPKV_EINVAL;   // 16-byte rows
  if (batch < 1 || batch > p->shape.max_batch || n_new < 0 || pt_stride < 1) return LOOPKV_EINVAL;
  if ((int64_t)n_new > (int64_t)p->shape.max_pages_per_seq * p->shape.page_tokens)
    return LOOPKV_EINVAL;
  if (n_new == 0) return LOOPKV_OK;
  const size_t i = (size_t)loop * p->shape.num_layers + layer;
  hipError_t e = launch_append(make_geom(p), p->desc_dev + i, p->desc[i],
                               static_cast<const uint16_t*>(k_new),
                               static_cast<const uint16_t*>(v_new), batch, n_new, n_new_dev,
                               seq_lens, page_table, pt_stride, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LOOPKV_OK : LOOPKV_EHIP;
}

}  // extern "C"

namespace {

// Both decode entry points: `static_ws` takes the split partials and merge counters from the
// per-device static array instead of the plan's arena.
loopkv_status decode_impl(loopkv_plan p, int32_t layer, int32_t loop, const void* q, int32_t batch,
                          const int32_t* seq_lens, const int32_t* page_table, int32_t pt_stride,
                          const loopkv_decode_opts* opts, float* out, void* stream, bool static_ws) {
  if (!cell_ok(p, layer, loop)) return LOOPKV_EINVAL;
  if (!q || !seq_lens || !page_table || !out) return LOOPKV_EINVAL;
  if ((uintptr_t)q % 16 != 0) return LOOPKV_EINVAL;   // read in 16-byte pieces
  if (batch < 1 || batch > p->shape.max_batch || pt_stride < 1) return LOOPKV_EINVAL;
  loopkv_decode_opts o;
  std::memset(&o, 0, sizeof(o));
  if (opts) o = *opts;
  if (!std::isfinite(o.tau) || o.tau < 0.f) return LOOPKV_EINVAL;
  if (!std::isfinite(o.sm_scale) || o.sm_scale < 0.f) return LOOPKV_EINVAL;
  if (o.split_tokens != LOOPKV_SPLIT_AUTO && (o.split_tokens < 0 || o.split_tokens % kGroup != 0))
    return LOOPKV_EINVAL;
  Geom g = make_geom(p);
  const int64_t ctx = decode_ctx(p, pt_stride);
  if (o.split_tokens == LOOPKV_SPLIT_AUTO) o.split_tokens = auto_split(p, batch, ctx);
  if (o.fetch_mask_dev && (int64_t)o.mask_stride < ctx) return LOOPKV_EINVAL;
  const int64_t n_split = o.split_tokens ? (ctx + o.split_tokens - 1) / o.split_tokens : 1;
  float* partials = p->partials_dev;
  int32_t* counters = p->merge_dev;
  if (static_ws) {
    const uint64_t rows = (uint64_t)batch * g.H;
    if (rows * sizeof(int32_t) > kStaticWsCounterBytes ||
        rows * (uint64_t)n_split * (g.D + 2) * sizeof(float) > kStaticWsBytes - kStaticWsCounterBytes)
      return LOOPKV_ECAPACITY;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev != p->device) return LOOPKV_EINVAL;
    // set up (address looked up, counters cleared) by loopkv_plan_load on this device, so this
    // returns the kept address without a HIP call
    void* ws = static_workspace(dev, static_cast<hipStream_t>(stream));
    if (!ws) return LOOPKV_EHIP;
    counters = static_cast<int32_t*>(ws);
    partials = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + kStaticWsCounterBytes);
    g.max_splits = (int32_t)n_split;   // partial rows packed at this call's split count
  } else if (n_split > p->shape.max_splits) {
    return LOOPKV_ECAPACITY;
  }
  const size_t i = (size_t)loop * p->shape.num_layers + layer;
  DecodeCall c;
  c.desc_dev = p->desc_dev + i;
  c.q = static_cast<const uint16_t*>(q);
  c.seq_lens = seq_lens;
  c.page_table = page_table;
  c.pt_stride = pt_stride;
  c.batch = batch;
  c.tau = o.tau;
  c.sm_scale = o.sm_scale > 0.f ? o.sm_scale : 1.0f / std::sqrt((float)g.D);
  c.split_tokens = o.split_tokens;
  c.n_split = (int32_t)n_split;
  c.seed = o.seed_dev;
  c.mask = o.fetch_mask_dev;
  c.mask_stride = o.mask_stride;
  c.stats = o.stats_dev;
  c.out = out;
  c.partials = partials;
  c.counters = counters;
  c.order_by_len = 0;   // set by the launcher from the grid size
  c.sink_seed = o.no_sink_seed ? 0 : 1;
  hipError_t e = launch_decode(g, p->desc[i], c, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? LOOPKV_OK : LOOPKV_EHIP;
}

}  // namespace

extern "C" {

loopkv_status loopkv_decode_attention(loopkv_plan p, int32_t layer, int32_t loop,
                                      const void* q, int32_t batch, const int32_t* seq_lens,
                                      const int32_t* page_table, int32_t pt_stride,
                                      const loopkv_decode_opts* opts, float* out,
                                      void* stream) {
  return decode_impl(p, layer, loop, q, batch, seq_lens, page_table, pt_stride, opts, out, stream,
                     false);
}

loopkv_status loopkv_decode_attention_static(loopkv_plan p, int32_t layer, int32_t loop,
                                             const void* q, int32_t batch, const int32_t* seq_lens,
                                             const int32_t* page_table, int32_t pt_stride,
                                             const loopkv_decode_opts* opts, float* out,
                                             void* stream) {
  return decode_impl(p, layer, loop, q, batch, seq_lens, page_table, pt_stride, opts, out, stream,
                     true);
}

}  // extern "C"
