/*
 * loopkv.h -- C ABI of libloopkv: LoopKV's fused decode attention and its companion
 * quantize-append step, for one AMD Instinct MI355X (gfx950).
 *
 * Source of the operations: "Loop-Aware KV Cache Compression for Serving Looped
 * Transformers" (the LoopKV paper).
 *   - A cell is one (loop, layer) pair of a looped transformer; a plan gives each cell one
 *     storage option: 4-bit codes, 2-bit codes, or reuse of the final loop's KV at the same
 *     layer (section 3, "System Design"; section 3.1 C1; section 3.2 C2).
 *   - An INT4 cell stores values as a high and a low 2-bit plane; attention reads the high
 *     plane of every token and the low plane only for tokens whose weight reaches tau times
 *     a running maximum seeded by m0 (section 3.3 C3, "Read-time V precision").
 *   - One launch per cell reads its history pages through a per-cell descriptor built at plan
 *     load; split partials merge by log-sum-exp (section 3.4, "The unified kernel").
 *   - Optionally a sink (the first 32 tokens) and a recent window stay exact bf16; a 32-token
 *     page is quantized when it leaves the window, and the sink's largest score seeds the
 *     running maximum of the history (section 2.3, "Measuring KV damage"; section 3.2;
 *     section 3.4, "The unified kernel").
 *   - KIVI-style quantization (section 5.1, "Baselines"): keys per channel over a 32-token
 *     page, values per token over groups of channels, asymmetric, fp16 scale and zero point.
 *
 * Conventions for every entry point:
 *   - Pointers named *_dev are device pointers; all others are host pointers.
 *   - The caller owns every device buffer (arena, q, out, k_new, v_new, seq_lens, page
 *     table, seed, mask, stats). The library never allocates device memory; after
 *     loopkv_plan_load it only launches kernels and enqueues copies on the given stream, with
 *     no host synchronisation, so appends and decodes can be captured in a HIP graph.
 *   - Streams are hipStream_t passed as void*; NULL is the default stream.
 *   - Errors are status codes; nothing is thrown across the ABI. Host-side arguments are
 *     validated before anything is enqueued: on any status other than LOOPKV_OK nothing has
 *     been launched. Values that live in device memory (lengths, page ids) cannot be checked
 *     on the host; kernels clamp them and record a flag readable with loopkv_device_errors.
 *   - A plan handle is not thread-safe; calls on different handles are independent. Split
 *     decodes of one handle share its workspace and must be ordered (see
 *     loopkv_decode_attention).
 *   - loop and layer are 0-based; the final loop is num_loops - 1.
 */
#ifndef LOOPKV_H
#define LOOPKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct loopkv_plan_s* loopkv_plan; /* opaque; host memory owned by the library */

typedef enum {
  LOOPKV_OK = 0,
  LOOPKV_EINVAL = 1,    /* bad argument: null pointer, index or size out of range */
  LOOPKV_EPLAN = 2,     /* bad plan table: unknown code, or REUSE in the final loop */
  LOOPKV_ENOTSUP = 3,   /* a shape this library does not implement */
  LOOPKV_ECAPACITY = 4, /* arena smaller than loopkv_cache_bytes says, a split count
                           above shape.max_splits, or host memory exhausted */
  LOOPKV_EHIP = 5,      /* a HIP runtime call or kernel launch failed */
  LOOPKV_EINFEASIBLE = 6 /* loopkv_plan_solve: no plan meets the budgets */
} loopkv_status;

/* Plan codes, one uint8 per cell, indexed plan[loop * num_layers + layer]. */
enum { LOOPKV_REUSE = 0, LOOPKV_INT2 = 2, LOOPKV_INT4 = 4 };

/* Static shape of a cache. The key group is fixed at 32 tokens (one page of the paper);
 * a page of 16 tokens makes two pages per key group. */
typedef struct {
  int32_t num_layers;        /* L >= 1 */
  int32_t num_loops;         /* T >= 1 */
  int32_t num_kv_heads;      /* H >= 1 */
  int32_t num_q_heads;       /* must equal num_kv_heads (no grouped-query attention) */
  int32_t head_dim;          /* D; this library supports 128 */
  int32_t page_tokens;       /* tokens per physical page: 16 or 32 */
  int32_t v_group;           /* value channels per scale/zero: 32, 64 or 128 */
  int32_t max_batch;         /* requests per call, at most */
  int32_t max_pages_per_seq; /* page-table row capacity; context <= this * page_tokens */
  int32_t tail_tokens;       /* exact bf16 ring per (cell, request) for tokens not yet
                                quantized: 32..1024, a multiple of 32 (64 recommended);
                                with a window, at least window_tokens + 64 */
  int32_t max_splits;        /* split-K partials per row the workspace holds (>= 1) */
  int32_t sink_tokens;       /* 0 or 32: the first sink_tokens tokens of every request stay
                                exact bf16 and are never quantized */
  int32_t window_tokens;     /* 0, or a multiple of 32: a 32-token group past the sink is
                                quantized only once none of its tokens is among the last
                                window_tokens positions (0: as soon as it is complete) */
  int32_t reserved;          /* set to 0 */
  int64_t num_pages;         /* physical pages in each own-storage cell's pool */
} loopkv_shape;

/* Sizes, in bytes. The arena is: metadata | workspace | tails | sinks | pools. */
typedef struct {
  uint64_t arena_bytes;      /* total device bytes loopkv_plan_load needs */
  uint64_t pool_bytes;       /* page pools of all own-storage cells */
  uint64_t tail_bytes;       /* bf16 tail rings of all cells (REUSE cells keep their own) */
  uint64_t meta_bytes;       /* descriptors, quantized-group counters, error word, split
                                merge counters */
  uint64_t workspace_bytes;  /* split-K partials (the merge counters are in meta_bytes) */
  /* Bytes per token summed over every cell and head (algorithmic, excluding pool padding):
   * stored -- quantized KV kept (REUSE cells keep none);
   * read_hi_only / read_all_hot -- what one decode step reads per history token when no /
   * every low plane is fetched (a REUSE cell reads its source's bytes). */
  double stored_bytes_per_token;
  double read_bytes_per_token_hi_only;
  double read_bytes_per_token_all_hot;
  uint64_t sink_bytes;       /* bf16 sinks of all cells (REUSE cells keep their own) */
} loopkv_bytes;

/* split_tokens value that lets the library choose the split (loopkv_auto_split). */
enum { LOOPKV_SPLIT_AUTO = -1 };

/* Per-call decode options. */
typedef struct {
  float tau;                  /* V-precision threshold; 0 fetches every low plane, > 1 none */
  float sm_scale;             /* score scale; 0 means 1/sqrt(head_dim) */
  int32_t split_tokens;       /* 0: one split per (request, head) row; a multiple of 32: the
                                 history is cut into runs of this many tokens from token 0,
                                 each with its own running maximum, merged by log-sum-exp in
                                 split order inside the same launch (section 3.4, "The unified
                                 kernel": the last block of a row merges the partials);
                                 LOOPKV_SPLIT_AUTO: the split loopkv_auto_split returns */
  int32_t mask_stride;        /* row stride of fetch_mask_dev, in bytes */
  const float* seed_dev;      /* [batch, num_q_heads] running-max seeds in score units, or
                                 NULL for -infinity */
  uint8_t* fetch_mask_dev;    /* optional [batch, num_q_heads, mask_stride]: per history
                                 token, 1 if its low plane was read (hot), 0 if not (cold);
                                 1 for every history token of a cell read at 2 bits; tail
                                 entries are not written. NULL to skip. */
  unsigned long long* stats_dev; /* optional [4] counters, accumulated (not reset):
                                 [0] history (token, head) pairs read, [1] of those, pairs
                                 whose low plane was read, [2] pairs read from INT4 pools,
                                 [3] exact (token, head) pairs: sink, window and tail.
                                 NULL to skip. */
  int32_t no_sink_seed;       /* 0: with a sink, the running maximum starts at the larger of
                                 the seed and the sink's largest score (section 3.4); 1: at the
                                 seed alone */
} loopkv_decode_opts;

/* Device view of one cell, for inspection by callers and tests. */
typedef struct {
  int32_t code;               /* the plan code of this cell */
  int32_t read_bits;          /* bits of the pool this cell reads (the source's for REUSE) */
  int32_t gated;              /* 1 if the low plane is fetched only for hot tokens */
  int32_t head_block_bytes;   /* bytes of one head of one page */
  int64_t page_bytes;         /* num_kv_heads * head_block_bytes */
  void* read_pool_dev;        /* pool this cell reads (own, or the final loop's) */
  void* own_pool_dev;         /* pool this cell writes; NULL for REUSE */
  void* tail_k_dev;           /* bf16 [max_batch, tail_tokens, H, D] ring, slot = pos % tail */
  void* tail_v_dev;
  int32_t* qgroups_dev;       /* int32 [max_batch]: end of the quantized history in 32-token
                                 groups (own storage only; a REUSE cell reads its source's) */
  void* sink_k_dev;           /* bf16 [max_batch, sink_tokens, H, D] exact sink; NULL without */
  void* sink_v_dev;
} loopkv_cell_info;

/* Sizes of the arena for `shape` and `plan` (num_loops * num_layers codes), and the
 * stored / read bytes per token. The per-token figures follow the paper's byte model:
 * BF16 KV, KIVI-4 and the INT2 / shared-loop variants (section 2.2 "Looped transformers and
 * their KV cache", section 3.1 C1), a shared cell storing nothing and reading its source
 * (section 3.2 C2), the low plane counted only when read (section 3.3 C3), and the per-cell
 * totals of Table 5; with 32-channel value groups they reproduce the paper's KiB-per-token
 * figures exactly. out->stored_bytes_per_token excludes pool padding; arena_bytes includes
 * every region (metadata, split workspace, rings, sinks, pools), each 256-byte aligned.
 * Errors: LOOPKV_EINVAL (null pointer, bad shape field), LOOPKV_ENOTSUP (a shape outside the
 * library's support), LOOPKV_EPLAN (bad plan code, REUSE in the final loop), LOOPKV_ECAPACITY
 * (host memory exhausted). Pure host computation; no HIP call; `out` is written only on
 * LOOPKV_OK. */
loopkv_status loopkv_cache_bytes(const loopkv_shape* shape, const uint8_t* plan,
                                 loopkv_bytes* out);

/* Builds one descriptor per cell (section 3.4) in the caller's device arena and returns a
 * handle. The arena must hold at least loopkv_cache_bytes().arena_bytes bytes and be
 * 256-byte aligned. Counters and the error word are zeroed on `stream`; pools and tails are
 * not touched (their contents are defined only where appends wrote them). The plan table
 * is copied; `plan` may be freed after the call. */
loopkv_status loopkv_plan_load(const loopkv_shape* shape, const uint8_t* plan,
                               void* arena_dev, uint64_t arena_bytes, void* stream,
                               loopkv_plan* out);

/* Releases the handle (host memory only; the arena stays the caller's). NULL is a no-op. */
loopkv_status loopkv_plan_free(loopkv_plan plan);

/* Appends new tokens to every request of cell (layer, loop): the companion step that keeps
 * the cache in the form decode reads. Sources: KIVI-style asymmetric quantization with fp16
 * scale and zero point -- keys per channel over a 32-token group, values per token over
 * v_group channels (section 5.1, "Baselines"); an INT4 cell's value codes split into a high
 * and a low 2-bit plane (section 3.3, "Bit-plane V layout"); a page is quantized when it leaves
 * the exact window (section 2.3, "Measuring KV damage"; section 4, "Implementation"); a shared
 * (REUSE) cell keeps only its own exact tokens (section 3.2 C2). Codes are
 * clamp(floor((x - z) / s + 1/2)) decided as in fp64 from the bf16 inputs; s and z are rounded
 * to the nearest fp16 from fp64. Groups whose range exceeds the fp16 scale (a range above
 * 65504 * (2^bits - 1)) or whose minimum exceeds the fp16 range are not representable.
 *   k_new_dev, v_new_dev: bf16 [batch, n_new, num_kv_heads, head_dim], contiguous, 16-byte
 *   aligned (LOOPKV_EINVAL otherwise).
 *   n_new_dev: optional int32 [batch]: request b appends its first n_new_dev[b] rows
 *   (0 <= n_new_dev[b] <= n_new); NULL appends all n_new rows of every request.
 *   seq_lens_dev: int32 [batch], tokens each request held before this append.
 *   page_table_dev: int32 [batch, page_table_stride], logical page -> physical page id in
 *   [0, num_pages); one table serves every cell.
 * With m = the request's appended count, its last min(m, tail_tokens) tokens enter the
 * cell's bf16 ring, and those at positions below sink_tokens also enter its sink. With
 * n = seq_len + m, the quantized history of a request ends at group
 *   qend(n) = max(sink_tokens / 32, floor((n - window_tokens) / 32))
 * (groups below sink_tokens / 32 are the sink). For an own-storage cell, every group in
 * [qend(seq_len), qend(n)) -- the groups this append moves out of the window -- is quantized
 * into the cell's pool (KIVI-style, fp16 scale/zero, INT4 values split into hi/lo planes) and
 * the cell's counter becomes qend(n). A REUSE cell only fills its ring and sink: its history
 * is the final loop's pool, as far as that cell's counter says. n_new == 0 is a no-op.
 * Precondition (device data): the tokens of a group quantized by this call that precede it
 * are still in the ring, i.e. every earlier append of the request also ran. */
loopkv_status loopkv_quantize_append(loopkv_plan plan, int32_t layer, int32_t loop,
                                     const void* k_new_dev, const void* v_new_dev,
                                     int32_t batch, int32_t n_new,
                                     const int32_t* n_new_dev,
                                     const int32_t* seq_lens_dev,
                                     const int32_t* page_table_dev,
                                     int32_t page_table_stride, void* stream);

/* Decode attention of cell (layer, loop) for one query token per request.
 *   q_dev: bf16 [batch, num_q_heads, head_dim], 16-byte aligned (LOOPKV_EINVAL otherwise);
 *   out_dev: fp32 [batch, num_q_heads, head_dim].
 *   seq_lens_dev: int32 [batch], context length including the newest token.
 * With n = seq_len, S = sink_tokens and g = max(S / 32, min(source counter, qend(n))):
 * sink = tokens [0, min(n, S)), read exactly from the cell's own sink; history = tokens
 * [S, 32*g), read from the pool the cell's descriptor names; tail = tokens [32*g, n), read
 * exactly from the cell's own ring (at most tail_tokens of them). Scores are
 * sm_scale * q . k^; softmax over sink, history and tail; history values of an INT4 pool
 * decode at full precision for hot tokens and to the middle of their high-plane bucket for
 * cold ones (section 3.3), with the running maximum of each split seeded by the seed joined
 * with the sink's largest score. A request with seq_len 0 gets zeros. opts may be NULL
 * (tau 0, default scale, no split). Every call is one kernel launch, split or not.
 * Value range: any finite fp16 value scale (the weights are rescaled per wave by powers of
 * two, section 3.3 keeps a scale per group); exact (bf16) sink, window and tail values must
 * be below 2^118 in magnitude. History scores are formed on the matrix cores from q * s_K
 * rounded to 24 bits relative to the largest |q * s_K| of its 32-channel block (about fp32's
 * precision for the score); in a block whose largest |q * s_K| is below 2^-110 the
 * score's absolute error stays below 2^-100, and every q * s_K must be finite in fp32.
 * Workspace: the split partials and the merge counters are one region of the plan's arena,
 * so split decodes of one plan (split_tokens != 0) must not overlap in time: issue them on
 * one stream (or order the streams), as the calls of one model step are. Errors:
 * LOOPKV_EINVAL (null pointer, misaligned q, batch or stride out of range, tau or sm_scale
 * negative or not finite, split_tokens not a multiple of 32 nor LOOPKV_SPLIT_AUTO, a mask
 * stride below the context), LOOPKV_ECAPACITY (more splits than shape.max_splits),
 * LOOPKV_EHIP (the launch failed). */
loopkv_status loopkv_decode_attention(loopkv_plan plan, int32_t layer, int32_t loop,
                                      const void* q_dev, int32_t batch,
                                      const int32_t* seq_lens_dev,
                                      const int32_t* page_table_dev,
                                      int32_t page_table_stride,
                                      const loopkv_decode_opts* opts, float* out_dev,
                                      void* stream);

/* loopkv_decode_attention for callers that cannot allocate device memory or must not touch
 * the plan's arena workspace (code under HIP graph capture that owns no workspace, tight
 * serving loops, harnesses that forbid allocation): identical arguments, semantics, results
 * (bit for bit) and errors, except that the split partials and merge counters live in a fixed
 * 4 MiB device array of the library, one per GPU, whose address is looked up (and whose
 * counters are cleared) by loopkv_plan_load on that GPU. The call allocates nothing and
 * issues only the decode launch. Limit: batch * num_kv_heads <= 16384 and
 * batch * num_kv_heads * (number of splits) <= 7939 (the partials' 4 MiB - 64 KiB), else
 * LOOPKV_ECAPACITY before anything is enqueued; shape.max_splits does not apply. The device
 * current at the call must be the plan's (LOOPKV_EINVAL otherwise). Every call on a GPU shares
 * that GPU's array: split calls that overlap in time on one GPU (two streams, two threads, two
 * plans) race and give wrong results; the counters are back at zero after every call. */
loopkv_status loopkv_decode_attention_static(loopkv_plan plan, int32_t layer, int32_t loop,
                                             const void* q_dev, int32_t batch,
                                             const int32_t* seq_lens_dev,
                                             const int32_t* page_table_dev,
                                             int32_t page_table_stride,
                                             const loopkv_decode_opts* opts, float* out_dev,
                                             void* stream);

/* The split_tokens a decode with LOOPKV_SPLIT_AUTO uses for `batch` requests and a page table
 * of `page_table_stride` entries (context c = min(max_pages_per_seq, stride) * page_tokens):
 * n = min(ceil(4 * CUs / (batch * num_kv_heads)), 64, shape.max_splits, floor(c / 1024)) splits
 * (enough that the rows fill every compute unit of the device with four rows' waves, at most
 * 64 far blocks per row as in section 3.4, none shorter than 1024 tokens); 0 (no split) when
 * n <= 1, else ceil(c / n) rounded up to a multiple of 32. Deterministic for a device, so a
 * caller (or a test) can reproduce the fetch mask. Host only. Errors: LOOPKV_EINVAL. */
loopkv_status loopkv_auto_split(loopkv_plan plan, int32_t batch, int32_t page_table_stride,
                                int32_t* split_tokens);

/* Fills `out` with the device view of cell (layer, loop). Host only. */
loopkv_status loopkv_get_cell_info(loopkv_plan plan, int32_t layer, int32_t loop,
                                   loopkv_cell_info* out);

/* Waits for `stream`, then returns in *flags the OR of the device-side flags kernels raised
 * since the last call, and clears them: 1 = a length out of range, 2 = a page id out of
 * range, 4 = more tail tokens than the ring holds. */
loopkv_status loopkv_device_errors(loopkv_plan plan, void* stream, uint32_t* flags);

/* Budgets of loopkv_plan_solve. */
typedef struct {
  double max_damage;          /* the plan's damage (sum of its cells' damages) must not exceed
                                 this; a negative value means no damage budget */
  double max_stored_bytes;    /* stored bytes per token over all cells (loopkv_cache_bytes'
                                 stored_bytes_per_token) must not exceed this; <= 0: no budget */
  double hot_fraction;        /* in [0, 1]: share of INT4 low planes counted as read (1: every
                                 plane, as the paper's read figures count them) */
} loopkv_plan_budget;

/* What a plan costs: summed damage, stored and read bytes per token (read as counted above). */
typedef struct {
  double damage;
  double stored_bytes_per_token;
  double read_bytes_per_token;
} loopkv_plan_cost;

/* The planner (section 1; section 3.1 "Allocation"; Appendix "Layer-only allocation"): chooses
 * one option per cell -- INT4, INT2, or for loops before the last REUSE of the final loop's KV
 * at the same layer -- that minimises the bytes read per decode step subject to the damage and
 * storage budgets, exactly (a multiple-choice knapsack solved by dynamic programming over the
 * layers). A plan's damage is the sum of its cells' damages (section 2.4: damages add up); a
 * reusing cell stores nothing and reads its source's bytes. Among plans with the fewest read
 * bytes it returns one with the least damage, then the least storage.
 *   shape: num_loops <= 5, num_loops * num_layers <= 256; its heads, head_dim and v_group set
 *   the byte model (the one loopkv_cache_bytes uses).
 *   damage: host double [num_loops][num_layers][3], options ordered INT4, INT2, REUSE; the
 *   final loop's REUSE entry is ignored; the others must be finite.
 *   plan_out: host uint8 [num_loops * num_layers] (plan[loop * num_layers + layer]).
 *   cost_out: optional (NULL to skip).
 * Host only, no HIP call; it allocates about T^3 * L^4 / 4 bytes of host memory for the
 * program's back-pointers (5 MB for 4 x 24 cells, 85 MB for 4 x 48) and frees them before it
 * returns. LOOPKV_EINFEASIBLE when no plan meets the budgets (plan_out is then untouched);
 * LOOPKV_ENOTSUP beyond the size limits above; LOOPKV_ECAPACITY if that memory is not
 * available. */
loopkv_status loopkv_plan_solve(const loopkv_shape* shape, const double* damage,
                                const loopkv_plan_budget* budget, uint8_t* plan_out,
                                loopkv_plan_cost* cost_out);

/* Static string naming a status. */
const char* loopkv_status_string(loopkv_status status);

#ifdef __cplusplus
}
#endif

#endif /* LOOPKV_H */
