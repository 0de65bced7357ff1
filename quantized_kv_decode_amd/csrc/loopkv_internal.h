// Internal definitions shared by the host side of libloopkv and its HIP kernels.
//
// Page layout (what a page holds follows "Loop-Aware KV Cache Compression for Serving
// Looped Transformers", section 3.3 "Bit-plane V layout" and section 3.4 "Layout"; the byte
// order below is this library's choice). A page is H head blocks, head-major. One head
// block of a page of P tokens, D channels and NVG value groups:
//
//   KSZ  4*D          fp16 (scale, zero) per channel of the key group starting in this page
//   KC   P*D*bits/8   key codes, token-major 32-bit words W[t][w] at word t*(D*bits/32) + w
//                       INT4: word w holds channels 8w..8w+7; channel 8w + i (i < 4) in bits
//                             8i..8i+3, channel 8w + 4 + i in bits 8i+4..8i+7
//                       INT2: word w holds channels 16w..16w+15; channel 16w + 4k + i
//                             (k, i < 4) in bits 8i+2k..8i+2k+1
//   VC   P*D/4        INT4 high plane / INT2 codes, W[cb][t] at word cb*P + t,
//                       channel 16*cb + i in bits 2i..2i+1
//   VSZ  4*P*NVG      fp16 (scale, zero) per (token, value group), token-major
//   VLO  P*D/4        INT4 low plane, token-major W[t][cb] at word t*(D/16) + cb, so one
//                       token's low plane is D/4 contiguous bytes
//
// Token-major key rows give each lane of a wave one contiguous load of 32 channels of one
// token, the operand of the score MFMA: masking a key word's nibbles (or 2-bit fields) into
// bytes leaves four consecutive channels per register, so the codes enter the MFMA with no
// reordering. Column-major value words give each lane contiguous 16-byte loads of several
// tokens of the same channels; the token-major low plane makes a hot token's fetch one
// contiguous D/4-byte row.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "loopkv.h"

namespace loopkv {

constexpr int kGroup = 32;     // tokens per key quantization group
constexpr int kHeadDim = 128;  // the only head_dim this library implements

enum DeviceError : uint32_t {
  kErrLength = 1u,  // a sequence length outside [0, max context]
  kErrPage = 2u,    // a page id outside [0, num_pages)
  kErrTail = 4u,    // more unquantized tokens than the ring holds
};

struct Layout {
  int32_t ksz, kc, vc, vsz, vlo, total;
};

__host__ __device__ constexpr Layout head_layout(int bits, int page_tokens, int head_dim, int nvg) {
  Layout l{};
  l.ksz = 0;
  l.kc = 4 * head_dim;
  l.vc = l.kc + page_tokens * head_dim * bits / 8;
  l.vsz = l.vc + page_tokens * head_dim / 4;
  l.vlo = l.vsz + 4 * page_tokens * nvg;
  l.total = l.vlo + (bits == 4 ? page_tokens * head_dim / 4 : 0);
  return l;
}

// End of the quantized history of a request holding n tokens, in 32-token groups: groups
// below sink / 32 are the exact sink, and a group past it is quantized once none of its
// tokens is among the last `window` positions ("Loop-Aware KV Cache Compression for Serving
// Looped Transformers", section 2.3 "Measuring KV damage", section 3.4 "The unified kernel").
__host__ __device__ inline int64_t quantized_end(int64_t n, int sink, int window) {
  const int64_t hs = sink / kGroup;
  const int64_t x = n - window;
  const int64_t he = x > 0 ? x / kGroup : 0;
  return he > hs ? he : hs;
}

// One descriptor per cell, built by loopkv_plan_load and kept in the arena.
struct CellDesc {
  uint8_t* read_pool;         // pool read by decode: own, or the final loop's (REUSE)
  uint8_t* own_pool;          // pool written by append; null for REUSE
  uint16_t* tail_k;           // bf16 ring [max_batch][tail_tokens][H][D]
  uint16_t* tail_v;
  uint16_t* sink_k;           // bf16 [max_batch][sink][H][D]; null without a sink
  uint16_t* sink_v;
  int32_t* src_qgroups;       // quantized-group counters of the cell whose pool is read
  int32_t* own_qgroups;       // this cell's counters (written by append for own storage)
  int64_t read_page_bytes;
  int64_t own_page_bytes;
  int32_t read_bits;          // 2 or 4
  int32_t own_bits;           // 0 (REUSE), 2 or 4
  int32_t gated;              // read_bits == 4
  int32_t code;
};

// Static shape, passed by value to every kernel.
struct Geom {
  int32_t H;             // kv heads (= q heads)
  int32_t D;             // head dim
  int32_t P;             // page tokens
  int32_t nvg;           // value groups per head
  int32_t v_group;       // channels per value group
  int32_t tail;          // ring tokens
  int32_t sink;          // exact sink tokens (0 or 32)
  int32_t window;        // exact window tokens
  int32_t max_ctx;       // max_pages_per_seq * P
  int32_t max_splits;
  int64_t num_pages;
  uint32_t* err;         // device error word
  int32_t cus;           // compute units of the device
};

// Host-side checks and the byte model shared by the API and the planner.
loopkv_status check_shape(const loopkv_shape* s);
// Algorithmic bytes of one (token, head) stored at `bits` (with_lo: an INT4 cell's low plane).
double token_head_bytes(int bits, int D, int nvg, bool with_lo);

// Launchers implemented next to their kernels.
hipError_t launch_append(const Geom& g, const CellDesc* desc_dev, const CellDesc& desc_host,
                         const uint16_t* k_new, const uint16_t* v_new, int batch, int n_new,
                         const int32_t* n_new_dev, const int32_t* seq_lens,
                         const int32_t* page_table, int pt_stride, hipStream_t stream);

struct DecodeCall {
  const CellDesc* desc_dev;
  const uint16_t* q;
  const int32_t* seq_lens;
  const int32_t* page_table;
  int32_t pt_stride;
  int32_t batch;
  float tau;
  float sm_scale;
  int32_t split_tokens;   // 0 = one split
  int32_t n_split;
  const float* seed;
  uint8_t* mask;
  int32_t mask_stride;
  unsigned long long* stats;
  float* out;
  float* partials;        // [batch, H, max_splits, D + 2]
  int32_t* counters;      // [batch, H]: finished splits per row group, zero between launches
  int32_t order_by_len;   // launch needs more than one generation: longest requests first
  int32_t sink_seed;      // seed the running maximum with the sink's largest score
};

hipError_t launch_decode(const Geom& g, const CellDesc& desc_host, const DecodeCall& c,
                         hipStream_t stream);

// Fixed per-GPU workspace of loopkv_decode_attention_static (static_workspace.hip): merge
// counters in the first kStaticWsCounterBytes, split partials after them.
constexpr uint64_t kStaticWsBytes = 4ull << 20;          // 4 MiB per device
constexpr uint64_t kStaticWsCounterBytes = 64ull << 10;  // counters for up to 16384 rows
// Device address of the workspace on device `device`, which must be current. The first call
// for a device looks the address up and clears the counters on `stream` (waiting for it);
// later calls return the kept address without a HIP call. nullptr if a HIP call fails.
void* static_workspace(int device, hipStream_t stream);

}  // namespace loopkv
