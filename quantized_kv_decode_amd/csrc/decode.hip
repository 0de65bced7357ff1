// Fused decode attention over one cell's quantized history and exact tail.
//
// "Loop-Aware KV Cache Compression for Serving Looped Transformers":
//  - one launch per cell reads history pages through the cell's descriptor, which names the
//    pool to read (its own, or the final loop's for a reusing cell), the stored bits, and
//    whether the low value plane is gated (section 3.4, "One launch per cell");
//  - for each page the key codes are read first, so every score of the page is known before
//    its values are touched; a token is cold when exp(s - m) < tau for a running maximum m
//    that starts at the seed, and a cold token reads only the high plane and decodes to the
//    middle of its bucket (section 3.3, "Read-time V precision");
//  - the per-channel key scale/zero fold into the query once per page, and the per-token value
//    scale/zero fold into the attention weight and a running sum (Appendix, "History reader");
//  - split partials merge by log-sum-exp, which gives the exact softmax (section 3.4).
//
// Work mapping (CDNA4, wave64): one workgroup of 4 waves per (request, head, split). In each
// round every wave takes one 32-token group; the group maxima are combined across the waves
// through LDS as a prefix maximum, so the hot/cold decisions are exactly those of streaming
// the split group by group, whatever the number of waves. Each wave keeps its own online
// softmax state; the waves merge at the end.
#include "loopkv_internal.h"

namespace loopkv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

template <int NVG>
struct Smem {
  alignas(16) float q[kHeadDim];
  alignas(16) float red[kWaves][16][36];    // per-wave key partials [channel block][token]
  alignas(16) float wbuf[kWaves][NVG][32];  // per-wave value weights [value group][token]
  int hot_list[kWaves][32];
  float gmax[2][kWaves];
  float fin_acc[kWaves][kHeadDim];
  float fin_M[kWaves], fin_L[kWaves], fin_C[kWaves][NVG];
  unsigned long long cnt_hist, cnt_hot;
};

struct RowCtx {
  const CellDesc* d;
  const int32_t* pt_row;
  int64_t head_off;
  int64_t num_pages;
  int P;
  uint32_t* err;
};

__device__ __forceinline__ const uint8_t* page_block(const RowCtx& r, int logical_page) {
  int pid = r.pt_row[logical_page];
  if (pid < 0 || pid >= r.num_pages) {
    atomicOr(r.err, (uint32_t)kErrPage);
    pid = 0;
  }
  return r.d->read_pool + (int64_t)pid * r.d->read_page_bytes + r.head_off;
}

// Score of the lane's tokens: key partials over the lane's channels, reduced through LDS.
// Returns, in lanes 0..31, the log2-scaled score of token `lane` of the group.
template <int BITS, int NVG>
__device__ float group_scores(Smem<NVG>& sm, const RowCtx& r, const Layout& lay, int grp,
                              int w, int lane, float scale2) {
  constexpr int KCH = 32 / BITS;          // channels per code word
  constexpr int NCB = kHeadDim / KCH;     // channel blocks
  constexpr int KTOK = kGroup * NCB / 64;  // tokens per lane (8 for INT4, 4 for INT2)
  const int cb = lane % NCB, tq = lane / NCB;
  const int t0 = tq * KTOK;               // first token of the lane within the group
  const int P = r.P;
  const int gpage0 = grp * kGroup / P;
  const uint8_t* blk0 = page_block(r, gpage0);
  const uint8_t* blk = (P == kGroup) ? blk0 : page_block(r, gpage0 + t0 / P);
  const int tl = t0 % P;
  // Key scale / zero of the lane's channels, folded into the query.
  const uint32_t* ksz = reinterpret_cast<const uint32_t*>(blk0 + lay.ksz) + cb * KCH;
  float qs[KCH];
  float kappa = 0.f;
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const uint32_t sz = ksz[i];
    const float q = sm.q[cb * KCH + i];
    qs[i] = q * f16_lo(sz);
    kappa = fmaf(q, f16_hi(sz), kappa);
  }
  const uint32_t* kw = reinterpret_cast<const uint32_t*>(blk + lay.kc) + cb * P + tl;
#pragma unroll
  for (int j = 0; j < KTOK; ++j) {
    const uint32_t word = kw[j];
    float acc = kappa;
#pragma unroll
    for (int i = 0; i < KCH; ++i)
      acc = fmaf(qs[i], (float)((word >> (BITS * i)) & ((1u << BITS) - 1)), acc);
    sm.red[w][cb][t0 + j] = acc;
  }
  wave_lds_sync();
  float s2 = -INFINITY;
  if (lane < kGroup) {
    float raw = 0.f;
#pragma unroll
    for (int c = 0; c < NCB; ++c) raw += sm.red[w][c][lane];
    s2 = raw * scale2;
  }
  wave_lds_sync();
  return s2;
}

struct DecodeParams {
  Geom g;
  DecodeCall c;
};

template <int BITS, int NVG>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams prm) {
  const Geom& g = prm.g;
  const DecodeCall& c = prm.c;
  constexpr float VS = BITS == 4 ? 4.f : 1.f;   // acc units: out numerator = VS*acc + C
  __shared__ Smem<NVG> sm;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const CellDesc* d = c.desc_dev;
  const int H = g.H;

  if (tid < kHeadDim) {
    const uint16_t qv = c.q[((size_t)b * H + h) * kHeadDim + tid];
    sm.q[tid] = __uint_as_float((uint32_t)qv << 16);
  }
  if (tid == 0) { sm.cnt_hist = 0; sm.cnt_hot = 0; }

  // Row extent.
  const int64_t cap = min((int64_t)g.max_ctx, (int64_t)c.pt_stride * g.P);
  int len = c.seq_lens[b];
  if (len < 0 || len > cap) {
    if (tid == 0 && split == 0 && h == 0) atomicOr(g.err, (uint32_t)kErrLength);
    len = 0;
  }
  int hist_groups = min(d->src_qgroups[b], len / kGroup);
  hist_groups = max(hist_groups, 0);
  int tail_begin = hist_groups * kGroup;
  int n_tail = len - tail_begin;
  if (n_tail > g.tail) {
    if (tid == 0 && split == 0 && h == 0) atomicOr(g.err, (uint32_t)kErrTail);
    tail_begin = len - g.tail;
    n_tail = g.tail;
  }
  int gs = 0, ge = hist_groups;
  if (c.n_split > 1) {
    const int gps = c.split_tokens / kGroup;
    gs = min(split * gps, hist_groups);
    ge = min(gs + gps, hist_groups);
  }
  const bool do_tail = split == c.n_split - 1 && n_tail > 0;

  RowCtx r;
  r.d = d;
  r.pt_row = c.page_table + (size_t)b * c.pt_stride;
  r.P = g.P;
  r.num_pages = g.num_pages;
  r.err = g.err;
  const Layout lay = head_layout(BITS, g.P, kHeadDim, NVG);
  r.head_off = (int64_t)h * lay.total;
  const bool gated = d->gated != 0;
  const float scale2 = c.sm_scale * kLog2e;
  const float log2tau = c.tau > 0.f ? log2f(c.tau) : -INFINITY;
  float m_run = c.seed ? c.seed[(size_t)b * H + h] * kLog2e : -INFINITY;
  __syncthreads();

  float M = -INFINITY, Lsum = 0.f;
  float Csum[NVG];
  float acc[16];
#pragma unroll
  for (int i = 0; i < NVG; ++i) Csum[i] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  const int cbv = lane & 7, tq8 = lane >> 3;     // value mapping: 16 channels x 4 tokens
  const int vg_lane = (cbv * 16) / (kHeadDim / NVG);
  uint8_t* mask_row = c.mask ? c.mask + ((size_t)b * H + h) * c.mask_stride : nullptr;
  unsigned long long my_hot = 0;

  const int n_groups = ge - gs;
  const int rounds = (n_groups + kWaves - 1) / kWaves;
  for (int rd = 0; rd < rounds; ++rd) {
    const int grp = gs + rd * kWaves + w;
    const bool active = grp < ge;
    float s2 = -INFINITY;
    if (active) s2 = group_scores<BITS, NVG>(sm, r, lay, grp, w, lane, scale2);
    const float gmax_w = wave_max(s2);
    if (lane == 0) sm.gmax[rd & 1][w] = gmax_w;
    __syncthreads();
    float mpre = m_run, mall = m_run;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
      const float x = sm.gmax[rd & 1][i];
      if (i <= w) mpre = fmaxf(mpre, x);
      mall = fmaxf(mall, x);
    }
    m_run = mall;
    if (!active) continue;

    // Online softmax rescale for this wave.
    const float Mn = fmaxf(M, gmax_w);
    const float f = (M == -INFINITY) ? 0.f : exp2f(M - Mn);
    M = Mn;
    Lsum *= f;
#pragma unroll
    for (int i = 0; i < NVG; ++i) Csum[i] *= f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] *= f;

    bool hot = true;
    const int P = g.P;
    if (lane < kGroup) {
      const float p = exp2f(s2 - M);
      if (gated) hot = !((s2 - mpre) < log2tau);
      const uint8_t* blk = page_block(r, (grp * kGroup + lane) / P);
      const uint32_t* vsz = reinterpret_cast<const uint32_t*>(blk + lay.vsz) + (lane % P) * NVG;
      Lsum += p;
#pragma unroll
      for (int i = 0; i < NVG; ++i) {
        const uint32_t sz = vsz[i];
        const float wv = p * f16_lo(sz);
        Csum[i] = fmaf(p, f16_hi(sz), Csum[i]);
        if (gated && !hot) Csum[i] = fmaf(1.5f, wv, Csum[i]);
        sm.wbuf[w][i][lane] = wv;
      }
      if (mask_row) mask_row[(size_t)grp * kGroup + lane] = hot ? 1 : 0;
    }
    const unsigned long long ball = __ballot(lane < kGroup && hot);
    const uint32_t hotmask = (uint32_t)ball;
    if (lane < kGroup && hot) sm.hot_list[w][__popc(hotmask & ((1u << lane) - 1u))] = lane;
    wave_lds_sync();

    // High plane (INT4) or codes (INT2): lane = 16 channels x 4 tokens.
    {
      const int t0 = tq8 * 4;
      const uint8_t* blk = page_block(r, (grp * kGroup + t0) / P);
      const uint4 words = *reinterpret_cast<const uint4*>(
          reinterpret_cast<const uint32_t*>(blk + lay.vc) + cbv * P + (t0 % P));
      const float4 wt = *reinterpret_cast<const float4*>(&sm.wbuf[w][vg_lane][t0]);
      const uint32_t wd[4] = {words.x, words.y, words.z, words.w};
      const float wf[4] = {wt.x, wt.y, wt.z, wt.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = fmaf(wf[j], (float)((wd[j] >> (2 * i)) & 3u), acc[i]);
    }
    // Low plane of the hot tokens only, compacted: 8 hot tokens per pass.
    if (BITS == 4) {
      const int nhot = __popc(hotmask);
      my_hot += (lane == 0) ? (unsigned long long)nhot : 0ull;
      for (int k = 0; k < nhot; k += 8) {
        const int idx = k + tq8;
        if (idx < nhot) {
          const int t = sm.hot_list[w][idx];
          const uint8_t* blk = page_block(r, (grp * kGroup + t) / P);
          const uint32_t lo = reinterpret_cast<const uint32_t*>(blk + lay.vlo)[(t % P) * (kHeadDim / 16) + cbv];
          const float wq = 0.25f * sm.wbuf[w][vg_lane][t];
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[i] = fmaf(wq, (float)((lo >> (2 * i)) & 3u), acc[i]);
        }
      }
    }
    wave_lds_sync();
  }

  // Exact tail tokens (last split only), in chunks of 32, distributed over the waves.
  if (do_tail) {
    const int n_chunks = (n_tail + kGroup - 1) / kGroup;
    for (int ch = w; ch < n_chunks; ch += kWaves) {
      const int cb = lane & 15, tq = lane >> 4;   // keys: 8 channels x 8 tokens
      for (int j = 0; j < 8; ++j) {
        const int t = tq * 8 + j;
        const int pos = tail_begin + ch * kGroup + t;
        float part = 0.f;
        if (ch * kGroup + t < n_tail) {
          const size_t row = ((size_t)b * g.tail + (pos % g.tail)) * H + h;
          const uint4 kv = *reinterpret_cast<const uint4*>(d->tail_k + row * kHeadDim + cb * 8);
          const uint32_t kk[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            part = fmaf(sm.q[cb * 8 + 2 * i], bf16_lo(kk[i]), part);
            part = fmaf(sm.q[cb * 8 + 2 * i + 1], bf16_hi(kk[i]), part);
          }
        }
        sm.red[w][cb][t] = part;
      }
      wave_lds_sync();
      float s2 = -INFINITY;
      if (lane < kGroup && ch * kGroup + lane < n_tail) {
        float raw = 0.f;
#pragma unroll
        for (int cc = 0; cc < 16; ++cc) raw += sm.red[w][cc][lane];
        s2 = raw * scale2;
      }
      const float gm = wave_max(s2);
      const float Mn = fmaxf(M, gm);
      const float f = (M == -INFINITY) ? 0.f : exp2f(M - Mn);
      M = Mn;
      Lsum *= f;
#pragma unroll
      for (int i = 0; i < NVG; ++i) Csum[i] *= f;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] *= f;
      if (lane < kGroup) {
        const float p = (ch * kGroup + lane < n_tail) ? exp2f(s2 - M) : 0.f;
        Lsum += p;
        sm.wbuf[w][0][lane] = p * (1.f / VS);
      }
      wave_lds_sync();
      for (int j = 0; j < 4; ++j) {
        const int t = tq8 * 4 + j;
        if (ch * kGroup + t >= n_tail) break;
        const int pos = tail_begin + ch * kGroup + t;
        const size_t row = ((size_t)b * g.tail + (pos % g.tail)) * H + h;
        const uint4* vp = reinterpret_cast<const uint4*>(d->tail_v + row * kHeadDim + cbv * 16);
        const uint4 v0 = vp[0], v1 = vp[1];
        const uint32_t vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        const float wt = sm.wbuf[w][0][t];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          acc[2 * i] = fmaf(wt, bf16_lo(vv[i]), acc[2 * i]);
          acc[2 * i + 1] = fmaf(wt, bf16_hi(vv[i]), acc[2 * i + 1]);
        }
      }
      wave_lds_sync();
    }
  }

  // Merge the waves: sum lanes, then combine the four softmax states.
  Lsum = wave_sum(lane < kGroup ? Lsum : 0.f);
#pragma unroll
  for (int i = 0; i < NVG; ++i) Csum[i] = wave_sum(lane < kGroup ? Csum[i] : 0.f);
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v = acc[i];
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    acc[i] = v;
  }
  if (lane < 8) {
#pragma unroll
    for (int i = 0; i < 16; ++i) sm.fin_acc[w][lane * 16 + i] = acc[i];
  }
  if (lane == 0) {
    sm.fin_M[w] = M;
    sm.fin_L[w] = Lsum;
#pragma unroll
    for (int i = 0; i < NVG; ++i) sm.fin_C[w][i] = Csum[i];
    if (c.stats) {
      atomicAdd(&sm.cnt_hot, my_hot);
    }
  }
  __syncthreads();
  if (tid < kHeadDim) {
    float Mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) Mx = fmaxf(Mx, sm.fin_M[i]);
    float num = 0.f, den = 0.f;
    if (Mx != -INFINITY) {
      const int vg = tid / (kHeadDim / NVG);
#pragma unroll
      for (int i = 0; i < kWaves; ++i) {
        const float fw = sm.fin_M[i] == -INFINITY ? 0.f : exp2f(sm.fin_M[i] - Mx);
        num = fmaf(fw, VS * sm.fin_acc[i][tid] + sm.fin_C[i][vg], num);
        den = fmaf(fw, sm.fin_L[i], den);
      }
    }
    const size_t row = (size_t)b * H + h;
    if (c.n_split == 1) {
      c.out[row * kHeadDim + tid] = den > 0.f ? num / den : 0.f;
    } else {
      float* part = c.partials + (row * g.max_splits + split) * (kHeadDim + 2);
      part[2 + tid] = num;
      if (tid == 0) { part[0] = Mx; part[1] = den; }
    }
  }
  if (tid == 0 && c.stats) {
    const unsigned long long nh = (unsigned long long)(ge - gs) * kGroup;
    atomicAdd(&c.stats[0], nh);
    if (gated) {
      atomicAdd(&c.stats[1], sm.cnt_hot);
      atomicAdd(&c.stats[2], nh);
    }
    if (do_tail) atomicAdd(&c.stats[3], (unsigned long long)n_tail);
  }
}

// Log-sum-exp merge of the split partials of each (request, head), in split order.
__global__ __launch_bounds__(kHeadDim) void merge_kernel(Geom g, DecodeCall c) {
  const int h = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const size_t row = (size_t)b * g.H + h;
  const float* base = c.partials + row * g.max_splits * (kHeadDim + 2);
  float Mx = -INFINITY;
  for (int s = 0; s < c.n_split; ++s) Mx = fmaxf(Mx, base[s * (kHeadDim + 2)]);
  float num = 0.f, den = 0.f;
  if (Mx != -INFINITY) {
    for (int s = 0; s < c.n_split; ++s) {
      const float* p = base + s * (kHeadDim + 2);
      const float fw = p[0] == -INFINITY ? 0.f : exp2f(p[0] - Mx);
      num = fmaf(fw, p[2 + tid], num);
      den = fmaf(fw, p[1], den);
    }
  }
  c.out[row * kHeadDim + tid] = den > 0.f ? num / den : 0.f;
}

template <int BITS>
hipError_t launch_bits(const Geom& g, const DecodeCall& c, hipStream_t stream) {
  DecodeParams prm{g, c};
  const dim3 grid((unsigned)c.n_split, (unsigned)g.H, (unsigned)c.batch);
  switch (g.nvg) {
    case 1: decode_kernel<BITS, 1><<<grid, kThreads, 0, stream>>>(prm); break;
    case 2: decode_kernel<BITS, 2><<<grid, kThreads, 0, stream>>>(prm); break;
    case 4: decode_kernel<BITS, 4><<<grid, kThreads, 0, stream>>>(prm); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const Geom& g, const CellDesc& dh, const DecodeCall& c, hipStream_t stream) {
  hipError_t e = dh.read_bits == 4 ? launch_bits<4>(g, c, stream) : launch_bits<2>(g, c, stream);
  if (e != hipSuccess || c.n_split == 1) return e;
  merge_kernel<<<dim3((unsigned)g.H, (unsigned)c.batch), kHeadDim, 0, stream>>>(g, c);
  return hipGetLastError();
}

}  // namespace loopkv
