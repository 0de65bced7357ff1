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
// through LDS as a prefix maximum, so the hot/cold decisions are exactly those of streaming the
// split group by group, whatever the number of waves. Each wave keeps its own online-softmax
// state; the waves merge at the end.
//
// Latency hiding: every data-independent load of a wave's next group (key codes and scales,
// value high plane or INT2 codes, value scales) is issued one round ahead into registers; the
// low planes of a round's hot tokens are loaded in that round and accumulated in the next.
//
// Code unpacking: a 2- or 4-bit code placed in the low bits of an fp8 (E4M3) byte converts
// exactly to code * u, with u the value of byte 0x01, because E4M3's subnormals and first
// binade are evenly spaced up to 15 * u. One masked word thus yields four codes as floats with
// two packed conversions; the constant u (and the factor 4 of codes sitting two bits up in
// their byte) folds into the query or into the per-channel output scale.
#include "loopkv_internal.h"

namespace loopkv {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr float kLog2e = 1.4426950408889634f;

typedef float float2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}
// Bytes 0,1 (hi = false) or 2,3 (hi = true) of w as fp8 -> two floats.
template <bool HI>
__device__ __forceinline__ float2v cvt2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
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

// 16 two-bit codes of a word (channel i at bits 2i) as floats in "scaled units": channel i is
// returned as code * u * (i odd ? 4 : 1).
__device__ __forceinline__ void unpack16(uint32_t w, float (&x)[16]) {
  const uint32_t m0 = w & 0x03030303u, m1 = w & 0x0C0C0C0Cu;
  const uint32_t w4 = w >> 4;
  const uint32_t m2 = w4 & 0x03030303u, m3 = w4 & 0x0C0C0C0Cu;
  float2v a = cvt2<false>(m0), b = cvt2<true>(m0);   // channels 0,4 | 8,12
  float2v c = cvt2<false>(m1), d = cvt2<true>(m1);   // 1,5 | 9,13 (x4)
  float2v e = cvt2<false>(m2), f = cvt2<true>(m2);   // 2,6 | 10,14
  float2v g = cvt2<false>(m3), h = cvt2<true>(m3);   // 3,7 | 11,15 (x4)
  x[0] = a.x; x[4] = a.y; x[8] = b.x; x[12] = b.y;
  x[1] = c.x; x[5] = c.y; x[9] = d.x; x[13] = d.y;
  x[2] = e.x; x[6] = e.y; x[10] = f.x; x[14] = f.y;
  x[3] = g.x; x[7] = g.y; x[11] = h.x; x[15] = h.y;
}

// 8 four-bit codes of a word (channel i at bits 4i) as floats: code * u.
__device__ __forceinline__ void unpack8(uint32_t w, float (&x)[8]) {
  const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
  float2v a = cvt2<false>(lo), b = cvt2<true>(lo);   // 0,2 | 4,6
  float2v c = cvt2<false>(hi), d = cvt2<true>(hi);   // 1,3 | 5,7
  x[0] = a.x; x[2] = a.y; x[4] = b.x; x[6] = b.y;
  x[1] = c.x; x[3] = c.y; x[5] = d.x; x[7] = d.y;
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
  unsigned long long cnt_hot;
};

// Per-lane registers of one group, loaded one round ahead.
template <int BITS, int NVG>
struct GroupRegs {
  static constexpr int KCW = BITS == 4 ? 2 : 1;   // uint4 of key code words
  static constexpr int KSW = BITS == 4 ? 2 : 4;   // uint4 of key (s, z) words
  uint4 kc[KCW];
  uint4 ksz[KSW];
  uint4 vc;
  uint32_t vsz[NVG];
};

struct RowCtx {
  const uint8_t* pool;
  int64_t page_bytes;
  const int32_t* pt_row;
  int64_t head_off;
  int64_t num_pages;
  uint32_t* err;
};

__device__ __forceinline__ const uint8_t* page_block(const RowCtx& r, int logical_page) {
  int pid = r.pt_row[logical_page];
  if (pid < 0 || pid >= r.num_pages) {
    atomicOr(r.err, (uint32_t)kErrPage);
    pid = 0;
  }
  return r.pool + (int64_t)pid * r.page_bytes + r.head_off;
}

template <int BITS, int NVG, int P>
__device__ __forceinline__ void load_group(GroupRegs<BITS, NVG>& g, const RowCtx& r, const Layout& lay,
                                           int grp, int lane) {
  constexpr int KCH = 32 / BITS;
  constexpr int NCB = kHeadDim / KCH;
  constexpr int KTOK = kGroup * NCB / 64;
  const int cb = lane % NCB, tq = lane / NCB;
  const int t0 = tq * KTOK;
  const int lp0 = grp * (kGroup / P);
  const uint8_t* blk0 = page_block(r, lp0);
  const uint8_t* blk1 = P == kGroup ? blk0 : page_block(r, lp0 + 1);
  {  // key codes of KTOK tokens of channel block cb
    const uint8_t* b = t0 < P ? blk0 : blk1;
    const uint4* p = reinterpret_cast<const uint4*>(b + lay.kc + 4 * (cb * P + t0 % P));
#pragma unroll
    for (int i = 0; i < GroupRegs<BITS, NVG>::KCW; ++i) g.kc[i] = p[i];
  }
  {  // key (s, z) of the lane's channels, stored with the group's first page
    const uint4* p = reinterpret_cast<const uint4*>(blk0 + lay.ksz + 4 * cb * KCH);
#pragma unroll
    for (int i = 0; i < GroupRegs<BITS, NVG>::KSW; ++i) g.ksz[i] = p[i];
  }
  {  // value codes / high plane: 16 channels x 4 tokens
    const int cbv = lane & 7, t4 = (lane >> 3) * 4;
    const uint8_t* b = t4 < P ? blk0 : blk1;
    g.vc = *reinterpret_cast<const uint4*>(b + lay.vc + 4 * (cbv * P + t4 % P));
  }
  {  // value (s, z) of token `lane` (lanes 0..31)
    const int t = lane & 31;
    const uint8_t* b = t < P ? blk0 : blk1;
    const uint32_t* p = reinterpret_cast<const uint32_t*>(b + lay.vsz) + (t % P) * NVG;
#pragma unroll
    for (int i = 0; i < NVG; ++i) g.vsz[i] = p[i];
  }
}

struct DecodeParams {
  Geom g;
  DecodeCall c;
};

template <int BITS, int NVG, int P>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeParams prm) {
  const Geom& g = prm.g;
  const DecodeCall& c = prm.c;
  constexpr int KCH = 32 / BITS;
  constexpr int NCB = kHeadDim / KCH;
  constexpr int KTOK = kGroup * NCB / 64;
  constexpr float VS = BITS == 4 ? 4.f : 1.f;   // true numerator = VS * acc + C
  __shared__ Smem<NVG> sm;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const CellDesc* d = c.desc_dev;
  const int H = g.H;
  const float u = cvt2<false>(1u).x;            // value of fp8 byte 0x01
  const float inv_u = 1.0f / u;

  if (tid < kHeadDim) {
    const uint16_t qv = c.q[((size_t)b * H + h) * kHeadDim + tid];
    sm.q[tid] = __uint_as_float((uint32_t)qv << 16);
  }
  if (tid == 0) sm.cnt_hot = 0;

  // Row extent.
  const int64_t cap = min((int64_t)g.max_ctx, (int64_t)c.pt_stride * P);
  int len = c.seq_lens[b];
  if (len < 0 || len > cap) {
    if (tid == 0 && split == 0 && h == 0) atomicOr(g.err, (uint32_t)kErrLength);
    len = 0;
  }
  int hist_groups = max(min(d->src_qgroups[b], len / kGroup), 0);
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
  r.pool = d->read_pool;
  r.page_bytes = d->read_page_bytes;
  r.pt_row = c.page_table + (size_t)b * c.pt_stride;
  r.num_pages = g.num_pages;
  r.err = g.err;
  const Layout lay = head_layout(BITS, P, kHeadDim, NVG);
  r.head_off = (int64_t)h * lay.total;
  const bool gated = d->gated != 0;
  const float scale2 = c.sm_scale * kLog2e;
  const float log2tau = c.tau > 0.f ? log2f(c.tau) : -INFINITY;
  float m_run = c.seed ? c.seed[(size_t)b * H + h] * kLog2e : -INFINITY;

  const int cb = lane % NCB, tq = lane / NCB;      // key mapping
  const int cbv = lane & 7, tq8 = lane >> 3;       // value mapping: 16 channels x 4 tokens
  const int vg_lane = (cbv * 16) / (kHeadDim / NVG);
  uint8_t* mask_row = c.mask ? c.mask + ((size_t)b * H + h) * c.mask_stride : nullptr;

  const int n_groups = ge - gs;
  const int rounds = (n_groups + kWaves - 1) / kWaves;
  GroupRegs<BITS, NVG> cur, nxt;
  if (gs + w < ge) load_group<BITS, NVG, P>(cur, r, lay, gs + w, lane);
  __syncthreads();

  // The lane's query channels, scaled by 1/u (and by 1/4 for INT2 codes two bits up).
  float qv[KCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const float q = sm.q[cb * KCH + i];
    qv[i] = (BITS == 2 && (i & 1)) ? q * 0.25f * inv_u : q * inv_u;
  }
  float qraw[KCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) qraw[i] = sm.q[cb * KCH + i];

  float M = -INFINITY, Lsum = 0.f;
  float Csum[NVG];
  float acc[16];
#pragma unroll
  for (int i = 0; i < NVG; ++i) Csum[i] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  // Low planes loaded last round, accumulated this round (up to 4 hot tokens per lane).
  uint32_t lo_word[4] = {0u, 0u, 0u, 0u};
  float lo_wt[4] = {0.f, 0.f, 0.f, 0.f};
  unsigned long long my_hot = 0;

  for (int rd = 0; rd < rounds; ++rd) {
    const int grp = gs + rd * kWaves + w;
    const bool active = grp < ge;
    const int nxt_grp = grp + kWaves;
    if (nxt_grp < ge) load_group<BITS, NVG, P>(nxt, r, lay, nxt_grp, lane);

    // ---- scores of the group (key codes read first, section 3.3)
    float s2 = -INFINITY;
    if (active) {
      float qs[KCH], kappa = 0.f;
      const uint32_t* kszw = reinterpret_cast<const uint32_t*>(cur.ksz);
#pragma unroll
      for (int i = 0; i < KCH; ++i) {
        const uint32_t sz = kszw[i];
        qs[i] = qv[i] * f16_lo(sz);
        kappa = fmaf(qraw[i], f16_hi(sz), kappa);
      }
      const uint32_t* kw = reinterpret_cast<const uint32_t*>(cur.kc);
      float part[KTOK];
#pragma unroll
      for (int j = 0; j < KTOK; ++j) {
        float a = kappa;
        if (BITS == 4) {
          float x[8];
          unpack8(kw[j], x);
#pragma unroll
          for (int i = 0; i < 8; ++i) a = fmaf(qs[i], x[i], a);
        } else {
          float x[16];
          unpack16(kw[j], x);
#pragma unroll
          for (int i = 0; i < 16; ++i) a = fmaf(qs[i], x[i], a);
        }
        part[j] = a;
      }
      float* red = &sm.red[w][cb][tq * KTOK];
#pragma unroll
      for (int j = 0; j < KTOK; j += 4)
        *reinterpret_cast<float4*>(red + j) = make_float4(part[j], part[j + 1], part[j + 2], part[j + 3]);
      wave_lds_sync();
      // all 64 lanes: lane l sums channel blocks [half*NCB/2, +NCB/2) of token l & 31
      const int t = lane & 31, half = lane >> 5;
      float raw = 0.f;
#pragma unroll
      for (int k = 0; k < NCB / 2; ++k) raw += sm.red[w][half * (NCB / 2) + k][t];
      raw += __shfl_xor(raw, 32);
      s2 = raw * scale2;
    }
    const float gmax_w = wave_max(active ? s2 : -INFINITY);
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

    if (active) {
      // ---- online softmax rescale, then last round's low planes
      const float Mn = fmaxf(M, gmax_w);
      const float f = (M == -INFINITY) ? 0.f : exp2f(M - Mn);
      M = Mn;
      Lsum *= f;
#pragma unroll
      for (int i = 0; i < NVG; ++i) Csum[i] *= f;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[i] *= f;
      if (BITS == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          if (lo_wt[k] != 0.f) {
            float x[16];
            unpack16(lo_word[k], x);
            const float wq = lo_wt[k] * f;
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[i] = fmaf(wq, x[i], acc[i]);
          }
        }
      }

      // ---- per token (lanes 0..31): weight, hot/cold, value scale/zero folds
      bool hot = true;
      if (lane < kGroup) {
        const float p = exp2f(s2 - M);
        if (gated) hot = !((s2 - mpre) < log2tau);
        Lsum += p;
#pragma unroll
        for (int i = 0; i < NVG; ++i) {
          const uint32_t sz = cur.vsz[i];
          const float wv = p * f16_lo(sz);
          Csum[i] = fmaf(p, f16_hi(sz), Csum[i]);
          if (gated && !hot) Csum[i] = fmaf(1.5f, wv, Csum[i]);
          sm.wbuf[w][i][lane] = wv;
        }
        if (mask_row) mask_row[(size_t)grp * kGroup + lane] = hot ? 1 : 0;
      }
      const uint32_t hotmask = (uint32_t)__ballot(lane < kGroup && hot);
      if (BITS == 4 && lane < kGroup && hot) sm.hot_list[w][__popc(hotmask & ((1u << lane) - 1u))] = lane;
      wave_lds_sync();

      // ---- issue the low-plane loads of the hot tokens (accumulated next round)
      if (BITS == 4) {
        const int nhot = __popc(hotmask);
        my_hot += nhot;
        const int lp0 = grp * (kGroup / P);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int idx = 8 * k + tq8;
          lo_wt[k] = 0.f;
          if (idx < nhot) {
            const int t = sm.hot_list[w][idx];
            const uint8_t* blk = page_block(r, lp0 + t / P);
            lo_word[k] = reinterpret_cast<const uint32_t*>(blk + lay.vlo)[(t % P) * (kHeadDim / 16) + cbv];
            lo_wt[k] = 0.25f * sm.wbuf[w][vg_lane][t];
          }
        }
      }

      // ---- high plane (INT4) or codes (INT2) of all 32 tokens
      {
        const float4 wt = *reinterpret_cast<const float4*>(&sm.wbuf[w][vg_lane][tq8 * 4]);
        const uint32_t wd[4] = {cur.vc.x, cur.vc.y, cur.vc.z, cur.vc.w};
        const float wf[4] = {wt.x, wt.y, wt.z, wt.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float x[16];
          unpack16(wd[j], x);
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[i] = fmaf(wf[j], x[i], acc[i]);
        }
      }
      wave_lds_sync();
    }
    cur = nxt;
  }
  // Low planes of the last round.
  if (BITS == 4) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if (lo_wt[k] != 0.f) {
        float x[16];
        unpack16(lo_word[k], x);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] = fmaf(lo_wt[k], x[i], acc[i]);
      }
    }
  }

  // Exact tail tokens (last split only), in chunks of 32, distributed over the waves.
  if (do_tail) {
    const int n_chunks = (n_tail + kGroup - 1) / kGroup;
    for (int ch = w; ch < n_chunks; ch += kWaves) {
      const int cbt = lane & 15, tqt = lane >> 4;   // keys: 8 channels x 8 tokens
      for (int j = 0; j < 8; ++j) {
        const int t = tqt * 8 + j;
        const int pos = tail_begin + ch * kGroup + t;
        float part = 0.f;
        if (ch * kGroup + t < n_tail) {
          const size_t row = ((size_t)b * g.tail + (pos % g.tail)) * H + h;
          const uint4 kv = *reinterpret_cast<const uint4*>(d->tail_k + row * kHeadDim + cbt * 8);
          const uint32_t kk[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            part = fmaf(sm.q[cbt * 8 + 2 * i], bf16_lo(kk[i]), part);
            part = fmaf(sm.q[cbt * 8 + 2 * i + 1], bf16_hi(kk[i]), part);
          }
        }
        sm.red[w][cbt][t] = part;
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
        sm.wbuf[w][0][lane] = p * (u / VS);         // into scaled units (x u)
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
          // channel 2i is even (scale u), channel 2i+1 is odd (scale 4u)
          acc[2 * i] = fmaf(wt, bf16_lo(vv[i]), acc[2 * i]);
          acc[2 * i + 1] = fmaf(4.f * wt, bf16_hi(vv[i]), acc[2 * i + 1]);
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
    acc[i] = v * ((i & 1) ? 0.25f * inv_u : inv_u);   // back from scaled units
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
    if (c.stats && BITS == 4) atomicAdd(&sm.cnt_hot, my_hot);
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

template <int BITS, int P>
hipError_t launch_bp(const Geom& g, const DecodeCall& c, hipStream_t stream) {
  DecodeParams prm{g, c};
  const dim3 grid((unsigned)c.n_split, (unsigned)g.H, (unsigned)c.batch);
  switch (g.nvg) {
    case 1: decode_kernel<BITS, 1, P><<<grid, kThreads, 0, stream>>>(prm); break;
    case 2: decode_kernel<BITS, 2, P><<<grid, kThreads, 0, stream>>>(prm); break;
    case 4: decode_kernel<BITS, 4, P><<<grid, kThreads, 0, stream>>>(prm); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const Geom& g, const CellDesc& dh, const DecodeCall& c, hipStream_t stream) {
  hipError_t e;
  if (dh.read_bits == 4)
    e = g.P == 32 ? launch_bp<4, 32>(g, c, stream) : launch_bp<4, 16>(g, c, stream);
  else
    e = g.P == 32 ? launch_bp<2, 32>(g, c, stream) : launch_bp<2, 16>(g, c, stream);
  if (e != hipSuccess || c.n_split == 1) return e;
  merge_kernel<<<dim3((unsigned)g.H, (unsigned)c.batch), kHeadDim, 0, stream>>>(g, c);
  return hipGetLastError();
}

}  // namespace loopkv
