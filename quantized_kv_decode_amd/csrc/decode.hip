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
// Work mapping (CDNA4, wave64): one workgroup of NW waves per (request, head, split). In each
// round every wave takes one 32-token group; the group maxima are combined across the waves
// through LDS as a prefix maximum, so the hot/cold decisions are exactly those of streaming the
// split group by group, whatever NW is. Each wave keeps its own online-softmax state; the waves
// merge at the end. NW is chosen so that every workgroup of a launch is resident at once.
//
// Latency hiding: every data-independent load of a wave's next group (key codes and scales,
// value high plane or INT2 codes, value scales) is issued one round ahead into a second set of
// registers (the round loop alternates the two sets); the low planes of a round's hot tokens
// are loaded in that round and accumulated in the next. Pool and tail pointers are global and
// page-table / descriptor reads constant address space, so the loads are global (not flat)
// and uniform indices become scalar loads.
//
// Code unpacking: a 2- or 4-bit code placed in the low bits of an fp8 (E4M3) byte converts
// exactly to code * u, with u the value of byte 0x01, because E4M3's subnormals and first
// binade are evenly spaced up to 15 * u. One masked word thus yields four codes as floats with
// two packed conversions; the constant u (and the factor 4 of codes sitting two bits up in
// their byte) folds into the query or into the per-channel output scale.
#include "loopkv_internal.h"

#define LKV_GLOBAL __attribute__((address_space(1)))
#define LKV_CONST __attribute__((address_space(4)))

namespace loopkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

typedef float float2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef const LKV_GLOBAL uint8_t* gbytes;

template <class T>
__device__ __forceinline__ const LKV_GLOBAL T* gp(gbytes p) {
  return reinterpret_cast<const LKV_GLOBAL T*>(p);
}
// Generic -> global / constant address space (data the kernel only reads).
template <class T>
__device__ __forceinline__ const LKV_GLOBAL T* as_global(const T* p) {
  return (const LKV_GLOBAL T*)(p);
}
template <class T>
__device__ __forceinline__ const LKV_CONST T* as_const(const T* p) {
  return (const LKV_CONST T*)(p);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w & 0xFFFFu));
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(w >> 16));
}
// Bytes 0,1 (HI = false) or 2,3 (HI = true) of w as fp8 -> two floats.
template <bool HI>
__device__ __forceinline__ float2v cvt2(uint32_t w) {
  return __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Maximum over lanes 0..31 (the values of lanes 32..63 duplicate them), broadcast to all.
__device__ __forceinline__ float max32(float v) {
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                   0, __builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, false)));   // quad xor 1
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                   0, __builtin_bit_cast(int, v), 0x4E, 0xF, 0xF, false)));   // quad xor 2
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                   0, __builtin_bit_cast(int, v), 0x141, 0xF, 0xF, false)));  // half-row mirror
  v = fmaxf(v, __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
                   0, __builtin_bit_cast(int, v), 0x140, 0xF, 0xF, false)));  // row mirror
  const float a = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
  const float b = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
  return fmaxf(a, b);
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

template <int NVG, int NW>
struct Smem {
  alignas(16) float q[kHeadDim];
  alignas(16) float red[NW][16][36];    // per-wave key partials [channel block][token]
  alignas(16) float wbuf[NW][NVG][32];  // per-wave value weights [value group][token]
  int hot_list[NW][32];
  float gmax[2][NW];
  float fin_acc[NW][kHeadDim];
  float fin_M[NW], fin_L[NW], fin_C[NW][NVG];
  unsigned long long cnt_hot;
};

// Per-lane registers of one group, loaded one round ahead.
template <int BITS, int NVG>
struct GroupRegs {
  static constexpr int KCW = BITS == 4 ? 2 : 1;   // 16-byte loads of key code words
  static constexpr int KSW = BITS == 4 ? 2 : 4;   // 16-byte loads of key (s, z) words
  u32x4 kc[KCW];
  u32x4 ksz[KSW];
  u32x4 vc;
  uint32_t vsz[NVG];
};

struct RowCtx {
  gbytes pool;
  int64_t page_bytes;
  const LKV_CONST int32_t* pt_row;
  int64_t head_off;
  int64_t num_pages;
  uint32_t* err;
};

__device__ __forceinline__ gbytes page_block(const RowCtx& r, int logical_page) {
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
  gbytes blk0 = page_block(r, lp0);
  gbytes blk1 = P == kGroup ? blk0 : page_block(r, lp0 + 1);
  {  // key codes of KTOK tokens of channel block cb
    gbytes bb = t0 < P ? blk0 : blk1;
    const LKV_GLOBAL u32x4* p = gp<u32x4>(bb + lay.kc + 4 * (cb * P + t0 % P));
#pragma unroll
    for (int i = 0; i < GroupRegs<BITS, NVG>::KCW; ++i) g.kc[i] = p[i];
  }
  {  // key (s, z) of the lane's channels, stored with the group's first page
    const LKV_GLOBAL u32x4* p = gp<u32x4>(blk0 + lay.ksz + 4 * cb * KCH);
#pragma unroll
    for (int i = 0; i < GroupRegs<BITS, NVG>::KSW; ++i) g.ksz[i] = p[i];
  }
  {  // value codes / high plane: 16 channels x 4 tokens
    const int cbv = lane & 7, t4 = (lane >> 3) * 4;
    gbytes bb = t4 < P ? blk0 : blk1;
    g.vc = *gp<u32x4>(bb + lay.vc + 4 * (cbv * P + t4 % P));
  }
  {  // value (s, z) of token `lane` (lanes 0..31)
    const int t = lane & 31;
    gbytes bb = t < P ? blk0 : blk1;
    const LKV_GLOBAL uint32_t* p = gp<uint32_t>(bb + lay.vsz) + (t % P) * NVG;
#pragma unroll
    for (int i = 0; i < NVG; ++i) g.vsz[i] = p[i];
  }
}

// Softmax and value accumulation state of one wave.
template <int NVG>
struct WaveState {
  float M, Lsum, m_run;
  float Csum[NVG];
  float acc[16];                 // scaled units, channels 16*cbv + i
  uint32_t lo_word[4];           // low planes loaded last round
  float lo_wt[4];                // their weights (0: nothing loaded)
  unsigned long long hot;
};

struct RoundConst {
  float scale2, log2tau, u;
  bool gated;
  int w, lane, gs, ge;
  uint8_t* mask_row;
};

template <int BITS, int NVG, int P, int NW>
__device__ __forceinline__ void round_body(Smem<NVG, NW>& sm, WaveState<NVG>& st,
                                           const GroupRegs<BITS, NVG>& cur, GroupRegs<BITS, NVG>& nxt,
                                           const RowCtx& r, const Layout& lay, const RoundConst& k,
                                           const float (&qv)[32 / BITS], int rd) {
  constexpr int KCH = 32 / BITS;
  constexpr int NCB = kHeadDim / KCH;
  constexpr int KTOK = kGroup * NCB / 64;
  const int w = k.w, lane = k.lane;
  const int cb = lane % NCB, tq = lane / NCB;
  const int cbv = lane & 7, tq8 = lane >> 3;
  const int vg_lane = (cbv * 16) / (kHeadDim / NVG);
  const int grp = k.gs + rd * NW + w;
  const bool active = grp < k.ge;
  const int nxt_grp = grp + NW;
  if (nxt_grp < k.ge) load_group<BITS, NVG, P>(nxt, r, lay, nxt_grp, lane);

  // ---- scores of the group (key codes read first, section 3.3)
  float s2 = -INFINITY;
  if (active) {
    float qs[KCH], ke = 0.f, ko = 0.f;
    const uint32_t* kszw = reinterpret_cast<const uint32_t*>(cur.ksz);
#pragma unroll
    for (int i = 0; i < KCH; ++i) {
      const uint32_t sz = kszw[i];
      qs[i] = qv[i] * f16_lo(sz);
      if (BITS == 2 && (i & 1)) ko = fmaf(qv[i], f16_hi(sz), ko);
      else ke = fmaf(qv[i], f16_hi(sz), ke);
    }
    // qv carries 1/u (and 1/4 on odd INT2 channels): kappa = sum_c q_c * z_c
    const float kappa = (BITS == 2 ? fmaf(4.f, ko, ke) : ke) * k.u;
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
    // all 64 lanes: lane l sums half of the channel blocks of token l & 31
    const int t = lane & 31, half = lane >> 5;
    float raw = 0.f;
#pragma unroll
    for (int kk = 0; kk < NCB / 2; ++kk) raw += sm.red[w][half * (NCB / 2) + kk][t];
    raw += __shfl_xor(raw, 32);
    s2 = raw * k.scale2;
  }
  const float gmax_w = active ? max32(s2) : -INFINITY;
  if (lane == 0) sm.gmax[rd & 1][w] = gmax_w;
  __syncthreads();
  float mpre = st.m_run, mall = st.m_run;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const float x = sm.gmax[rd & 1][i];
    if (i <= w) mpre = fmaxf(mpre, x);
    mall = fmaxf(mall, x);
  }
  st.m_run = mall;
  if (!active) return;

  // ---- online softmax: rescale only when the wave's maximum grows
  if (gmax_w > st.M) {
    if (st.M != -INFINITY) {
      const float f = exp2f(st.M - gmax_w);
      st.Lsum *= f;
#pragma unroll
      for (int i = 0; i < NVG; ++i) st.Csum[i] *= f;
#pragma unroll
      for (int i = 0; i < 16; ++i) st.acc[i] *= f;
#pragma unroll
      for (int i = 0; i < 4; ++i) st.lo_wt[i] *= f;
    }
    st.M = gmax_w;
  }
  // ---- last round's low planes
  if (BITS == 4) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (st.lo_wt[kk] != 0.f) {
        float x[16];
        unpack16(st.lo_word[kk], x);
#pragma unroll
        for (int i = 0; i < 16; ++i) st.acc[i] = fmaf(st.lo_wt[kk], x[i], st.acc[i]);
      }
    }
  }

  // ---- per token (lanes 0..31): weight, hot/cold, value scale/zero folds
  bool hot = true;
  if (lane < kGroup) {
    const float p = exp2f(s2 - st.M);
    if (k.gated) hot = !((s2 - mpre) < k.log2tau);
    st.Lsum += p;
#pragma unroll
    for (int i = 0; i < NVG; ++i) {
      const uint32_t sz = cur.vsz[i];
      const float wv = p * f16_lo(sz);
      float cz = p * f16_hi(sz);
      if (k.gated && !hot) cz = fmaf(1.5f, wv, cz);
      st.Csum[i] += cz;
      sm.wbuf[w][i][lane] = wv;
    }
    if (k.mask_row) k.mask_row[(size_t)grp * kGroup + lane] = hot ? 1 : 0;
  }
  const uint32_t hotmask = (uint32_t)__ballot(lane < kGroup && hot);
  if (BITS == 4 && lane < kGroup && hot) sm.hot_list[w][__popc(hotmask & ((1u << lane) - 1u))] = lane;
  wave_lds_sync();

  // ---- issue the low-plane loads of the hot tokens (accumulated next round)
  if (BITS == 4) {
    const int nhot = __popc(hotmask);
    st.hot += nhot;
    const int lp0 = grp * (kGroup / P);
    gbytes blk0 = page_block(r, lp0);
    gbytes blk1 = P == kGroup ? blk0 : page_block(r, lp0 + 1);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int idx = 8 * kk + tq8;
      st.lo_wt[kk] = 0.f;
      if (8 * kk < nhot && idx < nhot) {
        const int t = sm.hot_list[w][idx];
        gbytes blk = t < P ? blk0 : blk1;
        st.lo_word[kk] = gp<uint32_t>(blk + lay.vlo)[(t % P) * (kHeadDim / 16) + cbv];
        st.lo_wt[kk] = 0.25f * sm.wbuf[w][vg_lane][t];
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
      for (int i = 0; i < 16; ++i) st.acc[i] = fmaf(wf[j], x[i], st.acc[i]);
    }
  }
  wave_lds_sync();
}

struct DecodeParams {
  Geom g;
  DecodeCall c;
};

template <int BITS, int NVG, int P, int NW>
__global__ __launch_bounds__(64 * NW) void decode_kernel(DecodeParams prm) {
  const Geom& g = prm.g;
  const DecodeCall& c = prm.c;
  constexpr int KCH = 32 / BITS;
  constexpr int NCB = kHeadDim / KCH;
  constexpr float VS = BITS == 4 ? 4.f : 1.f;   // true numerator = VS * acc + C
  static_assert(NW >= 2, "the final merge uses 128 threads");
  __shared__ Smem<NVG, NW> sm;
  const int split = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const LKV_CONST CellDesc* d = as_const(c.desc_dev);
  const int H = g.H;
  const float u = cvt2<false>(1u).x;            // value of fp8 byte 0x01
  const float inv_u = 1.0f / u;

  if (tid < kHeadDim) {
    const uint16_t qb = c.q[((size_t)b * H + h) * kHeadDim + tid];
    sm.q[tid] = __uint_as_float((uint32_t)qb << 16);
  }
  if (tid == 0) sm.cnt_hot = 0;

  // Row extent.
  const int64_t cap = min((int64_t)g.max_ctx, (int64_t)c.pt_stride * P);
  int len = as_const(c.seq_lens)[b];
  if (len < 0 || len > cap) {
    if (tid == 0 && split == 0 && h == 0) atomicOr(g.err, (uint32_t)kErrLength);
    len = 0;
  }
  int hist_groups = max(min(as_const((const int32_t*)d->src_qgroups)[b], len / kGroup), 0);
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
  r.pool = as_global((const uint8_t*)d->read_pool);
  r.page_bytes = d->read_page_bytes;
  r.pt_row = as_const(c.page_table) + (size_t)b * c.pt_stride;
  r.num_pages = g.num_pages;
  r.err = g.err;
  const Layout lay = head_layout(BITS, P, kHeadDim, NVG);
  r.head_off = (int64_t)h * lay.total;

  RoundConst k;
  k.gated = d->gated != 0;
  k.scale2 = c.sm_scale * kLog2e;
  k.log2tau = c.tau > 0.f ? log2f(c.tau) : -INFINITY;
  k.u = u;
  k.w = w;
  k.lane = lane;
  k.gs = gs;
  k.ge = ge;
  k.mask_row = c.mask ? c.mask + ((size_t)b * H + h) * c.mask_stride : nullptr;

  WaveState<NVG> st;
  st.M = -INFINITY;
  st.Lsum = 0.f;
  st.m_run = c.seed ? c.seed[(size_t)b * H + h] * kLog2e : -INFINITY;
  st.hot = 0;
#pragma unroll
  for (int i = 0; i < NVG; ++i) st.Csum[i] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) st.acc[i] = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) { st.lo_word[i] = 0u; st.lo_wt[i] = 0.f; }

  const int cb = lane % NCB;
  const int cbv = lane & 7, tq8 = lane >> 3;
  const int rounds = (ge - gs + NW - 1) / NW;
  GroupRegs<BITS, NVG> ra, rb;
  if (gs + w < ge) load_group<BITS, NVG, P>(ra, r, lay, gs + w, lane);
  __syncthreads();

  // The lane's query channels, scaled by 1/u (and by 1/4 for INT2 codes two bits up).
  float qv[KCH];
#pragma unroll
  for (int i = 0; i < KCH; ++i) {
    const float q = sm.q[cb * KCH + i];
    qv[i] = (BITS == 2 && (i & 1)) ? q * 0.25f * inv_u : q * inv_u;
  }

  for (int rd = 0; rd < rounds; rd += 2) {
    round_body<BITS, NVG, P, NW>(sm, st, ra, rb, r, lay, k, qv, rd);
    if (rd + 1 < rounds) round_body<BITS, NVG, P, NW>(sm, st, rb, ra, r, lay, k, qv, rd + 1);
  }
  // Low planes of the last round.
  if (BITS == 4) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (st.lo_wt[kk] != 0.f) {
        float x[16];
        unpack16(st.lo_word[kk], x);
#pragma unroll
        for (int i = 0; i < 16; ++i) st.acc[i] = fmaf(st.lo_wt[kk], x[i], st.acc[i]);
      }
    }
  }

  // Exact tail tokens (last split only), in chunks of 32, distributed over the waves.
  if (do_tail) {
    const LKV_GLOBAL uint16_t* tail_k = as_global((const uint16_t*)d->tail_k);
    const LKV_GLOBAL uint16_t* tail_v = as_global((const uint16_t*)d->tail_v);
    const int n_chunks = (n_tail + kGroup - 1) / kGroup;
    for (int ch = w; ch < n_chunks; ch += NW) {
      const int cbt = lane & 15, tqt = lane >> 4;   // keys: 8 channels x 8 tokens
      for (int j = 0; j < 8; ++j) {
        const int t = tqt * 8 + j;
        const int pos = tail_begin + ch * kGroup + t;
        float part = 0.f;
        if (ch * kGroup + t < n_tail) {
          const size_t row = ((size_t)b * g.tail + (pos % g.tail)) * H + h;
          const u32x4 kv = *reinterpret_cast<const LKV_GLOBAL u32x4*>(tail_k + row * kHeadDim + cbt * 8);
          const uint32_t kk4[4] = {kv.x, kv.y, kv.z, kv.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            part = fmaf(sm.q[cbt * 8 + 2 * i], bf16_lo(kk4[i]), part);
            part = fmaf(sm.q[cbt * 8 + 2 * i + 1], bf16_hi(kk4[i]), part);
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
        s2 = raw * k.scale2;
      }
      const float gm = wave_max(s2);
      const float Mn = fmaxf(st.M, gm);
      const float f = (st.M == -INFINITY) ? 0.f : exp2f(st.M - Mn);
      st.M = Mn;
      st.Lsum *= f;
#pragma unroll
      for (int i = 0; i < NVG; ++i) st.Csum[i] *= f;
#pragma unroll
      for (int i = 0; i < 16; ++i) st.acc[i] *= f;
      if (lane < kGroup) {
        const float p = (ch * kGroup + lane < n_tail) ? exp2f(s2 - st.M) : 0.f;
        st.Lsum += p;
        sm.wbuf[w][0][lane] = p * (u / VS);         // into scaled units (x u)
      }
      wave_lds_sync();
      for (int j = 0; j < 4; ++j) {
        const int t = tq8 * 4 + j;
        if (ch * kGroup + t >= n_tail) break;
        const int pos = tail_begin + ch * kGroup + t;
        const size_t row = ((size_t)b * g.tail + (pos % g.tail)) * H + h;
        const LKV_GLOBAL u32x4* vp = reinterpret_cast<const LKV_GLOBAL u32x4*>(tail_v + row * kHeadDim + cbv * 16);
        const u32x4 v0 = vp[0], v1 = vp[1];
        const uint32_t vv[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
        const float wt = sm.wbuf[w][0][t];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          // channel 2i is even (scale u), channel 2i+1 is odd (scale 4u)
          st.acc[2 * i] = fmaf(wt, bf16_lo(vv[i]), st.acc[2 * i]);
          st.acc[2 * i + 1] = fmaf(4.f * wt, bf16_hi(vv[i]), st.acc[2 * i + 1]);
        }
      }
      wave_lds_sync();
    }
  }

  // Merge the waves: sum lanes, then combine the NW softmax states.
  const float Lsum = wave_sum(lane < kGroup ? st.Lsum : 0.f);
  float Csum[NVG];
#pragma unroll
  for (int i = 0; i < NVG; ++i) Csum[i] = wave_sum(lane < kGroup ? st.Csum[i] : 0.f);
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v = st.acc[i];
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
    sm.fin_M[w] = st.M;
    sm.fin_L[w] = Lsum;
#pragma unroll
    for (int i = 0; i < NVG; ++i) sm.fin_C[w][i] = Csum[i];
    if (c.stats && BITS == 4) atomicAdd(&sm.cnt_hot, st.hot);
  }
  __syncthreads();
  if (tid < kHeadDim) {
    float Mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < NW; ++i) Mx = fmaxf(Mx, sm.fin_M[i]);
    float num = 0.f, den = 0.f;
    if (Mx != -INFINITY) {
      const int vg = tid / (kHeadDim / NVG);
#pragma unroll
      for (int i = 0; i < NW; ++i) {
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
    if (k.gated) {
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

// Waves per workgroup: 3 lets four workgroups of the register budget these kernels use
// (at most 168 VGPRs, three waves per SIMD) share a CU, so 4 (request, head) rows per CU run
// in one generation.
constexpr int kNW = 3;

template <int BITS, int P>
hipError_t launch_bp(const Geom& g, const DecodeCall& c, hipStream_t stream) {
  DecodeParams prm{g, c};
  const dim3 grid((unsigned)c.n_split, (unsigned)g.H, (unsigned)c.batch);
  switch (g.nvg) {
    case 1: decode_kernel<BITS, 1, P, kNW><<<grid, 64 * kNW, 0, stream>>>(prm); break;
    case 2: decode_kernel<BITS, 2, P, kNW><<<grid, 64 * kNW, 0, stream>>>(prm); break;
    case 4: decode_kernel<BITS, 4, P, kNW><<<grid, 64 * kNW, 0, stream>>>(prm); break;
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
