// Fused decode attention over one cell's quantized history and exact tail.
//
// "Loop-Aware KV Cache Compression for Serving Looped Transformers":
//  - one launch per cell reads history pages through the cell's descriptor, which names the
//    pool to read (its own, or the final loop's for a reusing cell), the stored bits, and
//    whether the low value plane is gated (section 3.4, "The unified kernel");
//  - for each page the key codes are read first, so every score of the page is known before
//    its values are touched; a token is cold when exp(s - m) < tau for a running maximum m
//    that starts at the seed, and a cold token reads only the high plane and decodes to the
//    middle of its bucket (section 3.3, "Read-time V precision");
//  - the per-channel key scale/zero fold into the query once per page, and the per-token value
//    scale/zero fold into the attention weight and a running sum (Appendix, "History reader");
//  - split partials merge by log-sum-exp, which gives the exact softmax; the workgroup that
//    finishes a row's last split does it, so every decode is one launch (section 3.4).
//
// Work mapping (CDNA4, wave64): one workgroup per (request, RB heads, split), NW waves per
// (request, head) row: RB = 4 rows (16 waves, one workgroup filling a CU) when the launch
// still gives every CU a workgroup, else RB = 1. In each round every wave takes two
// consecutive 32-token groups of its row, lanes 0..31 the first and lanes 32..63 the second.
// The group maxima are combined across the waves through LDS as a prefix maximum, so the
// hot/cold decisions are exactly those of streaming the split group by group.
// Each wave keeps its own online-softmax state; the waves merge at the end.
//
// Latency hiding: each part of a wave's next two groups (key codes and scales, value scales,
// value high plane or INT2 codes) is loaded right after this round's last use of the same
// registers, so it has about a round to arrive; page ids are read a round before the loads
// that use them; the low planes of a round's hot tokens are loaded in that round and added in
// the next, before that round's barrier, where a wave would otherwise wait for the others.
//
// Arithmetic:
//  - keys: the scores of a round's 64 tokens are four block-scaled fp8 MFMAs (16 tokens x 128
//    channels each, v_mfma_scale_f32_16x16x128_f8f6f4). Operand B is the key codes: a 4-bit
//    or 2-bit code in the low bits of an fp8 (E4M3) byte is exactly code * 2^-9 (E4M3's
//    subnormals and first binade are evenly spaced up to 15 * 2^-9), so masking the stored
//    words into bytes is the whole conversion. Operand A is q * s_K (the key scale folded
//    into the query, per group and channel) written as a 24-bit integer relative to the
//    largest magnitude of its 32-channel scale block, offset by 2^23 and split into six
//    base-16 digits (rows of fp8 integers 0..15), plus a constant row that removes the offset;
//    each row and block carries its power of two in the MFMA's E8M0 block scale. Every
//    product and block sum is exact, so the score keeps fp32 accuracy (22 bits of q * s_K per
//    block) and the hot/cold test sees fp32-accurate scores. The key zero point enters as the
//    accumulator's initial value (sum over channels of q * z_K).
//  - values (INT4 high plane, INT2 codes): two tokens' words are interleaved with one byte
//    permute so each 16-bit half holds one token's channels; a code moved to mantissa bits 4..9
//    and OR-ed with the exponent of 1.0 is the fp16 number 1 + c/64, 1 + c/16 or 1 + c/4, and one
//    v_dot2_f32_f16 accumulates both tokens' weighted codes in fp32. The constant offset
//    (the sum of the fp16 weights) is removed once at the end.
#include "loopkv_internal.h"

#define LKV_GLOBAL __attribute__((address_space(1)))
#define LKV_CONST __attribute__((address_space(4)))

namespace loopkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
// Value weights enter the dot2 path as fp16 numbers K * p * s (p <= 1 the softmax weight, s the
// token's fp16 value scale, K a per-wave power of two). K starts at 2^24, so every non-zero fp16
// scale (>= 2^-24) gives weights >= p, and drops whenever a scale would push K * s past 2^15:
// weights stay finite and normal for any fp16 scale. Exact tokens use fp32 weights with K at
// most 2^8, which keeps their sums finite for bf16 values below 2^118.
constexpr float kWInit = 16777216.f;     // 2^24
constexpr float kWMax = 32768.f;         // 2^15: largest K * s
constexpr float kWExact = 256.f;         // 2^8: largest K while exact tokens are added

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
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
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float dot2(half2v a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(a, __builtin_bit_cast(half2v, b), c, false);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// max(a, b) as one v_max_f32. The values here are scores or -inf, never NaN, so the NaN
// quieting that fmaxf adds to every operand is not needed.
__device__ __forceinline__ float dmax(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float dmax3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}
// Maximum within each 16-lane row, broadcast to the row.
__device__ __forceinline__ float row_max16(float v) {
  v = dmax(v, dpp_mov<0xB1>(v));    // quad xor 1
  v = dmax(v, dpp_mov<0x4E>(v));    // quad xor 2
  v = dmax(v, dpp_mov<0x141>(v));   // half-row mirror
  v = dmax(v, dpp_mov<0x140>(v));   // row mirror
  return v;
}
// Sum within each 16-lane row, broadcast to the row (the same value in every lane: each step
// adds the same two partial sums in either order).
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  return v;
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
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

// (x & m) | o in one VALU op. VOP3 takes no literal constant and at most one SGPR on gfx950,
// so the mask is held in a VGPR and the OR constant in an SGPR (Masks below).
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t m, uint32_t o) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(m), "s"(o));
  return r;
}
struct Masks {
  uint32_t one, m89, m67, m45;   // fp16 1.0 in both halves; code bits 8..9 / 6..7 / 4..5 of both
};

// Offset unit of value channel i (of 16) in dot2_pair: its code sits at mantissa bits 8..9,
// 6..7 or 4..5, so it enters as 1 + code * kF[i] with kF = 1/4, 1/16 or 1/64.
__device__ constexpr float kF[8] = {1.f / 64, 1.f / 16, 1.f / 64, 1.f / 16, 1.f / 4, 1.f / 64, 1.f / 16, 1.f / 4};

// acc[c] += w0 * code(t0, c) + w1 * code(t1, c) for the 16 channels of two tokens' 2-bit code
// words, in offset units: channel c's code enters as the fp16 number 1 + code * kF[c % 8]. Two
// shifts of the interleaved word bring all eight codes of a half into mantissa bits 4..9.
__device__ __forceinline__ void dot2_pair(uint32_t w0, uint32_t w1, half2v wp, const Masks& mk,
                                          float (&acc)[16]) {
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    // channels 8*half .. 8*half+7 of token t0 in bits 0..15, of token t1 in bits 16..31
    const uint32_t s = __builtin_amdgcn_perm(w1, w0, half ? 0x07060302u : 0x05040100u);
    const uint32_t l4 = s << 4, r6 = s >> 6;   // bits 0..3 -> 4..7; bits 10..15 -> 4..9
    float* a = acc + 8 * half;
    a[0] = dot2(wp, and_or(l4, mk.m45, mk.one), a[0]);
    a[1] = dot2(wp, and_or(l4, mk.m67, mk.one), a[1]);
    a[2] = dot2(wp, and_or(s, mk.m45, mk.one), a[2]);
    a[3] = dot2(wp, and_or(s, mk.m67, mk.one), a[3]);
    a[4] = dot2(wp, and_or(s, mk.m89, mk.one), a[4]);
    a[5] = dot2(wp, and_or(r6, mk.m45, mk.one), a[5]);
    a[6] = dot2(wp, and_or(r6, mk.m67, mk.one), a[6]);
    a[7] = dot2(wp, and_or(r6, mk.m89, mk.one), a[7]);
  }
}

template <int NVG, int NW>
struct Smem {
  alignas(16) float q[kHeadDim];
  // Score-MFMA operand A per wave: [group of the pair][32-channel block][row][32 channels].
  // Rows 0..5 (the pair's first group) and 8..13 (its second) hold the base-16 digits of
  // q * s_K, rows 6 and 14 the constant -1 of the digits' offset, the others stay zero.
  alignas(16) uint8_t akey[NW][2][4][16][32];
  // Per-wave value weights [round parity][wave][value group][token of pair] and hot tokens
  // (token of pair, page id); the low planes of a round are added in the next one, which reads
  // that round's copies.
  alignas(16) _Float16 wbuf[2][NW][NVG][64];
  float tail_w[NW][kGroup];               // exact-token weights of a chunk
  float sink_max[NW];                     // largest sink score each wave saw
  // Hot tokens of a round, compacted: address of the token's low-plane row, and its value
  // weights / 4 as fp16 (a low code is a quarter of a high-plane step), with a zero after the
  // last so that tokens are read in pairs.
  unsigned long long hot_addr[2][NW][64];
  alignas(4) _Float16 hot_w[2][NW][NVG][66];
  float gmax[2][NW][2];
  float fin_acc[NW][kHeadDim];
  float fin_M[NW], fin_L[NW], fin_C[NW][NVG];
  unsigned long long cnt_hot;
};

// Per-lane registers of one pair of groups. Each part is reloaded for the next round right
// after this round's last use of it, so one set of registers keeps a round of loads in flight.
template <int BITS, int NVG>
struct PairRegs {
  static constexpr int KCT = BITS == 4 ? 4 : 2;   // key-code words per lane and tile
  uint32_t kc[4][KCT];   // 32 channels of one token of each 16-token tile
  u32x4 ksz;             // (s, z) of the lane's four channels 4u..4u+3 in its group
  u32x4 vc[2];
  uint32_t vsz[NVG];
};

struct RowCtx {
  gbytes pool;                      // read pool, advanced to this head's block in page 0
  uint32_t page_bytes;
  uint32_t num_pages;
  const LKV_GLOBAL int32_t* pt_row;
  uint32_t* err;
};

// Page ids of one round's pair of groups: with PPG pages per 32-token group, entry j < 2*PPG is
// the page of group (first group of the pair + j / PPG), page j % PPG of it. Lane j % (2*PPG)
// loads entry j, a round before the pair's data; the ids are then read back wave-uniform.
template <int P>
__device__ __forceinline__ int load_pair_ids(const RowCtx& r, int g, int ge, int lane) {
  constexpr int PPG = kGroup / P;
  const int j = lane & (2 * PPG - 1);
  const int gg = min(g + j / PPG, ge - 1);   // never past the history
  return r.pt_row[gg * PPG + j % PPG];
}

// A page id outside the pool is reported (by one lane: the id is wave-uniform) and replaced
// by page 0.
__device__ __forceinline__ int checked_page_u(const RowCtx& r, int pid, int lane) {
  if ((uint32_t)pid >= r.num_pages) {
    if (lane == 0) atomicOr(r.err, (uint32_t)kErrPage);
    pid = 0;
  }
  return pid;
}
__device__ __forceinline__ gbytes page_at(const RowCtx& r, int pid) {
  // pid * page_bytes as one 32x32->64 multiply whose scalar operand is the page size; the
  // pool base (also scalar) is added separately, so it never has to live in vector registers.
  uint64_t off, carry;
  asm("v_mad_u64_u32 %0, %1, %2, %3, 0" : "=v"(off), "=s"(carry) : "v"(pid), "s"(r.page_bytes));
  (void)carry;
  return r.pool + off;
}

// Byte offsets of a lane's loads inside its head block (fixed for the kernel).
struct LaneOffs {
  uint32_t kc, ksz, vc, vsz;
};

template <int BITS, int NVG, int P>
__device__ __forceinline__ LaneOffs lane_offsets(const Layout& lay, int lane) {
  const int hl = lane & 31;
  const int cbv = hl & 7, tv = (hl >> 3) * 8;
  LaneOffs o;
  // key codes: token lane % 16 of a tile, channels 32 * (lane / 16) .. + 31 (token-major rows)
  o.kc = lay.kc + (lane & 15) * (kHeadDim * BITS / 8) + (lane >> 4) * (32 * BITS / 8);
  o.ksz = lay.ksz + 16 * hl;                     // key (s, z) of channels 4hl .. 4hl + 3
  o.vc = lay.vc + 4 * (cbv * P + tv % P);        // value codes / high plane: 16 ch x 8 tokens
  o.vsz = lay.vsz + 4 * (hl % P) * NVG;          // value (s, z) of token hl
  return o;
}

// Page addresses of one pair of groups: the page of each 16-token key tile and the page of the
// lane's group's key scales (wave-uniform within each half), and the page of the lane's token.
struct PairPages {
  gbytes kt[4];
  gbytes ksz;
  gbytes tok;
  int tok_pid;
};

template <int P>
__device__ __forceinline__ PairPages pair_pages(const RowCtx& r, int idv, int lane) {
  constexpr int PPG = kGroup / P;
  int pid[2 * PPG];
  gbytes pg[2 * PPG];
#pragma unroll
  for (int j = 0; j < 2 * PPG; ++j) {
    pid[j] = checked_page_u(r, __builtin_amdgcn_readlane(idv, j), lane);
    pg[j] = r.pool + (uint64_t)(uint32_t)pid[j] * r.page_bytes;
  }
  PairPages pp;
#pragma unroll
  for (int k = 0; k < 4; ++k) pp.kt[k] = pg[PPG == 1 ? k / 2 : k];
  const bool second = lane >= 32;
  pp.ksz = second ? pg[PPG] : pg[0];
  if (PPG == 1) {
    pp.tok_pid = second ? pid[1] : pid[0];
  } else {
    const bool hi16 = (lane & 16) != 0;
    pp.tok_pid = second ? (hi16 ? pid[3] : pid[2]) : (hi16 ? pid[1] : pid[0]);
  }
  pp.tok = page_at(r, pp.tok_pid);
  return pp;
}

template <int BITS, int P, int NVG>
__device__ __forceinline__ void load_kc(PairRegs<BITS, NVG>& g, const PairPages& pp, const LaneOffs& o) {
  constexpr int ROW = kHeadDim * BITS / 8;   // bytes of one token's key codes
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    // with 32-token pages the second tile of a group is 16 rows further in the same page
    const gbytes a = pp.kt[k] + o.kc + (P == kGroup && (k & 1) ? 16 * ROW : 0);
    if constexpr (BITS == 4) {
      const u32x4 v = *gp<u32x4>(a);
      g.kc[k][0] = v.x; g.kc[k][1] = v.y; g.kc[k][2] = v.z; g.kc[k][3] = v.w;
    } else {
      const uint64_t v = *gp<uint64_t>(a);
      g.kc[k][0] = (uint32_t)v; g.kc[k][1] = (uint32_t)(v >> 32);
    }
  }
}
template <int BITS, int NVG>
__device__ __forceinline__ void load_vsz(PairRegs<BITS, NVG>& g, const PairPages& pp, const LaneOffs& o) {
  const LKV_GLOBAL uint32_t* p = gp<uint32_t>(pp.tok + o.vsz);
#pragma unroll
  for (int i = 0; i < NVG; ++i) g.vsz[i] = p[i];
}
template <int BITS, int NVG>
__device__ __forceinline__ void load_vc(PairRegs<BITS, NVG>& g, const PairPages& pp, const LaneOffs& o) {
  const LKV_GLOBAL u32x4* p = gp<u32x4>(pp.tok + o.vc);
  g.vc[0] = p[0];
  g.vc[1] = p[1];
}

// Softmax and value accumulation state of one wave.
template <int NVG>
struct WaveState {
  float M, Lsum, m_run, W;       // W: sum of the fp16 value weights (offset of acc)
  float K;                       // value-weight multiplier (a power of two)
  float Csum[NVG];
  // Value accumulator of channels 16*cbv + i in offset units: the high plane / INT2 codes enter
  // through dot2 as w' * (1 + code * f_i) with w' = K * weight and f_i = kF[i % 8], and W
  // collects the w'; low planes and exact tail values are added without the offset. True
  // weighted sum of channel i = (acc[i] - W) / (f_i * K).
  float acc[16];
  uint32_t lo_word[8];           // low planes of last round's hot tokens, two per lane and pass
  int nlo;                       // last round's hot count
  unsigned long long hot;
};

// Multiplies the value state (accumulators and their offset) by r, a power of two: exact.
template <int NVG>
__device__ __forceinline__ void scale_values(WaveState<NVG>& st, float r) {
  st.W *= r;
#pragma unroll
  for (int i = 0; i < 16; ++i) st.acc[i] *= r;
}

struct RoundConst {
  float scale2, log2tau;
  bool gated;
  int w, lane, gs, ge;
  uint8_t* mask_row;
  Masks mk;
};

// Score-MFMA constants of a lane: scale offsets of A row lane % 16 in each group of the pair
// (-1: a zero row), and the byte addresses of lanes holding the exponent of block lane / 16 in
// the pair's first and second group. A row r: digit rows 0..5 / 8..13 scale by 2^(4m + E - 13)
// (E8M0 byte 4m + E + 114), offset rows 6 / 14 by 2^(E + 1).
struct KeyLaneConst {
  int sofs0, sofs1, eaddr0, eaddr1;
};
__device__ __forceinline__ KeyLaneConst key_lane_const(int lane) {
  KeyLaneConst c;
  const int ar = lane & 15;
  c.sofs0 = ar <= 5 ? 114 + 4 * ar : ar == 6 ? 128 : -1;
  c.sofs1 = ar >= 8 && ar <= 13 ? 114 + 4 * (ar - 8) : ar == 14 ? 128 : -1;
  const int q = lane >> 4;
  const int src = q == 0 ? 0 : q == 1 ? 16 : q == 2 ? 4 : 20;
  c.eaddr0 = 4 * src;          // a lane whose channels fall in block lane / 16, first group
  c.eaddr1 = 4 * (32 + src);   // and second group
  return c;
}

constexpr int kCodeScale = 127 + 9;   // E8M0 2^9: a code c in an fp8 byte is c * 2^-9

// Key codes of one 16-token tile (32 channels of one token per lane) as fp8 bytes: four
// consecutive channels per register (the stored field order makes the masks enough).
template <int BITS>
__device__ __forceinline__ v8i spread_codes(const uint32_t (&w)[BITS == 4 ? 4 : 2]) {
  v8i b;
  if constexpr (BITS == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      b[2 * j] = (int)(w[j] & 0x0F0F0F0Fu);
      b[2 * j + 1] = (int)((w[j] >> 4) & 0x0F0F0F0Fu);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int k = 0; k < 4; ++k) b[4 * j + k] = (int)((w[j] >> (2 * k)) & 0x03030303u);
  }
  return b;
}

__device__ __forceinline__ v4f mfma_keys(const v8i& a, const v8i& b, const v4f& c, int scale_a) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, scale_a, 0, kCodeScale);
}

// Sum of a float over lanes l and l ^ 16 (rows 0+1 and 2+3 of the wave).
__device__ __forceinline__ float add_swap16(float v) {
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

// Adds the low planes loaded in the previous round (parity pr), before this round changes the
// wave's maximum, so that round's weights still apply. Pass j covers hot tokens 16j .. 16j+15:
// lane (slot, cbv) holds channels 16*cbv.. of tokens 16j + 2*slot and 16j + 2*slot + 1, which
// enter like a high-plane token pair (offset units, weights / 4).
template <int NVG, int NW>
__device__ __forceinline__ void add_prev_lo(Smem<NVG, NW>& sm, WaveState<NVG>& st, int pr, int w,
                                            int lane, const Masks& mk) {
  const int slot = lane >> 3;
  const int vg_lane = ((lane & 7) * 16) / (kHeadDim / NVG);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    if (16 * j < st.nlo) {
      const int idx = 16 * j + 2 * slot;
      uint32_t wpair = *reinterpret_cast<const uint32_t*>(&sm.hot_w[pr][w][vg_lane][idx]);
      if (idx >= st.nlo) wpair = 0u;
      const half2v wp = __builtin_bit_cast(half2v, wpair);
      st.W = dot2(wp, mk.one, st.W);
      dot2_pair(st.lo_word[2 * j], st.lo_word[2 * j + 1], wp, mk, st.acc);
    }
  }
}

template <int BITS, int NVG, int P, int NW>
__device__ __forceinline__ void round_body(Smem<NVG, NW>& sm, WaveState<NVG>& st,
                                           PairRegs<BITS, NVG>& cur, int& pid_cur, int& nid,
                                           const RowCtx& r, const RoundConst& k, int rd) {
  const int w = k.w;
  // The lane index, opaque to the compiler: values derived from it are formed again in every
  // round instead of being kept live (in registers, or spilled) across the loop.
  int lane = k.lane;
  asm volatile("" : "+v"(lane));
  constexpr Layout lay_r = head_layout(BITS, P, kHeadDim, NVG);
  const LaneOffs lo = lane_offsets<BITS, NVG, P>(lay_r, lane);
  const int half = lane >> 5, hl = lane & 31;
  const int cbv = lane & 7;
  const int vg_lane = (cbv * 16) / (kHeadDim / NVG);
  const int gA = k.gs + rd * 2 * NW + 2 * w;
  const bool active = gA < k.ge;
  const bool validB = gA + 1 < k.ge;
  const bool my_valid = half ? validB : active;
  // The next pair's pages (ids read last round); the ids of the pair after it. All loads are
  // issued on every round, also when the wave has no next pair (then it re-reads the split's
  // last group, which is cached): with a fixed number of loads per round every wait leaves
  // the younger loads in flight.
  const PairPages np = pair_pages<P>(r, nid, lane);
  nid = load_pair_ids<P>(r, gA + 4 * NW, k.ge, lane);

  // ---- scores of both groups (key codes read first, section 3.3)
  // Every step below runs also on a wave without groups this round (its scores are -inf and
  // its weights 0): then every path through the round consumes the same loads.
  float s2;
  {
    // Operand A: lane (half, hl) holds channels 4hl .. 4hl+3 of group `half` of the pair;
    // q * s_K (the key scale folded into the query, Appendix "History reader") and q * z_K.
    const float4 qf = *reinterpret_cast<const float4*>(&sm.q[4 * hl]);
    const float qv[4] = {qf.x, qf.y, qf.z, qf.w};
    const uint32_t szw[4] = {cur.ksz.x, cur.ksz.y, cur.ksz.z, cur.ksz.w};
    float qs[4], ke = 0.f, am = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      qs[i] = fmaf(qv[i], f16_lo(szw[i]), 0.f);   // fp16 operand: one v_fma_mix_f32
      ke = fmaf(qv[i], f16_hi(szw[i]), ke);
      am = dmax(am, fabsf(qs[i]));
    }
    cur.ksz = *gp<u32x4>(np.ksz + lo.ksz);   // next round's key scales
    // kappa = sum over the group's 128 channels of q * z_K: the 32 lanes of the half
    ke = add_swap16(row_sum16(ke));
    // The MFMA scales A row r by one E8M0 value per 32 channels, from lane r + 16 * b of its
    // scale operand for block b: b = 0 takes channels 0..15 and 32..47, b = 1 64..79 and
    // 96..111, b = 2 16..31 and 48..63, b = 3 80..95 and 112..127 (bytes 0..15 or 16..31 of
    // the lanes holding channels 0..63 or 64..127). Here the largest |q * s_K| of the lane's
    // block (8 lanes: quads 0 and 2, or 1 and 3, of its 16-lane row): |q * s_K| < 2^E.
    am = dmax(am, dpp_mov<0xB1>(am));
    am = dmax(am, dpp_mov<0x4E>(am));
    am = dmax(am, dpp_mov<0x128>(am));
    const int E = __builtin_amdgcn_frexp_expf(am);
    const float sc = __builtin_ldexpf(1.f, 22 - E);
    // 2^23 + q * s_K * 2^(22 - E), rounded: 24 bits, six base-16 digits
    uint32_t X[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) X[i] = (uint32_t)fmaf(qs[i], sc, 8388608.5f);
    const uint32_t a01 = __builtin_amdgcn_perm(X[1], X[0], 0x05010400u);   // X0.b0 X1.b0 X0.b1 X1.b1
    const uint32_t a23 = __builtin_amdgcn_perm(X[3], X[2], 0x05010400u);
    const uint32_t l01 = a01 & 0x0F0F0F0Fu, h01 = (a01 >> 4) & 0x0F0F0F0Fu;
    const uint32_t l23 = a23 & 0x0F0F0F0Fu, h23 = (a23 >> 4) & 0x0F0F0F0Fu;
    const uint32_t c01 = __builtin_amdgcn_perm(X[1], X[0], 0x05010602u);   // X0.b2 X1.b2 ..
    const uint32_t c23 = __builtin_amdgcn_perm(X[3], X[2], 0x05010602u);
    const uint32_t cc = __builtin_amdgcn_perm(c23, c01, 0x05040100u);      // X0.b2 X1.b2 X2.b2 X3.b2
    // digit m of the four channels, one byte each, into row (8 * half + m) of the block's A
    uint8_t* arow = &sm.akey[w][half][hl >> 3][half * 8][4 * (hl & 7)];
    *reinterpret_cast<uint32_t*>(arow + 0 * 32) = __builtin_amdgcn_perm(l23, l01, 0x05040100u);
    *reinterpret_cast<uint32_t*>(arow + 1 * 32) = __builtin_amdgcn_perm(h23, h01, 0x05040100u);
    *reinterpret_cast<uint32_t*>(arow + 2 * 32) = __builtin_amdgcn_perm(l23, l01, 0x07060302u);
    *reinterpret_cast<uint32_t*>(arow + 3 * 32) = __builtin_amdgcn_perm(h23, h01, 0x07060302u);
    *reinterpret_cast<uint32_t*>(arow + 4 * 32) = cc & 0x0F0F0F0Fu;
    *reinterpret_cast<uint32_t*>(arow + 5 * 32) = (cc >> 4) & 0x0F0F0F0Fu;
    // scale of A row r = lane % 16, block lane / 16: digit m carries 2^(4m + E - 22), the
    // offset row -2^(E + 1), times the fp8 units 2^9 of a digit byte; E of that block comes
    // from a lane of the block in each half
    const KeyLaneConst kl = key_lane_const(lane);
    const int eA = __builtin_amdgcn_ds_bpermute(kl.eaddr0, E);
    const int eB = __builtin_amdgcn_ds_bpermute(kl.eaddr1, E);
    const int scA = kl.sofs0 < 0 ? 127 : min(max(eA + kl.sofs0, 0), 254);
    const int scB = kl.sofs1 < 0 ? 127 : min(max(eB + kl.sofs1, 0), 254);
    wave_lds_sync();
    // Operand B: the codes of tiles 0, 1 (first group) and 2, 3 (second group). D rows 0..7 take
    // the first group (lanes 0..31), rows 8..15 the second (lanes 32..63); both accumulators
    // start at kappa in row 0 / row 8. One A and one B operand are live at a time.
    const v4f c0 = {(lane & 16) ? 0.f : ke, 0.f, 0.f, 0.f};
    // tiles 0 and 2 (the first 16 tokens of each group), then tiles 1 and 3: one accumulator,
    // one A and one B operand live at a time; A is read again from LDS for the second pair
    float z[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      v4f d;
      {
        const v8i A0 = *reinterpret_cast<const v8i*>(&sm.akey[w][0][lane >> 4][lane & 15][0]);
        d = mfma_keys(A0, spread_codes<BITS>(cur.kc[t]), c0, scA);
      }
      __builtin_amdgcn_sched_barrier(0);
      {
        const v8i A1 = *reinterpret_cast<const v8i*>(&sm.akey[w][1][lane >> 4][lane & 15][0]);
        d = mfma_keys(A1, spread_codes<BITS>(cur.kc[2 + t]), d, scB);
      }
      __builtin_amdgcn_sched_barrier(0);
      // token t of a tile: rows in lanes t, t + 16 (first group) or t + 32, t + 48 (second)
      z[t] = add_swap16(d[0] + d[1] + d[2] + d[3]);
    }
    load_kc<BITS, P, NVG>(cur, np, lo);   // next round's key codes
    const float raw = (lane & 16) ? z[1] : z[0];   // lane = token of the pair, as below
    s2 = my_valid ? raw * k.scale2 : -INFINITY;
  }
  const float rm = row_max16(s2);
  const float gmA = dmax(lane_f(rm, 0), lane_f(rm, 16));
  const float gmB = dmax(lane_f(rm, 32), lane_f(rm, 48));
  // Running maximum before each of the wave's two groups (4-bit history only: 2-bit history
  // has no low plane to gate). The 2-bit waves still meet once per round: in lockstep the
  // workgroup's waves stream neighbouring head blocks of the same pages together, which
  // measured 1-2% faster than letting them drift apart.
  float mpreA = 0.f, mpreB = 0.f;
  if (BITS == 2) __syncthreads();
  if (BITS == 4) {
    if (lane == 0) {
      sm.gmax[rd & 1][w][0] = gmA;
      sm.gmax[rd & 1][w][1] = gmB;
    }
    // Last round's low planes, before this round can move the wave's maximum; done before the
    // barrier, while the other waves are still forming their scores.
    add_prev_lo<NVG, NW>(sm, st, (rd + 1) & 1, w, lane, k.mk);
    __syncthreads();
    // Group maxima of this round in stream order: wave i's groups are 2i and 2i+1.
    const float* gx = &sm.gmax[rd & 1][0][0];
    float mall = st.m_run;
#pragma unroll
    for (int j = 0; j < 2 * NW; j += 2) mall = dmax3(mall, gx[j], gx[j + 1]);
    mpreA = dmax(st.m_run, gx[0]);      // everything up to this wave's first group
#pragma unroll
    for (int i = 1; i < NW; ++i)
      if (i <= w) mpreA = dmax3(mpreA, gx[2 * i - 1], gx[2 * i]);
    mpreB = dmax(mpreA, gmB);
    st.m_run = mall;
  }

  // ---- online softmax: rescale only when the wave's maximum grows
  const float gm = dmax(gmA, gmB);
  if (gm > st.M) {
    if (st.M != -INFINITY) {
      const float f = fexp2(st.M - gm);
      st.Lsum *= f;
      st.W *= f;
#pragma unroll
      for (int i = 0; i < NVG; ++i) st.Csum[i] *= f;
#pragma unroll
      for (int i = 0; i < 16; ++i) st.acc[i] *= f;
    }
    st.M = gm;
  }
  const int pr = rd & 1;

  // ---- value-weight multiplier: K * s <= 2^15 for every value scale of this round's tokens
  {
    float smax = 0.f;
    if (my_valid) {
#pragma unroll
      for (int i = 0; i < NVG; ++i) smax = dmax(smax, f16_lo(cur.vsz[i]));
    }
    if (__ballot(smax * st.K > kWMax)) {   // rare: the first rounds, or a larger scale
      const int e = __builtin_amdgcn_frexp_expf(wave_max(smax));   // smax < 2^e
      const float kn = __builtin_ldexpf(1.f, 15 - e);
      scale_values(st, kn / st.K);
      st.K = kn;
    }
  }

  // ---- per token (every lane): weight, hot/cold, value scale/zero folds
  bool hot = false;
  _Float16 wv[NVG];   // the token's value weights (K * p * s, fp16)
  if (my_valid) {
    const float p = fexp2(s2 - st.M);
    hot = !(k.gated && (s2 - (half ? mpreB : mpreA)) < k.log2tau);
    st.Lsum += p;
    const float pw = p * st.K;
#pragma unroll
    for (int i = 0; i < NVG; ++i) {
      const uint32_t sz = cur.vsz[i];
      // Csum gathers p * z, plus p * 1.5 * s for a cold token (middle of its bucket)
      const float zc = (k.gated && !hot) ? fmaf(1.5f, f16_lo(sz), f16_hi(sz)) : f16_hi(sz);
      st.Csum[i] = fmaf(p, zc, st.Csum[i]);
      // K * weight, rounded to nearest fp16: the value codes and the offset W both use
      // this rounded weight, and its error is unbiased (a truncated weight would bias the code
      // sum, which the zero term largely cancels in the output)
      wv[i] = (_Float16)fmaf(pw, f16_lo(sz), 0.f);
      sm.wbuf[pr][w][i][lane] = wv[i];
    }
    if (k.mask_row) k.mask_row[(size_t)(gA + half) * kGroup + hl] = hot ? 1 : 0;
  } else {
#pragma unroll
    for (int i = 0; i < NVG; ++i) {
      wv[i] = (_Float16)0.f;
      sm.wbuf[pr][w][i][lane] = wv[i];
    }
  }
  load_vsz<BITS, NVG>(cur, np, lo);   // next round's value scales
  const unsigned long long hotmask = __ballot(hot);
  const int nhot = __popcll(hotmask);
  if (BITS == 4 && hot) {
    const int pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(hotmask >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)hotmask, 0u));
    constexpr Layout lay = head_layout(BITS, P, kHeadDim, NVG);
    sm.hot_addr[pr][w][pos] = (unsigned long long)(page_at(r, pid_cur) + lay.vlo + (hl % P) * (kHeadDim / 4));
#pragma unroll
    for (int i = 0; i < NVG; ++i) {
      sm.hot_w[pr][w][i][pos] = wv[i] * (_Float16)0.25f;
      if (pos == nhot - 1) sm.hot_w[pr][w][i][pos + 1] = (_Float16)0.f;
    }
  }
  wave_lds_sync();

  // ---- low-plane loads of the hot tokens, two per lane and pass, added next round
  if (BITS == 4) {
    st.hot += nhot;
    const int slot = lane >> 3;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (16 * j < nhot) {
        const int idx = 16 * j + 2 * slot;
#pragma unroll
        for (int e = 0; e < 2; ++e)
          if (idx + e < nhot)
            st.lo_word[2 * j + e] = gp<uint32_t>((gbytes)sm.hot_addr[pr][w][idx + e])[cbv];
      }
    }
    st.nlo = nhot;
  }

  // ---- high plane (INT4) or codes (INT2): 8 tokens of the lane's group, in 4 token pairs
  {
    const int tb = half * 32 + (hl >> 3) * 8;
    const uint4 wq = *reinterpret_cast<const uint4*>(&sm.wbuf[pr][w][vg_lane][tb]);
    const half2v p0 = __builtin_bit_cast(half2v, wq.x);   // tokens tb, tb + 1
    const half2v p1 = __builtin_bit_cast(half2v, wq.y);
    const half2v p2 = __builtin_bit_cast(half2v, wq.z);
    const half2v p3 = __builtin_bit_cast(half2v, wq.w);
    const uint32_t ones = k.mk.one;
    st.W = dot2(p0, ones, st.W);
    st.W = dot2(p1, ones, st.W);
    st.W = dot2(p2, ones, st.W);
    st.W = dot2(p3, ones, st.W);
    dot2_pair(cur.vc[0].x, cur.vc[0].y, p0, k.mk, st.acc);
    dot2_pair(cur.vc[0].z, cur.vc[0].w, p1, k.mk, st.acc);
    dot2_pair(cur.vc[1].x, cur.vc[1].y, p2, k.mk, st.acc);
    dot2_pair(cur.vc[1].z, cur.vc[1].w, p3, k.mk, st.acc);
  }
  load_vc<BITS, NVG>(cur, np, lo);   // next round's value codes
  pid_cur = np.tok_pid;
  wave_lds_sync();
}

// Device-scope coherent float store and load (relaxed atomics at agent scope): they bypass
// the non-coherent per-XCD L2, so another workgroup on any XCD sees the stored value.
__device__ __forceinline__ void store_device(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_device(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct DecodeParams {
  Geom g;
  DecodeCall c;
};

typedef const LKV_GLOBAL uint16_t* gu16;

// Exact (bf16) tokens of one row: the sink and the tail (the window and any tokens not yet
// quantized), read from the cell's own buffers. Rows of both are [request][slot][head][D].
struct ExactRow {
  gu16 sink_k, sink_v, ring_k, ring_v;
  size_t sink_row0, ring_row0;   // (request, slot 0, head) row index of each buffer
  int H, ring, sink_n, tail_begin, n_tail;
};

// 16 bytes (8 channels) of a bf16 row as floats.
__device__ __forceinline__ void bf16x8(const u32x4 w, float (&x)[8]) {
  x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x); x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
  x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z); x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
}

// Largest score (log2 units) over the sink tokens 8r + j, j = w, w + NW, ..., of one wave: lanes
// 16r .. 16r + 15 take token row r, eight channels each, and a row sum gives the score.
template <int NW>
__device__ __forceinline__ float sink_wave_max(const ExactRow& x, gu16 q, float scale2, int w,
                                               int lane) {
  const int cbt = lane & 15, tr = lane >> 4;
  float qf[8];
  bf16x8(*reinterpret_cast<const LKV_GLOBAL u32x4*>(q + cbt * 8), qf);
  float mx = -INFINITY;
  static_assert(8 % NW == 0, "the waves split the eight tokens of a token row evenly");
#pragma unroll
  for (int jj = 0; jj < 8 / NW; ++jj) {
    const int t = tr * 8 + w + jj * NW;
    const size_t row = x.sink_row0 + (size_t)min(t, x.sink_n - 1) * x.H;
    float kf[8];
    bf16x8(*reinterpret_cast<const LKV_GLOBAL u32x4*>(x.sink_k + row * kHeadDim + cbt * 8), kf);
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaf(qf[i], kf[i], a);
    a = row_sum16(a);
    if (t < x.sink_n) mx = dmax(mx, a * scale2);
  }
  return dmax(dmax(lane_f(mx, 0), lane_f(mx, 16)), dmax(lane_f(mx, 32), lane_f(mx, 48)));
}

// Softmax state update for one chunk of exact tokens: chunk ch of the row's exact list (chunk 0
// is the sink when there is one; the others are 32-token runs of the tail). Keys: lanes
// 16r .. 16r + 15 hold token row r (tokens 8r .. 8r + 7), eight channels each; values: lanes
// 8r' .. 8r' + 7 hold tokens 4r' .. 4r' + 3, sixteen channels each, which is the layout of acc.
// Both halves' loads are issued before the scores are formed.
template <int NVG, int NW>
__device__ __forceinline__ void exact_chunk(Smem<NVG, NW>& sm, WaveState<NVG>& st, const ExactRow& x,
                                            int ch, int has_sink, float scale2, float inv_vs,
                                            int w, int lane) {
  const bool is_sink = has_sink && ch == 0;
  const int cw = ch - has_sink;
  const int n_c = is_sink ? x.sink_n : min(kGroup, x.n_tail - cw * kGroup);
  const gu16 kb = is_sink ? x.sink_k : x.ring_k;
  const gu16 vb = is_sink ? x.sink_v : x.ring_v;
  const size_t row0 = is_sink ? x.sink_row0 : x.ring_row0;
  const int ring = is_sink ? (1 << 30) : x.ring;
  const int slot0 = is_sink ? 0 : (x.tail_begin + cw * kGroup) % x.ring;
  auto row_of = [&](int t) -> size_t {
    int slot = slot0 + min(t, n_c - 1);
    if (slot >= ring) slot -= ring;
    return row0 + (size_t)slot * x.H;
  };
  const int cbt = lane & 15, tr = lane >> 4;
  const int cbv = lane & 7, tq = lane >> 3;
  u32x4 kk[8], vv[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    kk[j] = *reinterpret_cast<const LKV_GLOBAL u32x4*>(kb + row_of(tr * 8 + j) * kHeadDim + cbt * 8);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const LKV_GLOBAL u32x4* vp =
        reinterpret_cast<const LKV_GLOBAL u32x4*>(vb + row_of(tq * 4 + j) * kHeadDim + cbv * 16);
    vv[2 * j] = vp[0];
    vv[2 * j + 1] = vp[1];
  }
  float qf[8];
  {
    const float4 a = *reinterpret_cast<const float4*>(&sm.q[cbt * 8]);
    const float4 b = *reinterpret_cast<const float4*>(&sm.q[cbt * 8 + 4]);
    qf[0] = a.x; qf[1] = a.y; qf[2] = a.z; qf[3] = a.w;
    qf[4] = b.x; qf[5] = b.y; qf[6] = b.z; qf[7] = b.w;
  }
  float s2[8];
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float kf[8];
    bf16x8(kk[j], kf);
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaf(qf[i], kf[i], a);
    a = row_sum16(a);
    s2[j] = tr * 8 + j < n_c ? a * scale2 : -INFINITY;
    mx = dmax(mx, s2[j]);
  }
  mx = dmax(dmax(lane_f(mx, 0), lane_f(mx, 16)), dmax(lane_f(mx, 32), lane_f(mx, 48)));
  if (mx > st.M) {
    if (st.M != -INFINITY) {
      const float f = fexp2(st.M - mx);
      st.Lsum *= f;
      st.W *= f;
#pragma unroll
      for (int i = 0; i < NVG; ++i) st.Csum[i] *= f;
#pragma unroll
      for (int i = 0; i < 16; ++i) st.acc[i] *= f;
    }
    st.M = mx;
  }
  float p[8], psum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    p[j] = fexp2(s2[j] - st.M);   // exp2(-inf) = 0 for tokens past the chunk
    psum += p[j];
  }
  if (st.K > kWExact) {
    scale_values(st, kWExact / st.K);
    st.K = kWExact;
  }
  const float vs_inv = st.K * inv_vs;
  if (cbt == 0) {
    st.Lsum += psum;
    // weight in offset units (before the channel's kF): p * K / VS
    float* tw = &sm.tail_w[w][tr * 8];
    *reinterpret_cast<float4*>(tw) = make_float4(p[0] * vs_inv, p[1] * vs_inv, p[2] * vs_inv, p[3] * vs_inv);
    *reinterpret_cast<float4*>(tw + 4) = make_float4(p[4] * vs_inv, p[5] * vs_inv, p[6] * vs_inv, p[7] * vs_inv);
  }
  wave_lds_sync();
  const float4 wq = *reinterpret_cast<const float4*>(&sm.tail_w[w][tq * 4]);
  const float wt[4] = {wq.x, wq.y, wq.z, wq.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t v8[8] = {vv[2 * j].x, vv[2 * j].y, vv[2 * j].z, vv[2 * j].w,
                            vv[2 * j + 1].x, vv[2 * j + 1].y, vv[2 * j + 1].z, vv[2 * j + 1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      // exact values, offset-free, in channel c's units (kF[c % 8])
      st.acc[2 * i] = fmaf(kF[(2 * i) % 8] * wt[j], bf16_lo(v8[i]), st.acc[2 * i]);
      st.acc[2 * i + 1] = fmaf(kF[(2 * i + 1) % 8] * wt[j], bf16_hi(v8[i]), st.acc[2 * i + 1]);
    }
  }
  wave_lds_sync();
}


constexpr int kMaxOrderBatch = 1024;   // larger batches keep the launch order

template <int BITS, int NVG, int P, int NW, int RB>
__global__ __launch_bounds__(64 * NW * RB) __attribute__((amdgpu_waves_per_eu(NW == 8 ? 2 : 4, NW == 8 ? 2 : 4)))
void decode_kernel(DecodeParams prm) {
  const Geom& g = prm.g;
  const DecodeCall& c = prm.c;
  constexpr float VS = BITS == 4 ? 4.f : 1.f;   // value units of acc: true = VS * code
  static_assert(NW >= 2, "the final merge uses 128 threads");
  // RB rows (heads of one request) per workgroup, NW waves each, one workgroup per CU: with
  // several workgroups per CU the SIMDs' oldest-first issue runs them one after another and
  // leaves the last alone on the CU. With 4-bit history the rows also share the round barrier
  // that the running maximum needs.
  __shared__ Smem<NVG, NW> sm_rows[RB];
  const int wave = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int rsub = wave / NW;
  Smem<NVG, NW>& sm = sm_rows[rsub];
  const int w = wave - rsub * NW;
  // The dispatcher deals workgroups to the XCDs round-robin by linear index, so with the split
  // as the fastest grid index an XCD would get the same split of every request (with ragged
  // lengths, all the empty or all the full ones). The split is rotated by the request's
  // position instead, so every XCD sees every split.
  const int split = (int)((blockIdx.x + blockIdx.z) % gridDim.x), h = blockIdx.y * RB + rsub;
  const int tid = (int)threadIdx.x - rsub * 64 * NW;   // thread index among the row's waves
  const int lane = tid & 63;
  const LKV_CONST CellDesc* d = as_const(c.desc_dev);
  const int H = g.H;
  const int64_t cap = min((int64_t)g.max_ctx, (int64_t)c.pt_stride * P);

  // When the launch takes more than one generation of workgroups: longest requests first.
  // Workgroup z takes the request of rank z by length (descending, ties by index), so the
  // dispatcher starts the longest rows first and the short ones fill the end of the launch.
  int b = blockIdx.z;
  if (c.order_by_len && c.batch > 1 && c.batch <= kMaxOrderBatch) {
    __shared__ int s_len[kMaxOrderBatch];
    __shared__ int s_b;
    for (int i = threadIdx.x; i < c.batch; i += blockDim.x)
      s_len[i] = (int)min(max((int64_t)as_const(c.seq_lens)[i], (int64_t)0), cap);
    __syncthreads();
    for (int i = threadIdx.x; i < c.batch; i += blockDim.x) {
      const int li = s_len[i];
      int rank = 0;
      for (int j = 0; j < c.batch; ++j) {
        const int lj = s_len[j];
        rank += (lj > li) | ((lj == li) & (j < i));
      }
      if (rank == (int)blockIdx.z) s_b = i;
    }
    __syncthreads();
    b = s_b;
  }
  if (tid < kHeadDim) {
    const uint16_t qb = c.q[((size_t)b * H + h) * kHeadDim + tid];
    sm.q[tid] = __uint_as_float((uint32_t)qb << 16);
  }
  if (tid == 0) sm.cnt_hot = 0;
  {
    // The wave's score-MFMA operand A: zero rows, and the constant -1 (fp8 0xB8) in the offset
    // rows 6 (first group of a pair) and 14 (second); the digit rows are rewritten every round.
    uint8_t* ak = &sm.akey[w][0][0][0][0];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int chunk = lane + 64 * i;                 // 16-byte chunk of the wave's 4 KB
      const int buf = chunk >> 7, row = (chunk >> 1) & 15;
      const uint32_t v = row == 6 + 8 * buf ? 0xB8B8B8B8u : 0u;
      *reinterpret_cast<uint4*>(ak + 16 * chunk) = make_uint4(v, v, v, v);
    }
  }

  // Row extent.
  int len = as_const(c.seq_lens)[b];
  if (len < 0 || len > cap) {
    if (tid == 0 && split == 0 && h == 0) atomicOr(g.err, (uint32_t)kErrLength);
    len = 0;
  }
  // Sink [0, sink_n), history groups [hs, he), tail [32 he, len): the history ends where the
  // source's quantized history ends, and never past this request's own window.
  const int hs = g.sink / kGroup;
  const int sink_n = min(len, g.sink);
  const int he = max(hs, (int)min((int64_t)as_const((const int32_t*)d->src_qgroups)[b],
                                  quantized_end(len, g.sink, g.window)));
  int tail_begin = he * kGroup;
  int n_tail = max(len - tail_begin, 0);
  if (n_tail > g.tail) {
    if (tid == 0 && split == 0 && h == 0) atomicOr(g.err, (uint32_t)kErrTail);
    tail_begin = len - g.tail;
    n_tail = g.tail;
  }
  // Splits are runs of split_tokens from token 0; each takes its groups of [hs, he).
  int gs = hs, ge = he;
  if (c.n_split > 1) {
    const int gps = c.split_tokens / kGroup;
    gs = min(max(split * gps, hs), he);
    ge = min(max((split + 1) * gps, hs), he);
  }
  const bool last_split = split == c.n_split - 1;
  const bool do_exact = last_split && (n_tail > 0 || sink_n > 0);

  constexpr Layout lay = head_layout(BITS, P, kHeadDim, NVG);
  RowCtx r;
  r.pool = as_global((const uint8_t*)d->read_pool) + (size_t)h * lay.total;
  r.page_bytes = (uint32_t)d->read_page_bytes;
  r.num_pages = (uint32_t)min(g.num_pages, (int64_t)INT32_MAX);
  r.pt_row = as_global(c.page_table) + (size_t)b * c.pt_stride;
  r.err = g.err;

  RoundConst k;
  k.gated = BITS == 4 && d->gated != 0;
  k.scale2 = c.sm_scale * kLog2e;
  k.log2tau = c.tau > 0.f ? log2f(c.tau) : -INFINITY;
  k.w = w;
  k.lane = lane;
  k.gs = gs;
  k.ge = ge;
  k.mask_row = c.mask ? c.mask + ((size_t)b * H + h) * c.mask_stride : nullptr;
  k.mk.one = 0x3C003C00u;
  k.mk.m89 = 0x03000300u;
  k.mk.m67 = 0x00C000C0u;
  k.mk.m45 = 0x00300030u;

  WaveState<NVG> st;
  st.M = -INFINITY;
  st.Lsum = 0.f;
  st.W = 0.f;
  st.K = kWInit;
  st.m_run = c.seed ? c.seed[(size_t)b * H + h] * kLog2e : -INFINITY;

  ExactRow ex;
  ex.sink_k = as_global((const uint16_t*)d->sink_k);
  ex.sink_v = as_global((const uint16_t*)d->sink_v);
  ex.ring_k = as_global((const uint16_t*)d->tail_k);
  ex.ring_v = as_global((const uint16_t*)d->tail_v);
  ex.sink_row0 = (size_t)b * g.sink * H + h;
  ex.ring_row0 = (size_t)b * g.tail * H + h;
  ex.H = H;
  ex.ring = g.tail;
  ex.sink_n = sink_n;
  ex.tail_begin = tail_begin;
  ex.n_tail = n_tail;
  // The sink's largest score seeds every split's running maximum (the history of a 2-bit
  // pool has no low plane to gate, so it needs no seed).
  const bool sink_seed = k.gated && c.sink_seed && sink_n > 0 && gs < ge;
  if (sink_seed) {
    const float mx = sink_wave_max<NW>(ex, as_global(c.q) + ((size_t)b * H + h) * kHeadDim,
                                       k.scale2, w, lane);
    if (lane == 0) sm.sink_max[w] = mx;
  }
  st.hot = 0;
#pragma unroll
  for (int i = 0; i < NVG; ++i) st.Csum[i] = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) st.acc[i] = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) st.lo_word[i] = 0u;
  st.nlo = 0;

  const int rounds = (ge - gs + 2 * NW - 1) / (2 * NW);
  const LaneOffs offs = lane_offsets<BITS, NVG, P>(lay, lane);
  PairRegs<BITS, NVG> regs;
  int nid = 0;         // page ids of the next round's pair
  int pid_cur = 0;     // page holding the lane's token this round
  if (rounds > 0) {
    // the next round's ids go out before this round's data, as inside the loop
    const int gA = gs + 2 * w;
    const int id0 = load_pair_ids<P>(r, gA, ge, lane);
    nid = load_pair_ids<P>(r, gA + 2 * NW, ge, lane);
    const PairPages pp = pair_pages<P>(r, id0, lane);
    load_kc<BITS, P, NVG>(regs, pp, offs);
    regs.ksz = *gp<u32x4>(pp.ksz + offs.ksz);
    load_vsz<BITS, NVG>(regs, pp, offs);
    load_vc<BITS, NVG>(regs, pp, offs);
    pid_cur = pp.tok_pid;
  }
  __syncthreads();
  if (sink_seed) {
#pragma unroll
    for (int i = 0; i < NW; ++i) st.m_run = dmax(st.m_run, sm.sink_max[i]);
  }

  for (int rd = 0; rd < rounds; ++rd) round_body<BITS, NVG, P, NW>(sm, st, regs, pid_cur, nid, r, k, rd);
  // Low planes of the last round.
  if (BITS == 4 && rounds > 0) add_prev_lo<NVG, NW>(sm, st, (rounds - 1) & 1, w, lane, k.mk);

  // Exact tokens (last split only): the sink, then the tail in chunks of 32, spread over the
  // row's waves.
  if (do_exact) {
    const int has_sink = sink_n > 0 ? 1 : 0;
    const int n_chunks = has_sink + (n_tail + kGroup - 1) / kGroup;
    for (int ch = w; ch < n_chunks; ch += NW)
      exact_chunk<NVG, NW>(sm, st, ex, ch, has_sink, k.scale2, 1.f / VS, w, lane);
  }

  // Merge the waves: sum lanes, then combine the NW softmax states.
  const float Lsum = wave_sum(st.Lsum);
  float Csum[NVG];
#pragma unroll
  for (int i = 0; i < NVG; ++i) Csum[i] = wave_sum(st.Csum[i]);
  float W = st.W;
  W += __shfl_xor(W, 8);
  W += __shfl_xor(W, 16);
  W += __shfl_xor(W, 32);
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    float v = st.acc[i];
    v += __shfl_xor(v, 8);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    // offset units: channel i carries code * kF[i % 8], weights x K
    acc[i] = (v - W) * (1.f / (kF[i % 8] * st.K));
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
      store_device(&part[2 + tid], num);
      if (tid == 0) { store_device(&part[0], Mx); store_device(&part[1], den); }
    }
  }
  // Split partials: the workgroup that finishes a row group's last split merges them
  // (section 3.4: the last block of a row merges the partial results by log-sum-exp), so a
  // split decode is one launch. The counter of the row group is back at zero afterwards.
  if (c.n_split > 1) {
    __shared__ int s_last;
    int* counter = c.counters + (size_t)b * H + (int)blockIdx.y * RB;
    // The partials went out as device-coherent stores; once they are complete (vmcnt 0) in
    // every thread of the workgroup, the count is raised. No agent-scope fence: on this chip
    // that writes back and invalidates the whole L2 of the XCD, in every wave.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0)
      s_last = __hip_atomic_fetch_add(counter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == c.n_split - 1;
    __syncthreads();
    if (s_last) {
      // device-coherent loads: the other workgroups' partials, never a stale cached copy
      if (tid < kHeadDim) {
        const size_t row = (size_t)b * H + h;
        const float* base = c.partials + row * g.max_splits * (kHeadDim + 2);
        float Mx = -INFINITY;
        for (int sp = 0; sp < c.n_split; ++sp) Mx = fmaxf(Mx, load_device(&base[sp * (kHeadDim + 2)]));
        float num = 0.f, den = 0.f;
        if (Mx != -INFINITY) {
          for (int sp = 0; sp < c.n_split; ++sp) {
            const float* pp = base + sp * (kHeadDim + 2);
            const float m = load_device(&pp[0]);
            const float fw = m == -INFINITY ? 0.f : exp2f(m - Mx);
            num = fmaf(fw, load_device(&pp[2 + tid]), num);
            den = fmaf(fw, load_device(&pp[1]), den);
          }
        }
        c.out[row * kHeadDim + tid] = den > 0.f ? num / den : 0.f;
      }
      if (threadIdx.x == 0) __hip_atomic_store(counter, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (tid == 0 && c.stats) {
    const unsigned long long nh = (unsigned long long)(ge - gs) * kGroup;
    atomicAdd(&c.stats[0], nh);
    if (k.gated) {
      atomicAdd(&c.stats[1], sm.cnt_hot);
      atomicAdd(&c.stats[2], nh);
    }
    if (do_exact) atomicAdd(&c.stats[3], (unsigned long long)(n_tail + sink_n));
  }
}

// Waves per (request, head) row. With four rows per workgroup, one workgroup fills a CU at
// four waves per SIMD (128 VGPRs). One-row workgroups take eight waves (two per SIMD, up to
// 256 VGPRs) when the launch is a single generation of workgroups with splits of at least 1024
// tokens: a small launch (few requests, so split rows) then runs half as many rounds per
// workgroup, which is its latency.
#ifndef LOOPKV_NW2
#define LOOPKV_NW2 4
#endif
#ifndef LOOPKV_NW4
#define LOOPKV_NW4 4
#endif

template <int BITS, int P, int RB, int NW>
hipError_t launch_bprw(const Geom& g, const DecodeCall& c, hipStream_t stream) {
  DecodeParams prm{g, c};
  const dim3 grid((unsigned)c.n_split, (unsigned)(g.H / RB), (unsigned)c.batch);
  // one workgroup fills a CU
  prm.c.order_by_len = (int64_t)grid.x * grid.y * grid.z > (int64_t)g.cus;
  const unsigned threads = 64 * NW * RB;
  switch (g.nvg) {
    case 1: decode_kernel<BITS, 1, P, NW, RB><<<grid, threads, 0, stream>>>(prm); break;
    case 2: decode_kernel<BITS, 2, P, NW, RB><<<grid, threads, 0, stream>>>(prm); break;
    case 4: decode_kernel<BITS, 4, P, NW, RB><<<grid, threads, 0, stream>>>(prm); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Four heads per workgroup (one workgroup per CU) when the head count allows and that still
// gives every CU a workgroup; otherwise one head per workgroup, so a small launch (few requests,
// short rows) spreads over four times as many CUs.
template <int BITS, int P>
hipError_t launch_bp(const Geom& g, const DecodeCall& c, hipStream_t stream) {
  const int64_t wg4 = (int64_t)c.n_split * (g.H / 4) * c.batch;
  if (g.H % 4 == 0 && wg4 >= g.cus)
    return launch_bprw<BITS, P, 4, BITS == 2 ? LOOPKV_NW2 : LOOPKV_NW4>(g, c, stream);
  const int64_t wg1 = (int64_t)c.n_split * g.H * c.batch;
  const int64_t span = c.n_split > 1 ? (int64_t)c.split_tokens
                                     : std::min<int64_t>(g.max_ctx, (int64_t)c.pt_stride * P);
  if (wg1 <= g.cus && span >= 32 * kGroup) return launch_bprw<BITS, P, 1, 8>(g, c, stream);
  return launch_bprw<BITS, P, 1, 4>(g, c, stream);
}

}  // namespace

hipError_t launch_decode(const Geom& g, const CellDesc& dh, const DecodeCall& c, hipStream_t stream) {
  if (dh.read_bits == 4)
    return g.P == 32 ? launch_bp<4, 32>(g, c, stream) : launch_bp<4, 16>(g, c, stream);
  return g.P == 32 ? launch_bp<2, 32>(g, c, stream) : launch_bp<2, 16>(g, c, stream);
}

}  // namespace loopkv
