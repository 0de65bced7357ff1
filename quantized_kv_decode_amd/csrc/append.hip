// Quantize-append: the companion step that moves new tokens into a cell's storage.
//
// "Loop-Aware KV Cache Compression for Serving Looped Transformers": the sink stays exact,
// and a 32-token page is quantized into its cell's pool when it leaves the exact window
// (section 2.3, "Measuring KV damage"; section 4); KIVI-style asymmetric quantization, keys
// per channel over the page, values per token over channel groups (section 5.1); an INT4 cell
// stores its value codes as a high and a low 2-bit plane (section 3.3, "Bit-plane V layout").
// Here a group is quantized by the append that moves it out of the window (with no window:
// the append that completes it); until then its tokens stay exact in a per-(cell, request)
// bf16 ring, and the sink's tokens are also kept in a bf16 sink of their own.
//
// Rounding (bit-exact by construction): scale = fp16_rne((max - min) / (2^b - 1)) and
// zero = fp16_rne(min), each rounded once from a double; code = clamp(floor((x - zero) /
// scale + 1/2), 0, 2^b - 1) in double precision; a zero scale gives code 0.
#include "loopkv_internal.h"

namespace loopkv {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Round a double to the nearest fp16 (ties to even) and return its bits. One rounding,
// straight from the double's significand.
__device__ uint16_t f64_to_f16_bits(double x) {
  const uint64_t bits = (uint64_t)__double_as_longlong(x);
  const uint32_t sign = (uint32_t)(bits >> 48) & 0x8000u;
  const int exp = (int)((bits >> 52) & 0x7FF);
  const uint64_t mant = bits & ((1ull << 52) - 1);
  if (exp == 0x7FF) return (uint16_t)(sign | 0x7C00u | (mant ? 0x200u : 0u));
  if (exp == 0) return (uint16_t)sign;  // double subnormals are far below fp16's range
  const uint64_t sig = (1ull << 52) | mant;  // value = sig * 2^(exp - 1075)
  int e = exp - 1023 + 15;                   // biased fp16 exponent if normal
  int shift = e >= 1 ? 42 : 42 + (1 - e);    // bits dropped from sig
  if (shift > 53) return (uint16_t)sign;     // below half the smallest subnormal
  uint64_t m = sig >> shift;
  const uint64_t rem = sig & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (m & 1))) ++m;
  if (e >= 1) {
    if (m == (1ull << 11)) { m >>= 1; ++e; }
    if (e >= 31) return (uint16_t)(sign | 0x7C00u);
    return (uint16_t)(sign | ((uint32_t)e << 10) | (uint32_t)(m & 0x3FF));
  }
  return (uint16_t)(sign | (uint32_t)m);  // subnormal; m == 0x400 is the smallest normal
}

__device__ double f16_bits_to_f64(uint16_t h) {
  const int e = (h >> 10) & 0x1F;
  const int m = h & 0x3FF;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? __longlong_as_double(0x7FF8000000000000ll) : __longlong_as_double(0x7FF0000000000000ll);
  else v = ldexp((double)(1024 + m), e - 25);
  return (h & 0x8000) ? -v : v;
}

__device__ __forceinline__ int quant_code(double x, double s, double z, int levels) {
  if (s == 0.0) return 0;
  double c = floor((x - z) / s + 0.5);
  c = c < 0.0 ? 0.0 : (c > (double)levels ? (double)levels : c);
  return (int)c;
}

// The same code from an fp32 estimate. With x exact (bf16), s and z exact (fp16) and
// u = (x - z) * rcp(s) + 1/2 formed in fp32, |u - ((x - z) / s + 1/2)| < 6e-6 whenever the
// result can land inside [0, levels] (a relative error below 2^-22 on values up to 17). So
// when u is at least kBand = 1e-5 away from an integer, floor(u) is the floor of the exact
// value, which the fp64 rule also reaches (its own error is ~1e-15); nearer a boundary, or for
// values that are not finite, the fp64 rule decides. The estimate saves the fp64 division.
__device__ __forceinline__ int quant_code_fast(float x, float s32, float z32, double s, double z,
                                               int levels) {
  constexpr float kBand = 1e-5f;
  if (s32 == 0.f) return 0;
  const float u = fmaf(x - z32, __builtin_amdgcn_rcpf(s32), 0.5f);
  const float f = floorf(u);
  const float d = fminf(u - f, f + 1.f - u);   // distance to the nearest integer
  if (!(d >= kBand) || !(u < 4096.f)) return quant_code((double)x, s, z, levels);
  return (int)fminf(fmaxf(f, 0.f), (float)levels);
}

__device__ __forceinline__ void raise_error(uint32_t* err, uint32_t flag) { atomicOr(err, flag); }

// One workgroup of 128 threads quantizes one 32-token key group that leaves the window, of one
// (request, head), into the cell's pool. blockIdx = (group index within this call, head,
// request). With FUSED (calls of at most 32 tokens) the workgroup of group index 0 also copies
// the call's tokens of its head into the ring (and the sink) and sets the request's counter,
// which saves the separate ring launch on a decode step: the ring slots it writes (positions
// old .. old+31) never alias the slots the group reads (positions between old-window-31 and
// old-window+31) in a ring of at least window + 64 tokens.
// Tokens request b appends in this call: n_new_dev[b] if given (clamped to [0, n_new]).
__device__ __forceinline__ int appended(const int32_t* n_new_dev, int n_new, int b) {
  if (!n_new_dev) return n_new;
  const int m = n_new_dev[b];
  return m < 0 ? 0 : (m > n_new ? n_new : m);
}

template <int BITS, bool FUSED>
__global__ __launch_bounds__(128) void quantize_group_kernel(
    Geom g, const CellDesc* __restrict__ descp, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, int n_new, const int32_t* __restrict__ n_new_dev,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ page_table, int pt_stride) {
  constexpr int L = (1 << BITS) - 1;
  const int h = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const CellDesc d = *descp;   // a copy: the stores below cannot alias it
  const int old = seq_lens[b];
  const int64_t nw = (int64_t)old + appended(n_new_dev, n_new, b);
  const int64_t cap = min((int64_t)g.max_ctx, (int64_t)pt_stride * g.P);
  if (old < 0 || nw > cap) {
    if (blockIdx.x == 0 && h == 0 && tid == 0) raise_error(g.err, kErrLength);
    return;
  }
  if (n_new_dev && (n_new_dev[b] < 0 || n_new_dev[b] > n_new) && blockIdx.x == 0 && h == 0 && tid == 0)
    raise_error(g.err, kErrLength);
  const int64_t q0 = quantized_end(old, g.sink, g.window);   // history end before the call
  const int64_t q1 = quantized_end(nw, g.sink, g.window);    // and after it
  const int grp = (int)q0 + (int)blockIdx.x;
  const bool has_group = grp < q1;

  // The group's keys as their bf16 bits (rows 16-byte aligned): half the LDS of an fp32 tile, so
  // that more of a decode step's workgroups are resident at once.
  __shared__ __attribute__((aligned(16))) uint16_t ks[kGroup][kHeadDim + 8];
  __shared__ __attribute__((aligned(16))) uint32_t kszs[kHeadDim];   // per channel: fp16 s | z << 16
  __shared__ int64_t page_base[kGroup / 16];

  const int H = g.H, D = g.D;   // D == kHeadDim (checked on the host)
  // Staging: thread (t, part) takes channels 32 part .. 32 part + 31 of the group's token t,
  // four 16-byte loads each of K and V, all requested before anything waits on them (with the
  // group's page ids). Tokens before `old` come from the ring, later ones from this call's input.
  const int t = tid >> 2, part = tid & 3, c0 = part * 32;
  u32x4 kw[4], vw[4];
  int pid = 0;
  if (has_group) {
    if (tid < kGroup / g.P) pid = page_table[(size_t)b * pt_stride + grp * kGroup / g.P + tid];
    const int pos = grp * kGroup + t;
    const bool fresh = pos >= old;
    int slot = (grp * kGroup) % g.tail + t;   // ring slot of the token
    if (slot >= g.tail) slot -= g.tail;
    const size_t row = fresh ? ((size_t)b * n_new + (pos - old)) * H + h
                             : ((size_t)b * g.tail + slot) * H + h;
    const u32x4* kp = reinterpret_cast<const u32x4*>((fresh ? k_new : d.tail_k) + row * D + c0);
    const u32x4* vp = reinterpret_cast<const u32x4*>((fresh ? v_new : d.tail_v) + row * D + c0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kw[i] = kp[i];
      vw[i] = vp[i];
    }
  }
  if (FUSED && blockIdx.x == 0) {
    // The call's tokens of this head into the ring (and the sink): 16 bytes per thread.
    const int m = (int)(nw - old);
    for (int e = tid; e < m * (kHeadDim / 8); e += 128) {
      const int i = e / (kHeadDim / 8), ch = (e % (kHeadDim / 8)) * 8;
      const size_t src = (((size_t)b * n_new + i) * g.H + h) * g.D + ch;
      const size_t dst = (((size_t)b * g.tail + (old + i) % g.tail) * g.H + h) * g.D + ch;
      const u32x4 kx = *reinterpret_cast<const u32x4*>(k_new + src);
      const u32x4 vx = *reinterpret_cast<const u32x4*>(v_new + src);
      *reinterpret_cast<u32x4*>(d.tail_k + dst) = kx;
      *reinterpret_cast<u32x4*>(d.tail_v + dst) = vx;
      if (old + i < g.sink) {
        const size_t sd = (((size_t)b * g.sink + old + i) * g.H + h) * g.D + ch;
        *reinterpret_cast<u32x4*>(d.sink_k + sd) = kx;
        *reinterpret_cast<u32x4*>(d.sink_v + sd) = vx;
      }
    }
    if (h == 0 && tid == 0) d.own_qgroups[b] = (int)q1;
  }
  if (!has_group) return;

  float vv[32];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t vx[4] = {vw[i].x, vw[i].y, vw[i].z, vw[i].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      vv[8 * i + 2 * j] = __uint_as_float(vx[j] << 16);
      vv[8 * i + 2 * j + 1] = __uint_as_float(vx[j] & 0xFFFF0000u);
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) *reinterpret_cast<u32x4*>(&ks[t][c0 + 8 * i]) = kw[i];
  // Physical pages holding the group (one for 32-token pages, two for 16-token pages).
  if (tid < kGroup / g.P) {
    if (pid < 0 || pid >= g.num_pages) {
      raise_error(g.err, kErrPage);
      page_base[tid] = -1;
    } else {
      page_base[tid] = (int64_t)pid * d.own_page_bytes;
    }
  }
  __syncthreads();
  for (int i = 0; i < kGroup / g.P; ++i)
    if (page_base[i] < 0) return;

  const Layout lay = head_layout(BITS, g.P, D, g.nvg);
  const int64_t hoff = (int64_t)h * lay.total;
  // The head block of the page holding token tt of the group, and tt's row in that page.
  auto tok_block = [&](int tt, int* tl) -> uint8_t* {
    *tl = tt % g.P;
    return d.own_pool + page_base[tt / g.P] + hoff;
  };

  // Values: the thread's 32 channels of token t; a group wider than 32 channels combines its
  // min/max across the neighbouring lanes that hold its other channels.
  {
    float mnf = vv[0], mxf = vv[0];
#pragma unroll
    for (int c = 1; c < 32; ++c) {
      mnf = vv[c] < mnf ? vv[c] : mnf;
      mxf = vv[c] > mxf ? vv[c] : mxf;
    }
    for (int w = 1; w < g.v_group / 32; w <<= 1) {
      const float omn = __shfl_xor(mnf, w), omx = __shfl_xor(mxf, w);
      mnf = omn < mnf ? omn : mnf;
      mxf = omx > mxf ? omx : mxf;
    }
    const double mn = mnf, mx = mxf;
    const uint16_t sb = f64_to_f16_bits((mx - mn) / (double)L);
    const uint16_t zb = f64_to_f16_bits(mn);
    const double s = f16_bits_to_f64(sb), z = f16_bits_to_f64(zb);
    const float s32 = (float)s, z32 = (float)z;   // exact: fp16 values
    int tl;
    uint8_t* blk = tok_block(t, &tl);
    // two 16-channel words (channel 16 cb + i at bits 2i): the high plane / INT2 codes, and for
    // INT4 the low plane
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      uint32_t hiw = 0, low = 0;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const uint32_t c = (uint32_t)quant_code_fast(vv[16 * half + i], s32, z32, s, z, L);
        if (BITS == 4) {
          hiw |= (c >> 2) << (2 * i);
          low |= (c & 3u) << (2 * i);
        } else {
          hiw |= c << (2 * i);
        }
      }
      const int cb = 2 * part + half;
      reinterpret_cast<uint32_t*>(blk + lay.vc)[cb * g.P + tl] = hiw;
      if (BITS == 4) reinterpret_cast<uint32_t*>(blk + lay.vlo)[tl * (kHeadDim / 16) + cb] = low;
    }
    if (c0 % g.v_group == 0)
      reinterpret_cast<uint32_t*>(blk + lay.vsz)[tl * g.nvg + c0 / g.v_group] =
          (uint32_t)sb | ((uint32_t)zb << 16);
  }

  // Keys: thread = channel; min/max over the group's tokens (all 32 staged values read first).
  {
    const int c = tid;
    float x[kGroup];
#pragma unroll
    for (int tt = 0; tt < kGroup; ++tt) x[tt] = __uint_as_float((uint32_t)ks[tt][c] << 16);
    float mnf = x[0], mxf = x[0];
#pragma unroll
    for (int tt = 1; tt < kGroup; ++tt) {
      mnf = x[tt] < mnf ? x[tt] : mnf;
      mxf = x[tt] > mxf ? x[tt] : mxf;
    }
    const double mn = mnf, mx = mxf;
    const uint16_t sb = f64_to_f16_bits((mx - mn) / (double)L);
    const uint16_t zb = f64_to_f16_bits(mn);
    const uint32_t szw = (uint32_t)sb | ((uint32_t)zb << 16);
    kszs[c] = szw;
    uint8_t* blk = d.own_pool + page_base[0] + hoff;
    reinterpret_cast<uint32_t*>(blk + lay.ksz)[c] = szw;
  }
  __syncthreads();

  // Key codes of the thread's own token t, channels c0 .. c0 + 31 (still in registers from the
  // staging loads), packed straight into its token-major words: KPW channels per word, in the
  // field order that masking a word into bytes turns into four consecutive channels per 32-bit
  // register (INT4: channel 8w + i in bits 8i..8i+3, 8w + 4 + i in bits 8i+4..8i+7; INT2:
  // channel 16w + 4k + i in bits 8i+2k..8i+2k+1).
  {
    uint32_t szv[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(&kszs[c0 + 4 * i]);
      szv[4 * i] = v.x; szv[4 * i + 1] = v.y; szv[4 * i + 2] = v.z; szv[4 * i + 3] = v.w;
    }
    uint32_t code[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const uint32_t w2 = kw[i / 8][(i % 8) / 2];
      const float xv = __uint_as_float((i & 1) ? (w2 & 0xFFFF0000u) : (w2 << 16));
      const float s32 = (float)__builtin_bit_cast(_Float16, (uint16_t)(szv[i] & 0xFFFFu));
      const float z32 = (float)__builtin_bit_cast(_Float16, (uint16_t)(szv[i] >> 16));
      code[i] = (uint32_t)quant_code_fast(xv, s32, z32, (double)s32, (double)z32, L);
    }
    constexpr int KPW = 32 / BITS;
    constexpr int NKW = kHeadDim / KPW;   // words per token
    constexpr int TW = 32 / KPW;          // words of the thread's 32 channels
    uint32_t word[TW];
#pragma unroll
    for (int w = 0; w < TW; ++w) {
      word[w] = 0;
#pragma unroll
      for (int f = 0; f < KPW; ++f) {
        const int ch = BITS == 4 ? (f % 2) * 4 + f / 2 : 4 * (f % 4) + f / 4;
        word[w] |= code[w * KPW + ch] << (BITS * f);
      }
    }
    int tl;
    uint8_t* blk = tok_block(t, &tl);
    uint32_t* dst = reinterpret_cast<uint32_t*>(blk + lay.kc) + tl * NKW + part * TW;
    if constexpr (TW == 4) {
      u32x4 o;
      o.x = word[0]; o.y = word[1]; o.z = word[2]; o.w = word[3];
      *reinterpret_cast<u32x4*>(dst) = o;
    } else {
      *reinterpret_cast<uint2*>(dst) = make_uint2(word[0], word[1]);
    }
  }
}

// Copies the last min(n_new, tail) new tokens of each request into the cell's ring and, for
// an own-storage cell, sets its quantized-group counter. blockIdx = (chunk, request).
__global__ __launch_bounds__(256) void tail_write_kernel(
    Geom g, const CellDesc* __restrict__ descp, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, int n_new, const int32_t* __restrict__ n_new_dev,
    const int32_t* __restrict__ seq_lens, int pt_stride) {
  const CellDesc& d = *descp;
  const int b = blockIdx.y;
  const int old = seq_lens[b];
  const int m = appended(n_new_dev, n_new, b);
  const int64_t nw = (int64_t)old + m;
  const int64_t cap = min((int64_t)g.max_ctx, (int64_t)pt_stride * g.P);
  if (old < 0 || nw > cap) return;  // flagged by the quantize kernel
  const int first = m > g.tail ? m - g.tail : 0;
  const int chunks_per_tok = g.H * g.D / 8;  // 16-byte chunks per token
  // Tokens at positions below the sink length also enter the sink.
  const int n_sink_new = old < g.sink ? min(m, g.sink - old) : 0;
  if (blockIdx.x == 0) {
    for (int e = threadIdx.x; e < n_sink_new * chunks_per_tok; e += blockDim.x) {
      const int i = e / chunks_per_tok, r = e % chunks_per_tok;
      const size_t src = ((size_t)b * n_new + i) * (size_t)(g.H * g.D) + (size_t)r * 8;
      const size_t dst = ((size_t)b * g.sink + old + i) * (size_t)(g.H * g.D) + (size_t)r * 8;
      *reinterpret_cast<uint4*>(d.sink_k + dst) = *reinterpret_cast<const uint4*>(k_new + src);
      *reinterpret_cast<uint4*>(d.sink_v + dst) = *reinterpret_cast<const uint4*>(v_new + src);
    }
  }
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t total = (int64_t)(m - first) * chunks_per_tok;
  if (e < total) {
    const int i = first + (int)(e / chunks_per_tok);
    const int r = (int)(e % chunks_per_tok);
    const size_t src = ((size_t)b * n_new + i) * (size_t)(g.H * g.D) + (size_t)r * 8;
    const int slot = (int)((old + i) % g.tail);
    const size_t dst = ((size_t)b * g.tail + slot) * (size_t)(g.H * g.D) + (size_t)r * 8;
    *reinterpret_cast<uint4*>(d.tail_k + dst) = *reinterpret_cast<const uint4*>(k_new + src);
    *reinterpret_cast<uint4*>(d.tail_v + dst) = *reinterpret_cast<const uint4*>(v_new + src);
  }
  if (blockIdx.x == 0 && threadIdx.x == 0 && d.own_pool)
    d.own_qgroups[b] = (int)quantized_end(nw, g.sink, g.window);
}

}  // namespace

hipError_t launch_append(const Geom& g, const CellDesc* desc_dev, const CellDesc& dh,
                         const uint16_t* k_new, const uint16_t* v_new, int batch, int n_new,
                         const int32_t* n_new_dev, const int32_t* seq_lens,
                         const int32_t* page_table, int pt_stride, hipStream_t stream) {
  if (dh.own_pool) {
    // A call of n tokens moves at most ceil(n / 32) groups of a request out of the window.
    const dim3 grid((unsigned)((n_new + kGroup - 1) / kGroup), (unsigned)g.H, (unsigned)batch);
    const bool fused = n_new <= kGroup && g.tail >= g.window + 2 * kGroup && g.D == 128;
    if (dh.own_bits == 4) {
      if (fused) quantize_group_kernel<4, true><<<grid, 128, 0, stream>>>(g, desc_dev, k_new, v_new, n_new, n_new_dev, seq_lens, page_table, pt_stride);
      else quantize_group_kernel<4, false><<<grid, 128, 0, stream>>>(g, desc_dev, k_new, v_new, n_new, n_new_dev, seq_lens, page_table, pt_stride);
    } else {
      if (fused) quantize_group_kernel<2, true><<<grid, 128, 0, stream>>>(g, desc_dev, k_new, v_new, n_new, n_new_dev, seq_lens, page_table, pt_stride);
      else quantize_group_kernel<2, false><<<grid, 128, 0, stream>>>(g, desc_dev, k_new, v_new, n_new, n_new_dev, seq_lens, page_table, pt_stride);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (fused) return hipSuccess;
  }
  // The ring kernel must follow the quantize kernel: that one reads ring slots this one
  // may overwrite. Both are on `stream`, so they run in order.
  const int first = n_new > g.tail ? n_new - g.tail : 0;
  const int64_t chunks = (int64_t)(n_new - first) * (g.H * g.D / 8);
  const dim3 grid2((unsigned)((chunks + 255) / 256), (unsigned)batch);
  tail_write_kernel<<<grid2, 256, 0, stream>>>(g, desc_dev, k_new, v_new, n_new, n_new_dev,
                                               seq_lens, pt_stride);
  return hipGetLastError();
}

}  // namespace loopkv
