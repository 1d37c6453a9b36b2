// gfx950 matrix-core kernels for the delta apply y = W x + U diag(sigma) (V x)
// ("Delta-CoMe: Training-Free Delta-Compression with Mixed-Precision for
// LLMs", Approach: 8/3/2-bit singular vectors; "Delta-CoMe - 清华联合OpenBMB...",
// technical principles).
//
// The 3- and 2-bit codes go straight into v_mfma_scale_f32_16x16x128_f8f6f4
// as its B operand: a 2-bit code zero-extended into an fp4 (e2m1) nibble is
// the value q/2, a 3-bit code zero-extended into an fp6 (e2m3) field is q/8,
// so unpacking a word is one AND and one shift for 16 (or ~10) codes.  The
// activations are the A operand as fp8 (e4m3) pieces with E8M0 block scales:
// x (bf16, 8 significant bits) = hi + lo exactly; t' (fp32) = hi + mid + lo
// to 12 bits.  The zero point is folded out of the inner loop:
//   sum_j s (q_j - z) x_j = s (sum_j q_j x_j - z sum_j x_j).
//
// Operand layout of 16x16x128 on gfx950 (checked on the hardware):
//   D[i][j]: lane l holds column j = l%16, rows i = 4(l/16) + r.
//   A (fp8):  lane l, row l%16, lane group g = l/16, byte e: hardware
//             k = 16g + e (e < 16) or 48 + 16g + e (e >= 16).
//   B (fp4/fp6): lane l, column l%16, element e: k = 32g + e.
//   Scale operand of lane l: E8M0 of the block k in [32g, 32g+32).
// A lane of B holds the 32 codes of chunk g of a 128-code run as even codes
// (elements 0..15) then odd codes (16..31), so k = 32g + e carries code
// c(k) = 32(k/32) + 2(k%16) + (k%32 >= 16); the A side is written in the
// same order.  The 8-bit pairs (two per matrix at the 1/16 budget) run on
// the vector ALU with the fp16 dequantized weights fp16(s(q - z)).
#include <hip/hip_runtime.h>

#include "dc_internal.h"

namespace dc {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kFmtFp8 = 0, kFmtFp6 = 2, kFmtFp4 = 4;
constexpr int kScaleFp4Code = 128;   // 2^1: fp4 element q/2 -> q
constexpr int kScaleFp6Code = 130;   // 2^3: fp6 element q/8 -> q
constexpr int kXFrag = 256;          // bytes of x fragments per (token, 128-group)

__device__ __forceinline__ float f16f(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// E8M0 byte of a block whose largest magnitude is m, chosen so that
// m * 2^-E lies in [128, 256) (fits e4m3, whose largest value is 448).
__device__ __forceinline__ int block_scale_byte(float m) {
  if (!(m > 0.f)) return 127;
  int e = (int)((__float_as_uint(m) >> 23) & 0xFF);   // biased exponent of m
  if (e == 0) e = 1;                                   // subnormal m: treat as 2^-126
  int b = e - 7;                                       // 127 + (e - 127) - 7
  return b < 10 ? 10 : (b > 253 ? 253 : b);
}

__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// fp8 (e4m3) byte of v (|v| < 448), and its value back in fp32.
__device__ __forceinline__ uint32_t fp8_of(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.f, 0, false) & 0xFFu;
}
__device__ __forceinline__ float fp8_val(uint32_t byte) { return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0); }

// Position of element j (0..127) of a 128-run in the fp8 A fragments:
// lane group g and byte e, so that it meets code j of the B operand.
__device__ __forceinline__ void a_pos(int j, int& g, int& e) {
  const int a = j >> 5, w = j & 31, p = w & 1, h = w >> 1;
  if (a < 2) { g = 2 * a + p; e = h; }
  else { g = 2 * (a - 2) + p; e = 16 + h; }
}

// B operand from the 32 codes of one lane at 2 bits (two words): fp4 nibbles,
// even codes first.  Elements 0..7 = even codes of w0, 8..15 = even of w1,
// 16..23 = odd of w0, 24..31 = odd of w1.
__device__ __forceinline__ v8i b_fp4(uint32_t w0, uint32_t w1) {
  v8i b = {0, 0, 0, 0, 0, 0, 0, 0};
  b[0] = (int)(w0 & 0x33333333u);
  b[1] = (int)(w1 & 0x33333333u);
  b[2] = (int)((w0 >> 2) & 0x33333333u);
  b[3] = (int)((w1 >> 2) & 0x33333333u);
  return b;
}

// B operand from 32 codes at 3 bits (a 96-bit run w0,w1,w2): fp6 fields of
// 6 bits, even codes in fields 0..15, odd codes in 16..31.
__device__ __forceinline__ v8i b_fp6(uint32_t w0, uint32_t w1, uint32_t w2) {
  v8i b = {0, 0, 0, 0, 0, 0, 0, 0};
  b[0] = (int)(w0 & 0xC71C71C7u);
  b[1] = (int)(w1 & 0x71C71C71u);
  b[2] = (int)(w2 & 0x1C71C71Cu);
  const uint32_t s0 = __builtin_amdgcn_alignbit(w1, w0, 3);
  const uint32_t s1 = __builtin_amdgcn_alignbit(w2, w1, 3);
  const uint32_t s2 = w2 >> 3;
  b[3] = (int)(s0 & 0xC71C71C7u);
  b[4] = (int)(s1 & 0x71C71C71u);
  b[5] = (int)(s2 & 0x1C71C71Cu);
  return b;
}

// Keeps the source registers of a chain of matrix-core ops allocated until
// its result has been read back into `d`.  Without it the register allocator
// may hand an A operand or scale VGPR of an op still in flight to a load
// issued after it (observed: an LDS load landing in the A and scale VGPRs of
// the preceding v_mfma_scale changed its result).
__device__ __forceinline__ void hold(f32x4& d, const v8i& a0, const v8i& a1, const v8i& b, int s0, int s1, int sb) {
  asm volatile("" : "+v"(d) : "v"(a0), "v"(a1), "v"(b), "v"(s0), "v"(s1), "v"(sb));
}
__device__ __forceinline__ void hold(f32x4& d, const v8i& a0, const v8i& a1, const v8i& a2, const v8i& b, int s0,
                                     int s1, int s2, int sb) {
  asm volatile("" : "+v"(d) : "v"(a0), "v"(a1), "v"(a2), "v"(b), "v"(s0), "v"(s1), "v"(s2), "v"(sb));
}

__device__ __forceinline__ f32x4 mma(const v8i& a, const v8i& b, f32x4 c, int sa, int fmt_b, int sb) {
  if (fmt_b == kFmtFp4)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, kFmtFp8, kFmtFp4, 0, sa, 0, sb);
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, kFmtFp8, kFmtFp6, 0, sa, 0, sb);
}

struct Seg {
  int b, lo, n;
  const uint8_t* vc;
  const uint32_t* vs;
  const uint8_t* uc;
  const uint32_t* us;
};

__device__ __forceinline__ Seg seg_of(const Tenant& tn, const Layout& L, int which) {
  Seg s;
  const int rv = which == 0 ? DC_REG_VC8 : (which == 1 ? DC_REG_VC3 : DC_REG_VC2);
  s.b = which == 0 ? 8 : (which == 1 ? 3 : 2);
  s.lo = which == 0 ? 0 : (which == 1 ? tn.n8 : tn.n8 + tn.n3);
  s.n = which == 0 ? tn.n8 : (which == 1 ? tn.n3 : tn.n2);
  s.vc = tn.base + L.off[rv];
  s.vs = reinterpret_cast<const uint32_t*>(tn.base + L.off[rv + 3]);
  s.uc = tn.base + L.off[rv + 6];
  s.us = reinterpret_cast<const uint32_t*>(tn.base + L.off[rv + 9]);
  return s;
}

struct SegArg {
  int32_t v[DC_MAX_TENANTS + 1];
};

// ------------------------------------------------------- split-K combine
// Work items of one output block add their partial sums in a fixed order:
// each item stores its partials with device-coherent stores, waits until
// they have completed, then bumps the block's arrival counter; the item that
// arrives last reads every partial back with device-coherent loads.  Only
// these accesses bypass the per-XCD L2s; nothing writes back or invalidates a
// whole L2 (which a device-scope fence would).
__device__ __forceinline__ void st_dev(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// True in every thread of the item that arrives last of `total`.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, int total, int* flag) {
  __builtin_amdgcn_s_waitcnt(0);   // this thread's partial stores are complete
  __syncthreads();
  if (threadIdx.x == 0)
    *flag = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(total - 1);
  __syncthreads();
  return *flag != 0;
}

// ------------------------------------------------------------------- prep
// Block 0 routes the tokens (stable counting sort by tenant; bucket n holds
// the backbone-only tokens).  Every other wave turns one (token, 128-group)
// of x into fp8 hi/lo A fragments, their E8M0 scales and the group sum.
__global__ void __launch_bounds__(256) k_prep(const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
                                              int32_t T, int32_t in, int32_t n, int32_t mode, SegArg seg,
                                              int32_t* __restrict__ offs, int32_t* __restrict__ perm,
                                              uint32_t* __restrict__ flags, uint8_t* __restrict__ xf,
                                              uint32_t* __restrict__ xsc, float* __restrict__ xsum,
                                              uint16_t* __restrict__ xt, uint32_t* __restrict__ cnt, int32_t ncnt) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {
    for (int i = tid; i < ncnt; i += blockDim.x) cnt[i] = 0u;
    if (mode != 1) {
      for (int p = tid; p < T; p += blockDim.x) perm[p] = p;
      if (tid == 0) {
        if (mode == 0) { offs[0] = 0; offs[1] = T; offs[2] = T; }
        else { for (int k = 0; k <= n; ++k) offs[k] = seg.v[k]; offs[n + 1] = T; }
        *flags = 0;
      }
      return;
    }
    __shared__ int cnt[DC_MAX_TENANTS + 1];
    __shared__ int next[DC_MAX_TENANTS + 1];
    __shared__ int bkt[256];
    __shared__ int bad;
    for (int b = tid; b <= n; b += blockDim.x) cnt[b] = 0;
    if (tid == 0) bad = 0;
    __syncthreads();
    for (int t = tid; t < T; t += blockDim.x) {
      int k = ids[t];
      if (k < -1 || k >= n) { bad = 1; k = -1; }
      atomicAdd(&cnt[k < 0 ? n : k], 1);
    }
    __syncthreads();
    if (tid == 0) {
      int s = 0;
      for (int b = 0; b <= n; ++b) { offs[b] = s; next[b] = s; s += cnt[b]; }
      offs[n + 1] = s;
      *flags = bad ? 1u : 0u;
    }
    __syncthreads();
    for (int c0 = 0; c0 < T; c0 += blockDim.x) {
      const int t = c0 + tid;
      int b = -1;
      if (t < T) { const int k = ids[t]; b = (k < 0 || k >= n) ? n : k; }
      bkt[tid] = b;
      __syncthreads();
      if (t < T) {
        int rank = 0;
        for (int j = 0; j < tid; ++j) rank += (bkt[j] == b);
        perm[next[b] + rank] = t;
      }
      __syncthreads();
      if (t < T) atomicAdd(&next[b], 1);
      __syncthreads();
    }
    return;
  }
  const int gi_n = in / kGroup;
  const size_t item = (size_t)(blockIdx.x - 1) * 4 + (tid >> 6);
  if (item >= (size_t)T * gi_n) return;
  const int lane = tid & 63;
  const int t = (int)(item / gi_n), gi = (int)(item % gi_n);
  const uint16_t* xr = x + (size_t)t * in + (size_t)gi * kGroup;
  const uint16_t x0 = xr[lane], x1 = xr[lane + 64];
  const float v0 = __uint_as_float((uint32_t)x0 << 16);   // element j = lane (chunk lane/32)
  const float v1 = __uint_as_float((uint32_t)x1 << 16);   // element j = lane + 64 (chunk 2 + lane/32)
  if (xt) {  // bf16 B tiles of the backbone product: k = 128 gi + j -> step k/32, lane group (k%32)/8
    const int tiles = (T + 15) / 16, tl = t & 15, tt = t >> 4;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int k = gi * kGroup + lane + 64 * h;
      const int l = 16 * ((k & 31) >> 3) + tl;
      xt[(((size_t)(k >> 5) * tiles + tt) * 64 + l) * 8 + (k & 7)] = h ? x1 : x0;
    }
  }
  float m0 = fabsf(v0), m1 = fabsf(v1);
#pragma unroll
  for (int s = 16; s >= 1; s >>= 1) {
    m0 = fmaxf(m0, __shfl_xor(m0, s, 64));
    m1 = fmaxf(m1, __shfl_xor(m1, s, 64));
  }
  const int b0 = block_scale_byte(m0), b1 = block_scale_byte(m1);
  uint8_t* fr = xf + item * kXFrag;
  {
    const float v = v0 * pow2f(127 - b0);
    const uint32_t h = fp8_of(v);
    const uint32_t lo = fp8_of((v - fp8_val(h)) * 32.f);
    int g, e;
    a_pos(lane, g, e);
    fr[g * 64 + e] = (uint8_t)h;
    fr[g * 64 + 32 + e] = (uint8_t)lo;
  }
  {
    const float v = v1 * pow2f(127 - b1);
    const uint32_t h = fp8_of(v);
    const uint32_t lo = fp8_of((v - fp8_val(h)) * 32.f);
    int g, e;
    a_pos(lane + 64, g, e);
    fr[g * 64 + e] = (uint8_t)h;
    fr[g * 64 + 32 + e] = (uint8_t)lo;
  }
  float s = v0 + v1;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) s += __shfl_xor(s, m, 64);
  // chunk scales: lanes 0..31 hold chunks 0 (b0) and 2 (b1), lanes 32..63 chunks 1 and 3
  const int c1 = __shfl(b0, 32, 64), c3 = __shfl(b1, 32, 64);
  if (lane == 0) {
    xsc[item] = (uint32_t)b0 | ((uint32_t)c1 << 8) | ((uint32_t)b1 << 16) | ((uint32_t)c3 << 24);
    xsum[item] = s;
  }
}

// ------------------------------------------------------------------ V side
// Work item (block): tenant k = blockIdx.y; blockIdx.x = rank block rb *
// v_slices + input slice s.  Rank blocks: the 8-bit rows (vector ALU, fp16
// dequantized weights), then 64-rank blocks of the 3-bit and of the 2-bit
// segment (four 16-rank tiles, one per wave, on the matrix cores).  An item
// covers kVSlice 128-groups of the input; it issues all of its loads up
// front, writes a partial sum per (token, rank), and the last item of a rank
// block to arrive adds the slices in slice order and writes t = sigma * sum.
struct VsideLds {
  int4 frag[kVSlice][kVRows][4][4];   // [group][token row][lane group][hi0 hi1 lo0 lo1]
  uint32_t sc[kVSlice][kVRows];       // E8M0 words
  float xs[kVSlice][kVRows];          // group sums
  int last;
};

template <int B>
struct CodeW;
template <>
struct CodeW<2> { uint32_t w[2]; };
template <>
struct CodeW<3> { uint32_t w[3]; };

template <int B>
__device__ __forceinline__ CodeW<B> load_codes(const uint32_t* row, int gi, int q) {
  CodeW<B> c;
  if constexpr (B == 2) {
    const uint2 v = *reinterpret_cast<const uint2*>(row + (size_t)gi * 8 + 2 * q);
    c.w[0] = v.x; c.w[1] = v.y;
  } else {
    const uint32_t* wp = row + (size_t)gi * 12 + 3 * q;
#pragma unroll
    for (int i = 0; i < B; ++i) c.w[i] = wp[i];
  }
  return c;
}

template <int B>
__device__ __forceinline__ v8i b_op(const CodeW<B>& c) {
  if constexpr (B == 2) return b_fp4(c.w[0], c.w[1]);
  else return b_fp6(c.w[0], c.w[1], c.w[2]);
}

// Stage x fragments of token rows [pb, pb + kVRows) and groups [g0, g0+kVSlice)
// into LDS: thread tid moves int4 (tid & 3) of lane group (tid>>2)&3 of row
// (tid>>4)&7 for groups (tid>>7) + 2u; threads < 128 also move one
// (group, row) scale word and sum.
__device__ __forceinline__ void x_stage(VsideLds& S, const uint8_t* __restrict__ xf, const uint32_t* __restrict__ xsc,
                                        const float* __restrict__ xsum, const int32_t* __restrict__ perm, int gi_n,
                                        int g0, int pb, int nt) {
  const int tid = threadIdx.x;
  const int part = tid & 3, qq = (tid >> 2) & 3, row = (tid >> 4) & 7, gh = tid >> 7;
  const int tok = row < nt ? perm[pb + row] : -1;
  int4 v[kVSlice / 2];
#pragma unroll
  for (int u = 0; u < kVSlice / 2; ++u) {
    const int gl = gh + 2 * u, gi = g0 + gl;
    v[u] = make_int4(0, 0, 0, 0);
    if (tok >= 0 && gi < gi_n) v[u] = reinterpret_cast<const int4*>(xf + ((size_t)tok * gi_n + gi) * kXFrag + qq * 64)[part];
  }
  uint32_t scw = 0x7F7F7F7Fu;
  float xsv = 0.f;
  const int sr = tid & 7, sg = tid >> 3;   // (row, group) of the scale/sum this thread moves
  if (tid < kVRows * kVSlice) {
    const int stok = sr < nt ? perm[pb + sr] : -1;
    if (stok >= 0 && g0 + sg < gi_n) {
      scw = xsc[(size_t)stok * gi_n + g0 + sg];
      xsv = xsum[(size_t)stok * gi_n + g0 + sg];
    }
  }
#pragma unroll
  for (int u = 0; u < kVSlice / 2; ++u) S.frag[gh + 2 * u][row][qq][part] = v[u];
  if (tid < kVRows * kVSlice) {
    S.sc[sg][sr] = scw;
    S.xs[sg][sr] = xsv;
  }
}

// 8-bit rows of a tenant over one input slice, all tokens; partial sums
// (without sigma) to part[p][i].
__device__ void vside_8bit(const Tenant& tn, const Layout& L, int in, int s, const uint16_t* __restrict__ x,
                           const int32_t* __restrict__ perm, int p0, int p1, float* __restrict__ part, int rs) {
  constexpr int kQ = kVSlice * kGroup / 4 / 256;   // quads per thread per slice (2)
  __shared__ float red[4][8];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const Seg sg = seg_of(tn, L, 0);
  const int np = (int)round_up(sg.n, 4);
  const int q0 = s * kVSlice * kGroup / 4, nq = in / 4;
  for (int i = 0; i < sg.n; ++i) {
    const uint8_t* row = sg.vc + (size_t)i * in;   // 8-bit group bitstreams are plain bytes
    float w[kQ][4];
#pragma unroll
    for (int m = 0; m < kQ; ++m) {
      const int qd = q0 + tid + 256 * m;
#pragma unroll
      for (int u = 0; u < 4; ++u) w[m][u] = 0.f;
      if (qd < nq) {
        const uint32_t e = sg.vs[(size_t)(qd * 4 / kGroup) * np + i];
        const uint32_t c4 = *reinterpret_cast<const uint32_t*>(row + (size_t)qd * 4);
        const float sc = f16f(e & 0xFFFFu), z = f16f(e >> 16);
#pragma unroll
        for (int u = 0; u < 4; ++u) w[m][u] = (float)(_Float16)(sc * ((float)((c4 >> (8 * u)) & 0xFFu) - z));
      }
    }
    for (int pc = p0; pc < p1; pc += 8) {
      const int nt = min(8, p1 - pc);
      float acc[8];
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) {
        acc[t8] = 0.f;
        if (t8 < nt) {
          const uint16_t* xr = x + (size_t)perm[pc + t8] * in;
#pragma unroll
          for (int m = 0; m < kQ; ++m) {
            const int qd = q0 + tid + 256 * m;
            if (qd < nq) {
              const uint2 xv = *reinterpret_cast<const uint2*>(xr + (size_t)qd * 4);
              acc[t8] += w[m][0] * __uint_as_float(xv.x << 16) + w[m][1] * __uint_as_float(xv.x & 0xFFFF0000u) +
                         w[m][2] * __uint_as_float(xv.y << 16) + w[m][3] * __uint_as_float(xv.y & 0xFFFF0000u);
            }
          }
        }
      }
#pragma unroll
      for (int t8 = 0; t8 < 8; ++t8) {
        float v = acc[t8];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
        if (lane == 0) red[wave][t8] = v;
      }
      __syncthreads();
      if (tid < nt) st_dev(part + (size_t)(pc + tid) * rs + i, (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]));
      __syncthreads();
    }
  }
}

// One 16-rank tile per wave over one input slice, all tokens in passes of kVRows.
template <int B>
__device__ void vside_tiles(const Seg& sg, int tile, int in, int s, const int32_t* __restrict__ perm, int p0,
                            int p1, const uint8_t* __restrict__ xf, const uint32_t* __restrict__ xsc,
                            const float* __restrict__ xsum, float* __restrict__ part, int rs, VsideLds& S) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, q = lane >> 4;
  const int gi_n = in / kGroup;
  const int g0 = s * kVSlice;
  const int li = tile * 16 + col;
  const bool rv = li < sg.n;
  const int np = (int)round_up(sg.n, 4);
  const uint32_t* row = reinterpret_cast<const uint32_t*>(sg.vc) + (size_t)(rv ? li : 0) * gi_n * 4 * B;
  const uint32_t* vsp = sg.vs + (rv ? li : 0);
  const int fmt = B == 2 ? kFmtFp4 : kFmtFp6;
  const int bsc = B == 2 ? kScaleFp4Code : kScaleFp6Code;
  // every code and scale/zero word of the slice, issued at once
  CodeW<B> cw[kVSlice];
  uint32_t zw[kVSlice];
#pragma unroll
  for (int u = 0; u < kVSlice; ++u) {
    const int gi = g0 + u < gi_n ? g0 + u : gi_n - 1;
    cw[u] = load_codes<B>(row, gi, q);
    zw[u] = vsp[(size_t)gi * np];
  }
  for (int pb = p0; pb < p1; pb += kVRows) {
    const int nt = min(kVRows, p1 - pb);
    __syncthreads();   // LDS reuse across passes
    x_stage(S, xf, xsc, xsum, perm, gi_n, g0, pb, nt);
    __syncthreads();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kVSlice; ++u) {
      if (g0 + u < gi_n) {
        v8i ah = {0, 0, 0, 0, 0, 0, 0, 0}, al = ah;
        int sh = 127;
        if (col < kVRows) {
          const int4* fr = S.frag[u][col][q];
          const int4 h0 = fr[0], h1 = fr[1], l0 = fr[2], l1 = fr[3];
          ah = v8i{h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
          al = v8i{l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
          sh = (int)((S.sc[u][col] >> (8 * q)) & 0xFFu);
        }
        v8i bop = b_op<B>(cw[u]);
        if (!rv) bop = v8i{0, 0, 0, 0, 0, 0, 0, 0};
        const int sl = sh - 5;
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
        d = mma(ah, bop, d, sh, fmt, bsc);
        d = mma(al, bop, d, sl, fmt, bsc);
        hold(d, ah, al, bop, sh, sl, bsc);
        const float sc = f16f(zw[u] & 0xFFFFu), z = f16f(zw[u] >> 16);
        if (q < 2) {   // D rows 4q+r < 8 are the staged tokens
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r] += sc * (d[r] - z * S.xs[u][4 * q + r]);
        }
      }
    }
    if (rv && q < 2) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pd = pb + 4 * q + r;
        if (4 * q + r < nt) st_dev(part + (size_t)pd * rs + sg.lo + li, acc[r]);
      }
    }
  }
}

__global__ void __launch_bounds__(256) k_vside(TenantTable tt, int32_t out, int32_t in,
                                               const uint16_t* __restrict__ x, const int32_t* __restrict__ offs,
                                               const int32_t* __restrict__ perm, const uint8_t* __restrict__ xf,
                                               const uint32_t* __restrict__ xsc, const float* __restrict__ xsum,
                                               float* __restrict__ vpart, float* __restrict__ tv, int32_t rs,
                                               int32_t T, uint32_t* __restrict__ cnt, int32_t vbmax) {
  const int k = blockIdx.y;
  const int p0 = offs[k], p1 = offs[k + 1];
  if (p0 >= p1) return;
  const Tenant tn = tt.t[k];
  const int ns = v_slices(in);
  const int rb = blockIdx.x / ns, s = blockIdx.x % ns;
  if (rb >= v_blocks(tn.n8, tn.n3, tn.n2)) return;
  Layout L;
  layout_of(out, in, tn.n8, tn.n3, tn.n2, &L);
  __shared__ VsideLds S;
  const int tid = threadIdx.x, wave = tid >> 6;
  float* part = vpart + (size_t)s * T * rs;
  const int b3 = (tn.n3 + 63) / 64;
  int lo, hi;   // global rank range of the block
  int b = rb;
  if (tn.n8 > 0 && b == 0) {
    vside_8bit(tn, L, in, s, x, perm, p0, p1, part, rs);
    lo = 0; hi = tn.n8;
  } else {
    if (tn.n8 > 0) --b;
    if (b < b3) {
      const Seg sg = seg_of(tn, L, 1);
      vside_tiles<3>(sg, b * 4 + wave, in, s, perm, p0, p1, xf, xsc, xsum, part, rs, S);
      lo = sg.lo + b * 64; hi = min(sg.lo + sg.n, lo + 64);
    } else {
      const Seg sg = seg_of(tn, L, 2);
      vside_tiles<2>(sg, (b - b3) * 4 + wave, in, s, perm, p0, p1, xf, xsc, xsum, part, rs, S);
      lo = sg.lo + (b - b3) * 64; hi = min(sg.lo + sg.n, lo + 64);
    }
  }
  // last arriving slice of this rank block adds the slices in order
  if (!arrive_last(&cnt[(size_t)k * vbmax + rb], ns, &S.last)) return;
  const float* sigma = reinterpret_cast<const float*>(tn.base + L.off[DC_REG_SIGMA]);
  const int nr = hi - lo, cells = (p1 - p0) * nr;
  for (int c = tid; c < cells; c += 256) {
    const int p = p0 + c / nr, i = lo + c % nr;
    float v = 0.f;
    for (int j = 0; j < ns; ++j) v += ld_dev(vpart + ((size_t)j * T + p) * rs + i);
    tv[(size_t)p * rs + i] = sigma[i] * v;
  }
}

// ------------------------------------------------------------------ U side
// Work item (block): blockIdx.x = 128-row output group g, blockIdx.y =
// tenant k (n = the backbone-only bucket), blockIdx.z = rank slice su of
// kUPass chunks of 128 ranks (3-bit chunks first, then 2-bit).  Wave w builds
// the A fragments of t'_i = s_ig t_i (three fp8 pieces, E8M0 block scales)
// for chunk w of the slice: lane (token row i, lane group gq) writes exactly
// the 32-byte rows an MFMA lane (i, gq) reads.  Then every wave runs its two
// 16-row output tiles against the slice; its codes were loaded before the
// A-prep.  The slice's partial sum_i (q_oi - z_ig) t'_i goes to upart; the
// last slice to arrive adds the slices in order, the 8-bit pairs and W x,
// rounds once to bf16 and writes y.
struct UsideLds {
  int4 frag[kUPass][3][4][16][2];   // [chunk][piece][lane group][token row][32 bytes]
  uint8_t sc[kUPass][16][4];        // E8M0 of piece 0 per (chunk, token row, K-block)
  float cz[16][16];                 // partial sum_i z t' per (token row, slot)
  int last;
};

struct UChunk {
  int which;   // 1: 3-bit segment, 2: 2-bit segment
  int c;       // chunk index inside the segment
};

__device__ __forceinline__ UChunk chunk_of(int ci, int nc3) {
  UChunk u;
  if (ci < nc3) { u.which = 1; u.c = ci; }
  else { u.which = 2; u.c = ci - nc3; }
  return u;
}

__global__ void __launch_bounds__(256, 2) k_uside(TenantTable tt, int32_t n, int32_t out, int32_t in,
                                                  const int32_t* __restrict__ offs, const int32_t* __restrict__ perm,
                                                  const float* __restrict__ tv, int32_t rs,
                                                  const float* __restrict__ ybase, float* __restrict__ upart,
                                                  int32_t T, uint32_t* __restrict__ cnt, int32_t vbmax,
                                                  uint16_t* __restrict__ y) {
  const int g = blockIdx.x, k = blockIdx.y, su = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, q = lane >> 4;
  const int p0 = offs[k], p1 = offs[k + 1];
  if (p0 >= p1) return;
  const int go = out / kGroup;
  if (k == n) {  // backbone-only tokens
    if (su != 0) return;
    for (int idx = tid; idx < (p1 - p0) * kGroup; idx += 256) {
      const int t = perm[p0 + idx / kGroup];
      const int o = g * kGroup + idx % kGroup;
      y[(size_t)t * out + o] = to_bf16(ybase ? ybase[(size_t)t * out + o] : 0.f);
    }
    return;
  }
  const Tenant tn = tt.t[k];
  const int nsu = u_slices(tn.n3, tn.n2);
  if (su >= nsu) return;
  Layout L;
  layout_of(out, in, tn.n8, tn.n3, tn.n2, &L);
  __shared__ UsideLds S;
  const Seg seg3 = seg_of(tn, L, 1), seg2 = seg_of(tn, L, 2);
  const int kb3 = (seg3.n + kKBlock - 1) / kKBlock, kb2 = (seg2.n + kKBlock - 1) / kKBlock;
  const int nc3 = (kb3 + 3) / 4, nc = nc3 + (kb2 + 3) / 4;
  const int orow[2] = {g * kGroup + wave * 32 + col, g * kGroup + wave * 32 + 16 + col};
  // codes of the slice for this wave's two tiles
  uint32_t cw[kUPass][2][3];
#pragma unroll
  for (int cb = 0; cb < kUPass; ++cb) {
#pragma unroll
    for (int h = 0; h < 2; ++h) { cw[cb][h][0] = 0u; cw[cb][h][1] = 0u; cw[cb][h][2] = 0u; }
    const int ci = su * kUPass + cb;
    if (ci < nc) {
      const UChunk u = chunk_of(ci, nc3);
      const Seg& sg = u.which == 1 ? seg3 : seg2;
      const int kb = 4 * u.c + q;
      if (kb < (u.which == 1 ? kb3 : kb2)) {
        const uint32_t* base = reinterpret_cast<const uint32_t*>(sg.uc);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          int nw;
          const uint32_t* wp = base + u_kblock_word(orow[h], kb, sg.n, sg.b, &nw);
          cw[cb][h][0] = wp[0];
          if (nw > 1) cw[cb][h][1] = wp[1];
          if (nw > 2) cw[cb][h][2] = wp[2];
        }
      }
    }
  }
  float* part = upart + (size_t)su * T * out;
  // A-prep role: token row pi = lane % 16, lane group gq = lane / 16; ranks of
  // run 0 start at mA = 32(gq/2) + (gq&1) (stride 2), run 1 at 64 + mA.
  const int pi = col, gq = q;
  const int mA = 32 * (gq >> 1) + (gq & 1);
  for (int pb = p0; pb < p1; pb += 16) {
    const int nt = min(16, p1 - pb);
    float czp = 0.f;
    {
      const int ci = su * kUPass + wave;
      int4 pk[3][2];
      int sbA = 127, sbB = 127;
#pragma unroll
      for (int pc = 0; pc < 3; ++pc) { pk[pc][0] = make_int4(0, 0, 0, 0); pk[pc][1] = pk[pc][0]; }
      if (ci < nc) {
        const UChunk u = chunk_of(ci, nc3);
        const Seg& sg = u.which == 1 ? seg3 : seg2;
        const int np = (int)round_up(sg.n, 4);
        const bool tok_ok = pi < nt;
        const float* tvr = tv + (size_t)(pb + (tok_ok ? pi : 0)) * rs + sg.lo + u.c * 128;
        const uint32_t* usr = sg.us + (size_t)g * np + u.c * 128;
        const int lim = sg.n - u.c * 128;
#pragma unroll
        for (int run = 0; run < 2; ++run) {
          float tpv[16];
          uint32_t zz[16];
          float mx = 0.f;
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int m = 64 * run + mA + 2 * e;
            const bool ok = tok_ok && m < lim;
            const uint32_t w = ok ? usr[m] : 0u;
            const float t = ok ? tvr[m] : 0.f;
            tpv[e] = f16f(w & 0xFFFFu) * t;
            zz[e] = w >> 16;
            mx = fmaxf(mx, fabsf(tpv[e]));
          }
          mx = fmaxf(mx, __shfl_xor(mx, 16, 64));   // partner lane group holds the other parity
          const int sb = block_scale_byte(mx);
          if (run == 0) sbA = sb; else sbB = sb;
          const float inv = pow2f(127 - sb), fwd = pow2f(sb - 127);
          uint32_t wd[3][4] = {{0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}, {0u, 0u, 0u, 0u}};
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const float x0 = tpv[e] * inv;
            const uint32_t h0 = fp8_of(x0);
            const float r1 = (x0 - fp8_val(h0)) * 32.f;
            const uint32_t h1 = fp8_of(r1);
            const float r2 = (r1 - fp8_val(h1)) * 32.f;
            const uint32_t h2 = fp8_of(r2);
            const float back = (fp8_val(h0) + (fp8_val(h1) + fp8_val(h2) * (1.f / 32.f)) * (1.f / 32.f)) * fwd;
            czp += f16f(zz[e]) * back;   // zero for missing ranks and empty token rows
            wd[0][e >> 2] |= h0 << (8 * (e & 3));
            wd[1][e >> 2] |= h1 << (8 * (e & 3));
            wd[2][e >> 2] |= h2 << (8 * (e & 3));
          }
#pragma unroll
          for (int pc = 0; pc < 3; ++pc)
            pk[pc][run] = make_int4((int)wd[pc][0], (int)wd[pc][1], (int)wd[pc][2], (int)wd[pc][3]);
        }
      }
      __syncthreads();   // LDS reuse across token tiles
#pragma unroll
      for (int pc = 0; pc < 3; ++pc) {
        S.frag[wave][pc][gq][pi][0] = pk[pc][0];
        S.frag[wave][pc][gq][pi][1] = pk[pc][1];
      }
      if ((gq & 1) == 0) {
        S.sc[wave][pi][gq >> 1] = (uint8_t)sbA;
        S.sc[wave][pi][2 + (gq >> 1)] = (uint8_t)sbB;
      }
      S.cz[pi][wave * 4 + gq] = czp;
    }
    __syncthreads();
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int cb = 0; cb < kUPass; ++cb) {
      const int ci = su * kUPass + cb;
      if (ci < nc) {
        const bool three = ci < nc3;
        const int4* f0 = S.frag[cb][0][q][col];
        const int4* f1 = S.frag[cb][1][q][col];
        const int4* f2 = S.frag[cb][2][q][col];
        const v8i a0 = {f0[0].x, f0[0].y, f0[0].z, f0[0].w, f0[1].x, f0[1].y, f0[1].z, f0[1].w};
        const v8i a1 = {f1[0].x, f1[0].y, f1[0].z, f1[0].w, f1[1].x, f1[1].y, f1[1].z, f1[1].w};
        const v8i a2 = {f2[0].x, f2[0].y, f2[0].z, f2[0].w, f2[1].x, f2[1].y, f2[1].z, f2[1].w};
        const int s0 = S.sc[cb][col][q];
        const int bsc = three ? kScaleFp6Code : kScaleFp4Code;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const v8i bop = three ? b_fp6(cw[cb][h][0], cw[cb][h][1], cw[cb][h][2]) : b_fp4(cw[cb][h][0], cw[cb][h][1]);
          const int fmt = three ? kFmtFp6 : kFmtFp4;
          const int s1 = s0 - 5, s2 = s0 - 10;
          f32x4 d = {0.f, 0.f, 0.f, 0.f};
          d = mma(a0, bop, d, s0, fmt, bsc);
          d = mma(a1, bop, d, s1, fmt, bsc);
          d = mma(a2, bop, d, s2, fmt, bsc);
          hold(d, a0, a1, a2, bop, s0, s1, s2, bsc);
          acc[h] += d;
        }
      }
    }
    // partial of this slice: acc - sum_i z t'
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * q + r;
      if (row < nt) {
        float cz = 0.f;
#pragma unroll
        for (int u = 0; u < 16; ++u) cz += S.cz[row][u];
#pragma unroll
        for (int h = 0; h < 2; ++h) st_dev(part + (size_t)(pb + row) * out + orow[h], acc[h][r] - cz);
      }
    }
  }
  // last arriving slice: add the slices in order, the 8-bit pairs and W x
  if (!arrive_last(&cnt[(size_t)n * vbmax + (size_t)k * go + g], nsu, &S.last)) return;
  const Seg s8 = seg_of(tn, L, 0);
  const int np8 = (int)round_up(s8.n, 4);
  const int ol = tid & 127, o = g * kGroup + ol;
  float u8[8];
  const int n8c = min(s8.n, 8);
  for (int i = 0; i < n8c; ++i) {
    const uint32_t e = s8.us[(size_t)g * np8 + i];
    u8[i] = (float)(_Float16)(f16f(e & 0xFFFFu) * ((float)s8.uc[(size_t)o * s8.n + i] - f16f(e >> 16)));
  }
  for (int p = p0 + (tid >> 7); p < p1; p += 2) {
    float v = 0.f;
    for (int j = 0; j < nsu; ++j) v += ld_dev(upart + ((size_t)j * T + p) * out + o);
    for (int i = 0; i < s8.n; ++i) {
      float uh;
      if (i < n8c) uh = u8[i];
      else {
        const uint32_t e = s8.us[(size_t)g * np8 + i];
        uh = (float)(_Float16)(f16f(e & 0xFFFFu) * ((float)s8.uc[(size_t)o * s8.n + i] - f16f(e >> 16)));
      }
      v += uh * tv[(size_t)p * rs + i];
    }
    const int t = perm[p];
    if (ybase) v += ybase[(size_t)t * out + o];
    y[(size_t)t * out + o] = to_bf16(v);
  }
}

}  // namespace

int launch_apply(const ApplyArgs& a) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  uint32_t* flags = reinterpret_cast<uint32_t*>(a.ws + a.wl.flags);
  int32_t* offs = reinterpret_cast<int32_t*>(a.ws + a.wl.offs);
  int32_t* perm = reinterpret_cast<int32_t*>(a.ws + a.wl.perm);
  float* tv = reinterpret_cast<float*>(a.ws + a.wl.tv);
  float* ybase = a.W ? reinterpret_cast<float*>(a.ws + a.wl.ybase) : nullptr;
  float* vpart = reinterpret_cast<float*>(a.ws + a.wl.vpart);
  float* upart = reinterpret_cast<float*>(a.ws + a.wl.upart);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(a.ws + a.wl.cnt);
  const int go = a.out / kGroup;
  const int ncnt = a.n * (a.wl.vb + go);
  const size_t items = (size_t)a.T * (a.in / kGroup);
  uint8_t* xf = a.ws + a.wl.xf;
  uint32_t* xsc = reinterpret_cast<uint32_t*>(a.ws + a.wl.xsc);
  float* xsum = reinterpret_cast<float*>(a.ws + a.wl.xsum);
  uint16_t* xt = a.W ? reinterpret_cast<uint16_t*>(a.ws + a.wl.xt) : nullptr;
  SegArg seg{};
  if (a.mode == 2)
    for (int k = 0; k <= a.n; ++k) seg.v[k] = a.seg[k];
  auto mark = [&](int s) {
    if (a.events && a.events[s]) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(a.events[s]), st);
  };
  mark(DC_STAGE_ROUTE);
  mark(DC_STAGE_XPREP);
  hipLaunchKernelGGL(k_prep, dim3((unsigned)(1 + (items + 3) / 4)), dim3(256), 0, st, a.x, a.ids, a.T, a.in, a.n,
                     a.mode, seg, offs, perm, flags, xf, xsc, xsum, xt, cnt, ncnt);
  mark(DC_STAGE_BASE);
  if (a.W) launch_base(a.W, xt, ybase, a.out, a.in, a.T, a.stream);
  mark(DC_STAGE_VSIDE);
  if (a.wl.vb > 0)
    hipLaunchKernelGGL(k_vside, dim3((unsigned)(a.wl.vb * v_slices(a.in)), (unsigned)a.n), dim3(256), 0, st,
                       *a.tenants, a.out, a.in, a.x, offs, perm, xf, xsc, xsum, vpart, tv, a.wl.rs, a.T, cnt,
                       a.wl.vb);
  mark(DC_STAGE_USIDE);
  hipLaunchKernelGGL(k_uside, dim3((unsigned)go, (unsigned)(a.n + 1), (unsigned)a.wl.us), dim3(256), 0, st,
                     *a.tenants, a.n, a.out, a.in, offs, perm, tv, a.wl.rs, ybase, upart, a.T, cnt, a.wl.vb, a.y);
  mark(DC_STAGE_COUNT);
  return (int)hipGetLastError();
}

}  // namespace dc
