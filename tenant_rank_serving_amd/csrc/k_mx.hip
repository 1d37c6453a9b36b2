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

// ------------------------------------------------------------------- prep
// Block 0 routes the tokens (stable counting sort by tenant; bucket n holds
// the backbone-only tokens).  Every other wave turns one (token, 128-group)
// of x into fp8 hi/lo A fragments, their E8M0 scales and the group sum.
__global__ void __launch_bounds__(256) k_prep(const uint16_t* __restrict__ x, const int32_t* __restrict__ ids,
                                              int32_t T, int32_t in, int32_t n, int32_t mode, SegArg seg,
                                              int32_t* __restrict__ offs, int32_t* __restrict__ perm,
                                              uint32_t* __restrict__ flags, uint8_t* __restrict__ xf,
                                              uint32_t* __restrict__ xsc, float* __restrict__ xsum) {
  const int tid = threadIdx.x;
  if (blockIdx.x == 0) {
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
  const float v0 = __uint_as_float((uint32_t)xr[lane] << 16);          // element j = lane (chunk lane/32)
  const float v1 = __uint_as_float((uint32_t)xr[lane + 64] << 16);     // element j = lane + 64 (chunk 2 + lane/32)
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
// blockIdx.y = tenant, blockIdx.x = task.  Task 0 of a tenant with 8-bit
// pairs runs them on the vector ALU; every other task is four 16-rank tiles
// of the 3- or 2-bit segment, one per wave, each over the whole input.
__device__ void vside_8bit(const Tenant& tn, const Layout& L, int in, const uint16_t* __restrict__ x,
                           const int32_t* __restrict__ perm, int p0, int p1, float* __restrict__ tv, int rs) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const Seg sg = seg_of(tn, L, 0);
  const float* sigma = reinterpret_cast<const float*>(tn.base + L.off[DC_REG_SIGMA]);
  const int np = (int)round_up(sg.n, 4);
  const int gi_n = in / kGroup;
  for (int i = wave; i < sg.n; i += 4) {
    const uint8_t* row = sg.vc + (size_t)i * in;   // 8-bit group bitstreams are plain bytes
    for (int pc = p0; pc < p1; pc += 8) {
      const int nt = min(8, p1 - pc);
      int tok[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) tok[q] = perm[pc + (q < nt ? q : 0)];
      float acc[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[q] = 0.f;
      for (int j0 = lane * 4; j0 < in; j0 += 256) {
        const uint32_t e = sg.vs[(size_t)(j0 / kGroup) * np + i];
        const float s = f16f(e & 0xFFFFu), z = f16f(e >> 16);
        const uint32_t c4 = *reinterpret_cast<const uint32_t*>(row + j0);
        float w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) w[u] = (float)(_Float16)(s * ((float)((c4 >> (8 * u)) & 0xFFu) - z));
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          if (q < nt) {
            const uint2 xv = *reinterpret_cast<const uint2*>(x + (size_t)tok[q] * in + j0);
            acc[q] += w[0] * __uint_as_float(xv.x << 16) + w[1] * __uint_as_float(xv.x & 0xFFFF0000u) +
                      w[2] * __uint_as_float(xv.y << 16) + w[3] * __uint_as_float(xv.y & 0xFFFF0000u);
          }
        }
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        float v = acc[q];
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
        acc[q] = v;
      }
      if (lane == 0)
        for (int q = 0; q < nt; ++q) tv[(size_t)(pc + q) * rs + i] = sigma[i] * acc[q];
    }
  }
  (void)gi_n;
}

template <int B>
__device__ void vside_tile(const Seg& sg, int tile, const float* __restrict__ sigma, int in,
                           const int32_t* __restrict__ perm, int p0, int p1, const uint8_t* __restrict__ xf,
                           const uint32_t* __restrict__ xsc, const float* __restrict__ xsum,
                           float* __restrict__ tv, int rs) {
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, q = lane >> 4;
  const int gi_n = in / kGroup;
  const int li = tile * 16 + col;                 // local rank held by this lane (column)
  const bool rv = li < sg.n;
  const int np = (int)round_up(sg.n, 4);
  const uint32_t* row = reinterpret_cast<const uint32_t*>(sg.vc) + (size_t)(rv ? li : 0) * gi_n * 4 * B;
  const int fmt = B == 2 ? kFmtFp4 : kFmtFp6;
  const int bsc = B == 2 ? kScaleFp4Code : kScaleFp6Code;
  for (int pb = p0; pb < p1; pb += 64) {
    const int nt = min(64, p1 - pb);
    const int ntt = (nt + 15) >> 4;
    int arow[4];     // token (original index) of A row `col` in token tile tt, or -1
    int drow[4][4];  // token of D row 4q+r in token tile tt, or -1
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
      const int pa = pb + tt * 16 + col;
      arow[tt] = (tt < ntt && pa < p1) ? perm[pa] : -1;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int pd = pb + tt * 16 + 4 * q + r;
        drow[tt][r] = (tt < ntt && pd < p1) ? perm[pd] : -1;
      }
    }
    f32x4 acc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int gi = 0; gi < gi_n; ++gi) {
      v8i bop;
      if (B == 2) {
        const uint2 w = *reinterpret_cast<const uint2*>(row + (size_t)gi * 8 + 2 * q);
        bop = b_fp4(w.x, w.y);
      } else {
        const uint32_t* wp = row + (size_t)gi * 12 + 3 * q;
        bop = b_fp6(wp[0], wp[1], wp[2]);
      }
      if (!rv) bop = v8i{0, 0, 0, 0, 0, 0, 0, 0};
      const uint32_t e = rv ? sg.vs[(size_t)gi * np + li] : 0u;
      const float s = f16f(e & 0xFFFFu), z = f16f(e >> 16);
#pragma unroll
      for (int tt = 0; tt < 4; ++tt) {
        if (tt < ntt) {
          v8i ah = {0, 0, 0, 0, 0, 0, 0, 0}, al = {0, 0, 0, 0, 0, 0, 0, 0};
          int sh = 127;
          if (arow[tt] >= 0) {
            const size_t item = (size_t)arow[tt] * gi_n + gi;
            const int4* fp = reinterpret_cast<const int4*>(xf + item * kXFrag + q * 64);
            const int4 h0 = fp[0], h1 = fp[1], l0 = fp[2], l1 = fp[3];
            ah = v8i{h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
            al = v8i{l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
            sh = (int)((xsc[item] >> (8 * q)) & 0xFFu);
          }
          f32x4 d = {0.f, 0.f, 0.f, 0.f};
          d = mma(ah, bop, d, sh, fmt, bsc);
          d = mma(al, bop, d, sh - 5, fmt, bsc);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int tk = drow[tt][r];
            const float X = tk >= 0 ? xsum[(size_t)tk * gi_n + gi] : 0.f;
            acc[tt][r] += s * (d[r] - z * X);
          }
        }
      }
    }
    if (rv) {
      const float sig = sigma[sg.lo + li];
#pragma unroll
      for (int tt = 0; tt < 4; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pd = pb + tt * 16 + 4 * q + r;
          if (tt < ntt && pd < p1) tv[(size_t)pd * rs + sg.lo + li] = sig * acc[tt][r];
        }
    }
  }
}

__global__ void __launch_bounds__(256) k_vside(TenantTable tt, int32_t out, int32_t in,
                                               const uint16_t* __restrict__ x, const int32_t* __restrict__ offs,
                                               const int32_t* __restrict__ perm, const uint8_t* __restrict__ xf,
                                               const uint32_t* __restrict__ xsc, const float* __restrict__ xsum,
                                               float* __restrict__ tv, int32_t rs) {
  const int k = blockIdx.y;
  const int p0 = offs[k], p1 = offs[k + 1];
  if (p0 >= p1) return;
  const Tenant tn = tt.t[k];
  Layout L;
  layout_of(out, in, tn.n8, tn.n3, tn.n2, &L);
  int task = blockIdx.x;
  if (tn.n8 > 0) {
    if (task == 0) { vside_8bit(tn, L, in, x, perm, p0, p1, tv, rs); return; }
    --task;
  }
  const float* sigma = reinterpret_cast<const float*>(tn.base + L.off[DC_REG_SIGMA]);
  const int wave = threadIdx.x >> 6;
  const int t3 = (tn.n3 + 15) / 16, t2 = (tn.n2 + 15) / 16;
  const int k3 = (t3 + 3) / 4, k2 = (t2 + 3) / 4;
  if (task < k3) {
    const int tile = task * 4 + wave;
    if (tile < t3) vside_tile<3>(seg_of(tn, L, 1), tile, sigma, in, perm, p0, p1, xf, xsc, xsum, tv, rs);
  } else if (task < k3 + k2) {
    const int tile = (task - k3) * 4 + wave;
    if (tile < t2) vside_tile<2>(seg_of(tn, L, 2), tile, sigma, in, perm, p0, p1, xf, xsc, xsum, tv, rs);
  }
}

// ------------------------------------------------------------------ U side
// blockIdx.x = 128-row output group g, blockIdx.y = tenant (n = the
// backbone-only bucket).  Wave w owns rows 32w..32w+31 of the group (two
// 16-row tiles).  Per 128-rank chunk the block builds the A fragments of
// t'_i = s_ig t_i (three fp8 pieces) in LDS; y = sum_i q_oi t'_i
// - sum_i z_ig t'_i + (8-bit pairs) + W x, rounded once to bf16.
struct UsideLds {
  uint8_t frag[3][4][16][32];   // [piece][lane group][token row][byte]
  uint8_t sc[16][4];            // E8M0 of piece 0 per (token row, K-block)
  float cz[16][16];             // partial sum_i z t' per (token row, thread slot)
};

__global__ void __launch_bounds__(256) k_uside(TenantTable tt, int32_t n, int32_t out, int32_t in,
                                               const int32_t* __restrict__ offs, const int32_t* __restrict__ perm,
                                               const float* __restrict__ tv, int32_t rs,
                                               const float* __restrict__ ybase, uint16_t* __restrict__ y) {
  const int g = blockIdx.x, k = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, q = lane >> 4;
  const int p0 = offs[k], p1 = offs[k + 1];
  if (p0 >= p1) return;
  if (k == n) {  // backbone-only tokens
    for (int idx = tid; idx < (p1 - p0) * kGroup; idx += 256) {
      const int t = perm[p0 + idx / kGroup];
      const int o = g * kGroup + idx % kGroup;
      y[(size_t)t * out + o] = to_bf16(ybase ? ybase[(size_t)t * out + o] : 0.f);
    }
    return;
  }
  const Tenant tn = tt.t[k];
  Layout L;
  layout_of(out, in, tn.n8, tn.n3, tn.n2, &L);
  __shared__ UsideLds S;
  // A-prep thread role: token row ai = tid/16, K-block kb4 = (tid/4)%4, part = tid%4 (8 ranks)
  const int ai = tid >> 4, kb4 = (tid >> 2) & 3, part = tid & 3;
  for (int pb = p0; pb < p1; pb += 16) {
    const int nt = min(16, p1 - pb);
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    float czp = 0.f;   // this thread's share of sum_i z t' for token row ai
    for (int which = 1; which <= 2; ++which) {
      const Seg sg = seg_of(tn, L, which);
      if (sg.n == 0) continue;
      const int np = (int)round_up(sg.n, 4);
      const int kbn = (sg.n + kKBlock - 1) / kKBlock;
      const int fmt = sg.b == 2 ? kFmtFp4 : kFmtFp6;
      const int bsc = sg.b == 2 ? kScaleFp4Code : kScaleFp6Code;
      for (int c = 0; c < (kbn + 3) / 4; ++c) {
        __syncthreads();
        {  // A-prep: 8 ranks of K-block (4c + kb4) for token row ai
          const int m0 = kb4 * 32 + part * 8;              // rank offset inside the 128-rank chunk
          float tp[8];
          float mx = 0.f;
          const bool tok_ok = ai < nt;
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const int li = c * 128 + m0 + u;
            float v = 0.f;
            if (tok_ok && li < sg.n) {
              const uint32_t e = sg.us[(size_t)g * np + li];
              v = f16f(e & 0xFFFFu) * tv[(size_t)(pb + ai) * rs + sg.lo + li];
            }
            tp[u] = v;
            mx = fmaxf(mx, fabsf(v));
          }
          mx = fmaxf(mx, __shfl_xor(mx, 1, 64));
          mx = fmaxf(mx, __shfl_xor(mx, 2, 64));
          const int sb = block_scale_byte(mx);
          const float inv = pow2f(127 - sb), fwd = pow2f(sb - 127);
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            const float v = tp[u] * inv;
            const uint32_t h0 = fp8_of(v);
            const float r1 = (v - fp8_val(h0)) * 32.f;
            const uint32_t h1 = fp8_of(r1);
            const float r2 = (r1 - fp8_val(h1)) * 32.f;
            const uint32_t h2 = fp8_of(r2);
            const float back = (fp8_val(h0) + (fp8_val(h1) + fp8_val(h2) * (1.f / 32.f)) * (1.f / 32.f)) * fwd;
            const int li = c * 128 + m0 + u;
            if (li < sg.n && ai < nt) {
              const uint32_t e = sg.us[(size_t)g * np + li];
              czp += f16f(e >> 16) * back;
            }
            int ag, ae;
            a_pos(m0 + u, ag, ae);
            S.frag[0][ag][ai][ae] = (uint8_t)h0;
            S.frag[1][ag][ai][ae] = (uint8_t)h1;
            S.frag[2][ag][ai][ae] = (uint8_t)h2;
          }
          if (part == 0) S.sc[ai][kb4] = (uint8_t)sb;
        }
        __syncthreads();
        // A operand: token row col, lane group q
        const int4* f0 = reinterpret_cast<const int4*>(&S.frag[0][q][col][0]);
        const int4* f1 = reinterpret_cast<const int4*>(&S.frag[1][q][col][0]);
        const int4* f2 = reinterpret_cast<const int4*>(&S.frag[2][q][col][0]);
        const v8i a0 = {f0[0].x, f0[0].y, f0[0].z, f0[0].w, f0[1].x, f0[1].y, f0[1].z, f0[1].w};
        const v8i a1 = {f1[0].x, f1[0].y, f1[0].z, f1[0].w, f1[1].x, f1[1].y, f1[1].z, f1[1].w};
        const v8i a2 = {f2[0].x, f2[0].y, f2[0].z, f2[0].w, f2[1].x, f2[1].y, f2[1].z, f2[1].w};
        const int s0 = S.sc[col][q];
        const int kb = 4 * c + q;
        const uint32_t* ucw = reinterpret_cast<const uint32_t*>(sg.uc);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int o = g * kGroup + wave * 32 + h * 16 + col;   // output row of this lane's B column
          v8i bop = {0, 0, 0, 0, 0, 0, 0, 0};
          if (kb < kbn) {
            int nw;
            const uint32_t* wp = ucw + u_kblock_word(o, kb, sg.n, sg.b, &nw);
            uint32_t w[3] = {0u, 0u, 0u};
            for (int i = 0; i < nw; ++i) w[i] = wp[i];
            bop = sg.b == 2 ? b_fp4(w[0], w[1]) : b_fp6(w[0], w[1], w[2]);
          }
          f32x4 d = {0.f, 0.f, 0.f, 0.f};
          d = mma(a0, bop, d, s0, fmt, bsc);
          d = mma(a1, bop, d, s0 - 5, fmt, bsc);
          d = mma(a2, bop, d, s0 - 10, fmt, bsc);
          acc[h] += d;
        }
      }
    }
    // sum_i z t' per token row: reduce the 16 thread slots of each row
    __syncthreads();
    S.cz[ai][tid & 15] = czp;
    __syncthreads();
    // 8-bit pairs on the vector ALU, then the epilogue.  Lane: column o, token rows 4q+r.
    const Seg s8 = seg_of(tn, L, 0);
    const int np8 = (int)round_up(s8.n, 4);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int o = g * kGroup + wave * 32 + h * 16 + col;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 4 * q + r;
        if (row >= nt) continue;
        float v = acc[h][r];
        float cz = 0.f;
        for (int u = 0; u < 16; ++u) cz += S.cz[row][u];
        v -= cz;
        for (int i = 0; i < s8.n; ++i) {
          const uint32_t e = s8.us[(size_t)g * np8 + i];
          const float uh = (float)(_Float16)(f16f(e & 0xFFFFu) * ((float)s8.uc[(size_t)o * s8.n + i] - f16f(e >> 16)));
          v += uh * tv[(size_t)(pb + row) * rs + i];
        }
        const int t = perm[pb + row];
        if (ybase) v += ybase[(size_t)t * out + o];
        y[(size_t)t * out + o] = to_bf16(v);
      }
    }
    __syncthreads();   // S.cz is rewritten by the next token tile
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
  const size_t items = (size_t)a.T * (a.in / kGroup);
  uint8_t* xf = a.ws + a.wl.xf;
  uint32_t* xsc = reinterpret_cast<uint32_t*>(a.ws + a.wl.xsc);
  float* xsum = reinterpret_cast<float*>(a.ws + a.wl.xsum);
  SegArg seg{};
  if (a.mode == 2)
    for (int k = 0; k <= a.n; ++k) seg.v[k] = a.seg[k];
  auto mark = [&](int s) {
    if (a.events && a.events[s]) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(a.events[s]), st);
  };
  mark(DC_STAGE_ROUTE);
  mark(DC_STAGE_XPREP);
  hipLaunchKernelGGL(k_prep, dim3((unsigned)(1 + (items + 3) / 4)), dim3(256), 0, st, a.x, a.ids, a.T, a.in, a.n,
                     a.mode, seg, offs, perm, flags, xf, xsc, xsum);
  mark(DC_STAGE_BASE);
  if (a.W) launch_base(a.W, a.x, ybase, a.out, a.in, a.T, a.stream);
  mark(DC_STAGE_VSIDE);
  int tasks = 0;
  for (int k = 0; k < a.n; ++k) {
    const Tenant& t = a.tenants->t[k];
    const int k3 = ((t.n3 + 15) / 16 + 3) / 4, k2 = ((t.n2 + 15) / 16 + 3) / 4;
    const int nt = (t.n8 > 0 ? 1 : 0) + k3 + k2;
    tasks = nt > tasks ? nt : tasks;
  }
  if (tasks > 0)
    hipLaunchKernelGGL(k_vside, dim3((unsigned)tasks, (unsigned)a.n), dim3(256), 0, st, *a.tenants, a.out, a.in, a.x,
                       offs, perm, xf, xsc, xsum, tv, a.wl.rs);
  mark(DC_STAGE_USIDE);
  hipLaunchKernelGGL(k_uside, dim3((unsigned)(a.out / kGroup), (unsigned)(a.n + 1)), dim3(256), 0, st, *a.tenants,
                     a.n, a.out, a.in, offs, perm, tv, a.wl.rs, ybase, a.y);
  mark(DC_STAGE_COUNT);
  return (int)hipGetLastError();
}

}  // namespace dc
