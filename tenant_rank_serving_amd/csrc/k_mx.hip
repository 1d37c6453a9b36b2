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
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kFmtFp8 = 0, kFmtFp6 = 2, kFmtFp4 = 4;
constexpr int kScaleFp4Code = 128;   // 2^1: fp4 element q/2 -> q
constexpr int kScaleFp6Code = 130;   // 2^3: fp6 element q/8 -> q
constexpr int kXFrag = 256;          // bytes of x fragments per (token, 128-group)
constexpr int kBufFlags = 0x00020000; // buffer resource word 3: raw 32-bit dwords, bounds-checked

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
__device__ __forceinline__ void hold(f32x4& d, const v8i& a, const v8i& b, int s0, int sb) {
  asm volatile("" : "+v"(d) : "v"(a), "v"(b), "v"(s0), "v"(sb));
}
__device__ __forceinline__ void hold(f32x4& d, const v8i& a0, const v8i& a1, const v8i& b, int s0, int s1, int sb) {
  asm volatile("" : "+v"(d) : "v"(a0), "v"(a1), "v"(b), "v"(s0), "v"(s1), "v"(sb));
}
__device__ __forceinline__ void hold(f32x4& d, const v8i& a0, const v8i& a1, const v8i& a2, const v8i& b, int s0,
                                     int s1, int s2, int sb) {
  asm volatile("" : "+v"(d) : "v"(a0), "v"(a1), "v"(a2), "v"(b), "v"(s0), "v"(s1), "v"(s2), "v"(sb));
}

// v from lane l ^ X (X < 32) by ds_swizzle: no lane-address register, unlike
// a general shuffle.
template <int X>
__device__ __forceinline__ float swz_xor(float v) {
  static_assert(X > 0 && X < 32, "swizzle lanes stay within 32-lane halves");
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (X << 10) | 0x1F));
}

// Workgroup barrier that orders LDS only: unlike __syncthreads() it does not
// wait for the wave's global loads and stores in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ v8i v8_of(const uint4& a, const uint4& b) {
  return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
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
// the backbone-only tokens) and lists the buckets that have tokens, each with
// its tenant record and routed range, so that the V and U blocks of buckets
// with tokens come first in their grids and find everything they need in one
// load.  Its barriers order LDS only: they do not wait for its global
// stores, which only later kernels read.  Every other wave turns one (token,
// 128-group) of x into fp8 hi/lo A fragments, their E8M0 scales and the
// group sum; the other blocks also zero t and, when the backbone product is
// split over K, W x (both are accumulated with float atomics).
__device__ __forceinline__ void list_active(const Tenant& mine, int32_t n, const int* so,
                                            ActEntry* __restrict__ act) {
  __shared__ int wcnt[4];
  const int tid = threadIdx.x, b = tid, lane = tid & 63, wave = tid >> 6;
  const bool live = b <= n && so[b + 1] > so[b];
  const uint64_t m = __ballot(live);
  if (lane == 0) wcnt[wave] = __popcll(m);
  lds_barrier();
  int pos = __popcll(m & ((1ull << lane) - 1)), total = 0;
  for (int w = 0; w < 4; ++w) {
    if (w < wave) pos += wcnt[w];
    total += wcnt[w];
  }
  if (live) {
    ActEntry e;
    e.base = b < n ? mine.base : nullptr;
    e.n8 = b < n ? mine.n8 : 0;
    e.n3 = b < n ? mine.n3 : 0;
    e.n2 = b < n ? mine.n2 : 0;
    e.k = b;
    e.p0 = so[b];
    e.p1 = so[b + 1];
    act[pos] = e;
  }
  if (b <= n && b >= total) {   // the rest of the list: empty entries
    ActEntry e{};
    e.k = -1;
    act[b] = e;
  }
}

__global__ void __launch_bounds__(256) k_prep(TenantTable tt, const uint16_t* __restrict__ x,
                                              const int32_t* __restrict__ ids,
                                              int32_t T, int32_t in, int32_t n, int32_t mode, SegArg seg,
                                              int32_t* __restrict__ offs, int32_t* __restrict__ perm,
                                              ActEntry* __restrict__ act,
                                              uint32_t* __restrict__ flags, uint8_t* __restrict__ xf,
                                              uint32_t* __restrict__ xsc, float* __restrict__ xsum,
                                              uint16_t* __restrict__ xt, float* __restrict__ tv, int32_t ntv,
                                              float* __restrict__ yb, int32_t nyb) {
  const int tid = threadIdx.x;
  // t accumulates atomically: zeroed by the blocks after the first (the
  // first block's barriers would wait for its stores to finish)
  if (blockIdx.x > 0) {
    for (int i = (blockIdx.x - 1) * 256 + tid; i < ntv; i += (gridDim.x - 1) * 256) tv[i] = 0.f;
    for (int i = (blockIdx.x - 1) * 256 + tid; i < nyb; i += (gridDim.x - 1) * 256) yb[i] = 0.f;   // W x, when split over K
  }
  if (blockIdx.x == 0) {
    static_assert(DC_MAX_TENANTS + 1 <= 256, "one thread per bucket");
    __shared__ int so[DC_MAX_TENANTS + 2];   // bucket starts
    // thread b's tenant record, read first: the kernel arguments live in
    // memory and the indexing is per thread
    Tenant mine{};
    if (tid < n) mine = tt.t[tid];
    if (mode != 1) {
      for (int p = tid; p < T; p += blockDim.x) perm[p] = p;
      if (tid == 0) {
        if (mode == 0) { so[0] = 0; so[1] = T; so[2] = T; }
        else { for (int k = 0; k <= n; ++k) so[k] = seg.v[k]; so[n + 1] = T; }
        for (int k = 0; k <= n + 1; ++k) offs[k] = so[k];
        *flags = 0;
      }
      lds_barrier();
      list_active(mine, n, so, act);
      return;
    }
    __shared__ int cnt[DC_MAX_TENANTS + 1];   // tokens per bucket
    __shared__ int next[DC_MAX_TENANTS + 1];
    __shared__ __attribute__((aligned(16))) int bkt[256];
    __shared__ int bad;
    __shared__ int wsum[4];
    for (int b = tid; b <= n; b += blockDim.x) cnt[b] = 0;
    if (tid == 0) bad = 0;
    lds_barrier();
    int b0 = -1;   // bucket of token tid (the first chunk is kept for the placement below)
    for (int t = tid; t < T; t += blockDim.x) {
      int k = ids[t];
      if (k < -1 || k >= n) { bad = 1; k = -1; }
      const int b = k < 0 ? n : k;
      if (t == tid) b0 = b;
      atomicAdd(&cnt[b], 1);
    }
    lds_barrier();
    {  // exclusive scan of the bucket counts, one thread per bucket
      const int lane = tid & 63, wv = tid >> 6;
      const int c = tid <= n ? cnt[tid] : 0;
      int v = c;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int u = __shfl_up(v, d, 64);
        if (lane >= d) v += u;
      }
      if (lane == 63) wsum[wv] = v;
      lds_barrier();
      for (int w = 0; w < wv; ++w) v += wsum[w];
      if (tid <= n) {
        offs[tid] = v - c;
        so[tid] = v - c;
        next[tid] = v - c;
      }
      if (tid == n) {
        offs[n + 1] = v;
        so[n + 1] = v;
      }
      if (tid == 0) *flags = bad ? 1u : 0u;
    }
    lds_barrier();
    list_active(mine, n, so, act);
    for (int c0 = 0; c0 < T; c0 += blockDim.x) {
      const int t = c0 + tid;
      int b = -1;
      if (t < T) {
        if (c0 == 0) {
          b = b0;
        } else {
          const int k = ids[t];
          b = (k < 0 || k >= n) ? n : k;
        }
      }
      bkt[tid] = b;
      lds_barrier();
      if (t < T) {   // rank among the chunk's earlier tokens of its bucket: four per LDS read
        int rank = 0;
        const int4* b4 = reinterpret_cast<const int4*>(bkt);
#pragma unroll 4
        for (int j4 = 0; j4 < (tid >> 2); ++j4) {
          const int4 v = b4[j4];
          rank += (v.x == b) + (v.y == b) + (v.z == b) + (v.w == b);
        }
        for (int j = tid & ~3; j < tid; ++j) rank += (bkt[j] == b);
        perm[next[b] + rank] = t;
      }
      lds_barrier();
      if (t < T) atomicAdd(&next[b], 1);
      lds_barrier();
    }
    return;
  }
  const int gi_n = in / kGroup;
  const size_t item = (size_t)(blockIdx.x - 1) * 4 + (tid >> 6);
  if (item >= (size_t)T * gi_n) return;
  const int lane = tid & 63;
  const int t = (int)(item / gi_n), gi = (int)(item % gi_n);
  // sorted position of token t, as block 0 routes it (bucket, then token
  // order): the fragments, scales and sums are stored in that order
  int ps = t;
  if (mode == 1) {
    auto bucket = [&](int u) { const int kk = ids[u]; return (kk < 0 || kk >= n) ? n : kk; };
    const int bt = bucket(t);
    ps = 0;
    for (int c0 = 0; c0 < T; c0 += 64) {
      const int u = c0 + lane;
      bool before = false;
      if (u < T) {
        const int b = bucket(u);
        before = b < bt || (b == bt && u < t);
      }
      ps += __popcll(__ballot(before));
    }
  }
  const size_t sitem = (size_t)ps * gi_n + gi;
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
  uint8_t* fr = xf + sitem * kXFrag;
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
    xsc[sitem] = (uint32_t)b0 | ((uint32_t)c1 << 8) | ((uint32_t)b1 << 16) | ((uint32_t)c3 << 24);
    xsum[sitem] = s;
  }
}

// ------------------------------------------------------------------ V side
// Work item (block): tenant k = blockIdx.y; blockIdx.x = rank block rb *
// v_slices + input slice s.  Rank blocks: the 8-bit rows (vector ALU, fp16
// dequantized weights), then blocks of kVRanks ranks of the 3-bit and of the
// 2-bit segment on the matrix cores: wave w takes kVTiles 16-rank tiles, all
// waves the same kVSlice input groups.  Tokens go in passes of kVRows; per
// pass the block stages the x fragments of its slice into LDS once and every
// wave reads them as the A operand (rows 0-7 the hi pieces, rows 8-15 the lo
// pieces of the pass's tokens).  A wave's codes stream through a register
// ring kVDepth groups deep: the loads of group u + kVDepth go out before the
// matrix-core ops of group u (a later pass reloads them, from L2).  The
// kVTiles ops of a group share one A operand and are independent.  sigma * (partial V x)
// is added into t with float atomics; t is zeroed by the prep kernel.
struct VLds {
  int4 frag[kVSlice][kVRows][17];     // [group][token row][lane group * 4 + (hi0 hi1 lo0 lo1)], padded row
  uint32_t sc[kVSlice][kVRows];       // E8M0 words of the hi pieces
  float xs[kVSlice][kVRows];          // group sums of x
};

typedef int i32x4 __attribute__((ext_vector_type(4)));
struct U3 {
  uint32_t a, b, c;
};

// One group of one lane's codes (B words per tile) and its scale/zero words.
template <int B>
struct VGrp {
  uint32_t w[kVTiles][B];
  uint32_t z[kVTiles];
};

// Buffer resources of a segment's V codes and scale/zero words, and per tile
// the byte offset of the lane's word block (codes, 16-rank tile-major: one
// wave load reads 64 consecutive blocks) and of its rank's scale/zero column
// (rank 0 of the segment for ranks past its end); the group goes into the
// uniform offset.
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x3 __attribute__((ext_vector_type(3)));
struct VBuf {
  __amdgpu_buffer_rsrc_t rc, rz;
  uint32_t oc[kVTiles], oz[kVTiles];
};

template <int B>
__device__ __forceinline__ void v_load_grp(VGrp<B>& c, const VBuf& p, int np, int gi) {
#pragma unroll
  for (int h = 0; h < kVTiles; ++h) {
    if constexpr (B == 2) {
      const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(p.rc, p.oc[h], gi * 64 * B * 4, 0);
      c.w[h][0] = v.x;
      c.w[h][1] = v.y;
    } else {
      const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(p.rc, p.oc[h], gi * 64 * B * 4, 0);
      c.w[h][0] = v.x;
      c.w[h][1] = v.y;
      c.w[h][2] = v.z;
    }
    c.z[h] = __builtin_amdgcn_raw_buffer_load_b32(p.rz, p.oz[h], gi * np * 4, 0);
  }
}

// x fragments, scale words and group sums of sorted rows [pb, pb + kVRows)
// for groups [g0, g0 + kVSlice), staged into LDS in two steps so that the
// loads can go out ahead of the code ring.  Thread tid moves int4 (tid & 15)
// of the fragment of row (tid >> 4) & 7 for groups (tid >> 7) + 2u; threads
// < 128 move the scale word and group sum of row tid & 7 and group
// (tid >> 3) & 15.  Rows past the pass repeat its last row and are never
// read; groups past the input repeat its last group.
struct VStage {
  i32x4 v[kVSlice / 2];
  uint32_t scw;
  float xsv;
};

__device__ __forceinline__ void v_stage_load(VStage& st, const uint8_t* __restrict__ xf,
                                             const uint32_t* __restrict__ xsc, const float* __restrict__ xsum,
                                             int gi_n, int g0, int pb, int nt) {
  const int tid = threadIdx.x;
  const int k16 = tid & 15, rw = (tid >> 4) & 7, gh = tid >> 7;
  const size_t row = (size_t)(pb + min(rw, nt - 1)) * gi_n;
#pragma unroll
  for (int u = 0; u < kVSlice / 2; ++u) {
    const int gi = min(g0 + gh + 2 * u, gi_n - 1);
    st.v[u] = reinterpret_cast<const i32x4*>(xf + (row + gi) * kXFrag)[k16];
  }
  const int sr = tid & 7, sgl = (tid >> 3) & (kVSlice - 1);
  const size_t srow = (size_t)(pb + min(sr, nt - 1)) * gi_n + min(g0 + sgl, gi_n - 1);
  st.scw = xsc[srow];
  st.xsv = xsum[srow];
}

__device__ __forceinline__ void v_stage_store(VLds& S, const VStage& st) {
  const int tid = threadIdx.x;
  const int k16 = tid & 15, rw = (tid >> 4) & 7, gh = tid >> 7;
#pragma unroll
  for (int u = 0; u < kVSlice / 2; ++u)
    S.frag[gh + 2 * u][rw][k16] = make_int4(st.v[u].x, st.v[u].y, st.v[u].z, st.v[u].w);
  if (tid < kVRows * kVSlice) {
    const int sr = tid & 7, sgl = (tid >> 3) & (kVSlice - 1);
    S.sc[sgl][sr] = st.scw;
    S.xs[sgl][sr] = st.xsv;
  }
}

__device__ __forceinline__ void hold2(f32x4& d0, f32x4& d1, const v8i& a, const v8i& b0, const v8i& b1, int sa,
                                      int sb) {
  asm volatile("" : "+v"(d0), "+v"(d1) : "v"(a), "v"(b0), "v"(b1), "v"(sa), "v"(sb));
}

// kVTiles 16-rank tiles of one wave (starting at tile0 of the segment) over
// one input slice, all tokens; the block's other waves run the same slice.
// live_wave: any of the wave's tiles holds a rank of the segment.
template <int B>
__device__ void vside_blk(const Seg& sg, int tbase, int tile0, bool live_wave, int in, int s,
                          const int32_t* __restrict__ perm, int p0, int p1, const uint8_t* __restrict__ xf,
                          const uint32_t* __restrict__ xsc, const float* __restrict__ xsum,
                          const float* __restrict__ sigma, float* __restrict__ tv, int rs, VLds& S) {
  static_assert(kVTiles == 2, "hold2 covers two tiles");
  constexpr int fmt = B == 2 ? kFmtFp4 : kFmtFp6;
  constexpr int bsc = B == 2 ? kScaleFp4Code : kScaleFp6Code;
  constexpr int kDepth = B == 2 ? kVDepth : kVDepth / 2;   // ring depth in groups (3-bit groups are larger)
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, q = lane >> 4;
  const int gi_n = in / kGroup;
  const int g0 = s * kVSlice;
  const int gn = min(kVSlice, gi_n - g0);   // groups in this slice
  const int glast = g0 + gn - 1;
  const int np = (int)round_up(sg.n, 4);
  const int npass = (p1 - p0 + kVRows - 1) / kVRows;
  VBuf P;
  P.rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(sg.vc), 0, (int)round_up(sg.n, 16) * gi_n * 16 * B,
                                          kBufFlags);
  P.rz = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint32_t*>(sg.vs), 0, gi_n * np * 4, kBufFlags);
  int li[kVTiles];
  bool rv[kVTiles];
  float sig[kVTiles];
#pragma unroll
  for (int h = 0; h < kVTiles; ++h) {
    li[h] = (tile0 + h) * 16 + col;
    rv[h] = li[h] < sg.n;
    // tile-major codes: lane (col, q) of tile t reads the b words of block
    // (t, group, q, col), i.e. lane * b words into the tile's group block
    P.oc[h] = (uint32_t)(((tile0 + h) * gi_n * 64 + lane) * 4 * B);
    P.oz[h] = (uint32_t)(4 * (rv[h] ? li[h] : 0));
    sig[h] = rv[h] ? sigma[sg.lo + li[h]] : 0.f;
  }
  const int tr = col & 7;              // token row of this lane's A operand
  const int piece = col >> 3;          // 0: hi pieces, 1: lo pieces
  for (int ip = 0; ip < npass; ++ip) {
    const int pb = p0 + ip * kVRows;
    const int nt = min(kVRows, p1 - pb);
    VStage st;
    v_stage_load(st, xf, xsc, xsum, gi_n, g0, pb, nt);   // ahead of the ring: vmcnt is in order
    VGrp<B> ring[kDepth] = {};   // defined on every path: no values carried across passes
    if (live_wave) {
#pragma unroll
      for (int d = 0; d < kDepth; ++d) v_load_grp<B>(ring[d], P, np, min(g0 + d, glast));
    }
    __syncthreads();   // LDS reuse across passes
    v_stage_store(S, st);
    __syncthreads();
    if (!live_wave) continue;
    const bool live = tr < nt;
    f32x4 acc[kVTiles];
#pragma unroll
    for (int h = 0; h < kVTiles; ++h) acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < kVSlice; ++u) {
      const VGrp<B> c = ring[u % kDepth];
      if (u + kDepth < kVSlice)   // refill the slot with group u + kDepth (resolved at compile time)
        v_load_grp<B>(ring[u % kDepth], P, np, min(g0 + u + kDepth, glast));
      const int4* fr = S.frag[u][tr] + 4 * q + 2 * piece;
      const int4 f0 = fr[0], f1 = fr[1];
      const v8i a = live ? v8i{f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w} : v8i{0, 0, 0, 0, 0, 0, 0, 0};
      const int sa = live ? (int)((S.sc[u][tr] >> (8 * q)) & 0xFFu) - 5 * piece : 127;
      v8i bo[kVTiles];
      f32x4 d[kVTiles];
#pragma unroll
      for (int h = 0; h < kVTiles; ++h) {
        bo[h] = B == 2 ? b_fp4(c.w[h][0], c.w[h][1]) : b_fp6(c.w[h][0], c.w[h][1], c.w[h][2]);
        d[h] = mma(a, bo[h], f32x4{0.f, 0.f, 0.f, 0.f}, sa, fmt, bsc);
      }
      hold2(d[0], d[1], a, bo[0], bo[1], sa, bsc);
      // D rows 0-7 (lane groups 0, 1): hi products of tokens 0-7, which also
      // take the zero-point term; rows 8-15: lo products, added at the end.
      // Groups past the input (u >= gn) are clamped duplicates: scale 0.
      const bool gv = u < gn;
      float xsr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) xsr[r] = S.xs[u][(4 * q + r) & 7];
#pragma unroll
      for (int h = 0; h < kVTiles; ++h) {
        const float sc = gv ? f16f(c.z[h] & 0xFFFFu) : 0.f, z = q < 2 ? f16f(c.z[h] >> 16) : 0.f;
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[h][r] += sc * (d[h][r] - z * xsr[r]);
      }
      // the group's sums land in acc here: without this the compiler defers
      // them to the end of the pass and keeps every group's products live
      asm volatile("" : "+v"(acc[0]), "+v"(acc[1]));
    }
#pragma unroll
    for (int h = 0; h < kVTiles; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[h][r] += __shfl_xor(acc[h][r], 32, 64);
    if (q < 2) {
#pragma unroll
      for (int h = 0; h < kVTiles; ++h)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (rv[h] && 4 * q + r < nt) atomicAdd(tv + (size_t)(pb + 4 * q + r) * rs + tbase + li[h], sig[h] * acc[h][r]);
    }
  }
}

// 8-bit rows of a tenant over one input slice on the vector ALU with the fp16
// dequantized weights fp16(s (q - z)).  Thread tid owns 8 inputs of the
// slice, a pass's kVRows token rows and 4 rows at a time; the block sums per
// (row, token) and adds sigma * partial into t.
__device__ void vside_8bit(const Tenant& tn, const Layout& L, int in, int s, const uint16_t* __restrict__ x,
                           const int32_t* __restrict__ perm, int p0, int p1, float* __restrict__ tv, int rs) {
  __shared__ float red[4][4][kVRows];   // [wave][row][token row]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const Seg sg = seg_of(tn, L, 0);
  const float* sigma = reinterpret_cast<const float*>(tn.base + L.off[DC_REG_SIGMA]);
  const int np = (int)round_up(sg.n, 4);
  const int i0 = s * kVSlice * kGroup + 8 * tid;   // first input of this thread
  const bool ok = i0 < in;
  const int ic = ok ? i0 : 0;
  const int gi = ic / kGroup;
  for (int pb = p0; pb < p1; pb += kVRows) {
    const int nt = min(kVRows, p1 - pb);
    uint4 xv[kVRows];
#pragma unroll
    for (int t = 0; t < kVRows; ++t)
      xv[t] = *reinterpret_cast<const uint4*>(x + (size_t)perm[pb + min(t, nt - 1)] * in + ic);
    for (int r0 = 0; r0 < sg.n; r0 += 4) {
      uint2 cw[4];
      uint32_t e[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = min(r0 + u, sg.n - 1);
        cw[u] = *reinterpret_cast<const uint2*>(sg.vc + (size_t)i * in + ic);
        e[u] = sg.vs[(size_t)gi * np + i];
      }
      // partials of the live (row, token) pairs only: with two 8-bit rows and
      // a few tokens most of the 4 x kVRows pairs are padding
      const int nu = min(4, sg.n - r0);
      float part[4][kVRows];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (u >= nu) break;
        const float sc = f16f(e[u] & 0xFFFFu), z = f16f(e[u] >> 16);
        const uint32_t cwu[2] = {cw[u].x, cw[u].y};
        float w[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) w[j] = (float)(_Float16)(sc * ((float)((cwu[j >> 2] >> (8 * (j & 3))) & 0xFFu) - z));
#pragma unroll
        for (int t = 0; t < kVRows; ++t) {
          if (t >= nt) break;
          const uint32_t xw[4] = {xv[t].x, xv[t].y, xv[t].z, xv[t].w};
          float a = 0.f;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            a += w[2 * j] * __uint_as_float(xw[j] << 16) + w[2 * j + 1] * __uint_as_float(xw[j] & 0xFFFF0000u);
          part[u][t] = ok ? a : 0.f;
        }
      }
      // their wave sums
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int t = 0; t < kVRows; ++t) {
          if (u < nu && t < nt) {
            float v = part[u][t];
            v += swz_xor<1>(v);
            v += swz_xor<2>(v);
            v += swz_xor<4>(v);
            v += swz_xor<8>(v);
            v += swz_xor<16>(v);
            v += __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));   // lanes 32-63
            if (lane == 0) red[wave][u][t] = v;
          }
        }
      __syncthreads();
      if (tid < 4 * kVRows) {
        const int u = tid / kVRows, t = tid % kVRows;
        if (r0 + u < sg.n && t < nt)
          atomicAdd(tv + (size_t)(pb + t) * rs + r0 + u,
                    sigma[r0 + u] * ((red[0][u][t] + red[1][u][t]) + (red[2][u][t] + red[3][u][t])));
      }
      __syncthreads();
    }
  }
}

__global__ void __launch_bounds__(256) k_vside(int32_t n, int32_t out, int32_t in,
                                               const uint16_t* __restrict__ x, const ActEntry* __restrict__ act,
                                               const int32_t* __restrict__ perm, const uint8_t* __restrict__ xf,
                                               const uint32_t* __restrict__ xsc, const float* __restrict__ xsum,
                                               float* __restrict__ tv, int32_t rs) {
  const ActEntry e = act[blockIdx.y];   // the blockIdx.y-th bucket with tokens
  const int p0 = e.p0, p1 = e.p1;
  if (p0 >= p1 || e.k >= n) return;     // empty entry, or the backbone-only bucket
  Tenant tn;
  tn.base = e.base;
  tn.n8 = e.n8;
  tn.n3 = e.n3;
  tn.n2 = e.n2;
  tn.pad_ = 0;
  const int ns = v_slices(in);
  int b = blockIdx.x / ns;
  const int s = blockIdx.x % ns;
  if (b >= v_blocks(tn.n8, tn.n3, tn.n2)) return;
  Layout L;
  layout_of(out, in, tn.n8, tn.n3, tn.n2, &L);
  if (tn.n8 > 0) {
    if (b == 0) { vside_8bit(tn, L, in, s, x, perm, p0, p1, tv, rs); return; }
    --b;
  }
  __shared__ VLds S;
  const float* sigma = reinterpret_cast<const float*>(tn.base + L.off[DC_REG_SIGMA]);
  const int wave = threadIdx.x >> 6;
  const int b3 = (tn.n3 + kVRanks - 1) / kVRanks;
  const bool three = b < b3;
  const int tile0 = ((three ? b : b - b3) * 4 + wave) * kVTiles;
  const int sn = three ? tn.n3 : tn.n2;
  if (three)
    vside_blk<3>(seg_of(tn, L, 1), t_base(tn.n8, tn.n3, 1), tile0, tile0 * 16 < sn, in, s, perm, p0, p1, xf, xsc,
                 xsum, sigma, tv, rs, S);
  else
    vside_blk<2>(seg_of(tn, L, 2), t_base(tn.n8, tn.n3, 2), tile0, tile0 * 16 < sn, in, s, perm, p0, p1, xf, xsc,
                 xsum, sigma, tv, rs, S);
}

// ------------------------------------------------------------------ U side
// Work item (block of kUWaves waves): 128-row output group g = blockIdx.x
// (one scale group) of tenant k = blockIdx.y (n = the backbone-only bucket),
// all ranks, tokens in passes of up to kURows.  Wave w takes the 16-row tile
// 16w..16w+15.  The ranks go in 128-rank chunks, 3-bit chunks first.  Per
// pass, for a window of chunks at a time, the whole block first turns
// t'_i = s_ig t_i into three fp8 pieces with E8M0 block scales (thread:
// chunk, K-block, 4 ranks, four token rows) and writes them to LDS as A
// operands: token r, piece p goes to row (r % 4) + 4p of matrix-core op
// r / 4, so one op takes all three pieces of four tokens.  After one barrier
// every wave runs its tile over the window's chunks with no further
// synchronization, one op per four live tokens per chunk, the codes of the
// next kUDepth chunks in flight in a register ring (buffer loads on one
// resource for the tenant's whole buffer, the region in the uniform offset).
// The epilogue sums each token's three piece rows, takes sum_i z_ig t'_i
// off, adds the 8-bit pairs and W x and rounds once to bf16.
constexpr int kURows = 8;     // token rows per pass
constexpr int kUWaves = 8;    // waves per block, one 16-row tile each
constexpr int kU8Max = 2;     // 8-bit pairs whose U weights a lane keeps in registers
constexpr int kUDepth = 4;    // chunks of codes in flight per lane
constexpr int kUWin = 16;     // A operands per window (chunks x ops): 16 chunks with one op, 8 with two
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

struct ULds {
  uint16_t frag[kUWin][4][16][16];   // [chunk * ops + op][lane group][A row][32 bytes]
  uint8_t sc[kUWin][kURows][4];      // E8M0 of the hi piece per (chunk, token row, K-block)
  float cz[kUWaves][kURows];         // per-wave partial sums of z t' per token row
};

__global__ void __launch_bounds__(kUWaves * 64) k_uside(int32_t n, int32_t out, int32_t in,
                                                        const ActEntry* __restrict__ act,
                                                        const int32_t* __restrict__ perm,
                                                        const float* __restrict__ tv, int32_t rs, int32_t T,
                                                        const float* __restrict__ ybase,
                                                        uint16_t* __restrict__ y) {
  const int g = blockIdx.x;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, q = lane >> 4;
  const ActEntry e = act[blockIdx.y];   // the blockIdx.y-th bucket with tokens
  const int p0 = e.p0, p1 = e.p1;
  if (p0 >= p1) return;
  if (e.k == n) {  // backbone-only tokens
    for (int idx = tid; idx < (p1 - p0) * kGroup; idx += kUWaves * 64) {
      const int t = perm[p0 + idx / kGroup];
      const int o = g * kGroup + idx % kGroup;
      y[(size_t)t * out + o] = to_bf16(ybase ? ybase[(size_t)t * out + o] : 0.f);
    }
    return;
  }
  __shared__ ULds S;
  Tenant tn;
  tn.base = e.base;
  tn.n8 = e.n8;
  tn.n3 = e.n3;
  tn.n2 = e.n2;
  tn.pad_ = 0;
  Layout L;
  layout_of(out, in, tn.n8, tn.n3, tn.n2, &L);
  const Seg seg3 = seg_of(tn, L, 1), seg2 = seg_of(tn, L, 2), s8 = seg_of(tn, L, 0);
  const int tb3 = t_base(tn.n8, tn.n3, 1), tb2 = t_base(tn.n8, tn.n3, 2);
  const int np3 = (int)round_up(seg3.n, 4), np2 = (int)round_up(seg2.n, 4);
  const int nc3 = (seg3.n + 127) / 128, nc = nc3 + (seg2.n + 127) / 128;
  const int gn = out / kGroup;
  const int orow = g * kGroup + wave * 16 + col;
  const __amdgpu_buffer_rsrc_t rt =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(tv), 0, T * rs * 4, kBufFlags);
  // the tenant's whole packed buffer: code and scale regions go in the uniform offset
  const __amdgpu_buffer_rsrc_t rten =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(tn.base), 0, (int)L.total, kBufFlags);
  const int oc3 = (int)L.off[DC_REG_UC3], oc2 = (int)L.off[DC_REG_UC2];
  const int ou3 = (int)L.off[DC_REG_US3] + g * np3 * 4, ou2 = (int)L.off[DC_REG_US2] + g * np2 * 4;
  // the lane's byte offset of K-block kb of its row in the 3- or 2-bit code region
  const int rw3 = (int)u_row_words(seg3.n, 3), rw2 = (int)u_row_words(seg2.n, 2);
  const int kbn3 = (seg3.n + kKBlock - 1) / kKBlock, kbn2 = (seg2.n + kKBlock - 1) / kKBlock;
  auto load = [&](uint32_t (&w)[3], int c) __attribute__((always_inline)) {
    c = min(c, nc - 1);
    const bool three = c < nc3;
    const int b = three ? 3 : 2;
    const int kbn = three ? kbn3 : kbn2, rw = three ? rw3 : rw2;
    const int kb = min(4 * (three ? c : c - nc3) + q, kbn - 1);
    const int wl = rw - (kbn - 1) * b;   // words of the last K-block
    const int off = ((orow >> 4) * 16 * rw + kb * 16 * b + (orow & 15) * (kb == kbn - 1 ? wl : b)) * 4;
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rten, off, three ? oc3 : oc2, 0);
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
  };
  // fp16 dequantized 8-bit U weights of this lane's output row (first kU8Max
  // pairs); loaded behind the first window's A-prep inputs and codes
  float u8w[kU8Max];
  auto load_u8w = [&]() __attribute__((always_inline)) {
    const int np8 = (int)round_up(s8.n, 4);
#pragma unroll
    for (int i = 0; i < kU8Max; ++i) {
      const int ii = min(i, s8.n > 0 ? s8.n - 1 : 0);
      const uint32_t e = s8.n > 0 ? s8.us[(size_t)g * np8 + ii] : 0u;
      const float code = s8.n > 0 ? (float)s8.uc[(size_t)orow * s8.n + ii] : 0.f;
      u8w[i] = (float)(_Float16)(f16f(e & 0xFFFFu) * (code - f16f(e >> 16)));
    }
  };
  // rows 12-15 of every op carry no piece: zero once
  for (int i = tid; i < kUWin * 4 * 4; i += kUWaves * 64) {   // i = operand:4 lane group:2 row:2
    uint4* p = reinterpret_cast<uint4*>(S.frag[i >> 4][(i >> 2) & 3][12 + (i & 3)]);
    p[0] = make_uint4(0, 0, 0, 0);
    p[1] = make_uint4(0, 0, 0, 0);
  }
  // A-prep role: K-block kb4 and ranks m0..m0+3 of a chunk (which chunk and
  // rows depend on the pass: see aprep)
  const int kb4 = (tid >> 3) & 3, part = tid & 7;
  const int m0 = kb4 * 32 + part * 4;
  const int lg_even = 2 * (kb4 & 1), hw = (kb4 >= 2 ? 8 : 0) + part;   // lane group, 16-bit word
  const int ps = col >> 2, tr4 = col & 3;   // MFMA lane's A row: piece ps of token 4 op + tr4
  for (int pb = p0; pb < p1; pb += kURows) {
    const int nt = min(kURows, p1 - pb);
    const int nops = (nt + 3) >> 2;   // matrix-core ops per tile and chunk
    const int wcap = kUWin / nops;     // chunks per window (a multiple of kUDepth)
    uint32_t cr[kUDepth][3];
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    // A operands of chunks [cw0, cw0 + wc) for the pass's token rows.  Thread
    // tid takes chunk pcl of the window and rows 4h..4h+3: with one op per
    // chunk the 512 threads cover 16 chunks x rows 0-3, with two 8 chunks x
    // both halves.  The first window's loads go out ahead of the code ring's
    // first loads (vmcnt is in order: behind them they would wait for the
    // whole burst).
    const int pcl = nops == 1 ? tid >> 5 : (tid & 255) >> 5;
    const int hh = nops == 1 ? 0 : tid >> 8;
    auto aprep = [&](int cw0, int wc, bool first) __attribute__((always_inline)) {
      const int c = cw0 + pcl;
      const bool cok = pcl < wc;
      const bool three = c < nc3;
      const int sn = three ? seg3.n : seg2.n;
      const int li = (three ? c : c - nc3) * kGroup + m0;
      const u32x4 usw = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rten, li * 4, three ? ou3 : ou2, 0));
      f32x4 tt[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        tt[r] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rt, ((pb + min(4 * hh + r, nt - 1)) * rs + (three ? tb3 : tb2) + li) * 4, 0, 0));
      if (first) {
#pragma unroll
        for (int d = 0; d < kUDepth; ++d) load(cr[d], d);
        if (pb == p0) load_u8w();
      }
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int r = 4 * hh + r4;
        if (r >= nt) break;   // rows past the pass's tokens: their D rows are never read
        float tp[4];
        float mx = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bool ok = cok && li + u < sn;
          tp[u] = ok ? f16f(usw[u] & 0xFFFFu) * tt[r4][u] : 0.f;
          mx = fmaxf(mx, fabsf(tp[u]));
        }
        mx = fmaxf(mx, swz_xor<1>(mx));
        mx = fmaxf(mx, swz_xor<2>(mx));
        mx = fmaxf(mx, swz_xor<4>(mx));
        const int sb = block_scale_byte(mx);
        const float inv = pow2f(127 - sb), fwd = pow2f(sb - 127);
        // three fp8 pieces, two values per conversion: the low half of word w[pc]
        // holds ranks u = 0, 2 (even lane group), the high half ranks 1, 3
        float rr[4] = {tp[0] * inv, tp[1] * inv, tp[2] * inv, tp[3] * inv};
        float bk[4] = {0.f, 0.f, 0.f, 0.f};
        uint32_t w[3];
        float sc_pc = 1.f;
#pragma unroll
        for (int pc = 0; pc < 3; ++pc) {
          int ww = __builtin_amdgcn_cvt_pk_fp8_f32(rr[0], rr[2], 0, false);
          ww = __builtin_amdgcn_cvt_pk_fp8_f32(rr[1], rr[3], ww, true);
          w[pc] = (uint32_t)ww;
          const f32x2 e02 = __builtin_amdgcn_cvt_pk_f32_fp8(ww, false), e13 = __builtin_amdgcn_cvt_pk_f32_fp8(ww, true);
          bk[0] += e02.x * sc_pc; bk[2] += e02.y * sc_pc; bk[1] += e13.x * sc_pc; bk[3] += e13.y * sc_pc;
          rr[0] = (rr[0] - e02.x) * 32.f; rr[2] = (rr[2] - e02.y) * 32.f;
          rr[1] = (rr[1] - e13.x) * 32.f; rr[3] = (rr[3] - e13.y) * 32.f;
          sc_pc *= 1.f / 32.f;
        }
        float cz = 0.f;   // sum over the thread's ranks of z t' (zero for masked ranks and rows)
#pragma unroll
        for (int u = 0; u < 4; ++u) cz += f16f(usw[u] >> 16) * (bk[u] * fwd);
        cz += swz_xor<1>(cz);
        cz += swz_xor<2>(cz);
        cz += swz_xor<4>(cz);
        cz += swz_xor<8>(cz);
        cz += swz_xor<16>(cz);
        const float cz_hi = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cz), 32));   // lanes 32-63
        if (lane == 0) S.cz[wave][r] += cz + cz_hi;
        if (cok) {
          const int fi = pcl * nops + hh;
#pragma unroll
          for (int pc = 0; pc < 3; ++pc) {
            S.frag[fi][lg_even][r4 + 4 * pc][hw] = (uint16_t)w[pc];
            S.frag[fi][lg_even + 1][r4 + 4 * pc][hw] = (uint16_t)(w[pc] >> 16);
          }
          if (part == 0) S.sc[pcl][r][kb4] = (uint8_t)sb;
        }
        __builtin_amdgcn_sched_barrier(0);   // one token row at a time: bounded register use
      }
    };
    // chunk c (window-local cl): matrix-core ops with the codes in cur, then
    // the loads of chunk c + kUDepth into cur
    auto step = [&](int c, int cl, uint32_t (&cur)[3]) __attribute__((always_inline)) {
      const bool three = c < nc3;
      const v8i bop = three ? b_fp6(cur[0], cur[1], cur[2]) : b_fp4(cur[0], cur[1]);
      const int bs = three ? kScaleFp6Code : kScaleFp4Code;
#pragma unroll
      for (int op = 0; op < 2; ++op) {
        if (op < nops) {   // one A operand at a time: its registers are free again after hold()
          const uint4* f = reinterpret_cast<const uint4*>(S.frag[cl * nops + op][q][col]);
          const v8i a = v8_of(f[0], f[1]);
          const int sa = ps < 3 ? (int)S.sc[cl][4 * op + tr4][q] - 5 * ps : 127;
          f32x4 d = {0.f, 0.f, 0.f, 0.f};
          d = three ? mma(a, bop, d, sa, kFmtFp6, kScaleFp6Code) : mma(a, bop, d, sa, kFmtFp4, kScaleFp4Code);
          hold(d, a, bop, sa, bs);
          acc[op] += d;
        }
      }
      load(cur, c + kUDepth);
      asm volatile("" : "+v"(acc[0]), "+v"(acc[1]));   // sums land here, not deferred to the end
    };
    __syncthreads();   // the previous pass's operands and sums are consumed
    if (lane < kURows) S.cz[wave][lane] = 0.f;   // this wave's z t' sums of the pass
    if (nc == 0 && pb == p0) load_u8w();
    for (int cw0 = 0; cw0 < nc; cw0 += wcap) {
      const int wc = min(wcap, nc - cw0);
      if (cw0 > 0) __syncthreads();   // the previous window's operands are consumed
      aprep(cw0, wc, cw0 == 0);
      __syncthreads();
      int c0 = cw0;
      for (; c0 + kUDepth <= cw0 + wc; c0 += kUDepth) {
#pragma unroll
        for (int d = 0; d < kUDepth; ++d) step(c0 + d, c0 + d - cw0, cr[d]);
      }
      // tail of the last window: fewer than kUDepth chunks (uniform guards)
#pragma unroll
      for (int d = 0; d < kUDepth - 1; ++d)
        if (c0 + d < cw0 + wc) step(c0 + d, c0 + d - cw0, cr[d]);
    }
    // ---- epilogue: each token's three piece rows, sum_i z t' per token row, 8-bit pairs, W x, one rounding
    f32x4 tot[2];
#pragma unroll
    for (int op = 0; op < 2; ++op) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = acc[op][r] + swz_xor<16>(acc[op][r]);   // pieces 0+1, 2+(zero row)
        tot[op][r] = v + __shfl_xor(v, 32, 64);
      }
    }
    __syncthreads();
    if (q < 2) {   // lane group q writes the tokens of op q
      const f32x4 tq = q == 0 ? tot[0] : tot[1];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rw = 4 * q + r;
        if (rw < nt) {
          const int tk = perm[pb + rw];
          float cz = 0.f;
#pragma unroll
          for (int w8 = 0; w8 < kUWaves; ++w8) cz += S.cz[w8][rw];
          float v = tq[r] - cz;
#pragma unroll
          for (int i = 0; i < kU8Max; ++i)
            if (i < s8.n) v += u8w[i] * tv[(size_t)(pb + rw) * rs + i];
          for (int i = kU8Max; i < s8.n; ++i) {   // more 8-bit pairs than kept in registers
            const uint32_t e = s8.us[(size_t)g * round_up(s8.n, 4) + i];
            const float uh = (float)(_Float16)(f16f(e & 0xFFFFu) * ((float)s8.uc[(size_t)orow * s8.n + i] - f16f(e >> 16)));
            v += uh * tv[(size_t)(pb + rw) * rs + i];
          }
          y[(size_t)tk * out + orow] = to_bf16(v + (ybase ? ybase[(size_t)tk * out + orow] : 0.f));
        }
      }
    }
  }
}

}  // namespace

// Segments of at least this many tokens take the dense prefill form.
constexpr int kDenseMin = 256;

int launch_apply(const ApplyArgs& a) {
  if (a.mode == 2 && a.wl.drp > 0) {
    bool dense = true;
    for (int k = 0; k < a.n; ++k) {
      const int nt = a.seg[k + 1] - a.seg[k];
      if (nt > 0 && nt < kDenseMin) dense = false;
    }
    if (dense) return launch_dense_prefill(a);
  }
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  uint32_t* flags = reinterpret_cast<uint32_t*>(a.ws + a.wl.flags);
  int32_t* offs = reinterpret_cast<int32_t*>(a.ws + a.wl.offs);
  int32_t* perm = reinterpret_cast<int32_t*>(a.ws + a.wl.perm);
  ActEntry* act = reinterpret_cast<ActEntry*>(a.ws + a.wl.act);
  float* tv = reinterpret_cast<float*>(a.ws + a.wl.vpart);
  float* ybase = a.W ? reinterpret_cast<float*>(a.ws + a.wl.ybase) : nullptr;
  const size_t items = (size_t)a.T * (a.in / kGroup);
  uint8_t* xf = a.ws + a.wl.xf;
  uint32_t* xsc = reinterpret_cast<uint32_t*>(a.ws + a.wl.xsc);
  float* xsum = reinterpret_cast<float*>(a.ws + a.wl.xsum);
  // the B tiles of x feed the split-K backbone product only
  uint16_t* xt = a.W && base_splits(a.out, a.in, a.T) > 0 ? reinterpret_cast<uint16_t*>(a.ws + a.wl.xt) : nullptr;
  SegArg seg{};
  if (a.mode == 2)
    for (int k = 0; k <= a.n; ++k) seg.v[k] = a.seg[k];
  auto mark = [&](int s) {
    if (a.events && a.events[s]) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(a.events[s]), st);
  };
  mark(DC_STAGE_ROUTE);
  mark(DC_STAGE_XPREP);
  const int nyb = a.W && base_splits(a.out, a.in, a.T) > 1 ? a.T * a.out : 0;
  hipLaunchKernelGGL(k_prep, dim3((unsigned)(1 + (items + 3) / 4)), dim3(256), 0, st, *a.tenants, a.x, a.ids, a.T,
                     a.in, a.n, a.mode, seg, offs, perm, act, flags, xf, xsc, xsum, xt, tv, a.T * a.wl.rs, ybase, nyb);
  mark(DC_STAGE_BASE);
  if (a.W) launch_base(a.W, a.x, xt, ybase, a.out, a.in, a.T, a.stream);
  mark(DC_STAGE_VSIDE);
  if (a.wl.vb > 0)
    hipLaunchKernelGGL(k_vside, dim3((unsigned)(a.wl.vb * v_slices(a.in)), (unsigned)a.n), dim3(256), 0, st,
                       a.n, a.out, a.in, a.x, act, perm, xf, xsc, xsum, tv, a.wl.rs);
  mark(DC_STAGE_USIDE);
  hipLaunchKernelGGL(k_uside, dim3((unsigned)(a.out / kGroup), (unsigned)(a.n + 1)), dim3(kUWaves * 64), 0, st,
                     a.n, a.out, a.in, act, perm, tv, a.wl.rs, a.T, ybase, a.y);
  mark(DC_STAGE_COUNT);
  return (int)hipGetLastError();
}

}  // namespace dc
