// gfx950 kernels of the dense prefill form: tenants whose segments hold many
// tokens ("Delta-CoMe - 清华联合OpenBMB...", application scenarios: many
// fine-tuned models served together; "Delta-CoMe: Training-Free
// Delta-Compression with Mixed-Precision for LLMs", Approach: 8/3/2-bit
// singular vectors).  Per tenant and segment of tokens:
//   t = sigma (V x)   with V dequantized from its packed codes,
//   y = W x + U t     with U dequantized from its packed codes,
// as tiled matrix-core products (v_mfma_f32_16x16x32_f16) whose operand
// tiles are dequantized in registers on their way into LDS: the fp16 values
// fp16(s (q - z)) of the packer's quantizer, exact.  x enters as fp16 after a
// power-of-two rescale per token (bf16 values convert exactly, unless they
// lie 2^24 below the token's largest); t is carried as fp16 hi + lo after a
// power-of-two rescale per token (about 22 significant bits), so the U
// product takes two matrix-core ops per tile where the V product takes one.
//
// Ranks are laid out segment by segment, each segment padded to a multiple
// of 32 (its K-blocks of 32 ranks never straddle two widths): padded rank
// p = p0(segment) + local rank.  t is stored fp32 [T][ldt] in that order,
// zero in the padding; the largest |t| of each token is kept as its bits
// (atomic max: order-free) for the U product's rescale.
#include <hip/hip_runtime.h>

#include "dc_internal.h"

namespace dc {
namespace {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kPfBufFlags = 0x00020000;   // buffer resource word 3: raw 32-bit dwords, bounds-checked

constexpr int kPT = 128;                 // rows and tokens per tile
constexpr int kPVK = 64;                 // V product: inputs per K chunk (half a 128-group)
constexpr int kPVPad = kPVK * 2 + 16;    // its LDS row stride in bytes (conflict-free 16-byte reads)
constexpr int kPUK = 32;                 // U product: ranks per K chunk (one K-block)
constexpr int kPUPad = kPUK * 2 + 16;
constexpr int kPGroup = 8;               // row tiles per group of the per-XCD tile order

__device__ __forceinline__ float f16v(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }
__device__ __forceinline__ uint32_t f16b(float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); }
__device__ __forceinline__ float pow2(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }
__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// Exponent e with m 2^-e in [2^14, 2^15) for a magnitude m (0 for m = 0),
// kept where 2^-e and 2^e are normal floats.
__device__ __forceinline__ int scale_exp(float m) {
  if (!(m > 0.f)) return 0;
  int E = (int)((__float_as_uint(m) >> 23) & 0xFF) - 127;
  if (E < -126) E = -126;
  const int e = E - 14;
  return e < -126 ? -126 : (e > 126 ? 126 : e);
}

// Code k (compile-time) of a 32-code bitstream at b bits held in w.
template <int B, int K>
__device__ __forceinline__ uint32_t code_of(const uint32_t* w) {
  constexpr int bit = B * K, wi = bit >> 5, sh = bit & 31;
  if constexpr (sh + B > 32)
    return ((w[wi] >> sh) | (w[wi + 1] << (32 - sh))) & ((1u << B) - 1);
  else
    return (w[wi] >> sh) & ((1u << B) - 1);
}

// fp16 bits of s (q - z) for codes K0 .. K0 + N - 1 of w, two per word of
// out; ONE: one scale word for all (a V chunk), else one per code (a U run).
// Two codes at a time in packed fp16: 0x6400 | q is the fp16 value 1024 + q,
// and the zero point is an integer of at most 8 bits (the quantizer's), so
// (1024 + q) - (1024 + z) = q - z exactly and one fp16 multiply rounds
// s (q - z) once, as the fp32 product rounded to fp16 would.
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
template <int B, int K0, int E, int N, bool ONE>
struct Dequant {
  static __device__ __forceinline__ void run(const uint32_t* w, const uint32_t* sz, uint32_t* out) {
    if constexpr (E < N) {
      const uint32_t qq = code_of<B, K0 + E>(w) | (code_of<B, K0 + E + 1>(w) << 16) | 0x64006400u;
      const uint32_t sp = ONE ? (sz[0] & 0xFFFFu) * 0x10001u : (sz[E] & 0xFFFFu) | (sz[E + 1] << 16);
      const uint32_t zp = ONE ? (sz[0] >> 16) * 0x10001u : (sz[E] >> 16) | (sz[E + 1] & 0xFFFF0000u);
      const h2 d = __builtin_bit_cast(h2, qq) - (__builtin_bit_cast(h2, zp) + h2{(_Float16)1024.0f, (_Float16)1024.0f});
      out[E / 2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(h2, sp) * d);
      Dequant<B, K0, E + 2, N, ONE>::run(w, sz, out);
    }
  }
};

struct PfSeg {
  int32_t ovc, ovs;     // byte offsets in the tenant's buffer: V codes, V scale | zero << 16 [in/128][pad4(n)]
  int32_t ouc, ous;     // U codes, U scale | zero << 16 [out/128][pad4(n)]
  int32_t b, n, p0, glo;   // width, pairs, first padded rank, first global rank
};

// The operand loads go through one buffer resource over the tenant's whole
// packed buffer: every load is issued on every path (an offset of total, its
// size, is out of range and reads zeros), so the waits for them are exact.
struct PfTenant {
  const uint8_t* base;  // the packed buffer
  int32_t total;        // its bytes
  int32_t pad_;
  PfSeg s[3];           // 8-, 3- and 2-bit segments
  int32_t osig;         // byte offset of sigma in the buffer
  int32_t rp;           // padded rank rows of the V product (a multiple of 128)
  int32_t kp;           // padded ranks of the U product's K (a multiple of 32)
  int32_t s0, nt;       // the segment's tokens
};

struct PfBatch {
  PfTenant t[kPfBatch];
};

__device__ __forceinline__ int seg_of_pad(const PfTenant& tn, int p) {
  return p < tn.s[1].p0 ? 0 : (p < tn.s[2].p0 ? 1 : 2);
}

// Segment w of a tenant by selects on constant indices (a per-lane index into
// the kernel-argument record would load it through memory per lane).
__device__ __forceinline__ PfSeg seg_sel(const PfTenant& tn, int w) {
  return w == 0 ? tn.s[0] : (w == 1 ? tn.s[1] : tn.s[2]);
}

// Tile (o0, t0) of block b of a product with nto row tiles and ntt token
// tiles: consecutive block ids go round-robin over the 8 XCDs, so each XCD
// takes a contiguous range of tiles, ordered as groups of kPGroup row tiles
// x all token tiles (the blocks one XCD runs together share rows and tokens
// in its L2).
__device__ __forceinline__ bool tile_of(int nto, int ntt, int& o0, int& t0) {
  const int total = nto * ntt;
  if (blockIdx.x >= (unsigned)total) return false;
  const int xcd = blockIdx.x & 7, j8 = blockIdx.x >> 3;
  const int tile = xcd * (total >> 3) + min(xcd, total & 7) + j8;
  const int g = tile / (kPGroup * ntt), rem = tile - g * (kPGroup * ntt);
  const int gs = min(kPGroup, nto - g * kPGroup);
  o0 = (g * kPGroup + rem % gs) * kPT;
  t0 = (rem / gs) * kPT;
  return true;
}

// ----------------------------------------------------------------- V product
// C[p][tok] = sum_k V̂[p][k] x'[tok][k], x' = x 2^-e(tok); t = sigma_p C 2^e.
// Block = 128 padded ranks x 128 tokens, 4 waves of 64 x 64, K in chunks of
// 64 inputs through two LDS buffers.  Staging thread: rank row tid/2, code
// chunk tid%2 of the K chunk (32 codes, one word run), and token rows
// 32 it + tid/8, 8 inputs each.
__global__ void __launch_bounds__(256, 2) k_pf_v(PfBatch pb, const uint16_t* xh, int32_t in,
                                                 int32_t ldt, const float* __restrict__ xsc, float* __restrict__ tw,
                                                 uint32_t* __restrict__ tmax) {
  const PfTenant& tn = pb.t[blockIdx.y];
  const int N = tn.nt, s0 = tn.s0;
  int o0, t0;
  if (!tile_of(tn.rp / kPT, (N + kPT - 1) / kPT, o0, t0)) return;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kPT * kPVPad];   // [stage][V, x][row][bytes]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int gi = in / kGroup;
  // this thread's rank row and its segment
  const int arow = tid >> 1, qs = tid & 1;
  const int p = o0 + arow;
  // every wave's 32 rows are one K-block of one segment (segments are padded
  // to 32 ranks): the segment is the same on every lane
  const PfSeg sg = seg_sel(tn, __builtin_amdgcn_readfirstlane(seg_of_pad(tn, p)));
  const int li = p - sg.p0;
  const bool valid = li < sg.n;
  const int np4 = (int)round_up(sg.n, 4);
  // token rows of the x' staging (x rescaled per token to fp16 by the prep kernel)
  const uint16_t* xp[4];
  int so[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = it * 32 + (tid >> 3), c = tid & 7;
    const int tok = s0 + min(t0 + row, N - 1);
    xp[it] = xh + (size_t)tok * in + c * 8;
    so[it] = row * kPVPad + c * 16;
  }
  u32x4 ca, cb;   // the code words as loaded: unpacked in swrite, so that
  uint32_t sz;    // the loads stay in flight during the chunk's matrix-core ops
  u32x4 rx[4];
  const int nk = in / kPVK;
  const __amdgpu_buffer_rsrc_t rten =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(tn.base), 0, tn.total, kPfBufFlags);
  // the lane's code words of chunk q of group g: 8 words (an 8-bit chunk
  // uses 8, a 3-bit one 3, a 2-bit one 2; the rest is unused), two 16-byte
  // loads at a dword-aligned offset; rows past the segment read zeros
  auto gload = [&](int kc) __attribute__((always_inline)) {
    const int g = kc >> 1, q = 2 * (kc & 1) + qs;
    const int wo = sg.b == 8 ? (li * gi + g) * 32 + q * 8 : (int)v_chunk_word(li, g, q, gi, sg.b);
    const int oc = valid ? sg.ovc + wo * 4 : tn.total;
    ca = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rten, oc, 0, 0));
    cb = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rten, valid ? oc + 16 : tn.total, 0, 0));
    sz = __builtin_amdgcn_raw_buffer_load_b32(rten, valid ? sg.ovs + (g * np4 + li) * 4 : tn.total, 0, 0);
#pragma unroll
    for (int it = 0; it < 4; ++it) rx[it] = *reinterpret_cast<const u32x4*>(xp[it] + (size_t)kc * kPVK);
  };
  auto swrite = [&](int s) __attribute__((always_inline)) {
    // the chunk's loads are used from here on (not hoisted into the matrix-core ops)
    asm volatile("" : "+v"(ca), "+v"(cb), "+v"(sz), "+v"(rx[0]), "+v"(rx[1]), "+v"(rx[2]), "+v"(rx[3]));
    const uint32_t cw[8] = {ca.x, ca.y, ca.z, ca.w, cb.x, cb.y, cb.z, cb.w};
    uint32_t h[16];
    if (sg.b == 8) Dequant<8, 0, 0, 32, true>::run(cw, &sz, h);
    else if (sg.b == 3) Dequant<3, 0, 0, 32, true>::run(cw, &sz, h);
    else Dequant<2, 0, 0, 32, true>::run(cw, &sz, h);
    uint4* dst = reinterpret_cast<uint4*>(&lds[s][0][arow * kPVPad + qs * 64]);
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = make_uint4(h[4 * j], h[4 * j + 1], h[4 * j + 2], h[4 * j + 3]);
#pragma unroll
    for (int it = 0; it < 4; ++it)
      *reinterpret_cast<uint4*>(&lds[s][1][so[it]]) = make_uint4(rx[it].x, rx[it].y, rx[it].z, rx[it].w);
  };
  const int wo = wave >> 1, wt = wave & 1;
  const int ra = (64 * wo + (lane & 15)) * kPVPad + (lane >> 4) * 16;
  const int rb = (64 * wt + (lane & 15)) * kPVPad + (lane >> 4) * 16;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  gload(0);
  swrite(0);
  __syncthreads();
  for (int kc = 0; kc < nk; ++kc) {
    const int s = kc & 1;
    gload(min(kc + 1, nk - 1));   // the last chunk loads itself again (unused)
    __builtin_amdgcn_sched_barrier(0);   // the loads go out before the chunk's matrix-core ops
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      uint4 a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const uint4*>(&lds[s][0][ra + 16 * i * kPVPad + ks * 64]);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const uint4*>(&lds[s][1][rb + 16 * j * kPVPad + ks * 64]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a[i]), __builtin_bit_cast(h8, b[j]),
                                                             acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);   // the chunk's ops before the wait for the next chunk's loads
    swrite(s ^ 1);   // after the last chunk: unused
    __syncthreads();
  }
  // epilogue: lane holds token column (lane & 15) of token tile j and padded
  // ranks 4 (lane >> 4) .. +3 of rank tile i; sigma of those 16 ranks first
  // (zero in the padding)
  float sgm[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pp = o0 + 64 * wo + 16 * i + 4 * (lane >> 4) + r;
      const PfSeg sr = seg_sel(tn, seg_of_pad(tn, pp));
      const int l = pp - sr.p0;
      sgm[i][r] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                 rten, l < sr.n ? tn.osig + (sr.glo + l) * 4 : tn.total, 0, 0));
    }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tl = t0 + 64 * wt + 16 * j + (lane & 15);
    if (tl >= N) continue;
    const int tok = s0 + tl;
    const float fwd = 1.f / xsc[tok];   // a power of two: exact
    float mx = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int p4 = o0 + 64 * wo + 16 * i + 4 * (lane >> 4);
      f32x4 v;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        v[r] = sgm[i][r] * acc[i][j][r] * fwd;
        mx = fmaxf(mx, fabsf(v[r]));
      }
      *reinterpret_cast<f32x4*>(tw + (size_t)tok * ldt + p4) = v;
    }
    atomicMax(tmax + tok, __float_as_uint(mx));
  }
}

// ----------------------------------------------------------------- t split
// In place, per token row of the launch's tenants: t'[p] = t[p] 2^-e(tok)
// as fp16 hi = fp16(t') and lo = fp16(t' - hi): once per (token, rank), not
// once per row tile of the U product.  Each 8 ranks' 32 bytes become their 8
// hi values, then their 8 lo values, so that the U product's staging copies
// them into its operand tiles as they are.  Thread: 8 consecutive ranks of
// one token.
__global__ void __launch_bounds__(256) k_pf_t(float* __restrict__ tw, const uint32_t* __restrict__ tmax, int32_t tok0,
                                              int32_t ntok, int32_t ldt) {
  const int per = ldt / 8;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (size_t)ntok * per) return;
  const int tok = tok0 + (int)(i / per), c = (int)(i % per) * 8;
  const float tinv = pow2(-scale_exp(__uint_as_float(tmax[tok])));
  f32x4* p = reinterpret_cast<f32x4*>(tw + (size_t)tok * ldt + c);
  const f32x4 v0 = p[0], v1 = p[1];
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const float x0 = (e < 4 ? v0[e] : v1[e - 4]) * tinv, x1 = (e < 4 ? v0[e + 1] : v1[e - 3]) * tinv;
    const uint32_t h0 = f16b(x0), h1 = f16b(x1);
    hi[e / 2] = h0 | (h1 << 16);
    lo[e / 2] = f16b(x0 - f16v(h0)) | (f16b(x1 - f16v(h1)) << 16);
  }
  reinterpret_cast<uint4*>(p)[0] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  reinterpret_cast<uint4*>(p)[1] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

// ----------------------------------------------------------------- U product
// C[o][tok] = sum_p Û[o][p] (t_hi + t_lo)[tok][p], t' = t 2^-e(tok);
// y = bf16(W x + C 2^e).  Block = 128 rows x 128 tokens, K in chunks of one
// K-block of 32 padded ranks.  Staging thread: row tid/2, 16 ranks (half
// tid%2 of the K-block) of U and of t.
__global__ void __launch_bounds__(256, 2) k_pf_u(PfBatch pb, int32_t out, int32_t ldt, const float* tw,
                                                 const uint32_t* __restrict__ tmax, const float* __restrict__ ybase,
                                                 uint16_t* __restrict__ y) {
  const PfTenant& tn = pb.t[blockIdx.y];
  const int N = tn.nt, s0 = tn.s0;
  int o0, t0;
  if (!tile_of(out / kPT, (N + kPT - 1) / kPT, o0, t0)) return;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][3][kPT * kPUPad];   // [stage][U, t hi, t lo][row][bytes]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int arow = tid >> 1, hs = tid & 1;
  const int o = o0 + arow;
  const int og = o0 / kGroup;   // the tile's 128-row scale group
  const int tl_s = min(t0 + arow, N - 1);
  const int tok_s = s0 + tl_s;
  // fp16 hi and lo values (k_pf_t) of the tenant's t rows, through a buffer
  // resource: its loads stay where they are issued
  const __amdgpu_buffer_rsrc_t rtw = __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(tw + (size_t)s0 * ldt), 0,
                                                                       N * ldt * 4, kPfBufFlags);
  const int tofs = (tl_s * ldt + 16 * hs) * 4;
  // a chunk's loads as they arrive (unpacked in swrite, so that they stay
  // in flight during the matrix-core ops of the chunks before it)
  struct In {
    u32x4 cd, szr[4];   // code bytes, scale words
    f32x4 tr[4];        // t pairs
    uint32_t cd4;
    int csh, cli0, cn, bsel;
  };
  In r0, r1;
  const int nk = tn.kp / kPUK;
  const __amdgpu_buffer_rsrc_t rten =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(tn.base), 0, tn.total, kPfBufFlags);
  auto gload = [&](In& r, int kc) __attribute__((always_inline)) {
    const int pk = kc * kPUK;
    const PfSeg sg = seg_sel(tn, seg_of_pad(tn, pk));
    const int kbl = (pk - sg.p0) / kPUK, li0 = kbl * kPUK + 16 * hs;
    const int np4 = (int)round_up(sg.n, 4);
    r.bsel = sg.b;
    // This thread's codes, the same loads for every width: 20 bytes from the
    // dword below byte a, shifted down by a % 4.  8-bit: bytes [out][n8],
    // its 16 codes from byte o n8 + li0 (the bytes past the segment's pairs
    // meet zero scales below); 3/2-bit: the row's words of K-block kbl.
    int nw;
    const int a = sg.b == 8 ? sg.ouc + o * sg.n + li0 : sg.ouc + 4 * (int)u_kblock_word(o, kbl, sg.n, sg.b, &nw);
    const int ad = a & ~3;
    r.csh = a & 3;
    r.cli0 = li0;
    r.cn = sg.n;
    r.cd = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rten, ad, 0, 0));
    r.cd4 = __builtin_amdgcn_raw_buffer_load_b32(rten, ad + 16, 0, 0);
    // the 16 scale words, four 16-byte loads (pad4 rows, li0 a multiple of
    // 16: aligned); words past the segment's pairs are zeroed in swrite (a
    // zero scale makes their values zero)
    const int os = sg.ous + (og * np4 + li0) * 4;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r.szr[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rten, os + 16 * j, 0, 0));
#pragma unroll
    for (int j = 0; j < 4; ++j)
      r.tr[j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rtw, tofs + (pk + 4 * j) * 4, 0, 0));
  };
  auto swrite = [&](In& r, int s) __attribute__((always_inline)) {
    // the chunk's loads are used from here on (not hoisted into the matrix-core ops)
    asm volatile("" : "+v"(r.cd), "+v"(r.cd4), "+v"(r.szr[0]), "+v"(r.szr[1]), "+v"(r.szr[2]), "+v"(r.szr[3]),
                 "+v"(r.tr[0]), "+v"(r.tr[1]), "+v"(r.tr[2]), "+v"(r.tr[3]));
    const int csh = r.csh;
    const uint32_t cw[4] = {__builtin_amdgcn_alignbyte(r.cd.y, r.cd.x, csh), __builtin_amdgcn_alignbyte(r.cd.z, r.cd.y, csh),
                            __builtin_amdgcn_alignbyte(r.cd.w, r.cd.z, csh), __builtin_amdgcn_alignbyte(r.cd4, r.cd.w, csh)};
    uint32_t sz[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) sz[e] = r.szr[e >> 2][e & 3];
    if (r.cli0 + 16 > r.cn) {   // the segment's last K-block: words past its pairs are another row's
#pragma unroll
      for (int e = 0; e < 16; ++e) sz[e] = r.cli0 + e < r.cn ? sz[e] : 0u;
    }
    const int bsel = r.bsel;
    uint32_t h[8];
    if (bsel == 8) {   // cw holds this thread's 16 codes, one byte each
      Dequant<8, 0, 0, 16, false>::run(cw, sz, h);
    } else if (bsel == 3) {   // cw holds the K-block's 32 codes: this half's 16 from bit 48 hs
      // (the halves select their bits before one dequant: a branch on hs
      // would run both dequants on every wave, half the lanes idle)
      const uint32_t w[2] = {hs ? (cw[1] >> 16) | (cw[2] << 16) : cw[0], hs ? cw[2] >> 16 : cw[1]};
      Dequant<3, 0, 0, 16, false>::run(w, sz, h);
    } else {   // 2-bit: this half's 16 codes are word hs
      const uint32_t w[1] = {hs ? cw[1] : cw[0]};
      Dequant<2, 0, 0, 16, false>::run(w, sz, h);
    }
    uint4* da = reinterpret_cast<uint4*>(&lds[s][0][arow * kPUPad + hs * 32]);
    da[0] = make_uint4(h[0], h[1], h[2], h[3]);
    da[1] = make_uint4(h[4], h[5], h[6], h[7]);
    // t' arrives as 8 hi values then 8 lo values per 8 ranks (k_pf_t): the
    // operand tiles take them as they are
    uint4* dh = reinterpret_cast<uint4*>(&lds[s][1][arow * kPUPad + hs * 32]);
    uint4* dl = reinterpret_cast<uint4*>(&lds[s][2][arow * kPUPad + hs * 32]);
    dh[0] = __builtin_bit_cast(uint4, r.tr[0]);
    dl[0] = __builtin_bit_cast(uint4, r.tr[1]);
    dh[1] = __builtin_bit_cast(uint4, r.tr[2]);
    dl[1] = __builtin_bit_cast(uint4, r.tr[3]);
  };
  const int wo = wave >> 1, wt = wave & 1;
  const int ra = (64 * wo + (lane & 15)) * kPUPad + (lane >> 4) * 16;
  const int rb = (64 * wt + (lane & 15)) * kPUPad + (lane >> 4) * 16;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  // chunk kc is in LDS stage kc & 1 while the registers hold chunk kc + 1
  // and take chunk kc + 2 (two register sets, the loop unrolled by two)
  auto mma_chunk = [&](int s) __attribute__((always_inline)) {
    uint4 a[4], bh[4], bl[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const uint4*>(&lds[s][0][ra + 16 * i * kPUPad]);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      bh[j] = *reinterpret_cast<const uint4*>(&lds[s][1][rb + 16 * j * kPUPad]);
      bl[j] = *reinterpret_cast<const uint4*>(&lds[s][2][rb + 16 * j * kPUPad]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a[i]), __builtin_bit_cast(h8, bh[j]),
                                                           acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8, a[i]), __builtin_bit_cast(h8, bl[j]),
                                                           acc[i][j], 0, 0, 0);
      }
  };
  if (nk > 0) {
    gload(r0, 0);
    swrite(r0, 0);
    gload(r1, min(1, nk - 1));
    __syncthreads();
    for (int kc = 0; kc < nk; kc += 2) {
      gload(r0, min(kc + 2, nk - 1));   // past the last chunk: the last again (unused)
      asm volatile("" ::: "memory");   // the loads go out before the chunk's matrix-core ops
      __builtin_amdgcn_sched_barrier(0);
      mma_chunk(0);
      __builtin_amdgcn_sched_barrier(0);   // the chunk's ops before the wait for the next chunk's loads
      swrite(r1, 1);
      __syncthreads();
      if (kc + 1 >= nk) break;
      gload(r1, min(kc + 3, nk - 1));
      asm volatile("" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
      mma_chunk(1);
      __builtin_amdgcn_sched_barrier(0);
      swrite(r0, 0);
      __syncthreads();
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tl = t0 + 64 * wt + 16 * j + (lane & 15);
    if (tl >= N) continue;
    const int tok = s0 + tl;
    const float fwd = pow2(scale_exp(__uint_as_float(tmax[tok])));
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = o0 + 64 * wo + 16 * i + 4 * (lane >> 4);
      f32x4 v = acc[i][j] * fwd;
      if (ybase) v += *reinterpret_cast<const f32x4*>(ybase + (size_t)tok * out + m);
      const uint32_t q0 = to_bf16(v[0]) | ((uint32_t)to_bf16(v[1]) << 16);
      const uint32_t q1 = to_bf16(v[2]) | ((uint32_t)to_bf16(v[3]) << 16);
      *reinterpret_cast<uint2*>(y + (size_t)tok * out + m) = make_uint2(q0, q1);
    }
  }
}

// Per token: the rescale 2^-e of x (largest |x| into [2^14, 2^15)) and the
// rescaled row x' = fp16(x 2^-e) [T][in] that the V product's staging copies
// (once per token, not once per rank tile); clears the token's largest |t|
// and the call's status word.  One wave per token.
__global__ void __launch_bounds__(256) k_pf_prep(const uint16_t* __restrict__ x, int32_t T, int32_t in,
                                                 float* __restrict__ xsc, uint16_t* __restrict__ xh,
                                                 uint32_t* __restrict__ tmax, uint32_t* __restrict__ flags) {
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (blockIdx.x == 0 && threadIdx.x == 0) *flags = 0u;
  if (tok >= T) return;
  const uint16_t* row = x + (size_t)tok * in;
  float m = 0.f;
  for (int k = lane * 8; k < in; k += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + k);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j)
      m = fmaxf(m, fmaxf(fabsf(__uint_as_float(w[j] << 16)), fabsf(__uint_as_float(w[j] & 0xFFFF0000u))));
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
  const float xi = pow2(-scale_exp(m));   // the same on every lane
  if (lane == 0) {
    xsc[tok] = xi;
    tmax[tok] = 0u;
  }
  // bf16 values times a power of two convert to fp16 exactly (unless 2^24
  // below the token's largest); the second read of the row is from L2
  uint16_t* orow = xh + (size_t)tok * in;
  for (int k = lane * 8; k < in; k += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(row + k);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float lo = __uint_as_float(w[j] << 16) * xi, hi = __uint_as_float(w[j] & 0xFFFF0000u) * xi;
      o[j] = f16b(lo) | (f16b(hi) << 16);
    }
    *reinterpret_cast<uint4*>(orow + k) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

}  // namespace

int pf_rank_pad(int n8, int n3, int n2) {
  const size_t kp = round_up((size_t)n8, kKBlock) + round_up((size_t)n3, kKBlock) + round_up((size_t)n2, kKBlock);
  return kp > 0 ? (int)round_up(kp, kPT) : kPT;
}

int launch_dense_prefill(const ApplyArgs& a) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  const MatArgs& A = a.mat[0];   // a prefill call has one matrix
  float* ybase = A.W ? reinterpret_cast<float*>(a.ws + a.wl.mat[0].ybase) : nullptr;
  float* tw = reinterpret_cast<float*>(a.ws + a.wl.dt);
  float* xsc = reinterpret_cast<float*>(a.ws + a.wl.dxs);
  uint32_t* tmax = reinterpret_cast<uint32_t*>(a.ws + a.wl.dtm);
  uint32_t* flags = reinterpret_cast<uint32_t*>(a.ws + a.wl.flags);
  // x' (fp16 [T][in]) in the region of the decode kernels' x fragments, which
  // this form does not use (2 T in bytes either way)
  uint16_t* xh = reinterpret_cast<uint16_t*>(a.ws + a.wl.xf);
  if (A.W) launch_tiled_base(A.W, a.x, ybase, A.out, a.in, a.T, a.stream);
  hipLaunchKernelGGL(k_pf_prep, dim3((unsigned)((a.T + 3) / 4)), dim3(256), 0, st, a.x, a.T, a.in, xsc, xh, tmax,
                     flags);
  int k = 0;
  while (k < a.n) {   // tenants with tokens, kPfBatch per launch
    PfBatch b{};
    int cnt = 0;
    unsigned tv = 0, tu = 0;
    for (; k < a.n && cnt < kPfBatch; ++k) {
      const int s0 = a.seg[k], nt = a.seg[k + 1] - a.seg[k];
      if (nt == 0) continue;
      const Tenant& tn = A.tenants->t[k];
      Layout L;
      layout_of(A.out, a.in, tn.n8, tn.n3, tn.n2, &L);
      PfTenant& p = b.t[cnt];
      p.base = tn.base;
      p.total = (int32_t)L.total;
      const int ns[3] = {tn.n8, tn.n3, tn.n2};
      int p0 = 0, glo = 0;
      for (int w = 0; w < 3; ++w) {
        PfSeg& sg = p.s[w];
        sg.b = w == 0 ? 8 : (w == 1 ? 3 : 2);
        sg.n = ns[w];
        sg.p0 = p0;
        sg.glo = glo;
        sg.ovc = (int32_t)L.off[DC_REG_VC8 + w];
        sg.ovs = (int32_t)L.off[DC_REG_VS8 + w];
        sg.ouc = (int32_t)L.off[DC_REG_UC8 + w];
        sg.ous = (int32_t)L.off[DC_REG_US8 + w];
        p0 += (int)round_up((size_t)ns[w], kKBlock);
        glo += ns[w];
      }
      p.osig = (int32_t)L.off[DC_REG_SIGMA];
      p.kp = p0;
      p.rp = pf_rank_pad(tn.n8, tn.n3, tn.n2);
      p.s0 = s0;
      p.nt = nt;
      const unsigned ntt = (unsigned)((nt + kPT - 1) / kPT);
      tv = max(tv, (unsigned)(p.rp / kPT) * ntt);
      tu = max(tu, (unsigned)(A.out / kPT) * ntt);
      ++cnt;
    }
    if (cnt == 0) break;
    // grid x a multiple of 8, so that blockIdx.x mod 8 is the XCD the tile order assumes
    hipLaunchKernelGGL(k_pf_v, dim3((tv + 7) / 8 * 8, (unsigned)cnt), dim3(256), 0, st, b, xh, a.in, a.wl.drp, xsc,
                       tw, tmax);
    const int tok0 = b.t[0].s0, ntok = b.t[cnt - 1].s0 + b.t[cnt - 1].nt - tok0;   // the batch's segments are contiguous
    const size_t nth = (size_t)ntok * (a.wl.drp / 8);
    hipLaunchKernelGGL(k_pf_t, dim3((unsigned)((nth + 255) / 256)), dim3(256), 0, st, tw, tmax, tok0, ntok, a.wl.drp);
    hipLaunchKernelGGL(k_pf_u, dim3((tu + 7) / 8 * 8, (unsigned)cnt), dim3(256), 0, st, b, A.out, a.wl.drp, tw, tmax,
                       ybase, A.y);
  }
  return (int)hipGetLastError();
}

}  // namespace dc
