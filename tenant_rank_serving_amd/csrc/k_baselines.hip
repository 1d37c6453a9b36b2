// gfx950 kernels of the two baselines the pages compare Delta-CoMe with at
// the same storage ("Delta-CoMe: Training-Free Delta-Compression with
// Mixed-Precision for LLMs", Experimental setup and Key results: low-rank
// SVD compression and BitDelta at 1/16): the delta part of
//   low-rank   y = W x + U (sigma * (V x)),  U, V fp16, sigma fp32
//   BitDelta   y = W x + alpha S x,          S in {+1, -1}, one bit each
// for tokens routed to tenants.  The routing, the x fragments and the
// backbone product come from the Delta-CoMe kernels of the same call.
//
// BitDelta.  A sign bit goes straight into v_mfma_scale_f32_16x16x128_f8f6f4
// as an fp4 (e2m1) B element: (bit << 3) | 1 is -0.5 for a set bit and +0.5
// for a clear one, so the product with the B scale 2^1 is -S x.  The words
// keep the entries of a lane's 32 columns interleaved by nibble, so shifting
// by s and one AND-OR give the s-th dword of the B operand.  x is the A
// operand as fp8 hi/lo pieces with E8M0 block scales (rows 0-7 hi, rows 8-15
// lo), the same fragments the Delta-CoMe V side reads.
//
// Low-rank.  v_mfma_f32_16x16x32_f16: the fp16 V rows and U columns are B
// operands loaded as they are stored (one 16-byte load per lane per 32-step
// tile).  x becomes fp16 after a power-of-two rescale per 128 inputs (bf16
// values in fp16's normal range convert exactly); t = sigma (V x) becomes
// hi + lo fp16 pieces after a power-of-two rescale per token (A rows 0-7 hi,
// rows 8-15 lo), about 22 significant bits.
#include <hip/hip_runtime.h>

#include "dc_internal.h"

namespace dc {
namespace {

#include "mx_common.h"
#include "combine.h"
#include "vstage.h"

typedef _Float16 h8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ f32x4 mma16(const h8& a, const h8& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ h8 h8_of(const uint4& v) { return __builtin_bit_cast(h8, v); }

// ------------------------------------------------------------------ BitDelta
// The B operand of one lane from its word: dword s holds entries of nibble
// positions 8s..8s+7 as (bit << 3) | 1.
__device__ __forceinline__ v8i b_sign(uint32_t w) {
  v8i b = {0, 0, 0, 0, 0, 0, 0, 0};
  b[0] = (int)(((w << 3) & 0x88888888u) | 0x11111111u);
  b[1] = (int)(((w << 2) & 0x88888888u) | 0x11111111u);
  b[2] = (int)(((w << 1) & 0x88888888u) | 0x11111111u);
  b[3] = (int)((w & 0x88888888u) | 0x11111111u);
  return b;
}

constexpr int kBdDepth = 8;   // groups of sign words a wave keeps in flight

// The backbone value of output (token tk, row o): W x, or the sum of its K
// ranges in range order when the product was split in more than two.
__device__ __forceinline__ float base_of(const MatParams& P, int T, int tk, int o) {
  if (!P.ybase) return 0.f;
  if (P.nks <= kMaxAtomicTerms) return P.ybase[(size_t)tk * P.out + o];
  const size_t rstride = (size_t)T * P.out;
  const float* src = P.bpt + (size_t)tk * P.out + o;
  float v = 0.f;
  for (int r0 = 0; r0 < P.nks; r0 += 8) {
    float a[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) a[j] = r0 + j < P.nks ? src[(r0 + j) * rstride] : 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      if (r0 + j < P.nks) v += a[j];
  }
  return v;
}

struct BdGroup {
  const ActEntry* act;   // [m][nact]
  const MatParams* mp;   // [m]
  int32_t nact, ns, T, n;
};

// Block = one work item (up to 8 token rows) x kBdRows output rows x one
// input slice of kVSlice groups: wave w takes the two 16-row tiles
// 2w, 2w+1 of the block.  The slice's x fragments are staged in LDS once;
// the wave's sign words stream through a register ring kBdDepth groups deep.
// With more than one slice the partials are stored and the block of the
// item and rows that arrives last adds them in slice order; that block (or
// the only one) writes y = bf16(W x - alpha (-S x)).  Items of the
// backbone-only bucket write bf16(W x) from their first slice's blocks.
__global__ void __launch_bounds__(256) k_bd(int32_t in, const int32_t* __restrict__ perm,
                                            const uint8_t* __restrict__ xf, const uint32_t* __restrict__ xsc,
                                            const float* __restrict__ xsum, BdGroup g) {
  const int mj = blockIdx.y / g.nact, item = blockIdx.y % g.nact;
  const MatParams P = g.mp[mj];
  const ActEntry e = g.act[blockIdx.y];
  const int p0 = e.p0, p1 = e.p1;
  if (p0 >= p1) return;
  const int ns = g.ns;
  const int rb = blockIdx.x / ns, s = blockIdx.x % ns;
  const int out = P.out;
  if (rb * kBdRows >= out) return;
  const bool delta = e.k < g.n;
  if (!delta && s > 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, q = lane >> 4;
  const int nt = p1 - p0;
  const int tile0 = rb * (kBdRows / 16) + 2 * wave;
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  float alpha = 0.f;
  if (delta) {
    __shared__ VLds S;
    const int gi_n = in / kGroup;
    const int g0 = s * kVSlice;
    const int gn = min(kVSlice, gi_n - g0);
    const int glast = g0 + gn - 1;
    alpha = *reinterpret_cast<const float*>(e.base);
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(e.base + kAlign), 0, (out / 16) * gi_n * 64 * 4, kBufFlags);
    uint32_t oc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) oc[h] = (uint32_t)(((tile0 + h) * gi_n * 64 + lane) * 4);
    VStage st;
    v_stage_load(st, xf, xsc, xsum, gi_n, g0, tok8_of(e.tok), nt);   // ahead of the ring: vmcnt is in order
    uint32_t ring[kBdDepth][2];
#pragma unroll
    for (int d = 0; d < kBdDepth; ++d)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        ring[d][h] = __builtin_amdgcn_raw_buffer_load_b32(rc, oc[h], min(g0 + d, glast) * 256, 0);
    v_stage_store(S, st);
    __syncthreads();
    const int tr = col & 7, piece = col >> 3;
    const bool live = tr < nt;
#pragma unroll
    for (int u = 0; u < kVSlice; ++u) {
      uint32_t c[2] = {ring[u % kBdDepth][0], ring[u % kBdDepth][1]};
      if (u + kBdDepth < kVSlice) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
          ring[u % kBdDepth][h] =
              __builtin_amdgcn_raw_buffer_load_b32(rc, oc[h], min(g0 + u + kBdDepth, glast) * 256, 0);
      }
      if (u < gn) {   // groups past the input are clamped duplicates
        const int4* fr = S.frag[u][tr] + 4 * q + 2 * piece;
        const int4 f0 = fr[0], f1 = fr[1];
        const v8i a = live ? v8i{f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w} : v8i{0, 0, 0, 0, 0, 0, 0, 0};
        const int sa = live ? (int)((S.sc[u][tr] >> (8 * q)) & 0xFFu) - 5 * piece : 127;
        const v8i b0 = b_sign(c[0]), b1 = b_sign(c[1]);
        acc[0] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b0, acc[0], kFmtFp8, kFmtFp4, 0, sa, 0,
                                                                  kScaleFp4Code);
        acc[1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b1, acc[1], kFmtFp8, kFmtFp4, 0, sa, 0,
                                                                  kScaleFp4Code);
        hold2(acc[0], acc[1], a, b0, b1, sa, kScaleFp4Code);
      }
    }
    // rows 8-15 hold the lo pieces' products: fold them onto rows 0-7
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[h][r] += __shfl_xor(acc[h][r], 32, 64);
    if (ns > 1) {
      if (q < 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (4 * q + r < nt)
              st_dev(P.vpt + ((size_t)s * g.T + p0 + 4 * q + r) * out + (tile0 + h) * 16 + col, acc[h][r]);
      }
      __shared__ int last;
      if (!arrive_last(&P.vcnt[item * P.vb + rb], ns, &last)) return;
      if (q < 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float v = 0.f;
            if (4 * q + r < nt) {
              const float* src = P.vpt + (size_t)(p0 + 4 * q + r) * out + (tile0 + h) * 16 + col;
              for (int s0 = 0; s0 < ns; ++s0) v += ld_dev(src + (size_t)s0 * g.T * out);
            }
            acc[h][r] = v;
          }
      }
    }
  }
  if (q >= 2) return;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rw = 4 * q + r;
      if (rw < nt) {
        const int tk = perm[p0 + rw];
        const int o = (tile0 + h) * 16 + col;
        P.y[(size_t)tk * out + o] = to_bf16(base_of(P, g.T, tk, o) - alpha * acc[h][r]);
      }
    }
}

// ------------------------------------------------------------ low-rank, V
struct LrVGroup {
  const ActEntry* act;           // [m][nact]
  const MatParams* mp;           // [m]
  BaseSum bs[kMaxGroup];
  int32_t red0[kMaxGroup + 1];   // first partial-sum block of each matrix (prefix over the group)
  int32_t red_rows;              // leading grid rows of partial-sum blocks
  int32_t nact, ns, T, n;
};

constexpr int kLrSteps = kLrSlice / 32;   // 32-input steps per slice

struct LrVLds {
  uint4 xa[kLrSteps][kVRows][4];        // fp16 x of the slice: [step][token row][lane group], 8 halves each
  float sc[kLrSlice / kGroup][kVRows];  // power of two undoing each 128-group's rescale
};

// Block = one work item x kLrRanks ranks x one input slice of kLrSlice:
// wave w takes the 16-rank tile 4b + w over the slice's steps, all of whose
// V loads go out before x is staged.  A row m < 8 is token m; rows 8-15
// are zero.  sigma * (partial V x) goes to t as in the Delta-CoMe V side
// (atomics onto zero for up to two slices, else stored and added in slice
// order by the last block).  Leading grid rows add the backbone product's K
// ranges in range order (more than two ranges).
__global__ void __launch_bounds__(256) k_lr_v(int32_t in, const uint16_t* __restrict__ x,
                                              const int32_t* __restrict__ perm, const uint32_t* __restrict__ xsc,
                                              LrVGroup g) {
  if ((int)blockIdx.y < g.red_rows) {
    const int idx = blockIdx.y * gridDim.x + blockIdx.x;
#pragma unroll
    for (int j = 0; j < kMaxGroup; ++j)
      if (idx >= g.red0[j] && idx < g.red0[j + 1]) base_sum(g.bs[j], idx - g.red0[j]);
    return;
  }
  const int yy = blockIdx.y - g.red_rows;
  const int mj = yy / g.nact, item = yy % g.nact;
  const MatParams P = g.mp[mj];
  const ActEntry e = g.act[yy];
  const int p0 = e.p0, p1 = e.p1;
  if (p0 >= p1 || e.k >= g.n) return;
  const int r = e.n8;
  const int ns = g.ns;
  const int b = blockIdx.x / ns, s = blockIdx.x % ns;
  if (b * kLrRanks >= r) return;
  const VOut vo{P.tv, P.vpt, P.vcnt, P.rs, ns, g.T, P.vb};
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, q = lane >> 4;
  const int nt = p1 - p0;
  const int k0 = s * kLrSlice;
  const int nst = min(kLrSteps, (in - k0) / 32);   // steps of this slice (in is a multiple of 128)
  const int tile = b * (kLrRanks / 16) + wave;
  const bool live_wave = tile * 16 < r;
  // the wave's V operands for the whole slice
  const int in32 = in / 32;
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(e.base + lowrank_v_offset(r)), 0, (int)(round_up(r, 16) * in * 2), kBufFlags);
  uint4 bv[kLrSteps];
  const uint32_t ob = (uint32_t)(((tile * in32 + k0 / 32) * 64 + lane) * 16);
#pragma unroll
  for (int j = 0; j < kLrSteps; ++j) {
    bv[j] = uint4{0u, 0u, 0u, 0u};
    if (live_wave && j < nst) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rv, ob, j * 64 * 16, 0);
      bv[j] = uint4{v.x, v.y, v.z, v.w};
    }
  }
  // stage x: thread = token row tid / 32, 16 inputs (tid % 32) * 16 of the slice
  __shared__ LrVLds S;
  {
    const int rw = tid >> 5, c = tid & 31;
    const int kk = c * 16;
    if (kk < nst * 32) {
      const int prow = p0 + min(rw, nt - 1);
      const int tk = perm[prow];
      const int gi = (k0 + kk) / kGroup;
      const uint32_t w = xsc[(size_t)tk * (in / kGroup) + gi];   // scale words in token order
      const int bmax = max(max((int)(w & 0xFFu), (int)((w >> 8) & 0xFFu)),
                           max((int)((w >> 16) & 0xFFu), (int)(w >> 24)));
      const float f = pow2f(127 - bmax);   // |x| * f < 256
      const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)tk * in + k0 + kk);
      const uint4 v0 = src[0], v1 = src[1];
      const uint32_t xw[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
      uint32_t hw[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float lo = __uint_as_float(xw[j] << 16) * f, hi = __uint_as_float(xw[j] & 0xFFFF0000u) * f;
        hw[j] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
      }
      // inputs kk..kk+15 = step kk/32, lane groups (kk%32)/8 and +1
      const int stp = kk / 32, lg = (kk % 32) / 8;
      S.xa[stp][rw][lg] = uint4{hw[0], hw[1], hw[2], hw[3]};
      S.xa[stp][rw][lg + 1] = uint4{hw[4], hw[5], hw[6], hw[7]};
      if ((kk % kGroup) == 0) S.sc[kk / kGroup][rw] = pow2f(bmax - 127);
    }
  }
  __syncthreads();
  if (live_wave) {
    const bool arow = col < 8;   // A rows 8-15 are zero
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int gq = 0; gq < kLrSteps / 4; ++gq) {
      if (4 * gq < nst) {   // whole 128-groups: in is a multiple of 128
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint4 av = arow ? S.xa[4 * gq + j][col][q] : uint4{0u, 0u, 0u, 0u};
          d = mma16(h8_of(av), h8_of(bv[4 * gq + j]), d);
        }
        if (q < 2) {
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) acc[rr] += d[rr] * S.sc[gq][4 * q + rr];
        }
      }
    }
    if (q < 2) {
      const int rank = tile * 16 + col;
      if (rank < r) {
        const float sg = reinterpret_cast<const float*>(e.base)[rank];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          if (4 * q + rr < nt) v_put(vo, s, p0 + 4 * q + rr, rank, sg * acc[rr]);
      }
    }
  }
  v_combine(vo, item, b, p0, p1, b * kLrRanks, min(kLrRanks, r - b * kLrRanks));
}

// ------------------------------------------------------------ low-rank, U
struct LrUGroup {
  const ActEntry* act;   // [m][nact]
  const MatParams* mp;   // [m]
  int32_t nact, T, n;
};

constexpr int kLrWin = 8;   // 32-rank steps of t staged at a time

struct LrULds {
  uint4 ta[kLrWin][16][4];   // A operands: [step][row (0-7 hi, 8-15 lo)][lane group], 8 halves each
  float sc[kVRows];          // power of two undoing each token's rescale
  float inv[kVRows];         // the rescale
};

// Block = one work item x 128 output rows (wave w: the tiles 2w, 2w+1 of the
// block), all ranks in windows of kLrWin steps.  Per token, t is rescaled by
// a power of two so that its largest magnitude lies in [2^14, 2^15) and split
// into fp16 hi + lo; the U operands of a window go out before it is staged.
// Epilogue: y = bf16(W x + 2^e (hi + lo products)).  Items of the
// backbone-only bucket (or of a tenant with r = 0) write bf16(W x).
__global__ void __launch_bounds__(256) k_lr_u(int32_t in, const int32_t* __restrict__ perm, LrUGroup g) {
  const int mj = blockIdx.y / g.nact;
  const MatParams P = g.mp[mj];
  const ActEntry e = g.act[blockIdx.y];
  const int p0 = e.p0, p1 = e.p1;
  if (p0 >= p1) return;
  const int out = P.out;
  const int rb = blockIdx.x;
  if (rb * 128 >= out) return;
  const int r = e.k < g.n ? e.n8 : 0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, q = lane >> 4;
  const int nt = p1 - p0;
  const int tile0 = rb * 8 + 2 * wave;
  f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  __shared__ LrULds S;
  if (r > 0) {
    const int nsteps = (r + 31) / 32;
    const __amdgpu_buffer_rsrc_t ru = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(e.base + lowrank_u_offset(in, r)), 0, out * nsteps * 64, kBufFlags);
    uint32_t ou[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) ou[h] = (uint32_t)(((tile0 + h) * nsteps * 64 + lane) * 16);
    const int rw = tid >> 5, c = tid & 31;   // staging: token row, 8 ranks
    {  // the rescale of each token: largest |t| over its ranks
      float m = 0.f;
      if (rw < nt) {
        const float* tr = P.tv + (size_t)(p0 + rw) * P.rs;
        for (int i = c; i < r; i += 32) m = fmaxf(m, fabsf(tr[i]));
      }
#pragma unroll
      for (int d = 16; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
      if (c == 0) {
        int E = (int)((__float_as_uint(m) >> 23) & 0xFF) - 127;   // m in [2^E, 2^(E+1)) (normal m)
        if (!(m > 0.f)) E = 14;                                    // all zero: no rescale
        E = E < -113 ? -113 : E;                                   // 2^(14-E) stays a normal float
        S.sc[rw] = pow2f(E - 14 < -126 ? -126 : (E - 14 > 127 ? 127 : E - 14));
        S.inv[rw] = pow2f(14 - E > 127 ? 127 : 14 - E);
      }
    }
    for (int w0 = 0; w0 < nsteps; w0 += kLrWin) {
      const int wn = min(kLrWin, nsteps - w0);
      uint4 bu[kLrWin][2];
#pragma unroll
      for (int j = 0; j < kLrWin; ++j)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bu[j][h] = uint4{0u, 0u, 0u, 0u};
          if (j < wn) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(ru, ou[h], (w0 + j) * 64 * 16, 0);
            bu[j][h] = uint4{v.x, v.y, v.z, v.w};
          }
        }
      __syncthreads();   // the scales are written; the previous window's operands are consumed
      {
        const int i0 = w0 * 32 + c * 8;
        const float inv = S.inv[rw];
        const float* tr = P.tv + (size_t)(p0 + min(rw, nt - 1)) * P.rs;
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          uint32_t hh[2], ll[2];
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            const int i = i0 + 2 * j + k;
            const float v = (rw < nt && i < r) ? tr[i] * inv : 0.f;
            const _Float16 h = (_Float16)v;
            hh[k] = __builtin_bit_cast(uint16_t, h);
            ll[k] = __builtin_bit_cast(uint16_t, (_Float16)(v - (float)h));
          }
          hw[j] = hh[0] | (hh[1] << 16);
          lw[j] = ll[0] | (ll[1] << 16);
        }
        S.ta[c / 4][rw][c % 4] = uint4{hw[0], hw[1], hw[2], hw[3]};
        S.ta[c / 4][8 + rw][c % 4] = uint4{lw[0], lw[1], lw[2], lw[3]};
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < kLrWin; ++j) {
        if (j < wn) {
          const h8 a = h8_of(S.ta[j][col][q]);
          acc[0] = mma16(a, h8_of(bu[j][0]), acc[0]);
          acc[1] = mma16(a, h8_of(bu[j][1]), acc[1]);
        }
      }
    }
    // rows 8-15 hold the lo pieces' products: fold them onto rows 0-7
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) acc[h][rr] += __shfl_xor(acc[h][rr], 32, 64);
  }
  if (q >= 2) return;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int rw = 4 * q + rr;
      if (rw < nt) {
        const int tk = perm[p0 + rw];
        const int o = (tile0 + h) * 16 + col;
        const float yb = P.ybase ? P.ybase[(size_t)tk * out + o] : 0.f;
        P.y[(size_t)tk * out + o] = to_bf16(yb + (r > 0 ? acc[h][rr] * S.sc[rw] : 0.f));
      }
    }
}

}  // namespace

int launch_baseline(const BaselineLaunch& a) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  if (a.kind == kKindBitdelta) {
    BdGroup g{a.act, a.mp, a.nact, a.ns, a.T, a.n};
    const unsigned gx = (unsigned)((a.outmax / kBdRows) * a.ns);
    hipLaunchKernelGGL(k_bd, dim3(gx, (unsigned)(a.m * a.nact)), dim3(256), 0, st, a.in, a.perm, a.xf, a.xsc,
                       a.xsum, g);
    return (int)hipGetLastError();
  }
  LrVGroup vg{};
  vg.act = a.act;
  vg.mp = a.mp;
  vg.nact = a.nact;
  vg.ns = a.ns;
  vg.T = a.T;
  vg.n = a.n;
  const int gx = a.vbmax > 0 ? a.vbmax * a.ns : 1;
  int red = 0;
  for (int j = 0; j < a.m; ++j) {
    vg.red0[j] = red;
    if (a.bpt[j]) {
      vg.bs[j] = BaseSum{a.bpt[j], a.ybase[j], a.nks, a.out[j], a.T};
      red += (a.out[j] / 64) * ((a.T + 7) / 8);
    }
  }
  for (int j = a.m; j <= kMaxGroup; ++j) vg.red0[j] = red;
  vg.red_rows = (red + gx - 1) / gx;
  if (a.vbmax > 0 || red > 0) {
    const unsigned gy = (unsigned)(vg.red_rows + (a.vbmax > 0 ? a.m * a.nact : 0));
    hipLaunchKernelGGL(k_lr_v, dim3((unsigned)gx, gy), dim3(256), 0, st, a.in, a.x, a.perm, a.xsc, vg);
  }
  LrUGroup ug{a.act, a.mp, a.nact, a.T, a.n};
  hipLaunchKernelGGL(k_lr_u, dim3((unsigned)(a.outmax / 128), (unsigned)(a.m * a.nact)), dim3(256), 0, st, a.in,
                     a.perm, ug);
  return (int)hipGetLastError();
}

}  // namespace dc
