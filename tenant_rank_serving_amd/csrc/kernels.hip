// gfx950 kernels of libdeltacome.so: the shared-backbone product and the
// fp16 dequantizer.  The delta apply itself is in k_mx.hip.
//
// The apply is y = W_base x + U diag(sigma) (V x) per token, with the delta's
// singular pairs stored at 8, 3 and 2 bits in successive rank groups
// ("Delta-CoMe: Training-Free Delta-Compression with Mixed-Precision for
// LLMs", Approach and Key results; "Delta-CoMe - 清华联合OpenBMB...", technical
// principles).  Sums are fp32; the output is rounded to bf16 once.
#include <hip/hip_runtime.h>

#include "dc_internal.h"

namespace dc {
namespace {


typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
constexpr int kBufFlags = 0x00020000;   // buffer resource word 3: raw 32-bit dwords, bounds-checked


__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float f16_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

struct SegInfo {
  int b, lo, n;        // width, first global rank, count
  const uint8_t* vc;   // V codes region
  const uint32_t* vs;  // V scale/zero
  const uint8_t* uc;   // U codes region
  const uint32_t* us;  // U scale/zero
};

__host__ __device__ inline SegInfo seg_info(const Tenant& tn, const Layout& L, int which) {
  SegInfo s;
  const int rv[3] = {DC_REG_VC8, DC_REG_VC3, DC_REG_VC2};
  s.b = which == 0 ? 8 : (which == 1 ? 3 : 2);
  s.lo = which == 0 ? 0 : (which == 1 ? tn.n8 : tn.n8 + tn.n3);
  s.n = which == 0 ? tn.n8 : (which == 1 ? tn.n3 : tn.n2);
  s.vc = tn.base + L.off[rv[which]];
  s.vs = reinterpret_cast<const uint32_t*>(tn.base + L.off[rv[which] + 3]);
  s.uc = tn.base + L.off[rv[which] + 6];
  s.us = reinterpret_cast<const uint32_t*>(tn.base + L.off[rv[which] + 9]);
  return s;
}

// Code k (0..31) of a 32-code unit held in b words.
template <int B>
__device__ __forceinline__ uint32_t unit_code(const uint32_t* w, int k) {
  if constexpr (B == 8) {
    return (w[k >> 2] >> ((k & 3) * 8)) & 0xFFu;
  } else if constexpr (B == 2) {
    return (w[k >> 4] >> ((k & 15) * 2)) & 3u;
  } else {
    const int bit = 3 * k;
    const int wi = bit >> 5, sh = bit & 31;
    uint64_t v = w[wi] >> sh;
    if (sh > 29) v |= (uint64_t)w[wi + 1] << (32 - sh);
    return (uint32_t)v & 7u;
  }
}

// ----------------------------------------------------------- backbone GEMM
// ybase[t][o] = sum_j W[o][j] x[t][j] in fp32 with v_mfma_f32_16x16x32_bf16
// (A operand: lane l holds row l%16 of W, k = 8(l/16) .. +8 of a 32-step; B
// operand: token l%16, the same k; result: token l%16, rows 4(l/16) .. +4).
//
// Tiled form for many tokens (T > 256): 128 rows of W x 128 tokens per block,
// K in chunks of 64 staged through LDS in two buffers, rows padded by 16
// bytes so that the 16-byte operand reads of 8 consecutive lanes hit distinct
// banks.  Wave (wo, wt) computes the 64 x 64 quarter, 4 x 4 ops per 32-step.
// The next chunk's global loads are in flight while the current one is
// multiplied; one barrier per chunk (two or four chunks ahead in registers
// measured slower).  x is read in its row-major layout;
// tokens past T read the last token, and their columns are not stored.
// Consecutive workgroup ids go round-robin over the 8 XCDs, so tiles are
// numbered per XCD: each XCD takes a contiguous range of tiles, ordered as
// groups of 8 row tiles x all token tiles, so that the blocks it runs at one
// time share W rows and x rows in its L2.
constexpr int kGT = 128;                // rows of W and tokens per tile
constexpr int kGK = 64;                 // K per stage
constexpr int kGPad = kGK * 2 + 16;     // LDS row stride, bytes
constexpr int kGGroup = 8;              // row tiles per group

// One product c32[n][m] = sum_k A[m][k] B[n][k mod kb] (fp32, row stride
// ldc); A is [M][K] row-major (M a multiple of 128, K of 64), B [N][ldb].
constexpr int kGBatch = 8;

struct GemmOp {
  const uint16_t* A;
  const uint16_t* B;
  int32_t M, N, K, ldb, kb, ldc;
  float* c32;
};

// Up to kGBatch independent products per launch (blockIdx.y selects one;
// blocks past a product's tile count return at once).
struct GemmBatch {
  GemmOp op[kGBatch];
};
static_assert(kMaxGroup <= kGBatch, "a grouped call's backbone products fit one launch");

__global__ void __launch_bounds__(256, 2) k_gemm(GemmBatch gb) {
  const GemmOp& op = gb.op[blockIdx.y];
  const uint16_t* __restrict__ W = op.A;
  const uint16_t* __restrict__ x = op.B;
  const int out = op.M, T = op.N, in = op.K;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kGT * kGPad];   // [stage][W, x][row][144 B]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int nto = out / kGT, ntt = (T + kGT - 1) / kGT, total = nto * ntt;
  if (blockIdx.x >= (unsigned)total) return;
  const int xcd = blockIdx.x & 7, j8 = blockIdx.x >> 3;
  const int tile = xcd * (total >> 3) + min(xcd, total & 7) + j8;
  const int g = tile / (kGGroup * ntt), rem = tile - g * (kGGroup * ntt);
  const int gs = min(kGGroup, nto - g * kGGroup);
  const int o0 = (g * kGGroup + rem % gs) * kGT, t0 = (rem / gs) * kGT;
  // staging: piece it of a thread is row 32 it + tid/8, bytes 16 (tid%8) .. +16 of the chunk
  const uint16_t* wp[4];
  const uint16_t* xp[4];
  int so[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int row = it * 32 + (tid >> 3), c = tid & 7;
    wp[it] = W + (size_t)(o0 + row) * in + c * 8;
    xp[it] = x + (size_t)min(t0 + row, T - 1) * op.ldb + c * 8;
    so[it] = row * kGPad + c * 16;
  }
  // one chunk in flight, in register slot 0 (written this way, with the slot
  // index and a nested loop, the compiler keeps the loaded values in
  // registers; a flat loop over chunks made it stage them through scratch
  // memory, 4x slower)
  uint4 rw[1][4], rx[1][4];
  const int nk = in / kGK;
  auto gload = [&](int slot, int kc) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      rw[slot][it] = *reinterpret_cast<const uint4*>(wp[it] + (size_t)kc * kGK);
      rx[slot][it] = *reinterpret_cast<const uint4*>(xp[it] + (size_t)((kc * kGK) % op.kb));
    }
  };
  auto swrite = [&](int s, int slot) __attribute__((always_inline)) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      *reinterpret_cast<uint4*>(&lds[s][0][so[it]]) = rw[slot][it];
      *reinterpret_cast<uint4*>(&lds[s][1][so[it]]) = rx[slot][it];
    }
  };
  const int wo = wave >> 1, wt = wave & 1;
  const int ra = (64 * wo + (lane & 15)) * kGPad + (lane >> 4) * 16;
  const int rb = (64 * wt + (lane & 15)) * kGPad + (lane >> 4) * 16;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  gload(0, 0);
  swrite(0, 0);
  __syncthreads();
  for (int k0 = 0; k0 < nk; ++k0) {
#pragma unroll
    for (int d = 0; d < 1; ++d) {
      const int kc = k0 + d, s = kc & 1;
      // unconditional (the last chunk loads itself again), so that the loop
      // has no branch and the stores to LDS below wait for these loads only
      gload(0, min(kc + 1, nk - 1));
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        uint4 a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const uint4*>(&lds[s][0][ra + 16 * i * kGPad + ks * 64]);
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const uint4*>(&lds[s][1][rb + 16 * j * kGPad + ks * 64]);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                               __builtin_bit_cast(bf16x8, b[j]), acc[i][j], 0, 0, 0);
      }
      swrite(s ^ 1, 0);   // after the last chunk: unused
      __syncthreads();
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int tok = t0 + 64 * wt + 16 * j + (lane & 15);
    if (tok >= T) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = o0 + 64 * wo + 16 * i + 4 * (lane >> 4);   // rows m .. m+3 of this lane
      const f32x4 c = acc[i][j];
      *reinterpret_cast<f32x4*>(op.c32 + (size_t)tok * op.ldc + m) = c;
    }
  }
}

unsigned gemm_tiles(int M, int N) { return (unsigned)(M / kGT) * (unsigned)((N + kGT - 1) / kGT); }

// Split-K form for a few token groups (T <= 256): kBaseRows rows of W per
// block (wave w: rows 16w..16w+15) and one range of at most kSKSteps K-steps
// (blockIdx.y), so that the 8 waves share x: at the start wave w copies the
// 16-token tile w % 4 of x for half w / 4 of the range straight into LDS with
// direct-to-LDS loads (a fixed count, all in flight at once), next to the
// first kSKDepth K-steps of its W rows; after one barrier the loop streams W
// kSKDepth steps ahead with no further synchronization.  The partial sums
// go through LDS transposed, so that one wave instruction covers 64
// consecutive rows of one token.  A single range stores them; two ranges add
// them into ybase (zeroed by the prep kernel) with float atomics, which is
// order-independent for two terms; with more ranges every range stores its
// partial into bpt, and the blocks of the next kernel (the V side) add them
// in range order into ybase (the same bits on every run).
// kSKSteps (K-steps per range: 4 KB of x for 64 tokens each, 64 KB of LDS)
// is shared with the host's workspace sizing.
constexpr int kSKDepth = 8;    // W K-steps in flight per wave
typedef __attribute__((address_space(3))) void base_lds_t;

__device__ __forceinline__ void lds_barrier() {   // orders LDS only: W loads stay in flight
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The matrices of one launch (a group of matrices that read the same x):
// row block blockIdx.x belongs to the last matrix whose first row block is
// at or before it.
struct BaseMats {
  BaseMat m[kMaxGroup];
  int32_t nm;
};

__global__ void __launch_bounds__(kBaseWaves * 64) k_base_sk(BaseMats bms, const uint16_t* __restrict__ xt, int32_t in,
                                                 int32_t T, int32_t nks) {
  int mj = 0;
#pragma unroll
  for (int j = 1; j < kMaxGroup; ++j)
    if (j < bms.nm && (int)blockIdx.x >= bms.m[j].rb0) mj = j;
  const BaseMat bm = mj == 0 ? bms.m[0] : (mj == 1 ? bms.m[1] : (mj == 2 ? bms.m[2] : bms.m[3]));
  const uint16_t* __restrict__ W = bm.W;
  float* __restrict__ ybase = bm.ybase;
  float* __restrict__ bpt = bm.bpt;
  const int out = bm.out;
  __shared__ __attribute__((aligned(16))) uint4 xs[kSKSteps][4][64];   // [step][token tile][lane] B tiles
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r0 = (blockIdx.x - bm.rb0) * kBaseRows;
  const int t0 = blockIdx.z * 64;
  const int tiles = (T + 15) / 16;
  const int nall = in / 32;
  const int s0 = blockIdx.y * kSKSteps, nst = min(kSKSteps, nall - s0);   // this block's K-steps
  // x: wave w copies token tile w % 4 for the steps of half w / 4 of the range
  // (the last tile again past T: masked below)
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(xt), 0, nall * tiles * 1024, kBufFlags);
  const int tile = min(t0 / 16 + (wave & 3), tiles - 1);
  constexpr int kXSteps = kSKSteps * 4 / kBaseWaves;   // steps of x each wave copies
#pragma unroll
  for (int j = 0; j < kXSteps; ++j) {
    const int st = (wave >> 2) * kXSteps + j;
    const int ks = s0 + min(st, nst - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (base_lds_t*)&xs[st][wave & 3][0], 16,
                                             (ks * tiles + tile) * 1024 + lane * 16, 0, 0, 0);
  }
  // W: lane l holds row l%16 of the wave's 16, k = 8(l/16) .. +8 of a step
  const uint16_t* wa = W + (size_t)(r0 + 16 * wave + (lane & 15)) * in + (size_t)s0 * 32 + (lane >> 4) * 8;
  uint4 a[kSKDepth];
  auto load_a = [&](int slot, int st) __attribute__((always_inline)) {
    a[slot] = *reinterpret_cast<const uint4*>(wa + (size_t)min(st, nst - 1) * 32);
  };
#pragma unroll
  for (int d = 0; d < kSKDepth; ++d) load_a(d, d);
  uint32_t keep[4];   // all ones for a lane whose token exists
#pragma unroll
  for (int j = 0; j < 4; ++j) keep[j] = t0 + 16 * j + (lane & 15) < T ? ~0u : 0u;
  f32x4 acc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  lds_barrier();   // every wave's x copies have landed (the fence waits for them)
#pragma unroll
  for (int st = 0; st < kSKSteps; ++st) {
    const uint32_t live = st < nst ? ~0u : 0u;   // zero for the steps past the range
    uint4 av = a[st % kSKDepth];
    if (st + kSKDepth < kSKSteps) load_a(st % kSKDepth, st + kSKDepth);
    av.x &= live; av.y &= live; av.z &= live; av.w &= live;
    const bf16x8 ab = __builtin_bit_cast(bf16x8, av);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 bv = xs[st][j][lane];
      bv.x &= keep[j]; bv.y &= keep[j]; bv.z &= keep[j]; bv.w &= keep[j];
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, __builtin_bit_cast(bf16x8, bv), acc[j], 0, 0, 0);
    }
  }
  // D layout: lane holds token column lane%16 of tile j and rows 4(lane/16)+i
  // of the wave's 16; transpose to [token][row] (padded) over the x copies
  lds_barrier();
  constexpr int kRed = kBaseRows + 1;   // padded row of the transposed sums
  static_assert(64 * kRed * 4 <= (int)sizeof(xs), "the transposed sums fit over the x copies");
  float* red = reinterpret_cast<float*>(&xs[0][0][0]);   // [64 tokens][kRed]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(16 * j + (lane & 15)) * kRed + 16 * wave + 4 * (lane >> 4) + i] = acc[j][i];
  lds_barrier();
  const int ntok = min(64, T - t0);
  if (nks <= kMaxAtomicTerms) {
    for (int tl = wave; tl < ntok; tl += kBaseWaves) {   // wave: tokens wave, wave + 8, ..; lane: rows
#pragma unroll
      for (int rr = lane; rr < kBaseRows; rr += 64) {
        float* dst = ybase + (size_t)(t0 + tl) * out + r0 + rr;
        const float v = red[tl * kRed + rr];
        if (nks > 1)
          atomicAdd(dst, v);
        else
          *dst = v;
      }
    }
    return;
  }
  float* part = bpt + blockIdx.y * (size_t)T * out;   // this range's partials
  for (int tl = wave; tl < ntok; tl += kBaseWaves)
#pragma unroll
    for (int rr = lane; rr < kBaseRows; rr += 64) part[(size_t)(t0 + tl) * out + r0 + rr] = red[tl * kRed + rr];
}

// -------------------------------------------------------------- dequantize
// Exact fp32 value s*(q - z) of element pos of singular vector i (V_i when
// is_v, pos < in; else U_i, pos < out), from the tenant's packed codes.
__device__ __forceinline__ float dq_seg(const SegInfo& sg, bool is_v, int i, int pos, int in) {
  const int li = i - sg.lo;
  const int np = (int)round_up(sg.n, 4);
  uint32_t code, sz;
  if (is_v) {
    const int gi = in / kGroup;
    const int kk = pos % kGroup;
    const uint32_t* vw = reinterpret_cast<const uint32_t*>(sg.vc);
    const uint32_t* unit = sg.b == 8 ? vw + ((size_t)li * gi + pos / kGroup) * 32 + (kk / 32) * 8
                                     : vw + v_chunk_word(li, pos / kGroup, kk / 32, gi, sg.b);
    code = sg.b == 8 ? unit_code<8>(unit, kk % 32) : (sg.b == 3 ? unit_code<3>(unit, kk % 32) : unit_code<2>(unit, kk % 32));
    sz = sg.vs[(size_t)(pos / kGroup) * np + li];
  } else {
    if (sg.b == 8) {
      code = sg.uc[(size_t)pos * sg.n + li];
    } else {
      int nw;
      const uint32_t* wp = reinterpret_cast<const uint32_t*>(sg.uc) + u_kblock_word(pos, li / kKBlock, sg.n, sg.b, &nw);
      code = sg.b == 3 ? unit_code<3>(wp, li % kKBlock) : unit_code<2>(wp, li % kKBlock);
    }
    sz = sg.us[(size_t)(pos / kGroup) * np + li];
  }
  return f16_to_f32(sz & 0xFFFFu) * ((float)code - f16_to_f32(sz >> 16));   // exact in fp32
}

__device__ __forceinline__ float dq_value(const Tenant& tn, const Layout& L, bool is_v, int i, int pos, int in) {
  const int which = i < tn.n8 ? 0 : (i < tn.n8 + tn.n3 ? 1 : 2);
  return dq_seg(seg_info(tn, L, which), is_v, i, pos, in);
}

// fp16 bits of s*(q-z) for every element of U [r][out] and V [r][in].
__global__ void __launch_bounds__(256) k_dequant(Tenant tn, int32_t out, int32_t in, uint16_t* __restrict__ u16,
                                                 uint16_t* __restrict__ v16) {
  const int r = tn.n8 + tn.n3 + tn.n2;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t nv = (size_t)r * in, nu = (size_t)r * out;
  if (idx >= nv + nu) return;
  Layout L;
  layout_of(out, in, tn.n8, tn.n3, tn.n2, &L);
  const bool is_v = idx < nv;
  const int len = is_v ? in : out;
  const size_t e = is_v ? idx : idx - nv;
  const int i = (int)(e / len), pos = (int)(e % len);
  const uint16_t h = __builtin_bit_cast(uint16_t, (_Float16)dq_value(tn, L, is_v, i, pos, in));
  (is_v ? v16 : u16)[(size_t)i * len + pos] = h;
}

}  // namespace

int launch_base(const BaseMat* mats, int m, const uint16_t* x, const uint16_t* xt, int in, int T, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int nks = base_splits(in, T);
  if (nks > 0) {
    BaseMats bms{};
    int rows = 0;
    for (int j = 0; j < m; ++j) {
      bms.m[j] = mats[j];
      rows = mats[j].rb0 + mats[j].out / kBaseRows;
    }
    bms.nm = m;
    const dim3 g((unsigned)rows, (unsigned)nks, (unsigned)((T + 63) / 64));
    hipLaunchKernelGGL(k_base_sk, g, dim3(kBaseWaves * 64), 0, st, bms, xt, in, T, nks);
  } else {   // every matrix of the group in one launch of the tiled product
    GemmBatch gb{};
    unsigned tiles = 0;
    for (int j = 0; j < m; ++j) {
      GemmOp& op = gb.op[j];
      op.A = mats[j].W;
      op.B = x;
      op.M = mats[j].out;
      op.N = T;
      op.K = in;
      op.ldb = in;
      op.kb = in;
      op.ldc = mats[j].out;
      op.c32 = mats[j].ybase;
      const unsigned tj = gemm_tiles(mats[j].out, T);
      tiles = tj > tiles ? tj : tiles;
    }
    hipLaunchKernelGGL(k_gemm, dim3(tiles, (unsigned)m), dim3(256), 0, st, gb);
  }
  return (int)hipGetLastError();
}

int launch_tiled_base(const uint16_t* W, const uint16_t* x, float* ybase, int out, int in, int T, void* stream) {
  GemmOp op{};
  op.A = W;
  op.B = x;
  op.M = out;
  op.N = T;
  op.K = in;
  op.ldb = in;
  op.kb = in;
  op.ldc = out;
  op.c32 = ybase;
  GemmBatch gb{};
  gb.op[0] = op;
  hipLaunchKernelGGL(k_gemm, dim3(gemm_tiles(out, T)), dim3(256), 0, reinterpret_cast<hipStream_t>(stream), gb);
  return (int)hipGetLastError();
}

int launch_dequant(const Tenant& t, int32_t out, int32_t in, uint16_t* u16, uint16_t* v16, void* stream) {
  const size_t r = (size_t)t.n8 + t.n3 + t.n2;
  const size_t total = r * ((size_t)in + out);
  if (total == 0) return 0;
  hipLaunchKernelGGL(k_dequant, dim3((unsigned)((total + 255) / 256)), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), t, out, in, u16, v16);
  return (int)hipGetLastError();
}

}  // namespace dc
