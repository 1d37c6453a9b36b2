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

__device__ __forceinline__ SegInfo seg_info(const Tenant& tn, const Layout& L, int which) {
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
// ybase[t][o] = sum_j W[o][j] x[t][j] in fp32 with v_mfma_f32_16x16x32_bf16.
// Work item (block): 16 whole rows of W (one contiguous stretch of memory)
// and NT tiles of 16 tokens (blockIdx.y selects the group of 64 tokens).
// Each wave takes a quarter of the input columns for all 16 rows and all
// tokens, so every element of W is read once per 64 tokens.  W loads run
// kWDepth K-steps ahead of the matrix cores, x loads (1 KB B tiles written by
// the prep kernel) kXDepth steps ahead.  The step loop has no branches, so
// each step waits only for its own loads.  The four waves add their sums
// through LDS.
constexpr int kWDepth = 8;
constexpr int kXDepth = 4;

template <int NT>
__global__ void __launch_bounds__(256) k_base(const uint16_t* __restrict__ W, const uint16_t* __restrict__ xt,
                                              float* __restrict__ ybase, int32_t out, int32_t in, int32_t T,
                                              int32_t tg0) {
  __shared__ float red[4][16][65];   // [wave][row][token], padded
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r0 = blockIdx.x * 16;
  const int t0 = (tg0 + blockIdx.y) * 64;
  const int tiles = (T + 15) / 16;              // token tiles of x in total
  const int kspan = in / 4;                     // a multiple of 32: in is a multiple of 128
  const int kw = wave * kspan;
  const int nst = kspan / 32;                   // K-steps of this wave
  const int nsp = (nst + kWDepth - 1) / kWDepth * kWDepth;   // padded with zero steps
  const uint16_t* wa = W + (size_t)(r0 + (lane & 15)) * in + kw + (lane >> 4) * 8;
  // B tile (k-step kt, token tile tt) is 1 KB: lane l holds token 16tt + l%16, k = 32kt + 8(l/16) .. +8
  const uint16_t* xb = xt + ((size_t)(kw / 32) * tiles + t0 / 16) * 512 + lane * 8;
  uint32_t keep[NT];   // all ones for a lane whose token exists
#pragma unroll
  for (int j = 0; j < NT; ++j) keep[j] = t0 + 16 * j + (lane & 15) < T ? ~0u : 0u;
  f32x4 acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 a[kWDepth], b[kXDepth][NT];
  auto load_a = [&](int slot, int st) {
    a[slot] = *reinterpret_cast<const uint4*>(wa + (size_t)min(st, nst - 1) * 32);
  };
  auto load_b = [&](int slot, int st) {
    const uint16_t* p = xb + (size_t)min(st, nst - 1) * tiles * 512;
#pragma unroll
    for (int j = 0; j < NT; ++j) b[slot][j] = *reinterpret_cast<const uint4*>(p + j * 512);
  };
  auto step = [&](int sa, int sb, int st) {
    const uint32_t live = st < nst ? ~0u : 0u;   // zero for the padding steps
    uint4 av = a[sa];
    av.x &= live; av.y &= live; av.z &= live; av.w &= live;
    const bf16x8 ab = __builtin_bit_cast(bf16x8, av);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
      uint4 bv = b[sb][j];
      bv.x &= keep[j]; bv.y &= keep[j]; bv.z &= keep[j]; bv.w &= keep[j];
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ab, __builtin_bit_cast(bf16x8, bv), acc[j], 0, 0, 0);
    }
  };
#pragma unroll
  for (int d = 0; d < kWDepth; ++d) load_a(d, d);
#pragma unroll
  for (int d = 0; d < kXDepth; ++d) load_b(d, d);
  int s0 = 0;
  for (; s0 < nsp - kWDepth; s0 += kWDepth) {
#pragma unroll
    for (int d = 0; d < kWDepth; ++d) {
      step(d, d % kXDepth, s0 + d);
      load_a(d, s0 + d + kWDepth);
      load_b(d % kXDepth, s0 + d + kXDepth);
    }
  }
#pragma unroll
  for (int d = 0; d < kWDepth; ++d) {   // last kWDepth steps: no W loads left
    step(d, d % kXDepth, s0 + d);
    if (d + kXDepth < kWDepth) load_b(d % kXDepth, s0 + d + kXDepth);
  }
  // D layout: lane holds token column lane%16 of tile j and rows 4(lane/16)+i
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][4 * (lane >> 4) + i][16 * j + (lane & 15)] = acc[j][i];
  __syncthreads();
  const int ntok = min(64, T - t0);
  for (int c = tid; c < 16 * 64; c += 256) {
    const int row = c & 15, tl = c >> 4;   // consecutive threads: consecutive rows of one token
    if (tl < ntok)
      ybase[(size_t)(t0 + tl) * out + r0 + row] = (red[0][row][tl] + red[1][row][tl]) + (red[2][row][tl] + red[3][row][tl]);
  }
}

// Split-K form for a few token groups (T <= 256): 64 rows of W per block
// (wave w: rows 16w..16w+15) and one range of at most kSKSteps K-steps
// (blockIdx.y), so that the 4 waves share x: at the start each wave copies
// its 16-token tile of x for the whole range straight into LDS with
// direct-to-LDS loads (a fixed count, all in flight at once), next to the
// first kSKDepth K-steps of its W rows; after one barrier the loop streams W
// kSKDepth steps ahead with no further synchronization.  The partial sums
// go through LDS transposed, so that one wave instruction adds 64
// consecutive rows of one token into ybase (zeroed by the prep kernel) with
// float atomics; a single range stores them.
constexpr int kSKSteps = 16;   // K-steps per range: 4 KB of x (64 tokens) each, 64 KB of LDS
constexpr int kSKDepth = 8;    // W K-steps in flight per wave
typedef __attribute__((address_space(3))) void base_lds_t;

__device__ __forceinline__ void lds_barrier() {   // orders LDS only: W loads stay in flight
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__global__ void __launch_bounds__(256) k_base_sk(const uint16_t* __restrict__ W, const uint16_t* __restrict__ xt,
                                                 float* __restrict__ ybase, int32_t out, int32_t in, int32_t T,
                                                 int32_t nks) {
  __shared__ __attribute__((aligned(16))) uint4 xs[kSKSteps][4][64];   // [step][token tile][lane] B tiles
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r0 = blockIdx.x * 64;
  const int t0 = blockIdx.z * 64;
  const int tiles = (T + 15) / 16;
  const int nall = in / 32;
  const int s0 = blockIdx.y * kSKSteps, nst = min(kSKSteps, nall - s0);   // this block's K-steps
  // x: wave w copies token tile w (the last tile again past T: masked below)
  const __amdgpu_buffer_rsrc_t rx =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(xt), 0, nall * tiles * 1024, kBufFlags);
  const int tile = min(t0 / 16 + wave, tiles - 1);
#pragma unroll
  for (int st = 0; st < kSKSteps; ++st) {
    const int ks = s0 + min(st, nst - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rx, (base_lds_t*)&xs[st][wave][0], 16,
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
  float* red = reinterpret_cast<float*>(&xs[0][0][0]);   // [64][65]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[(16 * j + (lane & 15)) * 65 + 16 * wave + 4 * (lane >> 4) + i] = acc[j][i];
  lds_barrier();
  const int ntok = min(64, T - t0);
  for (int tl = wave; tl < ntok; tl += 4) {   // wave: tokens wave, wave + 4, ..; lane: row
    float* dst = ybase + (size_t)(t0 + tl) * out + r0 + lane;
    const float v = red[tl * 65 + lane];
    if (nks > 1)
      atomicAdd(dst, v);
    else
      *dst = v;
  }
}

// -------------------------------------------------------------- dequantize
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
  const int which = i < tn.n8 ? 0 : (i < tn.n8 + tn.n3 ? 1 : 2);
  const SegInfo sg = seg_info(tn, L, which);
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
  const float v = f16_to_f32(sz & 0xFFFFu) * ((float)code - f16_to_f32(sz >> 16));  // exact in fp32
  const uint16_t h = __builtin_bit_cast(uint16_t, (_Float16)v);
  (is_v ? v16 : u16)[(size_t)i * len + pos] = h;
}

}  // namespace

int base_splits(int out, int in, int T) {
  return T <= 256 ? (in / 32 + kSKSteps - 1) / kSKSteps : 0;
}

int launch_base(const uint16_t* W, const uint16_t* xt, float* ybase, int out, int in, int T, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int nks = base_splits(out, in, T);
  if (nks > 0) {
    const dim3 g((unsigned)(out / 64), (unsigned)nks, (unsigned)((T + 63) / 64));
    hipLaunchKernelGGL(k_base_sk, g, dim3(256), 0, st, W, xt, ybase, out, in, T, nks);
    return (int)hipGetLastError();
  }
  // full groups of 64 tokens, then the tail group with its own tile count
  const int full = T / 64, tail = (T % 64 + 15) / 16;
  const dim3 gf((unsigned)(out / 16), (unsigned)full), gt((unsigned)(out / 16), 1u);
  if (full > 0) hipLaunchKernelGGL(k_base<4>, gf, dim3(256), 0, st, W, xt, ybase, out, in, T, 0);
  switch (tail) {
    case 1: hipLaunchKernelGGL(k_base<1>, gt, dim3(256), 0, st, W, xt, ybase, out, in, T, full); break;
    case 2: hipLaunchKernelGGL(k_base<2>, gt, dim3(256), 0, st, W, xt, ybase, out, in, T, full); break;
    case 3: hipLaunchKernelGGL(k_base<3>, gt, dim3(256), 0, st, W, xt, ybase, out, in, T, full); break;
    case 4: hipLaunchKernelGGL(k_base<4>, gt, dim3(256), 0, st, W, xt, ybase, out, in, T, full); break;
    default: break;
  }
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
