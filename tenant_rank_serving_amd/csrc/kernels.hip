// gfx950 kernels of libdeltacome.so: routing, activation staging, the V-side
// and U-side of the mixed-precision delta apply, the shared-backbone product
// and the fp16 dequantizer.
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

constexpr int kTok = 8;      // tokens per register chunk in the delta kernels
constexpr int kRankChunk = 256;  // ranks staged in LDS by the U-side kernel

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

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

// ---------------------------------------------------------------- routing
struct SegArg {
  int32_t v[DC_MAX_TENANTS + 1];
};

// Counting sort of the tokens by tenant, stable.  Bucket n collects the
// backbone-only tokens (id -1, or an id outside [0, n), which also raises
// the flag word).  Writes offs[0..n+1] and perm[sorted position] = token.
__global__ void __launch_bounds__(1024) k_route(const int32_t* __restrict__ ids, int32_t T, int32_t n,
                                                int32_t mode, SegArg seg, int32_t* __restrict__ offs,
                                                int32_t* __restrict__ perm, uint32_t* __restrict__ flags) {
  const int tid = threadIdx.x;
  if (mode != 1) {
    for (int p = tid; p < T; p += blockDim.x) perm[p] = p;
    if (tid == 0) {
      if (mode == 0) {
        offs[0] = 0; offs[1] = T; offs[2] = T;
      } else {
        for (int k = 0; k <= n; ++k) offs[k] = seg.v[k];
        offs[n + 1] = T;
      }
      *flags = 0;
    }
    return;
  }
  __shared__ int cnt[DC_MAX_TENANTS + 1];
  __shared__ int next[DC_MAX_TENANTS + 1];
  __shared__ int bkt[1024];
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
    if (t < T) {
      const int k = ids[t];
      b = (k < 0 || k >= n) ? n : k;
    }
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
}

// ------------------------------------------------------- activation staging
// xs[p][j] = fp32(x[perm[p]][j]); four elements per thread.
__global__ void __launch_bounds__(256) k_xprep(const uint16_t* __restrict__ x, const int32_t* __restrict__ perm,
                                               float* __restrict__ xs, int32_t T, int32_t in) {
  const size_t q = (size_t)blockIdx.x * blockDim.x + threadIdx.x;  // quad index
  const size_t per_row = (size_t)in / 4;
  if (q >= per_row * T) return;
  const int p = (int)(q / per_row);
  const int j = (int)(q % per_row) * 4;
  const uint2 v = *reinterpret_cast<const uint2*>(x + (size_t)perm[p] * in + j);
  float4 o;
  o.x = __uint_as_float(v.x << 16);
  o.y = __uint_as_float(v.x & 0xFFFF0000u);
  o.z = __uint_as_float(v.y << 16);
  o.w = __uint_as_float(v.y & 0xFFFF0000u);
  *reinterpret_cast<float4*>(xs + (size_t)p * in + j) = o;
}

// ------------------------------------------------------------------ V side
// One wave per (tenant, rank): t[p][i] = sigma_i * sum_j s*(q_ij - z) x_pj for
// the tenant's tokens p.  Lanes walk 32-code units along the vector.
template <int B>
__device__ void vside_row(const uint32_t* __restrict__ row, const uint32_t* __restrict__ vs, int np, int li,
                          int in, const float* __restrict__ xs, int pc, int nt, int lane, float acc[kTok]) {
  const int units = in / 32;
  for (int u = lane; u < units; u += 64) {
    const uint32_t e = vs[(size_t)(u >> 2) * np + li];
    const float s = f16_to_f32(e & 0xFFFFu), z = f16_to_f32(e >> 16);
    uint32_t w[B];
#pragma unroll
    for (int q = 0; q < B; ++q) w[q] = row[(size_t)u * B + q];
#pragma unroll
    for (int k4 = 0; k4 < 32; k4 += 4) {
      float val[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        val[q] = s * ((float)unit_code<B>(w, k4 + q) - z);   // exact in fp32
        if constexpr (B == 8) val[q] = (float)(_Float16)val[q];  // 8-bit pairs: the fp16 dequantized value
      }
#pragma unroll
      for (int tt = 0; tt < kTok; ++tt) {
        if (tt < nt) {
          const float4 xv = *reinterpret_cast<const float4*>(xs + (size_t)(pc + tt) * in + u * 32 + k4);
          acc[tt] += val[0] * xv.x + val[1] * xv.y + val[2] * xv.z + val[3] * xv.w;
        }
      }
    }
  }
}

__global__ void __launch_bounds__(256) k_vside(TenantTable tt, int32_t out, int32_t in,
                                               const int32_t* __restrict__ offs, const float* __restrict__ xs,
                                               float* __restrict__ tv, int32_t rs) {
  const int k = blockIdx.y;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const Tenant tn = tt.t[k];
  const int r = tn.n8 + tn.n3 + tn.n2;
  const int i = blockIdx.x * 4 + wave;
  if (i >= r) return;
  const int p0 = offs[k], p1 = offs[k + 1];
  if (p0 >= p1) return;
  Layout L;
  layout_of(out, in, tn.n8, tn.n3, tn.n2, &L);
  const int which = i < tn.n8 ? 0 : (i < tn.n8 + tn.n3 ? 1 : 2);
  const SegInfo sg = seg_info(tn, L, which);
  const int li = i - sg.lo;
  const int np = (int)round_up(sg.n, 4);
  const int gi = in / kGroup;
  const uint32_t* row = reinterpret_cast<const uint32_t*>(sg.vc) + (size_t)li * gi * 4 * sg.b;
  const float sigma = reinterpret_cast<const float*>(tn.base + L.off[DC_REG_SIGMA])[i];
  for (int pc = p0; pc < p1; pc += kTok) {
    const int nt = min(kTok, p1 - pc);
    float acc[kTok];
#pragma unroll
    for (int q = 0; q < kTok; ++q) acc[q] = 0.f;
    if (sg.b == 8) vside_row<8>(row, sg.vs, np, li, in, xs, pc, nt, lane, acc);
    else if (sg.b == 3) vside_row<3>(row, sg.vs, np, li, in, xs, pc, nt, lane, acc);
    else vside_row<2>(row, sg.vs, np, li, in, xs, pc, nt, lane, acc);
#pragma unroll
    for (int q = 0; q < kTok; ++q) {
      float v = acc[q];
#pragma unroll
      for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
      acc[q] = v;
    }
    if (lane == 0)
      for (int q = 0; q < nt; ++q) tv[(size_t)(pc + q) * rs + i] = sigma * acc[q];
  }
}

// ------------------------------------------------------------------ U side
// One block of 128 threads per (128-row output group g, tenant); thread =
// output row.  t'_i = s_ig * t_i is staged in LDS; y = sum_i q_oi t'_i -
// sum_i z_ig t'_i, plus the backbone product, rounded once to bf16 and
// written at the token's original position.  Tenant index n is the
// backbone-only bucket.
__global__ void __launch_bounds__(128) k_uside(TenantTable tt, int32_t n, int32_t out, int32_t in,
                                               const int32_t* __restrict__ offs, const int32_t* __restrict__ perm,
                                               const float* __restrict__ tv, int32_t rs,
                                               const float* __restrict__ ybase, uint16_t* __restrict__ y) {
  const int g = blockIdx.x, k = blockIdx.y, tid = threadIdx.x;
  const int o = g * kGroup + tid;
  const int p0 = offs[k], p1 = offs[k + 1];
  if (p0 >= p1) return;
  if (k == n) {
    for (int p = p0; p < p1; ++p) {
      const int t = perm[p];
      const float v = ybase ? ybase[(size_t)t * out + o] : 0.f;
      y[(size_t)t * out + o] = f32_to_bf16(v);
    }
    return;
  }
  const Tenant tn = tt.t[k];
  Layout L;
  layout_of(out, in, tn.n8, tn.n3, tn.n2, &L);
  __shared__ float tp[kRankChunk][kTok];
  __shared__ float s8[kRankChunk], z8[kRankChunk];
  __shared__ float red[kTok][128];
  for (int pc = p0; pc < p1; pc += kTok) {
    const int nt = min(kTok, p1 - pc);
    float acc[kTok], cz[kTok];
#pragma unroll
    for (int q = 0; q < kTok; ++q) { acc[q] = 0.f; cz[q] = 0.f; }
    for (int which = 0; which < 3; ++which) {
      const SegInfo sg = seg_info(tn, L, which);
      if (sg.n == 0) continue;
      const int np = (int)round_up(sg.n, 4);
      const int n32 = (int)round_up(sg.n, kKBlock);
      for (int c0 = 0; c0 < sg.n; c0 += kRankChunk) {
        const int c1 = min(c0 + kRankChunk, n32);
        __syncthreads();
        for (int li = c0 + tid; li < c1; li += 128) {
          const uint32_t e = li < sg.n ? sg.us[(size_t)g * np + li] : 0u;
          const float s = f16_to_f32(e & 0xFFFFu), z = f16_to_f32(e >> 16);
          if (sg.b == 8) {  // 8-bit pairs use the fp16 dequantized values: keep t, s, z apart
            s8[li - c0] = s;
            z8[li - c0] = z;
          }
#pragma unroll
          for (int q = 0; q < kTok; ++q) {
            const float tvv = (q < nt && li < sg.n) ? tv[(size_t)(pc + q) * rs + sg.lo + li] : 0.f;
            if (sg.b == 8) {
              tp[li - c0][q] = tvv;
            } else {        // 3/2-bit: t' = s t, and the zero point folded into sum_i z t'
              const float tpv = s * tvv;
              tp[li - c0][q] = tpv;
              cz[q] += z * tpv;
            }
          }
        }
        __syncthreads();
        if (sg.b == 8) {
          const uint8_t* rowc = sg.uc + (size_t)o * sg.n;
          for (int li = c0; li < min(c0 + kRankChunk, sg.n); ++li) {
            const float uh = (float)(_Float16)(s8[li - c0] * ((float)rowc[li] - z8[li - c0]));
#pragma unroll
            for (int q = 0; q < kTok; ++q) acc[q] += uh * tp[li - c0][q];
          }
        } else {
          const uint32_t* uc = reinterpret_cast<const uint32_t*>(sg.uc);
          for (int kb = c0 / kKBlock; kb < c1 / kKBlock; ++kb) {
            int nw;
            const uint32_t* wp = uc + u_kblock_word(o, kb, sg.n, sg.b, &nw);
            uint32_t w[3] = {0u, 0u, 0u};
            for (int q = 0; q < nw; ++q) w[q] = wp[q];
            for (int kk = 0; kk < 32; ++kk) {
              const float c = (float)(sg.b == 3 ? unit_code<3>(w, kk) : unit_code<2>(w, kk));
              const int li = kb * 32 + kk - c0;
#pragma unroll
              for (int q = 0; q < kTok; ++q) acc[q] += c * tp[li][q];
            }
          }
        }
      }
    }
    // Deterministic tree reduction of sum_i z t' over the block.
#pragma unroll
    for (int q = 0; q < kTok; ++q) red[q][tid] = cz[q];
    __syncthreads();
    for (int h = 64; h >= 1; h >>= 1) {
      if (tid < h)
#pragma unroll
        for (int q = 0; q < kTok; ++q) red[q][tid] += red[q][tid + h];
      __syncthreads();
    }
    for (int q = 0; q < nt; ++q) {
      const int t = perm[pc + q];
      float v = acc[q] - red[q][0];
      if (ybase) v += ybase[(size_t)t * out + o];
      y[(size_t)t * out + o] = f32_to_bf16(v);
    }
    __syncthreads();
  }
}

// ----------------------------------------------------------- backbone GEMM
// ybase[t][o] = sum_j W[o][j] x[t][j] in fp32 with v_mfma_f32_16x16x32_bf16:
// each wave computes 16 rows x 16 tokens.
__global__ void __launch_bounds__(256) k_base(const uint16_t* __restrict__ W, const uint16_t* __restrict__ x,
                                              float* __restrict__ ybase, int32_t out, int32_t in, int32_t T) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int o0 = (blockIdx.x * 4 + wave) * 16;
  const int t0 = blockIdx.y * 16;
  if (o0 >= out) return;
  const int row = o0 + (lane & 15);
  const int kq = (lane >> 4) * 8;
  const int tok = t0 + (lane & 15);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const uint16_t* wp = W + (size_t)row * in + kq;
  const uint16_t* xp = x + (size_t)(tok < T ? tok : 0) * in + kq;
  for (int k0 = 0; k0 < in; k0 += 32) {
    const uint4 a = *reinterpret_cast<const uint4*>(wp + k0);
    uint4 b = *reinterpret_cast<const uint4*>(xp + k0);
    if (tok >= T) b = make_uint4(0, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                  acc, 0, 0, 0);
  }
  if (tok < T) {
#pragma unroll
    for (int j = 0; j < 4; ++j) ybase[(size_t)tok * out + o0 + (lane >> 4) * 4 + j] = acc[j];
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
    const uint32_t* grp = reinterpret_cast<const uint32_t*>(sg.vc) + ((size_t)li * gi + pos / kGroup) * 4 * sg.b;
    const int kk = pos % kGroup;
    const uint32_t* unit = grp + (kk / 32) * sg.b;
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

int launch_apply(const ApplyArgs& a) {
  hipStream_t st = reinterpret_cast<hipStream_t>(a.stream);
  uint32_t* flags = reinterpret_cast<uint32_t*>(a.ws + a.wl.flags);
  int32_t* offs = reinterpret_cast<int32_t*>(a.ws + a.wl.offs);
  int32_t* perm = reinterpret_cast<int32_t*>(a.ws + a.wl.perm);
  float* xs = reinterpret_cast<float*>(a.ws + a.wl.xs);
  float* tv = reinterpret_cast<float*>(a.ws + a.wl.tv);
  float* ybase = a.W ? reinterpret_cast<float*>(a.ws + a.wl.ybase) : nullptr;
  SegArg seg{};
  if (a.mode == 2)
    for (int k = 0; k <= a.n; ++k) seg.v[k] = a.seg[k];
  auto mark = [&](int s) {
    if (a.events && a.events[s]) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(a.events[s]), st);
  };
  mark(DC_STAGE_ROUTE);
  hipLaunchKernelGGL(k_route, dim3(1), dim3(1024), 0, st, a.ids, a.T, a.n, a.mode, seg, offs, perm, flags);
  mark(DC_STAGE_XPREP);
  const size_t quads = (size_t)a.T * a.in / 4;
  hipLaunchKernelGGL(k_xprep, dim3((unsigned)((quads + 255) / 256)), dim3(256), 0, st, a.x, perm, xs, a.T, a.in);
  mark(DC_STAGE_BASE);
  if (a.W)
    hipLaunchKernelGGL(k_base, dim3((unsigned)((a.out / 16 + 3) / 4), (unsigned)((a.T + 15) / 16)), dim3(256), 0, st,
                       a.W, a.x, ybase, a.out, a.in, a.T);
  mark(DC_STAGE_VSIDE);
  if (a.rmax > 0)
    hipLaunchKernelGGL(k_vside, dim3((unsigned)((a.rmax + 3) / 4), (unsigned)a.n), dim3(256), 0, st, *a.tenants,
                       a.out, a.in, offs, xs, tv, a.wl.rs);
  mark(DC_STAGE_USIDE);
  hipLaunchKernelGGL(k_uside, dim3((unsigned)(a.out / kGroup), (unsigned)(a.n + 1)), dim3(128), 0, st, *a.tenants,
                     a.n, a.out, a.in, offs, perm, tv, a.wl.rs, ybase, a.y);
  mark(DC_STAGE_COUNT);
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
