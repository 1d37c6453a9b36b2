// gfx950 kernels of libdeltacome.so: quantize and pack one delta on the GPU.
//
// The compression step of the pages keeps the singular pairs in descending
// singular-value order, the first n8 at 8 bits, the next n3 at 3 and the
// next n2 at 2 ("Delta-CoMe - 清华联合OpenBMB...", technical principles;
// "Delta-CoMe: Training-Free Delta-Compression with Mixed-Precision for
// LLMs", Approach).  The quantizer (per 128-element group: min/max range
// with zero included, fp16 scale rounded once from fp64, integer zero,
// round half to even) and the packed format are this library's, stated in
// include/deltacome.h; the results are bit-identical to dc_pack on the host.
#include <hip/hip_runtime.h>

#include "dc_internal.h"

namespace dc {
namespace {

__global__ void __launch_bounds__(256) k_pack_zero(uint32_t* __restrict__ p, size_t nwords,
                                                   uint32_t* __restrict__ flag) {
  const size_t i0 = (size_t)blockIdx.x * 256 + threadIdx.x;
  for (size_t i = i0; i < nwords; i += (size_t)gridDim.x * 256) p[i] = 0u;
  if (i0 == 0) *flag = 0u;
}

// Quantizer of one 128-element group held two values per lane (elements
// 2l, 2l+1 in lane l): fp32 min/max (exact) of the range with zero included,
// then fp64 arithmetic.  Returns false (for every lane) on a non-finite value
// or an fp16 overflow of the scale; the clamps are compare-and-select, as
// in the host quantizer (an all-zero group keeps z = -0.0).
struct GroupQ {
  uint32_t q0, q1;   // codes of the lane's two elements
  uint32_t sz;       // fp16 scale | fp16 zero << 16
};

__device__ __forceinline__ bool quant_group(float2 wv, int b, GroupQ& g) {
  if (__ballot(!isfinite(wv.x) || !isfinite(wv.y))) return false;
  float mn = fminf(0.f, fminf(wv.x, wv.y)), mx = fmaxf(0.f, fmaxf(wv.x, wv.y));
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    mn = fminf(mn, __shfl_xor(mn, d, 64));
    mx = fmaxf(mx, __shfl_xor(mx, d, 64));
  }
  const int maxq = (1 << b) - 1;
  uint16_t sh = f64_to_f16(((double)mx - (double)mn) / (double)maxq);
  if ((sh & 0x7FFF) == 0) sh = 0x3C00;   // 1.0
  if ((sh & 0x7C00) == 0x7C00) return false;
  const double s = f16_to_f64(sh);
  auto clampq = [&](double v) {
    if (v < 0.0) v = 0.0;
    if (v > (double)maxq) v = (double)maxq;
    return v;
  };
  const double z = clampq(rint(-(double)mn / s));
  g.q0 = (uint32_t)clampq(rint((double)wv.x / s) + z);
  g.q1 = (uint32_t)clampq(rint((double)wv.y / s) + z);
  g.sz = (uint32_t)sh | ((uint32_t)f64_to_f16(z) << 16);
  return true;
}

// Segment (width, first pair, count) of pair i.
__device__ __forceinline__ void seg_of_pair(int i, int n8, int n3, int n2, int& which, int& b, int& lo, int& n) {
  which = i < n8 ? 0 : (i < n8 + n3 ? 1 : 2);
  b = which == 0 ? 8 : (which == 1 ? 3 : 2);
  lo = which == 0 ? 0 : (which == 1 ? n8 : n8 + n3);
  n = which == 0 ? n8 : (which == 1 ? n3 : n2);
}

constexpr int kPackBatch = 2;   // groups whose loads a wave issues before the first is quantized
constexpr int kUParts = 8;      // waves per (128-row group, K-block) on the U side: 4 pairs each

// Region byte offsets of the packed buffer (computed once on the host; the
// host rejects buffers of 2 GiB or more, so 32 bits suffice).
struct PackOffs {
  uint32_t off[DC_REG_COUNT];
};

// V side and the U side of 8-bit pairs: items (pair i, 128-element group),
// V groups first, kPackBatch consecutive items per wave; the wave writes
// every word of its groups itself (no atomics).
__device__ __forceinline__ void quant_v_item(int w, float2 wv, int32_t out, int32_t in, int32_t n8, int32_t n3,
                                             int32_t n2, const PackOffs& L, const float* __restrict__ sigma,
                                             uint8_t* __restrict__ dst, uint32_t* __restrict__ flag);

__global__ void __launch_bounds__(256) k_quant_v(int32_t out, int32_t in, int32_t n8, int32_t n3, int32_t n2,
                                                 PackOffs L, const float* __restrict__ U, const float* __restrict__ sigma,
                                                 const float* __restrict__ V, uint8_t* __restrict__ dst,
                                                 uint32_t* __restrict__ flag) {
  const int lane = threadIdx.x & 63;
  const int r = n8 + n3 + n2, gi = in / kGroup, go = out / kGroup;
  const int nv = r * gi, nall = nv + n8 * go;
  const int w0 = (int)(blockIdx.x * 4 + (threadIdx.x >> 6)) * kPackBatch;
  if (w0 >= nall) return;
  float2 wv[kPackBatch];
#pragma unroll
  for (int j = 0; j < kPackBatch; ++j) {   // all loads first (items past the end reload the last one)
    const int w = min(w0 + j, nall - 1);
    const bool vs = w < nv;
    const int wl = vs ? w : w - nv;
    const int ng = vs ? gi : go;
    const int i = wl / ng, grp = wl % ng;
    const float* src = (vs ? V + (size_t)i * in : U + (size_t)i * out) + (size_t)grp * kGroup;
    wv[j] = reinterpret_cast<const float2*>(src)[lane];
  }
#pragma unroll
  for (int j = 0; j < kPackBatch; ++j)
    if (w0 + j < nall) quant_v_item(w0 + j, wv[j], out, in, n8, n3, n2, L, sigma, dst, flag);
}

__device__ __forceinline__ void quant_v_item(int w, float2 wv, int32_t out, int32_t in, int32_t n8, int32_t n3,
                                             int32_t n2, const PackOffs& L, const float* __restrict__ sigma,
                                             uint8_t* __restrict__ dst, uint32_t* __restrict__ flag) {
  const int lane = threadIdx.x & 63;
  const int r = n8 + n3 + n2, gi = in / kGroup;
  const int nv = r * gi;
  const bool vside = w < nv;
  const int wl = vside ? w : w - nv;
  const int ng = vside ? gi : out / kGroup;
  const int i = wl / ng, grp = wl % ng;
  int which, b, lo, n;
  seg_of_pair(i, n8, n3, n2, which, b, lo, n);
  const int li = i - lo;
  if (vside && grp == 0 && lane == 0) {   // sigma, stored unquantized
    const float sg = sigma[i];
    if (!isfinite(sg)) atomicOr(flag, 1u);
    reinterpret_cast<float*>(dst + L.off[DC_REG_SIGMA])[i] = sg;
  }
  GroupQ g;
  if (!quant_group(wv, b, g)) {
    if (lane == 0) atomicOr(flag, 1u);
    return;
  }
  const int np = (int)round_up((size_t)n, 4);
  // region offsets by selects on constant indices (a computed index would put L in scratch)
  const size_t off_sz = vside ? (which == 0 ? L.off[DC_REG_VS8] : (which == 1 ? L.off[DC_REG_VS3] : L.off[DC_REG_VS2]))
                              : L.off[DC_REG_US8];
  if (lane == 0) reinterpret_cast<uint32_t*>(dst + off_sz)[(size_t)grp * np + li] = g.sz;   // [group][pad4(n)]
  if (!vside) {   // 8-bit U codes: bytes [out][n8], one writer per byte
    const int o0 = grp * kGroup + 2 * lane;
    uint8_t* uc = dst + L.off[DC_REG_UC8];
    uc[(size_t)o0 * n8 + li] = (uint8_t)g.q0;
    uc[(size_t)(o0 + 1) * n8 + li] = (uint8_t)g.q1;
    return;
  }
  if (b == 8) {   // [n8][Gi][32] words: word w = codes 4w..4w+3 (lanes 2w, 2w+1)
    const uint32_t mine = g.q0 | (g.q1 << 8);
    const uint32_t nb = __shfl_down(mine, 1, 64);
    if ((lane & 1) == 0)
      reinterpret_cast<uint32_t*>(dst + L.off[DC_REG_VC8])[((size_t)li * gi + grp) * 32 + (lane >> 1)] = mine | (nb << 16);
    return;
  }
  // 3/2-bit: lane l holds codes 2m, 2m+1 (m = l % 16) of chunk l / 16; its 2b
  // bits sit at bit 2bm of the chunk's b-word stream; OR over the 16 lanes
  const int m = lane & 15, bit = 2 * b * m;
  const uint64_t c = (uint64_t)(g.q0 | (g.q1 << b));
  uint32_t wd[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) {
    const int sh = bit - 32 * j;   // position of c inside word j
    wd[j] = sh >= 32 || sh <= -2 * b ? 0u : (uint32_t)(sh >= 0 ? c << sh : c >> -sh);
  }
#pragma unroll
  for (int d = 1; d < 16; d <<= 1)
#pragma unroll
    for (int j = 0; j < 3; ++j) wd[j] |= __shfl_xor(wd[j], d, 64);
  if (m < b) {   // lane m of the chunk writes word m
    uint32_t* words = reinterpret_cast<uint32_t*>(dst + (which == 1 ? L.off[DC_REG_VC3] : L.off[DC_REG_VC2])) +
                      v_chunk_word(li, grp, lane >> 4, gi, b);
    words[m] = m == 0 ? wd[0] : (m == 1 ? wd[1] : wd[2]);
  }
}

// U side of 3- and 2-bit pairs: one wave per (128-row group, K-block of 32
// pairs of one segment, one of kUParts parts of the K-block).  It quantizes
// its pairs (each pair's 128 rows, two per lane), ORs their codes into
// registers holding the words of the lane's two rows, and ORs those into
// memory (the parts of a K-block share the words; OR is order-free).
__global__ void __launch_bounds__(256) k_quant_u(int32_t out, int32_t in, int32_t n8, int32_t n3, int32_t n2,
                                                 PackOffs L, const float* __restrict__ U, uint8_t* __restrict__ dst,
                                                 uint32_t* __restrict__ flag) {
  const int lane = threadIdx.x & 63;
  const int go = out / kGroup;
  const int kb3 = (n3 + kKBlock - 1) / kKBlock, kb2 = (n2 + kKBlock - 1) / kKBlock;
  const int w = (int)(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (w >= go * (kb3 + kb2) * kUParts) return;
  const int qt = w % kUParts, grp = (w / kUParts) % go, kbi = (w / kUParts) / go;
  const bool three = kbi < kb3;
  const int b = three ? 3 : 2, n = three ? n3 : n2, lo = three ? n8 : n8 + n3, kb = three ? kbi : kbi - kb3;
  const int np = (int)round_up((size_t)n, 4);
  uint32_t* us = reinterpret_cast<uint32_t*>(dst + (three ? L.off[DC_REG_US3] : L.off[DC_REG_US2]));
  uint32_t* uc = reinterpret_cast<uint32_t*>(dst + (three ? L.off[DC_REG_UC3] : L.off[DC_REG_UC2]));
  uint32_t r0w[3] = {0u, 0u, 0u}, r1w[3] = {0u, 0u, 0u};   // the K-block's words of rows 2l and 2l+1
  constexpr int kPer = kKBlock / kUParts;   // pairs per wave
  const int k0 = qt * kPer, k1 = min(min(kKBlock, n - kb * kKBlock), k0 + kPer);
  if (k0 >= k1) return;
  float2 wv[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {   // the wave's pairs' loads go out together
    const int lj = kb * kKBlock + min(k0 + j, k1 - 1);
    wv[j] = reinterpret_cast<const float2*>(U + (size_t)(lo + lj) * out + (size_t)grp * kGroup)[lane];
  }
  for (int k = k0; k < k1; ++k) {
    const int li = kb * kKBlock + k;
    GroupQ g;
    float2 cur = wv[0];
#pragma unroll
    for (int j = 1; j < kPer; ++j)
      if (k - k0 == j) cur = wv[j];
    if (!quant_group(cur, b, g)) {
      if (lane == 0) atomicOr(flag, 1u);
      return;
    }
    if (lane == 0) us[(size_t)grp * np + li] = g.sz;
    const int bit = b * k, wi = bit >> 5, sh = bit & 31;
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const uint32_t lo0 = wi == j ? g.q0 << sh : 0u, lo1 = wi == j ? g.q1 << sh : 0u;
      const uint32_t hi0 = (wi + 1 == j && sh + b > 32) ? g.q0 >> (32 - sh) : 0u;
      const uint32_t hi1 = (wi + 1 == j && sh + b > 32) ? g.q1 >> (32 - sh) : 0u;
      r0w[j] |= lo0 | hi0;
      r1w[j] |= lo1 | hi1;
    }
  }
  const int o0 = grp * kGroup + 2 * lane;
  int nw;
  uint32_t* w0 = uc + u_kblock_word(o0, kb, n, b, &nw);
  uint32_t* w1 = uc + u_kblock_word(o0 + 1, kb, n, b, &nw);
  for (int j = 0; j < nw; ++j) {
    const uint32_t a = j == 0 ? r0w[0] : (j == 1 ? r0w[1] : r0w[2]);
    const uint32_t c = j == 0 ? r1w[0] : (j == 1 ? r1w[1] : r1w[2]);
    if (a) atomicOr(w0 + j, a);
    if (c) atomicOr(w1 + j, c);
  }
}

// ------------------------------------------------------------ error table
// "Enhancing Delta Compression in LLMs via SVD-based Quantization Error
// Minimization", §2.1 eq. 5: quantizing row i of V at b bits costs about
// sigma_i^2 times the squared norm of (V̂_i - V_i) X over calibration columns
// X.  Two kernels: every (row, width) difference row V̂_i - V_i (the same
// quantizer as the packer; width 0 = the row dropped, -V_i), then one
// product of the stacked differences with X whose epilogue sums the squares.
struct ErrWidths {
  int32_t b[DC_ERR_MAX_WIDTHS];
  int32_t nw;
};

// One wave per (row i, 128-group): the group at every width, two elements
// per lane; dv row (i, k) holds V̂_i - V_i at width k (fp32: the fp16 value
// minus an fp32 value within a factor two of it is exact).
__global__ void __launch_bounds__(256) k_err_dv(int32_t r, int32_t in, const float* __restrict__ V, ErrWidths W,
                                                float* __restrict__ dv, uint32_t* __restrict__ flag) {
  const int lane = threadIdx.x & 63;
  const int gi = in / kGroup;
  const int w = (int)(blockIdx.x * 4 + (threadIdx.x >> 6));
  if (w >= r * gi) return;
  const int i = w / gi, grp = w % gi;
  const float2 wv = reinterpret_cast<const float2*>(V + (size_t)i * in + (size_t)grp * kGroup)[lane];
  for (int k = 0; k < W.nw; ++k) {
    const int b = W.b[k];
    float2 d = make_float2(-wv.x, -wv.y);
    if (b > 0) {
      GroupQ g;
      if (quant_group(wv, b, g)) {
        const float sc = (float)f16_to_f64((uint16_t)(g.sz & 0xFFFFu)), z = (float)f16_to_f64((uint16_t)(g.sz >> 16));
        d.x = (float)(_Float16)(sc * ((float)g.q0 - z)) - wv.x;
        d.y = (float)(_Float16)(sc * ((float)g.q1 - z)) - wv.y;
      } else if (lane == 0) {
        atomicOr(flag, 1u);
      }
    } else if (__ballot(!isfinite(wv.x) || !isfinite(wv.y)) && lane == 0) {
      atomicOr(flag, 1u);
    }
    reinterpret_cast<float2*>(dv + ((size_t)i * W.nw + k) * in + (size_t)grp * kGroup)[lane] = d;
  }
}

// err[row] = sigma_i^2 sum_c (sum_j dv[row][j] X[j][c])^2, row = i nw + k:
// block = 64 rows x every column in chunks of 64; thread = 4 rows x 4
// columns of a chunk; K in steps of 32 through LDS.  Products in fp32, the
// squares and their sums in fp64, in a fixed order.
constexpr int kErrRows = 64, kErrCols = 64, kErrK = 32;

__global__ void __launch_bounds__(256) k_err_gemm(int32_t R, int32_t in, int32_t ncal, int32_t nw,
                                                  const float* __restrict__ dv, const float* __restrict__ X,
                                                  const float* __restrict__ sigma, double* __restrict__ err) {
  __shared__ float As[kErrK][kErrRows + 4];   // [k][row]
  __shared__ float Bs[kErrK][kErrCols + 4];   // [k][column]
  const int tid = threadIdx.x, tx = tid & 15, ty = tid >> 4;
  const int row0 = blockIdx.x * kErrRows;
  double ss[4] = {0.0, 0.0, 0.0, 0.0};
  for (int c0 = 0; c0 < ncal; c0 += kErrCols) {
    float acc[4][4] = {};
    for (int k0 = 0; k0 < in; k0 += kErrK) {
      {  // A: row tid / 4, k (tid % 4) * 8 .. +8
        const int ar = tid >> 2, ak = (tid & 3) * 8;
        float4 a0 = make_float4(0.f, 0.f, 0.f, 0.f), a1 = a0;
        if (row0 + ar < R) {
          const float4* src = reinterpret_cast<const float4*>(dv + (size_t)(row0 + ar) * in + k0 + ak);
          a0 = src[0];
          a1 = src[1];
        }
        As[ak + 0][ar] = a0.x; As[ak + 1][ar] = a0.y; As[ak + 2][ar] = a0.z; As[ak + 3][ar] = a0.w;
        As[ak + 4][ar] = a1.x; As[ak + 5][ar] = a1.y; As[ak + 6][ar] = a1.z; As[ak + 7][ar] = a1.w;
      }
      {  // B: k tid / 8, columns (tid % 8) * 8 .. +8
        const int bk = tid >> 3, bc = (tid & 7) * 8;
        const float* src = X + (size_t)(k0 + bk) * ncal + c0 + bc;
#pragma unroll
        for (int j = 0; j < 8; ++j) Bs[bk][bc + j] = c0 + bc + j < ncal ? src[j] : 0.f;
      }
      __syncthreads();
#pragma unroll 8
      for (int kk = 0; kk < kErrK; ++kk) {
        float a[4], b[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          a[q] = As[kk][4 * ty + q];
          b[q] = Bs[kk][4 * tx + q];
        }
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int c = 0; c < 4; ++c) acc[q][c] = fmaf(a[q], b[c], acc[q][c]);
      }
      __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
      for (int c = 0; c < 4; ++c) ss[q] += (double)acc[q][c] * (double)acc[q][c];   // columns past ncal are 0
  }
  // sum over the 16 threads of a row group (consecutive lanes), in a fixed order
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) ss[q] += __shfl_xor(ss[q], d, 64);
  if (tx == 0) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int row = row0 + 4 * ty + q;
      if (row < R) {
        const double sg = (double)sigma[row / nw];
        err[row] = sg * sg * ss[q];
      }
    }
  }
}

}  // namespace

int launch_pack(int32_t out, int32_t in, int32_t n8, int32_t n3, int32_t n2, const float* U, const float* sigma,
                const float* V, uint8_t* dst, uint32_t* flag, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  Layout Lh;
  layout_of(out, in, n8, n3, n2, &Lh);
  PackOffs L;
  for (int k = 0; k < DC_REG_COUNT; ++k) L.off[k] = (uint32_t)Lh.off[k];
  const size_t nwords = Lh.total / 4;
  const size_t zb = std::max<size_t>(std::min<size_t>((nwords + 255) / 256, 4096), 1);   // one block clears the flag
  hipLaunchKernelGGL(k_pack_zero, dim3((unsigned)zb), dim3(256), 0, st,
                     reinterpret_cast<uint32_t*>(dst), nwords, flag);
  const int r = n8 + n3 + n2, gi = in / kGroup, go = out / kGroup;
  const int64_t wv = ((int64_t)r * gi + (int64_t)n8 * go + kPackBatch - 1) / kPackBatch;   // waves
  if (wv > 0)
    hipLaunchKernelGGL(k_quant_v, dim3((unsigned)((wv + 3) / 4)), dim3(256), 0, st, out, in, n8, n3, n2, L, U, sigma,
                       V, dst, flag);
  const int64_t wu = (int64_t)go * ((n3 + kKBlock - 1) / kKBlock + (n2 + kKBlock - 1) / kKBlock) * kUParts;
  if (wu > 0)
    hipLaunchKernelGGL(k_quant_u, dim3((unsigned)((wu + 3) / 4)), dim3(256), 0, st, out, in, n8, n3, n2, L, U, dst,
                       flag);
  return (int)hipGetLastError();
}

int launch_error_table(int32_t r, int32_t in, int32_t ncal, const float* sigma, const float* V, const float* X,
                       const int32_t* widths, int32_t nw, double* err, uint32_t* flag, float* dv, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  ErrWidths W{};
  for (int k = 0; k < nw; ++k) W.b[k] = widths[k];
  W.nw = nw;
  hipLaunchKernelGGL(k_pack_zero, dim3(1), dim3(256), 0, st, reinterpret_cast<uint32_t*>(err), (size_t)0, flag);
  const int64_t waves = (int64_t)r * (in / kGroup);
  if (waves > 0) {
    hipLaunchKernelGGL(k_err_dv, dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, st, r, in, V, W, dv, flag);
    const int32_t R = r * nw;
    hipLaunchKernelGGL(k_err_gemm, dim3((unsigned)((R + kErrRows - 1) / kErrRows)), dim3(256), 0, st, R, in, ncal, nw,
                       dv, X, sigma, err);
  }
  return (int)hipGetLastError();
}

}  // namespace dc
