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

#include <type_traits>

#include "dc_internal.h"

namespace dc {
namespace {

#include "mx_common.h"
#include "combine.h"
#include "vstage.h"

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

// The region offsets of a work item's packed buffer (sizes are not carried).
__device__ __forceinline__ void layout_of_item(const ActEntry& e, Layout* L) {
#pragma unroll
  for (int i = 0; i < DC_REG_COUNT; ++i) L->off[i] = e.off[i];
  L->total = e.total;
}

struct SegArg {
  int32_t v[DC_MAX_TENANTS + 1];
};

// Rows of the routing permutation the routing block keeps in LDS for the
// work items' token lists (past them it reads them back from memory).
constexpr int kPermLds = 2048;

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
// Work items of the buckets with tokens, in bucket order: thread b (bucket
// b) gets its items' first list position and count, and every thread the
// list length.  The same for every matrix of a group (the buckets are the
// routing's), so it is worked out once.
struct ActPos {
  int pos, items, total;
};
__device__ __forceinline__ ActPos act_positions(int32_t n, const int* so) {
  __shared__ int wsum[4];
  const int tid = threadIdx.x, b = tid, lane = tid & 63, wave = tid >> 6;
  // work items of bucket b: its rows in chunks of kChunkRows
  const int rows = b <= n ? so[b + 1] - so[b] : 0;
  const int items = (rows + kChunkRows - 1) / kChunkRows;
  int v = items;   // inclusive scan over the buckets
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int u = __shfl_up(v, d, 64);
    if (lane >= d) v += u;
  }
  if (lane == 63) wsum[wave] = v;
  lds_barrier();
  int pos = v - items, total = 0;
  for (int w = 0; w < 4; ++w) {
    if (w < wave) pos += wsum[w];
    total += wsum[w];
  }
  lds_barrier();   // wsum is read: a next call may write it
  return ActPos{pos, items, total};
}

// Bucket b's work items of one matrix (its tenant record, region offsets and
// derived U sizes, rows) at list positions pos .. pos + items - 1.
template <class TokAt>
__device__ __forceinline__ void act_write_bucket(const Tenant& mine, int b, int32_t n, const int* so, int pos,
                                                 int items, ActEntry* __restrict__ act, int32_t out, int32_t in,
                                                 bool layouts, TokAt tok_at) {
  ActEntry e{};
  e.base = b < n ? mine.base : nullptr;
  e.n8 = b < n ? mine.n8 : 0;
  e.n3 = b < n ? mine.n3 : 0;
  e.n2 = b < n ? mine.n2 : 0;
  e.k = b;
  if (layouts && b < n && items > 0) {
    Layout L;
    layout_of(out, in, e.n8, e.n3, e.n2, &L);
#pragma unroll
    for (int i = 0; i < DC_REG_COUNT; ++i) e.off[i] = (uint32_t)L.off[i];
    e.total = (uint32_t)L.total;
    e.tb3 = t_base(e.n8, e.n3, 1);
    e.tb2 = t_base(e.n8, e.n3, 2);
    e.np8 = (int)round_up(e.n8, 4);
    e.np3 = (int)round_up(e.n3, 4);
    e.np2 = (int)round_up(e.n2, 4);
    e.nc3 = (e.n3 + kGroup - 1) / kGroup;
    e.nc = e.nc3 + (e.n2 + kGroup - 1) / kGroup;
    e.rw3 = u_row_words(e.n3, 3);
    e.rw2 = u_row_words(e.n2, 2);
    e.kbn3 = (e.n3 + kKBlock - 1) / kKBlock;
    e.kbn2 = (e.n2 + kKBlock - 1) / kKBlock;
    e.wl3 = e.rw3 - (e.kbn3 - 1) * 3;
    e.wl2 = e.rw2 - (e.kbn2 - 1) * 2;
  }
  for (int j = 0; j < items; ++j) {
    e.p0 = so[b] + j * kChunkRows;
    e.p1 = min(so[b] + (j + 1) * kChunkRows, so[b + 1]);
#pragma unroll
    for (int r = 0; r < kChunkRows; ++r) e.tok[r] = tok_at(min(e.p0 + r, e.p1 - 1));
    act[pos + j] = e;
  }
}

template <int M>
struct GroupTables {
  TenantTable t[M];
};

// Per matrix of the group: its work-item list and what prep clears.
struct PrepMats {
  MatParams params[kMaxGroup];
  MatParams* mp;              // where they go in the workspace
  ActEntry* act[kMaxGroup];
  float* tv[kMaxGroup];       // t, when its slices add up atomically
  int32_t ntv[kMaxGroup];
  float* yb[kMaxGroup];       // W x, when its two K ranges add up atomically
  int32_t nyb[kMaxGroup];
  uint32_t* cnt[kMaxGroup];   // arrival counters of the fixed-order sums
  int32_t ncnt[kMaxGroup];
  int32_t layouts;            // Delta-CoMe buffers: the work items carry their region offsets
};

// (matrix j, bucket b) pair of thread tid (j-major over M (n + 1) pairs): its
// tenant record goes out with the routing's first loads.
template <int M>
__device__ __forceinline__ Tenant first_record(const GroupTables<M>& gt, int32_t n) {
  const int tid = threadIdx.x, nb = n + 1;
  const int j = tid / nb, b = tid - j * nb;
  return tid < M * nb && b < n ? gt.t[j].t[b] : Tenant{};
}

// Every matrix's work-item list: the buckets' items (thread tid takes the
// pairs tid, tid + 256, ..., so the matrices' lists are written side by
// side), then empty entries up to cap.
template <int M, class TokAt>
__device__ __forceinline__ void act_write_all(const GroupTables<M>& gt, const Tenant& first, int32_t n,
                                              const int* so, const ActPos& ap, int32_t cap, const PrepMats& pm,
                                              int32_t in, TokAt tok_at) {
  __shared__ int spos[DC_MAX_TENANTS + 1], sitems[DC_MAX_TENANTS + 1];
  const int tid = threadIdx.x, nb = n + 1;
  if (tid < nb) {
    spos[tid] = ap.pos;
    sitems[tid] = ap.items;
  }
  lds_barrier();
  for (int idx = tid; idx < M * nb; idx += blockDim.x) {
    const int j = idx / nb, b = idx - j * nb;
    const Tenant mine = idx == tid ? first : (b < n ? gt.t[j].t[b] : Tenant{});
    act_write_bucket(mine, b, n, so, spos[b], sitems[b], pm.act[j], pm.params[j].out, in, pm.layouts != 0, tok_at);
  }
#pragma unroll
  for (int j = 0; j < M; ++j)
    for (int i = ap.total + tid; i < cap; i += blockDim.x) {   // the rest of the list: empty entries
      ActEntry e{};
      e.k = -1;
      pm.act[j][i] = e;
    }
}

template <int M>
__global__ void __launch_bounds__(256) k_prep(GroupTables<M> gt, const uint16_t* __restrict__ x,
                                              const int32_t* __restrict__ ids,
                                              int32_t T, int32_t in, int32_t n, int32_t mode, SegArg seg,
                                              int32_t* __restrict__ offs, int32_t* __restrict__ perm,
                                              uint32_t* __restrict__ flags, uint8_t* __restrict__ xf,
                                              uint32_t* __restrict__ xsc, float* __restrict__ xsum,
                                              uint16_t* __restrict__ xt, PrepMats pm, int32_t cap) {
  const int tid = threadIdx.x;
  // zeroed by the blocks after the first (the first block's barriers would
  // wait for its stores to finish)
  if (blockIdx.x > 0) {
    const int i0 = (blockIdx.x - 1) * 256 + tid, di = (gridDim.x - 1) * 256;
#pragma unroll
    for (int j = 0; j < M; ++j) {
      for (int i = i0; i < pm.ntv[j]; i += di) pm.tv[j][i] = 0.f;
      for (int i = i0; i < pm.nyb[j]; i += di) pm.yb[j][i] = 0.f;
      for (int i = i0; i < pm.ncnt[j]; i += di) pm.cnt[j][i] = 0u;
    }
  }
  if (blockIdx.x == 0) {
    static_assert(DC_MAX_TENANTS + 1 <= 256, "one thread per bucket");
#pragma unroll
    for (int j = 0; j < M; ++j)
      if (tid == j) pm.mp[j] = pm.params[j];
    __shared__ int so[DC_MAX_TENANTS + 2];   // bucket starts
    // token tid's tenant id, then thread b's tenant records: both in flight
    // together (the kernel arguments live in memory and the indexing is per
    // thread)
    const int k_first = mode == 1 && tid < T ? ids[tid] : -1;
    const Tenant first = first_record(gt, n);
    if (mode != 1) {
      for (int p = tid; p < T; p += blockDim.x) perm[p] = p;
      if (tid == 0) {
        if (mode == 0) { so[0] = 0; so[1] = T; so[2] = T; }
        else { for (int k = 0; k <= n; ++k) so[k] = seg.v[k]; so[n + 1] = T; }
        for (int k = 0; k <= n + 1; ++k) offs[k] = so[k];
        *flags = 0;
      }
      lds_barrier();
      const ActPos ap = act_positions(n, so);
      act_write_all(gt, first, n, so, ap, cap, pm, in, [](int p) { return p; });
      return;
    }
    __shared__ int cnt[DC_MAX_TENANTS + 1];   // tokens per bucket
    __shared__ int next[DC_MAX_TENANTS + 1];
    __shared__ __attribute__((aligned(16))) int bkt[256];
    __shared__ int bad;
    __shared__ int wsum[4];
    __shared__ int permL[kPermLds];   // the permutation's first kPermLds rows, for the work items
    for (int b = tid; b <= n; b += blockDim.x) cnt[b] = 0;
    if (tid == 0) bad = 0;
    lds_barrier();
    int b0 = -1;   // bucket of token tid (the first chunk is kept for the placement below)
    for (int t = tid; t < T; t += blockDim.x) {
      int k = t == tid ? k_first : ids[t];
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
        const int pos = next[b] + rank;
        perm[pos] = t;
        if (pos < kPermLds) permL[pos] = t;
      }
      lds_barrier();
      if (t < T) atomicAdd(&next[b], 1);
      lds_barrier();
    }
    // past kPermLds rows the work items read the permutation back from
    // memory: a full barrier makes this block's stores of it visible
    if (T > kPermLds) __syncthreads();
    const ActPos ap = act_positions(n, so);
    auto tok_at = [&](int p) { return p < kPermLds ? permL[p] : perm[p]; };
    act_write_all(gt, first, n, so, ap, cap, pm, in, tok_at);
    return;
  }
  const int gi_n = in / kGroup;
  const size_t item = (size_t)(blockIdx.x - 1) * 4 + (tid >> 6);
  if (item >= (size_t)T * gi_n) return;
  const int lane = tid & 63;
  const int t = (int)(item / gi_n), gi = (int)(item % gi_n);
  // fragments, scales and sums in token order (the V side finds a work
  // item's tokens in the item)
  const size_t sitem = (size_t)t * gi_n + gi;
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
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
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


// kVTiles 16-rank tiles of one wave (starting at tile0 of the segment) over
// one input slice, all tokens; the block's other waves run the same slice.
// live_wave: any of the wave's tiles holds a rank of the segment.
template <int B>
__device__ void vside_blk(const Seg& sg, int tbase, int tile0, bool live_wave, int in, int s,
                          const Tok8 tok, int p0, int p1, const uint8_t* __restrict__ xf,
                          const uint32_t* __restrict__ xsc, const float* __restrict__ xsum,
                          const float* __restrict__ sigma, const VOut& vo, VLds& S) {
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
  static_assert(kChunkRows == kVRows, "a work item is one pass");
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
    sig[h] = rv[h] ? gload(sigma + sg.lo + li[h]) : 0.f;   // a global load: a flat one would make every wait drain
  }
  const int tr = col & 7;              // token row of this lane's A operand
  const int piece = col >> 3;          // 0: hi pieces, 1: lo pieces
  {
    const int pb = p0;
    const int nt = min(kVRows, p1 - pb);
    VStage st;
    v_stage_load(st, xf, xsc, xsum, gi_n, g0, tok, nt);   // ahead of the ring: vmcnt is in order
    // Every wave issues the ring's first loads, also one with no rank of the
    // segment (its code offsets are past the region: out of range, no memory
    // request): loads on every path keep the waits for the x tiles exact.
    VGrp<B> ring[kDepth];
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {   // in group order: the first group's wait leaves the rest in flight
      v_load_grp<B>(ring[d], P, np, min(g0 + d, glast));
      __builtin_amdgcn_sched_barrier(0);
    }
    v_stage_store(S, st);
    __syncthreads();
    if (!live_wave) return;
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
          if (rv[h] && 4 * q + r < nt) v_put(vo, s, pb + 4 * q + r, tbase + li[h], sig[h] * acc[h][r]);
    }
  }
}

// 8-bit rows of a tenant over one input slice on the vector ALU with the fp16
// dequantized weights fp16(s (q - z)).  Thread tid owns 8 inputs of the
// slice, a pass's kVRows token rows and 4 rows at a time; the block sums per
// (row, token) and adds sigma * partial into t.
__device__ void vside_8bit(const Tenant& tn, const Layout& L, int in, int s, const uint16_t* __restrict__ x,
                           const Tok8 tok, int p0, int p1, const VOut& vo) {
  constexpr int kR = 2;   // rows per step: few live registers, so the V kernel fits 4 waves per SIMD
  __shared__ float red[4][kR][kVRows];   // [wave][row][token row]
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
      xv[t] = *reinterpret_cast<const uint4*>(x + (size_t)pick8u(tok, min(t, nt - 1)) * in + ic);
    for (int r0 = 0; r0 < sg.n; r0 += kR) {
      uint2 cw[kR];
      uint32_t e[kR];
#pragma unroll
      for (int u = 0; u < kR; ++u) {
        const int i = min(r0 + u, sg.n - 1);
        cw[u] = *reinterpret_cast<const uint2*>(sg.vc + (size_t)i * in + ic);
        e[u] = sg.vs[(size_t)gi * np + i];
      }
      // partials of the live (row, token) pairs only: with a few tokens most
      // of the kR x kVRows pairs are padding
      const int nu = min(kR, sg.n - r0);
      float part[kR][kVRows];
#pragma unroll
      for (int u = 0; u < kR; ++u) {
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
      for (int u = 0; u < kR; ++u)
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
      if (tid < kR * kVRows) {
        const int u = tid / kVRows, t = tid % kVRows;
        if (r0 + u < sg.n && t < nt)
          v_put(vo, s, pb + t, r0 + u, sigma[r0 + u] * ((red[0][u][t] + red[1][u][t]) + (red[2][u][t] + red[3][u][t])));
      }
      __syncthreads();
    }
  }
}

// The V-side launch of a group of matrices: leading grid rows add the
// backbone partials of matrices whose W x has more than two K ranges, then
// one row of blocks per (matrix, work item).
struct VGroup {
  const ActEntry* act;           // [m][nact] work items
  const MatParams* mp;           // [m] per-matrix parameters (workspace)
  BaseSum bs[kMaxGroup];
  int32_t red0[kMaxGroup + 1];   // first partial-sum block of each matrix (prefix over the group)
  int32_t red_rows;              // grid rows of partial-sum blocks
  int32_t nact;                  // work items per matrix
  int32_t ns, T;                 // V-side input slices, tokens
  int32_t m;                     // matrices of the group
  uint32_t mmagic, nsmagic;      // ceil(2^32 / m), ceil(2^32 / ns) (when above 1): division by multiply-high
};

// q / d for the block indices here (q < 2^16): the multiply-high by
// ceil(2^32 / d) is exact for q < 2^32 / d; d = 1 passes magic 0.
__device__ __forceinline__ int div_magic(int q, uint32_t magic) {
  return magic == 0u ? q : (int)__umulhi((uint32_t)q, magic);
}
inline uint32_t magic_of(int d) {
  return d > 1 ? (uint32_t)((0x100000000ull + (uint64_t)d - 1) / (uint64_t)d) : 0u;
}

__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) k_vside(int32_t n, int32_t in, const uint16_t* __restrict__ x,
                                               const int32_t* __restrict__ perm, const uint8_t* __restrict__ xf,
                                               const uint32_t* __restrict__ xsc, const float* __restrict__ xsum,
                                               VGroup g) {
  if ((int)blockIdx.y < g.red_rows) {   // the backbone product's partial sums
    const int idx = blockIdx.y * gridDim.x + blockIdx.x;
#pragma unroll
    for (int j = 0; j < kMaxGroup; ++j)
      if (idx >= g.red0[j] && idx < g.red0[j + 1]) base_sum(g.bs[j], idx - g.red0[j]);
    return;
  }
  const int yy = blockIdx.y - g.red_rows;
  // rows item-major, matrix fastest: every matrix's work items (listed
  // first) run before the empty entries of any
  const int item = div_magic(yy, g.mmagic);
  const int mj = yy - item * g.m;
  const MatParams P = g.mp[mj];
  const ActEntry e = g.act[mj * g.nact + item];   // the item-th work item of matrix mj
  const VOut vo{P.tv, P.vpt, P.vcnt, P.rs, g.ns, g.T, P.vb};
  const int out = P.out;
  const int p0 = e.p0, p1 = e.p1;
  if (p0 >= p1 || e.k >= n) return;     // empty entry, or the backbone-only bucket
  Tenant tn;
  tn.base = e.base;
  tn.n8 = e.n8;
  tn.n3 = e.n3;
  tn.n2 = e.n2;
  tn.pad_ = 0;
  const int ns = vo.ns;
  const int bv = div_magic(blockIdx.x, g.nsmagic);   // rank block (counter index)
  int b = bv;
  const int s = blockIdx.x - bv * ns;
  if (b >= v_blocks(tn.n8, tn.n3, tn.n2)) return;
  Layout L;
  layout_of_item(e, &L);
  if (tn.n8 > 0) {
    if (b == 0) {
      vside_8bit(tn, L, in, s, x, tok8_of(e.tok), p0, p1, vo);
      v_combine(vo, item, bv, p0, p1, 0, tn.n8);
      return;
    }
    --b;
  }
  __shared__ VLds S;
  const float* sigma = reinterpret_cast<const float*>(tn.base + L.off[DC_REG_SIGMA]);
  const int wave = threadIdx.x >> 6;
  const int b3 = (tn.n3 + kVRanks - 1) / kVRanks;
  const bool three = b < b3;
  const int tile0 = ((three ? b : b - b3) * 4 + wave) * kVTiles;
  const int sn = three ? tn.n3 : tn.n2;
  const int tb = t_base(tn.n8, tn.n3, three ? 1 : 2);
  if (three)
    vside_blk<3>(seg_of(tn, L, 1), tb, tile0, tile0 * 16 < sn, in, s, tok8_of(e.tok), p0, p1, xf, xsc, xsum, sigma, vo, S);
  else
    vside_blk<2>(seg_of(tn, L, 2), tb, tile0, tile0 * 16 < sn, in, s, tok8_of(e.tok), p0, p1, xf, xsc, xsum, sigma, vo, S);
  // ranks of this block: kVRanks consecutive ranks of its segment
  const int rb0 = (three ? b : b - b3) * kVRanks;
  v_combine(vo, item, bv, p0, p1, tb + rb0, min(kVRanks, sn - rb0));
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
// The first window's loads go out as one burst: A-prep inputs, the 8-bit
// pairs' inputs, the ring, W x; the barriers order LDS only and leave the
// burst in flight.
// The epilogue sums each token's three piece rows, takes sum_i z_ig t'_i
// off, adds the 8-bit pairs and W x and rounds once to bf16.
constexpr int kURows = 8;     // token rows per pass
constexpr int kUWaves = 8;    // waves per block, one 16-row tile each
constexpr int kU8Max = 2;     // 8-bit pairs whose U weights a lane keeps in registers
constexpr int kUDepth = 4;    // chunks of codes in flight per lane (register ring)
constexpr int kUWin = 16;     // A operands per window (chunks x ops): 16 chunks with one op, 8 with two

struct ULds {
  uint16_t frag[kUWin][4][16][16];   // [chunk * ops + op][lane group][A row][32 bytes]
  uint8_t sc[kUWin][kURows][4];      // E8M0 of the hi piece per (chunk, token row, K-block)
  float cz[kUWaves][kURows];         // per-wave partial sums of z t' per token row
};

// The U-side launch of a group of matrices: one row of blocks per (matrix,
// work item), blocks past a matrix's output groups return at once.
struct UGroup {
  const ActEntry* act;   // [m][nact] work items
  const MatParams* mp;   // [m] per-matrix parameters (workspace)
  int32_t nact;
  int32_t m;             // matrices of the group
  uint32_t mmagic;       // ceil(2^32 / m) for m > 1 (div_magic)
};

__global__ void __launch_bounds__(kUWaves * 64) __attribute__((amdgpu_waves_per_eu(4))) k_uside(int32_t n, int32_t in, const int32_t* __restrict__ perm,
                                                        int32_t T, UGroup ug) {
  const int g = blockIdx.x;
  // rows item-major, matrix fastest: every matrix's work items (listed
  // first) run before the empty entries of any
  const int yy = blockIdx.y;
  const int item = div_magic(yy, ug.mmagic);
  const int mj = yy - item * ug.m;
  const MatParams P = ug.mp[mj];
  const ActEntry e = ug.act[mj * ug.nact + item];
  // every field in hand before the first branch: one scalar round trip
  asm volatile("" ::"s"(P.tv), "s"(P.ybase), "s"(P.y), "s"(P.out), "s"(P.rs), "s"(e.base), "s"(e.n8), "s"(e.n3),
               "s"(e.n2), "s"(e.k), "s"(e.p0), "s"(e.p1), "s"(n), "s"(in), "s"(perm), "s"(T));
  asm volatile("" ::"s"(e.off[DC_REG_UC8]), "s"(e.off[DC_REG_UC3]), "s"(e.off[DC_REG_UC2]), "s"(e.off[DC_REG_US8]),
               "s"(e.off[DC_REG_US3]), "s"(e.off[DC_REG_US2]), "s"(e.total));
  asm volatile("" ::"s"(e.tb3), "s"(e.tb2), "s"(e.np8), "s"(e.np3), "s"(e.np2), "s"(e.nc3), "s"(e.nc), "s"(e.rw3),
               "s"(e.rw2), "s"(e.kbn3), "s"(e.kbn2), "s"(e.wl3), "s"(e.wl2));
  const Tok8 etok = tok8_of(e.tok);
  const int out = P.out;
  if (g * kGroup >= out) return;
  const int rs = P.rs;
  const float* __restrict__ tv = P.tv;
  const float* __restrict__ ybase = P.ybase;
  uint16_t* __restrict__ y = P.y;
  const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 15, q = lane >> 4;
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
  const int n8 = e.n8, n3 = e.n3, n2 = e.n2;
  const int tb3 = e.tb3, tb2 = e.tb2;
  const int nc3 = e.nc3, nc = e.nc, nc2 = nc - nc3;
  const int tot = (int)e.total;
  const int orow = g * kGroup + wave * 16 + col;
  const __amdgpu_buffer_rsrc_t rt =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(tv), 0, T * rs * 4, kBufFlags);
  // the tenant's whole packed buffer; an offset of tot (its size) is out of
  // range: such a load returns zeros without a memory request
  const __amdgpu_buffer_rsrc_t rten =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(e.base), 0, tot, kBufFlags);
  const int ou3 = (int)e.off[DC_REG_US3] + g * e.np3 * 4, ou2 = (int)e.off[DC_REG_US2] + g * e.np2 * 4;
  // Codes of chunk c of this lane: K-block kb = 4c + q of row orow.  Full
  // K-blocks of a 16-row tile sit 16 b words apart and hold b words per row;
  // the last one holds wl words per row; past it nothing (offset tot).
  const int row = orow & 15, tile = orow >> 4;
  const int a3 = (int)e.off[DC_REG_UC3] + (tile * 16 * e.rw3 + q * 16 * 3 + row * 3) * 4;
  const int l3 = (int)e.off[DC_REG_UC3] + (tile * 16 * e.rw3 + (e.kbn3 - 1) * 16 * 3 + row * e.wl3) * 4;
  const int a2 = (int)e.off[DC_REG_UC2] + (tile * 16 * e.rw2 + q * 16 * 2 + row * 2) * 4;
  const int l2 = (int)e.off[DC_REG_UC2] + (tile * 16 * e.rw2 + (e.kbn2 - 1) * 16 * 2 + row * e.wl2) * 4;
  const int kl3 = e.kbn3 - 1, kl2 = e.kbn2 - 1;
  auto load3 = [&](uint32_t (&w)[3], int c) __attribute__((always_inline)) {
    const int kb = 4 * c + q;
    const int off = kb < kl3 ? a3 + c * (4 * 16 * 3 * 4) : (kb == kl3 ? l3 : tot);
    const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rten, off, 0, 0);
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
  };
  auto load2 = [&](uint32_t (&w)[2], int j) __attribute__((always_inline)) {
    const int kb = 4 * j + q;
    const int off = kb < kl2 ? a2 + j * (4 * 16 * 2 * 4) : (kb == kl2 ? l2 : tot);
    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rten, off, 0, 0);
    w[0] = v.x;
    w[1] = v.y;
  };
  // 8-bit U weights of this lane's output row (first kU8Max pairs): scale
  // word and code, loaded behind the first window's A-prep inputs and codes,
  // dequantized to fp16 in the epilogue
  uint32_t u8s[kU8Max], u8c[kU8Max];
  // (with no 8-bit pairs both point at the buffer's first word: every load stays inside it)
  const int ous8 = n8 > 0 ? (int)e.off[DC_REG_US8] + g * e.np8 * 4 : 0;
  const int ouc8 = n8 > 0 ? (int)e.off[DC_REG_UC8] + orow * n8 : 0;
  auto load_u8 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kU8Max; ++i) {   // unconditional (unused past n8): straight-line waits
      const int i8 = min(i, max(n8 - 1, 0));
      u8s[i] = __builtin_amdgcn_raw_buffer_load_b32(rten, ous8 + i8 * 4, 0, 0);
      u8c[i] = __builtin_amdgcn_raw_buffer_load_b8(rten, ouc8 + i8, 0, 0);
    }
  };
  // rows 12-15 of every op carry no piece: zeroed once, behind the first loads
  auto zero_rows = [&]() __attribute__((always_inline)) {
    for (int i = tid; i < kUWin * 4 * 4; i += kUWaves * 64) {   // i = operand:4 lane group:2 row:2
      uint4* p = reinterpret_cast<uint4*>(S.frag[i >> 4][(i >> 2) & 3][12 + (i & 3)]);
      p[0] = make_uint4(0, 0, 0, 0);
      p[1] = make_uint4(0, 0, 0, 0);
    }
  };
  // A-prep role: K-block kb4 and ranks m0..m0+3 of a chunk (which chunk and
  // rows depend on the pass: see aprep)
  const int kb4 = (tid >> 3) & 3, part = tid & 7;
  const int m0 = kb4 * 32 + part * 4;
  const int lg_even = 2 * (kb4 & 1), hw = (kb4 >= 2 ? 8 : 0) + part;   // lane group, 16-bit word
  const int ps = col >> 2, tr4 = col & 3;   // MFMA lane's A row: piece ps of token 4 op + tr4
  static_assert(kChunkRows == kURows, "a work item is one pass");
  {
    const int pb = p0;
    const int nt = min(kURows, p1 - pb);
    const int nops = (nt + 3) >> 2;   // matrix-core ops per tile and chunk
    const int wcap = nops == 1 ? kUWin : kUWin / 2;   // chunks per window
    // The codes stream through two register rings: the 3-bit chunks (slot
    // c % 2) and the 2-bit chunks (slot j % 4).  Windows start their 3-bit
    // part on an even chunk and their 2-bit part on a multiple of 4, so the
    // slots of an unrolled loop are fixed; a step past the last chunk reloads
    // an out-of-range slot (zeros, no memory request).
    uint32_t cr3[2][3], cr2[4][2];
    f32x4 acc[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    // the epilogue's inputs, in flight during the pass: lane group q writes
    // tokens 2q and 2q + 1 of the pass (their original indices, then W x and
    // t of the 8-bit pairs).  The token indices go out right behind the
    // A-prep inputs: the W x loads, last in the burst, wait for them alone.
    int tko[2];
    float ybo[2] = {0.f, 0.f}, t8o[2][kU8Max];
    auto load_tko = [&]() __attribute__((always_inline)) {   // from the work item's token list
#pragma unroll
      for (int h = 0; h < 2; ++h) tko[h] = pick8(etok, min(2 * q + h, nt - 1));
    };
    auto epi_loads_t8 = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int rw = min(2 * q + h, nt - 1);
#pragma unroll
        for (int i = 0; i < kU8Max; ++i)
          t8o[h][i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rt, ((pb + rw) * rs + i) * 4, 0, 0));
      }
      load_u8();
    };
    // two loads whether or not there is a W x (then two distinct words of t,
    // unused): straight-line code, so the waits for earlier loads are exact
    auto epi_loads_yb = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int h = 0; h < 2; ++h) ybo[h] = gload(ybase ? ybase + (size_t)tko[h] * out + orow : tv + h);
    };
    auto epi_select = [&]() __attribute__((always_inline)) {   // values past what the matrix has are zero
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        ybo[h] = ybase ? ybo[h] : 0.f;
#pragma unroll
        for (int i = 0; i < kU8Max; ++i) t8o[h][i] = i < n8 ? t8o[h][i] : 0.f;
      }
    };
    // A operands of one window: its 3-bit chunks w3 .. w3 + n3w - 1, then
    // its 2-bit chunks j0 .. j0 + n2w - 1, at window-local chunk index pcl,
    // for the pass's token rows.  Thread tid takes chunk pcl and rows
    // 4h..4h+3: with one op per chunk the 512 threads cover 16 chunks x rows
    // 0-3, with two 8 chunks x both halves.  The inputs (scale/zero words, t)
    // are loaded apart from the math, so that the first window's code rings
    // and the epilogue's inputs go out in the same burst behind them (vmcnt
    // is in order: the math then waits for its own loads only).
    const int pcl = nops == 1 ? tid >> 5 : (tid & 255) >> 5;
    const int hh = nops == 1 ? 0 : tid >> 8;
    struct APIn {
      u32x4 usw;
      f32x4 tt[4];
    };
    // Threads past the window's chunks or their segment's ranks, and token
    // rows past the pass's, load nothing: their offset is the resource's
    // record count, out of range, so the load returns zeros without a memory
    // request (the math masks those values anyway).
    auto aprep_load = [&](int w3, int n3w, int j0, int n2w, APIn& ai) __attribute__((always_inline)) {
      const bool three = pcl < n3w;
      const int li = (three ? w3 + pcl : j0 + pcl - n3w) * kGroup + m0;
      const bool live = pcl < n3w + n2w && li < (three ? n3 : n2);
      ai.usw = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rten, live ? li * 4 + (three ? ou3 : ou2) : tot, 0, 0));
#pragma unroll
      for (int r = 0; r < 4; ++r)
        ai.tt[r] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                       rt, live && 4 * hh + r < nt ? ((pb + 4 * hh + r) * rs + (three ? tb3 : tb2) + li) * 4 : T * rs * 4,
                       0, 0));
    };
    auto aprep = [&](int w3, int n3w, int j0, int n2w, const APIn& ai) __attribute__((always_inline)) {
      const bool cok = pcl < n3w + n2w;
      const bool three = pcl < n3w;
      const int sn = three ? n3 : n2;
      const int li = (three ? w3 + pcl : j0 + pcl - n3w) * kGroup + m0;
      const u32x4 usw = ai.usw;
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int r = 4 * hh + r4;
        if (r >= nt) break;   // rows past the pass's tokens: their D rows are never read
        float tp[4];
        float mx = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const bool ok = cok && li + u < sn;
          tp[u] = ok ? f16f(usw[u] & 0xFFFFu) * ai.tt[r4][u] : 0.f;
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
    // the matrix-core ops of window-local chunk cl against B operand bop
    // (fp6 or fp4 codes); NOPS is the pass's ops per chunk
    auto mops = [&](auto nops_c, int cl, const v8i& bop, auto three_c) __attribute__((always_inline)) {
      constexpr int NOPS = decltype(nops_c)::value;
      constexpr bool THREE = decltype(three_c)::value;
#pragma unroll
      for (int op = 0; op < NOPS; ++op) {   // one A operand at a time: its registers are free again after hold()
        const uint4* f = reinterpret_cast<const uint4*>(S.frag[cl * NOPS + op][q][col]);
        const v8i a = v8_of(f[0], f[1]);
        int scv = S.sc[cl][4 * op + tr4][q];   // read by every lane (no branch): rows 12-15 take 127
        asm volatile("" : "+v"(scv));
        const int sa = ps < 3 ? scv - 5 * ps : 127;
        f32x4 d = {0.f, 0.f, 0.f, 0.f};
        d = THREE ? mma(a, bop, d, sa, kFmtFp6, kScaleFp6Code) : mma(a, bop, d, sa, kFmtFp4, kScaleFp4Code);
        hold(d, a, bop, sa, THREE ? kScaleFp6Code : kScaleFp4Code);
        acc[op] += d;
      }
      asm volatile("" : "+v"(acc[0]), "+v"(acc[1]));   // sums land here, not deferred to the end
    };
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using B3 = std::integral_constant<bool, true>;
    using B2 = std::integral_constant<bool, false>;
    // the matrix-core ops of one window; every step reloads its slot
    // (straight-line loads, exact waits), the ops of a step past the
    // window's chunks are skipped
    // The first round of each ring runs outside the loops and whether or not
    // the window has chunks of that width: in a loop, or behind a branch, the
    // wait for a slot must hold on every path into it, and would cover the
    // loads issued behind the slot's (W x among them).  A step past the
    // window's chunks skips its ops and reloads the chunk its slot holds
    // (past the last chunk that is out of range: zeros, no memory request).
    auto run = [&](auto nops_c, int w3, int n3w, int j0, int n2w) __attribute__((always_inline)) {
      auto step3 = [&](int c) __attribute__((always_inline)) {   // c - w3 even: slots 0 and 1
#pragma unroll
        for (int d = 0; d < 2; ++d) {
          const bool live = c + d < w3 + n3w;
          if (live) mops(nops_c, c + d - w3, b_fp6(cr3[d][0], cr3[d][1], cr3[d][2]), B3{});
          load3(cr3[d], live ? c + d + 2 : c + d);
        }
      };
      auto step2 = [&](int j) __attribute__((always_inline)) {   // j - j0 a multiple of 4: slots 0-3
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          const bool live = j + d < j0 + n2w;
          if (live) mops(nops_c, n3w + j + d - j0, b_fp4(cr2[d][0], cr2[d][1]), B2{});
          load2(cr2[d], live ? j + d + 4 : j + d);
        }
      };
      step3(w3);
      for (int c = w3 + 2; c < w3 + n3w; c += 2) step3(c);
      step2(j0);
      for (int j = j0 + 4; j < j0 + n2w; j += 4) step2(j);
    };
    // window w: 3-bit chunks [w3, w3 + n3w), then 2-bit chunks [j0, j0 + n2w)
    auto window = [&](int w3, int j0, int& n3w, int& n2w) __attribute__((always_inline)) {
      n3w = min(nc3 - w3, wcap);
      // all remaining 2-bit chunks if they fit (past the last one the ring
      // reads out of range), else whole ring rounds
      n2w = nc2 - j0 <= wcap - n3w ? nc2 - j0 : ((wcap - n3w) >> 2) << 2;
    };
    if (lane < kURows) S.cz[wave][lane] = 0.f;   // this wave's z t' sums of the pass
    int w3 = 0, j0 = 0;
    if (nc == 0) {   // no 3/2-bit chunks: only the 8-bit pairs and W x
      load_tko();
      epi_loads_t8();
      epi_loads_yb();
      zero_rows();
      __syncthreads();   // every wave's zeroed sums are seen
    } else {
      // the first window, outside any loop: one burst of loads (A-prep
      // inputs first, the token indices, the 8-bit pairs' inputs, both code
      // rings, then W x once the token indices are in), then the math
      int n3w, n2w;
      window(w3, j0, n3w, n2w);
      APIn ai;
      aprep_load(w3, n3w, j0, n2w, ai);
      __builtin_amdgcn_sched_barrier(0);
      load_tko();
      epi_loads_t8();
      __builtin_amdgcn_sched_barrier(0);
      load3(cr3[0], 0);
      load3(cr3[1], 1);
#pragma unroll
      for (int d = 0; d < 4; ++d) load2(cr2[d], d);
      __builtin_amdgcn_sched_barrier(0);
      epi_loads_yb();
      __builtin_amdgcn_sched_barrier(0);
      zero_rows();
      aprep(w3, n3w, j0, n2w, ai);
      lds_barrier_keep_vm();
      if (nops == 1) run(I1{}, w3, n3w, j0, n2w);
      else run(I2{}, w3, n3w, j0, n2w);
      w3 += n3w;
      j0 += n2w;
    }
    while (w3 < nc3 || j0 < nc2) {
      int n3w, n2w;
      window(w3, j0, n3w, n2w);
      lds_barrier_keep_vm();   // the previous window's operands are consumed
      APIn ai;
      aprep_load(w3, n3w, j0, n2w, ai);
      aprep(w3, n3w, j0, n2w, ai);
      lds_barrier_keep_vm();
      if (nops == 1) run(I1{}, w3, n3w, j0, n2w);
      else run(I2{}, w3, n3w, j0, n2w);
      w3 += n3w;
      j0 += n2w;
    }
    // ---- epilogue: each token's three piece rows, sum_i z t' per token row, 8-bit pairs, W x, one rounding
    f32x4 tot4[2];
#pragma unroll
    for (int op = 0; op < 2; ++op) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float v = acc[op][r] + swz_xor<16>(acc[op][r]);   // pieces 0+1, 2+(zero row)
        tot4[op][r] = v + __shfl_xor(v, 32, 64);
      }
    }
    // every wave's z t' sums were written before the last window's barrier
    epi_select();
    float u8w[kU8Max];
#pragma unroll
    for (int i = 0; i < kU8Max; ++i)
      u8w[i] = (float)(_Float16)(f16f(u8s[i] & 0xFFFFu) * ((float)u8c[i] - f16f(u8s[i] >> 16)));
    const uint32_t* __restrict__ us8 = reinterpret_cast<const uint32_t*>(e.base + e.off[DC_REG_US8]);
    const uint8_t* __restrict__ uc8 = e.base + e.off[DC_REG_UC8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {   // lane group q writes tokens 2q and 2q + 1
      const int rw = 2 * q + h;
      if (rw < nt) {
        const f32x4 tq = rw < 4 ? tot4[0] : tot4[1];
        const int r = rw & 3;
        float v = r == 0 ? tq[0] : (r == 1 ? tq[1] : (r == 2 ? tq[2] : tq[3]));
#pragma unroll
        for (int w8 = 0; w8 < kUWaves; ++w8) v -= S.cz[w8][rw];
#pragma unroll
        for (int i = 0; i < kU8Max; ++i)
          if (i < n8) v += u8w[i] * t8o[h][i];
        for (int i = kU8Max; i < n8; ++i) {   // more 8-bit pairs than kept in registers
          const uint32_t ew = us8[(size_t)g * e.np8 + i];
          const float uh = (float)(_Float16)(f16f(ew & 0xFFFFu) * ((float)uc8[(size_t)orow * n8 + i] - f16f(ew >> 16)));
          v += uh * tv[(size_t)(pb + rw) * rs + i];
        }
        y[(size_t)tko[h] * out + orow] = to_bf16(v + ybo[h]);
      }
    }
  }
}

}  // namespace

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
  const int m = a.m;
  uint32_t* flags = reinterpret_cast<uint32_t*>(a.ws + a.wl.flags);
  int32_t* offs = reinterpret_cast<int32_t*>(a.ws + a.wl.offs);
  int32_t* perm = reinterpret_cast<int32_t*>(a.ws + a.wl.perm);
  const size_t items = (size_t)a.T * (a.in / kGroup);
  uint8_t* xf = a.ws + a.wl.xf;
  uint32_t* xsc = reinterpret_cast<uint32_t*>(a.ws + a.wl.xsc);
  float* xsum = reinterpret_cast<float*>(a.ws + a.wl.xsum);
  bool any_w = false;
  for (int j = 0; j < m; ++j) any_w = any_w || a.mat[j].W;
  // the B tiles of x feed the split-K backbone product only
  uint16_t* xt = any_w && a.wl.nks > 0 ? reinterpret_cast<uint16_t*>(a.ws + a.wl.xt) : nullptr;
  auto wsp = [&](size_t off) { return a.ws + off; };
  PrepMats pm{};
  VGroup vg{};
  UGroup ug{};
  ActEntry* act_all = reinterpret_cast<ActEntry*>(wsp(a.wl.act));
  MatParams* mp = reinterpret_cast<MatParams*>(wsp(a.wl.params));
  pm.mp = mp;
  BaseMat bm[kMaxGroup];
  int nbm = 0, rb = 0, red = 0, vbmax = 0, outmax = 0;
  for (int j = 0; j < m; ++j) {
    const WsMat& M = a.wl.mat[j];
    const MatArgs& A = a.mat[j];
    ActEntry* act = act_all + (size_t)j * a.wl.nact;
    float* tv = reinterpret_cast<float*>(wsp(M.vpart));
    float* ybase = A.W ? reinterpret_cast<float*>(wsp(M.ybase)) : nullptr;
    float* bpt = reinterpret_cast<float*>(wsp(M.bpt));
    uint32_t* cnt = reinterpret_cast<uint32_t*>(wsp(M.cnt));
    // t is zeroed when its slices add up atomically, W x when its two K ranges do
    pm.act[j] = act;
    pm.tv[j] = tv;
    pm.ntv[j] = a.kind != kKindBitdelta && a.wl.ns <= kMaxAtomicTerms ? a.T * M.rs : 0;
    pm.yb[j] = ybase;
    pm.nyb[j] = A.W && a.wl.nks == kMaxAtomicTerms ? a.T * A.out : 0;
    pm.cnt[j] = cnt;
    pm.ncnt[j] = M.ncnt;
    pm.layouts = a.kind == kKindDeltaCoMe;
    if (A.W) bm[nbm++] = BaseMat{A.W, ybase, bpt, A.out, rb}, rb += A.out / kBaseRows;
    pm.params[j] = MatParams{tv,   reinterpret_cast<float*>(wsp(M.vpt)), cnt, ybase, A.y, bpt, A.out, M.rs, M.vb,
                             a.wl.nks};
    vg.red0[j] = red;
    if (A.W && a.wl.nks > kMaxAtomicTerms) {
      vg.bs[j] = BaseSum{bpt, ybase, a.wl.nks, A.out, a.T};
      red += (A.out / 64) * ((a.T + 7) / 8);
    }
    vbmax = max(vbmax, M.vb);
    outmax = max(outmax, A.out);
  }
  for (int j = m; j <= kMaxGroup; ++j) vg.red0[j] = red;
  SegArg seg{};
  if (a.mode == 2)
    for (int k = 0; k <= a.n; ++k) seg.v[k] = a.seg[k];
  auto mark = [&](int s) {
    if (a.events && a.events[s]) (void)hipEventRecord(reinterpret_cast<hipEvent_t>(a.events[s]), st);
  };
  mark(DC_STAGE_ROUTE);
  mark(DC_STAGE_XPREP);
  const dim3 gp((unsigned)(1 + (items + 3) / 4)), bp(256);
#define DC_PREP(M_)                                                                                             \
  {                                                                                                             \
    GroupTables<M_> gt;                                                                                         \
    for (int j = 0; j < M_; ++j) gt.t[j] = *a.mat[j].tenants;                                                  \
    hipLaunchKernelGGL(k_prep<M_>, gp, bp, 0, st, gt, a.x, a.ids, a.T, a.in, a.n, a.mode, seg, offs, perm,       \
                       flags, xf, xsc, xsum, xt, pm, a.wl.nact);                                                \
  }
  switch (m) {
    case 1: DC_PREP(1) break;
    case 2: DC_PREP(2) break;
    case 3: DC_PREP(3) break;
    default: DC_PREP(4) break;
  }
#undef DC_PREP
  mark(DC_STAGE_BASE);
  if (nbm > 0) launch_base(bm, nbm, a.x, xt, a.in, a.T, a.stream);
  if (a.kind != kKindDeltaCoMe) {
    BaselineLaunch b{};
    b.kind = a.kind;
    b.m = m;
    b.n = a.n;
    b.in = a.in;
    b.T = a.T;
    b.nact = a.wl.nact;
    b.ns = a.wl.ns;
    b.x = a.x;
    b.perm = perm;
    b.xf = xf;
    b.xsc = xsc;
    b.xsum = xsum;
    b.act = act_all;
    b.mp = mp;
    b.vbmax = vbmax;
    b.outmax = outmax;
    b.nks = a.wl.nks;
    for (int j = 0; j < m; ++j) {
      const bool sum = a.mat[j].W && a.wl.nks > kMaxAtomicTerms;
      b.bpt[j] = sum ? reinterpret_cast<const float*>(wsp(a.wl.mat[j].bpt)) : nullptr;
      b.ybase[j] = reinterpret_cast<float*>(wsp(a.wl.mat[j].ybase));
      b.out[j] = a.mat[j].out;
    }
    b.stream = a.stream;
    return launch_baseline(b);
  }
  mark(DC_STAGE_VSIDE);
  const int gx = vbmax > 0 ? vbmax * a.wl.ns : 1;
  vg.red_rows = (red + gx - 1) / gx;
  vg.nact = a.wl.nact;
  vg.act = act_all;
  vg.mp = mp;
  vg.ns = a.wl.ns;
  vg.T = a.T;
  vg.m = m;
  vg.mmagic = magic_of(m);
  vg.nsmagic = magic_of(a.wl.ns);
  if (vbmax > 0 || red > 0) {
    const unsigned gy = (unsigned)(vg.red_rows + (vbmax > 0 ? m * a.wl.nact : 0));
    hipLaunchKernelGGL(k_vside, dim3((unsigned)gx, gy), dim3(256), 0, st, a.n, a.in, a.x, perm, xf, xsc, xsum, vg);
  }
  mark(DC_STAGE_USIDE);
  ug.nact = a.wl.nact;
  ug.act = act_all;
  ug.mp = mp;
  ug.m = m;
  ug.mmagic = magic_of(m);
  hipLaunchKernelGGL(k_uside, dim3((unsigned)(outmax / kGroup), (unsigned)(m * a.wl.nact)), dim3(kUWaves * 64), 0,
                     st, a.n, a.in, perm, a.T, ug);
  mark(DC_STAGE_COUNT);
  return (int)hipGetLastError();
}

}  // namespace dc
