// Pieces shared by the V-side style kernels of the delta apply: where a
// block's partial results go and how slices of one output are added in a
// fixed order, the fixed-order sum of the backbone product's K ranges, and
// the staging of x fragments into LDS.  Included inside namespace dc,
// anonymous namespace, after mx_common.h and combine.h.
#pragma once

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Where a V-side block puts sigma * (its slice's part of V x): with at most
// kMaxAtomicTerms input slices, added into t (zeroed by prep) with float
// atomics (order-independent for two terms); with more, stored as the
// slice's partial and added in slice order by the block of the same ranks
// that finishes last (counter per bucket and rank block).
struct VOut {
  float* tv;         // t [T][rs], sorted rows
  float* vpt;        // partials [ns][T][rs] (ns > kMaxAtomicTerms)
  uint32_t* vcnt;    // arrival counters [n + 1][vb]
  int32_t rs, ns, T, vb;
};

__device__ __forceinline__ void v_put(const VOut& o, int s, int row, int rank, float v) {
  if (o.ns <= kMaxAtomicTerms)
    atomicAdd(o.tv + (size_t)row * o.rs + rank, v);
  else
    st_dev(o.vpt + ((size_t)s * o.T + row) * o.rs + rank, v);
}

// After every pass of the block of work item `item`: the last of the ns
// slices of ranks [r0, r0 + nr) adds the partials of rows [p0, p1) in slice
// order into t (the slices of an output are loaded kSliceBatch at a time).
constexpr int kSliceBatch = 8;   // all the slices of up to 16384 inputs
__device__ __forceinline__ void v_combine(const VOut& o, int item, int b, int p0, int p1, int r0, int nr) {
  if (o.ns <= kMaxAtomicTerms) return;
  __shared__ int last;
  if (!arrive_last(&o.vcnt[item * o.vb + b], o.ns, &last)) return;
  const size_t sstride = (size_t)o.T * o.rs;
  for (int i = threadIdx.x; i < (p1 - p0) * nr; i += blockDim.x) {
    const int row = p0 + i / nr, rank = r0 + i % nr;
    const float* src = o.vpt + (size_t)row * o.rs + rank;
    float v = 0.f;
    for (int s0 = 0; s0 < o.ns; s0 += kSliceBatch) {
      float p[kSliceBatch];
#pragma unroll
      for (int j = 0; j < kSliceBatch; ++j) p[j] = s0 + j < o.ns ? ld_dev(src + (s0 + j) * sstride) : 0.f;
#pragma unroll
      for (int j = 0; j < kSliceBatch; ++j)
        if (s0 + j < o.ns) v += p[j];
    }
    o.tv[(size_t)row * o.rs + rank] = v;
  }
}

// The backbone product's K-range partials (more than two ranges) added in
// range order into W x, by blocks of the V-side launch that run before its
// V-side blocks: block = 64 rows x 8 tokens, thread = one row, two tokens,
// all of an output's ranges loaded before the sum.
struct BaseSum {
  const float* bpt;   // [nks][T][out]
  float* ybase;       // [T][out]
  int32_t nks, out, T;
};


__device__ void base_sum(const BaseSum& bs, int idx) {
  const int ntb = (bs.T + 7) / 8;
  const int rb = idx / ntb, tb = idx % ntb;
  const int ro = rb * 64 + (threadIdx.x & 63), t0 = tb * 8 + 2 * (threadIdx.x >> 6);
  if (t0 >= bs.T) return;
  const bool two = t0 + 1 < bs.T;
  const size_t rstride = (size_t)bs.T * bs.out;
  const float* src = bs.bpt + (size_t)t0 * bs.out + ro;
  float v0 = 0.f, v1 = 0.f;
  for (int r0 = 0; r0 < bs.nks; r0 += 16) {
    float a[16], c[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const bool ok = r0 + j < bs.nks;
      a[j] = ok ? src[(r0 + j) * rstride] : 0.f;
      c[j] = ok && two ? src[(r0 + j) * rstride + bs.out] : 0.f;
    }
#pragma unroll
    for (int j = 0; j < 16; ++j)
      if (r0 + j < bs.nks) {
        v0 += a[j];
        v1 += c[j];
      }
  }
  bs.ybase[(size_t)t0 * bs.out + ro] = v0;
  if (two) bs.ybase[(size_t)(t0 + 1) * bs.out + ro] = v1;
}

// x fragments of kVSlice input groups for kVRows token rows, as the V-side
// blocks read them: [group][token row][lane group * 4 + (hi0 hi1 lo0 lo1)],
// rows padded to 17 int4 against bank conflicts.
struct VLds {
  int4 frag[kVSlice][kVRows][17];     // [group][token row][lane group * 4 + (hi0 hi1 lo0 lo1)], padded row
  uint32_t sc[kVSlice][kVRows];       // E8M0 words of the hi pieces
  float xs[kVSlice][kVRows];          // group sums of x
};

// A work item's token list, passed by value (in registers), and its entry
// i (0..7, per lane) by selects on constant indices.
struct Tok8 {
  int32_t v[8];
};
__device__ __forceinline__ Tok8 tok8_of(const int32_t (&t)[8]) {
  Tok8 r;
#pragma unroll
  for (int k = 0; k < 8; ++k) r.v[k] = t[k];
  return r;
}
__device__ __forceinline__ int pick8(const Tok8& t, int i) {
  int r = t.v[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) {
    r = i == k ? t.v[k] : r;
    asm volatile("" : "+v"(r));   // a chain of selects: not turned into an indexed private-memory table
  }
  return r;
}
// The same for an index that is the same on every lane (scalar selects).
__device__ __forceinline__ int pick8u(const Tok8& t, int i) {
  int r = t.v[0];
#pragma unroll
  for (int k = 1; k < 8; ++k) {
    r = i == k ? t.v[k] : r;
    asm volatile("" : "+s"(r));
  }
  return r;
}

// x fragments, scale words and group sums of a work item's token rows
// (tokens tok[0 .. nt), stored in token order) for groups [g0, g0 + kVSlice),
// staged into LDS in two steps so that the
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
                                             int gi_n, int g0, const Tok8 tok, int nt) {
  const int tid = threadIdx.x;
  const int k16 = tid & 15, rw = (tid >> 4) & 7, gh = tid >> 7;
  const size_t row = (size_t)pick8(tok, min(rw, nt - 1)) * gi_n;
#pragma unroll
  for (int u = 0; u < kVSlice / 2; ++u) {
    const int gi = min(g0 + gh + 2 * u, gi_n - 1);
    st.v[u] = reinterpret_cast<const i32x4*>(xf + (row + gi) * kXFrag)[k16];
  }
  const int sr = tid & 7, sgl = (tid >> 3) & (kVSlice - 1);
  const size_t srow = (size_t)pick8(tok, min(sr, nt - 1)) * gi_n + min(g0 + sgl, gi_n - 1);
  st.scw = xsc[srow];
  st.xsv = xsum[srow];
}

__device__ __forceinline__ void v_stage_store(VLds& S, const VStage& st) {
  const int tid = threadIdx.x;
  const int k16 = tid & 15, rw = (tid >> 4) & 7, gh = tid >> 7;
#pragma unroll
  for (int u = 0; u < kVSlice / 2; ++u)
    S.frag[gh + 2 * u][rw][k16] = make_int4(st.v[u].x, st.v[u].y, st.v[u].z, st.v[u].w);
  // every thread stores (threads tid and tid + 128 write the same values):
  // a conditional store would sink these loads behind the code loads that
  // follow them, and waiting for them would then drain those too
  {
    const int sr = tid & 7, sgl = (tid >> 3) & (kVSlice - 1);
    S.sc[sgl][sr] = st.scw;
    S.xs[sgl][sr] = st.xsv;
  }
}

