// Internal declarations shared by the host code and the gfx950 kernels of
// libdeltacome.so.  Not part of the public ABI (include/deltacome.h is).
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "../../include/deltacome.h"

#if defined(__HIPCC__)
#define DC_HD __host__ __device__
#else
#define DC_HD
#endif

namespace dc {

constexpr int kGroup = 128;   // elements per quantization group
constexpr int kAlign = 256;   // region alignment inside a packed buffer
constexpr int kKBlock = 32;   // ranks per K-block of the U code regions

DC_HD inline size_t round_up(size_t v, size_t m) { return (v + m - 1) / m * m; }

// IEEE fp64 -> fp16, round to nearest even, in one step from the fp64 bits
// (no fp32 intermediate, so no double rounding).
DC_HD inline uint16_t f64_to_f16(double d) {
  const uint64_t b = __builtin_bit_cast(uint64_t, d);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const int e = (int)((b >> 52) & 0x7FF);
  const uint64_t frac = b & ((1ull << 52) - 1);
  if (e == 0x7FF) return sign | (frac ? 0x7E00 : 0x7C00);
  if (e == 0) return sign;                  // |d| < 2^-1022: rounds to zero
  int E = e - 1023;                         // d = 1.frac * 2^E
  if (E > 15) return sign | 0x7C00;
  const uint64_t sig = frac | (1ull << 52); // 53-bit significand
  const int shift = (E >= -14) ? 42 : 42 + (-14 - E);
  if (shift >= 55) return sign;             // below half the smallest subnormal
  uint64_t q = sig >> shift;
  const uint64_t rem = sig & ((1ull << shift) - 1);
  const uint64_t half = 1ull << (shift - 1);
  if (rem > half || (rem == half && (q & 1))) ++q;
  if (E >= -14) {
    if (q == 2048) { q = 1024; ++E; }
    if (E > 15) return sign | 0x7C00;
    return (uint16_t)(sign | ((E + 15) << 10) | (q - 1024));
  }
  return (uint16_t)(sign | q);              // subnormal; q == 1024 is the smallest normal
}

// fp16 bits -> fp64 (exact; every fp16 value is an fp64 value).
DC_HD inline double f16_to_f64(uint16_t h) {
  const int e = (h >> 10) & 0x1F;
  const uint64_t m = h & 0x3FF;
  const uint64_t sign = (uint64_t)(h & 0x8000) << 48;
  if (e == 31) return __builtin_bit_cast(double, sign | 0x7FF0000000000000ull | (m << 42));
  if (e == 0) {   // subnormal: m * 2^-24, exact in fp64
    const double v = (double)m * 5.9604644775390625e-8;
    return (h & 0x8000) ? -v : v;
  }
  return __builtin_bit_cast(double, sign | ((uint64_t)(e - 15 + 1023) << 52) | (m << 42));
}

// Words one row of a 3- or 2-bit U code segment of n ranks takes: full
// K-blocks of 32 ranks take b words, the last one ceil(m*b/32) for its m ranks.
DC_HD inline int u_row_words(int n, int b) {
  if (n <= 0) return 0;
  const int kb = (n + kKBlock - 1) / kKBlock;
  const int m = n - kKBlock * (kb - 1);
  return (kb - 1) * b + (m * b + 31) / 32;
}

// Word offset of K-block kb of row o inside a 3- or 2-bit U code region of n
// ranks (16-row tiles, K-block by K-block), and the words it holds.
DC_HD inline size_t u_kblock_word(int o, int kb, int n, int b, int* nw) {
  const int kbn = (n + kKBlock - 1) / kKBlock;
  const int rw = u_row_words(n, b);
  const int w = (kb == kbn - 1) ? rw - (kbn - 1) * b : b;
  *nw = w;
  return (size_t)(o / 16) * 16 * rw + (size_t)kb * 16 * b + (size_t)(o % 16) * w;
}

// Word offset of the b words of chunk q (codes 32q..32q+31) of group grp of
// local rank i inside a 3- or 2-bit V code region of Gi groups: 16-rank
// tiles, [ceil(n/16)][Gi][4][16][b] words.
DC_HD inline size_t v_chunk_word(int i, int grp, int q, int gi, int b) {
  return ((((size_t)(i / 16) * gi + grp) * 4 + q) * 16 + (i % 16)) * b;
}

// Byte offsets of the DC_REG_* regions of a packed buffer and its total size.
// This is the format stated in include/deltacome.h.
struct Layout {
  size_t off[DC_REG_COUNT];
  size_t size[DC_REG_COUNT];
  size_t total;
};

DC_HD inline void layout_of(int32_t out, int32_t in, int32_t n8, int32_t n3, int32_t n2, Layout* L) {
  const size_t gi = (size_t)in / kGroup, go = (size_t)out / kGroup;
  const size_t r = (size_t)n8 + n3 + n2;
  size_t sz[DC_REG_COUNT];
  sz[DC_REG_SIGMA] = 4 * r;
  sz[DC_REG_VC8] = (size_t)n8 * gi * 16 * 8;
  sz[DC_REG_VC3] = round_up(n3, 16) * gi * 16 * 3;
  sz[DC_REG_VC2] = round_up(n2, 16) * gi * 16 * 2;
  sz[DC_REG_VS8] = gi * round_up(n8, 4) * 4;
  sz[DC_REG_VS3] = gi * round_up(n3, 4) * 4;
  sz[DC_REG_VS2] = gi * round_up(n2, 4) * 4;
  sz[DC_REG_UC8] = (size_t)out * n8;
  sz[DC_REG_UC3] = (size_t)out * 4 * u_row_words(n3, 3);
  sz[DC_REG_UC2] = (size_t)out * 4 * u_row_words(n2, 2);
  sz[DC_REG_US8] = go * round_up(n8, 4) * 4;
  sz[DC_REG_US3] = go * round_up(n3, 4) * 4;
  sz[DC_REG_US2] = go * round_up(n2, 4) * 4;
  size_t o = 0;
  for (int i = 0; i < DC_REG_COUNT; ++i) {
    o = round_up(o, kAlign);
    L->off[i] = o;
    L->size[i] = sz[i];
    o += sz[i];
  }
  L->total = round_up(o, kAlign);
}

// One tenant as the kernels see it (kernel-argument table, no device copy).
// Baseline calls: n8 holds the low-rank r (0 for BitDelta), n3 = n2 = 0.
struct Tenant {
  const uint8_t* base;
  int32_t n8, n3, n2;
  int32_t pad_;
};

struct TenantTable {
  Tenant t[DC_MAX_TENANTS];
};

// One work item of routed tokens, as the prep kernel lists them: the rows of
// a bucket in chunks of kChunkRows (bucket order; the rest of the list has
// p0 == p1): the tenant record (zero for the backbone-only bucket k == n)
// and the routed range [p0, p1).  The V-side and U-side blocks of different
// chunks of one tenant run side by side (the codes they share come from
// the caches after the first read).
struct ActEntry {
  const uint8_t* base;
  int32_t n8, n3, n2;
  int32_t k;
  int32_t p0, p1;
  // Delta-CoMe calls: byte offsets of the DC_REG_* regions of the tenant's
  // packed buffer and its size, worked out once per item by the routing
  // block (every wave of a V or U block would otherwise redo it in scalar
  // arithmetic); zero for the backbone-only bucket and the baselines
  uint32_t off[DC_REG_COUNT];
  uint32_t total;
  // Delta-CoMe calls, U side: the tenant's derived sizes, the same for every
  // block of the item (the U blocks' waves would otherwise each work them
  // out with scalar instructions, which the waves of a compute unit share):
  // t positions of the 3- and 2-bit segments; scale-row lengths (ranks
  // rounded up to 4) of the 8-, 3- and 2-bit segments; 128-rank chunks of
  // the 3-bit segment and of both; words per U row, K-blocks and words of
  // the last K-block of the 3- and 2-bit segments
  int32_t tb3, tb2;
  int32_t np8, np3, np2;
  int32_t nc3, nc;
  int32_t rw3, rw2, kbn3, kbn2, wl3, wl2;
  // the item's tokens (original indices) at routed rows p0 .. p1 - 1, the
  // last one repeated past p1: the x staging and the epilogue read them from
  // here instead of loading the permutation
  int32_t tok[8];
  uint32_t pad_[1];
};
static_assert(sizeof(ActEntry) == 176, "four scalar loads per block");
constexpr int kChunkRows = 8;   // token rows per work item (one V-side and one U-side pass)
static_assert(kChunkRows == sizeof(ActEntry::tok) / sizeof(int32_t), "one token per item row");
// Work items of a call of n tenants and T tokens: at most one partly filled
// chunk per bucket (n tenants + the backbone-only bucket) plus T / kChunkRows.
DC_HD inline int32_t act_capacity(int32_t n, int32_t T) { return n + 1 + (T + kChunkRows - 1) / kChunkRows; }

// Work decomposition of the matrix-core path (shared by host sizing and kernels).
constexpr int kVSlice = 16;   // 128-groups of the input per V-side work item
constexpr int kVRows = 8;     // token rows per V-side pass
constexpr int kVTiles = 2;    // 16-rank tiles per V-side wave
constexpr int kVRanks = 4 * 16 * kVTiles;   // ranks per V-side block (4 waves)
constexpr int kVDepth = 8;    // groups of codes a V-side wave keeps in flight
static_assert(kChunkRows == kVRows, "one V-side pass per work item");

// Split backbone product (T <= 256): K ranges of kSKSteps steps of 32,
// blocks of kBaseRows rows of W (one 16-row tile per wave).
constexpr int kSKSteps = 16;
constexpr int kBaseWaves = 8;
constexpr int kBaseRows = 16 * kBaseWaves;
DC_HD inline int base_splits(int in, int T) { return T <= 256 ? (in / 32 + kSKSteps - 1) / kSKSteps : 0; }

// Prefill segments of at least this many tokens can take the dense form
// (every non-empty segment of the call must have this many).
constexpr int kDenseMin = 256;

DC_HD inline int v_slices(int in) { return (in / kGroup + kVSlice - 1) / kVSlice; }
// V-side rank blocks of a tenant: [8-bit rows if any] [3-bit blocks] [2-bit blocks] of kVRanks
DC_HD inline int v_blocks(int n8, int n3, int n2) {
  return (n8 > 0 ? 1 : 0) + (n3 + kVRanks - 1) / kVRanks + (n2 + kVRanks - 1) / kVRanks;
}
// Rank positions of the V-side results: each bit-width segment starts on a multiple of 8.
DC_HD inline int t_base(int n8, int n3, int which) {
  return which == 0 ? 0 : (which == 1 ? (int)round_up((size_t)n8, 8) : (int)(round_up((size_t)n8, 8) + round_up((size_t)n3, 8)));
}
DC_HD inline int t_width(int n8, int n3, int n2) { return t_base(n8, n3, 2) + (int)round_up((size_t)n2, 8); }

// Sums of more than two partials are added in a fixed order by the work item
// that arrives last; two partials (or one) are added onto zero with float
// atomics, which is order-independent for two terms.
constexpr int kMaxAtomicTerms = 2;

// Matrices of one grouped call (they read the same x and tenant ids).
constexpr int kMaxGroup = DC_MAX_GROUP;

// Per-matrix parameters of a call, written into the workspace by the prep
// kernel: the V-side and U-side kernels select their matrix with one uniform
// load instead of indexing their kernel arguments.
struct MatParams {
  float* tv;           // t [T][rs]
  float* vpt;          // V-side slice partials [ns][T][rs] (BitDelta: [ns][T][out])
  uint32_t* vcnt;      // V-side arrival counters [nact][vb]
  const float* ybase;  // W x [T][out], null: delta only
  uint16_t* y;         // output [T][out]
  const float* bpt;    // W x partials [nks][T][out] (read by the BitDelta epilogue when nks > 2)
  int32_t out, rs, vb, nks;
};
static_assert(sizeof(MatParams) == 64, "one scalar load per kernel");

// Kinds of delta an apply call serves: Delta-CoMe's mixed-precision pairs,
// or one of the two baselines (include/deltacome.h: DC_KIND_*).
constexpr int kKindDeltaCoMe = 0;
constexpr int kKindLowrank = DC_KIND_LOWRANK;
constexpr int kKindBitdelta = DC_KIND_BITDELTA;

// Low-rank baseline: V side in blocks of kLrRanks ranks (4 waves x one
// 16-rank tile) over input slices of kLrSlice; t rows padded to 32 ranks.
constexpr int kLrSlice = 512;
constexpr int kLrRanks = 64;
DC_HD inline int lr_slices(int in) { return (in + kLrSlice - 1) / kLrSlice; }
DC_HD inline int lr_vblocks(int r) { return (r + kLrRanks - 1) / kLrRanks; }
// BitDelta: blocks of kBdRows output rows (4 waves x two 16-row tiles) over
// input slices of kVSlice groups.
constexpr int kBdRows = 128;

// Shape rules of a baseline delta: out and in positive multiples of 128;
// low-rank 0 <= r <= min(out, in); BitDelta r = 0.
DC_HD inline bool baseline_valid(int32_t kind, int32_t out, int32_t in, int32_t r) {
  if (out <= 0 || in <= 0 || out % kGroup || in % kGroup) return false;
  if (kind == DC_KIND_LOWRANK) return r >= 0 && r <= (out < in ? out : in);
  return kind == DC_KIND_BITDELTA && r == 0;
}

// Packed sizes of the baselines (the formats of include/deltacome.h).
DC_HD inline size_t lowrank_bytes(int32_t out, int32_t in, int32_t r) {
  const size_t v = round_up(4 * (size_t)r, kAlign);
  const size_t u = round_up(v + 2 * round_up((size_t)r, 16) * in, kAlign);
  return round_up(u + 2 * (size_t)out * round_up((size_t)r, 32), kAlign);
}
DC_HD inline size_t lowrank_v_offset(int32_t r) { return round_up(4 * (size_t)r, kAlign); }
DC_HD inline size_t lowrank_u_offset(int32_t in, int32_t r) {
  return round_up(lowrank_v_offset(r) + 2 * round_up((size_t)r, 16) * in, kAlign);
}
DC_HD inline size_t bitdelta_bytes(int32_t out, int32_t in) { return kAlign + (size_t)out * in / 8; }

// The part of a call's workspace that belongs to one matrix of the group.
struct WsMat {
  size_t ybase;   // fp32 [T][out] backbone product, original order
  size_t vpart;   // fp32 [T][rs] t = sigma * (V x), sorted order
  size_t vpt;     // fp32 [ns][T][rs] per-slice partials of t when ns > 2 (added in slice order)
  size_t bpt;     // fp32 [nks][T][out] per-range partials of W x when nks > 2 (added in range order)
  size_t cnt;     // uint32 arrival counters of the V rank blocks [nact][vb] when ns > 2
  int32_t out;    // rows of the matrix
  int32_t rs;     // row stride of vpart (max t_width over tenants)
  int32_t vb;     // max V-side rank blocks per tenant
  int32_t ncnt;   // counters in cnt
};

// Workspace layout of one apply call: the routing and the staged x shared by
// the group's matrices, then each matrix's part, then the dense prefill
// operands (single-matrix prefill calls only).
struct WsLayout {
  size_t flags;   // uint32 status word (+ padding to 256 B)
  size_t offs;    // int32 [n+2] bucket starts in sorted order (bucket n = backbone only)
  size_t perm;    // int32 [T] sorted position -> token index
  size_t xf;      // uint8 [T][in/128][256] fp8 hi/lo fragments of x (matrix-core A operand)
  size_t xsc;     // uint32 [T][in/128] E8M0 block scales of the hi fragments
  size_t xsum;    // fp32 [T][in/128] sums of x over each 128-group
  size_t xt;      // bf16 x in matrix-core B tiles: [in/32][ceil(T/16)][64 lanes][8]
  size_t act;     // ActEntry [m][nact] work items of the buckets with tokens, in bucket order, per matrix
  size_t params;  // MatParams [m]
  WsMat mat[kMaxGroup];
  size_t dt;      // prefill, dense form: fp32 t [T][drp] (padded ranks, segment by segment)
  size_t dxs;     // fp32 [T] power-of-two rescale of each token's x
  size_t dtm;     // uint32 [T] bits of each token's largest |t|
  size_t total;
  int32_t m;      // matrices of the group
  int32_t drp;    // padded rank rows of the dense form's t (0: no dense region)
  int32_t ns;     // V-side input slices
  int32_t nks;    // K ranges of the split backbone product (0: tiled product)
  int32_t nact;   // work-item capacity of each act list
};

// Per matrix j of the group: out[j], rs[j] (max t_width over its tenants),
// vb[j] (max v_blocks over its tenants).  drp: rank rows of the dense prefill
// operands (0 for decode calls; m must be 1 otherwise).
// kind: kKindDeltaCoMe, or a baseline (rs = t row stride for the low-rank
// baseline, vb = its V blocks; BitDelta: vb = output row blocks, no t).
inline bool ws_layout(int32_t T, int32_t in, int32_t n, int32_t m, const int32_t* out, const int32_t* rs,
                      const int32_t* vb, int32_t drp, WsLayout* W, int32_t kind = kKindDeltaCoMe) {
  if (T < 0 || n < 0 || m < 1 || m > kMaxGroup || (drp > 0 && (m != 1 || kind != kKindDeltaCoMe))) return false;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = round_up(o, kAlign); o = at + bytes; return at; };
  W->m = m;
  W->flags = take(256);
  W->offs = take(4 * ((size_t)n + 2));
  W->perm = take(4 * (size_t)T);
  W->nact = act_capacity(n, T);
  const size_t items = (size_t)T * (in / kGroup);
  W->xf = take(256 * items);   // 2 T in bytes: the dense prefill form keeps x' (fp16 [T][in]) here
  W->xsc = take(4 * items);
  W->xsum = take(4 * items);
  W->xt = take(2 * (size_t)in * round_up((size_t)T, 16));
  W->ns = kind == kKindLowrank ? lr_slices(in) : v_slices(in);
  W->nks = base_splits(in, T);
  W->act = take(sizeof(ActEntry) * (size_t)m * W->nact);
  W->params = take(sizeof(MatParams) * kMaxGroup);
  const bool bd = kind == kKindBitdelta;
  // BitDelta slices always meet in the last one (its epilogue needs the sum)
  const bool stored = bd ? W->ns > 1 : W->ns > kMaxAtomicTerms;
  for (int j = 0; j < m; ++j) {
    WsMat& M = W->mat[j];
    M.out = out[j];
    M.rs = rs[j] > 0 ? rs[j] : 8;
    M.vb = vb[j];
    M.ybase = take(4 * (size_t)T * M.out);
    M.vpart = take(bd ? 0 : 4 * (size_t)T * M.rs);
    M.vpt = take(stored ? 4 * (size_t)W->ns * T * (bd ? M.out : M.rs) : 0);
    M.bpt = take(W->nks > kMaxAtomicTerms ? 4 * (size_t)W->nks * T * M.out : 0);
    M.ncnt = stored ? W->nact * M.vb : 0;
    M.cnt = take(4 * (size_t)M.ncnt);
  }
  W->drp = drp;
  W->dt = take(drp > 0 ? 4 * (size_t)T * drp : 0);
  W->dxs = take(drp > 0 ? 4 * (size_t)T : 0);
  W->dtm = take(drp > 0 ? 4 * (size_t)T : 0);
  W->total = round_up(o, kAlign);
  return true;
}

}  // namespace dc

// Kernel launchers (defined in the .hip files).  All enqueue on `stream`
// and return a hipError_t as int.
namespace dc {
// One matrix of a call: its tenants, shape, backbone and output.
struct MatArgs {
  const TenantTable* tenants;  // host pointer: copied into kernel arguments
  int32_t out;
  int32_t rmax;
  const uint16_t* W;           // may be null
  uint16_t* y;
};

struct ApplyArgs {
  int32_t kind;                // kKindDeltaCoMe or a baseline (its tenant records: base, n8 = r)
  int32_t m;                   // matrices (1 except grouped calls)
  MatArgs mat[kMaxGroup];
  int32_t n;
  int32_t in;
  int32_t T;
  const uint16_t* x;
  const int32_t* ids;          // device, mode 1
  const int32_t* seg;          // host, mode 2 ([n+1])
  int32_t mode;                // 0 decode (all tokens tenant 0), 1 ids, 2 segments
  uint8_t* ws;
  WsLayout wl;
  void* stream;
  void* const* events;         // optional DC_STAGE_COUNT + 1 hipEvent_t, may be null
};
int launch_apply(const ApplyArgs& a);
// The delta kernels of a baseline call, after routing, x staging and the
// backbone product (launched by launch_apply).
struct BaselineLaunch {
  int32_t kind, m, n, in, T, nact, ns;
  const uint16_t* x;
  const int32_t* perm;
  const uint8_t* xf;
  const uint32_t* xsc;
  const float* xsum;
  const ActEntry* act;         // [m][nact]
  const MatParams* mp;         // [m], in the workspace
  int32_t vbmax, outmax;       // largest V blocks / out of the group
  // per matrix: W x partials to add in range order into ybase (low-rank
  // calls whose backbone product has more than two K ranges), else null
  const float* bpt[kMaxGroup];
  float* ybase[kMaxGroup];
  int32_t out[kMaxGroup];
  int32_t nks;
  void* stream;
};
int launch_baseline(const BaselineLaunch& b);
// The backbone product W x into ybase (fp32 [T][out]).  Split over
// base_splits(in, T) K ranges when T <= 256: with two ranges ybase must be
// zeroed before it runs (the ranges add into it); with more, the ranges store
// partials into bpt [nks][T][out], which the V-side kernel adds in range order
// into ybase.  T > 256: the tiled product.
// One matrix of a backbone launch.
struct BaseMat {
  const uint16_t* W;
  float* ybase;
  float* bpt;
  int32_t out;
  int32_t rb0;   // first kBaseRows-row block of this matrix in the launch
};
// The tiled product (T > 256) covers one matrix (m == 1).
int launch_base(const BaseMat* mats, int m, const uint16_t* x, const uint16_t* xt, int in, int T, void* stream);
// Padded rank rows of a tenant in the dense prefill form: each rank group
// rounded up to 32 (whole K-blocks), the sum to whole 128-row tiles (at
// least one tile).
int pf_rank_pad(int n8, int n3, int n2);
constexpr int kPfBatch = 8;   // tenants whose dense products share one launch
// Prefill with long segments: backbone product, then per batch of tenants
// the two products with their operands dequantized in registers
// (k_prefill.hip).
int launch_dense_prefill(const ApplyArgs& a);
// The tiled backbone product (any T): ybase [T][out] = x W^T.
int launch_tiled_base(const uint16_t* W, const uint16_t* x, float* ybase, int out, int in, int T, void* stream);
int launch_dequant(const Tenant& t, int32_t out, int32_t in, uint16_t* u16, uint16_t* v16, void* stream);
// The checks and launches of every apply entry point.  ws_limit > 0: the
// workspace is the library's scratch array of that many bytes (ws and
// ws_bytes are ignored); it is looked up only once the checks pass.
// views [m][n], W [m] (entries may be null), y [m].
dc_status run_apply(const dc_delta_view* views, int32_t m, int32_t n, const uint16_t* const* W, const uint16_t* x,
                    const int32_t* ids, const int32_t* seg, int32_t mode, uint16_t* const* y, int32_t T, void* ws,
                    size_t ws_bytes, void* stream, void* const* events, size_t ws_limit);
// Device address of the scratch array on the current device (null if it
// cannot be found); defined next to the array.
void* scratch_ptr();
// The error table of dc_error_table: difference rows into dv [r][nw][in],
// then their products with X; zeroes `flag` first.
int launch_error_table(int32_t r, int32_t in, int32_t ncal, const float* sigma, const float* V, const float* X,
                       const int32_t* widths, int32_t nw, double* err, uint32_t* flag, float* dv, void* stream);
int launch_pack(int32_t out, int32_t in, int32_t n8, int32_t n3, int32_t n2, const float* U, const float* sigma,
                const float* V, uint8_t* dst, uint32_t* flag, void* stream);
// On-device SVD of a delta (block Jacobi on the fp64 Gram matrix): the
// workspace regions, the sweep cap and the convergence bound.
constexpr int kSvdMaxSweeps = 40;
constexpr double kSvdTol = 1e-13;
struct SvdLayout {
  int m, mp;   // min(out, in) and its padding to a multiple of 64
  size_t G, W, Q, off, d, fac, perm, flag, total;
};
SvdLayout svd_layout(int32_t out, int32_t in, int32_t r);
// 0: done; 1: a non-finite entry; 2: not converged in kSvdMaxSweeps; -1: HIP error
int launch_svd(int32_t out, int32_t in, int32_t r, const float* A, float* U, float* sigma, float* V, uint8_t* ws,
               int32_t* sweeps_used, void* stream);

}  // namespace dc
