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
struct Tenant {
  const uint8_t* base;
  int32_t n8, n3, n2;
  int32_t pad_;
};

struct TenantTable {
  Tenant t[DC_MAX_TENANTS];
};

// One bucket of routed tokens that is not empty, as the prep kernel lists
// them (bucket order; the rest of the list has p0 == p1): the tenant record
// (zero for the backbone-only bucket k == n) and the routed range [p0, p1).
struct ActEntry {
  const uint8_t* base;
  int32_t n8, n3, n2;
  int32_t k;
  int32_t p0, p1;
};
static_assert(sizeof(ActEntry) == 32, "one 32-byte load per block");

// Work decomposition of the matrix-core path (shared by host sizing and kernels).
constexpr int kVSlice = 16;   // 128-groups of the input per V-side work item
constexpr int kVRows = 8;     // token rows per V-side pass
constexpr int kVTiles = 2;    // 16-rank tiles per V-side wave
constexpr int kVRanks = 4 * 16 * kVTiles;   // ranks per V-side block (4 waves)
constexpr int kVDepth = 8;    // groups of codes a V-side wave keeps in flight

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

// Workspace layout of one apply call.
struct WsLayout {
  size_t flags;   // uint32 status word (+ padding to 256 B)
  size_t offs;    // int32 [n+2] bucket starts in sorted order (bucket n = backbone only)
  size_t perm;    // int32 [T] sorted position -> token index
  size_t act;     // ActEntry [n+1] buckets with tokens first
  size_t xf;      // uint8 [T][in/128][256] fp8 hi/lo fragments of x (matrix-core A operand)
  size_t xsc;     // uint32 [T][in/128] E8M0 block scales of the hi fragments
  size_t xsum;    // fp32 [T][in/128] sums of x over each 128-group
  size_t xt;      // bf16 x in matrix-core B tiles: [in/32][ceil(T/16)][64 lanes][8]
  size_t ybase;   // fp32 [T][out] backbone product, original order
  size_t vpart;   // fp32 [T][rs] t = sigma * (V x), sorted order (accumulated over input slices)
  size_t dav;     // prefill, dense form: dnb slots of bf16 [drp][2 in] V operand (hi, lo)
  size_t dau;     // dnb slots of bf16 [out][3 drp] U operand (hi, hi, lo)
  size_t dtb;     // bf16 [T][3 drp] t of one segment (hi, lo, hi)
  size_t total;
  int32_t drp;    // rank rows of the dense operands (0: no dense region)
  int32_t dnb;    // operand slots: tenants whose dense products share one launch
  int32_t rs;     // row stride of vpart (max t_width over tenants)
  int32_t vb;     // max V-side rank blocks per tenant
};

// rs: max t_width over tenants; vbmax: max v_blocks over tenants.
// drp: rank rows of the dense prefill operands (0 for decode calls).
inline bool ws_layout(int32_t T, int32_t in, int32_t out, int32_t rs, int32_t n, bool with_base, int32_t vbmax,
                      int32_t drp, WsLayout* W) {
  if (T < 0 || n < 0) return false;
  W->vb = vbmax;
  size_t o = 0;
  auto take = [&](size_t bytes) { size_t at = round_up(o, kAlign); o = at + bytes; return at; };
  W->rs = rs > 0 ? rs : 8;
  W->flags = take(256);
  W->offs = take(4 * ((size_t)n + 2));
  W->perm = take(4 * (size_t)T);
  W->act = take(sizeof(ActEntry) * ((size_t)n + 1));
  const size_t items = (size_t)T * (in / kGroup);
  W->xf = take(256 * items);
  W->xsc = take(4 * items);
  W->xsum = take(4 * items);
  W->xt = take(with_base ? 2 * (size_t)in * round_up((size_t)T, 16) : 0);
  W->ybase = take(with_base ? 4 * (size_t)T * out : 0);
  W->vpart = take(4 * (size_t)T * W->rs);
  W->drp = drp;
  W->dnb = drp > 0 ? (n < 8 ? n : 8) : 0;
  W->dav = take(2 * (size_t)W->dnb * drp * 2 * in);
  W->dau = take(2 * (size_t)W->dnb * out * 3 * drp);
  W->dtb = take(2 * (size_t)T * 3 * drp);
  W->total = round_up(o, kAlign);
  return true;
}

}  // namespace dc

// Kernel launchers (defined in the .hip files).  All enqueue on `stream`
// and return a hipError_t as int.
namespace dc {
struct ApplyArgs {
  const TenantTable* tenants;  // host pointer: copied into kernel arguments
  int32_t n;
  int32_t out, in;
  int32_t rmax;
  int32_t T;
  const uint16_t* W;           // may be null
  const uint16_t* x;
  const int32_t* ids;          // device, mode 1
  const int32_t* seg;          // host, mode 2 ([n+1])
  int32_t mode;                // 0 decode (all tokens tenant 0), 1 ids, 2 segments
  uint16_t* y;
  uint8_t* ws;
  WsLayout wl;
  void* stream;
  void* const* events;         // optional DC_STAGE_COUNT + 1 hipEvent_t, may be null
};
int launch_apply(const ApplyArgs& a);
// K ranges of the split backbone product (0: the tiled product, T > 256;
// 1: one range; > 1: ybase must be zeroed before it runs, its ranges add
// into it).
int base_splits(int out, int in, int T);
int launch_base(const uint16_t* W, const uint16_t* x, const uint16_t* xt, float* ybase, int out, int in, int T,
                void* stream);
// Rank rows of the dense prefill operands of a tenant with r pairs (r rounded
// up to whole 128-row tiles, at least one tile).
int dense_rank_pad(int r);
// Prefill with long segments: backbone product, then per segment the
// tenant's operands and two dense products (see kernels.hip).
int launch_dense_prefill(const ApplyArgs& a);
int launch_dequant(const Tenant& t, int32_t out, int32_t in, uint16_t* u16, uint16_t* v16, void* stream);
int launch_pack(int32_t out, int32_t in, int32_t n8, int32_t n3, int32_t n2, const float* U, const float* sigma,
                const float* V, uint8_t* dst, uint32_t* flag, void* stream);
}  // namespace dc
