// Host side of libdeltacome.so: spec checks, the packed format, the RTN
// quantizer and the packer.  Plain C++17, no GPU code.
//
// The quantizer follows the compression steps of the pages: singular pairs in
// descending singular-value order, the first n8 kept at 8 bits, the next n3
// at 3, the next n2 at 2, the rest dropped ("Delta-CoMe - 清华联合OpenBMB...",
// technical principles; "Delta-CoMe: Training-Free Delta-Compression with
// Mixed-Precision for LLMs", Approach).  The per-group min/max RTN with an
// fp16 scale and zero is this library's storage format (include/deltacome.h).
#include <cmath>
#include <cstring>
#include <vector>

#include "dc_internal.h"

namespace {

using dc::Layout;

bool spec_ok(const dc_spec* s) {
  if (!s) return false;
  if (s->out <= 0 || s->in <= 0 || s->out % dc::kGroup || s->in % dc::kGroup) return false;
  if (s->n8 < 0 || s->n3 < 0 || s->n2 < 0) return false;
  const int64_t r = (int64_t)s->n8 + s->n3 + s->n2;
  const int64_t lim = s->out < s->in ? s->out : s->in;
  return r <= lim;
}

using dc::f16_to_f64;
using dc::f64_to_f16;

// Quantize one group of 128 values at `bits`; writes codes and the
// (scale, zero) fp16 bit patterns.  Returns false on non-finite input or
// fp16 scale overflow.
bool quantize_group(const float* w, int bits, uint8_t* codes, uint16_t* sh_out, uint16_t* z_out) {
  const int maxq = (1 << bits) - 1;
  double mn = 0.0, mx = 0.0;
  for (int k = 0; k < dc::kGroup; ++k) {
    const double v = (double)w[k];
    if (!std::isfinite(v)) return false;
    if (v < mn) mn = v;
    if (v > mx) mx = v;
  }
  uint16_t sh = f64_to_f16((mx - mn) / maxq);
  if ((sh & 0x7FFF) == 0) sh = 0x3C00;      // 1.0
  if ((sh & 0x7C00) == 0x7C00) return false;
  const double s = f16_to_f64(sh);
  double z = std::nearbyint(-mn / s);
  if (z < 0) z = 0;
  if (z > maxq) z = maxq;
  for (int k = 0; k < dc::kGroup; ++k) {
    double q = std::nearbyint((double)w[k] / s) + z;
    if (q < 0) q = 0;
    if (q > maxq) q = maxq;
    codes[k] = (uint8_t)q;
  }
  *sh_out = sh;
  *z_out = f64_to_f16(z);
  return true;
}

// Writes code c at b bits as element k of the bitstream starting at words.
inline void put_code(uint32_t* words, int b, size_t k, uint32_t c) {
  const size_t bit = (size_t)b * k;
  const size_t w = bit >> 5;
  const unsigned sh = (unsigned)(bit & 31);
  words[w] |= c << sh;
  if (sh + b > 32) words[w + 1] |= c >> (32 - sh);
}

inline uint32_t get_code(const uint32_t* words, int b, size_t k) {
  const size_t bit = (size_t)b * k;
  const size_t w = bit >> 5;
  const unsigned sh = (unsigned)(bit & 31);
  uint64_t v = words[w] >> sh;
  if (sh + b > 32) v |= (uint64_t)words[w + 1] << (32 - sh);
  return (uint32_t)(v & ((1u << b) - 1));
}

struct Seg { int b; int lo; int n; int reg_vc, reg_vs, reg_uc, reg_us; };

void segments(const dc_spec* s, Seg out[3]) {
  out[0] = {8, 0, s->n8, DC_REG_VC8, DC_REG_VS8, DC_REG_UC8, DC_REG_US8};
  out[1] = {3, s->n8, s->n3, DC_REG_VC3, DC_REG_VS3, DC_REG_UC3, DC_REG_US3};
  out[2] = {2, s->n8 + s->n3, s->n2, DC_REG_VC2, DC_REG_VS2, DC_REG_UC2, DC_REG_US2};
}

// Packs codes/scales into `out` (already zeroed, layout L).
dc_status pack_into(const dc_spec* s, const Layout& L, const uint8_t* cu, const uint8_t* cv,
                    const uint16_t* szu, const uint16_t* szv, const float* sigma, uint8_t* out) {
  const int gi = s->in / dc::kGroup, go = s->out / dc::kGroup;
  const int r = s->n8 + s->n3 + s->n2;
  std::memcpy(out + L.off[DC_REG_SIGMA], sigma, 4 * (size_t)r);
  Seg sg[3];
  segments(s, sg);
  for (const Seg& g : sg) {
    const uint32_t lim = 1u << g.b;
    // V codes: 8-bit [n][Gi][32] words, one bitstream per 128-element group;
    // 3- and 2-bit in 16-rank tiles, [ceil(n/16)][Gi][4][16][b] words.
    uint32_t* vc = reinterpret_cast<uint32_t*>(out + L.off[g.reg_vc]);
    for (int i = 0; i < g.n; ++i) {
      const uint8_t* row = cv + (size_t)(g.lo + i) * s->in;
      for (int grp = 0; grp < gi; ++grp) {
        for (int k = 0; k < dc::kGroup; ++k) {
          const uint32_t c = row[grp * dc::kGroup + k];
          if (c >= lim) return DC_ERR_RANGE;
          if (g.b == 8)
            put_code(vc + ((size_t)i * gi + grp) * 32, 8, k, c);
          else
            put_code(vc + dc::v_chunk_word(i, grp, k / 32, gi, g.b), g.b, k % 32, c);
        }
      }
    }
    // V scale/zero: [Gi][pad4(n)].
    uint32_t* vs = reinterpret_cast<uint32_t*>(out + L.off[g.reg_vs]);
    const size_t np = dc::round_up(g.n, 4);
    for (int i = 0; i < g.n; ++i)
      for (int grp = 0; grp < gi; ++grp) {
        const uint16_t* e = szv + ((size_t)(g.lo + i) * gi + grp) * 2;
        vs[(size_t)grp * np + i] = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
      }
    // U codes.
    if (g.b == 8) {
      uint8_t* uc = out + L.off[g.reg_uc];
      for (int i = 0; i < g.n; ++i) {
        const uint8_t* col = cu + (size_t)(g.lo + i) * s->out;
        for (int o = 0; o < s->out; ++o) uc[(size_t)o * g.n + i] = col[o];
      }
    } else {
      uint32_t* uc = reinterpret_cast<uint32_t*>(out + L.off[g.reg_uc]);
      for (int i = 0; i < g.n; ++i) {
        const uint8_t* col = cu + (size_t)(g.lo + i) * s->out;
        const int kb = i / dc::kKBlock, k = i % dc::kKBlock;
        for (int o = 0; o < s->out; ++o) {
          const uint32_t c = col[o];
          if (c >= lim) return DC_ERR_RANGE;
          int nw;
          uint32_t* words = uc + dc::u_kblock_word(o, kb, g.n, g.b, &nw);
          put_code(words, g.b, k, c);
        }
      }
    }
    // U scale/zero: [Go][pad4(n)].
    uint32_t* us = reinterpret_cast<uint32_t*>(out + L.off[g.reg_us]);
    for (int i = 0; i < g.n; ++i)
      for (int grp = 0; grp < go; ++grp) {
        const uint16_t* e = szu + ((size_t)(g.lo + i) * go + grp) * 2;
        us[(size_t)grp * np + i] = (uint32_t)e[0] | ((uint32_t)e[1] << 16);
      }
  }
  return DC_OK;
}

}  // namespace

extern "C" {

const char* dc_status_string(dc_status s) {
  switch (s) {
    case DC_OK: return "DC_OK";
    case DC_ERR_INVALID_ARG: return "DC_ERR_INVALID_ARG";
    case DC_ERR_SHAPE: return "DC_ERR_SHAPE";
    case DC_ERR_ALIGN: return "DC_ERR_ALIGN";
    case DC_ERR_BUFFER: return "DC_ERR_BUFFER";
    case DC_ERR_RANGE: return "DC_ERR_RANGE";
    case DC_ERR_HIP: return "DC_ERR_HIP";
    case DC_ERR_UNSUPPORTED: return "DC_ERR_UNSUPPORTED";
    default: return "DC_ERR_UNKNOWN";
  }
}

dc_status dc_check_spec(const dc_spec* spec) {
  if (!spec) return DC_ERR_INVALID_ARG;
  return spec_ok(spec) ? DC_OK : DC_ERR_SHAPE;
}

size_t dc_packed_bytes(const dc_spec* s) {
  if (!spec_ok(s)) return 0;
  Layout L;
  dc::layout_of(s->out, s->in, s->n8, s->n3, s->n2, &L);
  return L.total;
}

size_t dc_algorithmic_bytes(const dc_spec* s) {
  if (!spec_ok(s)) return 0;
  const size_t r = (size_t)s->n8 + s->n3 + s->n2;
  const size_t codes = ((size_t)8 * s->n8 + 3 * (size_t)s->n3 + 2 * (size_t)s->n2) *
                       ((size_t)s->out + s->in) / 8;
  return codes + r * (size_t)(s->in / dc::kGroup + s->out / dc::kGroup) * 4 + 4 * r;
}

dc_status dc_region(const dc_spec* s, int32_t region, size_t* offset, size_t* size) {
  if (!s || !offset || !size) return DC_ERR_INVALID_ARG;
  if (!spec_ok(s)) return DC_ERR_SHAPE;
  if (region < 0 || region >= DC_REG_COUNT) return DC_ERR_INVALID_ARG;
  Layout L;
  dc::layout_of(s->out, s->in, s->n8, s->n3, s->n2, &L);
  *offset = L.off[region];
  *size = L.size[region];
  return DC_OK;
}

dc_status dc_pack_codes(const dc_spec* s, const uint8_t* codes_u, const uint8_t* codes_v,
                        const uint16_t* sz_u, const uint16_t* sz_v, const float* sigma,
                        void* out, size_t out_bytes) {
  if (!s || !out) return DC_ERR_INVALID_ARG;
  if (!spec_ok(s)) return DC_ERR_SHAPE;
  const int r = s->n8 + s->n3 + s->n2;
  if (r > 0 && (!codes_u || !codes_v || !sz_u || !sz_v || !sigma)) return DC_ERR_INVALID_ARG;
  Layout L;
  dc::layout_of(s->out, s->in, s->n8, s->n3, s->n2, &L);
  if (out_bytes < L.total) return DC_ERR_BUFFER;
  std::memset(out, 0, L.total);
  return pack_into(s, L, codes_u, codes_v, sz_u, sz_v, sigma, static_cast<uint8_t*>(out));
}

dc_status dc_pack(const dc_spec* s, const float* U, const float* sigma, const float* V, void* out,
                  size_t out_bytes) {
  if (!s || !out) return DC_ERR_INVALID_ARG;
  if (!spec_ok(s)) return DC_ERR_SHAPE;
  const int r = s->n8 + s->n3 + s->n2;
  if (r > 0 && (!U || !V || !sigma)) return DC_ERR_INVALID_ARG;
  Layout L;
  dc::layout_of(s->out, s->in, s->n8, s->n3, s->n2, &L);
  if (out_bytes < L.total) return DC_ERR_BUFFER;
  const int gi = s->in / dc::kGroup, go = s->out / dc::kGroup;
  std::vector<uint8_t> cu((size_t)r * s->out), cv((size_t)r * s->in);
  std::vector<uint16_t> szu((size_t)r * go * 2), szv((size_t)r * gi * 2);
  for (int i = 0; i < r; ++i) {
    const int b = i < s->n8 ? 8 : (i < s->n8 + s->n3 ? 3 : 2);
    if (!std::isfinite(sigma[i])) return DC_ERR_RANGE;
    for (int g = 0; g < go; ++g)
      if (!quantize_group(U + (size_t)i * s->out + (size_t)g * dc::kGroup, b,
                          &cu[(size_t)i * s->out + (size_t)g * dc::kGroup],
                          &szu[((size_t)i * go + g) * 2], &szu[((size_t)i * go + g) * 2 + 1]))
        return DC_ERR_RANGE;
    for (int g = 0; g < gi; ++g)
      if (!quantize_group(V + (size_t)i * s->in + (size_t)g * dc::kGroup, b,
                          &cv[(size_t)i * s->in + (size_t)g * dc::kGroup],
                          &szv[((size_t)i * gi + g) * 2], &szv[((size_t)i * gi + g) * 2 + 1]))
        return DC_ERR_RANGE;
  }
  std::memset(out, 0, L.total);
  return pack_into(s, L, cu.data(), cv.data(), szu.data(), szv.data(), sigma,
                   static_cast<uint8_t*>(out));
}

dc_status dc_unpack(const dc_spec* s, const void* packed, size_t packed_bytes, uint8_t* codes_u,
                    uint8_t* codes_v, uint16_t* sz_u, uint16_t* sz_v, float* sigma) {
  if (!s || !packed) return DC_ERR_INVALID_ARG;
  if (!spec_ok(s)) return DC_ERR_SHAPE;
  const int r = s->n8 + s->n3 + s->n2;
  if (r > 0 && (!codes_u || !codes_v || !sz_u || !sz_v || !sigma)) return DC_ERR_INVALID_ARG;
  Layout L;
  dc::layout_of(s->out, s->in, s->n8, s->n3, s->n2, &L);
  if (packed_bytes < L.total) return DC_ERR_BUFFER;
  const uint8_t* in = static_cast<const uint8_t*>(packed);
  const int gi = s->in / dc::kGroup, go = s->out / dc::kGroup;
  std::memcpy(sigma, in + L.off[DC_REG_SIGMA], 4 * (size_t)r);
  Seg sg[3];
  segments(s, sg);
  for (const Seg& g : sg) {
    const uint32_t* vc = reinterpret_cast<const uint32_t*>(in + L.off[g.reg_vc]);
    for (int i = 0; i < g.n; ++i)
      for (int grp = 0; grp < gi; ++grp) {
        for (int k = 0; k < dc::kGroup; ++k) {
          const uint32_t c = g.b == 8 ? get_code(vc + ((size_t)i * gi + grp) * 32, 8, k)
                                      : get_code(vc + dc::v_chunk_word(i, grp, k / 32, gi, g.b), g.b, k % 32);
          codes_v[(size_t)(g.lo + i) * s->in + grp * dc::kGroup + k] = (uint8_t)c;
        }
      }
    const size_t np = dc::round_up(g.n, 4);
    const uint32_t* vs = reinterpret_cast<const uint32_t*>(in + L.off[g.reg_vs]);
    for (int i = 0; i < g.n; ++i)
      for (int grp = 0; grp < gi; ++grp) {
        const uint32_t e = vs[(size_t)grp * np + i];
        sz_v[((size_t)(g.lo + i) * gi + grp) * 2] = (uint16_t)(e & 0xFFFF);
        sz_v[((size_t)(g.lo + i) * gi + grp) * 2 + 1] = (uint16_t)(e >> 16);
      }
    if (g.b == 8) {
      const uint8_t* uc = in + L.off[g.reg_uc];
      for (int i = 0; i < g.n; ++i)
        for (int o = 0; o < s->out; ++o)
          codes_u[(size_t)(g.lo + i) * s->out + o] = uc[(size_t)o * g.n + i];
    } else {
      const uint32_t* uc = reinterpret_cast<const uint32_t*>(in + L.off[g.reg_uc]);
      for (int i = 0; i < g.n; ++i)
        for (int o = 0; o < s->out; ++o) {
          int nw;
          const uint32_t* words = uc + dc::u_kblock_word(o, i / dc::kKBlock, g.n, g.b, &nw);
          codes_u[(size_t)(g.lo + i) * s->out + o] = (uint8_t)get_code(words, g.b, i % dc::kKBlock);
        }
    }
    const uint32_t* us = reinterpret_cast<const uint32_t*>(in + L.off[g.reg_us]);
    for (int i = 0; i < g.n; ++i)
      for (int grp = 0; grp < go; ++grp) {
        const uint32_t e = us[(size_t)grp * np + i];
        sz_u[((size_t)(g.lo + i) * go + grp) * 2] = (uint16_t)(e & 0xFFFF);
        sz_u[((size_t)(g.lo + i) * go + grp) * 2 + 1] = (uint16_t)(e >> 16);
      }
  }
  return DC_OK;
}

}  // extern "C"
