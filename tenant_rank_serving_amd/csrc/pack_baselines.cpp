// Host side of the two baselines the pages compare Delta-CoMe with: sizes
// and packers of the fp16 low-rank delta and of the 1-bit BitDelta delta
// ("Delta-CoMe: Training-Free Delta-Compression with Mixed-Precision for
// LLMs", Experimental setup: low-rank SVD compression and BitDelta as
// baselines; the formats are this library's, include/deltacome.h).  Plain
// C++17, no GPU code.
#include <cmath>
#include <cstring>

#include "dc_internal.h"

namespace {

bool baseline_ok(int32_t kind, int32_t out, int32_t in, int32_t r) { return dc::baseline_valid(kind, out, in, r); }

// Slot of the 8-element run (row, col) of a 16-row, 32-column tile step:
// [rows/16][cols/32][64][8], slot (row % 16) + 16 ((col % 32) / 8).
size_t tile_index(size_t row, size_t col, size_t cols) {
  const size_t step = col / 32, slot = (row % 16) + 16 * ((col % 32) / 8);
  return (((row / 16) * (cols / 32) + step) * 64 + slot) * 8 + col % 8;
}

// Bit of a BitDelta word that holds entry k (0..31) of its 32 columns: even
// entries fill the low nibble positions first, so that a shift by s and a
// mask of one bit per nibble gives 8 entries in matrix-core element order.
int sign_bit(int k) {
  const int kp = (k % 2 == 0) ? k / 2 : 16 + k / 2;
  return 4 * (kp % 8) + kp / 8;
}

}  // namespace

extern "C" {

size_t dc_baseline_bytes(int32_t kind, int32_t out, int32_t in, int32_t r) {
  if (!baseline_ok(kind, out, in, r)) return 0;
  return kind == DC_KIND_LOWRANK ? dc::lowrank_bytes(out, in, r) : dc::bitdelta_bytes(out, in);
}

size_t dc_baseline_algorithmic_bytes(int32_t kind, int32_t out, int32_t in, int32_t r) {
  if (!baseline_ok(kind, out, in, r)) return 0;
  if (kind == DC_KIND_LOWRANK) return 2 * (size_t)r * ((size_t)out + in) + 4 * (size_t)r;
  return (size_t)out * in / 8 + 4;
}

dc_status dc_pack_lowrank(int32_t out, int32_t in, int32_t r, const uint16_t* U, const float* sigma,
                          const uint16_t* V, void* dst, size_t dst_bytes) {
  if (!dst) return DC_ERR_INVALID_ARG;
  if (!baseline_ok(DC_KIND_LOWRANK, out, in, r)) return DC_ERR_SHAPE;
  if (r > 0 && (!U || !sigma || !V)) return DC_ERR_INVALID_ARG;
  const size_t need = dc::lowrank_bytes(out, in, r);
  if (dst_bytes < need) return DC_ERR_BUFFER;
  uint8_t* b = static_cast<uint8_t*>(dst);
  std::memset(b, 0, need);
  if (r > 0) std::memcpy(b, sigma, 4 * (size_t)r);
  uint16_t* v = reinterpret_cast<uint16_t*>(b + dc::lowrank_v_offset(r));
  uint16_t* u = reinterpret_cast<uint16_t*>(b + dc::lowrank_u_offset(in, r));
  const size_t r32 = dc::round_up((size_t)r, 32);
  for (size_t i = 0; i < (size_t)r; ++i) {
    for (size_t k = 0; k < (size_t)in; ++k) v[tile_index(i, k, in)] = V[i * in + k];
    for (size_t o = 0; o < (size_t)out; ++o) u[tile_index(o, i, r32)] = U[i * out + o];
  }
  return DC_OK;
}

dc_status dc_pack_bitdelta(int32_t out, int32_t in, const uint8_t* signs, float alpha, void* dst,
                           size_t dst_bytes) {
  if (!dst || !signs) return DC_ERR_INVALID_ARG;
  if (!baseline_ok(DC_KIND_BITDELTA, out, in, 0)) return DC_ERR_SHAPE;
  if (!std::isfinite(alpha)) return DC_ERR_RANGE;
  const size_t need = dc::bitdelta_bytes(out, in);
  if (dst_bytes < need) return DC_ERR_BUFFER;
  uint8_t* b = static_cast<uint8_t*>(dst);
  std::memset(b, 0, dc::kAlign);
  std::memcpy(b, &alpha, 4);
  uint32_t* w = reinterpret_cast<uint32_t*>(b + dc::kAlign);
  const size_t gi = (size_t)in / dc::kGroup;
  for (size_t tile = 0; tile < (size_t)out / 16; ++tile)
    for (size_t g = 0; g < gi; ++g)
      for (size_t c = 0; c < 4; ++c)
        for (size_t i = 0; i < 16; ++i) {
          const uint8_t* row = signs + (tile * 16 + i) * in + g * dc::kGroup + c * 32;
          uint32_t word = 0;
          for (int k = 0; k < 32; ++k)
            if (row[k]) word |= 1u << sign_bit(k);
          w[((tile * gi + g) * 4 + c) * 16 + i] = word;
        }
  return DC_OK;
}

}  // extern "C"
