// The library's host-only C++ (the packer and unpacker, the region table,
// the bit allocation, the baseline packers) run under AddressSanitizer and
// UndefinedBehaviorSanitizer on seeded inputs and edge cases.  Built with g++
// by test_host_sanitized.py together with csrc/pack.cpp, csrc/alloc.cpp and
// csrc/pack_baselines.cpp; any out-of-bounds access, leak or undefined
// behaviour aborts the run, and every check below must hold.  Prints "OK".
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <random>
#include <vector>

#include "deltacome.h"

#define CHECK(c)                                                        \
  do {                                                                  \
    if (!(c)) {                                                         \
      std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #c); \
      return 1;                                                         \
    }                                                                   \
  } while (0)

namespace {

// Inputs of one delta: mode 0 Gaussian rows of varied magnitude, 1 all zero,
// 2 rows whose largest magnitude is 3e-5 (fp16-subnormal scales), 3 constant
// rows (zero range within each group except through the zero point).
void make_vectors(int mode, int r, int n, std::mt19937_64& g, std::vector<float>& a) {
  a.assign((size_t)r * n, 0.f);
  std::normal_distribution<float> nd(0.f, 1.f);
  std::uniform_real_distribution<float> ud(-6.f, 1.f);
  for (int i = 0; i < r; ++i) {
    const float mag = std::exp(ud(g));
    for (int j = 0; j < n; ++j) {
      float v = 0.f;
      if (mode == 0) v = nd(g) * mag;
      if (mode == 2) v = nd(g) * 1e-5f;
      if (mode == 3) v = 0.25f * (float)(i + 1);
      a[(size_t)i * n + j] = v;
    }
    if (mode == 2) {  // scale the row so its largest magnitude is exactly 3e-5
      float m = 0.f;
      for (int j = 0; j < n; ++j) m = std::fmax(m, std::fabs(a[(size_t)i * n + j]));
      if (m > 0.f)
        for (int j = 0; j < n; ++j) a[(size_t)i * n + j] *= 3e-5f / m;
    }
  }
}

int check_pack(const dc_spec& s, int mode, uint64_t seed) {
  std::mt19937_64 g(seed);
  const int r = s.n8 + s.n3 + s.n2;
  std::vector<float> U, V, sigma(r);
  make_vectors(mode, r, s.out, g, U);
  make_vectors(mode, r, s.in, g, V);
  for (int i = 0; i < r; ++i) sigma[i] = std::exp(-0.5f * (float)i);
  CHECK(dc_check_spec(&s) == DC_OK);
  const size_t bytes = dc_packed_bytes(&s);
  if (r == 0) {  // a delta with no pairs stores nothing
    CHECK(bytes == 0 && dc_algorithmic_bytes(&s) == 0);
    return 0;
  }
  CHECK(bytes > 0);
  CHECK(dc_algorithmic_bytes(&s) <= bytes);
  // every region inside the buffer, in storage order, not overlapping
  size_t end = 0;
  for (int reg = 0; reg < DC_REG_COUNT; ++reg) {
    size_t off = 0, sz = 0;
    CHECK(dc_region(&s, reg, &off, &sz) == DC_OK);
    CHECK(off >= end && off + sz <= bytes);
    end = off + sz;
  }
  size_t off = 0, sz = 0;
  CHECK(dc_region(&s, DC_REG_COUNT, &off, &sz) != DC_OK);
  // exact-size buffers: the sanitizers see any write past them
  std::vector<uint8_t> buf(bytes), buf2(bytes);
  CHECK(dc_pack(&s, U.data(), sigma.data(), V.data(), buf.data(), bytes) == DC_OK);
  CHECK(dc_pack(&s, U.data(), sigma.data(), V.data(), buf2.data(), bytes - 1) == DC_ERR_BUFFER);
  std::vector<uint8_t> cu((size_t)r * s.out), cv((size_t)r * s.in);
  std::vector<uint16_t> szu((size_t)r * (s.out / 128) * 2), szv((size_t)r * (s.in / 128) * 2);
  std::vector<float> sg(r);
  CHECK(dc_unpack(&s, buf.data(), bytes, cu.data(), cv.data(), szu.data(), szv.data(), sg.data()) == DC_OK);
  CHECK(dc_unpack(&s, buf.data(), bytes - 1, cu.data(), cv.data(), szu.data(), szv.data(), sg.data()) ==
        DC_ERR_BUFFER);
  for (int i = 0; i < r; ++i) CHECK(std::memcmp(&sg[i], &sigma[i], 4) == 0);
  // codes within their widths, and packing the unpacked arrays gives the same bytes
  for (int i = 0; i < r; ++i) {
    const int b = i < s.n8 ? 8 : (i < s.n8 + s.n3 ? 3 : 2);
    for (int j = 0; j < s.out; ++j) CHECK(cu[(size_t)i * s.out + j] < (1u << b));
    for (int j = 0; j < s.in; ++j) CHECK(cv[(size_t)i * s.in + j] < (1u << b));
  }
  std::memset(buf2.data(), 0xA5, bytes);
  CHECK(dc_pack_codes(&s, cu.data(), cv.data(), szu.data(), szv.data(), sg.data(), buf2.data(), bytes) == DC_OK);
  CHECK(std::memcmp(buf.data(), buf2.data(), bytes) == 0);
  if (s.n2 > 0) {  // a code past its segment's width is rejected
    const size_t at = (size_t)(s.n8 + s.n3) * s.out;
    const uint8_t keep = cu[at];
    cu[at] = 4;
    CHECK(dc_pack_codes(&s, cu.data(), cv.data(), szu.data(), szv.data(), sg.data(), buf2.data(), bytes) ==
          DC_ERR_RANGE);
    cu[at] = keep;
  }
  if (r > 0) {  // a non-finite input is rejected
    const float keep = V[0];
    V[0] = NAN;
    CHECK(dc_pack(&s, U.data(), sigma.data(), V.data(), buf2.data(), bytes) == DC_ERR_RANGE);
    V[0] = INFINITY;
    CHECK(dc_pack(&s, U.data(), sigma.data(), V.data(), buf2.data(), bytes) == DC_ERR_RANGE);
    V[0] = keep;
  }
  CHECK(dc_pack(&s, nullptr, sigma.data(), V.data(), buf2.data(), bytes) == DC_ERR_INVALID_ARG);
  CHECK(dc_pack(&s, U.data(), sigma.data(), V.data(), nullptr, bytes) == DC_ERR_INVALID_ARG);
  return 0;
}

// Smallest total error over all choices by enumeration (r * nb small).
double brute(int r, int nb, const int32_t* cost, const double* err, int64_t budget, bool* found) {
  double best = INFINITY;
  *found = false;
  std::vector<int> c(r, 0);
  for (;;) {
    int64_t used = 0;
    double e = 0.0;
    for (int i = 0; i < r; ++i) {
      used += cost[c[i]];
      e += err[(size_t)i * nb + c[i]];
    }
    if (used <= budget && e < best) {
      best = e;
      *found = true;
    }
    int i = 0;
    while (i < r && ++c[i] == nb) c[i++] = 0;
    if (i == r) break;
  }
  return best;
}

int check_alloc(uint64_t seed) {
  std::mt19937_64 g(seed);
  const int32_t cost[4] = {0, 2, 3, 8};
  for (int rep = 0; rep < 60; ++rep) {
    const int r = (int)(g() % 7);
    std::vector<double> err((size_t)r * 4);
    std::uniform_real_distribution<double> ud(0.0, 1.0);
    for (int i = 0; i < r; ++i) {  // error falls with the width, as in the error model
      const double e0 = ud(g) + 0.5;
      err[(size_t)i * 4 + 0] = e0;
      err[(size_t)i * 4 + 1] = e0 * ud(g) * 0.5;
      err[(size_t)i * 4 + 2] = err[(size_t)i * 4 + 1] * ud(g);
      err[(size_t)i * 4 + 3] = err[(size_t)i * 4 + 2] * ud(g) * 0.01;
    }
    const int64_t budget = (int64_t)(g() % (8 * (uint64_t)r + 3));
    std::vector<int32_t> choice(r > 0 ? r : 1, -1);
    double total = -1.0;
    const dc_status st = dc_allocate_bits(r, 4, cost, err.data(), budget, choice.data(), &total);
    bool found = false;
    const double best = brute(r, 4, cost, err.data(), budget, &found);
    CHECK(found ? st == DC_OK : st == DC_ERR_RANGE);
    if (st == DC_OK) {
      int64_t used = 0;
      double e = 0.0;
      for (int i = 0; i < r; ++i) {
        CHECK(choice[i] >= 0 && choice[i] < 4);
        used += cost[choice[i]];
        e += err[(size_t)i * 4 + choice[i]];
      }
      CHECK(used <= budget);
      CHECK(std::fabs(e - best) <= 1e-12 * (1.0 + best));
      CHECK(std::fabs(total - best) <= 1e-12 * (1.0 + best));
    }
  }
  // invalid arguments
  int32_t ch[2];
  double er[8] = {1, 0.5, 0.2, 0.1, 1, 0.5, 0.2, 0.1};
  const int32_t bad_cost[4] = {0, -1, 3, 8};
  CHECK(dc_allocate_bits(2, 4, cost, nullptr, 10, ch, nullptr) == DC_ERR_INVALID_ARG);
  CHECK(dc_allocate_bits(2, 4, bad_cost, er, 10, ch, nullptr) == DC_ERR_INVALID_ARG);
  CHECK(dc_allocate_bits(2, 0, cost, er, 10, ch, nullptr) == DC_ERR_INVALID_ARG);
  er[5] = NAN;
  CHECK(dc_allocate_bits(2, 4, cost, er, 10, ch, nullptr) == DC_ERR_INVALID_ARG);
  return 0;
}

int check_baselines(uint64_t seed) {
  std::mt19937_64 g(seed);
  const int shapes[][3] = {{128, 128, 0}, {128, 256, 1}, {256, 128, 17}, {384, 256, 33}};
  for (const auto& sh : shapes) {
    const int out = sh[0], in = sh[1], r = sh[2];
    const size_t bytes = dc_baseline_bytes(DC_KIND_LOWRANK, out, in, r);
    CHECK(r == 0 ? bytes == 0 : bytes > 0);
    std::vector<uint16_t> U((size_t)r * out + 1), V((size_t)r * in + 1);
    std::vector<float> sigma(r + 1, 1.f);
    for (auto& u : U) u = (uint16_t)(0x3000 | (g() & 0x3FF) | ((g() & 1) << 15));   // finite fp16
    for (auto& v : V) v = (uint16_t)(0x3000 | (g() & 0x3FF) | ((g() & 1) << 15));
    std::vector<uint8_t> dst(bytes > 0 ? bytes : 1);
    if (r > 0) {
      CHECK(dc_pack_lowrank(out, in, r, U.data(), sigma.data(), V.data(), dst.data(), bytes) == DC_OK);
      CHECK(dc_pack_lowrank(out, in, r, U.data(), sigma.data(), V.data(), dst.data(), bytes - 1) == DC_ERR_BUFFER);
      CHECK(dc_pack_lowrank(out, in, r, nullptr, sigma.data(), V.data(), dst.data(), bytes) == DC_ERR_INVALID_ARG);
    }
    const size_t bb = dc_baseline_bytes(DC_KIND_BITDELTA, out, in, 0);
    CHECK(bb >= (size_t)out * in / 8 + 4);
    std::vector<uint8_t> signs((size_t)out * in), bd(bb);
    for (auto& s : signs) s = (uint8_t)(g() & 1);
    CHECK(dc_pack_bitdelta(out, in, signs.data(), 0.125f, bd.data(), bb) == DC_OK);
    CHECK(dc_pack_bitdelta(out, in, signs.data(), 0.125f, bd.data(), bb - 1) == DC_ERR_BUFFER);
    CHECK(dc_pack_bitdelta(out, in, signs.data(), NAN, bd.data(), bb) == DC_ERR_RANGE);
    // the scale leads the buffer; past its header every sign is one stored bit
    float alpha;
    std::memcpy(&alpha, bd.data(), 4);
    CHECK(alpha == 0.125f);
    const size_t hdr = bb - (size_t)out * in / 8;
    size_t ones = 0, want = 0;
    for (size_t i = hdr; i < bb; ++i) ones += (size_t)__builtin_popcount(bd[i]);
    for (auto s : signs) want += s != 0;
    CHECK(ones == want);
  }
  CHECK(dc_baseline_bytes(DC_KIND_LOWRANK, 100, 128, 4) == 0);
  CHECK(dc_baseline_bytes(7, 128, 128, 4) == 0);
  return 0;
}

}  // namespace

int main() {
  const dc_spec specs[] = {
      {128, 128, 0, 0, 0},     {256, 256, 2, 8, 22},   {384, 128, 3, 0, 17},  {128, 384, 0, 33, 0},
      {512, 256, 5, 31, 65},   {128, 128, 1, 1, 1},    {256, 128, 0, 0, 100}, {1024, 512, 2, 20, 150},
  };
  uint64_t seed = 1;
  for (const dc_spec& s : specs)
    for (int mode = 0; mode < 4; ++mode)
      if (check_pack(s, mode, seed++)) {
        std::fprintf(stderr, "spec %d x %d (%d, %d, %d), mode %d\n", s.out, s.in, s.n8, s.n3, s.n2, mode);
        return 1;
      }
  const dc_spec bad[] = {{100, 128, 0, 0, 1}, {128, 0, 0, 0, 1}, {128, 128, -1, 0, 0}, {128, 128, 100, 100, 100}};
  for (const dc_spec& s : bad) CHECK(dc_check_spec(&s) != DC_OK && dc_packed_bytes(&s) == 0);
  CHECK(dc_check_spec(nullptr) == DC_ERR_INVALID_ARG);
  if (check_alloc(77)) return 1;
  if (check_baselines(99)) return 1;
  std::printf("OK\n");
  return 0;
}
