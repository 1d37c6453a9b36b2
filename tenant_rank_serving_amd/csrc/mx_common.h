// Device helpers of the gfx950 matrix-core delta kernels (shared by the
// decode kernels and the operand kernels).  Included inside namespace dc,
// anonymous namespace, of each .hip file that uses them.
//
// The 3- and 2-bit codes go straight into v_mfma_scale_f32_16x16x128_f8f6f4
// as its B operand: a 2-bit code zero-extended into an fp4 (e2m1) nibble is
// the value q/2, a 3-bit code zero-extended into an fp6 (e2m3) field is q/8,
// so unpacking a word is one AND and one shift for 16 (or ~10) codes.  The
// activations are the A operand as fp8 (e4m3) pieces with E8M0 block scales.
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
// same order.
#pragma once

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kFmtFp8 = 0, kFmtFp6 = 2, kFmtFp4 = 4;
constexpr int kScaleFp4Code = 128;   // 2^1: fp4 element q/2 -> q
constexpr int kScaleFp6Code = 130;   // 2^3: fp6 element q/8 -> q
constexpr int kXFrag = 256;          // bytes of x fragments per (token, 128-group)
constexpr int kBufFlags = 0x00020000; // buffer resource word 3: raw 32-bit dwords, bounds-checked

// A load the compiler emits as a global access: a flat load also counts
// against lgkmcnt, so every later LDS wait would wait for its memory trip too.
__device__ __forceinline__ float gload(const float* p) {
  return *(const __attribute__((address_space(1))) float*)p;
}

__device__ __forceinline__ float f16f(uint32_t h) { return (float)__builtin_bit_cast(_Float16, (uint16_t)h); }

__device__ __forceinline__ uint16_t to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

// E8M0 byte of a block whose largest magnitude is m, chosen so that
// m * 2^-E lies in [128, 256) (fits e4m3, whose largest value is 448).
__device__ __forceinline__ int block_scale_byte(float m) {
  if (!(m > 0.f)) return 127;
  int e = (int)((__float_as_uint(m) >> 23) & 0xFF);   // biased exponent of m
  if (e == 0) e = 1;                                   // subnormal m: treat as 2^-126
  int b = e - 7;                                       // 127 + (e - 127) - 7
  return b < 10 ? 10 : (b > 253 ? 253 : b);
}

__device__ __forceinline__ float pow2f(int e) { return __uint_as_float((uint32_t)(e + 127) << 23); }

// fp8 (e4m3) byte of v (|v| < 448), and its value back in fp32.
__device__ __forceinline__ uint32_t fp8_of(float v) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v, 0.f, 0, false) & 0xFFu;
}
__device__ __forceinline__ float fp8_val(uint32_t byte) { return __builtin_amdgcn_cvt_f32_fp8((int)byte, 0); }

// Position of element j (0..127) of a 128-run in the fp8 A fragments:
// lane group g and byte e, so that it meets code j of the B operand.
__device__ __forceinline__ void a_pos(int j, int& g, int& e) {
  const int a = j >> 5, w = j & 31, p = w & 1, h = w >> 1;
  if (a < 2) { g = 2 * a + p; e = h; }
  else { g = 2 * (a - 2) + p; e = 16 + h; }
}

// B operand from the 32 codes of one lane at 2 bits (two words): fp4 nibbles,
// even codes first.  Elements 0..7 = even codes of w0, 8..15 = even of w1,
// 16..23 = odd of w0, 24..31 = odd of w1.
__device__ __forceinline__ v8i b_fp4(uint32_t w0, uint32_t w1) {
  v8i b = {0, 0, 0, 0, 0, 0, 0, 0};
  b[0] = (int)(w0 & 0x33333333u);
  b[1] = (int)(w1 & 0x33333333u);
  b[2] = (int)((w0 >> 2) & 0x33333333u);
  b[3] = (int)((w1 >> 2) & 0x33333333u);
  return b;
}

// B operand from 32 codes at 3 bits (a 96-bit run w0,w1,w2): fp6 fields of
// 6 bits, even codes in fields 0..15, odd codes in 16..31.
__device__ __forceinline__ v8i b_fp6(uint32_t w0, uint32_t w1, uint32_t w2) {
  v8i b = {0, 0, 0, 0, 0, 0, 0, 0};
  b[0] = (int)(w0 & 0xC71C71C7u);
  b[1] = (int)(w1 & 0x71C71C71u);
  b[2] = (int)(w2 & 0x1C71C71Cu);
  const uint32_t s0 = __builtin_amdgcn_alignbit(w1, w0, 3);
  const uint32_t s1 = __builtin_amdgcn_alignbit(w2, w1, 3);
  const uint32_t s2 = w2 >> 3;
  b[3] = (int)(s0 & 0xC71C71C7u);
  b[4] = (int)(s1 & 0x71C71C71u);
  b[5] = (int)(s2 & 0x1C71C71Cu);
  return b;
}

// Keeps the source registers of a chain of matrix-core ops allocated until
// its result has been read back into `d`.  Without it the register allocator
// may hand an A operand or scale VGPR of an op still in flight to a load
// issued after it (observed: an LDS load landing in the A and scale VGPRs of
// the preceding v_mfma_scale changed its result).
__device__ __forceinline__ void hold(f32x4& d, const v8i& a, const v8i& b, int s0, int sb) {
  asm volatile("" : "+v"(d) : "v"(a), "v"(b), "v"(s0), "v"(sb));
}
__device__ __forceinline__ void hold(f32x4& d, const v8i& a0, const v8i& a1, const v8i& b, int s0, int s1, int sb) {
  asm volatile("" : "+v"(d) : "v"(a0), "v"(a1), "v"(b), "v"(s0), "v"(s1), "v"(sb));
}
__device__ __forceinline__ void hold(f32x4& d, const v8i& a0, const v8i& a1, const v8i& a2, const v8i& b, int s0,
                                     int s1, int s2, int sb) {
  asm volatile("" : "+v"(d) : "v"(a0), "v"(a1), "v"(a2), "v"(b), "v"(s0), "v"(s1), "v"(s2), "v"(sb));
}

__device__ __forceinline__ void hold2(f32x4& d0, f32x4& d1, const v8i& a, const v8i& b0, const v8i& b1, int sa,
                                      int sb) {
  asm volatile("" : "+v"(d0), "+v"(d1) : "v"(a), "v"(b0), "v"(b1), "v"(sa), "v"(sb));
}

// v from lane l ^ X (X < 32) by ds_swizzle: no lane-address register, unlike
// a general shuffle.
template <int X>
__device__ __forceinline__ float swz_xor(float v) {
  static_assert(X > 0 && X < 32, "swizzle lanes stay within 32-lane halves");
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), (X << 10) | 0x1F));
}

// Workgroup barrier that orders LDS only: unlike __syncthreads() it does not
// wait for the wave's global loads and stores in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// The same for a kernel with LDS-DMA loads in flight: a fence would wait for
// them too (vmcnt(0)).  The stores it orders are plain LDS stores (complete
// at lgkmcnt(0)); DMA-filled LDS is read only by the wave that loads it,
// after its own count-based wait.
__device__ __forceinline__ void lds_barrier_keep_vm() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ v8i v8_of(const uint4& a, const uint4& b) {
  return v8i{(int)a.x, (int)a.y, (int)a.z, (int)a.w, (int)b.x, (int)b.y, (int)b.z, (int)b.w};
}

__device__ __forceinline__ f32x4 mma(const v8i& a, const v8i& b, f32x4 c, int sa, int fmt_b, int sb) {
  if (fmt_b == kFmtFp4)
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, kFmtFp8, kFmtFp4, 0, sa, 0, sb);
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, kFmtFp8, kFmtFp6, 0, sa, 0, sb);
}

