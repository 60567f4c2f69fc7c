// Shared device helpers for the banded Sinkhorn attention kernels (gfx950).
//
// Tiles are 16 x 16.  Score tiles come from v_mfma_f32_16x16x32_bf16 (bf16
// inputs, one instruction per 32-wide k chunk) or v_mfma_f32_16x16x4f32
// (fp32 inputs, four instructions per 16-wide k chunk).  In both cases a lane
// feeds 16 contiguous bytes of its operand row per chunk: lane l reads row
// (l % 16) at byte offset 64 * chunk + 16 * (l / 16).  The k ordering inside
// a chunk is the same for both operands, so the contraction is exact.
//
// Result layout of a 16 x 16 tile C = A B^T (A rows m, B rows n):
//   lane l holds C[4 * (l / 16) + r][l % 16] in element r (r = 0..3).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sinkattn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f4;
typedef __attribute__((ext_vector_type(4))) uint32_t u4;
typedef __attribute__((ext_vector_type(2))) uint32_t u2;

typedef uint16_t bf16_t;  // storage type of bf16 tensors

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();
// s_waitcnt immediate that waits for every vector memory operation of the
// wave (vmcnt = 0) and leaves the LDS/scalar and export counters free
// (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
constexpr int kVmcnt0 = 0x0F70;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float log2_fast(float x) { return __builtin_amdgcn_logf(x); }

// log2(x) of a positive finite fp32 x as fp64, split as x = m 2^e with m in
// [sqrt(1/2), sqrt(2)): the exponent is exact and the fp32 log is taken of
// m only, so the absolute error stays near 2^-24 instead of growing with
// |log2 x| (one fp32 ulp of a potential near -17 is 2^-19).
__device__ __forceinline__ double log2_split(float x) {
  int e;
  float m = frexpf(x, &e);  // m in [1/2, 1)
  if (m < 0.70710678f) {
    m *= 2.f;
    --e;
  }
  return (double)e + (double)__builtin_amdgcn_logf(m);
}

__device__ __forceinline__ float bits_to_float(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t float_to_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// bf16 (stored as uint16) -> fp32, exact.
__device__ __forceinline__ float bf16_to_float(bf16_t h) { return bits_to_float(((uint32_t)h) << 16); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = float_to_bits(f);
  uint32_t lsb = (u >> 16) & 1u;
  return (u + 0x7fffu + lsb) >> 16;
}

// ---------------------------------------------------------------------------
// Element-type traits: bytes per element and the score-tile MMA of one chunk.
// ---------------------------------------------------------------------------
template <typename T> struct Elt;

template <> struct Elt<float> {
  static constexpr int kBytes = 4;
  // 16 contiguous bytes = 4 consecutive k values; four K=4 MFMAs.
  static __device__ __forceinline__ f4 mma_chunk(f4 acc, u4 a, u4 b) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bits_to_float(a.x), bits_to_float(b.x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bits_to_float(a.y), bits_to_float(b.y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bits_to_float(a.z), bits_to_float(b.z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(bits_to_float(a.w), bits_to_float(b.w), acc, 0, 0, 0);
    return acc;
  }
  static __device__ __forceinline__ float load(const float* p, size_t i) { return p[i]; }
};

template <> struct Elt<bf16_t> {
  static constexpr int kBytes = 2;
  // 16 contiguous bytes = 8 consecutive k values; one K=32 MFMA.
  static __device__ __forceinline__ f4 mma_chunk(f4 acc, u4 a, u4 b) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
  }
  static __device__ __forceinline__ float load(const bf16_t* p, size_t i) { return bf16_to_float(p[i]); }
};

// ---------------------------------------------------------------------------
// Cross-lane reductions.  "row" = the 16 lanes sharing l / 16.
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return bits_to_float((uint32_t)__builtin_amdgcn_update_dpp(0, (int)float_to_bits(x), CTRL, 0xf, 0xf, false));
}

// Sum over the 16 lanes of each row; every lane receives its row's total.
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp<0x141>(x);  // row_half_mirror
  x += dpp<0x140>(x);  // row_mirror
  return x;
}

__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<0xB1>(x));
  x = fmaxf(x, dpp<0x4E>(x));
  x = fmaxf(x, dpp<0x141>(x));
  x = fmaxf(x, dpp<0x140>(x));
  return x;
}

// gfx950 row swaps (a "row" is 16 lanes): permlane32_swap(a, b) returns
// ([a0, a1, b0, b1], [a2, a3, b2, b3]) and permlane16_swap(a, b) returns
// ([a0, b0, a2, b2], [a1, b1, a3, b3]) by row.
__device__ __forceinline__ void swap32(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(float_to_bits(a), float_to_bits(b), false, false);
  a = bits_to_float(r[0]);
  b = bits_to_float(r[1]);
}
__device__ __forceinline__ void swap16(float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane16_swap(float_to_bits(a), float_to_bits(b), false, false);
  a = bits_to_float(r[0]);
  b = bits_to_float(r[1]);
}

// Sum over the four rows (lanes l, l^16, l^32, l^48); every lane gets it.
__device__ __forceinline__ float cross_row_sum(float x) {
  float y = x;
  swap32(x, y);  // x = [x0, x1, x0, x1], y = [x2, x3, x2, x3]
  x += y;
  y = x;
  swap16(x, y);  // x = [z0, z0, z2, z2], y = [z1, z1, z3, z3]
  return x + y;
}

// Four row sums at once: on return row g of the result holds the sum over
// the four rows of c[g] (c[0..3] are consumed).
__device__ __forceinline__ float cross_row_sum4(float c0, float c1, float c2, float c3) {
  swap32(c0, c2);  // c0 = [c0_0, c0_1, c2_0, c2_1], c2 = [c0_2, c0_3, c2_2, c2_3]
  c0 += c2;
  swap32(c1, c3);
  c1 += c3;
  swap16(c0, c1);  // c0 = [A0, B0, A2, B2], c1 = [A1, B1, A3, B3]
  return c0 + c1;
}

__device__ __forceinline__ float cross_row_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16, 64));
  x = fmaxf(x, __shfl_xor(x, 32, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) { return cross_row_sum(row16_sum(x)); }
__device__ __forceinline__ float wave_max(float x) { return cross_row_max(row16_max(x)); }

// ---------------------------------------------------------------------------
// Global / LDS 16-byte accesses.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u4 ld16(const void* p) { return *reinterpret_cast<const u4*>(p); }
__device__ __forceinline__ void st16(void* p, u4 v) { *reinterpret_cast<u4*>(p) = v; }

// ---------------------------------------------------------------------------
// Streamed tile pairs in LDS (bf16 rows of RB >= 128 bytes).
// A stored row swizzles its 16-byte chunks: chunk c of row r sits at chunk
// position c ^ f(r).  The two read patterns of the MFMA operands are 128-bit
// reads of one chunk in each of 16 consecutive rows and transposed 64-bit
// reads of two chunks in each of 4 consecutive rows.  Measured on gfx950 (bank
// conflict counter, every XOR-linear f of the row's low 4 bits): with 256-byte
// rows (16 chunks) f(r) = (r ^ 2r) & 15 leaves both patterns free of bank
// conflicts, while the 3-bit f = (r & 3) << 1 | (r >> 2) & 1 costs 4 conflict
// cycles per 128-bit read and 2 per transposed read.  Rows of 8 chunks keep the
// 3-bit f (their chunk index has 3 bits).
// ---------------------------------------------------------------------------
template <int CPR>
__device__ __forceinline__ int sw_chunk(int chunk, int row) {
  if constexpr (CPR >= 16) return chunk ^ ((row ^ (row << 1)) & 15);
  else return chunk ^ (((row & 3) << 1) | ((row >> 2) & 1));
}

// LDS address (byte offset in the workgroup's LDS) of a pointer into it.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
// One wave-wide LDS DMA: lane l copies 16 bytes from base + off (its own
// off) to LDS bytes [lds + 16 l, lds + 16 l + 16).  Written as inline asm so
// that the compiler does not treat the transposed LDS reads of the streamed
// sweeps as possibly aliasing a DMA in flight (it would wait for every DMA
// before them); the sweeps order their DMAs and reads with explicit waits and
// barriers.  No register is written.  `lds` and `base` are wave-uniform.
// M0 (a reserved register, so its clobber is only advisory) is overwritten:
// the kernels that use this helper have no other M0 user (the compiler sets
// M0 only for its own LDS-DMA builtins and indirect register moves, neither
// of which they contain).
__device__ __forceinline__ void lds_dma16(const char* base, uint32_t off, uint32_t lds) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2"
      :
      : "s"(lds), "v"(off), "s"(base)
      : "memory", "m0");
}

__device__ __forceinline__ u2 ld_tr16(const char* p) {
  typedef short s4v __attribute__((ext_vector_type(4)));
  const s4v v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s4v*)(p));
  u2 r;
  __builtin_memcpy(&r, &v, 8);
  return r;
}

// Two floats to packed bf16 (element 0 in the low half), rounded to nearest
// even, one v_cvt_pk_bf16_f32 per pair.
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef float f2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f2v){a, b}, bf16x2v));
}

// hi + lo bf16 operands of 8 fp32 values (4 of tile 0, then 4 of tile 1)
__device__ __forceinline__ void split_hilo(const float (&v0)[4], const float (&v1)[4], u4& hi, u4& lo) {
  const float x[8] = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
  uint32_t h[4], l[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    h[q] = pack_bf16x2(x[2 * q], x[2 * q + 1]);
    l[q] = pack_bf16x2(x[2 * q] - bits_to_float(h[q] << 16), x[2 * q + 1] - bits_to_float(h[q] & 0xffff0000u));
  }
  hi = (u4){h[0], h[1], h[2], h[3]};
  lo = (u4){l[0], l[1], l[2], l[3]};
}

// Map a linear workgroup id to a logical one so that each XCD (ids are dealt
// to the 8 XCDs round-robin) receives a contiguous range of logical ids:
// neighbouring band blocks then share that XCD's L2.  `padded` is the launch
// size (a multiple of 8); logical ids >= the real count are idle.
__device__ __forceinline__ int xcd_remap(int id, int padded) {
  const int per = padded >> 3;
  return (id & 7) * per + (id >> 3);
}

}  // namespace sinkattn
