// Shared device helpers of the attention and LoRA-gradient kernels (gfx950): buffer
// loads with range checking, v_mfma_f32_32x32x16_bf16 operands, and 64-row tiles moved
// from global memory into LDS either row-major or transposed.
//
// MFMA operand layouts (lane = 0..63, 32 x 32 x 16): A[i][k] sits in lane
// i + 32 (k / 8), element k % 8; B[k][j] in lane j + 32 (k / 8); the result C[i][j] in
// lane j + 32 ((i / 4) % 2), register (i / 8) * 4 + i % 4.  A tile computed as C leaves
// 16 of its rows in each lane; reused as an operand of a product whose contraction
// runs over those rows, it is taken in the lane's own row order (pack8), and the other
// operand is read from a transposed LDS tile in that same order (tfrag): the sum over
// the contraction does not depend on its order.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsq {
namespace tiles {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kTileRows = 64;              // rows of a streamed tile
constexpr int kTPitch = kTileRows + 4;     // pitch of a transposed tile [column][row], elements

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));   // RNE
}
// x rounded to bf16 (nearest even), as a float
__device__ __forceinline__ float bf16_value(float x) { return __builtin_bit_cast(float, pack2(0.f, x) & 0xFFFF0000u); }
__device__ __forceinline__ float bf_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}
// 16 bytes at a range-checked per-lane offset (past the end: zeros)
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ bf16x8_t as_bf8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }
__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
// eight consecutive accumulator values (one k16 step of a reused C tile) as bf16
__device__ __forceinline__ bf16x8_t pack8(const f32x16_t& x, int base) {
  return as_bf8(make_uint4(pack2(x[base], x[base + 1]), pack2(x[base + 2], x[base + 3]),
                           pack2(x[base + 4], x[base + 5]), pack2(x[base + 6], x[base + 7])));
}
// Operand fragment from a transposed LDS tile t[col][row]: lane (i + 32 hh) takes rows
// r0 + 4 hh + {0..3} and r0 + 8 + 4 hh + {0..3} of line col, the row order pack8
// gives registers 8 s .. 8 s + 7 of a C tile (r0 = 16 s within a 32-row block).
__device__ __forceinline__ bf16x8_t tfrag(const uint16_t* t, int col, int r0, int hh) {
  const uint16_t* src = t + col * kTPitch + r0 + 4 * hh;
  const uint2 lo = *reinterpret_cast<const uint2*>(src);
  const uint2 hi = *reinterpret_cast<const uint2*>(src + 8);
  return as_bf8(make_uint4(lo.x, lo.y, hi.x, hi.y));
}

// One 64-row tile (rows row0.., W columns) of a row-major bf16 matrix moved global ->
// registers -> LDS, row-major (pitch W + 8) and/or transposed ([col][row], pitch
// kTPitch).  Unit u covers rows 2p, 2p+1 and 8 columns 8c with c = (u / 4) % (W / 8),
// p = u % 4 + 4 ((u / 4) / (W / 8)): a wave's load reads whole W-column row segments,
// and the transposed stores of 4 neighbouring lanes fill neighbouring LDS words.
// NT threads.  Rows past the buffer's range read as zero.
template <int W, int NT>
struct TileMover {
  static constexpr int CW = W / 8;                  // 16-byte chunks per row
  static constexpr int NU = 32 * CW / NT;           // units per thread
  static_assert(NU >= 1 && 32 * CW % NT == 0, "tile width and thread count");
  uint4 v[NU][2];
  __device__ __forceinline__ static int unit_p(int u) { return (u & 3) + 4 * ((u >> 2) / CW); }
  __device__ __forceinline__ static int unit_c(int u) { return (u >> 2) % CW; }
  __device__ __forceinline__ void load(rsrc_t res, int ld, int row0) {
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = threadIdx.x + NT * i, p = unit_p(u), c = unit_c(u);
#pragma unroll
      for (int r = 0; r < 2; ++r)
        v[i][r] = bload16(res, ((uint32_t)(row0 + 2 * p + r) * (uint32_t)ld + 8u * c) * 2u);
    }
  }
  __device__ __forceinline__ void store_rows(uint16_t* s) const {
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = threadIdx.x + NT * i, p = unit_p(u), c = unit_c(u);
#pragma unroll
      for (int r = 0; r < 2; ++r) *reinterpret_cast<uint4*>(s + (2 * p + r) * (W + 8) + 8 * c) = v[i][r];
    }
  }
  __device__ __forceinline__ void store_t(uint16_t* t) const {
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = threadIdx.x + NT * i, p = unit_p(u), c = unit_c(u);
      const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&v[i][0]);
      const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&v[i][1]);
#pragma unroll
      for (int j = 0; j < 4; ++j) {   // dword j = columns 8c + 2j, 8c + 2j + 1
        *reinterpret_cast<uint32_t*>(t + (8 * c + 2 * j) * kTPitch + 2 * p) = __builtin_amdgcn_perm(r1[j], r0[j], 0x05040100u);
        *reinterpret_cast<uint32_t*>(t + (8 * c + 2 * j + 1) * kTPitch + 2 * p) = __builtin_amdgcn_perm(r1[j], r0[j], 0x07060302u);
      }
    }
  }
};

// Row fragments kept in registers as the B operand of a product over W columns:
// step s holds columns 16 s + 8 hh .. + 7 of row `row` (zeros past the end).
template <int W>
__device__ __forceinline__ void row_frags(bf16x8_t (&f)[W / 16], rsrc_t res, int ld, int row, int hh) {
#pragma unroll
  for (int s = 0; s < W / 16; ++s) f[s] = as_bf8(bload16(res, ((uint32_t)row * (uint32_t)ld + 16u * s + 8u * hh) * 2u));
}

}  // namespace tiles
}  // namespace lsq
