// Fused dequant GEMMs of the frozen base, gfx950 (CDNA4), 64-wide waves.
//
// Every projection of the method computes Y = X W^T + s (X A^T) B^T forward and
// dX = dY W + s (dY B) A backward ("Fine-Tuning an 8B Parameter Model on a 4 GB
// Laptop GPU", section "LoRA and QLoRA: Train a Fraction of the Parameters"), with W
// stored as 4-bit NormalFloat codes and one absmax per 64 weights (section
// "Quantization: Shrink the Weights" of the same page) or as bf16.  Here the base
// term and the low-rank term are one MFMA contraction: the 4-bit codes are expanded
// to bf16 in registers, staged in LDS and fed to v_mfma_f32_32x32x16_bf16; the
// low-rank term is a K-extension (s*H or s*G as extra A columns against B or A^T as
// extra B columns) run after the main loop in the same accumulators.
//
// Dequantised weight = bf16_rne(fp32(level[code] * absmax)), absmax either stored
// as float32 or decoded from the 8-bit second level as
// fp32(fp32(fp32(c/127) * scale2) + mean) with no fused multiply-add.
//
// A launch whose tiles leave the last (or only) round of compute units part full cuts
// each tile of that round along K into pieces that fill it; the piece that finishes
// last adds the pieces' float32 sums (piece_of, combine_pieces).
//
// Tile: 256 x 256 outputs per 256-thread workgroup, 2 x 2 waves of 128 x 128
// (4 x 4 MFMA blocks of 32 x 32, 256 float accumulators per lane), K step 64,
// two LDS stages (row pitch 72 bf16 = 144 B keeps ds_read_b128 conflict-free).
// W orientation (forward): both operands are K-contiguous rows.  W^T orientation
// (backward): the contraction runs down W's rows, so each thread dequantises two
// adjacent rows and writes (w[n][j], w[n+1][j]) pairs, i.e. the transpose, into LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "lsq_internal.hpp"

namespace lsq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int PITCH = BK + 8;                    // bf16 elements per LDS row
constexpr int TILE_ELEMS = BM * PITCH;           // per operand per stage
constexpr int NTHREADS = 256;

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));   // RNE
}
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __builtin_bit_cast(float, u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __builtin_bit_cast(float, u & 0xFFFF0000u); }

// absmax of NF4 block b: stored float32, or decoded from the 8-bit second level.
template <int FMT>
__device__ __forceinline__ float block_absmax(const WeightRef& w, uint64_t b) {
  if constexpr (FMT == WF_NF4_DQ) {
#pragma clang fp contract(off)
    const float frac = (float)(int8_t)w.qabs[b] / 127.0f;   // IEEE division
    const float prod = frac * w.scale2[b / kDQGroup];
    return prod + *w.mean;
  } else {
    return w.absmax[b];
  }
}

// The 256-entry pair table at LDS offset 0: entry b = (level[b >> 4], level[b & 15]),
// the two levels of one packed code byte (element 2k in the high nibble).  One 8-byte
// LDS read per byte; the address is the byte value times 8.
__device__ __forceinline__ uint32_t deq_byte(const float2* lut2, uint32_t byte, float am) {
  const float2 l = lut2[byte];
  return pack_bf16x2(l.x * am, l.y * am);      // fp32 multiply, RNE to bf16
}

// 8 codes (one dword, byte k = code[2k] << 4 | code[2k+1]) -> 4 dwords of bf16 pairs
__device__ __forceinline__ void dequant8(uint32_t codes, float am, const float2* lut2, uint32_t out[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) out[k] = deq_byte(lut2, (codes >> (8 * k)) & 0xFFu, am);
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0xFFFFFFF0u;   // offset past every buffer: the load returns 0
// s_waitcnt operand: vector-memory count 0, the export and LDS/scalar counts unconstrained
constexpr int kWaitVm0 = 0x0F70;

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
}
// Same, for a buffer the caller knows to be the same across the wave: the fields are
// moved to scalar registers so the loads need no per-lane descriptor loop.
__device__ __forceinline__ rsrc_t make_rsrc_wave(const void* p, uint64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)bytes);
  void* q = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(q, (short)0, (int)n, 0x00020000);
}
__device__ __forceinline__ uint4 bload16(rsrc_t r, uint32_t off) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint2 bload8(rsrc_t r, uint32_t off) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint32_t bload4(rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

struct Smem {
  float2 lut2[256];                  // must stay first: LDS offset 0
  union {
    struct {
      uint16_t a[2][TILE_ELEMS];
      uint16_t w[2][TILE_ELEMS];
    } k;
    float out[128 * (BN + 4)];       // epilogue staging, one half tile (128 rows) at a time
  } u;
  uint32_t sk_flag;                  // a split tile's arrival count, read back by every thread
};

__device__ __forceinline__ void fill_lut2(Smem& sm, const float* levels) {
  const int b = threadIdx.x;          // the first 256 threads, one entry each
  if (b < 256) sm.lut2[b] = levels ? make_float2(levels[b >> 4], levels[b & 15]) : make_float2(0.f, 0.f);
}

// NF4 weight buffers as resources
struct WRes {
  rsrc_t codes, absmax, qabs, scale2;
  float mean;
};
template <int FMT>
__device__ __forceinline__ WRes make_wres(const WeightRef& w) {
  WRes r;
  const uint64_t numel = (uint64_t)w.n_out * (uint64_t)w.n_in;
  const uint64_t nblocks = (numel + kNF4Block - 1) / kNF4Block;
  if constexpr (FMT == WF_BF16) {
    r.codes = make_rsrc(w.w, numel * 2);
  } else {
    r.codes = make_rsrc(w.w, (numel + 1) / 2);
  }
  if constexpr (FMT == WF_NF4) r.absmax = make_rsrc(w.absmax, nblocks * 4);
  if constexpr (FMT == WF_NF4_DQ) {
    r.qabs = make_rsrc(w.qabs, nblocks);
    r.scale2 = make_rsrc(w.scale2, (nblocks + kDQGroup - 1) / kDQGroup * 4);
    r.mean = *w.mean;
  }
  return r;
}

// absmax of NF4 block b (b < nblocks): float32, or decoded from the 8-bit second level
// as fp32(fp32(fp32(c/127) * scale2) + mean) with the two roundings kept separate.
template <int FMT>
__device__ __forceinline__ float block_absmax_r(const WRes& r, uint32_t b) {
  if constexpr (FMT == WF_NF4_DQ) {
#pragma clang fp contract(off)
    const uint32_t word = bload4(r.qabs, b & ~3u);
    const int8_t c = (int8_t)((word >> (8 * (b & 3u))) & 0xFFu);
    const float frac = (float)c / 127.0f;
    const float s2 = __builtin_bit_cast(float, bload4(r.scale2, (b / kDQGroup) * 4));
    const float prod = frac * s2;
    return prod + r.mean;
  } else {
    return __builtin_bit_cast(float, bload4(r.absmax, b * 4));
  }
}

// ---- A operand (activations, K-contiguous rows): 256 rows x 64 k, 8 x 16 B per thread
struct ALoad { uint4 v[8]; };

// base: bf16 matrix with row stride ld; rows [0, rows_left) valid, columns [0, klim) valid
__device__ __forceinline__ void load_a(ALoad& r, rsrc_t res, uint32_t base_off, int ld, int rows_left, int k0, int klim) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = t + NTHREADS * i;
    const int row = c >> 3, kc = (c & 7) * 8;
    const bool ok = row < rows_left && k0 + kc < klim;
    const uint32_t off = base_off + ((uint32_t)row * (uint32_t)ld + (uint32_t)(k0 + kc)) * 2u;
    r.v[i] = bload16(res, ok ? off : kOOB);
  }
}
__device__ __forceinline__ void load_a_part(ALoad& r, rsrc_t res, uint32_t base_off, int ld, int rows_left, int k0,
                                            int klim, int q) {   // chunks 2q, 2q+1
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 2 * q; i < 2 * q + 2; ++i) {
    const int c = t + NTHREADS * i;
    const int row = c >> 3, kc = (c & 7) * 8;
    const bool ok = row < rows_left && k0 + kc < klim;
    const uint32_t off = base_off + ((uint32_t)row * (uint32_t)ld + (uint32_t)(k0 + kc)) * 2u;
    r.v[i] = bload16(res, ok ? off : kOOB);
  }
}
__device__ __forceinline__ void store_a_part(const ALoad& r, uint16_t* s, int q) {   // chunks 2q, 2q+1
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 2 * q; i < 2 * q + 2; ++i) {
    const int c = t + NTHREADS * i;
    const int row = c >> 3, kc = (c & 7) * 8;
    *reinterpret_cast<uint4*>(s + row * PITCH + kc) = r.v[i];
  }
}
__device__ __forceinline__ void store_a(const ALoad& r, uint16_t* s) {
#pragma unroll
  for (int q = 0; q < 4; ++q) store_a_part(r, s, q);
}

// ---- W operand, forward orientation: thread t owns row n0+t, k in [k0, k0+64)
template <int FMT, bool ALIGNED>
struct WFwd {
  uint4 raw[FMT == WF_BF16 ? 8 : 2];
  float am[4];
  __device__ __forceinline__ void load(const WRes& R, int n_out, int K, int n0, int k0) {
    const int n = n0 + threadIdx.x;
    const bool row_ok = n < n_out;
    if constexpr (FMT == WF_BF16) {
      const uint32_t base = ((uint32_t)n * (uint32_t)K + (uint32_t)k0) * 2u;
#pragma unroll
      for (int i = 0; i < 8; ++i) raw[i] = bload16(R.codes, (row_ok && k0 + 8 * i < K) ? base + 16u * i : kOOB);
    } else if constexpr (ALIGNED) {
      // K % 64 == 0: the 64 codes are one NF4 block, 32 bytes, 32-byte aligned
      const uint32_t f = (uint32_t)n * (uint32_t)K + (uint32_t)k0;
      const bool ok = row_ok && k0 < K;
      raw[0] = bload16(R.codes, ok ? f / 2 : kOOB);
      raw[1] = bload16(R.codes, ok ? f / 2 + 16u : kOOB);
      am[0] = ok ? block_absmax_r<FMT>(R, f / kNF4Block) : 0.f;
    } else {
      // K % 16 == 0: four chunks of 16 codes (8 bytes), each inside one block
      const uint32_t f0 = (uint32_t)n * (uint32_t)K + (uint32_t)k0;
      uint32_t* r32 = reinterpret_cast<uint32_t*>(raw);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool ok = row_ok && k0 + 16 * c < K;
        const uint32_t f = f0 + 16u * c;
        const uint2 v = bload8(R.codes, ok ? f / 2 : kOOB);
        r32[2 * c] = ok ? v.x : 0x77777777u;
        r32[2 * c + 1] = ok ? v.y : 0x77777777u;
        am[c] = ok ? block_absmax_r<FMT>(R, f / kNF4Block) : 0.f;
      }
    }
  }
  // quarter q of the store: 16 of the thread's 64 elements
  __device__ __forceinline__ void store_part(uint16_t* s, const float2* lut2, int q) const {
    uint16_t* row = s + threadIdx.x * PITCH;
    if constexpr (FMT == WF_BF16) {
#pragma unroll
      for (int i = 2 * q; i < 2 * q + 2; ++i) *reinterpret_cast<uint4*>(row + 8 * i) = raw[i];
    } else {
      const uint32_t* r32 = reinterpret_cast<const uint32_t*>(raw);
#pragma unroll
      for (int d = 2 * q; d < 2 * q + 2; ++d) {      // 2 dwords of codes = 16 elements
        uint32_t o[4];
        dequant8(r32[d], ALIGNED ? am[0] : am[q], lut2, o);
        *reinterpret_cast<uint4*>(row + 8 * d) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* s, const float2* lut2) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) store_part(s, lut2, q);
  }
};

// ---- W operand, backward orientation: thread t owns rows k0+2p, k0+2p+1 (p = t%32)
// and output columns j0 + 32c .. +32 (c = t/32); writes LDS[j][k] pairs.
template <int FMT, bool ALIGNED>
struct WBwd {
  uint4 raw[FMT == WF_BF16 ? 8 : 2];   // bf16: row0 64 B, row1 64 B; nf4: row0 16 B, row1 16 B
  float am[2][2];
  __device__ __forceinline__ void load(const WRes& R, int J, int k0, int krows, int j0) {
    const int p = threadIdx.x & 31, c = threadIdx.x >> 5;
    const int jc = j0 + 32 * c;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int kr = k0 + 2 * p + r;                 // row of W (contraction index)
      const bool ok = kr < krows;
      if constexpr (FMT == WF_BF16) {
        const uint32_t base = ((uint32_t)kr * (uint32_t)J + (uint32_t)jc) * 2u;
#pragma unroll
        for (int i = 0; i < 4; ++i) raw[4 * r + i] = bload16(R.codes, (ok && jc + 8 * i < J) ? base + 16u * i : kOOB);
      } else if constexpr (ALIGNED) {
        // J % 64 == 0: 32 codes = 16 bytes, half of one block
        const uint32_t f = (uint32_t)kr * (uint32_t)J + (uint32_t)jc;
        const bool ok2 = ok && jc < J;
        raw[r] = bload16(R.codes, ok2 ? f / 2 : kOOB);
        am[r][0] = ok2 ? block_absmax_r<FMT>(R, f / kNF4Block) : 0.f;
      } else {
        const uint32_t f0 = (uint32_t)kr * (uint32_t)J + (uint32_t)jc;
        uint32_t* r32 = reinterpret_cast<uint32_t*>(&raw[r]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const bool ok2 = ok && jc + 16 * h < J;
          const uint32_t f = f0 + 16u * h;
          const uint2 v = bload8(R.codes, ok2 ? f / 2 : kOOB);
          r32[2 * h] = ok2 ? v.x : 0x77777777u;
          r32[2 * h + 1] = ok2 ? v.y : 0x77777777u;
          am[r][h] = ok2 ? block_absmax_r<FMT>(R, f / kNF4Block) : 0.f;
        }
      }
    }
  }
  // quarter q of the store: codes dword q of both rows (8 columns)
  __device__ __forceinline__ void store_part(uint16_t* s, const float2* lut2, int q) const {
    const int p = threadIdx.x & 31, c = threadIdx.x >> 5;
    uint32_t* dst = reinterpret_cast<uint32_t*>(s + (32 * c) * PITCH + 2 * p);
    const int pitch32 = PITCH / 2;
    if constexpr (FMT == WF_BF16) {
      const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&raw[0]);
      const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&raw[4]);
#pragma unroll
      for (int w = 4 * q; w < 4 * q + 4; ++w) {
        dst[(2 * w) * pitch32] = __builtin_amdgcn_perm(r1[w], r0[w], 0x05040100u);
        dst[(2 * w + 1) * pitch32] = __builtin_amdgcn_perm(r1[w], r0[w], 0x07060302u);
      }
    } else {
      const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&raw[0]);
      const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&raw[1]);
      const float a0 = ALIGNED ? am[0][0] : am[0][q / 2];
      const float a1 = ALIGNED ? am[1][0] : am[1][q / 2];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float2 l0 = lut2[(r0[q] >> (8 * k)) & 0xFFu], l1 = lut2[(r1[q] >> (8 * k)) & 0xFFu];
        const int j = 8 * q + 2 * k;
        dst[j * pitch32] = pack_bf16x2(l0.x * a0, l1.x * a1);
        dst[(j + 1) * pitch32] = pack_bf16x2(l0.y * a0, l1.y * a1);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* s, const float2* lut2) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) store_part(s, lut2, q);
  }
};

// ---------------------------------------------------------------- fast path
// Used when every tile lies inside its matrices (K % 64 == 0, and in the W^T
// orientation every stacked segment's rows % 64 == 0).  Per-lane offsets are loop
// invariant; the K position moves in the scalar offset, so the loads cost no VALU.
// Rows past the end of a buffer read as zero through the buffer range check.

__device__ __forceinline__ uint4 bload16s(rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint32_t bload4s(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}
__device__ __forceinline__ uint32_t bload1s(rsrc_t r, uint32_t voff, uint32_t soff) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b8(r, voff, soff, 0);
}

// fp32(fp32(fp32(c/127) * scale2) + mean), the two roundings kept apart
__device__ __forceinline__ float dq_absmax(uint32_t code_byte, float scale2, float mean) {
#pragma clang fp contract(off)
  const float frac = (float)(int8_t)(uint8_t)code_byte / 127.0f;
  const float prod = frac * scale2;
  return prod + mean;
}

constexpr int NT_FAST = 512;    // fast path: 8 waves, two per SIMD

// A operand: 256 rows x 64 columns of a K-contiguous bf16 matrix (row stride ld);
// thread t moves 4 chunks of 16 B: rows (t >> 3) + 64 q, columns (t & 7) * 8.  The
// row sits in the per-lane offset, which the buffer range check covers (rows past
// the end read as zero); the column position is the scalar offset and stays inside
// the row as long as the caller only asks for tiles below the row length.
struct AFast {
  uint4 v[4];
  rsrc_t res;
  uint32_t voff[4];
  __device__ __forceinline__ void init(rsrc_t r, int ld) {
    res = r;
#pragma unroll
    for (int q = 0; q < 4; ++q)
      voff[q] = ((uint32_t)((threadIdx.x >> 3) + 64 * q) * (uint32_t)ld + (uint32_t)(threadIdx.x & 7) * 8u) * 2u;
  }
  __device__ __forceinline__ void load_q(uint32_t col0, int q) {   // col0 in elements
    v[q] = bload16s(res, voff[q], col0 * 2u);
  }
  // as load_q, or zeros (an out-of-range offset) when `zero` (wave-uniform)
  __device__ __forceinline__ void load_q_or_zero(uint32_t col0, int q, bool zero) {
    v[q] = bload16s(res, zero ? kOOB : voff[q], zero ? 0u : col0 * 2u);
  }
  __device__ __forceinline__ void store_q(uint16_t* s, int q) const {
    const int c = threadIdx.x + NT_FAST * q;
    *reinterpret_cast<uint4*>(s + (c >> 3) * PITCH + (c & 7) * 8) = v[q];
  }
};

// extension tile with 512 threads: NQ * 64 rows; LDS columns [c_lo, c_lo + kx) take
// source columns [0, kx) (kx <= 64), every other column of the 64 is zero
template <int NQ = 4>
__device__ __forceinline__ void ext_tile(uint16_t* s, rsrc_t res, uint32_t col_off_bytes, int ld, int rows, int kx,
                                         int c_lo = 0) {
#pragma unroll
  for (int q = 0; q < NQ; ++q) {
    const int c = threadIdx.x + NT_FAST * q;
    const int row = c >> 3, kc = (c & 7) * 8;
    const int src = kc - c_lo;
    const bool ok = row < rows && src >= 0 && src < kx;
    const uint4 v = bload16(res, ok ? col_off_bytes + ((uint32_t)row * (uint32_t)ld + (uint32_t)src) * 2u : kOOB);
    *reinterpret_cast<uint4*>(s + row * PITCH + kc) = v;
  }
}

// W operand, forward orientation: thread t owns row n0 + (t >> 1), k half 32 (t & 1)
// of one NF4 block (both halves share the block's absmax).  Rows are in the checked
// per-lane offset; load(k0) must only be called with k0 < K.
template <int FMT>
struct WFwdFast {
  // per-tile registers, carried from one K step to the next
  struct Regs {
    uint4 raw[FMT == WF_BF16 ? 4 : 1];
    uint32_t blk;      // absmax word (NF4) or 8-bit code (DQ)
    float s2;          // DQ second-level scale
  };
  // loop-invariant buffers and offsets
  rsrc_t codes, absq, sc2;
  float mean;
  uint32_t voff_w, voff_b, blk0;
  __device__ __forceinline__ static void clear(Regs& R) {
#pragma unroll
    for (int i = 0; i < (FMT == WF_BF16 ? 4 : 1); ++i) R.raw[i] = make_uint4(0, 0, 0, 0);
    R.blk = 0; R.s2 = 0.f;
  }
  // r: this thread's row within the tile of weight w starting at row n0; cap: tile rows
  __device__ __forceinline__ void init(const WeightRef& w, int n0, uint32_t r, int cap) {
    const int K = w.n_in;
    const int rows = w.n_out - n0 < cap ? w.n_out - n0 : cap;
    const uint32_t h = threadIdx.x & 1;
    const uint32_t kblk = (uint32_t)K / kNF4Block;
    mean = 0.f; voff_b = 0; blk0 = 0;
    if constexpr (FMT == WF_BF16) {
      codes = make_rsrc_wave(w.w + (uint64_t)n0 * K * 2, (uint64_t)(rows > 0 ? rows : 0) * K * 2);
      voff_w = (r * (uint32_t)K + 32u * h) * 2u;
    } else {
      codes = make_rsrc_wave(w.w + (uint64_t)n0 * K / 2, (uint64_t)(rows > 0 ? rows : 0) * K / 2);
      voff_w = r * (uint32_t)K / 2u + 16u * h;
      const uint64_t b0 = (uint64_t)n0 * kblk;
      const uint64_t nb = (uint64_t)(rows > 0 ? rows : 0) * kblk;
      voff_b = r * kblk;
      blk0 = (uint32_t)(b0 + voff_b);
      if constexpr (FMT == WF_NF4) {
        absq = make_rsrc_wave(w.absmax + b0, nb * 4);
      } else {
        absq = make_rsrc_wave(w.qabs + b0, nb);
        const uint64_t all = (uint64_t)w.n_out * kblk;
        sc2 = make_rsrc_wave(w.scale2, (all + kDQGroup - 1) / kDQGroup * 4);
        mean = *w.mean;
      }
    }
  }
  __device__ __forceinline__ void load(Regs& R, int k0) const {
    if constexpr (FMT == WF_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) R.raw[i] = bload16s(codes, voff_w + 16u * i, (uint32_t)k0 * 2u);
    } else {
      R.raw[0] = bload16s(codes, voff_w, (uint32_t)k0 / 2u);
      const uint32_t kb = (uint32_t)k0 / kNF4Block;
      if constexpr (FMT == WF_NF4) {
        R.blk = bload4s(absq, voff_b * 4u, kb * 4u);
      } else {
        R.blk = bload1s(absq, voff_b, kb);
        R.s2 = __builtin_bit_cast(float, bload4s(sc2, ((blk0 + kb) / kDQGroup) * 4u, 0));
      }
    }
  }
  __device__ __forceinline__ float absmax(const Regs& R) const {
    if constexpr (FMT == WF_NF4) return __builtin_bit_cast(float, R.blk);
    else return dq_absmax(R.blk, R.s2, mean);
  }
  // quarter q: 8 of the thread's 32 elements, one 16-byte LDS store
  __device__ __forceinline__ void store_part(const Regs& R, uint16_t* s, const float2* lut2, int q, float am) const {
    uint16_t* dst = s + (threadIdx.x >> 1) * PITCH + 32 * (threadIdx.x & 1) + 8 * q;
    if constexpr (FMT == WF_BF16) {
      *reinterpret_cast<uint4*>(dst) = R.raw[q];
    } else {
      uint32_t o[4];
      dequant8(reinterpret_cast<const uint32_t*>(&R.raw[0])[q], am, lut2, o);
      *reinterpret_cast<uint4*>(dst) = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
};

// W operand, backward orientation: thread t owns rows k0 + 2p, k0 + 2p + 1 (p = t & 31)
// and 16 output columns j0 + 16c (c = t >> 5), inside one NF4 block per row.
template <int FMT>
struct WBwdFast {
  struct Regs {
    uint4 raw[FMT == WF_BF16 ? 4 : 1];   // nf4: .x .y = row 0 codes, .z .w = row 1 codes
    uint32_t blk[2];
    float s2[2];
    float mean;
  };
  uint32_t voff_w[2], voff_b[2];
  uint32_t jblk;     // J / 64
  __device__ __forceinline__ static void clear(Regs& R) {
#pragma unroll
    for (int i = 0; i < (FMT == WF_BF16 ? 4 : 1); ++i) R.raw[i] = make_uint4(0, 0, 0, 0);
    R.blk[0] = R.blk[1] = 0; R.s2[0] = R.s2[1] = 0.f; R.mean = 0.f;
  }
  __device__ __forceinline__ void init_lane(int J) {
    const uint32_t p = threadIdx.x & 31, c = threadIdx.x >> 5;
    jblk = (uint32_t)J / kNF4Block;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const uint32_t row = 2 * p + r;
      if constexpr (FMT == WF_BF16) voff_w[r] = (row * (uint32_t)J + 16u * c) * 2u;
      else voff_w[r] = (row * (uint32_t)J + 16u * c) / 2u;
      voff_b[r] = row * jblk + (c >> 2);
    }
  }
  // tile (rows k0.., columns j0..) with k0 < n_out: every buffer is based at the
  // tile's first element, so the range check (per-lane offset only) ends at the matrix
  __device__ __forceinline__ void load(Regs& R, const WeightRef& w, int j0, int k0) const {
    const uint64_t J = (uint64_t)w.n_in;
    const uint64_t numel = (uint64_t)w.n_out * J;
    const uint64_t e0 = (uint64_t)k0 * J + (uint64_t)j0;
    const uint64_t nb = numel / kNF4Block, b0 = e0 / kNF4Block;
    if constexpr (FMT == WF_BF16) {
      const rsrc_t codes = make_rsrc(w.w + e0 * 2, (numel - e0) * 2);
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        R.raw[2 * r] = bload16s(codes, voff_w[r], 0);
        R.raw[2 * r + 1] = bload16s(codes, voff_w[r] + 16u, 0);
      }
    } else {
      const rsrc_t codes = make_rsrc(w.w + e0 / 2, (numel - e0) / 2);
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      const u32x2 c0 = __builtin_amdgcn_raw_buffer_load_b64(codes, voff_w[0], 0, 0);
      const u32x2 c1 = __builtin_amdgcn_raw_buffer_load_b64(codes, voff_w[1], 0, 0);
      R.raw[0] = make_uint4(c0.x, c0.y, c1.x, c1.y);
      if constexpr (FMT == WF_NF4) {
        const rsrc_t absq = make_rsrc(w.absmax + b0, (nb - b0) * 4);
        R.blk[0] = bload4s(absq, voff_b[0] * 4u, 0);
        R.blk[1] = bload4s(absq, voff_b[1] * 4u, 0);
      } else {
        const rsrc_t absq = make_rsrc(w.qabs + b0, nb - b0);
        const rsrc_t sc2 = make_rsrc(w.scale2, (nb + kDQGroup - 1) / kDQGroup * 4);
        R.mean = *w.mean;
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          R.blk[r] = bload1s(absq, voff_b[r], 0);
          R.s2[r] = __builtin_bit_cast(float, bload4s(sc2, (((uint32_t)b0 + voff_b[r]) / kDQGroup) * 4u, 0));
        }
      }
    }
  }
  __device__ __forceinline__ float absmax(const Regs& R, int r) const {
    if constexpr (FMT == WF_NF4) return __builtin_bit_cast(float, R.blk[r]);
    else return dq_absmax(R.blk[r], R.s2[r], R.mean);
  }
  // quarter q: columns 4q .. 4q+3 of the thread's 16, both rows -> 4 dword stores
  __device__ __forceinline__ void store_part(const Regs& R, uint16_t* s, const float2* lut2, int q, float a0,
                                             float a1) const {
    const int p = threadIdx.x & 31, c = threadIdx.x >> 5;
    uint32_t* dst = reinterpret_cast<uint32_t*>(s + (16 * c + 4 * q) * PITCH + 2 * p);
    constexpr int pitch32 = PITCH / 2;
    if constexpr (FMT == WF_BF16) {
      // row r dword w (columns 2w, 2w+1), w = 2q, 2q+1
      const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&R.raw[0]);
      const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&R.raw[2]);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int w = 2 * q + u;
        dst[(2 * u) * pitch32] = __builtin_amdgcn_perm(r1[w], r0[w], 0x05040100u);
        dst[(2 * u + 1) * pitch32] = __builtin_amdgcn_perm(r1[w], r0[w], 0x07060302u);
      }
    } else {
      const uint32_t* rr = reinterpret_cast<const uint32_t*>(&R.raw[0]);
      const uint32_t sh = (q & 1) * 16;
      const uint32_t w0 = rr[q >> 1] >> sh, w1 = rr[2 + (q >> 1)] >> sh;
#pragma unroll
      for (int k = 0; k < 2; ++k) {   // code bytes 2q + k -> columns 4q + 2k, 4q + 2k + 1
        const float2 l0 = lut2[(w0 >> (8 * k)) & 0xFFu], l1 = lut2[(w1 >> (8 * k)) & 0xFFu];
        dst[(2 * k) * pitch32] = pack_bf16x2(l0.x * a0, l1.x * a1);
        dst[(2 * k + 1) * pitch32] = pack_bf16x2(l0.y * a0, l1.y * a1);
      }
    }
  }
};

// ---- MFMA over one LDS stage (4 k16 steps), with fragments of step kk+1 read
// while step kk's 16 MFMAs run, and a quarter of the next stage's stores (the
// functor `work`) placed after each step's MFMAs so they execute in their shadow.
// Wave layout of a 256 x 256 tile: NT / 64 waves, 2 along m (128 rows each) and
// WNW = NT / 128 along n (256 / WNW columns each, JB = 8 / WNW blocks of 32).
template <int NT> struct Layout {
  static constexpr int WNW = NT / 128;
  static constexpr int JB = 8 / WNW;
};

template <int NT, class Work>
__device__ __forceinline__ void mma_stage(const uint16_t* sa, const uint16_t* sw, f32x16_t (&acc)[4][Layout<NT>::JB],
                                          Work&& work) {
  constexpr int WNW = Layout<NT>::WNW, JB = Layout<NT>::JB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WNW, wn = wave % WNW;
  const uint16_t* pa = sa + (wm * 128 + (lane & 31)) * PITCH + (lane >> 5) * 8;
  const uint16_t* pw = sw + (wn * (32 * JB) + (lane & 31)) * PITCH + (lane >> 5) * 8;
  bf16x8_t fa[2][4], fb[2][JB];
#pragma unroll
  for (int i = 0; i < 4; ++i) fa[0][i] = *reinterpret_cast<const bf16x8_t*>(pa + i * 32 * PITCH);
#pragma unroll
  for (int j = 0; j < JB; ++j) fb[0][j] = *reinterpret_cast<const bf16x8_t*>(pw + j * 32 * PITCH);
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    const int c = kk & 1, n = c ^ 1;
    if (kk + 1 < BK / 16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[n][i] = *reinterpret_cast<const bf16x8_t*>(pa + i * 32 * PITCH + (kk + 1) * 16);
#pragma unroll
      for (int j = 0; j < JB; ++j) fb[n][j] = *reinterpret_cast<const bf16x8_t*>(pw + j * 32 * PITCH + (kk + 1) * 16);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < JB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[c][i], fb[c][j], acc[i][j], 0, 0, 0);
    work(kk);
  }
}

// The low-rank stage: only its first ks_n k16 steps hold non-zero columns (the rank
// padded to 16, or 0 without adapters), so only those are multiplied; the work of all
// four steps still runs (it fills the next stage).  ks_n is wave-uniform.
template <int NT, class Work>
__device__ __forceinline__ void mma_stage_n(const uint16_t* sa, const uint16_t* sw, f32x16_t (&acc)[4][Layout<NT>::JB],
                                            int ks_n, Work&& work) {
  constexpr int WNW = Layout<NT>::WNW, JB = Layout<NT>::JB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WNW, wn = wave % WNW;
  const uint16_t* pa = sa + (wm * 128 + (lane & 31)) * PITCH + (lane >> 5) * 8;
  const uint16_t* pw = sw + (wn * (32 * JB) + (lane & 31)) * PITCH + (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    if (kk < ks_n) {
      bf16x8_t fa[4], fb[JB];
#pragma unroll
      for (int i = 0; i < 4; ++i) fa[i] = *reinterpret_cast<const bf16x8_t*>(pa + i * 32 * PITCH + kk * 16);
#pragma unroll
      for (int j = 0; j < JB; ++j) fb[j] = *reinterpret_cast<const bf16x8_t*>(pw + j * 32 * PITCH + kk * 16);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    work(kk);
  }
}

// Fragments of one k16 step: the wave's 4 row blocks of the activation tile and its JB
// column blocks of the weight tile.
template <int NT> struct Frag {
  bf16x8_t a[4], b[Layout<NT>::JB];
};

template <int NT>
__device__ __forceinline__ void read_frag(Frag<NT>& f, const uint16_t* sa, const uint16_t* sw, int kk) {
  constexpr int WNW = Layout<NT>::WNW, JB = Layout<NT>::JB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WNW, wn = wave % WNW;
  const uint16_t* pa = sa + (wm * 128 + (lane & 31)) * PITCH + (lane >> 5) * 8 + kk * 16;
  const uint16_t* pw = sw + (wn * (32 * JB) + (lane & 31)) * PITCH + (lane >> 5) * 8 + kk * 16;
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = *reinterpret_cast<const bf16x8_t*>(pa + i * 32 * PITCH);
#pragma unroll
  for (int j = 0; j < JB; ++j) f.b[j] = *reinterpret_cast<const bf16x8_t*>(pw + j * 32 * PITCH);
}

// One LDS stage whose workgroup barrier comes before its last k16 step, so that no wave
// starts a stage waiting on LDS.  The fragments of step kk + 1 are read while step kk
// multiplies.  The next stage's stores (work(q), q = 0..3) go after steps 0, 1, 2 and 2;
// `sync` (the barrier, and whatever must precede it) follows them, and step 3 then
// reads the next stage's first fragments from the other buffer (nsa, nsw) while it
// multiplies.  f[0] holds this stage's step-0 fragments on entry and the next stage's
// on exit.  Only steps below n_mul multiply (4; the low-rank stage: its non-zero k
// steps); n_mul is wave-uniform.  The products and their order per accumulator are
// those of one k16 step after another, as in mma_stage.
template <int NT, class Work, class Sync>
__device__ __forceinline__ void mma_stage_early(const uint16_t* sa, const uint16_t* sw, const uint16_t* nsa,
                                                const uint16_t* nsw, f32x16_t (&acc)[4][Layout<NT>::JB],
                                                Frag<NT> (&f)[2], int n_mul, Work&& work, Sync&& sync) {
  constexpr int JB = Layout<NT>::JB;
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    const int c = kk & 1;
    if (kk + 1 < BK / 16) {
      if (kk + 1 < n_mul) read_frag<NT>(f[c ^ 1], sa, sw, kk + 1);
    } else {
      read_frag<NT>(f[0], nsa, nsw, 0);
    }
    if (kk < n_mul) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f[c].a[i], f[c].b[j], acc[i][j], 0, 0, 0);
    }
    if (kk < 2) {
      work(kk);
    } else if (kk == 2) {
      work(2);
      work(3);
      sync();
    }
  }
}

// Epilogue through LDS: half a tile (128 rows) at a time, each thread then moves
// 4 consecutive columns per step with one 8- or 16-byte global access.
// out(m, n) for m < M_lim, n < N_lim; a bf16 or float32 residual is added first; the
// rotary embedding (float32) is applied to columns below rope_cols (counted from the
// start of the whole output, col_base = this group's first column) before rounding.
struct Epi {
  void* out = nullptr; int ldo = 0; bool f32 = false;
  const uint16_t* r16 = nullptr; const float* r32 = nullptr; int ldr = 0;
  const float2* rope_tab = nullptr; int rope_cols = 0, col_base = 0, seq = 1, hd = 128;
  // SwiGLU backward: the product is dact; with g, u from gu (float32 [M, ldgu], u at
  // column + N_lim) write dgate, dup as bf16 into out ([M, ldo], dup at column + N_lim)
  const float* gu = nullptr; int ldgu = 0;
};

__device__ __forceinline__ float sigmoid_f(float z) { return 1.0f / (1.0f + __expf(-z)); }

// SwiGLU backward of one element: with act = silu(g) u and silu(g) = g sigmoid(g),
// dgate = y u sigmoid(g) (1 + g (1 - sigmoid(g))) and dup = y g sigmoid(g) for
// y = d(act).  Both epilogues that run it use this one routine.
__device__ __forceinline__ void swiglu_bwd(float y, float g, float u, float& dg, float& du) {
  const float sg = sigmoid_f(g);
  dg = y * u * sg * (1.0f + g * (1.0f - sg));
  du = y * g * sg;
}

template <int NT>
__device__ __forceinline__ void epilogue(Smem& sm, f32x16_t (&acc)[4][Layout<NT>::JB], int m0, int n0, int M_lim,
                                         int N_lim, const Epi& E) {
  constexpr int WNW = Layout<NT>::WNW, JB = Layout<NT>::JB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WNW, wn = wave % WNW;
  constexpr int OP = BN + 4;
  constexpr int RS = NT / 64;            // rows apart of one thread's consecutive rows
  constexpr int RPT = 128 / RS;          // rows per thread per half tile
  constexpr int CH = RPT < 4 ? RPT : 4;  // rows per batch of global reads
  for (int half = 0; half < 2; ++half) {
    __syncthreads();
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
            const int c = wn * (32 * JB) + j * 32 + (lane & 31);
            sm.u.out[r * OP + c] = acc[i][j][v];
          }
    }
    __syncthreads();
    // Thread t handles column quad q = t % 64 of rows t / 64 + RS k.  Each batch of CH
    // rows issues all its global reads (residual, rotary table, or g and u) before it
    // uses any of them, so a batch waits on memory once, not once per row; rows past
    // M_lim read the last row and are not written.
    const int mbase = m0 + half * 128;
    const int q = threadIdx.x & 63, rt = threadIdx.x >> 6;
    const int n = n0 + 4 * q;
    if (n >= N_lim) continue;           // the next half starts at a barrier every thread reaches
    const bool full = n + 4 <= N_lim;
    const int gc = E.col_base + n;
    const bool rope = gc < E.rope_cols;
    const int hh = E.hd / 2, i0 = rope ? gc % E.hd : 0;
    const bool lo = i0 < hh;
    // what the batch reads: g and u, the rotary table, a float32 or a bf16 residual
    const int mode = E.gu ? 1 : rope ? 2 : (full && E.r32) ? 3 : (full && E.r16) ? 4 : 0;
#pragma unroll 1
    for (int c = 0; c < RPT; c += CH) {
      float4 pre[CH][2];
      int mrow[CH];
#pragma unroll
      for (int k = 0; k < CH; ++k) mrow[k] = min(mbase + rt + RS * (c + k), M_lim - 1);
      // one branch per batch, then CH rows of reads back to back
      if (mode == 1) {   // N_lim % 4 == 0 here
#pragma unroll
        for (int k = 0; k < CH; ++k) {
          pre[k][0] = *reinterpret_cast<const float4*>(E.gu + (int64_t)mrow[k] * E.ldgu + n);
          pre[k][1] = *reinterpret_cast<const float4*>(E.gu + (int64_t)mrow[k] * E.ldgu + N_lim + n);
        }
      } else if (mode == 2) {
#pragma unroll
        for (int k = 0; k < CH; ++k) {
          const float2* tab = E.rope_tab + (int64_t)(mrow[k] % E.seq) * hh + (i0 % hh);
          pre[k][0] = make_float4(tab[0].x, tab[0].y, tab[1].x, tab[1].y);
          pre[k][1] = make_float4(tab[2].x, tab[2].y, tab[3].x, tab[3].y);
        }
      } else if (mode == 3) {
#pragma unroll
        for (int k = 0; k < CH; ++k) pre[k][0] = *reinterpret_cast<const float4*>(E.r32 + (int64_t)mrow[k] * E.ldr + n);
      } else if (mode == 4) {
#pragma unroll
        for (int k = 0; k < CH; ++k) {
          const uint2 rr = *reinterpret_cast<const uint2*>(E.r16 + (int64_t)mrow[k] * E.ldr + n);
          pre[k][0] = make_float4(bf16_lo(rr.x), bf16_hi(rr.x), bf16_lo(rr.y), bf16_hi(rr.y));
        }
      }
#pragma unroll
      for (int k = 0; k < CH; ++k) {
        const int r = rt + RS * (c + k);
        const int m = mbase + r;
        if (m >= M_lim) break;
        const float4 v = *reinterpret_cast<const float4*>(&sm.u.out[r * OP + 4 * q]);
        float y[4] = {v.x, v.y, v.z, v.w};
        if (mode == 1) {
          const float gs[4] = {pre[k][0].x, pre[k][0].y, pre[k][0].z, pre[k][0].w};
          const float us[4] = {pre[k][1].x, pre[k][1].y, pre[k][1].z, pre[k][1].w};
          float dg[4], du[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) swiglu_bwd(y[e], gs[e], us[e], dg[e], du[e]);
          uint16_t* po = reinterpret_cast<uint16_t*>(E.out) + (int64_t)m * E.ldo + n;
          *reinterpret_cast<uint2*>(po) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
          *reinterpret_cast<uint2*>(po + N_lim) = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
          continue;
        }
        if (rope) {
          const float4 pv = *reinterpret_cast<const float4*>(&sm.u.out[r * OP + 4 * q + (lo ? hh : -hh)]);
          const float pr[4] = {pv.x, pv.y, pv.z, pv.w};
          const float cx[4] = {pre[k][0].x, pre[k][0].z, pre[k][1].x, pre[k][1].z};
          const float cy[4] = {pre[k][0].y, pre[k][0].w, pre[k][1].y, pre[k][1].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = lo ? y[e] * cx[e] - pr[e] * cy[e] : y[e] * cx[e] + pr[e] * cy[e];
        }
        const int64_t o = (int64_t)m * E.ldo + n;
        if (E.r16 || E.r32) {
          const int64_t ro = (int64_t)m * E.ldr + n;
          if (mode >= 3) {   // read in the batch above
            y[0] += pre[k][0].x; y[1] += pre[k][0].y; y[2] += pre[k][0].z; y[3] += pre[k][0].w;
          } else if (full && E.r32) {
            const float4 rr = *reinterpret_cast<const float4*>(E.r32 + ro);
            y[0] += rr.x; y[1] += rr.y; y[2] += rr.z; y[3] += rr.w;
          } else if (full) {
            const uint2 rr = *reinterpret_cast<const uint2*>(E.r16 + ro);
            y[0] += bf16_lo(rr.x); y[1] += bf16_hi(rr.x); y[2] += bf16_lo(rr.y); y[3] += bf16_hi(rr.y);
          } else if (E.r32) {
            for (int e = 0; e < 4 && n + e < N_lim; ++e) y[e] += E.r32[ro + e];
          } else {
            for (int e = 0; e < 4 && n + e < N_lim; ++e) y[e] += bf16_lo(E.r16[ro + e]);
          }
        }
        if (E.f32) {
          float* po = reinterpret_cast<float*>(E.out) + o;
          if (full) *reinterpret_cast<float4*>(po) = make_float4(y[0], y[1], y[2], y[3]);
          else for (int e = 0; e < 4 && n + e < N_lim; ++e) po[e] = y[e];
        } else {
          uint16_t* po = reinterpret_cast<uint16_t*>(E.out) + o;
          const uint32_t p0 = pack_bf16x2(y[0], y[1]), p1 = pack_bf16x2(y[2], y[3]);
          if (full) *reinterpret_cast<uint2*>(po) = make_uint2(p0, p1);
          else {
            const uint16_t h[4] = {(uint16_t)p0, (uint16_t)(p0 >> 16), (uint16_t)p1, (uint16_t)(p1 >> 16)};
            for (int e = 0; e < 4 && n + e < N_lim; ++e) po[e] = h[e];
          }
        }
      }
    }
  }
}

// SwiGLU forward epilogue of a paired tile: columns 0..127 are gate, 128..255 up, for
// outputs j0 .. j0 + 127.  act = bf16(silu(g) u); with gu set, g and u are also kept in
// float32 (gu [M, ldgu], up at column + I); with dact set (float32 d(act), [M, ldda]),
// the SwiGLU backward runs here as well and dgu ([M, lddgu], dup at column + I)
// receives dgate | dup in bf16.
template <int NT>
__device__ __forceinline__ void epilogue_swiglu(Smem& sm, f32x16_t (&acc)[4][Layout<NT>::JB], int m0, int j0, int M_lim,
                                                int I, uint16_t* act, int ldact, float* gu, int ldgu,
                                                const float* dact, int ldda, uint16_t* dgu, int lddgu) {
  constexpr int WNW = Layout<NT>::WNW, JB = Layout<NT>::JB;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WNW, wn = wave % WNW;
  constexpr int OP = BN + 4;
  for (int half = 0; half < 2; ++half) {
    __syncthreads();
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JB; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
            const int c = wn * (32 * JB) + j * 32 + (lane & 31);
            sm.u.out[r * OP + c] = acc[i][j][v];
          }
    }
    __syncthreads();
    const int mbase = m0 + half * 128;
#pragma unroll 4
    for (int it = 0; it < 4096 / NT; ++it) {
      const int idx = threadIdx.x + NT * it;           // 128 rows x 32 quads
      const int r = idx >> 5, q = idx & 31;
      const int m = mbase + r, j = j0 + 4 * q;
      if (m >= M_lim || j >= I) continue;              // I % 4 == 0
      const float4 g4 = *reinterpret_cast<const float4*>(&sm.u.out[r * OP + 4 * q]);
      const float4 u4 = *reinterpret_cast<const float4*>(&sm.u.out[r * OP + 128 + 4 * q]);
      const float gs[4] = {g4.x, g4.y, g4.z, g4.w}, us[4] = {u4.x, u4.y, u4.z, u4.w};
      float a[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = gs[e] * sigmoid_f(gs[e]) * us[e];
      *reinterpret_cast<uint2*>(act + (int64_t)m * ldact + j) = make_uint2(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]));
      if (gu) {
        *reinterpret_cast<float4*>(gu + (int64_t)m * ldgu + j) = g4;
        *reinterpret_cast<float4*>(gu + (int64_t)m * ldgu + I + j) = u4;
      }
      if (dact) {
        const float4 d4 = *reinterpret_cast<const float4*>(dact + (int64_t)m * ldda + j);
        const float ys[4] = {d4.x, d4.y, d4.z, d4.w};
        float dg[4], du[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) swiglu_bwd(ys[e], gs[e], us[e], dg[e], du[e]);
        uint16_t* po = dgu + (int64_t)m * lddgu + j;
        *reinterpret_cast<uint2*>(po) = make_uint2(pack_bf16x2(dg[0], dg[1]), pack_bf16x2(dg[2], dg[3]));
        *reinterpret_cast<uint2*>(po + I) = make_uint2(pack_bf16x2(du[0], du[1]), pack_bf16x2(du[2], du[3]));
      }
    }
  }
}

// (m tile, n tile) of linear tile t of an m_tiles x n_tiles grid.  Each XCD's run of
// the linear order covers about m_tiles / 8 rows of m tiles; inside a group of that
// many m rows the m tile varies fastest, so the tiles of one weight tile (one n) run at
// about the same time on one XCD and share its L2, as do the tiles of one activation
// row block across the group.
__device__ __forceinline__ void tile_mn(int t, int m_tiles, int n_tiles, int& mt, int& nt) {
  const int gm = m_tiles >= 16 ? m_tiles >> 3 : 1;
  const int g = t / (gm * n_tiles);
  const int m_in = m_tiles - g * gm < gm ? m_tiles - g * gm : gm;
  const int r = t - g * gm * n_tiles;
  mt = g * gm + r % m_in;
  nt = r / m_in;
}

__device__ __forceinline__ int xcd_tile(int bid, int nblocks_padded) {
  // Workgroups go round-robin over the 8 XCDs; give each XCD a contiguous run of
  // tiles (n fastest below) so the tiles sharing activation rows share one L2.
  const int per = nblocks_padded / 8;
  return (bid & 7) * per + (bid >> 3);
}

// ---- work of one fast-path workgroup: K stages [ks, ke) of one tile.  Without split
// tiles a workgroup runs one whole tile (xcd_tile order).  With them, the launch's
// tiles are n_whole whole tiles (full rounds of the compute units, possibly none) plus
// a tail of fewer tiles than compute units, each cut into `split` pieces of about
// nk / split K stages, so the last round is fuller.  Every XCD (bid & 7) gets the same
// share of both: its first n_whole / 8 workgroups run whole tiles, the rest the pieces
// of its tail / 8 tail tiles (so the pieces of one tile share an XCD).
struct Piece { int tile, ks, ke, slot, idx; };
__device__ __forceinline__ Piece piece_of(int total_tiles, int nk, int padded, int n_whole, int split) {
  Piece p;
  if (split <= 1) {
    p.tile = xcd_tile(blockIdx.x, padded);
    p.ks = 0; p.ke = p.tile < total_tiles ? nk : 0;
    p.slot = -1; p.idx = 0;
    return p;
  }
  const int x = blockIdx.x & 7, li = blockIdx.x >> 3;
  const int wx = n_whole / 8, tx = (total_tiles - n_whole) / 8;
  if (li < wx) {
    p.tile = x * wx + li;
    p.ks = 0; p.ke = nk;
    p.slot = -1; p.idx = 0;
  } else {
    const int q = li - wx;
    p.slot = x * tx + q / split;
    p.tile = n_whole + p.slot;
    p.idx = q - (q / split) * split;
    p.ks = p.idx * nk / split;
    p.ke = (p.idx + 1) * nk / split;
    if (q >= tx * split) p.ke = p.ks;   // past the XCD's pieces (none when the grid is exact)
  }
  return p;
}

// A tail tile's `split` pieces meet in part[slot][piece] and cnt[slot].  Each piece
// writes its float32 sums and then counts itself; the piece that counts last reads
// all of them back and adds them in piece order (so the result does not depend on
// which piece comes last), writes the tile and sets the counter back to zero.  Nobody
// waits on another piece.  The partial sums are written and read at device scope
// (the sc1 cache policy: through to the point where every XCD sees them, the form
// the compiler gives device-scope atomic loads and stores), so they need no L2
// write-back or invalidation; the writes are complete (vmcnt 0) before the count.
// Returns whether this workgroup writes the tile.
constexpr int kScopeDevice = 16;   // buffer cache-policy bits: sc1 = device scope

template <int NT>
__device__ __forceinline__ bool combine_pieces(f32x16_t (&acc)[4][Layout<NT>::JB], float* part, uint32_t* cnt,
                                               int slot, int piece, int split, uint32_t* flag) {
  constexpr int JB = Layout<NT>::JB;
  constexpr int TILE = BM * BN;
  typedef float f32x4 __attribute__((ext_vector_type(4)));
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const rsrc_t pres = make_rsrc_wave(part + (size_t)slot * split * TILE, (uint64_t)split * TILE * 4);
  const uint32_t own = (uint32_t)piece * (TILE * 4u);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const f32x4 t = {acc[i][j][4 * v], acc[i][j][4 * v + 1], acc[i][j][4 * v + 2], acc[i][j][4 * v + 3]};
        const uint32_t off = (uint32_t)((((i * JB + j) * 4 + v) * NT + threadIdx.x) * 16);
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, t), pres, own + off, 0, kScopeDevice);
      }
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  if (threadIdx.x == 0) *flag = atomicAdd(cnt + slot, 1u);
  __syncthreads();
  if (*flag != (uint32_t)(split - 1)) return false;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < JB; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const uint32_t off = (uint32_t)((((i * JB + j) * 4 + v) * NT + threadIdx.x) * 16);
        f32x4 t = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(pres, off, 0, kScopeDevice));
        for (int pc = 1; pc < split; ++pc)
          t += __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(pres, (uint32_t)pc * (TILE * 4u) + off,
                                                                               0, kScopeDevice));
        acc[i][j][4 * v] = t.x;
        acc[i][j][4 * v + 1] = t.y;
        acc[i][j][4 * v + 2] = t.z;
        acc[i][j][4 * v + 3] = t.w;
      }
  if (threadIdx.x == 0) cnt[slot] = 0;
  return true;
}

// ------------------------------------------------------------------ forward
template <int FMT, bool ALIGNED>
__global__ void __launch_bounds__(NTHREADS, 1) k_gemm_fwd(FwdArgs args, int n_tiles, int total_tiles, int padded) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  const int tile = xcd_tile(blockIdx.x, padded);
  if (tile >= total_tiles) return;
  // tile -> (m tile, group, n tile); n fastest so an XCD's run shares activation rows
  const int mt = tile / n_tiles;
  int rest = tile - mt * n_tiles;
  int g = 0;
  for (; g < args.n_groups - 1; ++g) {
    const int nt_g = (args.g[g].w.n_out + BN - 1) / BN;
    if (rest < nt_g) break;
    rest -= nt_g;
  }
  const FwdGroup& G = args.g[g];
  const int m0 = mt * BM, n0 = rest * BN;
  const int K = args.K;
  const int n_out = G.w.n_out;

  fill_lut2(sm, args.levels);

  f32x16_t acc[4][Layout<NTHREADS>::JB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

  const int rows_left = args.M - m0;
  const rsrc_t xres = make_rsrc(args.x + (int64_t)m0 * args.ldx, (uint64_t)(rows_left < BM ? rows_left : BM) * args.ldx * 2);
  const WRes wres = make_wres<FMT>(G.w);
  const int nk = (K + BK - 1) / BK;
  // Iteration 0 is the low-rank term: A columns from aext (s*H, bf16) against the bf16
  // copy of B, zero beyond kx (all zero when the adapters are off).  Iterations
  // 1..nk are the K tiles of X and W.  Two register sets keep tiles i+1 and i+2 in
  // flight; tile i+1 is written to the other LDS stage while stage i is multiplied.
  const int n_iter = nk + 1;
  {
    const bool has_ext = args.kx > 0 && G.bext != nullptr;
    const rsrc_t ares = make_rsrc(has_ext ? args.aext + (int64_t)m0 * args.ldaext : args.x,
                                  has_ext ? (uint64_t)(rows_left < BM ? rows_left : BM) * args.ldaext * 2 : 0);
    const int brows = n_out - n0 < BN ? n_out - n0 : BN;
    const rsrc_t bres = make_rsrc(has_ext ? G.bext + (int64_t)n0 * args.kx : args.x,
                                  has_ext ? (uint64_t)brows * args.kx * 2 : 0);
    ALoad ea, eb;
    load_a(ea, ares, (uint32_t)G.ext_col0 * 2u, args.ldaext, rows_left, 0, args.kx);
    load_a(eb, bres, 0, args.kx, brows, 0, args.kx);
    store_a(ea, sm.u.k.a[0]);
    store_a(eb, sm.u.k.w[0]);
  }

  ALoad ra;
  WFwd<FMT, ALIGNED> rw, rw_next;
#pragma unroll
    for (int q = 0; q < 4; ++q) load_a_part(ra, xres, 0, args.ldx, rows_left, 0, K, q);
    rw.load(wres, n_out, K, n0, 0);
    rw_next.load(wres, n_out, K, n0, BK);
    __syncthreads();
    for (int it = 0; it < n_iter; ++it) {
      const int cur = it & 1;
      uint16_t* na = sm.u.k.a[cur ^ 1];
      uint16_t* nw = sm.u.k.w[cur ^ 1];
      const int k_next2 = (it + 1) * BK;
      mma_stage<NTHREADS>(sm.u.k.a[cur], sm.u.k.w[cur], acc, [&](int q) {
        store_a_part(ra, na, q);
        load_a_part(ra, xres, 0, args.ldx, rows_left, k_next2, K, q);
        rw.store_part(nw, sm.lut2, q);
      });
      rw = rw_next;
      rw_next.load(wres, n_out, K, n0, (it + 2) * BK);
      __syncthreads();
    }

  Epi E;
  E.f32 = args.y32 != nullptr;
  E.out = E.f32 ? (void*)(args.y32 + G.out_col0) : (void*)(args.y + G.out_col0);
  E.ldo = args.ldy;
  E.r16 = args.resid ? args.resid + G.out_col0 : nullptr;
  E.r32 = args.resid32 ? args.resid32 + G.out_col0 : nullptr;
  E.ldr = args.ldr;
  E.rope_tab = args.rope_tab; E.rope_cols = args.rope_tab ? args.rope_cols : 0;
  E.col_base = G.out_col0; E.seq = args.seq; E.hd = args.head_dim;
  epilogue<NTHREADS>(sm, acc, m0, n0, args.M, n_out, E);
}

// ------------------------------------------------------------------ backward
template <int FMT, bool ALIGNED>
__global__ void __launch_bounds__(NTHREADS, 1) k_gemm_bwd(BwdArgs args, int n_tiles, int total_tiles, int padded) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  const int tile = xcd_tile(blockIdx.x, padded);
  if (tile >= total_tiles) return;
  const int mt = tile / n_tiles;
  const int nt = tile - mt * n_tiles;
  const int m0 = mt * BM, j0 = nt * BN;

  fill_lut2(sm, args.levels);

  f32x16_t acc[4][Layout<NTHREADS>::JB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

  const int rows_left = args.M - m0;
  const rsrc_t dres = make_rsrc(args.dy + (int64_t)m0 * args.lddy, (uint64_t)(rows_left < BM ? rows_left : BM) * args.lddy * 2);
  int seg_tiles[kMaxGroups];
  int total_k = 0;
  for (int s = 0; s < args.n_segs; ++s) {
    seg_tiles[s] = (args.seg[s].w.n_out + BK - 1) / BK;
    total_k += seg_tiles[s];
  }
  // Iteration 0 is the low-rank term (s*G against A^T, bf16); iterations 1..total_k
  // run over the K tiles of the stacked segments.  Same two-set pipeline as forward.
  const int n_iter = total_k + 1;
  {
    const bool has_ext = args.kx > 0;
    const rsrc_t ares = make_rsrc(has_ext ? args.aext + (int64_t)m0 * args.ldaext : args.dy,
                                  has_ext ? (uint64_t)(rows_left < BM ? rows_left : BM) * args.ldaext * 2 : 0);
    const int brows = args.N - j0 < BN ? args.N - j0 : BN;
    const rsrc_t bres = make_rsrc(has_ext ? args.bext + (int64_t)j0 * args.ldbext : args.dy,
                                  has_ext ? (uint64_t)brows * args.ldbext * 2 : 0);
    ALoad ea, eb;
    load_a(ea, ares, 0, args.ldaext, rows_left, 0, args.kx);
    load_a(eb, bres, 0, args.ldbext, brows, 0, args.kx);
    store_a(ea, sm.u.k.a[0]);
    store_a(eb, sm.u.k.w[0]);
  }
  // tile index t (0-based over the stacked segments) -> segment and row offset
  auto seg_of = [&](int t, int& s_out, int& k0_out) {
    int s = 0;
    if (t >= total_k) { s_out = args.n_segs - 1; k0_out = (seg_tiles[s_out] + 1) * BK; return; }   // zeros
    while (t >= seg_tiles[s]) { t -= seg_tiles[s]; ++s; }
    s_out = s; k0_out = t * BK;
  };
    auto load_a_q = [&](ALoad& ra, int t, int q) {
      int s, k0; seg_of(t, s, k0);
      load_a_part(ra, dres, (uint32_t)args.seg[s].a_col0 * 2u, args.lddy, rows_left, k0, args.seg[s].w.n_out, q);
    };
    auto load_w = [&](WBwd<FMT, ALIGNED>& rw, int t) {
      int s, k0; seg_of(t, s, k0);
      const WRes wres = make_wres<FMT>(args.seg[s].w);
      rw.load(wres, args.seg[s].w.n_in, k0, args.seg[s].w.n_out, j0);
    };
    ALoad ra;
    WBwd<FMT, ALIGNED> rw, rw_next;
#pragma unroll
    for (int q = 0; q < 4; ++q) load_a_q(ra, 0, q);
    load_w(rw, 0);
    load_w(rw_next, 1);
    __syncthreads();
    for (int it = 0; it < n_iter; ++it) {
      const int cur = it & 1;
      uint16_t* na = sm.u.k.a[cur ^ 1];
      uint16_t* nw = sm.u.k.w[cur ^ 1];
      mma_stage<NTHREADS>(sm.u.k.a[cur], sm.u.k.w[cur], acc, [&](int q) {
        store_a_part(ra, na, q);
        load_a_q(ra, it + 1, q);
        rw.store_part(nw, sm.lut2, q);
      });
      rw = rw_next;
      load_w(rw_next, it + 2);
      __syncthreads();
    }

  Epi E;
  E.f32 = args.out32 != nullptr;
  E.out = E.f32 ? (void*)args.out32 : (void*)args.out16;
  E.ldo = args.ldo;
  E.gu = args.gu32; E.ldgu = args.ldgu;
  E.r32 = args.resid32; E.ldr = args.ldo;
  epilogue<NTHREADS>(sm, acc, m0, j0, args.M, args.N, E);
}

// ------------------------------------------------- fast path, 512 threads
// 8 waves (2 per SIMD: while one waits on LDS or memory the other issues), each
// 128 x 64 of the tile.  Used when K % 64 == 0 (forward) or every stacked segment's
// rows % 64 == 0 (backward), so no tile straddles the end of a row.
// PAIRED (SwiGLU): groups 0 and 1 are gate and up with the same shape; a tile holds
// gate rows 128 t.. (waves 0-3 load them) and the same up rows (waves 4-7), and its
// epilogue writes silu(gate) * up.  The low-rank terms become one 2 kx wide extension:
// [H_gate | H_up] against [B_gate | 0] for the gate half and [0 | B_up] for the up half.
template <int FMT, bool PAIRED>
__global__ void __launch_bounds__(NT_FAST, 1) k_gemm_fwd_fast(FwdArgs args, int n_tiles, int total_tiles, int padded,
                                                              int n_whole, int split) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  const int K = args.K;
  const int nk = K / BK;
  const Piece pc = piece_of(total_tiles, nk, padded, n_whole, split);
  if (pc.ks >= pc.ke) return;
  const int tile = pc.tile, ks = pc.ks, ke = pc.ke;

  fill_lut2(sm, args.levels);

  {
    int mt, rest;
    tile_mn(tile, total_tiles / n_tiles, n_tiles, mt, rest);
    int g = 0;
    if constexpr (!PAIRED) {
      for (; g < args.n_groups - 1; ++g) {
        const int nt_g = (args.g[g].w.n_out + BN - 1) / BN;
        if (rest < nt_g) break;
        rest -= nt_g;
      }
    }
    const FwdGroup& G = args.g[g];
    const int m0 = mt * BM;
    const int n0 = PAIRED ? rest * (BN / 2) : rest * BN;
    const int n_out = G.w.n_out;

    constexpr int JB = Layout<NT_FAST>::JB;
    f32x16_t acc[4][JB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < JB; ++j) acc[i][j] = f32x16_t{};

    const int rows_left = args.M - m0;
    const int arows = rows_left < BM ? rows_left : BM;
    const rsrc_t xres = make_rsrc(args.x + (int64_t)m0 * args.ldx, (uint64_t)arows * args.ldx * 2);
    const int n_iter = ke - ks + 1;   // iteration 0: the low-rank term (first piece only)
    // The low-rank term goes with the tile's first piece; a later piece leaves stage
    // 0 unread (its low-rank stage multiplies nothing).
    const int ext_cols = ks > 0 ? 0
                         : PAIRED ? (args.kx > 0 ? 2 * args.kx : 0)
                                  : (args.kx > 0 && G.bext != nullptr ? args.kx : 0);
    if (ext_cols > 0) {
      if constexpr (PAIRED) {
        const int kx = args.kx;
        const rsrc_t ares = make_rsrc(args.aext + (int64_t)m0 * args.ldaext, (uint64_t)arows * args.ldaext * 2);
        ext_tile(sm.u.k.a[0], ares, (uint32_t)G.ext_col0 * 2u, args.ldaext, arows, 2 * kx);
        const int brows = n_out - n0 < BN / 2 ? n_out - n0 : BN / 2;
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const uint16_t* bx = args.g[hf].bext;
          const bool on = bx != nullptr;
          const rsrc_t bres = make_rsrc(on ? bx + (int64_t)n0 * kx : args.x, on ? (uint64_t)brows * kx * 2 : 0);
          ext_tile<2>(sm.u.k.w[0] + hf * (BN / 2) * PITCH, bres, 0, kx, on ? brows : 0, kx, hf * kx);
        }
      } else {
        const int brows = n_out - n0 < BN ? n_out - n0 : BN;
        const rsrc_t ares = make_rsrc(args.aext + (int64_t)m0 * args.ldaext, (uint64_t)arows * args.ldaext * 2);
        const rsrc_t bres = make_rsrc(G.bext + (int64_t)n0 * args.kx, (uint64_t)brows * args.kx * 2);
        ext_tile(sm.u.k.a[0], ares, (uint32_t)G.ext_col0 * 2u, args.ldaext, arows, args.kx);
        ext_tile(sm.u.k.w[0], bres, 0, args.kx, brows, args.kx);
      }
    }
    // A: one register set, each quarter reloaded for tile it+1 right after it is
    // stored; W: current and next tile in registers.  Loads past the piece are skipped.
    AFast ra;
    ra.init(xres, args.ldx);
    WFwdFast<FMT> ws;
    {
      const WeightRef& wsel = PAIRED ? args.g[threadIdx.x >> 8].w : G.w;   // wave-uniform
      const uint32_t r = PAIRED ? (threadIdx.x >> 1) & 127u : threadIdx.x >> 1;
      ws.init(wsel, n0, r, PAIRED ? BN / 2 : BN);
    }
    typename WFwdFast<FMT>::Regs rw, rw_next;
    WFwdFast<FMT>::clear(rw);
    WFwdFast<FMT>::clear(rw_next);
    const int k_first = ks * BK, k_end = ke * BK, k_last = k_end - BK;
#pragma unroll
    for (int q = 0; q < 4; ++q) ra.load_q((uint32_t)k_first, q);
    ws.load(rw, k_first);
    ws.load(rw_next, k_first + BK < k_end ? k_first + BK : k_first);   // unconditional, like the loop's prefetches
    // Drain the prologue's loads once: otherwise their order here, merged into the loop
    // head, sets the wait counts of every iteration.
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    __syncthreads();
    Frag<NT_FAST> fr[2];
    read_frag<NT_FAST>(fr[0], sm.u.k.a[0], sm.u.k.w[0], 0);
    // Iteration it dequantises W tile ks + it from R and then reloads R with tile
    // ks + it + 2.  The two register sets alternate by unrolling two iterations: a copy
    // between them would wait on the loads still in flight into the source.  Every
    // prefetch is issued on every path (the compiler counts only loads that are always
    // issued when it places its waits; a skipped-load branch makes it wait for every
    // load in flight).  Iteration 0, the low-rank stage, multiplies only its non-zero k
    // steps; the K stages follow in pairs, and an odd count of them gets one padding
    // stage: an activation tile past the piece loads as zeros (out-of-range offset), W
    // past it re-reads the piece's last tile, so the padding stage adds exact zeros.
    // Each stage's barrier comes before its last k16 step (mma_stage_early).
    auto step = [&](int it, typename WFwdFast<FMT>::Regs& R, auto low_rank) {
      const int cur = it & 1;
      uint16_t* na = sm.u.k.a[cur ^ 1];
      uint16_t* nw = sm.u.k.w[cur ^ 1];
      const int k_next = k_first + (it + 1) * BK;
      const bool past = k_next >= k_end;
      const float am = FMT == WF_BF16 ? 0.f : ws.absmax(R);
      auto work = [&](int q) {
        ra.store_q(na, q);
        ra.load_q_or_zero((uint32_t)k_next, q, past);
        ws.store_part(R, nw, sm.lut2, q, am);
      };
      auto sync = [&]() {
        ws.load(R, k_next + BK < k_last ? k_next + BK : k_last);
        __syncthreads();
        // let the scheduler interleave the next stage's fragment reads with the last
        // step's MFMAs (the same hint before the barrier, or with the plain NF4 scales,
        // costs spilled registers)
        if constexpr (FMT != WF_NF4) __builtin_amdgcn_iglp_opt(0);
      };
      mma_stage_early<NT_FAST>(sm.u.k.a[cur], sm.u.k.w[cur], na, nw, acc, fr,
                               decltype(low_rank)::value ? (ext_cols + 15) / 16 : BK / 16, work, sync);
    };
    step(0, rw, std::true_type{});
    for (int it = 1; it < n_iter; it += 2) {
      step(it, rw_next, std::false_type{});
      step(it + 1, rw, std::false_type{});
    }

    if (pc.slot >= 0 && !combine_pieces<NT_FAST>(acc, args.sk.part, args.sk.cnt, pc.slot, pc.idx, split, &sm.sk_flag))
      return;
    if constexpr (PAIRED) {
      epilogue_swiglu<NT_FAST>(sm, acc, m0, n0, args.M, n_out, args.y, args.ldy, args.gu32, args.ldgu, args.dact,
                               args.ldda, args.dgu, args.lddgu);
    } else {
      Epi E;
      E.f32 = args.y32 != nullptr;
      E.out = E.f32 ? (void*)(args.y32 + G.out_col0) : (void*)(args.y + G.out_col0);
      E.ldo = args.ldy;
      E.r16 = args.resid ? args.resid + G.out_col0 : nullptr;
      E.r32 = args.resid32 ? args.resid32 + G.out_col0 : nullptr;
      E.ldr = args.ldr;
      E.rope_tab = args.rope_tab; E.rope_cols = args.rope_tab ? args.rope_cols : 0;
      E.col_base = G.out_col0; E.seq = args.seq; E.hd = args.head_dim;
      epilogue<NT_FAST>(sm, acc, m0, n0, args.M, n_out, E);
    }
  }
}

template <int FMT>
__global__ void __launch_bounds__(NT_FAST, 1) k_gemm_bwd_fast(BwdArgs args, int n_tiles, int total_tiles, int padded,
                                                              int n_whole, int split) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  Smem& sm = *reinterpret_cast<Smem*>(smem_raw);
  int seg_tiles[kMaxGroups];
  int total_k = 0;
  for (int s = 0; s < args.n_segs; ++s) {
    seg_tiles[s] = args.seg[s].w.n_out / BK;
    total_k += seg_tiles[s];
  }
  const Piece pc = piece_of(total_tiles, total_k, padded, n_whole, split);
  if (pc.ks >= pc.ke) return;
  const int tile = pc.tile, ks = pc.ks, ke = pc.ke;

  fill_lut2(sm, args.levels);

  // stacked K tile t < total_k -> segment and first row
  auto seg_of = [&](int t, int& s_out, int& k0_out) {
    int s = 0;
    while (t >= seg_tiles[s]) { t -= seg_tiles[s]; ++s; }
    s_out = s; k0_out = t * BK;
  };
  WBwdFast<FMT> ws;
  ws.init_lane(args.N);

  {
    int mt, nt;
    tile_mn(tile, total_tiles / n_tiles, n_tiles, mt, nt);
    const int m0 = mt * BM, j0 = nt * BN;

    constexpr int JB = Layout<NT_FAST>::JB;
    f32x16_t acc[4][JB];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < JB; ++j) acc[i][j] = f32x16_t{};

    const int rows_left = args.M - m0;
    const int arows = rows_left < BM ? rows_left : BM;
    const rsrc_t dres = make_rsrc(args.dy + (int64_t)m0 * args.lddy, (uint64_t)arows * args.lddy * 2);
    // iteration 0: the low-rank term (kx <= 64), in the tile's first piece only
    const int ext_cols = ks > 0 ? 0 : args.kx;
    if (ext_cols > 0) {
      const int brows = args.N - j0 < BN ? args.N - j0 : BN;
      const rsrc_t ares = make_rsrc(args.aext + (int64_t)m0 * args.ldaext, (uint64_t)arows * args.ldaext * 2);
      const rsrc_t bres = make_rsrc(args.bext + (int64_t)j0 * args.ldbext, (uint64_t)brows * args.ldbext * 2);
      ext_tile(sm.u.k.a[0], ares, 0, args.ldaext, arows, args.kx);
      ext_tile(sm.u.k.w[0], bres, 0, args.ldbext, brows, args.kx);
    }
    AFast ra;
    ra.init(dres, args.lddy);
    typename WBwdFast<FMT>::Regs rw, rw_next;
    WBwdFast<FMT>::clear(rw);
    WBwdFast<FMT>::clear(rw_next);
    // loads past the piece re-read its last tile (see the forward kernel)
    auto load_w = [&](typename WBwdFast<FMT>::Regs& R, int t) {
      int s, k0; seg_of(t < ke ? t : ke - 1, s, k0);
      ws.load(R, args.seg[s].w, j0, k0);
    };
    {
      int s, k0; seg_of(ks, s, k0);
#pragma unroll
      for (int q = 0; q < 4; ++q) ra.load_q((uint32_t)(args.seg[s].a_col0 + k0), q);
    }
    load_w(rw, ks);
    load_w(rw_next, ks + 1);
    __builtin_amdgcn_s_waitcnt(kWaitVm0);   // see the forward kernel
    __syncthreads();
    const int n_iter = ke - ks + 1;
    // as in the forward kernel: two register sets for W alternating without copies,
    // prefetches on every path, the low-rank stage multiplying only its non-zero k
    // steps, then the K stages in pairs (one zero padding stage if their count is odd)
    auto step = [&](int it, typename WBwdFast<FMT>::Regs& R, auto low_rank) {
      const int cur = it & 1;
      uint16_t* na = sm.u.k.a[cur ^ 1];
      uint16_t* nw = sm.u.k.w[cur ^ 1];
      const bool past = ks + it + 1 >= ke;
      uint32_t col;
      { int s, k0; seg_of(past ? ke - 1 : ks + it + 1, s, k0); col = (uint32_t)(args.seg[s].a_col0 + k0); }
      const float a0 = FMT == WF_BF16 ? 0.f : ws.absmax(R, 0);
      const float a1 = FMT == WF_BF16 ? 0.f : ws.absmax(R, 1);
      auto work = [&](int q) {
        ra.store_q(na, q);
        ra.load_q_or_zero(col, q, past);
        ws.store_part(R, nw, sm.lut2, q, a0, a1);
      };
      if constexpr (decltype(low_rank)::value)
        mma_stage_n<NT_FAST>(sm.u.k.a[cur], sm.u.k.w[cur], acc, (ext_cols + 15) / 16, work);
      else
        mma_stage<NT_FAST>(sm.u.k.a[cur], sm.u.k.w[cur], acc, work);
      load_w(R, ks + it + 2);
      __syncthreads();
    };
    step(0, rw, std::true_type{});
    for (int it = 1; it < n_iter; it += 2) {
      step(it, rw_next, std::false_type{});
      step(it + 1, rw, std::false_type{});
    }

    if (pc.slot >= 0 && !combine_pieces<NT_FAST>(acc, args.sk.part, args.sk.cnt, pc.slot, pc.idx, split, &sm.sk_flag))
      return;
    Epi E;
    E.f32 = args.out32 != nullptr;
    E.out = E.f32 ? (void*)args.out32 : (void*)args.out16;
    E.ldo = args.ldo;
    E.gu = args.gu32; E.ldgu = args.ldgu;
    E.r32 = args.resid32; E.ldr = args.ldo;
    epilogue<NT_FAST>(sm, acc, m0, j0, args.M, args.N, E);
  }
}

// --------------------------------------------------------- standalone dequant
template <int FMT>
__global__ void k_dequant(WeightRef w, const float* levels, uint16_t* out) {
  const uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;   // element pair
  const uint64_t e = 2 * i;
  if (e >= (uint64_t)w.n_out * w.n_in) return;
  if constexpr (FMT == WF_BF16) {
    out[e] = reinterpret_cast<const uint16_t*>(w.w)[e];
    out[e + 1] = reinterpret_cast<const uint16_t*>(w.w)[e + 1];
  } else {
    const uint32_t byte = w.w[i];
    const float a0 = block_absmax<FMT>(w, e / kNF4Block);
    const float a1 = block_absmax<FMT>(w, (e + 1) / kNF4Block);
    const uint32_t pk = pack_bf16x2(levels[byte >> 4] * a0, levels[byte & 15u] * a1);
    out[e] = (uint16_t)(pk & 0xFFFFu);
    out[e + 1] = (uint16_t)(pk >> 16);
  }
}

template <class F>
hipError_t launch_fmt(int format, F&& f) {
  switch (format) {
    case WF_NF4: return f(std::integral_constant<int, WF_NF4>{});
    case WF_NF4_DQ: return f(std::integral_constant<int, WF_NF4_DQ>{});
    default: return f(std::integral_constant<int, WF_BF16>{});
  }
}

// compute units of the current device, read once per device
int cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess) cached[dev] = n;
  }
  return cached[dev];
}

// Grid of a fast launch of `total` tiles of nk K stages.  Split the tail (the tiles
// past the last full round of compute units, or all of them when there are fewer tiles
// than units) when scratch is given and the tail would leave the last round at most
// 7/8 full: each tail tile becomes `split` pieces, as many as fit the round (at most
// 8, each at least 4 K stages).
void plan_split(const SplitTiles& sk, int total, int nk, int& grid, int& n_whole, int& split) {
  grid = (total + 7) / 8 * 8;
  n_whole = total;
  split = 1;
  if (!sk.part || !sk.cnt) return;
  const int P = cu_count();
  if (P <= 0 || P % 8 != 0 || sk.slots < P) return;
  const int tail = total % P;
  if (tail == 0 || tail % 8 != 0 || tail > P / 8 * 7) return;
  int S = P / tail;
  if (S > 8) S = 8;
  if (S > nk / 4) S = nk / 4;
  if (S < 2) return;
  n_whole = total - tail;
  split = S;
  grid = n_whole + tail * S;
}

}  // namespace

hipError_t launch_gemm_fwd(const FwdArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.n_groups <= 0) return hipSuccess;
  if (a.kx > BK) return hipErrorInvalidValue;   // one extension tile in the forward
  const int m_tiles = (a.M + BM - 1) / BM;
  int n_tiles = 0;
  for (int g = 0; g < a.n_groups; ++g) n_tiles += (a.g[g].w.n_out + BN - 1) / BN;
  const int total = m_tiles * n_tiles;
  const int padded = (total + 7) / 8 * 8;
  const bool fast = (a.K % BK) == 0 && a.K >= BK && (a.ldx % 8) == 0;
  if (a.swiglu) {
    // paired gate | up tiles: same shape, adjacent low-rank columns, 2 kx <= 64
    if (!fast || a.n_groups != 2 || a.g[0].w.n_out != a.g[1].w.n_out || a.g[0].w.n_in != a.g[1].w.n_in ||
        a.g[0].w.n_out % 4 != 0 || 2 * a.kx > BK || (a.kx > 0 && a.g[1].ext_col0 != a.g[0].ext_col0 + a.kx) ||
        !a.y || a.y32 || a.resid || a.resid32 || a.rope_tab || a.ldy % 4 != 0 || (a.gu32 && a.ldgu % 4 != 0) ||
        (a.dact && (a.gu32 || !a.dgu || a.ldda % 4 != 0 || a.lddgu % 4 != 0 ||
                    (reinterpret_cast<uintptr_t>(a.dact) & 15) || (reinterpret_cast<uintptr_t>(a.dgu) & 7))))
      return hipErrorInvalidValue;
    const int pt = (a.g[0].w.n_out + BN / 2 - 1) / (BN / 2);
    const int ptotal = m_tiles * pt;
    int grid, n_whole, split;
    plan_split(a.sk, ptotal, a.K / BK, grid, n_whole, split);
    return launch_fmt(a.format, [&](auto fmt) {
      constexpr int F = decltype(fmt)::value;
      hipLaunchKernelGGL((k_gemm_fwd_fast<F, true>), dim3(grid), dim3(NT_FAST), sizeof(Smem), s, a, pt, ptotal, grid,
                         n_whole, split);
      return hipGetLastError();
    });
  }
  if (a.dact) return hipErrorInvalidValue;   // the SwiGLU backward rides on the paired tiles only
  int grid = padded, n_whole = total, split = 1;
  if (fast) plan_split(a.sk, total, a.K / BK, grid, n_whole, split);
  return launch_fmt(a.format, [&](auto fmt) {
    constexpr int F = decltype(fmt)::value;
    if (fast)
      hipLaunchKernelGGL((k_gemm_fwd_fast<F, false>), dim3(grid), dim3(NT_FAST), sizeof(Smem), s, a, n_tiles, total, grid,
                         n_whole, split);
    else hipLaunchKernelGGL((k_gemm_fwd<F, false>), dim3(padded), dim3(NTHREADS), sizeof(Smem), s, a, n_tiles, total, padded);
    return hipGetLastError();
  });
}

hipError_t launch_gemm_bwd(const BwdArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  const int m_tiles = (a.M + BM - 1) / BM;
  const int n_tiles = (a.N + BN - 1) / BN;
  const int total = m_tiles * n_tiles;
  const int padded = (total + 7) / 8 * 8;
  // fast path: whole NF4 blocks per W row, every segment a whole number of K tiles,
  // 16-byte aligned activation rows
  bool fast = (a.N % BK) == 0 && (a.lddy % 8) == 0 && a.n_segs > 0;
  for (int sg = 0; sg < a.n_segs; ++sg)
    fast = fast && (a.seg[sg].w.n_out % BK) == 0 && a.seg[sg].w.n_out >= BK && (a.seg[sg].a_col0 % 8) == 0;
  // The kernel takes the first 64 low-rank columns as one extra K tile; wider
  // low-rank terms (stacked q|k|v or gate|up at rank > 16) add the remaining columns
  // into the float32 result with a second, generic MFMA GEMM.
  if (a.kx > BK && !a.out32) return hipErrorInvalidValue;
  if (a.resid32 && (!a.out32 || a.gu32 || a.kx > BK)) return hipErrorInvalidValue;
  if (a.gu32 && (!a.out16 || a.out32 || a.N % 4 != 0 || a.ldo % 4 != 0 || a.ldgu % 4 != 0 || a.kx > BK))
    return hipErrorInvalidValue;
  BwdArgs k = a;
  if (k.kx > BK) k.kx = BK;
  int grid = padded, n_whole = total, split = 1;
  if (fast) {
    int total_k = 0;
    for (int sg = 0; sg < a.n_segs; ++sg) total_k += a.seg[sg].w.n_out / BK;
    plan_split(a.sk, total, total_k, grid, n_whole, split);
  }
  hipError_t e = launch_fmt(a.format, [&](auto fmt) {
    constexpr int F = decltype(fmt)::value;
    if (fast)
      hipLaunchKernelGGL(k_gemm_bwd_fast<F>, dim3(grid), dim3(NT_FAST), sizeof(Smem), s, k, n_tiles, total, grid, n_whole,
                         split);
    else hipLaunchKernelGGL((k_gemm_bwd<F, false>), dim3(padded), dim3(NTHREADS), sizeof(Smem), s, k, n_tiles, total, padded);
    return hipGetLastError();
  });
  if (e != hipSuccess || a.kx <= BK) return e;
  GemmArgs g;
  g.A = a.aext + BK; g.sAm = a.ldaext; g.sAk = 1;
  g.B = a.bext + BK; g.sBn = a.ldbext; g.sBk = 1;
  g.C = a.out32; g.sCm = a.ldo; g.sCn = 1; g.c_f32 = 1;
  g.M = a.M; g.N = a.N; g.K = a.kx - BK;
  g.alpha = 1.f; g.beta = 1.f;
  return launch_gemm_generic(g, s);
}

hipError_t launch_dequant(const WeightRef& w, int32_t format, const float* levels, uint16_t* out, hipStream_t s) {
  const uint64_t pairs = ((uint64_t)w.n_out * w.n_in + 1) / 2;
  const dim3 grid((unsigned)((pairs + 255) / 256));
  switch (format) {
    case WF_NF4: hipLaunchKernelGGL(k_dequant<WF_NF4>, grid, dim3(256), 0, s, w, levels, out); break;
    case WF_NF4_DQ: hipLaunchKernelGGL(k_dequant<WF_NF4_DQ>, grid, dim3(256), 0, s, w, levels, out); break;
    default: hipLaunchKernelGGL(k_dequant<WF_BF16>, grid, dim3(256), 0, s, w, levels, out); break;
  }
  return hipGetLastError();
}

// Kernels use the full 144 KiB stage buffers: allow the dynamic LDS size once.
hipError_t gemm_dequant_init() {
  hipError_t e = hipSuccess;
  auto set = [&](const void* k) {
    hipError_t r = hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)sizeof(Smem));
    if (r != hipSuccess) e = r;
  };
  set((const void*)k_gemm_fwd<WF_NF4, false>);
  set((const void*)k_gemm_fwd<WF_NF4_DQ, false>);
  set((const void*)k_gemm_fwd<WF_BF16, false>);
  set((const void*)k_gemm_bwd<WF_NF4, false>);
  set((const void*)k_gemm_bwd<WF_NF4_DQ, false>);
  set((const void*)k_gemm_bwd<WF_BF16, false>);
  set((const void*)k_gemm_fwd_fast<WF_NF4, false>);
  set((const void*)k_gemm_fwd_fast<WF_NF4, true>);
  set((const void*)k_gemm_fwd_fast<WF_NF4_DQ, false>);
  set((const void*)k_gemm_fwd_fast<WF_NF4_DQ, true>);
  set((const void*)k_gemm_fwd_fast<WF_BF16, false>);
  set((const void*)k_gemm_fwd_fast<WF_BF16, true>);
  set((const void*)k_gemm_bwd_fast<WF_NF4>);
  set((const void*)k_gemm_bwd_fast<WF_NF4_DQ>);
  set((const void*)k_gemm_bwd_fast<WF_BF16>);
  return e;
}

}  // namespace lsq
