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

// 8 codes (one dword, byte k = code[2k] << 4 | code[2k+1]) -> 4 dwords of bf16 pairs
__device__ __forceinline__ void dequant8(uint32_t codes, float am, const float* lut, uint32_t out[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t byte = (codes >> (8 * k)) & 0xFFu;
    const float a = lut[byte >> 4] * am;
    const float b = lut[byte & 15u] * am;
    out[k] = pack_bf16x2(a, b);
  }
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOOB = 0xFFFFFFF0u;   // offset past every buffer: the load returns 0

__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFF0ull ? 0xFFFFFFF0u : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)n, 0x00020000);
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
  union {
    struct {
      uint16_t a[2][TILE_ELEMS];
      uint16_t w[2][TILE_ELEMS];
    } k;
    float out[128 * (BN + 4)];       // epilogue staging, one half tile (128 rows) at a time
  } u;
  float lut[16];
};

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
__device__ __forceinline__ void store_a(const ALoad& r, uint16_t* s) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int c = t + NTHREADS * i;
    const int row = c >> 3, kc = (c & 7) * 8;
    *reinterpret_cast<uint4*>(s + row * PITCH + kc) = r.v[i];
  }
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
  __device__ __forceinline__ void store(uint16_t* s, const float* lut) const {
    uint16_t* row = s + threadIdx.x * PITCH;
    if constexpr (FMT == WF_BF16) {
#pragma unroll
      for (int i = 0; i < 8; ++i) *reinterpret_cast<uint4*>(row + 8 * i) = raw[i];
    } else {
      const uint32_t* r32 = reinterpret_cast<const uint32_t*>(raw);
#pragma unroll
      for (int q = 0; q < 8; ++q) {      // 8 dwords of codes = 64 elements
        uint32_t o[4];
        dequant8(r32[q], ALIGNED ? am[0] : am[q / 2], lut, o);
        *reinterpret_cast<uint4*>(row + 8 * q) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
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
  __device__ __forceinline__ void store(uint16_t* s, const float* lut) const {
    const int p = threadIdx.x & 31, c = threadIdx.x >> 5;
    uint32_t* dst = reinterpret_cast<uint32_t*>(s + (32 * c) * PITCH + 2 * p);
    const int pitch32 = PITCH / 2;
    if constexpr (FMT == WF_BF16) {
      const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&raw[0]);
      const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&raw[4]);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        dst[(2 * q) * pitch32] = __builtin_amdgcn_perm(r1[q], r0[q], 0x05040100u);
        dst[(2 * q + 1) * pitch32] = __builtin_amdgcn_perm(r1[q], r0[q], 0x07060302u);
      }
    } else {
      const uint32_t* r0 = reinterpret_cast<const uint32_t*>(&raw[0]);
      const uint32_t* r1 = reinterpret_cast<const uint32_t*>(&raw[1]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {           // 4 dwords per row = 32 codes
        const float a0 = ALIGNED ? am[0][0] : am[0][q / 2];
        const float a1 = ALIGNED ? am[1][0] : am[1][q / 2];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t b0 = (r0[q] >> (8 * k)) & 0xFFu, b1 = (r1[q] >> (8 * k)) & 0xFFu;
          const int j = 8 * q + 2 * k;
          dst[j * pitch32] = pack_bf16x2(lut[b0 >> 4] * a0, lut[b1 >> 4] * a1);
          dst[(j + 1) * pitch32] = pack_bf16x2(lut[b0 & 15u] * a0, lut[b1 & 15u] * a1);
        }
      }
    }
  }
};

// ---- MFMA over one LDS stage
template <int KSTEPS>
__device__ __forceinline__ void mma_stage(const uint16_t* sa, const uint16_t* sw, f32x16_t acc[4][4]) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const uint16_t* pa = sa + (wm * 128 + (lane & 31)) * PITCH + (lane >> 5) * 8;
  const uint16_t* pw = sw + (wn * 128 + (lane & 31)) * PITCH + (lane >> 5) * 8;
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) {
    bf16x8_t a[4], b[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = *reinterpret_cast<const bf16x8_t*>(pa + i * 32 * PITCH + kk * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) b[j] = *reinterpret_cast<const bf16x8_t*>(pw + j * 32 * PITCH + kk * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
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
};

__device__ __forceinline__ void epilogue(Smem& sm, f32x16_t acc[4][4], int m0, int n0, int M_lim, int N_lim,
                                         const Epi& E) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  constexpr int OP = BN + 4;
  for (int half = 0; half < 2; ++half) {
    __syncthreads();
    if (wm == half) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int r = i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
            const int c = wn * 128 + j * 32 + (lane & 31);
            sm.u.out[r * OP + c] = acc[i][j][v];
          }
    }
    __syncthreads();
    const int mbase = m0 + half * 128;
#pragma unroll 4
    for (int it = 0; it < 32; ++it) {
      const int idx = threadIdx.x + NTHREADS * it;     // 128 rows x 64 quads
      const int r = idx >> 6, q = idx & 63;
      const int m = mbase + r, n = n0 + 4 * q;
      if (m >= M_lim || n >= N_lim) continue;
      const float4 v = *reinterpret_cast<const float4*>(&sm.u.out[r * OP + 4 * q]);
      float y[4] = {v.x, v.y, v.z, v.w};
      const int gc = E.col_base + n;
      if (gc < E.rope_cols) {
        const int hh = E.hd / 2, i0 = gc % E.hd;
        const int lo = i0 < hh;
        const float4 pv = *reinterpret_cast<const float4*>(&sm.u.out[r * OP + 4 * q + (lo ? hh : -hh)]);
        const float pr[4] = {pv.x, pv.y, pv.z, pv.w};
        const float2* tab = E.rope_tab + (int64_t)(m % E.seq) * hh + (i0 % hh);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float2 cs = tab[e];
          y[e] = lo ? y[e] * cs.x - pr[e] * cs.y : y[e] * cs.x + pr[e] * cs.y;
        }
      }
      const int64_t o = (int64_t)m * E.ldo + n;
      const bool full = n + 4 <= N_lim;
      if (E.r16 || E.r32) {
        const int64_t ro = (int64_t)m * E.ldr + n;
        if (E.r32) {
          if (full) { const float4 rr = *reinterpret_cast<const float4*>(E.r32 + ro); y[0] += rr.x; y[1] += rr.y; y[2] += rr.z; y[3] += rr.w; }
          else for (int e = 0; e < 4 && n + e < N_lim; ++e) y[e] += E.r32[ro + e];
        } else if (full) {
          const uint2 rr = *reinterpret_cast<const uint2*>(E.r16 + ro);
          y[0] += bf16_lo(rr.x); y[1] += bf16_hi(rr.x); y[2] += bf16_lo(rr.y); y[3] += bf16_hi(rr.y);
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

__device__ __forceinline__ int xcd_tile(int bid, int nblocks_padded) {
  // Workgroups go round-robin over the 8 XCDs; give each XCD a contiguous run of
  // tiles (n fastest below) so the tiles sharing activation rows share one L2.
  const int per = nblocks_padded / 8;
  return (bid & 7) * per + (bid >> 3);
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

  if (threadIdx.x < 16) sm.lut[threadIdx.x] = args.levels ? args.levels[threadIdx.x] : 0.f;

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16_t{};

  const int rows_left = args.M - m0;
  const rsrc_t xres = make_rsrc(args.x + (int64_t)m0 * args.ldx, (uint64_t)(rows_left < BM ? rows_left : BM) * args.ldx * 2);
  const WRes wres = make_wres<FMT>(G.w);
  const int nk = (K + BK - 1) / BK;
  // The low-rank term runs as one extra K tile of the same loop: A columns from
  // aext (s*H, bf16), B columns from the bf16 copy of B, zero beyond kx.
  const bool has_ext = args.kx > 0 && G.bext != nullptr;
  ALoad ra, rb;
  WFwd<FMT, ALIGNED> rw;
  load_a(ra, xres, 0, args.ldx, rows_left, 0, K);
  rw.load(wres, n_out, K, n0, 0);
  __syncthreads();   // lut visible
  store_a(ra, sm.u.k.a[0]);
  rw.store(sm.u.k.w[0], sm.lut);
  __syncthreads();
  const int nsteps = nk + (has_ext ? 1 : 0);
  for (int kt = 0; kt < nsteps; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    const bool ext_next = has_ext && kt + 1 == nk;
    if (more) {
      load_a(ra, xres, 0, args.ldx, rows_left, (kt + 1) * BK, K);
      rw.load(wres, n_out, K, n0, (kt + 1) * BK);
    } else if (ext_next) {
      const rsrc_t ares = make_rsrc(args.aext + (int64_t)m0 * args.ldaext, (uint64_t)(rows_left < BM ? rows_left : BM) * args.ldaext * 2);
      const int brows = n_out - n0 < BN ? n_out - n0 : BN;
      const rsrc_t bres = make_rsrc(G.bext + (int64_t)n0 * args.kx, (uint64_t)brows * args.kx * 2);
      load_a(ra, ares, (uint32_t)G.ext_col0 * 2u, args.ldaext, rows_left, 0, args.kx);
      load_a(rb, bres, 0, args.kx, brows, 0, args.kx);
    }
    mma_stage<BK / 16>(sm.u.k.a[cur], sm.u.k.w[cur], acc);
    if (more) {
      store_a(ra, sm.u.k.a[cur ^ 1]);
      rw.store(sm.u.k.w[cur ^ 1], sm.lut);
    } else if (ext_next) {
      store_a(ra, sm.u.k.a[cur ^ 1]);
      store_a(rb, sm.u.k.w[cur ^ 1]);
    }
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
  epilogue(sm, acc, m0, n0, args.M, n_out, E);
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

  if (threadIdx.x < 16) sm.lut[threadIdx.x] = args.levels ? args.levels[threadIdx.x] : 0.f;

  f32x16_t acc[4][4];
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
  ALoad ra, rb;
  WBwd<FMT, ALIGNED> rw;
  int cur_seg = -1;
  WRes wres;
  auto issue = [&](int idx) {
    int s = 0;
    while (idx >= seg_tiles[s]) { idx -= seg_tiles[s]; ++s; }
    const BwdSeg& S = args.seg[s];
    if (s != cur_seg) { wres = make_wres<FMT>(S.w); cur_seg = s; }
    const int k0 = idx * BK;
    load_a(ra, dres, (uint32_t)S.a_col0 * 2u, args.lddy, rows_left, k0, S.w.n_out);
    rw.load(wres, S.w.n_in, k0, S.w.n_out, j0);
  };
  // The low-rank term (s*G against A^T) runs as one extra K tile of the same loop.
  const bool has_ext = args.kx > 0;
  issue(0);
  __syncthreads();
  store_a(ra, sm.u.k.a[0]);
  rw.store(sm.u.k.w[0], sm.lut);
  __syncthreads();
  const int nsteps = total_k + (has_ext ? 1 : 0);
  for (int kt = 0; kt < nsteps; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < total_k;
    const bool ext_next = has_ext && kt + 1 == total_k;
    if (more) {
      issue(kt + 1);
    } else if (ext_next) {
      const rsrc_t ares = make_rsrc(args.aext + (int64_t)m0 * args.ldaext, (uint64_t)(rows_left < BM ? rows_left : BM) * args.ldaext * 2);
      const int brows = args.N - j0 < BN ? args.N - j0 : BN;
      const rsrc_t bres = make_rsrc(args.bext + (int64_t)j0 * args.ldbext, (uint64_t)brows * args.ldbext * 2);
      load_a(ra, ares, 0, args.ldaext, rows_left, 0, args.kx);
      load_a(rb, bres, 0, args.ldbext, brows, 0, args.kx);
    }
    mma_stage<BK / 16>(sm.u.k.a[cur], sm.u.k.w[cur], acc);
    if (more) {
      store_a(ra, sm.u.k.a[cur ^ 1]);
      rw.store(sm.u.k.w[cur ^ 1], sm.lut);
    } else if (ext_next) {
      store_a(ra, sm.u.k.a[cur ^ 1]);
      store_a(rb, sm.u.k.w[cur ^ 1]);
    }
    __syncthreads();
  }
  Epi E;
  E.f32 = args.out32 != nullptr;
  E.out = E.f32 ? (void*)args.out32 : (void*)args.out16;
  E.ldo = args.ldo;
  epilogue(sm, acc, m0, j0, args.M, args.N, E);
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
hipError_t launch_fmt(int format, bool aligned, F&& f) {
  switch (format) {
    case WF_NF4: return aligned ? f(std::integral_constant<int, WF_NF4>{}, std::true_type{})
                                : f(std::integral_constant<int, WF_NF4>{}, std::false_type{});
    case WF_NF4_DQ: return aligned ? f(std::integral_constant<int, WF_NF4_DQ>{}, std::true_type{})
                                   : f(std::integral_constant<int, WF_NF4_DQ>{}, std::false_type{});
    default: return f(std::integral_constant<int, WF_BF16>{}, std::true_type{});
  }
}

}  // namespace

hipError_t launch_gemm_fwd(const FwdArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.n_groups <= 0) return hipSuccess;
  const int m_tiles = (a.M + BM - 1) / BM;
  int n_tiles = 0;
  for (int g = 0; g < a.n_groups; ++g) n_tiles += (a.g[g].w.n_out + BN - 1) / BN;
  const int total = m_tiles * n_tiles;
  const int padded = (total + 7) / 8 * 8;
  const bool aligned = (a.K % BK) == 0;
  return launch_fmt(a.format, aligned, [&](auto fmt, auto al) {
    auto kern = k_gemm_fwd<decltype(fmt)::value, decltype(al)::value>;
    hipLaunchKernelGGL(kern, dim3(padded), dim3(NTHREADS), sizeof(Smem), s, a, n_tiles, total, padded);
    return hipGetLastError();
  });
}

hipError_t launch_gemm_bwd(const BwdArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0) return hipSuccess;
  const int m_tiles = (a.M + BM - 1) / BM;
  const int n_tiles = (a.N + BN - 1) / BN;
  const int total = m_tiles * n_tiles;
  const int padded = (total + 7) / 8 * 8;
  const bool aligned = (a.N % BK) == 0;
  return launch_fmt(a.format, aligned, [&](auto fmt, auto al) {
    auto kern = k_gemm_bwd<decltype(fmt)::value, decltype(al)::value>;
    hipLaunchKernelGGL(kern, dim3(padded), dim3(NTHREADS), sizeof(Smem), s, a, n_tiles, total, padded);
    return hipGetLastError();
  });
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
  set((const void*)k_gemm_fwd<WF_NF4, true>);
  set((const void*)k_gemm_fwd<WF_NF4, false>);
  set((const void*)k_gemm_fwd<WF_NF4_DQ, true>);
  set((const void*)k_gemm_fwd<WF_NF4_DQ, false>);
  set((const void*)k_gemm_fwd<WF_BF16, true>);
  set((const void*)k_gemm_bwd<WF_NF4, true>);
  set((const void*)k_gemm_bwd<WF_NF4, false>);
  set((const void*)k_gemm_bwd<WF_NF4_DQ, true>);
  set((const void*)k_gemm_bwd<WF_NF4_DQ, false>);
  set((const void*)k_gemm_bwd<WF_BF16, true>);
  return e;
}

}  // namespace lsq
