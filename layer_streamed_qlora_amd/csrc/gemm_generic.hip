// Generic batched bf16 MFMA GEMM for the small products around the dequant GEMMs:
// the LoRA down projection s*X*A^T, the LoRA gradients (dY*B, dY^T*H, G^T*X) and the
// materialised causal attention (Q*K^T, P*V and their backward products).
//
// C(m, n) = alpha * sum_k A(m, k) * B(n, k) + beta * C(m, n), float32 accumulation.
// Either operand may be stored k-contiguous (loaded with 16-byte rows) or
// m/n-contiguous (loaded along m/n and transposed into LDS), so one kernel serves
// X*A^T, dY^T*H and P^T*dO alike.  Tile 128 x 64 (or 128 x 32 for rank-r outputs),
// K step 32, 4 waves of v_mfma_f32_32x32x16_bf16 blocks, double-buffered LDS.  Long
// contractions over few output tiles (the LoRA reductions over all tokens) are split
// over K with float32 partials summed afterwards in a fixed order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsq_internal.hpp"

namespace lsq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int GM = 128, GK = 32, GP = GK + 8;   // pitch in bf16
constexpr int GT = 256;

__device__ __forceinline__ uint16_t to_bf16(float x) {
  f32x2_t v = {x, 0.f};
  return (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t)) & 0xFFFFu);
}

__device__ __forceinline__ int64_t zoff(const ZStride& z, int zi, int zdiv) {
  return (int64_t)(zi / zdiv) * z.s1 + (int64_t)((zi % zdiv) / z.grp) * z.s2;
}

// Load a ROWS x GK tile of operand X (X(r, k) = base + r*sr + k*sk) into LDS [ROWS][GP].
template <int ROWS, bool KCONTIG>
struct TileLoad {
  static constexpr int NCH = ROWS * GK / 8;                // 16-byte chunks per tile
  static constexpr int CHUNKS = (NCH + GT - 1) / GT;       // per thread
  uint4 v[CHUNKS];
  __device__ __forceinline__ void load(const uint16_t* base, int64_t sr, int64_t sk, int rows_left, int k0, int klim) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = threadIdx.x + GT * i;
      if (c >= NCH) { v[i] = make_uint4(0, 0, 0, 0); continue; }
      if constexpr (KCONTIG) {
        const int r = c / (GK / 8), kc = (c % (GK / 8)) * 8;
        if (r < rows_left && k0 + kc < klim)
          v[i] = *reinterpret_cast<const uint4*>(base + (int64_t)r * sr + (k0 + kc));
        else
          v[i] = make_uint4(0, 0, 0, 0);
      } else {
        const int kr = c / (ROWS / 8), rc = (c % (ROWS / 8)) * 8;
        if (rc < rows_left && k0 + kr < klim)
          v[i] = *reinterpret_cast<const uint4*>(base + (int64_t)(k0 + kr) * sk + rc);
        else
          v[i] = make_uint4(0, 0, 0, 0);
      }
    }
  }
  __device__ __forceinline__ void store(uint16_t* s) const {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = threadIdx.x + GT * i;
      if (c >= NCH) continue;
      if constexpr (KCONTIG) {
        const int r = c / (GK / 8), kc = (c % (GK / 8)) * 8;
        *reinterpret_cast<uint4*>(s + r * GP + kc) = v[i];
      } else {
        const int kr = c / (ROWS / 8), rc = (c % (ROWS / 8)) * 8;
        const uint16_t* e = reinterpret_cast<const uint16_t*>(&v[i]);
#pragma unroll
        for (int q = 0; q < 8; ++q) s[(rc + q) * GP + kr] = e[q];
      }
    }
  }
};

// Tile GM x GNT: 4 waves; GNT = 64 -> 2 x 2 waves of 64 x 32, GNT = 32 -> 4 x 1 waves
// of 32 x 32 (narrow outputs such as the rank-r LoRA products).
template <bool AK, bool BK_, int GNT>
__global__ void __launch_bounds__(GT) k_gemm_generic(GemmArgs a) {
  constexpr int WNW = GNT / 32;            // waves along n
  constexpr int WMW = 4 / WNW;             // waves along m
  constexpr int MB = GM / WMW / 32;        // 32-row MFMA blocks per wave
  __shared__ __align__(16) uint16_t sA[2][GM * GP];
  __shared__ __align__(16) uint16_t sB[2][GNT * GP];
  const int zk = blockIdx.z;
  const int z = zk / a.ksplit, ks = zk - z * a.ksplit;
  const int m0 = blockIdx.x * GM, n0 = blockIdx.y * GNT;
  if (a.causal == 1 && n0 > m0 + GM - 1) return;          // tile fully above the diagonal
  const uint16_t* A = a.A + zoff(a.zA, z, a.zdiv) + (AK ? (int64_t)m0 * a.sAm : (int64_t)m0);
  const uint16_t* B = a.B + zoff(a.zB, z, a.zdiv) + (BK_ ? (int64_t)n0 * a.sBn : (int64_t)n0);
  int klim = a.K;
  if (a.causal == 2) klim = min(klim, m0 + GM);            // contraction k <= m only
  int kbeg = 0;
  if (a.causal == 3) kbeg = (m0 / GK) * GK;                 // contraction k >= m only
  if (a.ksplit > 1) {
    const int chunk = ((klim - kbeg + a.ksplit - 1) / a.ksplit + GK - 1) / GK * GK;
    kbeg = kbeg + ks * chunk;
    klim = min(klim, kbeg + chunk);
  }
  const int rows_a = a.M - m0, rows_b = a.N - n0;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WNW, wn = wave % WNW;
  f32x16_t acc[MB];
#pragma unroll
  for (int i = 0; i < MB; ++i) acc[i] = f32x16_t{};

  TileLoad<GM, AK> la;
  TileLoad<GNT, BK_> lb;
  const int nk = klim > kbeg ? (klim - kbeg + GK - 1) / GK : 0;
  if (nk > 0) {
    la.load(A, AK ? a.sAm : a.sAk, AK ? 1 : a.sAk, rows_a, kbeg, klim);
    lb.load(B, BK_ ? a.sBn : a.sBk, BK_ ? 1 : a.sBk, rows_b, kbeg, klim);
    la.store(sA[0]);
    lb.store(sB[0]);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int k0 = kbeg + (kt + 1) * GK;
      la.load(A, AK ? a.sAm : a.sAk, AK ? 1 : a.sAk, rows_a, k0, klim);
      lb.load(B, BK_ ? a.sBn : a.sBk, BK_ ? 1 : a.sBk, rows_b, k0, klim);
    }
#pragma unroll
    for (int kk = 0; kk < GK / 16; ++kk) {
      const bf16x8_t bfr = *reinterpret_cast<const bf16x8_t*>(&sB[cur][(wn * 32 + (lane & 31)) * GP + kk * 16 + (lane >> 5) * 8]);
#pragma unroll
      for (int i = 0; i < MB; ++i) {
        const bf16x8_t afr = *reinterpret_cast<const bf16x8_t*>(&sA[cur][(wm * MB * 32 + i * 32 + (lane & 31)) * GP + kk * 16 + (lane >> 5) * 8]);
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(afr, bfr, acc[i], 0, 0, 0);
      }
    }
    if (more) {
      la.store(sA[cur ^ 1]);
      lb.store(sB[cur ^ 1]);
    }
    __syncthreads();
  }
  // epilogue
  const int n = n0 + wn * 32 + (lane & 31);
  if (n >= a.N) return;
  if (a.ksplit > 1) {
    float* part = a.partial + ((int64_t)ks * (a.nz) + z) * (int64_t)a.M * a.N;
#pragma unroll
    for (int i = 0; i < MB; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + wm * MB * 32 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        if (m < a.M) part[(int64_t)m * a.N + n] = acc[i][v];
      }
    return;
  }
  const int64_t cz = zoff(a.zC, z, a.zdiv);
#pragma unroll
  for (int i = 0; i < MB; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + wm * MB * 32 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
      if (m >= a.M) continue;
      const int64_t o = cz + (int64_t)m * a.sCm + (int64_t)n * a.sCn;
      float y = a.alpha * acc[i][v];
      if (a.c_f32) {
        float* c = reinterpret_cast<float*>(a.C) + o;
        if (a.beta != 0.f) y += a.beta * *c;
        *c = y;
      } else {
        uint16_t* c = reinterpret_cast<uint16_t*>(a.C) + o;
        if (a.beta != 0.f) y += a.beta * __builtin_bit_cast(float, (uint32_t)*c << 16);
        *c = to_bf16(y);
      }
    }
}

// Sum the split-K partials in chunk order, then C = alpha * sum + beta * C.
__global__ void k_splitk_reduce(GemmArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t per = (int64_t)a.M * a.N;
  if (idx >= per * a.nz) return;
  const int z = (int)(idx / per);
  const int64_t mn = idx - (int64_t)z * per;
  const int m = (int)(mn / a.N), n = (int)(mn - (int64_t)m * a.N);
  float s = 0.f;
  for (int k = 0; k < a.ksplit; ++k) s += a.partial[((int64_t)k * a.nz + z) * per + mn];
  const int64_t o = zoff(a.zC, z, a.zdiv) + (int64_t)m * a.sCm + (int64_t)n * a.sCn;
  float y = a.alpha * s;
  if (a.c_f32) {
    float* c = reinterpret_cast<float*>(a.C) + o;
    if (a.beta != 0.f) y += a.beta * *c;
    *c = y;
  } else {
    uint16_t* c = reinterpret_cast<uint16_t*>(a.C) + o;
    if (a.beta != 0.f) y += a.beta * __builtin_bit_cast(float, (uint32_t)*c << 16);
    *c = to_bf16(y);
  }
}

}  // namespace

template <int GNT>
static void launch_tiles(const GemmArgs& a, hipStream_t s) {
  const dim3 grid((a.M + GM - 1) / GM, (a.N + GNT - 1) / GNT, a.nz * a.ksplit);
  const bool ak = a.sAk == 1, bk = a.sBk == 1;
  if (ak && bk) hipLaunchKernelGGL((k_gemm_generic<true, true, GNT>), grid, dim3(GT), 0, s, a);
  else if (ak) hipLaunchKernelGGL((k_gemm_generic<true, false, GNT>), grid, dim3(GT), 0, s, a);
  else if (bk) hipLaunchKernelGGL((k_gemm_generic<false, true, GNT>), grid, dim3(GT), 0, s, a);
  else hipLaunchKernelGGL((k_gemm_generic<false, false, GNT>), grid, dim3(GT), 0, s, a);
}

hipError_t launch_gemm_generic(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.nz <= 0) return hipSuccess;
  if (a.ksplit > 1 && !a.partial) return hipErrorInvalidValue;
  if (a.N <= 32) launch_tiles<32>(a, s);
  else launch_tiles<64>(a, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.ksplit <= 1) return e;
  const int64_t n = (int64_t)a.M * a.N * a.nz;
  hipLaunchKernelGGL(k_splitk_reduce, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace lsq
