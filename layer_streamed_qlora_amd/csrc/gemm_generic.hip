// Generic batched bf16 MFMA GEMM for the small products around the dequant GEMMs:
// the LoRA down projection s*X*A^T, the LoRA gradients (dY*B, dY^T*H, G^T*X) and the
// materialised causal attention (Q*K^T, P*V and their backward products).
//
// C(m, n) = alpha * sum_k A(m, k) * B(n, k) + beta * C(m, n), float32 accumulation.
// Either operand may be stored k-contiguous (loaded with 16-byte rows) or
// m/n-contiguous (loaded along m/n and transposed into LDS), so one kernel serves
// X*A^T, dY^T*H and P^T*dO alike.  Tile 128 x 64, K step 32, 4 waves of 64 x 32
// (2 x 1 blocks of v_mfma_f32_32x32x16_bf16), double-buffered LDS.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsq_internal.hpp"

namespace lsq {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

constexpr int GM = 128, GN = 64, GK = 32, GP = GK + 8;   // pitch in bf16
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
  static constexpr int CHUNKS = ROWS * GK / 8 / GT;   // 16-byte chunks per thread
  uint4 v[CHUNKS];
  __device__ __forceinline__ void load(const uint16_t* base, int64_t sr, int64_t sk, int rows_left, int k0, int klim) {
#pragma unroll
    for (int i = 0; i < CHUNKS; ++i) {
      const int c = threadIdx.x + GT * i;
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

template <bool AK, bool BK_>
__global__ void __launch_bounds__(GT) k_gemm_generic(GemmArgs a) {
  __shared__ __align__(16) uint16_t sA[2][GM * GP];
  __shared__ __align__(16) uint16_t sB[2][GN * GP];
  const int z = blockIdx.z;
  const int m0 = blockIdx.x * GM, n0 = blockIdx.y * GN;
  if (a.causal == 1 && n0 > m0 + GM - 1) return;          // tile fully above the diagonal
  const uint16_t* A = a.A + zoff(a.zA, z, a.zdiv) + (AK ? (int64_t)m0 * a.sAm : (int64_t)m0);
  const uint16_t* B = a.B + zoff(a.zB, z, a.zdiv) + (BK_ ? (int64_t)n0 * a.sBn : (int64_t)n0);
  int klim = a.K;
  if (a.causal == 2) klim = min(klim, m0 + GM);            // contraction k <= m only
  int kbeg = 0;
  if (a.causal == 3) kbeg = (m0 / GK) * GK;                 // contraction k >= m only
  const int rows_a = a.M - m0, rows_b = a.N - n0;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  f32x16_t acc[2] = {f32x16_t{}, f32x16_t{}};

  TileLoad<GM, AK> la;
  TileLoad<GN, BK_> lb;
  la.load(A, AK ? a.sAm : a.sAk, AK ? 1 : a.sAk, rows_a, kbeg, klim);
  lb.load(B, BK_ ? a.sBn : a.sBk, BK_ ? 1 : a.sBk, rows_b, kbeg, klim);
  la.store(sA[0]);
  lb.store(sB[0]);
  __syncthreads();
  const int nk = klim > kbeg ? (klim - kbeg + GK - 1) / GK : 0;
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
      for (int i = 0; i < 2; ++i) {
        const bf16x8_t afr = *reinterpret_cast<const bf16x8_t*>(&sA[cur][(wm * 64 + i * 32 + (lane & 31)) * GP + kk * 16 + (lane >> 5) * 8]);
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
  const int64_t cz = zoff(a.zC, z, a.zdiv);
  const int n = n0 + wn * 32 + (lane & 31);
  if (n >= a.N) return;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int m = m0 + wm * 64 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
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

}  // namespace

hipError_t launch_gemm_generic(const GemmArgs& a, hipStream_t s) {
  if (a.M <= 0 || a.N <= 0 || a.nz <= 0) return hipSuccess;
  const dim3 grid((a.M + GM - 1) / GM, (a.N + GN - 1) / GN, a.nz);
  const bool ak = a.sAk == 1, bk = a.sBk == 1;
  if (ak && bk) hipLaunchKernelGGL((k_gemm_generic<true, true>), grid, dim3(GT), 0, s, a);
  else if (ak) hipLaunchKernelGGL((k_gemm_generic<true, false>), grid, dim3(GT), 0, s, a);
  else if (bk) hipLaunchKernelGGL((k_gemm_generic<false, true>), grid, dim3(GT), 0, s, a);
  else hipLaunchKernelGGL((k_gemm_generic<false, false>), grid, dim3(GT), 0, s, a);
  return hipGetLastError();
}

}  // namespace lsq
