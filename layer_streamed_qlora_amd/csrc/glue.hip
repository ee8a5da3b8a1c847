// Decoder glue around the projections: RMSNorm, rotary embedding,
// SwiGLU (forward and backward) and small layout conversions of the LoRA operands.
// All of it is HBM-bound elementwise / row-wise work: one pass over its operands,
// float32 arithmetic, bf16 in and out.
//
// The layer is the Llama-style pre-norm decoder of the families the pages list (the
// lachieslifestyle.com Soup how-to, section "Step 5: Enable 4-bit layer streaming").
// RMSNorm: y = x g / sqrt(mean(x^2) + eps).  Rotary embedding in the rotate-half
// form, angle pos * theta^(-2i/hd) taken from a host-computed table.  silu(z) =
// z / (1 + exp(-z)).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsq_internal.hpp"
#include "rope.hpp"

namespace lsq {
namespace {

typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf(uint16_t h) { return __builtin_bit_cast(float, (uint32_t)h << 16); }
__device__ __forceinline__ uint16_t tobf(float x) {
  f32x2_t v = {x, 0.f};
  return (uint16_t)(__builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t)) & 0xFFFFu);
}

template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  __syncthreads();
  if (l == 0) red[w] = v;
  __syncthreads();
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) s += red[i];
  return s;
}

template <class T> __device__ __forceinline__ float ld(const T* p, int64_t i);
template <> __device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) { return bf(p[i]); }
template <> __device__ __forceinline__ float ld<float>(const float* p, int64_t i) { return p[i]; }

// one 256-thread block per row
template <class XT>
__global__ void __launch_bounds__(256) k_rmsnorm_fwd(const XT* x, const uint16_t* g, uint16_t* y, float* rstd,
                                                     int D, float eps) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const XT* xr = x + row * D;
  float ss = 0.f;
  for (int i = threadIdx.x; i < D; i += 256) { const float v = ld(xr, i); ss += v * v; }
  ss = block_sum<256>(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
  if (threadIdx.x == 0 && rstd) rstd[row] = r;
  uint16_t* yr = y + row * D;
  for (int i = threadIdx.x; i < D; i += 256) yr[i] = tobf(ld(xr, i) * r * bf(g[i]));
}

// dx = dres + r g dn - (r^3 / D) x sum(dn g x)
template <class XT>
__global__ void __launch_bounds__(256) k_rmsnorm_bwd(const float* dn, const XT* x, const uint16_t* g,
                                                     const float* rstd, const float* dres32, const uint16_t* dres16,
                                                     float* dx32, uint16_t* dx16, int D) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const float* dnr = dn + row * D;
  const XT* xr = x + row * D;
  float s = 0.f;
  for (int i = threadIdx.x; i < D; i += 256) s += dnr[i] * bf(g[i]) * ld(xr, i);
  s = block_sum<256>(s, red);
  const float r = rstd[row];
  const float c = r * r * r / (float)D * s;
  for (int i = threadIdx.x; i < D; i += 256) {
    float v = r * bf(g[i]) * dnr[i] - c * ld(xr, i);
    if (dres32) v += dres32[row * D + i];
    else if (dres16) v += bf(dres16[row * D + i]);
    if (dx32) dx32[row * D + i] = v;
    if (dx16) dx16[row * D + i] = tobf(v);
  }
}

// Row-in-registers forms of the two kernels above for rows of at most 8192 elements
// (D % 8 == 0): 16-byte accesses, 8 consecutive elements per thread per chunk, one read
// of every operand.
constexpr int kRowChunks = 4;

__device__ __forceinline__ void ld8(const uint16_t* p, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    v[2 * j] = __builtin_bit_cast(float, w[j] << 16);
    v[2 * j + 1] = __builtin_bit_cast(float, w[j] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void ld8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void st8(uint16_t* p, const float (&v)[8]) {
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    f32x2_t t = {v[2 * j], v[2 * j + 1]};
    w[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(t, bf16x2_t));
  }
  *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
}
__device__ __forceinline__ void st8(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}

template <class XT>
__global__ void __launch_bounds__(256) k_rmsnorm_fwd_v(const XT* x, const uint16_t* g, uint16_t* y, float* rstd,
                                                       int D, float eps) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const XT* xr = x + row * D;
  float xv[kRowChunks][8];
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kRowChunks; ++c) {
    const int i0 = (c * 256 + threadIdx.x) * 8;
    if (i0 < D) {
      ld8(xr + i0, xv[c]);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss += xv[c][e] * xv[c][e];
    }
  }
  ss = block_sum<256>(ss, red);
  const float r = 1.0f / sqrtf(ss / (float)D + eps);
  if (threadIdx.x == 0 && rstd) rstd[row] = r;
#pragma unroll
  for (int c = 0; c < kRowChunks; ++c) {
    const int i0 = (c * 256 + threadIdx.x) * 8;
    if (i0 < D) {
      float gv[8], o[8];
      ld8(g + i0, gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] = xv[c][e] * r * gv[e];
      st8(y + row * D + i0, o);
    }
  }
}

template <class XT>
__global__ void __launch_bounds__(256) k_rmsnorm_bwd_v(const float* dn, const XT* x, const uint16_t* g,
                                                       const float* rstd, const float* dres32, const uint16_t* dres16,
                                                       float* dx32, uint16_t* dx16, int D) {
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  float dv[kRowChunks][8], xv[kRowChunks][8];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kRowChunks; ++c) {
    const int i0 = (c * 256 + threadIdx.x) * 8;
    if (i0 < D) {
      float gv[8];
      ld8(dn + row * D + i0, dv[c]);
      ld8(x + row * D + i0, xv[c]);
      ld8(g + i0, gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) s += dv[c][e] * gv[e] * xv[c][e];
    }
  }
  s = block_sum<256>(s, red);
  const float r = rstd[row];
  const float cc = r * r * r / (float)D * s;
#pragma unroll
  for (int c = 0; c < kRowChunks; ++c) {
    const int i0 = (c * 256 + threadIdx.x) * 8;
    if (i0 < D) {
      float gv[8], v[8], rv[8];
      ld8(g + i0, gv);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = r * gv[e] * dv[c][e] - cc * xv[c][e];
      if (dres32) {
        ld8(dres32 + row * D + i0, rv);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += rv[e];
      } else if (dres16) {
        ld8(dres16 + row * D + i0, rv);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[e] += rv[e];
      }
      if (dx32) st8(dx32 + row * D + i0, v);
      if (dx16) st8(dx16 + row * D + i0, v);
    }
  }
}

// float32 -> bf16 with the inverse rotation on the first nh heads of each row's first
// `width` columns (row stride ld); one thread per (token, column pair or lone column)
__global__ void k_rope_bwd_convert(const float* src, uint16_t* dst, int ld, int width, int64_t T, int seq, int nh,
                                   int hd, const float2* tab, const float* add, int add_col0, int add_ld) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int half = hd / 2;
  const int rope_pairs = nh * half;                    // rotated column pairs per row
  const int rest = width - nh * hd;                     // plain columns per row
  const int per_row = rope_pairs + rest;
  if (idx >= T * per_row) return;
  const int64_t t = idx / per_row;
  const int c = (int)(idx % per_row);
  const float* s = src + t * ld;
  uint16_t* d = dst + t * ld;
  auto rd = [&](int col) {     // the row's value, plus the addend's when col >= add_col0
    float v = s[col];
    if (add && col >= add_col0) v += add[t * add_ld + (col - add_col0)];
    return v;
  };
  if (c < rope_pairs) {
    const int h = c / half, i = c % half;
    const int col = h * hd + i;
    const float2 cs = tab[(int64_t)(t % seq) * half + i];
    const float2 g = rope_inverse(rd(col), rd(col + half), cs);
    d[col] = tobf(g.x);
    d[col + half] = tobf(g.y);
  } else {
    const int col = nh * hd + (c - rope_pairs);
    d[col] = tobf(rd(col));
  }
}

// Same, 4 rotated column pairs or 8 plain columns per thread (hd % 8 == 0, ld % 8 == 0)
__global__ void k_rope_bwd_convert_v(const float* src, uint16_t* dst, int ld, int width, int64_t T, int seq, int nh,
                                     int hd, const float2* tab, const float* add, int add_col0, int add_ld) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int half = hd / 2, gp = half / 4;
  const int rope_groups = nh * gp;
  const int per_row = rope_groups + (width - nh * hd) / 8;
  if (idx >= T * per_row) return;
  const int64_t t = idx / per_row;
  const int c = (int)(idx % per_row);
  const float* sr = src + t * ld;
  uint16_t* dr = dst + t * ld;
  // 4 consecutive float32 of the row at col, plus the addend's when col >= add_col0
  auto rd4 = [&](int col) {
    float4 v = *reinterpret_cast<const float4*>(sr + col);
    if (add && col >= add_col0) {
      const float4 w = *reinterpret_cast<const float4*>(add + t * add_ld + (col - add_col0));
      v.x += w.x; v.y += w.y; v.z += w.z; v.w += w.w;
    }
    return v;
  };
  if (c < rope_groups) {
    const int h = c / gp, i = (c % gp) * 4;
    const int col = h * hd + i;
    const float4 d1 = rd4(col);
    const float4 d2 = rd4(col + half);
    const float4* tp = reinterpret_cast<const float4*>(tab + (int64_t)(t % seq) * half + i);
    const float4 c01 = tp[0], c23 = tp[1];                 // (cos, sin) of pairs i .. i+3
    const float a1[4] = {d1.x, d1.y, d1.z, d1.w}, a2[4] = {d2.x, d2.y, d2.z, d2.w};
    const float cs[4] = {c01.x, c01.z, c23.x, c23.z}, sn[4] = {c01.y, c01.w, c23.y, c23.w};
    uint32_t o1[2], o2[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const float2 g0 = rope_inverse(a1[2 * j], a2[2 * j], make_float2(cs[2 * j], sn[2 * j]));
      const float2 g1 = rope_inverse(a1[2 * j + 1], a2[2 * j + 1], make_float2(cs[2 * j + 1], sn[2 * j + 1]));
      f32x2_t u = {g0.x, g1.x};
      f32x2_t v = {g0.y, g1.y};
      o1[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(u, bf16x2_t));
      o2[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
    }
    *reinterpret_cast<uint2*>(dr + col) = make_uint2(o1[0], o1[1]);
    *reinterpret_cast<uint2*>(dr + col + half) = make_uint2(o2[0], o2[1]);
  } else {
    const int col = nh * hd + (c - rope_groups) * 8;
    const float4 a = rd4(col), b = rd4(col + 4);
    f32x2_t p0 = {a.x, a.y}, p1 = {a.z, a.w}, p2 = {b.x, b.y}, p3 = {b.z, b.w};
    *reinterpret_cast<uint4*>(dr + col) = make_uint4(__builtin_bit_cast(uint32_t, __builtin_convertvector(p0, bf16x2_t)),
                                                     __builtin_bit_cast(uint32_t, __builtin_convertvector(p1, bf16x2_t)),
                                                     __builtin_bit_cast(uint32_t, __builtin_convertvector(p2, bf16x2_t)),
                                                     __builtin_bit_cast(uint32_t, __builtin_convertvector(p3, bf16x2_t)));
  }
}

// x in place; one thread per (token, head, i < hd/2); tab = [seq][hd/2] (cos, sin)
__global__ void k_rope(uint16_t* qk, int ld, int64_t n, int seq, int nh, int hd, const float2* tab, int inverse) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int half = hd / 2;
  const int i = (int)(idx % half);
  const int64_t th = idx / half;
  const int h = (int)(th % nh);
  const int64_t t = th / nh;
  const int pos = (int)(t % seq);
  const float2 cs = tab[(int64_t)pos * half + i];
  uint16_t* p = qk + t * ld + (int64_t)h * hd;
  const float x1 = bf(p[i]), x2 = bf(p[i + half]);
  float y1, y2;
  if (!inverse) { y1 = x1 * cs.x - x2 * cs.y; y2 = x2 * cs.x + x1 * cs.y; }
  else { y1 = x1 * cs.x + x2 * cs.y; y2 = x2 * cs.x - x1 * cs.y; }
  p[i] = tobf(y1);
  p[i + half] = tobf(y2);
}

__device__ __forceinline__ float sigmoidf(float z) { return 1.0f / (1.0f + __expf(-z)); }

__global__ void k_swiglu_fwd(const float* gu, int I, uint16_t* act, int64_t n) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= n) return;
  const int64_t t = idx / I;
  const int j = (int)(idx % I);
  const float g = gu[t * 2 * I + j], u = gu[t * 2 * I + I + j];
  act[t * I + j] = tobf(g * sigmoidf(g) * u);
}

// dst[r, c] = scale * src[r, c] (transpose: dst[c, r]) for c < cols, 0 for cols <= c < pad_cols
__global__ void k_f32_to_bf16(const float* src, int64_t lds, uint16_t* dst, int64_t ldd, int rows, int cols,
                              int pad_cols, float scale, int transpose) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (int64_t)rows * pad_cols) return;
  const int r = (int)(idx / pad_cols), c = (int)(idx % pad_cols);
  const uint16_t v = c < cols ? tobf(scale * src[(int64_t)r * lds + c]) : (uint16_t)0;
  if (transpose) dst[(int64_t)c * ldd + r] = v;
  else dst[(int64_t)r * ldd + c] = v;
}

// grid.y = job; grid-stride over the job's elements
__global__ void k_convert_batch(ConvBatch b) {
  const ConvJob& j = b.job[blockIdx.y];
  const int64_t n = (int64_t)j.rows * j.pad_cols;
  for (int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < n; idx += (int64_t)gridDim.x * blockDim.x) {
    const int r = (int)(idx / j.pad_cols), c = (int)(idx % j.pad_cols);
    const uint16_t v = c < j.cols ? tobf(j.scale * j.src[(int64_t)r * j.lds + c]) : (uint16_t)0;
    if (j.transpose) j.dst[(int64_t)c * j.ldd + r] = v;
    else j.dst[(int64_t)r * j.ldd + c] = v;
  }
}

__global__ void k_fill_f32(float* p, int64_t n, float v) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < n) p[idx] = v;
}

__global__ void k_fill_u32(uint32_t* p, int64_t n, uint32_t v) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx < n) p[idx] = v;
}

}  // namespace

static inline unsigned blocks_for(int64_t n, int t) { return (unsigned)((n + t - 1) / t); }

hipError_t launch_rmsnorm_fwd(const uint16_t* x16, const float* x32, const uint16_t* g, uint16_t* y, float* rstd,
                              int32_t T, int32_t D, float eps, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const bool v = D % 8 == 0 && D <= 256 * 8 * kRowChunks;
  if (x32) {
    if (v) hipLaunchKernelGGL(k_rmsnorm_fwd_v<float>, dim3(T), dim3(256), 0, s, x32, g, y, rstd, D, eps);
    else hipLaunchKernelGGL(k_rmsnorm_fwd<float>, dim3(T), dim3(256), 0, s, x32, g, y, rstd, D, eps);
  } else {
    if (v) hipLaunchKernelGGL(k_rmsnorm_fwd_v<uint16_t>, dim3(T), dim3(256), 0, s, x16, g, y, rstd, D, eps);
    else hipLaunchKernelGGL(k_rmsnorm_fwd<uint16_t>, dim3(T), dim3(256), 0, s, x16, g, y, rstd, D, eps);
  }
  return hipGetLastError();
}

hipError_t launch_rmsnorm_bwd(const float* dn, const uint16_t* x16, const float* x32, const uint16_t* g,
                              const float* rstd, const float* dres32, const uint16_t* dres16, float* dx32,
                              uint16_t* dx16, int32_t T, int32_t D, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  const bool v = D % 8 == 0 && D <= 256 * 8 * kRowChunks;
  if (x32) {
    if (v) hipLaunchKernelGGL(k_rmsnorm_bwd_v<float>, dim3(T), dim3(256), 0, s, dn, x32, g, rstd, dres32, dres16, dx32, dx16, D);
    else hipLaunchKernelGGL(k_rmsnorm_bwd<float>, dim3(T), dim3(256), 0, s, dn, x32, g, rstd, dres32, dres16, dx32, dx16, D);
  } else {
    if (v) hipLaunchKernelGGL(k_rmsnorm_bwd_v<uint16_t>, dim3(T), dim3(256), 0, s, dn, x16, g, rstd, dres32, dres16, dx32, dx16, D);
    else hipLaunchKernelGGL(k_rmsnorm_bwd<uint16_t>, dim3(T), dim3(256), 0, s, dn, x16, g, rstd, dres32, dres16, dx32, dx16, D);
  }
  return hipGetLastError();
}

hipError_t launch_rope_bwd_convert(const float* src, uint16_t* dst, int32_t ld, int32_t width, int32_t T, int32_t seq,
                                   int32_t nh, int32_t hd, const float2* tab, hipStream_t s, const float* add,
                                   int32_t add_col0, int32_t add_ld) {
  if (width < nh * hd || width > ld) return hipErrorInvalidValue;
  if (add && (add_col0 < 0 || add_col0 > width || add_ld < width - add_col0)) return hipErrorInvalidValue;
  if (hd % 8 == 0 && ld % 8 == 0 && (width - nh * hd) % 8 == 0 && (reinterpret_cast<uintptr_t>(src) & 15) == 0 &&
      (reinterpret_cast<uintptr_t>(dst) & 15) == 0 &&
      (!add || (add_col0 % 4 == 0 && add_ld % 4 == 0 && (reinterpret_cast<uintptr_t>(add) & 15) == 0))) {
    const int64_t n = (int64_t)T * ((int64_t)nh * (hd / 8) + (width - nh * hd) / 8);
    if (n <= 0) return hipSuccess;
    hipLaunchKernelGGL(k_rope_bwd_convert_v, dim3(blocks_for(n, 256)), dim3(256), 0, s, src, dst, ld, width, (int64_t)T,
                       seq, nh, hd, tab, add, add_col0, add_ld);
    return hipGetLastError();
  }
  const int64_t per_row = (int64_t)nh * (hd / 2) + (width - nh * hd);
  const int64_t n = (int64_t)T * per_row;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rope_bwd_convert, dim3(blocks_for(n, 256)), dim3(256), 0, s, src, dst, ld, width, (int64_t)T, seq,
                     nh, hd, tab, add, add_col0, add_ld);
  return hipGetLastError();
}

hipError_t launch_rope_tab(uint16_t* qk, int32_t ld, int32_t T, int32_t seq, int32_t nh, int32_t hd, const float2* tab,
                           int32_t inverse, hipStream_t s) {
  const int64_t n = (int64_t)T * nh * (hd / 2);
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_rope, dim3(blocks_for(n, 256)), dim3(256), 0, s, qk, ld, n, seq, nh, hd, tab, inverse);
  return hipGetLastError();
}

hipError_t launch_swiglu_fwd(const float* gu, int32_t I, uint16_t* act, int32_t T, hipStream_t s) {
  const int64_t n = (int64_t)T * I;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_swiglu_fwd, dim3(blocks_for(n, 256)), dim3(256), 0, s, gu, I, act, n);
  return hipGetLastError();
}

hipError_t launch_f32_to_bf16(const float* src, int64_t lds, uint16_t* dst, int64_t ldd, int32_t rows, int32_t cols,
                              int32_t pad_cols, float scale, int32_t transpose, hipStream_t s) {
  const int64_t n = (int64_t)rows * pad_cols;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_f32_to_bf16, dim3(blocks_for(n, 256)), dim3(256), 0, s, src, lds, dst, ldd, rows, cols, pad_cols,
                     scale, transpose);
  return hipGetLastError();
}

hipError_t launch_convert_batch(const ConvBatch& b, hipStream_t s) {
  if (b.n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_convert_batch, dim3(64, b.n), dim3(256), 0, s, b);
  return hipGetLastError();
}

hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_f32, dim3(blocks_for(n, 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_fill_u32, dim3(blocks_for(n, 256)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace lsq
