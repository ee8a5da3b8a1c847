// AdamW update of the trainable adapters (gfx950).
//
// Only the low-rank adapters train; Adam keeps two float32 moments per trained value
// ("Fine-Tuning an 8B Parameter Model on a 4 GB Laptop GPU", sections "LoRA and
// QLoRA: Train a Fraction of the Parameters" and the "Optimizer states" item of why
// training is memory-hungry).  The update is AdamW with learning-rate-scaled
// decoupled decay; per element, in float32:
//     p <- p (1 - lr wd);  m <- beta1 m + (1 - beta1) g;  v <- beta2 v + (1 - beta2) g^2
//     p <- p - step_size m / (sqrt(v) / sqrt(1 - beta2^t) + eps),  step_size = lr / (1 - beta1^t)
//
// Pure streaming: 16 bytes read and 12 written per element, no reuse, so the bound is
// HBM bandwidth.  Every adapter tensor of every layer goes through one launch: the
// host splits the tensors into chunks of at most kAdamChunk elements (a table in
// device memory), one workgroup per chunk, 16-byte accesses where every pointer of
// the chunk is 16-byte aligned.
#include "lsq_internal.hpp"

namespace lsq {
namespace {

constexpr int kAdamThreads = 256;

__device__ __forceinline__ void adam1(float& p, float g, float& m, float& v, const AdamHyper& h) {
  p *= h.decay_mul;
  m = h.beta1 * m + h.one_m_beta1 * g;
  v = h.beta2 * v + h.one_m_beta2 * (g * g);
  const float denom = sqrtf(v) * h.inv_bc2_sqrt + h.eps;
  p -= h.step_size * (m / denom);
}

__global__ void __launch_bounds__(kAdamThreads) k_adamw(const AdamChunk* __restrict__ chunks, AdamHyper h) {
  const AdamChunk c = chunks[blockIdx.x];
  if (c.vec4) {
    float4* p4 = reinterpret_cast<float4*>(c.p);
    const float4* g4 = reinterpret_cast<const float4*>(c.g);
    float4* m4 = reinterpret_cast<float4*>(c.m);
    float4* v4 = reinterpret_cast<float4*>(c.v);
    const uint32_t n4 = c.n / 4;
    for (uint32_t i = threadIdx.x; i < n4; i += kAdamThreads) {
      float4 p = p4[i], m = m4[i], v = v4[i];
      const float4 g = g4[i];
      adam1(p.x, g.x, m.x, v.x, h);
      adam1(p.y, g.y, m.y, v.y, h);
      adam1(p.z, g.z, m.z, v.z, h);
      adam1(p.w, g.w, m.w, v.w, h);
      p4[i] = p;
      m4[i] = m;
      v4[i] = v;
    }
  } else {
    for (uint32_t i = threadIdx.x; i < c.n; i += kAdamThreads) {
      float p = c.p[i], m = c.m[i], v = c.v[i];
      adam1(p, c.g[i], m, v, h);
      c.p[i] = p;
      c.m[i] = m;
      c.v[i] = v;
    }
  }
}

}  // namespace

hipError_t launch_adamw(const AdamChunk* chunks, int32_t n_chunks, const AdamHyper& h, hipStream_t s) {
  if (n_chunks <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_adamw, dim3(n_chunks), dim3(kAdamThreads), 0, s, chunks, h);
  return hipGetLastError();
}

}  // namespace lsq
