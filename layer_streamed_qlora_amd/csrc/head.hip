// Output head and loss (gfx950): softmax statistics over vocabulary slices, the SFT
// or DPO loss, and the logit gradient.
//
// Streaming bounds the weights, not the logits: the tool the pages describe keeps the
// whole logits tensor resident, 8.71 GB at batch 8 on a 152k vocabulary ("Soup CLI
// fine-tunes Llama-3.1-8B on a 4 GB laptop GPU ...", third and fifth paragraphs).
// Here the logits of one vocabulary slice at a time (a float32 [T, vs] product of the
// head slice held in a device slot) are folded into per-token running statistics:
// the maximum m_t, the sum s_t of exp(z - m_t), and the label's logit.  The loss needs
// only log p_t(label) = z_label - (m_t + log s_t); the backward recomputes each slice's
// logits and forms dz = g_t (onehot(label) - exp(z - lse_t)) with g_t = dL/dlog p_t.
//
// Every reduction has a fixed order (lane butterflies, a fixed tree, sequences in
// order), so results do not depend on scheduling.  Sums of log-probabilities over a
// sequence run in float64: DPO subtracts nearly equal policy and reference sums.
#include <math.h>

#include "lsq_internal.hpp"
#include "tiles.hpp"

namespace lsq {
namespace {

// (m, s) pairs: m the maximum, s the sum of exp(x - m); m = -inf means "empty"
struct Ms {
  float m, s;
};
__device__ __forceinline__ Ms merge(Ms a, Ms b) {
  if (b.m == -INFINITY) return a;
  if (a.m == -INFINITY) return b;
  const float mm = fmaxf(a.m, b.m);
  return {mm, a.s * expf(a.m - mm) + b.s * expf(b.m - mm)};
}
__device__ __forceinline__ Ms add1(Ms a, float x) { return merge(a, Ms{x, 1.f}); }

__device__ __forceinline__ bool labelled(int lab, int vocab) { return lab >= 0 && lab < vocab; }

// One wave per token: fold the slice's logits Z[t, 0 .. vs) (columns v0 + j of the
// vocabulary) into the running (m, s) and pick up the label's logit.
__global__ void __launch_bounds__(256) k_ce_stats(const float* __restrict__ Z, int32_t ldz, int32_t vs, int32_t v0,
                                                  const int32_t* __restrict__ labels, int32_t T, int32_t vocab,
                                                  float* run_m, float* run_s, float* zlab, int32_t first) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;   // whole wave
  const float* row = Z + (int64_t)t * ldz;
  Ms a{-INFINITY, 0.f};
  const int n4 = vs >> 2;
  for (int i = lane; i < n4; i += 64) {
    const float4 v = reinterpret_cast<const float4*>(row)[i];
    a = add1(add1(add1(add1(a, v.x), v.y), v.z), v.w);
  }
  for (int i = 4 * n4 + lane; i < vs; i += 64) a = add1(a, row[i]);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const Ms b{__shfl_xor(a.m, off), __shfl_xor(a.s, off)};
    a = merge(a, b);   // merge(a, b) and merge(b, a) agree bitwise, so every lane ends equal
  }
  if (lane == 0) {
    const Ms r = first ? a : merge(Ms{run_m[t], run_s[t]}, a);
    run_m[t] = r.m;
    run_s[t] = r.s;
    const int lab = labels[t];
    const bool here = labelled(lab, vocab) && lab >= v0 && lab < v0 + vs;
    if (here) zlab[t] = row[lab - v0];
    else if (first) zlab[t] = 0.f;
  }
}

constexpr int kFinThreads = 1024;

__device__ double block_sum(double v, double* red) {
  red[threadIdx.x] = v;
  __syncthreads();
  for (int w = kFinThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) red[threadIdx.x] += red[threadIdx.x + w];
    __syncthreads();
  }
  const double r = red[0];
  __syncthreads();
  return r;
}

// One workgroup: per-sequence log-prob sums (float64, fixed order), the loss, and the
// per-sequence coefficient g = dL/dlog p of the policy's labelled tokens.
__global__ void __launch_bounds__(kFinThreads) k_loss_finalize(
    int32_t kind, float beta, int32_t T, int32_t seq, int32_t vocab, const int32_t* __restrict__ labels,
    const float* pm, const float* ps, const float* pz, const float* rm, const float* rs, const float* rz,
    float* coef, float* out) {
  __shared__ double red[kFinThreads];
  __shared__ double pol[1024], ref[1024];   // nseq <= 1024 (checked on the host)
  const int nseq = T / seq;
  double total = 0.0;
  for (int b = 0; b < nseq; ++b) {
    double ap = 0.0, ar = 0.0, cnt = 0.0;
    for (int i = threadIdx.x; i < seq; i += kFinThreads) {
      const int t = b * seq + i;
      if (!labelled(labels[t], vocab)) continue;
      ap += (double)pz[t] - ((double)pm[t] + log((double)ps[t]));
      if (rm) ar += (double)rz[t] - ((double)rm[t] + log((double)rs[t]));
      cnt += 1.0;
    }
    const double sp = block_sum(ap, red);
    const double sr = block_sum(ar, red);
    const double sc = block_sum(cnt, red);
    if (threadIdx.x == 0) { pol[b] = sp; ref[b] = sr; }
    total += sc;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double loss = 0.0;
    if (kind == LS_LOSS_SFT) {
      double sum = 0.0;
      for (int b = 0; b < nseq; ++b) sum += pol[b];
      loss = total > 0 ? -sum / total : 0.0;
      for (int b = 0; b < nseq; ++b) coef[b] = total > 0 ? (float)(-1.0 / total) : 0.f;
    } else {
      const int P = nseq / 2;
      for (int i = 0; i < P; ++i) {
        const double mg = (double)beta * ((pol[2 * i] - ref[2 * i]) - (pol[2 * i + 1] - ref[2 * i + 1]));
        // -log sigmoid(mg) = softplus(-mg), and sigmoid(-mg), written to stay finite
        const double sp = mg > 0 ? log1p(exp(-mg)) : -mg + log1p(exp(mg));
        const double sg = mg > 0 ? exp(-mg) / (1.0 + exp(-mg)) : 1.0 / (1.0 + exp(mg));
        loss += sp;
        coef[2 * i] = (float)(-(double)beta * sg / P);
        coef[2 * i + 1] = (float)((double)beta * sg / P);
      }
      loss /= P;
    }
    out[0] = (float)loss;
    out[1] = (float)total;
    for (int b = 0; b < nseq; ++b) {
      out[2 + b] = (float)pol[b];
      out[2 + nseq + b] = (float)ref[b];
    }
  }
}

// dz[t, j] = g_t (onehot(label_t)[v0 + j] - exp(Z[t, j] - lse_t)) as bf16 (the operand
// of the product back to the hidden state); 4 columns per thread.
__global__ void __launch_bounds__(256) k_ce_grad(const float* __restrict__ Z, int32_t ldz, int32_t vs, int32_t v0,
                                                 const int32_t* __restrict__ labels, int32_t T, int32_t seq,
                                                 int32_t vocab, const float* __restrict__ run_m,
                                                 const float* __restrict__ run_s, const float* __restrict__ coef,
                                                 uint16_t* __restrict__ dz) {
  const int64_t nq = (vs + 3) / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= nq * T) return;
  const int t = (int)(idx / nq);
  const int j0 = (int)(idx - (int64_t)t * nq) * 4;
  const int lab = labels[t];
  const float g = labelled(lab, vocab) ? coef[t / seq] : 0.f;
  const float lse = run_m[t] + logf(run_s[t]);
  const float* row = Z + (int64_t)t * ldz;
  uint16_t* drow = dz + (int64_t)t * ldz;
  float d[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int j = j0 + e;
    d[e] = 0.f;
    if (j < vs && g != 0.f) d[e] = g * (((v0 + j) == lab ? 1.f : 0.f) - expf(row[j] - lse));
  }
  if (j0 + 4 <= vs) {
    *reinterpret_cast<uint2*>(drow + j0) = make_uint2(tiles::pack2(d[0], d[1]), tiles::pack2(d[2], d[3]));
  } else {
    for (int e = 0; e < 4 && j0 + e < vs; ++e) drow[j0 + e] = (uint16_t)(tiles::pack2(d[e], 0.f) & 0xFFFFu);
  }
}

}  // namespace

hipError_t launch_ce_stats(const float* Z, int32_t ldz, int32_t vs, int32_t v0, const int32_t* labels, int32_t T,
                           int32_t vocab, float* m, float* s, float* zlab, bool first, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  hipLaunchKernelGGL(k_ce_stats, dim3((T + 3) / 4), dim3(256), 0, st, Z, ldz, vs, v0, labels, T, vocab, m, s, zlab,
                     first ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_loss_finalize(int32_t kind, float beta, int32_t T, int32_t seq, int32_t vocab, const int32_t* labels,
                                const float* pm, const float* ps, const float* pz, const float* rm, const float* rs,
                                const float* rz, float* coef, float* out, hipStream_t st) {
  if (T <= 0 || seq <= 0 || T % seq != 0 || T / seq > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_loss_finalize, dim3(1), dim3(kFinThreads), 0, st, kind, beta, T, seq, vocab, labels, pm, ps, pz,
                     rm, rs, rz, coef, out);
  return hipGetLastError();
}

hipError_t launch_ce_grad(const float* Z, int32_t ldz, int32_t vs, int32_t v0, const int32_t* labels, int32_t T,
                          int32_t seq, int32_t vocab, const float* m, const float* s, const float* coef, uint16_t* dz,
                          hipStream_t st) {
  if (T <= 0 || vs <= 0) return hipSuccess;
  const int64_t n = (int64_t)T * ((vs + 3) / 4);
  hipLaunchKernelGGL(k_ce_grad, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, Z, ldz, vs, v0, labels, T, seq,
                     vocab, m, s, coef, dz);
  return hipGetLastError();
}

}  // namespace lsq
