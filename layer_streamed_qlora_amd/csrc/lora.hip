// LoRA adapter gradients over the tokens of a step, gfx950.
//
// For a projection y = x W^T + s (x A^T) B^T the adapter gradients are dB = dY^T (s H)
// and dA = (s G)^T X with H = x A^T and G = dY B ("Fine-Tuning an 8B Parameter Model on
// a 4 GB Laptop GPU", section "LoRA and QLoRA: Train a Fraction of the Parameters":
// only A and B are trained).  Each is a contraction over the T tokens of two
// token-major bf16 matrices: C[m][n] = sum_t A[t][m] B[t][n], with m a feature of the
// activation (up to 29568 of them) and n one of the r adapter columns.
//
// One launch computes several such products (one decoder stage's dA and dB).  A
// workgroup owns 128 features x 64 adapter columns and a run of tokens; 64-token tiles
// of both operands go to LDS transposed ([column][token], built with byte permutes from
// token pairs) and feed v_mfma_f32_32x32x16_bf16 with the contraction over tokens.  The
// token runs of one output tile write float32 partials that a second kernel adds in
// run order, so results do not depend on scheduling.
//
// The other two products of the adapters, H = s x A^T and G = s dY B, contract over the
// features of a token-major matrix ([T, K] against [N, K], N = r or a few stacked r):
// `k_lora_fc` takes 128 tokens x 64 columns per workgroup over a run of K, the same
// split and fixed-order sum, and writes bf16.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "lsq_internal.hpp"
#include "tiles.hpp"

namespace lsq {
namespace {

using namespace tiles;

constexpr int TM = 128, TN = 64, TT = kTileRows;
constexpr int NT = 256;

struct TcKArgs {
  TcArgs a;
  int32_t tile0[kMaxTcJobs + 1];
  int32_t n_tiles[kMaxTcJobs];
  int32_t ksplit = 1, chunk = 0;
};

// Destination of result element (thread t, block jb, register v) of a C tile at
// (m0, n0), or nullptr if it is not kept: C[i = feature][j = column] sits in lane
// j + 32 hh, register v holding feature 32 w + (v / 4) * 8 + 4 hh + v % 4.
__device__ __forceinline__ float* tc_dest(const TcJob& J, int m0, int n0, int t, int jb, int v) {
  const int lane = t & 63, w = t >> 6;
  const int m = m0 + 32 * w + (v >> 2) * 8 + 4 * (lane >> 5) + (v & 3);
  const int n = n0 + 32 * jb + (lane & 31);
  if (m >= J.M || n >= J.N) return nullptr;
  const int d = n / J.ncols, nl = n - d * J.ncols;
  if (nl >= J.nvalid || J.C[d] == nullptr) return nullptr;
  return J.C[d] + (int64_t)m * J.scm + (int64_t)nl * J.scn;
}
__device__ __forceinline__ void tc_put(float* c, float val, float beta) {
  *c = beta != 0.f ? val + beta * *c : val;
}

__global__ void __launch_bounds__(NT) k_lora_tc(TcKArgs k) {
  __shared__ __align__(16) uint16_t sA[TM * kTPitch];
  __shared__ __align__(16) uint16_t sB[TN * kTPitch];
  const TcArgs& a = k.a;
  const int flat = (int)blockIdx.x / k.ksplit, split = (int)blockIdx.x - flat * k.ksplit;
  int j = 0;
  while (j + 1 < a.n_jobs && flat >= k.tile0[j + 1]) ++j;
  const TcJob& J = a.job[j];
  const int local = flat - k.tile0[j];
  const int mt = local / k.n_tiles[j], nt = local - mt * k.n_tiles[j];
  const int m0 = mt * TM, n0 = nt * TN;
  const int t0 = split * k.chunk, t1 = min(a.T, t0 + k.chunk);
  // buffers based at (token t0, column m0 / n0): tokens past T read as zero
  const uint64_t rows = (uint64_t)(a.T - t0);
  const rsrc_t ra = make_rsrc(J.A + (int64_t)t0 * J.lda + m0, (rows * J.lda - m0) * 2);
  const rsrc_t rb = make_rsrc(J.B + (int64_t)t0 * J.ldb + n0, (rows * J.ldb - n0) * 2);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, hh = lane >> 5;
  const bool two = n0 + 32 < J.N;            // second 32-column block in use
  f32x16_t acc[2] = {f32x16_t{}, f32x16_t{}};
  TileMover<TM, NT> ta;
  TileMover<TN, NT> tb;
  const int nst = t1 > t0 ? (t1 - t0 + TT - 1) / TT : 0;
  if (nst > 0) {
    ta.load(ra, J.lda, 0);
    tb.load(rb, J.ldb, 0);
  }
  for (int st = 0; st < nst; ++st) {
    __syncthreads();                         // the previous tiles are no longer read
    ta.store_t(sA);
    tb.store_t(sB);
    __syncthreads();
    if (st + 1 < nst) {
      ta.load(ra, J.lda, (st + 1) * TT);
      tb.load(rb, J.ldb, (st + 1) * TT);
    }
#pragma unroll
    for (int s = 0; s < TT / 16; ++s) {
      const bf16x8_t af = tfrag(sA, 32 * w + l32, 16 * s, hh);
      acc[0] = mfma(af, tfrag(sB, l32, 16 * s, hh), acc[0]);
      if (two) acc[1] = mfma(af, tfrag(sB, 32 + l32, 16 * s, hh), acc[1]);
    }
  }
  if (k.ksplit == 1) {
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if (float* c = tc_dest(J, m0, n0, threadIdx.x, jb, v)) tc_put(c, acc[jb][v], a.beta);
    return;
  }
  float* part = a.partial + ((int64_t)flat * k.ksplit + split) * (TM * TN);
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int v = 0; v < 16; ++v)
      if (tc_dest(J, m0, n0, threadIdx.x, jb, v)) part[(jb * 16 + v) * NT + threadIdx.x] = acc[jb][v];
}

// Sum of the token runs of one result element, in run order: block b covers element
// slot e = b % 32 of tile b / 32 for all NT thread positions.
__global__ void __launch_bounds__(NT) k_lora_tc_reduce(TcKArgs k) {
  const TcArgs& a = k.a;
  const int flat = (int)blockIdx.x >> 5, e = (int)blockIdx.x & 31;
  int j = 0;
  while (j + 1 < a.n_jobs && flat >= k.tile0[j + 1]) ++j;
  const int local = flat - k.tile0[j];
  const int mt = local / k.n_tiles[j], nt = local - mt * k.n_tiles[j];
  float* c = tc_dest(a.job[j], mt * TM, nt * TN, threadIdx.x, e >> 4, e & 15);
  if (!c) return;
  const float* src = a.partial + (int64_t)flat * k.ksplit * (TM * TN) + e * NT + threadIdx.x;
  float sum = 0.f;
  for (int sp = 0; sp < k.ksplit; ++sp) sum += src[(int64_t)sp * (TM * TN)];
  tc_put(c, sum, a.beta);
}

// --------------------------------------------------------- feature contraction
constexpr int FM = 128, FN = 64, FK = 64, FP = FK + 8;   // tokens, columns, K step, LDS pitch

struct FcKArgs {
  FcArgs a;
  int32_t tile0[kMaxFcJobs + 1];
  int32_t n_tiles[kMaxFcJobs];
  int32_t m_tiles = 0;
  int32_t ksplit = 1, chunk = 0;
};

// 64 rows x 64 columns of a row-major bf16 matrix: 8 threads per row, 2 chunks each;
// columns at or past klim and rows past the buffer's range read as zero.
struct FcLoad {
  uint4 v[2];
  __device__ __forceinline__ void load(rsrc_t res, int ld, int row0, int col0, int klim) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = threadIdx.x + NT * i, row = q >> 3, cc = (q & 7) * 8;
      const bool ok = col0 + cc < klim;
      v[i] = bload16(res, ok ? ((uint32_t)(row0 + row) * (uint32_t)ld + (uint32_t)(col0 + cc)) * 2u : 0xFFFFFFF0u);
    }
  }
  __device__ __forceinline__ void store(uint16_t* s) const {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int q = threadIdx.x + NT * i, row = q >> 3, cc = (q & 7) * 8;
      *reinterpret_cast<uint4*>(s + row * FP + cc) = v[i];
    }
  }
};

// Destination column / token of result element (thread t, block jb, register v) of a
// C tile at (t0, n0): C[i = token][j = column], lane j + 32 hh, register v holding
// token 32 w + (v / 4) * 8 + 4 hh + v % 4.  Returns false if outside the job.
__device__ __forceinline__ bool fc_pos(const FcJob& J, int T, int t0, int n0, int t, int jb, int v, int& tok, int& col) {
  const int lane = t & 63, w = t >> 6;
  tok = t0 + 32 * w + (v >> 2) * 8 + 4 * (lane >> 5) + (v & 3);
  col = n0 + 32 * jb + (lane & 31);
  return tok < T && col < J.N;
}

__global__ void __launch_bounds__(NT) k_lora_fc(FcKArgs k) {
  __shared__ __align__(16) uint16_t sA[FM * FP];
  __shared__ __align__(16) uint16_t sB[FN * FP];
  const FcArgs& a = k.a;
  const int flat = (int)blockIdx.x / k.ksplit, split = (int)blockIdx.x - flat * k.ksplit;
  int j = 0;
  while (j + 1 < a.n_jobs && flat >= k.tile0[j + 1]) ++j;
  const FcJob& J = a.job[j];
  const int local = flat - k.tile0[j];
  const int mt = local / k.n_tiles[j], nt = local - mt * k.n_tiles[j];
  const int t0 = mt * FM, n0 = nt * FN;
  const int kb = split * k.chunk, ke = min(J.K, kb + k.chunk);
  const rsrc_t rx = make_rsrc(J.X + (int64_t)t0 * J.ldx, ((uint64_t)(a.T - t0) * J.ldx) * 2);
  const rsrc_t rw = make_rsrc(J.W + (int64_t)n0 * J.K, ((uint64_t)(J.N - n0) * J.K) * 2);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l32 = lane & 31, hh = lane >> 5;
  const bool two = n0 + 32 < J.N;
  f32x16_t acc[2] = {f32x16_t{}, f32x16_t{}};
  FcLoad la0, la1, lb;
  const int nst = ke > kb ? (ke - kb + FK - 1) / FK : 0;
  if (nst > 0) {
    la0.load(rx, J.ldx, 0, kb, ke);
    la1.load(rx, J.ldx, 64, kb, ke);
    lb.load(rw, J.K, 0, kb, ke);
  }
  for (int st = 0; st < nst; ++st) {
    __syncthreads();
    la0.store(sA);
    la1.store(sA + 64 * FP);
    lb.store(sB);
    __syncthreads();
    if (st + 1 < nst) {
      const int kk = kb + (st + 1) * FK;
      la0.load(rx, J.ldx, 0, kk, ke);
      la1.load(rx, J.ldx, 64, kk, ke);
      lb.load(rw, J.K, 0, kk, ke);
    }
#pragma unroll
    for (int s = 0; s < FK / 16; ++s) {
      const bf16x8_t af = *reinterpret_cast<const bf16x8_t*>(sA + (32 * w + l32) * FP + 16 * s + 8 * hh);
      acc[0] = mfma(af, *reinterpret_cast<const bf16x8_t*>(sB + l32 * FP + 16 * s + 8 * hh), acc[0]);
      if (two) acc[1] = mfma(af, *reinterpret_cast<const bf16x8_t*>(sB + (32 + l32) * FP + 16 * s + 8 * hh), acc[1]);
    }
  }
  if (k.ksplit == 1) {
#pragma unroll
    for (int jb = 0; jb < 2; ++jb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        int tok, col;
        if (fc_pos(J, a.T, t0, n0, threadIdx.x, jb, v, tok, col))
          J.out[(int64_t)tok * J.ldo + col] = (uint16_t)(pack2(J.alpha * acc[jb][v], 0.f) & 0xFFFFu);
      }
    return;
  }
  float* part = a.partial + ((int64_t)flat * k.ksplit + split) * (FM * FN);
#pragma unroll
  for (int jb = 0; jb < 2; ++jb)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      int tok, col;
      if (fc_pos(J, a.T, t0, n0, threadIdx.x, jb, v, tok, col)) part[(jb * 16 + v) * NT + threadIdx.x] = acc[jb][v];
    }
}

__global__ void __launch_bounds__(NT) k_lora_fc_reduce(FcKArgs k) {
  const FcArgs& a = k.a;
  const int flat = (int)blockIdx.x >> 5, e = (int)blockIdx.x & 31;
  int j = 0;
  while (j + 1 < a.n_jobs && flat >= k.tile0[j + 1]) ++j;
  const FcJob& J = a.job[j];
  const int local = flat - k.tile0[j];
  const int mt = local / k.n_tiles[j], nt = local - mt * k.n_tiles[j];
  int tok, col;
  if (!fc_pos(J, a.T, mt * FM, nt * FN, threadIdx.x, e >> 4, e & 15, tok, col)) return;
  const float* src = a.partial + (int64_t)flat * k.ksplit * (FM * FN) + e * NT + threadIdx.x;
  float sum = 0.f;
  for (int sp = 0; sp < k.ksplit; ++sp) sum += src[(int64_t)sp * (FM * FN)];
  J.out[(int64_t)tok * J.ldo + col] = (uint16_t)(pack2(J.alpha * sum, 0.f) & 0xFFFFu);
}

}  // namespace

hipError_t launch_lora_tc(const TcArgs& a, hipStream_t s) {
  if (a.T <= 0 || a.n_jobs <= 0) return hipSuccess;
  if (a.n_jobs > kMaxTcJobs) return hipErrorInvalidValue;
  TcKArgs k;
  k.a = a;
  int tiles = 0;
  int64_t max_ld = 1;
  for (int j = 0; j < a.n_jobs; ++j) {
    const TcJob& J = a.job[j];
    if (!J.A || !J.B || J.M <= 0 || J.N <= 0 || J.ncols <= 0 || J.N > 3 * J.ncols || J.lda % 8 || J.ldb % 8 ||
        J.lda < J.M || J.ldb < J.N || (reinterpret_cast<uintptr_t>(J.A) & 15) || (reinterpret_cast<uintptr_t>(J.B) & 15))
      return hipErrorInvalidValue;
    k.tile0[j] = tiles;
    k.n_tiles[j] = (J.N + TN - 1) / TN;
    tiles += (J.M + TM - 1) / TM * k.n_tiles[j];
    max_ld = std::max<int64_t>(max_ld, std::max(J.lda, J.ldb));
  }
  k.tile0[a.n_jobs] = tiles;
  // token runs: about 1024 workgroups, within the partial buffer
  int ks = std::max(1, std::min(32, 1024 / std::max(1, tiles)));
  ks = std::min(ks, (a.T + TT - 1) / TT);
  while (ks > 1 && (int64_t)tiles * ks * TM * TN > a.partial_floats) --ks;
  if (!a.partial) ks = 1;
  k.chunk = ((a.T + ks - 1) / ks + TT - 1) / TT * TT;
  k.ksplit = (a.T + k.chunk - 1) / k.chunk;
  if ((int64_t)(std::min(a.T, k.chunk) + TT) * max_ld * 2 >= (int64_t)1 << 31) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_lora_tc, dim3((unsigned)(tiles * k.ksplit)), dim3(NT), 0, s, k);
  if (k.ksplit > 1) hipLaunchKernelGGL(k_lora_tc_reduce, dim3((unsigned)(tiles * 32)), dim3(NT), 0, s, k);
  return hipGetLastError();
}

}  // namespace lsq

namespace lsq {

hipError_t launch_lora_fc(const FcArgs& a, hipStream_t s) {
  if (a.T <= 0 || a.n_jobs <= 0) return hipSuccess;
  if (a.n_jobs > kMaxFcJobs) return hipErrorInvalidValue;
  FcKArgs k;
  k.a = a;
  k.m_tiles = (a.T + FM - 1) / FM;
  int tiles = 0, kmax = 0;
  int64_t max_ld = 1;
  for (int j = 0; j < a.n_jobs; ++j) {
    const FcJob& J = a.job[j];
    if (!J.X || !J.W || !J.out || J.K <= 0 || J.N <= 0 || J.K % 8 || J.ldx % 8 || J.ldx < J.K ||
        (reinterpret_cast<uintptr_t>(J.X) & 15) || (reinterpret_cast<uintptr_t>(J.W) & 15))
      return hipErrorInvalidValue;
    k.tile0[j] = tiles;
    k.n_tiles[j] = (J.N + FN - 1) / FN;
    tiles += k.m_tiles * k.n_tiles[j];
    kmax = std::max(kmax, J.K);
    max_ld = std::max<int64_t>(max_ld, std::max<int64_t>(J.ldx, J.K));
  }
  k.tile0[a.n_jobs] = tiles;
  if ((int64_t)(a.T + FM) * max_ld * 2 >= (int64_t)1 << 31) return hipErrorInvalidValue;
  // K runs: about 1024 workgroups, at least two K steps each, within the partial buffer
  int ks = std::max(1, std::min(64, 1024 / std::max(1, tiles)));
  ks = std::min(ks, std::max(1, kmax / (2 * FK)));
  while (ks > 1 && (int64_t)tiles * ks * FM * FN > a.partial_floats) --ks;
  if (!a.partial) ks = 1;
  k.chunk = ((kmax + ks - 1) / ks + FK - 1) / FK * FK;
  k.ksplit = (kmax + k.chunk - 1) / k.chunk;
  hipLaunchKernelGGL(k_lora_fc, dim3((unsigned)(tiles * k.ksplit)), dim3(NT), 0, s, k);
  if (k.ksplit > 1) hipLaunchKernelGGL(k_lora_fc_reduce, dim3((unsigned)(tiles * 32)), dim3(NT), 0, s, k);
  return hipGetLastError();
}

}  // namespace lsq
