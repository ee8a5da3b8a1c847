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
// `k_lora_fc` takes 16 tokens x up to 64 columns per workgroup over all of K, its
// sixteen waves on sixteenths of K added in a fixed order, and writes bf16.
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
// v_mfma_f32_16x16x32_bf16: A[i][k] in lane i + 16 (k / 8), element k % 8; B[k][j] in
// lane j + 16 (k / 8); C[i][j] in lane j + 16 (i / 4), register i % 4.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
constexpr int FT = 16;     // tokens per workgroup
constexpr int FN = 64;     // columns per workgroup at most (4 blocks of 16)
constexpr int FW = 16;     // waves per workgroup, each on 1/FW of K

struct FcKArgs {
  FcArgs a;
  int32_t tile0[kMaxFcJobs + 1];
  int32_t n_tiles[kMaxFcJobs];
};

// Workgroup: 16 tokens x NB blocks of 16 columns over the whole of K.  Each of its FW
// waves streams a contiguous 1/FW of K straight into MFMA operand registers (16 bytes
// per lane per step, FU steps in flight); the partial products are added in LDS in
// wave order.  NB is the launch's widest job in 16-column blocks (a narrower job's
// extra blocks read zeros).
template <int NB>
__global__ void __launch_bounds__(FW * 64) k_lora_fc(FcKArgs k) {
  constexpr int FU = NB == 1 ? 8 : 4;   // 32-wide K steps in flight per wave
  __shared__ __align__(16) f32x4_t red[FW][NB][64];    // [wave][column block][lane]
  const FcArgs& a = k.a;
  const int flat = blockIdx.x;
  int j = 0;
  while (j + 1 < a.n_jobs && flat >= k.tile0[j + 1]) ++j;
  const FcJob& J = a.job[j];
  const int local = flat - k.tile0[j];
  const int mt = local / k.n_tiles[j], nt = local - mt * k.n_tiles[j];
  const int t0 = mt * FT, n0 = nt * (16 * NB);
  const int nb_used = min(NB, (J.N - n0 + 15) / 16);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int row = lane & 15, kg = (lane >> 4) * 8;
  const rsrc_t rx = make_rsrc(J.X + (int64_t)t0 * J.ldx, ((uint64_t)(a.T - t0) * J.ldx) * 2);
  const rsrc_t rw = make_rsrc(J.W + (int64_t)n0 * J.K, ((uint64_t)(J.N - n0) * J.K) * 2);
  const uint32_t xoff = (uint32_t)row * (uint32_t)J.ldx * 2u;
  const int steps = (J.K + 31) / 32;
  const int per = (steps + FW - 1) / FW;
  const int s_beg = w * per, s_end = min(steps, s_beg + per);
  f32x4_t acc[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) acc[nb] = f32x4_t{};
  for (int s = s_beg; s < s_end; s += FU) {
    bf16x8_t av[FU], bv[FU][NB];
#pragma unroll
    for (int u = 0; u < FU; ++u) {
      const int kk = (s + u) * 32 + kg;
      const bool ok = s + u < s_end && kk < J.K;
      av[u] = as_bf8(bload16(rx, ok ? xoff + (uint32_t)kk * 2u : 0xFFFFFFF0u));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        bv[u][nb] = as_bf8(bload16(rw, (ok && nb < nb_used) ? ((uint32_t)(16 * nb + row) * (uint32_t)J.K + (uint32_t)kk) * 2u
                                                            : 0xFFFFFFF0u));
    }
    // keep every load of the group in flight before the first product waits on one
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < FU; ++u)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u], bv[u][nb], acc[nb], 0, 0, 0);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) red[w][nb][lane] = acc[nb];
  __syncthreads();
  if (w >= nb_used) return;
  const int nb = w;
  f32x4_t sum = red[0][nb][lane];
#pragma unroll
  for (int ww = 1; ww < FW; ++ww) sum += red[ww][nb][lane];
  const int col = n0 + 16 * nb + (lane & 15);
  if (col >= J.N) return;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const int tok = t0 + 4 * (lane >> 4) + v;
    if (tok < a.T) J.out[(int64_t)tok * J.ldo + col] = (uint16_t)(pack2(J.alpha * sum[v], 0.f) & 0xFFFFu);
  }
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
  int max_n = 0;
  for (int j = 0; j < a.n_jobs; ++j) max_n = std::max(max_n, a.job[j].N);
  const int nb = std::max(1, std::min(4, (max_n + 15) / 16));   // column blocks per workgroup
  FcKArgs k;
  k.a = a;
  const int m_tiles = (a.T + FT - 1) / FT;
  int tiles = 0;
  for (int j = 0; j < a.n_jobs; ++j) {
    const FcJob& J = a.job[j];
    if (!J.X || !J.W || !J.out || J.K <= 0 || J.N <= 0 || J.K % 8 || J.ldx % 8 || J.ldx < J.K ||
        (reinterpret_cast<uintptr_t>(J.X) & 15) || (reinterpret_cast<uintptr_t>(J.W) & 15) ||
        (uint64_t)FN * J.K * 2 >= (1ull << 31) || (uint64_t)FT * J.ldx * 2 + (uint64_t)J.K * 2 >= (1ull << 31))
      return hipErrorInvalidValue;
    k.tile0[j] = tiles;
    k.n_tiles[j] = (J.N + 16 * nb - 1) / (16 * nb);
    tiles += m_tiles * k.n_tiles[j];
  }
  k.tile0[a.n_jobs] = tiles;
  switch (nb) {
    case 1: hipLaunchKernelGGL(k_lora_fc<1>, dim3((unsigned)tiles), dim3(FW * 64), 0, s, k); break;
    case 2: hipLaunchKernelGGL(k_lora_fc<2>, dim3((unsigned)tiles), dim3(FW * 64), 0, s, k); break;
    case 3: hipLaunchKernelGGL(k_lora_fc<3>, dim3((unsigned)tiles), dim3(FW * 64), 0, s, k); break;
    default: hipLaunchKernelGGL(k_lora_fc<4>, dim3((unsigned)tiles), dim3(FW * 64), 0, s, k); break;
  }
  return hipGetLastError();
}

}  // namespace lsq
