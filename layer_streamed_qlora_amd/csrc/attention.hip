// Causal grouped-query attention, flash style, gfx950 (CDNA4), 64-wide waves.
//
// Scores S = c Q K^T (c = 1/sqrt(hd)), causal mask, P = softmax(S), O = P V; the
// backward gives dV = P^T dO, dP = dO V^T, dS = c P (dP - rowsum(dO * O)), dQ = dS K,
// dK = dS^T Q, with dK and dV summed over the query heads that share a key/value head
// ("Fine-Tuning an 8B Parameter Model on a 4 GB Laptop GPU": the decoder layer is the
// Llama-3.1-8B one, grouped-query attention with rotary positions applied to q, k).
//
// Nothing of size seq x seq is stored.  The forward keeps a running maximum and sum
// per query and writes O and the base-2 log-sum-exp L of the scaled scores; the
// backward recomputes P = exp2(S c log2(e) - L) tile by tile.  Every product takes
// bf16 operands (P and dS are rounded to bf16 as MFMA operands) and accumulates in
// float32 on v_mfma_f32_32x32x16_bf16.
//
// Products over d keep one operand in registers as row fragments; products whose
// contraction runs over a tile's rows reuse score tiles in the lanes' own row order
// and read the other operand from a transposed LDS tile (tiles.hpp).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

#include "lsq_internal.hpp"
#include "rope.hpp"
#include "tiles.hpp"

namespace lsq {
namespace {

using namespace tiles;

constexpr int KB = kTileRows;   // rows (keys or queries) per streamed tile
constexpr int PT = kTPitch;
constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------------ forward
// Workgroup: 128 queries of one (batch, q head), 4 waves x 32 queries.  Per 64-key
// tile each wave computes S^T = K Q^T (keys x queries: each lane holds one query).
// Two passes over the keys: the first finds each row's maximum and sum of exp, the
// second forms the normalised P, rounds it to bf16 (the operand of the second
// product) and accumulates O^T = V^T P^T.
template <int HD>
__global__ void __launch_bounds__(256) k_attn_fwd(AttnArgs a) {
  constexpr int NS = HD / 16, ND = HD / 32, PR = HD + 8;
  __shared__ __align__(16) uint16_t sk[KB * PR];
  __shared__ __align__(16) uint16_t svt[HD * PT];
  const int nqb = (a.S + 127) / 128;
  // the grid runs (batch, head) fastest and the query blocks longest first, so every
  // workgroup of the longest rows is dispatched before any of the next length
  const int qb = nqb - 1 - (int)blockIdx.y;
  const int bh = blockIdx.x, b = bh / a.hq, h = bh % a.hq, g = h / (a.hq / a.hkv);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, ql = lane & 31, hh = lane >> 5;
  const int qw = qb * 128 + 32 * w, q = qw + ql;
  const uint64_t head_bytes = (uint64_t)a.S * a.ldqkv * 2;
  const uint16_t* base = a.qkv + (int64_t)b * a.S * a.ldqkv;
  const rsrc_t rq = make_rsrc(base + h * HD, head_bytes);
  const rsrc_t rk = make_rsrc(base + a.qd + g * HD, head_bytes);
  const rsrc_t rv = make_rsrc(base + a.qd + a.kvd + g * HD, head_bytes);
  bf16x8_t qf[NS];
  row_frags<HD>(qf, rq, a.ldqkv, q, hh);

  const int last_key = min(qb * 128 + 127, a.S - 1);
  const int n_kb = last_key / KB + 1;
  const float cl = a.scale * kLog2e;
  // scaled scores (base 2) of the key tile at k0 against this lane's query, masked; a
  // tile whose keys all precede the wave's first query needs no mask (same values)
  auto scores = [&](f32x16_t (&s)[2], int k0) {
    const bool inside = k0 + KB - 1 <= qw && k0 + KB - 1 < a.S;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      s[kk] = f32x16_t{};
#pragma unroll
      for (int st = 0; st < NS; ++st)
        s[kk] = mfma(*reinterpret_cast<const bf16x8_t*>(sk + (32 * kk + ql) * PR + 16 * st + 8 * hh), qf[st], s[kk]);
      if (inside) {
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kk][v] = s[kk][v] * cl;
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = k0 + 32 * kk + (v >> 2) * 8 + 4 * hh + (v & 3);
          s[kk][v] = (key <= q && key < a.S) ? s[kk][v] * cl : -INFINITY;
        }
      }
    }
  };
  TileMover<HD, 256> tk, tv;
  // pass 1: row maximum m and sum l of exp2(t - m) (each lane half sums its own keys),
  // or the values an earlier forward over the same q, k recorded
  float m = -INFINITY, l = 0.f;
  float lt;
  if (a.stats_in) {
    const float2 st = a.stats_in[(int64_t)bh * a.S + min(q, a.S - 1)];
    m = st.x;
    lt = st.y;
    tk.load(rk, a.ldqkv, 0);
    tv.load(rv, a.ldqkv, 0);
  } else {
    tk.load(rk, a.ldqkv, 0);
    for (int kb = 0; kb < n_kb; ++kb) {
      __syncthreads();                    // the previous tile is no longer read
      tk.store_rows(sk);
      __syncthreads();
      if (kb + 1 < n_kb) {
        tk.load(rk, a.ldqkv, (kb + 1) * KB);
      } else {                            // the second pass starts from key 0
        tk.load(rk, a.ldqkv, 0);
        tv.load(rv, a.ldqkv, 0);
      }
      const int k0 = kb * KB;
      if (k0 > qw + 31) continue;         // tile entirely after this wave's queries
      f32x16_t s[2];
      scores(s, k0);
      float mb = -INFINITY;
  #pragma unroll
      for (int kk = 0; kk < 2; ++kk)
  #pragma unroll
        for (int v = 0; v < 16; ++v) mb = fmaxf(mb, s[kk][v]);
      mb = fmaxf(mb, __shfl_xor(mb, 32));
      const float mn = fmaxf(m, mb);
      const float mu = mn == -INFINITY ? 0.f : mn;
      float ls = 0.f;
  #pragma unroll
      for (int kk = 0; kk < 2; ++kk)
  #pragma unroll
        for (int v = 0; v < 16; ++v) ls += __builtin_amdgcn_exp2f(s[kk][v] - mu);
      l = l * __builtin_amdgcn_exp2f(m - mu) + ls;
      m = mn;
    }
    lt = l + __shfl_xor(l, 32);
  }
  const float inv = 1.f / lt;           // lt >= 1: the maximum's own term
  // pass 2: P = exp2(t - m) / l, rounded to bf16, times V
  f32x16_t o[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) o[d] = f32x16_t{};
  for (int kb = 0; kb < n_kb; ++kb) {
    __syncthreads();
    tk.store_rows(sk);
    tv.store_t(svt);
    __syncthreads();
    if (kb + 1 < n_kb) {
      tk.load(rk, a.ldqkv, (kb + 1) * KB);
      tv.load(rv, a.ldqkv, (kb + 1) * KB);
    }
    const int k0 = kb * KB;
    if (k0 > qw + 31) continue;
    f32x16_t s[2];
    scores(s, k0);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int v = 0; v < 16; ++v) s[kk][v] = __builtin_amdgcn_exp2f(s[kk][v] - m) * inv;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8_t pb = pack8(s[kk], 8 * st);
#pragma unroll
        for (int d = 0; d < ND; ++d) o[d] = mfma(tfrag(svt, 32 * d + ql, 32 * kk + 16 * st, hh), pb, o[d]);
      }
  }
  if (q < a.S) {
    const int64_t row = (int64_t)b * a.S + q;
    uint16_t* dst = a.out + row * a.ldo + h * HD;
    float* dst32 = a.out32 ? a.out32 + row * a.ldo + h * HD : nullptr;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int col = 32 * d + 8 * g4 + 4 * hh;
        const float4 v4 = make_float4(o[d][4 * g4], o[d][4 * g4 + 1], o[d][4 * g4 + 2], o[d][4 * g4 + 3]);
        *reinterpret_cast<uint2*>(dst + col) = make_uint2(pack2(v4.x, v4.y), pack2(v4.z, v4.w));
        if (dst32) *reinterpret_cast<float4*>(dst32 + col) = v4;
      }
    if (hh == 0 && a.lse) a.lse[(int64_t)bh * a.S + q] = m + __builtin_amdgcn_logf(lt);
    if (hh == 0 && a.stats_out) a.stats_out[(int64_t)bh * a.S + q] = make_float2(m, lt);
  }
}

// ------------------------------------------------------- backward: rowsum(dO * O)
template <int HD>
__global__ void k_attn_dd(AttnArgs a) {
  constexpr int TPR = HD / 8;                       // threads per (row, head)
  const int64_t idx = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;   // row * hq + head
  const int part = threadIdx.x % TPR;
  const int64_t n = (int64_t)a.batch * a.S * a.hq;
  float acc = 0.f;
  const bool ok = idx < n;
  const int64_t row = ok ? idx / a.hq : 0;
  const int head = ok ? (int)(idx % a.hq) : 0;
  if (ok) {
    // O in float32 (the product P V before rounding): sum_d dO O = sum_j P_j dP_j
    const uint4 x = *reinterpret_cast<const uint4*>(a.dout + row * a.lddo + head * HD + 8 * part);
    const float4 y0 = *reinterpret_cast<const float4*>(a.out32 + row * a.ldo + head * HD + 8 * part);
    const float4 y1 = *reinterpret_cast<const float4*>(a.out32 + row * a.ldo + head * HD + 8 * part + 4);
    acc = bf_lo(x.x) * y0.x + bf_hi(x.x) * y0.y + bf_lo(x.y) * y0.z + bf_hi(x.y) * y0.w +
          bf_lo(x.z) * y1.x + bf_hi(x.z) * y1.y + bf_lo(x.w) * y1.z + bf_hi(x.w) * y1.w;
  }
#pragma unroll
  for (int sh = TPR / 2; sh > 0; sh >>= 1) acc += __shfl_xor(acc, sh);
  if (ok && part == 0) {
    const int64_t bq = row / a.S, pos = row % a.S;
    a.dd[(bq * a.hq + head) * a.S + pos] = acc;
  }
}

// ------------------------------------------------------------ backward: dQ
// Workgroup: 128 queries of one (batch, q head), 4 waves x 32 queries, over the key
// tiles up to the diagonal: S^T = K Q^T and dP^T = V dO^T (keys x queries), dS, then
// dQ^T += K^T dS^T.
template <int HD>
__global__ void __launch_bounds__(256, 2) k_attn_dq(AttnArgs a) {   // two workgroups per CU (52 KB LDS each)
  constexpr int NS = HD / 16, ND = HD / 32, PR = HD + 8;
  __shared__ __align__(16) uint16_t sk[KB * PR];
  __shared__ __align__(16) uint16_t sv[KB * PR];
  __shared__ __align__(16) uint16_t skt[HD * PT];
  const int nqb = (a.S + 127) / 128;
  const int qb = nqb - 1 - (int)blockIdx.y;   // longest rows first, as in the forward
  const int bh = blockIdx.x, b = bh / a.hq, h = bh % a.hq, g = h / (a.hq / a.hkv);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, ql = lane & 31, hh = lane >> 5;
  const int qw = qb * 128 + 32 * w, q = qw + ql;
  const uint64_t head_bytes = (uint64_t)a.S * a.ldqkv * 2;
  const uint16_t* base = a.qkv + (int64_t)b * a.S * a.ldqkv;
  const rsrc_t rq = make_rsrc(base + h * HD, head_bytes);
  const rsrc_t rk = make_rsrc(base + a.qd + g * HD, head_bytes);
  const rsrc_t rv = make_rsrc(base + a.qd + a.kvd + g * HD, head_bytes);
  const rsrc_t rdo = make_rsrc(a.dout + (int64_t)b * a.S * a.lddo + h * HD, (uint64_t)a.S * a.lddo * 2);
  bf16x8_t qf[NS], of[NS];
  row_frags<HD>(qf, rq, a.ldqkv, q, hh);
  row_frags<HD>(of, rdo, a.lddo, q, hh);
  const bool qok = q < a.S;
  const float L = qok ? a.lse[(int64_t)bh * a.S + q] : 0.f;
  const float D = qok ? a.dd[(int64_t)bh * a.S + q] : 0.f;

  const int last_key = min(qb * 128 + 127, a.S - 1);
  const int n_kb = last_key / KB + 1;
  const float cl = a.scale * kLog2e;
  f32x16_t dq[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) dq[d] = f32x16_t{};
  TileMover<HD, 256> tk, tv;
  tk.load(rk, a.ldqkv, 0);
  tv.load(rv, a.ldqkv, 0);
  for (int kb = 0; kb < n_kb; ++kb) {
    __syncthreads();
    tk.store_rows(sk);
    tk.store_t(skt);
    tv.store_rows(sv);
    __syncthreads();
    if (kb + 1 < n_kb) {
      tk.load(rk, a.ldqkv, (kb + 1) * KB);
      tv.load(rv, a.ldqkv, (kb + 1) * KB);
    }
    const int k0 = kb * KB;
    if (k0 > qw + 31) continue;
    const bool inside = k0 + KB - 1 <= qw && k0 + KB - 1 < a.S;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        s = mfma(*reinterpret_cast<const bf16x8_t*>(sk + (32 * kk + ql) * PR + 16 * st + 8 * hh), qf[st], s);
        dp = mfma(*reinterpret_cast<const bf16x8_t*>(sv + (32 * kk + ql) * PR + 16 * st + 8 * hh), of[st], dp);
      }
      if (inside) {   // every key of the tile precedes the wave's first query
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = qok ? bf16_value(__builtin_amdgcn_exp2f(s[v] * cl - L)) : 0.f;
          s[v] = a.scale * p * (dp[v] - D);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int key = k0 + 32 * kk + (v >> 2) * 8 + 4 * hh + (v & 3);
          const bool ok = qok && key <= q && key < a.S;
          const float p = ok ? bf16_value(__builtin_amdgcn_exp2f(s[v] * cl - L)) : 0.f;
          s[v] = a.scale * p * (dp[v] - D);
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8_t db = pack8(s, 8 * st);
#pragma unroll
        for (int d = 0; d < ND; ++d) dq[d] = mfma(tfrag(skt, 32 * d + ql, 32 * kk + 16 * st, hh), db, dq[d]);
      }
    }
  }
  if (qok && a.dq16) {
    // bf16 with the inverse rotation: column c (< HD/2) pairs with c + HD/2, which this
    // lane holds in block d + ND/2 of the same register positions
    uint16_t* dst = a.dq16 + ((int64_t)b * a.S + q) * a.lddq16 + h * HD;
    const float2* tab = a.rope_tab + (int64_t)q * (HD / 2);
#pragma unroll
    for (int d = 0; d < ND / 2; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int col = 32 * d + 8 * g4 + 4 * hh;
        const float4 t01 = *reinterpret_cast<const float4*>(tab + col);
        const float4 t23 = *reinterpret_cast<const float4*>(tab + col + 2);
        const float2 cs[4] = {make_float2(t01.x, t01.y), make_float2(t01.z, t01.w), make_float2(t23.x, t23.y),
                              make_float2(t23.z, t23.w)};
        float2 g[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) g[e] = rope_inverse(dq[d][4 * g4 + e], dq[d + ND / 2][4 * g4 + e], cs[e]);
        *reinterpret_cast<uint2*>(dst + col) = make_uint2(pack2(g[0].x, g[1].x), pack2(g[2].x, g[3].x));
        *reinterpret_cast<uint2*>(dst + col + HD / 2) = make_uint2(pack2(g[0].y, g[1].y), pack2(g[2].y, g[3].y));
      }
  } else if (qok) {
    float* dst = a.dqkv + ((int64_t)b * a.S + q) * a.lddqkv + h * HD;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<float4*>(dst + 32 * d + 8 * g4 + 4 * hh) =
            make_float4(dq[d][4 * g4], dq[d][4 * g4 + 1], dq[d][4 * g4 + 2], dq[d][4 * g4 + 3]);
  }
}

// -------------------------------------------------------- backward: dK, dV
// Workgroup: 64 keys of one (batch, kv head), 2 waves x 32 keys, looping over the
// group's q heads in order and, per head, over the 64-query tiles from the diagonal
// on: S = Q K^T and dP = dO V^T (queries x keys: each lane holds one key), P, dS, then
// dV += P^T dO and dK += dS^T Q.  The sums over heads and tiles stay in registers, in
// a fixed order.  With n_half = 2 the group's q heads are split in two halves, one
// workgroup each: the first half's sums go to dqkv, the second's to dkv2.  The key
// block varies slowest over the grid, so the longest workgroups (the first key blocks,
// which see every query tile) start first and the short ones fill in behind them.
template <int HD>
__global__ void __launch_bounds__(128) k_attn_dkv(AttnArgs a, int n_half) {
  constexpr int NS = HD / 16, ND = HD / 32, PR = HD + 8;
  __shared__ __align__(16) uint16_t sq[KB * PR];
  __shared__ __align__(16) uint16_t sdo[KB * PR];
  __shared__ __align__(16) uint16_t sqt[HD * PT];
  __shared__ __align__(16) uint16_t sdot[HD * PT];
  __shared__ __align__(16) float sL[KB];
  __shared__ __align__(16) float sD[KB];
  const int n_bg = a.batch * a.hkv;
  const int bg = (int)blockIdx.x % n_bg, rest = (int)blockIdx.x / n_bg;
  const int hf = rest % n_half, kb = rest / n_half;
  const int b = bg / a.hkv, g = bg % a.hkv;
  const int nrep = a.hq / a.hkv;
  const int r0 = hf * (nrep / n_half), n_rep = nrep / n_half;   // this workgroup's q heads
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, kl = lane & 31, hh = lane >> 5;
  const int kw0 = kb * KB + 32 * w, key = kw0 + kl;
  const uint64_t head_bytes = (uint64_t)a.S * a.ldqkv * 2;
  const uint16_t* base = a.qkv + (int64_t)b * a.S * a.ldqkv;
  const rsrc_t rk = make_rsrc(base + a.qd + g * HD, head_bytes);
  const rsrc_t rv = make_rsrc(base + a.qd + a.kvd + g * HD, head_bytes);
  bf16x8_t kf[NS], vf[NS];
  row_frags<HD>(kf, rk, a.ldqkv, key, hh);
  row_frags<HD>(vf, rv, a.ldqkv, key, hh);
  const float cl = a.scale * kLog2e;
  f32x16_t dk[ND], dv[ND];
#pragma unroll
  for (int d = 0; d < ND; ++d) { dk[d] = f32x16_t{}; dv[d] = f32x16_t{}; }
  // iterations: query tiles qb = kb .. n_qb - 1 of each q head of the group in order;
  // the tiles (and row statistics) of iteration i + 1 load while iteration i computes
  const int n_qt = (a.S + KB - 1) / KB - kb;
  const int n_it = n_rep * n_qt;
  TileMover<HD, 128> tq, to;
  float lv = 0.f, dv_ = 0.f;
  auto fetch = [&](int i) {
    const int r = i / n_qt;
    const int q0 = (kb + i - r * n_qt) * KB;
    const int h = g * nrep + r0 + r;
    const int64_t bh = (int64_t)b * a.hq + h;
    tq.load(make_rsrc(base + h * HD, head_bytes), a.ldqkv, q0);
    to.load(make_rsrc(a.dout + (int64_t)b * a.S * a.lddo + h * HD, (uint64_t)a.S * a.lddo * 2), a.lddo, q0);
    // row statistics of the tile's queries (threads past the tile or the sequence read 0)
    const bool ok = threadIdx.x < KB && q0 + (int)threadIdx.x < a.S;
    const uint32_t off = ok ? (uint32_t)(q0 + threadIdx.x) * 4u : 0xFFFFFFF0u;
    lv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.lse + bh * a.S, (uint64_t)a.S * 4), off, 0, 0));
    dv_ = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.dd + bh * a.S, (uint64_t)a.S * 4), off, 0, 0));
  };
  fetch(0);
  for (int i = 0; i < n_it; ++i) {
    const int q0 = (kb + i % n_qt) * KB;
    __syncthreads();                  // the previous tiles are no longer read
    tq.store_rows(sq);
    tq.store_t(sqt);
    to.store_rows(sdo);
    to.store_t(sdot);
    if (threadIdx.x < KB) { sL[threadIdx.x] = lv; sD[threadIdx.x] = dv_; }
    __syncthreads();
    fetch(i + 1 < n_it ? i + 1 : i);  // issued on every iteration (the last re-reads its tile)
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      if (q0 + 32 * qs + 31 < kw0) continue;      // every query before this wave's keys
      f32x16_t s = f32x16_t{}, dp = f32x16_t{};
#pragma unroll
      for (int st = 0; st < NS; ++st) {
        s = mfma(*reinterpret_cast<const bf16x8_t*>(sq + (32 * qs + kl) * PR + 16 * st + 8 * hh), kf[st], s);
        dp = mfma(*reinterpret_cast<const bf16x8_t*>(sdo + (32 * qs + kl) * PR + 16 * st + 8 * hh), vf[st], dp);
      }
      // C[i = query][j = key]: register v holds query 32 qs + (v / 4) * 8 + 4 hh + v % 4;
      // no mask when every query of the slice follows every key of the wave
      const bool inside = q0 + 32 * qs >= kw0 + 31 && q0 + 32 * qs + 31 < a.S && kw0 + 31 < a.S;
      f32x16_t ds;
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int qi = 32 * qs + 8 * g4 + 4 * hh;
        const float4 L4 = *reinterpret_cast<const float4*>(&sL[qi]);
        const float4 D4 = *reinterpret_cast<const float4*>(&sD[qi]);
        const float Ls[4] = {L4.x, L4.y, L4.z, L4.w}, Ds[4] = {D4.x, D4.y, D4.z, D4.w};
        if (inside) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * g4 + e;
            const float p = bf16_value(__builtin_amdgcn_exp2f(s[v] * cl - Ls[e]));
            s[v] = p;
            ds[v] = a.scale * p * (dp[v] - Ds[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int v = 4 * g4 + e, qg = q0 + qi + e;
            const bool ok = key <= qg && qg < a.S && key < a.S;
            const float p = ok ? bf16_value(__builtin_amdgcn_exp2f(s[v] * cl - Ls[e])) : 0.f;
            s[v] = p;
            ds[v] = a.scale * p * (dp[v] - Ds[e]);
          }
        }
      }
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const bf16x8_t pa = pack8(s, 8 * st), da = pack8(ds, 8 * st);
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          dv[d] = mfma(pa, tfrag(sdot, 32 * d + kl, 32 * qs + 16 * st, hh), dv[d]);
          dk[d] = mfma(da, tfrag(sqt, 32 * d + kl, 32 * qs + 16 * st, hh), dk[d]);
        }
      }
    }
  }
  // C[i = key][j = d]: lane (d + 32 hh), register v holds key (v / 4) * 8 + 4 hh + v % 4
  float* dst = hf == 0 ? a.dqkv + a.qd : a.dkv2;
  const int64_t ld = hf == 0 ? a.lddqkv : 2 * (int64_t)a.kvd;
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int kr = kw0 + (v >> 2) * 8 + 4 * hh + (v & 3);
    if (kr >= a.S) continue;
    float* row = dst + ((int64_t)b * a.S + kr) * ld;
#pragma unroll
    for (int d = 0; d < ND; ++d) {
      row[g * HD + 32 * d + kl] = dk[d][v];
      row[a.kvd + g * HD + 32 * d + kl] = dv[d][v];
    }
  }
}

template <int HD>
hipError_t fwd_hd(const AttnArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_attn_fwd<HD>, dim3(a.batch * a.hq, (a.S + 127) / 128), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int HD>
hipError_t bwd_hd(const AttnArgs& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.batch * a.S * a.hq;
  const int per_block = 256 / (HD / 8);
  hipLaunchKernelGGL(k_attn_dd<HD>, dim3((unsigned)((rows + per_block - 1) / per_block)), dim3(256), 0, s, a);
  const int n_half = a.dkv2 ? 2 : 1;
  hipLaunchKernelGGL(k_attn_dkv<HD>, dim3((a.S + KB - 1) / KB * n_half * a.batch * a.hkv), dim3(128), 0, s, a, n_half);
  hipLaunchKernelGGL(k_attn_dq<HD>, dim3(a.batch * a.hq, (a.S + 127) / 128), dim3(256), 0, s, a);
  return hipGetLastError();
}

bool shape_ok(const AttnArgs& a) {
  return (a.hd == 64 || a.hd == 128) && a.hkv > 0 && a.hq % a.hkv == 0 && a.ldqkv % 8 == 0 && a.ldo % 8 == 0 &&
         a.qd % 8 == 0 && a.kvd % 8 == 0;
}

}  // namespace

hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t s) {
  if (a.batch <= 0 || a.S <= 0) return hipSuccess;
  if (!shape_ok(a) || !a.qkv || !a.out) return hipErrorInvalidValue;
  return a.hd == 64 ? fwd_hd<64>(a, s) : fwd_hd<128>(a, s);
}

hipError_t launch_attn_bwd(const AttnArgs& a, hipStream_t s) {
  if (a.batch <= 0 || a.S <= 0) return hipSuccess;
  if (!shape_ok(a) || !a.qkv || !a.out32 || !a.dout || !a.lse || !a.dd || !a.dqkv || a.lddo % 8 != 0 ||
      a.lddqkv % 4 != 0 || (a.dkv2 && (a.hq / a.hkv) % 2 != 0))
    return hipErrorInvalidValue;
  if (a.dq16 && (!a.rope_tab || a.lddq16 < a.qd || a.lddq16 % 4 != 0 || (reinterpret_cast<uintptr_t>(a.dq16) & 7) ||
                 (reinterpret_cast<uintptr_t>(a.rope_tab) & 15)))
    return hipErrorInvalidValue;
  return a.hd == 64 ? bwd_hd<64>(a, s) : bwd_hd<128>(a, s);
}

}  // namespace lsq
