// Host-side encoding of the frozen base: NF4 codebook, blockwise NF4 packing with
// optional double quantisation, config validation and the per-layer blob layout.
//
// The encoding is the 4-bit NormalFloat storage with nested quantisation of the
// scaling constants that "Fine-Tuning an 8B Parameter Model on a 4 GB Laptop GPU"
// (codeinktechnologies.com), section "Quantization: Shrink the Weights", describes;
// block 64 and the 8-bit / 256-block second level are the workload's parameters.
// Readings where the pages are silent (nibble order, ties, the second level) are
// spelled out next to the code that implements them.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <thread>
#include <vector>

#include "lsq_internal.hpp"

// Every operation below is rounded on its own, in the order written: no fused
// multiply-add, so the host encoder takes exactly the decisions it is specified to.
#pragma clang fp contract(off)

namespace lsq {

// ------------------------------------------------------------------ codebook
// Standard-normal quantile by bisection on erfc; 200 halvings reach adjacent doubles.
static double normal_quantile(double p) {
  double lo = -40.0, hi = 40.0;
  for (int i = 0; i < 200; ++i) {
    double mid = 0.5 * (lo + hi);
    double cdf = 0.5 * std::erfc(-mid / std::sqrt(2.0));
    if (cdf < p) lo = mid; else hi = mid;
    if (!(hi - lo > 0.0)) break;
  }
  return 0.5 * (lo + hi);
}

// NormalFloat levels (QLoRA paper, section 3): quantiles of equally spaced
// probabilities from delta toward 1/2 — 8 on the positive side, 7 on the negative
// side — plus an exact zero, divided by the largest magnitude, rounded once to
// float32.  delta = ((1 - 1/30) + (1 - 1/32)) / 2, kept exact.
void nf4_codebook_host(float out[16]) {
  const double d = 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0));
  double v[16];
  int n = 0;
  for (int i = 0; i < 8; ++i) v[n++] = normal_quantile(d + (i * (0.5 - d)) / 8.0);
  for (int i = 0; i < 7; ++i) v[n++] = -normal_quantile(d + (i * (0.5 - d)) / 7.0);
  v[n++] = 0.0;
  std::sort(v, v + 16);
  double mx = 0.0;
  for (double x : v) mx = std::max(mx, std::fabs(x));
  for (int i = 0; i < 16; ++i) out[i] = (float)(v[i] / mx);
}

// ------------------------------------------------------------------- packing
static inline float bf16_to_f32(uint16_t h) {
  uint32_t u = (uint32_t)h << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

namespace {
struct Nf4Quantiser {
  double mid[15];
  explicit Nf4Quantiser(const float* lv) {
    // midpoints of adjacent levels, exact in float64 for float32 levels
    for (int i = 0; i < 15; ++i) mid[i] = ((double)lv[i] + (double)lv[i + 1]) * 0.5;
  }
  // nearest level, ties to the higher index: the number of midpoints <= n
  inline uint8_t code(float n) const {
    double x = (double)n;
    int c = 0;
    for (int i = 0; i < 15; ++i) c += (x >= mid[i]);
    return (uint8_t)c;
  }
};
}  // namespace

static void pack_range(const uint16_t* w, uint64_t numel, uint64_t b0, uint64_t b1,
                       const Nf4Quantiser& q, uint8_t* packed, float* absmax) {
  uint8_t codes[kNF4Block];
  for (uint64_t b = b0; b < b1; ++b) {
    uint64_t e0 = b * kNF4Block;
    uint64_t e1 = std::min<uint64_t>(numel, e0 + kNF4Block);
    int n = (int)(e1 - e0);
    float am = 0.f;
    for (int i = 0; i < n; ++i) am = std::max(am, std::fabs(bf16_to_f32(w[e0 + i])));
    absmax[b] = am;
    if (am == 0.f) {
      for (int i = 0; i < n; ++i) codes[i] = 7;     // all-zero block: the exact 0 level
    } else {
      for (int i = 0; i < n; ++i) codes[i] = q.code(bf16_to_f32(w[e0 + i]) / am);  // fp32 division
    }
    // element 2k in the high nibble of byte k, 2k+1 in the low nibble; pad with 7
    for (int i = 0; i < n; i += 2) {
      uint8_t hi = codes[i];
      uint8_t lo = (i + 1 < n) ? codes[i + 1] : (uint8_t)7;
      packed[(e0 + i) / 2] = (uint8_t)((hi << 4) | lo);
    }
  }
}

static int pick_threads(int n_threads) {
  if (n_threads > 0) return n_threads;
  unsigned hc = std::thread::hardware_concurrency();
  return (int)std::max(1u, std::min(hc ? hc : 1u, 16u));
}

template <class F>
static void parallel_for(uint64_t n, int n_threads, F&& f) {
  int t = (int)std::min<uint64_t>((uint64_t)n_threads, std::max<uint64_t>(1, n / 64));
  if (t <= 1) { f(0, n); return; }
  std::vector<std::thread> th;
  uint64_t step = (n + t - 1) / t;
  for (int i = 0; i < t; ++i) {
    uint64_t a = i * step, b = std::min(n, a + step);
    if (a >= b) break;
    th.emplace_back([&, a, b] { f(a, b); });
  }
  for (auto& x : th) x.join();
}

// Second level over the absmax values (reading: symmetric int8 around one float32
// mean per tensor; the mean is the float64 sum in index order divided by the count;
// per group of 256 a float32 scale = max |fp32(a - mean)|; code =
// round-half-even(clamp(127 (a - mean) / scale, -127, 127)) in float64).
static void double_quantise(const float* a, uint64_t n, int n_threads, uint8_t* qabs, float* scale2, float* mean_out) {
  double sum = 0.0;
  for (uint64_t i = 0; i < n; ++i) sum += (double)a[i];
  const float mean = n ? (float)(sum / (double)n) : 0.f;
  *mean_out = mean;
  uint64_t ngroups = (n + kDQGroup - 1) / kDQGroup;
  parallel_for(ngroups, n_threads, [&](uint64_t g0, uint64_t g1) {
    for (uint64_t g = g0; g < g1; ++g) {
      uint64_t i0 = g * kDQGroup, i1 = std::min<uint64_t>(n, i0 + kDQGroup);
      float s = 0.f;
      for (uint64_t i = i0; i < i1; ++i) {
        const float c = a[i] - mean;      // float32 subtraction
        s = std::max(s, std::fabs(c));
      }
      scale2[g] = s;
      for (uint64_t i = i0; i < i1; ++i) {
        int c = 0;
        if (s != 0.f) {
          double t = ((double)a[i] - (double)mean) / (double)s * 127.0;
          t = std::min(127.0, std::max(-127.0, t));
          c = (int)std::nearbyint(t);
        }
        qabs[i] = (uint8_t)(int8_t)c;
      }
    }
  });
}

void pack_nf4_host(const uint16_t* w, uint64_t numel, bool double_quant, int n_threads,
                   uint8_t* packed, float* absmax, uint8_t* qabs, float* scale2, float* mean) {
  float lv[16];
  nf4_codebook_host(lv);
  Nf4Quantiser q(lv);
  uint64_t nblocks = (numel + kNF4Block - 1) / kNF4Block;
  n_threads = pick_threads(n_threads);
  parallel_for(nblocks, n_threads, [&](uint64_t b0, uint64_t b1) { pack_range(w, numel, b0, b1, q, packed, absmax); });
  if (double_quant) double_quantise(absmax, nblocks, n_threads, qabs, scale2, mean);
}

// ---------------------------------------------------------- config and layout
void proj_dims(const ls_config& c, int proj, int32_t* n_out, int32_t* n_in) {
  const int32_t h = c.hidden, q = c.n_heads * c.head_dim, kv = c.n_kv_heads * c.head_dim, I = c.intermediate;
  switch (proj) {
    case LS_PROJ_Q: *n_out = q; *n_in = h; break;
    case LS_PROJ_K: *n_out = kv; *n_in = h; break;
    case LS_PROJ_V: *n_out = kv; *n_in = h; break;
    case LS_PROJ_O: *n_out = h; *n_in = q; break;
    case LS_PROJ_GATE: *n_out = I; *n_in = h; break;
    case LS_PROJ_UP: *n_out = I; *n_in = h; break;
    default: *n_out = h; *n_in = I; break;
  }
}

bool validate_config(const ls_config& c, const char** why) {
#define REQ(cond, msg) do { if (!(cond)) { *why = msg; return false; } } while (0)
  REQ(c.n_layers >= 1, "n_layers must be >= 1");
  REQ(c.hidden >= 64 && c.hidden % 64 == 0, "hidden must be a positive multiple of 64");
  REQ(c.n_heads >= 1 && c.n_kv_heads >= 1 && c.n_heads % c.n_kv_heads == 0, "n_heads must be a multiple of n_kv_heads");
  REQ(c.head_dim == 64 || c.head_dim == 128, "head_dim must be 64 or 128");
  REQ((c.n_heads * c.head_dim) % 64 == 0 && (c.n_kv_heads * c.head_dim) % 64 == 0, "head widths must be multiples of 64");
  REQ(c.intermediate >= 16 && c.intermediate % 16 == 0, "intermediate must be a positive multiple of 16");
  REQ(c.rms_eps > 0.f && std::isfinite(c.rms_eps), "rms_eps must be positive");
  REQ(c.rope_theta > 1.f && std::isfinite(c.rope_theta), "rope_theta must be > 1");
  REQ(c.quant == LS_QUANT_NF4 || c.quant == LS_QUANT_BF16, "quant must be LS_QUANT_NF4 or LS_QUANT_BF16");
  REQ(c.quant != LS_QUANT_NF4 || c.nf4_block == 64, "nf4_block must be 64");
  REQ(c.double_quant == 0 || c.double_quant == 1, "double_quant must be 0 or 1");
  REQ(c.quant == LS_QUANT_NF4 || c.double_quant == 0, "double_quant needs NF4");
  REQ(c.lora_r >= 1 && c.lora_r <= 64, "lora_r must be in 1..64");
  REQ(std::isfinite(c.lora_alpha), "lora_alpha must be finite");
  REQ((c.lora_mask & ~0x7Fu) == 0, "lora_mask has bits beyond the 7 projections");
  REQ(c.n_buffers == 0 || (c.n_buffers >= 2 && c.n_buffers <= 64), "n_buffers must be 0 (auto) or in 2..64");
  REQ(c.max_tokens >= 1 && c.max_tokens <= (1 << 20), "max_tokens must be in 1..2^20");
  REQ(c.max_seq >= 1 && c.max_seq <= c.max_tokens && c.max_seq <= 8192, "max_seq must be in 1..min(max_tokens, 8192)");
  REQ(c.resident == 0 || c.resident == 1, "resident must be 0 or 1");
  REQ(c.adamw == 0 || c.adamw == 1, "adamw must be 0 or 1");
  REQ(c.profile >= LS_PROFILE_OFF && c.profile <= LS_PROFILE_GEMM, "profile must be 0, 1 or 2");
  REQ(c.vocab >= 0 && c.vocab <= (1 << 24), "vocab must be in 0..2^24");
  REQ(c.store == LS_STORE_HOST || c.store == LS_STORE_FILE, "store must be LS_STORE_HOST or LS_STORE_FILE");
  REQ(c.copy_split == 0 || c.copy_split == 1, "copy_split must be 0 or 1");
  REQ(c.profile_stride >= 0 && c.profile_stride <= 1 << 20, "profile_stride must be >= 0");
  REQ(c.store != LS_STORE_FILE || (c.store_path[0] != 0 && memchr(c.store_path, 0, sizeof(c.store_path)) != nullptr),
      "LS_STORE_FILE needs a NUL-terminated store_path");
#undef REQ
  return true;
}

BlobLayout make_layout(const ls_config& c) {
  BlobLayout L;
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) { off = align_up(off, kAlign); uint64_t o = off; off += bytes; return o; };
  L.off_g1 = take(2ull * c.hidden);
  L.off_g2 = take(2ull * c.hidden);
  for (int p = 0; p < LS_N_PROJ; ++p) {
    ProjLayout& P = L.p[p];
    proj_dims(c, p, &P.n_out, &P.n_in);
    P.numel = (uint64_t)P.n_out * (uint64_t)P.n_in;
    if (c.quant == LS_QUANT_BF16) {
      P.bytes_w = 2 * P.numel;
      P.off_w = take(P.bytes_w);
      continue;
    }
    P.nblocks = (P.numel + kNF4Block - 1) / kNF4Block;
    P.ngroups = (P.nblocks + kDQGroup - 1) / kDQGroup;
    P.bytes_w = (P.numel + 1) / 2;
    P.off_w = take(P.bytes_w);
    if (c.double_quant) {
      P.off_qabs = take(P.nblocks);
      P.off_scale2 = take(4 * P.ngroups);
      P.off_mean = take(4);
    } else {
      P.off_absmax = take(4 * P.nblocks);
    }
  }
  L.bytes = align_up(off, kAlign);
  return L;
}

}  // namespace lsq
