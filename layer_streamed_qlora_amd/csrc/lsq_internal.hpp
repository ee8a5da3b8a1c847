// Internal declarations shared by the host runtime and the HIP kernels of liblsq.
#pragma once
#include <string>
#include <vector>

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "../../include/ls.h"

namespace lsq {

constexpr int kNF4Block = 64;     // weights per first-level absmax
constexpr int kDQGroup = 256;     // absmax values per second-level scale
constexpr int kAlign = 256;       // byte alignment of every piece of a layer blob

inline uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

// ---------------------------------------------------------------- blob layout
// One layer blob holds g1, g2 (bf16 [hidden]) and, per projection, either the NF4
// pieces (packed codes, absmax or qabs+scale2+mean) or the bf16 matrix.  The same
// layout is used in pinned host memory and in every device slot, so a streamed run
// and a resident run read identical bytes at identical offsets.
struct ProjLayout {
  int32_t n_out = 0, n_in = 0;
  uint64_t numel = 0, nblocks = 0, ngroups = 0;
  uint64_t off_w = 0, bytes_w = 0;        // packed codes (NF4) or bf16 matrix
  uint64_t off_absmax = 0;                // float32 [nblocks]   (NF4, no DQ)
  uint64_t off_qabs = 0;                  // uint8  [nblocks]   (NF4 + DQ)
  uint64_t off_scale2 = 0;                // float32 [ngroups]  (NF4 + DQ)
  uint64_t off_mean = 0;                  // float32 [1]        (NF4 + DQ)
};

struct BlobLayout {
  uint64_t off_g1 = 0, off_g2 = 0;
  ProjLayout p[LS_N_PROJ];
  uint64_t bytes = 0;
};

bool validate_config(const ls_config& c, const char** why);
BlobLayout make_layout(const ls_config& c);
void proj_dims(const ls_config& c, int proj, int32_t* n_out, int32_t* n_in);

// ------------------------------------------------------------- host encoders
void nf4_codebook_host(float out[16]);
void pack_nf4_host(const uint16_t* w, uint64_t numel, bool double_quant, int n_threads,
                   uint8_t* packed, float* absmax, uint8_t* qabs, float* scale2, float* mean);

// ------------------------------------------------------------ kernel launches
// All launches are asynchronous on `s` and return hipGetLastError().

// Weight description handed to the fused dequant GEMMs (device pointers into a slot).
struct WeightRef {
  const uint8_t* w = nullptr;       // NF4 packed codes or bf16 matrix
  const float* absmax = nullptr;    // NF4 without DQ
  const uint8_t* qabs = nullptr;    // NF4 with DQ
  const float* scale2 = nullptr;
  const float* mean = nullptr;
  int32_t n_out = 0, n_in = 0;
};

enum WFormat { WF_NF4 = 0, WF_NF4_DQ = 1, WF_BF16 = 2 };

constexpr int kMaxGroups = 3;

// Y[:, col0_g : col0_g + n_out_g] = X W_g^T + Aext[:, acol_g : acol_g + kx] Bext_g^T (+ R)
// for up to three weights g that share the input X [M, K] (K = n_in of every g).
struct FwdGroup {
  WeightRef w;
  int32_t out_col0 = 0;            // first output column of this group
  int32_t ext_col0 = 0;            // first column of this group's extension operand in Aext
  const uint16_t* bext = nullptr;  // bf16 [n_out, kx]: LoRA B (already in bf16), row stride kx
};
// Scratch for split tiles in the fused dequant GEMMs.  With `part` set, a launch whose
// last (or only) round of 256 x 256 tiles leaves at least 1/8 of the compute units idle
// cuts each tile of that round along K into pieces, one workgroup each; the pieces of
// a tile meet in part (float32 partial tiles, room for `slots` tiles) and cnt ([slots]
// arrival counters, zero before the launch and left zero after it).  slots must be at
// least the number of compute units.  Launches that share one scratch must not overlap
// in time (one stream per scratch).
struct SplitTiles {
  float* part = nullptr;
  uint32_t* cnt = nullptr;
  int32_t slots = 0;
};
struct FwdArgs {
  const uint16_t* x = nullptr; int32_t ldx = 0;     // bf16 [M, K]
  int32_t M = 0, K = 0;
  int32_t n_groups = 0;
  FwdGroup g[kMaxGroups];
  const uint16_t* aext = nullptr; int32_t ldaext = 0; int32_t kx = 0;   // bf16 [M, >=kx]; kx multiple of 16, 0 = none
  const uint16_t* resid = nullptr;                  // bf16 residual added to Y (nullable)
  const float* resid32 = nullptr; int32_t ldr = 0;  // or float32 residual
  uint16_t* y = nullptr; float* y32 = nullptr; int32_t ldy = 0;   // bf16 or float32 output
  // rotary embedding on output columns [0, rope_cols) before rounding (q and k of
  // the fused q|k|v projection): tab[pos * hd/2 + i] = (cos, sin), pos = row % seq
  const float2* rope_tab = nullptr; int32_t rope_cols = 0, seq = 1, head_dim = 128;
  const float* levels = nullptr;                    // device float32[16] NF4 levels
  int32_t format = WF_NF4;
  // SwiGLU: groups 0, 1 = gate, up (same shape, K % 64 == 0, up's low-rank columns
  // right after gate's, 2 kx <= 64); y (bf16, [M, ldy]) = silu(gate) * up, and, if gu32
  // is set, gate and up in float32 ([M, ldgu], up at column + n_out)
  int32_t swiglu = 0;
  float* gu32 = nullptr; int32_t ldgu = 0;
  // SwiGLU backward in the same epilogue (the recomputed gate | up, run inside the
  // backward once d(act) is known): with dact (float32 [M, ldda]) set, dgu (bf16
  // [M, lddgu], dup at column + n_out) receives dgate | dup; gu32 must then be null
  const float* dact = nullptr; int32_t ldda = 0;
  uint16_t* dgu = nullptr; int32_t lddgu = 0;
  SplitTiles sk;
};
hipError_t launch_gemm_fwd(const FwdArgs& a, hipStream_t s);

// dX[M, N] = sum_g dY[:, acol_g : acol_g + n_out_g] W_g + Aext Bext^T, contraction over
// the stacked n_out of up to three weights sharing n_in = N.
struct BwdSeg {
  WeightRef w;
  int32_t a_col0 = 0;              // first column of this segment in dY
};
struct BwdArgs {
  const uint16_t* dy = nullptr; int32_t lddy = 0;   // bf16 [M, sum n_out]
  int32_t M = 0, N = 0;                             // N = n_in shared by the segments
  int32_t n_segs = 0;
  BwdSeg seg[kMaxGroups];
  const uint16_t* aext = nullptr; int32_t ldaext = 0; int32_t kx = 0;   // bf16 [M, kx]
  const uint16_t* bext = nullptr; int32_t ldbext = 0;                   // bf16 [N, kx]
  float* out32 = nullptr; uint16_t* out16 = nullptr; int32_t ldo = 0;  // exactly one set
  // float32 [M, ldo] added to the product before it is written (may be out32 itself:
  // every element is read and written by the same thread), nullable
  const float* resid32 = nullptr;
  const float* levels = nullptr;
  int32_t format = WF_NF4;
  // SwiGLU backward: the product is d(act); with gate, up from gu32 (float32 [M, ldgu],
  // up at column + N) out16 receives dgate | dup (bf16 [M, ldo], dup at column + N)
  const float* gu32 = nullptr; int32_t ldgu = 0;
  SplitTiles sk;
};
hipError_t launch_gemm_bwd(const BwdArgs& a, hipStream_t s);

// Generic batched bf16 MFMA GEMM: C(m,n) = alpha * sum_k A(m,k) B(n,k) + beta * C(m,n).
// Element addresses: A + zoffA + m*sAm + k*sAk with sAk == 1 (A_K) or sAm == 1 (A_M);
// likewise B.  Batch z in [0, nz): zoff = (z / zdiv) * s1 + ((z % zdiv) / zgrp) * s2.
struct ZStride { int64_t s1 = 0, s2 = 0; int32_t grp = 1; };
struct GemmArgs {
  const uint16_t* A = nullptr; int64_t sAm = 0, sAk = 0; ZStride zA;
  const uint16_t* B = nullptr; int64_t sBn = 0, sBk = 0; ZStride zB;
  void* C = nullptr; int64_t sCm = 0, sCn = 0; ZStride zC; int32_t c_f32 = 1;
  int32_t M = 0, N = 0, K = 0, nz = 1, zdiv = 1;
  float alpha = 1.f, beta = 0.f;
  int32_t causal = 0;   // 1: skip tiles with n0 > m_last; 2: contraction k <= m only; 3: k >= m only
  // split-K: ksplit > 1 splits the contraction into ksplit chunks whose float32
  // partial results go to `partial` ([ksplit][nz][M][N]); a second kernel sums the
  // chunks in order (deterministic) and applies alpha / beta.
  int32_t ksplit = 1;
  float* partial = nullptr;
};
hipError_t launch_gemm_generic(const GemmArgs& a, hipStream_t s);

// Products over tokens for the LoRA gradients, several per launch:
// C_d[m][n - d ncols] (=, or += with beta 1) sum_t A[t][m] B[t][n] for n in
// [d ncols, (d + 1) ncols), kept where n - d ncols < nvalid and C_d is set.
constexpr int kMaxTcJobs = 4;
struct TcJob {
  const uint16_t* A = nullptr; int32_t lda = 0; int32_t M = 0;   // bf16 [T, lda], 16-byte aligned
  const uint16_t* B = nullptr; int32_t ldb = 0; int32_t N = 0;   // bf16 [T, ldb], N <= 3 ncols
  float* C[3] = {nullptr, nullptr, nullptr};
  int64_t scm = 0, scn = 0;                                      // element (m, n') at m scm + n' scn
  int32_t ncols = 0, nvalid = 0;
};
struct TcArgs {
  TcJob job[kMaxTcJobs]; int32_t n_jobs = 0;
  int32_t T = 0;
  float beta = 0.f;
  float* partial = nullptr; int64_t partial_floats = 0;          // scratch for token runs
};
hipError_t launch_lora_tc(const TcArgs& a, hipStream_t s);

// Products over features for the LoRA down projections and gradients, several per
// launch: out[t][n] = bf16(alpha * sum_k X[t][k] W[n][k]) for t < T, n < N.
constexpr int kMaxFcJobs = 4;
struct FcJob {
  const uint16_t* X = nullptr; int32_t ldx = 0;   // bf16 [T, ldx], K contiguous, 16-byte aligned
  const uint16_t* W = nullptr;                    // bf16 [N, K]
  int32_t K = 0, N = 0;                           // K % 8 == 0
  float alpha = 1.f;
  uint16_t* out = nullptr; int32_t ldo = 0;       // bf16 [T, ldo]
};
struct FcArgs {
  FcJob job[kMaxFcJobs]; int32_t n_jobs = 0;
  int32_t T = 0;
};
hipError_t launch_lora_fc(const FcArgs& a, hipStream_t s);

// Causal grouped-query attention over batch sequences of S tokens, flash style.
// qkv: bf16 [batch * S, ldqkv], q heads at columns h * hd, k heads from qd, v heads
// from qd + kvd; q head h reads kv head h / (hq / hkv).  hd is 64 or 128.
struct AttnArgs {
  const uint16_t* qkv = nullptr; int32_t ldqkv = 0;
  int32_t qd = 0, kvd = 0;
  int32_t batch = 0, S = 0, hq = 0, hkv = 0, hd = 0;
  float scale = 0.f;                                  // 1 / sqrt(hd)
  uint16_t* out = nullptr; int32_t ldo = 0;           // O, bf16 [batch * S, ldo]
  float* out32 = nullptr;                             // O before rounding, float32, same layout (forward:
                                                      // written if set; backward: read)
  float* lse = nullptr;                               // [batch * hq * S] base-2 log-sum-exp of scale * log2(e) * S
  const uint16_t* dout = nullptr; int32_t lddo = 0;   // backward: dO, bf16 like O
  float* dd = nullptr;                                // backward scratch [batch * hq * S]: rowsum(dO * O)
  float* dqkv = nullptr; int32_t lddqkv = 0;          // backward: float32 dq | dk | dv, layout of qkv
  // backward, optional: float32 [batch * S, 2 kvd] (dk | dv).  When set and each kv head
  // has an even number of q heads, dk, dv of the second half of each group's q heads go
  // here, those of the first half to dqkv; the caller adds the two (see
  // launch_rope_bwd_convert).  When unset, dqkv receives the whole sums.
  float* dkv2 = nullptr;
  // backward, optional: dq in bf16 with the inverse rotary embedding already applied
  // (rope.hpp; rope_tab[pos * hd/2 + i] = (cos, sin)), [batch * S, lddq16], instead of
  // float32 in dqkv (whose q columns are then left as they were)
  uint16_t* dq16 = nullptr; int32_t lddq16 = 0;
  const float2* rope_tab = nullptr;
  // forward: per query row (m, l) = the row maximum of the base-2 scaled scores and the sum
  // of exp2(t - m), [batch * hq * S]; written if stats_out is set; if stats_in holds the
  // values of an earlier forward over the same q, k, the first pass is skipped
  float2* stats_out = nullptr;
  const float2* stats_in = nullptr;
};
// O and lse
hipError_t launch_attn_fwd(const AttnArgs& a, hipStream_t s);
// dq, dk, dv from dO, O, lse (dk, dv summed over each kv head's q heads)
hipError_t launch_attn_bwd(const AttnArgs& a, hipStream_t s);

// Batched float32 -> bf16 layout conversions (LoRA operands), one launch.
struct ConvJob {
  const float* src = nullptr; int64_t lds = 0;
  uint16_t* dst = nullptr; int64_t ldd = 0;
  int32_t rows = 0, cols = 0, pad_cols = 0, transpose = 0;
  float scale = 1.f;
};
constexpr int kMaxConvJobs = 32;
struct ConvBatch { ConvJob job[kMaxConvJobs]; int32_t n = 0; };
hipError_t launch_convert_batch(const ConvBatch& b, hipStream_t s);

// Glue kernels.
// x is bf16 (x16) or float32 (x32): exactly one is set
hipError_t launch_rmsnorm_fwd(const uint16_t* x16, const float* x32, const uint16_t* g, uint16_t* y, float* rstd,
                              int32_t T, int32_t D, float eps, hipStream_t s);
// dx = dres + rmsnorm_bwd(dn); x bf16 or float32; writes float32 and/or bf16
hipError_t launch_rmsnorm_bwd(const float* dn, const uint16_t* x16, const float* x32, const uint16_t* g,
                              const float* rstd, const float* dres32, const uint16_t* dres16, float* dx32,
                              uint16_t* dx16, int32_t T, int32_t D, hipStream_t s);
// The first `width` columns of float32 rows [T, stride ld] -> bf16 rows of the same
// stride, inverse rotary embedding (rope.hpp) on the first nh heads.  With add set,
// columns [add_col0, width) first get add[t * add_ld + column - add_col0] added
// (float32, same rounding order on every call).
hipError_t launch_rope_bwd_convert(const float* src, uint16_t* dst, int32_t ld, int32_t width, int32_t T, int32_t seq,
                                   int32_t nh, int32_t hd, const float2* tab, hipStream_t s,
                                   const float* add = nullptr, int32_t add_col0 = 0, int32_t add_ld = 0);
// rotary embedding in place on the first nh heads of a token-major [T, ld] bf16
// buffer; tab[pos * hd/2 + i] = (cos, sin) of pos * theta^(-2i/hd)
hipError_t launch_rope_tab(uint16_t* qk, int32_t ld, int32_t T, int32_t seq, int32_t nh, int32_t hd,
                           const float2* tab, int32_t inverse, hipStream_t s);
hipError_t launch_fill_f32(float* p, int64_t n, float v, hipStream_t s);
// p[0 .. n) = v (a bit pattern; the slot poisoning of LS_DEBUG_POISON)
hipError_t launch_fill_u32(uint32_t* p, int64_t n, uint32_t v, hipStream_t s);
hipError_t gemm_dequant_init();
// gu float32 [T, 2I] (gate | up) -> act bf16 [T, I]
hipError_t launch_swiglu_fwd(const float* gu, int32_t I, uint16_t* act, int32_t T, hipStream_t s);
// float32 [rows, cols] (row stride lds) -> bf16 [rows, ldd] scaled, columns >= cols zero up to ldd
hipError_t launch_f32_to_bf16(const float* src, int64_t lds, uint16_t* dst, int64_t ldd, int32_t rows,
                              int32_t cols, int32_t pad_cols, float scale, int32_t transpose, hipStream_t s);
hipError_t launch_dequant(const WeightRef& w, int32_t format, const float* levels, uint16_t* out, hipStream_t s);

// ---- AdamW over the adapters: one launch over a table of chunks, each at most
// kAdamChunk elements of one tensor (param p, gradient g, moments m, v).
constexpr int kAdamChunk = 8192;
struct AdamChunk {
  float* p;
  const float* g;
  float* m;
  float* v;
  uint32_t n;      // elements, 1 .. kAdamChunk
  uint32_t vec4;   // 1: every pointer 16-byte aligned and n % 4 == 0
};
// per-step constants, from the step count on the host in double precision
struct AdamHyper {
  float decay_mul;      // 1 - lr * weight_decay
  float beta1, one_m_beta1, beta2, one_m_beta2;
  float step_size;      // lr / (1 - beta1^t)
  float inv_bc2_sqrt;   // 1 / sqrt(1 - beta2^t)
  float eps;
};
hipError_t launch_adamw(const AdamChunk* chunks, int32_t n_chunks, const AdamHyper& h, hipStream_t s);

// ---- output head and loss over vocabulary slices (head.hip)
// fold a slice's float32 logits [T, vs] (row stride ldz, vocabulary columns v0..) into
// per-token running max m, sum s of exp(z - m), and the label's logit
hipError_t launch_ce_stats(const float* Z, int32_t ldz, int32_t vs, int32_t v0, const int32_t* labels, int32_t T,
                           int32_t vocab, float* m, float* s, float* zlab, bool first, hipStream_t st);
// per-sequence log-prob sums, the loss (LS_LOSS_SFT / LS_LOSS_DPO) and the per-sequence
// coefficient dL/dlog p; rm/rs/rz null for SFT.  out: loss, labelled tokens, policy
// sums [T/seq], reference sums [T/seq]
hipError_t launch_loss_finalize(int32_t kind, float beta, int32_t T, int32_t seq, int32_t vocab, const int32_t* labels,
                                const float* pm, const float* ps, const float* pz, const float* rm, const float* rs,
                                const float* rz, float* coef, float* out, hipStream_t st);
// dz = coef (onehot(label) - softmax) of a slice, bf16 [T, vs] with row stride ldz
hipError_t launch_ce_grad(const float* Z, int32_t ldz, int32_t vs, int32_t v0, const int32_t* labels, int32_t T,
                          int32_t seq, int32_t vocab, const float* m, const float* s, const float* coef, uint16_t* dz,
                          hipStream_t st);

// ---- adapter files (host only): the safetensors container with PEFT names and a
// CRC-32 record per tensor.  names/shapes come from the stack configuration.
struct AdapterEntry {
  std::string name;
  int32_t layer, proj, which;   // which: 0 = A [r, in], 1 = B [out, r]
  int64_t rows, cols;
  uint64_t offset = 0;          // byte offset of the data in the file's data section
};
std::vector<AdapterEntry> adapter_entries(const ls_config& c);
uint32_t crc32_bytes(const void* data, size_t n);
// Writes entries (with data[i] = host float32 rows*cols of entry i); "" or an error.
std::string adapter_write(const ls_config& c, const std::vector<AdapterEntry>& e,
                          const std::vector<const float*>& data, const std::string& path);
// Checks the file against the stack; on success fills file_bytes and the entries'
// offsets (absolute, into file_bytes).  "" or the first problem.
std::string adapter_check(const ls_config& c, const std::string& path, std::vector<AdapterEntry>* e,
                          std::vector<uint8_t>* file_bytes);

}  // namespace lsq
