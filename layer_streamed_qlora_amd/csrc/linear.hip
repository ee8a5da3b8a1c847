// One LoRA projection outside any context: Y = X deq(W)^T + (alpha / r) (X A^T) B^T on
// caller buffers, with the same kernels the streamed stack uses for each projection
// (the rank-r down product, then the fused dequant GEMM with the low-rank term as a
// K-extension).  The formula is the LoRA projection over a frozen 4-bit base of
// "Fine-Tuning an 8B Parameter Model on a 4 GB Laptop GPU", section "LoRA and QLoRA:
// Train a Fraction of the Parameters".
//
// ls_lora_linear takes its scratch as a caller workspace; ls_lora_linear_noalloc uses a
// fixed device array of this file instead, for callers that cannot allocate.  Scratch
// layout (both): s X A^T as bf16 [M, r16], A in bf16 [r16, n_in] (rows r .. r16 zero), B
// in bf16 [n_out, r16] (columns r .. r16 zero), each region 256-byte aligned with 256
// bytes of slack.
#include <hip/hip_runtime.h>

#include <mutex>

#include "lsq_internal.hpp"

using namespace lsq;

namespace {

constexpr int kMaxDevices = 64;
constexpr uint64_t kScratchBytes = 12ull << 20;   // the fixed scratch of the no-alloc variant

// The 16 NF4 levels on each device, written once at set-up.
static __device__ float nf4_levels[16];
// The scratch of ls_lora_linear_noalloc, one copy per device for the life of the
// process.  In host code this name is only a stand-in, not a device address: the
// address used everywhere is the one hipGetSymbolAddress returns for each device.
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

struct DeviceState {
  bool ready = false;
  float* levels = nullptr;
  uint8_t* scratch = nullptr;
};
std::mutex g_mu;
DeviceState g_dev[kMaxDevices];

uint64_t al(uint64_t x) { return (x + 255) / 256 * 256; }

struct WsLayout {
  uint64_t hs = 0, a16 = 0, b16 = 0, total = 0;
};

WsLayout ws_layout(int64_t M, int64_t n_in, int64_t n_out, int r16) {
  WsLayout L;
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) { const uint64_t o = off; off = al(off + bytes + 256); return o; };
  L.hs = take(2ull * M * r16);
  L.a16 = take(2ull * r16 * n_in);
  L.b16 = take(2ull * n_out * r16);
  L.total = off;
  return L;
}

// Per-device set-up, once, with the device current: the level table and the scratch
// address.  Synchronous (a caller that captures graphs makes one call first).
hipError_t device_setup(int dev, DeviceState** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  DeviceState& d = g_dev[dev];
  if (!d.ready) {
    void* p = nullptr;
    hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    d.scratch = static_cast<uint8_t*>(p);
    void* q = nullptr;
    e = hipGetSymbolAddress(&q, HIP_SYMBOL(nf4_levels));
    if (e != hipSuccess) return e;
    float lv[16];
    nf4_codebook_host(lv);
    e = hipMemcpy(q, lv, sizeof(lv), hipMemcpyHostToDevice);
    if (e != hipSuccess) return e;
    d.levels = static_cast<float*>(q);
    d.ready = true;
  }
  *out = &d;
  return hipSuccess;
}

thread_local std::string t_err;

ls_status bad(const char* msg) {
  t_err = msg;
  return LS_ERR_INVALID;
}

ls_status check_args(const ls_weight* w, const void* X, int32_t M, const float* A, const float* B, int32_t r,
                     const void* Y) {
  if (!w || !X || !Y) return bad("null weight, X or Y");
  if (M < 0) return bad("M must be >= 0");
  if (w->n_out <= 0 || w->n_out % 4 != 0 || w->n_in <= 0 || w->n_in % 16 != 0)
    return bad("need n_out a positive multiple of 4 and n_in a positive multiple of 16");
  if (w->quant != LS_QUANT_NF4 && w->quant != LS_QUANT_BF16) return bad("unknown quant");
  if (!w->w) return bad("null weight data");
  if (w->quant == LS_QUANT_NF4 && (w->double_quant ? (!w->qabs || !w->scale2 || !w->mean) : !w->absmax))
    return bad("null NF4 scales");
  if (r < 0 || r > 64) return bad("r must be in 0..64");
  if (r > 0 && (!A || !B)) return bad("null A or B with r > 0");
  if ((reinterpret_cast<uintptr_t>(X) & 15) != 0) return bad("X must be 16-byte aligned");
  return LS_OK;
}

WeightRef to_ref(const ls_weight* w) {
  WeightRef r;
  r.w = static_cast<const uint8_t*>(w->w);
  if (w->quant == LS_QUANT_NF4) {
    if (w->double_quant) {
      r.qabs = w->qabs; r.scale2 = w->scale2; r.mean = w->mean;
    } else {
      r.absmax = w->absmax;
    }
  }
  r.n_out = w->n_out;
  r.n_in = w->n_in;
  return r;
}

int fmt_of(const ls_weight* w) {
  if (w->quant == LS_QUANT_BF16) return WF_BF16;
  return w->double_quant ? WF_NF4_DQ : WF_NF4;
}

// The enqueue: scratch at `ws` (layout L).
ls_status run(const ls_weight* w, const void* X, int32_t M, const float* A, const float* B, int32_t r, float alpha,
              void* Y, uint8_t* ws, const WsLayout& L, const float* levels, hipStream_t s) {
  if (M == 0) return LS_OK;
  const int r16 = (r + 15) / 16 * 16;
  const int n_in = w->n_in, n_out = w->n_out;
  uint16_t* hs = reinterpret_cast<uint16_t*>(ws + L.hs);
  uint16_t* a16 = reinterpret_cast<uint16_t*>(ws + L.a16);
  uint16_t* b16 = reinterpret_cast<uint16_t*>(ws + L.b16);
  auto chk = [](hipError_t e) { if (e != hipSuccess) { t_err = hipGetErrorString(e); return LS_ERR_HIP; } return LS_OK; };
  ls_status st;
  if (r > 0) {
    // rows r .. r16 of A16 must read as zero (the scratch keeps earlier contents)
    if (r16 > r && (st = chk(launch_fill_u32(reinterpret_cast<uint32_t*>(a16 + (uint64_t)r * n_in),
                                             (int64_t)(r16 - r) * n_in / 2, 0u, s))))
      return st;
    ConvBatch cb;
    ConvJob j;
    j.src = A; j.lds = n_in; j.dst = a16; j.ldd = n_in; j.rows = r; j.cols = n_in; j.pad_cols = n_in;
    cb.job[cb.n++] = j;
    ConvJob k;
    k.src = B; k.lds = r; k.dst = b16; k.ldd = r16; k.rows = n_out; k.cols = r; k.pad_cols = r16;
    cb.job[cb.n++] = k;
    if ((st = chk(launch_convert_batch(cb, s)))) return st;
    FcArgs fa;
    fa.T = M;
    FcJob& fj = fa.job[fa.n_jobs++];
    fj.X = static_cast<const uint16_t*>(X); fj.ldx = n_in; fj.W = a16; fj.K = n_in; fj.N = r16;
    fj.alpha = alpha / (float)r; fj.out = hs; fj.ldo = r16;
    if ((st = chk(launch_lora_fc(fa, s)))) return st;
  }
  FwdArgs f;
  f.x = static_cast<const uint16_t*>(X); f.ldx = n_in; f.M = M; f.K = n_in; f.n_groups = 1;
  f.g[0].w = to_ref(w);
  f.g[0].bext = r > 0 ? b16 : nullptr;
  f.aext = hs; f.ldaext = r16; f.kx = r > 0 ? r16 : 0;
  f.y = static_cast<uint16_t*>(Y); f.ldy = n_out;
  f.levels = levels; f.format = fmt_of(w);
  return chk(launch_gemm_fwd(f, s));
}

}  // namespace

extern "C" {

uint64_t ls_lora_linear_workspace_bytes(int32_t M, int32_t n_in, int32_t n_out, int32_t r) {
  if (M < 0 || n_in < 0 || n_out < 0 || r < 0 || r > 64) return 0;
  return ws_layout(M, n_in, n_out, (r + 15) / 16 * 16).total;
}

ls_status ls_lora_linear(const ls_weight* w, const void* X, int32_t M, const float* A, const float* B, int32_t r,
                         float alpha, void* Y, void* workspace, uint64_t workspace_bytes, void* stream) {
  if (ls_status st = check_args(w, X, M, A, B, r, Y)) return st;
  const WsLayout L = ws_layout(M, w->n_in, w->n_out, (r + 15) / 16 * 16);
  if (!workspace || workspace_bytes < L.total) return bad("workspace missing or smaller than ls_lora_linear_workspace_bytes");
  if ((reinterpret_cast<uintptr_t>(workspace) & 255) != 0) return bad("workspace must be 256-byte aligned");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) { t_err = "hipGetDevice failed"; return LS_ERR_HIP; }
  DeviceState* d = nullptr;
  if (hipError_t e = device_setup(dev, &d); e != hipSuccess) { t_err = hipGetErrorString(e); return LS_ERR_HIP; }
  return run(w, X, M, A, B, r, alpha, Y, static_cast<uint8_t*>(workspace), L, d->levels, (hipStream_t)stream);
}

ls_status ls_lora_linear_noalloc(const ls_weight* w, const void* X, int32_t M, const float* A, const float* B,
                                 int32_t r, float alpha, void* Y, void* stream) {
  if (ls_status st = check_args(w, X, M, A, B, r, Y)) return st;
  const WsLayout L = ws_layout(M, w->n_in, w->n_out, (r + 15) / 16 * 16);
  if (L.total > kScratchBytes)
    return bad("sizes exceed the fixed scratch of ls_lora_linear_noalloc (12 MiB: "
               "ls_lora_linear_workspace_bytes must not exceed 12582912)");
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) { t_err = "hipGetDevice failed"; return LS_ERR_HIP; }
  DeviceState* d = nullptr;
  if (hipError_t e = device_setup(dev, &d); e != hipSuccess) { t_err = hipGetErrorString(e); return LS_ERR_HIP; }
  return run(w, X, M, A, B, r, alpha, Y, d->scratch, L, d->levels, (hipStream_t)stream);
}

const char* ls_lora_linear_error(void) { return t_err.c_str(); }

}  // extern "C"
