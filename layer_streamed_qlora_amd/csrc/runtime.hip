// Host runtime of liblsq: pinned layer store, the device slot pool with its copy
// stream and event fencing, the per-layer executor (forward, adapters-off reference
// pass, recompute backward) and the C ABI declared in include/ls.h.
//
// What is streamed and when follows the pages: the frozen base stays in host RAM and
// each decoder layer is copied into a two-buffer device pool so the next layer loads
// while the current one computes; backward reads every layer again for the
// checkpoint recomputation (the lachieslifestyle.com Soup how-to, section "What Soup
// layer streaming changes"); the copies run on a dedicated stream and peak device
// memory is bounded by one layer's worth of weights per slot ("Soup CLI fine-tunes
// Llama-3.1-8B on a 4 GB laptop GPU ...", second paragraph); the DPO reference is the
// same streamed layer with the adapters off (same page, third paragraph).
#include <hip/hip_runtime.h>

#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <array>
#include <atomic>
#include <cerrno>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "lsq_internal.hpp"

using namespace lsq;

namespace {

constexpr int kPad = 256;    // slack after every workspace region (8-element group loads)
constexpr int kMaxSplit = 16;
// compute units the split-tile scratch of the dequant GEMMs serves (MI355X: 256); on
// a device with more, the GEMMs run whole tiles only
constexpr int kSplitSlots = 256;

struct LoraReg {
  const float* A = nullptr;
  const float* B = nullptr;
  float* dA = nullptr;
  float* dB = nullptr;
};

// Byte offsets of every device region; the same function sizes the plan for
// ls_plan_bytes and carves the single device allocation in ls_create.
struct DevPlan {
  uint64_t total = 0;
  uint64_t slots = 0, ck = 0, xref = 0;
  // the activations a layer's forward or recompute writes and its backward reads: two
  // sets, layer l using set l % 2, so that the recompute of layer l - 1 can run while
  // the backward of layer l still reads its own
  uint64_t n1[2] = {}, qkv[2] = {}, att[2] = {}, hb[2] = {}, n2[2] = {}, gu[2] = {}, act[2] = {};
  uint64_t rstd1[2] = {}, rstd2[2] = {}, lse[2] = {}, o32[2] = {};
  uint64_t hs = 0, gs = 0, dd = 0, astats = 0;
  uint64_t dya = 0, dyb = 0, dh32 = 0, dh16 = 0, dgu = 0, datt = 0, dqkv = 0, dqkv32 = 0, dn32 = 0;
  uint64_t dkv2 = 0;   // dk | dv of the second half of each kv head's q heads, float32
  uint64_t lora = 0, lora_per_layer = 0, partial = 0, partial_bytes = 0;
  // split-tile scratch of the dequant GEMMs, one set per stream that launches them
  // (the compute stream and the recompute stream): float32 partial tiles, counters
  uint64_t skpart[2] = {}, skcnt[2] = {};
  uint64_t levels = 0, rope = 0;
  // AdamW: moments m then v (moment_elems floats each) and the chunk table
  uint64_t moments = 0, moment_elems = 0, adam_tab = 0, adam_max_chunks = 0;
  // output head: vocabulary slices of head_rows rows, each in one slot (pool index
  // n_layers + j); logits [T, ldz] float32, their gradient bf16, per-token statistics
  int32_t head_rows = 0, head_slices = 0, ldz = 0;
  uint64_t gfin = 0, hyn = 0, hynr = 0, hrstd = 0, hrstd2 = 0, hz = 0, hdz = 0, hdyn = 0;
  uint64_t hpm = 0, hps = 0, hpz = 0, hrm = 0, hrs = 0, hrz = 0, hcoef = 0;
  // per-layer LoRA operand offsets (relative to the layer's LoRA base)
  uint64_t a16[LS_N_PROJ] = {}, bx16[LS_N_PROJ] = {}, bxt16[LS_N_PROJ] = {};
  uint64_t at_qkv = 0, at_o = 0, at_gu = 0, at_d = 0;
  int n_slots = 0;
};

inline int r16_of(const ls_config& c) { return (c.lora_r + 15) / 16 * 16; }

DevPlan make_plan(const ls_config& c, const BlobLayout& L) {
  DevPlan P;
  uint64_t off = 0;
  auto take = [&](uint64_t bytes) { off = align_up(off, kAlign); uint64_t o = off; off += bytes + kPad; return o; };
  const uint64_t T = (uint64_t)c.max_tokens, h = c.hidden, I = c.intermediate;
  const uint64_t qd = (uint64_t)c.n_heads * c.head_dim, kvd = (uint64_t)c.n_kv_heads * c.head_dim;
  const uint64_t qkvd = qd + 2 * kvd;
  const uint64_t r16 = r16_of(c), R7 = 7 * r16;
  if (c.vocab > 0) {
    // rows per head slice: as many bf16 rows of the head as fit one layer slot, rounded
    // down to a multiple of 256 (64 for small slots)
    int64_t vs = (int64_t)(L.bytes / (2ull * (uint64_t)c.hidden));
    vs -= vs >= 256 ? vs % 256 : vs % 64;
    vs = std::max<int64_t>(1, std::min<int64_t>(vs, c.vocab));
    P.head_rows = (int32_t)vs;
    P.head_slices = (int32_t)((c.vocab + vs - 1) / vs);
    P.ldz = (int32_t)((vs + 63) / 64 * 64);
  }
  P.n_slots = c.resident ? c.n_layers + P.head_slices : c.n_buffers;
  P.slots = take(L.bytes * (uint64_t)P.n_slots);
  P.ck = take(2 * T * h * (uint64_t)c.n_layers);
  P.xref = take(2 * 2 * T * h);
  for (int k = 0; k < 2; ++k) {
    P.n1[k] = take(2 * T * h);
    P.qkv[k] = take(2 * T * qkvd);
    P.att[k] = take(2 * T * qd);
    P.hb[k] = take(4 * T * h);        // residual stream after attention, float32
    P.n2[k] = take(2 * T * h);
    // float32 gate | up outputs, or, with the paired gate | up kernel (2 r16 <= 64),
    // the down projection's float32 d(act) in the backward
    P.gu[k] = take(4 * T * (2 * r16 <= 64 ? 1 : 2) * I);
    P.act[k] = take(2 * T * I);
    P.rstd1[k] = take(4 * T);
    P.rstd2[k] = take(4 * T);
    P.lse[k] = take(4 * T * (uint64_t)c.n_heads);
    P.o32[k] = take(4 * T * qd);
  }
  // s X A^T of every layer, kept from the forward for the recompute and the dB products
  P.hs = take(2 * T * R7 * (uint64_t)c.n_layers);
  P.gs = take(2 * T * R7);
  P.dd = take(4 * T * (uint64_t)c.n_heads);
  // attention row statistics (max, sum) of every layer's forward, read by its recompute
  P.astats = take(8 * T * (uint64_t)c.n_heads * (uint64_t)c.n_layers);
  P.dya = take(2 * T * h);
  P.dyb = take(2 * T * h);
  P.dh32 = take(4 * T * h);
  P.dh16 = take(2 * T * h);
  P.dgu = take(2 * T * 2 * I);
  P.datt = take(2 * T * qd);
  P.dqkv = take(2 * T * qkvd);
  P.dqkv32 = take(4 * T * qkvd);
  P.dkv2 = take(4 * T * 2 * kvd);
  P.dn32 = take(4 * T * (std::max(h, qd)));
  // LoRA operands in bf16, per layer
  uint64_t lo = 0;
  auto ltake = [&](uint64_t bytes) { lo = align_up(lo, kAlign); uint64_t o = lo; lo += bytes + kPad; return o; };
  // A16 of projections that share an input are stacked contiguously, so one GEMM
  // computes the whole group's s*X*A^T: [q|k|v] and [gate|up] are [n*r16, n_in].
  P.a16[LS_PROJ_Q] = ltake(2 * 3 * r16 * h);
  P.a16[LS_PROJ_K] = P.a16[LS_PROJ_Q] + 2 * r16 * h;
  P.a16[LS_PROJ_V] = P.a16[LS_PROJ_Q] + 4 * r16 * h;
  P.a16[LS_PROJ_O] = ltake(2 * r16 * qd);
  P.a16[LS_PROJ_GATE] = ltake(2 * 2 * r16 * h);
  P.a16[LS_PROJ_UP] = P.a16[LS_PROJ_GATE] + 2 * r16 * h;
  P.a16[LS_PROJ_DOWN] = ltake(2 * r16 * I);
  for (int p = 0; p < LS_N_PROJ; ++p) {
    int32_t n_out, n_in;
    proj_dims(c, p, &n_out, &n_in);
    P.bx16[p] = ltake(2 * (uint64_t)n_out * r16);
    P.bxt16[p] = ltake(2 * (uint64_t)n_out * r16);
  }
  // A^T stacked per group, [n_in, group_r16]: q|k|v, o, gate|up, down
  P.at_qkv = ltake(2 * h * 3 * r16);
  P.at_o = ltake(2 * qd * r16);
  P.at_gu = ltake(2 * h * 2 * r16);
  P.at_d = ltake(2 * I * r16);
  P.lora_per_layer = align_up(lo, kAlign);
  P.lora = take(P.lora_per_layer * (uint64_t)c.n_layers);
  // split-K partials of the rank-r reductions: up to kMaxSplit chunks of [rows, r16]
  P.partial_bytes = 4ull * kMaxSplit * std::max<uint64_t>(std::max<uint64_t>(T, I), std::max<uint64_t>(h, qkvd)) * 3 * r16;
  P.partial = take(P.partial_bytes);
  {
    // only when some dequant GEMM has more 256 x 256 tiles than one round of compute units
    const uint64_t widest = std::max<uint64_t>(std::max<uint64_t>(qkvd, 2 * I), std::max<uint64_t>(std::max(h, qd), (uint64_t)P.head_rows));
    if ((T + 255) / 256 * ((widest + 255) / 256) > (uint64_t)kSplitSlots)
      for (int k = 0; k < 2; ++k) {
        P.skpart[k] = take(4ull * 256 * 256 * kSplitSlots);
        P.skcnt[k] = take(4ull * kSplitSlots);
      }
  }
  P.levels = take(64);
  P.rope = take(8ull * (uint64_t)c.max_seq * (uint64_t)(c.head_dim / 2));
  if (c.adamw) {
    for (const AdapterEntry& e : adapter_entries(c)) {
      const uint64_t n = (uint64_t)e.rows * (uint64_t)e.cols;
      P.moment_elems += n;
      P.adam_max_chunks += (n + kAdamChunk - 1) / kAdamChunk;
    }
    P.moments = take(8 * P.moment_elems);
    P.adam_tab = take(sizeof(AdamChunk) * P.adam_max_chunks);
  }
  if (c.vocab > 0) {
    P.gfin = take(2 * h);
    P.hyn = take(2 * T * h);
    P.hynr = take(2 * T * h);
    P.hrstd = take(4 * T);
    P.hrstd2 = take(4 * T);
    P.hz = take(4 * T * (uint64_t)P.ldz);
    P.hdz = take(2 * T * (uint64_t)P.ldz);
    P.hdyn = take(4 * T * h);
    P.hpm = take(4 * T); P.hps = take(4 * T); P.hpz = take(4 * T);
    P.hrm = take(4 * T); P.hrs = take(4 * T); P.hrz = take(4 * T);
    P.hcoef = take(4 * T);
  }
  P.total = align_up(off, kAlign);
  return P;
}

// Event-pair recorder for profile = 1.
struct Prof {
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  struct KRec { int cls; size_t e0, e1; double flop, bytes; };
  std::vector<KRec> krecs;
  std::vector<std::pair<size_t, size_t>> copies, computes;
  size_t origin = (size_t)-1;
  hipError_t next(hipEvent_t* ev, size_t* idx) {
    if (used == pool.size()) {
      hipEvent_t e;
      hipError_t r = hipEventCreate(&e);
      if (r != hipSuccess) return r;
      pool.push_back(e);
    }
    *idx = used;
    *ev = pool[used++];
    return hipSuccess;
  }
  void reset() { used = 0; krecs.clear(); copies.clear(); computes.clear(); origin = (size_t)-1; }
};

}  // namespace

struct ls_ctx {
  ls_config cfg{};
  BlobLayout lay;
  DevPlan plan;
  int device = 0;
  hipStream_t cs = nullptr, ps = nullptr;
  bool own_cs = false, own_ps = false;
  // side stream of the adapter-gradient reductions (dA, dB): they run beside the
  // backward's dequant GEMMs, forked after each G product and joined before the next
  // layer's recompute overwrites what they read
  hipStream_t side = nullptr;
  hipEvent_t fork_ev = nullptr, join_ev = nullptr;
  bool side_pending = false;
  // the backward's recompute stream: the recompute of layer l - 1 runs on it while the
  // compute stream runs the backward of layer l.  Per activation set k (layer % 2):
  // rec_done[k] after a recompute, bp_done[k] after the backward that read the set,
  // side_done[k] after that backward's adapter-gradient reductions
  hipStream_t rs = nullptr;
  hipEvent_t rec_done[2] = {}, bp_done[2] = {}, side_done[2] = {};
  bool bp_rec[2] = {}, side_rec[2] = {};
  bool in_recompute = false;            // enqueueing a recompute (LS_PROFILE_GEMM skips it)
  int prof_layer = -1;                  // the forward's layer being enqueued (profile_stride)
  std::vector<uint8_t*> host;
  std::vector<char> staged;
  uint8_t* dbase = nullptr;
  std::vector<int> slot_layer;
  std::vector<hipEvent_t> ready, consumed;
  std::vector<char> ready_rec, cons_rec;
  std::vector<std::array<LoraReg, LS_N_PROJ>> lora;
  uint64_t lora_version = 1;            // bumped by every ls_set_lora
  // AdamW chunk table (host copy kept alive while its upload may be pending)
  std::vector<AdamChunk> adam_host;
  uint64_t adam_version = 0;
  double adam_elems = 0;
  bool prof_collected = false;
  bool head_staged = false;
  bool fwd_ref = false;                 // the last forward also ran the reference pass
  // LS_STORE_FILE: the store file, one pinned staging buffer per slot, one read job per
  // pool index (fixed contents: a job may be enqueued again before its last run ends)
  struct ReadJob {
    ls_ctx* c;
    uint8_t* buf;
    uint64_t off, len;
  };
  int fd = -1;
  bool uncached = false;                // pages dropped from the OS cache after use
  uint64_t stride = 0;                  // blob bytes rounded up to 4096 (file offsets, read sizes)
  std::vector<uint8_t*> staging;
  std::vector<ReadJob> jobs;
  std::atomic<int> store_err{0};
  std::atomic<uint64_t> store_reads{0};
  float levels_h[16];
  // race detection (read from the environment at ls_create): LS_DEBUG_POISON=1 fills a
  // slot with 0xFF bytes on the copy stream once its last reader is done, before the
  // next copy lands in it; LS_DEBUG_COPY_DELAY_US=n holds the copy stream n
  // microseconds (a host function) between that point and the copy
  bool dbg_poison = false;
  uint32_t dbg_delay_us = 0;
  // state
  bool fwd_valid = false, fwd_lora = false;
  int fwd_T = 0, fwd_batch = 0, fwd_seq = 0;
  bool in_flight = false;
  ls_status sticky = LS_OK;
  std::string err;
  ls_stats stats{};
  Prof prof;

  template <class T> T* dp(uint64_t off) const { return reinterpret_cast<T*>(dbase + off); }
  // split-tile scratch of the dequant GEMMs launched on stream s (the recompute stream
  // has its own set: its GEMMs run beside the compute stream's)
  SplitTiles split_scratch(hipStream_t s) const {
    SplitTiles t;
    const int k = s == rs ? 1 : 0;
    if (plan.skpart[k] == 0) return t;
    t.part = dp<float>(plan.skpart[k]);
    t.cnt = dp<uint32_t>(plan.skcnt[k]);
    t.slots = kSplitSlots;
    return t;
  }
};

static std::string g_create_err;

static ls_status fail(ls_ctx* c, ls_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  if (c) {
    c->err = buf;
    if (st == LS_ERR_HIP) c->sticky = LS_ERR_HIP;
  } else {
    g_create_err = buf;
  }
  return st;
}

#define HIPCHK(ctx, expr)                                                                    \
  do {                                                                                       \
    hipError_t _e = (expr);                                                                  \
    if (_e != hipSuccess) return fail((ctx), LS_ERR_HIP, "%s failed: %s", #expr, hipGetErrorString(_e)); \
  } while (0)

// ------------------------------------------------------------------ profiling
namespace {

struct KTimer {
  ls_ctx* c;
  int cls;
  double flop, bytes;
  size_t i0 = 0;
  bool on;
  hipStream_t s;
  KTimer(ls_ctx* ctx, int k, double f, double b, hipStream_t st = nullptr)
      : c(ctx), cls(k), flop(f), bytes(b),
        on(ctx->cfg.profile == LS_PROFILE_ALL ||
           (ctx->cfg.profile == LS_PROFILE_GEMM && k == LS_KC_GEMM_FWD && !ctx->in_recompute &&
            (ctx->cfg.profile_stride <= 1 || (ctx->prof_layer >= 0 && ctx->prof_layer % ctx->cfg.profile_stride == 0)))),
        s(st ? st : ctx->cs) {
    if (on) {
      hipEvent_t e;
      // a failed record drops this launch from the statistics (never the run)
      if (c->prof.next(&e, &i0) != hipSuccess || hipEventRecord(e, s) != hipSuccess) on = false;
    }
  }
  ~KTimer() {
    if (!on) return;
    hipEvent_t e;
    size_t i1;
    if (c->prof.next(&e, &i1) == hipSuccess && hipEventRecord(e, s) == hipSuccess)
      c->prof.krecs.push_back({cls, i0, i1, flop, bytes});
  }
};

struct Span {   // copy or per-layer compute interval
  ls_ctx* c;
  hipStream_t s;
  bool copy;
  size_t i0 = 0;
  bool on;
  Span(ls_ctx* ctx, hipStream_t st, bool is_copy) : c(ctx), s(st), copy(is_copy), on(ctx->cfg.profile == LS_PROFILE_ALL) {
    if (on) {
      hipEvent_t e;
      if (c->prof.next(&e, &i0) == hipSuccess && hipEventRecord(e, s) == hipSuccess) {
        if (c->prof.origin == (size_t)-1) c->prof.origin = i0;
      } else {
        on = false;
      }
    }
  }
  ~Span() {
    if (!on) return;
    hipEvent_t e;
    size_t i1;
    if (c->prof.next(&e, &i1) == hipSuccess && hipEventRecord(e, s) == hipSuccess)
      (copy ? c->prof.copies : c->prof.computes).push_back({i0, i1});
  }
};

void collect_profile(ls_ctx* c) {
  Prof& P = c->prof;
  for (int k = 0; k < LS_KC_N; ++k) {
    c->stats.k_launches[k] = 0;
    c->stats.k_ms[k] = c->stats.k_flop[k] = c->stats.k_bytes[k] = 0.0;
  }
  c->stats.last_copy_ms = c->stats.last_compute_ms = c->stats.last_overlap_ms = c->stats.last_span_ms = 0.0;
  if (!c->cfg.profile) return;
  auto el = [&](size_t a, size_t b) {
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, P.pool[a], P.pool[b]) != hipSuccess) return 0.0;
    return (double)ms;
  };
  for (const auto& r : P.krecs) {
    c->stats.k_launches[r.cls] += 1;
    c->stats.k_ms[r.cls] += el(r.e0, r.e1);
    c->stats.k_flop[r.cls] += r.flop;
    c->stats.k_bytes[r.cls] += r.bytes;
  }
  if (P.origin == (size_t)-1) return;   // no copy / compute intervals were recorded
  std::vector<std::pair<double, double>> cp, cm;
  double last = 0.0;
  for (auto& iv : P.copies) { cp.push_back({el(P.origin, iv.first), el(P.origin, iv.second)}); last = std::max(last, cp.back().second); }
  for (auto& iv : P.computes) { cm.push_back({el(P.origin, iv.first), el(P.origin, iv.second)}); last = std::max(last, cm.back().second); }
  // compute intervals of the compute and the recompute stream overlap each other: merge
  // them into their union before measuring the overlap with the copies
  std::sort(cm.begin(), cm.end());
  std::vector<std::pair<double, double>> um;
  for (auto& a : cm) {
    if (!um.empty() && a.first <= um.back().second) um.back().second = std::max(um.back().second, a.second);
    else um.push_back(a);
  }
  cm.swap(um);
  double cps = 0, cms = 0, ov = 0;
  for (auto& a : cp) cps += a.second - a.first;
  for (auto& a : cm) cms += a.second - a.first;
  for (auto& a : cp)
    for (auto& b : cm) {
      const double lo = std::max(a.first, b.first), hi = std::min(a.second, b.second);
      if (hi > lo) ov += hi - lo;
    }
  c->stats.last_copy_ms = cps;
  c->stats.last_compute_ms = cms;
  c->stats.last_overlap_ms = ov;
  c->stats.last_span_ms = last;
}

// ------------------------------------------------------------------ file store
// Host function on the copy stream: read one blob (job->len bytes at job->off) into the
// staging buffer.  No HIP call here; a failure is recorded for ls_sync.
void store_read(void* p) {
  auto* j = static_cast<ls_ctx::ReadJob*>(p);
  uint64_t done = 0;
  while (done < j->len) {
    const ssize_t r = pread(j->c->fd, j->buf + done, j->len - done, (off_t)(j->off + done));
    if (r < 0 && errno == EINTR) continue;
    if (r <= 0) {
      int expected = 0;
      j->c->store_err.compare_exchange_strong(expected, r < 0 ? errno : EIO);
      return;
    }
    done += (uint64_t)r;
  }
  if (j->c->uncached) posix_fadvise(j->c->fd, (off_t)j->off, (off_t)j->len, POSIX_FADV_DONTNEED);
  j->c->store_reads.fetch_add(1);
}

// The host buffer a layer (or head slice) is staged through: its pinned blob, or, with
// the file store, the first staging buffer, cleared (the blob's padding stays zero).
uint8_t* stage_buffer(ls_ctx* c, int l) {
  if (c->fd < 0) return c->host[l];
  std::memset(c->staging[0], 0, c->stride);
  return c->staging[0];
}

// After staging: write the blob to its place in the store file.
ls_status store_write(ls_ctx* c, int l, const uint8_t* blob) {
  if (c->fd < 0) return LS_OK;
  uint64_t done = 0;
  while (done < c->stride) {
    const ssize_t r = pwrite(c->fd, blob + done, c->stride - done, (off_t)((uint64_t)l * c->stride + done));
    if (r < 0 && errno == EINTR) continue;
    if (r <= 0) return fail(c, LS_ERR_INVALID, "write to the store file failed: %s", strerror(r < 0 ? errno : EIO));
    done += (uint64_t)r;
  }
  if (c->uncached) {
    const off_t off = (off_t)((uint64_t)l * c->stride);
    if (fdatasync(c->fd) != 0) return fail(c, LS_ERR_INVALID, "flush of the store file failed: %s", strerror(errno));
    posix_fadvise(c->fd, off, (off_t)c->stride, POSIX_FADV_DONTNEED);
  }
  return LS_OK;
}

// ------------------------------------------------------------------ pool
// Host function on the copy stream (LS_DEBUG_COPY_DELAY_US): widens every window in
// which a missing event wait would let the compute stream read a slot being refilled.
void copy_delay(void* p) { usleep(*static_cast<const uint32_t*>(p)); }

uint8_t* slot_ptr(ls_ctx* c, int layer) {
  const int s = c->cfg.resident ? layer : layer % c->cfg.n_buffers;
  return c->dbase + c->plan.slots + (uint64_t)s * c->lay.bytes;
}

// Pieces of a blob.  With copy_split a decoder layer crosses the link as kPieces pieces
// in the order its forward and its recompute first read them: g1, g2 and q|k|v; o;
// gate|up; down (contiguous in the blob layout), each followed by its own ready event,
// so the compute stream can start on a layer whose later pieces are still in flight.
// The slot is released as a whole (one consumed event per slot): the next copy into it
// waits for the last reader of every piece.  Head slices, and every blob without
// copy_split, are one piece.
constexpr int kPieces = 4;

int n_pieces(const ls_ctx* c, int l) {
  return c->cfg.copy_split && !c->cfg.resident && l < c->cfg.n_layers ? kPieces : 1;
}

void piece_range(const ls_ctx* c, int l, int g, uint64_t* off, uint64_t* len) {
  if (n_pieces(c, l) == 1) {
    *off = 0;
    *len = c->lay.bytes;
    return;
  }
  const uint64_t b[kPieces + 1] = {0, c->lay.p[LS_PROJ_O].off_w, c->lay.p[LS_PROJ_GATE].off_w,
                                   c->lay.p[LS_PROJ_DOWN].off_w, c->lay.bytes};
  *off = b[g];
  *len = b[g + 1] - b[g];
}

// Enqueue on the copy stream: bring layer l into its slot unless the slot still holds it.
ls_status ensure_copy(ls_ctx* c, int l) {
  if (c->cfg.resident) return LS_OK;
  const int s = l % c->cfg.n_buffers;
  if (c->slot_layer[s] == l) { c->stats.slot_hits++; return LS_OK; }
  if (c->cons_rec[s]) HIPCHK(c, hipStreamWaitEvent(c->ps, c->consumed[s], 0));
  uint8_t* dst = slot_ptr(c, l);
  if (c->dbg_poison) {
    HIPCHK(c, launch_fill_u32(reinterpret_cast<uint32_t*>(dst), (int64_t)(c->lay.bytes / 4), 0xFFFFFFFFu, c->ps));
    c->stats.poison_fills += 1;
  }
  if (c->dbg_delay_us) HIPCHK(c, hipLaunchHostFunc(c->ps, copy_delay, &c->dbg_delay_us));
  // with the file store, the blob is first read into this slot's staging buffer (a host
  // function in stream order: it runs after the previous copy out of the buffer)
  if (c->fd >= 0) HIPCHK(c, hipLaunchHostFunc(c->ps, store_read, &c->jobs[l]));
  const uint8_t* src = c->fd >= 0 ? c->jobs[l].buf : c->host[l];
  const int np = n_pieces(c, l);
  for (int g = 0; g < np; ++g) {
    uint64_t off, len;
    piece_range(c, l, g, &off, &len);
    {
      Span sp(c, c->ps, true);
      HIPCHK(c, hipMemcpyAsync(dst + off, src + off, len, hipMemcpyHostToDevice, c->ps));
    }
    // a one-piece blob records every piece's event: a reader that waits per piece (the
    // next occupant of the slot may be split) then waits for the whole copy
    for (int k = np == 1 ? 0 : g; k < (np == 1 ? kPieces : g + 1); ++k) {
      HIPCHK(c, hipEventRecord(c->ready[s * kPieces + k], c->ps));
      c->ready_rec[s * kPieces + k] = 1;
    }
  }
  c->slot_layer[s] = l;
  c->stats.h2d_bytes += c->lay.bytes;
  c->stats.h2d_copies += 1;
  return LS_OK;
}

// Stream s (the compute stream unless given) waits for piece g of layer l (use_layer:
// every piece).
ls_status use_piece(ls_ctx* c, int l, int g, hipStream_t s = nullptr) {
  if (c->cfg.resident) return LS_OK;
  const int e = (l % c->cfg.n_buffers) * kPieces + g;
  if (c->ready_rec[e]) HIPCHK(c, hipStreamWaitEvent(s ? s : c->cs, c->ready[e], 0));
  return LS_OK;
}

ls_status use_layer(ls_ctx* c, int l, hipStream_t s = nullptr) {
  for (int g = 0; g < kPieces; ++g)
    if (ls_status st = use_piece(c, l, g, s)) return st;
  return LS_OK;
}

// Every reader of layer l's slot has been enqueued on the compute stream.
ls_status release_layer(ls_ctx* c, int l) {
  if (c->cfg.resident) return LS_OK;
  const int s = l % c->cfg.n_buffers;
  HIPCHK(c, hipEventRecord(c->consumed[s], c->cs));
  c->cons_rec[s] = 1;
  return LS_OK;
}

// Per-piece waits of one pass over a split layer: the pass's stream waits for a piece
// just before its first reader.  Disabled when the caller waited for the whole layer.
struct Fence {
  int l = 0;
  bool wait = false;
};
ls_status fence_wait(ls_ctx* c, const Fence& f, int g, hipStream_t s) { return f.wait ? use_piece(c, f.l, g, s) : LS_OK; }

// ------------------------------------------------------------------ executor
// s X A^T of layer l, bf16 [T, 7 r16] (row stride 7 r16), layers max_tokens rows apart
uint16_t* hs_of(const ls_ctx* c, int l) {
  return c->dp<uint16_t>(c->plan.hs) + (uint64_t)l * c->cfg.max_tokens * 7 * r16_of(c->cfg);
}

// The activation workspaces of set k (layer l uses set l % 2).
struct Acts {
  uint16_t *n1, *qkv, *att, *n2, *act;
  float *hb, *gu, *rstd1, *rstd2, *lse, *o32;
};
Acts acts_of(ls_ctx* c, int l) {
  const int k = l & 1;
  const DevPlan& P = c->plan;
  return Acts{c->dp<uint16_t>(P.n1[k]), c->dp<uint16_t>(P.qkv[k]), c->dp<uint16_t>(P.att[k]),
              c->dp<uint16_t>(P.n2[k]), c->dp<uint16_t>(P.act[k]), c->dp<float>(P.hb[k]),
              c->dp<float>(P.gu[k]), c->dp<float>(P.rstd1[k]), c->dp<float>(P.rstd2[k]),
              c->dp<float>(P.lse[k]), c->dp<float>(P.o32[k])};
}

struct Dims {
  int T, batch, seq, h, hq, hkv, hd, qd, kvd, qkvd, I, r, r16, R7;
  float s;
};

Dims dims_of(const ls_ctx* c, int batch, int seq) {
  Dims d;
  const ls_config& g = c->cfg;
  d.T = batch * seq; d.batch = batch; d.seq = seq;
  d.h = g.hidden; d.hq = g.n_heads; d.hkv = g.n_kv_heads; d.hd = g.head_dim;
  d.qd = d.hq * d.hd; d.kvd = d.hkv * d.hd; d.qkvd = d.qd + 2 * d.kvd;
  d.I = g.intermediate; d.r = g.lora_r; d.r16 = r16_of(g); d.R7 = 7 * d.r16;
  d.s = g.lora_alpha / (float)g.lora_r;
  return d;
}

int wformat(const ls_config& c) {
  if (c.quant == LS_QUANT_BF16) return WF_BF16;
  return c.double_quant ? WF_NF4_DQ : WF_NF4;
}

WeightRef wref(const ls_ctx* c, const uint8_t* blob, int p) {
  const ProjLayout& P = c->lay.p[p];
  WeightRef w;
  w.w = blob + P.off_w;
  if (c->cfg.quant == LS_QUANT_NF4) {
    if (c->cfg.double_quant) {
      w.qabs = blob + P.off_qabs;
      w.scale2 = reinterpret_cast<const float*>(blob + P.off_scale2);
      w.mean = reinterpret_cast<const float*>(blob + P.off_mean);
    } else {
      w.absmax = reinterpret_cast<const float*>(blob + P.off_absmax);
    }
  }
  w.n_out = P.n_out;
  w.n_in = P.n_in;
  return w;
}

bool lora_active(const ls_ctx* c, int l, int p) {
  return ((c->cfg.lora_mask >> p) & 1u) && c->lora[l][p].A && c->lora[l][p].B;
}

uint16_t* lora_base(ls_ctx* c, int l) { return c->dp<uint16_t>(c->plan.lora + (uint64_t)l * c->plan.lora_per_layer); }
uint16_t* lora_at(ls_ctx* c, int l, uint64_t off) { return reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(lora_base(c, l)) + off); }

double wbytes(const ls_ctx* c, int p) {   // stored bytes of projection p in a blob
  const ProjLayout& P = c->lay.p[p];
  if (c->cfg.quant == LS_QUANT_BF16) return (double)P.bytes_w;
  return (double)P.bytes_w + (c->cfg.double_quant ? (double)P.nblocks + 4.0 * P.ngroups : 4.0 * P.nblocks);
}

// bf16 copies of the adapters, one launch per layer: A16 [r16, in], Bx16 [out, r16],
// BxT16 [r16, out] and A^T stacked per group [in, group r16].
ls_status prep_lora(ls_ctx* c, int l, const Dims& d) {
  const int gcol[LS_N_PROJ] = {0, 1, 2, 0, 0, 1, 0};
  const uint64_t at_off[LS_N_PROJ] = {c->plan.at_qkv, c->plan.at_qkv, c->plan.at_qkv, c->plan.at_o,
                                      c->plan.at_gu, c->plan.at_gu, c->plan.at_d};
  const int gsize[LS_N_PROJ] = {3, 3, 3, 1, 2, 2, 1};
  ConvBatch cb;
  double bytes = 0;
  for (int p = 0; p < LS_N_PROJ; ++p) {
    if (!lora_active(c, l, p)) continue;
    const ProjLayout& P = c->lay.p[p];
    const LoraReg& R = c->lora[l][p];
    ConvJob j;
    j.src = R.A; j.lds = P.n_in; j.dst = lora_at(c, l, c->plan.a16[p]); j.ldd = P.n_in;
    j.rows = d.r; j.cols = P.n_in; j.pad_cols = P.n_in;
    cb.job[cb.n++] = j;
    j.src = R.B; j.lds = d.r; j.dst = lora_at(c, l, c->plan.bx16[p]); j.ldd = d.r16;
    j.rows = P.n_out; j.cols = d.r; j.pad_cols = d.r16;
    cb.job[cb.n++] = j;
    j.dst = lora_at(c, l, c->plan.bxt16[p]); j.ldd = P.n_out; j.transpose = 1;
    cb.job[cb.n++] = j;
    j.src = R.A; j.lds = P.n_in; j.dst = lora_at(c, l, at_off[p]) + gcol[p] * d.r16; j.ldd = (int64_t)gsize[p] * d.r16;
    j.rows = d.r; j.cols = P.n_in; j.pad_cols = P.n_in; j.transpose = 1;
    cb.job[cb.n++] = j;
    bytes += 4.0 * d.r * ((double)P.n_in + P.n_out) + 2.0 * 4 * d.r * ((double)P.n_in + P.n_out);
  }
  KTimer kt(c, LS_KC_LORA, 0.0, bytes);
  HIPCHK(c, launch_convert_batch(cb, c->cs));
  return LS_OK;
}

// Hs[:, col0 .. col0 + ng*r16) = s * X A_group^T
ls_status lora_down(ls_ctx* c, int l, const Dims& d, const uint16_t* x, int ldx, int p0, int ng, int K) {
  bool any = false;
  for (int p = p0; p < p0 + ng; ++p) any |= lora_active(c, l, p);
  if (!any) return LS_OK;
  FcArgs a;
  a.T = d.T;
  FcJob& j = a.job[a.n_jobs++];
  j.X = x; j.ldx = ldx; j.W = lora_at(c, l, c->plan.a16[p0]); j.K = K; j.N = ng * d.r16; j.alpha = d.s;
  j.out = hs_of(c, l) + p0 * d.r16; j.ldo = d.R7;
  KTimer kt(c, LS_KC_LORA, 2.0 * d.T * ng * d.r * K, 2.0 * d.T * K + 2.0 * ng * d.r * K + 2.0 * d.T * ng * d.r);
  HIPCHK(c, launch_lora_fc(a, c->cs));
  return LS_OK;
}

double fwd_gemm_flop(const Dims& d, int n_out, int K, bool lora) { return 2.0 * d.T * n_out * K + (lora ? 2.0 * d.T * n_out * d.r : 0.0); }

AttnArgs attn_args(const Dims& d, const uint16_t* qkv, uint16_t* out, float* lse) {
  AttnArgs a;
  a.qkv = qkv; a.ldqkv = d.qkvd; a.qd = d.qd; a.kvd = d.kvd;
  a.batch = d.batch; a.S = d.seq; a.hq = d.hq; a.hkv = d.hkv; a.hd = d.hd;
  a.scale = 1.0f / std::sqrt((float)d.hd);
  a.out = out; a.ldo = d.qd;
  a.lse = lse;
  return a;
}

// Causal attention forward, O = softmax(c Q K^T) V, plus the per-row log-sum-exp the
// backward uses to rebuild P; out32 (nullable) keeps O before rounding for the backward.
// stats_out / stats_in: the layer's per-row softmax statistics, kept by the forward and
// read back by the recompute so that it skips the statistics pass.
ls_status attn_fwd(ls_ctx* c, const Dims& d, const uint16_t* qkv, uint16_t* out, float* lse, float* out32,
                   float2* stats_out, const float2* stats_in, hipStream_t s) {
  const double fl = (stats_in ? 4.0 : 6.0) * d.batch * d.hq * (double)d.seq * (d.seq + 1) / 2 * d.hd;
  KTimer kt(c, LS_KC_ATTN, fl, 2.0 * d.T * (d.qkvd + d.qd) + 4.0 * d.T * d.hq + (out32 ? 4.0 * d.T * d.qd : 0.0), s);
  AttnArgs a = attn_args(d, qkv, out, lse);
  a.out32 = out32;
  a.stats_out = stats_out;
  a.stats_in = stats_in;
  HIPCHK(c, launch_attn_fwd(a, s));
  return LS_OK;
}

// Attention backward from dO (datt), O (att) and the log-sum-exp of the recompute ->
// dq in bf16, rotated back, in the q columns of dqkv16; float32 dk, dv in dqkv32 (summed
// over a kv head's q heads, fixed order).
ls_status attn_bwd(ls_ctx* c, const Dims& d, const Acts& x, const uint16_t* dout, float* dqkv32, uint16_t* dqkv16) {
  AttnArgs a = attn_args(d, x.qkv, x.att, x.lse);
  a.out32 = x.o32;
  a.dout = dout; a.lddo = d.qd;
  a.dd = c->dp<float>(c->plan.dd);
  a.dqkv = dqkv32; a.lddqkv = d.qkvd;
  // dq leaves the kernel in bf16 with the inverse rotation applied, straight into the
  // q columns of the bf16 dq | dk | dv the q|k|v backward reads
  a.dq16 = dqkv16; a.lddq16 = d.qkvd; a.rope_tab = c->dp<float2>(c->plan.rope);
  // with an even number of q heads per kv head, dK / dV run in two halves of the heads
  // (twice the workgroups, so the short key blocks fill in behind the long ones)
  a.dkv2 = (d.hq / d.hkv) % 2 == 0 ? c->dp<float>(c->plan.dkv2) : nullptr;
  const double fl = 2.5 * 4.0 * d.batch * d.hq * (double)d.seq * (d.seq + 1) / 2 * d.hd;
  KTimer kt(c, LS_KC_ATTN, fl, 2.0 * d.T * (d.qkvd + d.qd) + 4.0 * d.T * (d.qkvd + d.qd) + 8.0 * d.T * d.hq);
  HIPCHK(c, launch_attn_bwd(a, c->cs));
  return LS_OK;
}

enum FwdMode { MODE_FWD = 0, MODE_RECOMPUTE = 1 };

// The gate | up projection of layer l over n2 (bf16 [T, h]): weights, low-rank term
// (s X A^T columns from hs against the layer's B), levels; outputs are the caller's.
FwdArgs gate_up_args(ls_ctx* c, int l, const uint8_t* blob, const Dims& d, bool lora, const uint16_t* n2,
                     const uint16_t* hs) {
  FwdArgs f;
  f.x = n2; f.ldx = d.h; f.M = d.T; f.K = d.h; f.n_groups = 2;
  for (int i = 0; i < 2; ++i) {
    const int p = LS_PROJ_GATE + i;
    f.g[i].w = wref(c, blob, p);
    f.g[i].out_col0 = i * d.I;
    f.g[i].ext_col0 = p * d.r16;
    f.g[i].bext = lora && lora_active(c, l, p) ? lora_at(c, l, c->plan.bx16[p]) : nullptr;
  }
  f.aext = hs; f.ldaext = d.R7; f.kx = lora ? d.r16 : 0;
  f.levels = c->dp<float>(c->plan.levels); f.format = wformat(c->cfg);
  return f;
}

// SwiGLU rides in the gate | up GEMM's epilogue (paired gate / up tiles) when both
// low-rank terms fit one 64-column extension
bool paired_swiglu(const Dims& d) { return 2 * d.r16 <= 64; }

// One decoder layer forward from x_in (bf16 [T, h]), every launch on stream s, into
// the layer's activation set.  MODE_FWD writes x_out.  MODE_RECOMPUTE (the backward's
// recompute) keeps the attention output in float32 and skips the down projection,
// whose output the backward does not need; with the paired gate | up kernel it also
// stops before gate | up, which the backward runs (layer_backward), and otherwise it
// keeps gate and up in float32.
ls_status layer_forward(ls_ctx* c, int l, const uint8_t* blob, const Dims& d, const uint16_t* x_in, uint16_t* x_out,
                        bool lora, FwdMode mode, const Fence& fc, hipStream_t s) {
  const ls_config& g = c->cfg;
  const int fmt = wformat(g);
  const float* lv = c->dp<float>(c->plan.levels);
  const Acts x = acts_of(c, l);
  uint16_t* n1 = x.n1;
  uint16_t* qkv = x.qkv;
  uint16_t* att = x.att;
  float* hb = x.hb;
  uint16_t* n2 = x.n2;
  float* gu = x.gu;
  uint16_t* act = x.act;
  uint16_t* hs = hs_of(c, l);
  // the recompute reads the forward's s X A^T of this layer (same inputs, same kernel)
  const bool down = lora && mode == MODE_FWD;
  const uint16_t* g1 = reinterpret_cast<const uint16_t*>(blob + c->lay.off_g1);
  const uint16_t* g2 = reinterpret_cast<const uint16_t*>(blob + c->lay.off_g2);
  const double tb = 2.0 * d.T;
  ls_status fst;

  if ((fst = fence_wait(c, fc, 0, s))) return fst;
  {
    KTimer kt(c, LS_KC_GLUE, 0.0, 2 * tb * d.h, s);
    HIPCHK(c, launch_rmsnorm_fwd(x_in, nullptr, g1, n1, x.rstd1, d.T, d.h, g.rms_eps, s));
  }
  if (down) { ls_status st = lora_down(c, l, d, n1, d.h, LS_PROJ_Q, 3, d.h); if (st) return st; }
  {
    FwdArgs f;
    f.x = n1; f.ldx = d.h; f.M = d.T; f.K = d.h; f.n_groups = 3;
    const int cols[3] = {0, d.qd, d.qd + d.kvd};
    for (int i = 0; i < 3; ++i) {
      f.g[i].w = wref(c, blob, LS_PROJ_Q + i);
      f.g[i].out_col0 = cols[i];
      f.g[i].ext_col0 = (LS_PROJ_Q + i) * d.r16;
      f.g[i].bext = lora && lora_active(c, l, LS_PROJ_Q + i) ? lora_at(c, l, c->plan.bx16[LS_PROJ_Q + i]) : nullptr;
    }
    f.aext = hs; f.ldaext = d.R7; f.kx = lora ? d.r16 : 0;
    f.y = qkv; f.ldy = d.qkvd; f.levels = lv; f.format = fmt;
    // q and k leave the GEMM rotated (rotary embedding applied in float32 before rounding)
    f.rope_tab = c->dp<float2>(c->plan.rope); f.rope_cols = d.qd + d.kvd; f.seq = d.seq; f.head_dim = d.hd;
    KTimer kt(c, LS_KC_GEMM_FWD, fwd_gemm_flop(d, d.qkvd, d.h, lora),
              tb * d.h + wbytes(c, 0) + wbytes(c, 1) + wbytes(c, 2) + tb * d.qkvd, s);
    f.sk = c->split_scratch(s);
    HIPCHK(c, launch_gemm_fwd(f, s));
  }
  {
    float2* stats = c->dp<float2>(c->plan.astats) + (uint64_t)l * c->cfg.max_tokens * c->cfg.n_heads;
    ls_status st = attn_fwd(c, d, qkv, att, x.lse, mode == MODE_RECOMPUTE ? x.o32 : nullptr,
                            mode == MODE_FWD && lora ? stats : nullptr, mode == MODE_RECOMPUTE ? stats : nullptr, s);
    if (st) return st;
  }
  if (down) { ls_status st = lora_down(c, l, d, att, d.qd, LS_PROJ_O, 1, d.qd); if (st) return st; }
  if ((fst = fence_wait(c, fc, 1, s))) return fst;
  {
    FwdArgs f;
    f.x = att; f.ldx = d.qd; f.M = d.T; f.K = d.qd; f.n_groups = 1;
    f.g[0].w = wref(c, blob, LS_PROJ_O);
    f.g[0].ext_col0 = LS_PROJ_O * d.r16;
    f.g[0].bext = lora && lora_active(c, l, LS_PROJ_O) ? lora_at(c, l, c->plan.bx16[LS_PROJ_O]) : nullptr;
    f.aext = hs; f.ldaext = d.R7; f.kx = lora ? d.r16 : 0;
    f.resid = x_in; f.ldr = d.h;
    f.y32 = hb; f.ldy = d.h; f.levels = lv; f.format = fmt;
    KTimer kt(c, LS_KC_GEMM_FWD, fwd_gemm_flop(d, d.h, d.qd, lora), tb * d.qd + wbytes(c, 3) + 3 * tb * d.h, s);
    f.sk = c->split_scratch(s);
    HIPCHK(c, launch_gemm_fwd(f, s));
  }
  {
    KTimer kt(c, LS_KC_GLUE, 0.0, 2 * tb * d.h, s);
    HIPCHK(c, launch_rmsnorm_fwd(nullptr, hb, g2, n2, x.rstd2, d.T, d.h, g.rms_eps, s));
  }
  const bool fuse_swiglu = paired_swiglu(d);
  // with the paired kernel the recompute ends here: the backward runs the gate | up
  // GEMM itself, once d(act) is known, and does the SwiGLU backward in its epilogue
  if (mode == MODE_RECOMPUTE && fuse_swiglu) return LS_OK;
  if ((fst = fence_wait(c, fc, 2, s))) return fst;
  if (down) { ls_status st = lora_down(c, l, d, n2, d.h, LS_PROJ_GATE, 2, d.h); if (st) return st; }
  {
    FwdArgs f = gate_up_args(c, l, blob, d, lora, n2, hs);
    if (fuse_swiglu) {
      f.swiglu = 1; f.y = act; f.ldy = d.I;
    } else {   // the recompute keeps gate and up in float32 for the down projection's dX GEMM
      f.y32 = gu; f.ldy = 2 * d.I;
    }
    const double out_bytes = fuse_swiglu ? tb * d.I : 2 * tb * 2 * d.I;
    KTimer kt(c, LS_KC_GEMM_FWD, fwd_gemm_flop(d, 2 * d.I, d.h, lora), tb * d.h + wbytes(c, 4) + wbytes(c, 5) + out_bytes, s);
    f.sk = c->split_scratch(s);
    HIPCHK(c, launch_gemm_fwd(f, s));
  }
  if (!fuse_swiglu) {
    KTimer kt(c, LS_KC_GLUE, 0.0, 5 * tb * d.I, s);
    HIPCHK(c, launch_swiglu_fwd(gu, d.I, act, d.T, s));
  }
  if (down) { ls_status st = lora_down(c, l, d, act, d.I, LS_PROJ_DOWN, 1, d.I); if (st) return st; }
  if (mode == MODE_RECOMPUTE) return LS_OK;
  if ((fst = fence_wait(c, fc, 3, s))) return fst;
  {
    FwdArgs f;
    f.x = act; f.ldx = d.I; f.M = d.T; f.K = d.I; f.n_groups = 1;
    f.g[0].w = wref(c, blob, LS_PROJ_DOWN);
    f.g[0].ext_col0 = LS_PROJ_DOWN * d.r16;
    f.g[0].bext = lora && lora_active(c, l, LS_PROJ_DOWN) ? lora_at(c, l, c->plan.bx16[LS_PROJ_DOWN]) : nullptr;
    f.aext = hs; f.ldaext = d.R7; f.kx = lora ? d.r16 : 0;
    f.resid32 = hb; f.ldr = d.h;
    f.y = x_out; f.ldy = d.h; f.levels = lv; f.format = fmt;
    KTimer kt(c, LS_KC_GEMM_FWD, fwd_gemm_flop(d, d.h, d.I, lora), tb * d.I + wbytes(c, 6) + 3 * tb * d.h, s);
    f.sk = c->split_scratch(s);
    HIPCHK(c, launch_gemm_fwd(f, s));
  }
  return LS_OK;
}

// LoRA gradient products of projection p: Gs_p = s dY_p Bx16_p (bf16, into Gs),
// dB_p = dY_p^T Hs_p, dA_p = Gs_p^T X_p (float32, written or accumulated).
// Gs_p = s dY_p Bx16_p (bf16, into Gs) for the n projections p0.. whose output
// gradients sit side by side in dy (dY_p at dy + the sum of the earlier n_out), one launch.
ls_status lora_grads_G(ls_ctx* c, int l, const Dims& d, int p0, int n, const uint16_t* dy, int lddy) {
  FcArgs a;
  a.T = d.T;
  double flop = 0.0, bytes = 0.0;
  int col = 0;
  for (int i = 0; i < n; ++i) {
    const int p = p0 + i;
    const ProjLayout& P = c->lay.p[p];
    if (lora_active(c, l, p)) {
      FcJob& j = a.job[a.n_jobs++];
      j.X = dy + col; j.ldx = lddy; j.W = lora_at(c, l, c->plan.bxt16[p]); j.K = P.n_out; j.N = d.r16;
      j.alpha = d.s; j.out = c->dp<uint16_t>(c->plan.gs) + p * d.r16; j.ldo = d.R7;
      flop += 2.0 * d.T * P.n_out * d.r;
      bytes += 2.0 * d.T * P.n_out + 2.0 * P.n_out * d.r + 2.0 * d.T * d.r;
    }
    col += P.n_out;
  }
  if (a.n_jobs == 0) return LS_OK;
  KTimer kt(c, LS_KC_LORA, flop, bytes);
  HIPCHK(c, launch_lora_fc(a, c->cs));
  return LS_OK;
}

// dA and dB of the n projections p0.. that share the input x (float32, written or,
// with beta 1, accumulated), one launch: dA_p = Gs_p^T x over the stacked Gs columns
// of the group, dB_p = dY_p^T Hs_p with dY_p at dy + (sum of the earlier n_out).
ls_status lora_grads_AB(ls_ctx* c, int l, const Dims& d, int p0, int n, const uint16_t* dy, int lddy,
                        const uint16_t* x, int ldx, float beta) {
  TcArgs a;
  a.T = d.T; a.beta = beta;
  a.partial = c->dp<float>(c->plan.partial); a.partial_floats = (int64_t)(c->plan.partial_bytes / 4);
  const int n_in = c->lay.p[p0].n_in;
  double flop = 0.0, bytes = 0.0;
  TcJob ja;
  ja.A = x; ja.lda = ldx; ja.M = n_in;
  ja.B = c->dp<uint16_t>(c->plan.gs) + p0 * d.r16; ja.ldb = d.R7; ja.N = n * d.r16;
  ja.scm = 1; ja.scn = n_in; ja.ncols = d.r16; ja.nvalid = d.r;
  bool any_a = false;
  int col = 0;
  for (int i = 0; i < n; ++i) {
    const int p = p0 + i;
    const ProjLayout& P = c->lay.p[p];
    const LoraReg& R = c->lora[l][p];
    const bool on = lora_active(c, l, p);
    if (on && R.dA) { ja.C[i] = R.dA; any_a = true; flop += 2.0 * d.T * n_in * d.r; }
    if (on && R.dB) {
      TcJob jb;
      jb.A = dy + col; jb.lda = lddy; jb.M = P.n_out;
      jb.B = hs_of(c, l) + p * d.r16; jb.ldb = d.R7; jb.N = d.r16;
      jb.C[0] = R.dB; jb.scm = d.r; jb.scn = 1; jb.ncols = d.r16; jb.nvalid = d.r;
      a.job[a.n_jobs++] = jb;
      flop += 2.0 * d.T * P.n_out * d.r;
      bytes += 2.0 * d.T * P.n_out + 2.0 * d.T * d.r16 + 4.0 * P.n_out * d.r;
    }
    col += P.n_out;
  }
  if (any_a) {
    a.job[a.n_jobs++] = ja;
    bytes += 2.0 * d.T * n_in + 2.0 * d.T * n * d.r16 + 4.0 * n * n_in * d.r;
  }
  if (a.n_jobs == 0) return LS_OK;
  // everything read here was written on the compute stream before this point
  HIPCHK(c, hipEventRecord(c->fork_ev, c->cs));
  HIPCHK(c, hipStreamWaitEvent(c->side, c->fork_ev, 0));
  c->side_pending = true;
  KTimer kt(c, LS_KC_LORA, flop, bytes, c->side);
  HIPCHK(c, launch_lora_tc(a, c->side));
  return LS_OK;
}

// The compute stream waits for the adapter-gradient reductions enqueued so far.
ls_status join_side(ls_ctx* c) {
  if (!c->side_pending) return LS_OK;
  HIPCHK(c, hipEventRecord(c->join_ev, c->side));
  HIPCHK(c, hipStreamWaitEvent(c->cs, c->join_ev, 0));
  c->side_pending = false;
  return LS_OK;
}

// The backward of layer l on the compute stream, after its recompute (layer_forward in
// MODE_RECOMPUTE, enqueued by the caller) filled the layer's activation set.
ls_status layer_backward(ls_ctx* c, int l, const uint8_t* blob, const Dims& d, const uint16_t* x_in, const uint16_t* dy,
                         uint16_t* dx, float beta, const Fence& fc) {
  // the previous layer's reductions read the gradient buffers this layer overwrites
  ls_status st = join_side(c);
  if (st) return st;
  const ls_config& g = c->cfg;
  const int fmt = wformat(g);
  const float* lv = c->dp<float>(c->plan.levels);
  const Acts x = acts_of(c, l);
  uint16_t* n1 = x.n1;
  uint16_t* att = x.att;
  float* hb = x.hb;
  uint16_t* n2 = x.n2;
  float* gu = x.gu;
  uint16_t* act = x.act;
  uint16_t* gs = c->dp<uint16_t>(c->plan.gs);
  float* dh32 = c->dp<float>(c->plan.dh32);
  uint16_t* dh16 = c->dp<uint16_t>(c->plan.dh16);
  float* dqkv32 = c->dp<float>(c->plan.dqkv32);
  uint16_t* dgu = c->dp<uint16_t>(c->plan.dgu);
  uint16_t* datt = c->dp<uint16_t>(c->plan.datt);
  uint16_t* dqkv = c->dp<uint16_t>(c->plan.dqkv);
  float* dn32 = c->dp<float>(c->plan.dn32);
  const uint16_t* g1 = reinterpret_cast<const uint16_t*>(blob + c->lay.off_g1);
  const uint16_t* g2 = reinterpret_cast<const uint16_t*>(blob + c->lay.off_g2);
  const double tb = 2.0 * d.T;
  auto bwd_flop = [&](int n_out, int n_in) { return 2.0 * d.T * n_out * n_in + 2.0 * d.T * n_in * d.r; };

  // ---- down: y = h + act W_d^T + LoRA
  // With the paired gate | up kernel, the recompute stopped before gate | up: the down
  // projection's dX GEMM writes d(act) in float32 (into the gate | up buffer), then the
  // gate | up GEMM runs here and its epilogue writes act and, from d(act) and its own
  // float32 gate and up, dgate | dup.  Otherwise the recompute kept gate and up in
  // float32 and the dX GEMM's epilogue does the SwiGLU backward from them.
  const bool fuse_swiglu = paired_swiglu(d);
  if ((st = lora_grads_G(c, l, d, LS_PROJ_DOWN, 1, dy, d.h))) return st;
  if (!fuse_swiglu && (st = lora_grads_AB(c, l, d, LS_PROJ_DOWN, 1, dy, d.h, act, d.I, beta))) return st;
  if ((st = fence_wait(c, fc, 3, c->cs))) return st;
  {
    BwdArgs b;
    b.dy = dy; b.lddy = d.h; b.M = d.T; b.N = d.I; b.n_segs = 1;
    b.seg[0].w = wref(c, blob, LS_PROJ_DOWN); b.seg[0].a_col0 = 0;
    b.aext = gs + LS_PROJ_DOWN * d.r16; b.ldaext = d.R7; b.kx = d.r16;
    b.bext = lora_at(c, l, c->plan.at_d); b.ldbext = d.r16;
    b.levels = lv; b.format = fmt;
    if (fuse_swiglu) {
      b.out32 = gu; b.ldo = d.I;
    } else {
      b.out16 = dgu; b.ldo = 2 * d.I; b.gu32 = gu; b.ldgu = 2 * d.I;
    }
    const double out_bytes = fuse_swiglu ? 2 * tb * d.I : 2 * tb * 2 * d.I + tb * 2 * d.I;
    KTimer kt(c, LS_KC_GEMM_BWD, bwd_flop(d.h, d.I), tb * d.h + wbytes(c, 6) + out_bytes);
    b.sk = c->split_scratch(c->cs);
    HIPCHK(c, launch_gemm_bwd(b, c->cs));
  }
  if (fuse_swiglu) {
    if ((st = fence_wait(c, fc, 2, c->cs))) return st;
    {
      FwdArgs f = gate_up_args(c, l, blob, d, true, n2, hs_of(c, l));
      f.swiglu = 1; f.y = act; f.ldy = d.I;
      f.dact = gu; f.ldda = d.I; f.dgu = dgu; f.lddgu = 2 * d.I;
      // the recompute's GEMM: not one of the forward pass's launches LS_PROFILE_GEMM times
      c->in_recompute = true;
      {
        KTimer kt(c, LS_KC_GEMM_FWD, fwd_gemm_flop(d, 2 * d.I, d.h, true),
                  tb * d.h + wbytes(c, 4) + wbytes(c, 5) + tb * d.I + 2 * tb * d.I + tb * 2 * d.I);
        f.sk = c->split_scratch(c->cs);
        const hipError_t e = launch_gemm_fwd(f, c->cs);
        c->in_recompute = false;
        HIPCHK(c, e);
      }
    }
    if ((st = lora_grads_AB(c, l, d, LS_PROJ_DOWN, 1, dy, d.h, act, d.I, beta))) return st;
  }
  // ---- gate / up
  if ((st = lora_grads_G(c, l, d, LS_PROJ_GATE, 2, dgu, 2 * d.I))) return st;
  if ((st = lora_grads_AB(c, l, d, LS_PROJ_GATE, 2, dgu, 2 * d.I, n2, d.h, beta))) return st;
  {
    BwdArgs b;
    b.dy = dgu; b.lddy = 2 * d.I; b.M = d.T; b.N = d.h; b.n_segs = 2;
    b.seg[0].w = wref(c, blob, LS_PROJ_GATE); b.seg[0].a_col0 = 0;
    b.seg[1].w = wref(c, blob, LS_PROJ_UP); b.seg[1].a_col0 = d.I;
    b.aext = gs + LS_PROJ_GATE * d.r16; b.ldaext = d.R7; b.kx = 2 * d.r16;
    b.bext = lora_at(c, l, c->plan.at_gu); b.ldbext = 2 * d.r16;
    b.out32 = dn32; b.ldo = d.h; b.levels = lv; b.format = fmt;
    KTimer kt(c, LS_KC_GEMM_BWD, 2 * bwd_flop(d.I, d.h), tb * 2 * d.I + wbytes(c, 4) + wbytes(c, 5) + 2 * tb * d.h);
    b.sk = c->split_scratch(c->cs);
    HIPCHK(c, launch_gemm_bwd(b, c->cs));
  }
  {
    KTimer kt(c, LS_KC_GLUE, 0.0, 4 * tb * d.h);
    HIPCHK(c, launch_rmsnorm_bwd(dn32, nullptr, hb, g2, x.rstd2, nullptr, dy, dh32, dh16, d.T, d.h, c->cs));
  }
  // ---- o: h = x + att W_o^T + LoRA
  if ((st = lora_grads_G(c, l, d, LS_PROJ_O, 1, dh16, d.h))) return st;
  if ((st = lora_grads_AB(c, l, d, LS_PROJ_O, 1, dh16, d.h, att, d.qd, beta))) return st;
  {
    BwdArgs b;
    b.dy = dh16; b.lddy = d.h; b.M = d.T; b.N = d.qd; b.n_segs = 1;
    b.seg[0].w = wref(c, blob, LS_PROJ_O); b.seg[0].a_col0 = 0;
    b.aext = gs + LS_PROJ_O * d.r16; b.ldaext = d.R7; b.kx = d.r16;
    b.bext = lora_at(c, l, c->plan.at_o); b.ldbext = d.r16;
    b.out16 = datt; b.ldo = d.qd; b.levels = lv; b.format = fmt;
    KTimer kt(c, LS_KC_GEMM_BWD, bwd_flop(d.h, d.qd), tb * d.h + wbytes(c, 3) + tb * d.qd);
    b.sk = c->split_scratch(c->cs);
    HIPCHK(c, launch_gemm_bwd(b, c->cs));
  }
  if ((st = attn_bwd(c, d, x, datt, dqkv32, dqkv))) return st;
  {
    // dk | dv: the second half of the q heads joins here (see attn_bwd), then the
    // inverse rotation on dk and bf16 (dq is already in place)
    KTimer kt(c, LS_KC_GLUE, 0.0, 3 * tb * 2 * d.kvd);
    const float* dkv2 = (d.hq / d.hkv) % 2 == 0 ? c->dp<float>(c->plan.dkv2) : nullptr;
    HIPCHK(c, launch_rope_bwd_convert(dqkv32 + d.qd, dqkv + d.qd, d.qkvd, 2 * d.kvd, d.T, d.seq, d.hkv, d.hd,
                                      c->dp<float2>(c->plan.rope), c->cs, dkv2, 0, 2 * d.kvd));
  }
  // ---- q, k, v
  const int cols[3] = {0, d.qd, d.qd + d.kvd};
  if ((st = lora_grads_G(c, l, d, LS_PROJ_Q, 3, dqkv, d.qkvd))) return st;
  if ((st = lora_grads_AB(c, l, d, LS_PROJ_Q, 3, dqkv, d.qkvd, n1, d.h, beta))) return st;
  {
    BwdArgs b;
    b.dy = dqkv; b.lddy = d.qkvd; b.M = d.T; b.N = d.h; b.n_segs = 3;
    for (int i = 0; i < 3; ++i) { b.seg[i].w = wref(c, blob, LS_PROJ_Q + i); b.seg[i].a_col0 = cols[i]; }
    b.aext = gs; b.ldaext = d.R7; b.kx = 3 * d.r16;
    b.bext = lora_at(c, l, c->plan.at_qkv); b.ldbext = 3 * d.r16;
    b.out32 = dn32; b.ldo = d.h; b.levels = lv; b.format = fmt;
    KTimer kt(c, LS_KC_GEMM_BWD, bwd_flop(d.qkvd, d.h), tb * d.qkvd + wbytes(c, 0) + wbytes(c, 1) + wbytes(c, 2) + 2 * tb * d.h);
    b.sk = c->split_scratch(c->cs);
    HIPCHK(c, launch_gemm_bwd(b, c->cs));
  }
  // dx may alias dy (a one-layer stack): the side stream's dB product of the down
  // projection reads dy, so it must be done before dx is written over it
  {
    const uintptr_t a0 = reinterpret_cast<uintptr_t>(dx), b0 = reinterpret_cast<uintptr_t>(dy);
    const uintptr_t n = (uintptr_t)tb * (uintptr_t)d.h;
    if (a0 < b0 + n && b0 < a0 + n && (st = join_side(c))) return st;
  }
  {
    KTimer kt(c, LS_KC_GLUE, 0.0, 4 * tb * d.h);
    HIPCHK(c, launch_rmsnorm_bwd(dn32, x_in, nullptr, g1, x.rstd1, dh32, nullptr, nullptr, dx, d.T, d.h, c->cs));
  }
  // the set is free for the recompute of layer l - 2 once this backward and its
  // reductions are done with it
  const int k = l & 1;
  HIPCHK(c, hipEventRecord(c->bp_done[k], c->cs));
  c->bp_rec[k] = true;
  if (c->side_pending) {
    HIPCHK(c, hipEventRecord(c->side_done[k], c->side));
    c->side_rec[k] = true;
  } else {
    c->side_rec[k] = false;
  }
  return LS_OK;
}

uint16_t* ckpt(ls_ctx* c, int l) {
  return c->dp<uint16_t>(c->plan.ck) + (uint64_t)l * c->cfg.max_tokens * c->cfg.hidden;
}

ls_status check_usable(ls_ctx* c) {
  if (!c) return LS_ERR_INVALID;
  if (c->sticky != LS_OK) return c->sticky;
  return LS_OK;
}

}  // namespace

// ======================================================================= C ABI
extern "C" {

void ls_nf4_codebook(float out[16]) { nf4_codebook_host(out); }

ls_status ls_pack_nf4(const uint16_t* w, uint64_t numel, int32_t double_quant, int32_t n_threads, uint8_t* packed,
                      float* absmax, uint8_t* qabs, float* scale2, float* mean) {
  if (!w || !packed || !absmax || (double_quant && (!qabs || !scale2 || !mean))) return LS_ERR_INVALID;
  if (numel == 0) return LS_OK;
  pack_nf4_host(w, numel, double_quant != 0, n_threads, packed, absmax, qabs, scale2, mean);
  return LS_OK;
}

// n_buffers = 0: the deepest pool (at most 64 slots and at most one per layer) whose
// device plan fits `budget`, else 2 (which the budget check then refuses).  Resident
// contexts ignore the pool depth; they get 2.
static void resolve_depth(ls_config& cfg, const BlobLayout& L, uint64_t budget) {
  if (cfg.n_buffers != 0) return;
  cfg.n_buffers = 2;
  if (cfg.resident) return;
  for (int k = std::max(2, std::min(64, (int)cfg.n_layers)); k > 2; --k) {
    cfg.n_buffers = k;
    if (make_plan(cfg, L).total <= budget) return;
  }
  cfg.n_buffers = 2;
}

ls_status ls_plan_bytes(const ls_config* cfg_in, uint64_t* device_bytes, uint64_t* host_bytes, uint64_t* blob_bytes) {
  if (!cfg_in) return LS_ERR_INVALID;
  const char* why = nullptr;
  if (!validate_config(*cfg_in, &why)) { g_create_err = why; return LS_ERR_INVALID; }
  ls_config resolved = *cfg_in;
  const ls_config* cfg = &resolved;
  const BlobLayout L = make_layout(*cfg);
  resolve_depth(resolved, L, cfg_in->vram_budget ? cfg_in->vram_budget : UINT64_MAX);
  const DevPlan P = make_plan(*cfg, L);
  if (device_bytes) *device_bytes = P.total;
  if (host_bytes)
    *host_bytes = cfg->store == LS_STORE_FILE
                      ? (L.bytes + 4095) / 4096 * 4096 * (uint64_t)(cfg->resident ? 1 : cfg->n_buffers)
                      : L.bytes * (uint64_t)(cfg->n_layers + P.head_slices);
  if (blob_bytes) *blob_bytes = L.bytes;
  return LS_OK;
}

ls_status ls_create(const ls_config* cfg_in, void* compute_stream, void* copy_stream, ls_ctx** out) {
  if (!cfg_in || !out) return fail(nullptr, LS_ERR_INVALID, "null cfg or out");
  *out = nullptr;
  const char* why = nullptr;
  if (!validate_config(*cfg_in, &why)) return fail(nullptr, LS_ERR_INVALID, "invalid config: %s", why);
  if (compute_stream && compute_stream == copy_stream) return fail(nullptr, LS_ERR_INVALID, "copy stream must differ from compute stream");
  ls_config resolved = *cfg_in;
  const ls_config* cfg = &resolved;
  const BlobLayout L = make_layout(*cfg);
  uint64_t budget = cfg->vram_budget;
  if (budget == 0) {
    size_t fr = 0, tot = 0;
    hipError_t e = hipMemGetInfo(&fr, &tot);
    if (e != hipSuccess) return fail(nullptr, LS_ERR_HIP, "hipMemGetInfo failed: %s", hipGetErrorString(e));
    budget = fr;
  }
  // an automatic pool depth leaves half of the free memory to the caller's tensors
  resolve_depth(resolved, L, cfg_in->vram_budget ? budget : budget / 2);
  const DevPlan P = make_plan(*cfg, L);
  if (P.total > budget)
    return fail(nullptr, LS_ERR_BUDGET, "device plan %llu bytes exceeds budget %llu bytes",
                (unsigned long long)P.total, (unsigned long long)budget);

  ls_ctx* c = new ls_ctx();
  c->cfg = *cfg;
  c->lay = L;
  c->plan = P;
  auto bail = [&](ls_status st) { g_create_err = c->err; ls_destroy(c); return st; };
  if (hipGetDevice(&c->device) != hipSuccess) { c->err = "hipGetDevice failed"; return bail(LS_ERR_HIP); }
  if (compute_stream) c->cs = (hipStream_t)compute_stream;
  else if (hipStreamCreateWithFlags(&c->cs, hipStreamNonBlocking) == hipSuccess) c->own_cs = true;
  else { c->err = "compute stream creation failed"; return bail(LS_ERR_HIP); }
  if (copy_stream) c->ps = (hipStream_t)copy_stream;
  else if (hipStreamCreateWithFlags(&c->ps, hipStreamNonBlocking) == hipSuccess) c->own_ps = true;
  else { c->err = "copy stream creation failed"; return bail(LS_ERR_HIP); }
  if (hipStreamCreateWithFlags(&c->side, hipStreamNonBlocking) != hipSuccess) {
    c->side = nullptr;
    c->err = "side stream creation failed";
    return bail(LS_ERR_HIP);
  }
  if (hipStreamCreateWithFlags(&c->rs, hipStreamNonBlocking) != hipSuccess) {
    c->rs = nullptr;
    c->err = "recompute stream creation failed";
    return bail(LS_ERR_HIP);
  }
  if (hipEventCreateWithFlags(&c->fork_ev, hipEventDisableTiming) != hipSuccess ||
      hipEventCreateWithFlags(&c->join_ev, hipEventDisableTiming) != hipSuccess) {
    c->err = "event creation failed";
    return bail(LS_ERR_HIP);
  }
  for (int k = 0; k < 2; ++k)
    if (hipEventCreateWithFlags(&c->rec_done[k], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&c->bp_done[k], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&c->side_done[k], hipEventDisableTiming) != hipSuccess) {
      c->err = "event creation failed";
      return bail(LS_ERR_HIP);
    }
  if (gemm_dequant_init() != hipSuccess) { c->err = "kernel attribute setup failed"; return bail(LS_ERR_HIP); }
  if (const char* e = getenv("LS_DEBUG_POISON")) c->dbg_poison = e[0] == '1';
  if (const char* e = getenv("LS_DEBUG_COPY_DELAY_US")) c->dbg_delay_us = (uint32_t)std::min(1000000L, std::max(0L, atol(e)));

  const int nb = P.n_slots;
  c->slot_layer.assign(nb, -1);
  // ready events: one per piece of each slot; consumed events: one per slot
  c->ready.resize(nb * kPieces);
  c->consumed.resize(nb);
  c->ready_rec.assign(nb * kPieces, 0);
  c->cons_rec.assign(nb, 0);
  for (auto& e : c->ready)
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) { e = nullptr; c->err = "event creation failed"; return bail(LS_ERR_HIP); }
  for (auto& e : c->consumed)
    if (hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) { e = nullptr; c->err = "event creation failed"; return bail(LS_ERR_HIP); }
  c->lora.resize(cfg->n_layers);
  c->staged.assign(cfg->n_layers, 0);
  const int n_blobs = cfg->n_layers + P.head_slices;
  c->host.assign(n_blobs, nullptr);
  if (cfg->store == LS_STORE_FILE) {
    // the store is a file of n_blobs blobs, 4096 bytes apart.  Reads go through the page
    // cache into the pinned staging buffers (direct I/O cannot pin that memory), and
    // every blob's pages are dropped from the cache after it is staged and after each
    // read, so each read comes from the file's device rather than from RAM.
    c->stride = (L.bytes + 4095) / 4096 * 4096;
    c->fd = open(cfg->store_path, O_RDWR | O_CREAT | O_TRUNC, 0600);
    if (c->fd < 0) {
      c->err = std::string("cannot create the store file ") + cfg->store_path + ": " + strerror(errno);
      return bail(LS_ERR_INVALID);
    }
    if (ftruncate(c->fd, (off_t)(c->stride * (uint64_t)n_blobs)) != 0) {
      c->err = std::string("cannot size the store file: ") + strerror(errno);
      return bail(LS_ERR_INVALID);
    }
    const int n_stage = cfg->resident ? 1 : cfg->n_buffers;
    c->staging.assign(n_stage, nullptr);
    for (int i = 0; i < n_stage; ++i) {
      if (hipHostMalloc((void**)&c->staging[i], c->stride, hipHostMallocDefault) != hipSuccess) {
        c->staging[i] = nullptr;
        c->err = "pinned host allocation of the staging buffers failed";
        return bail(LS_ERR_OOM);
      }
      std::memset(c->staging[i], 0, c->stride);
    }
    c->uncached = posix_fadvise(c->fd, 0, 0, POSIX_FADV_DONTNEED) == 0;
    c->jobs.resize(n_blobs);
    for (int l = 0; l < n_blobs; ++l)
      c->jobs[l] = {c, c->staging[cfg->resident ? 0 : l % cfg->n_buffers], (uint64_t)l * c->stride, c->stride};
  } else {
    for (int l = 0; l < n_blobs; ++l) {
      if (hipHostMalloc((void**)&c->host[l], L.bytes, hipHostMallocDefault) != hipSuccess) {
        c->host[l] = nullptr;
        c->err = "pinned host allocation of the layer store failed";
        return bail(LS_ERR_OOM);
      }
      std::memset(c->host[l], 0, L.bytes);
    }
  }
  if (hipMalloc((void**)&c->dbase, P.total) != hipSuccess) {
    c->dbase = nullptr;
    c->err = "device allocation failed";
    return bail(LS_ERR_OOM);
  }
  // zero the whole plan once: unused LoRA columns and padding must read as 0
  if (hipMemsetAsync(c->dbase, 0, P.total, c->cs) != hipSuccess) { c->err = "device memset failed"; return bail(LS_ERR_HIP); }
  // NF4 levels and the rotary table, computed on the host
  nf4_codebook_host(c->levels_h);
  std::vector<float2> rope((size_t)cfg->max_seq * (cfg->head_dim / 2));
  for (int pos = 0; pos < cfg->max_seq; ++pos)
    for (int i = 0; i < cfg->head_dim / 2; ++i) {
      const double ang = (double)pos * std::pow((double)cfg->rope_theta, -2.0 * i / (double)cfg->head_dim);
      rope[(size_t)pos * (cfg->head_dim / 2) + i] = make_float2((float)std::cos(ang), (float)std::sin(ang));
    }
  if (hipMemcpyAsync(c->dbase + P.levels, c->levels_h, 64, hipMemcpyHostToDevice, c->cs) != hipSuccess ||
      hipMemcpyAsync(c->dbase + P.rope, rope.data(), rope.size() * sizeof(float2), hipMemcpyHostToDevice, c->cs) != hipSuccess ||
      hipStreamSynchronize(c->cs) != hipSuccess) {
    c->err = "upload of tables failed";
    return bail(LS_ERR_HIP);
  }
  c->stats.blob_bytes = L.bytes;
  c->stats.store_bytes = cfg->store == LS_STORE_FILE ? c->stride * (uint64_t)n_blobs
                                                    : L.bytes * (uint64_t)(cfg->n_layers + P.head_slices);
  c->stats.store_uncached = c->uncached ? 1 : 0;
  c->stats.n_slots = P.n_slots;
  c->stats.device_bytes = P.total;
  *out = c;
  return LS_OK;
}

ls_status ls_stage_layer(ls_ctx* c, int32_t layer, const ls_layer_host* w) {
  if (ls_status st = check_usable(c)) return st;
  if (!w || layer < 0 || layer >= c->cfg.n_layers) return fail(c, LS_ERR_INVALID, "bad layer index or null weights");
  if (!w->g1 || !w->g2) return fail(c, LS_ERR_INVALID, "null norm weights");
  for (int p = 0; p < LS_N_PROJ; ++p)
    if (!w->w[p]) return fail(c, LS_ERR_INVALID, "null weight for projection %d", p);
  if (c->in_flight) return fail(c, LS_ERR_STATE, "a forward/backward is in flight: call ls_sync first");
  uint8_t* blob = stage_buffer(c, layer);
  std::memcpy(blob + c->lay.off_g1, w->g1, 2ull * c->cfg.hidden);
  std::memcpy(blob + c->lay.off_g2, w->g2, 2ull * c->cfg.hidden);
  for (int p = 0; p < LS_N_PROJ; ++p) {
    const ProjLayout& P = c->lay.p[p];
    if (c->cfg.quant == LS_QUANT_BF16) {
      std::memcpy(blob + P.off_w, w->w[p], P.bytes_w);
      continue;
    }
    if (c->cfg.double_quant) {
      std::vector<float> absmax(P.nblocks);
      pack_nf4_host(w->w[p], P.numel, true, 0, blob + P.off_w, absmax.data(), blob + P.off_qabs,
                    reinterpret_cast<float*>(blob + P.off_scale2), reinterpret_cast<float*>(blob + P.off_mean));
    } else {
      pack_nf4_host(w->w[p], P.numel, false, 0, blob + P.off_w, reinterpret_cast<float*>(blob + P.off_absmax), nullptr,
                    nullptr, nullptr);
    }
  }
  if (ls_status st = store_write(c, layer, blob)) return st;
  c->staged[layer] = 1;
  // the backward reuses the forward's per-layer products, which were made from the
  // old weights: it needs a new forward
  c->fwd_valid = false;
  // a slot holding the old contents of this layer is stale now
  for (auto& sl : c->slot_layer)
    if (sl == layer) sl = -1;
  if (c->cfg.resident) {
    HIPCHK(c, hipMemcpyAsync(slot_ptr(c, layer), blob, c->lay.bytes, hipMemcpyHostToDevice, c->ps));
    HIPCHK(c, hipStreamSynchronize(c->ps));
    c->stats.h2d_bytes += c->lay.bytes;
    c->stats.h2d_copies += 1;
  }
  return LS_OK;
}

ls_status ls_set_lora(ls_ctx* c, int32_t layer, int32_t proj, const float* A, const float* B, float* dA, float* dB) {
  if (ls_status st = check_usable(c)) return st;
  if (layer < 0 || layer >= c->cfg.n_layers || proj < 0 || proj >= LS_N_PROJ)
    return fail(c, LS_ERR_INVALID, "bad layer or projection index");
  if (!A || !B) return fail(c, LS_ERR_INVALID, "null A or B");
  c->lora[layer][proj] = {A, B, dA, dB};
  ++c->lora_version;
  // the forward's s X A^T and the adapters' bf16 copies belong to the old registration
  c->fwd_valid = false;
  return LS_OK;
}

ls_status ls_forward(ls_ctx* c, const void* X, int32_t batch, int32_t seq, int32_t lora_on, void* Y, void* Y_ref) {
  if (ls_status st = check_usable(c)) return st;
  const int64_t T = (int64_t)batch * seq;
  if (batch < 0 || seq < 0 || T > c->cfg.max_tokens || seq > c->cfg.max_seq)
    return fail(c, LS_ERR_INVALID, "batch*seq must be in 0..max_tokens and seq <= max_seq");
  if (seq % 8 != 0) return fail(c, LS_ERR_INVALID, "seq must be a multiple of 8");
  if (T > 0 && (!X || !Y)) return fail(c, LS_ERR_INVALID, "null X or Y");
  for (int l = 0; l < c->cfg.n_layers; ++l)
    if (!c->staged[l]) return fail(c, LS_ERR_STATE, "layer %d not staged", l);
  c->fwd_valid = false;
  c->prof.reset();
  c->prof_collected = false;
  c->in_flight = true;
  if (T == 0) {
    c->fwd_valid = true; c->fwd_lora = lora_on != 0; c->fwd_T = 0; c->fwd_batch = batch; c->fwd_seq = seq;
    c->fwd_ref = Y_ref != nullptr;
    return LS_OK;
  }
  const Dims d = dims_of(c, batch, seq);
  const int L = c->cfg.n_layers;
  const bool lora = lora_on != 0;
  HIPCHK(c, hipMemcpyAsync(ckpt(c, 0), X, 2ull * T * d.h, hipMemcpyDeviceToDevice, c->cs));
  uint16_t* xr[2] = {c->dp<uint16_t>(c->plan.xref), c->dp<uint16_t>(c->plan.xref) + (uint64_t)c->cfg.max_tokens * d.h};
  ls_status st;
  if ((st = ensure_copy(c, 0))) return st;
  for (int l = 0; l < L; ++l) {
    for (int k = 1; k < c->cfg.n_buffers && l + k < L; ++k)
      if ((st = ensure_copy(c, l + k))) return st;
    // a split layer's pieces are waited for inside the (policy) pass, each before its
    // first reader
    const bool split = n_pieces(c, l) > 1;
    // the adapters' bf16 copies do not read the layer's blob: they go ahead of the wait
    // for its copy
    if (lora && (st = prep_lora(c, l, d))) return st;
    if (!split && (st = use_layer(c, l))) return st;
    {
      Span sp(c, c->cs, false);
      const uint8_t* blob = slot_ptr(c, l);
      uint16_t* out = l + 1 < L ? ckpt(c, l + 1) : (uint16_t*)Y;
      const Fence f1{l, split};
      c->prof_layer = l;
      st = layer_forward(c, l, blob, d, ckpt(c, l), out, lora, MODE_FWD, f1, c->cs);
      c->prof_layer = -1;
      if (st) return st;
      if (Y_ref) {
        // layer 0 reads the checkpoint copy of X, so Y may alias X
        const uint16_t* rin = l == 0 ? ckpt(c, 0) : xr[(l - 1) & 1];
        uint16_t* rout = l + 1 < L ? xr[l & 1] : (uint16_t*)Y_ref;
        const Fence f2{l, false};
        c->prof_layer = l;
        st = layer_forward(c, l, blob, d, rin, rout, false, MODE_FWD, f2, c->cs);
        c->prof_layer = -1;
        if (st) return st;
      }
    }
    if ((st = release_layer(c, l))) return st;
  }
  c->fwd_valid = true; c->fwd_lora = lora; c->fwd_T = (int)T; c->fwd_batch = batch; c->fwd_seq = seq;
  c->fwd_ref = Y_ref != nullptr;
  return LS_OK;
}

ls_status ls_backward(ls_ctx* c, const void* dY, void* dX, int32_t accumulate) {
  if (ls_status st = check_usable(c)) return st;
  if (!c->fwd_valid) return fail(c, LS_ERR_STATE, "ls_backward needs a preceding ls_forward");
  if (!c->fwd_lora) return fail(c, LS_ERR_STATE, "ls_backward needs a forward with lora_on = 1");
  const int L = c->cfg.n_layers;
  const float beta = accumulate ? 1.f : 0.f;
  c->in_flight = true;
  if (c->fwd_T == 0) {
    if (!accumulate)
      for (int l = 0; l < L; ++l)
        for (int p = 0; p < LS_N_PROJ; ++p) {
          if (!lora_active(c, l, p)) continue;
          const ProjLayout& P = c->lay.p[p];
          if (c->lora[l][p].dA) HIPCHK(c, launch_fill_f32(c->lora[l][p].dA, (int64_t)c->cfg.lora_r * P.n_in, 0.f, c->cs));
          if (c->lora[l][p].dB) HIPCHK(c, launch_fill_f32(c->lora[l][p].dB, (int64_t)c->cfg.lora_r * P.n_out, 0.f, c->cs));
        }
    return LS_OK;
  }
  if (!dY || !dX) return fail(c, LS_ERR_INVALID, "null dY or dX");
  const Dims d = dims_of(c, c->fwd_batch, c->fwd_seq);
  uint16_t* ping[2] = {c->dp<uint16_t>(c->plan.dya), c->dp<uint16_t>(c->plan.dyb)};
  const uint16_t* cur = (const uint16_t*)dY;
  ls_status st;
  // The recompute of layer l runs on the recompute stream: it waits for the layer's
  // pieces and for its activation set to be free (the backward of layer l + 2 and that
  // backward's reductions done with it).  The backward of layer l, on the compute
  // stream, waits for its recompute.  The recompute of layer l - 1 is enqueued before
  // the backward of layer l, so the two run side by side.  Everything the forward left
  // (checkpoints, s X A^T, row statistics, the activation sets) is ordered before the
  // first recompute by an event on the compute stream.  With LS_PROFILE_ALL every
  // recompute instead follows the backward before it, so that no recompute kernel's
  // timing includes time it shares the GPU with another layer's backward.
  const bool serial = c->cfg.profile == LS_PROFILE_ALL;
  auto rs_after_cs = [&]() -> ls_status {
    HIPCHK(c, hipEventRecord(c->fork_ev, c->cs));
    HIPCHK(c, hipStreamWaitEvent(c->rs, c->fork_ev, 0));
    return LS_OK;
  };
  if ((st = rs_after_cs())) return st;
  auto recompute = [&](int l) -> ls_status {
    const int k = l & 1;
    if (c->bp_rec[k]) HIPCHK(c, hipStreamWaitEvent(c->rs, c->bp_done[k], 0));
    if (c->side_rec[k]) HIPCHK(c, hipStreamWaitEvent(c->rs, c->side_done[k], 0));
    const bool split = n_pieces(c, l) > 1;
    ls_status s2;
    if (!split && (s2 = use_layer(c, l, c->rs))) return s2;
    {
      Span sp(c, c->rs, false);
      const Fence f{l, split};   // pieces 0, 1 (and 2 without the paired gate | up kernel)
      c->in_recompute = true;
      s2 = layer_forward(c, l, slot_ptr(c, l), d, ckpt(c, l), nullptr, true, MODE_RECOMPUTE, f, c->rs);
      c->in_recompute = false;
      if (s2) return s2;
    }
    HIPCHK(c, hipEventRecord(c->rec_done[k], c->rs));
    return LS_OK;
  };
  if ((st = ensure_copy(c, L - 1))) return st;
  if (!serial && (st = recompute(L - 1))) return st;
  for (int l = L - 1; l >= 0; --l) {
    for (int k = 1; k < c->cfg.n_buffers && l - k >= 0; ++k)
      if ((st = ensure_copy(c, l - k))) return st;
    if (serial) {
      if ((st = rs_after_cs()) || (st = recompute(l))) return st;
    } else if (l >= 1 && (st = recompute(l - 1))) {
      return st;
    }
    const bool split = n_pieces(c, l) > 1;
    HIPCHK(c, hipStreamWaitEvent(c->cs, c->rec_done[l & 1], 0));
    if (!split && (st = use_layer(c, l))) return st;
    uint16_t* out = l == 0 ? (uint16_t*)dX : ping[l & 1];
    {
      Span sp(c, c->cs, false);
      const Fence f{l, split};   // pieces 3 and (with the paired gate | up kernel) 2
      if ((st = layer_backward(c, l, slot_ptr(c, l), d, ckpt(c, l), cur, out, beta, f))) return st;
    }
    if ((st = release_layer(c, l))) return st;
    cur = out;
  }
  return join_side(c);   // the compute stream's completion covers dA and dB
}

ls_status ls_sync(ls_ctx* c) {
  if (!c) return LS_ERR_INVALID;
  if (c->sticky != LS_OK) return c->sticky;
  HIPCHK(c, hipStreamSynchronize(c->ps));
  HIPCHK(c, hipStreamSynchronize(c->side));
  HIPCHK(c, hipStreamSynchronize(c->rs));
  HIPCHK(c, hipStreamSynchronize(c->cs));
  HIPCHK(c, hipGetLastError());
  c->in_flight = false;
  collect_profile(c);
  c->prof_collected = true;
  if (const int e = c->store_err.load()) {
    c->sticky = LS_ERR_HIP;
    return fail(c, LS_ERR_HIP, "read from the store file failed: %s", strerror(e));
  }
  return LS_OK;
}

ls_status ls_get_stats(const ls_ctx* c, ls_stats* out) {
  if (!c || !out) return LS_ERR_INVALID;
  *out = c->stats;
  out->store_reads = c->store_reads.load();
  return LS_OK;
}

const char* ls_last_error(const ls_ctx* c) { return c ? c->err.c_str() : g_create_err.c_str(); }

void ls_destroy(ls_ctx* c) {
  if (!c) return;
  // best effort: nothing can be reported from here, every release is attempted
  if (c->cs) (void)hipStreamSynchronize(c->cs);
  if (c->ps) (void)hipStreamSynchronize(c->ps);
  if (c->side) (void)hipStreamSynchronize(c->side);
  if (c->rs) (void)hipStreamSynchronize(c->rs);
  for (auto e : c->prof.pool) (void)hipEventDestroy(e);
  if (c->fork_ev) (void)hipEventDestroy(c->fork_ev);
  if (c->join_ev) (void)hipEventDestroy(c->join_ev);
  for (int k = 0; k < 2; ++k) {
    if (c->rec_done[k]) (void)hipEventDestroy(c->rec_done[k]);
    if (c->bp_done[k]) (void)hipEventDestroy(c->bp_done[k]);
    if (c->side_done[k]) (void)hipEventDestroy(c->side_done[k]);
  }
  for (auto e : c->ready) if (e) (void)hipEventDestroy(e);
  for (auto e : c->consumed) if (e) (void)hipEventDestroy(e);
  if (c->dbase) (void)hipFree(c->dbase);
  for (auto p : c->host) if (p) (void)hipHostFree(p);
  for (auto p : c->staging) if (p) (void)hipHostFree(p);
  if (c->fd >= 0) {
    close(c->fd);
    unlink(c->cfg.store_path);
  }
  if (c->own_cs && c->cs) (void)hipStreamDestroy(c->cs);
  if (c->own_ps && c->ps) (void)hipStreamDestroy(c->ps);
  if (c->side) (void)hipStreamDestroy(c->side);
  if (c->rs) (void)hipStreamDestroy(c->rs);
  delete c;
}

ls_status ls_read_weight(ls_ctx* c, int32_t layer, int32_t proj, void* out) {
  if (ls_status st = check_usable(c)) return st;
  if (layer < 0 || layer >= c->cfg.n_layers || proj < 0 || proj >= LS_N_PROJ || !out)
    return fail(c, LS_ERR_INVALID, "bad layer/projection index or null out");
  if (!c->staged[layer]) return fail(c, LS_ERR_STATE, "layer %d not staged", layer);
  if (c->in_flight) return fail(c, LS_ERR_STATE, "a forward/backward is in flight: call ls_sync first");
  ls_status st;
  if ((st = ensure_copy(c, layer))) return st;
  if ((st = use_layer(c, layer))) return st;
  HIPCHK(c, launch_dequant(wref(c, slot_ptr(c, layer), proj), wformat(c->cfg), c->dp<float>(c->plan.levels),
                           (uint16_t*)out, c->cs));
  if ((st = release_layer(c, layer))) return st;
  HIPCHK(c, hipStreamSynchronize(c->cs));
  HIPCHK(c, hipStreamSynchronize(c->ps));
  return LS_OK;
}

ls_status ls_base_gemm(ls_ctx* c, int32_t layer, int32_t group, int32_t transposed, const void* X, int32_t M,
                       float* out) {
  if (ls_status st = check_usable(c)) return st;
  if (layer < 0 || layer >= c->cfg.n_layers || group < 0 || group > 3 || !X || !out || M < 1 || M > c->cfg.max_tokens)
    return fail(c, LS_ERR_INVALID, "bad layer/group index, null pointer, or M outside 1..max_tokens");
  if (!c->staged[layer]) return fail(c, LS_ERR_STATE, "layer %d not staged", layer);
  if (c->in_flight) return fail(c, LS_ERR_STATE, "a forward/backward is in flight: call ls_sync first");
  const Dims d = dims_of(c, 1, 1);
  const int fmt = wformat(c->cfg);
  const float* lv = c->dp<float>(c->plan.levels);
  static const int p0s[4] = {LS_PROJ_Q, LS_PROJ_O, LS_PROJ_GATE, LS_PROJ_DOWN};
  static const int ngs[4] = {3, 1, 2, 1};
  const int p0 = p0s[group], ng = ngs[group];
  ls_status st;
  if ((st = ensure_copy(c, layer))) return st;
  if ((st = use_layer(c, layer))) return st;
  const uint8_t* blob = slot_ptr(c, layer);
  int out_w = 0;
  for (int i = 0; i < ng; ++i) out_w += c->lay.p[p0 + i].n_out;
  const int n_in = c->lay.p[p0].n_in;
  if (!transposed) {
    FwdArgs f;
    f.x = (const uint16_t*)X; f.ldx = n_in; f.M = M; f.K = n_in; f.n_groups = ng;
    int col = 0;
    for (int i = 0; i < ng; ++i) {
      f.g[i].w = wref(c, blob, p0 + i);
      f.g[i].out_col0 = col;
      col += c->lay.p[p0 + i].n_out;
    }
    f.levels = lv; f.format = fmt;
    if (group == 2 && 2 * d.r16 <= 64) {
      // the forward's paired kernel: act is written to the workspace, gate and up in
      // float32 to out
      f.swiglu = 1; f.y = c->dp<uint16_t>(c->plan.act[0]); f.ldy = d.I;
      f.gu32 = out; f.ldgu = out_w;
    } else {
      f.y32 = out; f.ldy = out_w;
    }
    f.sk = c->split_scratch(c->cs);
    HIPCHK(c, launch_gemm_fwd(f, c->cs));
  } else {
    BwdArgs b;
    b.dy = (const uint16_t*)X; b.lddy = out_w; b.M = M; b.N = n_in; b.n_segs = ng;
    int col = 0;
    for (int i = 0; i < ng; ++i) {
      b.seg[i].w = wref(c, blob, p0 + i);
      b.seg[i].a_col0 = col;
      col += c->lay.p[p0 + i].n_out;
    }
    b.out32 = out; b.ldo = n_in; b.levels = lv; b.format = fmt;
    b.sk = c->split_scratch(c->cs);
    HIPCHK(c, launch_gemm_bwd(b, c->cs));
  }
  if ((st = release_layer(c, layer))) return st;
  HIPCHK(c, hipStreamSynchronize(c->cs));
  HIPCHK(c, hipStreamSynchronize(c->ps));
  return LS_OK;
}

// ------------------------------------------------------------ AdamW and adapter files
ls_status ls_adamw_step(ls_ctx* c, const ls_adamw* hp) {
  if (ls_status st = check_usable(c)) return st;
  if (!c->cfg.adamw) return fail(c, LS_ERR_STATE, "AdamW moments were not planned (ls_config.adamw = 0)");
  if (!hp) return fail(c, LS_ERR_INVALID, "null hyperparameters");
  const bool ok = std::isfinite(hp->lr) && hp->lr >= 0.f && hp->beta1 >= 0.f && hp->beta1 < 1.f &&
                  hp->beta2 >= 0.f && hp->beta2 < 1.f && std::isfinite(hp->eps) && hp->eps > 0.f &&
                  std::isfinite(hp->weight_decay) && hp->weight_decay >= 0.f && hp->step >= 1;
  if (!ok) return fail(c, LS_ERR_INVALID, "AdamW: need lr >= 0, beta1 and beta2 in [0, 1), eps > 0, weight_decay >= 0, step >= 1");
  if (c->adam_version != c->lora_version) {
    // one chunk table over every adapter tensor that has a gradient buffer; the
    // moments follow the plan's order (layer, projection, A then B)
    c->adam_host.clear();
    double elems = 0;
    float* m0 = c->dp<float>(c->plan.moments);
    float* v0 = m0 + c->plan.moment_elems;
    uint64_t moff = 0;
    auto al16 = [](const void* q) { return (reinterpret_cast<uintptr_t>(q) & 15u) == 0; };
    for (const AdapterEntry& e : adapter_entries(c->cfg)) {
      const uint64_t n = (uint64_t)e.rows * (uint64_t)e.cols;
      const LoraReg& R = c->lora[e.layer][e.proj];
      float* prm = const_cast<float*>(e.which ? R.B : R.A);
      const float* grd = e.which ? R.dB : R.dA;
      if (prm && grd && R.A && R.B) {
        for (uint64_t o = 0; o < n; o += kAdamChunk) {
          AdamChunk ch;
          ch.p = prm + o; ch.g = grd + o; ch.m = m0 + moff + o; ch.v = v0 + moff + o;
          ch.n = (uint32_t)std::min<uint64_t>(kAdamChunk, n - o);
          ch.vec4 = (ch.n % 4 == 0 && al16(ch.p) && al16(ch.g) && al16(ch.m) && al16(ch.v)) ? 1u : 0u;
          c->adam_host.push_back(ch);
        }
        elems += (double)n;
      }
      moff += n;
    }
    if (c->adam_host.size() > c->plan.adam_max_chunks) return fail(c, LS_ERR_INVALID, "internal: AdamW table overflow");
    if (!c->adam_host.empty())
      HIPCHK(c, hipMemcpyAsync(c->dbase + c->plan.adam_tab, c->adam_host.data(), c->adam_host.size() * sizeof(AdamChunk),
                               hipMemcpyHostToDevice, c->cs));
    c->adam_elems = elems;
    c->adam_version = c->lora_version;
  }
  AdamHyper h;
  const double lr = hp->lr, b1 = hp->beta1, b2 = hp->beta2;
  h.decay_mul = (float)(1.0 - lr * (double)hp->weight_decay);
  h.beta1 = hp->beta1; h.one_m_beta1 = (float)(1.0 - b1);
  h.beta2 = hp->beta2; h.one_m_beta2 = (float)(1.0 - b2);
  h.step_size = (float)(lr / (1.0 - std::pow(b1, (double)hp->step)));
  h.inv_bc2_sqrt = (float)(1.0 / std::sqrt(1.0 - std::pow(b2, (double)hp->step)));
  h.eps = hp->eps;
  if (c->prof_collected) { c->prof.reset(); c->prof_collected = false; }
  if (c->cfg.profile == LS_PROFILE_ALL && c->prof.origin == (size_t)-1) {
    hipEvent_t e;
    size_t i;
    if (c->prof.next(&e, &i) == hipSuccess && hipEventRecord(e, c->cs) == hipSuccess) c->prof.origin = i;
  }
  c->in_flight = true;
  {
    // algorithmic bytes: p, g, m, v read and p, m, v written, float32
    KTimer kt(c, LS_KC_OPTIM, 0.0, 28.0 * c->adam_elems);
    HIPCHK(c, launch_adamw(reinterpret_cast<const AdamChunk*>(c->dbase + c->plan.adam_tab),
                           (int32_t)c->adam_host.size(), h, c->cs));
  }
  return LS_OK;
}

ls_status ls_adamw_reset(ls_ctx* c) {
  if (ls_status st = check_usable(c)) return st;
  if (!c->cfg.adamw) return fail(c, LS_ERR_STATE, "AdamW moments were not planned (ls_config.adamw = 0)");
  HIPCHK(c, launch_fill_f32(c->dp<float>(c->plan.moments), (int64_t)(2 * c->plan.moment_elems), 0.f, c->cs));
  return LS_OK;
}

static ls_status require_adapters(ls_ctx* c, const std::vector<AdapterEntry>& es) {
  for (const AdapterEntry& e : es)
    if (!c->lora[e.layer][e.proj].A || !c->lora[e.layer][e.proj].B)
      return fail(c, LS_ERR_STATE, "adapter of layer %d projection %d is not registered", e.layer, e.proj);
  return LS_OK;
}

ls_status ls_save_adapters(ls_ctx* c, const char* path) {
  if (ls_status st = check_usable(c)) return st;
  if (!path) return fail(c, LS_ERR_INVALID, "null path");
  const std::vector<AdapterEntry> es = adapter_entries(c->cfg);
  if (ls_status st = require_adapters(c, es)) return st;
  std::vector<std::vector<float>> host(es.size());
  std::vector<const float*> ptrs(es.size());
  HIPCHK(c, hipStreamSynchronize(c->cs));
  for (size_t i = 0; i < es.size(); ++i) {
    const LoraReg& R = c->lora[es[i].layer][es[i].proj];
    host[i].resize((size_t)(es[i].rows * es[i].cols));
    HIPCHK(c, hipMemcpyAsync(host[i].data(), es[i].which ? R.B : R.A, host[i].size() * sizeof(float),
                             hipMemcpyDeviceToHost, c->cs));
    ptrs[i] = host[i].data();
  }
  HIPCHK(c, hipStreamSynchronize(c->cs));
  std::string err = adapter_write(c->cfg, es, ptrs, path);
  if (!err.empty()) return fail(c, LS_ERR_INVALID, "%s", err.c_str());
  err = adapter_check(c->cfg, path, nullptr, nullptr);
  if (!err.empty()) return fail(c, LS_ERR_INVALID, "read-back check of %s failed: %s", path, err.c_str());
  return LS_OK;
}

ls_status ls_load_adapters(ls_ctx* c, const char* path) {
  if (ls_status st = check_usable(c)) return st;
  if (!path) return fail(c, LS_ERR_INVALID, "null path");
  if (ls_status st = require_adapters(c, adapter_entries(c->cfg))) return st;
  std::vector<AdapterEntry> es;
  std::vector<uint8_t> bytes;
  const std::string err = adapter_check(c->cfg, path, &es, &bytes);
  if (!err.empty()) return fail(c, LS_ERR_INVALID, "%s: %s", path, err.c_str());
  for (const AdapterEntry& e : es) {
    const LoraReg& R = c->lora[e.layer][e.proj];
    HIPCHK(c, hipMemcpyAsync(const_cast<float*>(e.which ? R.B : R.A), bytes.data() + e.offset,
                             (size_t)(4 * e.rows * e.cols), hipMemcpyHostToDevice, c->cs));
  }
  HIPCHK(c, hipStreamSynchronize(c->cs));
  return LS_OK;
}

ls_status ls_check_adapter_file(const ls_config* cfg, const char* path, char* msg, size_t msg_len) {
  auto say = [&](const std::string& m) {
    if (msg && msg_len) {
      const size_t n = std::min(m.size(), msg_len - 1);
      memcpy(msg, m.data(), n);
      msg[n] = 0;
    }
  };
  if (!cfg || !path) { say("null cfg or path"); return LS_ERR_INVALID; }
  const char* why = nullptr;
  if (!validate_config(*cfg, &why)) { say(std::string("invalid config: ") + why); return LS_ERR_INVALID; }
  const std::string err = adapter_check(*cfg, path, nullptr, nullptr);
  say(err.empty() ? "ok" : err);
  return err.empty() ? LS_OK : LS_ERR_INVALID;
}

// ------------------------------------------------------------------ output head and loss
ls_status ls_stage_head(ls_ctx* c, const uint16_t* w, const uint16_t* g_final) {
  if (ls_status st = check_usable(c)) return st;
  if (c->cfg.vocab <= 0) return fail(c, LS_ERR_STATE, "no output head planned (ls_config.vocab = 0)");
  if (!w || !g_final) return fail(c, LS_ERR_INVALID, "null head or norm weight");
  if (c->in_flight) return fail(c, LS_ERR_STATE, "work is in flight: call ls_sync first");
  const int L = c->cfg.n_layers, S = c->plan.head_slices, vs = c->plan.head_rows;
  const uint64_t row = 2ull * c->cfg.hidden;
  for (int j = 0; j < S; ++j) {
    const int64_t r0 = (int64_t)j * vs, rows = std::min<int64_t>(vs, c->cfg.vocab - r0);
    uint8_t* blob = stage_buffer(c, L + j);
    std::memcpy(blob, reinterpret_cast<const uint8_t*>(w) + (uint64_t)r0 * row, (uint64_t)rows * row);
    if (ls_status st = store_write(c, L + j, blob)) return st;
    for (auto& sl : c->slot_layer)
      if (sl == L + j) sl = -1;
    if (c->cfg.resident) {
      HIPCHK(c, hipMemcpyAsync(slot_ptr(c, L + j), blob, c->lay.bytes, hipMemcpyHostToDevice, c->ps));
      HIPCHK(c, hipStreamSynchronize(c->ps));
      c->stats.h2d_bytes += c->lay.bytes;
      c->stats.h2d_copies += 1;
    }
  }
  HIPCHK(c, hipMemcpyAsync(c->dbase + c->plan.gfin, g_final, row, hipMemcpyHostToDevice, c->ps));
  HIPCHK(c, hipStreamSynchronize(c->ps));
  c->head_staged = true;
  return LS_OK;
}

// the bf16 head slice j held in its slot, as the GEMMs take a weight
static WeightRef head_ref(const ls_ctx* c, int j) {
  WeightRef r;
  r.w = slot_ptr(const_cast<ls_ctx*>(c), c->cfg.n_layers + j);
  r.n_out = std::min<int32_t>(c->plan.head_rows, c->cfg.vocab - j * c->plan.head_rows);
  r.n_in = c->cfg.hidden;
  return r;
}

ls_status ls_head_loss(ls_ctx* c, const void* Y, const void* Y_ref, const int32_t* labels, int32_t kind, float beta,
                       float* out, void* dY) {
  if (ls_status st = check_usable(c)) return st;
  if (c->cfg.vocab <= 0 || !c->head_staged) return fail(c, LS_ERR_STATE, "no output head staged");
  if (!c->fwd_valid || c->fwd_T == 0) return fail(c, LS_ERR_STATE, "ls_head_loss needs a preceding non-empty ls_forward");
  if (kind != LS_LOSS_SFT && kind != LS_LOSS_DPO) return fail(c, LS_ERR_INVALID, "unknown loss kind %d", kind);
  if (!Y || !labels || !out || !dY) return fail(c, LS_ERR_INVALID, "null Y, labels, out or dY");
  const int T = c->fwd_T, seq = c->fwd_seq, nseq = c->fwd_batch;
  if (nseq > 1024) return fail(c, LS_ERR_INVALID, "at most 1024 sequences per call");
  const bool dpo = kind == LS_LOSS_DPO;
  if (dpo) {
    if (!Y_ref) return fail(c, LS_ERR_INVALID, "DPO needs the reference output Y_ref");
    if (!c->fwd_ref) return fail(c, LS_ERR_STATE, "DPO needs a forward that ran the reference pass");
    if (nseq % 2 != 0) return fail(c, LS_ERR_INVALID, "DPO needs an even batch (chosen, rejected pairs)");
    if (!(beta > 0.f) || !std::isfinite(beta)) return fail(c, LS_ERR_INVALID, "DPO beta must be > 0");
  }
  const int L = c->cfg.n_layers, S = c->plan.head_slices, h = c->cfg.hidden, vocab = c->cfg.vocab;
  const int ldz = c->plan.ldz;
  const float* lv = c->dp<float>(c->plan.levels);
  uint16_t* yn = c->dp<uint16_t>(c->plan.hyn);
  uint16_t* ynr = c->dp<uint16_t>(c->plan.hynr);
  const uint16_t* gf = c->dp<uint16_t>(c->plan.gfin);
  float* rstd = c->dp<float>(c->plan.hrstd);
  float* Z = c->dp<float>(c->plan.hz);
  uint16_t* dZ = c->dp<uint16_t>(c->plan.hdz);
  float* dyn = c->dp<float>(c->plan.hdyn);
  float *pm = c->dp<float>(c->plan.hpm), *ps = c->dp<float>(c->plan.hps), *pz = c->dp<float>(c->plan.hpz);
  float *rm = c->dp<float>(c->plan.hrm), *rs = c->dp<float>(c->plan.hrs), *rz = c->dp<float>(c->plan.hrz);
  float* coef = c->dp<float>(c->plan.hcoef);
  const int32_t* lab = labels;
  if (c->prof_collected) { c->prof.reset(); c->prof_collected = false; }
  c->in_flight = true;
  ls_status st;
  auto logits = [&](const uint16_t* x, int j) -> ls_status {
    const WeightRef w = head_ref(c, j);
    FwdArgs a;
    a.x = x; a.ldx = h; a.M = T; a.K = h; a.n_groups = 1;
    a.g[0].w = w;
    a.y32 = Z; a.ldy = ldz; a.levels = lv; a.format = WF_BF16;
    a.sk = c->split_scratch(c->cs);
    KTimer kt(c, LS_KC_HEAD, 2.0 * T * w.n_out * h, 2.0 * T * h + 2.0 * w.n_out * h + 4.0 * T * w.n_out);
    HIPCHK(c, launch_gemm_fwd(a, c->cs));
    return LS_OK;
  };
  {
    KTimer kt(c, LS_KC_HEAD, 0.0, (dpo ? 2.0 : 1.0) * 4.0 * T * h);
    HIPCHK(c, launch_rmsnorm_fwd((const uint16_t*)Y, nullptr, gf, yn, rstd, T, h, c->cfg.rms_eps, c->cs));
    if (dpo)
      HIPCHK(c, launch_rmsnorm_fwd((const uint16_t*)Y_ref, nullptr, gf, ynr, c->dp<float>(c->plan.hrstd2), T, h,
                                   c->cfg.rms_eps, c->cs));
  }
  // pass 1 over the slices: softmax statistics of the policy (and the reference)
  if ((st = ensure_copy(c, L))) return st;
  for (int j = 0; j < S; ++j) {
    for (int k = 1; k < c->cfg.n_buffers && j + k < S; ++k)
      if ((st = ensure_copy(c, L + j + k))) return st;
    if ((st = use_layer(c, L + j))) return st;
    {
      Span sp(c, c->cs, false);
      const int vs = head_ref(c, j).n_out, v0 = j * c->plan.head_rows;
      if ((st = logits(yn, j))) return st;
      {
        KTimer kt(c, LS_KC_HEAD, 0.0, 4.0 * T * vs);
        HIPCHK(c, launch_ce_stats(Z, ldz, vs, v0, lab, T, vocab, pm, ps, pz, j == 0, c->cs));
      }
      if (dpo) {
        if ((st = logits(ynr, j))) return st;
        KTimer kt(c, LS_KC_HEAD, 0.0, 4.0 * T * vs);
        HIPCHK(c, launch_ce_stats(Z, ldz, vs, v0, lab, T, vocab, rm, rs, rz, j == 0, c->cs));
      }
    }
    if ((st = release_layer(c, L + j))) return st;
  }
  {
    KTimer kt(c, LS_KC_HEAD, 0.0, 16.0 * T);
    HIPCHK(c, launch_loss_finalize(kind, beta, T, seq, vocab, lab, pm, ps, pz, dpo ? rm : nullptr, dpo ? rs : nullptr,
                                   dpo ? rz : nullptr, coef, out, c->cs));
  }
  // pass 2, slices in reverse: recompute the logits, dz, and dyn += dz W_j
  if ((st = ensure_copy(c, L + S - 1))) return st;
  for (int j = S - 1; j >= 0; --j) {
    for (int k = 1; k < c->cfg.n_buffers && j - k >= 0; ++k)
      if ((st = ensure_copy(c, L + j - k))) return st;
    if ((st = use_layer(c, L + j))) return st;
    {
      Span sp(c, c->cs, false);
      const WeightRef w = head_ref(c, j);
      const int vs = w.n_out, v0 = j * c->plan.head_rows;
      if ((st = logits(yn, j))) return st;
      {
        KTimer kt(c, LS_KC_HEAD, 0.0, 4.0 * T * vs + 2.0 * T * vs);
        HIPCHK(c, launch_ce_grad(Z, ldz, vs, v0, lab, T, seq, vocab, pm, ps, coef, dZ, c->cs));
      }
      BwdArgs b;
      b.dy = dZ; b.lddy = ldz; b.M = T; b.N = h; b.n_segs = 1;
      b.seg[0].w = w;
      b.out32 = dyn; b.ldo = h; b.resid32 = j == S - 1 ? nullptr : dyn;
      b.levels = lv; b.format = WF_BF16;
      KTimer kt(c, LS_KC_HEAD, 2.0 * T * vs * h, 2.0 * T * vs + 2.0 * vs * h + 4.0 * T * h * (j == S - 1 ? 1 : 2));
      b.sk = c->split_scratch(c->cs);
      HIPCHK(c, launch_gemm_bwd(b, c->cs));
    }
    if ((st = release_layer(c, L + j))) return st;
  }
  {
    KTimer kt(c, LS_KC_HEAD, 0.0, 4.0 * T * h + 4.0 * T * h);
    HIPCHK(c, launch_rmsnorm_bwd(dyn, (const uint16_t*)Y, nullptr, gf, rstd, nullptr, nullptr, nullptr, (uint16_t*)dY,
                                 T, h, c->cs));
  }
  return LS_OK;
}

ls_status ls_set_profile(ls_ctx* c, int32_t profile) {
  if (ls_status st = check_usable(c)) return st;
  if (profile != LS_PROFILE_OFF && profile != LS_PROFILE_ALL && profile != LS_PROFILE_GEMM)
    return fail(c, LS_ERR_INVALID, "unknown profiling level %d", profile);
  if (c->in_flight) return fail(c, LS_ERR_STATE, "work is in flight: call ls_sync first");
  c->cfg.profile = profile;
  c->prof.reset();
  c->prof_collected = false;
  return LS_OK;
}

}  // extern "C"
