/*
 * ls.h — C ABI of the layer-streamed LoRA library (liblsq.so), MI355X / gfx950.
 *
 * What the library computes.  A frozen decoder stack lives in pinned host RAM, each
 * layer either NF4-packed (4-bit codes, one absmax per 64 weights, optionally a
 * second 8-bit level over the absmax values) or plain bf16.  Every layer is copied
 * into a small device pool on a dedicated copy stream so that the next layer loads
 * while the current one computes, and is copied again for the recompute backward
 * ("Soup: Fine-Tuning an 8B Model on a 4 GB Laptop GPU, One Layer at a Time",
 * first paragraph; the lachieslifestyle.com Soup how-to, section "What Soup layer
 * streaming changes"; "Soup CLI fine-tunes Llama-3.1-8B on a 4 GB laptop GPU ...",
 * second paragraph).  Every projection p in {q,k,v,o,gate,up,down} computes
 *     Y = X dequant(W_p)^T + (alpha/r) (X A_p^T) B_p^T
 * and the backward returns dX plus dA_p, dB_p for the trainable adapters
 * ("Fine-Tuning an 8B Parameter Model on a 4 GB Laptop GPU", section "LoRA and
 * QLoRA: Train a Fraction of the Parameters").  The layer is the Llama-style
 * pre-norm decoder (RMSNorm, rotary q/k, causal grouped-query attention, SwiGLU).
 *
 * Conventions for every entry point.
 *  - Plain C types only.  "Device pointer" = memory from hipMalloc (or a torch CUDA
 *    tensor's data_ptr()) on the context's device; "host pointer" = ordinary memory.
 *  - bf16 tensors are passed as void* / uint16_t* holding IEEE bfloat16 bit patterns,
 *    row-major.  Activations are token-major [T, features], T = batch * seq, token
 *    t = b * seq + s (position s inside its sequence).
 *  - Weights are [out_features, in_features] row-major.  LoRA A_p is [r, in] and
 *    B_p is [out, r], both float32.
 *  - Every call returns an ls_status; no exception crosses the ABI.  A failing call
 *    leaves a message for ls_last_error().  LS_ERR_HIP is sticky: once a HIP call
 *    has failed, every later call on that context returns LS_ERR_HIP.
 *  - Calls on one context must not run concurrently from several host threads.
 */
#ifndef LS_H_
#define LS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ls_status {
  LS_OK = 0,
  LS_ERR_INVALID = 1, /* bad argument: null pointer, size out of range, bad config */
  LS_ERR_STATE = 2,   /* call out of order (e.g. backward before forward, unstaged layer) */
  LS_ERR_BUDGET = 3,  /* the device-memory plan exceeds the budget; nothing allocated */
  LS_ERR_OOM = 4,     /* an allocation (pinned host or device) failed */
  LS_ERR_HIP = 5      /* a HIP runtime call or kernel launch failed (sticky) */
} ls_status;

enum { LS_QUANT_NF4 = 0, LS_QUANT_BF16 = 1 };

/* Projection indices, also the bit positions of ls_config.lora_mask. */
enum { LS_PROJ_Q = 0, LS_PROJ_K, LS_PROJ_V, LS_PROJ_O, LS_PROJ_GATE, LS_PROJ_UP, LS_PROJ_DOWN, LS_N_PROJ };

/*
 * Stack description.  Field meaning follows the streaming configuration the
 * lachieslifestyle.com how-to shows in "Step 5: Enable 4-bit layer streaming"
 * (quantization 4bit|none, stream_buffers, lora r / alpha / target modules).
 */
typedef struct ls_config {
  int32_t n_layers;        /* >= 1 */
  int32_t hidden;          /* model width h, multiple of 64 */
  int32_t n_heads;         /* query heads */
  int32_t n_kv_heads;      /* key/value heads; n_heads % n_kv_heads == 0 */
  int32_t head_dim;        /* 64 or 128; n_heads * head_dim and n_kv_heads * head_dim multiples of 64 */
  int32_t intermediate;    /* SwiGLU width I, multiple of 16 */
  float rms_eps;           /* RMSNorm epsilon */
  float rope_theta;        /* rotary base */
  int32_t quant;           /* LS_QUANT_NF4 or LS_QUANT_BF16 */
  int32_t nf4_block;       /* must be 64 */
  int32_t double_quant;    /* NF4 only: 1 = 8-bit absmax codes per group of 256 blocks */
  int32_t lora_r;          /* 1..64 */
  float lora_alpha;        /* LoRA scale is lora_alpha / lora_r */
  uint32_t lora_mask;      /* bit p set = adapter on projection p (bits 0..6) */
  int32_t n_buffers;       /* device slots in the streaming pool: 2..64, or 0 = the deepest
                              pool (at most one slot per layer) that fits vram_budget, or half
                              of the free device memory when vram_budget is 0 */
  int32_t max_tokens;      /* upper bound on batch * seq for every call */
  int32_t max_seq;         /* upper bound on seq (attention scratch is sized by it) */
  int32_t resident;        /* 1 = keep every layer on the device (same blob layout;
                              parity reference for the streamed mode) */
  uint64_t vram_budget;    /* bytes the plan may use; 0 = free device memory */
  int32_t profile;         /* LS_PROFILE_OFF, LS_PROFILE_ALL or LS_PROFILE_GEMM (see ls_set_profile) */
  int32_t adamw;           /* 1 = also plan float32 AdamW moments (m and v) for every
                              adapter of lora_mask and enable ls_adamw_step */
  int32_t vocab;           /* 0 = no output head; else rows of the frozen bf16 output head
                              [vocab, hidden] (ls_stage_head, ls_head_loss) */
  int32_t store;           /* LS_STORE_HOST: the frozen base in pinned host RAM;
                              LS_STORE_FILE: in the file store_path (one blob per layer and
                              head slice), read into one pinned staging buffer per slot */
  char store_path[256];    /* LS_STORE_FILE: NUL-terminated path; the file is created (or
                              truncated) by ls_create and removed by ls_destroy */
  int32_t copy_split;      /* 0 = each decoder layer crosses the link as one copy followed
                              by one ready event; 1 = as four pieces in the order the layer
                              first reads them (g1, g2 and q|k|v; o; gate|up; down), each
                              followed by its own ready event, and the compute stream waits
                              for a piece just before its first reader, so a layer starts
                              while its later pieces are still in flight.  Either way a slot
                              is refilled only after the last reader of the whole layer
                              (one consumed event per slot).  Streamed mode only (ignored
                              when resident); results are bitwise the same either way.  The
                              pool's buffer count is a setting in the lachieslifestyle.com
                              Soup how-to ("Step 5: Enable 4-bit layer streaming"), which
                              also lists small stream buffers among the causes of slow
                              training ("Common problems"); the split makes the unit the
                              compute waits for one projection group instead of a layer. */
  int32_t profile_stride;  /* LS_PROFILE_GEMM: time the forward dequant-GEMM launches of
                              every profile_stride-th layer only (layers 0, stride, 2 stride,
                              ...; 0 or 1 = every layer).  Every layer has the same shapes,
                              so a sample times the class while recording fewer events in
                              the stream. */
} ls_config;

/* Where the frozen base lives ("Soup CLI fine-tunes Llama-3.1-8B on a 4 GB laptop GPU
 * ...", third paragraph: the base stays in CPU RAM or on NVMe). */
enum { LS_STORE_HOST = 0, LS_STORE_FILE = 1 };

/* Host-side source weights for one layer (bf16 bit patterns, host pointers). */
typedef struct ls_layer_host {
  const uint16_t* w[LS_N_PROJ]; /* [out, in] row-major per projection */
  const uint16_t* g1;           /* [hidden] RMSNorm weight before attention */
  const uint16_t* g2;           /* [hidden] RMSNorm weight before the MLP */
} ls_layer_host;

/* Kernel classes timed when ls_config.profile = 1. */
enum {
  LS_KC_GEMM_FWD = 0, /* fused dequant GEMM, W orientation (forward and recompute) */
  LS_KC_GEMM_BWD = 1, /* fused dequant GEMM, W^T orientation (dX) */
  LS_KC_ATTN = 2,     /* attention products and softmax */
  LS_KC_LORA = 3,     /* LoRA down projection and dA / dB / G products, operand conversion */
  LS_KC_GLUE = 4,     /* RMSNorm, rotary embedding, SwiGLU */
  LS_KC_OPTIM = 5,    /* AdamW update of the adapters (ls_adamw_step) */
  LS_KC_HEAD = 6,     /* output head products, softmax statistics and loss (ls_head_loss) */
  LS_KC_N = 7
};

/* Losses of ls_head_loss. */
enum { LS_LOSS_SFT = 0, LS_LOSS_DPO = 1 };
#define LS_LABEL_IGNORE (-100)

typedef struct ls_stats {
  uint64_t blob_bytes;         /* bytes of one layer blob (same host and device) */
  uint64_t store_bytes;        /* pinned host bytes of the whole store */
  uint64_t device_bytes;       /* device bytes the plan allocated */
  uint64_t h2d_bytes;          /* host->device layer bytes copied since create */
  uint64_t h2d_copies;         /* layer copies since create */
  uint64_t slot_hits;          /* layer reads served by a slot that already held it */
  uint64_t store_reads;        /* LS_STORE_FILE: blobs read from the file since create */
  uint64_t store_uncached;     /* LS_STORE_FILE: 1 if every blob is dropped from the OS page cache
                                  after use, so each read comes from the file's device */
  uint64_t n_slots;            /* device slots of the pool (resident: one per blob) */
  uint64_t poison_fills;       /* LS_DEBUG_POISON: slots filled with 0xFF before a copy */
  double last_copy_ms;         /* profile=1: summed copy time of the last fwd+bwd */
  double last_compute_ms;      /* profile=1: summed per-layer compute time of last fwd+bwd */
  double last_overlap_ms;      /* profile=1: copy time that overlapped compute */
  double last_span_ms;         /* profile=1: first event to last event of last fwd+bwd */
  /* profile=1, per kernel class, over the last forward (+ backward): launches, summed
   * launch durations from HIP events on the stream each launch ran on, and the
   * algorithmic FLOPs and bytes of those launches (2*M*N*K per contraction; operands
   * read once, results written once).  The backward's dA / dB products (LS_KC_LORA) run
   * on the library's side stream beside the compute stream, so their durations include
   * time shared with other kernels. */
  uint64_t k_launches[LS_KC_N];
  double k_ms[LS_KC_N];
  double k_flop[LS_KC_N];
  double k_bytes[LS_KC_N];
} ls_stats;

typedef struct ls_ctx ls_ctx;

/*
 * ls_create — validate cfg, plan device memory, refuse if over budget, allocate.
 *   cfg:            host pointer, read during the call only.
 *   compute_stream: hipStream_t to run kernels on (NULL: the library makes one).
 *   copy_stream:    hipStream_t for host->device layer copies (NULL: library makes
 *                   one).  Must differ from compute_stream.
 *   out:            receives the context.
 * The plan is checked against cfg->vram_budget (or the device's free memory when 0)
 * before any allocation; if it does not fit the call returns LS_ERR_BUDGET and
 * allocates nothing (the pages' pre-flight refusal of runs that will not fit:
 * the lachieslifestyle.com how-to, "Step 7: Train and keep the log").  The library
 * owns the pinned store, the device slots, checkpoints and workspaces, and one more
 * stream of its own (default priority) on which ls_backward runs the adapter-gradient
 * reductions beside the compute stream; ls_backward's work on the compute stream
 * ends with a wait for them.
 * Race detection (environment, read here; for tests, results must not change):
 *   LS_DEBUG_POISON=1        before every copy into a slot, the copy stream first fills
 *                            the slot with 0xFF bytes (NF4 code 15, NaN scales), after
 *                            the event that says the slot's last reader is done;
 *   LS_DEBUG_COPY_DELAY_US=n the copy stream also sleeps n microseconds (host function,
 *                            n <= 1e6) between that fill and the copy.
 * A missing wait on either side of the pool then shows as changed results.
 */
ls_status ls_create(const ls_config* cfg, void* compute_stream, void* copy_stream, ls_ctx** out);

/*
 * ls_plan_bytes — the device and pinned-host bytes ls_create would allocate for cfg.
 * Pure host computation, no HIP call.  Returns LS_ERR_INVALID for a bad cfg.  With
 * n_buffers = 0 it plans the depth ls_create would pick under cfg->vram_budget; with
 * no budget either (it cannot query the device), the deepest pool: one slot per layer,
 * at most 64.
 */
ls_status ls_plan_bytes(const ls_config* cfg, uint64_t* device_bytes, uint64_t* host_bytes,
                        uint64_t* blob_bytes);

/*
 * ls_stage_layer — encode one layer into the pinned store (NF4 packing with
 * blockwise absmax and optional double quantisation, or a bf16 copy) on the host
 * CPU.  Synchronous: the caller's buffers may be freed on return.  A resident
 * context also copies the blob to its device copy of the layer.  Staging invalidates
 * the last forward (ls_backward returns LS_ERR_STATE until the next ls_forward).
 * Errors: LS_ERR_INVALID (layer index, null pointer), LS_ERR_STATE (a forward or
 * backward is in flight: call ls_sync first).
 */
ls_status ls_stage_layer(ls_ctx* ctx, int32_t layer, const ls_layer_host* w);

/*
 * ls_set_lora — register the adapter of (layer, proj).  The adapters are the only
 * trained values and stay on the GPU while the frozen base streams (the
 * lachieslifestyle.com how-to, its opening paragraph; kept in full precision:
 * "Fine-Tuning an 8B Parameter Model on a 4 GB Laptop GPU", section "LoRA and QLoRA:
 * Train a Fraction of the Parameters").  A [r, in], B [out, r] and the gradient
 * buffers dA, dB (same shapes) are float32 device pointers owned by the caller and
 * borrowed until re-set or ls_destroy.  Projections outside lora_mask need no
 * registration.  dA/dB may be NULL if no gradient is wanted.  A registration
 * invalidates the last forward: ls_backward then returns LS_ERR_STATE until the next
 * ls_forward (the backward reuses per-layer products of the forward's adapters).
 * Errors: LS_ERR_INVALID (index out of range, null A or B).
 */
ls_status ls_set_lora(ls_ctx* ctx, int32_t layer, int32_t proj, const float* A, const float* B,
                      float* dA, float* dB);

/*
 * ls_forward — enqueue the streamed forward over all layers on the compute stream.
 *   X:      device bf16 [batch*seq, hidden], read during the call's GPU work.
 *   Y:      device bf16 [batch*seq, hidden], the last layer's output.
 *   lora_on: 0 runs every projection base-only.
 *   Y_ref:  NULL, or device bf16 [batch*seq, hidden]: also run, per layer and on the
 *           same streamed slot, the adapters-off reference pass from X (the DPO
 *           reference model: "Soup CLI fine-tunes Llama-3.1-8B on a 4 GB laptop GPU
 *           ...", third paragraph).
 * The layer inputs are kept as bf16 checkpoints for ls_backward; X is copied to the
 * first one before anything else reads it, so Y may alias X (Y_ref must not alias Y).
 * Asynchronous: returns after enqueueing.  Errors: LS_ERR_INVALID (sizes beyond
 * max_tokens / max_seq, seq not a multiple of 8, null pointers), LS_ERR_STATE (a layer
 * not staged).
 */
ls_status ls_forward(ls_ctx* ctx, const void* X, int32_t batch, int32_t seq, int32_t lora_on,
                     void* Y, void* Y_ref);

/*
 * ls_backward — enqueue the recompute backward: for l = L-1 .. 0 re-stream layer l,
 * recompute its forward from the checkpoint, and back-propagate (every layer is read
 * again for the backward recomputation: the lachieslifestyle.com how-to, section
 * "What Soup layer streaming changes"; only the adapters receive gradients:
 * "Fine-Tuning an 8B Parameter Model on a 4 GB Laptop GPU", section "LoRA and QLoRA:
 * Train a Fraction of the Parameters").
 *   dY: device bf16 [T, hidden] gradient of the last layer's output.
 *   dX: device bf16 [T, hidden] receives the gradient of the stack input.
 *   accumulate: 0 = write dA/dB, 1 = add into the registered dA/dB buffers.
 * dX may alias dY: dY is read only by the last layer's backward and dX written only at
 * the end of the first layer's.  Requires a preceding ls_forward with lora_on = 1 on
 * this context (same T) with no ls_stage_layer or ls_set_lora since, else LS_ERR_STATE.
 * Deterministic: no atomics, fixed reduction order.  Errors: LS_ERR_STATE (no valid
 * forward), LS_ERR_INVALID (null dY or dX with T > 0).
 */
ls_status ls_backward(ls_ctx* ctx, const void* dY, void* dX, int32_t accumulate);

/* ls_sync — wait for the copy stream, the compute stream and the library's side and
 * recompute streams (the copies run on a dedicated stream beside the compute: "Soup CLI fine-tunes
 * Llama-3.1-8B on a 4 GB laptop GPU ...", second paragraph).  Returns the first
 * deferred HIP error, or LS_ERR_HIP with a message if a read from the LS_STORE_FILE
 * store failed; either makes the context's error sticky. */
ls_status ls_sync(ls_ctx* ctx);

/*
 * Profiling levels.  Timing is HIP events recorded around kernel launches on the
 * stream each runs on; each event is a packet in the stream and widens the gap before
 * the next kernel, so a timed run should record as few as it needs.  The backward runs
 * each layer's recompute on a stream of its own beside the previous layer's backward,
 * where a kernel's time would include the time it shares the GPU.
 *   LS_PROFILE_OFF:  no events.
 *   LS_PROFILE_ALL:  every launch (per-class times in ls_stats) and the copy / per-layer
 *                    compute intervals (overlap figures); the backward then runs each
 *                    recompute after the previous layer's backward, so that no
 *                    recompute kernel shares the GPU with another layer's backward.
 *   LS_PROFILE_GEMM: only the forward pass's dequant-GEMM launches (class
 *                    LS_KC_GEMM_FWD; the recompute's launches of that kernel, which
 *                    share the GPU with the backward, are not timed), of every layer
 *                    or of every ls_config.profile_stride-th layer.
 */
enum { LS_PROFILE_OFF = 0, LS_PROFILE_ALL = 1, LS_PROFILE_GEMM = 2 };

/* ls_set_profile — change the profiling level for the calls that follow (no work may be
 * in flight: call ls_sync first).  Errors: LS_ERR_INVALID (unknown level), LS_ERR_STATE. */
ls_status ls_set_profile(ls_ctx* ctx, int32_t profile);

/* ls_get_stats — counters since ls_create (host pointer out): bytes and copies of the
 * layer stream, slot reuse, peak device bytes and, when profiling, per-class kernel
 * times.  These are the figures the pages report for a streamed run: throughput next
 * to peak device memory, with the GPU's utilisation ("Soup CLI fine-tunes
 * Llama-3.1-8B on a 4 GB laptop GPU ...", first paragraph).  Errors: LS_ERR_INVALID
 * (null pointer).  Works on a context in the sticky error state. */
ls_status ls_get_stats(const ls_ctx* ctx, ls_stats* out);

/* ls_last_error — message of the last failing call on ctx (or of the last failing
 * ls_create / ls_plan_bytes when ctx is NULL).  Valid until the next call on the same
 * context.  A refused run says why (the how-to's "Step 7: Train and keep the log":
 * refuse, and keep the reason, rather than run wrong). */
const char* ls_last_error(const ls_ctx* ctx);

/* ls_destroy — wait for outstanding work and free everything the library owns: the
 * pinned store (or the store file, which is removed), the device plan, the streams and
 * events the library created.  Caller-owned buffers (activations, adapters, the
 * streams passed to ls_create) are untouched.  The pool and store it releases are the
 * ones of the pages' design ("Soup CLI fine-tunes Llama-3.1-8B on a 4 GB laptop GPU
 * ...", second paragraph).  NULL is a no-op. */
void ls_destroy(ls_ctx* ctx);

/*
 * ls_nf4_codebook — the 16 float32 NF4 levels the library uses, written to out[16]
 * (host pointer).  Computed on the host from the NormalFloat construction of the
 * QLoRA paper that "Fine-Tuning an 8B Parameter Model on a 4 GB Laptop GPU",
 * section "Quantization: Shrink the Weights", names.  No HIP call.
 */
void ls_nf4_codebook(float out[16]);

/*
 * ls_pack_nf4 — the library's host NF4 encoder for one tensor of numel bf16 values
 * (host pointers; no HIP call).  packed[ceil(numel/2)] receives the nibbles (element
 * 2k in the high nibble of byte k), absmax[ceil(numel/64)] the float32 block absmax.
 * If double_quant, qabs[nblocks], scale2[ceil(nblocks/256)] and mean[1] also receive
 * the second level (qabs/scale2/mean may be NULL otherwise).  n_threads <= 0 picks
 * the machine's core count (capped at 16).
 */
ls_status ls_pack_nf4(const uint16_t* w, uint64_t numel, int32_t double_quant, int32_t n_threads,
                      uint8_t* packed, float* absmax, uint8_t* qabs, float* scale2, float* mean);

/*
 * ls_read_weight — dequantise projection proj of a staged layer into device bf16
 * out [out, in] through the same path the GEMMs use (copy of the blob to a device
 * slot, then the dequant kernel).  Synchronous.  For checking the encoding.
 */
ls_status ls_read_weight(ls_ctx* ctx, int32_t layer, int32_t proj, void* out);

/*
 * ls_base_gemm — the frozen base term of one projection group of a staged layer, run
 * through the fused dequant-GEMM kernels that ls_forward and ls_backward launch for
 * that group, with the adapter term off.  The 4-bit expansion the pages describe
 * ("Fine-Tuning an 8B Parameter Model on a 4 GB Laptop GPU", section "Quantization:
 * Shrink the Weights") happens inside those kernels; this call makes it observable:
 * with one 1.0 per row of X and zeros elsewhere, out holds dequantised weights
 * exactly (a float32 sum of one product w * 1.0 and zeros).
 *   group: 0 = q|k|v (outputs q, k, v side by side), 1 = o, 2 = gate|up (outputs gate
 *          then up; the paired gate|up kernel of the forward when both adapter terms
 *          fit it, as in ls_forward), 3 = down.
 *   transposed = 0: out[M, sum n_out] = X[M, n_in] deq(W)^T  (the forward orientation)
 *   transposed = 1: out[M, n_in] = X[M, sum n_out] deq(W)   (the backward's W^T)
 *   X: device bf16, rows of the widths above; out: device float32, row-major with
 *   that width; 1 <= M <= max_tokens.
 * The layer reaches a slot as in ls_forward (copied from the store unless the context is
 * resident or the slot holds it).  Synchronous.  Errors: LS_ERR_INVALID (index, size,
 * null pointer), LS_ERR_STATE (layer not staged, work in flight).
 */
ls_status ls_base_gemm(ls_ctx* ctx, int32_t layer, int32_t group, int32_t transposed, const void* X, int32_t M,
                       float* out);

/* ---------------------------------------------------------------------------
 * One projection outside any context.  The frozen weight is already on the device in
 * the store's encoding (e.g. from ls_pack_nf4, copied by the caller); the projection is
 * the LoRA formula over a 4-bit base ("Fine-Tuning an 8B Parameter Model on a 4 GB
 * Laptop GPU", section "LoRA and QLoRA: Train a Fraction of the Parameters"), computed
 * by the kernels the streamed stack runs for each projection: the rank-r down product,
 * then the fused dequant GEMM with the low-rank term as a K-extension.
 * ------------------------------------------------------------------------- */
typedef struct ls_weight {
  int32_t quant;          /* LS_QUANT_NF4 or LS_QUANT_BF16 */
  int32_t double_quant;   /* NF4: 1 = qabs / scale2 / mean, 0 = absmax */
  int32_t n_out, n_in;    /* the weight is [n_out, n_in]; n_out % 4 == 0, n_in % 16 == 0 */
  const void* w;          /* device: NF4 codes, ceil(n_out n_in / 2) bytes (element 2k in
                             the high nibble of byte k), or bf16 [n_out, n_in] */
  const float* absmax;    /* device float32 [ceil(n_out n_in / 64)]   (NF4, no DQ) */
  const uint8_t* qabs;    /* device uint8 [ceil(n_out n_in / 64)]     (NF4 + DQ) */
  const float* scale2;    /* device float32 [ceil(nblocks / 256)]     (NF4 + DQ) */
  const float* mean;      /* device float32 [1]                       (NF4 + DQ) */
} ls_weight;

/* ls_lora_linear_workspace_bytes — bytes of device workspace ls_lora_linear needs for
 * these sizes (0 for invalid sizes).  No HIP call. */
uint64_t ls_lora_linear_workspace_bytes(int32_t M, int32_t n_in, int32_t n_out, int32_t r);

/*
 * ls_lora_linear — enqueue Y = X deq(W)^T + (alpha / r) (X A^T) B^T on `stream`.
 *   w:     host pointer to the weight description (read during the call).
 *   X:     device bf16 [M, n_in], 16-byte aligned.  Y: device bf16 [M, n_out].
 *   A, B:  device float32 [r, n_in] and [n_out, r]; r = 0 means base term only (A, B
 *          may then be NULL).  0 <= r <= 64.
 *   workspace: device, 256-byte aligned, at least ls_lora_linear_workspace_bytes; the
 *          caller owns it and must not touch it until the enqueued work is done.
 *   stream: hipStream_t, NULL = the default stream.
 * Every buffer is the caller's.  The first call on a device also writes the NF4 level
 * table to that device (synchronously).  Asynchronous otherwise.  Errors:
 * LS_ERR_INVALID (sizes, null or misaligned pointers, small workspace; message from
 * ls_lora_linear_error), LS_ERR_HIP (a launch failed).
 */
ls_status ls_lora_linear(const ls_weight* w, const void* X, int32_t M, const float* A, const float* B, int32_t r,
                         float alpha, void* Y, void* workspace, uint64_t workspace_bytes, void* stream);

/*
 * ls_lora_linear_noalloc — ls_lora_linear for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation, with its scratch in a fixed 12 MiB array of the library on each
 * device instead of a workspace argument; it calls no allocating routine.  Sizes whose
 * ls_lora_linear_workspace_bytes exceeds 12582912 are refused with LS_ERR_INVALID.  The
 * first call on a device does a synchronous set-up (make it before any capture).  Every
 * call on one device shares that array and leaves its contents behind: calls that may
 * overlap on one device (other streams, other host threads) race and must be serialised
 * by the caller.  Errors as ls_lora_linear.
 */
ls_status ls_lora_linear_noalloc(const ls_weight* w, const void* X, int32_t M, const float* A, const float* B,
                                 int32_t r, float alpha, void* Y, void* stream);

/* ls_lora_linear_error — message of the calling thread's last failing ls_lora_linear*
 * call. */
const char* ls_lora_linear_error(void);

/* ---------------------------------------------------------------------------
 * Training-loop closure: optimizer step and adapter files.
 * ------------------------------------------------------------------------- */

/*
 * AdamW hyperparameters.  Only the adapters train ("Fine-Tuning an 8B Parameter Model
 * on a 4 GB Laptop GPU", section "LoRA and QLoRA: Train a Fraction of the
 * Parameters") and Adam keeps two float32 tensors per trained value (same page, the
 * "Optimizer states" item of why training is memory-hungry).  The update is AdamW
 * with learning-rate-scaled decoupled decay, for every element:
 *     p <- p (1 - lr weight_decay)
 *     m <- beta1 m + (1 - beta1) g ;  v <- beta2 v + (1 - beta2) g^2
 *     p <- p - (lr / (1 - beta1^step)) m / (sqrt(v) / sqrt(1 - beta2^step) + eps)
 */
typedef struct ls_adamw {
  float lr;            /* >= 0 */
  float beta1, beta2;  /* in [0, 1) */
  float eps;           /* > 0 */
  float weight_decay;  /* >= 0 */
  int32_t step;        /* 1-based step number t of this update (bias correction) */
} ls_adamw;

/*
 * ls_adamw_step — enqueue one AdamW update of every registered adapter tensor (A and
 * B of each (layer, proj) in lora_mask whose gradient buffer is registered) from its
 * registered gradient (dA, dB), in one launch on the compute stream.  A and B are
 * updated in place (the pointers given to ls_set_lora; the library writes them), the
 * moments live in the library's plan (ls_config.adamw = 1; zero after ls_create or
 * ls_adamw_reset).  Asynchronous.  Errors: LS_ERR_STATE (adamw not planned),
 * LS_ERR_INVALID (hyperparameters out of range, null hp).
 */
ls_status ls_adamw_step(ls_ctx* ctx, const ls_adamw* hp);

/* ls_adamw_reset — enqueue zeroing of every AdamW moment (a new optimizer run). */
ls_status ls_adamw_reset(ls_ctx* ctx);

/*
 * Adapter files.  A release of the tool the pages describe saved adapters under key
 * names that made them load without taking effect, silently (the lachieslifestyle.com
 * how-to, "Step 2", the warning against version 0.72.0; "Soup CLI fine-tunes
 * Llama-3.1-8B on a 4 GB laptop GPU ...", the paragraph on runs that were wrong
 * anyway).  These files therefore carry an integrity record and a load either
 * applies every adapter tensor or refuses.
 *
 * Format: safetensors (8-byte little-endian header length, JSON header, raw data).
 * Tensor names follow the PEFT convention for Llama-style stacks,
 *   base_model.model.model.layers.<l>.self_attn.<q|k|v|o>_proj.lora_<A|B>.weight
 *   base_model.model.model.layers.<l>.mlp.<gate|up|down>_proj.lora_<A|B>.weight
 * dtype F32, A [r, in], B [out, r].  __metadata__ holds format = pt, lsq.n_layers,
 * lsq.r, lsq.mask, lsq.alpha and, per tensor, lsq.crc32.<name> = CRC-32 (the zlib
 * polynomial) of its data bytes as 8 lowercase hex digits.
 */

/*
 * ls_save_adapters — write every registered adapter of lora_mask to path (host
 * string), after waiting for the compute stream; then read the file back and check
 * it as ls_check_adapter_file does.  Synchronous.  Errors: LS_ERR_STATE (an adapter
 * of the mask is not registered), LS_ERR_INVALID (the file cannot be written, or the
 * check of what was written fails).
 */
ls_status ls_save_adapters(ls_ctx* ctx, const char* path);

/*
 * ls_load_adapters — check path against the context's stack (as ls_check_adapter_file)
 * and, only if every check passes, copy every tensor into the registered A and B
 * device buffers.  Synchronous.  Errors: LS_ERR_INVALID (the file fails a check; the
 * message names the first problem; no adapter was changed), LS_ERR_STATE (an adapter
 * of the mask is not registered).
 */
ls_status ls_load_adapters(ls_ctx* ctx, const char* path);

/*
 * ls_check_adapter_file — host-only check of path against cfg: exactly the expected
 * tensor names (every layer, every projection of lora_mask, A and B; none missing,
 * none extra), dtype F32 and the expected shapes, in-range and non-overlapping data
 * offsets, lsq.n_layers / lsq.r / lsq.mask equal to cfg's, and every CRC-32 present
 * and matching.  No HIP call.  Returns LS_OK or LS_ERR_INVALID; msg (host buffer of
 * msg_len bytes, may be NULL) receives the first problem or "ok".
 */
ls_status ls_check_adapter_file(const ls_config* cfg, const char* path, char* msg, size_t msg_len);

/* ---------------------------------------------------------------------------
 * Output head and loss.  Streaming bounds the weights, not the logits: the tool the
 * pages describe keeps the whole logits tensor resident (8.71 GB at batch 8 on a
 * 152k-token vocabulary: "Soup CLI fine-tunes Llama-3.1-8B on a 4 GB laptop GPU ...",
 * third and fifth paragraphs).  Here the frozen head streams through the same device
 * slots as the layers, in vocabulary slices that fit one slot, and the loss needs only
 * per-token softmax statistics: no [tokens, vocab] tensor is ever held.
 * ------------------------------------------------------------------------- */

/*
 * ls_stage_head — copy the frozen head into the pinned store: w [vocab, hidden] bf16
 * (host pointer, row-major) and the final RMSNorm weight g_final [hidden] bf16.  The
 * head is kept in 16 bits whatever ls_config.quant says (QLoRA keeps the output layer
 * in 16 bits).  Synchronous; the caller's buffers may be freed on return.  Errors:
 * LS_ERR_STATE (ls_config.vocab = 0, or work in flight), LS_ERR_INVALID (null).
 */
ls_status ls_stage_head(ls_ctx* ctx, const uint16_t* w, const uint16_t* g_final);

/*
 * ls_head_loss — enqueue, after ls_forward and before ls_backward (same batch, seq):
 * final RMSNorm of Y, logits = yn W^T slice by slice, the loss, and dY = dLoss/dY for
 * ls_backward (second, reversed pass over the slices).
 *   Y:      device bf16 [T, hidden], the ls_forward output (adapters on).
 *   Y_ref:  device bf16 [T, hidden], the ls_forward reference output; LS_LOSS_DPO only.
 *   labels: device int32 [T], the target id of each token in [0, vocab), or
 *           LS_LABEL_IGNORE for a token without loss; the caller aligns targets.
 *   kind:   LS_LOSS_SFT — mean over labelled tokens of -log softmax(logits)[label];
 *           LS_LOSS_DPO — sequences in pairs (2i chosen, 2i+1 rejected), a sequence's
 *           log-prob is the sum over its labelled tokens, loss = mean over pairs of
 *           -log sigmoid(beta [(pi_c - ref_c) - (pi_r - ref_r)]) (the pages name DPO
 *           over the streamed base, reference = adapters off: same paragraph three).
 *   beta:   DPO temperature, > 0 (ignored for SFT).
 *   out:    device float [2 + 2 batch]: loss, number of labelled tokens, per-sequence
 *           log-prob sums of the policy, then (DPO) of the reference.
 *   dY:     device bf16 [T, hidden] receives dLoss/dY.
 * Asynchronous.  Deterministic (fixed reduction orders).  Errors: LS_ERR_STATE (no head
 * staged, no matching forward, DPO without a reference pass), LS_ERR_INVALID (null
 * pointers, bad kind, beta <= 0, odd batch for DPO).  Labels out of range are treated
 * as ignored.
 */
ls_status ls_head_loss(ls_ctx* ctx, const void* Y, const void* Y_ref, const int32_t* labels, int32_t kind,
                       float beta, float* out, void* dY);

#ifdef __cplusplus
}
#endif
#endif /* LS_H_ */
