"""ctypes binding of liblsq.so — the C ABI in include/ls.h, same names.

Argument marshalling only: every step of the path runs in the library's HIP kernels.
Device pointers are plain integers (e.g. ``tensor.data_ptr()`` of a torch CUDA
tensor); torch is used by callers for device memory and streams, never here for
compute.  The library is loaded on first use and a missing build raises.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblsq.so")

LS_OK, LS_ERR_INVALID, LS_ERR_STATE, LS_ERR_BUDGET, LS_ERR_OOM, LS_ERR_HIP = range(6)
LS_QUANT_NF4, LS_QUANT_BF16 = 0, 1
LS_STORE_HOST, LS_STORE_FILE = 0, 1
LS_PROFILE_OFF, LS_PROFILE_ALL, LS_PROFILE_GEMM = 0, 1, 2
PROJS = ("q", "k", "v", "o", "gate", "up", "down")
LS_KC_N = 7
KERNEL_CLASSES = ("gemm_fwd", "gemm_bwd", "attn", "lora", "glue", "optim", "head")
LS_LOSS_SFT, LS_LOSS_DPO = 0, 1
LS_LABEL_IGNORE = -100


class LsError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"liblsq status {status}: {msg}")
        self.status = status


class ls_config(C.Structure):
    _fields_ = [
        ("n_layers", C.c_int32), ("hidden", C.c_int32), ("n_heads", C.c_int32), ("n_kv_heads", C.c_int32),
        ("head_dim", C.c_int32), ("intermediate", C.c_int32), ("rms_eps", C.c_float), ("rope_theta", C.c_float),
        ("quant", C.c_int32), ("nf4_block", C.c_int32), ("double_quant", C.c_int32), ("lora_r", C.c_int32),
        ("lora_alpha", C.c_float), ("lora_mask", C.c_uint32), ("n_buffers", C.c_int32), ("max_tokens", C.c_int32),
        ("max_seq", C.c_int32), ("resident", C.c_int32), ("vram_budget", C.c_uint64), ("profile", C.c_int32),
        ("adamw", C.c_int32), ("vocab", C.c_int32), ("store", C.c_int32), ("store_path", C.c_char * 256),
        ("copy_split", C.c_int32), ("profile_stride", C.c_int32),
    ]


class ls_adamw(C.Structure):
    _fields_ = [("lr", C.c_float), ("beta1", C.c_float), ("beta2", C.c_float), ("eps", C.c_float),
                ("weight_decay", C.c_float), ("step", C.c_int32)]


class ls_weight(C.Structure):
    _fields_ = [("quant", C.c_int32), ("double_quant", C.c_int32), ("n_out", C.c_int32), ("n_in", C.c_int32),
                ("w", C.c_void_p), ("absmax", C.c_void_p), ("qabs", C.c_void_p), ("scale2", C.c_void_p),
                ("mean", C.c_void_p)]


class ls_layer_host(C.Structure):
    _fields_ = [("w", C.c_void_p * 7), ("g1", C.c_void_p), ("g2", C.c_void_p)]


class ls_stats(C.Structure):
    _fields_ = [
        ("blob_bytes", C.c_uint64), ("store_bytes", C.c_uint64), ("device_bytes", C.c_uint64),
        ("h2d_bytes", C.c_uint64), ("h2d_copies", C.c_uint64), ("slot_hits", C.c_uint64),
        ("store_reads", C.c_uint64), ("store_uncached", C.c_uint64), ("n_slots", C.c_uint64), ("poison_fills", C.c_uint64),
        ("last_copy_ms", C.c_double), ("last_compute_ms", C.c_double), ("last_overlap_ms", C.c_double),
        ("last_span_ms", C.c_double),
        ("k_launches", C.c_uint64 * LS_KC_N), ("k_ms", C.c_double * LS_KC_N),
        ("k_flop", C.c_double * LS_KC_N), ("k_bytes", C.c_double * LS_KC_N),
    ]

    def as_dict(self):
        d = {f: getattr(self, f) for f, _ in self._fields_ if not f.startswith("k_")}
        d["kernels"] = {KERNEL_CLASSES[i]: {"launches": self.k_launches[i], "ms": self.k_ms[i],
                                            "flop": self.k_flop[i], "bytes": self.k_bytes[i]}
                        for i in range(LS_KC_N)}
        return d


# exported symbol -> (restype, argtypes)
SIGNATURES = {
    "ls_create": (C.c_int, [C.POINTER(ls_config), C.c_void_p, C.c_void_p, C.POINTER(C.c_void_p)]),
    "ls_plan_bytes": (C.c_int, [C.POINTER(ls_config), C.POINTER(C.c_uint64), C.POINTER(C.c_uint64),
                                C.POINTER(C.c_uint64)]),
    "ls_stage_layer": (C.c_int, [C.c_void_p, C.c_int32, C.POINTER(ls_layer_host)]),
    "ls_set_lora": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p]),
    "ls_forward": (C.c_int, [C.c_void_p, C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p]),
    "ls_backward": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32]),
    "ls_sync": (C.c_int, [C.c_void_p]),
    "ls_get_stats": (C.c_int, [C.c_void_p, C.POINTER(ls_stats)]),
    "ls_last_error": (C.c_char_p, [C.c_void_p]),
    "ls_destroy": (None, [C.c_void_p]),
    "ls_nf4_codebook": (None, [C.POINTER(C.c_float)]),
    "ls_pack_nf4": (C.c_int, [C.c_void_p, C.c_uint64, C.c_int32, C.c_int32, C.c_void_p, C.c_void_p, C.c_void_p,
                              C.c_void_p, C.c_void_p]),
    "ls_read_weight": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_void_p]),
    "ls_base_gemm": (C.c_int, [C.c_void_p, C.c_int32, C.c_int32, C.c_int32, C.c_void_p, C.c_int32, C.c_void_p]),
    "ls_lora_linear_workspace_bytes": (C.c_uint64, [C.c_int32, C.c_int32, C.c_int32, C.c_int32]),
    "ls_lora_linear": (C.c_int, [C.POINTER(ls_weight), C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p, C.c_int32,
                                 C.c_float, C.c_void_p, C.c_void_p, C.c_uint64, C.c_void_p]),
    "ls_lora_linear_noalloc": (C.c_int, [C.POINTER(ls_weight), C.c_void_p, C.c_int32, C.c_void_p, C.c_void_p,
                                         C.c_int32, C.c_float, C.c_void_p, C.c_void_p]),
    "ls_lora_linear_error": (C.c_char_p, []),
    "ls_adamw_step": (C.c_int, [C.c_void_p, C.POINTER(ls_adamw)]),
    "ls_adamw_reset": (C.c_int, [C.c_void_p]),
    "ls_save_adapters": (C.c_int, [C.c_void_p, C.c_char_p]),
    "ls_load_adapters": (C.c_int, [C.c_void_p, C.c_char_p]),
    "ls_check_adapter_file": (C.c_int, [C.POINTER(ls_config), C.c_char_p, C.c_char_p, C.c_size_t]),
    "ls_stage_head": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p]),
    "ls_set_profile": (C.c_int, [C.c_void_p, C.c_int32]),
    "ls_head_loss": (C.c_int, [C.c_void_p, C.c_void_p, C.c_void_p, C.c_void_p, C.c_int32, C.c_float, C.c_void_p,
                               C.c_void_p]),
}

_lib = None


def lib():
    """Load liblsq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() or "
                               "python layer_streamed_qlora_amd/build.py")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status, ctx=None):
    if status != LS_OK:
        msg = lib().ls_last_error(ctx)
        raise LsError(status, msg.decode() if msg else "")


def make_config(w, n_buffers=2, max_tokens=None, max_seq=None, resident=0, vram_budget=0, profile=0,
                lora_mask=0x7F, n_layers=None, adamw=0, vocab=0, store_path=None, copy_split=0,
                profile_stride=0) -> ls_config:
    """ls_config for a workload description (``synth.Workload``)."""
    return ls_config(
        n_layers=w.n_layers if n_layers is None else n_layers, hidden=w.hidden, n_heads=w.n_heads,
        n_kv_heads=w.n_kv_heads, head_dim=w.head_dim, intermediate=w.intermediate, rms_eps=w.rms_eps,
        rope_theta=w.rope_theta, quant=LS_QUANT_NF4 if w.quant == "nf4" else LS_QUANT_BF16, nf4_block=64,
        double_quant=int(w.double_quant), lora_r=w.lora_r, lora_alpha=w.lora_alpha, lora_mask=lora_mask,
        n_buffers=n_buffers, max_tokens=w.tokens if max_tokens is None else max_tokens,
        max_seq=w.seq if max_seq is None else max_seq, resident=resident, vram_budget=vram_budget, profile=profile,
        adamw=adamw, vocab=vocab, store=LS_STORE_FILE if store_path else LS_STORE_HOST,
        store_path=os.fsencode(store_path) if store_path else b"", copy_split=copy_split,
        profile_stride=profile_stride)


# ------------------------------------------------------------------ host calls
def ls_nf4_codebook() -> np.ndarray:
    out = (C.c_float * 16)()
    lib().ls_nf4_codebook(out)
    return np.frombuffer(out, dtype=np.float32).copy()


def ls_pack_nf4(w_bits: np.ndarray, double_quant: bool, n_threads: int = 0):
    """Host NF4 encoder of the library on bf16 bit patterns (uint16)."""
    w = np.ascontiguousarray(w_bits, dtype=np.uint16).reshape(-1)
    n = w.size
    nb = -(-n // 64)
    packed = np.zeros(-(-n // 2), np.uint8)
    absmax = np.zeros(nb, np.float32)
    qabs = np.zeros(nb, np.uint8) if double_quant else None
    scale2 = np.zeros(-(-nb // 256), np.float32) if double_quant else None
    mean = np.zeros(1, np.float32) if double_quant else None
    ptr = lambda a: a.ctypes.data if a is not None else None
    _check(lib().ls_pack_nf4(ptr(w), n, int(double_quant), n_threads, ptr(packed), ptr(absmax), ptr(qabs),
                             ptr(scale2), ptr(mean)))
    return packed, absmax, qabs, scale2, (mean[0] if double_quant else None)


def ls_lora_linear_workspace_bytes(M, n_in, n_out, r) -> int:
    return int(lib().ls_lora_linear_workspace_bytes(M, n_in, n_out, r))


def _linear_check(st):
    if st != LS_OK:
        msg = lib().ls_lora_linear_error()
        raise LsError(st, msg.decode() if msg else "")


def ls_lora_linear(w: ls_weight, X_ptr, M, A_ptr, B_ptr, r, alpha, Y_ptr, ws_ptr, ws_bytes, stream=0):
    """Y = X deq(W)^T + (alpha / r) (X A^T) B^T; device pointers as integers."""
    _linear_check(lib().ls_lora_linear(C.byref(w), X_ptr, M, A_ptr or None, B_ptr or None, r, alpha, Y_ptr,
                                       ws_ptr or None, ws_bytes, stream or None))


def ls_lora_linear_noalloc(w: ls_weight, X_ptr, M, A_ptr, B_ptr, r, alpha, Y_ptr, stream=0):
    """ls_lora_linear with the library's fixed device scratch (no workspace)."""
    _linear_check(lib().ls_lora_linear_noalloc(C.byref(w), X_ptr, M, A_ptr or None, B_ptr or None, r, alpha, Y_ptr,
                                               stream or None))


def ls_check_adapter_file(cfg: ls_config, path: str):
    """(status, message) of the library's host-only check of an adapter file."""
    buf = C.create_string_buffer(1024)
    st = lib().ls_check_adapter_file(C.byref(cfg), os.fsencode(path), buf, len(buf))
    return st, buf.value.decode()


def ls_plan_bytes(cfg: ls_config):
    d, h, b = C.c_uint64(), C.c_uint64(), C.c_uint64()
    _check(lib().ls_plan_bytes(C.byref(cfg), C.byref(d), C.byref(h), C.byref(b)))
    return d.value, h.value, b.value


# -------------------------------------------------------------------- context
class Context:
    """One ls_ctx.  Methods are the C entry points with Python arguments."""

    def __init__(self, cfg: ls_config, compute_stream: int = 0, copy_stream: int = 0):
        self.cfg = cfg
        h = C.c_void_p()
        _check(lib().ls_create(C.byref(cfg), compute_stream or None, copy_stream or None, C.byref(h)))
        self.h = h

    def close(self):
        if self.h:
            lib().ls_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _chk(self, st):
        _check(st, self.h)

    def stage_layer(self, layer: int, weights_bits: dict):
        """weights_bits: proj -> uint16 [out, in] (bf16 bits), 'g1'/'g2' -> uint16 [h]."""
        keep = {k: np.ascontiguousarray(v, dtype=np.uint16) for k, v in weights_bits.items()}
        lh = ls_layer_host()
        for i, p in enumerate(PROJS):
            lh.w[i] = keep[p].ctypes.data
        lh.g1 = keep["g1"].ctypes.data
        lh.g2 = keep["g2"].ctypes.data
        self._chk(lib().ls_stage_layer(self.h, layer, C.byref(lh)))

    def set_lora(self, layer, proj, A_ptr, B_ptr, dA_ptr=0, dB_ptr=0):
        self._chk(lib().ls_set_lora(self.h, layer, proj, A_ptr, B_ptr, dA_ptr or None, dB_ptr or None))

    def forward(self, X_ptr, batch, seq, lora_on, Y_ptr, Yref_ptr=0):
        self._chk(lib().ls_forward(self.h, X_ptr or None, batch, seq, int(lora_on), Y_ptr or None, Yref_ptr or None))

    def backward(self, dY_ptr, dX_ptr, accumulate=0):
        self._chk(lib().ls_backward(self.h, dY_ptr or None, dX_ptr or None, int(accumulate)))

    def sync(self):
        self._chk(lib().ls_sync(self.h))

    def stats(self) -> ls_stats:
        s = ls_stats()
        self._chk(lib().ls_get_stats(self.h, C.byref(s)))
        return s

    def read_weight(self, layer, proj, out_ptr):
        self._chk(lib().ls_read_weight(self.h, layer, proj, out_ptr))

    def base_gemm(self, layer, group, transposed, x_ptr, M, out_ptr):
        self._chk(lib().ls_base_gemm(self.h, layer, group, transposed, x_ptr, M, out_ptr))

    def adamw_step(self, step, lr, beta1=0.9, beta2=0.999, eps=1e-8, weight_decay=0.01):
        hp = ls_adamw(lr=lr, beta1=beta1, beta2=beta2, eps=eps, weight_decay=weight_decay, step=step)
        self._chk(lib().ls_adamw_step(self.h, C.byref(hp)))

    def adamw_reset(self):
        self._chk(lib().ls_adamw_reset(self.h))

    def save_adapters(self, path):
        self._chk(lib().ls_save_adapters(self.h, os.fsencode(path)))

    def load_adapters(self, path):
        self._chk(lib().ls_load_adapters(self.h, os.fsencode(path)))

    def set_profile(self, level):
        self._chk(lib().ls_set_profile(self.h, int(level)))

    def stage_head(self, w_bits: np.ndarray, g_bits: np.ndarray):
        """w_bits: uint16 [vocab, hidden] (bf16 bits), g_bits: uint16 [hidden]."""
        w = np.ascontiguousarray(w_bits, dtype=np.uint16)
        g = np.ascontiguousarray(g_bits, dtype=np.uint16)
        self._chk(lib().ls_stage_head(self.h, w.ctypes.data, g.ctypes.data))

    def head_loss(self, Y_ptr, Yref_ptr, labels_ptr, kind, beta, out_ptr, dY_ptr):
        self._chk(lib().ls_head_loss(self.h, Y_ptr or None, Yref_ptr or None, labels_ptr or None, int(kind),
                                     float(beta), out_ptr or None, dY_ptr or None))
