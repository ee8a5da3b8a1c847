"""Adapter files: names, integrity record, reference writer and checker
(TEST INFRASTRUCTURE ONLY; see ``oracle/__init__``).

What the pages fix: a release of the tool saved adapters under key names that made
them load without applying the learned weights, silently (the lachieslifestyle.com
how-to, "Step 2", the warning against version 0.72.0; "Soup CLI fine-tunes
Llama-3.1-8B on a 4 GB laptop GPU ...", the paragraph on runs that completed and were
wrong anyway).  So a load must either apply every trained tensor or refuse.

Readings taken:

* container: the safetensors layout (8-byte little-endian header length, a JSON
  header with dtype, shape and [begin, end) byte offsets per tensor and a string map
  ``__metadata__``, then the raw little-endian data);
* names: the PEFT convention for Llama-style stacks,
  ``base_model.model.model.layers.{l}.self_attn.{q,k,v,o}_proj.lora_{A,B}.weight`` and
  ``...layers.{l}.mlp.{gate,up,down}_proj.lora_{A,B}.weight``; A is [r, in], B is
  [out, r], float32 ("F32");
* integrity record in ``__metadata__``: ``lsq.n_layers``, ``lsq.r``, ``lsq.mask``,
  ``lsq.alpha`` (decimal text) and, per tensor, ``lsq.crc32.<name>`` = the CRC-32
  (ISO-HDLC, the zlib one) of its data bytes as 8 lowercase hex digits;
* a file is valid for a stack when it holds exactly the expected names (every layer,
  every projection of the mask, A and B), each with the expected dtype and shape,
  each with a matching CRC-32, and with n_layers / r / mask equal to the stack's.
"""
from __future__ import annotations

import json
import struct
import zlib

import numpy as np

PROJ_MODULE = ("self_attn.q_proj", "self_attn.k_proj", "self_attn.v_proj", "self_attn.o_proj",
               "mlp.gate_proj", "mlp.up_proj", "mlp.down_proj")


def peft_key(layer: int, proj: int, which: str) -> str:
    assert which in ("A", "B")
    return f"base_model.model.model.layers.{layer}.{PROJ_MODULE[proj]}.lora_{which}.weight"


def expected(n_layers: int, mask: int, r: int, dims):
    """name -> shape for a stack; dims[p] = (n_out, n_in)."""
    out = {}
    for l in range(n_layers):
        for p in range(7):
            if (mask >> p) & 1:
                n_out, n_in = dims[p]
                out[peft_key(l, p, "A")] = (r, n_in)
                out[peft_key(l, p, "B")] = (n_out, r)
    return out


def crc32_hex(a: np.ndarray) -> str:
    return f"{zlib.crc32(np.ascontiguousarray(a).tobytes()) & 0xFFFFFFFF:08x}"


def write(path: str, tensors: dict, n_layers: int, r: int, alpha: float, mask: int, crc=True):
    """Reference writer through the safetensors package (a library routine)."""
    from safetensors.numpy import save_file
    meta = {"format": "pt", "lsq.n_layers": str(n_layers), "lsq.r": str(r), "lsq.mask": str(mask),
            "lsq.alpha": repr(float(alpha))}
    if crc:
        for k, a in tensors.items():
            meta["lsq.crc32." + k] = crc32_hex(np.asarray(a, np.float32))
    save_file({k: np.ascontiguousarray(a, np.float32) for k, a in tensors.items()}, path, metadata=meta)


def read_raw(path: str):
    """(header dict, data bytes) by the published layout, without the package."""
    with open(path, "rb") as f:
        blob = f.read()
    (n,) = struct.unpack_from("<Q", blob, 0)
    header = json.loads(blob[8:8 + n].decode("utf-8"))
    return header, blob[8 + n:]


def check(path: str, n_layers: int, mask: int, r: int, dims) -> list:
    """Problems of the file for the stack ([] = valid), each naming what is wrong."""
    try:
        header, data = read_raw(path)
    except Exception as e:  # noqa: BLE001 - any parse failure is a problem to report
        return [f"unreadable: {e}"]
    meta = header.pop("__metadata__", {}) or {}
    want = expected(n_layers, mask, r, dims)
    probs = []
    for k in sorted(set(want) - set(header)):
        probs.append(f"missing {k}")
    for k in sorted(set(header) - set(want)):
        probs.append(f"unexpected {k}")
    for key, val in (("lsq.n_layers", n_layers), ("lsq.r", r), ("lsq.mask", mask)):
        if meta.get(key) != str(val):
            probs.append(f"metadata {key} = {meta.get(key)!r}, stack has {val}")
    for k in sorted(set(want) & set(header)):
        e = header[k]
        if e.get("dtype") != "F32" or tuple(e.get("shape", ())) != want[k]:
            probs.append(f"bad dtype/shape for {k}")
            continue
        b, en = e["data_offsets"]
        if not (0 <= b <= en <= len(data)) or en - b != 4 * want[k][0] * want[k][1]:
            probs.append(f"bad offsets for {k}")
            continue
        crc = f"{zlib.crc32(data[b:en]) & 0xFFFFFFFF:08x}"
        if meta.get("lsq.crc32." + k) != crc:
            probs.append(f"crc mismatch for {k}")
    return probs


def load(path: str):
    """name -> float32 array, through the safetensors package."""
    from safetensors.numpy import load_file
    return load_file(path)
