"""CPU checks of the library's adapter-file check (ls_check_adapter_file, host only)
against the oracle's checker on files the oracle writes, clean and with planted
corruptions, and of the AdamW moments in the device plan."""
import json
import struct

import numpy as np
import pytest

from layer_streamed_qlora_amd import binding as B
from layer_streamed_qlora_amd import synth
from oracle import adapters

TOY = synth.WORKLOADS["toy"]
PROJS = synth.PROJS


def dims(w=TOY):
    return [w.proj_shape(p) for p in PROJS]


def toy_tensors(w=TOY, mask=0x7F, seed=1):
    rng = np.random.default_rng(seed)
    return {k: rng.standard_normal(s).astype(np.float32) for k, s in adapters.expected(w.n_layers, mask, w.lora_r, dims(w)).items()}


def cfg(mask=0x7F, n_layers=None, r=None, adamw=0):
    c = B.make_config(TOY, lora_mask=mask, n_layers=n_layers, adamw=adamw)
    if r is not None:
        c.lora_r = r
    return c


def rewrite(path, edit_header=None, edit_data=None, raw=None):
    header, data = adapters.read_raw(path)
    if edit_header:
        edit_header(header)
    data = bytearray(data)
    if edit_data:
        edit_data(header, data)
    hb = json.dumps(header).encode()
    hb += b" " * (-len(hb) % 8)
    blob = struct.pack("<Q", len(hb)) + hb + bytes(data)
    if raw:
        blob = raw(blob)
    with open(path, "wb") as f:
        f.write(blob)


@pytest.fixture
def good(tmp_path):
    f = str(tmp_path / "good.safetensors")
    adapters.write(f, toy_tensors(), TOY.n_layers, TOY.lora_r, TOY.lora_alpha, 0x7F)
    return f


def verdicts(path, c=None, n_layers=None, mask=0x7F, r=None):
    c = c or cfg(mask, n_layers, r)
    st, msg = B.ls_check_adapter_file(c, path)
    probs = adapters.check(path, c.n_layers, c.lora_mask, c.lora_r, dims())
    return st, msg, probs


def test_oracle_written_file_passes(good):
    st, msg, probs = verdicts(good)
    assert st == B.LS_OK and msg == "ok" and probs == []


K0 = adapters.peft_key(1, 4, "A")
CASES = {
    # the no-op failure mode of the pages: names that a loader keyed on the expected ones never finds
    "renamed": (dict(edit_header=lambda h: h.update({k.replace("base_model.model.", ""): h.pop(k)
                                                      for k in [k for k in h if k != "__metadata__"]})), "tensor"),
    "peft_default_adapter_name": (dict(edit_header=lambda h: h.update({k.replace(".weight", ".default.weight"): h.pop(k)
                                                                        for k in [k for k in h if k != "__metadata__"]})), "tensor"),
    "flipped_bit": (dict(edit_data=lambda h, d: d.__setitem__(h[K0]["data_offsets"][0] + 9,
                                                              d[h[K0]["data_offsets"][0] + 9] ^ 0x10)), K0),
    "dropped": (dict(edit_header=lambda h: h.pop(K0)), K0),
    "wrong_shape": (dict(edit_header=lambda h: h[K0].update(shape=[TOY.hidden, TOY.lora_r])), K0),
    "wrong_dtype": (dict(edit_header=lambda h: h[K0].update(dtype="F16")), K0),
    "rank_metadata": (dict(edit_header=lambda h: h["__metadata__"].update({"lsq.r": "4"})), "lsq.r"),
    "no_crc": (dict(edit_header=lambda h: h["__metadata__"].pop("lsq.crc32." + K0)), K0),
    "no_metadata": (dict(edit_header=lambda h: h.pop("__metadata__")), "metadata"),
    "truncated": (dict(raw=lambda b: b[:-100]), "offsets"),
    "header_too_long": (dict(raw=lambda b: struct.pack("<Q", 1 << 40) + b[8:]), "header length"),
    "not_json": (dict(raw=lambda b: b[:8] + b"x" + b[9:]), "JSON"),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_planted_corruption_is_refused_by_both(good, case):
    kw, needle = CASES[case]
    rewrite(good, **kw)
    st, msg, probs = verdicts(good)
    assert st == B.LS_ERR_INVALID, msg
    assert probs, "the oracle checker must refuse it too"
    assert needle in msg, msg


def test_stack_mismatch_is_refused(good):
    for kw in (dict(n_layers=3), dict(mask=0x3F), dict(r=16)):
        st, msg, probs = verdicts(good, **kw)
        assert st == B.LS_ERR_INVALID and probs, (kw, msg)


def test_partial_mask_file(tmp_path):
    mask = 0b1010101
    f = str(tmp_path / "m.safetensors")
    adapters.write(f, toy_tensors(mask=mask), TOY.n_layers, TOY.lora_r, TOY.lora_alpha, mask)
    st, msg, probs = verdicts(f, mask=mask)
    assert st == B.LS_OK and probs == [], msg


def test_escaped_names_parse(good):
    """A JSON header that spells characters with \\u escapes is the same header."""
    header, data = adapters.read_raw(good)
    hb = json.dumps(header, ensure_ascii=True).replace('"F32"', '"\\u0046\\u00332"').encode()
    hb += b" " * (-len(hb) % 8)
    with open(good, "wb") as fh:
        fh.write(struct.pack("<Q", len(hb)) + hb + data)
    st, msg, _ = verdicts(good)
    assert st == B.LS_OK, msg


def test_crc32_of_library_matches_check_value(tmp_path):
    """The library's CRC-32 agrees with zlib's on a file the oracle writes: every record
    the oracle computed with zlib is accepted, and the catalogued check value holds in
    the oracle (so both implement the same CRC)."""
    assert adapters.crc32_hex(np.frombuffer(b"123456789", np.uint8)) == "cbf43926"
    f = str(tmp_path / "c.safetensors")
    t = {k: np.frombuffer(np.random.default_rng(5).bytes(4 * int(np.prod(s))), np.float32).reshape(s)
         for k, s in adapters.expected(TOY.n_layers, 0x7F, TOY.lora_r, dims()).items()}
    adapters.write(f, t, TOY.n_layers, TOY.lora_r, TOY.lora_alpha, 0x7F)
    assert B.ls_check_adapter_file(cfg(), f)[0] == B.LS_OK


def test_plan_holds_adamw_moments():
    d0, _, _ = B.ls_plan_bytes(cfg(adamw=0))
    d1, _, _ = B.ls_plan_bytes(cfg(adamw=1))
    elems = sum(TOY.lora_r * (n_out + n_in) for n_out, n_in in dims()) * TOY.n_layers
    assert d1 - d0 >= 8 * elems
    assert d1 - d0 <= 8 * elems + 64 * (elems // 8192 + 14 * TOY.n_layers) + 4096
