// Adapter files (host code): the safetensors container with PEFT tensor names and a
// CRC-32 record per tensor, written and checked so that a load either applies every
// adapter tensor or refuses.  The pages report a release of the tool whose adapters
// were saved under key names that made them load as a no-op, silently (the
// lachieslifestyle.com how-to, "Step 2", the warning against version 0.72.0;
// "Soup CLI fine-tunes Llama-3.1-8B on a 4 GB laptop GPU ...", the paragraph on runs
// that completed and were wrong anyway).
//
// Container: an 8-byte little-endian header length N, N bytes of JSON (padded with
// spaces to a multiple of 8), then the tensor data; each tensor entry gives dtype,
// shape and [begin, end) byte offsets into the data section; "__metadata__" is a map
// of strings.  Names: base_model.model.model.layers.<l>.self_attn.<q|k|v|o>_proj and
// ...mlp.<gate|up|down>_proj, then .lora_A.weight ([r, in]) or .lora_B.weight
// ([out, r]), float32.  Metadata: format, lsq.n_layers, lsq.r, lsq.mask, lsq.alpha,
// lsq.crc32.<name> (8 lowercase hex digits).
#include <algorithm>
#include <cerrno>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <string>
#include <vector>

#include "lsq_internal.hpp"

namespace lsq {
namespace {

const char* const kModule[LS_N_PROJ] = {"self_attn.q_proj", "self_attn.k_proj", "self_attn.v_proj",
                                        "self_attn.o_proj", "mlp.gate_proj",    "mlp.up_proj",
                                        "mlp.down_proj"};

// ---- CRC-32, reflected form of the polynomial 0x04C11DB7 (0xEDB88320 bit-reversed),
// initial value and final xor 0xFFFFFFFF: the CRC of zlib, PNG and Ethernet.
struct CrcTable {
  uint32_t t[256];
  CrcTable() {
    for (uint32_t i = 0; i < 256; ++i) {
      uint32_t r = i;
      for (int k = 0; k < 8; ++k) r = (r & 1u) ? (r >> 1) ^ 0xEDB88320u : r >> 1;
      t[i] = r;
    }
  }
};

// ---- JSON: the subset a safetensors header uses (objects, arrays, strings,
// non-negative integers), plus literals and signed/fractional numbers parsed and kept
// as text so that any well-formed header parses.
struct JVal {
  enum Kind { OBJ, ARR, STR, NUM, LIT } kind = LIT;
  std::string s;                                  // STR: decoded text, NUM/LIT: source text
  std::vector<std::pair<std::string, JVal>> obj;  // in file order
  std::vector<JVal> arr;
  const JVal* get(const std::string& k) const {
    for (const auto& kv : obj)
      if (kv.first == k) return &kv.second;
    return nullptr;
  }
};

struct JParser {
  const char* p;
  const char* e;
  std::string err;
  int depth = 0;
  void ws() {
    while (p < e && (*p == ' ' || *p == '\t' || *p == '\n' || *p == '\r')) ++p;
  }
  bool fail(const char* m) {
    if (err.empty()) err = m;
    return false;
  }
  static void put_utf8(std::string& o, uint32_t cp) {
    if (cp < 0x80) {
      o += (char)cp;
    } else if (cp < 0x800) {
      o += (char)(0xC0 | (cp >> 6));
      o += (char)(0x80 | (cp & 0x3F));
    } else if (cp < 0x10000) {
      o += (char)(0xE0 | (cp >> 12));
      o += (char)(0x80 | ((cp >> 6) & 0x3F));
      o += (char)(0x80 | (cp & 0x3F));
    } else {
      o += (char)(0xF0 | (cp >> 18));
      o += (char)(0x80 | ((cp >> 12) & 0x3F));
      o += (char)(0x80 | ((cp >> 6) & 0x3F));
      o += (char)(0x80 | (cp & 0x3F));
    }
  }
  bool hex4(uint32_t* v) {
    if (e - p < 4) return fail("short \\u escape");
    *v = 0;
    for (int i = 0; i < 4; ++i) {
      const char c = *p++;
      *v <<= 4;
      if (c >= '0' && c <= '9') *v |= (uint32_t)(c - '0');
      else if (c >= 'a' && c <= 'f') *v |= (uint32_t)(c - 'a' + 10);
      else if (c >= 'A' && c <= 'F') *v |= (uint32_t)(c - 'A' + 10);
      else return fail("bad \\u escape");
    }
    return true;
  }
  bool str(std::string& out) {
    if (p >= e || *p != '"') return fail("expected a string");
    ++p;
    out.clear();
    while (p < e && *p != '"') {
      const unsigned char c = (unsigned char)*p;
      if (c < 0x20) return fail("control character in a string");
      if (c != '\\') {
        out += (char)c;
        ++p;
        continue;
      }
      if (++p >= e) return fail("unterminated escape");
      const char x = *p++;
      switch (x) {
        case '"': out += '"'; break;
        case '\\': out += '\\'; break;
        case '/': out += '/'; break;
        case 'b': out += '\b'; break;
        case 'f': out += '\f'; break;
        case 'n': out += '\n'; break;
        case 'r': out += '\r'; break;
        case 't': out += '\t'; break;
        case 'u': {
          uint32_t cp;
          if (!hex4(&cp)) return false;
          if (cp >= 0xD800 && cp < 0xDC00) {   // surrogate pair
            uint32_t lo;
            if (e - p < 6 || p[0] != '\\' || p[1] != 'u') return fail("lone surrogate");
            p += 2;
            if (!hex4(&lo) || lo < 0xDC00 || lo >= 0xE000) return fail("bad surrogate pair");
            cp = 0x10000 + ((cp - 0xD800) << 10) + (lo - 0xDC00);
          }
          put_utf8(out, cp);
          break;
        }
        default: return fail("bad escape");
      }
    }
    if (p >= e) return fail("unterminated string");
    ++p;
    return true;
  }
  bool val(JVal& v) {
    if (++depth > 16) return fail("nesting too deep");
    ws();
    if (p >= e) return fail("unexpected end");
    bool ok;
    if (*p == '{') {
      v.kind = JVal::OBJ;
      ++p;
      ws();
      if (p < e && *p == '}') {
        ++p;
        ok = true;
      } else {
        ok = false;
        while (true) {
          ws();
          std::string k;
          if (!str(k)) break;
          ws();
          if (p >= e || *p != ':') { fail("expected ':'"); break; }
          ++p;
          v.obj.emplace_back(k, JVal());
          if (!val(v.obj.back().second)) break;
          ws();
          if (p < e && *p == ',') { ++p; continue; }
          if (p < e && *p == '}') { ++p; ok = true; break; }
          fail("expected ',' or '}'");
          break;
        }
      }
    } else if (*p == '[') {
      v.kind = JVal::ARR;
      ++p;
      ws();
      if (p < e && *p == ']') {
        ++p;
        ok = true;
      } else {
        ok = false;
        while (true) {
          v.arr.emplace_back();
          if (!val(v.arr.back())) break;
          ws();
          if (p < e && *p == ',') { ++p; continue; }
          if (p < e && *p == ']') { ++p; ok = true; break; }
          fail("expected ',' or ']'");
          break;
        }
      }
    } else if (*p == '"') {
      v.kind = JVal::STR;
      ok = str(v.s);
    } else if (*p == '-' || (*p >= '0' && *p <= '9')) {
      v.kind = JVal::NUM;
      const char* b = p;
      while (p < e && (strchr("+-0123456789.eE", *p) != nullptr)) ++p;
      v.s.assign(b, p);
      ok = true;
    } else {
      v.kind = JVal::LIT;
      static const char* const lits[3] = {"true", "false", "null"};
      ok = false;
      for (const char* l : lits) {
        const size_t n = strlen(l);
        if ((size_t)(e - p) >= n && strncmp(p, l, n) == 0) {
          v.s = l;
          p += n;
          ok = true;
          break;
        }
      }
      if (!ok) fail("unexpected character");
    }
    --depth;
    return ok;
  }
};

// non-negative decimal integer that fits in 63 bits
bool as_u63(const JVal& v, uint64_t* out) {
  if (v.kind != JVal::NUM || v.s.empty() || v.s.size() > 18) return false;
  uint64_t x = 0;
  for (char c : v.s) {
    if (c < '0' || c > '9') return false;
    x = x * 10 + (uint64_t)(c - '0');
  }
  *out = x;
  return true;
}

std::string json_escape(const std::string& s) {
  std::string o;
  for (char c : s) {
    if (c == '"' || c == '\\') { o += '\\'; o += c; }
    else if ((unsigned char)c < 0x20) { char b[8]; snprintf(b, sizeof b, "\\u%04x", (unsigned)c); o += b; }
    else o += c;
  }
  return o;
}

std::string hex8(uint32_t v) {
  char b[16];
  snprintf(b, sizeof b, "%08x", v);
  return b;
}

bool read_file(const std::string& path, std::vector<uint8_t>* out, std::string* err) {
  std::unique_ptr<FILE, int (*)(FILE*)> f(fopen(path.c_str(), "rb"), fclose);
  if (!f) { *err = "cannot open " + path + ": " + strerror(errno); return false; }
  if (fseek(f.get(), 0, SEEK_END) != 0) { *err = "cannot seek " + path; return false; }
  const long n = ftell(f.get());
  if (n < 0) { *err = "cannot size " + path; return false; }
  rewind(f.get());
  out->resize((size_t)n);
  if (n > 0 && fread(out->data(), 1, (size_t)n, f.get()) != (size_t)n) { *err = "cannot read " + path; return false; }
  return true;
}

}  // namespace

uint32_t crc32_bytes(const void* data, size_t n) {
  static const CrcTable T;
  const uint8_t* b = static_cast<const uint8_t*>(data);
  uint32_t c = 0xFFFFFFFFu;
  for (size_t i = 0; i < n; ++i) c = T.t[(c ^ b[i]) & 0xFFu] ^ (c >> 8);
  return c ^ 0xFFFFFFFFu;
}

std::vector<AdapterEntry> adapter_entries(const ls_config& c) {
  std::vector<AdapterEntry> v;
  for (int l = 0; l < c.n_layers; ++l)
    for (int p = 0; p < LS_N_PROJ; ++p) {
      if (!((c.lora_mask >> p) & 1u)) continue;
      int32_t n_out, n_in;
      proj_dims(c, p, &n_out, &n_in);
      for (int w = 0; w < 2; ++w) {
        AdapterEntry e;
        e.name = "base_model.model.model.layers." + std::to_string(l) + "." + kModule[p] +
                 (w == 0 ? ".lora_A.weight" : ".lora_B.weight");
        e.layer = l;
        e.proj = p;
        e.which = w;
        e.rows = w == 0 ? c.lora_r : n_out;
        e.cols = w == 0 ? n_in : c.lora_r;
        v.push_back(e);
      }
    }
  return v;
}

std::string adapter_write(const ls_config& c, const std::vector<AdapterEntry>& e, const std::vector<const float*>& data,
                          const std::string& path) {
  if (e.size() != data.size()) return "internal: entry and data counts differ";
  char alpha[64];
  snprintf(alpha, sizeof alpha, "%.9g", (double)c.lora_alpha);
  std::string h = "{\"__metadata__\":{\"format\":\"pt\",\"lsq.n_layers\":\"" + std::to_string(c.n_layers) +
                  "\",\"lsq.r\":\"" + std::to_string(c.lora_r) + "\",\"lsq.mask\":\"" +
                  std::to_string(c.lora_mask) + "\",\"lsq.alpha\":\"" + alpha + "\"";
  for (size_t i = 0; i < e.size(); ++i)
    h += ",\"lsq.crc32." + json_escape(e[i].name) + "\":\"" +
         hex8(crc32_bytes(data[i], (size_t)(4 * e[i].rows * e[i].cols))) + "\"";
  h += "}";
  uint64_t off = 0;
  for (size_t i = 0; i < e.size(); ++i) {
    const uint64_t n = (uint64_t)4 * e[i].rows * e[i].cols;
    h += ",\"" + json_escape(e[i].name) + "\":{\"dtype\":\"F32\",\"shape\":[" + std::to_string(e[i].rows) + "," +
         std::to_string(e[i].cols) + "],\"data_offsets\":[" + std::to_string(off) + "," + std::to_string(off + n) +
         "]}";
    off += n;
  }
  h += "}";
  while (h.size() % 8) h += ' ';
  std::unique_ptr<FILE, int (*)(FILE*)> f(fopen(path.c_str(), "wb"), fclose);
  if (!f) return "cannot create " + path + ": " + strerror(errno);
  uint8_t len[8];
  for (int i = 0; i < 8; ++i) len[i] = (uint8_t)((uint64_t)h.size() >> (8 * i));
  bool ok = fwrite(len, 1, 8, f.get()) == 8 && fwrite(h.data(), 1, h.size(), f.get()) == h.size();
  for (size_t i = 0; ok && i < e.size(); ++i) {
    const size_t n = (size_t)(e[i].rows * e[i].cols);
    ok = fwrite(data[i], sizeof(float), n, f.get()) == n;
  }
  if (!ok) return "write failed: " + path;
  if (fflush(f.get()) != 0) return "write failed: " + path;
  return "";
}

std::string adapter_check(const ls_config& c, const std::string& path, std::vector<AdapterEntry>* entries,
                          std::vector<uint8_t>* file_bytes) {
  std::vector<uint8_t> local;
  std::vector<uint8_t>& buf = file_bytes ? *file_bytes : local;
  std::string err;
  if (!read_file(path, &buf, &err)) return err;
  if (buf.size() < 8) return "file shorter than the 8-byte header length";
  uint64_t hn = 0;
  for (int i = 0; i < 8; ++i) hn |= (uint64_t)buf[i] << (8 * i);
  if (hn > buf.size() - 8 || hn > (100ull << 20)) return "header length " + std::to_string(hn) + " exceeds the file";
  const uint64_t data0 = 8 + hn, dsize = buf.size() - data0;
  JParser P{reinterpret_cast<const char*>(buf.data()) + 8, reinterpret_cast<const char*>(buf.data()) + data0, {}};
  JVal root;
  if (!P.val(root)) return "header is not valid JSON: " + P.err;
  P.ws();
  if (P.p != P.e) return "trailing bytes after the JSON header";
  if (root.kind != JVal::OBJ) return "header is not a JSON object";

  std::vector<AdapterEntry> want = adapter_entries(c);
  std::map<std::string, size_t> idx;
  for (size_t i = 0; i < want.size(); ++i) idx[want[i].name] = i;
  std::vector<char> seen(want.size(), 0);
  const JVal* meta = nullptr;
  std::vector<std::pair<uint64_t, uint64_t>> ranges;
  for (const auto& kv : root.obj) {
    if (kv.first == "__metadata__") {
      if (meta) return "duplicate __metadata__";
      if (kv.second.kind != JVal::OBJ) return "__metadata__ is not an object";
      meta = &kv.second;
      continue;
    }
    auto it = idx.find(kv.first);
    if (it == idx.end()) return "unexpected tensor " + kv.first + " (not an adapter of this stack)";
    if (seen[it->second]) return "duplicate tensor " + kv.first;
    seen[it->second] = 1;
    AdapterEntry& w = want[it->second];
    const JVal& t = kv.second;
    const JVal* dt = t.kind == JVal::OBJ ? t.get("dtype") : nullptr;
    const JVal* sh = t.kind == JVal::OBJ ? t.get("shape") : nullptr;
    const JVal* of = t.kind == JVal::OBJ ? t.get("data_offsets") : nullptr;
    if (!dt || dt->kind != JVal::STR || dt->s != "F32") return "tensor " + kv.first + ": dtype is not F32";
    uint64_t d0, d1, b, en;
    if (!sh || sh->kind != JVal::ARR || sh->arr.size() != 2 || !as_u63(sh->arr[0], &d0) || !as_u63(sh->arr[1], &d1) ||
        d0 != (uint64_t)w.rows || d1 != (uint64_t)w.cols)
      return "tensor " + kv.first + ": shape is not [" + std::to_string(w.rows) + ", " + std::to_string(w.cols) + "]";
    if (!of || of->kind != JVal::ARR || of->arr.size() != 2 || !as_u63(of->arr[0], &b) || !as_u63(of->arr[1], &en) ||
        b > en || en > dsize || en - b != (uint64_t)4 * w.rows * w.cols)
      return "tensor " + kv.first + ": data offsets out of range or of the wrong length";
    w.offset = data0 + b;
    ranges.push_back({b, en});
  }
  for (size_t i = 0; i < want.size(); ++i)
    if (!seen[i]) return "missing tensor " + want[i].name;
  std::sort(ranges.begin(), ranges.end());
  for (size_t i = 1; i < ranges.size(); ++i)
    if (ranges[i].first < ranges[i - 1].second) return "tensor data ranges overlap";
  if (!meta) return "no __metadata__ (the integrity record is missing)";
  auto mstr = [&](const std::string& k) -> const std::string* {
    const JVal* v = meta->get(k);
    return v && v->kind == JVal::STR ? &v->s : nullptr;
  };
  const std::pair<const char*, std::string> facts[3] = {{"lsq.n_layers", std::to_string(c.n_layers)},
                                                        {"lsq.r", std::to_string(c.lora_r)},
                                                        {"lsq.mask", std::to_string(c.lora_mask)}};
  for (const auto& f : facts) {
    const std::string* v = mstr(f.first);
    if (!v || *v != f.second)
      return std::string("metadata ") + f.first + " is " + (v ? "\"" + *v + "\"" : "absent") + ", the stack has " +
             f.second;
  }
  for (const AdapterEntry& w : want) {
    const std::string* v = mstr("lsq.crc32." + w.name);
    if (!v) return "no CRC-32 recorded for " + w.name;
    const std::string got = hex8(crc32_bytes(buf.data() + w.offset, (size_t)(4 * w.rows * w.cols)));
    if (*v != got) return "CRC-32 mismatch for " + w.name + " (recorded " + *v + ", data " + got + ")";
  }
  if (entries) *entries = std::move(want);
  return "";
}

}  // namespace lsq
