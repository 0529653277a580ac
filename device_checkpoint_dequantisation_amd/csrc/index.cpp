// Host side of libstmat: the metadata-only safetensors index and the descriptor planner.
//
// The pages ("Disk tier safetensors streaming design audit", "FastSageTensors capability
// audit" and "Strategy summary / Streaming safetensors mapping") describe an index built from
// the header alone: per tensor a dtype, a shape and data_offsets, with tensors loaded on demand.
// This file parses the safetensors header (8-byte little-endian length N, then N bytes of JSON)
// with its own strict JSON reader, checks that the offsets tile the data section, pairs quantised
// weights with their scale tensors and plans the work-unit table the grouped kernel consumes.
#include <fcntl.h>
#include <sys/stat.h>
#include <unistd.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <memory>
#include <new>
#include <stdexcept>
#include <tuple>
#include <string>
#include <unordered_map>
#include <utility>
#include <vector>

#include "index_impl.h"
#include "st_internal.h"

// ---------------------------------------------------------------------------------- errors

static thread_local std::string g_err;

extern "C" const char* st_last_error(void) { return g_err.c_str(); }

st_status st_fail(st_status code, const char* fmt, ...) {
    char buf[1024];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

static void st_clear() { g_err.clear(); }
void sti::clear_error() { st_clear(); }

namespace {

using sti::Output;
using sti::Tensor;

// ---------------------------------------------------------------------------------- dtypes

struct DtypeInfo {
    const char* name;
    uint32_t bits;
};
const DtypeInfo kDtypes[] = {
    {"BOOL", 8}, {"U8", 8},   {"I8", 8},   {"F8_E4M3", 8}, {"F8_E5M2", 8}, {"F8_E8M0", 8}, {"I16", 16},
    {"U16", 16}, {"F16", 16}, {"BF16", 16}, {"I32", 32},   {"U32", 32},    {"F32", 32},    {"I64", 64},
    {"U64", 64}, {"F64", 64}, {"F4", 4},   {"F6_E2M3", 6}, {"F6_E3M2", 6},
};
constexpr int kNumDtypes = sizeof(kDtypes) / sizeof(kDtypes[0]);

int dtype_of(const std::string& s) {
    for (int i = 0; i < kNumDtypes; ++i)
        if (s == kDtypes[i].name) return i;
    return -1;
}

// ---------------------------------------------------------------------------------- JSON

struct JVal {
    enum Type : uint8_t { Null, Bool, Int, BigInt, Float, Str, Arr, Obj } t = Null;
    bool b = false;
    int64_t i = 0;  // Int: value (may be negative)
    std::string s;
    std::vector<JVal> a;
    std::vector<std::pair<std::string, JVal>> o;
};

// Strict UTF-8 check (no overlongs, no encoded surrogates, nothing above U+10FFFF).
bool valid_utf8(const unsigned char* p, size_t n) {
    size_t i = 0;
    while (i < n) {
        unsigned c = p[i];
        if (c < 0x80) { ++i; continue; }
        size_t len;
        uint32_t cp, min;
        if ((c & 0xE0) == 0xC0) { len = 2; cp = c & 0x1F; min = 0x80; }
        else if ((c & 0xF0) == 0xE0) { len = 3; cp = c & 0x0F; min = 0x800; }
        else if ((c & 0xF8) == 0xF0) { len = 4; cp = c & 0x07; min = 0x10000; }
        else return false;
        if (i + len > n) return false;
        for (size_t k = 1; k < len; ++k) {
            unsigned d = p[i + k];
            if ((d & 0xC0) != 0x80) return false;
            cp = (cp << 6) | (d & 0x3F);
        }
        if (cp < min || cp > 0x10FFFF || (cp >= 0xD800 && cp <= 0xDFFF)) return false;
        i += len;
    }
    return true;
}

class JsonReader {
   public:
    JsonReader(const char* p, size_t n) : p_(p), end_(p + n) {}

    st_status parse(JVal& out) {
        ws();
        st_status r = value(out, 0);
        if (r) return r;
        ws();
        if (p_ != end_) return err("unexpected data after the JSON value");
        return ST_OK;
    }

   private:
    const char* p_;
    const char* end_;
    const char* begin_ = p_;

    st_status err(const char* what) {
        return st_fail(ST_E_JSON, "header is not valid JSON: %s at byte %zu", what, size_t(p_ - begin_));
    }
    void ws() {
        while (p_ < end_ && (*p_ == ' ' || *p_ == '\t' || *p_ == '\n' || *p_ == '\r')) ++p_;
    }
    bool lit(const char* s) {
        size_t n = strlen(s);
        if (size_t(end_ - p_) < n || memcmp(p_, s, n) != 0) return false;
        p_ += n;
        return true;
    }

    st_status value(JVal& v, int depth) {
        if (depth > 64) return err("nesting deeper than 64");
        if (p_ >= end_) return err("unexpected end");
        char c = *p_;
        if (c == '{') return object(v, depth);
        if (c == '[') return array(v, depth);
        if (c == '"') { v.t = JVal::Str; return string(v.s); }
        if (c == '-' || (c >= '0' && c <= '9')) return number(v);
        if (lit("true")) { v.t = JVal::Bool; v.b = true; return ST_OK; }
        if (lit("false")) { v.t = JVal::Bool; v.b = false; return ST_OK; }
        if (lit("null")) { v.t = JVal::Null; return ST_OK; }
        return err("unexpected character");
    }

    st_status object(JVal& v, int depth) {
        v.t = JVal::Obj;
        ++p_;
        ws();
        if (p_ < end_ && *p_ == '}') { ++p_; return ST_OK; }
        std::unordered_map<std::string, size_t> seen;
        for (;;) {
            ws();
            if (p_ >= end_ || *p_ != '"') return err("expected a string key");
            std::string key;
            if (st_status r = string(key)) return r;
            if (!seen.emplace(key, v.o.size()).second)
                return st_fail(ST_E_JSON, "duplicate key \"%s\" in header", key.c_str());
            ws();
            if (p_ >= end_ || *p_ != ':') return err("expected ':'");
            ++p_;
            ws();
            v.o.emplace_back(std::move(key), JVal());
            if (st_status r = value(v.o.back().second, depth + 1)) return r;
            ws();
            if (p_ < end_ && *p_ == ',') { ++p_; continue; }
            if (p_ < end_ && *p_ == '}') { ++p_; return ST_OK; }
            return err("expected ',' or '}'");
        }
    }

    st_status array(JVal& v, int depth) {
        v.t = JVal::Arr;
        ++p_;
        ws();
        if (p_ < end_ && *p_ == ']') { ++p_; return ST_OK; }
        for (;;) {
            ws();
            v.a.emplace_back();
            if (st_status r = value(v.a.back(), depth + 1)) return r;
            ws();
            if (p_ < end_ && *p_ == ',') { ++p_; continue; }
            if (p_ < end_ && *p_ == ']') { ++p_; return ST_OK; }
            return err("expected ',' or ']'");
        }
    }

    static int hex(char c) {
        if (c >= '0' && c <= '9') return c - '0';
        if (c >= 'a' && c <= 'f') return c - 'a' + 10;
        if (c >= 'A' && c <= 'F') return c - 'A' + 10;
        return -1;
    }
    bool u4(uint32_t& cp) {
        if (end_ - p_ < 4) return false;
        cp = 0;
        for (int k = 0; k < 4; ++k) {
            int h = hex(p_[k]);
            if (h < 0) return false;
            cp = cp * 16 + uint32_t(h);
        }
        p_ += 4;
        return true;
    }
    static void put_utf8(std::string& s, uint32_t cp) {
        if (cp < 0x80) s += char(cp);
        else if (cp < 0x800) { s += char(0xC0 | (cp >> 6)); s += char(0x80 | (cp & 0x3F)); }
        else if (cp < 0x10000) {
            s += char(0xE0 | (cp >> 12)); s += char(0x80 | ((cp >> 6) & 0x3F)); s += char(0x80 | (cp & 0x3F));
        } else {
            s += char(0xF0 | (cp >> 18)); s += char(0x80 | ((cp >> 12) & 0x3F));
            s += char(0x80 | ((cp >> 6) & 0x3F)); s += char(0x80 | (cp & 0x3F));
        }
    }

    st_status string(std::string& s) {
        ++p_;  // opening quote
        for (;;) {
            if (p_ >= end_) return err("unterminated string");
            unsigned char c = (unsigned char)*p_;
            if (c == '"') { ++p_; break; }
            if (c < 0x20) return err("control character in string");
            if (c != '\\') { s += char(c); ++p_; continue; }
            ++p_;
            if (p_ >= end_) return err("unterminated escape");
            char e = *p_++;
            switch (e) {
                case '"': s += '"'; break;
                case '\\': s += '\\'; break;
                case '/': s += '/'; break;
                case 'b': s += '\b'; break;
                case 'f': s += '\f'; break;
                case 'n': s += '\n'; break;
                case 'r': s += '\r'; break;
                case 't': s += '\t'; break;
                case 'u': {
                    uint32_t cp;
                    if (!u4(cp)) return err("bad \\u escape");
                    if (cp >= 0xDC00 && cp <= 0xDFFF)
                        return st_fail(ST_E_JSON, "string with an unpaired surrogate in header");
                    if (cp >= 0xD800 && cp <= 0xDBFF) {
                        uint32_t lo;
                        if (end_ - p_ < 6 || p_[0] != '\\' || p_[1] != 'u')
                            return st_fail(ST_E_JSON, "string with an unpaired surrogate in header");
                        p_ += 2;
                        if (!u4(lo)) return err("bad \\u escape");
                        if (lo < 0xDC00 || lo > 0xDFFF)
                            return st_fail(ST_E_JSON, "string with an unpaired surrogate in header");
                        cp = 0x10000 + ((cp - 0xD800) << 10) + (lo - 0xDC00);
                    }
                    put_utf8(s, cp);
                    break;
                }
                default: return err("invalid escape");
            }
        }
        return ST_OK;
    }

    st_status number(JVal& v) {
        const char* start = p_;
        bool neg = false;
        if (*p_ == '-') { neg = true; ++p_; }
        if (p_ >= end_ || !(*p_ >= '0' && *p_ <= '9')) return err("bad number");
        bool big = false;
        uint64_t mag = 0;
        if (*p_ == '0') ++p_;
        else
            while (p_ < end_ && *p_ >= '0' && *p_ <= '9') {
                uint64_t d = uint64_t(*p_ - '0');
                if (mag > (UINT64_MAX - d) / 10) big = true;
                else mag = mag * 10 + d;
                ++p_;
            }
        bool is_float = false;
        if (p_ < end_ && *p_ == '.') {
            ++p_;
            if (p_ >= end_ || !(*p_ >= '0' && *p_ <= '9')) return err("bad number");
            while (p_ < end_ && *p_ >= '0' && *p_ <= '9') ++p_;
            is_float = true;
        }
        if (p_ < end_ && (*p_ == 'e' || *p_ == 'E')) {
            ++p_;
            if (p_ < end_ && (*p_ == '+' || *p_ == '-')) ++p_;
            if (p_ >= end_ || !(*p_ >= '0' && *p_ <= '9')) return err("bad number");
            while (p_ < end_ && *p_ >= '0' && *p_ <= '9') ++p_;
            is_float = true;
        }
        (void)start;
        if (is_float) { v.t = JVal::Float; return ST_OK; }
        if (big || mag > uint64_t(INT64_MAX) + (neg ? 1 : 0)) { v.t = JVal::BigInt; return ST_OK; }
        v.t = JVal::Int;
        v.i = neg ? int64_t(0 - mag) : int64_t(mag);
        return ST_OK;
    }
};

// ---------------------------------------------------------------------------------- index

bool ends_with(const std::string& s, const char* suf) {
    size_t n = strlen(suf);
    return s.size() >= n && memcmp(s.data() + s.size() - n, suf, n) == 0;
}

const char* const kScaleSuffixes[] = {".scale_weight", ".weight_scale_inv", ".weight_scale_2", ".weight_scale"};

bool is_scale_name(const std::string& s) {
    for (const char* suf : kScaleSuffixes)
        if (ends_with(s, suf)) return true;
    return false;
}

std::string shape_str(const std::vector<int64_t>& sh) {
    std::string s = "[";
    for (size_t i = 0; i < sh.size(); ++i) s += (i ? "," : "") + std::to_string(sh[i]);
    return s + "]";
}

uint64_t round_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

}  // namespace


namespace {

std::string json_quote(const std::string& s) {
    std::string o = "\"";
    for (unsigned char c : s) {
        if (c == '"' || c == '\\') { o += '\\'; o += char(c); }
        else if (c < 0x20) { char b[8]; snprintf(b, sizeof b, "\\u%04x", c); o += b; }
        else o += char(c);
    }
    return o + "\"";
}

st_status check_name(const std::string& s) {
    if (s.find('\0') != std::string::npos) return st_fail(ST_E_JSON, "string with a NUL character in header");
    return ST_OK;
}

bool is_scalar(const Tensor& t) { return t.shape.empty() || (t.shape.size() == 1 && t.shape[0] == 1); }

st_status read_int(const JVal& v, const std::string& name, const char* field, int64_t& out) {
    if (v.t != JVal::Int || v.i < 0)
        return st_fail(ST_E_SHAPE, "%s: %s must hold non-negative integers below 2^63", name.c_str(), field);
    out = v.i;
    return ST_OK;
}

st_status parse_entries(st_index& ix, const JVal& root) {
    if (root.t != JVal::Obj) return st_fail(ST_E_JSON, "header is not a JSON object");
    ix.tensors.reserve(root.o.size());
    for (const auto& kv : root.o) {
        const std::string& name = kv.first;
        const JVal& val = kv.second;
        if (st_status r = check_name(name)) return r;
        if (name == "__metadata__") {
            if (val.t != JVal::Obj) return st_fail(ST_E_JSON, "__metadata__ must map strings to strings");
            std::string m = "{";
            for (size_t i = 0; i < val.o.size(); ++i) {
                if (val.o[i].second.t != JVal::Str) return st_fail(ST_E_JSON, "__metadata__ must map strings to strings");
                if (check_name(val.o[i].first) || check_name(val.o[i].second.s))
                    return st_fail(ST_E_JSON, "string with a NUL character in header");
                m += (i ? "," : "") + json_quote(val.o[i].first) + ":" + json_quote(val.o[i].second.s);
            }
            ix.metadata_json = m + "}";
            continue;
        }
        if (val.t != JVal::Obj || val.o.size() != 3)
            return st_fail(ST_E_SHAPE, "%s: entry must have exactly dtype, shape, data_offsets", name.c_str());
        const JVal *dt = nullptr, *sh = nullptr, *of = nullptr;
        for (const auto& f : val.o) {
            if (f.first == "dtype") dt = &f.second;
            else if (f.first == "shape") sh = &f.second;
            else if (f.first == "data_offsets") of = &f.second;
        }
        if (!dt || !sh || !of)
            return st_fail(ST_E_SHAPE, "%s: entry must have exactly dtype, shape, data_offsets", name.c_str());
        Tensor t;
        t.name = name;
        t.dtype = dt->t == JVal::Str ? dtype_of(dt->s) : -1;
        if (t.dtype < 0)
            return st_fail(ST_E_DTYPE, "%s: unknown dtype %s", name.c_str(), dt->t == JVal::Str ? dt->s.c_str() : "(not a string)");
        if (sh->t != JVal::Arr) return st_fail(ST_E_SHAPE, "%s: shape must be a list of non-negative integers", name.c_str());
        if (sh->a.size() > ST_MAX_NDIM) return st_fail(ST_E_SHAPE, "%s: more than %d dimensions", name.c_str(), ST_MAX_NDIM);
        for (const JVal& d : sh->a) {
            int64_t x;
            if (st_status r = read_int(d, name, "shape", x)) return r;
            t.shape.push_back(x);
        }
        if (of->t != JVal::Arr || of->a.size() != 2)
            return st_fail(ST_E_OFFSETS, "%s: data_offsets must be two non-negative integers", name.c_str());
        int64_t b = 0, e = 0;
        if (read_int(of->a[0], name, "data_offsets", b) || read_int(of->a[1], name, "data_offsets", e))
            return st_fail(ST_E_OFFSETS, "%s: data_offsets must be two non-negative integers", name.c_str());
        if (b > e) return st_fail(ST_E_OFFSETS, "%s: data_offsets begin %lld > end %lld", name.c_str(), (long long)b, (long long)e);
        t.begin = uint64_t(b);
        t.end = uint64_t(e);
        // numel * bits must equal the span; any zero dimension makes numel 0 whatever the others.
        bool zero = false;
        for (int64_t d : t.shape) zero |= d == 0;
        unsigned __int128 numel = 1;
        bool overflow = false;
        if (!zero)
            for (int64_t d : t.shape) {
                numel *= uint64_t(d);
                if (numel > (unsigned __int128)UINT64_MAX) { overflow = true; break; }
            }
        if (zero) numel = 0;
        unsigned __int128 bits = numel * kDtypes[t.dtype].bits;
        if (overflow || bits % 8 != 0 || bits / 8 != (unsigned __int128)(t.end - t.begin))
            return st_fail(ST_E_SHAPE, "%s: %s%s needs %s bytes, offsets span %llu", name.c_str(), kDtypes[t.dtype].name,
                           shape_str(t.shape).c_str(),
                           overflow ? "more than 2^64" : (bits % 8 ? "a fractional number of" : std::to_string((uint64_t)(bits / 8)).c_str()),
                           (unsigned long long)(t.end - t.begin));
        t.numel = uint64_t(numel);
        ix.by_name.emplace(name, uint32_t(ix.tensors.size()));
        ix.tensors.push_back(std::move(t));
    }
    return ST_OK;
}

st_status check_layout(const st_index& ix) {
    std::vector<uint32_t> order(ix.tensors.size());
    for (uint32_t i = 0; i < order.size(); ++i) order[i] = i;
    std::sort(order.begin(), order.end(), [&](uint32_t a, uint32_t b) {
        const Tensor &x = ix.tensors[a], &y = ix.tensors[b];
        return x.begin != y.begin ? x.begin < y.begin : x.end < y.end;
    });
    uint64_t pos = 0;
    for (uint32_t i : order) {
        const Tensor& t = ix.tensors[i];
        if (t.begin != pos)
            return st_fail(ST_E_OFFSETS, "%s: data_offsets [%llu, %llu] %s byte %llu", t.name.c_str(),
                           (unsigned long long)t.begin, (unsigned long long)t.end,
                           t.begin < pos ? "overlaps" : "leaves a gap before", (unsigned long long)pos);
        pos = t.end;
    }
    if (pos != ix.data_size)
        return st_fail(ST_E_OFFSETS, "tensors cover %llu bytes but the data section has %llu",
                       (unsigned long long)pos, (unsigned long long)ix.data_size);
    return ST_OK;
}

const Tensor* find(const st_index& ix, const std::string& name, int64_t* idx = nullptr) {
    auto it = ix.by_name.find(name);
    if (it == ix.by_name.end()) return nullptr;
    if (idx) *idx = it->second;
    return &ix.tensors[it->second];
}

// An MX weight (kind MXFP8 or MXFP4) of K logical columns (-1: not 2-D) with its E8M0 scale
// [M, K/32]; fills the output's kind, shape and scale.
st_status mx_output(const st_index& ix, const Tensor& t, const std::string& x, const Tensor& sc, int64_t sci,
                    st_kind kind, int64_t k, Output& o) {
    const char* kn = kind == ST_KIND_MXFP8 ? "MXFP8" : "MXFP4";
    if (t.shape.size() != 2 || k < 0)
        return st_fail(ST_E_SHAPE, "%s: %s weight must be 2-D, got %s", t.name.c_str(), kn, shape_str(t.shape).c_str());
    if (k % 32) return st_fail(ST_E_SHAPE, "%s: %s K=%lld is not a multiple of 32", t.name.c_str(), kn, (long long)k);
    if (find(ix, x + ".weight_scale_2"))
        return st_fail(ST_E_SCALE, "%s.weight_scale_2: an E8M0-scaled weight takes no weight_scale_2", x.c_str());
    const int64_t m = t.shape[0];
    if (sc.dtype != ST_DT_F8_E8M0 || sc.shape.size() != 2 || sc.shape[0] != m || sc.shape[1] != k / 32)
        return st_fail(ST_E_SCALE, "%s: must be F8_E8M0 [%lld,%lld], got %s%s", sc.name.c_str(), (long long)m,
                       (long long)(k / 32), kDtypes[sc.dtype].name, shape_str(sc.shape).c_str());
    if (k >= (int64_t(1) << 32))
        return st_fail(ST_E_SHAPE, "%s: %s K of 2^32 or more is not supported", t.name.c_str(), kn);
    o.kind = kind;
    o.shape = {m, k};
    o.numel = uint64_t(m) * uint64_t(k);
    o.scale = sci;
    return ST_OK;
}

st_status classify(st_index& ix) {
    std::vector<bool> used(ix.tensors.size(), false);
    for (uint32_t ti = 0; ti < ix.tensors.size(); ++ti) {
        const Tensor& t = ix.tensors[ti];
        if (is_scale_name(t.name)) continue;
        Output o;
        o.tensor = ti;
        o.shape = t.shape;
        o.numel = t.numel;
        const char* dn = kDtypes[t.dtype].name;
        if (t.dtype == ST_DT_BF16) o.kind = ST_KIND_PASS_BF16;
        else if (t.dtype == ST_DT_F16) o.kind = ST_KIND_CAST_F16;
        else if (t.dtype == ST_DT_F32) o.kind = ST_KIND_CAST_F32;
        else if (t.dtype == ST_DT_F8_E4M3) {
            if (!ends_with(t.name, ".weight"))
                return st_fail(ST_E_SCALE, "%s: float8 tensor without a scale (not named X.weight)", t.name.c_str());
            std::string x = t.name.substr(0, t.name.size() - 7);
            int64_t si = -1, bi = -1, mi = -1;
            const Tensor* st = find(ix, x + ".scale_weight", &si);
            const Tensor* sb = find(ix, x + ".weight_scale_inv", &bi);
            const Tensor* sm = find(ix, x + ".weight_scale", &mi);
            if (int(st != nullptr) + int(sb != nullptr) + int(sm != nullptr) > 1)
                return st_fail(ST_E_SCALE, "%s: more than one of scale_weight, weight_scale_inv, weight_scale present",
                               t.name.c_str());
            if (sm) {
                if (st_status r = mx_output(ix, t, x, *sm, mi, ST_KIND_MXFP8, t.shape.size() == 2 ? t.shape[1] : -1, o))
                    return r;
            } else if (st) {
                if (st->dtype != ST_DT_F32 || !is_scalar(*st))
                    return st_fail(ST_E_SCALE, "%s: scale_weight must be an fp32 scalar, got %s%s", st->name.c_str(),
                                   kDtypes[st->dtype].name, shape_str(st->shape).c_str());
                o.kind = ST_KIND_FP8_TENSOR;
                o.scale = si;
            } else if (sb) {
                if (t.shape.size() != 2)
                    return st_fail(ST_E_SHAPE, "%s: block-scaled float8 weight must be 2-D, got %s", t.name.c_str(),
                                   shape_str(t.shape).c_str());
                int64_t gm = (t.shape[0] + 127) / 128, gn = (t.shape[1] + 127) / 128;
                if (sb->dtype != ST_DT_F32 || sb->shape.size() != 2 || sb->shape[0] != gm || sb->shape[1] != gn)
                    return st_fail(ST_E_SCALE, "%s: must be F32 [%lld,%lld], got %s%s", sb->name.c_str(), (long long)gm,
                                   (long long)gn, kDtypes[sb->dtype].name, shape_str(sb->shape).c_str());
                if (t.numel >= (uint64_t(1) << 32) || t.shape[1] >= (int64_t(1) << 32))
                    return st_fail(ST_E_SHAPE, "%s: block-scaled float8 weights of 2^32 or more elements are not supported",
                                   t.name.c_str());
                o.kind = ST_KIND_FP8_BLOCK128;
                o.scale = bi;
            } else {
                return st_fail(ST_E_SCALE, "%s: float8 weight has no scale_weight, weight_scale_inv or weight_scale",
                               t.name.c_str());
            }
        } else if (t.dtype == ST_DT_U8 || t.dtype == ST_DT_F4) {
            if (!ends_with(t.name, ".weight"))
                return st_fail(ST_E_DTYPE, "%s: %s tensor is not an NVFP4 or MXFP4 weight", t.name.c_str(), dn);
            if (t.shape.size() != 2)
                return st_fail(ST_E_SHAPE, "%s: packed fp4 weight must be 2-D, got %s", t.name.c_str(),
                               shape_str(t.shape).c_str());
            std::string x = t.name.substr(0, t.name.size() - 7);
            int64_t m = t.shape[0];
            int64_t k = t.dtype == ST_DT_U8 ? t.shape[1] * 2 : t.shape[1];
            int64_t bsi = -1, gi = -1;
            const Tensor* bs = find(ix, x + ".weight_scale", &bsi);
            const Tensor* g = find(ix, x + ".weight_scale_2", &gi);
            if (bs && bs->dtype == ST_DT_F8_E8M0) {  // MXFP4
                if (st_status r = mx_output(ix, t, x, *bs, bsi, ST_KIND_MXFP4, k, o)) return r;
            } else {  // NVFP4
                if (k % 16)
                    return st_fail(ST_E_SHAPE, "%s: NVFP4 K=%lld is not a multiple of 16", t.name.c_str(), (long long)k);
                if (!bs || !g)
                    return st_fail(ST_E_SCALE, "%s: NVFP4 weight needs weight_scale and weight_scale_2", t.name.c_str());
                if (bs->dtype != ST_DT_F8_E4M3 || bs->shape.size() != 2 || bs->shape[0] != m || bs->shape[1] != k / 16)
                    return st_fail(ST_E_SCALE, "%s: must be F8_E4M3 [%lld,%lld], got %s%s", bs->name.c_str(),
                                   (long long)m, (long long)(k / 16), kDtypes[bs->dtype].name,
                                   shape_str(bs->shape).c_str());
                if (g->dtype != ST_DT_F32 || !is_scalar(*g))
                    return st_fail(ST_E_SCALE, "%s: weight_scale_2 must be an fp32 scalar", g->name.c_str());
                if (k >= (int64_t(1) << 32))
                    return st_fail(ST_E_SHAPE, "%s: NVFP4 K of 2^32 or more is not supported", t.name.c_str());
                o.kind = ST_KIND_NVFP4;
                o.shape = {m, k};
                o.numel = uint64_t(m) * uint64_t(k);
                o.scale = bsi;
                o.scale2 = gi;
            }
        } else {
            return st_fail(ST_E_DTYPE, "%s: dtype %s cannot be materialised as bf16", t.name.c_str(), dn);
        }
        if (o.scale >= 0) used[size_t(o.scale)] = true;
        if (o.scale2 >= 0) used[size_t(o.scale2)] = true;
        ix.outputs.push_back(std::move(o));
    }
    for (uint32_t ti = 0; ti < ix.tensors.size(); ++ti)
        if (is_scale_name(ix.tensors[ti].name) && !used[ti])
            return st_fail(ST_E_SCALE, "%s: scale tensor with no matching weight", ix.tensors[ti].name.c_str());
    std::stable_sort(ix.outputs.begin(), ix.outputs.end(), [&](const Output& a, const Output& b) {
        const Tensor &x = ix.tensors[a.tensor], &y = ix.tensors[b.tensor];
        return x.begin != y.begin ? x.begin < y.begin : x.name < y.name;
    });
    return ST_OK;
}

// `at[t]` (if given) is where tensor t's bytes sit in the device blob; by default the blob is the
// data section itself.
st_desc make_desc(const st_index& ix, const Output& o, uint32_t out_slot, uint64_t unit_begin, uint64_t* units,
                  const uint64_t* at) {
    // unit_begin + units stays below 2^32: build_table rejects larger tables before use
    st_desc d;
    memset(&d, 0, sizeof d);
    auto where = [&](size_t t) { return at ? at[t] : ix.tensors[t].begin; };
    d.src = where(o.tensor);
    d.scale = o.scale >= 0 ? where(size_t(o.scale)) : 0;
    d.scale2 = o.scale2 >= 0 ? where(size_t(o.scale2)) : 0;
    d.out = out_slot;
    const uint32_t unit_shift = stk::step_shift(o.kind, ix.out_dtype) + ix.unit_log2_scale;
    uint32_t div_shift = 0;
    if (o.kind == ST_KIND_FP8_BLOCK128) {
        uint32_t n = uint32_t(o.shape[1]);
        d.cols = n;
        d.grid_cols = (n + 127) / 128;
        if (n) {
            d.div_magic = stk::div_magic(n);
            div_shift = stk::div_shift(n);
        }
    } else if (o.kind == ST_KIND_NVFP4 || o.kind == ST_KIND_MXFP8 || o.kind == ST_KIND_MXFP4) {
        d.cols = uint32_t(o.shape[1]);
    }
    d.meta = uint32_t(o.kind) | unit_shift << 8 | div_shift << 16;
    *units = (o.numel + (uint64_t(1) << unit_shift) - 1) >> unit_shift;
    d.unit_begin = uint32_t(unit_begin);
    d.unit_end = uint32_t(unit_begin + *units);
    d.tail = uint32_t(o.numel - ((*units ? *units - 1 : 0) << unit_shift));
    return d;
}

}  // namespace

namespace {

// A work table from descriptors whose unit ranges are set, `units` in total: header, map,
// descriptors.
// Outputs larger than this (the MI355X's 256 MiB Infinity Cache) are written with streaming
// (non-temporal, system-scope) stores.  Measured against plain stores: +2 to +4% on the large
// checkpoints and their row shards, +7 to +11% on one rank's column shards; on the many-small
// checkpoint (211 MB of outputs) plain stores leave the outputs in that cache and the launch 10%
// shorter after a flush.
constexpr uint64_t kStreamStoreBytes = uint64_t(256) << 20;

std::vector<unsigned char> assemble(const std::vector<st_desc>& descs, uint64_t units, uint32_t out_dtype,
                                    uint64_t out_bytes) {
    const size_t k = descs.size();
    const uint64_t groups = (units + ST_UNITS_PER_GROUP - 1) / ST_UNITS_PER_GROUP;
    st_table_header h;
    memset(&h, 0, sizeof h);
    h.magic = ST_TABLE_MAGIC;
    h.n_desc = uint32_t(k);
    h.units = units;
    h.map_offset = sizeof(st_table_header);
    h.desc_offset = stk::table_desc_offset(groups);
    h.bytes = h.desc_offset + k * sizeof(st_desc);
    h.out_dtype = out_dtype;
    h.flags = out_bytes > kStreamStoreBytes ? ST_TABLE_STREAM_STORES : 0u;
    std::vector<unsigned char> t(h.bytes, 0);
    memcpy(t.data(), &h, sizeof h);
    if (k) memcpy(t.data() + h.desc_offset, descs.data(), k * sizeof(st_desc));
    uint32_t* map = reinterpret_cast<uint32_t*>(t.data() + h.map_offset);
    size_t d = 0;
    for (uint64_t g = 0; g < groups; ++g) {
        const uint64_t u = g * ST_UNITS_PER_GROUP;
        while (descs[d].unit_end <= u) ++d;  // skips outputs with no units
        map[g] = uint32_t(d);
    }
    return t;
}

}  // namespace

// Work-unit order.  The kernel gives XCD x the x-th contiguous eighth of the units.  Formats carry
// different bytes per unit (about 3 KB for fp8, 4 KB for a bf16 copy, 5 KB for NVFP4), so in file
// order an eighth that holds, say, a whole bf16 embedding carries more bytes than the rest and
// finishes last.  When the file-order eighths differ by more than kImbalance in bytes, every
// output of at least kPieceMinUnits units is cut into 8 equal pieces, piece p placed in the p-th
// eighth (slot p), and the smaller outputs fill the slots in file order, an eighth of their units
// each: each XCD then streams through one eighth of every large tensor.  Otherwise the file order
// is kept, since jumping between tensors costs a homogeneous checkpoint about 1% (measured on
// MI355X; the pieces gained 4.6% on a block-FP8 checkpoint with a bf16 embedding).
// A piece is one descriptor: unit_begin is set so that the kernel's element offset
// (unit - unit_begin) << shift lands inside the whole output (computed modulo 2^32), and only
// the output's last piece ends in its partial unit.
constexpr uint64_t kPieceMinUnits = 2048;
constexpr uint32_t kSlots = 8;
constexpr double kImbalance = 1.05;

// Bytes of the heaviest file-order eighth over the mean (1 when balanced).
double eighth_imbalance(const st_index& ix, const uint32_t* sel, size_t k, const std::vector<uint64_t>& nu,
                        uint64_t total) {
    if (total < kSlots) return 1.0;
    double eighth[kSlots] = {0};
    uint64_t pos = 0;
    double sum = 0;
    for (size_t j = 0; j < k; ++j) {
        if (!nu[j]) continue;
        const Output& o = ix.outputs[sel[j]];
        double bytes = double(o.numel) * double(sti::out_bytes(ix)) +
                       double(ix.tensors[o.tensor].end - ix.tensors[o.tensor].begin);
        if (o.scale >= 0) bytes += double(ix.tensors[size_t(o.scale)].end - ix.tensors[size_t(o.scale)].begin);
        const double per_unit = bytes / double(nu[j]);
        sum += bytes;
        uint64_t u = pos, end = pos + nu[j];
        while (u < end) {  // spread the output over the eighths its units fall in
            const uint32_t x = uint32_t(std::min<uint64_t>(kSlots - 1, u * kSlots / total));
            const uint64_t xe = x + 1 == kSlots ? end : std::min<uint64_t>(end, (uint64_t(x) + 1) * total / kSlots);
            const uint64_t stop = std::max<uint64_t>(xe, u + 1);
            eighth[x] += per_unit * double(stop - u);
            u = stop;
        }
        pos = end;
    }
    double mx = 0;
    for (double e : eighth) mx = std::max(mx, e);
    return sum > 0 ? mx / (sum / kSlots) : 1.0;
}

std::vector<unsigned char> sti::build_table(const st_index& ix, const uint32_t* sel, size_t k, uint64_t* units_out,
                                            const uint64_t* at) {
    std::vector<st_desc> whole(k);
    std::vector<uint64_t> nu(k);
    uint64_t total = 0;
    for (size_t j = 0; j < k; ++j) {
        whole[j] = make_desc(ix, ix.outputs[sel[j]], uint32_t(j), 0, &nu[j], at);
        total += nu[j];
        if (total >= (uint64_t(1) << 32)) throw std::length_error("2^32 or more work units");
    }
    const bool cut = eighth_imbalance(ix, sel, k, nu, total) > kImbalance;
    uint64_t small = 0;  // units of the outputs that are not cut
    for (size_t j = 0; j < k; ++j)
        if (!(cut && nu[j] >= kPieceMinUnits)) small += nu[j];
    struct Piece {
        size_t j;
        uint64_t first, count;
    };
    std::vector<std::vector<Piece>> slot(kSlots);
    uint64_t filled = 0;  // units of small outputs placed so far
    for (size_t j = 0; j < k; ++j) {
        if (cut && nu[j] >= kPieceMinUnits) {
            for (uint32_t p = 0; p < kSlots; ++p) {
                const uint64_t a = nu[j] * p / kSlots, e = nu[j] * (p + 1) / kSlots;
                slot[p].push_back({j, a, e - a});
            }
        } else {
            const uint64_t s = small ? std::min<uint64_t>(kSlots - 1, filled * kSlots / small) : 0;
            slot[s].push_back({j, 0, nu[j]});
            filled += nu[j];
        }
    }
    std::vector<st_desc> descs;
    descs.reserve(k + 8 * k);
    uint64_t pos = 0;
    for (const auto& sl : slot)
        for (const Piece& pc : sl) {
            st_desc d = whole[pc.j];
            const uint32_t shift = (d.meta >> 8) & 0xFFu;
            d.unit_begin = uint32_t(pos - pc.first);  // modulo 2^32, as the kernel subtracts
            d.unit_end = uint32_t(pos + pc.count);
            if (pc.first + pc.count != nu[pc.j]) d.tail = uint32_t(1) << shift;  // not the output's last unit
            descs.push_back(d);
            pos += pc.count;
        }
    *units_out = pos;
    uint64_t out_bytes = 0;
    for (size_t j = 0; j < k; ++j) out_bytes += ix.outputs[sel[j]].numel * sti::out_bytes(ix);
    return assemble(descs, pos, ix.out_dtype, out_bytes);
}

namespace {

// ---------------------------------------------------------------------------------- slices

// A slice with its bounds resolved against the output's matrix view [R, C].
struct Slice {
    uint64_t R, C, r0, r1, c0, c1;
    uint64_t rows() const { return r1 - r0; }
    uint64_t cols() const { return c1 - c0; }
    bool strided() const { return !(c0 == 0 && c1 == C); }
};

st_status resolve_slice(const st_index& ix, const st_slice& sl, Slice& g) {
    if (sl.output >= ix.outputs.size())
        return st_fail(ST_E_ARG, "slice of output %u, the index has %zu", sl.output, ix.outputs.size());
    const Output& o = ix.outputs[sl.output];
    const std::string& name = ix.tensors[o.tensor].name;
    if (sl.reserved) return st_fail(ST_E_ARG, "%s: slice.reserved must be 0", name.c_str());
    g.R = o.shape.empty() ? 1 : uint64_t(o.shape[0]);
    g.C = o.shape.size() <= 1 ? 1 : (g.R ? o.numel / g.R : 0);
    if (o.shape.size() > 1 && g.R == 0) {
        g.C = 1;
        for (size_t d = 1; d < o.shape.size(); ++d) g.C *= uint64_t(o.shape[d]);
    }
    const int64_t r1 = sl.row_end < 0 ? int64_t(g.R) : sl.row_end, c1 = sl.col_end < 0 ? int64_t(g.C) : sl.col_end;
    if (sl.row_begin < 0 || sl.row_begin > r1 || uint64_t(r1) > g.R || sl.col_begin < 0 || sl.col_begin > c1 ||
        uint64_t(c1) > g.C)
        return st_fail(ST_E_ARG, "%s: slice rows [%lld, %lld) cols [%lld, %lld) outside [%llu, %llu]", name.c_str(),
                       (long long)sl.row_begin, (long long)r1, (long long)sl.col_begin, (long long)c1,
                       (unsigned long long)g.R, (unsigned long long)g.C);
    g.r0 = uint64_t(sl.row_begin);
    g.r1 = uint64_t(r1);
    g.c0 = uint64_t(sl.col_begin);
    g.c1 = uint64_t(c1);
    if (o.kind == ST_KIND_FP8_BLOCK128 && (g.r0 % 128 || g.c0 % 128))
        return st_fail(ST_E_SHAPE, "%s: block-FP8 slices start at multiples of 128 (rows %llu, cols %llu)",
                       name.c_str(), (unsigned long long)g.r0, (unsigned long long)g.c0);
    if (o.kind == ST_KIND_NVFP4 && (g.c0 % 16 || g.cols() % 16))
        return st_fail(ST_E_SHAPE, "%s: NVFP4 column slices start at and span multiples of 16 (cols [%llu, %llu))",
                       name.c_str(), (unsigned long long)g.c0, (unsigned long long)g.c1);
    if ((o.kind == ST_KIND_MXFP8 || o.kind == ST_KIND_MXFP4) && (g.c0 % 32 || g.cols() % 32))
        return st_fail(ST_E_SHAPE, "%s: MX column slices start at and span multiples of 32 (cols [%llu, %llu))",
                       name.c_str(), (unsigned long long)g.c0, (unsigned long long)g.c1);
    if (g.strided() && (g.rows() * g.cols() >= (uint64_t(1) << 32) || g.C >= (uint64_t(1) << 32)))
        return st_fail(ST_E_SHAPE, "%s: a column slice needs fewer than 2^32 elements and rows shorter than 2^32",
                       name.c_str());
    return ST_OK;
}

st_desc make_slice_desc(const st_index& ix, const Output& o, const Slice& g, uint32_t out_slot, uint64_t unit_begin,
                        uint64_t* units) {
    st_desc d;
    memset(&d, 0, sizeof d);
    const Tensor& t = ix.tensors[o.tensor];
    const uint32_t bits = stk::source_bits(o.kind);
    const uint64_t first = g.r0 * g.C + g.c0;  // first source element
    d.src = t.begin + first * bits / 8;
    d.scale = o.scale >= 0 ? ix.tensors[size_t(o.scale)].begin : 0;
    d.scale2 = o.scale2 >= 0 ? ix.tensors[size_t(o.scale2)].begin : 0;
    d.out = out_slot;
    const uint64_t width = g.strided() ? g.cols() : g.C;  // the row length the kernel indexes by
    uint32_t div_shift = 0;
    if (o.kind == ST_KIND_FP8_BLOCK128) {
        d.grid_cols = uint32_t((g.C + 127) / 128);
        d.scale += 4 * ((g.r0 / 128) * d.grid_cols + g.c0 / 128);
    } else if (o.kind == ST_KIND_NVFP4) {
        d.scale += first / 16;
    } else if (o.kind == ST_KIND_MXFP8 || o.kind == ST_KIND_MXFP4) {
        d.scale += first / 32;
    }
    if (o.kind == ST_KIND_FP8_BLOCK128 || o.kind == ST_KIND_NVFP4 || o.kind == ST_KIND_MXFP8 ||
        o.kind == ST_KIND_MXFP4 || g.strided())
        d.cols = uint32_t(width);
    if ((o.kind == ST_KIND_FP8_BLOCK128 || g.strided()) && width) {
        d.div_magic = stk::div_magic(uint32_t(width));
        div_shift = stk::div_shift(uint32_t(width));
    }
    if (g.strided()) {
        d.pitch = uint32_t(g.C);
        const bool whole_chunks = g.cols() % stk::chunk_elems(o.kind) == 0;
        const bool aligned_rows = (g.C * bits / 8) % stk::load_word_bytes(o.kind) == 0 && (g.C * bits) % 8 == 0;
        if (!whole_chunks || !aligned_rows) d.flags = ST_DESC_EXACT;
    }
    const uint64_t numel = g.rows() * g.cols();
    const uint32_t unit_shift = stk::step_shift(o.kind, ix.out_dtype) + ix.unit_log2_scale;
    d.meta = uint32_t(o.kind) | unit_shift << 8 | div_shift << 16;
    *units = (numel + (uint64_t(1) << unit_shift) - 1) >> unit_shift;
    d.unit_begin = uint32_t(unit_begin);
    d.unit_end = uint32_t(unit_begin + *units);
    d.tail = uint32_t(numel - ((*units ? *units - 1 : 0) << unit_shift));
    return d;
}

// Unit order of a slice table.  Column slices of one output that cover the same rows (the
// tensor-parallel shards of a weight) read the same source rows, each a short segment of them; a
// segment's first and last 128-byte lines, and the lines of its NVFP4 / MX block scales, also hold
// bytes of the neighbouring segments.  Placed one after another, each slice fetches those shared
// lines again, long after its neighbour did.  So sibling column slices of packed fp4 weights are
// interleaved in bands of kBandUnits units: band b of every sibling, then band b + 1, ...  The bands
// of one row range run next to each other in the unit order, hence at about the same time on one
// XCD, and the shared lines come from its L2.  Measured on MI355X (8 column shards of every weight
// in one launch): NVFP4 4936 -> 5204 GB/s, MXFP4 5038 -> 5320 with bands of 16 units (bands of 64
// and 256 within 2%); the same order cost scaled FP8 3%, block FP8 5% and MXFP8 6%, whose shared
// lines are a smaller share of the reads while their writes then spread over eight outputs at once,
// so they keep the request order.  A band is a piece descriptor (unit_begin set so the kernel's
// element offset (unit - unit_begin) << shift lands inside the slice, modulo 2^32); only a slice's
// last band ends in its partial unit.  Other slices keep their place, in request order.
#ifndef ST_SLICE_BAND_UNITS
#define ST_SLICE_BAND_UNITS 16
#endif
#ifndef ST_SLICE_BAND_KINDS
#define ST_SLICE_BAND_KINDS ((1u << ST_KIND_NVFP4) | (1u << ST_KIND_MXFP4))
#endif
#ifndef ST_SLICE_SPLIT
#define ST_SLICE_SPLIT 1
#endif
constexpr uint64_t kBandUnits = ST_SLICE_BAND_UNITS;
constexpr bool kSplit = ST_SLICE_SPLIT != 0;
constexpr uint32_t kBandKinds = ST_SLICE_BAND_KINDS;

// A split descriptor for the slices j, j + 1, ..., j + S - 1 of the request if they are every column
// shard of their rows: one output, the same rows, equal widths W in column order covering [0, C) with
// S = C / W a power of two from 2 to 64, W a whole number of chunks, rows * C below 2^32, none
// exact-only, each shard below 2^32 bytes, and a kind planned that way (stk::split_kind).  *count = S.
bool split_desc(const st_index& ix, size_t j, const std::vector<Slice>& gs, const std::vector<st_desc>& descs,
                const st_slice* slices, size_t k, st_desc* d, uint64_t* units, size_t* count) {
    if (!kSplit) return false;
    const Slice& g0 = gs[j];
    const Output& o = ix.outputs[slices[j].output];
    if (!g0.strided() || g0.c0 != 0 || !stk::split_kind(o.kind)) return false;
    const uint64_t W = g0.cols(), C = g0.C;
    if (W == 0 || C % W) return false;
    const uint64_t S = C / W;
    if (S < 2 || S > 64 || (S & (S - 1)) || j + S > k) return false;
    if (W % stk::chunk_elems(o.kind) || W % 4 || g0.rows() * C >= (uint64_t(1) << 32) ||
        g0.rows() * W * sti::out_bytes(ix) >= (uint64_t(1) << 32))  // a shard's byte offsets are 32-bit
        return false;
    for (size_t i = 0; i < S; ++i) {
        const Slice& g = gs[j + i];
        if (slices[j + i].output != slices[j].output || g.r0 != g0.r0 || g.r1 != g0.r1 || g.c0 != i * W ||
            g.cols() != W || (descs[j + i].flags & ST_DESC_EXACT))
            return false;
    }
    Slice whole = g0;   // the same rows, every column: a contiguous source
    whole.c0 = 0;
    whole.c1 = C;
    *d = make_slice_desc(ix, o, whole, uint32_t(j), 0, units);
    d->flags = ST_DESC_SPLIT;
    d->pitch = uint32_t(C);
    d->cols = uint32_t(W);
    d->grid_cols = stk::ilog2(uint32_t(S));
    d->div_magic = stk::div_magic(uint32_t(W));
    d->meta = (d->meta & 0xFF00FFFFu) | stk::div_shift(uint32_t(W)) << 16;
    *count = size_t(S);
    return true;
}

std::vector<st_desc> interleave_column_slices(const st_index& ix, const std::vector<st_desc>& descs,
                                              const std::vector<uint64_t>& nu, const std::vector<Slice>& gs,
                                              const st_slice* slices, uint64_t* total) {
    const size_t k = descs.size();
    // complete shard sets first: split descriptors, placed where their first shard is
    std::vector<st_desc> split(k);
    std::vector<uint64_t> split_units(k, 0);
    std::vector<size_t> split_count(k, 0);
    std::vector<bool> in_split(k, false);
    for (size_t j = 0; j < k; ++j) {
        size_t S = 0;
        if (!in_split[j] && split_desc(ix, j, gs, descs, slices, k, &split[j], &split_units[j], &S)) {
            split_count[j] = S;
            for (size_t i = j; i < j + S; ++i) in_split[i] = true;
        }
    }
    // sibling groups of the remaining packed-fp4 column slices
    std::vector<int64_t> group(k, -1);   // first member of the slice's sibling group
    std::map<std::tuple<uint32_t, uint64_t, uint64_t>, size_t> first;
    std::vector<size_t> members(k, 0);
    for (size_t j = 0; j < k; ++j) {
        if (in_split[j] || !gs[j].strided() || (descs[j].flags & ST_DESC_EXACT) || nu[j] == 0) continue;
        if (!((kBandKinds >> (descs[j].meta & 0xFFu)) & 1u)) continue;
        auto key = std::make_tuple(slices[j].output, gs[j].r0, gs[j].r1);
        auto it = first.emplace(key, j).first;
        group[j] = int64_t(it->second);
        ++members[it->second];
    }
    std::vector<st_desc> out;
    out.reserve(k);
    uint64_t pos = 0;
    auto place = [&](size_t j, uint64_t a, uint64_t count) {
        st_desc d = descs[j];
        const uint32_t shift = (d.meta >> 8) & 0xFFu;
        d.unit_begin = uint32_t(pos - a);  // modulo 2^32, as the kernel subtracts
        d.unit_end = uint32_t(pos + count);
        if (a + count != nu[j]) d.tail = uint32_t(1) << shift;  // not the slice's last unit
        out.push_back(d);
        pos += count;
    };
    std::vector<bool> done(k, false);
    for (size_t j = 0; j < k; ++j) {
        if (done[j]) continue;
        if (split_count[j]) {
            st_desc d = split[j];
            d.unit_begin = uint32_t(pos);
            d.unit_end = uint32_t(pos + split_units[j]);
            out.push_back(d);
            pos += split_units[j];
            for (size_t i = j; i < j + split_count[j]; ++i) done[i] = true;
            continue;
        }
        if (group[j] < 0 || members[size_t(group[j])] < 2) {
            place(j, 0, nu[j]);
            done[j] = true;
            continue;
        }
        std::vector<size_t> sib;
        for (size_t i = j; i < k; ++i)
            if (group[i] == group[j] && !done[i]) sib.push_back(i);
        uint64_t most = 0;
        for (size_t i : sib) most = std::max(most, nu[i]);
        for (uint64_t a = 0; a < most; a += kBandUnits)
            for (size_t i : sib)
                if (a < nu[i]) place(i, a, std::min(kBandUnits, nu[i] - a));
        for (size_t i : sib) done[i] = true;
    }
    *total = pos;
    return out;
}

// The XCD balance of build_table, for slice tables: when the request-order eighths of the units
// differ by more than kImbalance in bytes (a bf16 embedding's row shards among fp8 ones, say), every
// descriptor of at least kSlicePieceMinUnits units is cut into 8 pieces, piece p placed in the p-th
// eighth, and the smaller descriptors fill the eighths in order.  Slices are cut only when their
// pieces stay large (2048 units or more): cutting every 2048-unit shard of the block-FP8 checkpoint
// into 256-unit pieces made one rank's column shard 7% slower (measured on MI355X), the XCDs then
// jumping between tensors every megabyte.  A piece keeps its descriptor's
// fields (column slice, split or exact-only alike) with its unit range re-based: the kernel's unit
// offset (unit - unit_begin) still lands on the piece's first unit of the slice, and only the piece
// holding the descriptor's last unit keeps its tail.
constexpr uint64_t kSlicePieceMinUnits = 8 * 2048;

std::vector<st_desc> balance_eighths(const st_index& ix, const std::vector<st_desc>& in, uint64_t total) {
    if (total < kSlots) return in;
    const size_t n = in.size();
    std::vector<uint64_t> at(n), cnt(n);
    double eighth[kSlots] = {0}, sum = 0;
    uint64_t pos = 0;
    for (size_t i = 0; i < n; ++i) {
        const st_desc& d = in[i];
        at[i] = pos;
        cnt[i] = uint64_t(d.unit_end) - pos;
        const uint32_t kind = d.meta & 0xFFu, shift = (d.meta >> 8) & 0xFFu;
        const double per_unit = double(uint64_t(1) << shift) * (double(stk::source_bits(kind)) / 8.0 + double(sti::out_bytes(ix)));
        sum += per_unit * double(cnt[i]);
        uint64_t u = pos;
        const uint64_t end = pos + cnt[i];
        while (u < end) {  // spread the descriptor over the eighths its units fall in
            const uint32_t x = uint32_t(std::min<uint64_t>(kSlots - 1, u * kSlots / total));
            const uint64_t xe = x + 1 == kSlots ? end : std::min<uint64_t>(end, (uint64_t(x) + 1) * total / kSlots);
            const uint64_t stop = std::max<uint64_t>(xe, u + 1);
            eighth[x] += per_unit * double(stop - u);
            u = stop;
        }
        pos = end;
    }
    double mx = 0;
    for (double e : eighth) mx = std::max(mx, e);
    if (sum <= 0 || mx / (sum / kSlots) <= kImbalance) return in;
    uint64_t small = 0;
    for (size_t i = 0; i < n; ++i)
        if (cnt[i] < kSlicePieceMinUnits) small += cnt[i];
    struct Piece {
        size_t i;
        uint64_t first, count;  // units of the descriptor
    };
    std::vector<std::vector<Piece>> slot(kSlots);
    uint64_t filled = 0;
    for (size_t i = 0; i < n; ++i) {
        if (cnt[i] >= kSlicePieceMinUnits) {
            for (uint32_t p = 0; p < kSlots; ++p) {
                const uint64_t a = cnt[i] * p / kSlots, e = cnt[i] * (p + 1) / kSlots;
                slot[p].push_back({i, a, e - a});
            }
        } else {
            const uint64_t s = small ? std::min<uint64_t>(kSlots - 1, filled * kSlots / small) : 0;
            slot[s].push_back({i, 0, cnt[i]});
            filled += cnt[i];
        }
    }
    std::vector<st_desc> out;
    out.reserve(n + 8 * n);
    uint64_t q = 0;
    for (const auto& sl : slot)
        for (const Piece& pc : sl) {
            st_desc d = in[pc.i];
            const uint32_t shift = (d.meta >> 8) & 0xFFu;
            const uint32_t first_in_slice = uint32_t(at[pc.i] - d.unit_begin) + uint32_t(pc.first);  // modulo 2^32
            d.unit_begin = uint32_t(q) - first_in_slice;
            d.unit_end = uint32_t(q + pc.count);
            if (pc.first + pc.count != cnt[pc.i]) d.tail = uint32_t(1) << shift;  // not the descriptor's last unit
            out.push_back(d);
            q += pc.count;
        }
    return out;
}

}  // namespace

namespace {

st_status plan(st_index& ix) {
    if (ix.outputs.size() >= (uint64_t(1) << 32)) return st_fail(ST_E_SHAPE, "more than 2^32 outputs");
    uint64_t pos = 0;
    ix.out_offset.resize(ix.outputs.size());
    for (size_t k = 0; k < ix.outputs.size(); ++k) {
        ix.out_offset[k] = pos;
        pos = round_up(pos + ix.outputs[k].numel * sti::out_bytes(ix), 256);
    }
    ix.arena_bytes = pos;
    std::vector<uint32_t> all(ix.outputs.size());
    for (size_t k = 0; k < all.size(); ++k) all[k] = uint32_t(k);
    try {
        ix.table = sti::build_table(ix, all.data(), all.size(), &ix.total_units);
    } catch (const std::length_error& e) {
        return st_fail(ST_E_SHAPE, "checkpoint too large for one work table: %s", e.what());
    }
    return ST_OK;
}

}  // namespace

// ---------------------------------------------------------------------------------- C ABI

extern "C" st_status st_header_size(const void* first8, uint64_t* header_bytes) {
    st_clear();
    if (!first8 || !header_bytes) return st_fail(ST_E_ARG, "st_header_size: null pointer");
    uint64_t n = 0;
    const unsigned char* p = (const unsigned char*)first8;
    for (int k = 7; k >= 0; --k) n = (n << 8) | p[k];
    if (n > ST_HEADER_CAP)
        return st_fail(ST_E_HEADER, "header length %llu exceeds the cap %llu", (unsigned long long)n, ST_HEADER_CAP);
    *header_bytes = 8 + n;
    return ST_OK;
}

extern "C" st_status st_index_build(const void* header_bytes, uint64_t header_len, uint64_t file_size,
                                    const st_plan_opts* opts, st_index** out) {
    st_clear();
    if (!out) return st_fail(ST_E_ARG, "st_index_build: out is null");
    *out = nullptr;
    if (!header_bytes && header_len) return st_fail(ST_E_ARG, "st_index_build: header_bytes is null");
    if (opts && ((opts->flags & ~3u) != 0 || (opts->flags & 3u) > ST_OUT_F32 || opts->unit_log2_scale > 6))
        return st_fail(ST_E_ARG,
                       "st_plan_opts: flags hold only an output type (0..2) and unit_log2_scale is at most 6 (got 0x%x, %u)",
                       opts->flags, opts->unit_log2_scale);
    if (header_len < 8 || file_size < 8)
        return st_fail(ST_E_HEADER, "file shorter than the 8-byte header length (%llu bytes)",
                       (unsigned long long)std::min(header_len, file_size));
    uint64_t hb;
    if (st_status r = st_header_size(header_bytes, &hb)) return r;
    uint64_t n = hb - 8;
    if (hb > file_size)
        return st_fail(ST_E_HEADER, "header length %llu runs past the end of the file (%llu bytes)", (unsigned long long)n,
                       (unsigned long long)file_size);
    if (hb > header_len)
        return st_fail(ST_E_ARG, "st_index_build: %llu header bytes given, the header needs %llu",
                       (unsigned long long)header_len, (unsigned long long)hb);
    const char* text = (const char*)header_bytes + 8;
    if (!valid_utf8((const unsigned char*)text, n)) return st_fail(ST_E_HEADER, "header is not UTF-8");
    std::unique_ptr<st_index> ix(new (std::nothrow) st_index);
    if (!ix) return st_fail(ST_E_NOMEM, "out of host memory");
    ix->header_len = n;
    ix->data_size = file_size - hb;
    ix->unit_log2_scale = opts ? opts->unit_log2_scale : 0;
    ix->out_dtype = opts ? (opts->flags & 3u) : uint32_t(ST_OUT_BF16);
    try {
        JVal root;
        if (st_status r = JsonReader(text, n).parse(root)) return r;
        if (st_status r = parse_entries(*ix, root)) return r;
        if (st_status r = check_layout(*ix)) return r;
        if (st_status r = classify(*ix)) return r;
        if (st_status r = plan(*ix)) return r;
    } catch (const std::bad_alloc&) {
        return st_fail(ST_E_NOMEM, "out of host memory while indexing the header");
    }
    *out = ix.release();
    return ST_OK;
}

extern "C" st_status st_index_open(const char* path, const st_plan_opts* opts, st_index** out) {
    st_clear();
    if (!out) return st_fail(ST_E_ARG, "st_index_open: out is null");
    *out = nullptr;
    if (!path) return st_fail(ST_E_ARG, "st_index_open: path is null");
    int fd = open(path, O_RDONLY | O_CLOEXEC);
    if (fd < 0) return st_fail(ST_E_IO, "cannot open %s", path);
    struct stat sb;
    if (fstat(fd, &sb) != 0) { close(fd); return st_fail(ST_E_IO, "cannot stat %s", path); }
    uint64_t size = uint64_t(sb.st_size);
    unsigned char first[8];
    if (size < 8 || pread(fd, first, 8, 0) != 8) {
        close(fd);
        return st_fail(ST_E_HEADER, "file shorter than the 8-byte header length (%llu bytes)", (unsigned long long)size);
    }
    uint64_t hb;
    if (st_status r = st_header_size(first, &hb)) { close(fd); return r; }
    if (hb > size) {
        close(fd);
        return st_fail(ST_E_HEADER, "header length %llu runs past the end of the file (%llu bytes)",
                       (unsigned long long)(hb - 8), (unsigned long long)size);
    }
    std::vector<char> buf;
    try { buf.resize(hb); } catch (const std::bad_alloc&) { close(fd); return st_fail(ST_E_NOMEM, "out of host memory"); }
    uint64_t got = 0;
    while (got < hb) {
        ssize_t r = pread(fd, buf.data() + got, hb - got, off_t(got));
        if (r <= 0) { close(fd); return st_fail(ST_E_IO, "read of %s header failed", path); }
        got += uint64_t(r);
    }
    close(fd);
    return st_index_build(buf.data(), hb, size, opts, out);
}

extern "C" void st_index_free(st_index* idx) { delete idx; }

extern "C" uint64_t st_index_data_offset(const st_index* idx) { return idx ? 8 + idx->header_len : 0; }
extern "C" uint64_t st_index_data_size(const st_index* idx) { return idx ? idx->data_size : 0; }
extern "C" uint64_t st_index_blob_bytes(const st_index* idx) { return idx ? round_up(idx->data_size + 64, 256) : 0; }
extern "C" size_t st_index_count(const st_index* idx) { return idx ? idx->tensors.size() : 0; }

extern "C" st_status st_index_tensor(const st_index* idx, size_t i, st_tensor_meta* out) {
    st_clear();
    if (!idx || !out) return st_fail(ST_E_ARG, "st_index_tensor: null pointer");
    if (i >= idx->tensors.size()) return st_fail(ST_E_ARG, "st_index_tensor: index %zu out of range (%zu)", i, idx->tensors.size());
    const Tensor& t = idx->tensors[i];
    memset(out, 0, sizeof *out);
    out->name = t.name.c_str();
    out->dtype = t.dtype;
    out->ndim = int32_t(t.shape.size());
    for (size_t d = 0; d < t.shape.size(); ++d) out->shape[d] = t.shape[d];
    out->begin = t.begin;
    out->end = t.end;
    return ST_OK;
}

extern "C" int64_t st_index_find(const st_index* idx, const char* name) {
    if (!idx || !name) return -1;
    int64_t i = -1;
    return find(*idx, name, &i) ? i : -1;
}

extern "C" const char* st_index_metadata_json(const st_index* idx) { return idx ? idx->metadata_json.c_str() : "{}"; }

extern "C" size_t st_index_num_outputs(const st_index* idx) { return idx ? idx->outputs.size() : 0; }

extern "C" st_status st_index_output(const st_index* idx, size_t k, st_output_info* out) {
    st_clear();
    if (!idx || !out) return st_fail(ST_E_ARG, "st_index_output: null pointer");
    if (k >= idx->outputs.size()) return st_fail(ST_E_ARG, "st_index_output: index %zu out of range (%zu)", k, idx->outputs.size());
    const Output& o = idx->outputs[k];
    memset(out, 0, sizeof *out);
    out->name = idx->tensors[o.tensor].name.c_str();
    out->kind = o.kind;
    out->ndim = int32_t(o.shape.size());
    for (size_t d = 0; d < o.shape.size(); ++d) out->shape[d] = o.shape[d];
    out->numel = o.numel;
    out->tensor = o.tensor;
    out->scale = o.scale;
    out->scale2 = o.scale2;
    return ST_OK;
}

extern "C" uint64_t st_index_output_offset(const st_index* idx, size_t k) {
    return idx && k < idx->out_offset.size() ? idx->out_offset[k] : 0;
}
extern "C" uint64_t st_index_output_arena_bytes(const st_index* idx) { return idx ? std::max<uint64_t>(256, idx->arena_bytes) : 0; }

extern "C" uint64_t st_index_traffic_bytes(const st_index* idx) {
    if (!idx) return 0;
    uint64_t w = 0;
    for (const Output& o : idx->outputs) w += o.numel * sti::out_bytes(*idx);
    return idx->data_size + w;
}

extern "C" uint64_t st_index_device_bytes(const st_index* idx) {
    if (!idx) return 0;
    uint64_t n = idx->outputs.size();
    return st_index_blob_bytes(idx) + round_up(idx->table.size(), 256) + round_up(n * sizeof(void*), 256) +
           st_index_output_arena_bytes(idx);
}

extern "C" const void* st_index_table(const st_index* idx, size_t* bytes, uint64_t* units) {
    if (!idx) return nullptr;
    if (bytes) *bytes = idx->table.size();
    if (units) *units = idx->total_units;
    return idx->table.data();
}

extern "C" const void* st_index_descs(const st_index* idx, size_t* n, size_t* bytes) {
    uint64_t units = 0;
    const void* t = st_index_table(idx, bytes, &units);
    if (n) *n = t ? size_t(units) : 0;
    return t;
}

extern "C" st_status st_index_table_subset(const st_index* idx, const uint32_t* sel, size_t k, void* dst,
                                           size_t dst_bytes, size_t* bytes, uint64_t* units) {
    st_clear();
    if (!idx || (k && !sel)) return st_fail(ST_E_ARG, "st_index_table_subset: null pointer");
    for (size_t j = 0; j < k; ++j)
        if (sel[j] >= idx->outputs.size())
            return st_fail(ST_E_ARG, "st_index_table_subset: output %u out of range (%zu)", sel[j], idx->outputs.size());
    uint64_t u = 0;
    std::vector<unsigned char> t;
    try {
        t = sti::build_table(*idx, sel, k, &u);
    } catch (const std::bad_alloc&) {
        return st_fail(ST_E_NOMEM, "out of host memory");
    } catch (const std::length_error& e) {
        return st_fail(ST_E_SHAPE, "st_index_table_subset: %s", e.what());
    }
    if (bytes) *bytes = t.size();
    if (units) *units = u;
    if (!dst) return ST_OK;
    if (dst_bytes < t.size())
        return st_fail(ST_E_ARG, "st_index_table_subset: dst holds %zu bytes, %zu needed", dst_bytes, t.size());
    memcpy(dst, t.data(), t.size());
    return ST_OK;
}

extern "C" st_status st_index_slice_numel(const st_index* idx, const st_slice* s, uint64_t* rows, uint64_t* cols) {
    st_clear();
    if (!idx || !s) return st_fail(ST_E_ARG, "st_index_slice_numel: null pointer");
    Slice g;
    st_status r = resolve_slice(*idx, *s, g);
    if (r != ST_OK) return r;
    if (rows) *rows = g.rows();
    if (cols) *cols = g.cols();
    return ST_OK;
}

extern "C" st_status st_index_table_slices(const st_index* idx, const st_slice* slices, size_t k, void* dst,
                                           size_t dst_bytes, size_t* bytes, uint64_t* units) {
    st_clear();
    if (!idx || (k && !slices)) return st_fail(ST_E_ARG, "st_index_table_slices: null pointer");
    std::vector<unsigned char> t;
    uint64_t pos = 0;
    try {
        std::vector<st_desc> descs(k);
        std::vector<uint64_t> nu(k);
        std::vector<Slice> gs(k);
        for (size_t j = 0; j < k; ++j) {
            st_status r = resolve_slice(*idx, slices[j], gs[j]);
            if (r != ST_OK) return r;
            descs[j] = make_slice_desc(*idx, idx->outputs[slices[j].output], gs[j], uint32_t(j), 0, &nu[j]);
            pos += nu[j];
            if (pos >= (uint64_t(1) << 32)) return st_fail(ST_E_SHAPE, "st_index_table_slices: 2^32 or more work units");
        }
        uint64_t out_bytes = 0;
        for (size_t j = 0; j < k; ++j) out_bytes += gs[j].rows() * gs[j].cols() * sti::out_bytes(*idx);
        descs = interleave_column_slices(*idx, descs, nu, gs, slices, &pos);
        descs = balance_eighths(*idx, descs, pos);
        t = assemble(descs, pos, idx->out_dtype, out_bytes);
    } catch (const std::bad_alloc&) {
        return st_fail(ST_E_NOMEM, "out of host memory");
    } catch (const std::length_error& e) {
        return st_fail(ST_E_SHAPE, "st_index_table_slices: %s", e.what());
    }
    if (bytes) *bytes = t.size();
    if (units) *units = pos;
    if (!dst) return ST_OK;
    if (dst_bytes < t.size())
        return st_fail(ST_E_ARG, "st_index_table_slices: dst holds %zu bytes, %zu needed", dst_bytes, t.size());
    memcpy(dst, t.data(), t.size());
    return ST_OK;
}

extern "C" uint32_t st_index_out_dtype(const st_index* idx) { return idx ? idx->out_dtype : uint32_t(ST_OUT_BF16); }
