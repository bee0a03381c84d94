// Minimal JSON reader/writer (objects, arrays, numbers, strings, true/false/null).
#include "nf_json.h"

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <sstream>

namespace nf {
namespace json {

static const Value kNull;

const Value& Value::at(const std::string& k) const {
  if (kind != Obj) return kNull;
  auto it = obj.find(k);
  return it == obj.end() ? kNull : it->second;
}

namespace {

struct Parser {
  const std::string& s;
  size_t i = 0;
  std::string err;
  explicit Parser(const std::string& t) : s(t) {}

  void ws() {
    while (i < s.size() && (s[i] == ' ' || s[i] == '\n' || s[i] == '\t' || s[i] == '\r')) ++i;
  }
  bool fail(const char* m) {
    if (err.empty()) err = std::string(m) + " at offset " + std::to_string(i);
    return false;
  }
  bool lit(const char* w) {
    const size_t n = strlen(w);
    if (s.compare(i, n, w) != 0) return false;
    i += n;
    return true;
  }
  bool string(std::string& out) {
    if (i >= s.size() || s[i] != '"') return fail("expected string");
    ++i;
    out.clear();
    while (i < s.size() && s[i] != '"') {
      char c = s[i++];
      if (c == '\\') {
        if (i >= s.size()) return fail("bad escape");
        char e = s[i++];
        switch (e) {
          case 'n': out += '\n'; break;
          case 't': out += '\t'; break;
          case 'r': out += '\r'; break;
          case 'b': out += '\b'; break;
          case 'f': out += '\f'; break;
          case 'u': {
            if (i + 4 > s.size()) return fail("bad \\u escape");
            const unsigned cp = (unsigned)strtoul(s.substr(i, 4).c_str(), nullptr, 16);
            i += 4;
            out += cp < 0x80 ? (char)cp : '?';
            break;
          }
          default: out += e;
        }
      } else {
        out += c;
      }
    }
    if (i >= s.size()) return fail("unterminated string");
    ++i;
    return true;
  }
  bool value(Value& v, int depth) {
    if (depth > 64) return fail("nesting too deep");
    ws();
    if (i >= s.size()) return fail("unexpected end");
    const char c = s[i];
    if (c == '{') {
      v.kind = Value::Obj;
      ++i;
      ws();
      if (i < s.size() && s[i] == '}') {
        ++i;
        return true;
      }
      while (true) {
        ws();
        std::string k;
        if (!string(k)) return false;
        ws();
        if (i >= s.size() || s[i] != ':') return fail("expected ':'");
        ++i;
        if (!value(v.obj[k], depth + 1)) return false;
        ws();
        if (i < s.size() && s[i] == ',') {
          ++i;
          continue;
        }
        if (i < s.size() && s[i] == '}') {
          ++i;
          return true;
        }
        return fail("expected ',' or '}'");
      }
    }
    if (c == '[') {
      v.kind = Value::Arr;
      ++i;
      ws();
      if (i < s.size() && s[i] == ']') {
        ++i;
        return true;
      }
      while (true) {
        v.arr.emplace_back();
        if (!value(v.arr.back(), depth + 1)) return false;
        ws();
        if (i < s.size() && s[i] == ',') {
          ++i;
          continue;
        }
        if (i < s.size() && s[i] == ']') {
          ++i;
          return true;
        }
        return fail("expected ',' or ']'");
      }
    }
    if (c == '"') {
      v.kind = Value::Str;
      return string(v.str);
    }
    if (lit("true")) {
      v.kind = Value::Bool;
      v.b = true;
      return true;
    }
    if (lit("false")) {
      v.kind = Value::Bool;
      v.b = false;
      return true;
    }
    if (lit("null")) {
      v.kind = Value::Null;
      return true;
    }
    char* end = nullptr;
    const double d = strtod(s.c_str() + i, &end);
    if (end == s.c_str() + i) return fail("bad value");
    i = end - s.c_str();
    v.kind = Value::Num;
    v.num = d;
    return true;
  }
};

}  // namespace

bool parse(const std::string& text, Value& out, std::string& err) {
  Parser p(text);
  out = Value();
  if (!p.value(out, 0)) {
    err = p.err;
    return false;
  }
  p.ws();
  if (p.i != text.size()) {
    err = "trailing characters after JSON value";
    return false;
  }
  return true;
}

bool parse_file(const char* path, Value& out, std::string& err) {
  std::ifstream f(path);
  if (!f) {
    err = std::string("cannot open ") + path;
    return false;
  }
  std::stringstream ss;
  ss << f.rdbuf();
  return parse(ss.str(), out, err);
}

std::string quote(const std::string& s) {
  std::string o = "\"";
  for (char c : s) {
    if (c == '"' || c == '\\') {
      o += '\\';
      o += c;
    } else if (c == '\n') {
      o += "\\n";
    } else {
      o += c;
    }
  }
  return o + "\"";
}

std::string num(double v) {
  if (!std::isfinite(v)) return "null";
  char buf[64];
  snprintf(buf, sizeof buf, "%.12g", v);
  return buf;
}

}  // namespace json
}  // namespace nf
