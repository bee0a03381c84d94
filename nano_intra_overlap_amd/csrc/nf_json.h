// Minimal JSON reader/writer for the profile tables and plans (host only).
#pragma once

#include <cstdio>
#include <map>
#include <memory>
#include <string>
#include <vector>

namespace nf {
namespace json {

struct Value {
  enum Kind { Null, Bool, Num, Str, Arr, Obj } kind = Null;
  bool b = false;
  double num = 0.0;
  std::string str;
  std::vector<Value> arr;
  std::map<std::string, Value> obj;

  bool is_obj() const { return kind == Obj; }
  bool is_arr() const { return kind == Arr; }
  bool is_num() const { return kind == Num; }
  bool has(const std::string& k) const { return kind == Obj && obj.count(k); }
  const Value& at(const std::string& k) const;
  double number(const std::string& k, double def) const {
    return has(k) && obj.at(k).is_num() ? obj.at(k).num : def;
  }
};

// Parse text; on error returns false and sets err.
bool parse(const std::string& text, Value& out, std::string& err);
bool parse_file(const char* path, Value& out, std::string& err);

// Writer helpers
std::string quote(const std::string& s);
std::string num(double v);

}  // namespace json
}  // namespace nf
