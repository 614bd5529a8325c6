// table.cpp -- table file parsing, identity checks, refusals and defaults.
// Host-only C++ (no HIP calls).
#include "table.hpp"

#include <cctype>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <initializer_list>
#include <sstream>

#include "variants.hpp"

namespace skg {

// ------------------------------------------------------------ a small JSON
// reader: objects, arrays, strings (with simple escapes), numbers, literals.
namespace {

struct JVal {
  enum Kind { NUL, BOOL, NUM, STR, ARR, OBJ } kind = NUL;
  bool b = false;
  double num = 0;
  std::string str;
  std::vector<JVal> arr;
  std::vector<std::pair<std::string, JVal>> obj;
  const JVal* get(const char* key) const {
    if (kind != OBJ) return nullptr;
    for (const auto& kv : obj)
      if (kv.first == key) return &kv.second;
    return nullptr;
  }
};

class JParser {
 public:
  explicit JParser(const std::string& s) : s_(s) {}
  bool parse(JVal* out, std::string* err) {
    if (!value(out, 0)) {
      *err = "malformed JSON near byte " + std::to_string(pos_);
      return false;
    }
    ws();
    if (pos_ != s_.size()) {
      *err = "trailing bytes after JSON value at byte " + std::to_string(pos_);
      return false;
    }
    return true;
  }

 private:
  const std::string& s_;
  size_t pos_ = 0;
  void ws() {
    while (pos_ < s_.size() && std::isspace(static_cast<unsigned char>(s_[pos_]))) ++pos_;
  }
  bool lit(const char* t) {
    const size_t n = std::strlen(t);
    if (s_.compare(pos_, n, t) != 0) return false;
    pos_ += n;
    return true;
  }
  bool string(std::string* out) {
    if (pos_ >= s_.size() || s_[pos_] != '"') return false;
    ++pos_;
    while (pos_ < s_.size() && s_[pos_] != '"') {
      char c = s_[pos_++];
      if (c == '\\') {
        if (pos_ >= s_.size()) return false;
        const char e = s_[pos_++];
        switch (e) {
          case '"': c = '"'; break;
          case '\\': c = '\\'; break;
          case '/': c = '/'; break;
          case 'n': c = '\n'; break;
          case 't': c = '\t'; break;
          case 'r': c = '\r'; break;
          case 'b': c = '\b'; break;
          case 'f': c = '\f'; break;
          case 'u': {  // keep ASCII only; others become '?'
            if (pos_ + 4 > s_.size()) return false;
            const unsigned long cp = std::strtoul(s_.substr(pos_, 4).c_str(), nullptr, 16);
            pos_ += 4;
            c = cp < 128 ? static_cast<char>(cp) : '?';
            break;
          }
          default: return false;
        }
      }
      out->push_back(c);
    }
    if (pos_ >= s_.size()) return false;
    ++pos_;
    return true;
  }
  bool value(JVal* v, int depth) {
    if (depth > 64) return false;
    ws();
    if (pos_ >= s_.size()) return false;
    const char c = s_[pos_];
    if (c == '{') {
      v->kind = JVal::OBJ;
      ++pos_;
      ws();
      if (pos_ < s_.size() && s_[pos_] == '}') { ++pos_; return true; }
      for (;;) {
        ws();
        std::string key;
        if (!string(&key)) return false;
        ws();
        if (pos_ >= s_.size() || s_[pos_] != ':') return false;
        ++pos_;
        JVal child;
        if (!value(&child, depth + 1)) return false;
        v->obj.emplace_back(std::move(key), std::move(child));
        ws();
        if (pos_ < s_.size() && s_[pos_] == ',') { ++pos_; continue; }
        if (pos_ < s_.size() && s_[pos_] == '}') { ++pos_; return true; }
        return false;
      }
    }
    if (c == '[') {
      v->kind = JVal::ARR;
      ++pos_;
      ws();
      if (pos_ < s_.size() && s_[pos_] == ']') { ++pos_; return true; }
      for (;;) {
        JVal child;
        if (!value(&child, depth + 1)) return false;
        v->arr.push_back(std::move(child));
        ws();
        if (pos_ < s_.size() && s_[pos_] == ',') { ++pos_; continue; }
        if (pos_ < s_.size() && s_[pos_] == ']') { ++pos_; return true; }
        return false;
      }
    }
    if (c == '"') { v->kind = JVal::STR; return string(&v->str); }
    if (lit("true")) { v->kind = JVal::BOOL; v->b = true; return true; }
    if (lit("false")) { v->kind = JVal::BOOL; v->b = false; return true; }
    if (lit("null")) { v->kind = JVal::NUL; return true; }
    if (c == '-' || std::isdigit(static_cast<unsigned char>(c))) {
      const char* start = s_.c_str() + pos_;
      char* end = nullptr;
      v->num = std::strtod(start, &end);
      if (end == start) return false;
      v->kind = JVal::NUM;
      pos_ += static_cast<size_t>(end - start);
      return true;
    }
    return false;
  }
};

bool as_int(const JVal* v, int* out) {
  if (!v || v->kind != JVal::NUM) return false;
  const double d = v->num;
  if (d < -2147483648.0 || d > 2147483647.0 || static_cast<double>(static_cast<int>(d)) != d) return false;
  *out = static_cast<int>(d);
  return true;
}

}  // namespace

// ------------------------------------------------------------------ identity
std::string Identity::str() const {
  return "arch=" + arch + ";hip=" + hip + ";cc=" + cc + ";space=" + space;
}

bool Identity::parse(const std::string& s, Identity* out) {
  Identity id;
  std::stringstream ss(s);
  std::string item;
  int seen = 0;
  while (std::getline(ss, item, ';')) {
    const size_t eq = item.find('=');
    if (eq == std::string::npos) return false;
    const std::string k = item.substr(0, eq), v = item.substr(eq + 1);
    if (k == "arch") { id.arch = v; seen |= 1; }
    else if (k == "hip") { id.hip = v; seen |= 2; }
    else if (k == "cc") { id.cc = v; seen |= 4; }
    else if (k == "space") { id.space = v; seen |= 8; }
    else return false;
  }
  if (seen != 15) return false;
  *out = id;
  return true;
}

// ----------------------------------------------------------------- names
const char* op_name(int op) {
  switch (op) {
    case OP_BF16: return "bf16";
    case OP_GATED: return "gated";
    case OP_FP8T: return "fp8_tensor";
    case OP_A8W8: return "a8w8_block";
    case OP_A8W8Q: return "a8w8_quant";
    case OP_PACKED + OP_BF16: return "bf16_packed";
    case OP_PACKED + OP_GATED: return "gated_packed";
    case OP_PACKED + OP_FP8T: return "fp8_tensor_packed";
    case OP_PACKED + OP_A8W8: return "a8w8_block_packed";
    case OP_PACKED + OP_A8W8Q: return "a8w8_quant_packed";
    default: return nullptr;
  }
}
int op_from_name(const std::string& s) {
  for (int op = 0; op < NUM_OPS; ++op)
    if (s == op_name(op)) return op;
  return -1;
}
int variant_from_name(const std::string& s) {
  for (int i = 0; i < kNumVariants; ++i)
    if (s == kVariants[i].name) return i;
  return -1;
}

int forced_variant() {
  const char* f = std::getenv("SKINNY_GEMM_FORCE");
  if (!f || !*f) return -1;
  return variant_from_name(f);
}

// ------------------------------------------------------------------ table
void Table::clear() {
  map_.clear();
  engaged_ = false;
  status_ = "none";
}

int Table::lookup(int op, int bucket, int N, int K) const {
  if (!engaged_) return -1;
  const auto it = map_.find(std::make_tuple(op, bucket, N, K));
  return it == map_.end() ? -1 : it->second;
}

int Table::load(const std::string& path, const Identity& self, std::string* err) {
  clear();
  std::ifstream f(path, std::ios::binary);
  if (!f) {
    *err = "cannot read table " + path;
    status_ = "none (" + *err + ")";
    return -1;
  }
  std::stringstream buf;
  buf << f.rdbuf();
  const std::string text = buf.str();
  JVal root;
  if (!JParser(text).parse(&root, err) || root.kind != JVal::OBJ) {
    if (err->empty()) *err = "table is not a JSON object";
    *err = path + ": " + *err;
    status_ = "none (" + *err + ")";
    return -1;
  }
  auto refuse = [&](const std::string& why) {
    status_ = "refused " + path + ": " + why;
    std::fprintf(stderr, "skinny_gemm: table %s refused: %s; built-in defaults stay in effect\n",
                 path.c_str(), why.c_str());
    return 0;
  };

  const JVal* id = root.get("identity");
  if (!id || id->kind != JVal::OBJ) return refuse("no identity header");
  auto field = [&](const char* k) -> std::string {
    const JVal* v = id->get(k);
    return (v && v->kind == JVal::STR) ? v->str : std::string();
  };
  const std::string t_arch = field("arch"), t_hip = field("hip"), t_cc = field("cc"), t_space = field("space");
  if (t_space.empty())
    return refuse("its identity has no selection-space token, so it predates the current kernel list: "
                  "re-tune for this build");
  if (t_space != self.space)
    return refuse("its selection-space token " + t_space + " differs from this build's " + self.space +
                  " (the kernel list changed): re-tune for this build");
  if (t_arch != self.arch) return refuse("made for " + t_arch + ", this device is " + self.arch);
  if (t_hip != self.hip)
    return refuse("tuned on HIP runtime " + t_hip + ", this process loaded " + self.hip +
                  ": tune and run with the same runtime");
  if (t_cc != self.cc) return refuse("built by compiler " + t_cc + ", this build is " + self.cc);
  if (const char* f = std::getenv("SKINNY_GEMM_FORCE"); f && *f)
    return refuse(std::string("SKINNY_GEMM_FORCE=") + f +
                  " reroutes the dispatch away from what the table measured");

  const JVal* entries = root.get("entries");
  if (!entries || entries->kind != JVal::ARR) return refuse("no entries list");
  std::map<std::tuple<int, int, int, int>, int> map;
  for (size_t i = 0; i < entries->arr.size(); ++i) {
    const JVal& e = entries->arr[i];
    const std::string where = "entry " + std::to_string(i);
    const JVal* opv = e.get("op");
    const JVal* ch = e.get("choice");
    int rows = 0, N = 0, K = 0;
    if (!opv || opv->kind != JVal::STR || !ch || ch->kind != JVal::STR || !as_int(e.get("rows"), &rows) ||
        !as_int(e.get("N"), &N) || !as_int(e.get("K"), &K))
      return refuse(where + " lacks op/rows/N/K/choice");
    const int op = op_from_name(opv->str);
    if (op < 0) return refuse(where + " names unknown op '" + opv->str + "'");
    if (bucket_of(rows) != rows) return refuse(where + ": rows " + std::to_string(rows) + " is not a rows bucket");
    if (N <= 0 || K <= 0) return refuse(where + ": N and K must be positive");
    const int v = variant_from_name(ch->str);
    if (v < 0) return refuse(where + " names variant '" + ch->str + "' that this build does not compile");
    if (!variant_supports(op, v, rows))
      return refuse(where + ": variant '" + ch->str + "' is not compiled for " + opv->str + " at rows " +
                    std::to_string(rows));
    const auto key = std::make_tuple(op, rows, N, K);
    if (map.count(key)) return refuse(where + " duplicates an earlier key");
    map[key] = v;
  }
  map_ = std::move(map);
  engaged_ = true;
  status_ = "engaged " + std::to_string(map_.size()) + " shapes from " + path + " (" + self.arch +
            ", runtime " + self.hip + ")";
  std::fprintf(stderr, "skinny_gemm: table engaged: %zu shapes from %s (%s, runtime %s)\n", map_.size(),
               path.c_str(), self.arch.c_str(), self.hip.c_str());
  return 0;
}

// --------------------------------------------------------------- defaults
// The untuned entry point: what runs with no table, and the incumbent a table
// entry has to beat.  A shape rule fitted to gfx950 measurements of the whole
// variant list over the decode shapes:
//  * x quantised in the call (A8W8 from bf16 x), row-major or packed weight:
//    the LDS tile with one K group per workgroup (quantisation runs in every
//    round of every workgroup) and K split S ways across workgroups: S = 8
//    up to 64 tiles of 64 weight rows, 4 up to 128, 2 up to 256, else 1;
//    from the rows-32 bucket eight-wave workgroups at S = 4, else two
//    fragments per wave at S = 2.
//  * other forms with a packed weight, by 16-row weight blocks: from 1024
//    blocks the LDS tile with one K group (x through LDS); from 384, up to
//    16 rows, eight waves of which four split K (direct x up to 4 rows from
//    512 blocks), then S = 2 or 1 tiles; at 256, direct x with K split over
//    4 waves up to 12 rows, then the LDS x tile (in-workgroup, then S = 2 or
//    4 splits); below, direct x up to 8 rows, then the in-workgroup split.
//  * A8W8 (row-major), rows up to 16: the LDS tile with one K group from
//    16384 weight rows, else eight waves (direct x up to 4 rows).
//  * rows 1..3, rows 4 unless the weight is fp8 or its rows are large, and
//    rows up to 6 when the weight is under 16 MiB: the VALU weight stream.
//    Two weight rows per wave for one row of x, four for more, eight for a
//    vocabulary-sized N (>= 65536) with more than one row of x; K split over
//    the 4 waves of a workgroup unless a weight row is under 2 KiB, where the
//    4 waves take different rows instead.
//  * rows 4..6 on weights of >= 16 MiB with rows of >= 8 KiB and >= 4096
//    rows: direct x, K split over eight waves.
//  * weights under 16 MiB above that: the LDS tile with 16 weight rows per
//    workgroup and K split over its 4 waves (no cross-workgroup combine),
//    direct x up to 64 rows.
//  * rows 6..16 where a weight row holds at least 4 KiB and the 16-row tiles
//    come in whole multiples of 256 (one or more per CU): the same.
//  * otherwise the LDS tile with K split S ways across workgroups, so that
//    the 64-row output tiles times S come to about 256 workgroups or more:
//    S = 4 up to 8192 weight rows (gate and up rows counted), 2 up to 16384,
//    else 1; at most 4 fragments of x rows per workgroup from the rows-64
//    bucket, and eight-wave workgroups from the rows-96 bucket.
// `allow_ws` false keeps to variants that need no split-K workspace.
namespace {

int first_supported(int op, int M, std::initializer_list<const char*> names) {
  for (const char* n : names) {
    const int v = variant_from_name(n);
    if (v >= 0 && variant_supports(op, v, M)) return v;
  }
  return -1;
}

int first_of_family(int op, int M, int fam) {
  for (int i = 0; i < kNumVariants; ++i)
    if (kVariants[i].family == fam && variant_supports(op, i, M)) return i;
  return -1;
}

int default_pick(int op, int M, int N, int K, bool allow_ws) {
  const int b = M > kMaxBucket ? kMaxBucket : bucket_of(M);
  const double wbytes = (double)N * K * op_w_bytes(op) * op_groups(op);
  const double wrows = (double)N * op_groups(op);
  const double rowb = (double)K * op_w_bytes(op);
  const double MiB = 1024.0 * 1024.0;
  const bool small_w = wbytes < 16 * MiB;
  const int bo = op_base(op);
  const bool pk = op_packed(op);
  // (x quantised in the kernel, or a packed weight: LDS tile family only)
  const bool gemv = !pk && bo != OP_A8W8Q && bo != OP_A8W8 &&
                    (b <= 3 || (b == 4 && bo != OP_FP8T && !(wrows >= 4096 && rowb >= 8192)) ||
                     (small_w && b <= 6));
  const double blocks = wrows / 16.0;   // 16-row weight blocks
  // S > 1 variants need the split-K workspace: without it, the same tile with S = 1
  auto ws_or = [&](const char* with_ws, const char* without) { return allow_ws ? with_ws : without; };
  int v = -1;
  if (pk && bo != OP_A8W8Q) {
    // packed weight (measured on gfx950): x through LDS with one K group when
    // blocks are plenty; eight-wave K split for few rows on mid-sized
    // weights; direct x for few rows on small ones
    const char* n = nullptr;
    if (blocks >= 1024) {
      n = b <= 16 ? "tlds_f1_s1_p4_m2" : "tlds_f1_s1_p4_m4";
    } else if (blocks >= 384) {
      n = (b <= 4 && blocks >= 512) ? "tlds_d_k4_f1_s1_p4_m2"
          : b <= 16                 ? "tlds_w8_k4_f1_s1_p4_m2"
          : b <= 32                 ? ws_or("tlds_f1_s2_p4_m2", "tlds_f1_s1_p4_m2")
          : b <= 64                 ? (blocks >= 512 ? "tlds_f1_s1_p4_m2" : ws_or("tlds_f1_s2_p4_m4", "tlds_f1_s1_p4_m4"))
          : b <= 96                 ? ws_or("tlds_w8_f1_s4_p4", "tlds_f1_s1_p4_m4")
                                    : ws_or("tlds_w8_f1_s2_p4_m4", "tlds_f1_s1_p4_m4");
    } else if (blocks >= 256) {
      n = b <= 12   ? "tlds_d_k4_f1_s1_p4_m1"
          : b <= 16 ? "tlds_k4_f1_s1_p4_m1"
          : b <= 32 ? ws_or("tlds_k2_f1_s2_p4_m2", "tlds_k4_f1_s1_p4_m2")
          : b <= 64 ? ws_or("tlds_f1_s4_p4_m4", "tlds_f1_s1_p4_m4")
          : b <= 96 ? ws_or("tlds_f1_s4_p4", "tlds_f1_s1_p4_m4")
                    : ws_or("tlds_f1_s2_p4_m4", "tlds_f1_s1_p4_m4");
    } else {
      n = b <= 8 ? "tlds_d_k4_f1_s1_p4_m1"
          : (b <= 64 || blocks < 128) ? "tlds_k4_f1_s1_p4_m1"
                                      : "tlds_w8_k4_f1_s1_p4_m2";
    }
    v = first_supported(op, M, {n, "tlds_k4_f1_s1_p4_m1", "tlds_f1_s1_p4_m2"});
  } else if (!pk && bo == OP_A8W8 && b <= 16) {
    // A8W8, few rows: the LDS tile beats the VALU stream from one row
    v = wrows >= 16384 ? first_supported(op, M, {"tlds_f1_s1_p4_m2", "tlds_f1_s1_p4_m4"})
                       : first_supported(op, M, {b <= 4 ? "tlds_d_w8_k8_f1_s1_p4_m2" : "tlds_w8_k4_f1_s1_p4_m2",
                                                 "tlds_k4_f1_s1_p4_m2"});
  } else if (gemv) {
    if (rowb < 2048) v = first_supported(op, M, {"gemv_r4_k1_p2", "gemv_r4_k2_p2"});
    else if (M == 1) v = first_supported(op, M, {"gemv_r2_k4_p1", "gemv_r4_k4_p1"});
    else if (N >= 65536) v = first_supported(op, M, {"gemv_r8_k4_p1", "gemv_r4_k4_p1", "gemv_r2_k4_p1"});
    else v = first_supported(op, M, {"gemv_r4_k4_p1", "gemv_r2_k4_p1", "gemv_r1_k4_p2"});
    if (v < 0) v = first_of_family(op, M, FAM_GEMV);
  } else if (bo != OP_A8W8Q && !small_w && b >= 4 && b <= 6 && wrows >= 4096 && rowb >= 8192) {
    // large weight rows, a few rows of x: direct x, K split over eight waves
    v = first_supported(op, M, {"tlds_d_w8_k8_f1_s1_p4_m2", "tlds_k4_f1_s1_p4_m2"});
  } else if (bo == OP_A8W8Q) {
    // x is quantised in every round, so K split over the waves of a workgroup
    // multiplies the quantisation each round waits for: one K group per
    // workgroup, and the chip filled through the cross-workgroup split
    const double tiles = wrows / 64.0;
    const int S = !allow_ws ? 1 : tiles <= 64 ? 8 : tiles <= 128 ? 4 : tiles <= 256 ? 2 : 1;
    if (b <= 16)
      v = S == 8 ? first_supported(op, M, {"tlds_f1_s8_p2", "tlds_f1_s8_p4_m2"})
          : S == 4 ? first_supported(op, M, {"tlds_f1_s4_p2", "tlds_f1_s4_p4_m2"})
          : S == 2 ? first_supported(op, M, {"tlds_f1_s2_p4_m2", "tlds_f1_s2_p4"})
                   : first_supported(op, M, {"tlds_f1_s1_p4", "tlds_f1_s1_p4_m2"});
    else
      v = S >= 4 ? first_supported(op, M, {"tlds_w8_f1_s4_p4_m4", "tlds_f1_s4_p4_m2"})
          : allow_ws ? first_supported(op, M, {"tlds_f2_s2_p2", "tlds_f1_s2_p4_m2"})
                     : first_supported(op, M, {"tlds_f1_s1_p4_m2", "tlds_f1_s1_p4_m4"});
  } else if (small_w) {
    if (b <= 64 && (b <= 32 || wbytes <= 4 * MiB))
      v = first_supported(op, M, {"tlds_d_k4_f1_s1_p4_m1", "tlds_k4_f1_s1_p4_m1", "tlds_k4_f1_s1_p4_m2"});
    else if (b <= 32 || wbytes <= 4 * MiB) v = first_supported(op, M, {"tlds_k4_f1_s1_p4_m1", "tlds_k4_f1_s1_p4_m2"});
    else if (b <= 64) v = first_supported(op, M, {"tlds_k4_f1_s1_p4_m2", "tlds_k4_f1_s1_p4_m1"});
    else v = first_supported(op, M, {"tlds_w8_k4_f1_s1_p4_m2", "tlds_k4_f1_s1_p4_m2"});
  } else if (b <= 16 && rowb >= 4096 && std::fmod(wrows, 16.0 * 256.0) == 0.0) {
    v = first_supported(op, M, {"tlds_k4_f1_s1_p4_m2", "tlds_k4_f1_s1_p4_m1"});
  } else {
    const int S = !allow_ws ? 1 : wrows <= 8192 ? 4 : wrows <= 16384 ? 2 : 1;
    // the capped variants (at most 4 or 2 fragments of x rows per workgroup)
    // also serve forms whose full-height tile does not fit the register budget
    if (S == 4)
      v = b <= 32 ? first_supported(op, M, {"tlds_f1_s4_p4", "tlds_f1_s4_p4_m4", "tlds_f1_s4_p4_m2"})
          : b <= 64 ? first_supported(op, M, {"tlds_f1_s4_p4_m4", "tlds_f1_s4_p4_m2"})
                    : first_supported(op, M, {"tlds_w8_f1_s4_p4_m4", "tlds_f1_s4_p4_m4", "tlds_f1_s4_p4_m2"});
    else if (S == 2)
      v = first_supported(op, M, {b <= 32 ? "tlds_f1_s2_p4" : "tlds_f1_s2_p4_m4", "tlds_f1_s2_p4_m4", "tlds_f1_s2_p4_m2"});
    else
      v = first_supported(op, M, {b <= 32 ? "tlds_f1_s1_p4" : "tlds_f1_s1_p4_m4", "tlds_f1_s1_p4_m4", "tlds_f1_s1_p4_m2"});
  }
  if (v < 0) v = first_supported(op, M, {"tile_f1_k4_p4", "tile_f1_k4_p2"});
  if (v < 0) v = first_of_family(op, M, FAM_TILE);
  if (v < 0) v = first_of_family(op, M, FAM_GEMV);
  return v;
}

}  // namespace

// A split-K choice whose output tiles would not fit the split-K tile state
// (only at M far beyond the skinny range) gives way to the rule's no-split
// choice, so the default always launches.
int default_variant(int op, int M, int N, int K) {
  const int v = default_pick(op, M, N, K, true);
  return v >= 0 && !split_tiles_fit(v, M, N) ? default_pick(op, M, N, K, false) : v;
}

}  // namespace skg
