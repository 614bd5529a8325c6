// table.hpp -- the per-device shape -> variant table and the dispatch decision.
//
// One table per device replaces per-kernel configs; each entry names the chosen
// variant for (op, rows bucket, N, K) and keeps every measured candidate beside
// it (mstar PR #1104, "What changed").  A table carries an identity header --
// architecture, HIP runtime, compiler, kernel-selection-space token -- and is
// refused, with one line on stderr, when any field differs from this build and
// device, when it predates the space token, or when a dispatch override is set
// (Strata PR #1297, "The second commit: the seam rework", items 1-2).  Refused
// or absent tables leave the built-in defaults in effect (mstar PR #1104, "What
// changed": products without a table keep today's defaults).  Host-only code.
#pragma once

#include <map>
#include <string>
#include <tuple>
#include <vector>

namespace skg {

struct Identity {
  std::string arch, hip, cc, space;
  std::string str() const;
  static bool parse(const std::string& s, Identity* out);
};

struct Decision {
  int variant;      // index into kVariants
  const char* source;  // "table", "default", "force"
};

class Table {
 public:
  // Load from `path` against `self`.  Returns 0 (loaded or refused: see
  // status()), or -1 if the file cannot be read or parsed (the previous state
  // is kept only if it was empty; a failed load always leaves defaults).
  int load(const std::string& path, const Identity& self, std::string* err);
  void clear();
  bool engaged() const { return engaged_; }
  const std::string& status() const { return status_; }
  // -1 on miss.
  int lookup(int op, int bucket, int N, int K) const;
  size_t size() const { return map_.size(); }

 private:
  std::map<std::tuple<int, int, int, int>, int> map_;
  bool engaged_ = false;
  std::string status_ = "none";
};

// Name of op id ("bf16", "gated", "fp8_tensor", "a8w8_block"), or nullptr.
const char* op_name(int op);
int op_from_name(const std::string& s);
int variant_from_name(const std::string& s);

// Built-in default for (op, M, N, K): the untuned entry point a table is
// measured against.
int default_variant(int op, int M, int N, int K);

// The dispatch override: $SKINNY_GEMM_FORCE=<variant name>, or -1.
int forced_variant();

}  // namespace skg
