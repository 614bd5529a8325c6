// abi.hip -- the C entry points declared in include/skinny_gemm.h: argument
// checks, dispatch (rows bucket -> table or default variant), the split-K
// workspaces, launch.
//
// A GEMM call allocates nothing, frees nothing and never synchronises: the
// only device memory it touches beyond its arguments is the split-K workspace
// that the caller registered (skinny_gemm_set_workspace) or, for
// skinny_gemm_run_static, the library's static device scratch below.  Which
// kernel runs is a pure function of (op, rows bucket, N, K, table), and of M
// past the last bucket.
#include <dlfcn.h>

#include <atomic>
#include <cctype>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <memory>
#include <mutex>
#include <set>
#include <string>
#include <tuple>
#include <unordered_map>
#include <vector>

#include "kernels_mt.hpp"
#include "kernels_pg.hpp"
#include "skinny_gemm.h"
#include "table.hpp"

// Split-K workspace layout (registered or static): kSplitCounters words of
// split-K tile state (three per output tile, split_tile_state in
// kernels.hpp), then the fp32 partials [S][G][M][N] of the call.
constexpr size_t kCntBytes = (size_t)skg::kSplitCounters * sizeof(unsigned);
// The static scratch of skinny_gemm_run_static: the counters and at most
// kStaticPartialBytes of partials.  Each device that runs the library holds
// its own copy until the process ends.  Host code never uses this name as an
// address (in host code it is a stand-in, not device memory): it takes each
// device's address from hipGetSymbolAddress once, with that device current.
constexpr size_t kStaticPartialBytes = (size_t)16 << 20;
static __device__ __align__(256) unsigned char scratch[kCntBytes + kStaticPartialBytes];

namespace skg {

__global__ void zero_kernel(unsigned short* y, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    y[i] = 0;
}

// Clears n words (the split-K tile state of a workspace).  A kernel, not
// hipMemsetAsync, so that it is an ordinary node if a caller captures it.
__global__ void zero_words_kernel(unsigned* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

namespace {

thread_local std::string g_err;

skg_status fail(skg_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

// ------------------------------------------------- process-wide settings
// Read once: the dispatch override and the dispatch log.
struct Settings {
  int force = -1;          // $SKINNY_GEMM_FORCE as a variant index, or -1
  bool log = false;        // $SKINNY_GEMM_LOG set and not "0"
  bool split_wait = true;  // $SKINNY_GEMM_SPLIT_WAIT not "0": split-K workgroups may wait for
                           // the tile's other splits (else the last to arrive adds every slice)
};
const Settings& settings() {
  static const Settings s = [] {
    Settings t;
    t.force = forced_variant();
    const char* lg = std::getenv("SKINNY_GEMM_LOG");
    t.log = lg && *lg && *lg != '0';
    const char* sw = std::getenv("SKINNY_GEMM_SPLIT_WAIT");
    t.split_wait = !(sw && sw[0] == '0' && sw[1] == '\0');
    return t;
  }();
  return s;
}

std::string hex32(uint32_t v) {
  char b[16];
  std::snprintf(b, sizeof b, "%08x", v);
  return b;
}

std::string self_dir() {
  Dl_info info;
  if (dladdr(reinterpret_cast<void*>(&skinny_gemm_last_error), &info) && info.dli_fname) {
    std::string p = info.dli_fname;
    const size_t s = p.rfind('/');
    return s == std::string::npos ? std::string(".") : p.substr(0, s);
  }
  return ".";
}

// Device facts for the identity and the default table path.
bool device_facts(std::string* arch, std::string* hipver) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) { (void)hipGetLastError(); return false; }
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) { (void)hipGetLastError(); return false; }
  std::string a = p.gcnArchName;
  const size_t c = a.find(':');
  *arch = c == std::string::npos ? a : a.substr(0, c);
  int rt = 0;
  if (hipRuntimeGetVersion(&rt) != hipSuccess) { (void)hipGetLastError(); rt = 0; }
  *hipver = std::to_string(rt);
  return true;
}

#define SKG_STR2(x) #x
#define SKG_STR(x) SKG_STR2(x)
std::string compiler_token() { return hex32(fnv1a(__clang_version__ " hip " SKG_STR(HIP_VERSION))); }

std::string space_token() { return hex32(kSpaceToken); }

bool self_identity(Identity* id) {
  std::string arch, hipv;
  if (!device_facts(&arch, &hipv)) return false;
  id->arch = arch;
  id->hip = hipv;
  id->cc = compiler_token();
  id->space = space_token();
  return true;
}

// ------------------------------------------------------------ dispatch
// One immutable table snapshot plus the decisions taken under it.  A load
// builds a new snapshot and publishes it; the old one is kept (never freed),
// so a call that read the old pointer keeps a valid object.  Loads must not
// run concurrently with calls (the header says so); the snapshot makes the
// calls themselves lock-free on the table.
struct Snapshot {
  Table table;
  mutable std::mutex mu;                                   // guards `cache`
  mutable std::unordered_map<uint64_t, int> cache;         // (op, bucket, N, K) -> variant
};

std::mutex g_mu;                                            // serialises loads
std::vector<std::unique_ptr<Snapshot>> g_snapshots;        // every snapshot ever published
std::atomic<const Snapshot*> g_snap{nullptr};

void publish(std::unique_ptr<Snapshot> s) {   // caller holds g_mu
  g_snap.store(s.get(), std::memory_order_release);
  g_snapshots.push_back(std::move(s));
}

// The first dispatch loads $SKINNY_GEMM_TABLE, else the table installed beside
// the library for this device.  Caller holds g_mu.
void lazy_load_locked() {
  auto s = std::make_unique<Snapshot>();
  Identity id;
  if (self_identity(&id)) {
    std::string path;
    if (const char* e = std::getenv("SKINNY_GEMM_TABLE"); e && *e) path = e;
    else path = self_dir() + "/configs/" + id.arch + "/skinny_gemm.json";
    if (FILE* f = std::fopen(path.c_str(), "rb")) {
      std::fclose(f);
      std::string err;
      if (s->table.load(path, id, &err) != 0)
        std::fprintf(stderr, "skinny_gemm: table %s not loaded: %s; built-in defaults stay in effect\n",
                     path.c_str(), err.c_str());
    }
  }
  publish(std::move(s));
}

const Snapshot* snapshot() {
  const Snapshot* s = g_snap.load(std::memory_order_acquire);
  if (s) return s;
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_snap.load(std::memory_order_relaxed)) lazy_load_locked();
  return g_snap.load(std::memory_order_acquire);
}

// The dispatch decision: the override, else the table entry of the rows
// bucket, else the built-in default.  Every M of one rows bucket compiles to
// the same kernels, so a decision depends on (op, bucket, N, K) only; past
// the last bucket it depends on M as well.
Decision decide(int op, int M, int N, int K) {
  const Snapshot* snap = snapshot();
  const Settings& cfg = settings();
  const int b = bucket_of(M);                              // 0: above the last bucket
  const uint64_t key = ((uint64_t)(unsigned)op << 58) ^ ((uint64_t)(unsigned)b << 48) ^
                       ((uint64_t)(unsigned)N << 24) ^ (uint64_t)(unsigned)K;
  // (rows past the last bucket are not cached: there the default also
  // depends on M, through the split-K tile limit)
  const bool keyable = b != 0 && N < (1 << 24) && K < (1 << 24);
  {
    std::lock_guard<std::mutex> lk(snap->mu);
    if (keyable) {
      const auto it = snap->cache.find(key);
      if (it != snap->cache.end())
        return Decision{it->second, it->second == cfg.force ? "force" : "cached"};
    }
  }
  Decision d{-1, "default"};
  if (cfg.force >= 0 && variant_supports(op, cfg.force, M)) {
    d = Decision{cfg.force, "force"};
  } else {
    const int tv = b ? snap->table.lookup(op, b, N, K) : -1;
    if (tv >= 0 && variant_supports(op, tv, M)) d = Decision{tv, "table"};
    else d = Decision{default_variant(op, M, N, K), "default"};
  }
  if (keyable) {
    std::lock_guard<std::mutex> lk(snap->mu);
    snap->cache.emplace(key, d.variant);
  }
  if (cfg.log)
    std::fprintf(stderr, "skinny_gemm: %s M=%d(bucket %d) N=%d K=%d -> %s [%s]\n", op_name(op), M, b, N, K,
                 d.variant >= 0 ? kVariants[d.variant].name : "none", d.source);
  return d;
}

// Where a decision came from, for skinny_gemm_query (not cached: the query
// states the source).
const char* decision_source(int op, int M, int N, int K, int v) {
  const Settings& cfg = settings();
  if (cfg.force >= 0 && v == cfg.force) return "force";
  const int b = bucket_of(M);
  const int tv = b ? snapshot()->table.lookup(op, b, N, K) : -1;
  return tv == v ? "table" : "default";
}

// ---------------------------------------------------------- argument checks
struct Buf {
  const void* p;
  size_t bytes;
  const char* name;
};

skg_status check_device_range(const Buf& b) {
  if (b.bytes == 0) return SKG_OK;
  if (!b.p) return fail(SKG_EINVAL, "%s is NULL", b.name);
  hipDeviceptr_t base = nullptr;
  size_t size = 0;
  if (hipMemGetAddressRange(&base, &size, const_cast<void*>(b.p)) != hipSuccess || !base) {
    (void)hipGetLastError();
    return fail(SKG_EINVAL, "%s (%p) is not HIP device memory", b.name, b.p);
  }
  const uintptr_t lo = reinterpret_cast<uintptr_t>(base), hi = lo + size;
  const uintptr_t p = reinterpret_cast<uintptr_t>(b.p);
  if (p < lo || p + b.bytes > hi || p + b.bytes < p)
    return fail(SKG_EINVAL, "%s needs %zu bytes but its allocation ends %zu bytes after it", b.name, b.bytes,
                (size_t)(hi - p));
  return SKG_OK;
}

bool overlap(const Buf& a, const Buf& b) {
  if (!a.bytes || !b.bytes) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + b.bytes && b0 < a0 + a.bytes;
}

skg_status validate(int op, const Args& a) {
  if (a.M < 0 || a.N < 0 || a.K < 0) return fail(SKG_EINVAL, "negative size M=%d N=%d K=%d", a.M, a.N, a.K);
  if (a.M == 0 || a.N == 0) return SKG_OK;
  const int km = op_k_multiple(op);
  if (a.K % km) return fail(SKG_EUNSUPPORTED, "%s needs K %% %d == 0 (K=%d)", op_name(op), km, a.K);
  const int base = op_base(op);
  const size_t M = a.M, N = a.N, K = a.K;
  const size_t G = op_groups(op);
  const size_t kb = (K + 127) / 128, nb = (N + 127) / 128;
  Buf bx{a.x, M * K * op_x_bytes(op), "x"};
  Buf bw{a.w, op_packed(op) ? packed_weight_bytes(op, a.N, a.K) : G * N * K * op_w_bytes(op), "W"};
  Buf by{a.y, M * N * 2, "y"};
  Buf b0{a.s0, 0, base == OP_A8W8 ? "x_scales" : "scales"};
  Buf b1{a.s1, 0, "w_scales"};
  Buf bo{a.xs_out, 0, "x_scales_out"};   // an output: may be NULL
  if (base == OP_FP8T) b0.bytes = 4;
  if (base == OP_A8W8 && K > 0) {
    b0.bytes = M * kb * 4;
    b1.bytes = nb * kb * 4;
  }
  if (base == OP_A8W8Q && K > 0) {
    b1.bytes = nb * kb * 4;
    if (a.xs_out) bo.bytes = M * kb * 4;
  }
  if (K > 0 && ((reinterpret_cast<uintptr_t>(a.x) | reinterpret_cast<uintptr_t>(a.w)) & 15))
    return fail(SKG_EUNSUPPORTED, "x and W must be 16-byte aligned (x=%p W=%p)", a.x, a.w);
  if (reinterpret_cast<uintptr_t>(a.y) & 1) return fail(SKG_EUNSUPPORTED, "y must be 2-byte aligned");
  if ((reinterpret_cast<uintptr_t>(a.s0) | reinterpret_cast<uintptr_t>(a.s1) |
       reinterpret_cast<uintptr_t>(a.xs_out)) & 3)
    return fail(SKG_EUNSUPPORTED, "scales must be 4-byte aligned");
  if (K == 0) {
    bx.bytes = bw.bytes = 0;
    b0.bytes = b1.bytes = bo.bytes = 0;
  }
  for (const Buf* b : {&bx, &bw, &by, &b0, &b1, &bo})
    if (skg_status st = check_device_range(*b)) return st;
  for (const Buf* b : {&bx, &bw, &b0, &b1})
    if (overlap(by, *b)) return fail(SKG_EINVAL, "y overlaps %s", b->name);
  for (const Buf* b : {&bx, &bw, &b1, &by})
    if (overlap(bo, *b)) return fail(SKG_EINVAL, "x_scales_out overlaps %s", b->name);
  if ((size_t)a.N * (size_t)G > 0x7fffffffu) return fail(SKG_EUNSUPPORTED, "N too large");
  return SKG_OK;
}

LaunchFn variant_fn(int op, int v, int M) {
  const VariantDesc& d = kVariants[v];
  const int fi = family_index(v);
  if (d.family == FAM_PG) {
    const int mi = gemv_mt_index(M);
    const GemvRow* t = op == OP_PACKED + OP_BF16   ? pg_table<OP_PACKED + OP_BF16>()
                       : op == OP_PACKED + OP_GATED ? pg_table<OP_PACKED + OP_GATED>()
                                                    : nullptr;
    return t && mi >= 0 ? t[fi].f[mi] : nullptr;
  }
  if (d.family == FAM_MT) {
    const LaunchFn* t = nullptr;
    switch (op) {
      case OP_BF16: t = mt_table<OP_BF16>(); break;
      case OP_A8W8: t = mt_table<OP_A8W8>(); break;
      case OP_PACKED + OP_BF16: t = mt_table<OP_PACKED + OP_BF16>(); break;
      case OP_PACKED + OP_A8W8: t = mt_table<OP_PACKED + OP_A8W8>(); break;
    }
    return t ? t[fi] : nullptr;
  }
  if (d.family == FAM_GEMV) {
    const int mi = gemv_mt_index(M);
    if (mi < 0) return nullptr;
    const GemvRow* t = nullptr;
    switch (op) {
      case OP_BF16: t = gemv_table<OP_BF16>(); break;
      case OP_GATED: t = gemv_table<OP_GATED>(); break;
      case OP_FP8T: t = gemv_table<OP_FP8T>(); break;
      case OP_A8W8: t = gemv_table<OP_A8W8>(); break;
      case OP_A8W8Q: t = gemv_table<OP_A8W8Q>(); break;
    }
    return t ? t[fi].f[mi] : nullptr;
  }
  const int fm = M > kMaxBucket ? kNumTileFM - 1 : tile_fm_index(M);
  const TileRow* t = nullptr;
  const bool lds = d.family == FAM_TLDS;
  switch (op) {
    case OP_BF16: t = lds ? tlds_table<OP_BF16>() : tile_table<OP_BF16>(); break;
    case OP_GATED: t = lds ? tlds_table<OP_GATED>() : tile_table<OP_GATED>(); break;
    case OP_FP8T: t = lds ? tlds_table<OP_FP8T>() : tile_table<OP_FP8T>(); break;
    case OP_A8W8: t = lds ? tlds_table<OP_A8W8>() : tile_table<OP_A8W8>(); break;
    case OP_A8W8Q: t = lds ? tlds_table<OP_A8W8Q>() : tile_table<OP_A8W8Q>(); break;
    case OP_PACKED + OP_BF16: t = lds ? tlds_table<OP_PACKED + OP_BF16>() : nullptr; break;
    case OP_PACKED + OP_GATED: t = lds ? tlds_table<OP_PACKED + OP_GATED>() : nullptr; break;
    case OP_PACKED + OP_FP8T: t = lds ? tlds_table<OP_PACKED + OP_FP8T>() : nullptr; break;
    case OP_PACKED + OP_A8W8: t = lds ? tlds_table<OP_PACKED + OP_A8W8>() : nullptr; break;
    case OP_PACKED + OP_A8W8Q: t = lds ? tlds_table<OP_PACKED + OP_A8W8Q>() : nullptr; break;
  }
  return t ? t[fi].f[fm] : nullptr;
}

// Bytes of split-K partials variant v of op needs for M rows (0: none), and
// whether its output tiles fit the split-K tile state.
size_t partial_bytes(int op, int v, int M, int N) {
  if (v < 0) return 0;
  if (kVariants[v].family == FAM_MT) return (size_t)tlds_ws_bytes(op, kVariants[v].p4, M, N);
  if (kVariants[v].family != FAM_TLDS) return 0;
  return (size_t)tlds_ws_bytes(op, kVariants[v].p1, M, N);
}
bool tiles_fit(int op, int v, int M, int N) {
  (void)op;
  return split_tiles_fit(v, M, N);
}

// ------------------------------------------------- registered workspaces
// Caller-owned device buffers for the split-K partials, registered per
// (device, stream) or per device (any stream of it that has none of its own).
struct WsReg {
  int dev;
  bool any;            // the device-wide registration
  hipStream_t stream;  // when !any
  char* p;
  size_t bytes;
};
std::mutex g_ws_mu;
std::vector<WsReg> g_ws;

bool capturing(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return cs != hipStreamCaptureStatusNone;
}

skg_status clear_counters(void* p, hipStream_t s) {
  hipLaunchKernelGGL(zero_words_kernel, dim3(64), dim3(256), 0, s, static_cast<unsigned*>(p),
                     (size_t)kSplitCounters);
  const hipError_t e = hipGetLastError();
  return e == hipSuccess ? SKG_OK : fail(SKG_ELAUNCH, "clearing the split-K counters: %s", hipGetErrorString(e));
}

skg_status register_ws(bool any, hipStream_t stream, void* ws, size_t bytes) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(SKG_EINVAL, "no current HIP device");
  }
  if (ws) {
    if (bytes < kCntBytes) return fail(SKG_EINVAL, "a workspace needs at least %zu bytes (has %zu)", kCntBytes, bytes);
    if (reinterpret_cast<uintptr_t>(ws) & 255) return fail(SKG_EUNSUPPORTED, "the workspace must be 256-byte aligned");
    if (skg_status st = check_device_range(Buf{ws, bytes, "workspace"})) return st;
    if (capturing(stream)) return fail(SKG_EINVAL, "register a workspace outside graph capture");
    if (skg_status st = clear_counters(ws, stream)) return st;
  }
  std::lock_guard<std::mutex> lk(g_ws_mu);
  for (size_t i = 0; i < g_ws.size(); ++i)
    if (g_ws[i].dev == dev && g_ws[i].any == any && (any || g_ws[i].stream == stream)) {
      g_ws.erase(g_ws.begin() + (long)i);
      break;
    }
  if (ws) g_ws.push_back(WsReg{dev, any, any ? nullptr : stream, static_cast<char*>(ws), bytes});
  return SKG_OK;
}

// The workspace for a call on `stream` of the current device: its own, else
// the device's; {nullptr, 0} if neither.
std::pair<char*, size_t> find_ws(hipStream_t stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return {nullptr, 0};
  }
  std::lock_guard<std::mutex> lk(g_ws_mu);
  const WsReg* anyr = nullptr;
  for (const WsReg& r : g_ws) {
    if (r.dev != dev) continue;
    if (!r.any && r.stream == stream) return {r.p, r.bytes};
    if (r.any) anyr = &r;
  }
  return anyr ? std::make_pair(anyr->p, anyr->bytes) : std::make_pair((char*)nullptr, (size_t)0);
}

// --------------------------------------------- the static scratch, per device
constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices] = {};
bool g_static_cleared[kMaxDevices] = {};   // counters cleared by a launch outside capture

// This device's copy of `scratch`: its address is taken once per device with
// that device current; the counters are cleared (stream-ordered, before the
// call's kernel) until one clear has run outside graph capture, after which
// every launch leaves them consistent for the next.
skg_status static_scratch(hipStream_t s, char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return fail(SKG_EINVAL, "no current HIP device");
  }
  if (dev < 0 || dev >= kMaxDevices) return fail(SKG_EUNSUPPORTED, "device %d beyond the static scratch table", dev);
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return fail(SKG_ELAUNCH, "hipGetSymbolAddress of the static scratch failed on device %d", dev);
    }
    g_static_ptr[dev] = ptr;
  }
  if (!g_static_cleared[dev]) {
    if (skg_status st = clear_counters(g_static_ptr[dev], s)) return st;
    if (!capturing(s)) g_static_cleared[dev] = true;
  }
  *out = static_cast<char*>(g_static_ptr[dev]);
  return SKG_OK;
}

// ------------------------------------------------------------------ launch
enum class WsFrom { kRegistered, kStatic };

skg_status launch(int op, int v, const Args& a_in, hipStream_t s, WsFrom from) {
  Args a = a_in;
  if (a.K == 0) {
    const size_t n = (size_t)a.M * a.N;
    const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, s, static_cast<unsigned short*>(a.y), n);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? SKG_OK : fail(SKG_ELAUNCH, "zero fill launch: %s", hipGetErrorString(e));
  }
  const LaunchFn fn = v >= 0 ? variant_fn(op, v, a.M) : nullptr;
  if (!fn)
    return fail(SKG_EUNSUPPORTED, "variant %s is not compiled for %s at M=%d", v >= 0 ? kVariants[v].name : "(none)",
                op_name(op), a.M);
  if (const size_t need = partial_bytes(op, v, a.M, a.N)) {
    if (!tiles_fit(op, v, a.M, a.N))
      return fail(SKG_EUNSUPPORTED, "%s: more output tiles than split-K counters", kVariants[v].name);
    // the kernels address the partials through a 32-bit buffer range
    if (need >= (size_t)1 << 32)
      return fail(SKG_EUNSUPPORTED, "%s at M=%d N=%d: %zu bytes of split-K partials exceed the 4 GiB the kernels address",
                  kVariants[v].name, a.M, a.N, need);
    char* base = nullptr;
    if (from == WsFrom::kStatic) {
      if (need > kStaticPartialBytes)
        return fail(SKG_EUNSUPPORTED,
                    "%s at M=%d N=%d needs %zu bytes of split-K partials; the static scratch holds %zu",
                    kVariants[v].name, a.M, a.N, need, kStaticPartialBytes);
      if (skg_status st = static_scratch(s, &base)) return st;
    } else {
      const auto ws = find_ws(s);
      if (!ws.first || ws.second < need + kCntBytes)
        return fail(SKG_EUNSUPPORTED,
                    "%s at M=%d N=%d needs a split-K workspace of %zu bytes on this stream (registered: %zu); "
                    "see skinny_gemm_set_workspace",
                    kVariants[v].name, a.M, a.N, need + kCntBytes, ws.second);
      base = ws.first;
    }
    a.cnt = reinterpret_cast<unsigned*>(base);
    a.ws = reinterpret_cast<float*>(base + kCntBytes);
  }
  if (op_base(op) == OP_A8W8 && kVariants[v].family == FAM_GEMV) {
    const size_t smem = (size_t)(kGemvMT[gemv_mt_index(a.M)] + 1) * a.kb * sizeof(float);
    if (smem > 64 * 1024)
      return fail(SKG_EUNSUPPORTED, "K=%d needs %zu bytes of A8W8 scale staging (limit 65536)", a.K, smem);
  }
  const hipError_t e = fn(a, s);
  if (e != hipSuccess)
    return fail(SKG_ELAUNCH, "%s %s launch: %s", op_name(op), kVariants[v].name, hipGetErrorString(e));
  return SKG_OK;
}

Args make_args(int op, const void* x, const void* w, const float* s0, const float* s1, void* y, int M, int N,
               int K, float* xs_out) {
  const int base = op_base(op);
  Args a{x, w, s0, s1, y, M, N, K, (K + 127) / 128, nullptr, nullptr, base == OP_A8W8Q ? xs_out : nullptr};
  a.split_wait = settings().split_wait ? 0 : -1;   // the launch decides 1 or 0 unless waits are off
  if (base != OP_FP8T && base != OP_A8W8) a.s0 = nullptr;
  if (base != OP_A8W8 && base != OP_A8W8Q) a.s1 = nullptr;
  return a;
}

skg_status run_op(int op, const void* x, const void* w, const float* s0, const float* s1, void* y, int M, int N,
                  int K, hipStream_t s, float* xs_out, WsFrom from) {
  const Args a = make_args(op, x, w, s0, s1, y, M, N, K, xs_out);
  if (skg_status st = validate(op, a)) return st;
  if (M == 0 || N == 0) return SKG_OK;
  const Decision d = decide(op, M, N, K);
  return launch(op, d.variant, a, s, from);
}

int copy_out(const std::string& s, char* buf, int len) {
  if (!buf || len <= 0) return SKG_EINVAL;
  std::snprintf(buf, (size_t)len, "%s", s.c_str());
  return (int)s.size() < len ? SKG_OK : SKG_EINVAL;
}

}  // namespace
}  // namespace skg

using namespace skg;

extern "C" {

skg_status skinny_gemm_bf16(const void* x, const void* W, const float* scales, void* y, int M, int N, int K,
                            hipStream_t stream) {
  return run_op(OP_BF16, x, W, scales, nullptr, y, M, N, K, stream, nullptr, WsFrom::kRegistered);
}

skg_status skinny_gemm_gated(const void* x, const void* W, const float* scales, void* y, int M, int N, int K,
                             hipStream_t stream) {
  return run_op(OP_GATED, x, W, scales, nullptr, y, M, N, K, stream, nullptr, WsFrom::kRegistered);
}

skg_status skinny_gemm_fp8_tensor(const void* x, const void* W, const float* scales, void* y, int M, int N, int K,
                                  hipStream_t stream) {
  return run_op(OP_FP8T, x, W, scales, nullptr, y, M, N, K, stream, nullptr, WsFrom::kRegistered);
}

skg_status skinny_gemm_a8w8_block(const void* x, const void* W, const float* x_scales, const float* w_scales,
                                  void* y, int M, int N, int K, hipStream_t stream) {
  return run_op(OP_A8W8, x, W, x_scales, w_scales, y, M, N, K, stream, nullptr, WsFrom::kRegistered);
}

skg_status skinny_gemm_a8w8_block_quant(const void* x, const void* W, const float* w_scales, float* x_scales_out,
                                        void* y, int M, int N, int K, hipStream_t stream) {
  return run_op(OP_A8W8Q, x, W, nullptr, w_scales, y, M, N, K, stream, x_scales_out, WsFrom::kRegistered);
}

skg_status skinny_gemm_bf16_packed(const void* x, const void* W_packed, const float* scales, void* y, int M, int N,
                                   int K, hipStream_t stream) {
  return run_op(OP_PACKED + OP_BF16, x, W_packed, scales, nullptr, y, M, N, K, stream, nullptr, WsFrom::kRegistered);
}

skg_status skinny_gemm_gated_packed(const void* x, const void* W_packed, const float* scales, void* y, int M, int N,
                                    int K, hipStream_t stream) {
  return run_op(OP_PACKED + OP_GATED, x, W_packed, scales, nullptr, y, M, N, K, stream, nullptr,
                WsFrom::kRegistered);
}

skg_status skinny_gemm_fp8_tensor_packed(const void* x, const void* W_packed, const float* scales, void* y, int M,
                                         int N, int K, hipStream_t stream) {
  return run_op(OP_PACKED + OP_FP8T, x, W_packed, scales, nullptr, y, M, N, K, stream, nullptr, WsFrom::kRegistered);
}

skg_status skinny_gemm_a8w8_block_packed(const void* x, const void* W_packed, const float* x_scales,
                                         const float* w_scales, void* y, int M, int N, int K, hipStream_t stream) {
  return run_op(OP_PACKED + OP_A8W8, x, W_packed, x_scales, w_scales, y, M, N, K, stream, nullptr,
                WsFrom::kRegistered);
}

skg_status skinny_gemm_a8w8_block_quant_packed(const void* x, const void* W_packed, const float* w_scales,
                                               float* x_scales_out, void* y, int M, int N, int K,
                                               hipStream_t stream) {
  return run_op(OP_PACKED + OP_A8W8Q, x, W_packed, nullptr, w_scales, y, M, N, K, stream, x_scales_out,
                WsFrom::kRegistered);
}

size_t skinny_gemm_workspace_bytes(int op, int M, int N, int K) {
  if (!op_name(op) || M <= 0 || N <= 0 || K <= 0 || K % op_k_multiple(op)) return 0;
  const Decision d = decide(op, M, N, K);
  const size_t need = partial_bytes(op, d.variant, M, N);
  return need ? need + kCntBytes : 0;
}

skg_status skinny_gemm_set_workspace(hipStream_t stream, void* workspace, size_t bytes) {
  return register_ws(false, stream, workspace, bytes);
}

skg_status skinny_gemm_set_device_workspace(void* workspace, size_t bytes, hipStream_t stream) {
  return register_ws(true, stream, workspace, bytes);
}

skg_status skinny_gemm_run_static(int op, const void* x, const void* W, const float* s0, const float* s1, void* y,
                                  int M, int N, int K, hipStream_t stream) {
  if (!op_name(op)) return fail(SKG_EINVAL, "unknown op %d", op);
  float* xs_out = op_base(op) == OP_A8W8Q ? const_cast<float*>(s0) : nullptr;   // its s0 is the x-scale output
  return run_op(op, x, W, s0, s1, y, M, N, K, stream, xs_out, WsFrom::kStatic);
}

size_t skinny_gemm_static_scratch_bytes(void) { return kStaticPartialBytes; }

size_t skinny_gemm_packed_weight_bytes(int op, int N, int K) {
  if (!op_name(op) || N <= 0 || K <= 0 || K % op_k_multiple(op)) return 0;
  return packed_weight_bytes(op, N, K);
}

skg_status skinny_gemm_pack_weight(int op, const void* W, void* W_packed, int N, int K, hipStream_t stream) {
  if (!op_name(op)) return fail(SKG_EINVAL, "unknown op %d", op);
  if (N < 0 || K < 0) return fail(SKG_EINVAL, "negative size N=%d K=%d", N, K);
  if (N == 0 || K == 0) return SKG_OK;
  const int km = op_k_multiple(op);
  if (K % km) return fail(SKG_EUNSUPPORTED, "%s needs K %% %d == 0 (K=%d)", op_name(op), km, K);
  if ((size_t)N * (size_t)op_groups(op) > 0x7fffffffu) return fail(SKG_EUNSUPPORTED, "N too large");
  if ((reinterpret_cast<uintptr_t>(W) | reinterpret_cast<uintptr_t>(W_packed)) & 15)
    return fail(SKG_EUNSUPPORTED, "W and W_packed must be 16-byte aligned");
  const Buf bw{W, (size_t)op_groups(op) * N * K * op_w_bytes(op), "W"};
  const Buf bp{W_packed, packed_weight_bytes(op, N, K), "W_packed"};
  for (const Buf* b : {&bw, &bp})
    if (skg_status st = check_device_range(*b)) return st;
  if (overlap(bw, bp)) return fail(SKG_EINVAL, "W_packed overlaps W");
  const hipError_t e = launch_pack(op, W, W_packed, N, K, stream);
  return e == hipSuccess ? SKG_OK : fail(SKG_ELAUNCH, "pack launch: %s", hipGetErrorString(e));
}

const char* skinny_gemm_last_error(void) { return g_err.c_str(); }

skg_status skinny_gemm_calib_read(const void* buf, size_t bytes, int grid, int sweep, unsigned* sink,
                                  hipStream_t stream) {
  if (grid < 1 || grid > 65536) return fail(SKG_EINVAL, "grid %d outside 1..65536", grid);
  if (sweep != 0 && sweep != 1) return fail(SKG_EINVAL, "sweep must be 0 or 1 (%d)", sweep);
  if (bytes == 0 || bytes % 16 || (reinterpret_cast<uintptr_t>(buf) & 15) || (reinterpret_cast<uintptr_t>(sink) & 3))
    return fail(SKG_EUNSUPPORTED, "buf must be 16-byte aligned, its size a nonzero multiple of 16, sink 4-byte aligned");
  const Buf bb{buf, bytes, "buf"}, bs{sink, 256 * sizeof(unsigned), "sink"};
  for (const Buf* b : {&bb, &bs})
    if (skg_status st = check_device_range(*b)) return st;
  if (overlap(bb, bs)) return fail(SKG_EINVAL, "sink overlaps buf");
  const hipError_t e = launch_calib_read(buf, (unsigned long long)(bytes / 16), grid, sweep, sink, stream);
  return e == hipSuccess ? SKG_OK : fail(SKG_ELAUNCH, "calib read launch: %s", hipGetErrorString(e));
}

skg_status skinny_gemm_calib_mfma(int grid, int iters, unsigned* sink, hipStream_t stream) {
  if (grid < 1 || grid > 65536 || iters < 1 || iters > (1 << 20))
    return fail(SKG_EINVAL, "grid %d (1..65536) or iters %d (1..2^20) out of range", grid, iters);
  if (reinterpret_cast<uintptr_t>(sink) & 3) return fail(SKG_EUNSUPPORTED, "sink must be 4-byte aligned");
  const Buf bs{sink, 256 * sizeof(unsigned), "sink"};
  if (skg_status st = check_device_range(bs)) return st;
  const hipError_t e = launch_calib_mfma(grid, iters, sink, stream);
  return e == hipSuccess ? SKG_OK : fail(SKG_ELAUNCH, "calib mfma launch: %s", hipGetErrorString(e));
}

skg_status skinny_gemm_load_table(const char* path) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto s = std::make_unique<Snapshot>();
  Identity id;
  if (!self_identity(&id)) {
    publish(std::move(s));
    return fail(SKG_ETABLE, "no HIP device: cannot establish the table identity");
  }
  std::string p;
  if (path && *path) p = path;
  else if (const char* e = std::getenv("SKINNY_GEMM_TABLE"); e && *e) p = e;
  else p = self_dir() + "/configs/" + id.arch + "/skinny_gemm.json";
  std::string err;
  const int rc = s->table.load(p, id, &err);
  publish(std::move(s));
  if (rc != 0) return fail(SKG_ETABLE, "%s", err.c_str());
  return SKG_OK;
}

skg_status skinny_gemm_load_table_as(const char* path, const char* identity) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto s = std::make_unique<Snapshot>();
  Identity id;
  if (!identity || !Identity::parse(identity, &id)) {
    publish(std::move(s));
    return fail(SKG_EINVAL, "identity must read arch=..;hip=..;cc=..;space=..");
  }
  if (!path || !*path) {
    publish(std::move(s));
    return SKG_OK;  // explicit "no table"
  }
  std::string err;
  const int rc = s->table.load(path, id, &err);
  publish(std::move(s));
  if (rc != 0) return fail(SKG_ETABLE, "%s", err.c_str());
  return SKG_OK;
}

skg_status skinny_gemm_identity(char* buf, int len) {
  Identity id;
  if (!self_identity(&id)) return fail(SKG_EUNSUPPORTED, "no HIP device");
  return copy_out(id.str(), buf, len);
}

int skinny_gemm_table_status(char* buf, int len) {
  const Snapshot* s = g_snap.load(std::memory_order_acquire);
  if (!s) {
    if (buf && len > 0) std::snprintf(buf, (size_t)len, "%s", "none");
    return 0;
  }
  if (buf && len > 0) std::snprintf(buf, (size_t)len, "%s", s->table.status().c_str());
  return s->table.engaged() ? 1 : 0;
}

skg_status skinny_gemm_query(int op, int M, int N, int K, char* buf, int len) {
  if (!op_name(op)) return fail(SKG_EINVAL, "unknown op %d", op);
  if (M <= 0 || N <= 0 || K < 0) return fail(SKG_EINVAL, "query needs M, N > 0 and K >= 0");
  const Decision d = decide(op, M, N, K);
  if (d.variant < 0) return fail(SKG_EUNSUPPORTED, "no variant for M=%d", M);
  return copy_out(std::string(kVariants[d.variant].name) + " " + decision_source(op, M, N, K, d.variant), buf, len);
}

int skinny_gemm_num_variants(int op) { return op_name(op) ? kNumVariants : 0; }

skg_status skinny_gemm_variant_name(int op, int variant, char* buf, int len) {
  if (!op_name(op) || variant < 0 || variant >= kNumVariants) return fail(SKG_EINVAL, "no such variant");
  return copy_out(kVariants[variant].name, buf, len);
}

int skinny_gemm_variant_supports(int op, int variant, int M) {
  if (!op_name(op) || variant < 0 || variant >= kNumVariants || M <= 0) return 0;
  return variant_supports(op, variant, M) ? 1 : 0;
}

skg_status skinny_gemm_run_variant(int op, int variant, const int* knobs, const void* x, const void* W,
                                   const float* s0, const float* s1, void* y, int M, int N, int K,
                                   hipStream_t stream) {
  if (!op_name(op)) return fail(SKG_EINVAL, "unknown op %d", op);
  if (variant < 0 || variant >= kNumVariants) return fail(SKG_EINVAL, "no variant %d", variant);
  if (knobs) return fail(SKG_EINVAL, "knobs are reserved: pass NULL");
  float* xs_out = op_base(op) == OP_A8W8Q ? const_cast<float*>(s0) : nullptr;   // its s0 is the x-scale output
  const Args a = make_args(op, x, W, s0, s1, y, M, N, K, xs_out);
  if (skg_status st = validate(op, a)) return st;
  if (M == 0 || N == 0) return SKG_OK;
  if (!variant_supports(op, variant, M))
    return fail(SKG_EUNSUPPORTED, "variant %s does not run %s at M=%d", kVariants[variant].name, op_name(op), M);
  return launch(op, variant, a, stream, WsFrom::kRegistered);
}

size_t skinny_gemm_variant_workspace_bytes(int op, int variant, int M, int N) {
  if (!op_name(op) || variant < 0 || variant >= kNumVariants || M <= 0 || N <= 0) return 0;
  const size_t need = partial_bytes(op, variant, M, N);
  return need ? need + kCntBytes : 0;
}

}  // extern "C"
