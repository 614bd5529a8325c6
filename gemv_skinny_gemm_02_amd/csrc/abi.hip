// abi.hip -- the C entry points declared in include/skinny_gemm.h: argument
// checks, dispatch (rows bucket -> table or default variant), launch.
#include <dlfcn.h>

#include <cctype>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <set>
#include <string>
#include <tuple>

#include "kernels.hpp"
#include "skinny_gemm.h"
#include "table.hpp"

namespace skg {

__global__ void zero_kernel(unsigned short* y, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    y[i] = 0;
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

std::mutex g_mu;
Table g_table;
bool g_table_tried = false;  // a load (explicit or lazy) has happened

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
bool device_facts(std::string* arch, std::string* product, std::string* hipver) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) { (void)hipGetLastError(); return false; }
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) != hipSuccess) { (void)hipGetLastError(); return false; }
  std::string a = p.gcnArchName;
  const size_t c = a.find(':');
  *arch = c == std::string::npos ? a : a.substr(0, c);
  std::string name = p.name, low;
  for (char ch : name) low.push_back(static_cast<char>(std::tolower(static_cast<unsigned char>(ch))));
  *product = "unknown";
  for (size_t i = 0; i + 2 < low.size(); ++i) {
    if (low[i] == 'm' && low[i + 1] == 'i' && std::isdigit(static_cast<unsigned char>(low[i + 2]))) {
      size_t j = i + 2;
      while (j < low.size() && std::isalnum(static_cast<unsigned char>(low[j]))) ++j;
      *product = low.substr(i, j - i);
      break;
    }
  }
  int rt = 0;
  if (hipRuntimeGetVersion(&rt) != hipSuccess) { (void)hipGetLastError(); rt = 0; }
  *hipver = std::to_string(rt);
  return true;
}

#define SKG_STR2(x) #x
#define SKG_STR(x) SKG_STR2(x)
std::string compiler_token() { return hex32(fnv1a(__clang_version__ " hip " SKG_STR(HIP_VERSION))); }

std::string space_token() { return hex32(kSpaceToken); }

bool self_identity(Identity* id, std::string* product) {
  std::string arch, prod, hipv;
  if (!device_facts(&arch, &prod, &hipv)) return false;
  id->arch = arch;
  id->hip = hipv;
  id->cc = compiler_token();
  id->space = space_token();
  if (product) *product = prod;
  return true;
}

// Lazy table load on the first dispatch: $SKINNY_GEMM_TABLE, else the table
// installed beside the library for this device.  Caller holds g_mu.
void ensure_table_locked() {
  if (g_table_tried) return;
  g_table_tried = true;
  Identity id;
  std::string product;
  if (!self_identity(&id, &product)) return;
  std::string path;
  if (const char* e = std::getenv("SKINNY_GEMM_TABLE"); e && *e) path = e;
  else path = self_dir() + "/configs/" + id.arch + "/skinny_gemm.json";
  (void)product;
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f) return;  // no table: defaults
  std::fclose(f);
  std::string err;
  if (g_table.load(path, id, &err) != 0)
    std::fprintf(stderr, "skinny_gemm: table %s not loaded: %s; built-in defaults stay in effect\n", path.c_str(),
                 err.c_str());
}

std::set<std::tuple<int, int, int, int, int>> g_logged;

Decision decide(int op, int M, int N, int K) {
  std::lock_guard<std::mutex> lk(g_mu);
  ensure_table_locked();
  Decision d{-1, "default"};
  const int fv = forced_variant();
  if (fv >= 0 && variant_supports(op, fv, M)) {
    d = Decision{fv, "force"};
  } else {
    const int b = bucket_of(M);
    const int tv = b ? g_table.lookup(op, b, N, K) : -1;
    if (tv >= 0 && variant_supports(op, tv, M)) d = Decision{tv, "table"};
    else d = Decision{default_variant(op, M, N, K), "default"};
  }
  if (const char* lg = std::getenv("SKINNY_GEMM_LOG"); lg && *lg && *lg != '0') {
    const auto key = std::make_tuple(op, bucket_of(M), N, K, d.variant);
    if (g_logged.insert(key).second)
      std::fprintf(stderr, "skinny_gemm: %s M=%d(bucket %d) N=%d K=%d -> %s [%s]\n", op_name(op), M, bucket_of(M), N,
                   K, d.variant >= 0 ? kVariants[d.variant].name : "none", d.source);
  }
  return d;
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

// ------------------------------------------------------ split-K workspace
// fp32 partials of the tlds variants with S > 1: one buffer per device,
// allocated (kWsInit bytes, or more when a call needs it) by the first call
// on the device that is not under graph capture, and kept for the life of
// the process.  Calls on one stream are ordered, so they share it safely;
// calls that run concurrently on different streams of one device race on it.
constexpr size_t kWsCap = 256ull << 20;
constexpr size_t kWsInit = 64ull << 20;
constexpr size_t kCntBytes = (size_t)kSplitCounters * sizeof(unsigned);  // counters precede the partials
std::mutex g_ws_mu;
std::map<int, std::pair<void*, size_t>> g_ws;

bool capturing(hipStream_t s) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(s, &cs) != hipSuccess) {
    (void)hipGetLastError();
    return false;
  }
  return cs != hipStreamCaptureStatusNone;
}

float* workspace(hipStream_t s, size_t bytes, std::string* why) {
  if (bytes > kWsCap) {
    *why = "split-K partials of " + std::to_string(bytes) + " bytes exceed the " + std::to_string(kWsCap) +
           "-byte workspace cap";
    return nullptr;
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    *why = "no current device";
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_ws_mu);
  auto& e = g_ws[dev];
  if (e.first && e.second >= bytes + kCntBytes) return static_cast<float*>(e.first);
  if (capturing(s)) {
    *why = "the split-K workspace must be allocated outside graph capture (make one call eagerly first)";
    return nullptr;
  }
  if (e.first) {
    (void)hipDeviceSynchronize();   // the old buffer may still be in use
    (void)hipFree(e.first);
    e = {nullptr, 0};
  }
  const size_t want = std::max(bytes + kCntBytes, kWsInit);
  void* p = nullptr;
  if (hipMalloc(&p, want) != hipSuccess) {
    (void)hipGetLastError();
    *why = "hipMalloc of the split-K workspace failed";
    return nullptr;
  }
  // the arrival counters start at zero; each launch leaves them at zero
  if (hipMemset(p, 0, kCntBytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(p);
    *why = "clearing the split-K counters failed";
    return nullptr;
  }
  e = {p, want};
  return static_cast<float*>(p);
}

// The first call on a device (outside capture) allocates the workspace so
// that later captured calls find it.
void prime_workspace(hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return;
  }
  {
    std::lock_guard<std::mutex> lk(g_ws_mu);
    if (g_ws.count(dev)) return;
  }
  std::string why;
  (void)workspace(s, kWsInit, &why);
}

skg_status launch(int op, int v, const Args& a_in, hipStream_t s) {
  Args a = a_in;
  if (a.K == 0) {
    const size_t n = (size_t)a.M * a.N;
    const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_kernel, dim3(grid), dim3(256), 0, s, static_cast<unsigned short*>(a.y), n);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? SKG_OK : fail(SKG_ELAUNCH, "zero fill launch: %s", hipGetErrorString(e));
  }
  const LaunchFn fn = v >= 0 ? variant_fn(op, v, a.M) : nullptr;
  if (fn && kVariants[v].family == FAM_TLDS) {
    const size_t need = (size_t)tlds_ws_bytes(op, kVariants[v].p1, a.M, a.N);
    if (need) {
      const int fm = a.M > kMaxBucket ? kNumTileFM - 1 : tile_fm_index(a.M);
      if (tlds_tiles(kVariants[v].p0, kVariants[v].p4 / kVariants[v].p5, tlds_fm(kTileFM[fm], kVariants[v].p3), a.M,
                     a.N) >
          (unsigned long long)kSplitCounters)
        return fail(SKG_EUNSUPPORTED, "%s: more output tiles than split-K counters", kVariants[v].name);
      std::string why;
      float* base = workspace(s, need, &why);
      if (!base) return fail(SKG_EUNSUPPORTED, "%s: %s", kVariants[v].name, why.c_str());
      a.cnt = reinterpret_cast<unsigned*>(base);
      a.ws = reinterpret_cast<float*>(reinterpret_cast<char*>(base) + kCntBytes);
    }
  }
  if (fn && op == OP_A8W8 && kVariants[v].family == FAM_GEMV) {
    const size_t smem = (size_t)(kGemvMT[gemv_mt_index(a.M)] + 1) * a.kb * sizeof(float);
    if (smem > 64 * 1024)
      return fail(SKG_EUNSUPPORTED, "K=%d needs %zu bytes of A8W8 scale staging (limit 65536)", a.K, smem);
  }
  if (!fn)
    return fail(SKG_EUNSUPPORTED, "variant %s is not compiled for %s at M=%d", v >= 0 ? kVariants[v].name : "(none)",
                op_name(op), a.M);
  const hipError_t e = fn(a, s);
  if (e != hipSuccess)
    return fail(SKG_ELAUNCH, "%s %s launch: %s", op_name(op), kVariants[v].name, hipGetErrorString(e));
  return SKG_OK;
}

skg_status run_op(int op, const void* x, const void* w, const float* s0, const float* s1, void* y, int M, int N,
                  int K, hipStream_t s, float* xs_out = nullptr) {
  const int base = op_base(op);
  Args a{x, w, s0, s1, y, M, N, K, (K + 127) / 128, nullptr, nullptr, base == OP_A8W8Q ? xs_out : nullptr};
  if (base != OP_FP8T && base != OP_A8W8) a.s0 = nullptr;
  if (base != OP_A8W8 && base != OP_A8W8Q) a.s1 = nullptr;
  if (skg_status st = validate(op, a)) return st;
  if (M == 0 || N == 0) return SKG_OK;
  prime_workspace(s);
  const Decision d = decide(op, M, N, K);
  skg_status st = launch(op, d.variant, a, s);
  if (st == SKG_EUNSUPPORTED && d.variant >= 0 && kVariants[d.variant].family == FAM_TLDS) {
    // no split-K workspace here (e.g. first call under graph capture): the
    // untuned default without a K split needs none
    const int fb = default_variant_no_ws(op, M, N, K);
    if (fb >= 0 && fb != d.variant) st = launch(op, fb, a, s);
  }
  return st;
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
  return run_op(OP_BF16, x, W, scales, nullptr, y, M, N, K, stream);
}

skg_status skinny_gemm_gated(const void* x, const void* W, const float* scales, void* y, int M, int N, int K,
                             hipStream_t stream) {
  return run_op(OP_GATED, x, W, scales, nullptr, y, M, N, K, stream);
}

skg_status skinny_gemm_fp8_tensor(const void* x, const void* W, const float* scales, void* y, int M, int N, int K,
                                  hipStream_t stream) {
  return run_op(OP_FP8T, x, W, scales, nullptr, y, M, N, K, stream);
}

skg_status skinny_gemm_a8w8_block(const void* x, const void* W, const float* x_scales, const float* w_scales,
                                  void* y, int M, int N, int K, hipStream_t stream) {
  return run_op(OP_A8W8, x, W, x_scales, w_scales, y, M, N, K, stream);
}

skg_status skinny_gemm_a8w8_block_quant(const void* x, const void* W, const float* w_scales, float* x_scales_out,
                                        void* y, int M, int N, int K, hipStream_t stream) {
  return run_op(OP_A8W8Q, x, W, nullptr, w_scales, y, M, N, K, stream, x_scales_out);
}

skg_status skinny_gemm_bf16_packed(const void* x, const void* W_packed, const float* scales, void* y, int M, int N,
                                   int K, hipStream_t stream) {
  return run_op(OP_PACKED + OP_BF16, x, W_packed, scales, nullptr, y, M, N, K, stream);
}

skg_status skinny_gemm_gated_packed(const void* x, const void* W_packed, const float* scales, void* y, int M, int N,
                                    int K, hipStream_t stream) {
  return run_op(OP_PACKED + OP_GATED, x, W_packed, scales, nullptr, y, M, N, K, stream);
}

skg_status skinny_gemm_fp8_tensor_packed(const void* x, const void* W_packed, const float* scales, void* y, int M,
                                         int N, int K, hipStream_t stream) {
  return run_op(OP_PACKED + OP_FP8T, x, W_packed, scales, nullptr, y, M, N, K, stream);
}

skg_status skinny_gemm_a8w8_block_packed(const void* x, const void* W_packed, const float* x_scales,
                                         const float* w_scales, void* y, int M, int N, int K, hipStream_t stream) {
  return run_op(OP_PACKED + OP_A8W8, x, W_packed, x_scales, w_scales, y, M, N, K, stream);
}

skg_status skinny_gemm_a8w8_block_quant_packed(const void* x, const void* W_packed, const float* w_scales,
                                               float* x_scales_out, void* y, int M, int N, int K,
                                               hipStream_t stream) {
  return run_op(OP_PACKED + OP_A8W8Q, x, W_packed, nullptr, w_scales, y, M, N, K, stream, x_scales_out);
}

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
  g_table_tried = true;
  Identity id;
  std::string product;
  if (!self_identity(&id, &product)) {
    g_table.clear();
    return fail(SKG_ETABLE, "no HIP device: cannot establish the table identity");
  }
  std::string p;
  if (path && *path) p = path;
  else if (const char* e = std::getenv("SKINNY_GEMM_TABLE"); e && *e) p = e;
  else p = self_dir() + "/configs/" + id.arch + "/skinny_gemm.json";
  std::string err;
  if (g_table.load(p, id, &err) != 0) return fail(SKG_ETABLE, "%s", err.c_str());
  return SKG_OK;
}

skg_status skinny_gemm_load_table_as(const char* path, const char* identity) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_table_tried = true;
  Identity id;
  if (!identity || !Identity::parse(identity, &id)) {
    g_table.clear();
    return fail(SKG_EINVAL, "identity must read arch=..;hip=..;cc=..;space=..");
  }
  if (!path || !*path) {
    g_table.clear();
    return SKG_OK;  // explicit "no table"
  }
  std::string err;
  if (g_table.load(path, id, &err) != 0) return fail(SKG_ETABLE, "%s", err.c_str());
  return SKG_OK;
}

skg_status skinny_gemm_identity(char* buf, int len) {
  Identity id;
  if (!self_identity(&id, nullptr)) return fail(SKG_EUNSUPPORTED, "no HIP device");
  return copy_out(id.str(), buf, len);
}

int skinny_gemm_table_status(char* buf, int len) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (buf && len > 0) std::snprintf(buf, (size_t)len, "%s", g_table.status().c_str());
  return g_table.engaged() ? 1 : 0;
}

skg_status skinny_gemm_query(int op, int M, int N, int K, char* buf, int len) {
  if (!op_name(op)) return fail(SKG_EINVAL, "unknown op %d", op);
  if (M <= 0 || N <= 0 || K < 0) return fail(SKG_EINVAL, "query needs M, N > 0 and K >= 0");
  const Decision d = decide(op, M, N, K);
  if (d.variant < 0) return fail(SKG_EUNSUPPORTED, "no variant for M=%d", M);
  return copy_out(std::string(kVariants[d.variant].name) + " " + d.source, buf, len);
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
  Args a{x, W, s0, s1, y, M, N, K, (K + 127) / 128, nullptr, nullptr, nullptr};
  const int base = op_base(op);
  if (base == OP_A8W8Q) a.xs_out = const_cast<float*>(s0);   // its s0 is the x-scale output
  if (base != OP_FP8T && base != OP_A8W8) a.s0 = nullptr;
  if (base != OP_A8W8 && base != OP_A8W8Q) a.s1 = nullptr;
  if (skg_status st = validate(op, a)) return st;
  if (M == 0 || N == 0) return SKG_OK;
  if (!variant_supports(op, variant, M))
    return fail(SKG_EUNSUPPORTED, "variant %s does not run %s at M=%d", kVariants[variant].name, op_name(op), M);
  return launch(op, variant, a, stream);
}

}  // extern "C"
