// C ABI of the gfx950 triangle multiplicative update: argument rules, the
// workspace layout, the device check, and the three launches.
//
// Argument rules follow the page "Triangle Multiplicative Update (SM100 /
// SM103 / SM107)", section "Served today, and the typed declines" (widths,
// required parameters, aliasing as byte ranges before any launch, 32-bit
// extents), re-targeted to gfx950. The workspace holds the channel-major a, b
// and y planes (sections "Overview" and "Prepared class API").

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "trimul.h"
#include "trimul_kernels.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return TRIMUL_OK;
}

constexpr long long kLimit = 1LL << 31;

long long n_pad_of(long long N) { return (N + 63) / 64 * 64; }

size_t plane_bytes(int B, int N, int c) {
  const size_t e = size_t(c) * size_t(B) * size_t(N) * size_t(n_pad_of(N));
  return (e * 2 + 255) / 256 * 256;
}

// Shape rules shared by every entry point (no pointers, no device).
int check_shape(int B, int N, int c_z, int c, int direction) {
  if (direction != TRIMUL_OUTGOING && direction != TRIMUL_INCOMING)
    return fail(TRIMUL_E_INVALID, "direction must be 0 (outgoing) or 1 (incoming), got %d", direction);
  if (B < 1 || N < 1) return fail(TRIMUL_E_INVALID, "B and N must be >= 1 (got B=%d, N=%d)", B, N);
  if (c_z <= 0 || c_z % 32 != 0) return fail(TRIMUL_E_INVALID, "c_z must be a positive multiple of 32, got %d", c_z);
  if (c <= 0) return fail(TRIMUL_E_INVALID, "c must be positive, got %d", c);
  if (c_z != c)
    return fail(TRIMUL_E_UNSUPPORTED, "c_z != c (c_z=%d, c=%d) is outside the kernel envelope", c_z, c);
  if (c != 128 && c != 256)
    return fail(TRIMUL_E_UNSUPPORTED, "c_z = c must be 128 or 256, got %d", c);
  const long long xe = (long long)B * N * N * c_z;
  const long long pe = 2LL * c * B * N * n_pad_of(N);
  if (xe >= kLimit)
    return fail(TRIMUL_E_UNSUPPORTED, "extent B*N*N*c_z = %lld is not below 2^31", xe);
  if (pe >= kLimit)
    return fail(TRIMUL_E_UNSUPPORTED, "extent 2*c*B*N*n_pad = %lld is not below 2^31", pe);
  return ok();
}

struct Range {
  const char* name;
  uintptr_t lo, hi;  // [lo, hi)
};

bool overlaps(const Range& a, const Range& b) {
  return a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

int check_args(const void* x, const void* mask, const void* norm_in_w, const void* norm_in_b,
               const void* p_in_w, const void* p_in_b, const void* g_in_w, const void* g_in_b,
               const void* norm_out_w, const void* norm_out_b, const void* p_out_w,
               const void* p_out_b, const void* g_out_w, const void* g_out_b, int B, int N,
               int c_z, int c, int direction, float eps, const void* out, const void* workspace,
               size_t workspace_bytes) {
  int st = check_shape(B, N, c_z, c, direction);
  if (st != TRIMUL_OK) return st;
  if (!(eps >= 0.0f) || eps != eps || eps > 3.0e38f)
    return fail(TRIMUL_E_INVALID, "eps must be finite and >= 0");
  struct Req {
    const char* name;
    const void* p;
  } req[] = {{"x", x},           {"norm_in_weight", norm_in_w}, {"norm_in_bias", norm_in_b},
             {"p_in_weight", p_in_w}, {"g_in_weight", g_in_w}, {"norm_out_weight", norm_out_w},
             {"norm_out_bias", norm_out_b}, {"p_out_weight", p_out_w}, {"g_out_weight", g_out_w},
             {"out", out},       {"workspace", workspace}};
  for (const Req& r : req)
    if (r.p == nullptr) return fail(TRIMUL_E_INVALID, "%s is required (got NULL)", r.name);

  const size_t pairs = size_t(B) * N * N;
  const size_t need = trimul_workspace_bytes(B, N, c, direction);
  if (workspace_bytes < need)
    return fail(TRIMUL_E_INVALID, "workspace too small: %zu bytes given, %zu needed", workspace_bytes, need);

  Range rd[] = {
      {"x", uintptr_t(x), uintptr_t(x) + pairs * c_z * 2},
      {"mask", uintptr_t(mask), mask ? uintptr_t(mask) + pairs * 2 : uintptr_t(mask)},
      {"norm_in_weight", uintptr_t(norm_in_w), uintptr_t(norm_in_w) + size_t(c_z) * 2},
      {"norm_in_bias", uintptr_t(norm_in_b), uintptr_t(norm_in_b) + size_t(c_z) * 2},
      {"p_in_weight", uintptr_t(p_in_w), uintptr_t(p_in_w) + size_t(2 * c) * c_z * 2},
      {"p_in_bias", uintptr_t(p_in_b), p_in_b ? uintptr_t(p_in_b) + size_t(2 * c) * 2 : uintptr_t(p_in_b)},
      {"g_in_weight", uintptr_t(g_in_w), uintptr_t(g_in_w) + size_t(2 * c) * c_z * 2},
      {"g_in_bias", uintptr_t(g_in_b), g_in_b ? uintptr_t(g_in_b) + size_t(2 * c) * 2 : uintptr_t(g_in_b)},
      {"norm_out_weight", uintptr_t(norm_out_w), uintptr_t(norm_out_w) + size_t(c) * 2},
      {"norm_out_bias", uintptr_t(norm_out_b), uintptr_t(norm_out_b) + size_t(c) * 2},
      {"p_out_weight", uintptr_t(p_out_w), uintptr_t(p_out_w) + size_t(c_z) * c * 2},
      {"p_out_bias", uintptr_t(p_out_b), p_out_b ? uintptr_t(p_out_b) + size_t(c_z) * 2 : uintptr_t(p_out_b)},
      {"g_out_weight", uintptr_t(g_out_w), uintptr_t(g_out_w) + size_t(c_z) * c_z * 2},
      {"g_out_bias", uintptr_t(g_out_b), g_out_b ? uintptr_t(g_out_b) + size_t(c_z) * 2 : uintptr_t(g_out_b)},
  };
  Range wr[] = {
      {"out", uintptr_t(out), uintptr_t(out) + pairs * c_z * 2},
      {"workspace", uintptr_t(workspace), uintptr_t(workspace) + need},
  };
  // Tensors are read or written in 16-byte vectors; the mask and the
  // projection biases are read one element at a time.
  for (const Range& r : rd) {
    const bool scalar = !std::strcmp(r.name, "mask") || std::strstr(r.name, "_bias") != nullptr;
    const bool ln_vec = !std::strncmp(r.name, "norm_", 5);
    const uintptr_t align = (scalar && !ln_vec) ? 2 : 16;
    if (r.lo % align != 0) return fail(TRIMUL_E_INVALID, "%s must be %d-byte aligned", r.name, int(align));
  }
  for (const Range& r : wr)
    if (r.lo % 16 != 0) return fail(TRIMUL_E_INVALID, "%s must be 16-byte aligned", r.name);
  for (const Range& w : wr)
    for (const Range& r : rd)
      if (overlaps(w, r))
        return fail(TRIMUL_E_INVALID, "%s overlaps %s as byte ranges (must be disjoint)", w.name, r.name);
  if (overlaps(wr[0], wr[1])) return fail(TRIMUL_E_INVALID, "out overlaps workspace as byte ranges");
  return ok();
}

// Per-device facts, taken once per device.
struct DeviceInfo {
  bool known = false;
  bool gfx950 = false;
  int cus = 0;
  char arch[64] = {0};
};
constexpr int kMaxDevices = 64;
DeviceInfo g_dev[kMaxDevices];
std::mutex g_dev_mu;

int device_info(int dev, DeviceInfo& out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(TRIMUL_E_DEVICE, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.known) {
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess)
      return fail(TRIMUL_E_DEVICE, "hipGetDeviceProperties(%d): %s", dev, hipGetErrorString(e));
    std::snprintf(d.arch, sizeof(d.arch), "%s", prop.gcnArchName);
    d.gfx950 = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.known = true;
  }
  out = d;
  return TRIMUL_OK;
}

int current_device_check(DeviceInfo& info) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TRIMUL_E_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  int st = device_info(dev, info);
  if (st != TRIMUL_OK) return st;
  if (!info.gfx950)
    return fail(TRIMUL_E_UNSUPPORTED, "device %d is %s; only gfx950 (MI355X) is served", dev, info.arch);
  return TRIMUL_OK;
}

typedef const uint16_t* cbf;

int run(int first_stage, int last_stage, const void* x, const void* mask, const void* norm_in_w,
        const void* norm_in_b, const void* p_in_w, const void* p_in_b, const void* g_in_w,
        const void* g_in_b, const void* norm_out_w, const void* norm_out_b, const void* p_out_w,
        const void* p_out_b, const void* g_out_w, const void* g_out_b, int B, int N, int c_z,
        int c, int direction, float eps, void* out, void* workspace, size_t workspace_bytes,
        void* stream) {
  int st = check_args(x, mask, norm_in_w, norm_in_b, p_in_w, p_in_b, g_in_w, g_in_b, norm_out_w,
                      norm_out_b, p_out_w, p_out_b, g_out_w, g_out_b, B, N, c_z, c, direction, eps,
                      out, workspace, workspace_bytes);
  if (st != TRIMUL_OK) return st;
  DeviceInfo info;
  st = current_device_check(info);
  if (st != TRIMUL_OK) return st;

  const int n_pad = int(n_pad_of(N));
  const size_t pb = plane_bytes(B, N, c);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  uint16_t* plane_a = reinterpret_cast<uint16_t*>(ws);
  uint16_t* plane_b = reinterpret_cast<uint16_t*>(ws + pb);
  uint16_t* plane_y = reinterpret_cast<uint16_t*>(ws + 2 * pb);
  hipStream_t s = static_cast<hipStream_t>(stream);

  for (int stage = first_stage; stage <= last_stage; ++stage) {
    hipError_t e = hipSuccess;
    if (stage == 1) {
      trimul::K1Args a;
      a.x = cbf(x);
      a.mask = cbf(mask);
      a.ln_w = cbf(norm_in_w);
      a.ln_b = cbf(norm_in_b);
      a.p_in = cbf(p_in_w);
      a.p_in_b = cbf(p_in_b);
      a.g_in = cbf(g_in_w);
      a.g_in_b = cbf(g_in_b);
      a.plane_a = plane_a;
      a.plane_b = plane_b;
      a.B = B;
      a.N = N;
      a.n_pad = n_pad;
      a.c_z = c_z;
      a.c = c;
      a.incoming = direction == TRIMUL_INCOMING;
      a.nchunk = (N + 63) / 64;
      a.ntiles = trimul::k1_tiles(B, N);
      a.div_nchunk = trimul::make_fast_div(uint32_t(a.nchunk));
      a.div_N = trimul::make_fast_div(uint32_t(N));
      a.eps = eps;
      const int groups = c / 128;
      int grid = info.cus / groups;
      if (grid < 1) grid = 1;
      if (grid > a.ntiles) grid = a.ntiles;
      e = trimul::launch_k1(a, grid, s);
    } else if (stage == 2) {
      trimul::K2Args a;
      a.plane_a = plane_a;
      a.plane_b = plane_b;
      a.plane_y = plane_y;
      a.B = B;
      a.N = N;
      a.n_pad = n_pad;
      a.c = c;
      trimul::k2_plan(a);
      e = trimul::launch_k2(a, info.cus, s);
    } else {
      trimul::K3Args a;
      a.plane_y = plane_y;
      a.x = cbf(x);
      a.ln_in_w = cbf(norm_in_w);
      a.ln_in_b = cbf(norm_in_b);
      a.ln_out_w = cbf(norm_out_w);
      a.ln_out_b = cbf(norm_out_b);
      a.p_out = cbf(p_out_w);
      a.p_out_b = cbf(p_out_b);
      a.g_out = cbf(g_out_w);
      a.g_out_b = cbf(g_out_b);
      a.out = static_cast<uint16_t*>(out);
      a.B = B;
      a.N = N;
      a.n_pad = n_pad;
      a.c_z = c_z;
      a.c = c;
      a.nchunk = (N + 63) / 64;
      a.ntiles = trimul::k3_tiles(B, N);
      a.div_nchunk = trimul::make_fast_div(uint32_t(a.nchunk));
      a.eps = eps;
      int grid = info.cus;
      if (grid > a.ntiles) grid = a.ntiles;
      e = trimul::launch_k3(a, grid, s);
    }
    if (e != hipSuccess) return fail(TRIMUL_E_DEVICE, "stage %d launch failed: %s", stage, hipGetErrorString(e));
  }
  return ok();
}

// ---- fixed device scratch for trimul_forward_noalloc ----
//
// The a, b and y planes of the allocation-free entry point live in this
// file-scope device array, one copy per GPU, held until the process ends. In
// host code `scratch` names a host-side stand-in, not a device address: the
// device address is taken once per device with hipGetSymbolAddress (with that
// device current) and only that pointer is ever passed to the kernels.
constexpr size_t kScratchBytes = size_t(TRIMUL_NOALLOC_SCRATCH_BYTES);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

void* g_scratch_ptr[kMaxDevices] = {};
std::mutex g_scratch_mu;

// The current device's copy of `scratch` (looked up on the first call per
// device and kept); nullptr with the reason in g_err on failure.
void* scratch_for_current_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    fail(TRIMUL_E_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    fail(TRIMUL_E_DEVICE, "device index %d out of range", dev);
    return nullptr;
  }
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      fail(TRIMUL_E_DEVICE, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
           hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

struct trimul_graph_s {
  hipGraphExec_t exec;
  int device;
};

extern "C" {

const char* trimul_version(void) { return "trimul-gfx950 0.1.0"; }

const char* trimul_last_error(void) { return g_err.c_str(); }

int trimul_n_pad(int N) { return N < 0 ? 0 : int(n_pad_of(N)); }

size_t trimul_workspace_bytes(int B, int N, int c, int direction) {
  if (direction != TRIMUL_OUTGOING && direction != TRIMUL_INCOMING) return 0;
  if (B < 1 || N < 1 || c < 1) return 0;
  return 3 * plane_bytes(B, N, c);
}

int trimul_check_support(int B, int N, int c_z, int c, int direction, int device) {
  int st = check_shape(B, N, c_z, c, direction);
  if (st != TRIMUL_OK || device < 0) return st;
  DeviceInfo info;
  st = device_info(device, info);
  if (st != TRIMUL_OK) return st;
  if (!info.gfx950)
    return fail(TRIMUL_E_UNSUPPORTED, "device %d is %s; only gfx950 (MI355X) is served", device, info.arch);
  return ok();
}

int trimul_validate(const void* x, const void* mask, const void* norm_in_w, const void* norm_in_b,
                    const void* p_in_w, const void* p_in_b, const void* g_in_w, const void* g_in_b,
                    const void* norm_out_w, const void* norm_out_b, const void* p_out_w,
                    const void* p_out_b, const void* g_out_w, const void* g_out_b, int B, int N,
                    int c_z, int c, int direction, float eps, const void* out,
                    const void* workspace, size_t workspace_bytes) {
  return check_args(x, mask, norm_in_w, norm_in_b, p_in_w, p_in_b, g_in_w, g_in_b, norm_out_w,
                    norm_out_b, p_out_w, p_out_b, g_out_w, g_out_b, B, N, c_z, c, direction, eps,
                    out, workspace, workspace_bytes);
}

int trimul_forward(const void* x, const void* mask, const void* norm_in_w, const void* norm_in_b,
                   const void* p_in_w, const void* p_in_b, const void* g_in_w, const void* g_in_b,
                   const void* norm_out_w, const void* norm_out_b, const void* p_out_w,
                   const void* p_out_b, const void* g_out_w, const void* g_out_b, int B, int N,
                   int c_z, int c, int direction, float eps, void* out, void* workspace,
                   size_t workspace_bytes, void* stream) {
  return run(1, 3, x, mask, norm_in_w, norm_in_b, p_in_w, p_in_b, g_in_w, g_in_b, norm_out_w,
             norm_out_b, p_out_w, p_out_b, g_out_w, g_out_b, B, N, c_z, c, direction, eps, out,
             workspace, workspace_bytes, stream);
}

int trimul_forward_stage(int stage, const void* x, const void* mask, const void* norm_in_w,
                         const void* norm_in_b, const void* p_in_w, const void* p_in_b,
                         const void* g_in_w, const void* g_in_b, const void* norm_out_w,
                         const void* norm_out_b, const void* p_out_w, const void* p_out_b,
                         const void* g_out_w, const void* g_out_b, int B, int N, int c_z, int c,
                         int direction, float eps, void* out, void* workspace,
                         size_t workspace_bytes, void* stream) {
  if (stage < 1 || stage > 3) return fail(TRIMUL_E_INVALID, "stage must be 1, 2 or 3, got %d", stage);
  return run(stage, stage, x, mask, norm_in_w, norm_in_b, p_in_w, p_in_b, g_in_w, g_in_b,
             norm_out_w, norm_out_b, p_out_w, p_out_b, g_out_w, g_out_b, B, N, c_z, c, direction,
             eps, out, workspace, workspace_bytes, stream);
}

int trimul_forward_noalloc(const void* x, const void* mask, const void* norm_in_w,
                           const void* norm_in_b, const void* p_in_w, const void* p_in_b,
                           const void* g_in_w, const void* g_in_b, const void* norm_out_w,
                           const void* norm_out_b, const void* p_out_w, const void* p_out_b,
                           const void* g_out_w, const void* g_out_b, int B, int N, int c_z, int c,
                           int direction, float eps, void* out, void* stream) {
  int st = check_shape(B, N, c_z, c, direction);
  if (st != TRIMUL_OK) return st;
  const size_t need = trimul_workspace_bytes(B, N, c, direction);
  if (need > kScratchBytes)
    return fail(TRIMUL_E_UNSUPPORTED,
                "B=%d, N=%d, c=%d needs %zu bytes of planes, above the %zu-byte fixed scratch of "
                "trimul_forward_noalloc; call trimul_forward with a workspace",
                B, N, c, need, kScratchBytes);
  DeviceInfo info;
  st = current_device_check(info);
  if (st != TRIMUL_OK) return st;
  void* ws = scratch_for_current_device();
  if (ws == nullptr) return TRIMUL_E_DEVICE;
  return run(1, 3, x, mask, norm_in_w, norm_in_b, p_in_w, p_in_b, g_in_w, g_in_b, norm_out_w,
             norm_out_b, p_out_w, p_out_b, g_out_w, g_out_b, B, N, c_z, c, direction, eps, out,
             ws, kScratchBytes, stream);
}

int trimul_graph_create(const void* x, const void* mask, const void* norm_in_w,
                        const void* norm_in_b, const void* p_in_w, const void* p_in_b,
                        const void* g_in_w, const void* g_in_b, const void* norm_out_w,
                        const void* norm_out_b, const void* p_out_w, const void* p_out_b,
                        const void* g_out_w, const void* g_out_b, int B, int N, int c_z, int c,
                        int direction, float eps, void* out, void* workspace,
                        size_t workspace_bytes, trimul_graph_t* graph) {
  if (!graph) return fail(TRIMUL_E_INVALID, "graph (the handle's destination) is NULL");
  *graph = nullptr;
  int st = check_args(x, mask, norm_in_w, norm_in_b, p_in_w, p_in_b, g_in_w, g_in_b, norm_out_w,
                      norm_out_b, p_out_w, p_out_b, g_out_w, g_out_b, B, N, c_z, c, direction, eps,
                      out, workspace, workspace_bytes);
  if (st != TRIMUL_OK) return st;
  // device properties are read (and cached) before the capture starts
  DeviceInfo info;
  st = current_device_check(info);
  if (st != TRIMUL_OK) return st;
  int dev = -1;
  hipGetDevice(&dev);

  hipStream_t cs = nullptr;
  hipError_t e = hipStreamCreateWithFlags(&cs, hipStreamNonBlocking);
  if (e != hipSuccess) return fail(TRIMUL_E_DEVICE, "hipStreamCreateWithFlags: %s", hipGetErrorString(e));
  e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
  if (e != hipSuccess) {
    hipStreamDestroy(cs);
    return fail(TRIMUL_E_DEVICE, "hipStreamBeginCapture: %s", hipGetErrorString(e));
  }
  st = run(1, 3, x, mask, norm_in_w, norm_in_b, p_in_w, p_in_b, g_in_w, g_in_b, norm_out_w,
           norm_out_b, p_out_w, p_out_b, g_out_w, g_out_b, B, N, c_z, c, direction, eps, out,
           workspace, workspace_bytes, cs);
  const std::string run_err = g_err;
  hipGraph_t g = nullptr;
  e = hipStreamEndCapture(cs, &g);   // always end the capture, whatever run() returned
  hipStreamDestroy(cs);
  if (st != TRIMUL_OK) {
    if (g) hipGraphDestroy(g);
    return fail(st, "capture: %s", run_err.c_str());
  }
  if (e != hipSuccess || !g) return fail(TRIMUL_E_DEVICE, "hipStreamEndCapture: %s", hipGetErrorString(e));
  hipGraphExec_t exec = nullptr;
  e = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
  hipGraphDestroy(g);
  if (e != hipSuccess) return fail(TRIMUL_E_DEVICE, "hipGraphInstantiate: %s", hipGetErrorString(e));
  *graph = new trimul_graph_s{exec, dev};
  return ok();
}

int trimul_graph_launch(trimul_graph_t graph, void* stream) {
  if (!graph) return fail(TRIMUL_E_INVALID, "graph handle is NULL");
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TRIMUL_E_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev != graph->device)
    return fail(TRIMUL_E_INVALID, "graph was created on device %d but device %d is current", graph->device, dev);
  e = hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(TRIMUL_E_DEVICE, "hipGraphLaunch: %s", hipGetErrorString(e));
  return ok();
}

int trimul_graph_destroy(trimul_graph_t graph) {
  if (!graph) return ok();
  hipError_t e = hipGraphExecDestroy(graph->exec);
  delete graph;
  if (e != hipSuccess) return fail(TRIMUL_E_DEVICE, "hipGraphExecDestroy: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
