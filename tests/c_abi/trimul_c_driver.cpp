// A plain C-ABI consumer of libtrimul.so: no Python, no torch. Reads the
// inputs of one call as raw bf16 bit patterns from a directory, allocates
// device buffers with the HIP runtime, sizes the workspace with
// trimul_workspace_bytes, runs trimul_forward on a stream it creates, and
// writes the output's bits back.
//
// usage: trimul_c_driver DIR B N C DIRECTION(0|1) HAS_MASK HAS_BIAS
//   DIR/x.bin [B,N,N,C], DIR/mask.bin [B,N,N] (if HAS_MASK), DIR/<param>.bin for
//   the twelve parameters (the four projection biases only if HAS_BIAS);
//   writes DIR/out.bin [B,N,N,C]. Exit status 0 on success.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "trimul.h"

static bool read_file(const std::string& path, std::vector<unsigned short>& v, size_t n) {
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f) return false;
  v.resize(n);
  const size_t got = std::fread(v.data(), 2, n, f);
  std::fclose(f);
  return got == n;
}

static void* upload(const std::vector<unsigned short>& v) {
  void* d = nullptr;
  if (hipMalloc(&d, v.size() * 2) != hipSuccess) return nullptr;
  if (hipMemcpy(d, v.data(), v.size() * 2, hipMemcpyHostToDevice) != hipSuccess) return nullptr;
  return d;
}

int main(int argc, char** argv) {
  if (argc != 8) {
    std::fprintf(stderr, "usage: %s DIR B N C DIRECTION HAS_MASK HAS_BIAS\n", argv[0]);
    return 2;
  }
  const std::string dir = argv[1];
  const int B = std::atoi(argv[2]), N = std::atoi(argv[3]), C = std::atoi(argv[4]);
  const int direction = std::atoi(argv[5]);
  const bool has_mask = std::atoi(argv[6]) != 0, has_bias = std::atoi(argv[7]) != 0;
  const size_t pairs = size_t(B) * N * N;

  struct Param {
    const char* name;
    size_t n;
    bool optional;
  } params[] = {
      {"norm_in_weight", size_t(C), false}, {"norm_in_bias", size_t(C), false},
      {"p_in_weight", size_t(2 * C) * C, false}, {"p_in_bias", size_t(2 * C), true},
      {"g_in_weight", size_t(2 * C) * C, false}, {"g_in_bias", size_t(2 * C), true},
      {"norm_out_weight", size_t(C), false}, {"norm_out_bias", size_t(C), false},
      {"p_out_weight", size_t(C) * C, false}, {"p_out_bias", size_t(C), true},
      {"g_out_weight", size_t(C) * C, false}, {"g_out_bias", size_t(C), true},
  };
  std::vector<unsigned short> host;
  void* dev[12] = {};
  for (int i = 0; i < 12; ++i) {
    if (params[i].optional && !has_bias) continue;
    if (!read_file(dir + "/" + params[i].name + ".bin", host, params[i].n)) {
      std::fprintf(stderr, "cannot read %s\n", params[i].name);
      return 1;
    }
    if (!(dev[i] = upload(host))) return 1;
  }
  if (!read_file(dir + "/x.bin", host, pairs * C)) return 1;
  void* x = upload(host);
  void* mask = nullptr;
  if (has_mask) {
    if (!read_file(dir + "/mask.bin", host, pairs)) return 1;
    mask = upload(host);
  }
  void* out = nullptr;
  const size_t ws_bytes = trimul_workspace_bytes(B, N, C, direction);
  void* ws = nullptr;
  if (!x || hipMalloc(&out, pairs * C * 2) != hipSuccess || ws_bytes == 0 ||
      hipMalloc(&ws, ws_bytes) != hipSuccess)
    return 1;
  hipStream_t stream;
  if (hipStreamCreate(&stream) != hipSuccess) return 1;

  const int st = trimul_forward(x, mask, dev[0], dev[1], dev[2], dev[3], dev[4], dev[5], dev[6], dev[7],
                                dev[8], dev[9], dev[10], dev[11], B, N, C, C, direction, 1e-5f, out,
                                ws, ws_bytes, stream);
  if (st != TRIMUL_OK) {
    std::fprintf(stderr, "trimul_forward: status %d: %s\n", st, trimul_last_error());
    return 1;
  }
  if (hipStreamSynchronize(stream) != hipSuccess) return 1;
  host.resize(pairs * C);
  if (hipMemcpy(host.data(), out, pairs * C * 2, hipMemcpyDeviceToHost) != hipSuccess) return 1;
  FILE* f = std::fopen((dir + "/out.bin").c_str(), "wb");
  if (!f || std::fwrite(host.data(), 2, host.size(), f) != host.size()) return 1;
  std::fclose(f);
  std::printf("trimul_c_driver: %s, B=%d N=%d c=%d direction=%d ok\n", trimul_version(), B, N, C, direction);
  return 0;
}
