// The host code of the Q4_0 library -- the C ABI's argument validation and
// the GGUF reader, which parses untrusted bytes from the model's pieces --
// run under AddressSanitizer and UndefinedBehaviorSanitizer on the CPU.  The
// kernel launchers are stubs that count their calls, so no HIP kernel runs
// and no GPU is needed.
//
//   san_driver abi            every entry point with bad and good arguments
//   san_driver gguf LIST      LIST: one case per line, the ';'-separated
//                             paths of one byte stream; every table entry,
//                             metadata value and tensor of an opened file is
//                             read.  Prints one status per case.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <fstream>
#include <string>
#include <vector>

#include "q4.h"
#include "q4_kernels.h"

namespace q4 {
static int g_launches = 0;
hipError_t launch_matvec(const uint8_t*, const float*, float*, int64_t, int64_t, int64_t,
                         hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_lmhead_argmax(const uint8_t*, const float*, int32_t*, float*, float*, int64_t,
                                int64_t, int64_t, void*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
size_t lmhead_workspace_bytes(int64_t M) { return static_cast<size_t>(M) * 256; }
int64_t lmhead_noalloc_max_m() { return 64; }
hipError_t launch_lmhead_argmax_noalloc(const uint8_t*, const float*, int32_t*, float*, int64_t,
                                        int64_t, int64_t, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
const char* matvec_route(int64_t, int64_t, bool) { return "stub"; }
const char* matmul_route(int64_t, int64_t, int64_t, size_t, int, int* splits) {
  if (splits) *splits = 1;
  return "stub";
}
hipError_t launch_matmul(const uint8_t*, const float*, float*, const float*, int64_t, int64_t,
                         int64_t, void*, size_t, int, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
size_t matmul_workspace_bytes(int64_t, int64_t, int64_t, int) { return 0; }
// stub plan: the add is fused only for M > 48 (so small M in place needs workspace)
bool matmul_residual_fused(int64_t M, int64_t, int64_t, size_t, int) { return M > 48; }
size_t matmul_residual_workspace_bytes(int64_t M, int64_t N, int64_t, int) {
  return M > 48 ? 0 : static_cast<size_t>(M * N) * sizeof(float);
}
int matmul_small_per_cu() { return 1; }
void launch_matmul_small(const uint8_t*, const float*, float*, float*, int64_t, int64_t, int64_t,
                         int, int, hipStream_t) {}
hipError_t launch_embed(const uint8_t*, const int32_t*, float*, int64_t, int64_t, int64_t,
                        hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_quantize(const float*, uint8_t*, int64_t, int64_t, int32_t*, hipStream_t) {
  ++g_launches;
  return hipSuccess;
}
}  // namespace q4

static int g_fail = 0;
#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    const int before_ = q4::g_launches;                                                 \
    const int got_ = (call);                                                            \
    const bool launched_ = q4::g_launches != before_;                                   \
    if (got_ != (want) || launched_ != ((want) == Q4_OK)) {                             \
      fprintf(stderr, "FAIL line %d: %s -> %d (launched %d), want %d\n", __LINE__,     \
              #call, got_, launched_ ? 1 : 0, (want));                                  \
      ++g_fail;                                                                         \
    }                                                                                   \
  } while (0)

static int run_abi() {
  alignas(16) static float buf[256];
  alignas(16) static int32_t idx[64];
  alignas(16) static uint8_t ws[64 * 256];
  const float* mis = reinterpret_cast<const float*>(reinterpret_cast<const char*>(buf) + 4);
  const int64_t BIG = INT64_MAX, NEG = INT64_MIN;
  const int64_t sizes[] = {0, 1, 31, 32, 33, 64, 96, 3072, 12288, int64_t(1) << 22,
                           (int64_t(1) << 30) + 32, int64_t(1) << 31, int64_t(1) << 40, BIG, -1, NEG};

  // q4_matvec
  EXPECT(q4_matvec(buf, buf, buf, 1, 4, 64, nullptr), Q4_OK);
  EXPECT(q4_matvec(buf, buf, buf, 8, 4, 64, nullptr), Q4_OK);
  EXPECT(q4_matvec(nullptr, buf, buf, 1, 4, 64, nullptr), Q4_ERR_NULL);
  EXPECT(q4_matvec(buf, nullptr, buf, 1, 4, 64, nullptr), Q4_ERR_NULL);
  EXPECT(q4_matvec(buf, buf, nullptr, 1, 4, 64, nullptr), Q4_ERR_NULL);
  EXPECT(q4_matvec(buf, mis, buf, 1, 4, 64, nullptr), Q4_ERR_ALIGN);
  EXPECT(q4_matvec(buf, buf, buf, 9, 4, 64, nullptr), Q4_ERR_SHAPE);
  // q4_matmul
  EXPECT(q4_matmul(buf, buf, buf, 1500, 1280, 1280, nullptr, 0, nullptr), Q4_OK);
  EXPECT(q4_matmul(buf, buf, buf, 1500, 1280, 1280, ws, sizeof ws, nullptr), Q4_OK);
  EXPECT(q4_matmul(buf, buf, buf, 16, 64, 64, const_cast<float*>(mis), 64, nullptr), Q4_ERR_ALIGN);
  EXPECT(q4_matmul(buf, buf, buf, 16, 64, 48, nullptr, 0, nullptr), Q4_ERR_SHAPE);
  EXPECT(q4_matmul(buf, buf, nullptr, 16, 64, 64, nullptr, 0, nullptr), Q4_ERR_NULL);
  // q4_embed_rows
  EXPECT(q4_embed_rows(buf, idx, buf, 38, 131072, 3072, nullptr), Q4_OK);
  EXPECT(q4_embed_rows(buf, nullptr, buf, 1, 4, 32, nullptr), Q4_ERR_NULL);
  EXPECT(q4_embed_rows(buf, idx, buf, 0, 4, 32, nullptr), Q4_ERR_SHAPE);
  // q4_lmhead_argmax
  EXPECT(q4_lmhead_argmax(buf, buf, idx, nullptr, 1, 4, 32, ws, 256, nullptr), Q4_OK);
  EXPECT(q4_lmhead_argmax(buf, buf, idx, buf, 64, 4, 32, ws, sizeof ws, nullptr), Q4_OK);
  EXPECT(q4_lmhead_argmax(buf, buf, idx, nullptr, 2, 4, 32, ws, 256, nullptr), Q4_ERR_WORKSPACE);
  EXPECT(q4_lmhead_argmax(buf, buf, idx, nullptr, 1, 4, 32, nullptr, 256, nullptr), Q4_ERR_WORKSPACE);
  EXPECT(q4_lmhead_argmax(buf, buf, idx, nullptr, 65, 4, 32, ws, sizeof ws, nullptr), Q4_ERR_SHAPE);
  // q4_lmhead_argmax_noalloc
  EXPECT(q4_lmhead_argmax_noalloc(buf, buf, idx, buf, 64, 4, 32, nullptr), Q4_OK);
  EXPECT(q4_lmhead_argmax_noalloc(buf, buf, idx, buf, 65, 4, 32, nullptr), Q4_ERR_SHAPE);
  EXPECT(q4_lmhead_argmax_noalloc(buf, buf, nullptr, buf, 1, 4, 32, nullptr), Q4_ERR_NULL);
  EXPECT(q4_lmhead_argmax_noalloc(buf, mis, idx, buf, 1, 4, 32, nullptr), Q4_ERR_ALIGN);
  // q4_decode_chain
  {
    q4_matvec_step st[3] = {{buf, buf, buf, 64, 64}, {buf, buf, buf, 3072, 4096},
                            {buf, buf, buf, 1, 32}};
    EXPECT(q4_decode_chain(st, 3, nullptr, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                           nullptr), Q4_OK);
    EXPECT(q4_decode_chain(st, 3, buf, 131072, 3072, buf, idx, buf, buf, ws, 256, nullptr), Q4_OK);
    EXPECT(q4_decode_chain(st, 0, buf, 10, 64, buf, idx, nullptr, nullptr, ws, 256, nullptr), Q4_OK);
    EXPECT(q4_decode_chain(st, 0, nullptr, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                           nullptr), Q4_ERR_SHAPE);
    EXPECT(q4_decode_chain(nullptr, 2, nullptr, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                           nullptr), Q4_ERR_NULL);
    EXPECT(q4_decode_chain(st, 65, nullptr, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                           nullptr), Q4_ERR_SHAPE);
    EXPECT(q4_decode_chain(st, 3, buf, 131072, 3072, buf, idx, buf, buf, nullptr, 0, nullptr),
           Q4_ERR_WORKSPACE);
    EXPECT(q4_decode_chain(st, 3, buf, 131072, 3072, buf, idx, buf, const_cast<float*>(mis), ws,
                           256, nullptr), Q4_ERR_ALIGN);
    q4_matvec_step bad[2] = {{buf, buf, buf, 64, 64}, {buf, buf, buf, 64, 48}};
    EXPECT(q4_decode_chain(bad, 2, nullptr, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                           nullptr), Q4_ERR_SHAPE);
    bad[1].K = 64;
    bad[1].y = nullptr;
    EXPECT(q4_decode_chain(bad, 2, nullptr, 0, 0, nullptr, nullptr, nullptr, nullptr, nullptr, 0,
                           nullptr), Q4_ERR_NULL);
    for (int64_t a : sizes)
      for (int64_t b : sizes) {
        q4_matvec_step one = {buf, buf, buf, a, b};
        q4_decode_chain(&one, 1, buf, a, b, buf, idx, buf, buf, ws, sizeof ws, nullptr);
      }
  }
  // q4_matmul_residual: in place where the add is a second launch (the
  // stub plan: M <= 48) needs M*N floats of workspace
  EXPECT(q4_matmul_residual(buf, buf, buf, buf, 2, 16, 64, nullptr, 0, nullptr), Q4_ERR_WORKSPACE);
  EXPECT(q4_matmul_residual(buf, buf, buf, buf, 2, 16, 64, ws, 2 * 16 * 4, nullptr), Q4_OK);
  EXPECT(q4_matmul_residual(buf, buf, nullptr, buf, 2, 16, 64, ws, sizeof ws, nullptr), Q4_ERR_NULL);
  // q4_quantize
  EXPECT(q4_quantize(buf, ws, 4, 64, idx, nullptr), Q4_OK);
  EXPECT(q4_quantize(buf, ws, 4, 64, reinterpret_cast<int32_t*>(ws + 2), nullptr), Q4_ERR_ALIGN);
  EXPECT(q4_quantize(nullptr, ws, 4, 64, nullptr, nullptr), Q4_ERR_NULL);

  // Every entry point over every combination of extreme sizes: each is
  // refused or accepted without overflow (UBSan would stop the run).
  for (int64_t a : sizes)
    for (int64_t b : sizes)
      for (int64_t c : sizes) {
        q4_matvec(buf, buf, buf, a, b, c, nullptr);
        q4_matmul(buf, buf, buf, a, b, c, nullptr, 0, nullptr);
        q4_matmul_workspace_bytes(a, b, c);
        q4_matmul_residual(buf, buf, buf, buf, a, b, c, nullptr, 0, nullptr);
        q4_matmul_residual_workspace_bytes(a, b, c);
        q4_matmul_route(a, b, c, 0, nullptr);
        q4_matvec_route(b, c, 1);
        q4_embed_rows(buf, idx, buf, a, b, c, nullptr);
        q4_lmhead_argmax(buf, buf, idx, buf, a, b, c, ws, sizeof ws, nullptr);
        q4_lmhead_argmax_workspace_bytes(a, b, c);
        q4_lmhead_argmax_noalloc(buf, buf, idx, buf, a, b, c, nullptr);
        q4_quantize(buf, ws, b, c, nullptr, nullptr);
        q4_row_bytes(c);
      }
  for (int s = -3; s < 12; ++s)
    if (!q4_status_string(s)) {
      fprintf(stderr, "FAIL: status string %d\n", s);
      ++g_fail;
    }
  if (g_fail) return 1;
  puts("abi ok");
  return 0;
}

static void walk(q4_gguf* g) {
  const int64_t nm = q4_gguf_metadata_count(g);
  for (int64_t i = 0; i < nm; ++i) {
    const char* key = nullptr;
    uint32_t vt = 0;
    if (q4_gguf_metadata_key(g, i, &key, &vt) != Q4_OK) continue;
    int64_t iv;
    double fv;
    const char* sv;
    uint64_t n;
    uint32_t et;
    q4_gguf_metadata_int(g, key, &iv);
    q4_gguf_metadata_float(g, key, &fv);
    if (q4_gguf_metadata_string(g, key, &sv, &n) == Q4_OK && n) {
      volatile char c = sv[n - 1];
      (void)c;
    }
    q4_gguf_metadata_array(g, key, &et, &n);
  }
  const int64_t nt = q4_gguf_tensor_count(g);
  for (int64_t i = 0; i < nt; ++i) {
    const char* name = nullptr;
    uint32_t type = 0, nd = 0;
    int64_t dims[4];
    uint64_t off = 0, nb = 0;
    if (q4_gguf_tensor_info(g, i, &name, &type, &nd, dims, &off, &nb) != Q4_OK) continue;
    if (q4_gguf_find_tensor(g, name) != i) {
      fprintf(stderr, "FAIL: find_tensor(%s)\n", name);
      ++g_fail;
    }
    if (nb > (uint64_t(1) << 28)) continue;
    std::vector<uint8_t> dst(nb + 1);
    q4_gguf_read_tensor(g, i, dst.data(), nb);
    if (nb) q4_gguf_read_tensor(g, i, dst.data(), nb - 1);
  }
  q4_gguf_find_tensor(g, "");
  q4_gguf_version(g);
  q4_gguf_alignment(g);
  q4_gguf_data_offset(g);
}

static int run_gguf(const char* list) {
  std::ifstream in(list);
  std::string line;
  while (std::getline(in, line)) {
    std::vector<std::string> parts;
    size_t s = 0;
    for (;;) {
      const size_t e = line.find(';', s);
      parts.push_back(line.substr(s, e == std::string::npos ? std::string::npos : e - s));
      if (e == std::string::npos) break;
      s = e + 1;
    }
    std::vector<const char*> paths;
    for (auto& p : parts) paths.push_back(p.c_str());
    q4_gguf* g = nullptr;
    const int st = q4_gguf_open(paths.data(), static_cast<int64_t>(paths.size()), &g);
    if (st == Q4_OK) {
      walk(g);
      q4_gguf_close(g);
    } else if (g != nullptr) {
      fprintf(stderr, "FAIL: handle set on error\n");
      ++g_fail;
    }
    printf("%d\n", st);
  }
  return g_fail ? 1 : 0;
}

int main(int argc, char** argv) {
  if (argc >= 2 && strcmp(argv[1], "abi") == 0) return run_abi();
  if (argc >= 3 && strcmp(argv[1], "gguf") == 0) return run_gguf(argv[2]);
  fprintf(stderr, "usage: san_driver abi | gguf LIST\n");
  return 2;
}
