// Host-side driver run under AddressSanitizer and UndefinedBehaviorSanitizer
// (built and run by tests/test_sanitizers.py, CPU only): the oracle and the
// input generator on small ragged shapes with exactly sized heap buffers, and
// the C ABI's host validation (api.cpp) with every kernel launch and the four
// HIP runtime calls it makes replaced by stubs defined here, so no GPU and no
// HIP runtime is involved. Exits 0 when every check holds; a sanitizer report
// aborts the process.

#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "launch.hpp"
#include "rmsnorm_mi355x.h"

// ------------------------------------------------------------ stubs

namespace {
int g_launches = 0;
int64_t g_last_M = -1, g_last_N = -1;
}  // namespace

extern "C" hipError_t hipGetLastError(void) { return hipSuccess; }
extern "C" hipError_t hipGetDevice(int* d) {
  *d = 0;
  return hipSuccess;
}
extern "C" hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int) {
  *v = attr == hipDeviceAttributeMultiprocessorCount ? 256 : 160 * 1024;
  return hipSuccess;
}
extern "C" hipError_t hipFuncSetAttribute(const void*, hipFuncAttribute, int) {
  return hipSuccess;
}

namespace rmsn {
static hipError_t record(int64_t M, int64_t N) {
  ++g_launches;
  g_last_M = M;
  g_last_N = N;
  return hipSuccess;
}
hipError_t launch_fwd_f32(const FwdCall& c) { return record(c.M, c.N); }
hipError_t launch_fwd_f16(const FwdCall& c) { return record(c.M, c.N); }
hipError_t launch_fwd_bf16(const FwdCall& c) { return record(c.M, c.N); }
hipError_t launch_fwd_quant_f32(const FwdCall& c) { return record(c.M, c.N); }
hipError_t launch_fwd_quant_f16(const FwdCall& c) { return record(c.M, c.N); }
hipError_t launch_fwd_quant_bf16(const FwdCall& c) { return record(c.M, c.N); }
hipError_t launch_ln_fwd_f32(const FwdCall& c) { return record(c.M, c.N); }
hipError_t launch_ln_fwd_f16(const FwdCall& c) { return record(c.M, c.N); }
hipError_t launch_ln_fwd_bf16(const FwdCall& c) { return record(c.M, c.N); }
hipError_t launch_qk(const QKCall& c, int) { return record(c.tokens, c.N); }
hipError_t launch_bwd(const BwdCall& c) { return record(c.M, c.N); }
hipError_t launch_ln_bwd(const BwdCall& c) { return record(c.M, c.N); }
hipError_t noalloc_scratch(void** out) {
  static unsigned char fake[256];  // never dereferenced: the launch is a stub too
  *out = fake;
  return hipSuccess;
}
}  // namespace rmsn

// ------------------------------------------------------------ oracle / gen

extern "C" {
void gen_normal(uint64_t, uint32_t, int64_t, int64_t, int, double, int64_t, void*, int);
void gen_uniform(uint64_t, uint32_t, int64_t, double, double, int, void*, int);
uint64_t gen_splitmix64(uint64_t);
void gen_bits(uint64_t, uint32_t, int64_t, uint64_t*);
void oracle_decode(const void*, int64_t, int, double*);
void oracle_round(const double*, int64_t, int, void*);
void oracle_rmsnorm_fwd(const void*, const void*, int64_t, int64_t, float, int, int, double*,
                        void*, double*, float*, double*);
void oracle_rmsnorm_fused_add_fwd(const void*, const void*, const void*, int64_t, int64_t, float,
                                  int, int, void*, double*, void*, double*, float*, double*);
void oracle_rmsnorm_fused_add_bwd(const void*, const void*, const double*, const void*,
                                  const void*, int64_t, int64_t, int, int, double*, void*,
                                  double*, double*, double*, double*);
void oracle_rmsnorm_bwd(const void*, const void*, const double*, const void*, int64_t, int64_t,
                        int, int, double*, void*, double*, double*, double*, double*);
void oracle_rmsnorm_quant_fwd(const void*, const void*, const void*, int64_t, int64_t, float, int,
                              int, int, float, void*, uint8_t*, double*, double*, float*, float*);
void oracle_rmsnorm_heads_fwd(void*, const void*, int64_t, int64_t, int64_t, int64_t, float, int,
                              int, float*);
void oracle_layernorm_fwd(const void*, const void*, const void*, int64_t, int64_t, float, int, int,
                          double*, void*, double*, double*, float*, float*, double*);
void oracle_layernorm_bwd(const void*, const void*, const double*, const double*, const void*,
                          int64_t, int64_t, int, int, double*, void*, double*, double*, double*,
                          double*, double*, double*, double*, double*);
void oracle_rmsnorm_mx_fwd(const void*, const void*, const void*, int64_t, int64_t, float, int,
                           int, int, void*, uint8_t*, double*, uint8_t*, double*);
}

namespace {

int g_fail = 0;

void check(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "check failed at line %d: %s\n", line, what);
    ++g_fail;
  }
}
#define CHECK(x) check((x), #x, __LINE__)

size_t esize(int dt) { return dt == RMSN_F32 ? 4 : 2; }

// A storage array of n values of format dt, seeded normals.
std::vector<unsigned char> normals(int64_t rows, int64_t cols, int dt, uint64_t seed) {
  std::vector<unsigned char> v(static_cast<size_t>(rows * cols) * esize(dt));
  gen_normal(seed, 1, rows, cols, dt, 1.0, 0, v.data(), 2);
  return v;
}

std::vector<unsigned char> uniforms(int64_t n, int dt, uint64_t seed) {
  std::vector<unsigned char> v(static_cast<size_t>(n) * esize(dt));
  gen_uniform(seed, 4, n, 0.5, 1.5, dt, v.data(), 1);
  return v;
}

void run_generator() {
  for (int dt : {0, 1, 2, 3}) {
    const size_t es = dt == 3 ? 8 : esize(dt);
    std::vector<unsigned char> a(7 * 13 * es), b(5 * es);
    gen_normal(11, 2, 7, 13, dt, 100.0, 3, a.data(), 3);
    gen_uniform(11, 3, 5, -1.0, 1.0, dt, b.data(), 4);
  }
  std::vector<uint64_t> bits(9);
  gen_bits(5, 1, 9, bits.data());
  CHECK(gen_splitmix64(0) != 0);
}

void run_oracle() {
  const int pairs[][2] = {{0, 0}, {1, 1}, {1, 0}, {2, 2}, {2, 0}};
  for (const auto& p : pairs) {
    const int xd = p[0], gd = p[1];
    for (int64_t N : {1, 7, 64}) {
      const int64_t M = 3;
      auto x = normals(M, N, xd, 1 + N), r = normals(M, N, xd, 2 + N),
           dy = normals(M, N, xd, 3 + N), g = uniforms(N, gd, 4 + N);
      std::vector<double> ye(M * N), re(M), ms(M), c(M), a(M), s(N), dg(N), dxe(M * N);
      std::vector<float> rf(M), sf(M);
      std::vector<unsigned char> y(M * N * esize(xd)), h(M * N * esize(xd)), dx(M * N * esize(xd));
      oracle_rmsnorm_fwd(x.data(), g.data(), M, N, 1e-5f, xd, gd, ye.data(), y.data(), re.data(),
                         rf.data(), ms.data());
      oracle_rmsnorm_fwd(x.data(), g.data(), M, N, 0.0f, xd, gd, nullptr, nullptr, nullptr,
                         nullptr, nullptr);
      oracle_rmsnorm_fused_add_fwd(x.data(), r.data(), g.data(), M, N, 1e-5f, xd, gd, h.data(),
                                   ye.data(), y.data(), re.data(), rf.data(), ms.data());
      oracle_rmsnorm_bwd(dy.data(), x.data(), re.data(), g.data(), M, N, xd, gd, dxe.data(),
                         dx.data(), dg.data(), c.data(), a.data(), s.data());
      oracle_rmsnorm_fused_add_bwd(dy.data(), x.data(), re.data(), g.data(), r.data(), M, N, xd,
                                   gd, nullptr, dx.data(), dg.data(), nullptr, nullptr, nullptr);
      std::vector<uint8_t> q(M * N);
      std::vector<double> qe(M * N), se(M);
      for (int mode : {1, 2})
        oracle_rmsnorm_quant_fwd(x.data(), mode == 1 ? r.data() : nullptr, g.data(), M, N, 1e-5f,
                                 xd, gd, mode, 0.0125f, mode == 1 ? h.data() : nullptr, q.data(),
                                 qe.data(), se.data(), sf.data(), rf.data());
      std::vector<double> me(M), m2(M), c1(M), c2(M), a1(M), a2(M), sg(N), sb(N), db(N);
      std::vector<float> mf(M);
      oracle_layernorm_fwd(x.data(), g.data(), g.data(), M, N, 1e-5f, xd, gd, ye.data(), y.data(),
                           me.data(), m2.data(), mf.data(), rf.data(), a.data());
      oracle_layernorm_fwd(x.data(), g.data(), nullptr, M, N, 1e-5f, xd, gd, nullptr, nullptr,
                           me.data(), m2.data(), nullptr, nullptr, nullptr);
      oracle_layernorm_bwd(dy.data(), x.data(), me.data(), m2.data(), g.data(), M, N, xd, gd,
                           dxe.data(), dx.data(), dg.data(), db.data(), c1.data(), c2.data(),
                           a1.data(), a2.data(), sg.data(), sb.data());
      if (N % 32 == 0) {
        std::vector<uint8_t> sc(M * N / 32);
        std::vector<double> am(M * N / 32);
        for (int elem : {4, 5})  // e4m3, e2m1 element codes
          oracle_rmsnorm_mx_fwd(x.data(), r.data(), g.data(), M, N, 1e-5f, xd, gd, elem, h.data(),
                                q.data(), qe.data(), sc.data(), am.data());
      }
      std::vector<double> d(M * N);
      oracle_decode(x.data(), M * N, xd, d.data());
      oracle_round(d.data(), M * N, xd, y.data());
      CHECK(std::memcmp(y.data(), x.data(), y.size()) == 0);  // decode then round is exact
    }
    // Per-head forward over a strided buffer sized exactly to its last head.
    const int64_t T = 3, H = 2, D = 8, S = 20;
    const int64_t n = (T - 1) * S + H * D;
    auto buf = normals(1, n, xd, 9);
    auto g = uniforms(D, gd, 10);
    std::vector<float> rs(T * H);
    oracle_rmsnorm_heads_fwd(buf.data(), g.data(), T, H, D, S, 1e-6f, xd, gd, rs.data());
  }
}

// ------------------------------------------------------------ ABI validation

// Fake, well-separated, 256-byte-aligned device addresses: the stubs never
// dereference them.
void* addr(int k) { return reinterpret_cast<void*>(static_cast<uintptr_t>(k) << 28); }

void run_abi() {
  void *A = addr(1), *B = addr(2), *C = addr(3), *D = addr(4), *E = addr(5), *F = addr(6),
       *G = addr(7);
  float* Cf = static_cast<float*>(C);
  float* Ff = static_cast<float*>(F);
  hipStream_t st = nullptr;
  int before = g_launches;
  CHECK(rmsnorm_fwd(A, B, C, nullptr, 4, 64, 1e-5f, RMSN_BF16, RMSN_BF16, st) == RMSN_OK);
  CHECK(g_launches == before + 1 && g_last_M == 4 && g_last_N == 64);
  CHECK(rmsnorm_fwd(A, B, C, nullptr, 0, 64, 1e-5f, RMSN_BF16, RMSN_BF16, st) == RMSN_OK);
  CHECK(g_launches == before + 1);  // M == 0 launches nothing
  CHECK(rmsnorm_fwd(A, B, C, nullptr, 4, 64, 1e-5f, 7, RMSN_BF16, st) == RMSN_ERR_DTYPE);
  CHECK(rmsnorm_fwd(A, B, C, nullptr, -1, 64, 1e-5f, RMSN_BF16, RMSN_BF16, st) == RMSN_ERR_SHAPE);
  CHECK(rmsnorm_fwd(A, B, C, nullptr, 4, int64_t(RMSN_MAX_N) + 1, 1e-5f, RMSN_BF16, RMSN_BF16,
                    st) == RMSN_ERR_SHAPE);
  CHECK(rmsnorm_fwd(A, B, C, nullptr, int64_t(1) << 40, int64_t(1) << 30, 1e-5f, RMSN_BF16,
                    RMSN_BF16, st) == RMSN_ERR_SHAPE);
  CHECK(rmsnorm_fwd(nullptr, B, C, nullptr, 4, 64, 1e-5f, RMSN_BF16, RMSN_BF16, st) ==
        RMSN_ERR_NULL);
  CHECK(rmsnorm_fwd(A, B, C, nullptr, 4, 64, -1.0f, RMSN_BF16, RMSN_BF16, st) == RMSN_ERR_EPS);
  CHECK(rmsnorm_fwd(A, B, C, nullptr, 4, 64, NAN, RMSN_BF16, RMSN_BF16, st) == RMSN_ERR_EPS);
  CHECK(rmsnorm_fwd(static_cast<char*>(A) + 1, B, C, nullptr, 4, 64, 1e-5f, RMSN_BF16, RMSN_BF16,
                    st) == RMSN_ERR_ALIGN);
  CHECK(rmsnorm_fwd(A, B, static_cast<char*>(A) + 64, nullptr, 4, 64, 1e-5f, RMSN_BF16, RMSN_BF16,
                    st) == RMSN_ERR_OVERLAP);
  CHECK(rmsnorm_fwd(A, B, A, nullptr, 4, 64, 1e-5f, RMSN_BF16, RMSN_BF16, st) == RMSN_OK);
  CHECK(rmsnorm_fused_add_fwd(A, D, B, C, Ff, 4, 64, 1e-5f, RMSN_BF16, RMSN_F32, st) == RMSN_OK);
  CHECK(rmsnorm_fused_add_fwd(A, D, B, D, nullptr, 4, 64, 1e-5f, RMSN_BF16, RMSN_BF16, st) ==
        RMSN_ERR_OVERLAP);
  for (int mode = 0; mode <= 5; ++mode) {
    const int want = mode == 0 || mode == 5 ? RMSN_ERR_MODE : RMSN_OK;
    CHECK(rmsnorm_quant_fwd(A, nullptr, B, C, Ff, mode, nullptr, 4, 64, 1e-5f, RMSN_BF16,
                            RMSN_BF16, st) == want);
  }
  CHECK(rmsnorm_quant_fwd(A, nullptr, B, C, Ff, RMSN_QUANT_MXFP8, nullptr, 4, 48, 1e-5f,
                          RMSN_BF16, RMSN_BF16, st) == RMSN_ERR_SHAPE);
  CHECK(rmsnorm_qk_fwd(A, static_cast<char*>(A) + 32 * 128 * 2, B, D, 16, 32, 8, 128, 48 * 128,
                       48 * 128, 1e-6f, RMSN_BF16, RMSN_BF16, st) == RMSN_OK);
  CHECK(rmsnorm_qk_fwd(A, static_cast<char*>(A) + 2, B, D, 16, 32, 8, 128, 48 * 128, 48 * 128,
                       1e-6f, RMSN_BF16, RMSN_BF16, st) != RMSN_OK);
  CHECK(rmsnorm_qk_fwd(A, nullptr, B, nullptr, 16, 32, 0, 128, 32 * 128, 0, 1e-6f, RMSN_BF16,
                       RMSN_BF16, st) == RMSN_OK);
  CHECK(layernorm_fwd(A, B, D, C, Ff, static_cast<float*>(G), 4, 64, 1e-5f, RMSN_F16, RMSN_F16,
                      st) == RMSN_OK);
  // Backward: workspace sizes and validation.
  for (int64_t M : {1, 3, 255, 256, 257, 16384, 16385, 131072})
    for (int64_t N : {1, 7, 8192, 8193, 100000}) {
      const size_t ws = rmsnorm_bwd_workspace_size(M, N), lws = layernorm_bwd_workspace_size(M, N);
      const int64_t target = N > 32768 ? ((int64_t(1) << 22) + N - 1) / N : 256;
      const int64_t by_rows = (M + 63) / 64;
      const int64_t blocks = (M < target ? M : target) > by_rows ? (M < target ? M : target) : by_rows;
      CHECK(ws >= static_cast<size_t>(blocks * N * 4));
      CHECK(lws >= ws && ws % 256 == 0 && lws % 256 == 0);
    }
  CHECK(rmsnorm_bwd_workspace_size(0, 64) == 0 && rmsnorm_bwd_workspace_size(4, 0) == 0);
  const size_t ws = rmsnorm_bwd_workspace_size(64, 256);
  CHECK(rmsnorm_bwd(A, B, Cf, D, E, Ff, G, ws, 64, 256, RMSN_BF16, RMSN_BF16, st) == RMSN_OK);
  CHECK(rmsnorm_bwd(A, B, Cf, D, E, Ff, G, ws - 4, 64, 256, RMSN_BF16, RMSN_BF16, st) ==
        RMSN_ERR_WORKSPACE);
  CHECK(rmsnorm_bwd(A, B, Cf, D, E, Ff, F, ws, 64, 256, RMSN_BF16, RMSN_BF16, st) ==
        RMSN_ERR_OVERLAP);
  CHECK(rmsnorm_fused_add_bwd(A, B, Cf, D, addr(8), E, Ff, G, ws, 64, 256, RMSN_BF16, RMSN_BF16,
                              st) == RMSN_OK);
  const size_t lws = layernorm_bwd_workspace_size(64, 256);
  CHECK(layernorm_bwd(A, B, Cf, static_cast<float*>(addr(8)), D, E, Ff, static_cast<float*>(addr(9)),
                      G, lws, 64, 256, RMSN_BF16, RMSN_BF16, st) == RMSN_OK);
  CHECK(rmsnorm_bwd_noalloc(A, B, Cf, D, E, Ff, 64, 256, RMSN_BF16, RMSN_BF16, st) == RMSN_OK);
  CHECK(rmsnorm_bwd_noalloc(A, B, Cf, D, E, Ff, 65537, 8192, RMSN_BF16, RMSN_BF16, st) ==
        RMSN_ERR_SCRATCH);
  for (int s = -10; s <= 1; ++s) CHECK(rmsnorm_status_string(s) != nullptr);
  CHECK(std::strcmp(rmsnorm_status_string(12345), "unknown status") == 0);
  CHECK(rmsnorm_last_hip_error() == 0);
}

}  // namespace

int main() {
  run_generator();
  run_oracle();
  run_abi();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("sanitizer driver: all checks passed (%d stub launches)\n", g_launches);
  return 0;
}
