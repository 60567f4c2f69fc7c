// The C-ABI's rejected-argument cases, run against a host build of the
// validation layer under AddressSanitizer and UndefinedBehaviorSanitizer.
// Every call must return its status code without reaching a launcher.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "sinkattn.h"

extern int g_stub_calls;

static int g_failures = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      std::printf("FAILED line %d: %s\n", __LINE__, #cond);       \
      ++g_failures;                                               \
    }                                                             \
  } while (0)

static sinkattn_shape shape(int B = 1, int H = 2, int L = 256, int d = 64, int dtype = SINKATTN_F32,
                            const int32_t* lengths = nullptr, int dustbin = 0) {
  sinkattn_shape s;
  std::memset(&s, 0, sizeof(s));
  s.B = B;
  s.H = H;
  s.L = L;
  s.d = d;
  s.dtype = dtype;
  s.lengths = lengths;
  s.dustbin = dustbin;
  return s;
}

int main() {
  void* fake = reinterpret_cast<void*>(uintptr_t(0x10000));  // never dereferenced
  float* ff = static_cast<float*>(fake);
  char* misaligned = static_cast<char*>(fake) + 4;
  const int32_t* fake_len = static_cast<const int32_t*>(fake);

  // workspace sizes of invalid shapes
  sinkattn_shape s = shape();
  EXPECT(sinkattn_workspace_bytes(nullptr, 64, 2) == 0);
  sinkattn_shape bad_d = shape(1, 2, 256, 48);
  EXPECT(sinkattn_workspace_bytes(&bad_d, 64, 2) == 0);
  EXPECT(sinkattn_workspace_bytes(&s, 0, 2) == 0);
  EXPECT(sinkattn_workspace_bytes(&s, 64, -1) == 0);
  sinkattn_shape l0 = shape(1, 2, 0);
  EXPECT(sinkattn_workspace_bytes(&l0, 64, 2) == 0);
  sinkattn_shape bad_t = shape(1, 2, 256, 64, 7);
  EXPECT(sinkattn_workspace_bytes(&bad_t, 64, 2) == 0);
  EXPECT(sinkattn_workspace_bytes(&s, 600, 2) == 0);
  sinkattn_shape dust_nolen = shape(1, 2, 256, 64, SINKATTN_F32, nullptr, 1);
  EXPECT(sinkattn_workspace_bytes(&dust_nolen, 64, 2) == 0);
  sinkattn_shape huge = shape(256, 256, 8);
  EXPECT(sinkattn_workspace_bytes(&huge, 17, 2) == 0);
  sinkattn_shape slice = shape(1, 1, 1 << 24, 128, SINKATTN_BF16);
  EXPECT(sinkattn_workspace_bytes(&slice, 64, 2) == 0);
  const size_t nb = sinkattn_workspace_bytes(&s, 64, 2);
  EXPECT(nb > 0);
  sinkattn_shape with_len = shape(2, 2, 256, 64, SINKATTN_F32, fake_len, 1);
  EXPECT(sinkattn_workspace_bytes(&with_len, 64, 2) > 0);

  // tail offsets
  EXPECT(sinkattn_tail_offset(&s, 2, 3, 0) == (size_t)-1);
  EXPECT(sinkattn_tail_offset(&s, 2, -1, 1) == (size_t)-1);
  EXPECT(sinkattn_tail_offset(nullptr, 2, 0, 0) == (size_t)-1);
  EXPECT(sinkattn_tail_offset(&s, 2, 1, 0) == 2u * 256u * 8u);

  // forward
  auto fwd = [&](const sinkattn_shape* sh, int W, int T, int R, void* Q, void* ws, size_t bytes) {
    return sinkattn_forward(Q, fake, fake, W, T, R, ff, ff, sh, ff, ff, ff, ws, bytes, nullptr);
  };
  EXPECT(fwd(&s, 64, 3, 2, nullptr, fake, nb) == SINKATTN_EINVAL);
  EXPECT(fwd(&s, 64, 3, 2, fake, nullptr, nb) == SINKATTN_EINVAL);
  EXPECT(fwd(&s, 0, 3, 2, fake, fake, nb) == SINKATTN_EINVAL);
  EXPECT(fwd(&s, 64, -1, 2, fake, fake, nb) == SINKATTN_EINVAL);
  EXPECT(fwd(&s, 64, 3, -2, fake, fake, nb) == SINKATTN_EINVAL);
  EXPECT(fwd(&s, 64, 3, 2, misaligned, fake, nb) == SINKATTN_EINVAL);
  EXPECT(fwd(&bad_d, 64, 3, 2, fake, fake, nb) == SINKATTN_EUNSUPPORTED);
  EXPECT(fwd(nullptr, 64, 3, 2, fake, fake, nb) == SINKATTN_EINVAL);
  EXPECT(fwd(&s, 64, 3, 2, fake, fake, 1024) == SINKATTN_EWORKSPACE);
  EXPECT(fwd(&huge, 17, 3, 2, fake, fake, nb) == SINKATTN_EUNSUPPORTED);
  EXPECT(sinkattn_forward(fake, fake, fake, 64, 3, 2, ff, ff, &s, nullptr, ff, ff, fake, nb, nullptr) ==
         SINKATTN_EINVAL);

  // early-stopping forward
  int t_used = -7;
  auto conv = [&](int T_max, int R, double tol, int every, size_t bytes, int* tu) {
    return sinkattn_forward_converge(fake, fake, fake, 64, T_max, R, ff, ff, &s, tol, every, ff, ff, ff, fake,
                                     bytes, tu, nullptr, nullptr);
  };
  EXPECT(conv(10, 0, 1e-3, 2, nb, &t_used) == SINKATTN_EINVAL);
  EXPECT(conv(10, 2, 1e-3, 0, nb, &t_used) == SINKATTN_EINVAL);
  EXPECT(conv(10, 2, -1.0, 2, nb, &t_used) == SINKATTN_EINVAL);
  EXPECT(conv(10, 2, NAN, 2, nb, &t_used) == SINKATTN_EINVAL);
  EXPECT(conv(-1, 2, 1e-3, 2, nb, &t_used) == SINKATTN_EINVAL);
  EXPECT(conv(10, 2, 1e-3, 2, nb, nullptr) == SINKATTN_EINVAL);
  EXPECT(conv(10, 2, 1e-3, 2, 1024, &t_used) == SINKATTN_EWORKSPACE);
  EXPECT(t_used == -7);

  // backward
  auto bwd = [&](int R, void* dO, size_t bytes) {
    return sinkattn_backward(fake, fake, fake, 64, 3, R, ff, ff, &s, ff, dO, fake, bytes, ff, ff, ff, nullptr,
                             nullptr);
  };
  EXPECT(bwd(2, nullptr, nb) == SINKATTN_EINVAL);
  EXPECT(bwd(9, fake, nb) == SINKATTN_EUNSUPPORTED);
  EXPECT(bwd(-1, fake, nb) == SINKATTN_EINVAL);
  EXPECT(bwd(2, fake, 16) == SINKATTN_EWORKSPACE);
  EXPECT(bwd(2, misaligned, nb) == SINKATTN_EINVAL);

  // certificate
  double eta[9];
  int sel = -3;
  auto cert = [&](int R_max, double tau, double* e) {
    return sinkattn_tail_certificate(fake, fake, fake, 64, 3, R_max, ff, ff, &s, ff, fake, fake, nb, ff, ff, ff, ff,
                                     ff, e, tau, &sel, nullptr);
  };
  EXPECT(cert(0, 1e-5, eta) == SINKATTN_EINVAL);
  EXPECT(cert(9, 1e-5, eta) == SINKATTN_EUNSUPPORTED);
  EXPECT(cert(2, -1.0, eta) == SINKATTN_EINVAL);
  EXPECT(cert(2, NAN, eta) == SINKATTN_EINVAL);
  EXPECT(cert(2, 1e-5, nullptr) == SINKATTN_EINVAL);
  EXPECT(sel == -3);

  // contraction diagnostic
  EXPECT(sinkattn_block_contraction(fake, fake, 64, &s, 0, ff, nullptr, nullptr) == SINKATTN_EINVAL);
  EXPECT(sinkattn_block_contraction(fake, fake, 64, &s, 200, ff, nullptr, nullptr) == SINKATTN_EINVAL);
  EXPECT(sinkattn_block_contraction(fake, fake, 16, &s, 9, ff, nullptr, nullptr) == SINKATTN_EINVAL);
  EXPECT(sinkattn_block_contraction(fake, fake, 64, &s, 16, nullptr, nullptr, nullptr) == SINKATTN_EINVAL);

  // timing and strings
  EXPECT(sinkattn_timing_collect(nullptr, nullptr) == SINKATTN_EINVAL);
  EXPECT(sinkattn_timing_enable(1) == SINKATTN_OK);
  double ms = -1.0;
  long long steps = -1;
  EXPECT(sinkattn_timing_collect(&ms, &steps) == SINKATTN_OK && ms == 0.0 && steps == 0);
  EXPECT(sinkattn_timing_enable(0) == SINKATTN_OK);
  for (int code = -7; code <= 0; ++code) EXPECT(std::strcmp(sinkattn_status_string(code), "unknown status") != 0);
  EXPECT(std::strcmp(sinkattn_status_string(99), "unknown status") == 0);
  EXPECT(sinkattn_measure_peaks(nullptr, nullptr, nullptr, nullptr) == SINKATTN_EINVAL);
  double cyc = 0.0;
  EXPECT(sinkattn_measure_lds(288, 0, nullptr, nullptr) == SINKATTN_EINVAL);
  EXPECT(sinkattn_measure_lds(280, 0, &cyc, nullptr) == SINKATTN_EINVAL);
  EXPECT(sinkattn_measure_lds(336, 0, &cyc, nullptr) == SINKATTN_EINVAL);
  EXPECT(sinkattn_measure_lds(272, 1, &cyc, nullptr) == SINKATTN_EINVAL);
  EXPECT(sinkattn_measure_lds(256, 2, &cyc, nullptr) == SINKATTN_EINVAL);
  EXPECT(sinkattn_version() >= 10000);

  EXPECT(g_stub_calls == 0);
  if (g_failures == 0) std::printf("all checks passed\n");
  return g_failures == 0 ? 0 : 1;
}
