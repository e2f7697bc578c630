// MFMA lane-layout self-check: multiplies small integer-valued matrices with
// the operand/accumulator conventions of gdn_common.hpp and compares with the
// exact host product.  Diagnostics only (synchronous, allocates a few KB).
#include <vector>

#include "gdn_common.hpp"
#include "gdn_internal.h"

namespace gdn {

// X [16][KS] and Yt [16][KS] row-major (contiguous along k); C [16][16].
template <typename E>
__global__ void selftest_kernel(const E *X, const E *Yt, float *C) {
  using M = Mma<E>;
  const int lane = threadIdx.x;
  const int lr = lane & 15, lg = lane >> 4;
  auto a = M::ld(X + lr * M::KS + M::EPL * lg);
  auto b = M::ld(Yt + lr * M::KS + M::EPL * lg);
  f32x4 c = M::mma(a, b, zero4());
#pragma unroll
  for (int i = 0; i < 4; ++i) C[(4 * lg + i) * 16 + lr] = c[i];
}

template <typename E>
static int check_one() {
  using M = Mma<E>;
  constexpr int KS = M::KS;
  std::vector<E> x(16 * KS), y(16 * KS);
  std::vector<float> xf(16 * KS), yf(16 * KS);
  for (int m = 0; m < 16; ++m)
    for (int k = 0; k < KS; ++k) {
      xf[m * KS + k] = (float)((m * 7 + k * 3) % 11 - 5);
      yf[m * KS + k] = (float)((m * 5 + k * 2) % 9 - 4);
      x[m * KS + k] = (E)xf[m * KS + k];
      y[m * KS + k] = (E)yf[m * KS + k];
    }
  E *dx = nullptr, *dy = nullptr;
  float *dc = nullptr;
  if (hipMalloc(&dx, sizeof(E) * 16 * KS) != hipSuccess) return 10;
  if (hipMalloc(&dy, sizeof(E) * 16 * KS) != hipSuccess) return 11;
  if (hipMalloc(&dc, sizeof(float) * 256) != hipSuccess) return 12;
  int rc = 0;
  if (hipMemcpy(dx, x.data(), sizeof(E) * 16 * KS, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemcpy(dy, y.data(), sizeof(E) * 16 * KS, hipMemcpyHostToDevice) != hipSuccess)
    rc = 13;
  std::vector<float> c(256, -1.f);
  if (!rc) {
    selftest_kernel<E><<<1, 64>>>(dx, dy, dc);
    if (hipDeviceSynchronize() != hipSuccess) rc = 14;
  }
  if (!rc && hipMemcpy(c.data(), dc, sizeof(float) * 256, hipMemcpyDeviceToHost) != hipSuccess)
    rc = 15;
  if (!rc) {
    for (int m = 0; m < 16 && !rc; ++m)
      for (int n = 0; n < 16; ++n) {
        float ref = 0.f;
        for (int k = 0; k < KS; ++k) ref += xf[m * KS + k] * yf[n * KS + k];
        if (c[m * 16 + n] != ref) {
          rc = 1;
          break;
        }
      }
  }
  (void)hipFree(dx);
  (void)hipFree(dy);
  (void)hipFree(dc);
  return rc;
}

int run_selftest() {
  int rc = check_one<bf16>();
  if (rc) return rc;
  rc = check_one<float>();
  if (rc) return 100 + rc;
  return 0;
}

}  // namespace gdn
