// Device self-test of the int8 score instruction (Karume v0.8.0 release
// notes, "Fixes": the attention's int8 dot is not taken on faith; a canary
// runs the instruction and an emulation against a known answer at first use,
// and the library fails loudly if the instruction disagrees).
//
// One wave multiplies a fixed 16 x 64 by 64 x 16 int8 pattern twice: with
// v_mfma_i32_16x16x64_i8 (the instruction every int8-K score uses, in the
// lane layout the kernels rely on) and with plain integer multiply-adds from
// LDS.  The host compares both with the exact product it computes itself.
// The result goes to a file-scope device array, so the test allocates
// nothing; it runs once per device and the outcome is kept.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "ka_launch.h"

namespace ka {
namespace {

constexpr int kCanaryMaxDevices = 64;
__device__ int g_canary[2 * 256];  // [instruction | emulation][16 x 16]

// Entries of the pattern: every code from -127 to 127 appears, with mixed
// signs in every row and column.
__host__ __device__ inline int canary_a(int i, int k) { return ((i * 67 + k * 29 + 11) % 255) - 127; }
__host__ __device__ inline int canary_b(int k, int j) { return ((k * 41 + j * 83 + 5) % 255) - 127; }

__global__ __launch_bounds__(64) void i8_canary_kernel() {
  typedef __attribute__((ext_vector_type(4))) int i32x4;
  __shared__ signed char sa[16][64];
  __shared__ signed char sb[64][16];
  const int l = threadIdx.x;
  for (int i = l; i < 16 * 64; i += 64) {
    sa[i / 64][i % 64] = (signed char)canary_a(i / 64, i % 64);
    sb[i / 16][i % 16] = (signed char)canary_b(i / 16, i % 16);
  }
  __syncthreads();
  // instruction: A[l % 16][16 (l / 16) + j], B[16 (l / 16) + j][l % 16]
  union { i32x4 v; signed char c[16]; } a, b;
  for (int j = 0; j < 16; ++j) {
    a.c[j] = sa[l % 16][16 * (l / 16) + j];
    b.c[j] = sb[16 * (l / 16) + j][l % 16];
  }
  i32x4 d = {0, 0, 0, 0};
  d = __builtin_amdgcn_mfma_i32_16x16x64_i8(a.v, b.v, d, 0, 0, 0);
  for (int i = 0; i < 4; ++i) g_canary[(4 * (l / 16) + i) * 16 + (l % 16)] = d[i];
  // emulation: this lane's four outputs by integer multiply-adds
  for (int i = 0; i < 4; ++i) {
    const int row = 4 * (l / 16) + i, col = l % 16;
    int acc = 0;
    for (int k = 0; k < 64; ++k) acc += (int)sa[row][k] * (int)sb[k][col];
    g_canary[256 + row * 16 + col] = acc;
  }
}

std::mutex g_canary_mu;
int g_canary_state[kCanaryMaxDevices];  // 0 untested, 1 passed, 2 failed
char g_canary_msg[kCanaryMaxDevices][160];

}  // namespace

hipError_t int8_self_test(bool* passed, const char** why) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kCanaryMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_canary_mu);
  if (g_canary_state[dev] == 0) {
    hipLaunchKernelGGL(i8_canary_kernel, dim3(1), dim3(64), 0, nullptr);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    int got[2 * 256];
    if ((e = hipMemcpyFromSymbol(got, HIP_SYMBOL(g_canary), sizeof got)) != hipSuccess) return e;
    int bad_mfma = 0, bad_emul = 0;
    for (int r = 0; r < 16; ++r)
      for (int c = 0; c < 16; ++c) {
        int want = 0;
        for (int k = 0; k < 64; ++k) want += canary_a(r, k) * canary_b(k, c);
        bad_mfma += got[r * 16 + c] != want;
        bad_emul += got[256 + r * 16 + c] != want;
      }
    g_canary_state[dev] = bad_mfma == 0 && bad_emul == 0 ? 1 : 2;
    snprintf(g_canary_msg[dev], sizeof g_canary_msg[dev],
             "int8 score self-test on device %d: instruction %d / 256 wrong, emulation %d / 256 wrong",
             dev, bad_mfma, bad_emul);
  }
  *passed = g_canary_state[dev] == 1;
  *why = g_canary_msg[dev];
  return hipSuccess;
}

}  // namespace ka
