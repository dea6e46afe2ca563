// Device self-test of the int8 score instruction (Karume v0.8.0 release
// notes, "Fixes": the attention's int8 dot is not taken on faith; a canary
// runs the instruction and an emulation against a known answer at first use,
// and the library fails loudly if the instruction disagrees).
//
// One wave multiplies fixed int8 patterns with each instruction the int8-K
// scores use, in the lane layout the kernels rely on -- 16 x 64 by 64 x 16 on
// v_mfma_i32_16x16x64_i8 (decode) and 32 x 32 by 32 x 32 on
// v_mfma_i32_32x32x32_i8 (prefill) -- and again with plain integer
// multiply-adds from LDS.  The host compares all with the exact products it
// computes itself.
// The result goes to a file-scope device array, so the test allocates
// nothing; it runs once per device and the outcome is kept.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "ka_launch.h"

namespace ka {
namespace {

constexpr int kCanaryMaxDevices = 64;
// [16x16x64: instruction | emulation][16 x 16], then [32x32x32: instruction |
// emulation][32 x 32]
constexpr int kCanaryInts = 2 * 256 + 2 * 1024;
__device__ int g_canary[kCanaryInts];

// Entries of the pattern: every code from -127 to 127 appears, with mixed
// signs in every row and column.
__host__ __device__ inline int canary_a(int i, int k) { return ((i * 67 + k * 29 + 11) % 255) - 127; }
__host__ __device__ inline int canary_b(int k, int j) { return ((k * 41 + j * 83 + 5) % 255) - 127; }

__global__ __launch_bounds__(64) void i8_canary_kernel() {
  typedef __attribute__((ext_vector_type(4))) int i32x4;
  typedef __attribute__((ext_vector_type(16))) int i32x16;
  __shared__ signed char sa[16][64];
  __shared__ signed char sb[64][16];
  __shared__ signed char ta[32][32];
  __shared__ signed char tb[32][32];
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
  // 32 x 32 x 32: A[l % 32][16 (l / 32) + j], B[16 (l / 32) + j][l % 32],
  // D register i at row 8 (i / 4) + 4 (l / 32) + i % 4, column l % 32
  for (int i = l; i < 32 * 32; i += 64) {
    ta[i / 32][i % 32] = (signed char)canary_a(i / 32, i % 32);
    tb[i / 32][i % 32] = (signed char)canary_b(i / 32, i % 32);
  }
  __syncthreads();
  for (int j = 0; j < 16; ++j) {
    a.c[j] = ta[l % 32][16 * (l / 32) + j];
    b.c[j] = tb[16 * (l / 32) + j][l % 32];
  }
  i32x16 e = {};
  e = __builtin_amdgcn_mfma_i32_32x32x32_i8(a.v, b.v, e, 0, 0, 0);
  for (int i = 0; i < 16; ++i) {
    const int row = 8 * (i / 4) + 4 * (l / 32) + i % 4, col = l % 32;
    g_canary[512 + row * 32 + col] = e[i];
    int acc = 0;
    for (int k = 0; k < 32; ++k) acc += (int)ta[row][k] * (int)tb[k][col];
    g_canary[512 + 1024 + row * 32 + col] = acc;
  }
}

std::mutex g_canary_mu;
int g_canary_state[kCanaryMaxDevices];  // 0 untested, 1 passed, 2 failed
char g_canary_msg[kCanaryMaxDevices][200];

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
    static int got[kCanaryInts];  // under the mutex
    if ((e = hipMemcpyFromSymbol(got, HIP_SYMBOL(g_canary), sizeof got)) != hipSuccess) return e;
    int bad16 = 0, bad32 = 0, bad_emul = 0;
    for (int r = 0; r < 16; ++r)
      for (int c = 0; c < 16; ++c) {
        int want = 0;
        for (int k = 0; k < 64; ++k) want += canary_a(r, k) * canary_b(k, c);
        bad16 += got[r * 16 + c] != want;
        bad_emul += got[256 + r * 16 + c] != want;
      }
    for (int r = 0; r < 32; ++r)
      for (int c = 0; c < 32; ++c) {
        int want = 0;
        for (int k = 0; k < 32; ++k) want += canary_a(r, k) * canary_b(k, c);
        bad32 += got[512 + r * 32 + c] != want;
        bad_emul += got[512 + 1024 + r * 32 + c] != want;
      }
    g_canary_state[dev] = bad16 == 0 && bad32 == 0 && bad_emul == 0 ? 1 : 2;
    snprintf(g_canary_msg[dev], sizeof g_canary_msg[dev],
             "int8 score self-test on device %d: 16x16x64 instruction %d / 256 wrong, 32x32x32 "
             "instruction %d / 1024 wrong, emulation %d / 1280 wrong",
             dev, bad16, bad32, bad_emul);
  }
  *passed = g_canary_state[dev] == 1;
  *why = g_canary_msg[dev];
  return hipSuccess;
}

}  // namespace ka
