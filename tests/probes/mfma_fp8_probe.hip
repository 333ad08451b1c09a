// Test-only probe of gfx950's FP8 matrix-core accumulation: n independent
// v_mfma_f32_16x16x128_f8f6f4 products (E4M3 x E4M3, C = 0), one wave each.
// The GPU parity tests bound the accumulation error of this instruction; this
// probe measures it so that the bound is checked on the device itself.
//
// Layout (both operands alike): lane l holds 32 bytes; a[i][l] is lane l's A
// operand of product i, b[i][l] its B operand. D[r][c] sums, over the four
// lane groups g and the 32 byte positions p, A[lane r + 16 g][p] times
// B[lane c + 16 g][p]; lane l's four results are D[4 (l / 16) + q][l % 16].
#include <hip/hip_runtime.h>

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(64) void mfma_fp8_probe_kernel(const v8i* __restrict__ a,
                                                            const v8i* __restrict__ b,
                                                            v4f* __restrict__ out, int n) {
  const int i = blockIdx.x;
  if (i >= n) return;
  const int lane = threadIdx.x;
  const v8i av = a[(size_t)i * 64 + lane];
  const v8i bv = b[(size_t)i * 64 + lane];
  v4f c = {0.f, 0.f, 0.f, 0.f};
  c = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bv, c, 0, 0, 0, 0, 0, 0);
  out[(size_t)i * 64 + lane] = c;
}

// a, b: device [n][64][32] bytes; out: device [n][64][4] float32. Returns the
// launch's hipError_t.
extern "C" int mfma_fp8_probe(const void* a, const void* b, void* out, int n, void* stream) {
  if (n <= 0) return 0;
  hipLaunchKernelGGL(mfma_fp8_probe_kernel, dim3(n), dim3(64), 0, static_cast<hipStream_t>(stream),
                     static_cast<const v8i*>(a), static_cast<const v8i*>(b), static_cast<v4f*>(out),
                     n);
  return (int)hipGetLastError();
}
