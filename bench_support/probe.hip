// Matrix-core throughput probe for the benchmark's measured ceilings: every
// wave runs rounds of four independent v_mfma_f32_32x32x16_bf16 chains with
// no memory traffic in the loop, so the rate it reaches is what the matrix
// cores deliver at the clock they hold under sustained MFMA load. Built into
// its own library (bench_support/libmoba_probe.so); nothing on the MoBA path
// uses it.
#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_loop_kernel(float *out, int iters, float seed) {
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)(seed * (float)((j + threadIdx.x) & 7));
    b[j] = (__bf16)(seed * (float)((j * 3 + threadIdx.x) & 7));
  }
  floatx16 c[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) c[u][i] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int u = 0; u < 4; ++u) c[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[u], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += c[u][i];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

// Launches `blocks` workgroups of 256 threads (4 waves), each wave running
// `iters` rounds of 4 MFMAs (32x32x16 bf16: 32768 FLOP each); out must hold
// blocks * 256 floats (device). Returns the hipError_t of the launch.
extern "C" int moba_probe_mfma_bf16(int blocks, int iters, float *out, hipStream_t stream) {
  if (blocks <= 0 || iters <= 0 || !out) return (int)hipErrorInvalidValue;
  mfma_loop_kernel<<<dim3((unsigned)blocks), dim3(256), 0, stream>>>(out, iters, 1e-3f);
  return (int)hipGetLastError();
}
