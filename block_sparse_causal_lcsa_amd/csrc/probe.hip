// lcsa_mfma_probe: sustained throughput of the bf16 matrix core, for the measurement harness (not part
// of the attention method). Each wave keeps its operands in registers and issues back-to-back
// 32x32x16 bf16 MFMAs over four independent accumulators, so the matrix core is the only limit.
#include <hip/hip_runtime.h>

#include "lcsa_internal.h"
#include "lcsa_probe.h"

namespace lcsa {
namespace {

typedef __bf16 probe_bf16x8 __attribute__((ext_vector_type(8)));
typedef float probe_f32x16 __attribute__((ext_vector_type(16)));

__global__ __launch_bounds__(256) void mfma_probe_kernel(float* sink, int iters) {
  probe_bf16x8 x, y;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    x[i] = (__bf16)(1e-3f * float(lane) + float(i));
    y[i] = (__bf16)(0.5f * float(i));
  }
  probe_f32x16 acc[4] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int m = 0; m < 8; ++m) acc[m & 3] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(x, y, acc[m & 3], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 16; ++j) s += acc[i][j];
  sink[size_t(blockIdx.x) * blockDim.x + threadIdx.x] = s;
}

}  // namespace
}  // namespace lcsa

using namespace lcsa;

extern "C" lcsa_status lcsa_mfma_probe(int32_t workgroups, int32_t iters, float* sink, double* flop, void* stream) {
  if (workgroups < 1 || workgroups > (1 << 20) || iters < 1 || iters > (1 << 24))
    return fail(LCSA_ERR_INVALID, "lcsa_mfma_probe: workgroups %d or iters %d out of range", workgroups, iters);
  if (!sink || reinterpret_cast<uintptr_t>(sink) % 4)
    return fail(LCSA_ERR_INVALID, "lcsa_mfma_probe: sink is NULL or misaligned");
  if (flop) *flop = double(workgroups) * 4.0 * double(iters) * 8.0 * 2.0 * 32.0 * 32.0 * 16.0;
  (void)hipGetLastError();
  mfma_probe_kernel<<<workgroups, 256, 0, static_cast<hipStream_t>(stream)>>>(sink, iters);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return hip_status(e, "lcsa_mfma_probe: launch");
  return LCSA_OK;
}
