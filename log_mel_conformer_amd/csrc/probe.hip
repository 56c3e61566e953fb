// A measurement aid, not part of the encoder: the matrix cores' sustained
// bf16 rate on the current device, a second denominator beside the nominal
// 2.5 PFLOP/s for the GEMMs' rooflines (the nominal figure assumes the
// 2.4 GHz peak clock, which matrix-core-heavy work does not hold). Each
// wavefront runs `iters` rounds of eight independent
// v_mfma_f32_32x32x16_bf16 on register operands: no memory traffic, only
// matrix-core issue, four wavefronts per SIMD. Measured rates rise with
// the length of the run as the clock settles (1.86 PFLOP/s over 1.4 ms,
// 2.06 over 5 ms on one box), so the caller should time a few ms.
#include "common.h"

namespace ae {
namespace {

__global__ void __launch_bounds__(256) k_mfma_probe(int iters, float* sink) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (bf16)(0.001f * (float)(lane + e));
    b[e] = (bf16)(0.002f * (float)(lane - e));
  }
  f32x16 acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = f32x16{};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[k][v];
  // a store the compiler cannot rule out keeps the products live; the sum
  // never takes this value for these operands
  if (s == 1234567.0f) sink[0] = s;
}

}  // namespace
}  // namespace ae

/* Matrix-core rate probe (see include/ae.h). */
extern "C" ae_status ae_probe_mfma(int32_t iters, float* sink, int64_t* flops, hipStream_t s) {
  if (iters < 1 || !sink || !flops)
    return ae::set_error(AE_ERR_INVALID, "ae_probe_mfma: iters >= 1, sink and flops are needed");
  int dev = 0, cus = 0;
  AE_HIP_TRY(hipGetDevice(&dev));
  AE_HIP_TRY(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
  const int blocks = 4 * (cus > 0 ? cus : 1);  // four 4-wavefront blocks per CU
  hipLaunchKernelGGL(ae::k_mfma_probe, dim3(blocks), dim3(256), 0, s, iters, sink);
  AE_HIP_TRY(hipGetLastError());
  *flops = (int64_t)blocks * 4 * iters * 8 * (2LL * 32 * 32 * 16);
  return AE_OK;
}
