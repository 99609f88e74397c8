// Measurement aid, not part of the attention path: the bf16 MFMA rate that the
// whole chip sustains when it does nothing else. "Flash Attention FA1->FA4 /
// pre-training practice" (sections 2.2 and 2.3) quotes its kernels' speed as a
// share of the GPU's theoretical peak; on this chip the published dense bf16
// peak assumes the top clock, which is not held under a full matrix load, so
// the benchmark reports this figure next to it.
//
// Every wavefront runs `nit` rounds of eight independent 32x32x16 bf16 MFMA
// chains on register operands and then stores one float per lane, so no MFMA
// can be removed. 2 * 32 * 32 * 16 FLOP per MFMA.
//
// extern "C" int calib_mfma_bf16(float* out, int blocks, int nit, hipStream_t stream)
//   out:    device buffer of blocks * 256 floats (written);
//   blocks: workgroups of 256 threads (4 wavefronts), 1 .. 65536;
//   nit:    rounds per wavefront, 1 .. 2^24.
//   Returns 0, or -1 for arguments out of range, or the launch error.
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int CHAINS = 8;

__global__ __launch_bounds__(256) void mfma_loop_kernel(float* out, int nit) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(1e-3f * (float)(threadIdx.x + i));
    b[i] = (__bf16)(1e-3f * (float)(i - (int)threadIdx.x));
  }
  f32x16 acc[CHAINS];
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) acc[c] = f32x16{};
  for (int it = 0; it < nit; ++it) {
#pragma unroll
    for (int c = 0; c < CHAINS; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CHAINS; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" int calib_mfma_bf16(float* out, int blocks, int nit, hipStream_t stream) {
  if (out == nullptr || blocks < 1 || blocks > 65536 || nit < 1 || nit > (1 << 24)) return -1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256), 0, stream, out, nit);
  return (int)hipGetLastError();
}
