// Measurement aid, not part of the attention path: the bf16 MFMA rate that the
// whole chip sustains when it does nothing else. "Flash Attention FA1->FA4 /
// pre-training practice" (sections 2.2 and 2.3) quotes its kernels' speed as a
// share of the GPU's theoretical peak; on this chip the published dense bf16
// peak assumes the top clock, which is not held under a full matrix load, so
// the benchmark reports this figure next to it.
//
// Every wavefront runs `nit` rounds of eight independent 32x32x16 bf16 MFMA
// chains on register operands and then stores one float per lane, so no MFMA
// can be removed. The operands are eight pseudo-random A and eight B fragments
// per lane (values of magnitude 2^-2 .. 2^2 with random mantissas and signs),
// taken in a different pairing by every MFMA of a round: the matrix units
// draw more power on changing random data than on constant operands, and
// attention feeds them changing data. 2 * 32 * 32 * 16 FLOP per MFMA.
//
#include <hip/hip_runtime.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int CHAINS = 8;

// bf16 bits from a counter: sign and 7 mantissa bits random, exponent 125 .. 129
__device__ __forceinline__ unsigned short rand_bf16(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return (unsigned short)(((x >> 15) & 0x8000u) | ((125u + (x >> 8) % 5u) << 7) | (x & 0x7fu));
}

template <bool RANDOM>
__global__ __launch_bounds__(256) void mfma_loop_kernel(float* out, int nit) {
  bf16x8 a[8], b[8];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const unsigned id = ((blockIdx.x * 256u + threadIdx.x) * 8u + f) * 8u + i;
      a[f][i] = __builtin_bit_cast(__bf16, rand_bf16(2u * id));
      b[f][i] = __builtin_bit_cast(__bf16, rand_bf16(2u * id + 1u));
    }
  f32x16 acc[CHAINS];
#pragma unroll
  for (int c = 0; c < CHAINS; ++c) acc[c] = f32x16{};
  for (int it = 0; it < nit; it += 8) {
#pragma unroll
    for (int r = 0; r < 8; ++r)
#pragma unroll
      for (int c = 0; c < CHAINS; ++c)
        acc[c] = RANDOM ? __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(c + r) & 7], b[(c + 3 * r + 1) & 7], acc[c], 0, 0, 0)
                        : __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CHAINS; ++c)
#pragma unroll
    for (int i = 0; i < 16; ++i) s += acc[c][i];
  out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" int calib_mfma_bf16(float* out, int blocks, int nit, int random, hipStream_t stream) {
  if (out == nullptr || blocks < 1 || blocks > 65536 || nit < 8 || nit > (1 << 24) || nit % 8 != 0) return -1;
  if (random)
    hipLaunchKernelGGL(mfma_loop_kernel<true>, dim3(blocks), dim3(256), 0, stream, out, nit);
  else
    hipLaunchKernelGGL(mfma_loop_kernel<false>, dim3(blocks), dim3(256), 0, stream, out, nit);
  return (int)hipGetLastError();
}
