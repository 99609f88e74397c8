// Measurement aids, not part of the attention path: the bf16 MFMA rate that
// the whole chip sustains when it does nothing else, and how the matrix pipe
// and the vector ALU of one SIMD share it between two wavefronts. "Flash Attention FA1->FA4 /
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

typedef short s16x4 __attribute__((vector_size(8)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

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


// Co-issue probe: one workgroup of 8 wavefronts per CU (80 KB of LDS keeps it
// alone there); wavefronts w and w + 4 share a SIMD. Wavefronts 0-3 run the
// attention step's matrix stream: per pair of MFMAs one K fragment read with
// ds_read_b128 and two transposed V halves read with ds_read_b64_tr_b16,
// loaded two pairs ahead, then one 32x32x16 MFMA on each (1 KB of LDS per
// MFMA, as in the forward's main loop). Wavefronts 4-7 run a softmax-shaped
// vector stream: per score an FMA with the scale, exp2, a sum-tree add, half
// a bf16 pair pack and an FMA that feeds the next round. MODE 0: the matrix
// stream alone; 1: both streams; 2: the vector stream alone; 3: the vector
// stream on all 8 wavefronts (two per SIMD); 4: the matrix stream on all 8
// wavefronts (two per SIMD sharing one pipe, both reading LDS). Every wavefront stores the
// shader-clock cycles of its stream (s_memtime, read-only). A 32x32x16 bf16
// MFMA is 32768 FLOP; at the published 2.5 PFLOP/s over 1024 SIMDs at 2.4 GHz
// that is 32 cycles, the figure the matrix stream is measured against.
template <int MODE>
__global__ __launch_bounds__(512) void coissue_kernel(unsigned long long* cycles, float* out, int nit) {
  __shared__ __attribute__((aligned(16))) unsigned short lds[40960];
  const int w = threadIdx.x / 64, lane = threadIdx.x % 64;
  for (int i = threadIdx.x; i < 40960; i += 512) lds[i] = rand_bf16(blockIdx.x * 40960u + i);
  __syncthreads();
  float res = 0.f;
  const unsigned long long t0 = __builtin_amdgcn_s_memtime();
  const bool matrix = (w < 4 && MODE <= 1) || MODE == 4;
  const bool vector = !matrix && ((w >= 4 && (MODE == 1 || MODE == 2)) || MODE == 3);
  if (matrix) {
    bf16x8 q[8], p[8];
#pragma unroll
    for (int f = 0; f < 8; ++f)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned id = ((blockIdx.x * 512u + threadIdx.x) * 8u + f) * 8u + i;
        q[f][i] = __builtin_bit_cast(__bf16, rand_bf16(2u * id));
        p[f][i] = __builtin_bit_cast(__bf16, rand_bf16(2u * id + 1u));
      }
    f32x16 acc[6];
#pragma unroll
    for (int c = 0; c < 6; ++c) acc[c] = f32x16{};
    // this wavefront's 16 KB: K fragments in the first 8 KB, V in the second
    const unsigned char* region = (const unsigned char*)lds + (w & 3) * 16384;
    for (int it = 0; it < nit; ++it) {
      const unsigned char* kb = region + ((lane + it) & 63) * 16;
      const unsigned char* vb = region + 8192 + ((lane + it) & 63) * 8;
      bf16x8 kr[3], vr[3];
      auto load = [&](int u, bf16x8& k, bf16x8& v) {
        k = *(const bf16x8*)(kb + (u & 7) * 1024 + (u >> 3) * 16);
        const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + ((2 * u) & 15) * 512 + (u >> 3) * 8));
        const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + ((2 * u + 1) & 15) * 512 + (u >> 3) * 8));
        v = __builtin_bit_cast(bf16x8, __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7));
      };
      load(0, kr[0], vr[0]);
      load(1, kr[1], vr[1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 32; ++u) {
        if (u + 2 < 32) load(u + 2, kr[(u + 2) % 3], vr[(u + 2) % 3]);
        __builtin_amdgcn_sched_barrier(0);
        acc[u & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[u % 3], q[u & 7], acc[u & 1], 0, 0, 0);
        acc[2 + (u & 3)] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[u % 3], p[u & 7], acc[2 + (u & 3)], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int c = 0; c < 6; ++c)
#pragma unroll
      for (int i = 0; i < 16; ++i) res += acc[c][i];
  } else if (vector) {
    float sc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) sc[i] = (float)((threadIdx.x * 37 + i * 11) % 97) * 0.01f;
    const float c = 1.4426950f, c1 = 1.0e-3f, m = 0.75f;
    float lsum = 0.f;
    unsigned pk = 0u;
    for (int it = 0; it < 3 * nit; ++it) {
      float pr[32];
#pragma unroll
      for (int i = 0; i < 32; ++i) pr[i] = __builtin_amdgcn_exp2f(fmaf(sc[i], c, -m));
      float t[8];
#pragma unroll
      for (int g = 0; g < 8; ++g) t[g] = (pr[4 * g] + pr[4 * g + 1]) + (pr[4 * g + 2] + pr[4 * g + 3]);
      lsum += ((t[0] + t[1]) + (t[2] + t[3])) + ((t[4] + t[5]) + (t[6] + t[7]));
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        bf16x2 b2;
        b2[0] = (__bf16)pr[2 * i];
        b2[1] = (__bf16)pr[2 * i + 1];
        pk ^= __builtin_bit_cast(unsigned, b2);
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) sc[i] = fmaf(pr[i], c1, sc[i]);
    }
    res = lsum + __uint_as_float(pk & 0x3fffffffu);
  }
  const unsigned long long t1 = __builtin_amdgcn_s_memtime();
  out[(size_t)blockIdx.x * 512 + threadIdx.x] = res;
  if (lane == 0) cycles[(size_t)blockIdx.x * 8 + w] = (matrix || vector) ? t1 - t0 : 0ull;
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

// cycles: blocks * 8 per-wavefront cycle counts (0 for a wavefront with no
// stream); out: blocks * 512 floats. Each matrix wavefront issues 64 * nit
// MFMAs, each vector wavefront handles 96 * nit scores per lane (so that in
// mode 1 the vector stream outlasts the matrix stream).
extern "C" int calib_coissue(unsigned long long* cycles, float* out, int blocks, int nit, int mode,
                             hipStream_t stream) {
  if (cycles == nullptr || out == nullptr || blocks < 1 || blocks > 65536 || nit < 1 || nit > (1 << 20) ||
      mode < 0 || mode > 4)
    return -1;
  switch (mode) {
    case 0: hipLaunchKernelGGL(coissue_kernel<0>, dim3(blocks), dim3(512), 0, stream, cycles, out, nit); break;
    case 1: hipLaunchKernelGGL(coissue_kernel<1>, dim3(blocks), dim3(512), 0, stream, cycles, out, nit); break;
    case 2: hipLaunchKernelGGL(coissue_kernel<2>, dim3(blocks), dim3(512), 0, stream, cycles, out, nit); break;
    case 3: hipLaunchKernelGGL(coissue_kernel<3>, dim3(blocks), dim3(512), 0, stream, cycles, out, nit); break;
    default: hipLaunchKernelGGL(coissue_kernel<4>, dim3(blocks), dim3(512), 0, stream, cycles, out, nit); break;
  }
  return (int)hipGetLastError();
}
