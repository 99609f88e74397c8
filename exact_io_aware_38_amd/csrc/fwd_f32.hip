// Forward attention in fp32 (vector ALU), for inputs that must not pass
// through bf16.
//
// Same recurrence as the bf16 path (online softmax, "Flash Attention FA1->FA4
// / pre-training practice" §1.2; (m, l, u) state of "AI 大模型之
// FlashAttention_01" §4.1), kept in the natural-log domain with expf so that
// the result stays within a few fp32 ulps of the exact one. One thread owns
// one query row; K/V tiles of 16 keys are staged through LDS and read by all
// threads as broadcasts.
#include "common.h"
#include "kernels.h"

namespace attn {

namespace {

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  float* o;
  float* lse;
  int Hq, Hkv, Sq, Sk, g, causal;
  float scale;
  int hsq, hsk;      // head strides in rows (see Problem)
};

template <int D>
__global__ __launch_bounds__(128) void fwd_f32_kernel(F32Args a) {
  constexpr int BR = 128;
  constexpr int BC = 16;
  __shared__ float sk[BC * D];
  __shared__ float sv[BC * D];

  const int tid = threadIdx.x;
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int hkv = hq / a.g;
  const int row = blockIdx.x * BR + tid;
  const bool valid = row < a.Sq;
  const int off = (a.causal == 2) ? (a.Sk - a.Sq) : 0;
  const int last_row = min((int)(blockIdx.x + 1) * BR, a.Sq) - 1;
  int kend = a.causal ? min(a.Sk, last_row + off + 1) : a.Sk;
  if (kend < 0) kend = 0;
  const int lim = a.causal ? min(kend - 1, row + off) : kend - 1;   // last visible key of this row

  float q[D], o[D];
  const float* qp = a.q + (((size_t)b * a.Hq + hq) * a.hsq + (valid ? row : 0)) * D;
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = valid ? qp[c] : 0.f;
    o[c] = 0.f;
  }
  float m = kNegInf, l = 0.f;
  const float* kg = a.k + ((size_t)b * a.Hkv + hkv) * (size_t)a.hsk * D;
  const float* vg = a.v + ((size_t)b * a.Hkv + hkv) * (size_t)a.hsk * D;

  for (int key0 = 0; key0 < kend; key0 += BC) {
    __syncthreads();
    for (int e = tid; e < BC * D; e += BR) {
      const int key = key0 + e / D;
      sk[e] = key < kend ? kg[(size_t)key * D + e % D] : 0.f;
      sv[e] = key < kend ? vg[(size_t)key * D + e % D] : 0.f;
    }
    __syncthreads();
    float s[BC];
    float mt = kNegInf;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < D; ++c) acc = __builtin_fmaf(q[c], sk[j * D + c], acc);
      s[j] = (key0 + j <= lim) ? acc * a.scale : kNegInf;
      mt = fmaxf(mt, s[j]);
    }
    const float mnew = fmaxf(m, mt);
    if (mnew == kNegInf) continue;      // nothing visible yet for this row
    const float alpha = expf(m - mnew);   // m = -inf on the first visible tile gives 0
    l *= alpha;
#pragma unroll
    for (int c = 0; c < D; ++c) o[c] *= alpha;
#pragma unroll
    for (int j = 0; j < BC; ++j) {
      const float p = expf(s[j] - mnew);
      l += p;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] = __builtin_fmaf(p, sv[j * D + c], o[c]);
    }
    m = mnew;
  }
  if (!valid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = a.o + (((size_t)b * a.Hq + hq) * a.hsq + row) * D;
#pragma unroll
  for (int c = 0; c < D; ++c) op[c] = o[c] * inv;
  if (a.lse != nullptr) a.lse[((size_t)b * a.Hq + hq) * a.hsq + row] = l > 0.f ? m + logf(l) : kNegInf;
}

}  // namespace

hipError_t launch_fwd_f32(const Problem& p, const float* q, const float* k, const float* v, float* o,
                          float* lse, hipStream_t s) {
  F32Args a{q, k, v, o, lse, p.Hq, p.Hkv, p.Sq, p.Sk, p.Hq / p.Hkv, p.causal, p.scale, p.hsq, p.hsk};
  dim3 grid((p.Sq + 127) / 128, p.Hq, p.B);
  timing_begin(s, "fwd_f32");
  if (p.d == 64)
    hipLaunchKernelGGL((fwd_f32_kernel<64>), grid, dim3(128), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<128>), grid, dim3(128), 0, s, a);
  const hipError_t e = hipGetLastError();
  timing_end(s);
  return e;
}

}  // namespace attn
