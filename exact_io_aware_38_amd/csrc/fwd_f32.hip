// Forward attention in fp32 (vector ALU), for inputs that must not pass
// through bf16.
//
// Same recurrence as the bf16 path (online softmax, "Flash Attention FA1->FA4
// / pre-training practice" §1.2; (m, l, u) state of "AI 大模型之
// FlashAttention_01" §4.1), kept in the natural-log domain with expf so that
// the result stays within a few fp32 ulps of the exact one. Half a wavefront
// owns one query row, splitting its keys 16 ways and its channels 2 ways; K/V
// tiles of 64 keys are staged through LDS for the workgroup's rows.
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

// Thirty-two lanes own one query row: lane = kl + 16 dh, where kl (0..15)
// picks every 16th key of each 64-key tile and dh the half of the channels the
// lane keeps (q and the output accumulator for D/2 channels each). A score is
// the lane's partial dot product plus its partner's (lane ^ 16). Every lane
// runs the online softmax over its own keys; at the end the 16 partial states
// (m, l, u) of a row are merged with the same rescaling rule. K and V tiles are
// staged in LDS for the workgroup's 8 rows.
template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(F32Args a) {
  constexpr int ROWS = 8;                       // query rows per workgroup (32 lanes each)
  constexpr int BC = 64;                        // keys per tile
  constexpr int KPL = BC / 16;                  // keys per lane per tile
  constexpr int DH = D / 2;                     // channels per lane
  __shared__ float sk[BC * D];
  __shared__ float sv[BC * D];

  const int tid = threadIdx.x;
  const int kl = tid & 15, dh = (tid >> 4) & 1;
  const int hq = blockIdx.y;
  const int b = blockIdx.z;
  const int hkv = hq / a.g;
  const int row = blockIdx.x * ROWS + (tid >> 5);
  const bool valid = row < a.Sq;
  const int off = (a.causal == 2) ? (a.Sk - a.Sq) : 0;
  const int last_row = min((int)(blockIdx.x + 1) * ROWS, a.Sq) - 1;
  int kend = a.causal ? min(a.Sk, last_row + off + 1) : a.Sk;
  if (kend < 0) kend = 0;
  const int lim = a.causal ? min(kend - 1, row + off) : kend - 1;   // last visible key of this row

  float q[DH], u[DH];
  const float* qp = a.q + (((size_t)b * a.Hq + hq) * a.hsq + (valid ? row : 0)) * D + dh * DH;
#pragma unroll
  for (int c = 0; c < DH; ++c) {
    q[c] = valid ? qp[c] : 0.f;
    u[c] = 0.f;
  }
  float m = kNegInf, l = 0.f;
  const float* kg = a.k + ((size_t)b * a.Hkv + hkv) * (size_t)a.hsk * D;
  const float* vg = a.v + ((size_t)b * a.Hkv + hkv) * (size_t)a.hsk * D;

  for (int key0 = 0; key0 < kend; key0 += BC) {
    __syncthreads();
    for (int e = tid * 4; e < BC * D; e += 256 * 4) {
      const int key = key0 + e / D;
      f32x4 kx = f32x4{0.f, 0.f, 0.f, 0.f}, vx = kx;
      if (key < kend) {
        kx = *(const f32x4*)(kg + (size_t)key * D + e % D);
        vx = *(const f32x4*)(vg + (size_t)key * D + e % D);
      }
      *(f32x4*)(sk + e) = kx;
      *(f32x4*)(sv + e) = vx;
    }
    __syncthreads();
    float s[KPL];
    float mt = kNegInf;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const int j = kl + 16 * i;
      const float* kr = sk + j * D + dh * DH;
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < DH; ++c) acc = __builtin_fmaf(q[c], kr[c], acc);
      acc += __shfl_xor(acc, 16);
      s[i] = (key0 + j <= lim) ? acc * a.scale : kNegInf;
      mt = fmaxf(mt, s[i]);
    }
    const float mnew = fmaxf(m, mt);
    if (mnew == kNegInf) continue;              // nothing visible yet for this lane
    const float alpha = expf(m - mnew);         // m = -inf before the first visible key gives 0
    l *= alpha;
#pragma unroll
    for (int c = 0; c < DH; ++c) u[c] *= alpha;
#pragma unroll
    for (int i = 0; i < KPL; ++i) {
      const float p = expf(s[i] - mnew);
      l += p;
      const float* vr = sv + (kl + 16 * i) * D + dh * DH;
#pragma unroll
      for (int c = 0; c < DH; ++c) u[c] = __builtin_fmaf(p, vr[c], u[c]);
    }
    m = mnew;
  }
  // merge the 16 lanes' states of the row: m = max, l and u rescaled to it and summed
  float mr = m;
#pragma unroll
  for (int x = 1; x < 16; x <<= 1) mr = fmaxf(mr, __shfl_xor(mr, x));
  const float w = (mr == kNegInf) ? 0.f : expf(m - mr);
  l *= w;
#pragma unroll
  for (int x = 1; x < 16; x <<= 1) l += __shfl_xor(l, x);
#pragma unroll
  for (int c = 0; c < DH; ++c) {
    float t = u[c] * w;
#pragma unroll
    for (int x = 1; x < 16; x <<= 1) t += __shfl_xor(t, x);
    u[c] = t;
  }
  if (!valid) return;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* op = a.o + (((size_t)b * a.Hq + hq) * a.hsq + row) * D + dh * DH;
  // lane kl writes channels kl, kl + 16, ... of its half
#pragma unroll
  for (int c = 0; c < DH; ++c)
    if (c % 16 == kl) op[c] = u[c] * inv;
  if (a.lse != nullptr && tid % 32 == 0)
    a.lse[((size_t)b * a.Hq + hq) * a.hsq + row] = l > 0.f ? mr + logf(l) : kNegInf;
}

}  // namespace

hipError_t launch_fwd_f32(const Problem& p, const float* q, const float* k, const float* v, float* o,
                          float* lse, hipStream_t s) {
  F32Args a{q, k, v, o, lse, p.Hq, p.Hkv, p.Sq, p.Sk, p.Hq / p.Hkv, p.causal, p.scale, p.hsq, p.hsk};
  dim3 grid((p.Sq + 7) / 8, p.Hq, p.B);
  timing_begin(s, "fwd_f32");
  if (p.d == 64)
    hipLaunchKernelGGL((fwd_f32_kernel<64>), grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<128>), grid, dim3(256), 0, s, a);
  const hipError_t e = hipGetLastError();
  timing_end(s);
  return e;
}

}  // namespace attn
