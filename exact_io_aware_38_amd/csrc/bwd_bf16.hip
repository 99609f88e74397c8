// Backward attention in bf16 on gfx950 MFMA, by recomputation.
//
// The forward kept only O and the per-row lse. Following "AI 大模型之
// FlashAttention_01", sections "反向传播为什么可以重算" and "训练与部署 注意力
// 反向的完整链式关系", the probabilities are rebuilt tile by tile as
// P = exp(s - lse), then dV = P^T dO, dP = dO V^T, dS = P o (dP - D) with the
// softmax-Jacobian row term D_i = sum_j P_ij dP_ij, dQ = scale dS K and
// dK = scale dS^T Q. Since sum_j P_ij v_j = O_i, the row term equals
// dO_i . O_i, which a first pass computes from the saved output; masked
// probabilities are exactly zero, so their gradients are too.
//
// Three kernels, all on the caller's stream:
//  1. bwd_pre:  D_i = dO_i . O_i and lse2_i = lse_i * log2(e) (+inf for rows
//               that see no key, which makes every rebuilt probability 0);
//  2. bwd_dkdv: one workgroup per (KV head, 128-key tile); loops over the query
//               heads that share the KV head and over 64-row query tiles,
//               accumulating dK^T and dV^T in registers (no atomics);
//  3. bwd_dq:   one workgroup per (query head, 128-row query tile); loops over
//               64-key tiles, accumulating dQ^T in registers.
// The dK/dV and dQ passes both rebuild S and dP, which costs two GEMMs more
// than a single pass with atomic dQ but keeps the result deterministic.
#include "common.h"
#include "kernels.h"

#include <algorithm>
#include <cstdio>

namespace attn {

namespace {

// Element offset in a row-major [rows][D] bf16 LDS tile whose 16-byte chunks
// are XOR-swizzled per row (chunk_swizzle), so that both 16-byte row reads
// and transposed 8-byte reads are free of bank conflicts. col must be a
// multiple of 4.
template <int D>
__device__ __forceinline__ int swz(int row, int col) {
  return row * D + (((col >> 3) ^ chunk_swizzle<D>(row)) << 3) + (col & 7);
}

struct BwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* o;
  const bf16* dout;
  const float* lse;
  bf16* dq;
  bf16* dk;
  bf16* dv;
  float* lse2;    // workspace [B, Hq, Sq]
  float* delta;   // workspace [B, Hq, Sq]
  int B, Hq, Hkv, Sq, Sk, g, causal;
  float scale;
  float c;        // scale * log2(e)
  int n_ktiles, total_kv;
  int n_qtiles, total_q;
};

template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a, size_t rows) {
  constexpr int LPR = D / 8;       // lanes per row, 8 elements each
  constexpr int RPB = 256 / LPR;   // rows per block
  const size_t row = (size_t)blockIdx.x * RPB + threadIdx.x / LPR;
  const int c = threadIdx.x % LPR;
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 ov = *(const bf16x8*)(a.o + row * D + c * 8);
    const bf16x8 dv = *(const bf16x8*)(a.dout + row * D + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)ov[e], (float)dv[e], acc);
  }
#pragma unroll
  for (int s = LPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s);
  if (row < rows && c == 0) {
    a.delta[row] = acc;
    const float l = a.lse[row];
    a.lse2[row] = (l == kNegInf) ? __builtin_huge_valf() : l * kLog2e;
  }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int BQ = 64;           // query rows per staged tile
  constexpr int NT = 256;
  constexpr int DC = D / 16;
  constexpr int MB = D / 32;
  constexpr int CH_ROW = D / 8;
  constexpr int CH_THR = BQ * CH_ROW / NT;
  static_assert((BQ * CH_ROW) % NT == 0, "tile must split evenly");

  __shared__ __attribute__((aligned(16))) bf16 sq[2][BQ * D];
  __shared__ __attribute__((aligned(16))) bf16 sdo[2][BQ * D];
  __shared__ __attribute__((aligned(16))) float slse[2][BQ];
  __shared__ __attribute__((aligned(16))) float sdel[2][BQ];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int off = (a.causal == 2) ? (a.Sk - a.Sq) : 0;

  const int W = xcd_logical_id(blockIdx.x, a.total_kv);
  const int kt = W % a.n_ktiles;
  const int rest = W / a.n_ktiles;
  const int hkv = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int k0 = kt * 128;
  const int kw0 = k0 + 32 * wid;
  const int key = kw0 + l32;
  const bool kvalid = key < a.Sk;
  const bool wave_keys = kw0 < a.Sk;
  const int wave_kmax = min(kw0 + 31, a.Sk - 1);

  // K and V fragments: B operands of S = Q K^T and dP = dO V^T (column = key)
  bf16x8 kf[DC], vf[DC];
  {
    const size_t kvrow = (((size_t)b * a.Hkv + hkv) * a.Sk + (kvalid ? key : 0)) * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      if (kvalid) {
        kf[dc] = *(const bf16x8*)(a.k + kvrow + 16 * dc + 8 * hi);
        vf[dc] = *(const bf16x8*)(a.v + kvrow + 16 * dc + 8 * hi);
      } else {
        kf[dc] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        vf[dc] = kf[dc];
      }
    }
  }
  f32x16 dkt[MB], dvt[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    dkt[mb] = f32x16{};
    dvt[mb] = f32x16{};
  }

  const int n_qt = (a.Sq + BQ - 1) / BQ;
  const int qt_lo = a.causal ? min(n_qt, max(0, k0 - off) / BQ) : 0;
  const int per_head = n_qt - qt_lo;
  const int iters = a.g * per_head;

  u32x4 qreg[CH_THR], dreg[CH_THR];
  float lreg = 0.f, dlreg = 0.f;
  auto load_tile = [&](int it) {
    const int hq = hkv * a.g + it / per_head;
    const int q0 = (qt_lo + it % per_head) * BQ;
    const size_t base = ((size_t)b * a.Hq + hq) * a.Sq;
#pragma unroll
    for (int i = 0; i < CH_THR; ++i) {
      const int c = tid + i * NT;
      const int row = c / CH_ROW;
      const int col = c % CH_ROW;
      const int qi = q0 + row;
      if (qi < a.Sq) {
        qreg[i] = *(const u32x4*)(a.q + (base + qi) * D + col * 8);
        dreg[i] = *(const u32x4*)(a.dout + (base + qi) * D + col * 8);
      } else {
        qreg[i] = u32x4{0u, 0u, 0u, 0u};
        dreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    if (tid < BQ) {
      const int qi = q0 + tid;
      lreg = qi < a.Sq ? a.lse2[base + qi] : __builtin_huge_valf();
      dlreg = qi < a.Sq ? a.delta[base + qi] : 0.f;
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH_THR; ++i) {
      const int c = tid + i * NT;
      const int row = c / CH_ROW;
      const int col = c % CH_ROW;
      *(u32x4*)(&sq[buf][swz<D>(row, col * 8)]) = qreg[i];
      *(u32x4*)(&sdo[buf][swz<D>(row, col * 8)]) = dreg[i];
    }
    if (tid < BQ) {
      slse[buf][tid] = lreg;
      sdel[buf][tid] = dlreg;
    }
  };

  if (iters > 0) {
    load_tile(0);
    store_tile(0);
  }
  const int L = lane & 15;
  const int dhalf = (lane >> 4) & 1;
  for (int it = 0; it < iters; ++it) {
    __syncthreads();
    const int cur = it & 1;
    if (it + 1 < iters) load_tile(it + 1);
    const int q0 = (qt_lo + it % per_head) * BQ;
    // skip when the wavefront has no key, or no query of this tile sees any of its keys
    const bool skip = !wave_keys || (a.causal && kw0 > q0 + BQ - 1 + off);
    if (!skip) {
      const bf16* tq = sq[cur];
      const bf16* tdo = sdo[cur];
      // ---- S = Q K^T and dP = dO V^T: rows = 64 queries (2 blocks), columns = 32 keys
      f32x16 s[2], dp[2];
      s[0] = s[1] = dp[0] = dp[1] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const bf16x8 aq = *(const bf16x8*)(tq + swz<D>(32 * qb + l32, 16 * dc + 8 * hi));
          const bf16x8 ad = *(const bf16x8*)(tdo + swz<D>(32 * qb + l32, 16 * dc + 8 * hi));
          s[qb] = mfma32(aq, kf[dc], s[qb]);
          dp[qb] = mfma32(ad, vf[dc], dp[qb]);
        }
      }
      const bool need_mask = a.causal && (wave_kmax > q0 + off);
      // ---- P = exp2(s*c - lse2), dS = P o (dP - D)
      bf16x8 pf[4], dsf[4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float p[16], ds[16];
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int r = 32 * qb + 8 * i4 + 4 * hi;     // first of 4 consecutive query rows
          const f32x4 l2 = *(const f32x4*)(&slse[cur][r]);
          const f32x4 dl = *(const f32x4*)(&sdel[cur][r]);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * i4 + e;
            float pv = fast_exp2(__builtin_fmaf(s[qb][i], a.c, -l2[e]));
            if (need_mask && key > q0 + r + e + off) pv = 0.f;
            p[i] = pv;
            ds[i] = pv * (dp[qb][i] - dl[e]);
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          pf[2 * qb + h] = to_bf16x8(p[8 * h + 0], p[8 * h + 1], p[8 * h + 2], p[8 * h + 3],
                                     p[8 * h + 4], p[8 * h + 5], p[8 * h + 6], p[8 * h + 7]);
          dsf[2 * qb + h] = to_bf16x8(ds[8 * h + 0], ds[8 * h + 1], ds[8 * h + 2], ds[8 * h + 3],
                                      ds[8 * h + 4], ds[8 * h + 5], ds[8 * h + 6], ds[8 * h + 7]);
        }
      }
      // ---- dV^T += dO^T P and dK^T += Q^T dS: rows = d, columns = keys, reduction over queries
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int qc = 0; qc < 4; ++qc) {
          const int r0 = 16 * qc + 4 * hi + (L >> 2);
          const int col = 32 * mb + 16 * dhalf + 4 * (L & 3);
          const bf16x8 ado = cat4(lds_read_tr(tdo + swz<D>(r0, col)), lds_read_tr(tdo + swz<D>(r0 + 8, col)));
          const bf16x8 aqt = cat4(lds_read_tr(tq + swz<D>(r0, col)), lds_read_tr(tq + swz<D>(r0 + 8, col)));
          dvt[mb] = mfma32(ado, pf[qc], dvt[mb]);
          dkt[mb] = mfma32(aqt, dsf[qc], dkt[mb]);
        }
      }
    }
    if (it + 1 < iters) store_tile(cur ^ 1);
  }

  if (!kvalid) return;
  const size_t kvrow = (((size_t)b * a.Hkv + hkv) * a.Sk + key) * D;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      bf16x4 rk, rv;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rk[e] = (bf16)(dkt[mb][4 * i4 + e] * a.scale);
        rv[e] = (bf16)(dvt[mb][4 * i4 + e]);
      }
      *(bf16x4*)(a.dk + kvrow + 32 * mb + 8 * i4 + 4 * hi) = rk;
      *(bf16x4*)(a.dv + kvrow + 32 * mb + 8 * i4 + 4 * hi) = rv;
    }
}

template <int D>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a) {
  constexpr int BK = 64;           // keys per staged tile
  constexpr int NT = 256;
  constexpr int DC = D / 16;
  constexpr int MB = D / 32;
  constexpr int CH_ROW = D / 8;
  constexpr int CH_THR = BK * CH_ROW / NT;
  static_assert((BK * CH_ROW) % NT == 0, "tile must split evenly");

  __shared__ __attribute__((aligned(16))) bf16 sk[2][BK * D];
  __shared__ __attribute__((aligned(16))) bf16 sv[2][BK * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int off = (a.causal == 2) ? (a.Sk - a.Sq) : 0;

  const int W = xcd_logical_id(blockIdx.x, a.total_q);
  const int qt = a.n_qtiles - 1 - (W % a.n_qtiles);
  const int rest = W / a.n_qtiles;
  const int hq = rest % a.Hq;
  const int b = rest / a.Hq;
  const int hkv = hq / a.g;
  const int p0 = qt * 128 + 32 * wid;
  const int pos = p0 + l32;
  const bool valid = pos < a.Sq;
  const bool wave_rows = p0 < a.Sq;
  const int wave_maxpos = min(p0 + 31, a.Sq - 1);
  const int wg_last = min(qt * 128 + 128, a.Sq) - 1;
  int kend = a.causal ? min(a.Sk, wg_last + off + 1) : a.Sk;
  if (kend < 0) kend = 0;
  const int ntiles = (kend + BK - 1) / BK;
  int kend_w = a.causal ? min(kend, wave_maxpos + off + 1) : kend;
  if (!wave_rows) kend_w = 0;
  const int mask_from = a.causal ? min(kend, p0 + off + 1) : kend;
  const int lim = a.causal ? min(kend - 1, pos + off) : kend - 1;

  const size_t qrow = ((size_t)b * a.Hq + hq) * a.Sq + (valid ? pos : 0);
  bf16x8 qf[DC], df[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    if (valid) {
      qf[dc] = *(const bf16x8*)(a.q + qrow * D + 16 * dc + 8 * hi);
      df[dc] = *(const bf16x8*)(a.dout + qrow * D + 16 * dc + 8 * hi);
    } else {
      qf[dc] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      df[dc] = qf[dc];
    }
  }
  const float l2 = valid ? a.lse2[qrow] : __builtin_huge_valf();
  const float dl = valid ? a.delta[qrow] : 0.f;

  const bf16* kg = a.k + ((size_t)b * a.Hkv + hkv) * (size_t)a.Sk * D;
  const bf16* vg = a.v + ((size_t)b * a.Hkv + hkv) * (size_t)a.Sk * D;
  u32x4 kreg[CH_THR], vreg[CH_THR];
  auto load_tile = [&](int t) {
    const int key0 = t * BK;
#pragma unroll
    for (int i = 0; i < CH_THR; ++i) {
      const int c = tid + i * NT;
      const int row = c / CH_ROW;
      const int col = c % CH_ROW;
      const int kk = key0 + row;
      if (kk < kend) {
        kreg[i] = *(const u32x4*)(kg + (size_t)kk * D + col * 8);
        vreg[i] = *(const u32x4*)(vg + (size_t)kk * D + col * 8);
      } else {
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
        vreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int i = 0; i < CH_THR; ++i) {
      const int c = tid + i * NT;
      const int row = c / CH_ROW;
      const int col = c % CH_ROW;
      *(u32x4*)(&sk[buf][swz<D>(row, col * 8)]) = kreg[i];
      *(u32x4*)(&sv[buf][swz<D>(row, col * 8)]) = vreg[i];
    }
  };

  f32x16 dqt[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) dqt[mb] = f32x16{};

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  const int L = lane & 15;
  const int dhalf = (lane >> 4) & 1;
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    const int cur = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const int key0 = t * BK;
    if (key0 < kend_w) {
      const bf16* tk = sk[cur];
      const bf16* tv = sv[cur];
      // ---- S^T = K Q^T and dP^T = V dO^T: rows = 64 keys (2 blocks), columns = 32 queries
      f32x16 s[2], dp[2];
      s[0] = s[1] = dp[0] = dp[1] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 ak = *(const bf16x8*)(tk + swz<D>(32 * kb + l32, 16 * dc + 8 * hi));
          const bf16x8 av = *(const bf16x8*)(tv + swz<D>(32 * kb + l32, 16 * dc + 8 * hi));
          s[kb] = mfma32(ak, qf[dc], s[kb]);
          dp[kb] = mfma32(av, df[dc], dp[kb]);
        }
      }
      const bool need_mask = key0 + BK > mask_from;
      bf16x8 dsf[4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        float ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float pv = fast_exp2(__builtin_fmaf(s[kb][i], a.c, -l2));
          const int kk = key0 + 32 * kb + 8 * (i >> 2) + 4 * hi + (i & 3);
          if (need_mask && kk > lim) pv = 0.f;
          ds[i] = pv * (dp[kb][i] - dl);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h)
          dsf[2 * kb + h] = to_bf16x8(ds[8 * h + 0], ds[8 * h + 1], ds[8 * h + 2], ds[8 * h + 3],
                                      ds[8 * h + 4], ds[8 * h + 5], ds[8 * h + 6], ds[8 * h + 7]);
      }
      // ---- dQ^T += K^T dS^T: rows = d, columns = queries, reduction over 64 keys
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const int r0 = 16 * kc + 4 * hi + (L >> 2);
          const int col = 32 * mb + 16 * dhalf + 4 * (L & 3);
          const bf16x8 akt = cat4(lds_read_tr(tk + swz<D>(r0, col)), lds_read_tr(tk + swz<D>(r0 + 8, col)));
          dqt[mb] = mfma32(akt, dsf[kc], dqt[mb]);
        }
      }
    }
    if (t + 1 < ntiles) store_tile(cur ^ 1);
  }

  if (!valid) return;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i4 = 0; i4 < 4; ++i4) {
      bf16x4 r;
#pragma unroll
      for (int e = 0; e < 4; ++e) r[e] = (bf16)(dqt[mb][4 * i4 + e] * a.scale);
      *(bf16x4*)(a.dq + qrow * D + 32 * mb + 8 * i4 + 4 * hi) = r;
    }
}

template <int D>
hipError_t launch_bwd_d(BwdArgs& a, hipStream_t s, char* log, size_t log_n) {
  const size_t rows = (size_t)a.B * a.Hq * a.Sq;
  constexpr int RPB = 256 / (D / 8);
  timing_begin(s, "bwd_pre");
  hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s, a, rows);
  hipError_t e = hipGetLastError();
  timing_end(s);
  if (e != hipSuccess) return e;
  if (a.total_kv > 0) {
    timing_begin(s, "bwd_dkdv");
    hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3(a.total_kv), dim3(256), 0, s, a);
    e = hipGetLastError();
    timing_end(s);
    if (e != hipSuccess) return e;
  }
  if (a.total_q > 0) {
    timing_begin(s, "bwd_dq");
    hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3(a.total_q), dim3(256), 0, s, a);
    e = hipGetLastError();
    timing_end(s);
    if (e != hipSuccess) return e;
  }
  if (log != nullptr && log_n > 0)
    snprintf(log, log_n,
             "attn_bwd: bwd_pre<d=%d> grid=%zu; bwd_dkdv<d=%d> grid=%d (128 keys x 64-row query tiles); "
             "bwd_dq<d=%d> grid=%d (128 rows x 64-key tiles)",
             D, (rows + RPB - 1) / RPB, D, a.total_kv, D, a.total_q);
  return hipSuccess;
}

}  // namespace

size_t bwd_workspace_bytes(const Problem& p) {
  const size_t rows = (size_t)p.B * p.Hq * p.Sq;
  return ((rows * sizeof(float) + 255) / 256) * 256 * 2;
}

hipError_t launch_bwd_bf16(const Problem& p, const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws,
                           hipStream_t s, char* log, size_t log_n) {
  BwdArgs a{};
  a.q = (const bf16*)q;
  a.k = (const bf16*)k;
  a.v = (const bf16*)v;
  a.o = (const bf16*)o;
  a.dout = (const bf16*)dout;
  a.lse = lse;
  a.dq = (bf16*)dq;
  a.dk = (bf16*)dk;
  a.dv = (bf16*)dv;
  const size_t rows = (size_t)p.B * p.Hq * p.Sq;
  a.lse2 = (float*)ws;
  a.delta = (float*)((char*)ws + ((rows * sizeof(float) + 255) / 256) * 256);
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Sq = p.Sq;
  a.Sk = p.Sk;
  a.g = p.Hq / p.Hkv;
  a.causal = p.causal;
  a.scale = p.scale;
  a.c = p.scale * kLog2e;
  a.n_ktiles = (p.Sk + 127) / 128;
  a.total_kv = p.B * p.Hkv * a.n_ktiles;
  a.n_qtiles = (p.Sq + 127) / 128;
  a.total_q = p.B * p.Hq * a.n_qtiles;
  return p.d == 64 ? launch_bwd_d<64>(a, s, log, log_n) : launch_bwd_d<128>(a, s, log, log_n);
}

}  // namespace attn
