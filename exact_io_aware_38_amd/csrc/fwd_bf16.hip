// Forward attention in bf16 on gfx950 MFMA: tiled prefill and split-key decode.
//
// Method: the online-softmax recurrence of "Flash Attention FA1->FA4 /
// pre-training practice" §1.2, kept in the unnormalised (m, l, u) form of "AI
// 大模型之 FlashAttention_01" §4.1 / "瓦片状态如何保持精确语义": per query row,
// a running max m, a running denominator l and an accumulator u are rescaled
// by exp(m_old - m_new) whenever a key tile raises the max, and O = u / l at
// the end, with lse = m + ln l kept for the backward. Scores never leave the
// registers (the fusion of §1.3 of the first page); the outer loop runs over
// query tiles and the inner one over key tiles (the loop order of §4.3 of
// the second page). Key tiles above the causal diagonal are never loaded
// (§2.1 of the first page), and the rescale is skipped when no row of the
// wavefront raised its max (§2.3 of the first page, with threshold 0).
//
// Mapping to CDNA4:
//  * a wavefront owns 32*NB query rows as MFMA columns and computes the
//    transposed score tile S^T = K Q^T (rows = keys), so that every lane holds
//    the scores of one query row: the row max and sum reduce inside the lane
//    plus one swap between lane halves, and the probabilities sit in the
//    exact register layout the B operand of O^T = V^T P^T expects;
//  * K and V tiles (64 keys) are staged through LDS, double-buffered, shared by
//    the NW wavefronts of the workgroup; V^T fragments come from
//    ds_read_b64_tr_b16 on the row-major V tile;
//  * exp2 with log2(e) folded into the score scale: one FMA and one v_exp_f32
//    per score.
#include "common.h"
#include "kernels.h"

#include <algorithm>

namespace attn {

namespace {

template <int D>
struct FwdTile {
  static constexpr int BC = 64;          // keys per tile
  static constexpr int KS = D + 8;       // K row stride in LDS (bf16), 16 B pad
  static constexpr int VS = D + 16;      // V row stride in LDS (bf16), 32 B pad
  static constexpr int K_ELEMS = BC * KS;
  static constexpr int V_ELEMS = BC * VS;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
};

struct FwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  float* part_o;     // split path: [nsplit, B, Hq, Sq, D]
  float* part_lse;   // split path: [nsplit, B, Hq, Sq]
  int B, Hq, Hkv, Sq, Sk, g, causal;
  float c;           // scale * log2(e)
  int hw, n_hgroups, rows_per_wg, n_ptiles, total_wgs;
  int nsplit, split_keys;
};

template <int D, int NW, int NB, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(FwdArgs a) {
  using T = FwdTile<D>;
  constexpr int BC = T::BC;
  constexpr int NT = NW * 64;
  constexpr int CH_ROW = D / 8;             // 16-byte chunks per row
  constexpr int CH_THR = BC * CH_ROW / NT;  // chunks per thread per tensor per tile
  static_assert((BC * CH_ROW) % NT == 0, "tile must split evenly over the threads");
  constexpr int QW = 32 * NB;
  constexpr int MB = D / 32;                // 32-row blocks of O^T (over d)
  constexpr int DC = D / 16;                // 16-wide reduction chunks over d

  __shared__ __attribute__((aligned(16))) bf16 smem[2 * T::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int off = (a.causal == 2) ? (a.Sk - a.Sq) : 0;

  int b, hkv, kbeg, kend, split = 0;
  int hq[NB], pos[NB];
  bool colv[NB];
  int wave_minpos, wave_maxpos;
  bool wave_rows;

  if constexpr (!SPLIT) {
    const int W = xcd_logical_id(blockIdx.x, a.total_wgs);
    const int ptile = a.n_ptiles - 1 - (W % a.n_ptiles);   // longest causal tiles first
    int rest = W / a.n_ptiles;
    const int hgrp = rest % a.n_hgroups;
    rest /= a.n_hgroups;
    hkv = rest % a.Hkv;
    b = rest / a.Hkv;
    const int head = hkv * a.g + hgrp * a.hw + (wid % a.hw);
    const int p0 = ptile * a.rows_per_wg + QW * (wid / a.hw);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      hq[nb] = head;
      pos[nb] = p0 + 32 * nb + l32;
      colv[nb] = pos[nb] < a.Sq;
    }
    wave_rows = p0 < a.Sq;
    wave_minpos = p0;
    wave_maxpos = min(p0 + QW - 1, a.Sq - 1);
    const int wg_last = min((ptile + 1) * a.rows_per_wg, a.Sq) - 1;
    kbeg = 0;
    kend = a.causal ? min(a.Sk, wg_last + off + 1) : a.Sk;
  } else {
    const int W = blockIdx.x;
    split = W % a.nsplit;
    const int rest = W / a.nsplit;
    hkv = rest % a.Hkv;
    b = rest / a.Hkv;
    // column n packs (query head of the group, position): n = hg * Sq + position
    const int n = l32;
    colv[0] = n < a.g * a.Sq;
    hq[0] = hkv * a.g + (colv[0] ? n / a.Sq : 0);
    pos[0] = colv[0] ? n % a.Sq : 0;
    wave_rows = true;
    wave_minpos = 0;
    wave_maxpos = a.Sq - 1;
    kbeg = split * a.split_keys;
    kend = min(a.Sk, kbeg + a.split_keys);
    if (a.causal) kend = min(kend, a.Sq - 1 + off + 1);
  }
  if (kend < kbeg) kend = kbeg;
  const int ntiles = (kend - kbeg + BC - 1) / BC;
  // keys this wavefront must process, and the first key that some of its rows cannot see
  int kend_w = a.causal ? min(kend, wave_maxpos + off + 1) : kend;
  if (!wave_rows) kend_w = kbeg;
  const int mask_from = a.causal ? min(kend, wave_minpos + off + 1) : kend;

  // Q fragments (B operand of S^T = K Q^T): lane holds row pos, d = 16*dc + 8*hi .. +7
  bf16x8 qf[NB][DC];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const bf16* qp = a.q + (((size_t)b * a.Hq + hq[nb]) * a.Sq + (colv[nb] ? pos[nb] : 0)) * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      if (colv[nb]) {
        qf[nb][dc] = *(const bf16x8*)(qp + 16 * dc + 8 * hi);
      } else {
        qf[nb][dc] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
      }
    }
  }

  const bf16* kg = a.k + ((size_t)b * a.Hkv + hkv) * (size_t)a.Sk * D;
  const bf16* vg = a.v + ((size_t)b * a.Hkv + hkv) * (size_t)a.Sk * D;

  u32x4 kreg[CH_THR], vreg[CH_THR];
  auto load_tile = [&](int t) {
    const int key0 = kbeg + t * BC;
#pragma unroll
    for (int i = 0; i < CH_THR; ++i) {
      const int c = tid + i * NT;
      const int row = c / CH_ROW;
      const int col = c % CH_ROW;
      const int key = key0 + row;
      if (key < kend) {
        kreg[i] = *(const u32x4*)(kg + (size_t)key * D + col * 8);
        vreg[i] = *(const u32x4*)(vg + (size_t)key * D + col * 8);
      } else {
        kreg[i] = u32x4{0u, 0u, 0u, 0u};
        vreg[i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
  };
  auto store_tile = [&](int buf) {
    bf16* sk = smem + buf * T::BUF;
    bf16* sv = sk + T::K_ELEMS;
#pragma unroll
    for (int i = 0; i < CH_THR; ++i) {
      const int c = tid + i * NT;
      const int row = c / CH_ROW;
      const int col = c % CH_ROW;
      *(u32x4*)(sk + row * T::KS + col * 8) = kreg[i];
      *(u32x4*)(sv + row * T::VS + col * 8) = vreg[i];
    }
  };

  f32x16 acc[MB][NB];
  float m2[NB], lsum[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m2[nb] = kNegInf;
    lsum[nb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb][nb] = f32x16{};
  }

  if (ntiles > 0) {
    load_tile(0);
    store_tile(0);
  }
  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();
    const int cur = t & 1;
    if (t + 1 < ntiles) load_tile(t + 1);
    const int key0 = kbeg + t * BC;
    if (key0 < kend_w) {
      const bf16* sk = smem + cur * T::BUF;
      const bf16* sv = sk + T::K_ELEMS;
      // ---- scores S^T = K Q^T: rows = 64 keys (2 blocks), columns = query rows
      f32x16 s[2][NB];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s[kb][nb] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 ak = *(const bf16x8*)(sk + (32 * kb + l32) * T::KS + 16 * dc + 8 * hi);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) s[kb][nb] = mfma32(ak, qf[nb][dc], s[kb][nb]);
        }
      }
      // ---- mask (diagonal and ragged tiles only), before the max
      if (key0 + BC > mask_from) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int lim = a.causal ? min(kend - 1, pos[nb] + off) : kend - 1;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * hi + (i & 3);
              if (key > lim) s[kb][nb][i] = kNegInf;
            }
          }
      }
      // ---- online softmax update
      bf16x8 pf[4][NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float mx = s[0][nb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][nb][i]);
        mx = max_halves(mx);
        const float mnew = fmaxf(m2[nb], mx * a.c);
        const bool grow = mnew > m2[nb];
        if (wave_any(grow)) {
          const float alpha = grow ? fast_exp2(m2[nb] - mnew) : 1.f;
          lsum[nb] *= alpha;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[mb][nb] *= alpha;
        }
        m2[nb] = mnew;
        const float msub = (mnew == kNegInf) ? 0.f : mnew;
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              p[e] = fast_exp2(__builtin_fmaf(s[kb][nb][8 * h + e], a.c, -msub));
              ps += p[e];
            }
            pf[2 * kb + h][nb] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
          }
        lsum[nb] += ps;
      }
      // ---- O^T += V^T P^T: rows = d, columns = query rows, reduction over 64 keys
      const int L = lane & 15;
      const int dhalf = (lane >> 4) & 1;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          const bf16* vp = sv + (16 * kc + 4 * hi + (L >> 2)) * T::VS + 32 * mb + 16 * dhalf + 4 * (L & 3);
          const bf16x8 av = cat4(lds_read_tr(vp), lds_read_tr(vp + 8 * T::VS));
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma32(av, pf[kc][nb], acc[mb][nb]);
        }
      }
    }
    if (t + 1 < ntiles) store_tile(cur ^ 1);
  }

  // ---- epilogue: O = u / l, lse = ln(2) * (m2 + log2 l)
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float lt = sum_halves(lsum[nb]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse_v = lt > 0.f ? (m2[nb] + __log2f(lt)) * kLn2 : kNegInf;
    if (!colv[nb]) continue;
    if constexpr (!SPLIT) {
      bf16* op = a.o + (((size_t)b * a.Hq + hq[nb]) * a.Sq + pos[nb]) * D;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          bf16x4 r;
          r[0] = (bf16)(acc[mb][nb][4 * q4 + 0] * inv);
          r[1] = (bf16)(acc[mb][nb][4 * q4 + 1] * inv);
          r[2] = (bf16)(acc[mb][nb][4 * q4 + 2] * inv);
          r[3] = (bf16)(acc[mb][nb][4 * q4 + 3] * inv);
          *(bf16x4*)(op + 32 * mb + 8 * q4 + 4 * hi) = r;
        }
      if (a.lse != nullptr && hi == 0) a.lse[((size_t)b * a.Hq + hq[nb]) * a.Sq + pos[nb]] = lse_v;
    } else {
      const size_t row = (((size_t)split * a.B + b) * a.Hq + hq[nb]) * a.Sq + pos[nb];
      float* pp = a.part_o + row * D;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          f32x4 r;
          r[0] = acc[mb][nb][4 * q4 + 0] * inv;
          r[1] = acc[mb][nb][4 * q4 + 1] * inv;
          r[2] = acc[mb][nb][4 * q4 + 2] * inv;
          r[3] = acc[mb][nb][4 * q4 + 3] * inv;
          *(f32x4*)(pp + 32 * mb + 8 * q4 + 4 * hi) = r;
        }
      if (hi == 0) a.part_lse[row] = lse_v;
    }
  }
}

// ---------------------------------------------------------------------------
// Pipelined prefill kernel.
//
// Workgroup = 4 wavefronts x 64 query rows (two 32-column MFMA blocks each).
// Key/value tiles of 64 keys are copied HBM -> LDS by the DMA path of
// global_load_lds (no staging registers) into a ring of 4 stages, issued two
// tiles ahead. Iteration j computes S(j) = K_j Q^T, then issues the P V
// product of tile j-1, then runs the softmax of tile j on the vector ALU while
// those MFMAs execute; the accumulator is rescaled only when some row's max
// grew by more than RESCALE_T (log2 units), so rescales are rare and the
// probabilities stay below 2^RESCALE_T. u / l is unchanged by the choice of
// reference max, so the result is the same as rescaling on every increase.
// LDS tiles are unpadded [64][D] bf16 rows whose 16-byte chunks are XOR
// swizzled: K by (row & 7) for conflict-free 16-byte row reads, V by
// 2*(row & 3) for conflict-free transposed reads.
// ---------------------------------------------------------------------------
constexpr float RESCALE_T = 8.0f;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void glb_void;

__device__ __forceinline__ void dma16(const void* g, lds_void* l) {
  __builtin_amdgcn_global_load_lds((glb_void*)g, l, 16, 0, 0);
}

template <int D>
struct Ring {
  static constexpr int BC = 64;
  static constexpr int TILE = BC * D * 2;       // bytes of one K or V tile
  static constexpr int STAGE = 2 * TILE;        // K then V
  static constexpr int NSTAGE = 4;
  static constexpr int INSTR = D / 32;          // DMA instructions per wavefront per tensor per tile
};

template <int D, int NB>
__global__ __launch_bounds__(256) void fwd_prefill_kernel(FwdArgs a) {
  using R = Ring<D>;
  constexpr int BC = R::BC;
  constexpr int QW = 32 * NB;
  constexpr int MB = D / 32;
  constexpr int DC = D / 16;
  constexpr int CPR = D / 8;                    // 16-byte chunks per row
  constexpr int RB = 2 * D;                     // bytes per row

  __shared__ __attribute__((aligned(1024))) char smem[R::NSTAGE * R::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int off = (a.causal == 2) ? (a.Sk - a.Sq) : 0;

  const int W = xcd_logical_id(blockIdx.x, a.total_wgs);
  const int ptile = a.n_ptiles - 1 - (W % a.n_ptiles);   // longest causal tiles first
  int rest = W / a.n_ptiles;
  const int hgrp = rest % a.n_hgroups;
  rest /= a.n_hgroups;
  const int hkv = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int head = hkv * a.g + hgrp * a.hw + (wid % a.hw);
  const int p0 = ptile * a.rows_per_wg + QW * (wid / a.hw);
  int pos[NB];
  bool colv[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    pos[nb] = p0 + 32 * nb + l32;
    colv[nb] = pos[nb] < a.Sq;
  }
  const int wg_last = min((ptile + 1) * a.rows_per_wg, a.Sq) - 1;
  int kend = a.causal ? min(a.Sk, wg_last + off + 1) : a.Sk;
  if (kend < 0) kend = 0;
  const int ntiles = (kend + BC - 1) / BC;
  const int wave_maxpos = min(p0 + QW - 1, a.Sq - 1);
  int kend_w = a.causal ? min(kend, wave_maxpos + off + 1) : kend;
  if (p0 >= a.Sq || kend_w < 0) kend_w = 0;
  const int nt_w = (kend_w + BC - 1) / BC;      // tiles this wavefront computes (a prefix)
  const int mask_from = a.causal ? max(0, min(kend, p0 + off + 1)) : kend;

  // Q fragments: B operand of S^T = K Q^T (column = query row, d = 16*dc + 8*hi .. +7)
  bf16x8 qf[NB][DC];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const bf16* qp = a.q + (((size_t)b * a.Hq + head) * a.Sq + (colv[nb] ? pos[nb] : 0)) * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      qf[nb][dc] = colv[nb] ? *(const bf16x8*)(qp + 16 * dc + 8 * hi)
                            : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }

  const bf16* kg = a.k + ((size_t)b * a.Hkv + hkv) * (size_t)a.Sk * D;
  const bf16* vg = a.v + ((size_t)b * a.Hkv + hkv) * (size_t)a.Sk * D;

  // DMA of tile t into stage t % NSTAGE: lane i of instruction n writes LDS chunk
  // P = (wid*INSTR + n)*64 + i, i.e. row P / CPR, physical chunk P % CPR, which
  // holds logical chunk (physical ^ swizzle(row)). Rows past kend repeat row kend-1
  // (finite data whose probabilities are masked to 0).
  auto issue = [&](int t) {
    const int key0 = t * BC;
    char* stage = smem + (t % R::NSTAGE) * R::STAGE;
#pragma unroll
    for (int n = 0; n < R::INSTR; ++n) {
      const int P = (wid * R::INSTR + n) * 64 + lane;
      const int row = P / CPR;
      const int phys = P % CPR;
      const size_t key = (size_t)min(key0 + row, kend - 1);
      dma16(kg + key * D + (phys ^ (row & 7)) * 8, (lds_void*)(stage + (wid * R::INSTR + n) * 1024));
      dma16(vg + key * D + (phys ^ ((row & 3) << 1)) * 8,
            (lds_void*)(stage + R::TILE + (wid * R::INSTR + n) * 1024));
    }
  };

  f32x16 acc[MB][NB];
  float m2[NB], lsum[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    m2[nb] = kNegInf;
    lsum[nb] = 0.f;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb][nb] = f32x16{};
  }
  bf16x8 pf[4][NB];
#pragma unroll
  for (int kc = 0; kc < 4; ++kc)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) pf[kc][nb] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});

  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);
  const int L = lane & 15;
  const int dhalf = (lane >> 4) & 1;

  for (int j = 0; j <= ntiles; ++j) {
    // tile j has landed in LDS for every wavefront (each waits for its own DMA,
    // the barrier for everybody's); also, every wavefront is done with tile j-2
    if (j + 1 < ntiles) {
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * R::INSTR) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    if (j + 2 < ntiles) issue(j + 2);

    const char* stK = smem + (j % R::NSTAGE) * R::STAGE;
    const char* stV = smem + ((j + R::NSTAGE - 1) % R::NSTAGE) * R::STAGE + R::TILE;
    const int key0 = j * BC;
    const bool do_s = j < nt_w;
    const bool do_pv = j >= 1 && j - 1 < nt_w;

    f32x16 s[2][NB];
    if (do_s) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) s[kb][nb] = f32x16{};
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const int r = 32 * kb + l32;
          const bf16x8 ak = *(const bf16x8*)(stK + r * RB + (((2 * dc + hi) ^ (r & 7)) << 4));
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) s[kb][nb] = mfma32(ak, qf[nb][dc], s[kb][nb]);
        }
      }
    }
    if (do_pv) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
          bf16x4 h[2];
#pragma unroll
          for (int t = 0; t < 2; ++t) {
            const int r = 16 * kc + 8 * t + 4 * hi + (L >> 2);
            const int c = (4 * mb + 2 * dhalf + ((L & 3) >> 1)) ^ ((r & 3) << 1);
            h[t] = lds_read_tr((const bf16*)(stV + r * RB + (c << 4) + ((L & 1) << 3)));
          }
          const bf16x8 av = cat4(h[0], h[1]);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) acc[mb][nb] = mfma32(av, pf[kc][nb], acc[mb][nb]);
        }
      }
    }
    if (do_s) {
      if (key0 + BC > mask_from) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
            const int lim = a.causal ? min(kend - 1, pos[nb] + off) : kend - 1;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * hi + (i & 3);
              if (key > lim) s[kb][nb][i] = kNegInf;
            }
          }
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float mx = s[0][nb][0];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][nb][i]);
        mx = max_halves(mx) * a.c;
        // move the reference max only when the row max grew by more than RESCALE_T
        const bool grow = mx > m2[nb] + RESCALE_T;
        if (wave_any(grow)) {
          const float mnew = grow ? mx : m2[nb];
          const float alpha = grow ? fast_exp2(m2[nb] - mnew) : 1.f;
          lsum[nb] *= alpha;
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[mb][nb] *= alpha;
          m2[nb] = mnew;
        }
        const float msub = (m2[nb] == kNegInf) ? 0.f : m2[nb];
        float ps = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            float p[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              p[e] = fast_exp2(__builtin_fmaf(s[kb][nb][8 * h + e], a.c, -msub));
              ps += p[e];
            }
            pf[2 * kb + h][nb] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
          }
        lsum[nb] += ps;
      }
    }
  }

#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const float lt = sum_halves(lsum[nb]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse_v = lt > 0.f ? (m2[nb] + __log2f(lt)) * kLn2 : kNegInf;
    if (!colv[nb]) continue;
    bf16* op = a.o + (((size_t)b * a.Hq + head) * a.Sq + pos[nb]) * D;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 r;
        r[0] = (bf16)(acc[mb][nb][4 * q4 + 0] * inv);
        r[1] = (bf16)(acc[mb][nb][4 * q4 + 1] * inv);
        r[2] = (bf16)(acc[mb][nb][4 * q4 + 2] * inv);
        r[3] = (bf16)(acc[mb][nb][4 * q4 + 3] * inv);
        *(bf16x4*)(op + 32 * mb + 8 * q4 + 4 * hi) = r;
      }
    if (a.lse != nullptr && hi == 0) a.lse[((size_t)b * a.Hq + head) * a.Sq + pos[nb]] = lse_v;
  }
}

// Merge of the per-slice partial results (the update of §1.2 of the first page
// applied to whole slices): lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s.
template <int D>
__global__ __launch_bounds__(64) void combine_split_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_lse,
                                                           bf16* __restrict__ o, float* __restrict__ lse,
                                                           int nsplit, size_t rows) {
  const size_t row = blockIdx.x;
  if (row >= rows) return;
  const int lane = threadIdx.x;
  float m = kNegInf;
  for (int s = 0; s < nsplit; ++s) m = fmaxf(m, part_lse[(size_t)s * rows + row]);
  constexpr int PER = D / 64;
  float accv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) accv[j] = 0.f;
  float tot = 0.f;
  if (m != kNegInf) {
    for (int s = 0; s < nsplit; ++s) {
      const float ls = part_lse[(size_t)s * rows + row];
      const float w = __expf(ls - m);      // exp(-inf) = 0 for empty slices
      tot += w;
      if (w != 0.f) {
        const float* po = part_o + ((size_t)s * rows + row) * D;
#pragma unroll
        for (int j = 0; j < PER; ++j) accv[j] += w * po[lane * PER + j];
      }
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) o[row * D + lane * PER + j] = (bf16)(accv[j] * inv);
  if (lse != nullptr && lane == 0) lse[row] = tot > 0.f ? m + __logf(tot) : kNegInf;
}

template <int D>
hipError_t launch_prefill_d(const FwdArgs& a, hipStream_t s) {
  timing_begin(s, "fwd_prefill_bf16");
  hipLaunchKernelGGL((fwd_prefill_kernel<D, 2>), dim3(a.total_wgs), dim3(256), 0, s, a);
  const hipError_t e = hipGetLastError();
  timing_end(s);
  return e;
}

template <int D>
hipError_t launch_split_d(const FwdArgs& a, int rows, hipStream_t s) {
  timing_begin(s, "fwd_split_bf16");
  hipLaunchKernelGGL((fwd_bf16_kernel<D, 1, 1, true>), dim3(a.nsplit * a.B * a.Hkv), dim3(64), 0, s, a);
  hipError_t e = hipGetLastError();
  timing_end(s);
  if (e != hipSuccess) return e;
  timing_begin(s, "combine_split");
  hipLaunchKernelGGL((combine_split_kernel<D>), dim3(rows), dim3(64), 0, s, a.part_o, a.part_lse,
                     a.o, a.lse, a.nsplit, (size_t)rows);
  e = hipGetLastError();
  timing_end(s);
  return e;
}

FwdArgs base_args(const Problem& p, const void* q, const void* k, const void* v, void* o, float* lse) {
  FwdArgs a{};
  a.q = (const bf16*)q;
  a.k = (const bf16*)k;
  a.v = (const bf16*)v;
  a.o = (bf16*)o;
  a.lse = lse;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Sq = p.Sq;
  a.Sk = p.Sk;
  a.g = p.Hq / p.Hkv;
  a.causal = p.causal;
  a.c = p.scale * kLog2e;
  return a;
}

}  // namespace

PrefillPlan plan_prefill(const Problem& p) {
  PrefillPlan pl{};
  const int g = p.Hq / p.Hkv;
  pl.hw = (g % 4 == 0) ? 4 : (g % 2 == 0) ? 2 : 1;
  pl.n_hgroups = g / pl.hw;
  pl.rows_per_wg = 4 * 64 / pl.hw;
  pl.n_ptiles = (p.Sq + pl.rows_per_wg - 1) / pl.rows_per_wg;
  pl.total_wgs = p.B * p.Hkv * pl.n_hgroups * pl.n_ptiles;
  return pl;
}

SplitPlan plan_split(const Problem& p) {
  SplitPlan sp{};
  const int g = p.Hq / p.Hkv;
  sp.use = (long long)g * p.Sq <= 32;
  if (!sp.use) return sp;
  const int tiles = (p.Sk + 63) / 64;
  const int units = p.B * p.Hkv;
  int ns = (2048 + units - 1) / units;
  ns = std::max(1, std::min(ns, tiles / 4));
  const int tiles_per = std::max(1, (tiles + ns - 1) / ns);
  ns = std::max(1, (tiles + tiles_per - 1) / tiles_per);
  sp.nsplit = ns;
  sp.split_keys = tiles_per * 64;
  const size_t rows = (size_t)p.B * p.Hq * p.Sq;
  const size_t o_bytes = (size_t)ns * rows * p.d * sizeof(float);
  const size_t l_bytes = (size_t)ns * rows * sizeof(float);
  sp.ws_bytes = ((o_bytes + 255) / 256) * 256 + l_bytes;
  return sp;
}

hipError_t launch_fwd_prefill_bf16(const Problem& p, const PrefillPlan& pl, const void* q,
                                   const void* k, const void* v, void* o, float* lse, hipStream_t s) {
  FwdArgs a = base_args(p, q, k, v, o, lse);
  a.hw = pl.hw;
  a.n_hgroups = pl.n_hgroups;
  a.rows_per_wg = pl.rows_per_wg;
  a.n_ptiles = pl.n_ptiles;
  a.total_wgs = pl.total_wgs;
  if (a.total_wgs == 0) return hipSuccess;
  return p.d == 64 ? launch_prefill_d<64>(a, s) : launch_prefill_d<128>(a, s);
}

hipError_t launch_fwd_split_bf16(const Problem& p, const SplitPlan& sp, const void* q,
                                 const void* k, const void* v, void* o, float* lse, void* ws,
                                 hipStream_t s) {
  FwdArgs a = base_args(p, q, k, v, o, lse);
  a.nsplit = sp.nsplit;
  a.split_keys = sp.split_keys;
  const size_t rows = (size_t)p.B * p.Hq * p.Sq;
  const size_t o_bytes = (size_t)sp.nsplit * rows * p.d * sizeof(float);
  a.part_o = (float*)ws;
  a.part_lse = (float*)((char*)ws + ((o_bytes + 255) / 256) * 256);
  return p.d == 64 ? launch_split_d<64>(a, (int)rows, s) : launch_split_d<128>(a, (int)rows, s);
}

}  // namespace attn
