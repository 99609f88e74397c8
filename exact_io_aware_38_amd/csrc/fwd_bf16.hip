// Forward attention in bf16 on gfx950 MFMA: tiled prefill and split-key decode.
//
// Method: the online-softmax recurrence of "Flash Attention FA1->FA4 /
// pre-training practice" §1.2, kept in the unnormalised (m, l, u) form of "AI
// 大模型之 FlashAttention_01" §4.1 / "瓦片状态如何保持精确语义": per query row,
// a running max m, a running denominator l and an accumulator u are rescaled
// by exp(m_old - m_new) when a key tile raises the max, and O = u / l at the
// end, with lse = m + ln l kept for the backward. Scores never leave the
// registers (the fused kernel of §1.3 of the first page); the outer loop runs
// over query tiles and the inner one over key tiles (the loop order of §4.3 of
// the second page). Key tiles above the causal diagonal are never loaded (§2.1
// of the first page), and the rescale is skipped unless some row's max grew
// by more than RESCALE_T (§2.3 of the first page describes the skip; with a
// threshold the probabilities stay below 2^RESCALE_T and u / l is unchanged).
//
// Mapping to CDNA4:
//  * a wavefront owns 32 query rows as MFMA columns and computes the transposed
//    score tile S^T = K Q^T (rows = keys), so every lane holds the scores of one
//    query row: the row max and sum reduce inside the lane plus one swap between
//    lane halves, and the probabilities already sit in the B-operand layout of
//    O^T = V^T P^T;
//  * V is first transposed once per call into a [d][keys] workspace whose keys
//    are permuted inside each group of 16 so that one 16-byte LDS read yields
//    the 8 keys an MFMA lane needs (transposed LDS reads are several times
//    slower than row reads on this chip);
//  * K and V^T tiles (64 keys) go HBM -> LDS through the DMA path of
//    global_load_lds into a 4-stage ring, issued two tiles ahead;
//  * two wavefronts share each SIMD and run the per-tile steps in opposite
//    orders so that one's softmax (vector ALU) overlaps the other's MFMAs;
//  * exp2 with log2(e) folded into the score scale: one FMA and one v_exp_f32
//    per score.
#include "common.h"
#include "kernels.h"
#include "tiles.h"

#include <algorithm>
#include <type_traits>

namespace attn {

namespace {

constexpr float RESCALE_T = 8.0f;   // log2 units
constexpr int BC = 64;               // keys per tile

struct FwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* vt;    // prefill: transposed V, [B, Hkv, D, skp], keys permuted by vt_perm
  bf16* o;
  float* lse;
  float* part_o;     // split path: [nsplit, B, Hq, Sq, D]
  float* part_lse;   // split path: [nsplit, B, Hq, Sq]
  int B, Hq, Hkv, Sq, Sk, g, causal;
  int skp;           // Sk rounded up to the key tile
  float c;           // scale * log2(e)
  int hw, n_hgroups, rows_per_wg, n_ptiles, total_wgs;
  int nsplit, split_keys;
};

// ---------------------------------------------------------------------------
// Prefill: 8 wavefronts (two per SIMD) x 32 query rows per workgroup.
// Phase A wavefronts do S(j), P(j-1)V(j-1), softmax(j) per step; phase B
// wavefronts do softmax(j-1), P(j-1)V(j-1), S(j).
// ---------------------------------------------------------------------------
template <int D>
struct Ring {
  static constexpr int TILE = BC * D * 2;       // bytes of one K or V^T tile
  static constexpr int STAGE = 2 * TILE;        // K then V^T
  static constexpr int NSTAGE = 4;
  static constexpr int INSTR = D / 64;          // DMA instructions per wavefront per tensor per tile
};

template <int D>
__global__ __launch_bounds__(512) void fwd_prefill_kernel(FwdArgs a) {
  using R = Ring<D>;
  constexpr int MB = D / 32;
  constexpr int DC = D / 16;
  constexpr int CPR = D / 8;                    // 16-byte chunks per K row
  constexpr int RB = 2 * D;                     // bytes per K row

  __shared__ __attribute__((aligned(1024))) char smem[R::NSTAGE * R::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bool phase_b = wid >= 4;
  const int off = (a.causal == 2) ? (a.Sk - a.Sq) : 0;

  const int W = xcd_logical_id(blockIdx.x, a.total_wgs);
  const int ptile = a.n_ptiles - 1 - (W % a.n_ptiles);   // longest causal tiles first
  int rest = W / a.n_ptiles;
  const int hgrp = rest % a.n_hgroups;
  rest /= a.n_hgroups;
  const int hkv = rest % a.Hkv;
  const int b = rest / a.Hkv;
  // the two phases take alternating 32-row blocks, which keeps their causal work equal
  const int slot = (wid & 3) * 2 + (wid >> 2);
  const int head = hkv * a.g + hgrp * a.hw + slot % a.hw;
  const int p0 = ptile * a.rows_per_wg + 32 * (slot / a.hw);
  const int pos = p0 + l32;
  const bool colv = pos < a.Sq;
  const int wg_last = min((ptile + 1) * a.rows_per_wg, a.Sq) - 1;
  int kend = a.causal ? min(a.Sk, wg_last + off + 1) : a.Sk;
  if (kend < 0) kend = 0;
  const int ntiles = (kend + BC - 1) / BC;
  const int wave_maxpos = min(p0 + 31, a.Sq - 1);
  int kend_w = a.causal ? min(kend, wave_maxpos + off + 1) : kend;
  if (p0 >= a.Sq || kend_w < 0) kend_w = 0;
  const int nt_w = (kend_w + BC - 1) / BC;       // tiles this wavefront computes (a prefix)
  const int mask_from = a.causal ? max(0, min(kend, p0 + off + 1)) : kend;
  const int lim = a.causal ? min(kend - 1, pos + off) : kend - 1;

  bf16x8 qf[DC];
  {
    const bf16* qp = a.q + (((size_t)b * a.Hq + head) * a.Sq + (colv ? pos : 0)) * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      qf[dc] = colv ? *(const bf16x8*)(qp + 16 * dc + 8 * hi) : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    // Re-define the fragments after they arrived: the compiler then knows no
    // load is pending on them inside the loop, where a wait on the memory
    // counter would also wait for the K/V prefetch in flight.
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      u32x4 t = __builtin_bit_cast(u32x4, qf[dc]);
      asm volatile("" : "+v"(t));
      qf[dc] = __builtin_bit_cast(bf16x8, t);
    }
  }
  const bf16* kg = a.k + ((size_t)b * a.Hkv + hkv) * (size_t)a.Sk * D;
  const bf16* vtg = a.vt + ((size_t)b * a.Hkv + hkv) * (size_t)D * a.skp;

  // Per-lane DMA geometry: lane i of instruction n writes LDS chunk
  // P = (wid*INSTR + n)*64 + i of a tile, i.e. K row P / CPR, physical chunk
  // P % CPR (V^T row P / 8, physical chunk P % 8), and loads the logical chunk
  // (physical ^ swizzle(row)) from global memory.
  int krow[R::INSTR], koff[R::INSTR], voff[R::INSTR];
#pragma unroll
  for (int n = 0; n < R::INSTR; ++n) {
    const int P = (wid * R::INSTR + n) * 64 + lane;
    krow[n] = P / CPR;
    koff[n] = ((P % CPR) ^ chunk_swizzle<D>(krow[n])) * 8;
    const int vrow = P / 8;
    voff[n] = vrow * a.skp + ((P % 8) ^ vt_swizzle(vrow)) * 8;
  }
  // DMA instruction q (0 .. 2*INSTR-1) of tile t: K for even q, V^T for odd q.
  auto issue_one = [&](int t, int q) {
    const int key0 = t * BC;
    char* stage = smem + (t % R::NSTAGE) * R::STAGE;
    const int n = q >> 1;
    if ((q & 1) == 0) {
      // rows past kend repeat row kend-1 (finite data; their probabilities are masked to 0)
      const bf16* ks = (key0 + BC <= kend) ? kg + (size_t)key0 * D + krow[n] * D + koff[n]
                                           : kg + (size_t)min(key0 + krow[n], kend - 1) * D + koff[n];
      dma16(ks, (lds_void*)(stage + (wid * R::INSTR + n) * 1024));
    } else {
      dma16(vtg + key0 + voff[n], (lds_void*)(stage + R::TILE + (wid * R::INSTR + n) * 1024));
    }
  };
  auto issue = [&](int t) {
#pragma unroll
    for (int q = 0; q < 2 * R::INSTR; ++q) issue_one(t, q);
  };

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};
  float m2 = kNegInf, lsum = 0.f;
  bf16x8 pf[4];
  f32x16 s[2];

  // One basic block of MFMAs: S(j) = K_j Q^T (16 MFMAs, 2 chains) interleaved
  // one-for-one with O^T += V_{j-1}^T P_{j-1}^T (16 MFMAs, MB chains); with the
  // two products alternating, a chain's next MFMA issues at least four MFMAs
  // after its previous one (a dependent MFMA waits ~150 cycles for its
  // predecessor). LDS operand fragments are loaded two pairs ahead so that
  // their latency is covered by the MFMAs in between.
  auto mma = [&](auto do_s, auto do_pv, int j, int dma_tile) {
    const char* stK = smem + (j % R::NSTAGE) * R::STAGE;
    const char* stV = smem + ((j + R::NSTAGE - 1) % R::NSTAGE) * R::STAGE + R::TILE;
    constexpr int NP = 2 * DC;                 // MFMA pairs (= 4 * MB for the PV half)
    auto kfrag = [&](int i) {                  // pair i: kb = i & 1, dc = i >> 1
      const int r = 32 * (i & 1) + l32;
      return *(const bf16x8*)(stK + r * RB + (((2 * (i >> 1) + hi) ^ chunk_swizzle<D>(r)) << 4));
    };
    auto vfrag = [&](int i) {                  // pair i: mb = i % MB, kc = i / MB
      const int d = 32 * (i % MB) + l32;
      return *(const bf16x8*)(stV + d * (2 * BC) + (((2 * (i / MB) + hi) ^ vt_swizzle(d)) << 4));
    };
    bf16x8 kq[3], vq[3];
    if constexpr (do_s.value) {
      s[0] = s[1] = f32x16{};
      kq[0] = kfrag(0);
      kq[1] = kfrag(1);
    }
    if constexpr (do_pv.value) {
      vq[0] = vfrag(0);
      vq[1] = vfrag(1);
    }
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      if (i + 2 < NP) {
        if constexpr (do_s.value) kq[(i + 2) % 3] = kfrag(i + 2);
        if constexpr (do_pv.value) vq[(i + 2) % 3] = vfrag(i + 2);
      }
      __builtin_amdgcn_sched_barrier(0);   // keep the reads two pairs ahead of their MFMAs
      if constexpr (do_s.value) s[i & 1] = mfma32(kq[i % 3], qf[i >> 1], s[i & 1]);
      if constexpr (do_pv.value) acc[i % MB] = mfma32(vq[i % 3], pf[i / MB], acc[i % MB]);
      // the prefetch of a later tile rides in the shadow of the MFMAs
      constexpr int EVERY = NP / (2 * R::INSTR);
      if (i % EVERY == EVERY - 1 && dma_tile >= 0) issue_one(dma_tile, i / EVERY);
    }
  };
  auto softmax = [&](int j) {
    const int key0 = j * BC;
    float v[32];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      v[i] = s[0][i];
      v[16 + i] = s[1][i];
    }
    if (key0 + BC > mask_from) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const int key = key0 + 32 * (i >> 4) + 8 * ((i & 15) >> 2) + 4 * hi + (i & 3);
        if (key > lim) v[i] = kNegInf;
      }
    }
    const float mx = max_halves(tree_max32(v)) * a.c;
    // move the reference max only when the row max grew by more than RESCALE_T
    const bool grow = mx > m2 + RESCALE_T;
    if (wave_any(grow)) {
      const float mnew = grow ? mx : m2;
      const float alpha = grow ? fast_exp2(m2 - mnew) : 1.f;
      lsum *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] *= alpha;
      m2 = mnew;
    }
    const float msub = (m2 == kNegInf) ? 0.f : m2;
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = fast_exp2(__builtin_fmaf(v[i], a.c, -msub));
#pragma unroll
    for (int q = 0; q < 4; ++q)
      pf[q] = to_bf16x8(v[8 * q + 0], v[8 * q + 1], v[8 * q + 2], v[8 * q + 3], v[8 * q + 4], v[8 * q + 5],
                        v[8 * q + 6], v[8 * q + 7]);
    lsum += tree_sum32(v);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;

  if (ntiles > 0) issue(0);
  if (ntiles > 1) issue(1);
  for (int j = 0; j <= ntiles; ++j) {
    // tile j has landed in LDS for every wavefront (each waits for its own DMA,
    // the barrier for all of them), and every wavefront is done with tile j-2
    if (j + 1 < ntiles) {
      asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(2 * R::INSTR) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    }
    const int dma_tile = (j + 2 < ntiles) ? j + 2 : -1;
    const bool ds = j < nt_w;                  // scores of tile j
    const bool dp = j >= 1 && j - 1 < nt_w;    // P V of tile j-1
    if (phase_b && dp) softmax(j - 1);
    if (ds && dp) {
      mma(T_{}, T_{}, j, dma_tile);
    } else if (ds) {
      mma(T_{}, F_{}, j, dma_tile);
    } else if (dp) {
      mma(F_{}, T_{}, j, dma_tile);
    } else if (dma_tile >= 0) {
      issue(dma_tile);
    }
    if (!phase_b && ds) softmax(j);
  }

  const float lt = sum_halves(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse_v = lt > 0.f ? (m2 + __log2f(lt)) * kLn2 : kNegInf;
  if (!colv) return;
  bf16* op = a.o + (((size_t)b * a.Hq + head) * a.Sq + pos) * D;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 r;
      r[0] = (bf16)(acc[mb][4 * q4 + 0] * inv);
      r[1] = (bf16)(acc[mb][4 * q4 + 1] * inv);
      r[2] = (bf16)(acc[mb][4 * q4 + 2] * inv);
      r[3] = (bf16)(acc[mb][4 * q4 + 3] * inv);
      *(bf16x4*)(op + 32 * mb + 8 * q4 + 4 * hi) = r;
    }
  if (a.lse != nullptr && hi == 0) a.lse[((size_t)b * a.Hq + head) * a.Sq + pos] = lse_v;
}

// ---------------------------------------------------------------------------
// Split-key decode: one wavefront per (key slice, KV head, batch); its 32
// MFMA columns pack (query head of the group, query row) pairs, so each K/V
// byte of the slice is read once for all of them. Writes the slice's
// normalised partial output and lse; combine_split_kernel merges the slices.
// ---------------------------------------------------------------------------
template <int D>
struct SplitTile {
  static constexpr int KS = D + 8;       // K row stride in LDS (bf16), 16 B pad
  static constexpr int VS = D + 16;      // V row stride in LDS (bf16), 32 B pad
  static constexpr int K_ELEMS = BC * KS;
  static constexpr int V_ELEMS = BC * VS;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
};

template <int D>
__global__ __launch_bounds__(64) void fwd_split_kernel(FwdArgs a) {
  using T = SplitTile<D>;
  constexpr int CH_ROW = D / 8;
  constexpr int CH_THR = BC * CH_ROW / 64;
  constexpr int MB = D / 32;
  constexpr int DC = D / 16;

  __shared__ __attribute__((aligned(16))) bf16 smem[2 * T::BUF];

  const int lane = threadIdx.x;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int off = (a.causal == 2) ? (a.Sk - a.Sq) : 0;
  const int W = blockIdx.x;
  const int split = W % a.nsplit;
  const int rest = W / a.nsplit;
  const int hkv = rest % a.Hkv;
  const int b = rest / a.Hkv;
  // column n packs (query head of the group, query row): n = hg * Sq + row
  const bool colv = l32 < a.g * a.Sq;
  const int hq = hkv * a.g + (colv ? l32 / a.Sq : 0);
  const int pos = colv ? l32 % a.Sq : 0;
  const int kbeg = split * a.split_keys;
  int kend = min(a.Sk, kbeg + a.split_keys);
  if (a.causal) kend = min(kend, a.Sq - 1 + off + 1);
  if (kend < kbeg) kend = kbeg;
  const int ntiles = (kend - kbeg + BC - 1) / BC;
  const int lim = a.causal ? min(kend - 1, pos + off) : kend - 1;
  const int mask_from = a.causal ? max(kbeg, min(kend, off + 1)) : kend;

  bf16x8 qf[DC];
  {
    const bf16* qp = a.q + (((size_t)b * a.Hq + hq) * a.Sq + pos) * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      qf[dc] = colv ? *(const bf16x8*)(qp + 16 * dc + 8 * hi) : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
  }
  const bf16* kg = a.k + ((size_t)b * a.Hkv + hkv) * (size_t)a.Sk * D;
  const bf16* vg = a.v + ((size_t)b * a.Hkv + hkv) * (size_t)a.Sk * D;

  u32x4 kreg[CH_THR], vreg[CH_THR];
  auto load_tile = [&](int t) {
    const int key0 = kbeg + t * BC;
#pragma unroll
    for (int i = 0; i < CH_THR; ++i) {
      const int c = lane + i * 64;
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
      const int c = lane + i * 64;
      const int row = c / CH_ROW;
      const int col = c % CH_ROW;
      *(u32x4*)(sk + row * T::KS + col * 8) = kreg[i];
      *(u32x4*)(sv + row * T::VS + col * 8) = vreg[i];
    }
  };

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};
  float m2 = kNegInf, lsum = 0.f;

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
    const int key0 = kbeg + t * BC;
    const bf16* sk = smem + cur * T::BUF;
    const bf16* sv = sk + T::K_ELEMS;
    f32x16 s[2];
    s[0] = s[1] = f32x16{};
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        s[kb] = mfma32(*(const bf16x8*)(sk + (32 * kb + l32) * T::KS + 16 * dc + 8 * hi), qf[dc], s[kb]);
    if (key0 + BC > mask_from) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = key0 + 32 * kb + 8 * (i >> 2) + 4 * hi + (i & 3);
          if (key > lim) s[kb][i] = kNegInf;
        }
    }
    float mx = fmaxf(s[0][0], s[1][0]);
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, fmaxf(s[0][i], s[1][i]));
    mx = max_halves(mx) * a.c;
    const bool grow = mx > m2 + RESCALE_T;
    if (wave_any(grow)) {
      const float mnew = grow ? mx : m2;
      const float alpha = grow ? fast_exp2(m2 - mnew) : 1.f;
      lsum *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] *= alpha;
      m2 = mnew;
    }
    const float msub = (m2 == kNegInf) ? 0.f : m2;
    bf16x8 pf[4];
    float ps = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float p[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = fast_exp2(__builtin_fmaf(s[kb][8 * h + e], a.c, -msub));
          ps += p[e];
        }
        pf[2 * kb + h] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
      }
    lsum += ps;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const bf16* vp = sv + (16 * kc + 4 * hi + (L >> 2)) * T::VS + 32 * mb + 16 * dhalf + 4 * (L & 3);
        acc[mb] = mfma32(cat4(lds_read_tr(vp), lds_read_tr(vp + 8 * T::VS)), pf[kc], acc[mb]);
      }
    if (t + 1 < ntiles) store_tile(cur ^ 1);
  }

  const float lt = sum_halves(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse_v = lt > 0.f ? (m2 + __log2f(lt)) * kLn2 : kNegInf;
  if (!colv) return;
  const size_t row = (((size_t)split * a.B + b) * a.Hq + hq) * a.Sq + pos;
  float* pp = a.part_o + row * D;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      f32x4 r;
      r[0] = acc[mb][4 * q4 + 0] * inv;
      r[1] = acc[mb][4 * q4 + 1] * inv;
      r[2] = acc[mb][4 * q4 + 2] * inv;
      r[3] = acc[mb][4 * q4 + 3] * inv;
      *(f32x4*)(pp + 32 * mb + 8 * q4 + 4 * hi) = r;
    }
  if (hi == 0) a.part_lse[row] = lse_v;
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
hipError_t launch_prefill_d(const FwdArgs& a, bf16* vt, hipStream_t s) {
  hipError_t e = hipSuccess;
  if (a.skp > 0) {
    timing_begin(s, "transpose_v");
    hipLaunchKernelGGL((transpose_rows_kernel<D>), dim3(a.skp / BC, a.Hkv, a.B), dim3(256), 0, s, a.v, vt,
                       a.Hkv, a.Sk, a.skp);
    e = hipGetLastError();
    timing_end(s);
    if (e != hipSuccess) return e;
  }
  timing_begin(s, "fwd_prefill_bf16");
  hipLaunchKernelGGL((fwd_prefill_kernel<D>), dim3(a.total_wgs), dim3(512), 0, s, a);
  e = hipGetLastError();
  timing_end(s);
  return e;
}

template <int D>
hipError_t launch_split_d(const FwdArgs& a, int rows, hipStream_t s) {
  timing_begin(s, "fwd_split_bf16");
  hipLaunchKernelGGL((fwd_split_kernel<D>), dim3(a.nsplit * a.B * a.Hkv), dim3(64), 0, s, a);
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
  a.skp = ((p.Sk + BC - 1) / BC) * BC;
  a.c = p.scale * kLog2e;
  return a;
}

}  // namespace

PrefillPlan plan_prefill(const Problem& p) {
  PrefillPlan pl{};
  const int g = p.Hq / p.Hkv;
  pl.hw = (g % 4 == 0) ? 4 : (g % 2 == 0) ? 2 : 1;
  pl.n_hgroups = g / pl.hw;
  pl.rows_per_wg = 8 * 32 / pl.hw;
  pl.n_ptiles = (p.Sq + pl.rows_per_wg - 1) / pl.rows_per_wg;
  pl.total_wgs = p.B * p.Hkv * pl.n_hgroups * pl.n_ptiles;
  const size_t skp = (size_t)((p.Sk + BC - 1) / BC) * BC;
  pl.ws_bytes = (size_t)p.B * p.Hkv * p.d * skp * 2;
  return pl;
}

SplitPlan plan_split(const Problem& p) {
  SplitPlan sp{};
  const int g = p.Hq / p.Hkv;
  sp.use = (long long)g * p.Sq <= 32;
  if (!sp.use) return sp;
  const int tiles = (p.Sk + BC - 1) / BC;
  const int units = p.B * p.Hkv;
  int ns = (2048 + units - 1) / units;
  ns = std::max(1, std::min(ns, tiles / 4));
  const int tiles_per = std::max(1, (tiles + ns - 1) / ns);
  ns = std::max(1, (tiles + tiles_per - 1) / tiles_per);
  sp.nsplit = ns;
  sp.split_keys = tiles_per * BC;
  const size_t rows = (size_t)p.B * p.Hq * p.Sq;
  const size_t o_bytes = (size_t)ns * rows * p.d * sizeof(float);
  const size_t l_bytes = (size_t)ns * rows * sizeof(float);
  sp.ws_bytes = ((o_bytes + 255) / 256) * 256 + l_bytes;
  return sp;
}

hipError_t launch_fwd_prefill_bf16(const Problem& p, const PrefillPlan& pl, const void* q, const void* k,
                                   const void* v, void* o, float* lse, void* ws, hipStream_t s) {
  FwdArgs a = base_args(p, q, k, v, o, lse);
  a.hw = pl.hw;
  a.n_hgroups = pl.n_hgroups;
  a.rows_per_wg = pl.rows_per_wg;
  a.n_ptiles = pl.n_ptiles;
  a.total_wgs = pl.total_wgs;
  a.vt = (const bf16*)ws;
  if (a.total_wgs == 0) return hipSuccess;
  return p.d == 64 ? launch_prefill_d<64>(a, (bf16*)ws, s) : launch_prefill_d<128>(a, (bf16*)ws, s);
}

hipError_t launch_fwd_split_bf16(const Problem& p, const SplitPlan& sp, const void* q, const void* k,
                                 const void* v, void* o, float* lse, void* ws, hipStream_t s) {
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
