// Forward attention on MXFP8 inputs (gfx950 block-scaled FP8 MFMA).
//
// "Flash Attention FA1->FA4 / pre-training practice" §2.2: FA3 runs
// attention in FP8, at twice the bf16 matrix rate, and keeps it accurate by
// quantising per block. Here the blocks are the OCP Microscaling ones: 32
// E4M3 values share one power-of-two scale (an E8M0 byte). gfx950's
// v_mfma_scale_f32_32x32x64_f8f6f4 applies such scales itself: each row of
// A and column of B takes one scale byte per 32 values of the reduction, so
// the scales of Q, K and V cost nothing inside the loop.
//
// Operand formats (produced by the quantisers below):
//  * Q, K: codes [B, H, S, d] (row-major, like the bf16 tensors), scales
//    [B, H, S, d/32]: one per 32 channels of a row;
//  * V, transposed and tiled by 64 keys: codes [B, Hkv, Skp/64, d, 64]
//    (Skp = Sk rounded up to 64, the padding zero), scales
//    [B, Hkv, Skp/64, d, 2]: one per 32 keys of a channel. A tile's codes are
//    8 KB and its scales 256 bytes, each contiguous (a plain [d, Skp]
//    transpose would read 64-byte pieces 32 KB apart in long sequences). V is blocked along the keys because the P V product
//    sums over them, and it is stored transposed because V^T is the A
//    operand of O^T = V^T P^T.
//
// The recurrence is the bf16 prefill's (online softmax over 64-key tiles,
// two wavefronts per SIMD in opposite phases, an LDS ring fed by LDS DMA),
// with these changes:
//  * the ring has 8 stages and the DMA runs three tiles ahead, so the
//    workgroup needs a barrier only every other step (the barrier held the
//    eight wavefronts in lockstep around the softmax; halving it saves 3 %);
//  * the main loop is compiled once per phase, so that each phase keeps its
//    scores in the registers its MFMAs write: with one loop for both, every
//    step copied the 32 score registers after the MFMAs (16 v_mov_b64), and
//    this kernel is bound by its vector instruction issue (11 % faster
//    without the copies, bit-identical output);
//  * operand layout of v_mfma_scale_f32_32x32x64_f8f6f4 (measured with an
//    in-bounds probe of the builtin): lane l holds row (A) or column (B)
//    l % 32; its operand bytes 0..15 lie in k-block 0 (k 0..31), bytes 16..31
//    in k-block 1 (k 32..63); the scale byte of lane half h applies to
//    k-block h of that row or column, i.e. to bytes 16h .. 16h+15 of both
//    lane halves; opsel n picks byte n of the scale register. Here lane half
//    h supplies the h-th 16 values of each k-block, so each k-block is 32
//    consecutive channels (one MX block of Q or K) or 32 consecutive keys
//    (one MX block of V);
//  * scores: S^T = K Q^T on 32x32x64 FP8 MFMAs (two per 32x32 block at
//    d = 128). The A operand of block c takes key rows in the order
//    kappa_c(r) = 32 c + 16 ((r >> 2) & 1) + 4 (r >> 3) + (r & 3), so that
//    accumulator register i of block c in lane half H is key 32 c + 16 H + i;
//  * probabilities: rounded to E4M3 (v_cvt_pk_fp8_f32, nearest even) and fed
//    from registers as the B operand of O^T = V^T P^T: byte 16 c + i of lane
//    half H is key 32 c + 16 H + i, exactly the k slot the layout above gives
//    it; the matching A operand is two 16-byte LDS reads of the V^T tile
//    (keys 16 H .. +15 and 32 + 16 H .. +15). To keep small probabilities
//    out of the E4M3 subnormals, P is formed relative to m - 6 (2^6 times the probability)
//    and the reference max moves only when a row max grows by more than 2, so
//    P stays <= 2^8 < 448; the denominator carries the same factor, so u / l
//    is unchanged and lse subtracts it.
#include "common.h"
#include "kernels.h"
#include "tiles.h"

#include <cstdio>

namespace attn {

namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint8_t u8;

constexpr int F8_BC = 64;               // keys per tile
constexpr float F8_RESCALE_T = 2.0f;    // log2 units
constexpr float F8_PSHIFT = 6.0f;       // P = 2^6 exp2(s - m) <= 2^(6 + F8_RESCALE_T)
constexpr int E8M0_ONE = 127;           // scale byte of 1.0

struct Fp8Args {
  const u8* q;
  const u8* qs;
  const u8* k;
  const u8* ks;
  const u8* vt;
  const u8* vs;
  bf16* o;
  float* lse;
  int B, Hq, Hkv, Sq, Sk, Skp, g, causal;
  float c;                              // scale * log2(e)
  int hw, n_hgroups, rows_per_wg, n_ptiles, total_wgs;
};

// D = 128 stage: [K tile | V^T tile | K scales | V scales]
template <int D>
struct Fp8Ring {
  static constexpr int KT = F8_BC * D;          // K tile bytes (64 rows of D)
  static constexpr int VT = D * F8_BC;          // V^T tile bytes (D rows of 64 keys)
  static constexpr int KS = F8_BC * (D / 32);   // K scale bytes
  static constexpr int VS = D * 2;              // V scale bytes
  static constexpr int K_OFF = 0;
  static constexpr int V_OFF = KT;
  static constexpr int KS_OFF = KT + VT;
  static constexpr int VS_OFF = KS_OFF + KS;
  static constexpr int STAGE = VS_OFF + VS;
  static constexpr int VST = VT + VS;           // a V^T tile and its scales (decode ring slot)
  static constexpr int NSTAGE = 8;
};

// S^T / O^T product with per-lane E8M0 scales (byte OPA of sa for the A
// operand's 32 values, byte OPB of sb for the B operand's); both formats E4M3.
template <int OPA, int OPB>
__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, int sa, i32x8 b, int sb, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, OPA, sa, OPB, sb);
}

// Key row that lane row r of the score A operand loads for key block c.
__device__ __forceinline__ int kappa(int c, int r) { return 32 * c + 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

// LDS chunk swizzles (16-byte chunks XOR-permuted per row): K rows are 128
// bytes, V^T rows 64. With them each 16-lane group of a 16-byte fragment read
// touches 16 distinct 16-byte bank groups (the 16 key rows kappa_c(r),
// r = 0..15 or 16..31, resp. 16 consecutive channels).
__device__ __forceinline__ int swz_k(int row) { return ((row >> 1) & 3) | (((row >> 4) & 1) << 2); }
__device__ __forceinline__ int swz_v(int row) { return (row >> 2) & 3; }

__device__ __forceinline__ i32x8 cat_u32x4(u32x4 a, u32x4 b) {
  return __builtin_bit_cast(i32x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

template <int D>
__global__ __launch_bounds__(512) void fwd_fp8_kernel(Fp8Args a) {
  static_assert(D == 128, "the FP8 path is built for d = 128");
  using R = Fp8Ring<D>;
  constexpr int DC = D / 64;                    // MFMAs per 32x32 score block
  constexpr int MB = D / 32;                    // 32-channel blocks of the output
  constexpr int NSB = D / 32;                   // scale bytes per Q or K row
  static_assert(R::NSTAGE == 8, "the main loop is unrolled by the ring size");
  static_assert(R::KT == 8 * 1024 && R::VT == 8 * 1024, "one 1 KB DMA instruction per wavefront per tensor");

  __shared__ __attribute__((aligned(1024))) char smem[R::NSTAGE * R::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bool phase_b = wid >= 4;

  int t, rest;
  xcd_tile_order(a.total_wgs, a.n_ptiles, t, rest);
  const int ptile = a.n_ptiles - 1 - t;                    // longest causal tiles first
  const int hgrp = rest % a.n_hgroups;
  rest /= a.n_hgroups;
  const int hkv = rest % a.Hkv;
  const int b = rest / a.Hkv;

  const int off = (a.causal == 2) ? (a.Sk - a.Sq) : 0;
  const int slot = (wid & 3) * 2 + (wid >> 2);
  const int head = hkv * a.g + hgrp * a.hw + slot % a.hw;
  const int p0 = ptile * a.rows_per_wg + 32 * (slot / a.hw);
  const int pos = p0 + l32;
  const bool colv = pos < a.Sq;
  const int wg_last = min((ptile + 1) * a.rows_per_wg, a.Sq) - 1;
  int kend = a.causal ? min(a.Sk, wg_last + off + 1) : a.Sk;
  if (kend < 0) kend = 0;
  const int ntiles = (kend + F8_BC - 1) / F8_BC;
  const int mask_from = a.causal ? max(0, min(kend, p0 + off + 1)) : kend;
  const int lim = a.causal ? min(kend - 1, pos + off) : kend - 1;

  // Q fragments (B operand of S^T): lane (hi, l32) holds row pos, channels
  // 64 dc + 16 hi .. +15 (k-block 0) and 64 dc + 32 + 16 hi .. +15 (k-block
  // 1). Lane half hi supplies the scale of k-block hi, i.e. of channel block
  // 2 dc + hi, in byte 2 dc of qsc (the row's four scale bytes shifted right
  // by 8 hi). Rows past Sq hold zeros (scale byte 0, not NaN).
  i32x8 qf[DC];
  int qsc;
  {
    const size_t row = ((size_t)b * a.Hq + head) * a.Sq + (colv ? pos : 0);
    const u8* qp = a.q + row * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      qf[dc] = colv ? cat_u32x4(*(const u32x4*)(qp + 64 * dc + 16 * hi), *(const u32x4*)(qp + 64 * dc + 32 + 16 * hi))
                    : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    qsc = colv ? (int)((*(const uint32_t*)(a.qs + row * NSB)) >> (8 * hi)) : 0;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qf[dc] = settle(qf[dc]);
    qsc = settle(qsc);
  }
  const size_t kvh = (size_t)b * a.Hkv + hkv;
  const u8* kg = wave_uniform(a.k + kvh * (size_t)a.Sk * D);
  const u8* ksg = wave_uniform(a.ks + kvh * (size_t)a.Sk * NSB);
  const u8* vtg = wave_uniform(a.vt + kvh * (size_t)D * a.Skp);
  const u8* vsg = wave_uniform(a.vs + kvh * (size_t)(a.Skp / F8_BC) * (2 * D));

  // LDS read offsets. K: block c, d-chunk dc, k-block hh (bytes 16 hh .. of
  // the lane's 32): row kappa_c(l32), logical chunk 4 dc + 2 hh + hi. V^T:
  // channel row 32 mb + l32 (mb is an immediate offset: it does not change
  // the row's swizzle bits), logical chunk 2 hh + hi.
  uint32_t kb[2][DC][2], vb[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int kr = kappa(c, l32);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh)
        kb[c][dc][hh] = R::K_OFF + kr * D + (((4 * dc + 2 * hh + hi) ^ swz_k(kr)) << 4);
  }
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) vb[hh] = R::V_OFF + l32 * F8_BC + (((2 * hh + hi) ^ swz_v(l32)) << 4);
  const uint32_t ksb0 = R::KS_OFF + 4 * kappa(0, l32), ksb1 = R::KS_OFF + 4 * kappa(1, l32);
  const uint32_t vsb = R::VS_OFF + 2 * l32 + hi;

  // DMA geometry: wavefront wid writes the 1 KB of LDS at wid * 1024 of the K
  // tile and of the V^T tile; lane i the 16-byte chunk P = 64 wid + i.
  // K: row P / 8, physical chunk P % 8; V^T: channel P / 4, chunk P % 4.
  uint32_t koff, voff;
  {
    const int P = wid * 64 + lane;
    const int kr = P / 8, vr = P / 4;
    koff = kr * D + (((P % 8) ^ swz_k(kr)) << 4);
    voff = vr * F8_BC + (((P % 4) ^ swz_v(vr)) << 4);
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);
  const uint32_t ldsw = lds0 + wid * 1024;
  // wavefronts 0 and 1 also load the tile's K scales and V scales (4 bytes a lane)
  const bool scale_dma = wid < 2;

  struct Dma {
    u32x4 rk, rv, rs;
  };
  auto dma_for = [&](int t) __attribute__((always_inline)) {
    Dma d;
    const int tt = min(t, ntiles - 1);
    const int key0 = tt * F8_BC;
    d.rk = buffer_rsrc(kg + (size_t)key0 * D, (uint32_t)(kend - key0) * D);
    d.rv = buffer_rsrc(vtg + (size_t)tt * (D * F8_BC), D * F8_BC);
    if (wid == 0) d.rs = buffer_rsrc(ksg + (size_t)key0 * NSB, (uint32_t)(kend - key0) * NSB);
    else d.rs = buffer_rsrc(vsg + (size_t)tt * (2 * D), 2 * D);
    return d;
  };
  // DMA instruction QI into ring slot SLOT: 0 = K, 1 = V^T, 2 = scales
  auto issue_one = [&](auto slot_, auto qi_, const Dma& d) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_)::value;
    constexpr int QI = decltype(qi_)::value;
    if constexpr (QI == 0) dma16b_at<SLOT * R::STAGE + R::K_OFF>(d.rk, koff, 0u, ldsw);
    else if constexpr (QI == 1) dma16b_at<SLOT * R::STAGE + R::V_OFF>(d.rv, voff, 0u, ldsw);
    else if (scale_dma) {
      if (wid == 0) dma4b_at<SLOT * R::STAGE + R::KS_OFF>(d.rs, 4 * lane, 0u, lds0);
      else dma4b_at<SLOT * R::STAGE + R::VS_OFF>(d.rs, 4 * lane, 0u, lds0);
    }
  };

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};
  float m2 = kNegInf, lsum = 0.f;
  i32x8 pf = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
  f32x16 s[2];

  // Step j (slot position POS = j mod 4): S(j) = K_j Q^T (4 MFMAs, two
  // chains: pair i is key block i & 1, d-chunk i >> 1) interleaved with
  // O^T += V_{j-1}^T P_{j-1}^T (one MFMA per 32-channel block), operand
  // fragments one pair ahead; the DMA of tile j+2 is spread over the pairs.
  auto mma = [&](auto pos_, auto do_s, auto do_pv, int j) __attribute__((always_inline)) {
    constexpr int POS = decltype(pos_)::value;
    constexpr bool DS = decltype(do_s)::value;
    constexpr bool DP = decltype(do_pv)::value;
    constexpr int SK = POS;                     // K of tile j
    constexpr int SV = (POS + 7) % 8;           // V of tile j-1
    constexpr int SD = (POS + 3) % 8;           // DMA target: tile j+3
    const char* stk = smem + SK * R::STAGE;
    const char* stv = smem + SV * R::STAGE;
    auto kfrag = [&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      return cat_u32x4(*(const u32x4*)(stk + kb[i & 1][i >> 1][0]), *(const u32x4*)(stk + kb[i & 1][i >> 1][1]));
    };
    auto vfrag = [&](auto mc) __attribute__((always_inline)) {
      constexpr int mb = decltype(mc)::value;
      return cat_u32x4(*(const u32x4*)(stv + vb[0] + mb * 32 * F8_BC), *(const u32x4*)(stv + vb[1] + mb * 32 * F8_BC));
    };
    Dma d;
    if constexpr (DS) d = dma_for(j + 3);
    int ksc[2] = {0, 0}, vsc[MB];
    i32x8 kq[2], vq[2];
    if constexpr (DS) {
      ksc[0] = (int)(*(const uint32_t*)(stk + ksb0) >> (8 * hi));
      ksc[1] = (int)(*(const uint32_t*)(stk + ksb1) >> (8 * hi));
      kq[0] = kfrag(std::integral_constant<int, 0>{});
    }
    if constexpr (DP) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) vsc[mb] = (int)*(const u8*)(stv + vsb + mb * 64);
      vq[0] = vfrag(std::integral_constant<int, 0>{});
    }
    __builtin_amdgcn_s_setprio(1);
    static_for<4>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i + 1 < 4) {
        if constexpr (DS) kq[(i + 1) & 1] = kfrag(std::integral_constant<int, i + 1>{});
        if constexpr (DP) vq[(i + 1) & 1] = vfrag(std::integral_constant<int, i + 1>{});
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (DS)
        s[i & 1] = mfma_f8<2 * (i >> 1), 2 * (i >> 1)>(kq[i & 1], ksc[i & 1], qf[i >> 1], qsc,
                                                         i < 2 ? f32x16{} : s[i & 1]);
      if constexpr (DP) acc[i] = mfma_f8<0, 0>(vq[i & 1], vsc[i], pf, E8M0_ONE, acc[i]);
      if constexpr (DS && i < 3) issue_one(std::integral_constant<int, SD>{}, std::integral_constant<int, i>{}, d);
    });
    __builtin_amdgcn_s_setprio(0);
  };
  auto softmax = [&](int j) __attribute__((always_inline)) {
    const int key0 = j * F8_BC;
    float v[32];                                // v[u]: key key0 + 32 (u >> 4) + 16 hi + (u & 15)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      v[i] = s[0][i];
      v[16 + i] = s[1][i];
    }
    if (key0 + F8_BC > mask_from) {
#pragma unroll
      for (int u = 0; u < 32; ++u)
        if (key0 + 32 * (u >> 4) + 16 * hi + (u & 15) > lim) v[u] = kNegInf;
    }
    const float mx = max_halves(tree_max32(v)) * a.c;
    const bool grow = mx > m2 + F8_RESCALE_T;
    if (wave_any(grow)) {
      const float mnew = grow ? mx : m2;
      const float alpha = grow ? fast_exp2(m2 - mnew) : 1.f;
      lsum *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] *= alpha;
      m2 = mnew;
    }
    const float msub = (m2 == kNegInf) ? 0.f : m2 - F8_PSHIFT;
#pragma unroll
    for (int u = 0; u < 32; ++u) v[u] = fast_exp2(__builtin_fmaf(v[u], a.c, -msub));
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      int x = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * w], v[4 * w + 1], 0, false);
      pf[w] = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * w + 2], v[4 * w + 3], x, true);
    }
    lsum += tree_sum32(v);
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // Even step j: every wavefront's DMA of tiles j and j+1 has landed (each
  // waits for its own: 2 or 3 instructions may still be in flight, those of
  // tile j+2), and every wavefront is done with step j-1. Odd steps need no
  // barrier: their tiles were covered by the previous one, and the slot a
  // step's DMA overwrites (tile j-5, ring of 8, DMA three tiles ahead) was
  // last read in step j-4, which every wavefront had finished at the last
  // barrier.
  auto sync = [&]() __attribute__((always_inline)) {
    if (scale_dma) asm volatile("s_waitcnt vmcnt(3)\n\ts_barrier" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(2)\n\ts_barrier" ::: "memory");
  };
  // one copy of the loop per phase (see the header)
  auto run = [&](auto pb_) __attribute__((always_inline)) {
    constexpr bool PB = decltype(pb_)::value;
    auto full = [&](auto pos_, int j) __attribute__((always_inline)) {
      if constexpr (decltype(pos_)::value % 2 == 0) sync();
      if constexpr (PB) softmax(j - 1);
      mma(pos_, T_{}, T_{}, j);
      if constexpr (!PB) softmax(j);
    };

    if (ntiles > 0) {
      const Dma d0 = dma_for(0), d1 = dma_for(1), d2 = dma_for(2);
      static_for<3>([&](auto qi) __attribute__((always_inline)) { issue_one(I0{}, qi, d0); });
      static_for<3>([&](auto qi) __attribute__((always_inline)) { issue_one(I1{}, qi, d1); });
      static_for<3>([&](auto qi) __attribute__((always_inline)) { issue_one(I2{}, qi, d2); });
      sync();
      mma(I0{}, T_{}, F_{}, 0);
      if constexpr (!PB) softmax(0);
    }
    int j = 1;
    for (; j + 7 < ntiles; j += 8) {
      static_for<8>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        full(std::integral_constant<int, (k + 1) % 8>{}, j + k);
      });
    }
    static_for<7>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      if (j + k < ntiles) full(std::integral_constant<int, k + 1>{}, j + k);
    });
    if (ntiles > 0) {
      if constexpr (PB) softmax(ntiles - 1);
      switch (ntiles & 7) {
        case 0: mma(I0{}, F_{}, T_{}, ntiles); break;
        case 1: mma(I1{}, F_{}, T_{}, ntiles); break;
        case 2: mma(I2{}, F_{}, T_{}, ntiles); break;
        case 3: mma(I3{}, F_{}, T_{}, ntiles); break;
        case 4: mma(std::integral_constant<int, 4>{}, F_{}, T_{}, ntiles); break;
        case 5: mma(std::integral_constant<int, 5>{}, F_{}, T_{}, ntiles); break;
        case 6: mma(std::integral_constant<int, 6>{}, F_{}, T_{}, ntiles); break;
        default: mma(std::integral_constant<int, 7>{}, F_{}, T_{}, ntiles); break;
      }
    }
  };
  if (phase_b) run(T_{});
  else run(F_{});
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  const float lt = sum_halves(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse_v = lt > 0.f ? (m2 - F8_PSHIFT + __log2f(lt)) * kLn2 : kNegInf;
  if (!colv) return;
  const size_t orow = ((size_t)b * a.Hq + head) * a.Sq + pos;
  bf16* op = a.o + orow * D;
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
  if (a.lse != nullptr && hi == 0) a.lse[orow] = lse_v;
}

// ---------------------------------------------------------------------------
// Split-key decode on MXFP8 operands: one 64-lane wavefront per (key slice,
// KV head, batch); its 32 MFMA columns pack (query head of the group, query
// row) pairs, so every K/V byte of the slice is read once for all of them.
// Decode streams K and V once and is bound by the loads in flight (about
// eight wavefronts per CU): K fragments go straight from HBM into registers
// (range-checked buffer loads), those of the next 64-key tile as soon as
// the score MFMAs have read the current ones; V^T tiles (contiguous 8 KB in
// the tiled layout) go through a 2-slot LDS ring of the wavefront, the next
// one issued by LDS DMA at the start of each tile. Writes the slice's
// normalised partial output and lse for the merge kernel.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void fwd_fp8_split_kernel(Fp8Args a, float* __restrict__ part_o,
                                                           float* __restrict__ part_lse, int nsplit,
                                                           int split_keys) {
  static_assert(D == 128, "the FP8 path is built for d = 128");
  using R = Fp8Ring<D>;
  constexpr int DC = D / 64;
  constexpr int MB = D / 32;
  constexpr int NSB = D / 32;
  __shared__ __attribute__((aligned(1024))) char smem[2 * R::VST];
  const int lane = threadIdx.x;
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int off = (a.causal == 2) ? (a.Sk - a.Sq) : 0;
  const int W = blockIdx.x;
  const int split = W % nsplit;
  const int rest = W / nsplit;
  const int hkv = rest % a.Hkv;
  const int b = rest / a.Hkv;
  // column n packs (query head of the group, query row): n = hg * Sq + row
  const bool colv = l32 < a.g * a.Sq;
  const int hq = hkv * a.g + (colv ? l32 / a.Sq : 0);
  const int pos = colv ? l32 % a.Sq : 0;
  const int kbeg = split * split_keys;
  int kend = min(a.Sk, kbeg + split_keys);
  if (a.causal) kend = min(kend, a.Sq - 1 + off + 1);
  if (kend < kbeg) kend = kbeg;
  const int ntiles = (kend - kbeg + F8_BC - 1) / F8_BC;
  const int lim = a.causal ? min(kend - 1, pos + off) : kend - 1;
  const int mask_from = a.causal ? max(kbeg, min(kend, off + 1)) : kend;

  // Q fragments and scales as in the prefill kernel (unused columns hold zeros)
  i32x8 qf[DC];
  int qsc;
  {
    const size_t row = ((size_t)b * a.Hq + hq) * a.Sq + pos;
    const u8* qp = a.q + row * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      qf[dc] = colv ? cat_u32x4(*(const u32x4*)(qp + 64 * dc + 16 * hi), *(const u32x4*)(qp + 64 * dc + 32 + 16 * hi))
                    : i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    qsc = colv ? (int)((*(const uint32_t*)(a.qs + row * NSB)) >> (8 * hi)) : 0;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qf[dc] = settle(qf[dc]);
    qsc = settle(qsc);
  }
  const size_t kvh = (size_t)b * a.Hkv + hkv;
  // whole-head buffers: K rows past Sk read zeros (their scores are masked).
  // The int byte ranges cannot overflow: Sk < 2^24 and a code row is
  // D = 128 bytes, so Sk * D < 2^31 (scale rows are 4 bytes).
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.k + kvh * (size_t)a.Sk * D), (short)0, a.Sk * D, 0x00020000);
  const __amdgpu_buffer_rsrc_t rks =
      __builtin_amdgcn_make_buffer_rsrc((void*)(a.ks + kvh * (size_t)a.Sk * NSB), (short)0, a.Sk * NSB, 0x00020000);
  // per-lane offsets: K row kappa_c(l32) of the tile, channels 64 dc + 16 hi (+32)
  const uint32_t kro0 = (uint32_t)kappa(0, l32) * D + 16 * hi;
  const uint32_t kso0 = (uint32_t)kappa(0, l32) * NSB;
  // V^T tiles go through a 2-slot LDS ring of this wavefront by LDS DMA, one
  // tile ahead: instruction n (0..7) writes chunks 64 n + lane, i.e. channel
  // row 16 n + lane / 4, physical chunk lane % 4 holding logical chunk
  // (lane % 4) ^ swz_v(row) (the swizzle does not depend on n); the tile's
  // 256 scale bytes follow the codes.
  const uint32_t vdma = (uint32_t)(lane >> 2) * F8_BC + ((((lane & 3) ^ swz_v(lane >> 2))) << 4);
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);
  const u32x4 rvd = buffer_rsrc(a.vt + kvh * (size_t)D * a.Skp, (uint32_t)(D * a.Skp));
  const u32x4 rvsd = buffer_rsrc(a.vs + kvh * (size_t)(a.Skp / F8_BC) * (2 * D), (uint32_t)((a.Skp / F8_BC) * 2 * D));
  uint32_t vb[2];
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) vb[hh] = l32 * F8_BC + (((2 * hh + hi) ^ swz_v(l32)) << 4);
  const uint32_t vsb = R::VT + 2 * l32 + hi;

  i32x8 kf[2][DC];
  int ksc[2];
  auto load_k = [&](int t) __attribute__((always_inline)) {
    const uint32_t key0 = (uint32_t)(kbeg + t * F8_BC);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t base = (key0 + 32 * c) * D + kro0;
#pragma unroll
      for (int dc = 0; dc < DC; ++dc)
        kf[c][dc] = cat_u32x4(__builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, base + 64 * dc, 0, 0)),
                              __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, base + 64 * dc + 32, 0, 0)));
      ksc[c] = (int)(__builtin_amdgcn_raw_buffer_load_b32(rks, (key0 + 32 * c) * NSB + kso0, 0, 0) >> (8 * hi));
    }
  };
  auto dma_v = [&](int t, auto slot_) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_)::value;
    const uint32_t key0 = (uint32_t)(kbeg + t * F8_BC);
    static_for<8>([&](auto nc) __attribute__((always_inline)) {
      constexpr int n = decltype(nc)::value;
      dma16b_at<SLOT * R::VST + n * 1024>(rvd, vdma + (key0 / F8_BC) * (D * F8_BC), (uint32_t)(n * 1024), lds0);
    });
    dma4b_at<SLOT * R::VST + R::VT>(rvsd, (key0 / F8_BC) * (2 * D) + 4 * lane, 0u, lds0);
  };

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};
  float m2 = kNegInf, lsum = 0.f;
  if (ntiles > 0) {
    load_k(0);
    dma_v(0, std::integral_constant<int, 0>{});
  }
  auto tile = [&](int t, auto slot_) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_)::value;
    // K(t) (registers) and V(t) (slot SLOT) have landed; V(t+1) goes out now,
    // K(t+1) once the score MFMAs have read K(t)
#pragma unroll
    for (int c = 0; c < 2; ++c) {
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) kf[c][dc] = settle(kf[c][dc]);
      ksc[c] = settle(ksc[c]);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (t + 1 < ntiles) dma_v(t + 1, std::integral_constant<int, SLOT ^ 1>{});
    f32x16 s[2];
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
#pragma unroll
      for (int c = 0; c < 2; ++c)
        s[c] = dc == 0 ? mfma_f8<0, 0>(kf[c][0], ksc[c], qf[0], qsc, f32x16{})
                       : mfma_f8<2, 2>(kf[c][1], ksc[c], qf[1], qsc, s[c]);
    if (t + 1 < ntiles) load_k(t + 1);
    const int key0 = kbeg + t * F8_BC;
    float v[32];                                // v[u]: key key0 + 32 (u >> 4) + 16 hi + (u & 15)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      v[i] = s[0][i];
      v[16 + i] = s[1][i];
    }
    if (key0 + F8_BC > mask_from) {
      const int rel = lim - key0 - 16 * hi;
#pragma unroll
      for (int u = 0; u < 32; ++u)
        if (32 * (u >> 4) + (u & 15) > rel) v[u] = kNegInf;
    }
    const float mx = max_halves(tree_max32(v)) * a.c;
    const bool grow = mx > m2 + F8_RESCALE_T;
    if (wave_any(grow)) {
      const float mnew = grow ? mx : m2;
      const float alpha = grow ? fast_exp2(m2 - mnew) : 1.f;
      lsum *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] *= alpha;
      m2 = mnew;
    }
    const float msub = (m2 == kNegInf) ? 0.f : m2 - F8_PSHIFT;
#pragma unroll
    for (int u = 0; u < 32; ++u) v[u] = fast_exp2(__builtin_fmaf(v[u], a.c, -msub));
    i32x8 pf;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      int x = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * w], v[4 * w + 1], 0, false);
      pf[w] = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * w + 2], v[4 * w + 3], x, true);
    }
    lsum += tree_sum32(v);
    const char* sv = smem + SLOT * R::VST;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const i32x8 vq = cat_u32x4(*(const u32x4*)(sv + vb[0] + mb * 32 * F8_BC),
                                 *(const u32x4*)(sv + vb[1] + mb * 32 * F8_BC));
      const int vs = (int)*(const u8*)(sv + vsb + mb * 64);
      acc[mb] = mfma_f8<0, 0>(vq, vs, pf, E8M0_ONE, acc[mb]);
    }
  };
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    tile(t, std::integral_constant<int, 0>{});
    tile(t + 1, std::integral_constant<int, 1>{});
  }
  if (t < ntiles) tile(t, std::integral_constant<int, 0>{});
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  const float lt = sum_halves(lsum);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse_v = lt > 0.f ? (m2 - F8_PSHIFT + __log2f(lt)) * kLn2 : kNegInf;
  if (!colv) return;
  const size_t row = (((size_t)split * a.B + b) * a.Hq + hq) * a.Sq + pos;
  float* pp = part_o + row * D;
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
  if (hi == 0) part_lse[row] = lse_v;
}

// ---------------------------------------------------------------------------
// MXFP8 quantisers. Block exponent: the smallest e with amax <= 448 * 2^e
// (amax = f 2^E with f in [0.5, 1) and 448 = 0.875 * 2^9 give
// e = E - 9 + (f > 0.875)), 0 for an all-zero block, clamped to [-127, 127];
// elements are x * 2^-e (exact) rounded to E4M3, nearest even.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.f)) return 0;
  int E;
  const float f = frexpf(amax, &E);
  const int e = E - 9 + (f > 0.875f ? 1 : 0);
  return max(-127, min(127, e));
}

// Four bf16 pairs scaled by 2^-e into 8 E4M3 bytes (two words).
__device__ __forceinline__ u32x2 e4m3x8(const float* x, int e) {
  u32x2 r;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    int t = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[4 * w], -e), ldexpf(x[4 * w + 1], -e), 0, false);
    t = __builtin_amdgcn_cvt_pk_fp8_f32(ldexpf(x[4 * w + 2], -e), ldexpf(x[4 * w + 3], -e), t, true);
    r[w] = (uint32_t)t;
  }
  return r;
}

// Rows of 32-element blocks: 4 lanes per block, 8 bf16 each.
__global__ __launch_bounds__(256) void mx_quant_rows_kernel(const bf16* __restrict__ x, u8* __restrict__ codes,
                                                            u8* __restrict__ scales, long long nblocks) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long blk = t >> 2;
  const int part = (int)(t & 3);
  const bool valid = blk < nblocks;
  float xv[8];
  u32x4 raw = u32x4{0u, 0u, 0u, 0u};
  if (valid) raw = *(const u32x4*)(x + blk * 32 + part * 8);
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    xv[2 * i] = __uint_as_float(raw[i] << 16);
    xv[2 * i + 1] = __uint_as_float(raw[i] & 0xffff0000u);
    amax = fmaxf(amax, fmaxf(fabsf(xv[2 * i]), fabsf(xv[2 * i + 1])));
  }
  amax = fmaxf(amax, __shfl_xor(amax, 1));
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  const int e = mx_exponent(amax);
  if (!valid) return;
  *(u32x2*)(codes + blk * 32 + part * 8) = e4m3x8(xv, e);
  if (part == 0) scales[blk] = (u8)(e + 127);
}

// V [BH, Sk, D] bf16 -> V^T codes [BH, Skp/64, D, 64] and scales [BH, Skp/64, D, 2].
// A grid of at most one resident round of 256-thread workgroups strides over
// the (head, 64-key tile) units and loads the next unit's 16 KB into registers
// while it quantises the current one from LDS. In LDS the tile is 64 key rows
// of 256 bytes; the 16-byte chunk k of row r sits at chunk k ^ 4 ((r / 16) % 4),
// so the four 16-key groups of a wave read different banks. Lane (kq, cl) of
// wave w quantises keys 16 kq .. 16 kq + 15 of channels 32 w + cl and
// 32 w + 16 + cl; the two lanes of one 32-key block take the larger of their
// amax values, and each of the wave's two code stores fills 1 KB of the V^T
// tile (16 channel rows of 64 bytes). Writing whole rows this way took the
// kernel from 4.1 to 5.8 TB/s of algorithmic bytes; the earlier layout wrote
// 8-byte pieces into 64 different rows per store. Keys past Sk count as zeros.
template <int D>
__global__ __launch_bounds__(256) void mx_quant_vt_kernel(const bf16* __restrict__ v, u8* __restrict__ codes,
                                                          u8* __restrict__ scales, int Sk, int Skp, int units) {
  static_assert(D == 128, "the LDS swizzle and the lane map assume 16 chunks of 8 channels");
  __shared__ __attribute__((aligned(16))) unsigned char tile[F8_BC * 2 * D];
  constexpr int NCH = F8_BC * D / 8 / 256;       // 16-byte chunks each thread stages
  const int ntile = Skp / F8_BC;
  const int w = threadIdx.x / 64, L = threadIdx.x % 64, kq = L & 3, cl = L >> 2;
  u32x4 raw[NCH];
  auto load = [&](int u) {
    const int key0 = (u % ntile) * F8_BC;
    const bf16* src = v + ((size_t)(u / ntile) * Sk + key0) * D;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ch = threadIdx.x + j * 256, r = ch / (D / 8), c16 = ch % (D / 8);
      raw[j] = u32x4{0u, 0u, 0u, 0u};
      if (key0 + r < Sk) raw[j] = *(const u32x4*)(src + (size_t)r * D + 8 * c16);
    }
  };
  load(blockIdx.x);
  for (int u = blockIdx.x; u < units; u += gridDim.x) {
    __syncthreads();                             // the previous unit's reads are done
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
      const int ch = threadIdx.x + j * 256, r = ch / (D / 8), c16 = ch % (D / 8);
      *(u32x4*)(tile + r * 2 * D + 16 * (c16 ^ (4 * ((r >> 4) & 3)))) = raw[j];
    }
    __syncthreads();
    if (u + (int)gridDim.x < units) load(u + gridDim.x);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = 32 * w + 16 * j + cl;
      float x[16];
      float amax = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 16 * kq + i;
        const uint16_t h = *(const uint16_t*)(tile + r * 2 * D + 16 * ((c >> 3) ^ (4 * kq)) + 2 * (c & 7));
        x[i] = __uint_as_float((uint32_t)h << 16);
        amax = fmaxf(amax, fabsf(x[i]));
      }
      amax = fmaxf(amax, __shfl_xor(amax, 1));   // the other half of the 32-key block
      const int e = mx_exponent(amax);
      const size_t row = (size_t)u * D + c;      // channel row of the V^T tile
      const u32x2 lo = e4m3x8(x, e), hi = e4m3x8(x + 8, e);
      *(u32x4*)(codes + row * F8_BC + 16 * kq) = u32x4{lo[0], lo[1], hi[0], hi[1]};
      if ((kq & 1) == 0) scales[row * 2 + kq / 2] = (u8)(e + 127);
    }
  }
}

}  // namespace

int fp8_padded_keys(int Sk) { return (Sk + F8_BC - 1) / F8_BC * F8_BC; }

hipError_t launch_mx_quant_rows(const void* x, void* codes, void* scales, long long rows, int d, hipStream_t s) {
  const long long nblocks = rows * (d / 32);
  if (nblocks == 0) return hipSuccess;
  const long long threads = nblocks * 4;
  timing_begin(s, "mx_quant_rows");
  hipLaunchKernelGGL(mx_quant_rows_kernel, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s,
                     (const bf16*)x, (u8*)codes, (u8*)scales, nblocks);
  const hipError_t e = hipGetLastError();
  timing_end(s);
  return e;
}

hipError_t launch_mx_quant_vt(const void* v, void* codes, void* scales, int BH, int Sk, int d, hipStream_t s) {
  const int Skp = fp8_padded_keys(Sk);
  const long long units = (long long)BH * (Skp / F8_BC);   // < 2^31: BH * Sk is checked
  if (units == 0) return hipSuccess;
  (void)d;                                       // validated: 128
  timing_begin(s, "mx_quant_vt");
  // one resident round: 256 CUs x 8 workgroups of 4 waves (54 VGPRs, 16 KB LDS each)
  const long long grid = units < 2048 ? units : 2048;
  hipLaunchKernelGGL((mx_quant_vt_kernel<128>), dim3((unsigned)grid), dim3(256), 0, s, (const bf16*)v, (u8*)codes,
                     (u8*)scales, Sk, Skp, (int)units);
  const hipError_t e = hipGetLastError();
  timing_end(s);
  return e;
}

size_t fp8_workspace_bytes(const Problem& p) {
  const SplitPlan sp = plan_split(p);
  return sp.use ? sp.ws_bytes : 0;
}

hipError_t launch_fwd_fp8(const Problem& p, const void* q8, const void* qs, const void* k8, const void* ks,
                          const void* vt8, const void* vs, void* o, float* lse, void* ws, hipStream_t s, char* log,
                          size_t log_n) {
  const PrefillPlan pl = plan_prefill(p);
  Fp8Args a{};
  a.q = (const u8*)q8;
  a.qs = (const u8*)qs;
  a.k = (const u8*)k8;
  a.ks = (const u8*)ks;
  a.vt = (const u8*)vt8;
  a.vs = (const u8*)vs;
  a.o = (bf16*)o;
  a.lse = lse;
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Sq = p.Sq;
  a.Sk = p.Sk;
  a.Skp = fp8_padded_keys(p.Sk);
  a.g = p.Hq / p.Hkv;
  a.causal = p.causal;
  a.c = p.scale * kLog2e;
  const SplitPlan sp = plan_split(p);
  if (sp.use) {
    // decode-shaped: every grouped query row of a KV head in one wavefront, keys split
    const size_t rows = (size_t)p.B * p.Hq * p.Sq;
    const size_t o_bytes = (size_t)sp.nsplit * rows * p.d * sizeof(float);
    float* part_o = (float*)ws;
    float* part_lse = (float*)((char*)ws + ((o_bytes + 255) / 256) * 256);
    if (log != nullptr && log_n > 0)
      snprintf(log, log_n, "fwd_fp8_split<d=%d> grid=%d (%d key slices of %d keys, MXFP8 MFMA) + combine_split rows=%zu",
               p.d, sp.nsplit * p.B * p.Hkv, sp.nsplit, sp.split_keys, rows);
    timing_begin(s, "fwd_fp8_split");
    hipLaunchKernelGGL((fwd_fp8_split_kernel<128>), dim3(sp.nsplit * p.B * p.Hkv), dim3(64), 0, s, a, part_o,
                       part_lse, sp.nsplit, sp.split_keys);
    hipError_t e = hipGetLastError();
    timing_end(s);
    if (e != hipSuccess) return e;
    return launch_combine_split(p, sp, ws, o, lse, s);
  }
  a.hw = pl.hw;
  a.n_hgroups = pl.n_hgroups;
  a.rows_per_wg = pl.rows_per_wg;
  a.n_ptiles = pl.n_ptiles;
  a.total_wgs = pl.total_wgs;
  if (log != nullptr && log_n > 0)
    snprintf(log, log_n, "fwd_fp8<d=%d> grid=%d (%d query rows x %d heads per workgroup, 64-key tiles, MXFP8 MFMA)",
             p.d, pl.total_wgs, pl.rows_per_wg, pl.hw);
  if (a.total_wgs == 0) return hipSuccess;
  timing_begin(s, "fwd_fp8");
  hipLaunchKernelGGL((fwd_fp8_kernel<128>), dim3(a.total_wgs), dim3(512), 0, s, a);
  const hipError_t e = hipGetLastError();
  timing_end(s);
  return e;
}

}  // namespace attn
