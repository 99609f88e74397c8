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
// Kernels, all on the caller's stream:
//  1. bwd_dq:    one workgroup per (query head, 128-row tile); forms its rows'
//                D_i = dO_i . O_i and lse2_i = lse_i * log2(e) (+inf for rows
//                that see no key and for padding rows, which makes every
//                rebuilt probability 0), writes them packed per 32 rows for
//                the next pass (lse2 and -D), then loops over 32-key tiles, accumulating
//                dQ^T in registers;
//  2. bwd_dkdv:  one workgroup per (KV head, 128-key tile); loops over the
//                query heads that share the KV head and over 32-row query
//                tiles, accumulating dK^T and dV^T in registers (no atomics).
// The dK/dV and dQ passes both rebuild S and dP, which costs two GEMMs more
// than a single pass with atomic dQ but keeps the result deterministic. (A
// separate pass computing the row terms first measured 1 % slower on the
// whole training step than forming them in the dQ pass.)
//
// Fused path (attn_bwd_fused): a first pass, bwd_pre, forms the row terms and
// clears a float32 dQ workspace; the dK/dV pass also forms dQ = dS K for its
// 128 keys and adds it into that workspace with vector atomic adds, so S and
// dP are rebuilt once; dq_convert scales and rounds it into dq afterwards. The order in which workgroups add
// into a dQ row varies from run to run, so the float32 sums (and at times the
// bf16 result) do too. On this chip it is the slower form: every (128-key
// tile, query row) pair costs d float32 atomic adds, about 1.1e9 for the
// 8K-token training shape, and float32 atomic adds retire at roughly 3.4e11
// per second chip-wide (a tenth of the rate of plain stores of the same
// pattern), which alone takes longer than the whole two-kernel backward.
//
// Mapping to CDNA4: in the dK/dV pass the two wavefronts that share a SIMD
// split each tile's work (scores and elementwise terms on one, the gradient
// products on the other), so one's vector work runs under the other's MFMAs.
// In the dQ pass each wavefront's step j interleaves, MFMA by MFMA, the score
// and dP products of tile j+1, the dQ products of tile j-1 and the
// elementwise work (P, dS) of tile j; two workgroups share each CU. Tiles arrive by LDS DMA ahead
// of their first use, in rings sized so that no slot is rewritten while any
// wavefront still reads it.
#include "common.h"
#include "kernels.h"
#include "tiles.h"

#include <algorithm>
#include <cstdio>
#include <type_traits>
#include <utility>

namespace attn {

namespace {

constexpr int BT = 32;        // rows of a pipeline tile (queries for dK/dV, keys for dQ)
constexpr int KV_WG = 128;    // keys per dK/dV workgroup (4 wavefronts x 32)
// 32-query column blocks per dQ wavefront. With one, a wavefront needs under
// 256 registers, so two workgroups share each CU and the two wavefronts on a
// SIMD fill each other's stalls (measured 4 % faster than two blocks, which
// let each K, V or K^T fragment feed two MFMAs but held 512 registers).
constexpr int DQ_NCB = 1;
constexpr int Q_WG = 4 * 32 * DQ_NCB;         // queries per dQ workgroup (4 wavefronts)

// Score MFMAs with the accumulator in VGPRs (the elementwise code reads every
// score; AGPR accumulators would need one v_accvgpr_read per score), issued
// as inline assembly because the kernels otherwise compile with AGPR
// accumulators (the gradient accumulators do not fit next to everything else
// in the 256 VGPRs). The compiler does not track hazards through inline
// assembly: score_settle() must follow the last MFMA of a chain before any
// other instruction reads the accumulator (an MFMA result needs up to 19
// wait states before a non-MFMA read); chained MFMAs with the same
// accumulator as srcC and vdst issue back to back.
__device__ __forceinline__ void mfma_first(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_next(f32x16& acc, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void score_settle(f32x16& x, f32x16& y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
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
  float* ld;      // [B, Hq, sqp / 32][64]: lse2 of 32 rows, then -D of the same rows
  float* dqacc;   // fused path: [B, Hq, sqp, D] float32 sums of dS K (NULL on the two-kernel path)
  int B, Hq, Hkv, Sq, Sk, g, causal;
  int hsq, hsk;   // head strides in rows (see Problem)
  int sqp;        // Sq rounded up to 64
  float scale;
  float c;        // scale * log2(e)
  int n_ktiles, total_kv;
  int n_qtiles, total_q;
  DropParams drop;
};

// Sequence s of a packed launch as a problem of batch 1: lengths, data
// pointers and its lse2/D block from the table (the head strides stay the
// packed totals).
template <int D>
__device__ __forceinline__ void rebase(BwdArgs& a, const SeqTable& T, int s) {
  a.Sq = T.sq[s];
  a.Sk = T.sk[s];
  a.sqp = (a.Sq + TILE_ROWS - 1) / TILE_ROWS * TILE_ROWS;
  a.n_ktiles = (a.Sk + KV_WG - 1) / KV_WG;
  a.n_qtiles = (a.Sq + Q_WG - 1) / Q_WG;
  const size_t qo = (size_t)T.q0[s] * D, ko = (size_t)T.k0[s] * D;
  a.q += qo;
  a.o += qo;
  a.dout += qo;
  a.dq += qo;
  a.lse += T.q0[s];
  a.k += ko;
  a.v += ko;
  a.dk += ko;
  a.dv += ko;
  a.ld += (size_t)T.aux[s] * a.Hq * 2;         // aux: padded query rows of the earlier sequences
}

// Tab (here and in the two gradient kernels): NoTable for one dense problem,
// SeqTable for a packed launch.
template <int D, typename Tab>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a, Tab T) {
  constexpr int LPR = D / 8;       // lanes per row, 8 elements each
  constexpr int RPB = 256 / LPR;   // rows per block
  size_t blk = blockIdx.x;
  if constexpr (std::is_same_v<Tab, SeqTable>) {
    const SeqCoord sc = seq_coord(T);
    rebase<D>(a, T, sc.seq);
    blk = sc.t;
  }
  const size_t rows = (size_t)a.B * a.Hq * a.sqp;
  const size_t prow = blk * RPB + threadIdx.x / LPR;   // padded row
  const int c = threadIdx.x % LPR;
  const size_t head = prow / a.sqp;
  const int pos = (int)(prow % a.sqp);
  const bool valid = prow < rows && pos < a.Sq;
  const size_t row = head * a.hsq + pos;
  float acc = 0.f;
  if (valid) {
    const bf16x8 ov = *(const bf16x8*)(a.o + row * D + c * 8);
    const bf16x8 dv = *(const bf16x8*)(a.dout + row * D + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)ov[e], (float)dv[e], acc);
  }
#pragma unroll
  for (int s = LPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s);
  if (a.dqacc != nullptr && prow < rows) {
    // fused path: clear this row's dQ sums (padding rows too; nothing reads them)
    float* z = a.dqacc + prow * D + c * 8;
    *(f32x4*)z = f32x4{0.f, 0.f, 0.f, 0.f};
    *(f32x4*)(z + 4) = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (prow < rows && c == 0) {
    float l2 = __builtin_huge_valf(), dl = 0.f;
    if (valid) {
      const float l = a.lse[row];
      l2 = (l == kNegInf) ? __builtin_huge_valf() : l * kLog2e;
      dl = acc;
    }
    float* ldb = a.ld + (head * (a.sqp / BT) + pos / BT) * (2 * BT);
    ldb[pos % BT] = l2;
    ldb[BT + pos % BT] = -dl;
  }
}

// ---------------------------------------------------------------------------
// dK, dV. A workgroup of 8 wavefronts owns 128 keys as four 32-key blocks;
// the two wavefronts that share a SIMD (w and w + 4) share block w mod 4,
// whose keys are their MFMA columns, and split the work of each 32-row query
// tile between them:
//  * the score wavefront (w < 4) computes S = Q K^T and dP = dO V^T (rows =
//    queries) with K and V held in registers, then P = 2^(S c - lse2) and
//    dS = P (dP - D), and hands the bf16 fragments of P and dS to its partner
//    through LDS, one lane to the same lane; without dropout the dP
//    accumulator starts at -D (stored negated for this), so that it ends as
//    dP - D and dS is one multiply per score (1 % on the training step);
//  * the gradient wavefront (w >= 4) accumulates dV^T += dO^T P and
//    dK^T += Q^T dS (rows = d) one step later, reading dO^T and Q^T with
//    transposing LDS reads of the row-major tiles the score wavefront used,
//    and issues all the tile DMA.
// The partner's gradient MFMAs fill the matrix pipe while the score wavefront
// does its vector work.
//
// LDS: a 4-slot ring of [Q | dO] row tiles (tile t loaded at the start of
// step t-1, read in steps t and t+1) with its lse2/-D blocks, and a 2-slot
// exchange buffer of P and dS fragments (written in step t, read in step t+1).
// ---------------------------------------------------------------------------
// DROP (here and in the dQ kernel): dropout with the forward's mask, so that
// dV takes P Z and dS = P (Z dP - D), Z = keep / (1 - p).
// FUSED: the gradient wavefronts also form dQ = dS K of each query tile over
// the workgroup's 128 keys and add it into a.dqacc. Wavefront w takes the
// 32-channel block w mod (D/32) of dQ and the key chunks 8 (D/32) / 4 of its
// share (all 128 keys at D = 128, half of them at D = 64): its B operand (K
// for 16 keys x 32 channels per MFMA) is loaded into registers once, its A
// operand (dS, 32 queries x 16 keys) is read transposed from the exchange
// buffer of all four key blocks. The 16 sums per lane are added with vector
// atomics after the step's MFMAs; the barrier's wait leaves them in flight
// (vector memory operations complete in issue order, so waiting until at most
// that many are outstanding covers the tile DMA issued before them).
template <int D, bool CAUSAL, typename Tab, bool DROP, bool FUSED>
__global__ __launch_bounds__(512) void bwd_dkdv_kernel(BwdArgs a, Tab T) {
  constexpr int DC = D / 16;
  constexpr int MB = D / 32;
  constexpr int CPR = D / 8;                    // 16-byte chunks per row
  constexpr int RB = 2 * D;                     // bytes per row
  constexpr int TB = BT * RB;                   // bytes of a 32-row tile
  constexpr int RING = 4;
  constexpr int SLOT = 2 * TB;                  // [Q | dO]
  constexpr int LB = 2 * BT * 4;                // lse2/D of a tile
  constexpr int L_OFF = RING * SLOT;
  constexpr int X_OFF = L_OFF + RING * LB;
  constexpr int XB = 64 * 64;                   // exchange bytes per key block: 64 lanes x (P, dS)
  constexpr int XSLOT = 4 * XB;
  constexpr int INSTR = TB / 4096;              // DMA instructions per gradient wavefront per tensor
  constexpr int NDMA = 2 * INSTR + 1;           // ... per step: Q, dO, lse2/D
  static_assert(INSTR >= 1, "four wavefronts share each tile's DMA");
  __shared__ __attribute__((aligned(1024))) char smem[X_OFF + 2 * XSLOT];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kb = wid & 3;                       // key block, shared by the SIMD's two wavefronts
  const bool grad = wid >= 4;
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int kt, hkv, b;
  if constexpr (std::is_same_v<Tab, SeqTable>) {
    const SeqCoord sc = seq_coord(T);
    rebase<D>(a, T, sc.seq);
    kt = sc.t;
    hkv = sc.unit;
    b = 0;
  } else {
    int bh;
    xcd_tile_order(a.total_kv, a.n_ktiles, kt, bh);
    hkv = bh % a.Hkv;
    b = bh / a.Hkv;
  }
  const int off = (a.causal == 2) ? (a.Sk - a.Sq) : 0;
  const int k0 = kt * KV_WG;
  const int key = k0 + 32 * kb + l32;
  const bool kvalid = key < a.Sk;

  const int n_qt = (a.Sq + BT - 1) / BT;
  const int qt_lo = a.causal ? min(n_qt, max(0, k0 - off) / BT) : 0;
  const int per_head = n_qt - qt_lo;
  const int n = a.g * per_head;                 // pipeline tiles: (query head, 32-row tile)

  // Tile sequence: for each query head of the group, the 32-row tiles from
  // the last one down to the first one that sees a key of this workgroup.
  // Walking down keeps every workgroup of a head on the same tile at the same
  // time (they all start at the last tile), so each tile is fetched into L2
  // once and then served to all of them. (On the fused path this also has the
  // workgroups of a head add into the same dQ rows at about the same time; a
  // walk rotated per key tile was measured no faster, since the atomic adds
  // are bound by their chip-wide rate, not by contention.)
  auto advance = [&](int& hq, int& q0) __attribute__((always_inline)) {
    q0 -= BT;
    if (q0 < qt_lo * BT) {
      q0 = (n_qt - 1) * BT;
      ++hq;
    }
  };
  // step j: the tiles j (score wavefronts) and j - 1 (gradient wavefronts)
  // have landed for every wavefront (the gradient wavefronts wait for all
  // their DMA, the barrier makes it visible to all), the exchange slot of
  // tile j - 1 is complete, and every wavefront is done with step j - 1.
  constexpr int NATOM = 16;                     // fused path: atomic adds per gradient wavefront and step
  bool atoms_out = false;                       // some are in flight (gradient wavefronts)
  auto sync = [&]() __attribute__((always_inline)) {
    if (grad) {
      if (FUSED && atoms_out)
        asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NATOM) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory");
    } else {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  const char* lds = smem;

  if (!grad) {
    // ---------------- score wavefront ----------------
    // K and V fragments: B operands of S = Q K^T and dP = dO V^T (column = key)
    bf16x8 kf[DC], vf[DC];
    {
      const size_t kvrow = (((size_t)b * a.Hkv + hkv) * a.hsk + (kvalid ? key : 0)) * D;
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
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        kf[dc] = settle(kf[dc]);
        vf[dc] = settle(vf[dc]);
      }
    }
    // A-operand fragments of S and dP: row l32 (query), logical chunk 2 dc + hi
    uint32_t rb[DC];
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) rb[dc] = l32 * RB + (((2 * dc + hi) ^ chunk_swizzle<D>(l32)) << 4);
    const uint32_t lb = L_OFF + 16 * hi;
    const uint32_t xw = X_OFF + kb * XB + lane * 16;
    int hq = hkv * a.g, q0 = (n_qt - 1) * BT;

    auto step = [&](auto pos_, auto mask_) __attribute__((always_inline)) {
      constexpr int POS = decltype(pos_)::value;
      constexpr bool MASK = decltype(mask_)::value;
      const char* tile = lds + POS * SLOT;
      auto frag = [&](int k) __attribute__((always_inline)) {   // op k: S (even) / dP (odd), d-chunk k / 2
        return *(const bf16x8*)(tile + rb[k >> 1] + (k & 1) * TB);
      };
      f32x4 l2v[4], dlv[4];
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        l2v[i4] = *(const f32x4*)(lds + lb + POS * LB + 32 * i4);
        dlv[i4] = *(const f32x4*)(lds + lb + POS * LB + 4 * BT + 32 * i4);
      }
      f32x16 s, dp;
      bf16x8 f[3];
      f[0] = frag(0);
      f[1] = frag(1);
      // the dP accumulator starts at -D of its rows, so that it ends as dP - D
      if constexpr (!DROP)
        dp = __builtin_shufflevector(__builtin_shufflevector(dlv[0], dlv[1], 0, 1, 2, 3, 4, 5, 6, 7),
                                     __builtin_shufflevector(dlv[2], dlv[3], 0, 1, 2, 3, 4, 5, 6, 7), 0, 1, 2, 3, 4, 5,
                                     6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
      static_for<2 * DC>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        if constexpr (k + 2 < 2 * DC) f[(k + 2) % 3] = frag(k + 2);
        __builtin_amdgcn_sched_barrier(0);      // keep the reads two MFMAs ahead of their use
        if constexpr (k < 2) {
          if constexpr (k & 1) {
            if constexpr (DROP)
              mfma_first(dp, f[k % 3], vf[k >> 1]);
            else
              mfma_next(dp, f[k % 3], vf[k >> 1]);
          } else {
            mfma_first(s, f[k % 3], kf[k >> 1]);
          }
        } else {
          if constexpr (k & 1)
            mfma_next(dp, f[k % 3], vf[k >> 1]);
          else
            mfma_next(s, f[k % 3], kf[k >> 1]);
        }
      });
      score_settle(s, dp);
      // accumulator register v holds query q0 + 8 (v >> 2) + 4 hi + (v & 3)
      float p[16], ds[16];
      u32x4 dx;                                 // dropout: block of query rows q0 + 8g + 4hi .. +3
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float pv = fast_exp2(__builtin_fmaf(s[v], a.c, -l2v[v >> 2][v & 3]));
        if constexpr (MASK) {
          if (key > q0 + 8 * (v >> 2) + 4 * hi + (v & 3) + off) pv = 0.f;
        }
        if constexpr (DROP) {
          // this lane's key is byte (key & 3) of word (v & 3) of the block
          if ((v & 3) == 0)
            dx = dropout_block(a.drop, (uint32_t)(q0 + 8 * (v >> 2) + 4 * hi) >> 2, (uint32_t)key >> 2,
                               (uint32_t)(b * a.Hq + hq));
          const float z = ((dx[v & 3] >> (8 * (key & 3))) & 0xffu) >= a.drop.thr ? a.drop.scale : 0.f;
          p[v] = pv * z;
          ds[v] = pv * (z * dp[v] + dlv[v >> 2][v & 3]);
        } else {
          p[v] = pv;
          ds[v] = pv * dp[v];
        }
      }
      char* xs = smem + xw + (POS & 1) * XSLOT;
      *(bf16x8*)(xs + 0 * 1024) = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
      *(bf16x8*)(xs + 1 * 1024) = to_bf16x8(p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]);
      *(bf16x8*)(xs + 2 * 1024) = to_bf16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
      *(bf16x8*)(xs + 3 * 1024) = to_bf16x8(ds[8], ds[9], ds[10], ds[11], ds[12], ds[13], ds[14], ds[15]);
      advance(hq, q0);
    };
    using M_ = std::integral_constant<bool, CAUSAL>;
    // Causal masking is needed only where some key of the workgroup lies
    // above some query of the tile. The walk runs down to the diagonal, so
    // with one query head per KV head these are the last tiles: the first
    // n_um steps run unmasked, the rest masked (the loops switch at a multiple
    // of 4 so slot positions stay compile-time). With several query heads per
    // KV head every step is masked. Without a causal mask nothing needs
    // masking: rows past Sq have lse2 = +inf, so their P and dS are 0.
    int n_um = n;
    if (CAUSAL) {
      n_um = 0;
      if (a.g == 1) {
        // tile qt is unmasked iff its first row sees the workgroup's last key
        const int x = k0 + KV_WG - 1 - off;
        const int lowest_unmasked = x <= 0 ? 0 : (x + BT - 1) / BT;
        n_um = min(n, max(0, n_qt - max(lowest_unmasked, qt_lo)));
      }
    }
    int j = 0;
    for (; j + 3 < n_um; j += 4) {
      sync();
      step(I0{}, F_{});
      sync();
      step(I1{}, F_{});
      sync();
      step(I2{}, F_{});
      sync();
      step(I3{}, F_{});
    }
    for (; j + 3 < n; j += 4) {
      sync();
      step(I0{}, M_{});
      sync();
      step(I1{}, M_{});
      sync();
      step(I2{}, M_{});
      sync();
      step(I3{}, M_{});
    }
    if (j < n) {
      sync();
      step(I0{}, M_{});
    }
    if (j + 1 < n) {
      sync();
      step(I1{}, M_{});
    }
    if (j + 2 < n) {
      sync();
      step(I2{}, M_{});
    }
    if (n > 0) sync();                          // the gradient wavefronts' step n
    return;
  }

  // ---------------- gradient wavefront ----------------
  // DMA geometry of instruction i: LDS chunk P = (kb*INSTR + i)*64 + lane of a
  // tile, i.e. row P / CPR, physical chunk P % CPR, loading the logical chunk
  // (physical ^ swizzle(row)); byte offsets relative to the tile's first row.
  uint32_t roff[INSTR];
#pragma unroll
  for (int i = 0; i < INSTR; ++i) {
    const int P = (kb * INSTR + i) * 64 + lane;
    const int rr = P / CPR;
    roff[i] = rr * RB + (((P % CPR) ^ chunk_swizzle<D>(rr)) << 4);
  }
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const uint32_t ldsw = __builtin_amdgcn_readfirstlane(lds0 + kb * INSTR * 1024);
  // DMA of the tiles in sequence order; past the last tile it reloads the last
  // one into a slot nobody reads any more, which keeps the per-step DMA count
  // uniform. Buffer descriptors are rebuilt only when the head changes; rows
  // past Sq are out of the row buffers' range and read zeros.
  int dhq = hkv * a.g, dq0 = (n_qt - 1) * BT, issued = 0, dh = -1;
  u32x4 rq, rd, rl;
  struct Dma {
    uint32_t vr[INSTR];
    uint32_t sl;
  };
  auto next_dma = [&]() __attribute__((always_inline)) {
    if (dhq != dh) {
      dh = dhq;
      const size_t h = (size_t)b * a.Hq + dhq;
      rq = buffer_rsrc(a.q + h * a.hsq * D, (uint32_t)a.Sq * RB);
      rd = buffer_rsrc(a.dout + h * a.hsq * D, (uint32_t)a.Sq * RB);
      rl = buffer_rsrc(a.ld + h * (a.sqp / BT) * (2 * BT), (uint32_t)a.sqp * 8);
    }
    Dma o;
#pragma unroll
    for (int i = 0; i < INSTR; ++i) o.vr[i] = roff[i] + (uint32_t)dq0 * RB;
    o.sl = (uint32_t)(dq0 / BT) * LB;
    if (++issued < n) advance(dhq, dq0);
    return o;
  };
  // DMA instruction QI (0 .. NDMA-1) of a tile into ring slot S
  auto dma_one = [&](auto s_, auto qi_, const Dma& o) __attribute__((always_inline)) {
    constexpr int S = decltype(s_)::value;
    constexpr int QI = decltype(qi_)::value;
    constexpr int i = QI % INSTR;
    if constexpr (QI < INSTR)
      dma16b_at<S * SLOT + i * 1024>(rq, o.vr[i], 0u, ldsw);
    else if constexpr (QI < 2 * INSTR)
      dma16b_at<S * SLOT + TB + i * 1024>(rd, o.vr[i], 0u, ldsw);
    else                                        // every gradient wavefront loads the same 256 bytes
      dma4b_at<L_OFF + S * LB>(rl, (uint32_t)lane * 4, o.sl, lds0);
  };
  // Transposing reads: the A operand of dV^T += dO^T P for d-block mb and
  // 16-query chunk qc is two 4-query reads at rows 16 qc + 4 hi + (L >> 2)
  // (+8) and columns 32 mb + 16 dhalf + 4 (L & 3) of the dO tile (Q tile for
  // dK^T); their query order is the register order of the P and dS fragments.
  // The row swizzle does not change with qc, so qc is an immediate offset.
  uint32_t vb[MB][2];
  {
    const int L = lane & 15, dhalf = (lane >> 4) & 1;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 4 * hi + (L >> 2) + 8 * h;
        const int c = 32 * mb + 16 * dhalf + 4 * (L & 3);
        vb[mb][h] = r * RB + (((c >> 3) ^ chunk_swizzle<D>(r)) << 4) + (c & 7) * 2;
      }
  }
  const uint32_t xr = X_OFF + kb * XB + lane * 16;

  // Fused dQ. Channel block dblk = kb mod MB, key chunks kc0 .. kc0 + NKC - 1
  // (16 keys each, chunk kc in key block kc / 2). B operand: lane l holds
  // channel 32 dblk + (l mod 32) and keys 16 kc + 8 (l / 32) + 0..7, loaded once.
  // A operand (dS, rows = the tile's 32 queries): two transposing 4-key reads
  // per MFMA from the exchange entries the score wavefronts wrote, where the
  // lane of key kk (and half h) holds queries 4 c .. 4 c + 3 for chunk
  // c = 2 (v / 4) + h of its registers v; within a 16-lane group lane L reads
  // key kk0 + L / 4 at query chunk c = 4 (group & 1) + (L & 3), so that output
  // lane j holds query 16 (group & 1) + j.
  constexpr int NKC = 2 * MB;                   // key chunks per wavefront
  const int dblk = kb % MB;
  const int kc0 = (kb / MB) * NKC;
  bf16x8 ktf[FUSED ? NKC : 1];
  uint32_t xq = 0;
  if constexpr (FUSED) {
    const bf16* kcol = a.k + ((size_t)b * a.Hkv + hkv) * a.hsk * D + 32 * dblk + l32;
#pragma unroll
    for (int i = 0; i < NKC; ++i) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kk = k0 + 16 * (kc0 + i) + 8 * hi + e;
        ktf[i][e] = kk < a.Sk ? kcol[(size_t)kk * D] : (bf16)0.f;
      }
    }
#pragma unroll
    for (int i = 0; i < NKC; ++i) ktf[i] = settle(ktf[i]);
    const int L = lane & 15, c = 4 * ((lane >> 4) & 1) + (L & 3);
    xq = X_OFF + 2048 + (8 * hi + (L >> 2)) * 16 + 512 * (c & 1) + 1024 * (c >> 2) + 8 * ((c >> 1) & 1);
  }
  int ghq = hkv * a.g, gq0 = (n_qt - 1) * BT;   // query tile whose gradients the step forms

  f32x16 dkt[MB], dvt[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    dkt[mb] = f32x16{};
    dvt[mb] = f32x16{};
  }
  // step j at slot position POS = j mod 4: DMA of tile j + 1, issued first
  // so that it has the whole step to land, then the gradients of tile j - 1
  // (if G)
  auto step = [&](auto pos_, auto g_) __attribute__((always_inline)) {
    constexpr int POS = decltype(pos_)::value;
    constexpr bool G = decltype(g_)::value;
    constexpr int SG = (POS + 3) % RING;        // rows of tile j - 1
    constexpr int SD = (POS + 1) % RING;        // DMA target: tile j + 1
    const Dma o = next_dma();
    static_for<NDMA>([&](auto qi) __attribute__((always_inline)) { dma_one(std::integral_constant<int, SD>{}, qi, o); });
    if constexpr (G) {
      const char* xs = lds + xr + ((POS + 1) & 1) * XSLOT;
      bf16x8 pf[2], dsf[2];
      pf[0] = *(const bf16x8*)(xs + 0 * 1024);
      pf[1] = *(const bf16x8*)(xs + 1 * 1024);
      dsf[0] = *(const bf16x8*)(xs + 2 * 1024);
      dsf[1] = *(const bf16x8*)(xs + 3 * 1024);
      const char* tile = lds + SG * SLOT;
      // gradient op g: chain g % 2MB (dV^T for < MB, dK^T above), query chunk g / 2MB
      auto gfrag = [&](int g) __attribute__((always_inline)) {
        const int ch = g % (2 * MB), qc = g / (2 * MB);
        const char* t = tile + (ch < MB ? TB : 0) + qc * 16 * RB;
        return cat4(lds_read_tr((const bf16*)(t + vb[ch % MB][0])), lds_read_tr((const bf16*)(t + vb[ch % MB][1])));
      };
      // fused dQ op i: key chunk kc0 + i of the exchange slot of tile j - 1
      const char* xs_q = lds + xq + ((POS + 1) & 1) * XSLOT;
      auto qfrag = [&](int i) __attribute__((always_inline)) {
        const int kc = kc0 + i;
        const char* t = xs_q + (kc >> 1) * XB + (kc & 1) * 256;
        return cat4(lds_read_tr((const bf16*)t), lds_read_tr((const bf16*)(t + 64)));
      };
      constexpr int NG = 4 * MB;                  // dV^T and dK^T MFMAs
      constexpr int NQ = FUSED ? NKC : 0;         // dQ MFMAs, one after every two gradient ones
      constexpr int NOPS = NG + NQ;
      // op k -> (is a dQ op, index within its kind)
      auto is_q = [](int k) constexpr { return FUSED && k % 3 == 2; };
      auto idx = [](int k) constexpr { return FUSED ? (k % 3 == 2 ? k / 3 : k - (k + 1) / 3) : k; };
      auto frag = [&](int k) __attribute__((always_inline)) { return is_q(k) ? qfrag(idx(k)) : gfrag(idx(k)); };
      f32x16 dqa;
      bf16x8 f[3];
      f[0] = frag(0);
      f[1] = frag(1);
      static_for<NOPS>([&](auto kc) __attribute__((always_inline)) {
        constexpr int k = decltype(kc)::value;
        if constexpr (k + 2 < NOPS) f[(k + 2) % 3] = frag(k + 2);
        __builtin_amdgcn_sched_barrier(0);      // keep the reads two MFMAs ahead of their use
        constexpr int g = idx(k);
        if constexpr (is_q(k)) {
          dqa = mfma32(f[k % 3], ktf[g], g == 0 ? f32x16{} : dqa);
        } else {
          constexpr int ch = g % (2 * MB), qc = g / (2 * MB);
          if constexpr (ch < MB)
            dvt[ch] = mfma32(f[k % 3], pf[qc], dvt[ch]);
          else
            dkt[ch - MB] = mfma32(f[k % 3], dsf[qc], dkt[ch - MB]);
        }
      });
      if constexpr (FUSED) {
        static_assert(NQ > 0 && NOPS % 3 == 0, "every third op is a dQ op");
        // accumulator register i: query gq0 + 8 (i / 4) + 4 hi + (i % 4), channel 32 dblk + l32
        float* dst = a.dqacc + ((size_t)(b * a.Hq + ghq) * a.sqp + gq0 + 4 * hi) * D + 32 * dblk + l32;
#pragma unroll
        for (int i = 0; i < NATOM; ++i)
          __hip_atomic_fetch_add(dst + (8 * (i >> 2) + (i & 3)) * D, dqa[i], __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        atoms_out = true;
        advance(ghq, gq0);
      }
    }
  };
  if (n > 0) {
    {
      const Dma o0 = next_dma();
      static_for<NDMA>([&](auto qi) __attribute__((always_inline)) { dma_one(I0{}, qi, o0); });
    }
    sync();
    step(I0{}, F_{});                           // j = 0: DMA only
    int j = 1;
    for (; j + 3 <= n; j += 4) {
      sync();
      step(I1{}, T_{});
      sync();
      step(I2{}, T_{});
      sync();
      step(I3{}, T_{});
      sync();
      step(I0{}, T_{});
    }
    if (j <= n) {
      sync();
      step(I1{}, T_{});
    }
    if (j + 1 <= n) {
      sync();
      step(I2{}, T_{});
    }
    if (j + 2 <= n) {
      sync();
      step(I3{}, T_{});
    }
  }
  // no LDS DMA may still be in flight when the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  if (!kvalid) return;
  const size_t kvrow = (((size_t)b * a.Hkv + hkv) * a.hsk + key) * D;
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
// ---------------------------------------------------------------------------
// dQ. Wavefront w owns queries p + 32 NCB w .. as NCB blocks of 32 MFMA
// columns: S^T = K Q^T and dP^T = V dO^T (rows = 32 keys) take Q and dO from
// registers, dQ^T += K^T dS^T (rows = d) takes dS^T from the score
// accumulators and K^T from transposing LDS reads of the row-major K tile;
// each K, V or K^T fragment read from LDS feeds NCB MFMAs. A 4-slot ring of
// [K | V] row tiles: key tile t is loaded at the start of step t-2 and read in
// steps t-1 (K, V) and t+1 (K^T).
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL, typename Tab, bool DROP>
__global__ __launch_bounds__(256, (DQ_NCB == 1 && !DROP) ? 2 : 1) void bwd_dq_kernel(BwdArgs a, Tab T) {
  constexpr int NCB = DQ_NCB;
  constexpr int DC = D / 16;
  constexpr int MB = D / 32;
  constexpr int NU = DC;                        // units per step: 2 row fragments + 1 K^T fragment each
  constexpr int CPR = D / 8;
  constexpr int RB = 2 * D;                     // bytes per row
  constexpr int TB = BT * RB;
  constexpr int INSTR = TB / 4096;
  constexpr int NDMA = 2 * INSTR;               // K, V
  constexpr int RING = 4;
  static_assert(2 * MB == NU, "one K^T fragment per unit");
  __shared__ __attribute__((aligned(1024))) char smem[RING * 2 * TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;

  int qtile, hq, b;
  if constexpr (std::is_same_v<Tab, SeqTable>) {
    const SeqCoord sc = seq_coord(T);
    rebase<D>(a, T, sc.seq);
    qtile = sc.t;
    hq = sc.unit;
    b = 0;
  } else {
    int bh;
    xcd_tile_order(a.total_q, a.n_qtiles, qtile, bh);
    hq = bh % a.Hq;
    b = bh / a.Hq;
  }
  const int off = (a.causal == 2) ? (a.Sk - a.Sq) : 0;
  const int qb = a.n_qtiles - 1 - qtile;        // longest causal tiles first
  const int hkv = hq / a.g;
  const int p0 = qb * Q_WG + 32 * NCB * wid;    // first query of the wavefront
  const int wg_last = min(qb * Q_WG + Q_WG, a.Sq) - 1;
  int kend = a.causal ? min(a.Sk, wg_last + off + 1) : a.Sk;
  if (kend < 0) kend = 0;
  const int n = (kend + BT - 1) / BT;

  const size_t hrow = (size_t)b * a.Hq + hq;
  int pos[NCB], lim[NCB];
  bool valid[NCB];
  bf16x8 qf[NCB][DC], df[NCB][DC];
  float l2[NCB], dl[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    pos[cb] = p0 + 32 * cb + l32;
    valid[cb] = pos[cb] < a.Sq;
    lim[cb] = a.causal ? min(kend - 1, pos[cb] + off) : kend - 1;
    const size_t qrow = hrow * a.hsq + (valid[cb] ? pos[cb] : 0);
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      if (valid[cb]) {
        qf[cb][dc] = *(const bf16x8*)(a.q + qrow * D + 16 * dc + 8 * hi);
        df[cb][dc] = *(const bf16x8*)(a.dout + qrow * D + 16 * dc + 8 * hi);
      } else {
        qf[cb][dc] = __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
        df[cb][dc] = qf[cb][dc];
      }
    }
    // The row terms of this lane's query row, formed here rather than by a
    // preprocessing pass: D = dO . O over the row's channels (this lane's
    // half, then its partner lane's) and lse2 = lse log2(e), +inf where the
    // row sees no key or lies past Sq (every rebuilt probability is then 0).
    // They also go to the row's lse2/D block (D negated) for the dK/dV pass that follows.
    float dpart = 0.f, l = kNegInf;
    if (valid[cb]) {
#pragma unroll
      for (int dc = 0; dc < DC; ++dc) {
        const bf16x8 ov = *(const bf16x8*)(a.o + qrow * D + 16 * dc + 8 * hi);
#pragma unroll
        for (int e = 0; e < 8; ++e) dpart = __builtin_fmaf((float)ov[e], (float)df[cb][dc][e], dpart);
      }
      l = a.lse[qrow];
    }
    dl[cb] = sum_halves(dpart);
    l2[cb] = (l == kNegInf) ? __builtin_huge_valf() : l * kLog2e;
    if (hi == 0 && pos[cb] < a.sqp) {
      float* blk = a.ld + (hrow * (a.sqp / BT) + pos[cb] / BT) * (2 * BT);
      blk[pos[cb] % BT] = l2[cb];
      blk[BT + pos[cb] % BT] = -dl[cb];
    }
  }
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {       // only MFMAs read them: keep them in AGPRs
      qf[cb][dc] = settle(qf[cb][dc]);
      df[cb][dc] = settle(df[cb][dc]);
    }
    l2[cb] = settle(l2[cb]);
    dl[cb] = settle(dl[cb]);
  }
  // without dropout the dP^T accumulators start at -D of the lane's row, so
  // that they end as dP - D (a register tuple of its own, kept for the kernel)
  f32x16 ndl[NCB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int i = 0; i < 16; ++i) ndl[cb][i] = DROP ? 0.f : -dl[cb];

  const size_t kvh = (size_t)b * a.Hkv + hkv;
  const bf16* kg = a.k + kvh * (size_t)a.hsk * D;
  const bf16* vg = a.v + kvh * (size_t)a.hsk * D;
  uint32_t rb[DC];
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) rb[dc] = l32 * RB + (((2 * dc + hi) ^ chunk_swizzle<D>(l32)) << 4);
  // Transposing reads: the A operand of dQ^T += K^T dS^T for d-block mb and
  // 16-key chunk kc is two 4-key reads at rows 16 kc + 4 hi + (L >> 2) (+8)
  // and columns 32 mb + 16 dhalf + 4 (L & 3) of the K tile; their key order is
  // the register order of the dS^T fragments. The row swizzle does not change
  // with kc, so kc is an immediate offset.
  uint32_t vb[MB][2];
  {
    const int L = lane & 15, dhalf = (lane >> 4) & 1;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 4 * hi + (L >> 2) + 8 * h;
        const int c = 32 * mb + 16 * dhalf + 4 * (L & 3);
        vb[mb][h] = r * RB + (((c >> 3) ^ chunk_swizzle<D>(r)) << 4) + (c & 7) * 2;
      }
  }
  uint32_t roff[INSTR];
#pragma unroll
  for (int i = 0; i < INSTR; ++i) {
    const int P = (wid * INSTR + i) * 64 + lane;
    const int rr = P / CPR;
    roff[i] = rr * RB + (((P % CPR) ^ chunk_swizzle<D>(rr)) << 4);
  }
  const uint32_t ldsw = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem + wid * INSTR * 1024);
  // K / V rows of the KV head (rows past Sk are out of range and read zeros);
  // a key tile is a byte offset
  const u32x4 rk = buffer_rsrc(kg, (uint32_t)a.Sk * RB);
  const u32x4 rv = buffer_rsrc(vg, (uint32_t)a.Sk * RB);
  struct DmaOff {
    uint32_t vr[INSTR];                         // rows of the key tile (per lane)
  };
  // key tiles past the last one are clamped to it (reloaded into unread slots)
  auto dma_offsets = [&](int t) __attribute__((always_inline)) {
    DmaOff o;
    const uint32_t key = (uint32_t)min(t, n - 1) * BT;
#pragma unroll
    for (int i = 0; i < INSTR; ++i) o.vr[i] = roff[i] + key * RB;
    return o;
  };
  auto dma_one = [&](auto skv_, auto qi_, const DmaOff& o) __attribute__((always_inline)) {
    constexpr int SKV = decltype(skv_)::value;
    constexpr int QI = decltype(qi_)::value;
    constexpr int i = QI % INSTR;
    constexpr uint32_t part = i * 1024;
    if constexpr (QI < INSTR)
      dma16b_at<SKV * 2 * TB + part>(rk, o.vr[i], 0u, ldsw);
    else
      dma16b_at<SKV * 2 * TB + TB + part>(rv, o.vr[i], 0u, ldsw);
  };
  using C0 = std::integral_constant<int, 0>;

  f32x16 dqt[NCB][MB];
#pragma unroll
  for (int cb = 0; cb < NCB; ++cb)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) dqt[cb][mb] = f32x16{};
  // S^T of two tiles in flight; dP^T of one (the elementwise work of tile j
  // reads it before the dP^T products of tile j+1 start)
  f32x16 s_[2][NCB], dp_[NCB];
  bf16x8 dsf[2][NCB][2];                        // [tile parity][column block][16-key chunk]

  // One step j (slot position POS = j mod 4), after the DMA of tile j+2 (issued
  // first, so that it has the whole step to land), in two phases:
  //  1. unit u = 0 .. NU-1: S^T of tile j+1 from K fragment u (2 MFMAs), dQ^T of
  //     tile j-1 from K^T fragment u (d-block u % MB, 16-key chunk u / MB;
  //     2 MFMAs), and a share of the elementwise work (dS) of tile j;
  //  2. unit u: dP^T of tile j+1 from V fragment u (2 MFMAs).
  auto step = [&](auto pos_, auto g1, auto g2, auto ew, auto mask_, int j) __attribute__((always_inline)) {
    constexpr int POS = decltype(pos_)::value;
    constexpr int P = POS & 1;
    constexpr bool G1 = decltype(g1)::value;
    constexpr bool G2 = decltype(g2)::value;
    constexpr bool EW = decltype(ew)::value;
    constexpr bool MASK = decltype(mask_)::value;
    constexpr int SKV = (POS + 1) % RING;       // K, V rows of tile j+1
    constexpr int SKT = (POS + 3) % RING;       // K rows of tile j-1, read transposed
    constexpr int SD = (POS + 2) % RING;        // DMA target: tile j+2
    const char* lds = smem;
    auto kfr = [&](int u) __attribute__((always_inline)) { return *(const bf16x8*)(lds + rb[u] + SKV * 2 * TB); };
    auto vfr = [&](int u) __attribute__((always_inline)) { return *(const bf16x8*)(lds + rb[u] + SKV * 2 * TB + TB); };
    auto tfr = [&](int u) __attribute__((always_inline)) {
      const char* t = lds + SKT * 2 * TB + (u / MB) * 16 * RB;
      return cat4(lds_read_tr((const bf16*)(t + vb[u % MB][0])), lds_read_tr((const bf16*)(t + vb[u % MB][1])));
    };
    if constexpr (G1) {
      const DmaOff o = dma_offsets(j + 2);
      static_for<NDMA>([&](auto qi) __attribute__((always_inline)) { dma_one(std::integral_constant<int, SD>{}, qi, o); });
    }
    const int key0 = j * BT;
    bf16x8 fk[2], ft[2], fv[2];
    if constexpr (G1) fk[0] = kfr(0);
    if constexpr (G2) ft[0] = tfr(0);
    float dt[NCB][8];
    uint32_t dword[NCB];                        // dropout: this row's 4 bytes of the current key quad
    static_for<NU>([&](auto uc) __attribute__((always_inline)) {
      constexpr int u = decltype(uc)::value;
      if constexpr (u + 1 < NU) {
        if constexpr (G1) fk[(u + 1) & 1] = kfr(u + 1);
        if constexpr (G2) ft[(u + 1) & 1] = tfr(u + 1);
      }
      if constexpr (u + 1 == NU) {
        if constexpr (G1) fv[0] = vfr(0);
      }
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (G1) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          s_[P ^ 1][cb] = mfma32(fk[u & 1], qf[cb][u], u == 0 ? f32x16{} : s_[P ^ 1][cb]);
      }
      if constexpr (G2) {
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb)
          dqt[cb][u % MB] = mfma32(ft[u & 1], dsf[P ^ 1][cb][u / MB], dqt[cb][u % MB]);
      }
      if constexpr (EW) {
        // values [v0, v1) of the 16 NCB score registers (16 per column block)
        constexpr int v0 = (u * 16 * NCB) / NU;
        constexpr int v1 = ((u + 1) * 16 * NCB) / NU;
#pragma unroll
        for (int vv = v0; vv < v1; ++vv) {
          const int cb = vv >> 4;
          const int v = vv & 15;
          float p = fast_exp2(__builtin_fmaf(s_[P][cb][v], a.c, -l2[cb]));
          if constexpr (MASK) {
            if (key0 + 8 * (v >> 2) + 4 * hi + (v & 3) > lim[cb]) p = 0.f;
          }
          if constexpr (DROP) {
            if ((v & 3) == 0) {
              const u32x4 x = dropout_block(a.drop, (uint32_t)pos[cb] >> 2,
                                            (uint32_t)(key0 + 8 * (v >> 2) + 4 * hi) >> 2, (uint32_t)hrow);
              const int w = pos[cb] & 3;
              dword[cb] = w == 0 ? x[0] : w == 1 ? x[1] : w == 2 ? x[2] : x[3];
            }
            const float z = ((dword[cb] >> (8 * (v & 3))) & 0xffu) >= a.drop.thr ? a.drop.scale : 0.f;
            dt[cb][v & 7] = p * (z * dp_[cb][v] - dl[cb]);
          } else {
            dt[cb][v & 7] = p * dp_[cb][v];
          }
          pin(dt[cb][v & 7]);
          if ((v & 7) == 7) {
            dsf[P][cb][v >> 3] = to_bf16x8(dt[cb][0], dt[cb][1], dt[cb][2], dt[cb][3], dt[cb][4], dt[cb][5],
                                           dt[cb][6], dt[cb][7]);
            pin(dsf[P][cb][v >> 3]);
          }
        }
      }
    });
    if constexpr (G1) {
      static_for<NU>([&](auto uc) __attribute__((always_inline)) {
        constexpr int u = decltype(uc)::value;
        if constexpr (u + 1 < NU) fv[(u + 1) & 1] = vfr(u + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) dp_[cb] = mfma32(fv[u & 1], df[cb][u], u == 0 ? (DROP ? f32x16{} : ndl[cb]) : dp_[cb]);
      });
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // Causal masking is needed only for key tiles that reach past the first
  // query of the workgroup: the last ones of the walk. The first n_um steps
  // run unmasked, the rest masked (switching at a multiple of 4). Without a
  // causal mask nothing needs masking: keys past Sk have zero K rows, so their
  // dS never reaches dQ.
  using M_ = std::integral_constant<bool, CAUSAL>;
  int n_um = n;
  if (CAUSAL) {
    const int y = qb * Q_WG + off - (BT - 1);   // tile t is unmasked iff t * BT <= y
    n_um = y < 0 ? 0 : min(n, y / BT + 1);
  }
  auto full = [&](auto pos_, auto g2, auto mask_, int j) __attribute__((always_inline)) {
    step(pos_, T_{}, g2, T_{}, mask_, j);
  };
  // step j: tile j+1 has landed for every wavefront (each waits for all its
  // DMA, the barrier for all of them), and every wavefront is done with step
  // j-1
  auto sync = [&]() __attribute__((always_inline)) { asm volatile("s_waitcnt vmcnt(0)\n\ts_barrier" ::: "memory"); };

  if (n > 0) {
    {
      const DmaOff o0 = dma_offsets(0);         // tile 0; step -1 loads tile 1
      static_for<NDMA>([&](auto qi) __attribute__((always_inline)) { dma_one(C0{}, qi, o0); });
    }
    sync();
    step(I3{}, T_{}, F_{}, F_{}, F_{}, -1);
    sync();
    if (n_um > 0)
      full(I0{}, F_{}, F_{}, 0);
    else
      full(I0{}, F_{}, M_{}, 0);
  }
  int j = 1;
  for (; j + 3 < n_um; j += 4) {
    sync();
    full(I1{}, T_{}, F_{}, j);
    sync();
    full(I2{}, T_{}, F_{}, j + 1);
    sync();
    full(I3{}, T_{}, F_{}, j + 2);
    sync();
    full(I0{}, T_{}, F_{}, j + 3);
  }
  for (; j + 3 < n; j += 4) {
    sync();
    full(I1{}, T_{}, M_{}, j);
    sync();
    full(I2{}, T_{}, M_{}, j + 1);
    sync();
    full(I3{}, T_{}, M_{}, j + 2);
    sync();
    full(I0{}, T_{}, M_{}, j + 3);
  }
  if (j < n) {
    sync();
    full(I1{}, T_{}, M_{}, j);
  }
  if (j + 1 < n) {
    sync();
    full(I2{}, T_{}, M_{}, j + 1);
  }
  if (j + 2 < n) {
    sync();
    full(I3{}, T_{}, M_{}, j + 2);
  }
  if (n > 0) {
    switch (n & 3) {
      case 0: step(I0{}, F_{}, T_{}, F_{}, F_{}, n); break;
      case 1: step(I1{}, F_{}, T_{}, F_{}, F_{}, n); break;
      case 2: step(I2{}, F_{}, T_{}, F_{}, F_{}, n); break;
      default: step(I3{}, F_{}, T_{}, F_{}, F_{}, n); break;
    }
  }
  // no LDS DMA may still be in flight when the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

#pragma unroll
  for (int cb = 0; cb < NCB; ++cb) {
    if (!valid[cb]) continue;
    bf16* dst = a.dq + (hrow * a.hsq + pos[cb]) * D;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        bf16x4 r;
#pragma unroll
        for (int e = 0; e < 4; ++e) r[e] = (bf16)(dqt[cb][mb][4 * i4 + e] * a.scale);
        *(bf16x4*)(dst + 32 * mb + 8 * i4 + 4 * hi) = r;
      }
  }
}

// dq = bf16(scale * dqacc) for the rows of the problem (fused path): one thread
// per 8 channels of a row.
template <int D>
__global__ __launch_bounds__(256) void dq_convert_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;
  const size_t t = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = t / LPR;                   // (b Hq + h) Sq + i
  const int c = (int)(t % LPR);
  if (row >= (size_t)a.B * a.Hq * a.Sq) return;
  const size_t head = row / a.Sq;
  const size_t pos = row % a.Sq;
  const float* src = a.dqacc + (head * a.sqp + pos) * D + c * 8;
  const f32x4 x0 = *(const f32x4*)src, x1 = *(const f32x4*)(src + 4);
  const float s = a.scale;
  *(bf16x8*)(a.dq + (head * a.hsq + pos) * D + c * 8) =
      to_bf16x8(x0[0] * s, x0[1] * s, x0[2] * s, x0[3] * s, x1[0] * s, x1[1] * s, x1[2] * s, x1[3] * s);
}

struct WsLayout {
  size_t ld, dqacc, total;     // byte offsets of lse2/D and of the fused path's dQ sums; total bytes
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

WsLayout ws_layout(const Problem& p) {
  const size_t sqp = (size_t)((p.Sq + TILE_ROWS - 1) / TILE_ROWS) * TILE_ROWS;
  WsLayout w{};
  w.ld = 0;
  w.dqacc = align256((size_t)p.B * p.Hq * sqp * 2 * sizeof(float));
  w.total = w.dqacc + align256((size_t)p.B * p.Hq * sqp * p.d * sizeof(float));
  return w;
}

template <int D, bool CAUSAL, bool FUSED>
void launch_dkdv(const BwdArgs& a, hipStream_t s) {
  if (a.drop.thr != 0)
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, NoTable, true, FUSED>), dim3(a.total_kv), dim3(512), 0, s, a,
                       NoTable{});
  else
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL, NoTable, false, FUSED>), dim3(a.total_kv), dim3(512), 0, s, a,
                       NoTable{});
}

template <int D, bool CAUSAL>
void launch_dq(const BwdArgs& a, hipStream_t s) {
  if (a.drop.thr != 0)
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, NoTable, true>), dim3(a.total_q), dim3(256), 0, s, a, NoTable{});
  else
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL, NoTable, false>), dim3(a.total_q), dim3(256), 0, s, a, NoTable{});
}

template <int D>
hipError_t launch_bwd_d(BwdArgs& a, hipStream_t s, char* log, size_t log_n) {
  const size_t rows = (size_t)a.B * a.Hq * a.sqp;
  constexpr int RPB = 256 / (D / 8);
  const bool fused = a.dqacc != nullptr;
  hipError_t e = hipSuccess;
  if (fused && rows > 0) {
    timing_begin(s, "bwd_pre");
    hipLaunchKernelGGL((bwd_pre_kernel<D, NoTable>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s,
                       a, NoTable{});
    e = hipGetLastError();
    timing_end(s);
    if (e != hipSuccess) return e;
  }
  if (fused) {
    if (a.total_kv > 0) {
      timing_begin(s, "bwd_dkdvq");
      if (a.causal)
        launch_dkdv<D, true, true>(a, s);
      else
        launch_dkdv<D, false, true>(a, s);
      e = hipGetLastError();
      timing_end(s);
      if (e != hipSuccess) return e;
    }
    // with no key at all the sums stay at the zeros bwd_pre wrote: dq = 0
    const size_t threads = (size_t)a.B * a.Hq * a.Sq * (D / 8);
    timing_begin(s, "dq_convert");
    hipLaunchKernelGGL((dq_convert_kernel<D>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, a);
    e = hipGetLastError();
    timing_end(s);
    if (e != hipSuccess) return e;
    if (log != nullptr && log_n > 0)
      snprintf(log, log_n,
               "attn_bwd: bwd_pre<d=%d> grid=%zu (clears the dQ sums); "
               "bwd_dkdv<d=%d, fused dQ> grid=%d (128 keys x 32-row query tiles, 8 wavefronts, float32 atomic dQ); "
               "dq_convert<d=%d> grid=%zu",
               D, (rows + RPB - 1) / RPB, D, a.total_kv, D, (threads + 255) / 256);
    return hipSuccess;
  }
  // dQ first: it also writes the row terms (lse2, D) that the dK/dV pass reads
  if (a.total_q > 0) {
    timing_begin(s, "bwd_dq");
    if (a.causal)
      launch_dq<D, true>(a, s);
    else
      launch_dq<D, false>(a, s);
    e = hipGetLastError();
    timing_end(s);
    if (e != hipSuccess) return e;
  }
  if (a.total_kv > 0) {
    timing_begin(s, "bwd_dkdv");
    if (a.causal)
      launch_dkdv<D, true, false>(a, s);
    else
      launch_dkdv<D, false, false>(a, s);
    e = hipGetLastError();
    timing_end(s);
    if (e != hipSuccess) return e;
  }
  if (log != nullptr && log_n > 0)
    snprintf(log, log_n,
             "attn_bwd: bwd_dq<d=%d> grid=%d (%d rows x 32-key tiles; also the rows' lse2 and D); "
             "bwd_dkdv<d=%d> grid=%d (128 keys x 32-row query tiles, 8 wavefronts)",
             D, a.total_q, Q_WG, D, a.total_kv);
  return hipSuccess;
}

}  // namespace

size_t bwd_workspace_bytes(const Problem& p) { return ws_layout(p).dqacc; }
size_t bwd_fused_workspace_bytes(const Problem& p) { return ws_layout(p).total; }

hipError_t launch_bwd_bf16(const Problem& p, const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws,
                           bool fused, hipStream_t s, char* log, size_t log_n) {
  const WsLayout w = ws_layout(p);
  BwdArgs a{};
  a.dqacc = fused ? (float*)((char*)ws + w.dqacc) : nullptr;
  a.q = (const bf16*)q;
  a.k = (const bf16*)k;
  a.v = (const bf16*)v;
  a.o = (const bf16*)o;
  a.dout = (const bf16*)dout;
  a.lse = lse;
  a.dq = (bf16*)dq;
  a.dk = (bf16*)dk;
  a.dv = (bf16*)dv;
  a.ld = (float*)((char*)ws + w.ld);
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Sq = p.Sq;
  a.Sk = p.Sk;
  a.hsq = p.hsq;
  a.hsk = p.hsk;
  a.g = p.Hq / p.Hkv;
  a.causal = p.causal;
  a.sqp = (p.Sq + TILE_ROWS - 1) / TILE_ROWS * TILE_ROWS;
  a.scale = p.scale;
  a.c = p.scale * kLog2e;
  a.n_ktiles = (p.Sk + KV_WG - 1) / KV_WG;
  a.total_kv = p.B * p.Hkv * a.n_ktiles;
  a.n_qtiles = (p.Sq + Q_WG - 1) / Q_WG;
  a.total_q = p.B * p.Hq * a.n_qtiles;
  a.drop = p.drop;
  return p.d == 64 ? launch_bwd_d<64>(a, s, log, log_n) : launch_bwd_d<128>(a, s, log, log_n);
}

namespace {

template <int D>
hipError_t launch_bwd_packed_d(const BwdArgs& a, const SeqTable& Tkv, int gkv, const SeqTable& Tq, int gq,
                               hipStream_t s) {
  hipError_t e = hipSuccess;
  // dQ first: it also writes the row terms (lse2, D) that the dK/dV pass reads
  if (gq > 0) {
    timing_begin(s, "bwd_dq");
    if (a.causal)
      hipLaunchKernelGGL((bwd_dq_kernel<D, true, SeqTable, false>), dim3(gq), dim3(256), 0, s, a, Tq);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, false, SeqTable, false>), dim3(gq), dim3(256), 0, s, a, Tq);
    e = hipGetLastError();
    timing_end(s);
    if (e != hipSuccess) return e;
  }
  if (gkv > 0) {
    timing_begin(s, "bwd_dkdv");
    if (a.causal)
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, SeqTable, false, false>), dim3(gkv), dim3(512), 0, s, a, Tkv);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, SeqTable, false, false>), dim3(gkv), dim3(512), 0, s, a, Tkv);
    e = hipGetLastError();
    timing_end(s);
  }
  return e;
}

}  // namespace

size_t bwd_packed_workspace_bytes(const Problem& p, const SeqSpan* seqs, int n) {
  size_t rows = 0;
  for (int i = 0; i < n; ++i) rows += (size_t)((seqs[i].sq + TILE_ROWS - 1) / TILE_ROWS) * TILE_ROWS;
  return align256(rows * p.Hq * 2 * sizeof(float));
}

hipError_t launch_bwd_bf16_packed(const Problem& p, const SeqSpan* seqs, int n, const void* q, const void* k,
                                  const void* v, const void* o, const float* lse, const void* dout, void* dq,
                                  void* dk, void* dv, void* ws, hipStream_t s, char* log, size_t log_n) {
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
  a.ld = (float*)ws;
  a.B = 1;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.hsq = p.hsq;
  a.hsk = p.hsk;
  a.g = p.Hq / p.Hkv;
  a.causal = p.causal;
  a.scale = p.scale;
  a.c = p.scale * kLog2e;
  int nkv[SEQ_MAX], nq[SEQ_MAX], ld0[SEQ_MAX];
  int rows = 0;
  for (int i = 0; i < n; ++i) {
    const int sqp = (seqs[i].sq + TILE_ROWS - 1) / TILE_ROWS * TILE_ROWS;
    nkv[i] = (seqs[i].sk + KV_WG - 1) / KV_WG;
    nq[i] = (seqs[i].sq + Q_WG - 1) / Q_WG;
    ld0[i] = rows;
    rows += sqp;
  }
  SeqTable Tkv, Tq;
  const int gkv = build_seq_table(Tkv, seqs, n, p.Hkv, nkv, ld0);
  const int gq = build_seq_table(Tq, seqs, n, p.Hq, nq, ld0);
  if (log != nullptr && log_n > 0)
    snprintf(log, log_n,
             "bwd_dq<d=%d, packed> %d sequences grid=%d%s (also the rows' lse2 and D); "
             "bwd_dkdv<d=%d, packed> %d sequences grid=%d%s",
             p.d, Tq.n, gq, Tq.split8 ? " (per-XCD head split)" : "", p.d, Tkv.n, gkv,
             Tkv.split8 ? " (per-XCD head split)" : "");
  return p.d == 64 ? launch_bwd_packed_d<64>(a, Tkv, gkv, Tq, gq, s) : launch_bwd_packed_d<128>(a, Tkv, gkv, Tq, gq, s);
}

}  // namespace attn
