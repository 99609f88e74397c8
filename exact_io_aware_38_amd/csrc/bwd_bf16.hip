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
//  1. bwd_pre:   D_i = dO_i . O_i and lse2_i = lse_i * log2(e) (+inf for rows
//                that see no key and for padding rows, which makes every
//                rebuilt probability 0), packed per 32 rows;
//  2. transpose_rows (x3): Q^T, dO^T and K^T copies whose sequence index is
//                permuted inside groups of 16, so that every MFMA operand of
//                the two main kernels is one 16-byte LDS read;
//  3. bwd_dkdv:  one workgroup per (KV head, 128-key tile); loops over the
//                query heads that share the KV head and over 32-row query
//                tiles, accumulating dK^T and dV^T in registers (no atomics);
//  4. bwd_dq:    one workgroup per (query head, 128-row tile); loops over
//                32-key tiles, accumulating dQ^T in registers.
// The dK/dV and dQ passes both rebuild S and dP, which costs two GEMMs more
// than a single pass with atomic dQ but keeps the result deterministic.
//
// Mapping to CDNA4: the accumulators (dK^T and dV^T: 128 registers per lane
// at d = 128) plus the resident K/V fragments leave room for one wavefront per
// SIMD only, so the overlap of matrix and vector work comes from inside each
// wavefront: step j of the main loop interleaves, MFMA by MFMA, the score and
// dP products of tile j+1, the gradient products of tile j-1 and the
// elementwise work (P, dS) of tile j. Tiles arrive by LDS DMA three steps
// ahead of their first use, in rings sized so that no slot is rewritten while
// any wavefront still reads it.
#include "common.h"
#include "kernels.h"
#include "tiles.h"

#include <algorithm>
#include <cstdio>
#include <type_traits>

namespace attn {

namespace {

constexpr int BT = 32;        // rows of a pipeline tile (queries for dK/dV, keys for dQ)
constexpr int KV_WG = 128;    // keys per dK/dV workgroup (4 wavefronts x 32)
constexpr int Q_WG = 128;     // queries per dQ workgroup

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
  float* ld;      // [B, Hq, sqp / 32][64]: lse2 of 32 rows, then D of the same rows
  bf16* qt;       // [B, Hq, D, sqp]
  bf16* dot;      // [B, Hq, D, sqp]
  bf16* kt;       // [B, Hkv, D, skp]
  int B, Hq, Hkv, Sq, Sk, g, causal;
  int sqp, skp;   // Sq, Sk rounded up to 64
  float scale;
  float c;        // scale * log2(e)
  int n_ktiles, total_kv;
  int n_qtiles, total_q;
};

// Workgroup order: the 8 XCDs each receive a contiguous range of logical ids
// (xcd_logical_id), i.e. whole heads, whose tiles then share that XCD's L2.
// Inside the range, when it holds whole heads, the tile index varies slowest
// so that the longest causal tiles of all its heads start first.
__device__ __forceinline__ void wg_coords(int total, int tiles, int& tile, int& head) {
  const int W = xcd_logical_id(blockIdx.x, total);
  if ((total & 7) == 0) {
    const int R = total >> 3;
    if (R % tiles == 0) {
      const int nh = R / tiles;
      const int x = W / R, s = W % R;
      tile = s / nh;
      head = x * nh + s % nh;
      return;
    }
  }
  tile = W % tiles;
  head = W / tiles;
}

// 16-byte MFMA operand fragment of a 32-row LDS tile with D columns (rows of
// 2D bytes, chunks permuted by chunk_swizzle).
template <int D>
__device__ __forceinline__ bf16x8 row_frag(const char* tile, int row, int chunk) {
  return *(const bf16x8*)(tile + row * (2 * D) + ((chunk ^ chunk_swizzle<D>(row)) << 4));
}

// 16-byte fragment of a transposed tile: D rows of 32 sequence positions
// (64 bytes), chunks permuted by (row >> 2) & 3, which makes 16 consecutive
// rows at one logical chunk hit 16 distinct bank groups.
__device__ __forceinline__ int tr_swizzle(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ bf16x8 tr_frag(const char* tile, int row, int chunk) {
  return *(const bf16x8*)(tile + row * 64 + ((chunk ^ tr_swizzle(row)) << 4));
}

template <int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;       // lanes per row, 8 elements each
  constexpr int RPB = 256 / LPR;   // rows per block
  const size_t rows = (size_t)a.B * a.Hq * a.sqp;
  const size_t prow = (size_t)blockIdx.x * RPB + threadIdx.x / LPR;   // padded row
  const int c = threadIdx.x % LPR;
  const size_t head = prow / a.sqp;
  const int pos = (int)(prow % a.sqp);
  const bool valid = prow < rows && pos < a.Sq;
  const size_t row = head * a.Sq + pos;
  float acc = 0.f;
  if (valid) {
    const bf16x8 ov = *(const bf16x8*)(a.o + row * D + c * 8);
    const bf16x8 dv = *(const bf16x8*)(a.dout + row * D + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)ov[e], (float)dv[e], acc);
  }
#pragma unroll
  for (int s = LPR / 2; s > 0; s >>= 1) acc += __shfl_xor(acc, s);
  if (prow < rows && c == 0) {
    float l2 = __builtin_huge_valf(), dl = 0.f;
    if (valid) {
      const float l = a.lse[row];
      l2 = (l == kNegInf) ? __builtin_huge_valf() : l * kLog2e;
      dl = acc;
    }
    float* blk = a.ld + (head * (a.sqp / BT) + pos / BT) * (2 * BT);
    blk[pos % BT] = l2;
    blk[BT + pos % BT] = dl;
  }
}

// ---------------------------------------------------------------------------
// dK, dV. Wavefront w owns keys k0 + 32w .. +31 as MFMA columns: S = Q K^T and
// dP = dO V^T (rows = 32 queries) take K and V from registers; dV^T += dO^T P
// and dK^T += Q^T dS (rows = d) take P and dS straight from the score
// accumulators, which already have the B-operand layout.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int DC = D / 16;
  constexpr int MB = D / 32;
  constexpr int NOPS = 2 * DC;                  // MFMAs per product group per step (= 4 * MB)
  constexpr int CPR = D / 8;                    // 16-byte chunks per row
  constexpr int TB = BT * D * 2;                // bytes of a 32-row tile, row-major or transposed
  constexpr int INSTR = TB / 4096;              // DMA instructions per wavefront per tensor
  constexpr int NDMA = 4 * INSTR + 1;           // ... per tile: Q, dO, Q^T, dO^T, lse2/D
  constexpr int NQ = 3, NT = 5, NL = 4;         // ring slots
  constexpr int T_OFF = NQ * 2 * TB;
  constexpr int L_OFF = T_OFF + NT * 2 * TB;
  static_assert(NOPS >= NDMA, "one DMA per step at most");
  __shared__ __attribute__((aligned(1024))) char smem[L_OFF + NL * 2 * BT * 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int off = (a.causal == 2) ? (a.Sk - a.Sq) : 0;

  int kt, bh;
  wg_coords(a.total_kv, a.n_ktiles, kt, bh);
  const int hkv = bh % a.Hkv;
  const int b = bh / a.Hkv;
  const int k0 = kt * KV_WG;
  const int kw0 = k0 + 32 * wid;
  const int key = kw0 + l32;
  const bool kvalid = key < a.Sk;

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
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) {
      kf[dc] = settle(kf[dc]);
      vf[dc] = settle(vf[dc]);
    }
  }

  const int n_qt = (a.Sq + BT - 1) / BT;
  const int qt_lo = a.causal ? min(n_qt, max(0, k0 - off) / BT) : 0;
  const int per_head = n_qt - qt_lo;
  const int n = a.g * per_head;                 // pipeline tiles: (query head, 32-row tile)

  // Per-lane DMA geometry of instruction i: LDS chunk P = (wid*INSTR + i)*64 + lane
  // of a tile; row-major tile: row P / CPR, physical chunk P % CPR; transposed
  // tile: row P / 4, physical chunk P % 4; each lane loads the logical chunk.
  // Byte offsets are relative to the head's base (32-bit: a head is < 4 GiB).
  int rrow[INSTR];
  uint32_t rcol[INSTR], toff[INSTR];
#pragma unroll
  for (int i = 0; i < INSTR; ++i) {
    const int P = (wid * INSTR + i) * 64 + lane;
    rrow[i] = P / CPR;
    rcol[i] = ((P % CPR) ^ chunk_swizzle<D>(rrow[i])) * 16;
    const int tr = P / 4;
    toff[i] = (uint32_t)(tr * a.sqp + ((P & 3) ^ tr_swizzle(tr)) * 8) * 2;
  }
  auto tile_head = [&](int t) { return hkv * a.g + t / per_head; };
  auto tile_q0 = [&](int t) { return (qt_lo + t % per_head) * BT; };
  // DMA instruction qi (0 .. NDMA-1) of tile t into ring slots of tile ts
  // (ts >= t: past the last tile the last one is loaded again into slots
  // nobody reads, which keeps the per-step DMA count uniform)
  auto issue_one = [&](int ts, int hq, int q0, int qi) {
    const size_t hrow = (size_t)b * a.Hq + hq;
    if (qi < 2 * INSTR) {                       // Q (qi < INSTR) or dO rows; rows past Sq repeat row Sq-1
      const int i = qi % INSTR;
      const bf16* src = ((qi < INSTR) ? a.q : a.dout) + hrow * a.Sq * D;
      const uint32_t r = (uint32_t)min(q0 + rrow[i], a.Sq - 1);
      dma16s(src, r * (2 * D) + rcol[i],
             (lds_void*)(smem + (ts % NQ) * 2 * TB + (qi / INSTR) * TB + (wid * INSTR + i) * 1024));
    } else if (qi < 4 * INSTR) {                // Q^T or dO^T (zero past Sq)
      const int i = qi % INSTR;
      const bf16* src = ((qi < 3 * INSTR) ? a.qt : a.dot) + hrow * D * a.sqp + q0;
      dma16s(src, toff[i],
             (lds_void*)(smem + T_OFF + (ts % NT) * 2 * TB + ((qi - 2 * INSTR) / INSTR) * TB +
                         (wid * INSTR + i) * 1024));
    } else {                                    // lse2 and D of the 32 rows (every wavefront, same bytes)
      dma4s(a.ld + (hrow * (a.sqp / BT) + q0 / BT) * (2 * BT), lane * 4,
            (lds_void*)(smem + L_OFF + (ts % NL) * 2 * BT * 4));
    }
  };
  auto issue = [&](int t) {
    const int hq = tile_head(t), q0 = tile_q0(t);
#pragma unroll
    for (int qi = 0; qi < NDMA; ++qi) issue_one(t, hq, q0, qi);
  };

  f32x16 dkt[MB], dvt[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    dkt[mb] = f32x16{};
    dvt[mb] = f32x16{};
  }
  f32x16 s_[2], dp_[2];                         // scores and dP of two tiles in flight
  bf16x8 pf[2][2], dsf[2][2];                   // [tile parity][16-query chunk]

  // MFMA op k (0 .. NOPS-1) of the score group of the tile in ring slot sq:
  // S (even k) or dP (odd k) over d-chunk k / 2.
  auto g1_frag = [&](const char* sq, int k) {
    return row_frag<D>(sq + (k & 1) * TB, l32, 2 * (k >> 1) + hi);
  };
  // MFMA op k of the gradient group: chain k % (2 MB) (dV^T for < MB, dK^T
  // otherwise, d-block k % MB), 16-query chunk k / (2 MB).
  auto g2_frag = [&](const char* st, int k) {
    const int ch = k % (2 * MB);
    const int qc = k / (2 * MB);
    const int d = 32 * (ch % MB) + l32;
    return tr_frag(st + (ch < MB ? TB : 0), d, 2 * qc + hi);   // dO^T for dV, Q^T for dK
  };

  auto step = [&](auto par, auto g1, auto g2, auto ew, int j) {
    constexpr int P = decltype(par)::value;     // parity of tile j
    constexpr bool G1 = decltype(g1)::value;    // scores of tile j+1
    constexpr bool G2 = decltype(g2)::value;    // gradients of tile j-1
    constexpr bool EW = decltype(ew)::value;    // P, dS of tile j
    const char* sq = smem + ((j + 1) % NQ) * 2 * TB;
    const char* st = smem + T_OFF + ((j + NT - 1) % NT) * 2 * TB;
    const float* sl = (const float*)(smem + L_OFF + (j % NL) * 2 * BT * 4);
    const int t3 = j + 3;
    const int t3c = min(t3, n - 1);
    const int hq3 = tile_head(t3c);
    const int q03 = tile_q0(t3c);
    const int q0 = tile_q0(j);
    const bool need_mask = a.causal && (kw0 + 31 > q0 + off);

    f32x4 l2v[4], dlv[4];
    if constexpr (EW) {
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        l2v[i4] = *(const f32x4*)(sl + 8 * i4 + 4 * hi);
        dlv[i4] = *(const f32x4*)(sl + BT + 8 * i4 + 4 * hi);
      }
    }
    if constexpr (G1) s_[P ^ 1] = dp_[P ^ 1] = f32x16{};
    bf16x8 f1[3], f2[3];
    if constexpr (G1) {
      f1[0] = g1_frag(sq, 0);
      f1[1] = g1_frag(sq, 1);
    }
    if constexpr (G2) {
      f2[0] = g2_frag(st, 0);
      f2[1] = g2_frag(st, 1);
    }
    float pt[8], dt[8];
#pragma unroll
    for (int i = 0; i < NOPS; ++i) {
      if (i + 2 < NOPS) {
        if constexpr (G1) f1[(i + 2) % 3] = g1_frag(sq, i + 2);
        if constexpr (G2) f2[(i + 2) % 3] = g2_frag(st, i + 2);
      }
      __builtin_amdgcn_sched_barrier(0);        // keep the reads two MFMAs ahead of their use
      if constexpr (G1) {
        if (i & 1)
          dp_[P ^ 1] = mfma32(f1[i % 3], vf[i >> 1], dp_[P ^ 1]);
        else
          s_[P ^ 1] = mfma32(f1[i % 3], kf[i >> 1], s_[P ^ 1]);
      }
      if constexpr (G2) {
        const int ch = i % (2 * MB);
        const int qc = i / (2 * MB);
        if (ch < MB)
          dvt[ch] = mfma32(f2[i % 3], pf[P ^ 1][qc], dvt[ch]);
        else
          dkt[ch - MB] = mfma32(f2[i % 3], dsf[P ^ 1][qc], dkt[ch - MB]);
      }
      if constexpr (EW) {
        // values [v0, v1) of the 16 score registers; the first step only reads lse2 / D
        const int v0 = i == 0 ? 0 : ((i - 1) * 16) / (NOPS - 1);
        const int v1 = i == 0 ? 0 : (i * 16) / (NOPS - 1);
#pragma unroll
        for (int v = v0; v < v1; ++v) {
          const float l2 = l2v[v >> 2][v & 3];
          const float dl = dlv[v >> 2][v & 3];
          float p = fast_exp2(__builtin_fmaf(s_[P][v], a.c, -l2));
          if (need_mask && key > q0 + 8 * (v >> 2) + 4 * hi + (v & 3) + off) p = 0.f;
          pt[v & 7] = p;
          dt[v & 7] = p * (dp_[P][v] - dl);
          if ((v & 7) == 7) {
            pf[P][v >> 3] = to_bf16x8(pt[0], pt[1], pt[2], pt[3], pt[4], pt[5], pt[6], pt[7]);
            dsf[P][v >> 3] = to_bf16x8(dt[0], dt[1], dt[2], dt[3], dt[4], dt[5], dt[6], dt[7]);
          }
        }
      }
      if (i < NDMA && G1) issue_one(t3, hq3, q03, i);
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  // tiles 0 and 1 now; tile j+3 during step j (tile 2 during the scores of
  // tile 0). Every step that computes scores issues exactly NDMA DMA
  // instructions, so "all but the last NDMA" always means "the next tile".
  if (n > 0) {
    issue(0);
    issue(min(1, n - 1));
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NDMA) : "memory");
    // scores of tile 0 (parity 0): a step of parity 1 with only the score group
    step(P1{}, T_{}, F_{}, F_{}, -1);
  }
  // step j: tile j+1 has landed for every wavefront (each waits for its own
  // DMA, the barrier for all of them), and every wavefront is done with step j-1
  auto sync = [&](int j) {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NDMA) : "memory");
  };
  if (n > 0) {
    sync(0);
    step(P0{}, T_{}, F_{}, T_{}, 0);
  }
  int j = 1;
  for (; j + 1 < n; j += 2) {
    sync(j);
    step(P1{}, T_{}, T_{}, T_{}, j);
    sync(j + 1);
    step(P0{}, T_{}, T_{}, T_{}, j + 1);
  }
  if (j < n) {
    sync(j);
    step(P1{}, T_{}, T_{}, T_{}, j);
    ++j;
  }
  // gradients of the last tile: a step of parity n with only the gradient group
  if (n > 0) {
    if (n & 1)
      step(P1{}, F_{}, T_{}, F_{}, n);
    else
      step(P0{}, F_{}, T_{}, F_{}, n);
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

// ---------------------------------------------------------------------------
// dQ. Wavefront w owns queries p + 32w .. +31 as MFMA columns: S^T = K Q^T and
// dP^T = V dO^T (rows = 32 keys) take Q and dO from registers; dQ^T += K^T dS^T
// (rows = d) takes dS^T from the score accumulators.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void bwd_dq_kernel(BwdArgs a) {
  constexpr int DC = D / 16;
  constexpr int MB = D / 32;
  constexpr int NS = MB * 2;                    // steps: 2 score MFMAs + 1 gradient MFMA each
  constexpr int CPR = D / 8;
  constexpr int TB = BT * D * 2;
  constexpr int INSTR = TB / 4096;
  constexpr int NDMA = 3 * INSTR;               // K, V, K^T
  constexpr int NKV = 3, NT = 5;
  constexpr int T_OFF = NKV * 2 * TB;
  static_assert(NS >= NDMA, "one DMA per step at most");
  __shared__ __attribute__((aligned(1024))) char smem[T_OFF + NT * TB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const int off = (a.causal == 2) ? (a.Sk - a.Sq) : 0;

  int qtile, bh;
  wg_coords(a.total_q, a.n_qtiles, qtile, bh);
  const int qb = a.n_qtiles - 1 - qtile;        // longest causal tiles first
  const int hq = bh % a.Hq;
  const int b = bh / a.Hq;
  const int hkv = hq / a.g;
  const int p0 = qb * Q_WG + 32 * wid;
  const int pos = p0 + l32;
  const bool valid = pos < a.Sq;
  const int wg_last = min(qb * Q_WG + Q_WG, a.Sq) - 1;
  int kend = a.causal ? min(a.Sk, wg_last + off + 1) : a.Sk;
  if (kend < 0) kend = 0;
  const int n = (kend + BT - 1) / BT;
  const int mask_from = a.causal ? max(0, min(kend, p0 + off + 1)) : kend;
  const int lim = a.causal ? min(kend - 1, pos + off) : kend - 1;

  const size_t hrow = (size_t)b * a.Hq + hq;
  const size_t qrow = hrow * a.Sq + (valid ? pos : 0);
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
  float l2 = __builtin_huge_valf(), dl = 0.f;
  if (valid) {
    const float* blk = a.ld + (hrow * (a.sqp / BT) + pos / BT) * (2 * BT);
    l2 = blk[pos % BT];
    dl = blk[BT + pos % BT];
  }
#pragma unroll
  for (int dc = 0; dc < DC; ++dc) {
    qf[dc] = settle(qf[dc]);
    df[dc] = settle(df[dc]);
  }
  l2 = settle(l2);
  dl = settle(dl);

  const bf16* kg = a.k + ((size_t)b * a.Hkv + hkv) * (size_t)a.Sk * D;
  const bf16* vg = a.v + ((size_t)b * a.Hkv + hkv) * (size_t)a.Sk * D;
  const bf16* ktg = a.kt + ((size_t)b * a.Hkv + hkv) * (size_t)D * a.skp;
  int rrow[INSTR];
  uint32_t rcol[INSTR], toff[INSTR];
#pragma unroll
  for (int i = 0; i < INSTR; ++i) {
    const int P = (wid * INSTR + i) * 64 + lane;
    rrow[i] = P / CPR;
    rcol[i] = ((P % CPR) ^ chunk_swizzle<D>(rrow[i])) * 16;
    const int tr = P / 4;
    toff[i] = (uint32_t)(tr * a.skp + ((P & 3) ^ tr_swizzle(tr)) * 8) * 2;
  }
  // DMA instruction qi (0 .. NDMA-1) of tile t (K rows, V rows, K^T) into the
  // ring slots of tile ts (ts > t only past the last tile: see the dK/dV pass)
  auto issue_one = [&](int ts, int t, int qi) {
    const int key0 = t * BT;
    const int i = qi % INSTR;
    if (qi < 2 * INSTR) {                       // rows past kend repeat row kend-1 (their P is masked to 0)
      const bf16* src = (qi < INSTR) ? kg : vg;
      const uint32_t r = (uint32_t)min(key0 + rrow[i], kend - 1);
      dma16s(src, r * (2 * D) + rcol[i],
             (lds_void*)(smem + (ts % NKV) * 2 * TB + (qi / INSTR) * TB + (wid * INSTR + i) * 1024));
    } else {
      dma16s(ktg + key0, toff[i], (lds_void*)(smem + T_OFF + (ts % NT) * TB + (wid * INSTR + i) * 1024));
    }
  };
  auto issue = [&](int t) {
#pragma unroll
    for (int qi = 0; qi < NDMA; ++qi) issue_one(t, t, qi);
  };

  f32x16 dqt[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) dqt[mb] = f32x16{};
  f32x16 s_[2], dp_[2];
  bf16x8 dsf[2][2];                             // [tile parity][16-key chunk]

  // score op k (0 .. 2 DC - 1): S^T (even k) or dP^T (odd k) over d-chunk k / 2
  auto g1_frag = [&](const char* skv, int k) {
    return row_frag<D>(skv + (k & 1) * TB, l32, 2 * (k >> 1) + hi);
  };
  // gradient op k (0 .. 2 MB - 1): d-block k % MB, 16-key chunk k / MB
  auto g2_frag = [&](const char* st, int k) {
    const int d = 32 * (k % MB) + l32;
    return tr_frag(st, d, 2 * (k / MB) + hi);
  };

  auto step = [&](auto par, auto g1, auto g2, auto ew, int j) {
    constexpr int P = decltype(par)::value;
    constexpr bool G1 = decltype(g1)::value;
    constexpr bool G2 = decltype(g2)::value;
    constexpr bool EW = decltype(ew)::value;
    const char* skv = smem + ((j + 1) % NKV) * 2 * TB;
    const char* st = smem + T_OFF + ((j + NT - 1) % NT) * TB;
    const int t3 = j + 3;
    const int t3c = min(t3, n - 1);
    const int key0 = j * BT;
    const bool need_mask = key0 + BT > mask_from;
    if constexpr (G1) s_[P ^ 1] = dp_[P ^ 1] = f32x16{};
    bf16x8 f1[3], f2[2];
    if constexpr (G1) {
      f1[0] = g1_frag(skv, 0);
      f1[1] = g1_frag(skv, 1);
    }
    if constexpr (G2) f2[0] = g2_frag(st, 0);
    float dt[8];
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      // reads for the next step: score ops 2i+2, 2i+3, gradient op i+1
      if constexpr (G1) {
        if (2 * i + 2 < 2 * DC) f1[(2 * i + 2) % 3] = g1_frag(skv, 2 * i + 2);
      }
      if constexpr (G2) {
        if (i + 1 < NS) f2[(i + 1) & 1] = g2_frag(st, i + 1);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int k = 2 * i + u;
        if constexpr (G1) {
          if (k & 1)
            dp_[P ^ 1] = mfma32(f1[k % 3], df[k >> 1], dp_[P ^ 1]);
          else
            s_[P ^ 1] = mfma32(f1[k % 3], qf[k >> 1], s_[P ^ 1]);
        }
        if (u == 0) {
          if constexpr (G2) dqt[i % MB] = mfma32(f2[i & 1], dsf[P ^ 1][i / MB], dqt[i % MB]);
        }
        if (u == 0) {
          if constexpr (G1) {
            if (2 * i + 3 < 2 * DC) f1[(2 * i + 3) % 3] = g1_frag(skv, 2 * i + 3);
          }
        }
      }
      if constexpr (EW) {
        const int v0 = (i * 16) / NS;
        const int v1 = ((i + 1) * 16) / NS;
#pragma unroll
        for (int v = v0; v < v1; ++v) {
          float p = fast_exp2(__builtin_fmaf(s_[P][v], a.c, -l2));
          if (need_mask && key0 + 8 * (v >> 2) + 4 * hi + (v & 3) > lim) p = 0.f;
          dt[v & 7] = p * (dp_[P][v] - dl);
          if ((v & 7) == 7)
            dsf[P][v >> 3] = to_bf16x8(dt[0], dt[1], dt[2], dt[3], dt[4], dt[5], dt[6], dt[7]);
        }
      }
      if (i < NDMA && G1) issue_one(t3, t3c, i);
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using P0 = std::integral_constant<int, 0>;
  using P1 = std::integral_constant<int, 1>;

  // tiles 0 and 1 now; tile j+3 during step j (tile 2 during the scores of
  // tile 0). Every step that computes scores issues exactly NDMA DMA
  // instructions, so "all but the last NDMA" always means "the next tile".
  if (n > 0) {
    issue(0);
    issue(min(1, n - 1));
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NDMA) : "memory");
    step(P1{}, T_{}, F_{}, F_{}, -1);
  }
  auto sync = [&](int j) {
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NDMA) : "memory");
  };
  if (n > 0) {
    sync(0);
    step(P0{}, T_{}, F_{}, T_{}, 0);
  }
  int j = 1;
  for (; j + 1 < n; j += 2) {
    sync(j);
    step(P1{}, T_{}, T_{}, T_{}, j);
    sync(j + 1);
    step(P0{}, T_{}, T_{}, T_{}, j + 1);
  }
  if (j < n) {
    sync(j);
    step(P1{}, T_{}, T_{}, T_{}, j);
  }
  if (n > 0) {
    if (n & 1)
      step(P1{}, F_{}, T_{}, F_{}, n);
    else
      step(P0{}, F_{}, T_{}, F_{}, n);
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

struct WsLayout {
  size_t ld, qt, dot, kt, total;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

WsLayout ws_layout(const Problem& p) {
  const size_t sqp = (size_t)((p.Sq + TILE_ROWS - 1) / TILE_ROWS) * TILE_ROWS;
  const size_t skp = (size_t)((p.Sk + TILE_ROWS - 1) / TILE_ROWS) * TILE_ROWS;
  WsLayout w{};
  w.ld = 0;
  w.qt = align256((size_t)p.B * p.Hq * sqp * 2 * sizeof(float));
  w.dot = w.qt + align256((size_t)p.B * p.Hq * p.d * sqp * 2);
  w.kt = w.dot + align256((size_t)p.B * p.Hq * p.d * sqp * 2);
  w.total = w.kt + align256((size_t)p.B * p.Hkv * p.d * skp * 2);
  return w;
}

template <int D>
hipError_t launch_bwd_d(BwdArgs& a, hipStream_t s, char* log, size_t log_n) {
  const size_t rows = (size_t)a.B * a.Hq * a.sqp;
  constexpr int RPB = 256 / (D / 8);
  hipError_t e = hipSuccess;
  if (rows > 0) {
    timing_begin(s, "bwd_pre");
    hipLaunchKernelGGL((bwd_pre_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, s, a);
    e = hipGetLastError();
    timing_end(s);
    if (e != hipSuccess) return e;
    timing_begin(s, "bwd_transpose");
    hipLaunchKernelGGL((transpose_rows_kernel<D>), dim3(a.sqp / TILE_ROWS, a.Hq, a.B), dim3(256), 0, s,
                       a.q, a.qt, a.Hq, a.Sq, a.sqp);
    hipLaunchKernelGGL((transpose_rows_kernel<D>), dim3(a.sqp / TILE_ROWS, a.Hq, a.B), dim3(256), 0, s,
                       a.dout, a.dot, a.Hq, a.Sq, a.sqp);
    e = hipGetLastError();
    timing_end(s);
    if (e != hipSuccess) return e;
  }
  if (a.skp > 0) {
    timing_begin(s, "bwd_transpose");
    hipLaunchKernelGGL((transpose_rows_kernel<D>), dim3(a.skp / TILE_ROWS, a.Hkv, a.B), dim3(256), 0, s,
                       a.k, a.kt, a.Hkv, a.Sk, a.skp);
    e = hipGetLastError();
    timing_end(s);
    if (e != hipSuccess) return e;
  }
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
             "attn_bwd: bwd_pre<d=%d> grid=%zu; transpose_rows<d=%d> x3 (Q^T, dO^T, K^T); "
             "bwd_dkdv<d=%d> grid=%d (128 keys x 32-row query tiles); "
             "bwd_dq<d=%d> grid=%d (128 rows x 32-key tiles)",
             D, (rows + RPB - 1) / RPB, D, D, a.total_kv, D, a.total_q);
  return hipSuccess;
}

}  // namespace

size_t bwd_workspace_bytes(const Problem& p) { return ws_layout(p).total; }

hipError_t launch_bwd_bf16(const Problem& p, const void* q, const void* k, const void* v, const void* o,
                           const float* lse, const void* dout, void* dq, void* dk, void* dv, void* ws,
                           hipStream_t s, char* log, size_t log_n) {
  const WsLayout w = ws_layout(p);
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
  a.ld = (float*)((char*)ws + w.ld);
  a.qt = (bf16*)((char*)ws + w.qt);
  a.dot = (bf16*)((char*)ws + w.dot);
  a.kt = (bf16*)((char*)ws + w.kt);
  a.B = p.B;
  a.Hq = p.Hq;
  a.Hkv = p.Hkv;
  a.Sq = p.Sq;
  a.Sk = p.Sk;
  a.g = p.Hq / p.Hkv;
  a.causal = p.causal;
  a.sqp = (p.Sq + TILE_ROWS - 1) / TILE_ROWS * TILE_ROWS;
  a.skp = (p.Sk + TILE_ROWS - 1) / TILE_ROWS * TILE_ROWS;
  a.scale = p.scale;
  a.c = p.scale * kLog2e;
  a.n_ktiles = (p.Sk + KV_WG - 1) / KV_WG;
  a.total_kv = p.B * p.Hkv * a.n_ktiles;
  a.n_qtiles = (p.Sq + Q_WG - 1) / Q_WG;
  a.total_q = p.B * p.Hq * a.n_qtiles;
  return p.d == 64 ? launch_bwd_d<64>(a, s, log, log_n) : launch_bwd_d<128>(a, s, log, log_n);
}

}  // namespace attn
