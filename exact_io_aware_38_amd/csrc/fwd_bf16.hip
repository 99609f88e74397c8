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
// Without dropout the row max itself is formed only where it can matter: at
// the first tile, and where a lane's probabilities against the current
// reference sum to more than 2^RESCALE_T.
//
// Mapping to CDNA4:
//  * a wavefront owns 32 query rows as MFMA columns and computes the transposed
//    score tile S^T = K Q^T (rows = keys), so every lane holds the scores of one
//    query row: the row max and sum reduce inside the lane plus one swap between
//    lane halves, and the probabilities already sit in the B-operand layout of
//    O^T = V^T P^T;
//  * K and V tiles (64 keys, row-major, 16-byte chunks XOR-swizzled per row)
//    go HBM -> LDS through the LDS DMA path of buffer loads into a 4-stage
//    ring, issued two tiles ahead; the V^T operand of O^T = V^T P^T comes
//    from transposing LDS reads (ds_read_b64_tr_b16) of the row-major V
//    tile, which the swizzle keeps free of bank conflicts;
//  * two wavefronts share each SIMD and run the per-tile steps in opposite
//    orders so that one's softmax (vector ALU) overlaps the other's MFMAs;
//    the main loop is compiled once per order, so each keeps its scores in
//    the registers its MFMAs write;
//  * exp2 with log2(e) folded into the score scale: one FMA and one v_exp_f32
//    per score;
//  * each XCD takes whole heads and starts the longest causal query tiles of
//    all of them first (xcd_tile_order), so the launch ends on short tiles.
#include "common.h"
#include "kernels.h"
#include "tiles.h"

#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>

// Scratch of attn_fwd_noalloc: the split path's per-slice partials for
// callers that cannot allocate device memory. Every GPU the library runs on
// holds its own copy of this array until the process ends; host code never
// passes the array's name to a kernel (in host code it is only a handle), but
// the device address that hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[attn::NOALLOC_SCRATCH_BYTES];

namespace attn {

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

namespace {

constexpr float RESCALE_T = 8.0f;   // log2 units
constexpr float kRescaleSum = 256.0f;   // 2^RESCALE_T
constexpr int BC = 64;               // keys per tile

struct FwdArgs {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  bf16* o;
  float* lse;
  float* part_o;     // split path: [nsplit, B, Hq, Sq, D]
  float* part_lse;   // split path: [nsplit, B, Hq, Sq]
  int B, Hq, Hkv, Sq, Sk, g, causal;
  int hsq, hsk;      // head strides in rows (see Problem)
  float c;           // scale * log2(e)
  int hw, n_hgroups, rows_per_wg, n_ptiles, total_wgs;
  int nsplit, split_keys;
  DropParams drop;
};

// ---------------------------------------------------------------------------
// Prefill: 8 wavefronts (two per SIMD) x 32 query rows per workgroup.
// Phase A wavefronts do S(j), P(j-1)V(j-1), softmax(j) per step; phase B
// wavefronts do softmax(j-1), P(j-1)V(j-1), S(j).
// ---------------------------------------------------------------------------
template <int D>
struct Ring {
  static constexpr int TILE = BC * D * 2;       // bytes of one K or V tile
  static constexpr int STAGE = 2 * TILE;        // K then V
  static constexpr int NSTAGE = 4;
  static constexpr int INSTR = D / 64;          // DMA instructions per wavefront per tensor per tile
};

// Sequence s of a packed launch as a problem of batch 1: lengths and data
// pointers from the table (the head strides stay the packed totals).
template <int D>
__device__ __forceinline__ void rebase(FwdArgs& a, const SeqTable& T, int s) {
  a.Sq = T.sq[s];
  a.Sk = T.sk[s];
  const size_t qo = (size_t)T.q0[s] * D, ko = (size_t)T.k0[s] * D;
  a.q += qo;
  a.o += qo;
  if (a.lse != nullptr) a.lse += T.q0[s];
  a.k += ko;
  a.v += ko;
}

// Tab: NoTable for one dense [B, H, S, d] problem, SeqTable for a packed launch.
// DROP: dropout on the probabilities that multiply V (the denominator counts
// every visible key, as without dropout). POLY > 0: every POLY-th probability
// of a lane is formed by poly_exp2 on the FMA pipe instead of v_exp_f32 (an
// opt-in variant, ATTN_EXP2_POLY; slower on this chip, kept to measure it).
template <int D, typename Tab, bool DROP, int POLY = 0>
__global__ __launch_bounds__(512) void fwd_prefill_kernel(FwdArgs a, Tab T) {
  using R = Ring<D>;
  constexpr int MB = D / 32;
  constexpr int DC = D / 16;
  constexpr int CPR = D / 8;                    // 16-byte chunks per K row
  constexpr int RB = 2 * D;                     // bytes per K row
  constexpr int NP = 2 * DC;                    // MFMA pairs per step (= 4 * MB for the PV half)
  constexpr int NDMA = 2 * R::INSTR;            // DMA instructions per wavefront per step
  static_assert(R::NSTAGE == 4, "the main loop is unrolled by the ring size");

  __shared__ __attribute__((aligned(1024))) char smem[R::NSTAGE * R::STAGE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hi = lane >> 5;
  const bool phase_b = wid >= 4;

  int ptile, hgrp, hkv, b;                      // longest causal tiles first
  if constexpr (std::is_same_v<Tab, SeqTable>) {
    const SeqCoord c = seq_coord(T);
    rebase<D>(a, T, c.seq);
    ptile = T.ntile[c.seq] - 1 - c.t;
    hgrp = c.unit % a.n_hgroups;
    hkv = c.unit / a.n_hgroups;
    b = 0;
  } else {
    int t, rest;
    xcd_tile_order(a.total_wgs, a.n_ptiles, t, rest);
    ptile = a.n_ptiles - 1 - t;
    hgrp = rest % a.n_hgroups;
    rest /= a.n_hgroups;
    hkv = rest % a.Hkv;
    b = rest / a.Hkv;
  }
  const int off = (a.causal == 2) ? (a.Sk - a.Sq) : 0;
  // the two phases take alternating 32-row blocks, which keeps their causal work equal
  const int slot = (wid & 3) * 2 + (wid >> 2);
  const int head = hkv * a.g + hgrp * a.hw + slot % a.hw;
  // (batch, query head) index, wave-uniform: one scalar register carries it
  // from the Q load to the epilogue
  const int bh = __builtin_amdgcn_readfirstlane(b * a.Hq + head);
  const int p0 = ptile * a.rows_per_wg + 32 * (slot / a.hw);
  const int pos = p0 + l32;
  const bool colv = pos < a.Sq;
  const int wg_last = min((ptile + 1) * a.rows_per_wg, a.Sq) - 1;
  int kend = a.causal ? min(a.Sk, wg_last + off + 1) : a.Sk;
  if (kend < 0) kend = 0;
  const int ntiles = (kend + BC - 1) / BC;
  const int mask_from = a.causal ? max(0, min(kend, p0 + off + 1)) : kend;
  const int lim = a.causal ? min(kend - 1, pos + off) : kend - 1;

  bf16x8 qf[DC];
  {
    const bf16* qp = a.q + ((size_t)bh * a.hsq + (colv ? pos : 0)) * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      qf[dc] = colv ? *(const bf16x8*)(qp + 16 * dc + 8 * hi) : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
    // Re-define the fragments after they arrived: the compiler then knows no
    // load is pending on them inside the loop, where a wait on the memory
    // counter would also wait for the K/V prefetch in flight.
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qf[dc] = settle(qf[dc]);
  }
  const size_t kvh = ((size_t)b * a.Hkv + hkv) * (size_t)a.hsk * D;
  const bf16* kg = wave_uniform(a.k + kvh);
  const bf16* vg = wave_uniform(a.v + kvh);

  // Per-lane LDS read offsets (the ring slot and the constant parts of each
  // fragment's address are immediate offsets of the reads). K: row l32 (+32
  // for the second key block) at logical chunk 2 dc + hi. V: the A operand of
  // O^T = V^T P^T for d-block mb and 16-key chunk kc is two transposing 4-key
  // reads at rows 16 kc + 4 hi + (L >> 2) (+8), columns 32 mb + 16 dhalf +
  // 4 (L & 3); their keys line up with the register order of the P fragments.
  // The swizzle of those rows does not change with kc (16 kc adds nothing to
  // the row bits it uses), so kc is an immediate offset too.
  uint32_t kb[DC], vb[MB][2];
  auto lds_offsets = [&](int ln) __attribute__((always_inline)) {
    const int r32 = ln & 31, h32 = ln >> 5;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) kb[dc] = r32 * RB + (((2 * dc + h32) ^ chunk_swizzle<D>(r32)) << 4);
    const int L = ln & 15, dhalf = (ln >> 4) & 1;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = 4 * h32 + (L >> 2) + 8 * h;
        const int c = 32 * mb + 16 * dhalf + 4 * (L & 3);
        vb[mb][h] = R::TILE + r * RB + (((c >> 3) ^ chunk_swizzle<D>(r)) << 4) + (c & 7) * 2;
      }
  };
  lds_offsets(lane);

  // Per-lane DMA geometry (the same for K and V tiles): lane i of instruction
  // n writes LDS chunk P = (wid*INSTR + n)*64 + i of a tile, i.e. row P / CPR,
  // physical chunk P % CPR, and loads the logical chunk (physical ^
  // swizzle(row)); byte offsets relative to the tile's first key.
  uint32_t koff[R::INSTR];
#pragma unroll
  for (int n = 0; n < R::INSTR; ++n) {
    const int P = (wid * R::INSTR + n) * 64 + lane;
    const int krow = P / CPR;
    koff[n] = krow * RB + (((P % CPR) ^ chunk_swizzle<D>(krow)) << 4);
  }
  const uint32_t ldsw = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem + wid * R::INSTR * 1024);
  // DMA of key tile t (clamped to the last one: past it, the last tile is
  // reloaded into a slot nobody reads, which keeps the per-step DMA count
  // uniform). K and V rows past kend are out of the buffers' range and read
  // zeros: their scores are masked and their P is 0 (and 0 * 0 stays 0).
  struct Dma {
    u32x4 rk, rv;
  };
  auto dma_for = [&](int t) __attribute__((always_inline)) {
    Dma d;
    const int key0 = min(t, ntiles - 1) * BC;
    const uint32_t bytes = (uint32_t)(kend - key0) * RB;
    d.rk = buffer_rsrc(kg + (size_t)key0 * D, bytes);
    d.rv = buffer_rsrc(vg + (size_t)key0 * D, bytes);
    return d;
  };
  // DMA instruction QI (0 .. NDMA-1) into ring slot SLOT: K for even QI, V for odd
  auto issue_one = [&](auto slot_, auto qi_, const Dma& d) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_)::value;
    constexpr int QI = decltype(qi_)::value;
    constexpr int n = QI >> 1;
    if constexpr ((QI & 1) == 0)
      dma16b_at<SLOT * R::STAGE + n * 1024>(d.rk, koff[n], 0u, ldsw);
    else
      dma16b_at<SLOT * R::STAGE + R::TILE + n * 1024>(d.rv, koff[n], 0u, ldsw);
  };

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};
  float m2 = kNegInf, lsum = 0.f;
  bf16x8 pf[4];
  f32x16 s[2];

  // One basic block of MFMAs (step j, slot position POS = j mod 4): S(j) =
  // K_j Q^T (16 MFMAs, 2 chains) interleaved one-for-one with O^T +=
  // V_{j-1}^T P_{j-1}^T (16 MFMAs, MB chains), so a chain's next MFMA issues at
  // least four MFMAs after its previous one. LDS operand fragments are loaded
  // two pairs ahead; the DMA of tile j+2 rides in the shadow of the MFMAs.
  auto mma = [&](auto pos_, auto do_s, auto do_pv, int j) __attribute__((always_inline)) {
    constexpr int POS = decltype(pos_)::value;
    constexpr bool DS = decltype(do_s)::value;
    constexpr bool DP = decltype(do_pv)::value;
    constexpr int SK = POS;                     // K of tile j
    constexpr int SV = (POS + 3) % 4;           // V of tile j-1
    constexpr int SD = (POS + 2) % 4;           // DMA target: tile j+2
    const char* lds = smem;
    auto kfrag = [&](int i) __attribute__((always_inline)) {   // pair i: key block i & 1, d-chunk i >> 1
      return *(const bf16x8*)(lds + kb[i >> 1] + SK * R::STAGE + (i & 1) * 32 * RB);
    };
    static_assert(NP / MB == BC / 16, "one key chunk per MB pairs");
    auto vfrag = [&](int i) __attribute__((always_inline)) {   // pair i: d-block i % MB, key chunk i / MB
      const char* p = lds + SV * R::STAGE + (i / MB) * 16 * RB;
      return cat4(lds_read_tr((const bf16*)(p + vb[i % MB][0])), lds_read_tr((const bf16*)(p + vb[i % MB][1])));
    };
    Dma d;
    if constexpr (DS) d = dma_for(j + 2);
    bf16x8 kq[3], vq[3];
    if constexpr (DS) {
      kq[0] = kfrag(0);
      kq[1] = kfrag(1);
    }
    if constexpr (DP) {
      vq[0] = vfrag(0);
      vq[1] = vfrag(1);
    }
    constexpr int EVERY = NP / NDMA;
    // the partner wavefront is in its softmax meanwhile: issue priority keeps
    // its vector instructions from delaying this block's MFMA issue (measured
    // 2-3 % on the whole kernel)
    __builtin_amdgcn_s_setprio(1);
    static_for<NP>([&](auto ic) __attribute__((always_inline)) {
      constexpr int i = decltype(ic)::value;
      if constexpr (i + 2 < NP) {
        if constexpr (DS) kq[(i + 2) % 3] = kfrag(i + 2);
        if constexpr (DP) vq[(i + 2) % 3] = vfrag(i + 2);
      }
      __builtin_amdgcn_sched_barrier(0);   // keep the reads two pairs ahead of their MFMAs
      if constexpr (DS) s[i & 1] = mfma32(kq[i % 3], qf[i >> 1], i < 2 ? f32x16{} : s[i & 1]);
      if constexpr (DP) acc[i % MB] = mfma32(vq[i % 3], pf[i / MB], acc[i % MB]);
      if constexpr (DS && i % EVERY == EVERY - 1)
        issue_one(std::integral_constant<int, SD>{}, std::integral_constant<int, i / EVERY>{}, d);
    });
    __builtin_amdgcn_s_setprio(0);
  };
  // Phase A's full step. The V fragments of its first two P V products (V of
  // tile j-1, in LDS since step j-1) are read before the barrier (vpre), so
  // the block opens with those two MFMAs while the first K fragments of tile
  // j arrive (K of tile j may only be read after the barrier); from there the
  // P V stream runs two MFMAs ahead of the score stream, and the block ends
  // with two score MFMAs. Every chain sees its MFMAs in the same order as in
  // mma, so the result is the same bit for bit (measured 0.8-1.4 % faster at
  // d = 128).
  auto vpre = [&](auto pos_, bf16x8& v0, bf16x8& v1) __attribute__((always_inline)) {
    constexpr int SV = decltype(pos_)::value;   // stage of the tile whose V the next step reads
    const char* p = (const char*)smem + SV * R::STAGE;
    v0 = cat4(lds_read_tr((const bf16*)(p + vb[0][0])), lds_read_tr((const bf16*)(p + vb[0][1])));
    v1 = cat4(lds_read_tr((const bf16*)(p + vb[1][0])), lds_read_tr((const bf16*)(p + vb[1][1])));
  };
  auto mma_a = [&](auto pos_, int j, const bf16x8& vp0, const bf16x8& vp1) __attribute__((always_inline)) {
    constexpr int POS = decltype(pos_)::value;
    constexpr int SK = POS;                     // K of tile j
    constexpr int SV = (POS + 3) % 4;           // V of tile j-1
    constexpr int SD = (POS + 2) % 4;           // DMA target: tile j+2
    const char* lds = smem;
    auto kfrag = [&](int i) __attribute__((always_inline)) {
      return *(const bf16x8*)(lds + kb[i >> 1] + SK * R::STAGE + (i & 1) * 32 * RB);
    };
    auto vfrag = [&](int i) __attribute__((always_inline)) {
      const char* p = lds + SV * R::STAGE + (i / MB) * 16 * RB;
      return cat4(lds_read_tr((const bf16*)(p + vb[i % MB][0])), lds_read_tr((const bf16*)(p + vb[i % MB][1])));
    };
    const Dma d = dma_for(j + 2);
    bf16x8 kq[3], vq[3];
    kq[0] = kfrag(0);
    kq[1] = kfrag(1);
    vq[2] = vfrag(2);
    vq[0] = vfrag(3);
    constexpr int EVERY = NP / NDMA;
    __builtin_amdgcn_s_setprio(1);
    // op k: P V k for k < 2; then S t (k = 2 + 2t) and P V t + 2 (k = 3 + 2t);
    // S NP-2 and S NP-1 last. K and V fragments are loaded two MFMAs of their
    // own stream ahead; the DMA goes after every 2 EVERY MFMAs, as in mma.
    static_for<2 * NP>([&](auto kc) __attribute__((always_inline)) {
      constexpr int k = decltype(kc)::value;
      constexpr bool is_s = k >= 2 && (k >= 2 * NP - 2 || k % 2 == 0);
      constexpr int t = k >= 2 * NP - 2 ? k - NP : (k - 2) / 2;
      constexpr int v = k < 2 ? k : (k - 3) / 2 + 2;
      if constexpr (is_s) {
        if constexpr (t + 2 < NP) kq[(t + 2) % 3] = kfrag(t + 2);
        __builtin_amdgcn_sched_barrier(0);
        s[t & 1] = mfma32(kq[t % 3], qf[t >> 1], t < 2 ? f32x16{} : s[t & 1]);
      } else {
        if constexpr (v >= 2 && v + 2 < NP) vq[(v + 2) % 3] = vfrag(v + 2);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (v == 0)
          acc[0] = mfma32(vp0, pf[0], acc[0]);
        else if constexpr (v == 1)
          acc[1] = mfma32(vp1, pf[1 / MB], acc[1]);
        else
          acc[v % MB] = mfma32(vq[v % 3], pf[v / MB], acc[v % MB]);
      }
      if constexpr (k % 2 == 1 && (k / 2) % EVERY == EVERY - 1)
        issue_one(std::integral_constant<int, SD>{}, std::integral_constant<int, (k / 2) / EVERY>{}, d);
    });
    __builtin_amdgcn_s_setprio(0);
  };
  // The reference max m2 (log2 units) of this lane's row moves only when the
  // row max grew by more than RESCALE_T; the running sum and output are then
  // rescaled. msub is m2, or 0 while m2 = -inf.
  float msub = 0.f;
  auto move_max = [&](const float* v) __attribute__((always_inline)) {
    const float mx = max_halves(tree_max32(v)) * a.c;
    const bool grow = mx > m2 + RESCALE_T;
    if (!wave_any(grow)) return false;
    const float mnew = grow ? mx : m2;
    const float alpha = grow ? fast_exp2(m2 - mnew) : 1.f;
    lsum *= alpha;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] *= alpha;
    m2 = mnew;
    msub = (m2 == kNegInf) ? 0.f : m2;
    return true;
  };
  auto softmax = [&](int j) __attribute__((always_inline)) {
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
    if constexpr (DROP) {
      move_max(v);
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = fast_exp2(__builtin_fmaf(v[i], a.c, -msub));
      lsum += tree_sum32(v);
      // values 4g .. 4g+3 are keys 4 j4 .. 4 j4 + 3 of this lane's query row:
      // word (pos & 3) of block (pos / 4, j4)
#pragma unroll
      for (int g = 0; g < 8; ++g) {
        const uint32_t j4 = (uint32_t)(key0 + 32 * (g >> 2) + 8 * (g & 3) + 4 * hi) >> 2;
        const u32x4 x = dropout_block(a.drop, (uint32_t)pos >> 2, j4, (uint32_t)bh);
        const int w = pos & 3;
        const uint32_t word = w == 0 ? x[0] : w == 1 ? x[1] : w == 2 ? x[2] : x[3];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (((word >> (8 * t)) & 0xffu) < a.drop.thr) v[4 * g + t] = 0.f;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q)
        pf[q] = to_bf16x8(v[8 * q + 0], v[8 * q + 1], v[8 * q + 2], v[8 * q + 3], v[8 * q + 4], v[8 * q + 5],
                          v[8 * q + 6], v[8 * q + 7]);
    } else {
      // The probabilities are first taken against the current m2. While every
      // lane's sum of its 32 values stays within 2^RESCALE_T, no score of the
      // wavefront exceeds m2 + RESCALE_T, so m2 stays and the row max is not
      // needed; otherwise, and at tile 0 (the first tile of every row that
      // sees any key), the row max is formed and the rule applied. Either way
      // the result is the same. Groups of eight values are summed and packed
      // as they are formed; the four group sums make the same tree as
      // tree_sum32.
      auto probs = [&]() __attribute__((always_inline)) {
        float g[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float p[8];
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const float x = __builtin_fmaf(v[8 * q + i], a.c, -msub);
            p[i] = (POLY > 0 && i % POLY == POLY - 1) ? poly_exp2(x) : fast_exp2(x);
          }
          g[q] = ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
          pf[q] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
        }
        return (g[0] + g[1]) + (g[2] + g[3]);
      };
      float ts = probs();
      if (j == 0 || wave_any(!(ts <= kRescaleSum)))
        if (move_max(v)) ts = probs();
      lsum += ts;
    }
  };
  using T_ = std::true_type;
  using F_ = std::false_type;
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I3 = std::integral_constant<int, 3>;
  // step j: tile j has landed for every wavefront (each waits for its own
  // DMA, the barrier for all of them), and every wavefront is done with step
  // j-1. Every step that computes scores issues NDMA DMA instructions.
  auto sync = [&]() __attribute__((always_inline)) { asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(NDMA) : "memory"); };
  // Wavefronts whose rows see no key of a tile still run it (their scores are
  // all masked, so P = 0): the step sequence is the same for the whole workgroup.
  // The steps of one wavefront for its phase pb_, a compile-time constant:
  // each phase gets its own copy of the loop and keeps its scores in the
  // registers its MFMAs write (one loop for both copied them after every
  // MFMA block; the copies cost 3-5 % at d = 128 and 5-9 % at d = 64, with
  // bit-identical output).
  auto run = [&](auto pb_) __attribute__((always_inline)) {
    const bool pb = pb_;
    bf16x8 vp0, vp1;                            // phase A: V fragments read before the barrier
    auto full = [&](auto pos_, int j) __attribute__((always_inline)) {
      sync();
      if (pb) {
        softmax(j - 1);
        mma(pos_, T_{}, T_{}, j);
      } else {
        mma_a(pos_, j, vp0, vp1);
        softmax(j);
        vpre(pos_, vp0, vp1);
      }
    };
    if (ntiles > 0) {
      const Dma d0 = dma_for(0), d1 = dma_for(1);
      static_for<NDMA>([&](auto qi) __attribute__((always_inline)) { issue_one(I0{}, qi, d0); });
      static_for<NDMA>([&](auto qi) __attribute__((always_inline)) { issue_one(I1{}, qi, d1); });
      sync();
      mma(I0{}, T_{}, F_{}, 0);
      if (!pb) {
        softmax(0);
        vpre(I0{}, vp0, vp1);
      }
    }
    int j = 1;
    for (; j + 3 < ntiles; j += 4) {
      full(I1{}, j);
      full(I2{}, j + 1);
      full(I3{}, j + 2);
      full(I0{}, j + 3);
    }
    // the last steps get freshly computed offsets (from the lane index counted
    // again), so that no offset is held, or spilled, across the main loop
    lds_offsets((int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)));
    if (j < ntiles) full(I1{}, j);
    if (j + 1 < ntiles) full(I2{}, j + 1);
    if (j + 2 < ntiles) full(I3{}, j + 2);
    if (ntiles > 0) {
      // P V of the last tile (its V sits in slot (ntiles - 1) mod 4); no
      // barrier is needed since no DMA writes that slot any more
      if (pb) softmax(ntiles - 1);
      switch (ntiles & 3) {
        case 0: mma(I0{}, F_{}, T_{}, ntiles); break;
        case 1: mma(I1{}, F_{}, T_{}, ntiles); break;
        case 2: mma(I2{}, F_{}, T_{}, ntiles); break;
        default: mma(I3{}, F_{}, T_{}, ntiles); break;
      }
    }
  };
  if (phase_b) run(T_{});
  else run(F_{});
  // no LDS DMA may still be in flight when the workgroup's LDS is released
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  const float lt = sum_halves(lsum);
  float inv = lt > 0.f ? 1.f / lt : 0.f;
  if constexpr (DROP) inv *= a.drop.scale;
  const float lse_v = lt > 0.f ? (m2 + __log2f(lt)) * kLn2 : kNegInf;
  // this lane's row, from the lane index counted again (not held across the loop)
  const int ln = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int pos_e = p0 + (ln & 31), hi_e = ln >> 5;
  if (pos_e >= a.Sq) return;
  const size_t hbase = (size_t)bh * a.hsq;
  bf16* op = a.o + (hbase + pos_e) * D;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 r;
      r[0] = (bf16)(acc[mb][4 * q4 + 0] * inv);
      r[1] = (bf16)(acc[mb][4 * q4 + 1] * inv);
      r[2] = (bf16)(acc[mb][4 * q4 + 2] * inv);
      r[3] = (bf16)(acc[mb][4 * q4 + 3] * inv);
      *(bf16x4*)(op + 32 * mb + 8 * q4 + 4 * hi_e) = r;
    }
  if (a.lse != nullptr && hi_e == 0) a.lse[hbase + pos_e] = lse_v;
}

// ---------------------------------------------------------------------------
// Split-key decode: one wavefront per (key slice, KV head, batch); its 32
// MFMA columns pack (query head of the group, query row) pairs, so each K/V
// byte of the slice is read once for all of them. Writes the slice's
// normalised partial output and lse; combine_split_kernel merges the slices.
//
// The kernel streams K and V from HBM once, so it is sized for occupancy
// (about eight wavefronts per CU keep enough loads in flight): 32-key tiles,
// K fragments (the A operand of S^T = K Q^T) loaded straight into registers
// one tile ahead by range-checked buffer loads, V tiles by LDS DMA into a
// 2-slot ring (16 KB per wavefront at d = 128) and read transposed for
// O^T = V^T P^T.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void fwd_split_kernel(FwdArgs a) {
  constexpr int BK = 32;                        // keys per tile
  constexpr int MB = D / 32;
  constexpr int DC = D / 16;
  constexpr int RB = 2 * D;                     // bytes per K or V row
  constexpr int VT = BK * RB;                   // bytes of a V tile
  constexpr int NV = VT / 1024;                 // DMA instructions per V tile
  constexpr int CPR = D / 8;                    // 16-byte chunks per row
  __shared__ __attribute__((aligned(1024))) char smem[2 * VT];

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
  const int ntiles = (kend - kbeg + BK - 1) / BK;
  const int lim = a.causal ? min(kend - 1, pos + off) : kend - 1;
  const int mask_from = a.causal ? max(kbeg, min(kend, off + 1)) : kend;

  bf16x8 qf[DC];
  {
    const bf16* qp = a.q + (((size_t)b * a.Hq + hq) * a.hsq + pos) * D;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      qf[dc] = colv ? *(const bf16x8*)(qp + 16 * dc + 8 * hi) : __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) qf[dc] = settle(qf[dc]);
  }
  const size_t kvh = (size_t)b * a.Hkv + hkv;
  // whole-head buffers: rows past Sk read zeros (their scores are masked or,
  // for V, multiplied by P = 0). The byte range is an unsigned 32-bit count
  // (Sk < 2^24 rows of up to 256 bytes), passed bit for bit to the builtin's
  // int parameter.
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a.k + kvh * (size_t)a.hsk * D), (short)0, __builtin_bit_cast(int, (uint32_t)a.Sk * (uint32_t)RB),
      0x00020000);
  const u32x4 rv = buffer_rsrc(a.v + kvh * (size_t)a.hsk * D, (uint32_t)a.Sk * RB);
  // K fragment dc of key row l32: byte l32*RB + 16*hi + 32*dc of the tile
  const uint32_t kl = l32 * RB + 16 * hi;
  // V DMA: lane of instruction n writes LDS chunk P = 64 n + lane of the tile,
  // i.e. row P / CPR, physical chunk P % CPR, holding logical chunk
  // (physical ^ chunk_swizzle(row))
  uint32_t vo[NV];
#pragma unroll
  for (int n = 0; n < NV; ++n) {
    const int P = 64 * n + lane;
    const int r = P / CPR;
    vo[n] = r * RB + (((P % CPR) ^ chunk_swizzle<D>(r)) << 4);
  }
  const uint32_t lds0 = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)smem);

  auto load_k = [&](int t, bf16x8* kf) __attribute__((always_inline)) {
    const uint32_t base = kl + (uint32_t)(kbeg + t * BK) * RB;
#pragma unroll
    for (int dc = 0; dc < DC; ++dc)
      kf[dc] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, base + 32 * dc, 0, 0));
  };
  auto load_v = [&](int t, auto slot_) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_)::value;
    const uint32_t base = (uint32_t)(kbeg + t * BK) * RB;
    static_for<NV>([&](auto nc) __attribute__((always_inline)) {
      constexpr int n = decltype(nc)::value;
      dma16b_at<SLOT * VT + n * 1024>(rv, vo[n] + base, 0u, lds0);
    });
  };

  f32x16 acc[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};
  float m2 = kNegInf, lsum = 0.f;
  bf16x8 kcur[DC], knext[DC];
  const int L = lane & 15;
  const int dhalf = (lane >> 4) & 1;

  auto tile = [&](int t, auto slot_) __attribute__((always_inline)) {
    constexpr int SLOT = decltype(slot_)::value;
    // every load of tile t has arrived (the compiler waits on the memory
    // counter before the re-definition, which also covers the V DMA issued
    // with them); then the next tile's loads go out
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) kcur[dc] = settle(knext[dc]);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (t + 1 < ntiles) {
      load_k(t + 1, knext);
      load_v(t + 1, std::integral_constant<int, SLOT ^ 1>{});
    }
    const int key0 = kbeg + t * BK;
    f32x16 s = f32x16{};
#pragma unroll
    for (int dc = 0; dc < DC; ++dc) s = mfma32(kcur[dc], qf[dc], dc == 0 ? f32x16{} : s);
    if (key0 + BK > mask_from) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = key0 + 8 * (i >> 2) + 4 * hi + (i & 3);
        if (key > lim) s[i] = kNegInf;
      }
    }
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
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
    bf16x8 pf[2];
    float ps = 0.f;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float p[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = fast_exp2(__builtin_fmaf(s[8 * h + e], a.c, -msub));
        ps += p[e];
      }
      pf[h] = to_bf16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
    }
    lsum += ps;
    // O^T += V^T P^T: A operand rows d = 32 mb + l32, reduction slots = the 8
    // keys of P's register order, read transposed from the row-major V tile
    const char* sv = smem + SLOT * VT;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int kc = 0; kc < 2; ++kc) {
        const int r = 16 * kc + 4 * hi + (L >> 2);
        const int c = 32 * mb + 16 * dhalf + 4 * (L & 3);
        const bf16* p0 = (const bf16*)(sv + r * RB + (((c >> 3) ^ chunk_swizzle<D>(r)) << 4) + (c & 7) * 2);
        const bf16* p1 = (const bf16*)(sv + (r + 8) * RB + (((c >> 3) ^ chunk_swizzle<D>(r + 8)) << 4) + (c & 7) * 2);
        acc[mb] = mfma32(cat4(lds_read_tr(p0), lds_read_tr(p1)), pf[kc], acc[mb]);
      }
  };

  if (ntiles > 0) {
    load_k(0, knext);
    load_v(0, std::integral_constant<int, 0>{});
  }
  int t = 0;
  for (; t + 1 < ntiles; t += 2) {
    tile(t, std::integral_constant<int, 0>{});
    tile(t + 1, std::integral_constant<int, 1>{});
  }
  if (t < ntiles) tile(t, std::integral_constant<int, 0>{});

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
                                                           int nsplit, size_t rows, int Sq, int hsq) {
  const size_t row = blockIdx.x;
  if (row >= rows) return;
  const size_t orow = (row / Sq) * (size_t)hsq + row % Sq;   // (b, h, i) in the output's layout
  const int lane = threadIdx.x;
  // the slices' lse spread over the lanes, then a wavefront max
  float m = kNegInf;
  for (int s = lane; s < nsplit; s += 64) m = fmaxf(m, part_lse[(size_t)s * rows + row]);
#pragma unroll
  for (int sh = 32; sh >= 1; sh >>= 1) m = fmaxf(m, __shfl_xor(m, sh));
  constexpr int PER = D / 64;
  float accv[PER];
#pragma unroll
  for (int j = 0; j < PER; ++j) accv[j] = 0.f;
  float tot = 0.f;
  if (m != kNegInf) {
    // no branch on the weight: an empty slice has lse = -inf (weight 0) and a
    // zero partial, so the loads of several slices can be in flight together
#pragma unroll 4
    for (int s = 0; s < nsplit; ++s) {
      const float w = __expf(part_lse[(size_t)s * rows + row] - m);
      tot += w;
      const float* po = part_o + ((size_t)s * rows + row) * D + lane * PER;
#pragma unroll
      for (int j = 0; j < PER; ++j) accv[j] += w * po[j];
    }
  }
  const float inv = tot > 0.f ? 1.f / tot : 0.f;
#pragma unroll
  for (int j = 0; j < PER; ++j) o[orow * D + lane * PER + j] = (bf16)(accv[j] * inv);
  if (lse != nullptr && lane == 0) lse[orow] = tot > 0.f ? m + __logf(tot) : kNegInf;
}

// The dropout mask as keep bytes [B, Hq, Sq, Sk]: one thread per 4x4 block.
__global__ __launch_bounds__(256) void dropout_mask_kernel(DropParams dp, unsigned char* __restrict__ keep,
                                                           long long blocks, int iq, int jq, int Sq, int Sk) {
  const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
  if (t >= blocks) return;
  const int j4 = (int)(t % jq);
  const int i4 = (int)((t / jq) % iq);
  const long long bh = t / ((long long)jq * iq);
  const u32x4 x = dropout_block(dp, (uint32_t)i4, (uint32_t)j4, (uint32_t)bh);
  for (int w = 0; w < 4; ++w) {
    const int i = 4 * i4 + w;
    if (i >= Sq) break;
    unsigned char* row = keep + ((size_t)bh * Sq + i) * Sk;
    for (int u = 0; u < 4; ++u) {
      const int j = 4 * j4 + u;
      if (j < Sk) row[j] = ((x[w] >> (8 * u)) & 0xffu) >= dp.thr ? 1 : 0;
    }
  }
}

}  // namespace

// ATTN_EXP2_POLY=2 or 4: the dense d = 128 prefill without dropout forms every
// second or fourth probability with poly_exp2 (read at every call).
int exp2_poly_every() {
  const char* e = std::getenv("ATTN_EXP2_POLY");
  if (e == nullptr) return 0;
  if (std::strcmp(e, "2") == 0) return 2;
  if (std::strcmp(e, "4") == 0) return 4;
  return 0;
}

namespace {

template <int D>
hipError_t launch_prefill_d(const FwdArgs& a, hipStream_t s) {
  timing_begin(s, "fwd_prefill_bf16");
  const int poly = exp2_poly_every();
  if (a.drop.thr != 0)
    hipLaunchKernelGGL((fwd_prefill_kernel<D, NoTable, true>), dim3(a.total_wgs), dim3(512), 0, s, a, NoTable{});
  else if (D == 128 && poly == 4)
    hipLaunchKernelGGL((fwd_prefill_kernel<D, NoTable, false, 4>), dim3(a.total_wgs), dim3(512), 0, s, a, NoTable{});
  else if (D == 128 && poly == 2)
    hipLaunchKernelGGL((fwd_prefill_kernel<D, NoTable, false, 2>), dim3(a.total_wgs), dim3(512), 0, s, a, NoTable{});
  else
    hipLaunchKernelGGL((fwd_prefill_kernel<D, NoTable, false>), dim3(a.total_wgs), dim3(512), 0, s, a, NoTable{});
  const hipError_t e = hipGetLastError();
  timing_end(s);
  return e;
}

template <int D>
hipError_t launch_prefill_packed_d(const FwdArgs& a, const SeqTable& T, int grid, hipStream_t s) {
  timing_begin(s, "fwd_prefill_bf16");
  hipLaunchKernelGGL((fwd_prefill_kernel<D, SeqTable, false>), dim3(grid), dim3(512), 0, s, a, T);
  const hipError_t e = hipGetLastError();
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
                     a.o, a.lse, a.nsplit, (size_t)rows, a.Sq, a.hsq);
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
  a.hsq = p.hsq;
  a.hsk = p.hsk;
  a.g = p.Hq / p.Hkv;
  a.causal = p.causal;
  a.c = p.scale * kLog2e;
  a.drop = p.drop;
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
  pl.ws_bytes = 0;
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
  (void)ws;
  if (a.total_wgs == 0) return hipSuccess;
  return p.d == 64 ? launch_prefill_d<64>(a, s) : launch_prefill_d<128>(a, s);
}

hipError_t launch_fwd_prefill_bf16_packed(const Problem& p, const SeqSpan* seqs, int n, const void* q,
                                          const void* k, const void* v, void* o, float* lse, hipStream_t s,
                                          char* log, size_t log_n) {
  const PrefillPlan pl = plan_prefill(p);       // the head grouping depends only on Hq / Hkv
  FwdArgs a = base_args(p, q, k, v, o, lse);
  a.hw = pl.hw;
  a.n_hgroups = pl.n_hgroups;
  a.rows_per_wg = pl.rows_per_wg;
  int ntile[SEQ_MAX];
  for (int i = 0; i < n; ++i) ntile[i] = (seqs[i].sq + pl.rows_per_wg - 1) / pl.rows_per_wg;
  SeqTable T;
  const int grid = build_seq_table(T, seqs, n, p.Hkv * pl.n_hgroups, ntile, nullptr);
  if (log != nullptr && log_n > 0)
    snprintf(log, log_n, "fwd_prefill<d=%d, packed> %d sequences grid=%d (%d query rows x %d heads per workgroup%s)",
             p.d, T.n, grid, pl.rows_per_wg, pl.hw,
             T.split8 ? ", per-XCD head split" : "");
  if (grid == 0) return hipSuccess;
  return p.d == 64 ? launch_prefill_packed_d<64>(a, T, grid, s) : launch_prefill_packed_d<128>(a, T, grid, s);
}

hipError_t launch_dropout_mask(const Problem& p, unsigned char* keep, hipStream_t s) {
  const int iq = (p.Sq + 3) / 4, jq = (p.Sk + 3) / 4;
  const long long blocks = (long long)p.B * p.Hq * iq * jq;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)((blocks + 255) / 256)), dim3(256), 0, s, p.drop, keep,
                     blocks, iq, jq, p.Sq, p.Sk);
  return hipGetLastError();
}

hipError_t launch_combine_split(const Problem& p, const SplitPlan& sp, void* ws, void* o, float* lse,
                                hipStream_t s) {
  const size_t rows = (size_t)p.B * p.Hq * p.Sq;
  const size_t o_bytes = (size_t)sp.nsplit * rows * p.d * sizeof(float);
  const float* part_o = (const float*)ws;
  const float* part_lse = (const float*)((const char*)ws + ((o_bytes + 255) / 256) * 256);
  timing_begin(s, "combine_split");
  if (p.d == 64)
    hipLaunchKernelGGL((combine_split_kernel<64>), dim3(rows), dim3(64), 0, s, part_o, part_lse, (bf16*)o, lse,
                       sp.nsplit, rows, p.Sq, p.hsq);
  else
    hipLaunchKernelGGL((combine_split_kernel<128>), dim3(rows), dim3(64), 0, s, part_o, part_lse, (bf16*)o, lse,
                       sp.nsplit, rows, p.Sq, p.hsq);
  const hipError_t e = hipGetLastError();
  timing_end(s);
  return e;
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
