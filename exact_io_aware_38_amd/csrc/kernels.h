// Host-side launch interface between the C ABI (api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by the ABI layer and
// returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace attn {

// Optional per-kernel timing (diagnostics, off by default): while enabled on
// the calling thread, every launch is bracketed by two HIP events recorded on
// the launch's own stream.
void timing_begin(hipStream_t s, const char* kernel);
void timing_end(hipStream_t s);

// Problem description shared by the launchers (already validated).
// Row (b, h, i) of Q, O, dO, dQ and lse lives at packed row (b Hq + h) hsq + i,
// row (b, h, j) of K, V, dK, dV at (b Hkv + h) hsk + j: hsq = Sq and hsk = Sk
// for [B, H, S, d] tensors; a sequence inside head-major packed tensors
// [H, total, d] (B = 1, data pointers advanced to the sequence's first row)
// has the packed totals as head strides.
// Dropout on the attention probabilities: a probability is kept when its byte
// of the Philox stream (see philox4x32_10 and dropout_block) is >= thr, and
// kept values are multiplied by scale = 1 / (1 - thr / 256). thr = 0 means no
// dropout.
struct DropParams {
  uint32_t seed_lo, seed_hi, offset, thr;
  float scale;
};

struct Problem {
  int B, Hq, Hkv, Sq, Sk, d, causal;
  float scale;
  int hsq, hsk;     // head strides in rows
  DropParams drop;
};

// 0, or 2 / 4 when ATTN_EXP2_POLY asks the dense d = 128 bf16 prefill to form
// every second / fourth probability with the FMA-pipe exponential.
int exp2_poly_every();

// keep[B, Hq, Sq, Sk] (1 = kept) of the dropout mask the kernels regenerate.
hipError_t launch_dropout_mask(const Problem& p, unsigned char* keep, hipStream_t s);

// ---- packed batches in one launch -------------------------------------------
// A sequence of a head-major packed batch: its first packed query and key row
// and its lengths.
struct SeqSpan {
  int q0, k0, sq, sk;
};

// Up to SEQ_MAX sequences of a packed batch run as one grid. Workgroups are
// numbered sequence after sequence; every sequence has `units` independent
// units (heads or groups of heads) of ntile[i] tiles each. With split8 each
// of the 8 XCDs (the hardware deals consecutive workgroup ids to them in
// turn) takes units/8 units of every sequence, so the XCDs get equal work and
// each unit's K and V stay in one L2; wg0 then counts workgroups per XCD. The
// table travels in the kernel arguments.
constexpr int SEQ_MAX = 64;
struct SeqTable {
  int n, units, split8;
  int wg0[SEQ_MAX + 1];      // first workgroup of each sequence
  int ntile[SEQ_MAX];
  int q0[SEQ_MAX], k0[SEQ_MAX], sq[SEQ_MAX], sk[SEQ_MAX];
  int aux[SEQ_MAX];          // per-kernel offset (the backward's lse2/D block, in floats)
};

// Fills T with the sequences that have at least one tile; returns the grid
// size.
inline int build_seq_table(SeqTable& T, const SeqSpan* seqs, int n, int units, const int* ntile,
                           const int* aux) {
  T = SeqTable{};
  T.units = units;
  T.split8 = (units % 8) == 0;
  const int per = T.split8 ? units / 8 : units;
  int w = 0;
  for (int i = 0; i < n; ++i) {
    if (ntile[i] == 0) continue;
    const int j = T.n++;
    T.wg0[j] = w;
    T.ntile[j] = ntile[i];
    T.q0[j] = seqs[i].q0;
    T.k0[j] = seqs[i].k0;
    T.sq[j] = seqs[i].sq;
    T.sk[j] = seqs[i].sk;
    T.aux[j] = aux != nullptr ? aux[i] : 0;
    w += per * ntile[i];
  }
  T.wg0[T.n] = w;
  return T.split8 ? 8 * w : w;
}

// p carries Hq, Hkv, d, causal, scale and the packed totals as head strides
// (B = 1; Sq and Sk are taken per sequence). n <= SEQ_MAX.
hipError_t launch_fwd_prefill_bf16_packed(const Problem& p, const SeqSpan* seqs, int n, const void* q,
                                          const void* k, const void* v, void* o, float* lse, hipStream_t s,
                                          char* log, size_t log_n);
size_t bwd_packed_workspace_bytes(const Problem& p, const SeqSpan* seqs, int n);
hipError_t launch_bwd_bf16_packed(const Problem& p, const SeqSpan* seqs, int n, const void* q, const void* k,
                                  const void* v, const void* o, const float* lse, const void* dout, void* dq,
                                  void* dk, void* dv, void* ws, hipStream_t s, char* log, size_t log_n);

// ---- forward, bf16 ----------------------------------------------------------
// Tiled prefill: one workgroup per (query-row tile, group of query heads).
struct PrefillPlan {
  int hw;           // query heads packed into one workgroup
  int n_hgroups;    // (Hq/Hkv) / hw
  int rows_per_wg;  // query positions per workgroup
  int n_ptiles;     // ceil(Sq / rows_per_wg)
  int total_wgs;
  size_t ws_bytes;  // 0: K and V tiles are read in place
};
PrefillPlan plan_prefill(const Problem& p);
hipError_t launch_fwd_prefill_bf16(const Problem& p, const PrefillPlan& plan, const void* q,
                                   const void* k, const void* v, void* o, float* lse, void* ws,
                                   hipStream_t s);

// Split-key decode: every workgroup runs the recurrence over one slice of the
// keys for all query rows of one KV head, writing a normalised partial output
// and its lse; a second kernel merges the slices.
struct SplitPlan {
  bool use;         // problem qualifies for the split path
  int nsplit;       // number of key slices
  int split_keys;   // keys per slice (multiple of the key tile)
  size_t ws_bytes;  // workspace for the partials
};
SplitPlan plan_split(const Problem& p);
hipError_t launch_fwd_split_bf16(const Problem& p, const SplitPlan& plan, const void* q,
                                 const void* k, const void* v, void* o, float* lse,
                                 void* ws, hipStream_t s);
// Fixed scratch for callers that cannot allocate (attn_fwd_noalloc): a
// static device array of this many bytes per GPU, holding the split path's
// partials. noalloc_scratch() returns its address on the current device,
// looked up once per device.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)16 << 20;
hipError_t noalloc_scratch(void** ptr);
// The merge of a split launch's per-slice partials (in the workspace laid out
// by plan_split) into o (bf16) and lse.
hipError_t launch_combine_split(const Problem& p, const SplitPlan& plan, void* ws, void* o, float* lse,
                                hipStream_t s);

// ---- forward, fp32 ----------------------------------------------------------
hipError_t launch_fwd_f32(const Problem& p, const float* q, const float* k, const float* v,
                          float* o, float* lse, hipStream_t s);

// ---- backward, bf16 ---------------------------------------------------------
// Workspace of the two-kernel path (lse2/D), and of the fused path (the same
// lse2/D block followed by the float32 dQ sums).
size_t bwd_workspace_bytes(const Problem& p);
size_t bwd_fused_workspace_bytes(const Problem& p);
hipError_t launch_bwd_bf16(const Problem& p, const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout, void* dq,
                           void* dk, void* dv, void* ws, bool fused, hipStream_t s, char* log,
                           size_t log_n);

// ---- forward, MXFP8 ---------------------------------------------------------
// Keys of the transposed FP8 V rounded up to the 64-key tile.
int fp8_padded_keys(int Sk);
// x bf16 [rows, d] -> E4M3 codes [rows, d] and E8M0 scales [rows, d/32].
hipError_t launch_mx_quant_rows(const void* x, void* codes, void* scales, long long rows, int d, hipStream_t s);
// v bf16 [BH, Sk, d] -> V^T codes tiled by 64 keys [BH, Skp/64, d, 64] and scales
// [BH, Skp/64, d, 2].
hipError_t launch_mx_quant_vt(const void* v, void* codes, void* scales, int BH, int Sk, int d, hipStream_t s);
// Workspace of the FP8 forward: the split-key partials for decode-shaped
// problems (the same rule and layout as the bf16 split path), else 0.
size_t fp8_workspace_bytes(const Problem& p);
hipError_t launch_fwd_fp8(const Problem& p, const void* q8, const void* qs, const void* k8, const void* ks,
                          const void* vt8, const void* vs, void* o, float* lse, void* ws, hipStream_t s, char* log,
                          size_t log_n);

}  // namespace attn
