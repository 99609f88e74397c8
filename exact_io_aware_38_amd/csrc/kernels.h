// Host-side launch interface between the C ABI (api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by the ABI layer and
// returns the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

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
struct Problem {
  int B, Hq, Hkv, Sq, Sk, d, causal;
  float scale;
  int hsq, hsk;     // head strides in rows
};

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

// ---- forward, fp32 ----------------------------------------------------------
hipError_t launch_fwd_f32(const Problem& p, const float* q, const float* k, const float* v,
                          float* o, float* lse, hipStream_t s);

// ---- backward, bf16 ---------------------------------------------------------
size_t bwd_workspace_bytes(const Problem& p);
hipError_t launch_bwd_bf16(const Problem& p, const void* q, const void* k, const void* v,
                           const void* o, const float* lse, const void* dout, void* dq,
                           void* dk, void* dv, void* ws, hipStream_t s, char* log, size_t log_n);

}  // namespace attn
