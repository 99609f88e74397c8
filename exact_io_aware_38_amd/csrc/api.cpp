// C ABI of the attention library: argument validation, kernel selection,
// workspace sizing and the per-thread dispatch record (see include/attn.h).
#include "attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "kernels.h"

namespace {

// Per-thread kernel timing records (diagnostics).
struct TimedLaunch {
  const char* kernel;
  hipEvent_t begin, end;
};
struct TimingState {
  bool on = false;
  bool failed = false;
  std::vector<hipEvent_t> pool;   // events owned by this thread, reused across sessions
  size_t used = 0;
  std::vector<TimedLaunch> launches;
  const char* pending = nullptr;
  hipEvent_t pending_begin = nullptr;
};
thread_local TimingState g_timing;

hipEvent_t next_event() {
  TimingState& t = g_timing;
  if (t.used == t.pool.size()) {
    hipEvent_t e = nullptr;
    if (hipEventCreate(&e) != hipSuccess) {
      t.failed = true;
      return nullptr;
    }
    t.pool.push_back(e);
  }
  return t.pool[t.used++];
}

thread_local char g_dispatch[512] = "";

bool log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("ATTN_LOG");
    return e != nullptr && std::strcmp(e, "1") == 0;
  }();
  return on;
}

void record(const char* text) {
  std::snprintf(g_dispatch, sizeof(g_dispatch), "%s", text);
  if (log_enabled()) std::fprintf(stderr, "[attn] %s\n", g_dispatch);
}

int check_common(int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, float scale, int dtype) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 0) return ATTN_ERR_SHAPE;
  // every element offset must fit the kernels' 64-bit arithmetic and every
  // per-head index their 32-bit arithmetic
  const long long rows_q = (long long)B * Hq * Sq;
  const long long rows_k = (long long)B * Hkv * (long long)Sk;
  if (rows_q > (1LL << 31) - 1 || rows_k > (1LL << 31) - 1) return ATTN_ERR_SHAPE;
  if (Sq > (1 << 30) || Sk > (1 << 30)) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_GQA;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (causal < 0 || causal > 2) return ATTN_ERR_CAUSAL;
  if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_SCALE;
  return ATTN_OK;
}

attn::Problem make_problem(int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, float scale) {
  return attn::Problem{B, Hq, Hkv, Sq, Sk, d, causal, scale};
}

}  // namespace

namespace attn {

void timing_begin(hipStream_t s, const char* kernel) {
  TimingState& t = g_timing;
  if (!t.on) return;
  t.pending = kernel;
  t.pending_begin = next_event();
  if (t.pending_begin != nullptr && hipEventRecord(t.pending_begin, s) != hipSuccess) t.failed = true;
}

void timing_end(hipStream_t s) {
  TimingState& t = g_timing;
  if (!t.on || t.pending == nullptr || t.pending_begin == nullptr) return;
  hipEvent_t e = next_event();
  if (e == nullptr || hipEventRecord(e, s) != hipSuccess) {
    t.failed = true;
  } else {
    t.launches.push_back(TimedLaunch{t.pending, t.pending_begin, e});
  }
  t.pending = nullptr;
  t.pending_begin = nullptr;
}

}  // namespace attn

extern "C" {

int attn_timing_start(void) {
  TimingState& t = g_timing;
  t.on = true;
  t.failed = false;
  t.used = 0;
  t.launches.clear();
  return ATTN_OK;
}

int attn_timing_stop(char* buf, size_t n) {
  TimingState& t = g_timing;
  t.on = false;
  if (t.failed) return ATTN_ERR_HIP;
  // aggregate per kernel name, in order of first appearance
  std::vector<std::string> names;
  std::vector<double> total;
  std::vector<int> count;
  for (const TimedLaunch& l : t.launches) {
    if (hipEventSynchronize(l.end) != hipSuccess) return ATTN_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, l.begin, l.end) != hipSuccess) return ATTN_ERR_HIP;
    size_t i = 0;
    while (i < names.size() && names[i] != l.kernel) ++i;
    if (i == names.size()) {
      names.emplace_back(l.kernel);
      total.push_back(0.0);
      count.push_back(0);
    }
    total[i] += ms;
    count[i] += 1;
  }
  std::string out;
  for (size_t i = 0; i < names.size(); ++i) {
    char line[160];
    std::snprintf(line, sizeof(line), "%s %d %.6f\n", names[i].c_str(), count[i], total[i]);
    out += line;
  }
  t.launches.clear();
  t.used = 0;
  if (n > 0) {
    if (buf == nullptr) return ATTN_ERR_NULL;
    std::snprintf(buf, n, "%s", out.c_str());
  }
  return (int)out.size();
}

const char* attn_strerror(int status) {
  switch (status) {
    case ATTN_OK: return "success";
    case ATTN_ERR_NULL: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "invalid shape: need B, Hq, Hkv, Sq >= 1, Sk >= 0 and sizes that fit";
    case ATTN_ERR_GQA: return "Hq must be a multiple of Hkv";
    case ATTN_ERR_HEADDIM: return "head dim must be 64 or 128";
    case ATTN_ERR_DTYPE: return "unsupported dtype for this entry point";
    case ATTN_ERR_CAUSAL: return "causal must be 0 (none), 1 (top-left) or 2 (bottom-right)";
    case ATTN_ERR_WORKSPACE: return "workspace missing or smaller than the query returns";
    case ATTN_ERR_HIP: return "HIP runtime error while launching";
    case ATTN_ERR_SCALE: return "scale must be finite and > 0";
    default: return "unknown status";
  }
}

int attn_last_dispatch(char* buf, size_t n) {
  const int len = (int)std::strlen(g_dispatch);
  if (n == 0) return len;
  if (buf == nullptr) return ATTN_ERR_NULL;
  std::snprintf(buf, n, "%s", g_dispatch);
  return len;
}

size_t attn_fwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, int dtype) {
  if (check_common(B, Hq, Hkv, Sq, Sk, d, causal, 1.f, dtype) != ATTN_OK) return 0;
  if (dtype != ATTN_BF16) return 0;
  const attn::Problem p = make_problem(B, Hq, Hkv, Sq, Sk, d, causal, 1.f);
  const attn::SplitPlan sp = attn::plan_split(p);
  return sp.use ? sp.ws_bytes : attn::plan_prefill(p).ws_bytes;
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
             int Sq, int Sk, int d, int causal, float scale, int dtype, void* workspace,
             size_t workspace_bytes, void* stream) {
  // k and v are not read when there is no key
  if (q == nullptr || o == nullptr || (Sk != 0 && (k == nullptr || v == nullptr))) return ATTN_ERR_NULL;
  const int st = check_common(B, Hq, Hkv, Sq, Sk, d, causal, scale, dtype);
  if (st != ATTN_OK) return st;
  const attn::Problem p = make_problem(B, Hq, Hkv, Sq, Sk, d, causal, scale);
  hipStream_t s = (hipStream_t)stream;
  char text[512];
  hipError_t e;
  if (dtype == ATTN_F32) {
    e = attn::launch_fwd_f32(p, (const float*)q, (const float*)k, (const float*)v, (float*)o, lse, s);
    std::snprintf(text, sizeof(text), "attn_fwd: fwd_f32<d=%d> grid=(%d,%d,%d) block=128 (one row per thread, 16-key tiles)",
                  d, (Sq + 127) / 128, Hq, B);
  } else {
    const attn::SplitPlan sp = attn::plan_split(p);
    if (sp.use) {
      if (workspace_bytes < sp.ws_bytes || workspace == nullptr) return ATTN_ERR_WORKSPACE;
      e = attn::launch_fwd_split_bf16(p, sp, q, k, v, o, lse, workspace, s);
      std::snprintf(text, sizeof(text),
                    "attn_fwd: fwd_split_bf16<d=%d> grid=%d block=64 nsplit=%d keys/split=%d; combine_split<d=%d> grid=%d",
                    d, sp.nsplit * B * Hkv, sp.nsplit, sp.split_keys, d, B * Hq * Sq);
    } else {
      const attn::PrefillPlan pl = attn::plan_prefill(p);
      if (pl.ws_bytes > 0 && (workspace == nullptr || workspace_bytes < pl.ws_bytes)) return ATTN_ERR_WORKSPACE;
      e = attn::launch_fwd_prefill_bf16(p, pl, q, k, v, o, lse, workspace, s);
      std::snprintf(text, sizeof(text),
                    "attn_fwd: transpose_v<d=%d> grid=(%d,%d,%d); fwd_prefill_bf16<d=%d> grid=%d block=512 "
                    "heads/wg=%d rows/wg=%d key_tile=64 causal=%d",
                    d, (Sk + 63) / 64, Hkv, B, d, pl.total_wgs, pl.hw, pl.rows_per_wg, causal);
    }
  }
  if (e != hipSuccess) return ATTN_ERR_HIP;
  record(text);
  return ATTN_OK;
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, int dtype) {
  if (check_common(B, Hq, Hkv, Sq, Sk, d, causal, 1.f, dtype) != ATTN_OK) return 0;
  if (dtype != ATTN_BF16) return 0;
  return attn::bwd_workspace_bytes(make_problem(B, Hq, Hkv, Sq, Sk, d, causal, 1.f));
}

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal,
             float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  // k, v, dk and dv are neither read nor written when there is no key
  if (q == nullptr || o == nullptr || lse == nullptr || dout == nullptr || dq == nullptr ||
      (Sk != 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr)))
    return ATTN_ERR_NULL;
  const int st = check_common(B, Hq, Hkv, Sq, Sk, d, causal, scale, dtype);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  const attn::Problem p = make_problem(B, Hq, Hkv, Sq, Sk, d, causal, scale);
  const size_t need = attn::bwd_workspace_bytes(p);
  if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  char text[512];
  const hipError_t e = attn::launch_bwd_bf16(p, q, k, v, o, lse, dout, dq, dk, dv, workspace,
                                             (hipStream_t)stream, text, sizeof(text));
  if (e != hipSuccess) return ATTN_ERR_HIP;
  record(text);
  return ATTN_OK;
}

}  // extern "C"
