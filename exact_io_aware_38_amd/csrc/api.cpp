// C ABI of the attention library: argument validation, kernel selection,
// workspace sizing and the per-thread dispatch record (see include/attn.h).
#include "attn.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <cstdint>
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

// Alignment contract of include/attn.h: tensors and workspaces move in
// 16-byte vectors, lse and FP8 scale arrays in 4-byte words. NULL passes (the
// NULL checks come first and are per entry point).
bool misaligned(const void* p, uintptr_t a) { return p != nullptr && ((uintptr_t)p & (a - 1)) != 0; }
template <typename... P>
bool any16(P... p) { return (misaligned(p, 16) || ...); }

int check_common(int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, float scale, int dtype) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Sq < 1 || Sk < 0) return ATTN_ERR_SHAPE;
  // every element offset must fit the kernels' 64-bit arithmetic and every
  // per-head index their 32-bit arithmetic
  const long long rows_q = (long long)B * Hq * Sq;
  const long long rows_k = (long long)B * Hkv * (long long)Sk;
  if (rows_q > (1LL << 31) - 1 || rows_k > (1LL << 31) - 1) return ATTN_ERR_SHAPE;
  // the buffer loads take a head's byte range as a 32-bit count (2^24 rows of
  // 256 bytes at d = 128 would already wrap it)
  if (Sq >= (1 << 24) || Sk >= (1 << 24)) return ATTN_ERR_SHAPE;
  if (Hq % Hkv != 0) return ATTN_ERR_GQA;
  if (d != 64 && d != 128) return ATTN_ERR_HEADDIM;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (causal < 0 || causal > 2) return ATTN_ERR_CAUSAL;
  if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_ERR_SCALE;
  return ATTN_OK;
}

// Dropout parameters of the generator's contract (include/attn.h).
int make_drop(float p, unsigned long long seed, unsigned int offset, attn::DropParams& dp) {
  if (!std::isfinite(p) || p < 0.f || p >= 1.f) return ATTN_ERR_DROPOUT;
  const long thr = std::lrint(p * 256.f);
  if (thr > 255) return ATTN_ERR_DROPOUT;
  dp.seed_lo = (uint32_t)seed;
  dp.seed_hi = (uint32_t)(seed >> 32);
  dp.offset = offset;
  dp.thr = (uint32_t)thr;
  dp.scale = 256.f / (float)(256 - thr);
  return ATTN_OK;
}

attn::Problem make_problem(int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, float scale) {
  return attn::Problem{B, Hq, Hkv, Sq, Sk, d, causal, scale, Sq, Sk};
}

// Packed variable-length batches: host arrays of B+1 offsets, starting at 0
// and non-decreasing. Each sequence is then validated as a dense problem of
// batch 1 (with at least one row, so that the per-sequence checks apply).
int check_varlen(const int* cu_q, const int* cu_k, int B, int Hq, int Hkv, int d, int causal, float scale,
                 int dtype) {
  if (cu_q == nullptr || cu_k == nullptr) return ATTN_ERR_NULL;
  if (B < 1 || Hq < 1 || Hkv < 1) return ATTN_ERR_SHAPE;
  if (cu_q[0] != 0 || cu_k[0] != 0) return ATTN_ERR_SHAPE;
  for (int b = 0; b < B; ++b)
    if (cu_q[b + 1] < cu_q[b] || cu_k[b + 1] < cu_k[b]) return ATTN_ERR_SHAPE;
  // every packed row index of a head must fit the kernels' 32-bit arithmetic
  if ((long long)Hq * cu_q[B] > (1LL << 31) - 1 || (long long)Hkv * cu_k[B] > (1LL << 31) - 1)
    return ATTN_ERR_SHAPE;
  for (int b = 0; b < B; ++b) {
    const int st = check_common(1, Hq, Hkv, std::max(1, cu_q[b + 1] - cu_q[b]), cu_k[b + 1] - cu_k[b], d,
                                causal, scale, dtype);
    if (st != ATTN_OK) return st;
  }
  return ATTN_OK;
}

// Sequence b of a packed batch as a dense problem of batch 1 whose head
// strides are the packed totals (the data pointers are advanced to its first
// row by the caller).
attn::Problem seq_problem(const int* cu_q, const int* cu_k, int B, int b, int Hq, int Hkv, int d, int causal,
                          float scale) {
  attn::Problem p = make_problem(1, Hq, Hkv, cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b], d, causal, scale);
  p.hsq = cu_q[B];
  p.hsk = cu_k[B];
  return p;
}

// The whole packed batch as the launchers see it: batch 1, the packed totals
// as head strides (lengths come per sequence).
attn::Problem packed_problem(const int* cu_q, const int* cu_k, int B, int Hq, int Hkv, int d, int causal,
                             float scale) {
  attn::Problem p = make_problem(1, Hq, Hkv, 0, 0, d, causal, scale);
  p.hsq = cu_q[B];
  p.hsk = cu_k[B];
  return p;
}

// The sequences that `keep` selects, most work first, so that each packed
// launch starts its largest tiles first.
template <typename Keep>
std::vector<attn::SeqSpan> packed_order(const int* cu_q, const int* cu_k, int B, Keep keep) {
  std::vector<attn::SeqSpan> v;
  for (int b = 0; b < B; ++b) {
    const attn::SeqSpan sp{cu_q[b], cu_k[b], cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]};
    if (keep(sp)) v.push_back(sp);
  }
  std::stable_sort(v.begin(), v.end(), [](const attn::SeqSpan& a, const attn::SeqSpan& b) {
    return (long long)(a.sq + 1) * (a.sk + 1) > (long long)(b.sq + 1) * (b.sk + 1);
  });
  return v;
}

size_t fwd_ws(const attn::Problem& p, int dtype) {
  if (dtype != ATTN_BF16) return 0;
  const attn::SplitPlan sp = attn::plan_split(p);
  return sp.use ? sp.ws_bytes : attn::plan_prefill(p).ws_bytes;
}

// The forward's kernel selection and launch for one validated problem; the
// workspace must hold fwd_ws(p, dtype) bytes.
hipError_t fwd_launch(const attn::Problem& p, int dtype, const void* q, const void* k, const void* v, void* o,
                      float* lse, void* workspace, hipStream_t s, char* text, size_t text_n) {
  hipError_t e;
  if (dtype == ATTN_F32) {
    e = attn::launch_fwd_f32(p, (const float*)q, (const float*)k, (const float*)v, (float*)o, lse, s);
    std::snprintf(text, text_n, "fwd_f32<d=%d> grid=(%d,%d,%d) block=128 (one row per thread, 16-key tiles)",
                  p.d, (p.Sq + 127) / 128, p.Hq, p.B);
    return e;
  }
  const attn::SplitPlan sp = attn::plan_split(p);
  if (sp.use) {
    e = attn::launch_fwd_split_bf16(p, sp, q, k, v, o, lse, workspace, s);
    std::snprintf(text, text_n,
                  "fwd_split_bf16<d=%d> grid=%d block=64 nsplit=%d keys/split=%d; combine_split<d=%d> grid=%d",
                  p.d, sp.nsplit * p.B * p.Hkv, sp.nsplit, sp.split_keys, p.d, p.B * p.Hq * p.Sq);
    return e;
  }
  const attn::PrefillPlan pl = attn::plan_prefill(p);
  e = attn::launch_fwd_prefill_bf16(p, pl, q, k, v, o, lse, workspace, s);
  const int poly = p.d == 128 ? attn::exp2_poly_every() : 0;
  std::snprintf(text, text_n,
                "fwd_prefill_bf16<d=%d> grid=%d block=512 heads/wg=%d rows/wg=%d key_tile=64 causal=%d%s",
                p.d, pl.total_wgs, pl.hw, pl.rows_per_wg, p.causal,
                poly == 4 ? " exp2=poly every 4th" : poly == 2 ? " exp2=poly every 2nd" : "");
  return e;
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
    case ATTN_ERR_DROPOUT: return "dropout probability must lie in [0, 1) and round below 256/256";
    case ATTN_ERR_ALIGN: return "misaligned pointer: tensors and workspace need 16 bytes, lse and scales 4";
    case ATTN_ERR_SCRATCH: return "problem needs more scratch than the library's static buffer holds";
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
  return fwd_ws(make_problem(B, Hq, Hkv, Sq, Sk, d, causal, 1.f), dtype);
}

int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
             int Sq, int Sk, int d, int causal, float scale, int dtype, void* workspace,
             size_t workspace_bytes, void* stream) {
  // k and v are not read when there is no key
  if (q == nullptr || o == nullptr || (Sk != 0 && (k == nullptr || v == nullptr))) return ATTN_ERR_NULL;
  const int st = check_common(B, Hq, Hkv, Sq, Sk, d, causal, scale, dtype);
  if (st != ATTN_OK) return st;
  if (any16(q, k, v, o, workspace) || misaligned(lse, 4)) return ATTN_ERR_ALIGN;
  const attn::Problem p = make_problem(B, Hq, Hkv, Sq, Sk, d, causal, scale);
  if (fwd_ws(p, dtype) > 0 && (workspace == nullptr || workspace_bytes < fwd_ws(p, dtype))) return ATTN_ERR_WORKSPACE;
  char text[480], line[512];
  if (fwd_launch(p, dtype, q, k, v, o, lse, workspace, (hipStream_t)stream, text, sizeof(text)) != hipSuccess)
    return ATTN_ERR_HIP;
  std::snprintf(line, sizeof(line), "attn_fwd: %s", text);
  record(line);
  return ATTN_OK;
}

static_assert(attn::NOALLOC_SCRATCH_BYTES == ATTN_NOALLOC_SCRATCH_BYTES, "one scratch size");

int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                     int Sq, int Sk, int d, int causal, float scale, int dtype, void* stream) {
  if (q == nullptr || o == nullptr || (Sk != 0 && (k == nullptr || v == nullptr))) return ATTN_ERR_NULL;
  const int st = check_common(B, Hq, Hkv, Sq, Sk, d, causal, scale, dtype);
  if (st != ATTN_OK) return st;
  if (any16(q, k, v, o) || misaligned(lse, 4)) return ATTN_ERR_ALIGN;
  const attn::Problem p = make_problem(B, Hq, Hkv, Sq, Sk, d, causal, scale);
  const size_t need = fwd_ws(p, dtype);
  if (need > attn::NOALLOC_SCRATCH_BYTES) return ATTN_ERR_SCRATCH;
  void* scratch = nullptr;
  if (need > 0 && attn::noalloc_scratch(&scratch) != hipSuccess) return ATTN_ERR_HIP;
  char text[440], line[512];
  if (fwd_launch(p, dtype, q, k, v, o, lse, scratch, (hipStream_t)stream, text, sizeof(text)) != hipSuccess)
    return ATTN_ERR_HIP;
  std::snprintf(line, sizeof(line), "attn_fwd_noalloc%s: %s", need > 0 ? " (static scratch)" : "", text);
  record(line);
  return ATTN_OK;
}

size_t attn_bwd_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, int dtype) {
  if (check_common(B, Hq, Hkv, Sq, Sk, d, causal, 1.f, dtype) != ATTN_OK) return 0;
  if (dtype != ATTN_BF16) return 0;
  return attn::bwd_workspace_bytes(make_problem(B, Hq, Hkv, Sq, Sk, d, causal, 1.f));
}

namespace {
// attn_bwd and attn_bwd_fused: the two-kernel pass or the single pass with
// atomically accumulated dQ.
int bwd_entry(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
              void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, float scale,
              int dtype, void* workspace, size_t workspace_bytes, void* stream, bool fused) {
  // k, v, dk and dv are neither read nor written when there is no key
  if (q == nullptr || o == nullptr || lse == nullptr || dout == nullptr || dq == nullptr ||
      (Sk != 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr)))
    return ATTN_ERR_NULL;
  const int st = check_common(B, Hq, Hkv, Sq, Sk, d, causal, scale, dtype);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  if (any16(q, k, v, o, dout, dq, dk, dv, workspace) || misaligned(lse, 4)) return ATTN_ERR_ALIGN;
  const attn::Problem p = make_problem(B, Hq, Hkv, Sq, Sk, d, causal, scale);
  const size_t need = fused ? attn::bwd_fused_workspace_bytes(p) : attn::bwd_workspace_bytes(p);
  if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  char text[512];
  const hipError_t e = attn::launch_bwd_bf16(p, q, k, v, o, lse, dout, dq, dk, dv, workspace, fused,
                                             (hipStream_t)stream, text, sizeof(text));
  if (e != hipSuccess) return ATTN_ERR_HIP;
  record(text);
  return ATTN_OK;
}
}  // namespace

int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal,
             float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_entry(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Sq, Sk, d, causal, scale, dtype, workspace,
                   workspace_bytes, stream, false);
}

size_t attn_bwd_fused_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal, int dtype) {
  if (check_common(B, Hq, Hkv, Sq, Sk, d, causal, 1.f, dtype) != ATTN_OK) return 0;
  if (dtype != ATTN_BF16) return 0;
  return attn::bwd_fused_workspace_bytes(make_problem(B, Hq, Hkv, Sq, Sk, d, causal, 1.f));
}

int attn_bwd_fused(const void* q, const void* k, const void* v, const void* o, const float* lse, const void* dout,
                   void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal,
                   float scale, int dtype, void* workspace, size_t workspace_bytes, void* stream) {
  return bwd_entry(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Sq, Sk, d, causal, scale, dtype, workspace,
                   workspace_bytes, stream, true);
}

size_t attn_fwd_varlen_workspace_bytes(const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq,
                                       int Hkv, int d, int causal, int dtype) {
  if (check_varlen(cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, d, causal, 1.f, dtype) != ATTN_OK) return 0;
  size_t need = 0;       // only the sequences launched one by one on the split path use it
  for (int b = 0; b < B; ++b) {
    const attn::Problem p = seq_problem(cu_seqlens_q, cu_seqlens_k, B, b, Hq, Hkv, d, causal, 1.f);
    if (p.Sq > 0) need = std::max(need, fwd_ws(p, dtype));
  }
  return need;
}

int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse, const int* cu_seqlens_q,
                    const int* cu_seqlens_k, int B, int Hq, int Hkv, int d, int causal, float scale, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_varlen(cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, d, causal, scale, dtype);
  if (st != ATTN_OK) return st;
  const bool any_q = cu_seqlens_q[B] > 0, any_k = cu_seqlens_k[B] > 0;
  if ((any_q && (q == nullptr || o == nullptr)) || (any_q && any_k && (k == nullptr || v == nullptr)))
    return ATTN_ERR_NULL;
  if (any16(q, k, v, o, workspace) || misaligned(lse, 4)) return ATTN_ERR_ALIGN;
  const size_t need = attn_fwd_varlen_workspace_bytes(cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, d, causal, dtype);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  const hipStream_t s = (hipStream_t)stream;
  const size_t es = dtype == ATTN_F32 ? 4 : 2;
  char text[512] = "";
  int single = 0, packed = 0, launches = 0;
  // fp32, and decode-shaped bf16 sequences (split over the keys), one launch each
  for (int b = 0; b < B; ++b) {
    const attn::Problem p = seq_problem(cu_seqlens_q, cu_seqlens_k, B, b, Hq, Hkv, d, causal, scale);
    if (p.Sq == 0 || (dtype == ATTN_BF16 && !attn::plan_split(p).use)) continue;
    const size_t q0 = (size_t)cu_seqlens_q[b], k0 = (size_t)cu_seqlens_k[b];
    const char* kb = p.Sk > 0 ? (const char*)k + k0 * d * es : nullptr;
    const char* vb = p.Sk > 0 ? (const char*)v + k0 * d * es : nullptr;
    if (fwd_launch(p, dtype, (const char*)q + q0 * d * es, kb, vb, (char*)o + q0 * d * es,
                   lse != nullptr ? lse + q0 : nullptr, workspace, s, text, sizeof(text)) != hipSuccess)
      return ATTN_ERR_HIP;
    ++single;
  }
  // every other bf16 sequence: tiled prefill, up to SEQ_MAX sequences per launch
  if (dtype == ATTN_BF16) {
    const attn::Problem pp = packed_problem(cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, d, causal, scale);
    const std::vector<attn::SeqSpan> seqs =
        packed_order(cu_seqlens_q, cu_seqlens_k, B, [&](const attn::SeqSpan& sp) {
          attn::Problem p1 = pp;
          p1.Sq = sp.sq;
          p1.Sk = sp.sk;
          return sp.sq > 0 && !attn::plan_split(p1).use;
        });
    for (size_t i = 0; i < seqs.size(); i += attn::SEQ_MAX) {
      const int n = (int)std::min<size_t>(attn::SEQ_MAX, seqs.size() - i);
      if (attn::launch_fwd_prefill_bf16_packed(pp, seqs.data() + i, n, q, k, v, o, lse, s, text, sizeof(text)) !=
          hipSuccess)
        return ATTN_ERR_HIP;
      packed += n;
      ++launches;
    }
  }
  char summary[512];
  std::snprintf(summary, sizeof(summary),
                "attn_fwd_varlen: %d sequences of %d launched: %d in %d packed launches, %d one by one; last: %s",
                single + packed, B, packed, launches, single, text);
  record(summary);
  return ATTN_OK;
}

size_t attn_bwd_varlen_workspace_bytes(const int* cu_seqlens_q, const int* cu_seqlens_k, int B, int Hq,
                                       int Hkv, int d, int causal, int dtype) {
  if (check_varlen(cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, d, causal, 1.f, dtype) != ATTN_OK) return 0;
  if (dtype != ATTN_BF16) return 0;
  // the lse2/D blocks of every sequence (each packed launch reuses the start of it)
  const attn::Problem pp = packed_problem(cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, d, causal, 1.f);
  const std::vector<attn::SeqSpan> seqs =
      packed_order(cu_seqlens_q, cu_seqlens_k, B, [](const attn::SeqSpan& sp) { return sp.sq > 0; });
  return attn::bwd_packed_workspace_bytes(pp, seqs.data(), (int)seqs.size());
}

int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, const int* cu_seqlens_q,
                    const int* cu_seqlens_k, int B, int Hq, int Hkv, int d, int causal, float scale, int dtype,
                    void* workspace, size_t workspace_bytes, void* stream) {
  const int st = check_varlen(cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, d, causal, scale, dtype);
  if (st != ATTN_OK) return st;
  if (dtype != ATTN_BF16) return ATTN_ERR_DTYPE;
  const bool any_q = cu_seqlens_q[B] > 0, any_k = cu_seqlens_k[B] > 0;
  if ((any_q && (q == nullptr || o == nullptr || lse == nullptr || dout == nullptr || dq == nullptr)) ||
      (any_k && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr)))
    return ATTN_ERR_NULL;
  if (any16(q, k, v, o, dout, dq, dk, dv, workspace) || misaligned(lse, 4)) return ATTN_ERR_ALIGN;
  const size_t need = attn_bwd_varlen_workspace_bytes(cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, d, causal, dtype);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  // a sequence with keys but no query still takes part: its dK and dV rows
  // are written as zeros (no query tile reaches them)
  const attn::Problem pp = packed_problem(cu_seqlens_q, cu_seqlens_k, B, Hq, Hkv, d, causal, scale);
  const std::vector<attn::SeqSpan> seqs = packed_order(
      cu_seqlens_q, cu_seqlens_k, B, [](const attn::SeqSpan& sp) { return sp.sq > 0 || sp.sk > 0; });
  char text[512] = "";
  int launches = 0;
  for (size_t i = 0; i < seqs.size(); i += attn::SEQ_MAX) {
    const int n = (int)std::min<size_t>(attn::SEQ_MAX, seqs.size() - i);
    if (attn::launch_bwd_bf16_packed(pp, seqs.data() + i, n, q, k, v, o, lse, dout, dq, dk, dv, workspace,
                                     (hipStream_t)stream, text, sizeof(text)) != hipSuccess)
      return ATTN_ERR_HIP;
    ++launches;
  }
  char summary[512];
  std::snprintf(summary, sizeof(summary), "attn_bwd_varlen: %d sequences of %d launched in %d packed launches; last: %s",
                (int)seqs.size(), B, launches, text);
  record(summary);
  return ATTN_OK;
}
int attn_fwd_dropout(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq, int Hkv,
                     int Sq, int Sk, int d, int causal, float scale, float dropout_p, unsigned long long seed,
                     unsigned int offset, void* stream) {
  if (q == nullptr || o == nullptr || (Sk != 0 && (k == nullptr || v == nullptr))) return ATTN_ERR_NULL;
  int st = check_common(B, Hq, Hkv, Sq, Sk, d, causal, scale, ATTN_BF16);
  if (st != ATTN_OK) return st;
  if (any16(q, k, v, o) || misaligned(lse, 4)) return ATTN_ERR_ALIGN;
  attn::Problem p = make_problem(B, Hq, Hkv, Sq, Sk, d, causal, scale);
  st = make_drop(dropout_p, seed, offset, p.drop);
  if (st != ATTN_OK) return st;
  // the tiled prefill for every shape (the split-key decode has no dropout)
  const attn::PrefillPlan pl = attn::plan_prefill(p);
  if (attn::launch_fwd_prefill_bf16(p, pl, q, k, v, o, lse, nullptr, (hipStream_t)stream) != hipSuccess)
    return ATTN_ERR_HIP;
  char line[512];
  std::snprintf(line, sizeof(line),
                "attn_fwd_dropout: fwd_prefill<d=%d>%s grid=%d (%d query rows x %d heads per workgroup); "
                "keep when byte >= %u of 256",
                d, p.drop.thr ? " with dropout" : "", pl.total_wgs, pl.rows_per_wg, pl.hw, p.drop.thr);
  record(line);
  return ATTN_OK;
}

int attn_bwd_dropout(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Sq, int Sk,
                     int d, int causal, float scale, float dropout_p, unsigned long long seed, unsigned int offset,
                     void* workspace, size_t workspace_bytes, void* stream) {
  if (q == nullptr || o == nullptr || lse == nullptr || dout == nullptr || dq == nullptr ||
      (Sk != 0 && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr)))
    return ATTN_ERR_NULL;
  int st = check_common(B, Hq, Hkv, Sq, Sk, d, causal, scale, ATTN_BF16);
  if (st != ATTN_OK) return st;
  if (any16(q, k, v, o, dout, dq, dk, dv, workspace) || misaligned(lse, 4)) return ATTN_ERR_ALIGN;
  attn::Problem p = make_problem(B, Hq, Hkv, Sq, Sk, d, causal, scale);
  st = make_drop(dropout_p, seed, offset, p.drop);
  if (st != ATTN_OK) return st;
  const size_t need = attn::bwd_workspace_bytes(p);
  if (workspace == nullptr || workspace_bytes < need) return ATTN_ERR_WORKSPACE;
  char text[448], line[512];
  if (attn::launch_bwd_bf16(p, q, k, v, o, lse, dout, dq, dk, dv, workspace, false, (hipStream_t)stream, text,
                            sizeof(text)) != hipSuccess)
    return ATTN_ERR_HIP;
  std::snprintf(line, sizeof(line), "attn_bwd_dropout (keep when byte >= %u of 256): %s", p.drop.thr, text);
  record(line);
  return ATTN_OK;
}

int attn_dropout_mask(unsigned char* keep, int B, int Hq, int Sq, int Sk, float dropout_p,
                      unsigned long long seed, unsigned int offset, void* stream) {
  if (B < 1 || Hq < 1 || Sq < 1 || Sk < 0) return ATTN_ERR_SHAPE;
  if ((long long)B * Hq > (1LL << 31) - 1 || Sq >= (1 << 24) || Sk >= (1 << 24)) return ATTN_ERR_SHAPE;
  if (keep == nullptr && Sk > 0) return ATTN_ERR_NULL;
  attn::Problem p = make_problem(B, Hq, Hq, Sq, Sk, 64, 0, 1.f);
  const int st = make_drop(dropout_p, seed, offset, p.drop);
  if (st != ATTN_OK) return st;
  if (attn::launch_dropout_mask(p, keep, (hipStream_t)stream) != hipSuccess) return ATTN_ERR_HIP;
  char line[160];
  std::snprintf(line, sizeof(line), "attn_dropout_mask: B=%d Hq=%d Sq=%d Sk=%d, keep when byte >= %u of 256", B, Hq,
                Sq, Sk, p.drop.thr);
  record(line);
  return ATTN_OK;
}

int attn_fp8_padded_keys(int Sk) {
  if (Sk < 0 || Sk >= (1 << 24)) return ATTN_ERR_SHAPE;
  return attn::fp8_padded_keys(Sk);
}

int attn_mxfp8_quantize_rows(const void* x, void* codes, void* scales, long long rows, int d, void* stream) {
  if (rows < 0) return ATTN_ERR_SHAPE;
  if (d != 128) return ATTN_ERR_HEADDIM;
  if (rows > (1LL << 31) - 1) return ATTN_ERR_SHAPE;
  if (rows > 0 && (x == nullptr || codes == nullptr || scales == nullptr)) return ATTN_ERR_NULL;
  if (any16(x, codes)) return ATTN_ERR_ALIGN;
  if (attn::launch_mx_quant_rows(x, codes, scales, rows, d, (hipStream_t)stream) != hipSuccess) return ATTN_ERR_HIP;
  char line[128];
  std::snprintf(line, sizeof(line), "attn_mxfp8_quantize_rows: %lld rows of d=%d", rows, d);
  record(line);
  return ATTN_OK;
}

int attn_mxfp8_quantize_vt(const void* v, void* vt_codes, void* vt_scales, int BH, int Sk, int d, void* stream) {
  if (BH < 1 || Sk < 0 || Sk >= (1 << 24)) return ATTN_ERR_SHAPE;
  if ((long long)BH * Sk > (1LL << 31) - 1) return ATTN_ERR_SHAPE;
  if (d != 128) return ATTN_ERR_HEADDIM;
  if (Sk > 0 && (v == nullptr || vt_codes == nullptr || vt_scales == nullptr)) return ATTN_ERR_NULL;
  if (any16(v, vt_codes)) return ATTN_ERR_ALIGN;
  if (attn::launch_mx_quant_vt(v, vt_codes, vt_scales, BH, Sk, d, (hipStream_t)stream) != hipSuccess)
    return ATTN_ERR_HIP;
  char line[128];
  std::snprintf(line, sizeof(line), "attn_mxfp8_quantize_vt: %d heads x %d keys of d=%d (padded to %d)", BH, Sk, d,
                attn::fp8_padded_keys(Sk));
  record(line);
  return ATTN_OK;
}

size_t attn_fwd_fp8_workspace_bytes(int B, int Hq, int Hkv, int Sq, int Sk, int d, int causal) {
  if (check_common(B, Hq, Hkv, Sq, Sk, d, causal, 1.f, ATTN_BF16) != ATTN_OK || d != 128) return 0;
  return attn::fp8_workspace_bytes(make_problem(B, Hq, Hkv, Sq, Sk, d, causal, 1.f));
}

int attn_fwd_fp8(const void* q8, const void* q_scales, const void* k8, const void* k_scales, const void* vt8,
                 const void* vt_scales, void* o, float* lse, int B, int Hq, int Hkv, int Sq, int Sk, int d,
                 int causal, float scale, void* workspace, size_t workspace_bytes, void* stream) {
  if (q8 == nullptr || q_scales == nullptr || o == nullptr ||
      (Sk != 0 && (k8 == nullptr || k_scales == nullptr || vt8 == nullptr || vt_scales == nullptr)))
    return ATTN_ERR_NULL;
  const int st = check_common(B, Hq, Hkv, Sq, Sk, d, causal, scale, ATTN_BF16);
  if (st != ATTN_OK) return st;
  if (d != 128) return ATTN_ERR_HEADDIM;
  if (any16(q8, k8, vt8, o, workspace) || misaligned(q_scales, 4) || misaligned(k_scales, 4) ||
      misaligned(vt_scales, 4) || misaligned(lse, 4))
    return ATTN_ERR_ALIGN;
  const attn::Problem p = make_problem(B, Hq, Hkv, Sq, Sk, d, causal, scale);
  const size_t need = attn::fp8_workspace_bytes(p);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return ATTN_ERR_WORKSPACE;
  char text[400], line[480];
  if (attn::launch_fwd_fp8(p, q8, q_scales, k8, k_scales, vt8, vt_scales, o, lse, workspace, (hipStream_t)stream,
                           text, sizeof(text)) != hipSuccess)
    return ATTN_ERR_HIP;
  std::snprintf(line, sizeof(line), "attn_fwd_fp8: %s", text);
  record(line);
  return ATTN_OK;
}

}  // extern "C"
