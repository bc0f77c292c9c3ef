// C ABI of libmxfp4.so: argument checks, schedule choice, the library-owned
// split-K workspace, and the launches.  Every check runs on the host before
// anything is enqueued.
#include <stdlib.h>
#include <string.h>

#include <cmath>
#include <map>
#include <mutex>
#include <string>
#include <tuple>
#include <vector>

#include "../../include/mxfp4.h"
#include "mxfp4_internal.hpp"
#include "workspace_pool.hpp"

using namespace mxfp4;

namespace {

const int64_t kMaxBytes = (int64_t)1 << 31;  // 32-bit offsets inside the kernels

// The last HIP error this thread's calls into the library met.
thread_local hipError_t t_last_hip_error = hipSuccess;

mxfp4_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return MXFP4_OK;
  t_last_hip_error = e;
  return MXFP4_ERR_HIP;
}

inline bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

inline int64_t pad_to(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

// Process-wide options (testing and fallback).
int g_quant_mode = 0;  // 0: hardware convert, 1: software encoder
std::mutex g_opt_mu;
std::string g_schedule_override;
bool g_schedule_override_set = false;

// Schedule choice: the tuned table for the shapes measured on MI355X;
// otherwise the compiled schedule of least estimated time -- the fused
// kernels with 16-row tiles (fused_cost) against the large-M kernels
// (wide_cost), the large-M kernels alone when K is too long for the fused
// ones.  The choice is remembered per shape (choose).
int tiles_of(const Schedule &s, int M, int N) {
  return (N / (16 * s.nt * s.wn)) * ((M + 16 * s.mt - 1) / (16 * s.mt));
}

bool covers(const Schedule &s, int M, int N, int K) {
  if (s.split < 1 || N % (16 * s.nt * s.wn) != 0) return false;
  if (s.rb == 8 && (M > 8 || s.mt != 1)) return false;
  const int ks = (K + 127) / 128;
  if (s.epi == 2) {
    // stream-K: every workgroup has at least one iteration and at most the
    // K steps one workgroup covers; tickets for every tile
    const int64_t T = (int64_t)tiles_of(s, M, N) * ks;
    return s.split <= kMaxStreamKGroups && s.split <= T && (T + s.split - 1) / s.split <= s.wk * s.kpw &&
           tiles_of(s, M, N) <= kMaxSplitTiles;
  }
  // the wide kernel loops over K; the others cover wk * kpw steps per split
  if (!s.wide && (ks + s.split - 1) / s.split > s.wk * s.kpw) return false;
  if (s.split > 1 && tiles_of(s, M, N) > kMaxSplitTiles) return false;
  return true;
}

bool parse_name(const char *name, Schedule *out);

// Schedules measured best on MI355X for the shapes the benchmark times
// (cold inputs, graph replay).
struct Tuned {
  int M, N, K;
  const char *name;
};
const Tuned kTuned[] = {
    {16, 3072, 1536, "mt1_nt2_wn1_wk4_kpw3_split1"},
    {32, 4096, 512, "mt1_nt2_wn1_wk4_kpw1_split1"},
    {8, 2112, 7168, "mt1_nt1_wn1_wk14_kpw4_split1_r8"},
    {64, 7168, 2048, "mt1_nt2_wn4_wk4_kpw4_split1"},
    {256, 7168, 7168, "wide_mt4_nt7_w4_d2_split1"},
    // the leaderboard's other shapes
    {4, 2880, 512, "mt1_nt2_wn1_wk4_kpw1_split1"},
    {16, 2112, 7168, "mt1_nt1_wn4_wk4_kpw4_split4"},
    {32, 2880, 512, "mt1_nt2_wn1_wk4_kpw1_split1"},
    {256, 3072, 1536, "mt2_nt2_wn3_wk4_kpw3_split1"},
    // A given quantized (mxfp4_gemm_q); the large-M entry above serves it too
    {16, 3072, 1536, "mt1_nt1_wn1_wk8_kpw2_split1_pq"},
    {32, 4096, 512, "mt1_nt2_wn1_wk4_kpw1_split1_pq"},
    {8, 2112, 7168, "mt1_nt1_wn1_wk8_kpw8_split1_pq"},
    {64, 7168, 2048, "mt4_nt2_wn1_wk4_kpw4_split1_pq"},
    {4, 2880, 512, "mt1_nt2_wn1_wk4_kpw1_split1_pq"},
    {16, 2112, 7168, "mt1_nt1_wn1_wk8_kpw8_split1_pq"},
    {32, 2880, 512, "mt1_nt2_wn1_wk4_kpw1_split1_pq"},
    {256, 3072, 1536, "mt2_nt2_wn1_wk4_kpw4_split1_pq"},
};

// Estimated cost of a large-M schedule, in log-microseconds on the same
// scale as fused_cost: lines per CU as there (A as codes, quantized by the
// launch before; B codes and scales), and a split of K across workgroups.
// Fitted like fused_cost, to every large-M schedule of eight shapes with
// M 96-256 (N 2048-14336, K 1024-14336).
double wide_cost(const Schedule &s, int M, int N, int K) {
  const int ks = (K + 127) / 128;
  const int per = (ks + s.split - 1) / s.split;
  const double rows = 16.0 * s.mt, cols = 16.0 * s.nt;
  const double wgs = (double)tiles_of(s, M, N) * s.split;
  const double lines = (rows + cols) * per * 0.5 + rows / 64.0 * per * 2.0 + cols / 32.0 * per * 2.0;
  return 2.226 + 1.2177e-4 * std::ceil(wgs / 256.0) * lines + (s.split > 1 ? 1.012 : 0.0);
}

// The large-M schedule of least estimated cost (B in registers; the
// LDS-staged variants run only when named); on equal cost, fewer waves.
// It reads A quantized by its own launch, so it also serves callers that
// need a pre-quantized schedule.
bool pick_wide(int M, int N, int K, Schedule *out, double *cost_out = nullptr) {
  bool found = false;
  Schedule best{};
  double best_cost = 0;
  for (int v = 0; v < num_gemm_variants(); ++v) {
    Schedule s;
    gemm_variant_shape(v, &s);
    if (s.wide != 1) continue;
    for (s.split = 1; s.split <= 8; ++s.split) {
      if (!covers(s, M, N, K)) continue;
      const double cost = wide_cost(s, M, N, K);
      if (!found || cost < best_cost - 1e-12 || (cost < best_cost + 1e-12 && s.wk < best.wk)) {
        found = true;
        best_cost = cost;
        best = s;
      }
    }
  }
  if (found) {
    *out = best;
    if (cost_out) *cost_out = best_cost;
  }
  return found;
}

// Estimated cost of a fused schedule, in log-microseconds.
// A CU keeps only ~64 lines (128 bytes) outstanding to L2, so a workgroup's
// time grows with the lines it requests: A rows actually present (bf16, or
// codes when A arrives quantized -- read in 64-byte halves of their lines,
// one per step, so twice the lines of their bytes), B columns and B scales,
// over its K run;
// workgroups beyond one per CU queue behind others.  A split of K across
// workgroups costs its epilogue.  The weights were fitted to cold,
// graph-replayed timings of every compiled schedule on twelve decode shapes
// (M 1-64, N 1024-14336, K 4096-14336) on MI355X; picking by this cost came
// within 8 % of the best schedule on average, left-one-shape-out.
double fused_cost(const Schedule &s, int M, int N, int K, bool quantized_a, double *pad) {
  const int ks = (K + 127) / 128;
  const int per = (ks + s.split - 1) / s.split;  // K steps of one workgroup
  const double rows = M < 16 * s.mt ? M : 16 * s.mt;
  const double cols = 16.0 * s.nt * s.wn;
  const double wgs = (double)tiles_of(s, M, N) * s.split;
  const double a_lines = rows * per * (quantized_a ? 1.0 : 2.0);
  const double lines = a_lines + cols * per * 0.5 + cols / 32.0 * per * 2.0;
  const double per_cu = std::ceil(wgs / 256.0) * lines;
  *pad = (double)(s.wk * s.kpw - per) / (s.wk * s.kpw);
  return 1.978 + 1.215e-4 * per_cu + 0.02547 * s.split + (s.split > 1 ? 0.1405 : 0.0);
}

bool pick_schedule(int M, int N, int K, Schedule *out, bool need_pq = false) {
  for (const Tuned &t : kTuned)
    if (t.M == M && t.N == N && t.K == K) {
      // an entry serves the mode it was tuned for; large-M entries serve both
      // (that kernel reads A quantized in either case)
      Schedule s;
      if (parse_name(t.name, &s) && covers(s, M, N, K) && (s.wide || s.pq == (need_pq ? 1 : 0))) {
        *out = s;
        return true;
      }
    }
  // 16-row tiles: each workgroup then stages a quarter to a half as much A
  // as a 32- or 64-row tile would, and there are more workgroups to spread
  // B over; measured best at M = 32 and 64 as well as at M = 16
  const int mt = 1;
  bool found = false;
  Schedule best{};
  double best_cost = 0, best_pad = 0;
  for (int v = 0; v < num_gemm_variants(); ++v) {
    Schedule s;
    gemm_variant_shape(v, &s);
    if (s.mt != mt || s.pq != (need_pq ? 1 : 0) || s.wide || s.epi) continue;  // atomic and stream-K: named only
    // the estimate was fitted on power-of-two column tiles; the 96- and
    // 112-column tiles serve the shapes of the table
    if ((s.nt * s.wn) & (s.nt * s.wn - 1)) continue;
    if (!need_pq && (s.rb == 8) != (M <= 8)) continue;
    for (s.split = 1; s.split <= 16; ++s.split) {
      if (!covers(s, M, N, K)) continue;
      double pad = 0;
      const double cost = fused_cost(s, M, N, K, need_pq, &pad);
      // eight waves across 256 columns: measured the best where their steps
      // cover the workgroup's K run exactly (32 x 8192 x 8192: 13.6 against
      // 20.5 us), but the estimate overrates them with idle steps (160 x 5120 x
      // 1024: 7.8 against 5.6 us), so only exact covers are offered
      if (s.wn >= 8 && pad > 0) continue;
      // equal cost: the least idle K capacity, then the most waves
      const bool better = !found || cost < best_cost - 1e-12 ||
                          (cost < best_cost + 1e-12 &&
                           (pad < best_pad - 1e-12 || (pad < best_pad + 1e-12 && s.wn * s.wk > best.wn * best.wk)));
      if (better) {
        found = true;
        best_cost = cost;
        best_pad = pad;
        best = s;
      }
    }
  }
  // The large-M kernel competes on estimated time: above 64 rows it wins
  // unless K is short, and at fewer rows when K is long and N wide enough
  // (64 x 4096 x 14336: 17.5 against 30.8 us).  K beyond what 16 splits of
  // any fused kernel cover goes to it as well, since it loops over K.
  Schedule w;
  double w_cost = 0;
  if (pick_wide(M, N, K, &w, &w_cost) && (!found || w_cost < best_cost)) {
    *out = w;
    return true;
  }
  if (!found) return false;
  *out = best;
  return true;
}

// "mt1_nt1_wn2_wk4_kpw1_split2", with "_pq" appended for the pre-quantized mode
bool parse_name(const char *name, Schedule *out) {
  int mt, nt, wn, wk, kpw, split, used = 0;
  int v;
  if (strncmp(name, "wide_", 5) == 0 || strncmp(name, "widel_", 6) == 0) {
    // wide_: B in registers; widel_: B staged through LDS
    const int lds = name[4] == 'l';
    int w, d;
    if (sscanf(name + (lds ? 6 : 5), "mt%d_nt%d_w%d_d%d_split%d%n", &mt, &nt, &w, &d, &split, &used) != 5 ||
        name[(lds ? 6 : 5) + used] != 0)
      return false;
    v = find_gemm_variant(mt, nt, 1, w, d, 1, 16, lds ? 3 : 1);
  } else {
    // "..._split<n>" with "_pq", "_r8", "_at" or "_r8_at" appended, or
    // "..._streamk<G>" with "_r8" appended
    int epi = 0;
    if (sscanf(name, "mt%d_nt%d_wn%d_wk%d_kpw%d_split%d%n", &mt, &nt, &wn, &wk, &kpw, &split, &used) != 6) {
      used = 0;
      if (sscanf(name, "mt%d_nt%d_wn%d_wk%d_kpw%d_streamk%d%n", &mt, &nt, &wn, &wk, &kpw, &split, &used) != 6)
        return false;
      epi = 2;
    }
    int pq = 0, rb = 16;
    const char *rest = name + used;
    if (strncmp(rest, "_r8", 3) == 0) {
      rb = 8;
      rest += 3;
    }
    if (strcmp(rest, "_pq") == 0 && rb == 16 && epi == 0) {
      pq = 1;
    } else if (strcmp(rest, "_at") == 0 && epi == 0) {
      epi = 1;
    } else if (*rest != 0) {
      return false;
    }
    v = find_gemm_variant(mt, nt, wn, wk, kpw, pq, rb, 0, epi);
  }
  if (v < 0 || split < 1) return false;
  gemm_variant_shape(v, out);
  out->split = split;
  return true;
}

bool parse_schedule(const std::string &name, int M, int N, int K, Schedule *out) {
  Schedule s;
  if (!parse_name(name.c_str(), &s) || !covers(s, M, N, K)) return false;
  *out = s;
  return true;
}

// The name mxfp4_set_schedule_override accepts for a schedule.
void schedule_to_name(const Schedule &s, char *buf, size_t n) {
  if (s.wide)
    snprintf(buf, n, "%s_mt%d_nt%d_w%d_d%d_split%d", s.wide == 3 ? "widel" : "wide", s.mt, s.nt, s.wk, s.kpw, s.split);
  else
    snprintf(buf, n, "mt%d_nt%d_wn%d_wk%d_kpw%d_%s%d%s%s", s.mt, s.nt, s.wn, s.wk, s.kpw,
             s.epi == 2 ? "streamk" : "split", s.split, s.pq ? "_pq" : (s.rb == 8 ? "_r8" : ""),
             s.epi == 1 ? "_at" : "");
}

// The built-in choice depends only on the shape, the form of A and the
// compiled tables, so it is made once per shape: the search costs several
// microseconds of host time, a lookup well under one.  Bounded: the memo is
// emptied when it holds 4096 shapes.
struct ChoiceMemo {
  bool ok;
  Schedule s;
};
std::mutex g_memo_mu;
std::map<std::tuple<int, int, int, bool>, ChoiceMemo> g_memo;

bool choose(int M, int N, int K, Schedule *s, bool need_pq = false) {
  {
    std::lock_guard<std::mutex> lk(g_opt_mu);
    if (g_schedule_override_set)
      return parse_schedule(g_schedule_override, M, N, K, s) && (s->pq || !need_pq);
  }
  const auto key = std::make_tuple(M, N, K, need_pq);
  {
    std::lock_guard<std::mutex> lk(g_memo_mu);
    const auto it = g_memo.find(key);
    if (it != g_memo.end()) {
      if (it->second.ok) *s = it->second.s;
      return it->second.ok;
    }
  }
  Schedule r{};
  const bool ok = pick_schedule(M, N, K, &r, need_pq);
  {
    std::lock_guard<std::mutex> lk(g_memo_mu);
    if (g_memo.size() >= 4096) g_memo.clear();
    g_memo[key] = ChoiceMemo{ok, r};
  }
  if (ok) *s = r;
  return ok;
}

mxfp4_status_t check_gemm_args(const void *A, const void *Bq, const void *Bs, const void *C, int64_t M, int64_t N,
                               int64_t K) {
  if (!A || !Bq || !Bs || !C) return MXFP4_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1) return MXFP4_ERR_INVALID_ARG;
  if (!aligned(A, 16) || !aligned(Bq, 16) || !aligned(Bs, 16) || !aligned(C, 16)) return MXFP4_ERR_INVALID_ARG;
  if (K % 64 != 0 || N % 32 != 0) return MXFP4_ERR_UNSUPPORTED;
  if (M * K * 2 >= kMaxBytes || N * K / 2 >= kMaxBytes || M * N * 2 >= kMaxBytes ||
      pad_to(N, 256) * pad_to(K / 32, 8) >= kMaxBytes)
    return MXFP4_ERR_UNSUPPORTED;
  return MXFP4_OK;
}

// Library-owned workspaces, one per (device, stream).  A new buffer starts
// zeroed (the split-K tickets); the fill is a kernel launch on the stream
// that asked for it, not a memset.  Buffers replaced by larger ones stay
// allocated (see WorkspacePool), so graphs captured before a growth keep
// valid addresses; growth needs no synchronization.
int alloc_workspace(int device, void *stream, size_t bytes, void **out) {
  (void)device;  // the calling thread's current device
  void *p = nullptr;
  if (hipError_t e = hipMalloc(&p, bytes); e != hipSuccess) {
    t_last_hip_error = e;
    return MXFP4_ERR_HIP;
  }
  if (hipError_t e = launch_zero(p, bytes, (hipStream_t)stream); e != hipSuccess) {
    (void)hipFree(p);
    t_last_hip_error = e;
    return MXFP4_ERR_HIP;
  }
  *out = p;
  return MXFP4_OK;
}

WorkspacePool<int (*)(int, void *, size_t, void **)> g_ws(alloc_workspace);

mxfp4_status_t get_workspace(size_t need, hipStream_t stream, void **out) {
  *out = nullptr;
  if (need == 0) return MXFP4_OK;
  int dev = 0;
  if (hipError_t e0 = hipGetDevice(&dev); e0 != hipSuccess) return hip_status(e0);
  return (mxfp4_status_t)g_ws.get(dev, (void *)stream, need, out);
}

// Scratch of mxfp4_gemm_noalloc: a file-scope device array, one copy per
// GPU, held until the process ends.  Host code never uses its name as an
// address: the first call on a device looks the device copy's address up
// with hipGetSymbolAddress (with that device current) and keeps it, and
// every later use goes through the kept pointer.
static __device__ __align__(256) uint8_t scratch[MXFP4_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// The current device's scratch; on the first call for a device its ticket
// prefix is cleared with a fill kernel on `stream` (no memset, no
// allocation).
mxfp4_status_t scratch_of_current_device(hipStream_t stream, void **out) {
  int dev = 0;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) return hip_status(e);
  if (dev < 0 || dev >= kMaxDevices) return MXFP4_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)); e != hipSuccess) return hip_status(e);
    if (!p) return hip_status(hipErrorInvalidSymbol);
    if (hipError_t e = launch_zero(p, kTicketBytes, stream); e != hipSuccess) return hip_status(e);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return MXFP4_OK;
}

bool sw_quant() {
  std::lock_guard<std::mutex> lk(g_opt_mu);
  return g_quant_mode == 1;
}

}  // namespace

extern "C" {

size_t mxfp4_packed_bytes(int64_t rows, int64_t K) { return rows > 0 && K > 0 ? (size_t)(rows * K / 2) : 0; }

size_t mxfp4_raw_scale_bytes(int64_t rows, int64_t K) { return rows > 0 && K > 0 ? (size_t)(rows * (K / 32)) : 0; }

size_t mxfp4_shuffled_scale_bytes(int64_t rows, int64_t K) {
  return rows > 0 && K > 0 ? (size_t)(pad_to(rows, 256) * pad_to(K / 32, 8)) : 0;
}

size_t mxfp4_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M < 1 || N < 1 || K < 1 || K % 64 != 0 || N % 32 != 0) return 0;
  Schedule s;
  if (!choose((int)M, (int)N, (int)K, &s)) return 0;
  return gemm_workspace_bytes(s, (int)M, (int)N, (int)K);
}

const char *mxfp4_status_string(mxfp4_status_t st) {
  switch (st) {
    case MXFP4_OK: return "MXFP4_OK";
    case MXFP4_ERR_INVALID_ARG: return "MXFP4_ERR_INVALID_ARG: null pointer, non-positive size or misaligned pointer";
    case MXFP4_ERR_UNSUPPORTED: return "MXFP4_ERR_UNSUPPORTED: shape not handled (needs K % 64 == 0, N % 32 == 0)";
    case MXFP4_ERR_WORKSPACE: return "MXFP4_ERR_WORKSPACE: workspace missing or too small";
    case MXFP4_ERR_HIP: return "MXFP4_ERR_HIP: a HIP call or kernel launch failed";
  }
  return "MXFP4: unknown status";
}

const char *mxfp4_last_hip_error(void) {
  return t_last_hip_error == hipSuccess ? "hipSuccess" : hipGetErrorName(t_last_hip_error);
}

const char *mxfp4_gemm_schedule_name(int64_t M, int64_t N, int64_t K) {
  static thread_local char buf[96];
  if (M < 1 || N < 1 || K < 1 || K % 64 != 0 || N % 32 != 0) return nullptr;
  Schedule s;
  if (!choose((int)M, (int)N, (int)K, &s)) return nullptr;
  schedule_to_name(s, buf, sizeof(buf));
  return buf;
}

/* Testing and fallback knobs (declared in mxfp4.h). */
mxfp4_status_t mxfp4_set_quant_mode(int mode) {
  if (mode != 0 && mode != 1) return MXFP4_ERR_INVALID_ARG;
  std::lock_guard<std::mutex> lk(g_opt_mu);
  g_quant_mode = mode;
  return MXFP4_OK;
}

mxfp4_status_t mxfp4_set_schedule_override(const char *name) {
  std::lock_guard<std::mutex> lk(g_opt_mu);
  if (!name || !*name) {
    g_schedule_override_set = false;
    g_schedule_override.clear();
    return MXFP4_OK;
  }
  Schedule probe;
  if (!parse_name(name, &probe)) return MXFP4_ERR_INVALID_ARG;
  g_schedule_override = name;
  g_schedule_override_set = true;
  return MXFP4_OK;
}

mxfp4_status_t mxfp4_quantize(const void *x_bf16, int64_t rows, int64_t K, void *q, void *scales,
                              int shuffled_scales, mxfp4_stream_t stream) {
  if (!x_bf16 || !q || !scales) return MXFP4_ERR_INVALID_ARG;
  if (rows < 1 || K < 32) return MXFP4_ERR_INVALID_ARG;
  if (!aligned(x_bf16, 16) || !aligned(q, 16)) return MXFP4_ERR_INVALID_ARG;
  if (K % 32 != 0) return MXFP4_ERR_UNSUPPORTED;
  if (rows * K * 2 >= kMaxBytes || pad_to(rows, 256) * pad_to(K / 32, 8) >= kMaxBytes) return MXFP4_ERR_UNSUPPORTED;
  hipError_t e = launch_quantize(x_bf16, rows, K, q, scales, shuffled_scales != 0, sw_quant(), (hipStream_t)stream);
  return hip_status(e);
}

mxfp4_status_t mxfp4_preshuffle_b(const void *bq, const void *bs_raw, int64_t N, int64_t K, void *bq_shuffled,
                                  void *bs_shuffled, mxfp4_stream_t stream) {
  if (!bq || !bs_raw || !bq_shuffled || !bs_shuffled) return MXFP4_ERR_INVALID_ARG;
  if (N < 1 || K < 32) return MXFP4_ERR_INVALID_ARG;
  if (!aligned(bq, 16) || !aligned(bq_shuffled, 16)) return MXFP4_ERR_INVALID_ARG;
  if (N % 16 != 0 || K % 32 != 0) return MXFP4_ERR_UNSUPPORTED;
  if (N * K / 2 >= kMaxBytes || pad_to(N, 256) * pad_to(K / 32, 8) >= kMaxBytes) return MXFP4_ERR_UNSUPPORTED;
  hipError_t e = launch_preshuffle_b(bq, bs_raw, N, K, bq_shuffled, bs_shuffled, (hipStream_t)stream);
  return hip_status(e);
}

mxfp4_status_t mxfp4_prepare_b(const void *b_bf16, int64_t N, int64_t K, void *bq_shuffled, void *bs_shuffled,
                               mxfp4_stream_t stream) {
  if (!b_bf16 || !bq_shuffled || !bs_shuffled) return MXFP4_ERR_INVALID_ARG;
  if (N < 1 || K < 32) return MXFP4_ERR_INVALID_ARG;
  if (!aligned(b_bf16, 16) || !aligned(bq_shuffled, 16)) return MXFP4_ERR_INVALID_ARG;
  if (N % 16 != 0 || K % 32 != 0) return MXFP4_ERR_UNSUPPORTED;
  if (N * K * 2 >= kMaxBytes || pad_to(N, 256) * pad_to(K / 32, 8) >= kMaxBytes) return MXFP4_ERR_UNSUPPORTED;
  hipError_t e = launch_prepare_b(b_bf16, N, K, bq_shuffled, bs_shuffled, sw_quant(), (hipStream_t)stream);
  return hip_status(e);
}

mxfp4_status_t mxfp4_gemm_ex(const void *A, const void *Bq_sh, const void *Bs_sh, void *C, int64_t M, int64_t N,
                             int64_t K, void *workspace, size_t workspace_bytes, mxfp4_stream_t stream) {
  mxfp4_status_t st = check_gemm_args(A, Bq_sh, Bs_sh, C, M, N, K);
  if (st != MXFP4_OK) return st;
  Schedule s;
  if (!choose((int)M, (int)N, (int)K, &s)) return MXFP4_ERR_UNSUPPORTED;
  const size_t need = gemm_workspace_bytes(s, (int)M, (int)N, (int)K);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned(workspace, 256))) return MXFP4_ERR_WORKSPACE;
  GemmArgs a{A, Bq_sh, Bs_sh, C, workspace, (int)M, (int)N, (int)K};
  return hip_status(launch_gemm(s, a, sw_quant(), (hipStream_t)stream));
}

mxfp4_status_t mxfp4_gemm(const void *A, const void *Bq_sh, const void *Bs_sh, void *C, int64_t M, int64_t N,
                          int64_t K, mxfp4_stream_t stream) {
  mxfp4_status_t st = check_gemm_args(A, Bq_sh, Bs_sh, C, M, N, K);
  if (st != MXFP4_OK) return st;
  Schedule s;
  if (!choose((int)M, (int)N, (int)K, &s)) return MXFP4_ERR_UNSUPPORTED;
  const size_t need = gemm_workspace_bytes(s, (int)M, (int)N, (int)K);
  void *ws = nullptr;
  st = get_workspace(need, (hipStream_t)stream, &ws);
  if (st != MXFP4_OK) return st;
  GemmArgs a{A, Bq_sh, Bs_sh, C, ws, (int)M, (int)N, (int)K};
  return hip_status(launch_gemm(s, a, sw_quant(), (hipStream_t)stream));
}

mxfp4_status_t mxfp4_gemm_noalloc(const void *A, const void *Bq_sh, const void *Bs_sh, void *C, int64_t M, int64_t N,
                                  int64_t K, mxfp4_stream_t stream) {
  mxfp4_status_t st = check_gemm_args(A, Bq_sh, Bs_sh, C, M, N, K);
  if (st != MXFP4_OK) return st;
  Schedule s;
  if (!choose((int)M, (int)N, (int)K, &s)) return MXFP4_ERR_UNSUPPORTED;
  const size_t need = gemm_workspace_bytes(s, (int)M, (int)N, (int)K);
  if (need > (size_t)MXFP4_NOALLOC_SCRATCH_BYTES) return MXFP4_ERR_WORKSPACE;
  void *ws = nullptr;
  if (need > 0) {
    st = scratch_of_current_device((hipStream_t)stream, &ws);
    if (st != MXFP4_OK) return st;
  }
  GemmArgs a{A, Bq_sh, Bs_sh, C, ws, (int)M, (int)N, (int)K};
  return hip_status(launch_gemm(s, a, sw_quant(), (hipStream_t)stream));
}

mxfp4_status_t mxfp4_gemm_q(const void *Aq, const void *As_shuffled, const void *Bq_sh, const void *Bs_sh, void *C,
                            int64_t M, int64_t N, int64_t K, mxfp4_stream_t stream) {
  if (!As_shuffled) return MXFP4_ERR_INVALID_ARG;
  mxfp4_status_t st = check_gemm_args(Aq, Bq_sh, Bs_sh, C, M, N, K);
  if (st != MXFP4_OK) return st;
  if (pad_to(M, 256) * pad_to(K / 32, 8) >= kMaxBytes) return MXFP4_ERR_UNSUPPORTED;
  Schedule s;
  if (!choose((int)M, (int)N, (int)K, &s, true)) return MXFP4_ERR_UNSUPPORTED;
  void *ws = nullptr;
  st = get_workspace(gemm_workspace_bytes(s, (int)M, (int)N, (int)K), (hipStream_t)stream, &ws);
  if (st != MXFP4_OK) return st;
  GemmArgs a{nullptr, Bq_sh, Bs_sh, C, ws, (int)M, (int)N, (int)K};
  a.Aq = Aq;
  a.As = As_shuffled;
  return hip_status(launch_gemm(s, a, false, (hipStream_t)stream));
}

const char *mxfp4_gemm_q_schedule_name(int64_t M, int64_t N, int64_t K) {
  static thread_local char buf[96];
  if (M < 1 || N < 1 || K < 64 || K % 64 != 0 || N % 32 != 0) return nullptr;
  Schedule s;
  if (!choose((int)M, (int)N, (int)K, &s, true)) return nullptr;
  schedule_to_name(s, buf, sizeof(buf));
  return buf;
}

size_t mxfp4_list_schedules(int64_t M, int64_t N, int64_t K, int quantized_a, char *buf, size_t cap) {
  if (cap > 0 && buf) buf[0] = 0;
  if (M < 1 || N < 1 || K < 64 || K % 64 != 0 || N % 32 != 0) return 0;
  if (M * K * 2 >= kMaxBytes || N * K / 2 >= kMaxBytes || M * N * 2 >= kMaxBytes ||
      pad_to(N, 256) * pad_to(K / 32, 8) >= kMaxBytes)
    return 0;
  std::string out;
  char name[96];
  auto add = [&](const Schedule &s) {
    schedule_to_name(s, name, sizeof(name));
    out += name;
    out += '\n';
  };
  const bool q = quantized_a != 0;
  const int ks = (int)((K + 127) / 128);  // a split beyond this leaves workgroups without a step
  for (int v = 0; v < num_gemm_variants(); ++v) {  // fused kernels, ticketed epilogue
    Schedule s;
    gemm_variant_shape(v, &s);
    if (s.wide || s.epi || s.pq != (q ? 1 : 0)) continue;
    for (s.split = 1; s.split <= 16 && s.split <= ks; ++s.split)
      if (covers(s, (int)M, (int)N, (int)K)) add(s);
  }
  for (int v = 0; v < num_gemm_variants(); ++v) {  // large-M kernels
    Schedule s;
    gemm_variant_shape(v, &s);
    if (!s.wide) continue;
    for (s.split = 1; s.split <= 8 && s.split <= ks; ++s.split)
      if (covers(s, (int)M, (int)N, (int)K)) add(s);
  }
  if (cap > 0 && buf) {
    const size_t n = out.size() < cap - 1 ? out.size() : cap - 1;
    memcpy(buf, out.data(), n);
    buf[n] = 0;
  }
  return out.size();
}

mxfp4_status_t mxfp4_reserve(int64_t M, int64_t N, int64_t K, mxfp4_stream_t stream) {
  if (M < 1 || N < 1 || K < 1) return MXFP4_ERR_INVALID_ARG;
  if (K % 64 != 0 || N % 32 != 0) return MXFP4_ERR_UNSUPPORTED;
  Schedule s;
  if (!choose((int)M, (int)N, (int)K, &s)) return MXFP4_ERR_UNSUPPORTED;
  void *ws = nullptr;
  return get_workspace(gemm_workspace_bytes(s, (int)M, (int)N, (int)K), (hipStream_t)stream, &ws);
}

}  // extern "C"
