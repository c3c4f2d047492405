// C-ABI layer of libcsa: argument validation, device check, workspace layout,
// dispatch to the kernels and the optional kernel-timing instrumentation.
// Host code only.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "internal.hpp"

namespace {

thread_local std::string g_error;

csa_status fail(csa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_error = buf;
  return st;
}

csa_status hip_fail(hipError_t e, const char* what) {
  return fail(CSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// ---------------------------------------------------------------------------
// device check (once per device)
// ---------------------------------------------------------------------------
constexpr int kMaxDevices = 64;
std::once_flag g_dev_once[kMaxDevices];
int g_dev_ok[kMaxDevices];  // 1 = gfx950, 0 = other, -1 = query failed
char g_dev_arch[kMaxDevices][64];

csa_status check_device() {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(CSA_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
  std::call_once(g_dev_once[dev], [dev]() {
    hipDeviceProp_t p;
    if (hipGetDeviceProperties(&p, dev) != hipSuccess) {
      g_dev_ok[dev] = -1;
      return;
    }
    snprintf(g_dev_arch[dev], sizeof(g_dev_arch[dev]), "%s", p.gcnArchName);
    g_dev_ok[dev] = strncmp(p.gcnArchName, "gfx950", 6) == 0 ? 1 : 0;
  });
  if (g_dev_ok[dev] == -1) return fail(CSA_ERR_HIP, "hipGetDeviceProperties failed for device %d", dev);
  if (g_dev_ok[dev] == 0)
    return fail(CSA_ERR_UNSUPPORTED, "device %d is %s; this library runs on gfx950 (MI355X) only", dev,
                g_dev_arch[dev]);
  return CSA_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
int vec_elems(csa_dtype dt) { return dt == CSA_BF16 ? 8 : 4; }
bool dtype_ok(int dt) { return dt == CSA_F32 || dt == CSA_BF16; }
size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

#define CSA_REQUIRE(cond, ...)                                   \
  do {                                                           \
    if (!(cond)) return fail(CSA_ERR_INVALID_ARG, __VA_ARGS__);  \
  } while (0)

// ---------------------------------------------------------------------------
// kernel timing
// ---------------------------------------------------------------------------
std::atomic<bool> g_timing{false};
std::mutex g_timing_mu;
struct Family {
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending;
  double ms = 0.0;
  int64_t launches = 0;
};
std::map<std::string, Family> g_families;

long scores_ld(long max_cand) { return (max_cand + 3) & ~3L; }

// Rows of more than 1024 candidates get the top-k's first radix level from
// the indexer sweep.  The one-workgroup-per-row selector costs 12-15 us per
// row however short the row; on the sweep's histogram the multi-workgroup
// selector took 32 rows of 2048 candidates from 15.0 to 4.5 us (classifying
// only) and 64 rows of up to 8192 from 18.9 to 9.4 us.
bool use_hist(long max_cand) { return max_cand > 1024; }
// ... and, for few rows, a selector that spreads each row over workgroups.
int topk_chunks(long max_cand) { return (int)((max_cand + csa::kMChunk - 1) / csa::kMChunk); }
bool use_lists(long n_queries, long max_cand) {
  const long P = topk_chunks(max_cand);
  return use_hist(max_cand) && P <= csa::kMMaxChunks && n_queries * P <= csa::kMMaxWorkgroups;
}

// Workspace layout of csa_index_topk (each area 256-byte aligned):
//   scores [n_queries, scores_ld]            fp32
//   hist   [n_queries, 2^kTopkL1Bits]        uint32   (use_hist)
//   arrive [n_queries]                       uint32   (use_lists; right after hist)
//   counts [n_queries, P, 2]                 uint32   (use_lists)
//   gt     [n_queries, P, min(kMChunk, k)]   uint64   (use_lists)
//   eq     [n_queries, P, kMChunk]           uint64   (use_lists)
//   b1g1   [n_queries, 2]                    uint32   (use_lists; the decode path that finishes rows in the MQA)
struct IndexWs {
  size_t scores = 0, hist = 0, arrive = 0, counts = 0, gt = 0, eq = 0, b1g1 = 0, total = 0;
};
IndexWs index_ws(long n_queries, long max_cand, int k) {
  using csa::ws_add;
  using csa::ws_align;
  using csa::ws_bytes;
  IndexWs w;
  size_t at = ws_align(ws_bytes(n_queries, scores_ld(max_cand), sizeof(float)));
  if (use_hist(max_cand)) {
    w.hist = at;
    at = ws_add(at, ws_bytes(n_queries, 1u << csa::kTopkL1Bits, sizeof(uint32_t)));
    w.arrive = at;  // contiguous with hist: one clear covers both
    at = ws_align(ws_add(at, use_lists(n_queries, max_cand) ? ws_bytes(n_queries, sizeof(uint32_t)) : 0));
  }
  if (use_lists(n_queries, max_cand)) {
    const size_t P = (size_t)topk_chunks(max_cand);
    const size_t gtc = (size_t)(k < csa::kMChunk ? k : csa::kMChunk);
    w.counts = at;
    at = ws_align(ws_add(at, ws_bytes(n_queries, P, 2 * sizeof(uint32_t))));
    w.gt = at;
    at = ws_align(ws_add(at, ws_bytes(n_queries, P, gtc, sizeof(uint64_t))));
    w.eq = at;
    at = ws_align(ws_add(at, ws_bytes(n_queries, P, csa::kMChunk, sizeof(uint64_t))));
    w.b1g1 = at;
    at = ws_align(ws_add(at, ws_bytes(n_queries, 2 * sizeof(uint32_t))));
  }
  w.total = at;
  return w;
}

}  // namespace

namespace csa {

bool timing_enabled() { return g_timing.load(std::memory_order_relaxed); }

void timing_record(const char* family, hipEvent_t start, hipEvent_t stop) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  g_families[family].pending.emplace_back(start, stop);
}

}  // namespace csa

extern "C" {

int csa_abi_version(void) { return CSA_ABI_VERSION; }

const char* csa_last_error(void) { return g_error.c_str(); }

csa_status csa_timing_enable(int on) {
  g_timing.store(on != 0);
  return CSA_OK;
}

csa_status csa_timing_reset(void) {
  std::lock_guard<std::mutex> lk(g_timing_mu);
  for (auto& kv : g_families) {
    for (auto& pr : kv.second.pending) {
      (void)hipEventSynchronize(pr.second);
      (void)hipEventDestroy(pr.first);
      (void)hipEventDestroy(pr.second);
    }
  }
  g_families.clear();
  return CSA_OK;
}

csa_status csa_timing_read(const char* name, double* total_ms, int64_t* launches) {
  CSA_REQUIRE(name && total_ms && launches, "csa_timing_read: null argument");
  std::lock_guard<std::mutex> lk(g_timing_mu);
  auto it = g_families.find(name);
  if (it == g_families.end()) {
    *total_ms = 0.0;
    *launches = 0;
    return CSA_OK;
  }
  Family& f = it->second;
  for (auto& pr : f.pending) {
    hipError_t e = hipEventSynchronize(pr.second);
    float ms = 0.f;
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, pr.first, pr.second);
    (void)hipEventDestroy(pr.first);
    (void)hipEventDestroy(pr.second);
    if (e != hipSuccess) {
      f.pending.clear();
      return hip_fail(e, "csa_timing_read");
    }
    f.ms += ms;
    f.launches += 1;
  }
  f.pending.clear();
  *total_ms = f.ms;
  *launches = f.launches;
  return CSA_OK;
}

csa_status csa_project(csa_dtype in_dt, csa_dtype out_dt, int64_t M, int64_t N, int64_t K,
                       const void* X, int64_t ldx, const void* Wt, int64_t ldw, void* Y,
                       int64_t ldy, void* stream) {
  CSA_REQUIRE(dtype_ok(in_dt) && dtype_ok(out_dt), "csa_project: unknown dtype");
  CSA_REQUIRE(!(in_dt == CSA_F32 && out_dt == CSA_BF16),
              "csa_project: fp32 input with bf16 output is not supported");
  CSA_REQUIRE(M > 0 && N > 0 && K > 0, "csa_project: M, N, K must be positive (got %lld, %lld, %lld)",
              (long long)M, (long long)N, (long long)K);
  CSA_REQUIRE(M <= 0x7FFFFFFF && N <= 0x7FFFFFFF && K <= 0x7FFFFFFF, "csa_project: size exceeds 2^31-1");
  CSA_REQUIRE(K % 8 == 0, "csa_project: K must be a multiple of 8 (got %lld)", (long long)K);
  CSA_REQUIRE(X && Wt && Y, "csa_project: null pointer");
  CSA_REQUIRE(aligned16(X) && aligned16(Wt) && aligned16(Y), "csa_project: pointers must be 16-byte aligned");
  const int v = vec_elems(in_dt);
  CSA_REQUIRE(ldx >= K && ldw >= K && ldy >= N, "csa_project: leading dimension smaller than row length");
  CSA_REQUIRE(ldx % v == 0 && ldw % v == 0, "csa_project: ldx/ldw must keep rows 16-byte aligned");
  CSA_REQUIRE(ldy % vec_elems(out_dt) == 0, "csa_project: ldy must keep rows 16-byte aligned");
  csa_status st = check_device();
  if (st != CSA_OK) return st;
  hipError_t e = csa::launch_gemm(in_dt, out_dt, M, N, K, X, ldx, Wt, ldw, Y, ldy, (hipStream_t)stream);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "csa_project launch");
}

csa_status csa_project_pair(csa_dtype in_dt, int64_t M, int64_t K, const void* X, int64_t ldx, csa_dtype out_dt1,
                            int64_t N1, const void* Wt1, int64_t ldw1, void* Y1, int64_t ldy1, csa_dtype out_dt2,
                            int64_t N2, const void* Wt2, int64_t ldw2, void* Y2, int64_t ldy2, void* stream) {
  CSA_REQUIRE(dtype_ok(in_dt) && dtype_ok(out_dt1) && dtype_ok(out_dt2), "csa_project_pair: unknown dtype");
  CSA_REQUIRE(!(in_dt == CSA_F32 && (out_dt1 == CSA_BF16 || out_dt2 == CSA_BF16)),
              "csa_project_pair: fp32 input with bf16 output is not supported");
  CSA_REQUIRE(M > 0 && K > 0 && N1 > 0 && N2 > 0, "csa_project_pair: M, K, N1, N2 must be positive");
  CSA_REQUIRE(M <= 0x7FFFFFFF && K <= 0x7FFFFFFF && N1 <= 0x7FFFFFFF && N2 <= 0x7FFFFFFF,
              "csa_project_pair: size exceeds 2^31-1");
  CSA_REQUIRE(K % 8 == 0, "csa_project_pair: K must be a multiple of 8 (got %lld)", (long long)K);
  CSA_REQUIRE(X && Wt1 && Y1 && Wt2 && Y2, "csa_project_pair: null pointer");
  CSA_REQUIRE(aligned16(X) && aligned16(Wt1) && aligned16(Y1) && aligned16(Wt2) && aligned16(Y2),
              "csa_project_pair: pointers must be 16-byte aligned");
  const int v = vec_elems(in_dt);
  CSA_REQUIRE(ldx >= K && ldw1 >= K && ldw2 >= K && ldy1 >= N1 && ldy2 >= N2,
              "csa_project_pair: leading dimension smaller than row length");
  CSA_REQUIRE(ldx % v == 0 && ldw1 % v == 0 && ldw2 % v == 0,
              "csa_project_pair: ldx/ldw must keep rows 16-byte aligned");
  CSA_REQUIRE(ldy1 % vec_elems(out_dt1) == 0 && ldy2 % vec_elems(out_dt2) == 0,
              "csa_project_pair: ldy must keep rows 16-byte aligned");
  csa_status st = check_device();
  if (st != CSA_OK) return st;
  hipError_t e = csa::launch_gemm_pair(in_dt, M, K, X, ldx, out_dt1, N1, Wt1, ldw1, Y1, ldy1, out_dt2, N2, Wt2, ldw2,
                                       Y2, ldy2, (hipStream_t)stream);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "csa_project_pair launch");
}

namespace {
// Workspace of csa_project_backward: W = Wt^T [K, N] (for dX); dY^T [N, M8] and X^T [K, M8] (for dWt).
struct ProjBwdLayout {
  size_t w, dyt, xt, total;
};
ProjBwdLayout proj_bwd_layout(csa_dtype dt, int64_t M, int64_t N, int64_t K, bool want_dx, bool want_dw) {
  using csa::ws_add;
  using csa::ws_align;
  using csa::ws_bytes;
  const size_t e = dt == CSA_F32 ? 4 : 2;
  const uint64_t M8 = ((uint64_t)M + 7) / 8 * 8;
  ProjBwdLayout L;
  L.w = 0;
  L.dyt = want_dx ? ws_align(ws_bytes(K, N, e)) : 0;
  L.xt = ws_add(L.dyt, want_dw ? ws_align(ws_bytes(N, M8, e)) : 0);
  L.total = ws_add(L.xt, want_dw ? ws_align(ws_bytes(K, M8, e)) : 0);
  return L;
}
}  // namespace

csa_status csa_project_backward_workspace(csa_dtype in_dt, int64_t M, int64_t N, int64_t K, int want_dx, int want_dw,
                                          size_t* bytes) {
  CSA_REQUIRE(bytes, "csa_project_backward_workspace: null bytes");
  CSA_REQUIRE(dtype_ok(in_dt), "csa_project_backward_workspace: unknown dtype");
  CSA_REQUIRE(M >= 0 && N > 0 && K > 0, "csa_project_backward_workspace: bad sizes");
  *bytes = proj_bwd_layout(in_dt, M, N, K, want_dx != 0, want_dw != 0).total;
  CSA_REQUIRE(*bytes < csa::kWorkspaceTooBig, "csa_project_backward_workspace: sizes too large");
  return CSA_OK;
}

csa_status csa_project_backward(csa_dtype in_dt, csa_dtype out_dt, int64_t M, int64_t N, int64_t K, const void* X,
                                int64_t ldx, const void* Wt, int64_t ldw, const void* dY, int64_t ldy, void* dX,
                                int64_t ld_dx, void* dWt, int64_t ld_dw, void* workspace, size_t ws_bytes,
                                void* stream) {
  CSA_REQUIRE(dtype_ok(in_dt) && dtype_ok(out_dt), "csa_project_backward: unknown dtype");
  CSA_REQUIRE(!(in_dt == CSA_F32 && out_dt == CSA_BF16),
              "csa_project_backward: (F32 in, BF16 out) is not a supported combination");
  CSA_REQUIRE(M >= 0 && N > 0 && K > 0, "csa_project_backward: M >= 0, N > 0, K > 0 required");
  CSA_REQUIRE(N % 8 == 0 && K % 8 == 0, "csa_project_backward: N and K must be multiples of 8");
  CSA_REQUIRE(dY && (dX == nullptr || Wt) && (dWt == nullptr || X), "csa_project_backward: null pointer");
  CSA_REQUIRE(dWt == nullptr || M > 0, "csa_project_backward: dWt needs M > 0");
  const int v = vec_elems(in_dt);
  CSA_REQUIRE(aligned16(X) && aligned16(Wt) && aligned16(dY) && aligned16(dX) && aligned16(dWt) &&
                  aligned16(workspace),
              "csa_project_backward: pointers must be 16-byte aligned");
  CSA_REQUIRE(ldx >= K && ldw >= K && ldy >= N && ld_dx >= K && ld_dw >= K,
              "csa_project_backward: leading dimension smaller than row length");
  CSA_REQUIRE(ldx % v == 0 && ldw % v == 0 && ldy % v == 0, "csa_project_backward: input rows must stay 16-byte aligned");
  CSA_REQUIRE(ld_dx % vec_elems(out_dt) == 0 && ld_dw % vec_elems(out_dt) == 0,
              "csa_project_backward: output rows must stay 16-byte aligned");
  const ProjBwdLayout L = proj_bwd_layout(in_dt, M, N, K, dX != nullptr, dWt != nullptr);
  CSA_REQUIRE(L.total < csa::kWorkspaceTooBig, "csa_project_backward: sizes too large");
  if (L.total > 0 && (workspace == nullptr || ws_bytes < L.total))
    return fail(CSA_ERR_WORKSPACE, "csa_project_backward: workspace needs %zu bytes (got %zu)", L.total, ws_bytes);
  csa_status st = check_device();
  if (st != CSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const int64_t M8 = (M + 7) / 8 * 8;
  hipError_t e = hipSuccess;
  if (dX && M > 0) {  // dX [M, K] = dY [M, N] . W^T, W^T stored as W = Wt^T [K, N]
    e = csa::launch_transpose(in_dt, N, K, N, Wt, ldw, ws + L.w, N, s);
    if (e == hipSuccess) e = csa::launch_gemm(in_dt, out_dt, M, K, N, dY, ldy, ws + L.w, N, dX, ld_dx, s);
    if (e != hipSuccess) return hip_fail(e, "csa_project_backward (dX) launch");
  }
  if (dWt) {  // dWt [N, K] = dY^T [N, M] . X [M, K]; contraction over the (zero-padded) tokens
    e = csa::launch_transpose(in_dt, M, N, M8, dY, ldy, ws + L.dyt, M8, s);
    if (e == hipSuccess) e = csa::launch_transpose(in_dt, M, K, M8, X, ldx, ws + L.xt, M8, s);
    if (e == hipSuccess) e = csa::launch_gemm(in_dt, out_dt, N, K, M8, ws + L.dyt, M8, ws + L.xt, M8, dWt, ld_dw, s);
    if (e != hipSuccess) return hip_fail(e, "csa_project_backward (dWt) launch");
  }
  return CSA_OK;
}

csa_status csa_compress(csa_dtype dt, int64_t n, int32_t m, int32_t c, const void* Ca,
                        const void* Cb, const void* Za, const void* Zb, int64_t ld_in,
                        const void* Ba, const void* Bb, void* Ccomp, int64_t ld_out,
                        void* stream) {
  CSA_REQUIRE(dtype_ok(dt), "csa_compress: unknown dtype");
  CSA_REQUIRE(n >= 0, "csa_compress: n must be >= 0");
  CSA_REQUIRE(m >= 1 && m <= 64, "csa_compress: m must be in [1, 64] (got %d)", m);
  CSA_REQUIRE(c > 0 && c % 4 == 0, "csa_compress: c must be a positive multiple of 4 (got %d)", c);
  if (n / m == 0) return CSA_OK;
  CSA_REQUIRE(Ca && Cb && Za && Zb && Ba && Bb && Ccomp, "csa_compress: null pointer");
  CSA_REQUIRE(aligned16(Ca) && aligned16(Cb) && aligned16(Za) && aligned16(Zb) && aligned16(Ba) &&
                  aligned16(Bb) && aligned16(Ccomp),
              "csa_compress: pointers must be 16-byte aligned");
  const int v = vec_elems(dt);
  CSA_REQUIRE(ld_in >= c && ld_out >= c, "csa_compress: leading dimension smaller than c");
  CSA_REQUIRE(ld_in % v == 0 && ld_out % v == 0, "csa_compress: leading dimensions must keep rows 16-byte aligned");
  csa_status st = check_device();
  if (st != CSA_OK) return st;
  hipError_t e = csa::launch_compress(dt, n, m, c, Ca, Cb, Za, Zb, ld_in, Ba, Bb, Ccomp, ld_out,
                                      (hipStream_t)stream);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "csa_compress launch");
}

csa_status csa_compress_backward_workspace(int64_t n, int32_t m, int32_t c, size_t* bytes) {
  CSA_REQUIRE(bytes != nullptr, "csa_compress_backward_workspace: null bytes");
  CSA_REQUIRE(n >= 0, "csa_compress_backward_workspace: n must be >= 0");
  CSA_REQUIRE(m >= 1 && m <= 16, "csa_compress_backward_workspace: m must be in [1, 16] (got %d)", m);
  CSA_REQUIRE(c > 0 && c % 4 == 0, "csa_compress_backward_workspace: c must be a positive multiple of 4");
  *bytes = csa::compress_backward_workspace_bytes(n, m, c, 0, 0, false);
  CSA_REQUIRE(*bytes < csa::kWorkspaceTooBig, "csa_compress_backward_workspace: sizes too large");
  return CSA_OK;
}

csa_status csa_compress_backward(csa_dtype dt, int64_t n, int32_t m, int32_t c, const void* Ca, const void* Cb,
                                 const void* Za, const void* Zb, int64_t ld_in, const void* Ba, const void* Bb,
                                 const float* dCcomp, int64_t ld_dc, void* dCa, void* dCb, void* dZa, void* dZb,
                                 int64_t ld_out, float* dBa, float* dBb, void* workspace, size_t ws_bytes,
                                 void* stream) {
  CSA_REQUIRE(dtype_ok(dt), "csa_compress_backward: unknown dtype");
  CSA_REQUIRE(n >= 0, "csa_compress_backward: n must be >= 0");
  CSA_REQUIRE(m >= 1 && m <= 16, "csa_compress_backward: m must be in [1, 16] (got %d)", m);
  CSA_REQUIRE(c > 0 && c % 4 == 0, "csa_compress_backward: c must be a positive multiple of 4 (got %d)", c);
  CSA_REQUIRE(dBa && dBb && workspace, "csa_compress_backward: null pointer");
  const size_t need = csa::compress_backward_workspace_bytes(n, m, c, 0, 0, false);
  CSA_REQUIRE(need < csa::kWorkspaceTooBig, "csa_compress_backward: sizes too large");
  CSA_REQUIRE(ws_bytes >= need, "csa_compress_backward: workspace of %zu bytes is smaller than %zu", ws_bytes, need);
  CSA_REQUIRE(aligned16(workspace), "csa_compress_backward: workspace must be 16-byte aligned");
  const int v = vec_elems(dt);
  if (n > 0) {
    CSA_REQUIRE(Ca && Cb && Za && Zb && Ba && Bb && dCa && dCb && dZa && dZb, "csa_compress_backward: null pointer");
    CSA_REQUIRE(n / m == 0 || dCcomp != nullptr, "csa_compress_backward: null dCcomp");
    CSA_REQUIRE(aligned16(Ca) && aligned16(Cb) && aligned16(Za) && aligned16(Zb) && aligned16(Ba) &&
                    aligned16(Bb) && aligned16(dCa) && aligned16(dCb) && aligned16(dZa) && aligned16(dZb) &&
                    (dCcomp == nullptr || aligned16(dCcomp)),
                "csa_compress_backward: pointers must be 16-byte aligned");
    CSA_REQUIRE(ld_in >= c && ld_out >= c && ld_dc >= c, "csa_compress_backward: leading dimension smaller than c");
    CSA_REQUIRE(ld_in % v == 0 && ld_out % v == 0 && ld_dc % 4 == 0,
                "csa_compress_backward: leading dimensions must keep rows 16-byte aligned");
  }
  csa_status st = check_device();
  if (st != CSA_OK) return st;
  hipError_t e = csa::launch_compress_backward(dt, n, m, c, Ca, Cb, Za, Zb, ld_in, Ba, Bb, dCcomp, ld_dc, dCa, dCb,
                                               dZa, dZb, ld_out, dBa, dBb, workspace, (hipStream_t)stream);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "csa_compress_backward launch");
}

csa_status csa_compress_backward_varlen_workspace(int64_t n_seqs, int64_t n_blocks, int32_t m, int32_t c,
                                                 size_t* bytes) {
  CSA_REQUIRE(bytes != nullptr, "csa_compress_backward_varlen_workspace: null bytes");
  CSA_REQUIRE(n_seqs >= 0 && n_seqs <= 0x7FFFFFFF && n_blocks >= 0,
              "csa_compress_backward_varlen_workspace: bad n_seqs / n_blocks");
  CSA_REQUIRE(m >= 1 && m <= 16, "csa_compress_backward_varlen_workspace: m must be in [1, 16] (got %d)", m);
  CSA_REQUIRE(c > 0 && c % 4 == 0, "csa_compress_backward_varlen_workspace: c must be a positive multiple of 4");
  *bytes = csa::compress_backward_workspace_bytes(0, m, c, n_seqs, n_blocks, true);
  CSA_REQUIRE(*bytes < csa::kWorkspaceTooBig, "csa_compress_backward_varlen_workspace: sizes too large");
  return CSA_OK;
}

csa_status csa_compress_backward_varlen(csa_dtype dt, int64_t n_seqs, int32_t m, int32_t c, const void* Ca,
                                        const void* Cb, const void* Za, const void* Zb, int64_t ld_in,
                                        const void* Ba, const void* Bb, const int64_t* cu_seqlens,
                                        const int64_t* block_offset, int64_t n_blocks, const float* dCcomp,
                                        int64_t ld_dc, void* dCa, void* dCb, void* dZa, void* dZb, int64_t ld_out,
                                        float* dBa, float* dBb, void* workspace, size_t ws_bytes, void* stream) {
  CSA_REQUIRE(dtype_ok(dt), "csa_compress_backward_varlen: unknown dtype");
  CSA_REQUIRE(n_seqs >= 0 && n_seqs <= 0x7FFFFFFF && n_blocks >= 0, "csa_compress_backward_varlen: bad n_seqs / n_blocks");
  CSA_REQUIRE(m >= 1 && m <= 16, "csa_compress_backward_varlen: m must be in [1, 16] (got %d)", m);
  CSA_REQUIRE(c > 0 && c % 4 == 0, "csa_compress_backward_varlen: c must be a positive multiple of 4 (got %d)", c);
  CSA_REQUIRE(dBa && dBb && workspace, "csa_compress_backward_varlen: null pointer");
  const size_t need = csa::compress_backward_workspace_bytes(0, m, c, n_seqs, n_blocks, true);
  CSA_REQUIRE(need < csa::kWorkspaceTooBig, "csa_compress_backward_varlen: sizes too large");
  CSA_REQUIRE(ws_bytes >= need, "csa_compress_backward_varlen: workspace of %zu bytes is smaller than %zu", ws_bytes,
              need);
  CSA_REQUIRE(aligned16(workspace), "csa_compress_backward_varlen: workspace must be 16-byte aligned");
  CSA_REQUIRE(n_seqs > 0 || n_blocks == 0, "csa_compress_backward_varlen: blocks without sequences");
  const int v = vec_elems(dt);
  if (n_seqs > 0) {
    CSA_REQUIRE(Ca && Cb && Za && Zb && Ba && Bb && dCa && dCb && dZa && dZb && cu_seqlens && block_offset,
                "csa_compress_backward_varlen: null pointer");
    CSA_REQUIRE(n_blocks == 0 || dCcomp != nullptr, "csa_compress_backward_varlen: null dCcomp");
    CSA_REQUIRE(aligned16(Ca) && aligned16(Cb) && aligned16(Za) && aligned16(Zb) && aligned16(Ba) &&
                    aligned16(Bb) && aligned16(dCa) && aligned16(dCb) && aligned16(dZa) && aligned16(dZb) &&
                    (dCcomp == nullptr || aligned16(dCcomp)),
                "csa_compress_backward_varlen: pointers must be 16-byte aligned");
    CSA_REQUIRE(ld_in >= c && ld_out >= c && ld_dc >= c,
                "csa_compress_backward_varlen: leading dimension smaller than c");
    CSA_REQUIRE(ld_in % v == 0 && ld_out % v == 0 && ld_dc % 4 == 0,
                "csa_compress_backward_varlen: leading dimensions must keep rows 16-byte aligned");
  }
  csa_status st = check_device();
  if (st != CSA_OK) return st;
  hipError_t e = csa::launch_compress_backward_varlen(dt, n_seqs, n_blocks, m, c, Ca, Cb, Za, Zb, ld_in, Ba, Bb,
                                                      cu_seqlens, block_offset, dCcomp, ld_dc, dCa, dCb, dZa, dZb,
                                                      ld_out, dBa, dBb, workspace, (hipStream_t)stream);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "csa_compress_backward_varlen launch");
}

csa_status csa_compress_append(csa_dtype dt, int64_t B, int32_t m, int32_t c, const void* new_rows,
                               int64_t ld_new, void* ring, const void* Ba, const void* Bb,
                               const int64_t* t_new, const int64_t* kv_offset, void* Ccomp,
                               int64_t ld_out, void* stream) {
  CSA_REQUIRE(dtype_ok(dt), "csa_compress_append: unknown dtype");
  CSA_REQUIRE(B >= 0 && B <= 0x7FFFFFFF, "csa_compress_append: bad B");
  CSA_REQUIRE(m >= 1 && m <= 64, "csa_compress_append: m must be in [1, 64] (got %d)", m);
  CSA_REQUIRE(c > 0 && c % 4 == 0, "csa_compress_append: c must be a positive multiple of 4 (got %d)", c);
  if (B == 0) return CSA_OK;
  CSA_REQUIRE(new_rows && ring && Ba && Bb && t_new && kv_offset && Ccomp, "csa_compress_append: null pointer");
  CSA_REQUIRE(aligned16(new_rows) && aligned16(ring) && aligned16(Ba) && aligned16(Bb) && aligned16(Ccomp),
              "csa_compress_append: pointers must be 16-byte aligned");
  const int v = vec_elems(dt);
  CSA_REQUIRE(ld_new >= 4L * c && ld_out >= c, "csa_compress_append: leading dimension too small");
  CSA_REQUIRE(ld_new % v == 0 && ld_out % v == 0,
              "csa_compress_append: leading dimensions must keep rows 16-byte aligned");
  csa_status st = check_device();
  if (st != CSA_OK) return st;
  hipError_t e = csa::launch_compress_append(dt, B, m, c, new_rows, ld_new, ring, Ba, Bb, t_new, kv_offset, Ccomp,
                                             ld_out, (hipStream_t)stream);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "csa_compress_append launch");
}

csa_status csa_compress_append_pair(csa_dtype dt, int64_t B, int32_t m, const int64_t* t_new,
                                    const int64_t* kv_offset, int32_t c1, const void* new_rows1, int64_t ld_new1,
                                    void* ring1, const void* Ba1, const void* Bb1, void* Ccomp1, int64_t ld_out1,
                                    int32_t c2, const void* new_rows2, int64_t ld_new2, void* ring2,
                                    const void* Ba2, const void* Bb2, void* Ccomp2, int64_t ld_out2, void* stream) {
  CSA_REQUIRE(dtype_ok(dt), "csa_compress_append_pair: unknown dtype");
  CSA_REQUIRE(B >= 0 && B <= 0x3FFFFFFF, "csa_compress_append_pair: bad B");
  CSA_REQUIRE(m >= 1 && m <= 64, "csa_compress_append_pair: m must be in [1, 64] (got %d)", m);
  const int v = vec_elems(dt);
  const int32_t cs[2] = {c1, c2};
  const void* rows[2] = {new_rows1, new_rows2};
  const void* rings[2] = {ring1, ring2};
  const void* bas[2] = {Ba1, Ba2};
  const void* bbs[2] = {Bb1, Bb2};
  const void* outs[2] = {Ccomp1, Ccomp2};
  const int64_t lds_new[2] = {ld_new1, ld_new2}, lds_out[2] = {ld_out1, ld_out2};
  for (int x = 0; x < 2; ++x) {
    CSA_REQUIRE(cs[x] > 0 && cs[x] % 4 == 0, "csa_compress_append_pair: c%d must be a positive multiple of 4 (got %d)",
                x + 1, cs[x]);
  }
  if (B == 0) return CSA_OK;
  CSA_REQUIRE(t_new && kv_offset, "csa_compress_append_pair: null pointer");
  for (int x = 0; x < 2; ++x) {
    CSA_REQUIRE(rows[x] && rings[x] && bas[x] && bbs[x] && outs[x], "csa_compress_append_pair: null pointer (cache %d)",
                x + 1);
    CSA_REQUIRE(aligned16(rows[x]) && aligned16(rings[x]) && aligned16(bas[x]) && aligned16(bbs[x]) &&
                    aligned16(outs[x]),
                "csa_compress_append_pair: pointers must be 16-byte aligned (cache %d)", x + 1);
    CSA_REQUIRE(lds_new[x] >= 4L * cs[x] && lds_out[x] >= cs[x],
                "csa_compress_append_pair: leading dimension too small (cache %d)", x + 1);
    CSA_REQUIRE(lds_new[x] % v == 0 && lds_out[x] % v == 0,
                "csa_compress_append_pair: leading dimensions must keep rows 16-byte aligned (cache %d)", x + 1);
  }
  csa_status st = check_device();
  if (st != CSA_OK) return st;
  const csa::AppendCache a{c1, new_rows1, ld_new1, ring1, Ba1, Bb1, Ccomp1, ld_out1};
  const csa::AppendCache b{c2, new_rows2, ld_new2, ring2, Ba2, Bb2, Ccomp2, ld_out2};
  hipError_t e = csa::launch_compress_append_pair(dt, B, m, t_new, kv_offset, a, b, (hipStream_t)stream);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "csa_compress_append_pair launch");
}

csa_status csa_index_topk_workspace(int64_t n_queries, int64_t max_cand, int32_t n_hI, int32_t k,
                                    size_t* bytes) {
  CSA_REQUIRE(bytes, "csa_index_topk_workspace: null bytes");
  CSA_REQUIRE(n_queries >= 0 && max_cand >= 0, "csa_index_topk_workspace: negative size");
  CSA_REQUIRE(n_hI >= 1 && k >= 1, "csa_index_topk_workspace: n_hI and k must be >= 1");
  *bytes = index_ws(n_queries, max_cand, k).total;
  CSA_REQUIRE(*bytes < csa::kWorkspaceTooBig, "csa_index_topk_workspace: sizes too large");
  return CSA_OK;
}

}  // extern "C"

namespace {
// csa_index_topk; `clear` zeroes the histogram and arrival counters first
// (csa_decode relies on the selectors leaving them zero instead).  With
// `classified` not null, rows on the multi-workgroup path are only
// classified (TopkLists::b1g1) and *classified describes their lists, for
// the attention to finish them; classified->b1g1 stays null when the batch
// takes another path (the selection is then complete on return).
csa_status index_topk(csa_dtype dt, int64_t n_queries, int32_t n_hI, int32_t cI, int32_t m, int32_t k,
                      const void* qI, const float* wI, const void* KIcomp, const int32_t* q_seq,
                      const int64_t* q_pos, const int64_t* kv_offset, int64_t max_cand, int32_t* idx_out,
                      float* score_out, void* workspace, size_t ws_bytes, void* stream, bool clear,
                      csa::TopkLists* classified = nullptr) {
  if (classified) *classified = csa::TopkLists{};
  CSA_REQUIRE(dtype_ok(dt), "csa_index_topk: unknown dtype");
  CSA_REQUIRE(n_queries >= 0 && n_queries <= 0x7FFFFFFF, "csa_index_topk: bad n_queries");
  CSA_REQUIRE(n_hI >= 1 && n_hI <= 64, "csa_index_topk: n_hI must be in [1, 64] (got %d)", n_hI);
  CSA_REQUIRE(cI == 32 || cI == 64 || cI == 128 || cI == 256,
              "csa_index_topk: cI must be 32, 64, 128 or 256 (got %d)", cI);
  CSA_REQUIRE(m >= 1, "csa_index_topk: m must be >= 1");
  CSA_REQUIRE(k >= 1 && k <= (1 << 24), "csa_index_topk: k must be in [1, 2^24]");
  CSA_REQUIRE(max_cand >= 0 && max_cand <= 0x7FFFFFFF, "csa_index_topk: bad max_cand");
  if (n_queries == 0) return CSA_OK;
  CSA_REQUIRE(qI && wI && KIcomp && idx_out, "csa_index_topk: null pointer");
  CSA_REQUIRE(aligned16(qI) && aligned16(wI) && aligned16(KIcomp) && aligned16(idx_out),
              "csa_index_topk: pointers must be 16-byte aligned");
  size_t need = 0;
  csa_status st0 = csa_index_topk_workspace(n_queries, max_cand, n_hI, k, &need);
  if (st0 != CSA_OK) return st0;
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(CSA_ERR_WORKSPACE, "csa_index_topk: workspace needs %zu bytes (got %zu)", need, ws_bytes);
  CSA_REQUIRE(workspace == nullptr || aligned16(workspace), "csa_index_topk: workspace must be 16-byte aligned");
  csa_status st = check_device();
  if (st != CSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  float* scores = (float*)workspace;
  const long ld = scores_ld(max_cand);
  // the per-query sweep (q_seq or q_pos given) builds the level-1 histogram
  const IndexWs w = index_ws(n_queries, max_cand, k);
  char* ws = (char*)workspace;
  uint32_t* hist = nullptr;
  csa::TopkLists lists{};
  const bool sweep = q_seq || q_pos;
  const bool multi = sweep && use_lists(n_queries, max_cand);
  if (use_hist(max_cand) && sweep) {
    hist = (uint32_t*)(ws + w.hist);
  }
  if (hist && clear) {
    const long words = n_queries * (1L << csa::kTopkL1Bits) + (multi ? n_queries : 0);
    hipError_t e0 = csa::launch_hist_clear(hist, words, s);
    if (e0 != hipSuccess) return hip_fail(e0, "csa_index_topk histogram clear");
  }
  if (multi) {
    lists.arrive = (uint32_t*)(ws + w.arrive);
    lists.counts = (uint32_t*)(ws + w.counts);
    lists.gt = (uint64_t*)(ws + w.gt);
    lists.eq = (uint64_t*)(ws + w.eq);
    lists.P = topk_chunks(max_cand);
    lists.gtc = k < csa::kMChunk ? k : csa::kMChunk;
    if (classified) {
      lists.b1g1 = (uint32_t*)(ws + w.b1g1);
      lists.hist = hist;
    }
  }
  hipError_t e = csa::launch_indexer(dt, n_queries, n_hI, cI, m, qI, wI, KIcomp, q_seq, q_pos, kv_offset,
                                     max_cand, scores, ld, hist, k, s);
  if (e != hipSuccess) return hip_fail(e, "csa_index_topk indexer launch");
  e = csa::launch_topk(n_queries, m, scores, ld, q_pos, max_cand, k, hist, multi ? &lists : nullptr, idx_out,
                       score_out, s);
  if (e != hipSuccess) return hip_fail(e, "csa_index_topk top-k launch");
  if (classified && lists.b1g1) *classified = lists;
  return CSA_OK;
}

}  // namespace

extern "C" {

csa_status csa_index_topk(csa_dtype dt, int64_t n_queries, int32_t n_hI, int32_t cI, int32_t m,
                          int32_t k, const void* qI, const float* wI, const void* KIcomp,
                          const int32_t* q_seq, const int64_t* q_pos, const int64_t* kv_offset,
                          int64_t max_cand, int32_t* idx_out, float* score_out, void* workspace,
                          size_t ws_bytes, void* stream) {
  return index_topk(dt, n_queries, n_hI, cI, m, k, qI, wI, KIcomp, q_seq, q_pos, kv_offset, max_cand, idx_out,
                    score_out, workspace, ws_bytes, stream, true);
}

// Workspace of csa_index_topk_stream (each area 256-byte aligned): lists
// [n_queries, stream_ld(max_cand)] uint64, per-query state [n_queries, 4] uint32.
long stream_ld(long max_cand) { return (max_cand + 1) & ~1L; }

csa_status csa_index_topk_stream_workspace(int64_t n_queries, int64_t max_cand, size_t* bytes) {
  CSA_REQUIRE(bytes, "csa_index_topk_stream_workspace: null bytes");
  CSA_REQUIRE(n_queries >= 0 && n_queries <= 0x7FFFFFFF && max_cand >= 0 && max_cand <= 65535,
              "csa_index_topk_stream_workspace: bad size (max_cand <= 65535)");
  *bytes = csa::ws_add(csa::ws_align(csa::ws_bytes(n_queries, stream_ld(max_cand), sizeof(uint64_t))),
                       csa::ws_align(csa::ws_bytes(n_queries, 4 * sizeof(uint32_t))));
  return CSA_OK;
}

csa_status csa_index_topk_stream(csa_dtype dt, int64_t n_queries, int32_t n_hI, int32_t cI, int32_t m, int32_t k,
                                 const void* qI, const float* wI, const void* KIcomp, int64_t max_cand,
                                 int32_t* idx_out, float* score_out, void* workspace, size_t ws_bytes,
                                 void* stream) {
  CSA_REQUIRE(dtype_ok(dt), "csa_index_topk_stream: unknown dtype");
  CSA_REQUIRE(n_queries >= 0 && n_queries <= 0x7FFFFFFF, "csa_index_topk_stream: bad n_queries");
  CSA_REQUIRE(n_hI >= 1 && n_hI <= 64, "csa_index_topk_stream: n_hI must be in [1, 64] (got %d)", n_hI);
  CSA_REQUIRE(cI == 32 || cI == 64 || cI == 128 || cI == 256,
              "csa_index_topk_stream: cI must be 32, 64, 128 or 256 (got %d)", cI);
  CSA_REQUIRE(m >= 1, "csa_index_topk_stream: m must be >= 1");
  CSA_REQUIRE(k >= 1 && k <= (1 << 24), "csa_index_topk_stream: k must be in [1, 2^24]");
  CSA_REQUIRE(max_cand >= 0 && max_cand <= 65535, "csa_index_topk_stream: max_cand must be in [0, 65535]");
  if (n_queries == 0) return CSA_OK;
  CSA_REQUIRE(qI && wI && KIcomp && idx_out, "csa_index_topk_stream: null pointer");
  CSA_REQUIRE(aligned16(qI) && aligned16(wI) && aligned16(KIcomp) && aligned16(idx_out) && aligned16(score_out),
              "csa_index_topk_stream: pointers must be 16-byte aligned");
  if (!csa::indexer_stream_supported(dt, n_hI, cI, max_cand))
    return fail(CSA_ERR_UNSUPPORTED, "csa_index_topk_stream: n_hI = %d, cI = %d does not fit the streaming kernel",
                n_hI, cI);
  size_t need = 0;
  csa_status st = csa_index_topk_stream_workspace(n_queries, max_cand, &need);
  if (st != CSA_OK) return st;
  if (workspace == nullptr || ws_bytes < need)
    return fail(CSA_ERR_WORKSPACE, "csa_index_topk_stream: workspace needs %zu bytes (got %zu)", need, ws_bytes);
  CSA_REQUIRE(aligned16(workspace), "csa_index_topk_stream: workspace must be 16-byte aligned");
  st = check_device();
  if (st != CSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  const long ld = stream_ld(max_cand);
  uint64_t* lists = (uint64_t*)workspace;
  uint32_t* meta = (uint32_t*)((char*)workspace + csa::ws_align(csa::ws_bytes(n_queries, ld, sizeof(uint64_t))));
  hipError_t e = csa::launch_indexer_stream(dt, n_queries, n_hI, cI, m, qI, wI, KIcomp, nullptr, max_cand, lists,
                                            ld, meta, k, s);
  if (e != hipSuccess) return hip_fail(e, "csa_index_topk_stream indexer launch");
  e = csa::launch_topk_lists(n_queries, m, max_cand, k, lists, ld, meta, idx_out, score_out, s);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "csa_index_topk_stream top-k launch");
}

csa_status csa_sparse_mqa_workspace(int64_t n_queries, int32_t n_h, int32_t c, int32_t k, size_t* bytes) {
  CSA_REQUIRE(bytes, "csa_sparse_mqa_workspace: null bytes");
  CSA_REQUIRE(n_queries >= 0 && n_h >= 1 && c >= 1 && k >= 1, "csa_sparse_mqa_workspace: bad size");
  // the query has no dtype: cover both kernels' plans
  const size_t a = csa::mqa_workspace_bytes(n_queries, n_h, c, k, true);
  const size_t b = csa::mqa_workspace_bytes(n_queries, n_h, c, k, false);
  *bytes = a > b ? a : b;
  CSA_REQUIRE(*bytes < csa::kWorkspaceTooBig, "csa_sparse_mqa_workspace: sizes too large");
  return CSA_OK;
}

}  // extern "C"

namespace {
// csa_sparse_mqa; sel: see csa::TileSelect (csa_decode only)
csa_status sparse_mqa(csa_dtype dt, int64_t n_queries, int32_t n_h, int32_t c, int32_t k, float scale,
                      const void* q, const void* Ccomp, const int32_t* q_seq, const int64_t* kv_offset,
                      const int32_t* idx, void* o, float* lse, void* workspace, size_t ws_bytes, void* stream,
                      const csa::TileSelect* sel) {
  CSA_REQUIRE(dtype_ok(dt), "csa_sparse_mqa: unknown dtype");
  CSA_REQUIRE(n_queries >= 0 && n_queries <= 0x7FFFFFFF, "csa_sparse_mqa: bad n_queries");
  CSA_REQUIRE(n_h >= 1 && n_h <= 256, "csa_sparse_mqa: n_h must be in [1, 256] (got %d)", n_h);
  CSA_REQUIRE(csa::mqa_supported_c(c), "csa_sparse_mqa: c must be 64, 128, 256, 512 or 1024 (got %d)", c);
  CSA_REQUIRE(k >= 1 && k <= (1 << 24), "csa_sparse_mqa: k must be in [1, 2^24]");
  CSA_REQUIRE(scale == scale && scale > 0.f && scale < 1e30f, "csa_sparse_mqa: scale must be positive and finite");
  if (n_queries == 0) return CSA_OK;
  CSA_REQUIRE(q && Ccomp && idx && o, "csa_sparse_mqa: null pointer");
  CSA_REQUIRE(aligned16(q) && aligned16(Ccomp) && aligned16(idx) && aligned16(o),
              "csa_sparse_mqa: pointers must be 16-byte aligned");
  const size_t need = csa::mqa_workspace_bytes(n_queries, n_h, c, k, dt == CSA_BF16);
  CSA_REQUIRE(need < csa::kWorkspaceTooBig, "csa_sparse_mqa: sizes too large");
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(CSA_ERR_WORKSPACE, "csa_sparse_mqa: workspace needs %zu bytes (got %zu)", need, ws_bytes);
  CSA_REQUIRE(aligned16(workspace), "csa_sparse_mqa: workspace must be 16-byte aligned");
  csa_status st = check_device();
  if (st != CSA_OK) return st;
  hipError_t e = csa::launch_mqa(dt, n_queries, n_h, c, k, scale, q, Ccomp, q_seq, kv_offset, idx, o, lse,
                                 workspace, (hipStream_t)stream, sel);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "csa_sparse_mqa launch");
}

// The two stages of csa_decode / csa_decode_noalloc on a workspace laid out
// as [index_topk part | a | MQA part].  Where the attention can finish the
// selection (csa::mqa_tile_selects, and the batch takes the top-k's
// multi-workgroup path) the top-k launch only classifies, and the attention
// resolves each row's threshold itself (csa::TileSelect).
csa_status decode_stages(csa_dtype dt, int64_t n_queries, int32_t n_hI, int32_t cI, int32_t n_h, int32_t c,
                         int32_t m, int32_t k, float scale, const void* qI, const float* wI, const void* KIcomp,
                         const void* q, const void* Ccomp, const int32_t* q_seq, const int64_t* q_pos,
                         const int64_t* kv_offset, int64_t max_cand, int32_t* idx_out, float* score_out, void* o,
                         float* lse, char* ws, size_t a, size_t ws_bytes, void* stream, bool clear) {
  const bool fuse = csa::mqa_tile_selects(n_queries, n_h, c, k, dt == CSA_BF16);
  csa::TopkLists lists{};
  csa_status st = index_topk(dt, n_queries, n_hI, cI, m, k, qI, wI, KIcomp, q_seq, q_pos, kv_offset, max_cand,
                             idx_out, score_out, ws, a, stream, clear, fuse ? &lists : nullptr);
  if (st != CSA_OK) return st;
  csa::TileSelect sel{m, q_pos, max_cand, lists, idx_out, score_out};
  return sparse_mqa(dt, n_queries, n_h, c, k, scale, q, Ccomp, q_seq, kv_offset, idx_out, o, lse,
                    ws ? ws + a : nullptr, ws_bytes - a, stream, lists.b1g1 ? &sel : nullptr);
}
}  // namespace

extern "C" {

csa_status csa_sparse_mqa(csa_dtype dt, int64_t n_queries, int32_t n_h, int32_t c, int32_t k,
                          float scale, const void* q, const void* Ccomp, const int32_t* q_seq,
                          const int64_t* kv_offset, const int32_t* idx, void* o, float* lse,
                          void* workspace, size_t ws_bytes, void* stream) {
  return sparse_mqa(dt, n_queries, n_h, c, k, scale, q, Ccomp, q_seq, kv_offset, idx, o, lse, workspace, ws_bytes,
                    stream, nullptr);
}

csa_status csa_sparse_mqa_backward_workspace(int64_t n_queries, int32_t n_h, int32_t c, int32_t k, int64_t n_rows,
                                             size_t* bytes) {
  CSA_REQUIRE(bytes, "csa_sparse_mqa_backward_workspace: null bytes");
  CSA_REQUIRE(n_queries >= 0 && n_queries <= 0x7FFFFFFF, "csa_sparse_mqa_backward_workspace: bad n_queries");
  CSA_REQUIRE(n_h >= 1 && n_h <= 256, "csa_sparse_mqa_backward_workspace: n_h must be in [1, 256]");
  CSA_REQUIRE(c == 512, "csa_sparse_mqa_backward_workspace: c must be 512 (got %d)", c);
  CSA_REQUIRE(k >= 1 && k <= (1 << 20), "csa_sparse_mqa_backward_workspace: k must be in [1, 2^20]");
  CSA_REQUIRE(n_rows >= 0 && n_rows < 0x7FFFFFFF, "csa_sparse_mqa_backward_workspace: bad n_rows");
  *bytes = csa::mqa_backward_workspace_bytes(n_queries, n_h, k, n_rows);
  CSA_REQUIRE(*bytes < csa::kWorkspaceTooBig, "csa_sparse_mqa_backward_workspace: sizes too large");
  return CSA_OK;
}

csa_status csa_sparse_mqa_backward(csa_dtype dt, int64_t n_queries, int32_t n_h, int32_t c, int32_t k, float scale,
                                   const void* q, const void* Ccomp, int64_t n_rows, const int32_t* q_seq,
                                   const int64_t* kv_offset, const int32_t* idx, const void* o, const float* lse,
                                   const void* dO, void* dq, float* dCcomp, void* workspace, size_t ws_bytes,
                                   void* stream) {
  CSA_REQUIRE(dtype_ok(dt), "csa_sparse_mqa_backward: unknown dtype");
  if (dt != CSA_BF16) return fail(CSA_ERR_UNSUPPORTED, "csa_sparse_mqa_backward: only bf16 is supported");
  size_t need = 0;
  csa_status st = csa_sparse_mqa_backward_workspace(n_queries, n_h, c, k, n_rows, &need);
  if (st != CSA_OK) return st;
  CSA_REQUIRE(scale == scale && scale > 0.f && scale < 1e30f,
              "csa_sparse_mqa_backward: scale must be positive and finite");
  CSA_REQUIRE(n_rows == 0 || dCcomp, "csa_sparse_mqa_backward: null dCcomp");
  CSA_REQUIRE(aligned16(dCcomp), "csa_sparse_mqa_backward: dCcomp must be 16-byte aligned");
  if (n_queries > 0) {
    CSA_REQUIRE(q && idx && o && lse && dO && dq && (n_rows == 0 || Ccomp), "csa_sparse_mqa_backward: null pointer");
    CSA_REQUIRE(aligned16(q) && aligned16(Ccomp) && aligned16(idx) && aligned16(o) && aligned16(dO) && aligned16(dq),
                "csa_sparse_mqa_backward: pointers must be 16-byte aligned");
    if (workspace == nullptr || ws_bytes < need)
      return fail(CSA_ERR_WORKSPACE, "csa_sparse_mqa_backward: workspace needs %zu bytes (got %zu)", need, ws_bytes);
    CSA_REQUIRE(aligned16(workspace), "csa_sparse_mqa_backward: workspace must be 16-byte aligned");
  }
  if (n_queries == 0 && n_rows == 0) return CSA_OK;
  st = check_device();
  if (st != CSA_OK) return st;
  hipError_t e = csa::launch_mqa_backward(n_queries, n_h, k, scale, q, Ccomp, n_rows, q_seq, kv_offset, idx, o, lse,
                                          dO, dq, dCcomp, workspace, (hipStream_t)stream);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "csa_sparse_mqa_backward launch");
}

csa_status csa_decode_workspace(int64_t n_queries, int64_t max_cand, int32_t n_hI, int32_t n_h, int32_t c,
                                int32_t k, size_t* bytes) {
  CSA_REQUIRE(bytes, "csa_decode_workspace: null bytes");
  size_t a = 0, b = 0;
  csa_status st = csa_index_topk_workspace(n_queries, max_cand, n_hI, k, &a);
  if (st != CSA_OK) return st;
  st = csa_sparse_mqa_workspace(n_queries, n_h, c, k, &b);
  if (st != CSA_OK) return st;
  *bytes = csa::ws_add(csa::ws_align(a), b);
  CSA_REQUIRE(*bytes < csa::kWorkspaceTooBig, "csa_decode_workspace: sizes too large");
  return CSA_OK;
}

}  // extern "C"

namespace {

// Checks of csa_decode (and csa_decode_noalloc) that its two stages would
// otherwise make one after the other: the attention's are made here too, so a
// bad argument is refused before the selection launches anything.
csa_status decode_checks(const char* fn, int64_t n_queries, int32_t n_hI, int32_t n_h, int32_t c, int32_t k,
                         float scale, const void* q, const void* Ccomp, const int64_t* q_pos, int64_t max_cand,
                         const void* o) {
  CSA_REQUIRE(q_pos != nullptr || n_queries == 0, "%s: q_pos is required", fn);
  CSA_REQUIRE(n_h >= 1 && n_hI >= 1 && k >= 1 && n_queries >= 0 && max_cand >= 0, "%s: bad size", fn);
  CSA_REQUIRE(n_h <= 256, "%s: n_h must be in [1, 256] (got %d)", fn, n_h);
  CSA_REQUIRE(csa::mqa_supported_c(c), "%s: c must be 64, 128, 256, 512 or 1024 (got %d)", fn, c);
  CSA_REQUIRE(scale == scale && scale > 0.f && scale < 1e30f, "%s: scale must be positive and finite", fn);
  CSA_REQUIRE(n_queries == 0 || (q && Ccomp && o), "%s: null pointer", fn);
  CSA_REQUIRE(aligned16(q) && aligned16(Ccomp) && aligned16(o), "%s: pointers must be 16-byte aligned", fn);
  return CSA_OK;
}

// ---------------------------------------------------------------------------
// Scratch of csa_decode_noalloc: a file-scope device array, one copy per GPU
// (each holds it until the process ends).  Host code never passes the
// array's name: its device address is looked up once per device, with that
// device current, and kept.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = (size_t)32 << 20;
__device__ __align__(256) unsigned char scratch[kScratchBytes];
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

csa_status scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(CSA_ERR_UNSUPPORTED, "device ordinal %d out of range", dev);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "csa_decode_noalloc: address of the static scratch");
    if (p == nullptr) return fail(CSA_ERR_HIP, "csa_decode_noalloc: the static scratch has no device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return CSA_OK;
}

}  // namespace

extern "C" {

csa_status csa_decode(csa_dtype dt, int64_t n_queries, int32_t n_hI, int32_t cI, int32_t n_h, int32_t c, int32_t m,
                      int32_t k, float scale, const void* qI, const float* wI, const void* KIcomp, const void* q,
                      const void* Ccomp, const int32_t* q_seq, const int64_t* q_pos, const int64_t* kv_offset,
                      int64_t max_cand, int32_t* idx_out, float* score_out, void* o, float* lse, void* workspace,
                      size_t ws_bytes, void* stream) {
  csa_status st0 = decode_checks("csa_decode", n_queries, n_hI, n_h, c, k, scale, q, Ccomp, q_pos, max_cand, o);
  if (st0 != CSA_OK) return st0;
  size_t need = 0, a = 0;
  csa_status st = csa_decode_workspace(n_queries, max_cand, n_hI, n_h, c, k, &need);
  if (st != CSA_OK) return st;
  if (need > 0 && (workspace == nullptr || ws_bytes < need))
    return fail(CSA_ERR_WORKSPACE, "csa_decode: workspace needs %zu bytes (got %zu)", need, ws_bytes);
  csa_index_topk_workspace(n_queries, max_cand, n_hI, k, &a);
  a = align256(a);
  return decode_stages(dt, n_queries, n_hI, cI, n_h, c, m, k, scale, qI, wI, KIcomp, q, Ccomp, q_seq, q_pos,
                       kv_offset, max_cand, idx_out, score_out, o, lse, (char*)workspace, a, ws_bytes, stream, false);
}

csa_status csa_decode_noalloc(csa_dtype dt, int64_t n_queries, int32_t n_hI, int32_t cI, int32_t n_h, int32_t c,
                              int32_t m, int32_t k, float scale, const void* qI, const float* wI, const void* KIcomp,
                              const void* q, const void* Ccomp, const int32_t* q_seq, const int64_t* q_pos,
                              const int64_t* kv_offset, int64_t max_cand, int32_t* idx_out, float* score_out,
                              void* o, float* lse, void* stream) {
  CSA_REQUIRE(dtype_ok(dt), "csa_decode_noalloc: unknown dtype");
  csa_status st =
      decode_checks("csa_decode_noalloc", n_queries, n_hI, n_h, c, k, scale, q, Ccomp, q_pos, max_cand, o);
  if (st != CSA_OK) return st;
  if (n_queries == 0) return CSA_OK;
  // this dtype's own needs (csa_decode_workspace covers both dtypes)
  size_t a = 0;
  st = csa_index_topk_workspace(n_queries, max_cand, n_hI, k, &a);
  if (st != CSA_OK) return st;
  a = align256(a);
  const size_t b = csa::mqa_workspace_bytes(n_queries, n_h, c, k, dt == CSA_BF16);
  if (csa::ws_add(a, b) > kScratchBytes)
    return fail(CSA_ERR_WORKSPACE, "csa_decode_noalloc: these sizes need %zu bytes of scratch; the static scratch "
                "holds %zu (use csa_decode with a workspace)", a + b, kScratchBytes);
  st = check_device();
  if (st != CSA_OK) return st;
  void* ws = nullptr;
  st = scratch_of_current_device(&ws);
  if (st != CSA_OK) return st;
  // the scratch keeps whatever the last call left, laid out for that call's
  // sizes: the selection clears its histogram and counters first (a kernel,
  // not a memset)
  return decode_stages(dt, n_queries, n_hI, cI, n_h, c, m, k, scale, qI, wI, KIcomp, q, Ccomp, q_seq, q_pos,
                       kv_offset, max_cand, idx_out, score_out, o, lse, (char*)ws, a, a + b, stream, true);
}

csa_status csa_compress_varlen(csa_dtype dt, int64_t n_seqs, int32_t m, int32_t c, const void* Ca, const void* Cb,
                               const void* Za, const void* Zb, int64_t ld_in, const void* Ba, const void* Bb,
                               const int64_t* cu_seqlens, const int64_t* block_offset, int64_t n_blocks, void* Ccomp,
                               int64_t ld_out, void* stream) {
  CSA_REQUIRE(dtype_ok(dt), "csa_compress_varlen: unknown dtype");
  CSA_REQUIRE(n_seqs >= 0 && n_seqs <= 0x7FFFFFFF && n_blocks >= 0, "csa_compress_varlen: bad n_seqs / n_blocks");
  CSA_REQUIRE(m >= 1, "csa_compress_varlen: m must be >= 1 (got %d)", m);
  CSA_REQUIRE(c > 0 && c % 4 == 0, "csa_compress_varlen: c must be a positive multiple of 4 (got %d)", c);
  if (n_seqs == 0 || n_blocks == 0) return CSA_OK;
  CSA_REQUIRE(Ca && Cb && Za && Zb && Ba && Bb && cu_seqlens && block_offset && Ccomp,
              "csa_compress_varlen: null pointer");
  CSA_REQUIRE(aligned16(Ca) && aligned16(Cb) && aligned16(Za) && aligned16(Zb) && aligned16(Ba) && aligned16(Bb) &&
                  aligned16(Ccomp),
              "csa_compress_varlen: pointers must be 16-byte aligned");
  const int v = vec_elems(dt);
  CSA_REQUIRE(ld_in >= c && ld_out >= c, "csa_compress_varlen: leading dimension too small");
  CSA_REQUIRE(ld_in % v == 0 && ld_out % v == 0,
              "csa_compress_varlen: leading dimensions must keep rows 16-byte aligned");
  csa_status st = check_device();
  if (st != CSA_OK) return st;
  hipError_t e = csa::launch_compress_varlen(dt, n_seqs, m, c, Ca, Cb, Za, Zb, ld_in, Ba, Bb, cu_seqlens,
                                             block_offset, n_blocks, Ccomp, ld_out, (hipStream_t)stream);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "csa_compress_varlen launch");
}

// Workspace of csa_index_topk_varlen (each area 256-byte aligned): scores
// [n_tokens, scores_ld] fp32, q_pos [n_tokens] int64, q_seq [n_tokens] int32,
// block table [n_seqs + 1] int32.
csa_status csa_index_topk_varlen_workspace(int64_t n_seqs, int64_t n_tokens, int64_t max_cand, int32_t k,
                                           size_t* bytes) {
  CSA_REQUIRE(bytes, "csa_index_topk_varlen_workspace: null bytes");
  CSA_REQUIRE(n_seqs >= 0 && n_tokens >= 0 && max_cand >= 0 && k >= 1, "csa_index_topk_varlen_workspace: bad size");
  using csa::ws_add;
  using csa::ws_align;
  using csa::ws_bytes;
  *bytes = ws_add(ws_add(ws_align(ws_bytes(n_tokens, scores_ld(max_cand), sizeof(float))),
                         ws_align(ws_bytes(n_tokens, sizeof(int64_t)))),
                  ws_add(ws_align(ws_bytes(n_tokens, sizeof(int32_t))), ws_align(ws_bytes(n_seqs + 1, sizeof(int32_t)))));
  CSA_REQUIRE(*bytes < csa::kWorkspaceTooBig, "csa_index_topk_varlen_workspace: sizes too large");
  return CSA_OK;
}

csa_status csa_index_topk_varlen(csa_dtype dt, int64_t n_seqs, int64_t n_tokens, int32_t n_hI, int32_t cI, int32_t m,
                                 int32_t k, const void* qI, const float* wI, const void* KIcomp,
                                 const int64_t* cu_seqlens, const int64_t* kv_offset, int64_t max_cand,
                                 int32_t* idx_out, float* score_out, int32_t* q_seq_out, void* workspace,
                                 size_t ws_bytes, void* stream) {
  CSA_REQUIRE(dtype_ok(dt), "csa_index_topk_varlen: unknown dtype");
  CSA_REQUIRE(n_seqs >= 0 && n_seqs <= 0x7FFFFFFF && n_tokens >= 0 && n_tokens <= 0x7FFFFFFF,
              "csa_index_topk_varlen: bad n_seqs / n_tokens");
  CSA_REQUIRE(n_hI >= 1 && n_hI <= 64, "csa_index_topk_varlen: n_hI must be in [1, 64] (got %d)", n_hI);
  CSA_REQUIRE(cI == 32 || cI == 64 || cI == 128 || cI == 256,
              "csa_index_topk_varlen: cI must be 32, 64, 128 or 256 (got %d)", cI);
  CSA_REQUIRE(m >= 1, "csa_index_topk_varlen: m must be >= 1");
  CSA_REQUIRE(k >= 1 && k <= (1 << 24), "csa_index_topk_varlen: k must be in [1, 2^24]");
  CSA_REQUIRE(max_cand >= 0 && max_cand <= 0x7FFFFFFF, "csa_index_topk_varlen: bad max_cand");
  if (n_tokens == 0) return CSA_OK;
  CSA_REQUIRE(n_seqs >= 1, "csa_index_topk_varlen: tokens without sequences");
  CSA_REQUIRE(qI && wI && KIcomp && idx_out && cu_seqlens && kv_offset, "csa_index_topk_varlen: null pointer");
  CSA_REQUIRE(aligned16(qI) && aligned16(wI) && aligned16(KIcomp) && aligned16(idx_out),
              "csa_index_topk_varlen: pointers must be 16-byte aligned");
  size_t need = 0;
  csa_status st0 = csa_index_topk_varlen_workspace(n_seqs, n_tokens, max_cand, k, &need);
  if (st0 != CSA_OK) return st0;
  if (workspace == nullptr || ws_bytes < need)
    return fail(CSA_ERR_WORKSPACE, "csa_index_topk_varlen: workspace needs %zu bytes (got %zu)", need, ws_bytes);
  CSA_REQUIRE(aligned16(workspace), "csa_index_topk_varlen: workspace must be 16-byte aligned");
  csa_status st = check_device();
  if (st != CSA_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  char* ws = (char*)workspace;
  const long ld = scores_ld(max_cand);
  float* scores = (float*)ws;
  size_t at = align256((size_t)n_tokens * ld * sizeof(float));
  int64_t* q_pos = (int64_t*)(ws + at);
  at += align256((size_t)n_tokens * sizeof(int64_t));
  int32_t* q_seq = q_seq_out ? q_seq_out : (int32_t*)(ws + at);
  at += align256((size_t)n_tokens * sizeof(int32_t));
  int32_t* blk = (int32_t*)(ws + at);
  hipError_t e = csa::launch_indexer_varlen(dt, n_seqs, n_tokens, n_hI, cI, m, qI, wI, KIcomp, cu_seqlens, kv_offset,
                                            max_cand, scores, ld, blk, q_pos, q_seq, s);
  if (e != hipSuccess) return hip_fail(e, "csa_index_topk_varlen indexer launch");
  e = csa::launch_topk(n_tokens, m, scores, ld, q_pos, max_cand, k, nullptr, nullptr, idx_out, score_out, s);
  return e == hipSuccess ? CSA_OK : hip_fail(e, "csa_index_topk_varlen top-k launch");
}

}  // extern "C"

