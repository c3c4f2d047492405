// Internal launcher interface between the C-ABI layer (api.cpp) and the kernels.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa.h"

namespace csa {

// Workspace sizes use saturating arithmetic with 128-bit intermediates: a
// size that reaches kWorkspaceTooBig (far beyond any device) stays there, and
// every size query and every call refuses it, so no query returns a size that
// wrapped around.  Arguments are non-negative (checked before).
constexpr size_t kWorkspaceTooBig = (size_t)1 << 56;
inline size_t ws_sat(unsigned __int128 v) { return v >= kWorkspaceTooBig ? kWorkspaceTooBig : (size_t)v; }
inline size_t ws_bytes(uint64_t a, uint64_t b, uint64_t c = 1, uint64_t d = 1) {
  size_t v = ws_sat((unsigned __int128)a * b);
  v = ws_sat((unsigned __int128)v * c);
  return ws_sat((unsigned __int128)v * d);
}
inline size_t ws_add(size_t a, size_t b) { return ws_sat((unsigned __int128)a + b); }
inline size_t ws_align(size_t b) { return ws_sat(((unsigned __int128)b + 255) & ~(unsigned __int128)255); }

// Kernel timing (csa_timing_*): when enabled, launches carry a start/stop
// event pair in their own dispatch packet, so the elapsed time is the
// kernel's execution time, without the queueing before it.
bool timing_enabled();
void timing_record(const char* family, hipEvent_t start, hipEvent_t stop);

// Every kernel of the library is launched through here.
template <typename F, typename... Args>
hipError_t launch(const char* family, F kernel, dim3 grid, dim3 block, uint32_t lds, hipStream_t s,
                  Args... args) {
  hipEvent_t a = nullptr, b = nullptr;
  if (timing_enabled()) {
    if (hipEventCreate(&a) != hipSuccess) a = nullptr;
    if (a && hipEventCreate(&b) != hipSuccess) {
      (void)hipEventDestroy(a);
      a = nullptr;
      b = nullptr;
    }
  }
  hipExtLaunchKernelGGL(kernel, grid, block, lds, s, a, b, 0, args...);
  const hipError_t e = hipGetLastError();
  if (a) timing_record(family, a, b);
  return e;
}

hipError_t launch_gemm(csa_dtype in_dt, csa_dtype out_dt, long M, long N, long K, const void* X,
                       long ldx, const void* W, long ldw, void* Y, long ldy, hipStream_t s);

// Y1 = X W1 and Y2 = X W2 (one launch when X has at most 16 bf16 rows).
hipError_t launch_gemm_pair(csa_dtype in_dt, long M, long K, const void* X, long ldx, csa_dtype out1, long N1,
                            const void* W1, long ldw1, void* Y1, long ldy1, csa_dtype out2, long N2, const void* W2,
                            long ldw2, void* Y2, long ldy2, hipStream_t s);

// dst[c][r] = src[r][c] (r < R, c < C), zeros for R <= r < Rp; 16-byte granules.
hipError_t launch_transpose(csa_dtype dt, long R, long C, long Rp, const void* src, long lds, void* dst, long ldd,
                            hipStream_t s);

hipError_t launch_compress(csa_dtype dt, long n, int m, int c, const void* Ca, const void* Cb,
                           const void* Za, const void* Zb, long ld_in, const void* Ba,
                           const void* Bb, void* out, long ld_out, hipStream_t s);

// Packed sequences: sequence b's projected rows start at cu[b]; its blocks go
// to output rows boff[b] .. boff[b+1]-1 (nblk = boff[nseq] in total).
hipError_t launch_compress_varlen(csa_dtype dt, long nseq, int m, int c, const void* Ca, const void* Cb,
                                  const void* Za, const void* Zb, long ld_in, const void* Ba, const void* Bb,
                                  const int64_t* cu, const int64_t* boff, long nblk, void* out, long ld_out,
                                  hipStream_t s);

// Backward of eqs 3-4 (see csa_compress_backward and its _varlen form); the
// workspace holds the per-workgroup partial bias gradients.  The size is that
// of one sequence of n tokens, or (varlen) of nseq sequences with nblk blocks.
size_t compress_backward_workspace_bytes(long n, int m, int c, long nseq, long nblk, bool varlen);
hipError_t launch_compress_backward(csa_dtype dt, long n, int m, int c, const void* Ca, const void* Cb,
                                    const void* Za, const void* Zb, long ld_in, const void* Ba, const void* Bb,
                                    const float* dCcomp, long ld_dc, void* dCa, void* dCb, void* dZa, void* dZb,
                                    long ld_out, float* dBa, float* dBb, void* workspace, hipStream_t s);
hipError_t launch_compress_backward_varlen(csa_dtype dt, long nseq, long nblk, int m, int c, const void* Ca,
                                           const void* Cb, const void* Za, const void* Zb, long ld_in,
                                           const void* Ba, const void* Bb, const int64_t* cu, const int64_t* boff,
                                           const float* dCcomp, long ld_dc, void* dCa, void* dCb, void* dZa,
                                           void* dZb, long ld_out, float* dBa, float* dBb, void* workspace,
                                           hipStream_t s);

// One cache of csa_compress_append_pair.
struct AppendCache {
  int c;
  const void* rows;
  long ld_new;
  void* ring;
  const void* Ba;
  const void* Bb;
  void* out;
  long ld_out;
};
hipError_t launch_compress_append_pair(csa_dtype dt, long B, int m, const int64_t* t_new, const int64_t* kv_off,
                                       const AppendCache& a, const AppendCache& b, hipStream_t s);

// Decode-time append (one new token per sequence); see csa_compress_append.
hipError_t launch_compress_append(csa_dtype dt, long B, int m, int c, const void* rows, long ld_new, void* ring,
                                  const void* Ba, const void* Bb, const int64_t* t_new, const int64_t* kv_off,
                                  void* out, long ld_out, hipStream_t s);

// The top-k selector's first radix level: a histogram of the top kTopkL1Bits
// bits of each row's score keys (see score_key).
constexpr int kTopkL1Bits = 12;

// Scores of eq 8 for every query and candidate into `scores` [n_queries, ld_sc].
// When `hist` is not null (per-query sweep only) the kernel also adds the
// level-1 key histogram of each row with more than hist_min candidates into
// hist [n_queries, 2^kTopkL1Bits], which must be zero on entry; the selector
// reads those rows and leaves them zero again.
hipError_t launch_indexer(csa_dtype dt, long n_queries, int nhI, int cI, int m, const void* qI,
                          const float* wI, const void* K, const int32_t* q_seq,
                          const int64_t* q_pos, const int64_t* kv_offset, long max_cand,
                          float* scores, long ld_sc, uint32_t* hist, long hist_min, hipStream_t s);

// Packed sequences (prefill of several sequences in one call): sequence b owns
// rows cu[b] .. cu[b+1]-1 of qI / wI and keys from kv_offset[b].  Fills the
// per-token q_pos / q_seq [ntok] and the tiled kernel's block table blk
// [nseq + 1] (device buffers), then scores every token against its own
// sequence's causal candidates into scores [ntok, ld_sc].
hipError_t launch_indexer_varlen(csa_dtype dt, long nseq, long ntok, int nhI, int cI, int m, const void* qI,
                                 const float* wI, const void* K, const int64_t* cu, const int64_t* kv_offset,
                                 long max_cand, float* scores, long ld_sc, int32_t* blk, int64_t* q_pos,
                                 int32_t* q_seq, hipStream_t s);

hipError_t launch_hist_clear(uint32_t* hist, long n, hipStream_t s);

// bits of the streaming indexer's histogram bins (top bits of score_key)
constexpr int kStreamBitsTopk = 11;

// Streaming prefill selection (one sequence, query t at position t): the
// indexer appends to lists [n, ld_list] (index | score bits << 32) only the
// scores that can still be selected and writes per token meta [n, 4] =
// (threshold bin, count above it, list length, streamed); the list selector
// finishes the top-k from them.  indexer_stream_supported says whether the
// kernel's LDS holds the sizes.
bool indexer_stream_supported(csa_dtype dt, int nhI, int cI, long max_cand);
hipError_t launch_indexer_stream(csa_dtype dt, long n, int nhI, int cI, int m, const void* qI, const float* wI,
                                 const void* K, const int64_t* kv_offset, long max_cand, uint64_t* lists,
                                 long ld_list, uint32_t* meta, int k, hipStream_t s);
hipError_t launch_topk_lists(long n, int m, long max_cand, int k, const uint64_t* lists, long ld_list,
                             const uint32_t* meta, int32_t* idx_out, float* score_out, hipStream_t s);

// Long rows (with the indexer's histogram) can be selected by many
// workgroups per row: chunks of kMChunk keys, at most kMMaxChunks per row.
constexpr int kMChunk = 2048;
constexpr int kMMaxChunks = 64;
constexpr long kMMaxWorkgroups = 4096;  // bounds the list workspace

// Workspace areas of the multi-workgroup selector.  `arrive` [n_queries]
// must be zero on entry (it is cleared together with the histogram) and is
// zero again on exit; the lists need no initialisation.  List entries hold the candidate index in
// the low 32 bits and the fp32 score bits (gt) or the score key (eq) above.
struct TopkLists {
  uint32_t* arrive;  // [n_queries]
  uint32_t* counts;  // [n_queries, P, 2]
  uint64_t* gt;      // [n_queries, P, gtc]
  uint64_t* eq;      // [n_queries, P, kMChunk]
  int P;             // chunks per row: ceil(max_cand / kMChunk)
  int gtc;           // min(kMChunk, k)
  // Not null: the chunk workgroups only classify and publish their lists
  // and each row's (b1, g1) here ([n_queries, 2]); the rows are finished by
  // the decode attention (TileSelect), which also clears `hist`.  Rows with
  // at most k candidates are still written out whole by the top-k launch.
  uint32_t* b1g1 = nullptr;
  uint32_t* hist = nullptr;  // the level-1 histograms the lists were classified with
};

// The decode attention finishing the selection itself (see TopkLists::b1g1):
// every workgroup of the short-batch MQA kernel resolves its query's
// threshold from the published lists, takes the slots of its own split and
// writes them (workgroups of head tile 0) to idx_out / score_out.
struct TileSelect {
  int m;
  const int64_t* q_pos;
  long max_cand;
  TopkLists lists;
  int32_t* idx_out;
  float* score_out;  // nullable
};

// Eq 9 selection per row of `scores`; `hist` (nullable) is the level-1
// histogram produced by the indexer; `lists` (nullable, needs `hist`) selects
// the multi-workgroup path.
hipError_t launch_topk(long n_queries, int m, const float* scores, long ld_sc,
                       const int64_t* q_pos, long max_cand, int k, uint32_t* hist,
                       const TopkLists* lists, int32_t* idx_out, float* score_out, hipStream_t s);

bool mqa_supported_c(int c);
size_t mqa_workspace_bytes(long n_queries, int nh, int c, int k, bool bf16);
// sel (nullable; only where mqa_tile_selects): the attention finishes the
// selection of rows whose top-k launch only classified them (TileSelect);
// idx must then be sel->idx_out.
bool mqa_tile_selects(long n_queries, int nh, int c, int k, bool bf16);
hipError_t launch_mqa(csa_dtype dt, long n_queries, int nh, int c, int k, float scale,
                      const void* q, const void* C, const int32_t* q_seq,
                      const int64_t* kv_offset, const int32_t* idx, void* o, float* lse,
                      void* workspace, hipStream_t s, const TileSelect* sel = nullptr);

// Backward of eq 11 (see csa_sparse_mqa_backward): bf16, c = 512.
size_t mqa_backward_workspace_bytes(long n_queries, int nh, int k, long rows);
hipError_t launch_mqa_backward(long nq, int nh, int k, float scale, const void* q, const void* C, long rows,
                               const int32_t* q_seq, const int64_t* kv_off, const int32_t* idx, const void* o,
                               const float* lse, const void* dO, void* dq, float* dC, void* workspace,
                               hipStream_t s);

}  // namespace csa
