// Internal launcher interface between the C-ABI layer (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/csa.h"

namespace csa {

// Records a HIP event pair around the enclosed launches when kernel timing is
// enabled (csa_timing_enable); a no-op otherwise.
class TimedScope {
 public:
  TimedScope(const char* family, hipStream_t s);
  ~TimedScope();
  TimedScope(const TimedScope&) = delete;
  TimedScope& operator=(const TimedScope&) = delete;

 private:
  const char* family_;
  hipStream_t stream_;
  hipEvent_t start_ = nullptr;
};

hipError_t launch_gemm(csa_dtype in_dt, csa_dtype out_dt, long M, long N, long K, const void* X,
                       long ldx, const void* W, long ldw, void* Y, long ldy, hipStream_t s);

hipError_t launch_compress(csa_dtype dt, long n, int m, int c, const void* Ca, const void* Cb,
                           const void* Za, const void* Zb, long ld_in, const void* Ba,
                           const void* Bb, void* out, long ld_out, hipStream_t s);

// Scores of eq 8 for every query and candidate into `scores` [n_queries, ld_sc].
hipError_t launch_indexer(csa_dtype dt, long n_queries, int nhI, int cI, int m, const void* qI,
                          const float* wI, const void* K, const int32_t* q_seq,
                          const int64_t* q_pos, const int64_t* kv_offset, long max_cand,
                          float* scores, long ld_sc, hipStream_t s);

// Eq 9 selection per row of `scores`.
hipError_t launch_topk(long n_queries, int m, const float* scores, long ld_sc,
                       const int64_t* q_pos, long max_cand, int k, int32_t* idx_out,
                       float* score_out, hipStream_t s);

bool mqa_supported_c(int c);
size_t mqa_workspace_bytes(long n_queries, int nh, int c, int k);
hipError_t launch_mqa(csa_dtype dt, long n_queries, int nh, int c, int k, float scale,
                      const void* q, const void* C, const int32_t* q_seq,
                      const int64_t* kv_offset, const int32_t* idx, void* o, float* lse,
                      void* workspace, hipStream_t s);

}  // namespace csa
