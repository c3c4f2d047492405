/*
 * Host-side driver of the C ABI (include/csa.h) for the sanitizer build: every
 * entry point is called with arguments its checks must refuse, with sizes at
 * the edges of what they accept, and with empty batches.  No call here may
 * reach a kernel launch (there need not be a GPU): each must return its status
 * from the host checks.  Built with AddressSanitizer and UndefinedBehaviorSanitizer
 * on the host code of the library (tests/test_sanitize_cpu.py); any report
 * aborts the run.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "../include/csa.h"

static int failures = 0;

#define EXPECT(call, want)                                                                    \
  do {                                                                                        \
    const int got_ = (int)(call);                                                             \
    if (got_ != (int)(want)) {                                                                \
      fprintf(stderr, "line %d: %s returned %d, expected %d (%s)\n", __LINE__, #call, got_,   \
              (int)(want), csa_last_error());                                                 \
      ++failures;                                                                             \
    } else if ((want) != CSA_OK && csa_last_error()[0] == 0) {                                \
      fprintf(stderr, "line %d: %s set no error text\n", __LINE__, #call);                    \
      ++failures;                                                                             \
    }                                                                                         \
  } while (0)

/* any 16-byte aligned, never dereferenced address */
#define P ((void*)(uintptr_t)4096)
#define PF ((float*)(uintptr_t)4096)
#define PI ((int32_t*)(uintptr_t)4096)
#define PL ((int64_t*)(uintptr_t)4096)
#define MIS ((void*)(uintptr_t)4098)

int main(void) {
  size_t b = 0;
  const int64_t big = 0x7FFFFFFFLL;

  if (csa_abi_version() != 1) ++failures;

  /* projections */
  EXPECT(csa_project(CSA_BF16, CSA_BF16, 0, 8, 8, P, 8, P, 8, P, 8, NULL), CSA_ERR_INVALID_ARG);
  EXPECT(csa_project(CSA_BF16, CSA_BF16, 8, 8, 12, P, 16, P, 16, P, 8, NULL), CSA_ERR_INVALID_ARG);
  EXPECT(csa_project(CSA_BF16, CSA_BF16, 8, 8, 8, NULL, 8, P, 8, P, 8, NULL), CSA_ERR_INVALID_ARG);
  EXPECT(csa_project(CSA_BF16, CSA_BF16, 8, 8, 8, MIS, 8, P, 8, P, 8, NULL), CSA_ERR_INVALID_ARG);
  EXPECT(csa_project((csa_dtype)7, CSA_BF16, 8, 8, 8, P, 8, P, 8, P, 8, NULL), CSA_ERR_INVALID_ARG);
  EXPECT(csa_project(CSA_BF16, CSA_BF16, INT64_MAX, INT64_MAX, 8, P, 8, P, 8, P, INT64_MAX, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_project(CSA_BF16, CSA_BF16, 8, 8, 8, P, -8, P, 8, P, 8, NULL), CSA_ERR_INVALID_ARG);
  EXPECT(csa_project_pair(CSA_BF16, 8, 8, P, 8, CSA_BF16, 0, P, 8, P, 8, CSA_BF16, 8, P, 8, P, 8, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_project_pair(CSA_BF16, 8, 8, P, 8, CSA_BF16, 8, P, 8, P, 8, CSA_BF16, 8, NULL, 8, P, 8, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_project_pair(CSA_BF16, 8, 8, P, 8, CSA_BF16, 8, P, 8, P, 8, CSA_BF16, 8, P, 8, MIS, 8, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_project_backward_workspace(CSA_BF16, -1, 64, 32, 1, 1, &b), CSA_ERR_INVALID_ARG);
  EXPECT(csa_project_backward_workspace(CSA_BF16, big, big, big, 1, 1, &b), CSA_ERR_INVALID_ARG);
  EXPECT(csa_project_backward_workspace(CSA_BF16, 10, 64, 32, 1, 1, NULL), CSA_ERR_INVALID_ARG);
  EXPECT(csa_project_backward(CSA_BF16, CSA_BF16, 64, 60, 64, P, 64, P, 64, P, 60, P, 64, P, 64, P, 1 << 30, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_project_backward(CSA_BF16, CSA_BF16, 64, 64, 64, P, 64, P, 64, P, 64, P, 64, P, 64, P, 16, NULL),
         CSA_ERR_WORKSPACE);

  /* compression */
  EXPECT(csa_compress(CSA_BF16, 64, 0, 64, P, P, P, P, 256, P, P, P, 64, NULL), CSA_ERR_INVALID_ARG);
  EXPECT(csa_compress(CSA_BF16, 64, 4, 6, P, P, P, P, 256, P, P, P, 64, NULL), CSA_ERR_INVALID_ARG);
  EXPECT(csa_compress(CSA_BF16, 64, 4, 64, P, NULL, P, P, 256, P, P, P, 64, NULL), CSA_ERR_INVALID_ARG);
  EXPECT(csa_compress(CSA_BF16, 64, 4, 64, P, P, P, P, 60, P, P, P, 64, NULL), CSA_ERR_INVALID_ARG);
  EXPECT(csa_compress(CSA_BF16, -5, 4, 64, P, P, P, P, 256, P, P, P, 64, NULL), CSA_ERR_INVALID_ARG);
  EXPECT(csa_compress(CSA_BF16, 3, 4, 64, NULL, NULL, NULL, NULL, 64, NULL, NULL, NULL, 64, NULL), CSA_OK);
  EXPECT(csa_compress(CSA_BF16, INT64_MAX, 1, 64, P, P, P, P, INT64_MAX, P, P, P, INT64_MAX, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_compress_append(CSA_BF16, 2, 0, 64, P, 256, P, P, P, PL, PL, P, 64, NULL), CSA_ERR_INVALID_ARG);
  EXPECT(csa_compress_append(CSA_BF16, 2, 65, 64, P, 256, P, P, P, PL, PL, P, 64, NULL), CSA_ERR_INVALID_ARG);
  EXPECT(csa_compress_append(CSA_BF16, 2, 4, 64, P, 255, P, P, P, PL, PL, P, 64, NULL), CSA_ERR_INVALID_ARG);
  EXPECT(csa_compress_append(CSA_BF16, 2, 4, 64, P, 256, P, P, P, NULL, PL, P, 64, NULL), CSA_ERR_INVALID_ARG);
  EXPECT(csa_compress_append(CSA_BF16, 0, 4, 64, NULL, 256, NULL, P, P, PL, PL, P, 64, NULL), CSA_OK);
  EXPECT(csa_compress_backward_workspace(-1, 4, 64, &b), CSA_ERR_INVALID_ARG);
  EXPECT(csa_compress_backward_workspace(big, 16, 1 << 20, &b), CSA_OK); /* partials per workgroup row only */
  if (b >= ((size_t)1 << 40)) ++failures;
  EXPECT(csa_compress_backward(CSA_BF16, 64, 17, 64, P, P, P, P, 256, P, P, PF, 64, P, P, P, P, 256, PF, PF, P,
                               1 << 30, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_compress_backward(CSA_BF16, 64, 4, 64, P, P, P, P, 256, P, P, PF, 64, P, P, P, P, 256, PF, PF, P, 8,
                               NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_compress_varlen(CSA_BF16, 3, 0, 64, P, P, P, P, 256, P, P, PL, PL, 10, P, 64, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_compress_varlen(CSA_BF16, 3, 4, 64, P, P, P, P, 256, P, P, NULL, PL, 10, P, 64, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_compress_varlen(CSA_BF16, 3, 4, 64, P, P, P, P, 256, P, P, NULL, NULL, 0, P, 64, NULL), CSA_OK);
  EXPECT(csa_compress_backward_varlen_workspace(-1, 10, 4, 64, &b), CSA_ERR_INVALID_ARG);
  EXPECT(csa_compress_backward_varlen_workspace(big, big, 16, 1 << 20, &b), CSA_OK);
  EXPECT(csa_compress_backward_varlen_workspace(big + 1, 10, 4, 64, &b), CSA_ERR_INVALID_ARG);
  EXPECT(csa_compress_backward_varlen(CSA_BF16, 0, 4, 64, P, P, P, P, 256, P, P, PL, PL, 3, PF, 64, P, P, P, P,
                                      256, PF, PF, P, 1 << 30, NULL),
         CSA_ERR_INVALID_ARG);

  /* indexer + top-k */
  EXPECT(csa_index_topk_workspace(-1, 10, 4, 4, &b), CSA_ERR_INVALID_ARG);
  EXPECT(csa_index_topk_workspace(big, big, 64, 1 << 24, &b), CSA_ERR_INVALID_ARG);
  EXPECT(csa_index_topk_workspace(8, 32768, 64, 1024, NULL), CSA_ERR_INVALID_ARG);
  EXPECT(csa_index_topk_workspace(8, 32768, 64, 1024, &b), CSA_OK);
  if (b < (size_t)8 * 32768 * 4) ++failures;
  EXPECT(csa_index_topk(CSA_BF16, 4, 65, 128, 4, 16, P, PF, P, NULL, NULL, NULL, 100, PI, NULL, P, 1 << 20, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_index_topk(CSA_BF16, 4, 64, 96, 4, 16, P, PF, P, NULL, NULL, NULL, 100, PI, NULL, P, 1 << 20, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_index_topk(CSA_BF16, 4, 64, 128, 4, 0, P, PF, P, NULL, NULL, NULL, 100, PI, NULL, P, 1 << 20, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_index_topk(CSA_BF16, 4, 64, 128, 4, 16, NULL, PF, P, NULL, NULL, NULL, 100, PI, NULL, P, 1 << 20,
                        NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_index_topk(CSA_BF16, 4, 64, 128, 4, 16, P, PF, P, NULL, NULL, NULL, 100, PI, NULL, P, 10, NULL),
         CSA_ERR_WORKSPACE);
  EXPECT(csa_index_topk(CSA_BF16, 4, 64, 128, 4, 16, P, PF, P, NULL, NULL, NULL, big + 1, PI, NULL, P, 1 << 20,
                        NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_index_topk(CSA_BF16, 0, 64, 128, 4, 16, NULL, NULL, NULL, NULL, NULL, NULL, 100, NULL, NULL, NULL, 0,
                        NULL),
         CSA_OK);
  EXPECT(csa_index_topk_varlen_workspace(-1, 100, 30, 16, &b), CSA_ERR_INVALID_ARG);
  EXPECT(csa_index_topk_varlen_workspace(big, big, big, 16, &b), CSA_ERR_INVALID_ARG);
  EXPECT(csa_index_topk_varlen(CSA_BF16, 2, 100, 8, 96, 4, 16, P, PF, P, PL, PL, 30, PI, NULL, NULL, P, 1 << 30,
                               NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_index_topk_varlen(CSA_BF16, 0, 100, 8, 64, 4, 16, P, PF, P, PL, PL, 30, PI, NULL, NULL, P, 1 << 30,
                               NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_index_topk_varlen(CSA_BF16, 2, 100, 8, 64, 4, 16, P, PF, P, PL, PL, 30, PI, NULL, NULL, P, 8, NULL),
         CSA_ERR_WORKSPACE);

  /* streaming prefill selection */
  EXPECT(csa_index_topk_stream_workspace(-1, 100, &b), CSA_ERR_INVALID_ARG);
  EXPECT(csa_index_topk_stream_workspace(big, 65536, &b), CSA_ERR_INVALID_ARG);
  EXPECT(csa_index_topk_stream_workspace(big, 65535, &b), CSA_OK);
  EXPECT(csa_index_topk_stream(CSA_BF16, 100, 8, 96, 4, 16, P, PF, P, 25, PI, NULL, P, 1 << 30, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_index_topk_stream(CSA_BF16, 100, 8, 64, 4, 16, P, PF, P, 70000, PI, NULL, P, 1 << 30, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_index_topk_stream(CSA_BF16, 100, 8, 64, 4, 16, P, PF, P, 25, PI, (float*)MIS, P, 1 << 30, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_index_topk_stream(CSA_BF16, 100, 8, 64, 4, 16, P, PF, P, 25, PI, NULL, P, 8, NULL), CSA_ERR_WORKSPACE);
  EXPECT(csa_index_topk_stream(CSA_BF16, 0, 8, 64, 4, 16, NULL, NULL, NULL, 25, NULL, NULL, NULL, 0, NULL), CSA_OK);

  /* attention */
  EXPECT(csa_sparse_mqa_workspace(-1, 64, 512, 1024, &b), CSA_ERR_INVALID_ARG);
  EXPECT(csa_sparse_mqa_workspace(big, 256, 1024, 1 << 24, &b), CSA_OK); /* a large batch is not split */
  if (b != 0) ++failures;
  EXPECT(csa_sparse_mqa_workspace(1, 1, 64, 1 << 24, &b), CSA_OK); /* one query, many splits */
  EXPECT(csa_sparse_mqa_workspace(8, 64, 512, 1024, &b), CSA_OK);
  EXPECT(csa_sparse_mqa(CSA_BF16, 2, 64, 96, 1024, 0.04f, P, P, NULL, NULL, PI, P, NULL, P, 1 << 30, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_sparse_mqa(CSA_BF16, 2, 0, 512, 1024, 0.04f, P, P, NULL, NULL, PI, P, NULL, P, 1 << 30, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_sparse_mqa(CSA_BF16, 2, 64, 512, 1024, -1.f, P, P, NULL, NULL, PI, P, NULL, P, 1 << 30, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_sparse_mqa(CSA_BF16, 2, 64, 512, 1024, NAN, P, P, NULL, NULL, PI, P, NULL, P, 1 << 30, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_sparse_mqa(CSA_BF16, 2, 64, 512, 1024, 0.04f, P, P, NULL, NULL, PI, NULL, NULL, P, 1 << 30, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_sparse_mqa(CSA_BF16, 2, 64, 512, 1024, 0.04f, P, P, NULL, NULL, PI, P, NULL, P, 64, NULL),
         CSA_ERR_WORKSPACE);
  EXPECT(csa_sparse_mqa_backward_workspace(-1, 64, 512, 512, 100, &b), CSA_ERR_INVALID_ARG);
  EXPECT(csa_sparse_mqa_backward_workspace(big, 256, 512, 1 << 20, big - 1, &b), CSA_OK);
  EXPECT(csa_sparse_mqa_backward_workspace(big, 256, 512, 1 << 20, big, &b), CSA_ERR_INVALID_ARG);
  EXPECT(csa_sparse_mqa_backward(CSA_F32, 4, 64, 512, 64, 0.05f, P, P, 100, NULL, NULL, PI, P, PF, P, P, PF, P,
                                 1 << 30, NULL),
         CSA_ERR_UNSUPPORTED);
  EXPECT(csa_sparse_mqa_backward(CSA_BF16, 4, 64, 256, 64, 0.05f, P, P, 100, NULL, NULL, PI, P, PF, P, P, PF, P,
                                 1 << 30, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_sparse_mqa_backward(CSA_BF16, 4, 64, 512, 64, 0.05f, P, P, 100, NULL, NULL, PI, P, PF, P, P, PF, P,
                                 100, NULL),
         CSA_ERR_WORKSPACE);

  /* the decode step */
  EXPECT(csa_decode_workspace(8, 32768, 64, 64, 512, 1024, &b), CSA_OK);
  EXPECT(csa_decode_workspace(big, big, 64, 256, 1024, 1 << 24, &b), CSA_ERR_INVALID_ARG);
  EXPECT(csa_decode(CSA_BF16, 2, 8, 64, 16, 128, 4, 64, 0.1f, P, PF, P, P, P, NULL, NULL, NULL, 1000, PI, NULL, P,
                    NULL, P, 1 << 30, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_decode(CSA_BF16, 2, 8, 64, 16, 128, 4, 64, 0.1f, P, PF, P, P, MIS, NULL, PL, NULL, 1000, PI, NULL, P,
                    NULL, P, 1 << 30, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_decode(CSA_BF16, 2, 8, 64, 16, 128, 4, 64, 0.1f, P, PF, P, P, P, NULL, PL, NULL, 1000, PI, NULL, P,
                    NULL, P, 10, NULL),
         CSA_ERR_WORKSPACE);
  EXPECT(csa_decode(CSA_BF16, 0, 8, 64, 16, 128, 4, 64, 0.1f, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1000,
                    NULL, NULL, NULL, NULL, NULL, 0, NULL),
         CSA_OK);
  EXPECT(csa_decode_noalloc(CSA_BF16, 2, 8, 64, 16, 96, 4, 64, 0.1f, P, PF, P, P, P, NULL, PL, NULL, 1000, PI, NULL,
                            P, NULL, NULL),
         CSA_ERR_INVALID_ARG);
  EXPECT(csa_decode_noalloc(CSA_BF16, 64, 64, 128, 64, 512, 4, 1024, 0.04f, P, PF, P, P, P, NULL, PL, NULL, 131072,
                            PI, NULL, P, NULL, NULL),
         CSA_ERR_WORKSPACE);
  EXPECT(csa_decode_noalloc(CSA_BF16, big, 64, 128, 256, 1024, 4, 1 << 24, 0.04f, P, PF, P, P, P, NULL, PL, NULL,
                            big, PI, NULL, P, NULL, NULL),
         CSA_ERR_INVALID_ARG); /* sizes whose workspace arithmetic saturates */

  /* instrumentation */
  EXPECT(csa_timing_enable(0), CSA_OK);
  EXPECT(csa_timing_reset(), CSA_OK);
  {
    double ms = -1.0;
    int64_t n = -1;
    EXPECT(csa_timing_read("gemm", &ms, &n), CSA_OK);
    EXPECT(csa_timing_read(NULL, &ms, &n), CSA_ERR_INVALID_ARG);
  }

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("ABI_DRIVER_OK\n");
  return 0;
}
