/*
 * csa.h -- C ABI of the Compressed Sparse Attention (CSA) hot path on one
 * AMD Instinct MI355X (gfx950) GPU.
 *
 * The operations are those of the web page "Compressed Sparse Attention
 * (压缩稀疏注意力)" (cnblogs): the linear projections of eqs 1, 2, 5, 6, 7 and
 * 10; the softmax-gated overlapping compression of eqs 3-4 (section
 * "Compressed Key-Value Entries"); the lightning indexer of eq 8 with the
 * top-k selector of eq 9 (section "Lightning Indexer for Sparse Selection");
 * and the shared-key-value multi-query attention of eq 11 (section "Shared
 * Key-Value MQA").
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every array argument is a DEVICE pointer into memory the caller owns.
 *   Sizes, strides, scalars and the `bytes` out-parameters are host values.
 *   The library never allocates, frees or keeps device memory; scratch
 *   space is the caller-provided `workspace` sized by the *_workspace query.
 * - Every call enqueues its kernels on `stream` (a hipStream_t; NULL means
 *   the null stream) and returns without synchronising.  Outputs are valid
 *   once the stream has reached that point.
 * - Arrays are row-major.  A "leading dimension" (ld*) is the distance, in
 *   elements, between consecutive rows; it must be >= the row length.
 * - Device pointers must be 16-byte aligned and every leading dimension must
 *   keep rows 16-byte aligned (a multiple of 8 for bf16, 4 for fp32).
 * - Errors: argument validation happens before any launch.  A failing call
 *   returns a nonzero csa_status, enqueues nothing, leaves every output
 *   untouched and sets a thread-local message readable by csa_last_error().
 *   A failed launch returns CSA_ERR_HIP.  Faults inside kernels surface, as
 *   usual in HIP, at the caller's next synchronisation.  No C++ exception
 *   crosses this interface.
 * - The library is thread-safe.  Its global state: a per-device property
 *   cache filled once, the thread-local error text, the timing records of
 *   csa_timing_enable (guarded by a lock), and the static scratch array of
 *   csa_decode_noalloc with its per-device address (looked up once, under a
 *   lock; calls that use the array race as described there).  Calls that
 *   share a workspace or output buffer on the same device race unless they
 *   are ordered on one stream.
 * - Inputs must be finite (no NaN/Inf); behaviour on non-finite input is
 *   unspecified.
 * - The first call on a device checks that it is a gfx950 GPU and returns
 *   CSA_ERR_UNSUPPORTED otherwise.
 */
#ifndef CSA_H
#define CSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CSA_ABI_VERSION 1

typedef enum {
  CSA_OK = 0,
  CSA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misalignment, bad dtype */
  CSA_ERR_UNSUPPORTED = 2, /* device is not gfx950, or a shape the kernels do not cover */
  CSA_ERR_WORKSPACE = 3,   /* workspace missing or smaller than the query returned */
  CSA_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} csa_status;

typedef enum {
  CSA_F32 = 0, /* IEEE binary32 */
  CSA_BF16 = 1, /* bfloat16 (upper half of binary32), round-to-nearest-even on store */
  /* not dtypes: they make every int32 a value of this type, so an unknown
     dtype passed by a caller is refused (CSA_ERR_INVALID_ARG), not undefined */
  CSA_DTYPE_RANGE_MIN_ = -0x7FFFFFFF - 1,
  CSA_DTYPE_RANGE_MAX_ = 0x7FFFFFFF
} csa_dtype;

/* Version of this interface (CSA_ABI_VERSION of the built library). */
int csa_abi_version(void);

/* Message describing the last failure on the calling thread ("" if none).
 * The pointer stays valid until the thread's next failing call. */
const char* csa_last_error(void);

/*
 * csa_project -- Y = X . W   (eqs 1, 2, 5, 6, 7 and 10 are all of this form:
 * C^a = H W^aKV, C^b = H W^bKV, Z^a = H W^aZ, Z^b = H W^bZ, c^Q = H W^DQ,
 * q^I = c^Q W^UQ(indexer), w^I = H W^w, q = c^Q W^UQ(attention)).
 *
 *   X   [M, K]  row-major, leading dimension ldx, dtype in_dt
 *   Wt  [N, K]  W stored TRANSPOSED (row n holds column n of W, the way a
 *               linear layer keeps its weight), leading dimension ldw, in_dt
 *   Y   [M, N]  row-major, leading dimension ldy, dtype out_dt
 *
 * Products accumulate in fp32.  Supported (in_dt, out_dt): (F32, F32),
 * (BF16, BF16), (BF16, F32).  Several projections that share X are one call
 * with their weights stacked along N; a column slice of a wider Y is written
 * by passing Y + col0 with the wide ldy.  K must be a multiple of 8.
 * M, N, K > 0.
 */
csa_status csa_project(csa_dtype in_dt, csa_dtype out_dt, int64_t M, int64_t N, int64_t K,
                       const void* X, int64_t ldx, const void* Wt, int64_t ldw, void* Y,
                       int64_t ldy, void* stream);

/*
 * csa_project_pair -- Y1 = X . W1 and Y2 = X . W2 for two projections of the
 * same rows X whose outputs cannot share one stacked call (different output
 * dtypes or separate buffers): eqs 1, 2, 5 with eq 7 (H times the stacked
 * W^aKV | W^bKV | W^aZ | W^bZ | W^DQ, and H W^w), or eq 6 with eq 10 (c^Q W^UQ
 * of the indexer and of the attention).
 *
 *   X    [M, K]   row-major, leading dimension ldx, dtype in_dt
 *   Wt1  [N1, K]  W1 transposed as for csa_project, leading dimension ldw1
 *   Y1   [M, N1]  leading dimension ldy1, dtype out_dt1
 *   Wt2, Y2       likewise with N2, ldw2, ldy2, out_dt2
 *
 * Results are those of two csa_project calls.  With at most 16 bf16 rows
 * (one decode token per sequence) both products run in one launch, so a
 * small one (W^w) costs no launch of its own.  The same requirements as
 * csa_project hold for each product; the two outputs must not overlap.
 */
csa_status csa_project_pair(csa_dtype in_dt, int64_t M, int64_t K, const void* X, int64_t ldx, csa_dtype out_dt1,
                            int64_t N1, const void* Wt1, int64_t ldw1, void* Y1, int64_t ldy1, csa_dtype out_dt2,
                            int64_t N2, const void* Wt2, int64_t ldw2, void* Y2, int64_t ldy2, void* stream);

/*
 * csa_project_backward -- gradients of Y = X . W (eqs 1, 2, 5, 6, 7 and 10)
 * given dY, with W stored transposed as for csa_project:
 *
 *   dX  [M, K] = dY . W^T           (skipped when dX is NULL)
 *   dWt [N, K] = dY^T . X  (= (dL/dW)^T, the layout of Wt; skipped when dWt is NULL)
 *
 *   X [M, K], Wt [N, K], dY [M, N]  dtype in_dt, row-major with leading dimensions ldx, ldw, ldy
 *   dX, dWt                         dtype out_dt, leading dimensions ld_dx, ld_dw
 *
 * Both products run on the projection GEMM kernels after the operands are
 * transposed into the workspace (csa_project_backward_workspace bytes:
 * K x N for dX, (N + K) x roundup(M, 8) for dWt, elements of in_dt; the
 * token axis is zero-padded to a multiple of 8).  Accumulation is fp32.
 * Supported (in_dt, out_dt) as csa_project; N and K multiples of 8; dWt
 * needs M > 0.
 */
csa_status csa_project_backward_workspace(csa_dtype in_dt, int64_t M, int64_t N, int64_t K, int want_dx, int want_dw,
                                          size_t* bytes);
csa_status csa_project_backward(csa_dtype in_dt, csa_dtype out_dt, int64_t M, int64_t N, int64_t K, const void* X,
                                int64_t ldx, const void* Wt, int64_t ldw, const void* dY, int64_t ldy, void* dX,
                                int64_t ld_dx, void* dWt, int64_t ld_dw, void* workspace, size_t ws_bytes,
                                void* stream);

/*
 * csa_compress -- eqs 3-4: for every block i = 0 .. floor(n/m)-1 and channel j,
 * softmax over the 2m logits Z^a[m*i+r, j] + B^a[r, j] and
 * Z^b[m*(i-1)+r, j] + B^b[r, j] (r < m), then
 * Ccomp[i, j] = sum_r S^a_r C^a[m*i+r, j] + sum_r S^b_r C^b[m*(i-1)+r, j].
 * Block 0 has no b-terms (the page pads them with -inf logits and zero values).
 * Trailing rows n mod m form no block.  The same call produces the indexer
 * keys K^IComp from the indexer's own projections and biases.
 *
 *   Ca, Cb, Za, Zb  [n, c]  leading dimension ld_in (they may be column slices
 *                           of one [n, >= 4c] projection output)
 *   Ba, Bb          [m, c]  contiguous
 *   Ccomp           [floor(n/m), c]  leading dimension ld_out
 *   dt              dtype of every array (arithmetic is fp32)
 *
 * n >= 0 (n < m writes nothing), 1 <= m <= 64, c > 0 and a multiple of 4.
 */
csa_status csa_compress(csa_dtype dt, int64_t n, int32_t m, int32_t c, const void* Ca,
                        const void* Cb, const void* Za, const void* Zb, int64_t ld_in,
                        const void* Ba, const void* Bb, void* Ccomp, int64_t ld_out,
                        void* stream);

/*
 * csa_compress_append -- eqs 3-4 applied while decoding, one new token per
 * sequence (section "Compressed Key-Value Entries": every m consecutive
 * entries become one compressed entry, block i's softmax also spanning the
 * b-rows of block i-1).
 *
 * Sequence b's new token is token t = t_new[b] (0-based) of that sequence.
 * Its projected row, laid out [C^a | C^b | Z^a | Z^b] (4c values), starts at
 * new_rows + b * ld_new.  ring [B, 2m, 4c] keeps, per sequence, the rows of
 * its last 2m tokens (token t in slot t mod 2m); the call stores the new row
 * there.  When t completes block i = floor(t/m) (t mod m == m - 1), the
 * compressed entry of block i -- a-terms from the ring rows of block i,
 * b-terms from those of block i-1 (none for i = 0) -- is written to row
 * kv_offset[b] + i of Ccomp (leading dimension ld_out); otherwise Ccomp is
 * not touched.  The ring must already hold the rows of tokens t-2m+1 .. t-1
 * that exist (a prefill leaves its last 2m projected rows there); slots of
 * tokens before 0 are never read.  The caller owns every buffer and reserves
 * the Ccomp rows its sequences grow into.
 *
 *   new_rows  [B rows, >= 4c]  dtype dt, leading dimension ld_new
 *   ring      [B, 2m, 4c]      dtype dt, contiguous, read and written
 *   Ba, Bb    [m, c]           dtype dt, contiguous
 *   t_new, kv_offset  [B] int64 (device)
 *
 * B >= 0, 1 <= m <= 64, c > 0 and a multiple of 4.  Arithmetic is fp32 and
 * matches csa_compress on the same rows.
 */
csa_status csa_compress_append(csa_dtype dt, int64_t B, int32_t m, int32_t c, const void* new_rows,
                               int64_t ld_new, void* ring, const void* Ba, const void* Bb,
                               const int64_t* t_new, const int64_t* kv_offset, void* Ccomp,
                               int64_t ld_out, void* stream);

/*
 * csa_compress_append_pair -- csa_compress_append on two caches of the same
 * B sequences in one launch (the same section and equations): the main
 * cache (width c1) and the indexer's (width c2; "the same operation" on the
 * indexer's projections), both advanced with the same t_new and kv_offset.
 * Each cache's arguments mean what csa_compress_append's do; the limits are
 * the same per cache (B <= 2^30).  Results equal two csa_compress_append
 * calls.  The two caches must not overlap in memory.
 */
csa_status csa_compress_append_pair(csa_dtype dt, int64_t B, int32_t m, const int64_t* t_new,
                                    const int64_t* kv_offset, int32_t c1, const void* new_rows1, int64_t ld_new1,
                                    void* ring1, const void* Ba1, const void* Bb1, void* Ccomp1, int64_t ld_out1,
                                    int32_t c2, const void* new_rows2, int64_t ld_new2, void* ring2,
                                    const void* Ba2, const void* Bb2, void* Ccomp2, int64_t ld_out2, void* stream);

/*
 * csa_compress_backward -- gradients of eqs 3-4 (section "Compressed Key-Value
 * Entries") for one sequence, given dCcomp = dL/dCcomp.  For block i and
 * channel j, with S_r the softmax weights of its 2m pairs (value v_r, logit
 * l_r = Z_r + B_r) and out = Ccomp[i, j]:
 *
 *   dv_r = S_r * dCcomp[i, j],   dl_r = S_r * dCcomp[i, j] * (v_r - out),
 *
 * dl_r going to both Z_r and B_r.  Each projected row gets its a-gradients
 * (dCa, dZa) from its own block and its b-gradients (dCb, dZb) from the next
 * block; rows that no block reads get zeros.  The bias gradients sum over
 * blocks: dBa[r, j] = sum_i dl of a-row r of block i, dBb likewise over the
 * b-rows of blocks 1 .. floor(n/m)-1.
 *
 *   Ca, Cb, Za, Zb      [n, c]  forward inputs, leading dimension ld_in, dtype dt
 *   Ba, Bb              [m, c]  forward biases, contiguous, dtype dt
 *   dCcomp              [floor(n/m), c]  fp32, leading dimension ld_dc
 *   dCa, dCb, dZa, dZb  [n, c]  outputs, dtype dt, leading dimension ld_out
 *                       (they may be column slices of one [n, >= 4c] gradient
 *                       buffer, the layout of the forward projection output)
 *   dBa, dBb            [m, c]  fp32 outputs, contiguous, overwritten
 *   workspace           csa_compress_backward_workspace bytes, 16-byte aligned;
 *                       per-workgroup partial bias gradients, summed by a second
 *                       kernel in a fixed order (the result is deterministic)
 *
 * Arithmetic is fp32 (the forward statistics are recomputed from the inputs).
 * n >= 0, 1 <= m <= 16, c > 0 and a multiple of 4.  Every output row is
 * written exactly once; nothing is accumulated into the caller's buffers.
 */
csa_status csa_compress_backward_workspace(int64_t n, int32_t m, int32_t c, size_t* bytes);
csa_status csa_compress_backward(csa_dtype dt, int64_t n, int32_t m, int32_t c, const void* Ca, const void* Cb,
                                 const void* Za, const void* Zb, int64_t ld_in, const void* Ba, const void* Bb,
                                 const float* dCcomp, int64_t ld_dc, void* dCa, void* dCb, void* dZa, void* dZb,
                                 int64_t ld_out, float* dBa, float* dBb, void* workspace, size_t ws_bytes,
                                 void* stream);

/*
 * csa_compress_backward_varlen -- csa_compress_backward for several sequences
 * packed the way csa_compress_varlen takes them (same section and equations):
 * sequence b owns token rows cu_seqlens[b] .. cu_seqlens[b+1]-1 of Ca, Cb, Za,
 * Zb and of the four gradient outputs, and rows block_offset[b] ..
 * block_offset[b+1]-1 of dCcomp (its blocks, block_offset[b+1] - block_offset[b]
 * = floor(length / m), n_blocks = block_offset[n_seqs]).  Each sequence's
 * gradients are those of csa_compress_backward on its own rows (its block 0
 * has no b-terms; its rows that none of its blocks reads get zeros); dBa and
 * dBb sum over the blocks of every sequence, since the biases are shared.
 * Rows outside every sequence are not written.  cu_seqlens [n_seqs+1] and
 * block_offset [n_seqs+1] are int64 in device memory and must agree as stated;
 * they are not checked.  Other arguments, limits and the workspace rules as
 * csa_compress_backward, with the workspace sized by
 * csa_compress_backward_varlen_workspace.  n_seqs = 0 writes zero bias gradients.
 */
csa_status csa_compress_backward_varlen_workspace(int64_t n_seqs, int64_t n_blocks, int32_t m, int32_t c,
                                                 size_t* bytes);
csa_status csa_compress_backward_varlen(csa_dtype dt, int64_t n_seqs, int32_t m, int32_t c, const void* Ca,
                                        const void* Cb, const void* Za, const void* Zb, int64_t ld_in,
                                        const void* Ba, const void* Bb, const int64_t* cu_seqlens,
                                        const int64_t* block_offset, int64_t n_blocks, const float* dCcomp,
                                        int64_t ld_dc, void* dCa, void* dCb, void* dZa, void* dZb, int64_t ld_out,
                                        float* dBa, float* dBb, void* workspace, size_t ws_bytes, void* stream);

/*
 * csa_index_topk -- eq 8 scores and the eq 9 selection for a batch of queries.
 *
 * Query r belongs to sequence seq = q_seq[r] (q_seq NULL: 0) and sits at token
 * position pos = q_pos[r] (q_pos NULL: pos = r).  Its candidates are the
 * n_cand = min(floor(pos/m), max_cand) compressed blocks s < n_cand of that
 * sequence, whose keys are rows kv_offset[seq] + s of KIcomp (kv_offset
 * NULL: 0).  For a decode query appended after L context tokens, pass
 * pos = L: every one of the floor(L/m) cached blocks is a candidate.
 *
 *   score I[r, s] = sum_h wI[r, h] * max(0, qI[r, h, :] . KIcomp[kv_offset[seq] + s, :])
 *
 * idx_out[r, :] receives the min(k, n_cand) candidates with the largest
 * scores; equal scores are ordered by lower block index, and -0.0 equals
 * +0.0.  The order of indices within a row is unspecified (treat each row
 * as a set).  Slots beyond min(k, n_cand) hold -1.  If score_out is not NULL,
 * score_out[r, j] holds the fp32 score of idx_out[r, j] (-inf for -1 slots).
 *
 *   qI       [n_queries, n_hI, cI]  dtype dt, contiguous
 *   wI       [n_queries, n_hI]      fp32, contiguous
 *   KIcomp   [rows, cI]             dtype dt, contiguous
 *   q_seq    [n_queries] int32 or NULL;  q_pos [n_queries] int64 or NULL
 *   kv_offset[n_seqs] int64 or NULL
 *   idx_out  [n_queries, k] int32;  score_out [n_queries, k] fp32 or NULL
 *
 * Scores are fp32 (products of dt values, fp32 accumulation).  With q_seq and
 * q_pos both NULL (one sequence, query r at position r: a prefill) a tiled
 * kernel shares key tiles between neighbouring queries; otherwise each
 * query sweeps its own keys.  Supported: 1 <= n_hI <= 64, cI a multiple of
 * 32 up to 256, k >= 1, m >= 1, max_cand >= 0.
 */
csa_status csa_index_topk_workspace(int64_t n_queries, int64_t max_cand, int32_t n_hI, int32_t k,
                                    size_t* bytes);
csa_status csa_index_topk(csa_dtype dt, int64_t n_queries, int32_t n_hI, int32_t cI, int32_t m,
                          int32_t k, const void* qI, const float* wI, const void* KIcomp,
                          const int32_t* q_seq, const int64_t* q_pos, const int64_t* kv_offset,
                          int64_t max_cand, int32_t* idx_out, float* score_out, void* workspace,
                          size_t ws_bytes, void* stream);

/*
 * csa_index_topk_stream -- eqs 8-9 for the queries of one sequence's prefill
 * (query t at position t: the layout of csa_index_topk with q_seq, q_pos and
 * kv_offset NULL), without materialising the causal score matrix (section
 * "Lightning Indexer for Sparse Selection": only the top-k of each query's
 * scores is ever used).  While the indexer walks a query's candidates in
 * index order it keeps a histogram of its scores' keys and a running
 * threshold bin b -- the highest bin with at least k of the scores seen so
 * far at or above it -- and appends to the query's list, as (index, score)
 * pairs, only the scores in bins >= b; b only rises, and the final top-k
 * always lies at or above it, so nothing selectable is dropped.  The
 * selection then runs on the lists.  The selected set is the same as
 * csa_index_topk's; idx_out lists each row's selection in increasing index
 * order (csa_index_topk's order within a row is unspecified), and score_out
 * (nullable) gets the matching scores (-inf for -1 slots).
 *
 * The workspace (size from csa_index_topk_stream_workspace: lists of up to
 * max_cand 8-byte entries per query plus 16 bytes of per-query state) needs
 * no initialisation.  Arguments and limits otherwise as csa_index_topk, and:
 * max_cand <= 65535; the tiled kernel's LDS must hold the histograms, so some
 * (dtype, n_hI, cI) combinations return CSA_ERR_UNSUPPORTED (every shape with
 * cI <= 128 is supported).
 */
csa_status csa_index_topk_stream_workspace(int64_t n_queries, int64_t max_cand, size_t* bytes);
csa_status csa_index_topk_stream(csa_dtype dt, int64_t n_queries, int32_t n_hI, int32_t cI, int32_t m, int32_t k,
                                 const void* qI, const float* wI, const void* KIcomp, int64_t max_cand,
                                 int32_t* idx_out, float* score_out, void* workspace, size_t ws_bytes,
                                 void* stream);

/*
 * csa_sparse_mqa -- eq 11: shared key-value multi-query attention over the
 * selected compressed entries.  For query r of sequence seq (q_seq NULL: 0)
 * and head h, with the selected rows C_s = Ccomp[kv_offset[seq] + idx[r, j]]
 * (slots holding -1 are skipped):
 *
 *   o[r, h, :] = sum_s softmax_s(scale * q[r, h, :] . C_s) C_s
 *   lse[r, h]  = log sum_s exp(scale * q[r, h, :] . C_s)
 *
 * Each selected entry is both key and value.  A row with no valid slot gives
 * o = 0 and lse = -inf.  The page leaves the attention scale open; pass
 * 1/sqrt(c) for the usual choice.
 *
 *   q      [n_queries, n_h, c]  dtype dt, contiguous
 *   Ccomp  [rows, c]            dtype dt, contiguous
 *   idx    [n_queries, k] int32, entries in [-1, number of blocks of seq)
 *   o      [n_queries, n_h, c]  dtype dt;  lse [n_queries, n_h] fp32 or NULL
 *
 * Softmax and accumulation are fp32.  Supported: c in {64, 128, 256, 512,
 * 1024}, 1 <= n_h <= 256, 1 <= k <= 2^24.  Small batches split each query's
 * slots across workgroups and merge the partial results through the
 * workspace; when the workspace query returns 0 bytes (large batches),
 * `workspace` may be NULL.
 */
csa_status csa_sparse_mqa_workspace(int64_t n_queries, int32_t n_h, int32_t c, int32_t k,
                                    size_t* bytes);
csa_status csa_sparse_mqa(csa_dtype dt, int64_t n_queries, int32_t n_h, int32_t c, int32_t k,
                          float scale, const void* q, const void* Ccomp, const int32_t* q_seq,
                          const int64_t* kv_offset, const int32_t* idx, void* o, float* lse,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * csa_sparse_mqa_backward -- gradients of eq 11 (section "Shared Key-Value
 * MQA") given dO = dL/do.  With P[r, h, s] = exp(scale q[r, h] . C_s - lse[r, h])
 * over the selected rows C_s = Ccomp[kv_offset[seq] + idx[r, s]] (the
 * forward's softmax, from its lse) and D[r, h] = dO[r, h] . o[r, h]:
 *
 *   dS       = P * (dO[r, h] . C_s - D[r, h])
 *   dq[r, h] = scale * sum_s dS C_s
 *   dCcomp[kv_offset[seq] + idx[r, s]] += sum_h P dO[r, h] + scale * sum_h dS q[r, h]
 *
 * summed over every query and slot that selects a row (each selected entry
 * is both key and value, so both paths add to it).  Slots holding -1 add
 * nothing.
 *
 *   q, dO, o  [n_queries, n_h, c]  bf16, contiguous (o and lse are the forward's outputs)
 *   lse       [n_queries, n_h]     fp32
 *   Ccomp     [n_rows, c]          bf16, contiguous
 *   idx, q_seq, kv_offset          as csa_sparse_mqa
 *   dq        [n_queries, n_h, c]  bf16 output
 *   dCcomp    [n_rows, c]          fp32 output, overwritten (rows nobody selects get 0)
 *   workspace csa_sparse_mqa_backward_workspace bytes, 16-byte aligned
 *
 * Each query's key-gradient share of each selected row is written to the
 * workspace as a bf16 row (rounded once, after fp32 accumulation); the shares
 * are then grouped by row with a counting sort and summed in fp32.  Queries
 * are processed in passes of at most 2^21 (query, slot) pairs per 64-head
 * group, which bounds the workspace at about 2 GiB.  The order of the fp32
 * additions into dCcomp is not fixed (atomic adds at segment boundaries).
 * Supported: bf16, c = 512, 1 <= n_h <= 256, 1 <= k <= 2^20.  Entries of idx
 * must lie in [-1, number of rows of the query's sequence).
 */
csa_status csa_sparse_mqa_backward_workspace(int64_t n_queries, int32_t n_h, int32_t c, int32_t k, int64_t n_rows,
                                             size_t* bytes);
csa_status csa_sparse_mqa_backward(csa_dtype dt, int64_t n_queries, int32_t n_h, int32_t c, int32_t k, float scale,
                                   const void* q, const void* Ccomp, int64_t n_rows, const int32_t* q_seq,
                                   const int64_t* kv_offset, const int32_t* idx, const void* o, const float* lse,
                                   const void* dO, void* dq, float* dCcomp, void* workspace, size_t ws_bytes,
                                   void* stream);

/*
 * Packed sequences (a prefill of several sequences in one call).  Sequence b
 * owns projected rows cu_seqlens[b] .. cu_seqlens[b+1]-1 (cu_seqlens: n_seqs + 1
 * non-decreasing int64 on the device, cu_seqlens[0] = 0); each sequence is
 * compressed and attended on its own, as if it were the only one.
 *
 * csa_compress_varlen -- eqs 3-4 per sequence (section "Compressed Key-Value
 * Entries"): sequence b's floor(len_b / m) blocks go to Ccomp rows
 * block_offset[b] .. block_offset[b+1]-1 (block_offset: n_seqs + 1 int64 on the
 * device, the prefix sums of floor(len_b / m)); n_blocks = block_offset[n_seqs]
 * (host value).  Block 0 of every sequence has no b-terms.  Arguments and
 * limits otherwise as csa_compress.
 *
 * csa_index_topk_varlen -- eqs 8-9 for every token of every sequence (section
 * "Lightning Indexer for Sparse Selection"): token t of sequence b (row
 * cu_seqlens[b] + t) is a query at position t whose candidates are its own
 * sequence's blocks s < floor(t / m), KIcomp rows kv_offset[b] + s (kv_offset:
 * n_seqs int64 on the device, e.g. block_offset).  max_cand >= the largest
 * floor(t / m) of the batch.  Outputs per token as csa_index_topk; q_seq_out
 * (nullable, [n_tokens] int32) receives each token's sequence index, the
 * q_seq that csa_sparse_mqa takes for this batch.  The workspace (size from
 * csa_index_topk_varlen_workspace) needs no initialisation.
 */
csa_status csa_compress_varlen(csa_dtype dt, int64_t n_seqs, int32_t m, int32_t c, const void* Ca, const void* Cb,
                               const void* Za, const void* Zb, int64_t ld_in, const void* Ba, const void* Bb,
                               const int64_t* cu_seqlens, const int64_t* block_offset, int64_t n_blocks, void* Ccomp,
                               int64_t ld_out, void* stream);
csa_status csa_index_topk_varlen_workspace(int64_t n_seqs, int64_t n_tokens, int64_t max_cand, int32_t k,
                                           size_t* bytes);
csa_status csa_index_topk_varlen(csa_dtype dt, int64_t n_seqs, int64_t n_tokens, int32_t n_hI, int32_t cI, int32_t m,
                                 int32_t k, const void* qI, const float* wI, const void* KIcomp,
                                 const int64_t* cu_seqlens, const int64_t* kv_offset, int64_t max_cand,
                                 int32_t* idx_out, float* score_out, int32_t* q_seq_out, void* workspace,
                                 size_t ws_bytes, void* stream);

/*
 * csa_decode -- one decode step for a batch of queries: eqs 8 and 9
 * (csa_index_topk, per-query sweep) then eq 11 (csa_sparse_mqa) on the
 * selected entries, in one call.  Arguments are those of the two calls
 * (q_pos is required; idx_out receives the selection and is then read by
 * the attention).  Results equal csa_index_topk followed by csa_sparse_mqa.
 *
 * Workspace protocol (this is what the call saves over the two-call
 * sequence): the workspace must be zero-filled before its first use and
 * again whenever n_queries, max_cand or k change; every call leaves the
 * parts that must start at zero (score histograms, arrival counters) zero
 * again, so back-to-back calls need no clearing pass.  Calls that share a
 * workspace must not overlap.
 */
csa_status csa_decode_workspace(int64_t n_queries, int64_t max_cand, int32_t n_hI, int32_t n_h, int32_t c,
                                int32_t k, size_t* bytes);
csa_status csa_decode(csa_dtype dt, int64_t n_queries, int32_t n_hI, int32_t cI, int32_t n_h, int32_t c, int32_t m,
                      int32_t k, float scale, const void* qI, const float* wI, const void* KIcomp, const void* q,
                      const void* Ccomp, const int32_t* q_seq, const int64_t* q_pos, const int64_t* kv_offset,
                      int64_t max_cand, int32_t* idx_out, float* score_out, void* o, float* lse, void* workspace,
                      size_t ws_bytes, void* stream);

/*
 * csa_decode_noalloc -- csa_decode without a workspace argument, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation.  It calls no hipMalloc,
 * hipFree or allocating library routine.  Its scratch is one static device
 * array of 32 MiB per GPU, which the library holds until the process ends;
 * sizes whose scratch would not fit (the csa_index_topk workspace plus the
 * csa_sparse_mqa workspace for dt) are refused with CSA_ERR_WORKSPACE before
 * anything is launched.  The 8 x 131072-token, 32 x 8192-token and ragged
 * 64-sequence decode batches of c = 512 fit.
 *
 * Every call on a GPU shares that GPU's array, which keeps what the last call
 * left: each call first clears the parts that must start at zero (with a
 * kernel, so it may be captured in a graph), then proceeds as csa_decode.
 * Calls that overlap on one GPU (other streams, other host threads) race on
 * the array; serialise them.  Arguments, limits and results otherwise as
 * csa_decode (results are identical to it).
 */
csa_status csa_decode_noalloc(csa_dtype dt, int64_t n_queries, int32_t n_hI, int32_t cI, int32_t n_h, int32_t c,
                              int32_t m, int32_t k, float scale, const void* qI, const float* wI, const void* KIcomp,
                              const void* q, const void* Ccomp, const int32_t* q_seq, const int64_t* q_pos,
                              const int64_t* kv_offset, int64_t max_cand, int32_t* idx_out, float* score_out,
                              void* o, float* lse, void* stream);

/*
 * Kernel timing (instrumentation, off by default).  While enabled, every
 * kernel the library launches is bracketed by a pair of HIP events recorded
 * on the launch stream.  csa_timing_read synchronises on the recorded events
 * and returns, for the kernel family `name` ("gemm", "gemm_smallm"
 * (bf16 projections of 16 rows or fewer), "compress", "compress_append",
 * "indexer_sweep", "indexer_prefill", "varlen_meta", "hist_clear", "topk",
 * "mqa", "mqa_combine", and for the backward "compress_bwd",
 * "compress_bias_reduce", "mqa_bwd", "mqa_bwd_zero", "mqa_bwd_sort",
 * "mqa_bwd_reduce", "transpose"),
 * the summed duration in milliseconds and the number of launches since the
 * last reset.  Unknown names give 0 launches.
 */
csa_status csa_timing_enable(int on);
csa_status csa_timing_reset(void);
csa_status csa_timing_read(const char* name, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif

#endif /* CSA_H */
