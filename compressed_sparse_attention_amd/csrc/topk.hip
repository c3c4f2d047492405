// Top-k selector, eq 9 of "Compressed Sparse Attention": keep, per query, the
// min(k, n_cand) candidates with the largest indexer scores; equal scores go
// to the lower block index; -0.0 equals +0.0.
//
// One workgroup per query row.  Scores are mapped to order-preserving uint32
// keys (larger score -> larger key) and the k-th largest key T is found by an
// MSB-first radix select:
//   level 1: a 4096-bin histogram of the top 12 key bits -- built by the
//            indexer while it produced the scores (long rows), or here;
//   one ordered pass then selects every key whose 12-bit digit lies above the
//            threshold bin and compacts the keys inside it, in index order,
//            into a small candidate list;
//   levels 2-4: 8+8+4-bit histograms over the candidates only, then one
//            ordered pass over the candidates.
// Rows of up to 8192 candidates are held in registers, 32 consecutive keys per
// thread; longer rows are staged in LDS in segments of 32 x TPB keys
// (coalesced loads; one padding word per 32 keys, so the 64 lanes of a wave
// reading "their" 32 consecutive keys hit 64 different banks).  Thread t owns
// keys [32t, 32t+32) of a segment, so thread order is index order: an ordered pass is one burst
// read and classification per thread, one workgroup-wide exclusive scan, and
// an emit of the (few) selected keys.  Keys > T fill the
// first slots; among keys == T the lowest indices fill the rest, which is
// the tie-break.  The result, slot order included, is deterministic.
#include "common.hpp"
#include "internal.hpp"
#include "select.hpp"

namespace csa {
namespace {

__global__ void hist_clear_kernel(uint32_t* __restrict__ h, long n) {
  const long i = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) h[i] = 0u;
}

// REGS: rows of at most EPT x TPB candidates (max_cand bounds them), keys in
// registers.  Rows of up to 8192 candidates (every prefill row here) take
// 256 threads x 32 keys: at 19.5 KB of LDS and 93 VGPRs five rows share a
// CU, against three with the row staged in LDS (0.53 -> 0.38 ms for the
// 32768-token prefill; 512 x 16 and 1024 x 8 measured 0.41 and 0.65 ms).
constexpr int kShortTPB = 256;
constexpr int kShortEPT = 32;
template <int TPB, bool REGS, int EPT>
__global__ __launch_bounds__(TPB) void topk_kernel(int m, const float* __restrict__ scores, long ld,
                                                   const int64_t* __restrict__ q_pos, long max_cand,
                                                   int k, uint32_t* __restrict__ hist_g,
                                                   int32_t* __restrict__ idx_out,
                                                   float* __restrict__ score_out) {
  __shared__ SelectRowSmem<TPB, REGS> sm;
  const long r = blockIdx.x;
  const long pos = q_pos ? q_pos[r] : r;
  long ncl = pos > 0 ? pos / m : 0;
  ncl = ncl < max_cand ? ncl : max_cand;
  uint32_t* hrow = hist_g ? hist_g + r * kL1Bins : nullptr;
  select_row<TPB, REGS, EPT>(sm, scores + r * ld, ld, (int)ncl, k, hrow, hrow, idx_out + r * k,
                  score_out ? score_out + r * k : nullptr);
}

// ---------------------------------------------------------------------------
// Long rows with the indexer's level-1 histogram: many workgroups per row.
//
// A row of n_cand scores is cut into chunks of kMChunk keys, one 256-thread
// workgroup each (8 keys per thread), so the row is read by many CUs at once.
// Every chunk workgroup fetches the row's histogram, finds the threshold bin
// b1 itself, classifies its keys (digit > b1: selected; digit == b1:
// candidate) and appends both kinds, in index order, to per-chunk lists in
// the workspace.  The last chunk workgroup of a row to finish (a per-row
// arrival counter) then:
//   * copies the selected lists, chunk by chunk, to the first g1 slots;
//   * stages the candidate lists (all chunks, index order) in LDS, runs
//     levels 2-4 on them and emits the rest exactly as the one-workgroup
//     selector does.
// The output, slot order included, is the same as that selector's.
// ---------------------------------------------------------------------------
constexpr int kMTPB = 256;
constexpr int kMEPT = 8;
__global__ __launch_bounds__(kMTPB) void topk_multi_kernel(
    int m, const float* __restrict__ scores, long ld, const int64_t* __restrict__ q_pos, long max_cand, int k,
    uint32_t* __restrict__ hist_g, uint32_t* __restrict__ arrive, uint32_t* __restrict__ counts,
    uint64_t* __restrict__ gt_list, uint64_t* __restrict__ eq_list, int P, int gtc, int32_t* __restrict__ idx_out,
    float* __restrict__ score_out, uint32_t* __restrict__ b1g1) {
  __shared__ uint32_t s_wave[kMTPB / 64];
  __shared__ uint32_t s_res[2];
  __shared__ int s_last;
  __shared__ FinishSmem<kMTPB> fs;

  const int tid = threadIdx.x;
  const long r = blockIdx.x / P;
  const int j = (int)(blockIdx.x - r * P);
  const long pos = q_pos ? q_pos[r] : r;
  long ncl = pos > 0 ? pos / m : 0;
  ncl = ncl < max_cand ? ncl : max_cand;
  const int nc = (int)ncl;
  const float* row = scores + r * ld;
  int32_t* out = idx_out + r * k;
  float* sout = score_out ? score_out + r * k : nullptr;

  if (nc <= k) {  // every candidate is kept
    if (j == 0)
      for (int e = tid; e < k; e += kMTPB) {
        const bool live = e < nc;
        out[e] = live ? e : -1;
        if (sout) sout[e] = live ? row[e] : -INFINITY;
      }
    return;
  }
  const int Pr = (nc + kMChunk - 1) / kMChunk;
  if (j >= Pr) return;

  // ---- chunk phase ------------------------------------------------------------
  // this thread's keys: a .. a+7 (loads clamped into the row; keys past nc unused)
  const long a = (long)j * kMChunk + kMEPT * tid;
  const float4 v0 = *reinterpret_cast<const float4*>(row + (a < ld - 4 ? a : ld - 4));
  const float4 v1 = *reinterpret_cast<const float4*>(row + (a + 4 < ld - 4 ? a + 4 : ld - 4));
  // every chunk workgroup derives the threshold bin from the row's histogram
  level1_threshold<kMTPB>(hist_g + r * kL1Bins, (uint32_t)k, s_wave, s_res);
  const uint32_t b1 = s_res[0];
  const uint32_t g1 = s_res[1];

  const float sv[kMEPT] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
  uint32_t kv[kMEPT];
  uint32_t mg = 0, me = 0;
#pragma unroll
  for (int e = 0; e < kMEPT; ++e) {
    kv[e] = score_key(sv[e]);
    const bool valid = a + e < nc;
    const uint32_t d = kv[e] >> kL1Shift;
    mg |= (uint32_t)(valid && d > b1) << e;
    me |= (uint32_t)(valid && d == b1) << e;
  }
  uint32_t tot2;
  const uint32_t ex2 = block_excl_scan<kMTPB>(__popc(mg) | (__popc(me) << 16), s_wave, tot2);
  uint32_t pg = ex2 & 0xFFFFu, pe = ex2 >> 16;
  // list entries: index in the low word, score bits (gt) or key (eq) in the high word
  uint64_t* gl = gt_list + (r * P + j) * (long)gtc;
  uint64_t* el = eq_list + (r * P + j) * (long)kMChunk;
#pragma unroll
  for (int e = 0; e < kMEPT; ++e) {
    const uint64_t i = (uint64_t)(a + e);
    if ((mg >> e) & 1u) {
      if (pg < (uint32_t)gtc) st_agent(gl + pg, i | ((uint64_t)__float_as_uint(sv[e]) << 32));
      ++pg;
    }
    if ((me >> e) & 1u) st_agent(el + pe++, i | ((uint64_t)kv[e] << 32));
  }
  if (tid == 0) {
    const uint32_t ng = tot2 & 0xFFFFu;
    st_agent(counts + (r * P + j) * 2, ng < (uint32_t)gtc ? ng : (uint32_t)gtc);
    st_agent(counts + (r * P + j) * 2 + 1, tot2 >> 16);
  }
  if (b1g1) {  // classify only: the decode attention finishes the row
    if (j == 0 && tid == 0) {
      b1g1[2 * r] = b1;
      b1g1[2 * r + 1] = g1;
    }
    return;
  }
  // publish the lists, then count this chunk in; the last one finishes the row
  wait_stores();
  __syncthreads();
  if (tid == 0)
    s_last = __hip_atomic_fetch_add(arrive + r, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == (uint32_t)(Pr - 1);
  __syncthreads();
  if (!s_last) return;
  // every chunk of the row has read its histogram: leave it and the counter
  // zero for the next call
  {
    u32x4* h = reinterpret_cast<u32x4*>(hist_g + r * kL1Bins);
    for (int b = tid; b < kL1Bins / 4; b += kMTPB) h[b] = u32x4{0u, 0u, 0u, 0u};
    if (tid == 0) arrive[r] = 0u;
  }
  FinishPrefetch pf;
  finish_prefetch<kMTPB, true>(pf, Pr, counts + r * P * 2, gt_list + r * P * (long)gtc, gtc,
                               eq_list + r * P * (long)kMChunk, kMChunk);
  finish_row<kMTPB, true>(fs, pf, Pr, Pr, k, b1, g1, counts + r * P * 2, gt_list + r * P * (long)gtc, gtc,
                    eq_list + r * P * (long)kMChunk, kMChunk, 0u, (uint32_t)k, [&](uint32_t slot, uint32_t i, float sc) {
                      out[slot] = (int32_t)i;
                      if (sout) sout[slot] = sc;
                    });
}

// ---------------------------------------------------------------------------
// Streaming prefill selection, finishing phase.  Row r (the query at position
// r) exists only as the list the indexer appended (index | score bits << 32,
// in index order), with the threshold bin b of its running histogram (the
// k-th largest score lies in bin b), the count g1 of entries in higher bins
// and the list length.  Entries below b are dropped, those above are
// selected, and the k - g1 still needed come from bin b: levels of 8 + 8 + 5
// bits over bin b's entries (staged in LDS) find the k-th largest key T and
// how many entries equal to T to take (the lowest indices).  The emit is one
// ordered pass over the list: every selected entry, in index order.  Lists
// longer than kLTPB x kLEPT entries are walked in segments (re-read from
// global memory), and bin b's entries are staged in LDS while they fit
// (otherwise the levels re-read the list too).
// ---------------------------------------------------------------------------
constexpr int kLTPB = 256;
constexpr int kLEPT = 32;
constexpr int kLSeg = kLTPB * kLEPT;
constexpr int kLCap = 4096;
constexpr int kLShift = 32 - kStreamBitsTopk;

__global__ __launch_bounds__(kLTPB) void topk_list_kernel(int m, long max_cand, int k, const uint64_t* __restrict__ lists,
                                                         long ld_list, const uint32_t* __restrict__ meta,
                                                         int32_t* __restrict__ idx_out, float* __restrict__ score_out) {
  __shared__ uint32_t s_ckey[kLCap];
  __shared__ uint32_t s_cidx[kLCap];
  __shared__ uint32_t s_h[3][256];
  __shared__ uint32_t s_wave[kLTPB / 64];
  __shared__ uint32_t s_res[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const long r = blockIdx.x;
  long nc = r / m;
  nc = nc < max_cand ? nc : max_cand;
  int32_t* out = idx_out + r * k;
  float* sout = score_out ? score_out + r * k : nullptr;
  if (nc <= k) {  // every candidate is kept: the list holds all of them, entry e = candidate e
    for (int e = tid; e < k; e += kLTPB) {
      const bool live = e < nc;
      out[e] = live ? e : -1;
      if (sout) sout[e] = live ? __uint_as_float((uint32_t)(lists[r * ld_list + e] >> 32)) : -INFINITY;
    }
    return;
  }
  const u32x4 mt = *reinterpret_cast<const u32x4*>(meta + 4 * r);
  const uint32_t bstar = mt.x, g1 = mt.y;
  const long len = (long)mt.z < ld_list ? (long)mt.z : ld_list;
  const uint64_t* row = lists + r * ld_list;
  const int nseg = (int)((len + kLSeg - 1) / kLSeg);
  const int first = tid * kLEPT;

  // this thread's entries of segment sg: [sg * kLSeg + first, + kLEPT), 16-byte loads clamped into the list
  uint64_t ent[kLEPT];
  // Pairs (a, a + 1), a even: rows have an even pitch, so a pair whose first
  // entry is in the list lies inside the row (its second entry, if past the
  // list, is masked); pairs wholly past the list read the list's first pair
  // (every listed row has at least k + 1 >= 2 entries) and are masked.
  auto load_seg = [&](int sg) {
    const long base = (long)sg * kLSeg + first;
#pragma unroll
    for (int j = 0; j < kLEPT / 2; ++j) {
      const long a = base + 2 * j;
      const long at = a < len ? a : 0;
      const u32x4 v = *reinterpret_cast<const u32x4*>(row + at);
      ent[2 * j] = (uint64_t)v.x | ((uint64_t)v.y << 32);
      ent[2 * j + 1] = (uint64_t)v.z | ((uint64_t)v.w << 32);
    }
  };
  auto nvalid = [&](int sg) { return (int)max(0L, min((long)kLEPT, len - (long)sg * kLSeg - first)); };
  auto key_of = [](uint64_t e) { return score_key(__uint_as_float((uint32_t)(e >> 32))); };

  // ---- bin b's entries to LDS (index order), counted ------------------------------
  uint32_t n_eq = 0;
  for (int sg = 0; sg < nseg; ++sg) {
    load_seg(sg);
    const int nv = nvalid(sg);
    uint32_t me = 0;
#pragma unroll
    for (int e = 0; e < kLEPT; ++e) me |= (uint32_t)(e < nv && (key_of(ent[e]) >> kLShift) == bstar) << e;
    uint32_t tot;
    uint32_t p = n_eq + block_excl_scan<kLTPB>(__popc(me), s_wave, tot);
#pragma unroll
    for (int e = 0; e < kLEPT; ++e)
      if ((me >> e) & 1u) {
        if (p < (uint32_t)kLCap) {
          s_cidx[p] = (uint32_t)ent[e];
          s_ckey[p] = key_of(ent[e]);
        }
        ++p;
      }
    n_eq += tot;
  }
  for (int b = tid; b < 3 * 256; b += kLTPB) (&s_h[0][0])[b] = 0u;
  __syncthreads();
  const bool staged = n_eq <= (uint32_t)kLCap;

  // ---- levels over bin b's entries: 8, 8 and 5 more bits -----------------------------
  const int shifts[3] = {kLShift - 8, kLShift - 16, 0};
  const int widths[3] = {8, 8, kLShift - 16};
  uint32_t prefix = bstar << kLShift, pmask = 0xFFFFFFFFu << kLShift, need = (uint32_t)k - g1;
  for (int lv = 0; lv < 3; ++lv) {
    const int sh = shifts[lv];
    const uint32_t dm = (1u << widths[lv]) - 1u;
    uint32_t* h = s_h[lv];
    if (staged) {
      for (uint32_t e = tid; e < n_eq; e += kLTPB) {
        const uint32_t key = s_ckey[e];
        if ((key & pmask) == prefix) atomicAdd(&h[(key >> sh) & dm], 1u);
      }
    } else {
      for (int sg = 0; sg < nseg; ++sg) {
        load_seg(sg);
        const int nv = nvalid(sg);
#pragma unroll
        for (int e = 0; e < kLEPT; ++e) {
          const uint32_t key = key_of(ent[e]);
          if (e < nv && (key & pmask) == prefix) atomicAdd(&h[(key >> sh) & dm], 1u);
        }
      }
    }
    __syncthreads();
    if (wave == 0) {
      if (lane == 0) {
        s_res[0] = 0u;
        s_res[1] = 0u;
      }
      find_bin_wave(h, 1 << widths[lv], need, s_res);
    }
    __syncthreads();
    prefix |= s_res[0] << sh;
    pmask |= dm << sh;
    need -= s_res[1];
  }
  const uint32_t T = prefix;      // the k-th largest key
  const uint32_t take_eq = need;  // entries equal to T to take, lowest indices first

  // ---- ordered emit: every entry above T, and the first take_eq equal to T ----------
  uint32_t run1 = 0, run2 = 0;
  for (int sg = 0; sg < nseg; ++sg) {
    if (nseg > 1 || !staged) load_seg(sg);
    const int nv = nvalid(sg);
    uint32_t m1 = 0, m2 = 0;
#pragma unroll
    for (int e = 0; e < kLEPT; ++e) {
      const uint32_t key = key_of(ent[e]);
      m1 |= (uint32_t)(e < nv && key > T) << e;
      m2 |= (uint32_t)(e < nv && key == T) << e;
    }
    uint32_t tot;
    const uint32_t ex = block_excl_scan<kLTPB>(__popc(m1) | (__popc(m2) << 16), s_wave, tot);
    uint32_t p1 = run1 + (ex & 0xFFFFu), p2 = run2 + (ex >> 16);
    for (uint32_t mm = m1 | m2; mm; mm &= mm - 1) {
      const int e = __ffs(mm) - 1;
      const bool eq = (m2 >> e) & 1u;
      const uint32_t slot = eq ? (p2 < take_eq ? p1 + p2 : 0xFFFFFFFFu) : p1 + min(p2, take_eq);
      if (slot < (uint32_t)k) {
        out[slot] = (int32_t)(uint32_t)ent[e];
        if (sout) sout[slot] = __uint_as_float((uint32_t)(ent[e] >> 32));
      }
      if (eq) ++p2; else ++p1;
    }
    run1 += tot & 0xFFFFu;
    run2 += tot >> 16;
  }
}

template <int TPB, bool REGS, int EPT>
void launch_rows(long n_queries, int m, const float* scores, long ld_sc, const int64_t* q_pos, long max_cand,
            int k, uint32_t* hist, int32_t* idx_out, float* score_out, hipStream_t s) {
  (void)csa::launch("topk", topk_kernel<TPB, REGS, EPT>, dim3((unsigned)n_queries), dim3(TPB), 0, s, m, scores, ld_sc,
                    q_pos, max_cand, k, hist, idx_out, score_out);
}

}  // namespace

hipError_t launch_topk_lists(long n, int m, long max_cand, int k, const uint64_t* lists, long ld_list,
                             const uint32_t* meta, int32_t* idx_out, float* score_out, hipStream_t s) {
  if (n == 0) return hipSuccess;
  return launch("topk", topk_list_kernel, dim3((unsigned)n), dim3(kLTPB), 0, s, m, max_cand, k, lists, ld_list, meta,
                idx_out, score_out);
}

hipError_t launch_hist_clear(uint32_t* hist, long n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  return launch("hist_clear", hist_clear_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, hist, n);
}

hipError_t launch_topk(long n_queries, int m, const float* scores, long ld_sc,
                       const int64_t* q_pos, long max_cand, int k, uint32_t* hist,
                       const TopkLists* lists, int32_t* idx_out, float* score_out, hipStream_t s) {
  if (n_queries == 0) return hipSuccess;
  if (hist && lists) {
    (void)csa::launch("topk", topk_multi_kernel, dim3((unsigned)(n_queries * lists->P)), dim3(kMTPB), 0, s, m,
                      scores, ld_sc, q_pos, max_cand, k, hist, lists->arrive, lists->counts, lists->gt, lists->eq,
                      lists->P, lists->gtc, idx_out, score_out, lists->b1g1);
    return hipGetLastError();
  }
  if (max_cand <= kShortTPB * kShortEPT)  // every row fits in registers
    launch_rows<kShortTPB, true, kShortEPT>(n_queries, m, scores, ld_sc, q_pos, max_cand, k, hist, idx_out,
                                             score_out, s);
  else
    launch_rows<1024, false, kEPT>(n_queries, m, scores, ld_sc, q_pos, max_cand, k, hist, idx_out, score_out, s);
  return hipGetLastError();
}

}  // namespace csa
