// Top-k selector, eq 9 of "Compressed Sparse Attention": keep, per query, the
// min(k, n_cand) candidates with the largest indexer scores; equal scores go
// to the lower block index; -0.0 equals +0.0.
//
// One workgroup per query row.  Scores are mapped to order-preserving uint32
// keys and the k-th largest key T is found by a 4-pass MSB-first radix select
// (8-bit digits, 256-bin LDS histogram, the bin that crosses the remaining
// count found by one wave's prefix sum).  After it, exactly k - e keys are
// > T and e of the keys == T must be taken; the output pass walks the row in
// index order, one workgroup-wide round at a time, and a block-wide
// exclusive scan of packed (greater, equal) flags gives every kept index a
// deterministic slot: keys > T fill slots [0, k-e), the first e ties in
// index order fill [k-e, k).  The pass stops once both quotas are filled.
#include "common.hpp"
#include "internal.hpp"

namespace csa {
namespace {

template <int TPB>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_wave, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) s_wave[wave] = x;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < TPB / 64; ++w) {
    const uint32_t t = s_wave[w];
    before += (w < wave) ? t : 0u;
    all += t;
  }
  __syncthreads();
  total = all;
  return before + x - v;
}

template <int TPB>
__global__ __launch_bounds__(TPB) void topk_kernel(int m, const float* __restrict__ scores, long ld,
                                                   const int64_t* __restrict__ q_pos, long max_cand,
                                                   int k, int32_t* __restrict__ idx_out,
                                                   float* __restrict__ score_out) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_wave[TPB / 64];
  __shared__ uint32_t s_digit, s_above;

  const int tid = threadIdx.x;
  const long r = blockIdx.x;
  const long pos = q_pos ? q_pos[r] : r;
  long nc = pos > 0 ? pos / m : 0;
  nc = nc < max_cand ? nc : max_cand;
  const float* row = scores + r * ld;
  int32_t* out = idx_out + r * k;
  float* sout = score_out ? score_out + r * k : nullptr;

  if (nc <= k) {  // every candidate is kept
    for (int j = tid; j < k; j += TPB) {
      const bool live = j < nc;
      out[j] = live ? j : -1;
      if (sout) sout[j] = live ? row[j] : -INFINITY;
    }
    return;
  }

  uint32_t prefix = 0, pmask = 0, need = (uint32_t)k;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int i = tid; i < 256; i += TPB) hist[i] = 0;
    __syncthreads();
    for (long s = tid; s < nc; s += TPB) {
      const uint32_t key = score_key(row[s]);
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      uint32_t h[4], sum4 = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        h[q] = hist[255 - 4 * tid - q];
        sum4 += h[q];
      }
      uint32_t incl = sum4;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const uint32_t y = __shfl_up(incl, d);
        if (tid >= d) incl += y;
      }
      const uint32_t excl = incl - sum4;
      if (excl < need && incl >= need) {
        uint32_t cum = excl;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (cum + h[q] >= need) {
            s_digit = 255u - 4u * tid - q;
            s_above = cum;
            break;
          }
          cum += h[q];
        }
      }
    }
    __syncthreads();
    prefix |= s_digit << shift;
    pmask |= 255u << shift;
    need -= s_above;
  }

  const uint32_t T = prefix;
  const uint32_t take_eq = need;
  const uint32_t gt_total = (uint32_t)k - need;
  uint32_t base_gt = 0, base_eq = 0;
  for (long s0 = 0; s0 < nc; s0 += TPB) {
    const long s = s0 + tid;
    const bool live = s < nc;
    const float v = live ? row[s] : 0.f;
    const uint32_t key = score_key(v);
    const bool gt = live && key > T;
    const bool eq = live && key == T;
    uint32_t tot;
    const uint32_t ex = block_excl_scan<TPB>((gt ? 1u : 0u) | (eq ? 0x10000u : 0u), s_wave, tot);
    if (gt) {
      const uint32_t p = base_gt + (ex & 0xFFFFu);
      if (p < gt_total) {  // always true when the select is exact; keeps writes inside the row
        out[p] = (int32_t)s;
        if (sout) sout[p] = v;
      }
    } else if (eq) {
      const uint32_t rank = base_eq + (ex >> 16);
      if (rank < take_eq) {
        out[gt_total + rank] = (int32_t)s;
        if (sout) sout[gt_total + rank] = v;
      }
    }
    base_gt += tot & 0xFFFFu;
    base_eq += tot >> 16;
    if (base_gt >= gt_total && base_eq >= take_eq) break;
  }
}

}  // namespace

hipError_t launch_topk(long n_queries, int m, const float* scores, long ld_sc,
                       const int64_t* q_pos, long max_cand, int k, int32_t* idx_out,
                       float* score_out, hipStream_t s) {
  if (n_queries == 0) return hipSuccess;
  TimedScope t("topk", s);
  if (max_cand >= 16384)
    hipLaunchKernelGGL((topk_kernel<1024>), dim3((unsigned)n_queries), dim3(1024), 0, s, m, scores,
                       ld_sc, q_pos, max_cand, k, idx_out, score_out);
  else
    hipLaunchKernelGGL((topk_kernel<256>), dim3((unsigned)n_queries), dim3(256), 0, s, m, scores,
                       ld_sc, q_pos, max_cand, k, idx_out, score_out);
  return hipGetLastError();
}

}  // namespace csa
