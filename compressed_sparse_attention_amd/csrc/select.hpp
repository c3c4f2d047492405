// Radix-select building blocks of the top-k selector (eq 9 of "Compressed
// Sparse Attention": the min(k, n_cand) largest indexer scores per query,
// equal scores to the lower block index), shared by the selector kernels of
// topk.hip.
//
// Scores are compared as order-preserving uint32 keys (score_key).  The k-th
// largest key T is found MSB first: a 4096-bin histogram of the top 12 bits
// picks the threshold bin b1 (g1 keys lie in higher bins and are all
// selected); the keys inside b1 (the candidates) then go through 8 + 8 + 4-bit
// histograms.  Keys > T fill the first slots in index order; among keys == T
// the lowest indices fill the rest, which is the tie-break.
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace csa {

constexpr int kL1Bins = 1 << kTopkL1Bits;
constexpr int kL1Shift = 32 - kTopkL1Bits;
constexpr int kMSeg = 4096;  // candidates staged in LDS at once by finish_row
constexpr int kMUnroll = 8;  // list entries fetched per thread per batch
// a row handed to finish_row is cut into at most this many chunks
constexpr int kRowChunksMax = kMMaxChunks;

// Inverse of score_key (a -0.0 score comes back as +0.0).
__device__ __forceinline__ float key_score(uint32_t key) {
  const uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __uint_as_float(u);
}

// Exclusive scan over the workgroup; also returns the total.  Contains barriers.
template <int TPB>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_wave, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t x = wave_incl_scan(v);
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

// One wave finds the bin of a small histogram (nbins <= 256) where the count
// from the top reaches `need`; the caller follows with a barrier.
// nbins is 256 or 16.
__device__ __forceinline__ void find_bin_wave(const uint32_t* hist, int nbins, uint32_t need, uint32_t* s_out) {
  const int lane = threadIdx.x & 63;
  // lane l holds bins nbins-1-4l .. nbins-4-4l (highest first); lanes past the
  // histogram hold zeros
  uint32_t h[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int b = nbins - 1 - (4 * lane + q);
    h[q] = b >= 0 ? hist[b] : 0u;
  }
  const uint32_t local = h[0] + h[1] + h[2] + h[3];
  const uint32_t incl = wave_incl_scan(local);
  const uint32_t excl = incl - local;
  if (excl < need && incl >= need) {
    uint32_t cum = excl;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (cum < need && cum + h[q] >= need) {
        s_out[0] = (uint32_t)(nbins - 1 - (4 * lane + q));
        s_out[1] = cum;
      }
      cum += h[q];
    }
  }
}

// Level 1 from a row's 4096-bin histogram in global memory (more than k keys
// in the row): the threshold bin b1 -> s_res[0] and the count of keys in
// higher bins g1 -> s_res[1], valid after the call (it ends with a barrier).
template <int TPB>
__device__ __forceinline__ void level1_threshold(const uint32_t* __restrict__ hrow, uint32_t k, uint32_t* s_wave,
                                                 uint32_t* s_res) {
  constexpr int HPT = kL1Bins / TPB;  // bins per thread: [HPT*tid, HPT*tid + HPT)
  static_assert(HPT % 4 == 0, "bins per thread");
  const int tid = threadIdx.x;
  uint32_t hb[HPT];
  u32x4 hv[HPT / 4];
#pragma unroll
  for (int q = 0; q < HPT / 4; ++q) hv[q] = *reinterpret_cast<const u32x4*>(hrow + HPT * tid + 4 * q);
#pragma unroll
  for (int q = 0; q < HPT / 4; ++q) {
    hb[4 * q] = hv[q].x;
    hb[4 * q + 1] = hv[q].y;
    hb[4 * q + 2] = hv[q].z;
    hb[4 * q + 3] = hv[q].w;
  }
  if (tid == 0) {
    s_res[0] = 0u;
    s_res[1] = 0u;
  }
  uint32_t local = 0;
#pragma unroll
  for (int q = 0; q < HPT; ++q) local += hb[q];
  uint32_t tot;
  const uint32_t excl = block_excl_scan<TPB>(local, s_wave, tot);
  const uint32_t above = tot - excl - local;  // keys in bins above this thread's bins
  if (above < k && above + local >= k) {
    uint32_t cum = above;
#pragma unroll
    for (int q = HPT - 1; q >= 0; --q) {
      if (cum < k && cum + hb[q] >= k) {
        s_res[0] = (uint32_t)(HPT * tid + q);
        s_res[1] = cum;
      }
      cum += hb[q];
    }
  }
  __syncthreads();
}

constexpr int kCandCap = kL1Bins / 2;  // the candidate list (index, key) reuses the level-1 histogram's LDS
constexpr int kEPT = 32;                // keys per thread per segment of select_row

// Scanning bins from the highest digit down, finds the bin where the running
// count reaches `need`; writes the bin and the count strictly above it.
template <int TPB>
__device__ void find_bin(const uint32_t* hist, int nbins, uint32_t need, uint32_t* s_wave,
                         uint32_t* s_out) {
  const int per = (nbins + TPB - 1) / TPB;
  const int tid = threadIdx.x;
  uint32_t local = 0;
  for (int q = 0; q < per; ++q) {
    const int b = nbins - 1 - (tid * per + q);
    if (b >= 0) local += hist[b];
  }
  uint32_t total;
  const uint32_t excl = block_excl_scan<TPB>(local, s_wave, total);
  if (excl < need && excl + local >= need) {
    uint32_t cum = excl;
    for (int q = 0; q < per; ++q) {
      const int b = nbins - 1 - (tid * per + q);
      const uint32_t h = hist[b];
      if (cum + h >= need) {
        s_out[0] = (uint32_t)b;
        s_out[1] = cum;
        break;
      }
      cum += h;
    }
  }
  __syncthreads();
}

// LDS of select_row.  REGS: rows of at most 32 x TPB keys, held in registers
// (no key staging area: about a third of the LDS, so more rows per CU).
template <int TPB, bool REGS = false>
struct SelectRowSmem {
  uint32_t keys[REGS ? 1 : TPB * kEPT + TPB * kEPT / 32];
  // level-1 histogram; afterwards the candidate list: indices in [0, kCandCap),
  // their keys in [kCandCap, 2 kCandCap)
  uint32_t hist[kL1Bins];
  uint32_t h2[3][256];  // levels 2-4
  uint32_t wave[TPB / 64];
  uint32_t res[4];
};

// One workgroup of TPB threads selects row `row` [nc candidates; leading
// dimension ld, a multiple of 4 that is >= nc] into out[0..k) (and sout).
// hist_g (nullable) is the row's level-1 histogram built by the indexer
// sweep; hist_zero (nullable, the same histogram) is cleared once read, so
// the workspace is left zero for its next use.
//
// The row is staged in LDS in segments of 32 x TPB keys (coalesced loads; one
// padding word per 32 keys, so the 64 lanes of a wave reading "their" 32
// consecutive keys hit 64 different banks).  Thread t owns keys [32t, 32t+32)
// of a segment, so thread order is index order: an ordered pass is one burst
// read and classification per thread, one workgroup-wide exclusive scan, and
// an emit of the (few) selected keys.  Level 1 (without hist_g) is built
// here; one ordered pass then selects every key whose 12-bit digit lies
// above the threshold bin and compacts the keys inside it, in index order,
// into a candidate list; levels 2-4 run over the list (or, when it
// overflows, over the whole row again).  Not every thread returns at the
// same point: callers add nothing after it that needs a barrier.
//
// REGS (rows of at most 32 x TPB keys): thread t loads its 32 keys straight
// into registers (eight 16-byte loads 128 bytes apart) instead of staging the
// row in LDS; every pass reads them there, with loop indices that unroll to
// constants.  Results are identical.
template <int TPB, bool REGS = false, int EPT = kEPT>
__device__ __forceinline__ void select_row(SelectRowSmem<TPB, REGS>& sm, const float* __restrict__ row, long ld,
                                           int nc, int k, const uint32_t* hist_g, uint32_t* hist_zero,
                                           int32_t* __restrict__ out, float* __restrict__ sout) {
  static_assert(EPT % 4 == 0 && EPT <= 32 && (REGS || EPT == kEPT), "staging in LDS assumes 32 keys per thread");
  constexpr int SEG = TPB * EPT;     // keys per staged segment
  constexpr int VPT = SEG / 4 / TPB;  // float4 loads per thread per segment
  uint32_t* s_keys = sm.keys;
  uint32_t* s_hist = sm.hist;
  uint32_t(*s_h2)[256] = sm.h2;
  uint32_t* s_wave = sm.wave;
  uint32_t* s_res = sm.res;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  if (nc <= k) {  // every candidate is kept
    for (int j = tid; j < k; j += TPB) {
      const bool live = j < nc;
      out[j] = live ? j : -1;
      if (sout) sout[j] = live ? row[j] : -INFINITY;
    }
    return;
  }
  const int first = tid * EPT;  // this thread's keys: [first, first + EPT) of a segment
  // a vector value, not an array: a run-time index into it becomes register
  // selects (an indexed array would be placed in scratch memory)
  typedef uint32_t KeyRun __attribute__((ext_vector_type(EPT)));
  KeyRun kreg;
  if constexpr (REGS) {  // loads clamped into the row as in stage(); keys past nc are never used
    float4 v[EPT / 4];
#pragma unroll
    for (int j = 0; j < EPT / 4; ++j) {
      const long a = first + 4L * j;
      v[j] = *reinterpret_cast<const float4*>(row + (a < ld - 4 ? a : ld - 4));
    }
#pragma unroll
    for (int j = 0; j < EPT / 4; ++j) {
      kreg[4 * j] = score_key(v[j].x);
      kreg[4 * j + 1] = score_key(v[j].y);
      kreg[4 * j + 2] = score_key(v[j].z);
      kreg[4 * j + 3] = score_key(v[j].w);
    }
  }
  for (int b = tid; b < 3 * 256; b += TPB) (&s_h2[0][0])[b] = 0u;

  const int nseg = (nc + SEG - 1) / SEG;  // 1 when REGS
  const uint32_t* mykeys = s_keys + (REGS ? 0 : first + (first >> 5));
  // key e of this thread's run (e a constant after unrolling when REGS)
  auto key_at = [&](int e) __attribute__((always_inline)) -> uint32_t {
    if constexpr (REGS) return kreg[e];
    else return mykeys[e];
  };
  // Stage segment sg: coalesced 16-byte loads (all issued first) into padded
  // LDS.  Rows live in a workspace whose leading dimension is a multiple of 4
  // and >= nc, so a load clamped to [0, ld-4] stays in bounds; keys past nc
  // are staged but never used.
  auto stage = [&](int sg) {
    if constexpr (REGS) return;  // never called: a REGS row is one segment, already in registers
    __syncthreads();
    const long base = (long)sg * SEG;
    float4 buf[VPT];
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const long a = base + 4L * (tid + j * TPB);
      buf[j] = *reinterpret_cast<const float4*>(row + (a < ld - 4 ? a : ld - 4));
    }
    issue_fence();
#pragma unroll
    for (int j = 0; j < VPT; ++j) {
      const int i = 4 * (tid + j * TPB);
      const int a = i + (i >> 5);
      s_keys[a] = score_key(buf[j].x);
      s_keys[a + 1] = score_key(buf[j].y);
      s_keys[a + 2] = score_key(buf[j].z);
      s_keys[a + 3] = score_key(buf[j].w);
    }
    __syncthreads();
  };
  auto nvalid = [&](int sg) { return max(0, min(EPT, nc - sg * SEG - first)); };
  auto put = [&](uint32_t slot, int i, uint32_t kv) {
    if (slot < (uint32_t)k) {  // always true when the counts are exact; keeps writes in the row
      out[slot] = i;
      if (sout) sout[slot] = key_score(kv);
    }
  };
  // Ordered pass over the whole row: cls(key) in {0, 1, 2}.  Each thread reads
  // its 32 keys in one burst and records the classes as two bit masks; after
  // the workgroup scan it visits only the set bits.  Classes 1 and 2 are
  // numbered separately in index order and handed to emit1 / emit2.
  auto ordered_row = [&](auto&& cls, auto&& emit1, auto&& emit2, uint32_t& tot1,
                         uint32_t& tot2) __attribute__((always_inline)) {
    tot1 = 0;
    tot2 = 0;
    for (int sg = 0; sg < nseg; ++sg) {
      if (nseg > 1) stage(sg);
      const int nv = nvalid(sg);
      uint32_t m1 = 0, m2 = 0;
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const int c = cls(key_at(e));
        m1 |= (uint32_t)(c == 1 && e < nv) << e;
        m2 |= (uint32_t)(c == 2 && e < nv) << e;
      }
      uint32_t tot;
      const uint32_t ex = block_excl_scan<TPB>(__popc(m1) | (__popc(m2) << 16), s_wave, tot);
      uint32_t p1 = tot1 + (ex & 0xFFFFu), p2 = tot2 + (ex >> 16);
      for (uint32_t mm = m1 | m2; mm; mm &= mm - 1) {
        const int e = __ffs(mm) - 1;
        uint32_t kv;
        if constexpr (REGS) {
          kv = kreg[e];
        } else {
          kv = mykeys[e];
        }
        if ((m1 >> e) & 1u)
          emit1(sg * SEG + first + e, kv, p1++);
        else
          emit2(sg * SEG + first + e, kv, p2++);
      }
      tot1 += tot & 0xFFFFu;
      tot2 += tot >> 16;
    }
  };

  // the indexer's histogram is fetched together with the row
  constexpr int HPT = kL1Bins / TPB;  // bins per thread
  uint32_t hreg[HPT];
  if (hist_g) {
#pragma unroll
    for (int q = 0; q < HPT; ++q) hreg[q] = hist_g[q * TPB + tid];
  }
  if (!REGS && nseg == 1) stage(0);

  // ---- level 1: 12-bit digit ----------------------------------------------
  if (hist_g) {
#pragma unroll
    for (int q = 0; q < HPT; ++q) s_hist[q * TPB + tid] = hreg[q];
    if (hist_zero) {  // the caller's histogram is left zero for its next use
#pragma unroll
      for (int q = 0; q < HPT; ++q) hist_zero[q * TPB + tid] = 0u;
    }
    __syncthreads();
  } else {
    for (int b = tid; b < kL1Bins; b += TPB) s_hist[b] = 0u;
    __syncthreads();
    for (int sg = 0; sg < nseg; ++sg) {
      if (nseg > 1) stage(sg);
      const int nv = nvalid(sg);
#pragma unroll
      for (int e = 0; e < EPT; ++e)
        if (e < nv) atomicAdd(&s_hist[key_at(e) >> kL1Shift], 1u);
    }
    __syncthreads();
  }
  find_bin<TPB>(s_hist, kL1Bins, (uint32_t)k, s_wave, s_res);
  const uint32_t b1 = s_res[0];
  const uint32_t g1 = s_res[1];  // keys with a higher digit: all selected
  const uint32_t need1 = (uint32_t)k - g1;

  // Digit > b1: selected.  Digit == b1: candidate list, in index order.
  uint32_t* c_idx = s_hist;
  uint32_t* c_key = s_hist + kCandCap;
  uint32_t n_gt1, n_cand;
  ordered_row([&](uint32_t kv) -> int {
        const uint32_t d = kv >> kL1Shift;
        return d > b1 ? 1 : (d == b1 ? 2 : 0);
      },
      [&](int i, uint32_t kv, uint32_t p) { put(p, i, kv); },
      [&](int i, uint32_t kv, uint32_t p) {
        if (p < (uint32_t)kCandCap) {
          c_idx[p] = (uint32_t)i;
          c_key[p] = kv;
        }
      },
      n_gt1, n_cand);
  __syncthreads();
  const bool listed = n_cand <= (uint32_t)kCandCap;

  // ---- levels 2-4: 8 + 8 + 4 bits ---------------------------------------------
  const int shifts[3] = {12, 4, 0};
  const int widths[3] = {8, 8, 4};
  if (listed) {
    // The candidates fit in the list: one wave finishes the row, with wave-level
    // scans only (no workgroup barriers).
    if (wave != 0) return;
    const int lane = tid & 63;
    uint32_t prefix = b1 << kL1Shift, pmask = 0xFFFFFFFFu << kL1Shift, need = need1;
    for (int lv = 0; lv < 3; ++lv) {
      const int sh = shifts[lv];
      const uint32_t dm = (1u << widths[lv]) - 1u;
      uint32_t* h2 = s_h2[lv];
      for (int j = lane; j < (int)n_cand; j += 64) {
        const uint32_t kv = c_key[j];
        if ((kv & pmask) == prefix) atomicAdd(&h2[(kv >> sh) & dm], 1u);
      }
      __builtin_amdgcn_wave_barrier();
      find_bin_wave(h2, 1 << widths[lv], need, s_res);
      __builtin_amdgcn_wave_barrier();
      prefix |= s_res[0] << sh;
      pmask |= dm << sh;
      need -= s_res[1];
    }
    const uint32_t T = prefix;      // the k-th largest key
    const uint32_t take_eq = need;  // ties at T to take, lowest indices first
    const uint32_t gt2 = need1 - take_eq;
    // list positions [cpt*lane, cpt*lane + cpt); list order is index order
    const int cpt = ((int)n_cand + 63) / 64;
    const int f = lane * cpt;
    const int lim = max(0, min(cpt, (int)n_cand - f));
    uint32_t c1 = 0, c2 = 0;
    for (int e = 0; e < lim; ++e) {
      const uint32_t kv = c_key[f + e];
      c1 += kv > T;
      c2 += kv == T;
    }
    const uint32_t packed = c1 | (c2 << 16);
    const uint32_t ex = wave_incl_scan(packed) - packed;
    uint32_t p1 = ex & 0xFFFFu, p2 = ex >> 16;
    for (int e = 0; e < lim; ++e) {
      const uint32_t kv = c_key[f + e];
      const int i = (int)c_idx[f + e];
      if (kv > T) put(g1 + p1++, i, kv);
      if (kv == T) {
        if (p2 < take_eq) put(g1 + gt2 + p2, i, kv);
        ++p2;
      }
    }
    return;
  }

  // More candidates than the list holds: finish over the whole row.
  uint32_t prefix = b1 << kL1Shift, pmask = 0xFFFFFFFFu << kL1Shift, need = need1;
  for (int lv = 0; lv < 3; ++lv) {
    const int sh = shifts[lv];
    const uint32_t dm = (1u << widths[lv]) - 1u;
    uint32_t* h2 = s_h2[lv];
    for (int sg = 0; sg < nseg; ++sg) {
      if (nseg > 1) stage(sg);
      const int nv = nvalid(sg);
#pragma unroll
      for (int e = 0; e < EPT; ++e) {
        const uint32_t kv = key_at(e);
        if (e < nv && (kv & pmask) == prefix) atomicAdd(&h2[(kv >> sh) & dm], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) find_bin_wave(h2, 1 << widths[lv], need, s_res);
    __syncthreads();
    prefix |= s_res[0] << sh;
    pmask |= dm << sh;
    need -= s_res[1];
  }
  const uint32_t T = prefix;
  const uint32_t take_eq = need;
  const uint32_t gt2 = need1 - take_eq;
  uint32_t t1, t2;
  ordered_row([&](uint32_t kv) -> int {
        if ((kv >> kL1Shift) != b1) return 0;
        return kv > T ? 1 : (kv == T ? 2 : 0);
      },
      [&](int i, uint32_t kv, uint32_t p) { put(g1 + p, i, kv); },
      [&](int i, uint32_t kv, uint32_t p) {
        if (p < take_eq) put(g1 + gt2 + p, i, kv);
      },
      t1, t2);
}

// chunk holding list position e, given the exclusive prefix pre[0..P] of the
// per-chunk counts (pre[P] = total)
__device__ __forceinline__ int chunk_of(const uint32_t* pre, int P, uint32_t e) {
  int lo = 0, hi = P - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pre[mid] <= e) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Finishing phase of a row whose Pr (<= kRowChunksMax) chunks were classified
// against the level-1 threshold bin b1 by several workgroups of this launch
// (run by the last of them).  Chunk c published, with st_agent:
//   counts[2c]     selected entries (digit > b1)  at gt + c * gts,
//   counts[2c + 1] candidate entries (digit == b1) at eq + c * eqs,
// each list in index order; an entry holds the key's index in the low 32
// bits and the fp32 score bits (gt) or the score key (eq) above.
// Copies the selected entries, chunk by chunk, to the first g1 slots; stages
// the candidates in LDS, runs levels 2-4 on them and fills the remaining
// k - g1 slots.  Only slots in [s0, s1) are handed out: put(slot, index,
// score) once per such slot, by one thread (the whole row: [0, k)).  Every
// thread of the workgroup calls it; `fs` is its LDS.  SAME_LAUNCH: the lists
// were published by other workgroups of this launch and are read with
// agent-scope loads; otherwise (a previous launch wrote them) plain cached
// loads see them.
template <int TPB>
struct FinishSmem {
  uint32_t ckey[kMSeg];
  uint32_t cidx[kMSeg];
  uint32_t h2[3][256];
  uint32_t pg[kRowChunksMax + 1], pe[kRowChunksMax + 1];
  uint32_t wave[TPB / 64];
  uint32_t res[2];
};

// The first memory round trip of finish_row, which the caller issues as
// early as it can: the counts of chunks c < Pl (wave 0, lane c) and the first
// batch of each thread's list entries, threads laid out over Pl >= Pr chunks
// (a group of tpc threads per chunk).  Entries past a list's end, and chunks
// past the row's Pr, are filler from inside the lists and are ignored.
struct FinishPrefetch {
  uint64_t g[kMUnroll], e[kMUnroll];
  uint32_t cg, ce;
};

__device__ __forceinline__ int finish_tpc(int TPB, int Pl) {
  int p2 = 1;
  while (p2 < Pl) p2 <<= 1;
  return p2 >= TPB ? 1 : TPB / p2;
}

template <int TPB, bool SAME_LAUNCH>
__device__ __forceinline__ void finish_prefetch(FinishPrefetch& pf, int Pl, const uint32_t* __restrict__ counts,
                                                const uint64_t* __restrict__ gt, long gts,
                                                const uint64_t* __restrict__ eq, long eqs) {
  auto ld = [](const auto* p) { return SAME_LAUNCH ? ld_agent(p) : *p; };
  const int tid = threadIdx.x, lane = tid & 63;
  const int tpc = finish_tpc(TPB, Pl);
  const int c_first = tid / tpc, sub = tid % tpc;
  if (c_first < Pl) {
#pragma unroll
    for (int u = 0; u < kMUnroll; ++u) {
      const long e = sub + u * tpc;
      pf.g[u] = ld(gt + c_first * gts + (e < gts ? e : gts - 1));
      pf.e[u] = ld(eq + c_first * eqs + (e < eqs ? e : eqs - 1));
    }
  }
  pf.cg = pf.ce = 0u;
  if (tid < 64 && lane < Pl) {
    pf.cg = ld(counts + 2 * lane);
    pf.ce = ld(counts + 2 * lane + 1);
  }
}

template <int TPB, bool SAME_LAUNCH, typename Put>
__device__ void finish_row(FinishSmem<TPB>& fs, const FinishPrefetch& pf, int Pl, int Pr, int k, uint32_t b1,
                           uint32_t g1, const uint32_t* __restrict__ counts, const uint64_t* __restrict__ gt,
                           long gts, const uint64_t* __restrict__ eq, long eqs, uint32_t s0, uint32_t s1,
                           Put&& put) {
  static_assert(kRowChunksMax <= 64, "one wave scans the chunk counts");
  uint32_t* s_ckey = fs.ckey;
  uint32_t* s_cidx = fs.cidx;
  uint32_t(*s_h2)[256] = fs.h2;
  uint32_t* s_pg = fs.pg;
  uint32_t* s_pe = fs.pe;
  uint32_t* s_wave = fs.wave;
  uint32_t* s_res = fs.res;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  auto ld = [](const auto* p) { return SAME_LAUNCH ? ld_agent(p) : *p; };

  // A group of tpc threads serves each chunk (laid out over Pl chunks, as in
  // finish_prefetch, whose batch is this thread's first).
  const int tpc = finish_tpc(TPB, Pl);
  const int c_first = tid / tpc, sub = tid % tpc;
  for (int b = tid; b < 3 * 256; b += TPB) (&s_h2[0][0])[b] = 0u;
  if (wave == 0) {  // exclusive prefix of the per-chunk counts (Pr <= 64)
    const uint32_t cg = lane < Pr ? pf.cg : 0u, ce = lane < Pr ? pf.ce : 0u;
    const uint32_t ig = wave_incl_scan(cg), ie = wave_incl_scan(ce);
    s_pg[lane] = ig - cg;
    s_pe[lane] = ie - ce;
    if (lane == 63) {
      s_pg[64] = ig;
      s_pe[64] = ie;
    }
  }
  __syncthreads();  // s_pg[Pr], s_pe[Pr]: the totals (counts past Pr are zero)
  const uint32_t n_cand = s_pe[Pr];
  const int nseg = (int)((n_cand + kMSeg - 1) / kMSeg);

  auto put_key = [&](uint32_t slot, uint32_t i, uint32_t key) {
    if (slot >= s0 && slot < s1) put(slot, i, key_score(key));
  };
  // Both lists in one pass (chunk order = index order): selected entries go
  // straight to their slots; candidates go to LDS when they all fit.
  for (int c = c_first; c < Pr; c += TPB / tpc) {
    const uint32_t g0 = s_pg[c], ng = s_pg[c + 1] - g0;
    const uint32_t e0c = s_pe[c], ne = s_pe[c + 1] - e0c;
    const uint32_t nmax = nseg == 1 ? max(ng, ne) : ng;
    const uint64_t* gsrc = gt + c * gts;
    const uint64_t* esrc = eq + c * eqs;
    for (uint32_t base = sub; base < nmax; base += tpc * kMUnroll) {
      uint64_t eg[kMUnroll], ee[kMUnroll];
      if (c == c_first && base == (uint32_t)sub) {  // the batch of finish_prefetch
#pragma unroll
        for (int u = 0; u < kMUnroll; ++u) {
          eg[u] = pf.g[u];
          ee[u] = pf.e[u];
        }
      } else {
#pragma unroll
        for (int u = 0; u < kMUnroll; ++u) {
          const uint32_t e = base + u * tpc;
          eg[u] = ld(gsrc + (e < ng ? e : 0u));
          ee[u] = ld(esrc + (e < ne ? e : 0u));
        }
        issue_fence();
      }
#pragma unroll
      for (int u = 0; u < kMUnroll; ++u) {
        const uint32_t e = base + u * tpc;
        if (e < ng && g0 + e >= s0 && g0 + e < s1)
          put(g0 + e, (uint32_t)eg[u], __uint_as_float((uint32_t)(eg[u] >> 32)));
        if (nseg == 1 && e < ne) {
          s_cidx[e0c + e] = (uint32_t)ee[u];
          s_ckey[e0c + e] = (uint32_t)(ee[u] >> 32);
        }
      }
    }
  }
  __syncthreads();

  // More candidates than LDS holds: stage them kMSeg at a time from the lists.
  auto stage = [&](int sg) {
    __syncthreads();
    const uint32_t base = (uint32_t)sg * kMSeg;
    const uint32_t cnt = min((uint32_t)kMSeg, n_cand - base);
    for (uint32_t el_ = tid; el_ < cnt; el_ += TPB) {
      const uint32_t e = base + el_;
      const int c = chunk_of(s_pe, Pr, e);
      const uint64_t ent = ld(eq + c * eqs + (e - s_pe[c]));
      s_cidx[el_] = (uint32_t)ent;
      s_ckey[el_] = (uint32_t)(ent >> 32);
    }
    __syncthreads();
  };
  auto seg_count = [&](int sg) { return (int)min((uint32_t)kMSeg, n_cand - (uint32_t)sg * kMSeg); };

  const int shifts[3] = {12, 4, 0};
  const int widths[3] = {8, 8, 4};
  uint32_t prefix = b1 << kL1Shift, pmask = 0xFFFFFFFFu << kL1Shift;
  uint32_t need = (uint32_t)k - g1;
  for (int lv = 0; lv < 3; ++lv) {
    const int sh = shifts[lv];
    const uint32_t dm = (1u << widths[lv]) - 1u;
    uint32_t* h2 = s_h2[lv];
    for (int sg = 0; sg < nseg; ++sg) {
      if (nseg > 1) stage(sg);
      const int cnt = seg_count(sg);
      for (int e = tid; e < cnt; e += TPB) {
        const uint32_t key = s_ckey[e];
        if ((key & pmask) == prefix) atomicAdd(&h2[(key >> sh) & dm], 1u);
      }
    }
    __syncthreads();
    if (wave == 0) {
      if (lane == 0) {
        s_res[0] = 0u;
        s_res[1] = 0u;
      }
      find_bin_wave(h2, 1 << widths[lv], need, s_res);
    }
    __syncthreads();
    prefix |= s_res[0] << sh;
    pmask |= dm << sh;
    need -= s_res[1];
  }
  const uint32_t T = prefix;      // the k-th largest key
  const uint32_t take_eq = need;  // ties at T to take, lowest indices first
  const uint32_t gt2 = (uint32_t)k - g1 - take_eq;

  uint32_t run1 = 0, run2 = 0;
  for (int sg = 0; sg < nseg; ++sg) {
    if (nseg > 1) stage(sg);
    const int cnt = seg_count(sg);
    const int cpt = (cnt + TPB - 1) / TPB;
    const int f = tid * cpt;
    const int lim = max(0, min(cpt, cnt - f));
    uint32_t c1 = 0, c2 = 0;
    for (int e = 0; e < lim; ++e) {
      const uint32_t key = s_ckey[f + e];
      c1 += key > T;
      c2 += key == T;
    }
    uint32_t tot3;
    const uint32_t ex3 = block_excl_scan<TPB>(c1 | (c2 << 16), s_wave, tot3);
    uint32_t p1 = run1 + (ex3 & 0xFFFFu), p2 = run2 + (ex3 >> 16);
    for (int e = 0; e < lim; ++e) {
      const uint32_t key = s_ckey[f + e];
      const uint32_t i = s_cidx[f + e];
      if (key > T) put_key(g1 + p1++, i, key);
      if (key == T) {
        if (p2 < take_eq) put_key(g1 + gt2 + p2, i, key);
        ++p2;
      }
    }
    run1 += tot3 & 0xFFFFu;
    run2 += tot3 >> 16;
  }
}

}  // namespace csa
