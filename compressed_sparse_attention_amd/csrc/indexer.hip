// Lightning indexer, eq 8 of "Compressed Sparse Attention" (section "Lightning
// Indexer for Sparse Selection"):
//
//   I[t, s] = sum_h w[t, h] * ReLU(q^I[t, h] . K^IComp[s]),  s < n_cand(t).
//
// The head dot products are one contraction [heads x cI] . [cI x keys]; it
// runs on MFMA with heads as the 16-row M side and keys as the 16-column N
// side.  The accumulator then holds, per lane, 4 heads of one key, so ReLU,
// the head weight and the head sum are an in-register fused epilogue plus
// two cross-lane adds.
//
// Contraction slots are mapped so that a lane reads ONE contiguous run of a
// key row: in step kk, lane group g's slot j is dimension g*8*KK + 8*kk + j
// (KK = cI/32 steps).  The query fragments use the same map.
//
// Two kernels:
//  * indexer_sweep -- any query/sequence layout (decode, ragged batches).
//    A workgroup of four waves takes one query and a chunk of 512 of its
//    candidates; the query's heads and weights are staged once in LDS, and
//    every wave streams its run of 16-key groups straight from HBM into MFMA
//    operands with a rolling window of groups in flight.
//  * indexer_prefill -- one sequence, query t at position t.  A workgroup
//    owns 16 consecutive tokens (one per wave, its q^I held in registers; at
//    most 128 VGPRs, so four waves share each SIMD; 8 tokens when q^I is too
//    large for that) and walks the causal key prefix once in key tiles
//    staged through LDS, so each key tile is fetched once per 16 tokens.
//    Heaviest token blocks first.
#include "common.hpp"
#include "internal.hpp"
#include "select.hpp"
#include "sweep.hpp"

namespace csa {
namespace {

template <typename T, int KK, int NHT>
__global__ __launch_bounds__(64 * kSweepWaves) void indexer_sweep_kernel(
    int nhI, int m, const T* __restrict__ qI, const float* __restrict__ wI,
    const T* __restrict__ K, const int32_t* __restrict__ q_seq, const int64_t* __restrict__ q_pos,
    const int64_t* __restrict__ kv_off, long max_cand, float* __restrict__ scores, long ld_sc,
    int chunks, uint32_t* __restrict__ hist, long hist_min) {
  __shared__ SweepSmem<T, KK, NHT> sm;
  const int r = blockIdx.x / chunks;
  const int chunk = blockIdx.x - r * chunks;
  float* row = scores + (long)r * ld_sc;
  sweep_chunk<T, KK, NHT>(sm, r, (long)chunk * kSweepKeysPerWG, nhI, m, qI, wI, K, q_seq, q_pos, kv_off, max_cand,
                          hist ? hist + (long)r * (1 << kTopkL1Bits) : nullptr, hist_min,
                          [&](long s, float v) { row[s] = v; });
}

// ---------------------------------------------------------------------------
// prefill: tokens t0 .. t0+W-1 per workgroup (W waves x 1 token)
// ---------------------------------------------------------------------------
constexpr int kPfTokPerWave = 1;

// Waves (= tokens) per workgroup, from the VGPRs a token's q^I fragments take:
// 16 waves (128-VGPR budget each) up to 64, 8 waves (256) up to 96, else 4.
template <typename T, int KK, int NHT, bool STREAM = false>
constexpr int pf_waves() {
  constexpr int v = NHT * KK * (sizeof(T) == 2 ? 4 : 8);
  constexpr int w = v <= 64 ? 16 : (v <= 96 ? 8 : 4);
  // streaming keeps more state per wave: at most 8 waves (256 VGPRs each)
  return STREAM && w > 8 ? 8 : w;
}

// keys per LDS tile of the prefill kernel: 128 (measured faster than 64)
// while two tiles of key rows stay well inside LDS, else 64
template <typename T, int KK>
constexpr int pf_tile() {
  return 32 * KK * sizeof(T) <= 512 ? 128 : 64;
}

// Streaming selection (STREAM): each wave keeps, for its token, a histogram
// of 2^kStreamBits bins of the top bits of the score keys (score_key), two
// 16-bit counts per LDS word, and a running threshold bin b: the highest bin
// such that at least k of the scores seen so far lie in bins >= b.  b only
// rises, and every score of the final top-k lies in a bin >= the final b >=
// every earlier b, so a score below the current b can never be selected and
// is dropped; the others are appended, in index order, to the token's list as
// (index, score) entries.  The histogram counts only appended scores, which
// are all the scores of bins >= b: exact where it is read.
constexpr int kStreamBits = kStreamBitsTopk;
constexpr int kStreamBins = 1 << kStreamBits;
constexpr int kStreamWords = kStreamBins / 2;

// LDS of the prefill kernel: two key tiles, plus one histogram per wave when
// streaming.
template <typename T, int KK, int NHT, bool STREAM>
constexpr size_t pf_lds_bytes() {
  return 2 * (size_t)pf_tile<T, KK>() * (32 * KK + 32 / sizeof(T)) * sizeof(T) +
         (STREAM ? (size_t)pf_waves<T, KK, NHT, STREAM>() * kStreamWords * 4 : 0);
}

template <typename T, int KK, int NHT, bool STREAM>
constexpr bool pf_fits() {
  return pf_lds_bytes<T, KK, NHT, STREAM>() <= 160 * 1024;
}

template <typename T, int KK, int NHT, bool STREAM = false>
__global__ __launch_bounds__((64 * pf_waves<T, KK, NHT, STREAM>())) void indexer_prefill_kernel(int n, int nhI, int m,
                                                              const T* __restrict__ qI,
                                                              const float* __restrict__ wI,
                                                              const T* __restrict__ K,
                                                              const int64_t* __restrict__ kv_off,
                                                              long max_cand,
                                                              float* __restrict__ scores,
                                                              long ld_sc, int nseq,
                                                              const int64_t* __restrict__ cu,
                                                              const int32_t* __restrict__ blk,
                                                              uint64_t* __restrict__ lists, uint32_t* __restrict__ meta,
                                                              int k) {
  constexpr int kPfWaves = pf_waves<T, KK, NHT, STREAM>();
  constexpr int kPfTokens = kPfWaves * kPfTokPerWave;
  constexpr int kPfTile = pf_tile<T, KK>();
  constexpr int CI = 32 * KK;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int PITCH = CI + 2 * VEC;  // padded LDS row: rows 32 bytes apart, conflict-free fragment reads
  constexpr int CHUNKS = CI / VEC;
  constexpr int TILE_VECS = kPfTile * CHUNKS;
  static_assert(!STREAM || (pf_fits<T, KK, NHT, STREAM>() && kPfTokPerWave == 1), "streaming layout");
  __shared__ __attribute__((aligned(16))) T Ks[2][kPfTile * PITCH];
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[STREAM ? kPfWaves * kStreamWords : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  // Token block of this workgroup: positions p0 .. p0+kPfTokens-1 of one
  // sequence of length len, whose rows start at row0 and keys at kbase.
  // One sequence: the blocks in reverse order (heaviest first).  Several
  // (cu set): blk[b] .. blk[b+1]-1 are sequence b's blocks; the grid may hold
  // more workgroups than blocks.
  long p0, len, row0 = 0, kbase = kv_off ? kv_off[0] : 0;
  if (cu == nullptr) {
    const int nblocks = (n + kPfTokens - 1) / kPfTokens;
    p0 = (long)(nblocks - 1 - (int)blockIdx.x) * kPfTokens;
    len = n;
  } else {
    const int total = blk[nseq];
    if ((int)blockIdx.x >= total) return;
    const int j = total - 1 - (int)blockIdx.x;
    int lo = 0, hi = nseq - 1;  // the sequence b with blk[b] <= j < blk[b+1]
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (blk[mid] <= j) lo = mid; else hi = mid - 1;
    }
    p0 = (long)(j - blk[lo]) * kPfTokens;
    row0 = cu[lo];
    len = cu[lo + 1] - row0;
    kbase = kv_off[lo];
  }

  // candidate count of the last token of this block bounds the key range
  const long p_last = min(p0 + kPfTokens - 1, len - 1);
  long kend = p_last / m;
  kend = kend < max_cand ? kend : max_cand;
  if (kend <= 0) return;

  Frag<T> qa[kPfTokPerWave][NHT][KK];
  float wv[kPfTokPerWave][NHT][4];
  long tok[kPfTokPerWave], nc[kPfTokPerWave];
#pragma unroll
  for (int tt = 0; tt < kPfTokPerWave; ++tt) {
    const long pos = p0 + wave * kPfTokPerWave + tt;
    const bool live = pos < len;
    const long t = row0 + (live ? pos : 0);  // the token's row in qI / wI / scores
    tok[tt] = t;
    long c = live ? pos / m : 0;
    nc[tt] = c < max_cand ? c : max_cand;
#pragma unroll
    for (int mt = 0; mt < NHT; ++mt) {
      const int head = 16 * mt + c16;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qa[tt][mt][kk].load_clamped(qI + (t * nhI + head) * CI + 32 * kk + 8 * g, live && head < nhI, qI);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int h = 16 * mt + 4 * g + rr;
        wv[tt][mt][rr] = (live && h < nhI) ? wI[t * nhI + h] : 0.f;
      }
    }
  }

  // streaming state of this wave's token (wave-uniform)
  uint32_t* whist = s_hist + (STREAM ? wave * kStreamWords : 0);
  // (a token with at most k candidates never raises its threshold: all its scores are listed)
  const bool stream_tok = STREAM && nc[0] > 0;
  uint32_t bstar = 0, above = 0, nlist = 0;
  uint64_t* lrow = lists + (STREAM ? tok[0] * ld_sc : 0);
  if constexpr (STREAM) {
    for (int i = lane; i < kStreamWords / 4; i += 64)
      reinterpret_cast<u32x4*>(whist)[i] = u32x4{0u, 0u, 0u, 0u};
  }

  K += kbase * CI;
  const int ntiles = (int)((kend + kPfTile - 1) / kPfTile);
  constexpr int LOADS = (TILE_VECS + 64 * kPfWaves - 1) / (64 * kPfWaves);
  u32x4 stage[LOADS];
  auto fetch = [&](int tile) {
#pragma unroll
    for (int p = 0; p < LOADS; ++p) {
      const int v = tid + p * 64 * kPfWaves;
      const long key = (long)tile * kPfTile + v / CHUNKS;
      stage[p] = load16_clamped(K + key * CI + (v % CHUNKS) * VEC, v < TILE_VECS && key < kend, K);
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int p = 0; p < LOADS; ++p) {
      const int v = tid + p * 64 * kPfWaves;
      if (v < TILE_VECS)
        *reinterpret_cast<u32x4*>(&Ks[buf][(v / CHUNKS) * PITCH + (v % CHUNKS) * VEC]) = stage[p];
    }
  };

  fetch(0);
  stash(0);
  __syncthreads();
  for (int tile = 0; tile < ntiles; ++tile) {
    const int cur = tile & 1;
    if (tile + 1 < ntiles) fetch(tile + 1);
#pragma unroll
    for (int grp = 0; grp < kPfTile / 16; ++grp) {
      const long s = (long)tile * kPfTile + grp * 16 + c16;
      Frag<T> kb[KK];
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        kb[kk].load(&Ks[cur][(grp * 16 + c16) * PITCH + 32 * kk + 8 * g]);
#pragma unroll
      for (int tt = 0; tt < kPfTokPerWave; ++tt) {
        float part = 0.f;
#pragma unroll
        for (int mt = 0; mt < NHT; ++mt) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kk = 0; kk < KK; ++kk) mma(acc, qa[tt][mt][kk], kb[kk]);
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) part = fmaf(wv[tt][mt][rr], relu(acc[rr]), part);
        }
        part = wave_sum_xor_16_32(part);
        if constexpr (!STREAM) {
          if (g == 0 && s < nc[tt]) scores[tok[tt] * ld_sc + s] = part;
        } else if (stream_tok) {
          const uint32_t bin = score_key(part) >> (32 - kStreamBits);
          const bool pass = g == 0 && s < nc[tt] && bin >= bstar;
          const uint64_t bal = __ballot(pass);  // lanes 0..15 only: key order
          if (pass) {
            const uint32_t at = nlist + __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u);
            if (at < (uint32_t)ld_sc) lrow[at] = (uint64_t)s | ((uint64_t)__float_as_uint(part) << 32);
            atomicAdd(&whist[bin >> 1], 1u << ((bin & 1u) * 16));
          }
          const uint32_t np = __builtin_amdgcn_readfirstlane((uint32_t)__popcll(bal));
          nlist += np;
          above += np;
        }
      }
    }
    if constexpr (STREAM) {
      // Raise the threshold bin to the highest bin with at least k listed
      // scores at or above it, once at least k are listed.  One wave-parallel
      // search over the histogram: lane l sums bins 32l .. 32l+31, a suffix
      // scan from the top finds the lane where the count reaches k, and that
      // lane walks its 32 bins.  (This wave's LDS operations complete in
      // order: the counts include the additions above.)  Bins below the
      // current threshold hold partial counts, but the search stops at or
      // above it: the count at and above it is already >= k.
      if (stream_tok && above >= (uint32_t)k) {
        const u32x4* hw = reinterpret_cast<const u32x4*>(whist) + 4 * lane;
        uint32_t lsum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const u32x4 v = hw[q];
          lsum += ((v.x & 0xFFFFu) + (v.x >> 16)) + ((v.y & 0xFFFFu) + (v.y >> 16)) +
                  ((v.z & 0xFFFFu) + (v.z >> 16)) + ((v.w & 0xFFFFu) + (v.w >> 16));
        }
        // counts at or above this lane's bins: total minus the inclusive prefix below
        const uint32_t incl = wave_incl_scan(lsum);
        const uint32_t total = wave_last(incl);
        const uint32_t from_me = total - incl + lsum;  // bins >= 32 lane
        const uint32_t above_me = from_me - lsum;      // bins >= 32 (lane + 1)
        const uint64_t hit = __ballot(above_me < (uint32_t)k && from_me >= (uint32_t)k);
        const int hl = __builtin_ctzll(hit | (1ull << 63));  // exactly one lane holds the crossing
        uint32_t nb = 0, nab = 0;
        if (lane == hl) {  // walk this lane's 32 bins from the top (its words read again)
          uint32_t cum = above_me;
          bool found = false;
          for (int wdi = 15; wdi >= 0 && !found; --wdi) {
            const uint32_t wd = whist[16 * lane + wdi];
            for (int half = 1; half >= 0 && !found; --half) {
              const uint32_t c = half ? (wd >> 16) : (wd & 0xFFFFu);
              if (cum + c >= (uint32_t)k) {
                nb = (uint32_t)(32 * lane + 2 * wdi + half);
                nab = cum + c;
                found = true;
              }
              cum += c;
            }
          }
        }
        bstar = __builtin_amdgcn_readlane(nb, hl);
        above = __builtin_amdgcn_readlane(nab, hl);
      }
    }
    if (tile + 1 < ntiles) stash(cur ^ 1);
    __syncthreads();
  }
  if constexpr (STREAM) {
    // per token: threshold bin, count strictly above it, list length
    if (lane == 0 && p0 + wave < len) {
      uint32_t g1 = 0;
      if (stream_tok) g1 = above - ((whist[bstar >> 1] >> ((bstar & 1u) * 16)) & 0xFFFFu);
      *reinterpret_cast<u32x4*>(meta + 4 * tok[0]) = u32x4{bstar, g1, nlist, stream_tok ? 1u : 0u};
    }
  }
}

// ---------------------------------------------------------------------------
// Packed sequences: per-token sequence and position, and the tiled kernel's
// block table blk[b] = sum over b' < b of ceil(len_b' / wtok) (blk[nseq] =
// total), from cu (the sequences' first rows, cu[nseq] = total tokens).
// Workgroup 0 also builds the table.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void varlen_meta_kernel(int nseq, const int64_t* __restrict__ cu, long ntok, int wtok,
                                                          int32_t* __restrict__ blk, int64_t* __restrict__ q_pos,
                                                          int32_t* __restrict__ q_seq) {
  const long t = (long)blockIdx.x * 256 + threadIdx.x;
  if (t < ntok) {
    int lo = 0, hi = nseq - 1;  // the last sequence starting at or before t
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cu[mid] <= t) lo = mid; else hi = mid - 1;
    }
    q_pos[t] = t - cu[lo];
    q_seq[t] = lo;
  }
  if (blockIdx.x == 0) {
    __shared__ uint32_t s_wave[4];
    uint32_t run = 0;
    for (int b0 = 0; b0 < nseq; b0 += 256) {
      const int b = b0 + (int)threadIdx.x;
      const uint32_t v = b < nseq ? (uint32_t)((cu[b + 1] - cu[b] + wtok - 1) / wtok) : 0u;
      uint32_t tot;
      const uint32_t ex = block_excl_scan<256>(v, s_wave, tot);
      if (b < nseq) blk[b] = (int32_t)(run + ex);
      run += tot;
    }
    if (threadIdx.x == 0) blk[nseq] = (int32_t)run;
  }
}

template <typename T, int KK, int NHT>
hipError_t run_varlen(long nseq, long ntok, int nhI, int m, const void* qI, const float* wI, const void* K,
                      const int64_t* cu, const int32_t* blk, const int64_t* kv_off, long max_cand, float* scores,
                      long ld_sc, hipStream_t s) {
  constexpr int waves = pf_waves<T, KK, NHT>();
  // every sequence adds at most one partly filled block; surplus workgroups exit
  const long grid = (ntok + waves - 1) / waves + nseq;
  return launch("indexer_prefill", indexer_prefill_kernel<T, KK, NHT>, dim3((unsigned)grid), dim3(64 * waves), 0, s,
                (int)ntok, nhI, m, (const T*)qI, wI, (const T*)K, kv_off, max_cand, scores, ld_sc, (int)nseq, cu,
                blk, (uint64_t*)nullptr, (uint32_t*)nullptr, 0);
}

template <typename T>
int waves_of(int nhI, int cI) {
  const int nht = (nhI + 15) / 16;
  switch (cI / 32) {
    case 1: return nht == 1 ? pf_waves<T, 1, 1>() : nht == 2 ? pf_waves<T, 1, 2>() : nht == 3 ? pf_waves<T, 1, 3>() : pf_waves<T, 1, 4>();
    case 2: return nht == 1 ? pf_waves<T, 2, 1>() : nht == 2 ? pf_waves<T, 2, 2>() : nht == 3 ? pf_waves<T, 2, 3>() : pf_waves<T, 2, 4>();
    case 4: return nht == 1 ? pf_waves<T, 4, 1>() : nht == 2 ? pf_waves<T, 4, 2>() : nht == 3 ? pf_waves<T, 4, 3>() : pf_waves<T, 4, 4>();
    default: return nht == 1 ? pf_waves<T, 8, 1>() : nht == 2 ? pf_waves<T, 8, 2>() : nht == 3 ? pf_waves<T, 8, 3>() : pf_waves<T, 8, 4>();
  }
}

template <typename T, int KK>
hipError_t varlen_nht(long nseq, long ntok, int nhI, int m, const void* qI, const float* wI, const void* K,
                      const int64_t* cu, const int32_t* blk, const int64_t* kv_off, long max_cand, float* scores,
                      long ld_sc, hipStream_t s) {
  switch ((nhI + 15) / 16) {
    case 1: return run_varlen<T, KK, 1>(nseq, ntok, nhI, m, qI, wI, K, cu, blk, kv_off, max_cand, scores, ld_sc, s);
    case 2: return run_varlen<T, KK, 2>(nseq, ntok, nhI, m, qI, wI, K, cu, blk, kv_off, max_cand, scores, ld_sc, s);
    case 3: return run_varlen<T, KK, 3>(nseq, ntok, nhI, m, qI, wI, K, cu, blk, kv_off, max_cand, scores, ld_sc, s);
    default: return run_varlen<T, KK, 4>(nseq, ntok, nhI, m, qI, wI, K, cu, blk, kv_off, max_cand, scores, ld_sc, s);
  }
}

template <typename T>
hipError_t varlen_kk(long nseq, long ntok, int nhI, int cI, int m, const void* qI, const float* wI, const void* K,
                     const int64_t* cu, const int32_t* blk, const int64_t* kv_off, long max_cand, float* scores,
                     long ld_sc, hipStream_t s) {
  switch (cI / 32) {
    case 1: return varlen_nht<T, 1>(nseq, ntok, nhI, m, qI, wI, K, cu, blk, kv_off, max_cand, scores, ld_sc, s);
    case 2: return varlen_nht<T, 2>(nseq, ntok, nhI, m, qI, wI, K, cu, blk, kv_off, max_cand, scores, ld_sc, s);
    case 4: return varlen_nht<T, 4>(nseq, ntok, nhI, m, qI, wI, K, cu, blk, kv_off, max_cand, scores, ld_sc, s);
    case 8: return varlen_nht<T, 8>(nseq, ntok, nhI, m, qI, wI, K, cu, blk, kv_off, max_cand, scores, ld_sc, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int KK, int NHT>
hipError_t run(long nq, int nhI, int m, const void* qI, const float* wI, const void* K,
               const int32_t* q_seq, const int64_t* q_pos, const int64_t* kv_off, long max_cand,
               float* scores, long ld_sc, uint32_t* hist, long hist_min, hipStream_t s) {
  if (q_seq == nullptr && q_pos == nullptr) {
    constexpr int waves = pf_waves<T, KK, NHT>();
    const int nblocks = (int)((nq + waves * kPfTokPerWave - 1) / (waves * kPfTokPerWave));
    return launch("indexer_prefill", indexer_prefill_kernel<T, KK, NHT>, dim3(nblocks), dim3(64 * waves), 0, s,
                  (int)nq, nhI, m, (const T*)qI, wI, (const T*)K, kv_off, max_cand, scores, ld_sc, 0,
                  (const int64_t*)nullptr, (const int32_t*)nullptr, (uint64_t*)nullptr, (uint32_t*)nullptr, 0);
  } else {
    const unsigned chunks = (unsigned)((max_cand + kSweepKeysPerWG - 1) / kSweepKeysPerWG);
    return launch("indexer_sweep", indexer_sweep_kernel<T, KK, NHT>, dim3(chunks * (unsigned)nq),
                  dim3(64 * kSweepWaves), 0,
                  s, nhI, m, (const T*)qI, wI, (const T*)K, q_seq, q_pos, kv_off, max_cand, scores, ld_sc,
                  (int)chunks, hist, hist_min);
  }
}

template <typename T, int KK>
hipError_t pick_nht(long nq, int nhI, int m, const void* qI, const float* wI, const void* K,
                    const int32_t* q_seq, const int64_t* q_pos, const int64_t* kv_off,
                    long max_cand, float* scores, long ld_sc, uint32_t* hist, long hist_min, hipStream_t s) {
  switch ((nhI + 15) / 16) {
    case 1: return run<T, KK, 1>(nq, nhI, m, qI, wI, K, q_seq, q_pos, kv_off, max_cand, scores, ld_sc, hist, hist_min, s);
    case 2: return run<T, KK, 2>(nq, nhI, m, qI, wI, K, q_seq, q_pos, kv_off, max_cand, scores, ld_sc, hist, hist_min, s);
    case 3: return run<T, KK, 3>(nq, nhI, m, qI, wI, K, q_seq, q_pos, kv_off, max_cand, scores, ld_sc, hist, hist_min, s);
    default: return run<T, KK, 4>(nq, nhI, m, qI, wI, K, q_seq, q_pos, kv_off, max_cand, scores, ld_sc, hist, hist_min, s);
  }
}

template <typename T>
hipError_t pick_kk(long nq, int nhI, int cI, int m, const void* qI, const float* wI, const void* K,
                   const int32_t* q_seq, const int64_t* q_pos, const int64_t* kv_off,
                   long max_cand, float* scores, long ld_sc, uint32_t* hist, long hist_min, hipStream_t s) {
  switch (cI / 32) {
    case 1: return pick_nht<T, 1>(nq, nhI, m, qI, wI, K, q_seq, q_pos, kv_off, max_cand, scores, ld_sc, hist, hist_min, s);
    case 2: return pick_nht<T, 2>(nq, nhI, m, qI, wI, K, q_seq, q_pos, kv_off, max_cand, scores, ld_sc, hist, hist_min, s);
    case 4: return pick_nht<T, 4>(nq, nhI, m, qI, wI, K, q_seq, q_pos, kv_off, max_cand, scores, ld_sc, hist, hist_min, s);
    case 8: return pick_nht<T, 8>(nq, nhI, m, qI, wI, K, q_seq, q_pos, kv_off, max_cand, scores, ld_sc, hist, hist_min, s);
    default: return hipErrorInvalidValue;
  }
}

template <typename T, int KK, int NHT>
hipError_t run_stream(long n, int nhI, int m, const void* qI, const float* wI, const void* K, const int64_t* kv_off,
                      long max_cand, uint64_t* lists, long ld_list, uint32_t* meta, int k, hipStream_t s) {
  if constexpr (!pf_fits<T, KK, NHT, true>()) {
    return hipErrorInvalidValue;  // the host checks stream_supported first
  } else {
    constexpr int waves = pf_waves<T, KK, NHT, true>();
    const int nblocks = (int)((n + waves - 1) / waves);
    return launch("indexer_prefill", indexer_prefill_kernel<T, KK, NHT, true>, dim3(nblocks), dim3(64 * waves), 0, s,
                  (int)n, nhI, m, (const T*)qI, wI, (const T*)K, kv_off, max_cand, (float*)nullptr, ld_list, 0,
                  (const int64_t*)nullptr, (const int32_t*)nullptr, lists, meta, k);
  }
}

template <typename T, int KK>
hipError_t stream_nht(long n, int nhI, int m, const void* qI, const float* wI, const void* K, const int64_t* kv_off,
                      long max_cand, uint64_t* lists, long ld_list, uint32_t* meta, int k, hipStream_t s) {
  switch ((nhI + 15) / 16) {
    case 1: return run_stream<T, KK, 1>(n, nhI, m, qI, wI, K, kv_off, max_cand, lists, ld_list, meta, k, s);
    case 2: return run_stream<T, KK, 2>(n, nhI, m, qI, wI, K, kv_off, max_cand, lists, ld_list, meta, k, s);
    case 3: return run_stream<T, KK, 3>(n, nhI, m, qI, wI, K, kv_off, max_cand, lists, ld_list, meta, k, s);
    default: return run_stream<T, KK, 4>(n, nhI, m, qI, wI, K, kv_off, max_cand, lists, ld_list, meta, k, s);
  }
}

template <typename T, int KK>
bool fits_nht(int nhI) {
  switch ((nhI + 15) / 16) {
    case 1: return pf_fits<T, KK, 1, true>();
    case 2: return pf_fits<T, KK, 2, true>();
    case 3: return pf_fits<T, KK, 3, true>();
    default: return pf_fits<T, KK, 4, true>();
  }
}

template <typename T>
bool fits_kk(int nhI, int cI) {
  switch (cI / 32) {
    case 1: return fits_nht<T, 1>(nhI);
    case 2: return fits_nht<T, 2>(nhI);
    case 4: return fits_nht<T, 4>(nhI);
    case 8: return fits_nht<T, 8>(nhI);
    default: return false;
  }
}

}  // namespace

bool indexer_stream_supported(csa_dtype dt, int nhI, int cI, long max_cand) {
  // the streaming histogram counts up to 65535 scores per bin
  if (max_cand > 65535) return false;
  return dt == CSA_F32 ? fits_kk<float>(nhI, cI) : fits_kk<bf16_t>(nhI, cI);
}

hipError_t launch_indexer_stream(csa_dtype dt, long n, int nhI, int cI, int m, const void* qI, const float* wI,
                                 const void* K, const int64_t* kv_offset, long max_cand, uint64_t* lists,
                                 long ld_list, uint32_t* meta, int k, hipStream_t s) {
  if (n == 0 || max_cand == 0) return hipSuccess;
  const bool f32 = dt == CSA_F32;
  switch (cI / 32) {
    case 1: return f32 ? stream_nht<float, 1>(n, nhI, m, qI, wI, K, kv_offset, max_cand, lists, ld_list, meta, k, s)
                       : stream_nht<bf16_t, 1>(n, nhI, m, qI, wI, K, kv_offset, max_cand, lists, ld_list, meta, k, s);
    case 2: return f32 ? stream_nht<float, 2>(n, nhI, m, qI, wI, K, kv_offset, max_cand, lists, ld_list, meta, k, s)
                       : stream_nht<bf16_t, 2>(n, nhI, m, qI, wI, K, kv_offset, max_cand, lists, ld_list, meta, k, s);
    case 4: return f32 ? stream_nht<float, 4>(n, nhI, m, qI, wI, K, kv_offset, max_cand, lists, ld_list, meta, k, s)
                       : stream_nht<bf16_t, 4>(n, nhI, m, qI, wI, K, kv_offset, max_cand, lists, ld_list, meta, k, s);
    case 8: return f32 ? stream_nht<float, 8>(n, nhI, m, qI, wI, K, kv_offset, max_cand, lists, ld_list, meta, k, s)
                       : stream_nht<bf16_t, 8>(n, nhI, m, qI, wI, K, kv_offset, max_cand, lists, ld_list, meta, k, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_indexer(csa_dtype dt, long n_queries, int nhI, int cI, int m, const void* qI,
                          const float* wI, const void* K, const int32_t* q_seq,
                          const int64_t* q_pos, const int64_t* kv_offset, long max_cand,
                          float* scores, long ld_sc, uint32_t* hist, long hist_min, hipStream_t s) {
  if (n_queries == 0 || max_cand == 0) return hipSuccess;
  if (dt == CSA_F32)
    return pick_kk<float>(n_queries, nhI, cI, m, qI, wI, K, q_seq, q_pos, kv_offset, max_cand,
                          scores, ld_sc, hist, hist_min, s);
  return pick_kk<bf16_t>(n_queries, nhI, cI, m, qI, wI, K, q_seq, q_pos, kv_offset, max_cand,
                         scores, ld_sc, hist, hist_min, s);
}

hipError_t launch_indexer_varlen(csa_dtype dt, long nseq, long ntok, int nhI, int cI, int m, const void* qI,
                                 const float* wI, const void* K, const int64_t* cu, const int64_t* kv_offset,
                                 long max_cand, float* scores, long ld_sc, int32_t* blk, int64_t* q_pos,
                                 int32_t* q_seq, hipStream_t s) {
  if (nseq == 0 || ntok == 0) return hipSuccess;
  const int wtok = dt == CSA_F32 ? waves_of<float>(nhI, cI) : waves_of<bf16_t>(nhI, cI);
  hipError_t e = launch("varlen_meta", varlen_meta_kernel, dim3((unsigned)((ntok + 255) / 256)), dim3(256), 0, s,
                        (int)nseq, cu, ntok, wtok, blk, q_pos, q_seq);
  if (e != hipSuccess || max_cand == 0) return e;
  if (dt == CSA_F32)
    return varlen_kk<float>(nseq, ntok, nhI, cI, m, qI, wI, K, cu, blk, kv_offset, max_cand, scores, ld_sc, s);
  return varlen_kk<bf16_t>(nseq, ntok, nhI, cI, m, qI, wI, K, cu, blk, kv_offset, max_cand, scores, ld_sc, s);
}

}  // namespace csa
