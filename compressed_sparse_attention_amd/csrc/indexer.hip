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
template <typename T, int KK, int NHT>
constexpr int pf_waves() {
  constexpr int v = NHT * KK * (sizeof(T) == 2 ? 4 : 8);
  return v <= 64 ? 16 : (v <= 96 ? 8 : 4);
}

template <typename T, int KK, int NHT>
__global__ __launch_bounds__((64 * pf_waves<T, KK, NHT>())) void indexer_prefill_kernel(int n, int nhI, int m,
                                                              const T* __restrict__ qI,
                                                              const float* __restrict__ wI,
                                                              const T* __restrict__ K,
                                                              const int64_t* __restrict__ kv_off,
                                                              long max_cand,
                                                              float* __restrict__ scores,
                                                              long ld_sc) {
  constexpr int kPfWaves = pf_waves<T, KK, NHT>();
  constexpr int kPfTokens = kPfWaves * kPfTokPerWave;
  // keys per LDS tile: 128 (measured faster than 64) while two tiles of key
  // rows stay well inside LDS, else 64
  constexpr int kPfTile = 32 * KK * sizeof(T) <= 512 ? 128 : 64;
  constexpr int CI = 32 * KK;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int PITCH = CI + VEC;  // padded LDS row (elements)
  constexpr int CHUNKS = CI / VEC;
  constexpr int TILE_VECS = kPfTile * CHUNKS;
  __shared__ __attribute__((aligned(16))) T Ks[2][kPfTile * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const int nblocks = (n + kPfTokens - 1) / kPfTokens;
  const long t0 = (long)(nblocks - 1 - (int)blockIdx.x) * kPfTokens;  // heaviest first

  // candidate count of the last token of this block bounds the key range
  const long t_last = min(t0 + kPfTokens - 1, (long)n - 1);
  long kend = t_last / m;
  kend = kend < max_cand ? kend : max_cand;
  if (kend <= 0) return;

  Frag<T> qa[kPfTokPerWave][NHT][KK];
  float wv[kPfTokPerWave][NHT][4];
  long tok[kPfTokPerWave], nc[kPfTokPerWave];
#pragma unroll
  for (int tt = 0; tt < kPfTokPerWave; ++tt) {
    const long t = t0 + wave * kPfTokPerWave + tt;
    tok[tt] = t;
    long c = t < n ? t / m : 0;
    nc[tt] = c < max_cand ? c : max_cand;
    const bool live = t < n;
#pragma unroll
    for (int mt = 0; mt < NHT; ++mt) {
      const int head = 16 * mt + c16;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk)
        qa[tt][mt][kk].load_clamped(qI + (t * nhI + head) * CI + g * 8 * KK + 8 * kk, live && head < nhI, qI);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int h = 16 * mt + 4 * g + rr;
        wv[tt][mt][rr] = (live && h < nhI) ? wI[t * nhI + h] : 0.f;
      }
    }
  }

  if (kv_off) K += kv_off[0] * CI;
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
        kb[kk].load(&Ks[cur][(grp * 16 + c16) * PITCH + g * 8 * KK + 8 * kk]);
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
        if (g == 0 && s < nc[tt]) scores[tok[tt] * ld_sc + s] = part;
      }
    }
    if (tile + 1 < ntiles) stash(cur ^ 1);
    __syncthreads();
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
                  (int)nq, nhI, m, (const T*)qI, wI, (const T*)K, kv_off, max_cand, scores, ld_sc);
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

}  // namespace

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

}  // namespace csa
