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

namespace csa {
namespace {

constexpr int kSweepWaves = 4;
constexpr int kSweepKeysPerWG = 512;  // 128 keys (eight 16-key groups) per wave

template <typename T, int KK, int NHT>
__global__ __launch_bounds__(64 * kSweepWaves) void indexer_sweep_kernel(
    int nhI, int m, const T* __restrict__ qI, const float* __restrict__ wI,
    const T* __restrict__ K, const int32_t* __restrict__ q_seq, const int64_t* __restrict__ q_pos,
    const int64_t* __restrict__ kv_off, long max_cand, float* __restrict__ scores, long ld_sc,
    int chunks, uint32_t* __restrict__ hist) {
  constexpr int CI = 32 * KK;
  constexpr int NB = 1 << kTopkL1Bits;
  constexpr int NTH = 64 * kSweepWaves;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int QPITCH = CI + VEC;  // padded LDS row: the 16 lanes reading one k-slice hit distinct banks
  constexpr int QCH = CI / VEC;     // 16-byte pieces per query row
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[NB];
  __shared__ uint32_t s_touched[kSweepKeysPerWG];  // bins this chunk hit, in first-touch order
  __shared__ uint32_t s_ntouched;
  __shared__ __attribute__((aligned(16))) T s_q[16 * NHT * QPITCH];
  __shared__ float s_w[16 * NHT];

  const int r = blockIdx.x / chunks;
  const int chunk = blockIdx.x - r * chunks;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;

  // The query's heads and head weights are fetched first, by every wave,
  // before any wave issues key loads (a barrier orders the issue): a CU
  // serves its waves' requests roughly in issue order, so a query load queued
  // behind other waves' keys would hold the LDS staging (and with it every
  // MFMA) until most of the chunk had arrived.  Staging the query in LDS
  // (zero rows for padded heads; every wave then reads its fragments from
  // there) then waits only for these loads.
  constexpr int QPIECES = 16 * NHT * QCH;
  constexpr int QV = (QPIECES + NTH - 1) / NTH;
  u32x4 qv[QV];
#pragma unroll
  for (int i = 0; i < QV; ++i) {
    const int v = tid + i * NTH;
    const int head = v / QCH, pc = (v - head * QCH) * VEC;
    qv[i] = load16_clamped(qI + ((long)r * nhI + head) * CI + pc, v < QPIECES && head < nhI, qI);
  }
  const float wraw = wI[(long)r * nhI + (tid < nhI ? tid : 0)];
  const long pos = q_pos ? q_pos[r] : (long)r;
  const int seq = q_seq ? q_seq[r] : 0;
  long ncand = pos > 0 ? pos / m : 0;
  ncand = ncand < max_cand ? ncand : max_cand;
  const long chunk0 = (long)chunk * kSweepKeysPerWG;
  if (chunk0 >= ncand) return;
  const long off = kv_off ? kv_off[seq] : 0;
  const long chunk_end = min(chunk0 + (long)kSweepKeysPerWG, ncand);
  __syncthreads();  // every wave's query loads are issued before any key load

  // Each wave owns GPW consecutive 16-key groups of the chunk and keeps D of
  // them in flight: group gi is computed once its loads have landed and its
  // register slot is refilled with group gi + D right away.  A wave whose
  // loads all went out at once would sit in the issue queue (the memory
  // system back-pressures it) until most of its data had arrived, and only
  // then start its MFMAs; the rolling window lets a wave compute while its
  // later groups are still streaming in.  Lanes past the end of the chunk
  // read the chunk's first key instead; their scores are never stored.
  constexpr int GPW = kSweepKeysPerWG / (16 * kSweepWaves);
  constexpr int VPF = sizeof(T) == 2 ? 4 : 8;  // VGPRs per fragment
  constexpr int DB = 32 / (KK * VPF);  // 32 VGPRs of keys in flight per wave
  constexpr int D = DB < 1 ? 1 : (DB > GPW ? GPW : DB);
  const T* Kb = K + off * CI + g * 8 * KK;
  const long wbase = chunk0 + (long)wave * GPW * 16;
  Frag<T> kb[D][KK];
  auto issue = [&](int gi, int slot) {
    const long s = wbase + gi * 16 + c16;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) kb[slot][kk].load_clamped(Kb + s * CI + 8 * kk, s < chunk_end, Kb + 8 * kk);
  };
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d, d);  // in flight while the query is staged
  issue_fence();

#pragma unroll
  for (int i = 0; i < QV; ++i) {
    const int v = tid + i * NTH;
    const int head = v / QCH, pc = (v - head * QCH) * VEC;
    if (v < QPIECES)
      *reinterpret_cast<u32x4*>(&s_q[head * QPITCH + pc]) = head < nhI ? qv[i] : u32x4{0u, 0u, 0u, 0u};
  }
  if (tid < 16 * NHT) s_w[tid] = tid < nhI ? wraw : 0.f;
  if (hist) {
    for (int b = tid; b < NB / 4; b += NTH) reinterpret_cast<u32x4*>(s_hist)[b] = u32x4{0u, 0u, 0u, 0u};
    if (tid == 0) s_ntouched = 0u;
  }
  __syncthreads();
  Frag<T> qa[NHT][KK];
  float wv[NHT][4];
#pragma unroll
  for (int mt = 0; mt < NHT; ++mt) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) qa[mt][kk].load(&s_q[(16 * mt + c16) * QPITCH + g * 8 * KK + 8 * kk]);
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) wv[mt][rr] = s_w[16 * mt + 4 * g + rr];
  }

#pragma unroll
  for (int gi = 0; gi < GPW; ++gi) {
    const int slot = gi % D;
    float part = 0.f;
#pragma unroll
    for (int mt = 0; mt < NHT; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) mma(acc, qa[mt][kk], kb[slot][kk]);
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) part = fmaf(wv[mt][rr], relu(acc[rr]), part);
    }
    if (gi + D < GPW) {
      issue(gi + D, slot);
      issue_fence();
    }
    part = wave_sum_xor_16_32(part);
    const long s = wbase + gi * 16 + c16;
    if (g == 0 && s < chunk_end) {
      scores[(long)r * ld_sc + s] = part;
      if (hist) {
        const uint32_t b = score_key(part) >> (32 - kTopkL1Bits);
        if (atomicAdd(&s_hist[b], 1u) == 0u) s_touched[atomicAdd(&s_ntouched, 1u)] = b;
      }
    }
  }
  if (hist) {  // add the touched bins (at most one per key) into the row's histogram
    __syncthreads();
    uint32_t* hrow = hist + (long)r * NB;
    const uint32_t nt = s_ntouched;
    for (uint32_t e = tid; e < nt; e += NTH) {
      const uint32_t b = s_touched[e];
      atomicAdd(&hrow[b], s_hist[b]);
    }
  }
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
               float* scores, long ld_sc, uint32_t* hist, hipStream_t s) {
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
                  (int)chunks, hist);
  }
}

template <typename T, int KK>
hipError_t pick_nht(long nq, int nhI, int m, const void* qI, const float* wI, const void* K,
                    const int32_t* q_seq, const int64_t* q_pos, const int64_t* kv_off,
                    long max_cand, float* scores, long ld_sc, uint32_t* hist, hipStream_t s) {
  switch ((nhI + 15) / 16) {
    case 1: return run<T, KK, 1>(nq, nhI, m, qI, wI, K, q_seq, q_pos, kv_off, max_cand, scores, ld_sc, hist, s);
    case 2: return run<T, KK, 2>(nq, nhI, m, qI, wI, K, q_seq, q_pos, kv_off, max_cand, scores, ld_sc, hist, s);
    case 3: return run<T, KK, 3>(nq, nhI, m, qI, wI, K, q_seq, q_pos, kv_off, max_cand, scores, ld_sc, hist, s);
    default: return run<T, KK, 4>(nq, nhI, m, qI, wI, K, q_seq, q_pos, kv_off, max_cand, scores, ld_sc, hist, s);
  }
}

template <typename T>
hipError_t pick_kk(long nq, int nhI, int cI, int m, const void* qI, const float* wI, const void* K,
                   const int32_t* q_seq, const int64_t* q_pos, const int64_t* kv_off,
                   long max_cand, float* scores, long ld_sc, uint32_t* hist, hipStream_t s) {
  switch (cI / 32) {
    case 1: return pick_nht<T, 1>(nq, nhI, m, qI, wI, K, q_seq, q_pos, kv_off, max_cand, scores, ld_sc, hist, s);
    case 2: return pick_nht<T, 2>(nq, nhI, m, qI, wI, K, q_seq, q_pos, kv_off, max_cand, scores, ld_sc, hist, s);
    case 4: return pick_nht<T, 4>(nq, nhI, m, qI, wI, K, q_seq, q_pos, kv_off, max_cand, scores, ld_sc, hist, s);
    case 8: return pick_nht<T, 8>(nq, nhI, m, qI, wI, K, q_seq, q_pos, kv_off, max_cand, scores, ld_sc, hist, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_indexer(csa_dtype dt, long n_queries, int nhI, int cI, int m, const void* qI,
                          const float* wI, const void* K, const int32_t* q_seq,
                          const int64_t* q_pos, const int64_t* kv_offset, long max_cand,
                          float* scores, long ld_sc, uint32_t* hist, hipStream_t s) {
  if (n_queries == 0 || max_cand == 0) return hipSuccess;
  if (dt == CSA_F32)
    return pick_kk<float>(n_queries, nhI, cI, m, qI, wI, K, q_seq, q_pos, kv_offset, max_cand,
                          scores, ld_sc, hist, s);
  return pick_kk<bf16_t>(n_queries, nhI, cI, m, qI, wI, K, q_seq, q_pos, kv_offset, max_cand,
                         scores, ld_sc, hist, s);
}

}  // namespace csa
