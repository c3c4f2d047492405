// Per-query sweep of the lightning indexer, eq 8 of "Compressed Sparse
// Attention" (section "Lightning Indexer for Sparse Selection"):
//
//   I[t, s] = sum_h w[t, h] * ReLU(q^I[t, h] . K^IComp[s]),  s < n_cand(t),
//
// for one query and one chunk of kSweepKeysPerWG of its candidates, as the
// body of a workgroup of kSweepWaves waves (the per-query sweep kernel in
// indexer.hip).
//
// The head dot products run on MFMA with heads as the 16-row M side and keys
// as the 16-column N side, so the accumulator holds, per lane, 4 heads of one
// key: ReLU, the head weight and the head sum are an in-register epilogue
// plus two cross-lane adds.  Contraction slots are mapped so that a lane
// reads ONE contiguous run of a key row: in step kk, lane group g's slot j is
// dimension g*8*KK + 8*kk + j (KK = cI/32 steps); the query fragments use the
// same map.
#pragma once

#include "common.hpp"
#include "internal.hpp"

namespace csa {

constexpr int kSweepWaves = 4;
constexpr int kSweepKeysPerWG = 512;  // 128 keys (eight 16-key groups) per wave

// Candidates of query r: floor(q_pos[r] / m) (query r at position r when
// q_pos is null), capped at max_cand.
__device__ __forceinline__ long sweep_ncand(int r, int m, const int64_t* __restrict__ q_pos, long max_cand) {
  const long pos = q_pos ? q_pos[r] : (long)r;
  const long nc = pos > 0 ? pos / m : 0;
  return nc < max_cand ? nc : max_cand;
}

// LDS of sweep_chunk.
template <typename T, int KK, int NHT>
struct SweepSmem {
  static constexpr int QPITCH = 32 * KK + 16 / (int)sizeof(T);  // padded q^I row
  alignas(16) uint32_t hist[1 << kTopkL1Bits];
  uint32_t touched[kSweepKeysPerWG];  // bins this chunk hit, in first-touch order
  uint32_t ntouched;
  alignas(16) T q[16 * NHT * QPITCH];
  float w[16 * NHT];
};

// Scores of query r for candidates [chunk0, chunk0 + kSweepKeysPerWG) below
// n_cand: emit(s, score) is called once per key, by one lane.  When hist_row
// is not null and n_cand > hist_min, the level-1 key histogram of these
// scores (top kTopkL1Bits bits of score_key) is added into hist_row with
// device-scope atomics.  Returns n_cand; nothing is done (no barrier either)
// when chunk0 >= n_cand.  Every thread of the workgroup calls it.
template <typename T, int KK, int NHT, typename Emit>
__device__ __forceinline__ long sweep_chunk(SweepSmem<T, KK, NHT>& sm, int r, long chunk0, int nhI, int m,
                                            const T* __restrict__ qI, const float* __restrict__ wI,
                                            const T* __restrict__ K, const int32_t* __restrict__ q_seq,
                                            const int64_t* __restrict__ q_pos, const int64_t* __restrict__ kv_off,
                                            long max_cand, uint32_t* __restrict__ hist_row, long hist_min,
                                            Emit&& emit) {
  constexpr int CI = 32 * KK;
  constexpr int NB = 1 << kTopkL1Bits;
  constexpr int NTH = 64 * kSweepWaves;
  constexpr int VEC = 16 / sizeof(T);
  constexpr int QPITCH = SweepSmem<T, KK, NHT>::QPITCH;  // the 16 lanes reading one k-slice hit distinct banks
  constexpr int QCH = CI / VEC;                          // 16-byte pieces per query row
  uint32_t* s_hist = sm.hist;
  uint32_t* s_touched = sm.touched;
  uint32_t& s_ntouched = sm.ntouched;
  T* s_q = sm.q;
  float* s_w = sm.w;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int seq = q_seq ? q_seq[r] : 0;
  const long ncand = sweep_ncand(r, m, q_pos, max_cand);
  if (chunk0 >= ncand) return ncand;
  const long off = kv_off ? kv_off[seq] : 0;
  const long chunk_end = min(chunk0 + (long)kSweepKeysPerWG, ncand);
  const bool use_hist = hist_row != nullptr && ncand > hist_min;
  __syncthreads();  // every wave's query loads are issued before any key load

  // Each wave owns GPW consecutive 16-key groups of the chunk and keeps D of
  // them in flight: group gi is computed once its loads have landed and its
  // register slot is refilled with group gi + D right away.  A wave whose
  // loads all went out at once would sit in the issue queue (the memory
  // system back-pressures it) until most of its data had arrived, and only
  // then start its MFMAs; the rolling window lets a wave compute while its
  // later groups are still streaming in.  Lanes past the end of the chunk
  // read the chunk's first key instead; their scores are never emitted.
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
  if (use_hist) {
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
      emit(s, part);
      if (use_hist) {
        const uint32_t b = score_key(part) >> (32 - kTopkL1Bits);
        if (atomicAdd(&s_hist[b], 1u) == 0u) s_touched[atomicAdd(&s_ntouched, 1u)] = b;
      }
    }
  }
  if (use_hist) {  // add the touched bins (at most one per key) into the row's histogram
    __syncthreads();
    const uint32_t nt = s_ntouched;
    for (uint32_t e = tid; e < nt; e += NTH) {
      const uint32_t b = s_touched[e];
      atomicAdd(&hist_row[b], s_hist[b]);
    }
  }
  return ncand;
}

}  // namespace csa
