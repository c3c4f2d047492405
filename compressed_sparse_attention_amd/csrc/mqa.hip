// Shared key-value MQA, eq 11 of "Compressed Sparse Attention" (section
// "Shared Key-Value MQA"): every selected compressed entry C_s is both the key
// and the value of all n_h query heads of its token,
//
//   o[r, h] = sum_s softmax_s(scale * q[r, h] . C_s) C_s.
//
// A workgroup owns one query, one group of up to 64 heads and a contiguous
// range of its selection slots, which it walks in chunks of 64 slots (32 for
// rows over 1 KiB) with an online softmax.  Per chunk it gathers the selected
// rows of C^Comp ONCE
// into LDS and serves every head of the group from there (one read of a
// selected entry for all heads: the point of a shared key-value MQA):
//   * S^T = C_sel . q^T on MFMA, keys as M (rows read from LDS with 16-byte
//     reads), heads as N (query fragments straight from global memory).  The
//     accumulator holds one head per lane column, so the per-head max and sum
//     over keys are in-lane plus two cross-lane steps;
//   * P = exp2(S*scale*log2e - running max) goes to LDS as [head][key], with
//     each head's rescale factor for the running output;
//   * O^T = C_sel^T . P^T on MFMA, output dims as M split across the 4 waves,
//     heads as N.  The C^T operand comes from the same LDS rows through two
//     transposing LDS reads per fragment; P^T is one 16-byte read.
// With one split per query the workgroup normalises and writes o and lse
// itself.  Short batches (decode) split the slots across workgroups to fill
// the GPU; each split then writes its unnormalised output and (max, sum) per
// head, and the combine kernel merges the splits by log-sum-exp.
#include <atomic>

#include "common.hpp"
#include "internal.hpp"
#include "select.hpp"

#include <algorithm>

namespace csa {
namespace {

constexpr int kHG = 64;  // heads per pass (4 waves x 16)

// Copies ROWS rows of C (row ids in lanes 0..ROWS-1 of `myid`) into LDS rows
// row0 .. row0+ROWS-1 of Cs (pitch CPITCH elements), using one wave.  A slot
// with id -1 receives finite filler from `fallback`; its logit is masked to
// -inf, so it carries zero weight.  Every lane moves 16-byte pieces; up to
// MAXB pieces per lane are loaded before the first is stored, so the gather
// takes ceil(pieces / MAXB) memory round trips.  For c = 512 bf16 one wave
// instruction moves one 1 KiB row.
template <typename T, int CD, int ROWS, int CPITCH, int MAXB = 16>
__device__ __forceinline__ void wave_gather(const T* __restrict__ Cb, int myid, T* Cs, int row0, int lane,
                                            const void* fallback) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int LPR = CD / VEC;  // 16-byte pieces per row
  if constexpr (LPR <= 64) {
    constexpr int RPI = 64 / LPR;  // rows per instruction
    constexpr int N = (ROWS + RPI - 1) / RPI;
    constexpr int B = N < MAXB ? N : MAXB;
    const int sub = lane / LPR, pc = (lane % LPR) * VEC;
    for (int q0 = 0; q0 < N; q0 += B) {
      u32x4 buf[B];
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const int rl = (q0 + q) * RPI + sub;
        if constexpr (RPI == 1) {
          // one row per instruction: its id is wave-uniform (a scalar base address)
          const int id = __builtin_amdgcn_readlane(myid, q0 + q);
          const T* rowp = id >= 0 ? Cb + (long)id * CD : reinterpret_cast<const T*>(fallback);
          buf[q] = *reinterpret_cast<const u32x4*>(rowp + pc);
        } else {
          const int id = __shfl(myid, rl < ROWS ? rl : 0);
          buf[q] = load16_clamped(Cb + (long)id * CD + pc, rl < ROWS && id >= 0, fallback);
        }
      }
      issue_fence();
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const int rl = (q0 + q) * RPI + sub;
        if (rl < ROWS) *reinterpret_cast<u32x4*>(&Cs[(row0 + rl) * CPITCH + pc]) = buf[q];
      }
    }
  } else {
    constexpr int IPR = LPR / 64;  // instructions per row
    constexpr int N = ROWS * IPR;
    constexpr int B = N < MAXB ? N : MAXB;
    for (int q0 = 0; q0 < N; q0 += B) {
      u32x4 buf[B];
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const int rl = (q0 + q) / IPR;
        const int pc = (((q0 + q) % IPR) * 64 + lane) * VEC;
        const int id = __shfl(myid, rl);
        buf[q] = load16_clamped(Cb + (long)id * CD + pc, id >= 0, fallback);
      }
      issue_fence();
#pragma unroll
      for (int q = 0; q < B; ++q) {
        const int rl = (q0 + q) / IPR;
        const int pc = (((q0 + q) % IPR) * 64 + lane) * VEC;
        *reinterpret_cast<u32x4*>(&Cs[(row0 + rl) * CPITCH + pc]) = buf[q];
      }
    }
  }
}

template <typename T> __device__ __forceinline__ void store4(T* p, const float* v);
template <> __device__ __forceinline__ void store4<float>(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
template <> __device__ __forceinline__ void store4<bf16_t>(bf16_t* p, const float* v) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
}

// Selection slots per chunk of the 64-head-group kernel: 64 while a gathered
// row is at most 1 KiB, else 32 (keeps the chunk within ~70 KiB of LDS).
template <typename T, int DTW>
constexpr int group_chunk() {
  return 64 * DTW * (int)sizeof(T) <= 1024 ? 64 : 32;
}

template <typename T, int DTW>
__global__ __launch_bounds__(256) void mqa_kernel(int nh, int k, int nhg, int nsplit, int cps,
                                                  float scale_log2, const T* __restrict__ q,
                                                  const T* __restrict__ C,
                                                  const int32_t* __restrict__ q_seq,
                                                  const int64_t* __restrict__ kv_off,
                                                  const int32_t* __restrict__ idx, T* __restrict__ o,
                                                  float* __restrict__ lse, float* __restrict__ part_o,
                                                  float* __restrict__ part_ml) {
  constexpr int CD = 64 * DTW;  // head dim c
  constexpr int KS = group_chunk<T, DTW>();
  constexpr int VEC = 16 / sizeof(T);
  constexpr int CPITCH = CD + 2 * VEC;  // rows staggered by 32 bytes: conflict-free 16-byte fragment reads
  constexpr int PPITCH = KS + 2 * VEC;
  constexpr int KSTEPS = CD / 32;
  constexpr int VPF = sizeof(T) == 2 ? 4 : 8;          // VGPRs per fragment
  constexpr bool QREG = KSTEPS * VPF <= 64;             // keep the query fragments in registers
  __shared__ __attribute__((aligned(16))) T Cs[KS * CPITCH];
  __shared__ __attribute__((aligned(16))) T Ps[kHG * PPITCH];
  __shared__ int32_t s_rows[KS];
  __shared__ float s_alpha[kHG];
  __shared__ float s_l[kHG];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const long bid = blockIdx.x;
  const int j = (int)(bid % nsplit);
  const long rest = bid / nsplit;
  const int hg = (int)(rest % nhg);
  const long r = rest / nhg;
  const int h0 = hg * kHG;
  const int NT = min(4, (nh - h0 + 15) / 16);  // 16-head tiles in this group
  const int seq = q_seq ? q_seq[r] : 0;
  const long off = kv_off ? kv_off[seq] : 0;

  // running softmax state of the heads this wave scores (head h0 + 16*wave + c16)
  const int qhead = h0 + 16 * wave + c16;
  const bool qwave = wave < NT;
  float m_run = -INFINITY, l_run = 0.f;
  const T* qrow = q + (r * nh + qhead) * CD + 8 * g;

  Frag<T> qf[QREG ? KSTEPS : 1];
  if constexpr (QREG) {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[kk].load_clamped(qrow + 32 * kk, qwave && qhead < nh, q);
  }

  f32x4 acc_o[DTW][4];
#pragma unroll
  for (int dt = 0; dt < DTW; ++dt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc_o[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ch = 0; ch < cps; ++ch) {
    const int slot0 = (j * cps + ch) * KS;
    if (slot0 >= k) break;  // uniform across the workgroup
    {
      constexpr int RPW = KS / 4;  // rows gathered by each wave
      const int slot = slot0 + RPW * wave + lane;
      const int raw = idx[r * k + (slot < k ? slot : k - 1)];  // always in bounds
      const int myid = (lane < RPW && slot < k) ? raw : -1;
      if (lane < RPW) s_rows[RPW * wave + lane] = myid;
      wave_gather<T, CD, RPW, CPITCH>(C + off * CD, myid, Cs, RPW * wave, lane, q);
    }
    __syncthreads();

    if (qwave) {
      f32x4 acc[KS / 16];
#pragma unroll
      for (int mt = 0; mt < KS / 16; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
      for (int kk = 0; kk < KSTEPS; ++kk) {
        Frag<T> bq;
        if constexpr (QREG)
          bq = qf[kk];
        else
          bq.load_clamped(qrow + 32 * kk, qhead < nh, q);
#pragma unroll
        for (int mt = 0; mt < KS / 16; ++mt) {
          Frag<T> ac;
          ac.load(&Cs[(16 * mt + c16) * CPITCH + 32 * kk + 8 * g]);
          mma(acc[mt], ac, bq);
        }
      }
      float x[KS / 16][4];
      float cm = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < KS / 16; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int key = 16 * mt + 4 * g + rr;
          x[mt][rr] = s_rows[key] >= 0 ? acc[mt][rr] * scale_log2 : -INFINITY;
          cm = fmaxf(cm, x[mt][rr]);
        }
      cm = wave_max_xor_16_32(cm);
      const float m_new = fmaxf(m_run, cm);
      const bool none = (m_new == -INFINITY);
      const float alpha = none ? 1.f : exp2_fast(m_run - m_new);
      float sum = 0.f;
#pragma unroll
      for (int mt = 0; mt < KS / 16; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float p = none ? 0.f : exp2_fast(x[mt][rr] - m_new);
          sum += p;
          Ps[(16 * wave + c16) * PPITCH + 16 * mt + 4 * g + rr] = from_f32<T>(p);
        }
      sum = wave_sum_xor_16_32(sum);
      l_run = l_run * alpha + sum;
      m_run = m_new;
      if (g == 0) s_alpha[16 * wave + c16] = alpha;
    }
    __syncthreads();

#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      if (nt < NT) {
        const float a = s_alpha[16 * nt + c16];
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt) acc_o[dt][nt] *= a;
      }
    }
#pragma unroll
    for (int kk = 0; kk < KS / 32; ++kk) {
      Frag<T> bp[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        if (nt < NT) bp[nt].load(&Ps[(16 * nt + c16) * PPITCH + 32 * kk + 8 * g]);
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt) {
        const Frag<T> ac = frag_ct<T>(Cs, CPITCH, 32 * kk, (wave * DTW + dt) * 16, lane);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          if (nt < NT) mma(acc_o[dt][nt], ac, bp[nt]);
      }
    }
    __syncthreads();
  }

  if (nsplit == 1) {
    if (qwave && g == 0) {
      s_l[16 * wave + c16] = l_run;
      if (lse && qhead < nh)
        lse[r * nh + qhead] = (l_run > 0.f) ? (m_run + log2f(l_run)) * 0.6931471805599453f : -INFINITY;
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int head = h0 + 16 * nt + c16;
      if (nt < NT && head < nh) {
        const float l = s_l[16 * nt + c16];
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt) {
          float v[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) v[rr] = acc_o[dt][nt][rr] * inv;
          store4<T>(o + (r * nh + head) * CD + (wave * DTW + dt) * 16 + 4 * g, v);
        }
      }
    }
  } else {
    const long pbase = (r * nsplit + j) * (long)nh;
    if (qwave && g == 0 && qhead < nh) {
      part_ml[(pbase + qhead) * 2] = m_run;
      part_ml[(pbase + qhead) * 2 + 1] = l_run;
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int head = h0 + 16 * nt + c16;
      if (nt < NT && head < nh) {
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt) {
          float* dst = part_o + (pbase + head) * CD + (wave * DTW + dt) * 16 + 4 * g;
          *reinterpret_cast<float4*>(dst) =
              make_float4(acc_o[dt][nt][0], acc_o[dt][nt][1], acc_o[dt][nt][2], acc_o[dt][nt][3]);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Long bf16 batches with 128 <= c <= 512 (prefill): eight waves per
// (query, 64-head group), 64-slot chunks, double buffered.  While chunk i is
// scored and accumulated from one LDS buffer, the rows of chunk i+1 are in
// flight into registers (and the ids of chunk i+2 are being read), and are
// stored into the other buffer after the output update (the loop's barriers
// cover LDS only, so those loads stay in flight through them).  S^T is split over
// (16-head tile, 32-key half) with the per-head max and sum exchanged through
// LDS; O^T is split over the output dims (c/8 per wave).
// ---------------------------------------------------------------------------
constexpr int kG8Chunk = 64;
constexpr int kG8MaxStaged = 2048;  // slot ids of a split staged in LDS

template <int DTW>
__global__ __launch_bounds__(512) void mqa_group8_kernel(int nh, int k, int nhg, int nsplit, int cps,
                                                         float scale_log2, const bf16_t* __restrict__ q,
                                                         const bf16_t* __restrict__ C,
                                                         const int32_t* __restrict__ q_seq,
                                                         const int64_t* __restrict__ kv_off,
                                                         const int32_t* __restrict__ idx,
                                                         bf16_t* __restrict__ o, float* __restrict__ lse,
                                                         float* __restrict__ part_o,
                                                         float* __restrict__ part_ml) {
  constexpr int CD = 64 * DTW;
  constexpr int KS = kG8Chunk;
  constexpr int CPITCH = CD + 16;  // rows staggered by 32 bytes: conflict-free 16-byte fragment reads
  constexpr int PPITCH = KS + 16;
  constexpr int KSTEPS = CD / 32;
  constexpr int DTPW = CD / 16 / 8;  // output 16-dim tiles per wave
  constexpr int RPW = KS / 8;        // rows gathered per wave per chunk
  constexpr int LPR = CD / 8;        // 16-byte pieces per row
  constexpr int RPI = 64 / LPR;      // rows per wave instruction
  constexpr int NLD = RPW / RPI;     // row loads per lane per chunk
  __shared__ __attribute__((aligned(16))) bf16_t Cs[2][KS * CPITCH];
  __shared__ __attribute__((aligned(16))) bf16_t Ps[kHG * PPITCH];
  __shared__ int32_t s_rows[2][KS];
  __shared__ float s_red[2][2][kHG];
  __shared__ float s_alpha[kHG];
  __shared__ float s_l[kHG];
  __shared__ int32_t s_ids[kG8MaxStaged];
  __shared__ int s_ext[2][8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const long bid = blockIdx.x;
  const int j = (int)(bid % nsplit);
  const long rest = bid / nsplit;
  const int hg = (int)(rest % nhg);
  const long r = rest / nhg;
  const int h0 = hg * kHG;
  const int NT = min(4, (nh - h0 + 15) / 16);
  const int seq = q_seq ? q_seq[r] : 0;
  const long off = kv_off ? kv_off[seq] : 0;
  const bf16_t* Cb = C + off * CD;
  const int nch_all = min(cps, (k - j * cps * KS + KS - 1) / KS);  // chunks of this split (>= 1)
  const int sbeg = j * cps * KS, send = min(k, sbeg + nch_all * KS);

  const int ht = wave & 3, kh = wave >> 2;  // S^T work: head tile, key half
  const int qhead = h0 + 16 * ht + c16;
  const bool qlive = ht < NT;

  // The split's slot ids are staged in LDS once (when they fit).  Slots that
  // hold -1 contribute nothing; when the valid ids form a prefix of the split
  // (the selector pads rows with -1 at the end), the chunks past it are not
  // walked at all.
  const bool staged = send - sbeg <= kG8MaxStaged;
  int nch = nch_all;
  if (staged) {
    int first_bad = 0x7FFFFFFF, last_good = -1;
    for (int sl = sbeg + tid; sl < send; sl += 512) {
      const int id = idx[r * k + sl];
      s_ids[sl - sbeg] = id;
      if (id < 0) first_bad = min(first_bad, sl); else last_good = max(last_good, sl);
    }
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      first_bad = min(first_bad, __shfl_xor(first_bad, sh));
      last_good = max(last_good, __shfl_xor(last_good, sh));
    }
    if (lane == 0) {
      s_ext[0][wave] = first_bad;
      s_ext[1][wave] = last_good;
    }
    __syncthreads();
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      first_bad = min(first_bad, s_ext[0][w]);
      last_good = max(last_good, s_ext[1][w]);
    }
    if (last_good < first_bad) nch = max(0, (last_good - sbeg + KS) / KS);
  }

  // row ids of chunk c for this wave's RPW rows (lane < RPW), -1 past k
  auto load_ids = [&](int c) -> int {
    const int slot = (j * cps + c) * KS + RPW * wave + lane;
    const int raw = staged ? s_ids[min(slot, send - 1) - sbeg] : idx[r * k + (slot < k ? slot : k - 1)];
    return (lane < RPW && slot < send) ? raw : -1;
  };
  u32x4 stg[NLD];
  auto issue_rows = [&](int ids) {
    const int sub = lane / LPR, pc = (lane % LPR) * 8;
#pragma unroll
    for (int qd = 0; qd < NLD; ++qd) {
      if constexpr (RPI == 1) {  // one row per instruction: a wave-uniform (scalar) row address
        const int id = __builtin_amdgcn_readlane(ids, qd);
        const bf16_t* rowp = id >= 0 ? Cb + (long)id * CD : q;
        stg[qd] = *reinterpret_cast<const u32x4*>(rowp + pc);
      } else {
        const int id = __shfl(ids, qd * RPI + sub);
        stg[qd] = load16_clamped(Cb + (long)id * CD + pc, id >= 0, q);
      }
    }
    issue_fence();
  };
  auto store_rows = [&](int buf, int ids) {
    const int sub = lane / LPR, pc = (lane % LPR) * 8;
#pragma unroll
    for (int qd = 0; qd < NLD; ++qd)
      *reinterpret_cast<u32x4*>(&Cs[buf][(RPW * wave + qd * RPI + sub) * CPITCH + pc]) = stg[qd];
    if (lane < RPW) s_rows[buf][RPW * wave + lane] = ids;
  };

  // prologue: chunk 0 into buffer 0, chunk 1 in flight, ids of chunk 2
  // requested.  The query fragments are loaded before the first rows: their
  // wait (for the rows, which come later in issue order) then happens here,
  // not inside the chunk loop, where it would also wait for the loop's
  // prefetch of the next chunk.
  Frag<bf16_t> qf[KSTEPS];
#pragma unroll
  for (int kk = 0; kk < KSTEPS; ++kk) qf[kk].load_clamped(q + (r * nh + qhead) * CD + 32 * kk + 8 * g, qlive && qhead < nh, q);
  int ids_cur = load_ids(0);
  int ids_nxt = nch > 1 ? load_ids(1) : -1;
  issue_rows(ids_cur);
  store_rows(0, ids_cur);
  if (nch > 1) issue_rows(ids_nxt);
  int ids_nn = nch > 2 ? load_ids(2) : -1;
  __syncthreads();

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc_o[DTPW][4];
#pragma unroll
  for (int dt = 0; dt < DTPW; ++dt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc_o[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ch = 0; ch < nch; ++ch) {
    const int cur = ch & 1;
    const bf16_t* Cc = Cs[cur];
    // ---- S^T for keys 32*kh .. +31 of this chunk, head tile ht
    float x[2][4];
    float cm = -INFINITY;
    if (qlive) {
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) {
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          Frag<bf16_t> ac;
          ac.load(&Cc[(32 * kh + 16 * t + c16) * CPITCH + 32 * kk + 8 * g]);
          mma(acc[t], ac, qf[kk]);
        }
      }
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int key = 32 * kh + 16 * t + 4 * g + rr;
          x[t][rr] = s_rows[cur][key] >= 0 ? acc[t][rr] * scale_log2 : -INFINITY;
          cm = fmaxf(cm, x[t][rr]);
        }
      cm = wave_max_xor_16_32(cm);
      if (g == 0) s_red[0][kh][16 * ht + c16] = cm;
    }
    lds_barrier();
    // Lazy rescaling: the reference maximum m_run moves only when a chunk's
    // maximum exceeds it by more than 2^8, so the exponentials stay below 256
    // (exact in the fp32 sums and within bf16's range) and the O^T
    // accumulators are rescaled in the rare chunks where it moves.
    float alpha = 1.f;
    if (qlive) {
      const int hl = 16 * ht + c16;
      const float cmax = fmaxf(s_red[0][0][hl], s_red[0][1][hl]);
      const float m_new = (m_run == -INFINITY || cmax > m_run + 8.f) ? fmaxf(m_run, cmax) : m_run;
      const bool none = (m_new == -INFINITY);
      alpha = none ? 1.f : exp2_fast(m_run - m_new);
      float ps = 0.f;
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        float p[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          p[rr] = none ? 0.f : exp2_fast(x[t][rr] - m_new);
          ps += p[rr];
        }
        *reinterpret_cast<uint2*>(&Ps[hl * PPITCH + 32 * kh + 16 * t + 4 * g]) =
            make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
      }
      ps = wave_sum_xor_16_32(ps);
      if (g == 0) {
        s_red[1][kh][hl] = ps;
        if (kh == 0) s_alpha[hl] = alpha;
      }
      m_run = m_new;
    }
    lds_barrier();
    if (qlive) {
      const int hl = 16 * ht + c16;
      l_run = l_run * alpha + s_red[1][0][hl] + s_red[1][1][hl];
    }
    // ---- O^T for dims tiles DTPW*wave .. : C_sel^T x P^T
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      if (nt < NT) {
        const float a = s_alpha[16 * nt + c16];
        if (__builtin_amdgcn_read_exec() & __ballot(a != 1.f)) {  // some head of this tile moved its maximum
#pragma unroll
          for (int dt = 0; dt < DTPW; ++dt) acc_o[dt][nt] *= a;
        }
      }
    }
#pragma unroll
    for (int kk = 0; kk < KS / 32; ++kk) {
      Frag<bf16_t> bp[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        if (nt < NT) bp[nt].load(&Ps[(16 * nt + c16) * PPITCH + 32 * kk + 8 * g]);
#pragma unroll
      for (int dt = 0; dt < DTPW; ++dt) {
        const Frag<bf16_t> ac = frag_ct<bf16_t>(Cc, CPITCH, 32 * kk, (wave * DTPW + dt) * 16, lane);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          if (nt < NT) mma(acc_o[dt][nt], ac, bp[nt]);
      }
    }
    // ---- rows of chunk ch+1 land in the other buffer; chunk ch+2 goes in flight
    if (ch + 1 < nch) store_rows(cur ^ 1, ids_nxt);
    lds_barrier();
    if (ch + 2 < nch) {
      issue_rows(ids_nn);
      ids_nxt = ids_nn;
      ids_nn = ch + 3 < nch ? load_ids(ch + 3) : -1;
    }
  }

  if (nsplit == 1) {
    if (qlive && kh == 0 && g == 0) {
      s_l[16 * ht + c16] = l_run;
      if (lse && qhead < nh)
        lse[r * nh + qhead] = (l_run > 0.f) ? (m_run + log2f(l_run)) * 0.6931471805599453f : -INFINITY;
    }
    __syncthreads();
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int head = h0 + 16 * nt + c16;
      if (nt < NT && head < nh) {
        const float l = s_l[16 * nt + c16];
        const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
        for (int dt = 0; dt < DTPW; ++dt) {
          float v[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) v[rr] = acc_o[dt][nt][rr] * inv;
          store4<bf16_t>(o + (r * nh + head) * CD + (wave * DTPW + dt) * 16 + 4 * g, v);
        }
      }
    }
  } else {
    const long pbase = (r * nsplit + j) * (long)nh;
    if (qlive && kh == 0 && g == 0 && qhead < nh) {
      part_ml[(pbase + qhead) * 2] = m_run;
      part_ml[(pbase + qhead) * 2 + 1] = l_run;
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int head = h0 + 16 * nt + c16;
      if (nt < NT && head < nh) {
#pragma unroll
        for (int dt = 0; dt < DTPW; ++dt)
          *reinterpret_cast<float4*>(part_o + (pbase + head) * CD + (wave * DTPW + dt) * 16 + 4 * g) =
              make_float4(acc_o[dt][nt][0], acc_o[dt][nt][1], acc_o[dt][nt][2], acc_o[dt][nt][3]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Persistent form of the kernel above for c = 512 (long bf16 batches whose
// splits' slot ids fit in LDS).  One workgroup per CU walks the units
// u = blockIdx.x, blockIdx.x + gridDim.x, ... (unit = query, 64-head group,
// split) and keeps the chunk pipeline running across unit boundaries, so a
// unit's start does not pay its two dependent memory round trips (slot ids,
// then rows) with the CU otherwise idle: the next unit's slot ids are fetched
// during the current unit's first chunk and staged after it, its query
// fragments are fetched when the current unit finishes, and its first rows
// are gathered during the current unit's last chunk.  Rows go straight into
// LDS (global_load_lds issued from asm, one 1 KiB row per instruction), one
// chunk ahead; the top of each chunk waits for them explicitly.  A unit whose
// first rows could not be prefetched (the unit before had a single chunk)
// gathers them when it starts.  Barriers inside the unit loop are LDS-only:
// a plain barrier would also drain the row gathers and output stores in
// flight.  The next chunk's rows are requested one row per two k-steps of
// S^T: issued at once, a wave's eight direct-to-LDS loads stalled it for
// about 1200 cycles per chunk while the address path took them in.
// ---------------------------------------------------------------------------
constexpr int kStreamMaxStaged = 512;  // slot ids of a unit staged in LDS

struct G8Unit {
  long r;
  int h0, j, sbeg, send, nch, sb;  // sb: the s_ids buffer holding the unit's slot ids
  const bf16_t* Cb;
};

__global__ __launch_bounds__(512) void mqa_stream_kernel(long nunits, int nh, int k, int nhg, int nsplit, int cps,
                                                         float scale_log2, const bf16_t* __restrict__ q,
                                                         const bf16_t* __restrict__ C,
                                                         const int32_t* __restrict__ q_seq,
                                                         const int64_t* __restrict__ kv_off,
                                                         const int32_t* __restrict__ idx,
                                                         bf16_t* __restrict__ o, float* __restrict__ lse,
                                                         float* __restrict__ part_o,
                                                         float* __restrict__ part_ml) {
  constexpr int CD = 512;
  constexpr int KS = kG8Chunk;
  constexpr int CPITCH = CD + 16;  // rows staggered by 32 bytes: conflict-free 16-byte fragment reads
  constexpr int PPITCH = KS + 16;
  constexpr int KSTEPS = CD / 32;
  constexpr int DTPW = CD / 16 / 8;
  constexpr int RPW = KS / 8;  // rows gathered per wave per chunk
  __shared__ __attribute__((aligned(16))) bf16_t Cs[2][KS * CPITCH];
  __shared__ __attribute__((aligned(16))) bf16_t Ps[kHG * PPITCH];
  __shared__ int32_t s_rows[2][KS];
  __shared__ float s_red[2][2][kHG];
  __shared__ float s_alpha[kHG];
  __shared__ float s_l[kHG];
  __shared__ int32_t s_ids[2][kStreamMaxStaged];
  __shared__ int s_ext[2][8];
  __shared__ int s_flag[8];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int ht = wave & 3, kh = wave >> 2;
  const long stride = gridDim.x;

  auto describe = [&](long u, int sb) -> G8Unit {
    G8Unit d;
    d.j = (int)(u % nsplit);
    const long rest = u / nsplit;
    d.h0 = (int)(rest % nhg) * kHG;
    d.r = rest / nhg;
    const int seq = q_seq ? q_seq[d.r] : 0;
    d.Cb = C + (kv_off ? kv_off[seq] : 0) * CD;
    const int nch_all = min(cps, (k - d.j * cps * KS + KS - 1) / KS);
    d.sbeg = d.j * cps * KS;
    d.send = min(k, d.sbeg + nch_all * KS);
    d.nch = nch_all;
    d.sb = sb;
    return d;
  };
  // slot ids: fetched into a register, staged in LDS (with the test of a
  // -1-padded prefix that trims trailing chunks), then counted after a barrier
  int nid = -1;
  auto fetch_ids = [&](const G8Unit& d) { nid = idx[d.r * k + min(d.sbeg + tid, d.send - 1)]; };
  auto stage_ids = [&](const G8Unit& d) {
    const int sl = d.sbeg + tid;
    int first_bad = 0x7FFFFFFF, last_good = -1;
    if (sl < d.send) {
      s_ids[d.sb][tid] = nid;
      if (nid < 0) first_bad = sl; else last_good = sl;
    }
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) {
      first_bad = min(first_bad, __shfl_xor(first_bad, sh));
      last_good = max(last_good, __shfl_xor(last_good, sh));
    }
    if (lane == 0) {
      s_ext[0][wave] = first_bad;
      s_ext[1][wave] = last_good;
    }
  };
  auto count_chunks = [&](G8Unit& d) {
    int first_bad = 0x7FFFFFFF, last_good = -1;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      first_bad = min(first_bad, s_ext[0][w]);
      last_good = max(last_good, s_ext[1][w]);
    }
    if (last_good < first_bad) d.nch = max(0, (last_good - d.sbeg + KS) / KS);
  };
  // rows of chunk c of unit d into buffer b: wave w brings rows RPW w .. +RPW-1;
  // the wave's row ids come from one LDS read (lane i holds row i's id)
  auto gather = [&](const G8Unit& d, int c, int b) {
    const int sl0 = d.sbeg + c * KS + RPW * wave;
    const int lid = s_ids[d.sb][min(sl0 + lane, d.send - 1) - d.sbeg];
    const int myid = (lane < RPW && sl0 + lane < d.send) ? lid : -1;
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
      const int id = __builtin_amdgcn_readlane(myid, i);
      const bf16_t* src = id >= 0 ? d.Cb + (long)id * CD : q;  // -1: finite filler, weight 0
      const uint32_t base = (uint32_t)(size_t)(lds_char*)&Cs[b][(RPW * wave + i) * CPITCH];
      gather_row_lds(src + 8 * lane, __builtin_amdgcn_readfirstlane(base));
    }
    if (lane < RPW) s_rows[b][RPW * wave + lane] = myid;
  };
  // the unit's 64 query rows (one 1 KiB row per head) into buffer bf, eight per wave
  auto stage_q = [&](const G8Unit& d, int bf) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * wave + i;
      const int head = min(d.h0 + row, nh - 1);  // heads past nh: finite filler, never stored
      const uint32_t base = (uint32_t)(size_t)(lds_char*)&Cs[bf][row * CPITCH];
      gather_row_lds(q + (d.r * nh + head) * CD + 8 * lane, __builtin_amdgcn_readfirstlane(base));
    }
  };
  Frag<bf16_t> qf[KSTEPS];
  auto read_q = [&](int bf) {
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) qf[kk].load(&Cs[bf][(16 * ht + c16) * CPITCH + 32 * kk + 8 * g]);
  };
  auto load_q = [&](const G8Unit& d) {
    const int qhead = d.h0 + 16 * ht + c16;
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk)
      qf[kk].load_clamped(q + (d.r * nh + qhead) * CD + 32 * kk + 8 * g, qhead < nh, q);
  };

  long u = blockIdx.x;
  if (u >= nunits) return;
  G8Unit cu = describe(u, 0), nu;
  fetch_ids(cu);
  stage_ids(cu);
  __syncthreads();
  count_chunks(cu);
  bool has_nu = u + stride < nunits, nu_staged = false;
  if (has_nu) nu = describe(u + stride, 1);
  load_q(cu);
  bool q_loaded = true;
  bool q_lds = false;  // the current unit's query rows wait in the other row buffer
  int bufc = 0;
  bool first_in_buf = false;  // the current unit's chunk 0 is already in Cs[bufc] (or in flight to it)

  while (true) {
    if (!q_loaded && !q_lds) load_q(cu);
    q_loaded = false;
    if (cu.nch > 0 && !first_in_buf) gather(cu, 0, bufc);
    first_in_buf = false;
    const int NT = min(4, (nh - cu.h0 + 15) / 16);
    const int qhead = cu.h0 + 16 * ht + c16;
    const bool qlive = ht < NT;
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc_o[DTPW][4];
#pragma unroll
    for (int dt = 0; dt < DTPW; ++dt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc_o[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int ch = 0; ch < cu.nch; ++ch) {
      const int cur = bufc;
      // this wave's gathers of chunk ch (and everything it issued before
      // them) have landed; after the barrier, every wave's have
      wait_stores();
      lds_barrier();
      if (q_lds) {  // (chunk 0) fragments from the staged rows, read before chunk 1's rows replace them
        read_q(cur ^ 1);
        lds_barrier();
        q_lds = false;
      }
      // the next chunk goes in flight into the other buffer (free: chunk
      // ch - 1 was read before the barrier); the next unit's slot ids are
      // requested once this unit has started
      const bool g_cur = ch + 1 < cu.nch;
      const bool g_any = g_cur || (has_nu && nu_staged && nu.nch > 0);
      if (!g_cur && g_any) first_in_buf = true;
      if (ch == 0 && has_nu) fetch_ids(nu);
      // row ids of the chunk to gather (lane i holds row i's), one LDS read
      const int g_sb = g_cur ? cu.sb : nu.sb, g_sbeg = g_cur ? cu.sbeg : nu.sbeg;
      const int g_send = g_cur ? cu.send : nu.send;
      const int g_sl0 = (g_cur ? cu.sbeg + (ch + 1) * KS : nu.sbeg) + RPW * wave;
      const bf16_t* gCb = g_cur ? cu.Cb : nu.Cb;
      int gid = -1;
      if (g_any) {
        const int lid = s_ids[g_sb][min(g_sl0 + lane, g_send - 1) - g_sbeg];
        gid = (lane < RPW && g_sl0 + lane < g_send) ? lid : -1;
        if (lane < RPW) s_rows[cur ^ 1][RPW * wave + lane] = gid;
      }
      auto gissue = [&](int i) {
        const int id = __builtin_amdgcn_readlane(gid, i);
        const bf16_t* src = id >= 0 ? gCb + (long)id * CD : q;  // -1: finite filler, weight 0
        const uint32_t base = (uint32_t)(size_t)(lds_char*)&Cs[cur ^ 1][(RPW * wave + i) * CPITCH];
        gather_row_lds(src + 8 * lane, __builtin_amdgcn_readfirstlane(base));
      };
      const bf16_t* Cc = Cs[cur];
      float x[2][4];
      float cm = -INFINITY;
      // S^T (every wave, also over a head tile past nh: its results are
      // discarded): key fragments are read two steps ahead of their MFMAs
      // (the fences keep the compiler from sinking each read next to its
      // use), and one row of the next chunk is gathered every two steps
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
      {
        const bf16_t* ka = &Cc[(32 * kh + c16) * CPITCH + 8 * g];
        Frag<bf16_t> fa[3][2];
        fa[0][0].load(ka);
        fa[0][1].load(ka + 16 * CPITCH);
        fa[1][0].load(ka + 32);
        fa[1][1].load(ka + 16 * CPITCH + 32);
#pragma unroll
        for (int kk = 0; kk < KSTEPS; ++kk) {
          if ((kk & 1) == 0 && g_any) gissue(kk >> 1);
          if (kk + 2 < KSTEPS) {
            fa[(kk + 2) % 3][0].load(ka + 32 * (kk + 2));
            fa[(kk + 2) % 3][1].load(ka + 16 * CPITCH + 32 * (kk + 2));
          }
          issue_fence();
          mma(acc[0], fa[kk % 3][0], qf[kk]);
          mma(acc[1], fa[kk % 3][1], qf[kk]);
          issue_fence();
        }
      }
      if (qlive) {
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            const int key = 32 * kh + 16 * t + 4 * g + rr;
            x[t][rr] = s_rows[cur][key] >= 0 ? acc[t][rr] * scale_log2 : -INFINITY;
            cm = fmaxf(cm, x[t][rr]);
          }
        cm = wave_max_xor_16_32(cm);
      }
      // Numerators against the running reference maximum m_run.  Lazy
      // rescaling: m_run moves only when a chunk's maximum exceeds it by more
      // than 2^8 (so the exponentials stay below 256, exact in the fp32 sums
      // and within bf16's range), decided per head from both key halves'
      // maxima.  A wave that sees one of its heads exceed (or the unit's
      // first chunk) raises a flag; only then do the waves exchange maxima
      // and redo their numerators against the moved references, so most
      // chunks need one barrier here instead of two.
      const int hl = 16 * ht + c16;
      auto numerators = [&](float mref) {
        const bool none = (mref == -INFINITY);
        float ps = 0.f;
#pragma unroll
        for (int t = 0; t < 2; ++t) {
          float p[4];
#pragma unroll
          for (int rr = 0; rr < 4; ++rr) {
            p[rr] = none ? 0.f : exp2_fast(x[t][rr] - mref);
            ps += p[rr];
          }
          *reinterpret_cast<uint2*>(&Ps[hl * PPITCH + 32 * kh + 16 * t + 4 * g]) =
              make_uint2(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]));
        }
        ps = wave_sum_xor_16_32(ps);
        if (g == 0) s_red[1][kh][hl] = ps;
      };
      const bool moves = qlive && (m_run == -INFINITY || cm > m_run + 8.f);
      if (qlive) numerators(m_run);
      const bool wave_moves = __ballot(moves) != 0;
      if (lane == 0) s_flag[wave] = wave_moves;
      // the next unit's slot ids are staged behind this unit's first chunk
      const bool staging = ch == 0 && has_nu;
      if (staging) stage_ids(nu);
      lds_barrier();
      if (staging) {
        count_chunks(nu);
        nu_staged = true;
      }
      bool any_moves = false;
#pragma unroll
      for (int w = 0; w < 8; ++w) any_moves |= s_flag[w] != 0;
      float alpha = 1.f;
      if (any_moves) {
        if (qlive && g == 0) s_red[0][kh][hl] = cm;
        lds_barrier();
        if (qlive) {
          const float cmax = fmaxf(s_red[0][0][hl], s_red[0][1][hl]);
          const float m_new = (m_run == -INFINITY || cmax > m_run + 8.f) ? fmaxf(m_run, cmax) : m_run;
          alpha = m_new == -INFINITY ? 1.f : exp2_fast(m_run - m_new);
          numerators(m_new);
          if (g == 0 && kh == 0) s_alpha[hl] = alpha;
          m_run = m_new;
        }
        lds_barrier();
      }
      if (qlive) l_run = l_run * alpha + s_red[1][0][hl] + s_red[1][1][hl];
      if (any_moves) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          if (nt < NT) {
            const float a = s_alpha[16 * nt + c16];
            if (__builtin_amdgcn_read_exec() & __ballot(a != 1.f)) {  // some head of this tile moved its maximum
#pragma unroll
              for (int dt = 0; dt < DTPW; ++dt) acc_o[dt][nt] *= a;
            }
          }
        }
      }
      {  // O^T: all P fragments of the chunk first, the transposed C reads two steps ahead
        constexpr int NSTEP = (KS / 32) * DTPW;
        Frag<bf16_t> bp[KS / 32][4];
#pragma unroll
        for (int kk = 0; kk < KS / 32; ++kk)
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) bp[kk][nt].load(&Ps[(16 * nt + c16) * PPITCH + 32 * kk + 8 * g]);
        Frag<bf16_t> ac[3];
        ac[0] = frag_ct<bf16_t>(Cc, CPITCH, 0, (wave * DTPW) * 16, lane);
        ac[1] = frag_ct<bf16_t>(Cc, CPITCH, 32 * (1 / DTPW), (wave * DTPW + 1 % DTPW) * 16, lane);
#pragma unroll
        for (int st = 0; st < NSTEP; ++st) {
          if (st + 2 < NSTEP)
            ac[(st + 2) % 3] =
                frag_ct<bf16_t>(Cc, CPITCH, 32 * ((st + 2) / DTPW), (wave * DTPW + (st + 2) % DTPW) * 16, lane);
          issue_fence();
#pragma unroll
          for (int nt = 0; nt < 4; ++nt)
            if (nt < NT) mma(acc_o[st % DTPW][nt], ac[st % 3], bp[st / DTPW][nt]);
          issue_fence();
        }
      }
      bufc ^= 1;
    }

    // ---- finish the unit.  After the barrier every wave is done with this
    // unit's last rows, and the next unit's query rows go into their buffer
    // (one copy of each row, where fragment loads per wave fetched every
    // head tile's rows twice).
    q_lds = false;
    if (nsplit == 1) {
      if (qlive && kh == 0 && g == 0) {
        s_l[16 * ht + c16] = l_run;
        if (lse && qhead < nh)
          lse[cu.r * nh + qhead] = (l_run > 0.f) ? (m_run + log2f(l_run)) * 0.6931471805599453f : -INFINITY;
      }
      lds_barrier();
      if (has_nu) {
        stage_q(nu, bufc ^ 1);
        q_lds = true;
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int head = cu.h0 + 16 * nt + c16;
        if (nt < NT && head < nh) {
          const float l = s_l[16 * nt + c16];
          const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
          for (int dt = 0; dt < DTPW; ++dt) {
            float v[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) v[rr] = acc_o[dt][nt][rr] * inv;
            store4<bf16_t>(o + (cu.r * nh + head) * CD + (wave * DTPW + dt) * 16 + 4 * g, v);
          }
        }
      }
    } else {
      lds_barrier();
      if (has_nu) {
        stage_q(nu, bufc ^ 1);
        q_lds = true;
      }
      const long pbase = (cu.r * nsplit + cu.j) * (long)nh;
      if (qlive && kh == 0 && g == 0 && qhead < nh) {
        part_ml[(pbase + qhead) * 2] = m_run;
        part_ml[(pbase + qhead) * 2 + 1] = l_run;
      }
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int head = cu.h0 + 16 * nt + c16;
        if (nt < NT && head < nh) {
#pragma unroll
          for (int dt = 0; dt < DTPW; ++dt)
            *reinterpret_cast<float4*>(part_o + (pbase + head) * CD + (wave * DTPW + dt) * 16 + 4 * g) =
                make_float4(acc_o[dt][nt][0], acc_o[dt][nt][1], acc_o[dt][nt][2], acc_o[dt][nt][3]);
        }
      }
    }
    if (!has_nu) break;
    // ---- switch to the next unit
    u += stride;
    if (!nu_staged) {  // this unit had no chunk to stage it behind
      fetch_ids(nu);
      stage_ids(nu);
      __syncthreads();
      count_chunks(nu);
    }
    cu = nu;
    // s_l, s_ext and the other s_ids buffer are next written after the next
    // unit's first chunk barrier; a unit without chunks has none, and would
    // write s_l while waves still read it for this unit's stores
    if (cu.nch == 0) lds_barrier();
    has_nu = u + stride < nunits;
    nu_staged = false;
    if (has_nu) nu = describe(u + stride, cu.sb ^ 1);
  }
}

// ---------------------------------------------------------------------------
// Short batches (decode): one workgroup per (query, 16-head tile, split).
// The split's slots are walked in chunks of kTileRows gathered rows; the four
// waves share the chunk's keys for S^T (32 keys each, the per-head max and sum
// exchanged through LDS) and the output dims for O^T.  Block b maps to
// (unit, tile) so that the head tiles of one unit have the same b mod 8 and
// therefore run on the same XCD, where the gathered rows are reused from L2.
// Partial outputs are 16 heads x c fp32 per split.
// ---------------------------------------------------------------------------
constexpr int kTileRows = 128;

// SEL (c = 512, one 128-slot chunk per split): the selection of eq 9 is
// finished here rather than by the top-k launch, which only classified each
// row's chunks (TopkLists::b1g1).  Every workgroup resolves its query's
// threshold from the published lists (the top-k's finishing phase, LDS taken
// from the row-tile buffer before any row is gathered) but keeps only the
// slots of its own split; the workgroups of head tile 0 also write those
// slots to idx_out / score_out, and the one of split 0 clears the query's
// level-1 histogram for the next call.  The query's heads are loaded first,
// so their round trip overlaps the selection.
template <int DTW, bool SEL>
__global__ __launch_bounds__(256) void mqa_tile_kernel(int nq, int nh, int k, int nht, int nsplit, int cps,
                                                       float scale_log2, const bf16_t* __restrict__ q,
                                                       const bf16_t* __restrict__ C,
                                                       const int32_t* __restrict__ q_seq,
                                                       const int64_t* __restrict__ kv_off,
                                                       const int32_t* __restrict__ idx,
                                                       bf16_t* __restrict__ o, float* __restrict__ lse,
                                                       float* __restrict__ part_o,
                                                       float* __restrict__ part_ml, TileSelect sel) {
  constexpr int CD = 64 * DTW;
  constexpr int CPITCH = CD + 16;  // rows staggered by 32 bytes: conflict-free 16-byte fragment reads
  constexpr int PPITCH = kTileRows + 16;
  constexpr int KSTEPS = CD / 32;
  __shared__ __attribute__((aligned(16))) bf16_t Cs[kTileRows * CPITCH];
  __shared__ __attribute__((aligned(16))) bf16_t Ps[16 * PPITCH];
  __shared__ int32_t s_rows[kTileRows];
  __shared__ float s_red[2][4][16];
  __shared__ __attribute__((aligned(16))) bf16_t s_q[16 * CPITCH];  // the tile's 16 query heads
  __shared__ int32_t s_win[SEL ? kTileRows : 1];                      // SEL: this split's selection slots

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int b = blockIdx.x;
  const int grp = b / (8 * nht);
  const int rem = b - grp * 8 * nht;
  const int ht = rem >> 3;
  const long u = (long)grp * 8 + (rem & 7);
  if (u >= (long)nq * nsplit) return;
  const long r = u / nsplit;
  const int j = (int)(u - r * nsplit);
  const int head = 16 * ht + c16;  // this lane's head (B-operand column, output column)
  const bool hlive = head < nh;
  const int seq = q_seq ? q_seq[r] : 0;
  const long off = kv_off ? kv_off[seq] : 0;

  // the first chunk's row ids are loaded before the query fragments: the
  // gather depends on them, the fragments are needed only after it (SEL:
  // every load the selection starts with -- the query's position, b1 and
  // g1, the chunk counts and the first list entries -- goes out first, in
  // one round trip)
  const int slot_first = (j * cps) * kTileRows + (kTileRows / 4) * wave + lane;
  int raw_first = 0;
  FinishPrefetch pf;
  long sel_pos = 0;
  uint32_t sel_b1 = 0, sel_g1 = 0;
  if constexpr (SEL) {
    const int P = sel.lists.P, gtc = sel.lists.gtc;
    finish_prefetch<256, false>(pf, P, sel.lists.counts + r * P * 2, sel.lists.gt + r * P * (long)gtc, gtc,
                                sel.lists.eq + r * P * (long)kMChunk, kMChunk);
    sel_pos = sel.q_pos[r];
    sel_b1 = sel.lists.b1g1[2 * r];
    sel_g1 = sel.lists.b1g1[2 * r + 1];
  } else {
    raw_first = idx[r * k + (slot_first < k ? slot_first : k - 1)];
  }
  // the tile's 16 query heads: each wave stages 4 of them in LDS (16-byte
  // pieces).  The pieces are loaded here but written to LDS only after the
  // first chunk's gather has been issued, so that their round trip overlaps
  // the gather's instead of preceding it.
  constexpr int QCH = CD / 8;
  constexpr int QN = (4 * QCH + 63) / 64;
  u32x4 qv[QN];
#pragma unroll
  for (int i = 0; i < QN; ++i) {
    const int v = lane + 64 * i;
    const int hl = 4 * wave + v / QCH, pc = (v % QCH) * 8;
    const int hh = 16 * ht + hl;
    qv[i] = load16_clamped(q + (r * nh + hh) * CD + pc, v < 4 * QCH && hh < nh, q);
  }
  if constexpr (SEL) {
    static_assert(sizeof(FinishSmem<256>) <= sizeof(Cs), "the selection's LDS lives in the row-tile buffer");
    const uint32_t s0 = (uint32_t)(j * kTileRows), s1 = (uint32_t)min(k, (j + 1) * kTileRows);
    const long pos = sel_pos;
    long ncl = pos > 0 ? pos / sel.m : 0;
    ncl = ncl < sel.max_cand ? ncl : sel.max_cand;
    if (tid < kTileRows) s_win[tid] = (ncl <= k && s0 + tid < (uint32_t)ncl) ? (int32_t)(s0 + tid) : -1;
    __syncthreads();
    if (ncl > k) {  // uniform: rows of at most k candidates keep all of them (the top-k launch wrote them out)
      const int P = sel.lists.P, gtc = sel.lists.gtc;
      const int Pr = (int)((ncl + kMChunk - 1) / kMChunk);
      const uint32_t b1 = sel_b1, g1 = sel_g1;
      FinishSmem<256>& fs = *reinterpret_cast<FinishSmem<256>*>(Cs);
      int32_t* out = sel.idx_out + r * k;
      float* sout = sel.score_out ? sel.score_out + r * k : nullptr;
      finish_row<256, false>(fs, pf, P, Pr, k, b1, g1, sel.lists.counts + r * P * 2, sel.lists.gt + r * P * (long)gtc, gtc,
                      sel.lists.eq + r * P * (long)kMChunk, kMChunk, s0, s1,
                      [&](uint32_t slot, uint32_t i, float sc) {
                        s_win[slot - s0] = (int32_t)i;
                        if (ht == 0) {
                          out[slot] = (int32_t)i;
                          if (sout) sout[slot] = sc;
                        }
                      });
      if (ht == 0 && j == 0) {  // every chunk workgroup of the top-k launch has read it
        u32x4* h = reinterpret_cast<u32x4*>(sel.lists.hist + r * kL1Bins);
        for (int b = tid; b < kL1Bins / 4; b += 256) h[b] = u32x4{0u, 0u, 0u, 0u};
      }
    }
    __syncthreads();  // s_win complete; the row-tile buffer is free again
    raw_first = s_win[lane < kTileRows / 4 ? (kTileRows / 4) * wave + lane : 0];
  }
  Frag<bf16_t> qf[KSTEPS];

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 acc_o[DTW];
#pragma unroll
  for (int dt = 0; dt < DTW; ++dt) acc_o[dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ch = 0; ch < cps; ++ch) {
    const int slot0 = (j * cps + ch) * kTileRows;
    if (slot0 >= k) break;  // uniform
    {
      constexpr int RPW = kTileRows / 4;  // rows gathered by each wave
      const int slot = slot0 + RPW * wave + lane;
      const int raw = ch == 0 ? raw_first : idx[r * k + (slot < k ? slot : k - 1)];  // always in bounds
      const int myid = (lane < RPW && slot < k) ? raw : -1;
      if (lane < RPW) s_rows[RPW * wave + lane] = myid;
      // one wave per SIMD here: all of a wave's rows are in flight at once
      wave_gather<bf16_t, CD, RPW, CPITCH, RPW>(C + off * CD, myid, Cs, RPW * wave, lane, q);
    }
    if (ch == 0) {
#pragma unroll
      for (int i = 0; i < QN; ++i) {
        const int v = lane + 64 * i;
        if (v < 4 * QCH) *reinterpret_cast<u32x4*>(&s_q[(4 * wave + v / QCH) * CPITCH + (v % QCH) * 8]) = qv[i];
      }
    }
    __syncthreads();

    if (ch == 0) {
#pragma unroll
      for (int kk = 0; kk < KSTEPS; ++kk) qf[kk].load(&s_q[c16 * CPITCH + 32 * kk + 8 * g]);
    }
    // S^T for keys 32*wave .. 32*wave+31 (two 16-key M tiles), this tile's 16 heads
    f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kk = 0; kk < KSTEPS; ++kk) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        Frag<bf16_t> ac;
        ac.load(&Cs[(32 * wave + 16 * t + c16) * CPITCH + 32 * kk + 8 * g]);
        mma(acc[t], ac, qf[kk]);
      }
    }
    float x[2][4];
    float cm = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = 32 * wave + 16 * t + 4 * g + rr;
        x[t][rr] = s_rows[key] >= 0 ? acc[t][rr] * scale_log2 : -INFINITY;
        cm = fmaxf(cm, x[t][rr]);
      }
    cm = wave_max_xor_16_32(cm);
    if (g == 0) s_red[0][wave][c16] = cm;
    __syncthreads();
    cm = fmaxf(fmaxf(s_red[0][0][c16], s_red[0][1][c16]), fmaxf(s_red[0][2][c16], s_red[0][3][c16]));
    const float m_new = fmaxf(m_run, cm);
    const bool none = (m_new == -INFINITY);
    const float alpha = none ? 1.f : exp2_fast(m_run - m_new);
    float ps = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const float p = none ? 0.f : exp2_fast(x[t][rr] - m_new);
        ps += p;
        Ps[c16 * PPITCH + 32 * wave + 16 * t + 4 * g + rr] = f2bf(p);
      }
    ps = wave_sum_xor_16_32(ps);
    if (g == 0) s_red[1][wave][c16] = ps;
    __syncthreads();
    l_run = l_run * alpha + (s_red[1][0][c16] + s_red[1][1][c16]) + (s_red[1][2][c16] + s_red[1][3][c16]);
    m_run = m_new;

    // O^T for dims tiles wave*DTW .. : C_sel^T (2-byte LDS reads) x P^T
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt) acc_o[dt] *= alpha;
#pragma unroll
    for (int kk = 0; kk < kTileRows / 32; ++kk) {
      Frag<bf16_t> bp;
      bp.load(&Ps[c16 * PPITCH + 32 * kk + 8 * g]);
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt) {
        const Frag<bf16_t> ac = frag_ct<bf16_t>(Cs, CPITCH, 32 * kk, (wave * DTW + dt) * 16, lane);
        mma(acc_o[dt], ac, bp);
      }
    }
    __syncthreads();
  }

  if (!hlive) return;
  if (nsplit == 1) {
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt) {
      float v[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) v[rr] = acc_o[dt][rr] * inv;
      store4<bf16_t>(o + (r * nh + head) * CD + (wave * DTW + dt) * 16 + 4 * g, v);
    }
    if (wave == 0 && g == 0 && lse)
      lse[r * nh + head] = (l_run > 0.f) ? (m_run + log2f(l_run)) * 0.6931471805599453f : -INFINITY;
  } else {
    // the split's output normalised by its own sum, in bf16 (half the bytes
    // of the raw fp32 accumulators; the merge weights it by l_run again)
    const long pb = u * nh + head;
    const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
    bf16_t* po = reinterpret_cast<bf16_t*>(part_o);
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt) {
      float v[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) v[rr] = acc_o[dt][rr] * inv;
      store4<bf16_t>(po + pb * CD + (wave * DTW + dt) * 16 + 4 * g, v);
    }
    if (wave == 0 && g == 0) {
      part_ml[pb * 2] = m_run;
      part_ml[pb * 2 + 1] = l_run;
    }
  }
}

// Partials PT: float = the splits' raw accumulators; bf16_t = each split's
// output already divided by its own sum.
template <typename T, typename PT>
__global__ __launch_bounds__(256) void mqa_combine_kernel(long nrows, int nh, int c, int nsplit,
                                                          const PT* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          T* __restrict__ o, float* __restrict__ lse) {
  constexpr int U = 8;  // splits whose loads are in flight together
  const int groups = c / 4;
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long rh = gid / groups;
  if (rh >= nrows * nh) return;
  const int d4 = (int)(gid - rh * groups) * 4;
  const long r = rh / nh;
  const int h = (int)(rh - r * nh);
  const long b0 = r * nsplit * (long)nh + h;  // split j at b0 + j*nh
  // Online merge, U splits per batch: every split's (m, l) and partial output
  // of a batch are loaded together (one memory round trip per batch).
  float M = -INFINITY;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  for (int j0 = 0; j0 < nsplit; j0 += U) {
    float2 ml[U];
    float4 po[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const long b = b0 + (long)(j0 + u < nsplit ? j0 + u : 0) * nh;  // always in bounds
      ml[u] = *reinterpret_cast<const float2*>(part_ml + b * 2);
      if constexpr (sizeof(PT) == 4) {
        po[u] = *reinterpret_cast<const float4*>(part_o + b * c + d4);
      } else {
        const uint2 w = *reinterpret_cast<const uint2*>(part_o + b * c + d4);
        po[u] = make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                            __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
      }
    }
    issue_fence();
    float mb = M;
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (j0 + u < nsplit) mb = fmaxf(mb, ml[u].x);
    if (mb == -INFINITY) continue;  // nothing valid yet
    const float a = M == -INFINITY ? 0.f : exp2_fast(M - mb);
    L *= a;
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] *= a;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const float wgt = (j0 + u >= nsplit || ml[u].x == -INFINITY) ? 0.f : exp2_fast(ml[u].x - mb);
      L = fmaf(ml[u].y, wgt, L);
      const float wo = sizeof(PT) == 4 ? wgt : wgt * ml[u].y;
      acc[0] = fmaf(wo, po[u].x, acc[0]);
      acc[1] = fmaf(wo, po[u].y, acc[1]);
      acc[2] = fmaf(wo, po[u].z, acc[2]);
      acc[3] = fmaf(wo, po[u].w, acc[3]);
    }
    M = mb;
  }
  const float inv = (M == -INFINITY) ? 0.f : 1.f / L;
  float v[4] = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
  store4<T>(o + rh * c + d4, v);
  if (d4 == 0 && lse) lse[rh] = (M == -INFINITY) ? -INFINITY : (M + log2f(L)) * 0.6931471805599453f;
}

// Compute units of the current device (queried once per device; threads
// that race on the first query store the same value).
int compute_units() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int q = 0;
    n = hipDeviceGetAttribute(&q, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && q > 0 ? q : 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

struct Plan {
  bool tile;    // short-batch kernel (16-head tiles) instead of the 64-head-group kernels
  bool group8;  // eight-wave double-buffered 64-head-group kernel (bf16, 128 <= c <= 512)
  int nhg, nchunks, nsplit, cps;
};

constexpr long kTargetWGs = 512;  // two workgroups per CU

// Large batches: one workgroup per (query, 64-head group), no split.  Short
// bf16 batches (decode) use the 16-head tile kernel and split each query's
// slots into as many 128-row chunks per workgroup as keeps about kTargetWGs
// workgroups busy.  Other short batches split the 64-head-group kernel.
Plan plan(long nq, int nh, int c, int k, bool bf16) {
  Plan p;
  const long base = nq * ((nh + kHG - 1) / kHG);
  p.tile = bf16 && c <= 512 && base < kTargetWGs;
  p.group8 = !p.tile && bf16 && c >= 128 && c <= 512;
  if (p.tile) {
    p.nhg = (nh + 15) / 16;
    p.nchunks = (k + kTileRows - 1) / kTileRows;
    const long units = nq * p.nhg;
    long ns = (kTargetWGs + units - 1) / units;
    if (ns > p.nchunks) ns = p.nchunks;
    if (ns < 1) ns = 1;
    p.cps = (int)((p.nchunks + ns - 1) / ns);
  } else {
    p.nhg = (nh + kHG - 1) / kHG;
    const int ks = p.group8 ? kG8Chunk : ((long)c * (bf16 ? 2 : 4) <= 1024 ? 64 : 32);  // group_chunk<T, c/64>()
    p.nchunks = (k + ks - 1) / ks;
    long ns = base >= kTargetWGs ? 1 : (kTargetWGs + base - 1) / base;
    if (ns > p.nchunks) ns = p.nchunks;
    p.cps = (int)((p.nchunks + ns - 1) / ns);
  }
  p.nsplit = (p.nchunks + p.cps - 1) / p.cps;
  return p;
}

template <typename T, int DTW>
hipError_t run(long nq, int nh, int k, float scale, const void* q, const void* C,
               const int32_t* q_seq, const int64_t* kv_off, const int32_t* idx, void* o,
               float* lse, float* part_o, float* part_ml, const TileSelect* sel, hipStream_t s) {
  const Plan p = plan(nq, nh, 64 * DTW, k, sizeof(T) == 2);
  hipError_t e = hipSuccess;
  bool done = false;
  if constexpr (sizeof(T) == 2 && DTW <= 8) {
    if (p.tile) {
      const long units = nq * p.nsplit;
      const unsigned blocks = (unsigned)(((units + 7) / 8) * 8 * p.nhg);
      if constexpr (DTW == 8) {
        if (sel)
          e = launch("mqa", mqa_tile_kernel<DTW, true>, dim3(blocks), dim3(256), 0, s, (int)nq, nh, k, p.nhg,
                     p.nsplit, p.cps, scale * kLog2e, (const bf16_t*)q, (const bf16_t*)C, q_seq, kv_off, idx,
                     (bf16_t*)o, lse, part_o, part_ml, *sel);
      }
      if (!sel)
        e = launch("mqa", mqa_tile_kernel<DTW, false>, dim3(blocks), dim3(256), 0, s, (int)nq, nh, k, p.nhg,
                   p.nsplit, p.cps, scale * kLog2e, (const bf16_t*)q, (const bf16_t*)C, q_seq, kv_off, idx,
                   (bf16_t*)o, lse, part_o, part_ml, TileSelect{});
      done = true;
    }
  }
  if constexpr (sizeof(T) == 2 && DTW >= 2 && DTW <= 8) {
    if (!done && p.group8 && DTW == 8 && (long)p.cps * kG8Chunk <= kStreamMaxStaged) {
      const long units = nq * p.nhg * p.nsplit;
      const long grid = std::min(units, (long)compute_units());
      e = launch("mqa", mqa_stream_kernel, dim3((unsigned)grid), dim3(512), 0, s, units, nh, k, p.nhg, p.nsplit,
                 p.cps, scale * kLog2e, (const bf16_t*)q, (const bf16_t*)C, q_seq, kv_off, idx, (bf16_t*)o, lse,
                 part_o, part_ml);
      done = true;
    }
    if (!done && p.group8) {
      e = launch("mqa", mqa_group8_kernel<DTW>, dim3((unsigned)(nq * p.nhg * p.nsplit)), dim3(512), 0, s, nh, k,
                 p.nhg, p.nsplit, p.cps, scale * kLog2e, (const bf16_t*)q, (const bf16_t*)C, q_seq, kv_off, idx,
                 (bf16_t*)o, lse, part_o, part_ml);
      done = true;
    }
  }
  if (!done)
    e = launch("mqa", mqa_kernel<T, DTW>, dim3((unsigned)(nq * p.nhg * p.nsplit)), dim3(256), 0, s, nh, k,
               p.nhg, p.nsplit, p.cps, scale * kLog2e, (const T*)q, (const T*)C, q_seq, kv_off, idx, (T*)o,
               lse, part_o, part_ml);
  if (e != hipSuccess || p.nsplit == 1) return e;
  const long threads = nq * nh * (64 * DTW / 4);
  const dim3 cgrid((unsigned)((threads + 255) / 256));
  if (p.tile)  // the tile kernel leaves normalised bf16 partials
    return launch("mqa_combine", mqa_combine_kernel<T, bf16_t>, cgrid, dim3(256), 0, s, nq, nh, 64 * DTW, p.nsplit,
                  (const bf16_t*)part_o, (const float*)part_ml, (T*)o, lse);
  return launch("mqa_combine", mqa_combine_kernel<T, float>, cgrid, dim3(256), 0, s, nq, nh, 64 * DTW, p.nsplit,
                (const float*)part_o, (const float*)part_ml, (T*)o, lse);
}

template <typename T>
hipError_t pick(long nq, int nh, int c, int k, float scale, const void* q, const void* C,
                const int32_t* q_seq, const int64_t* kv_off, const int32_t* idx, void* o, float* lse,
                float* part_o, float* part_ml, const TileSelect* sel, hipStream_t s) {
  switch (c / 64) {
    case 1: return run<T, 1>(nq, nh, k, scale, q, C, q_seq, kv_off, idx, o, lse, part_o, part_ml, sel, s);
    case 2: return run<T, 2>(nq, nh, k, scale, q, C, q_seq, kv_off, idx, o, lse, part_o, part_ml, sel, s);
    case 4: return run<T, 4>(nq, nh, k, scale, q, C, q_seq, kv_off, idx, o, lse, part_o, part_ml, sel, s);
    case 8: return run<T, 8>(nq, nh, k, scale, q, C, q_seq, kv_off, idx, o, lse, part_o, part_ml, sel, s);
    case 16: return run<T, 16>(nq, nh, k, scale, q, C, q_seq, kv_off, idx, o, lse, part_o, part_ml, sel, s);
    default: return hipErrorInvalidValue;
  }
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

bool mqa_supported_c(int c) { return c == 64 || c == 128 || c == 256 || c == 512 || c == 1024; }

// The attention finishes the selection when every split is one 128-row chunk
// and the whole grid runs in one round (the kernel's LDS allows one workgroup
// per CU): in a second round the finishing phase would be paid again, which
// measured slower than the top-k launch finishing the rows (32 queries x 4
// splits x 4 head tiles: attention 15.4 -> 23.4 us for 10.5 us less top-k).
bool mqa_tile_selects(long n_queries, int nh, int c, int k, bool bf16) {
  if (n_queries <= 0 || c != 512) return false;
  const Plan p = plan(n_queries, nh, c, k, bf16);
  if (!p.tile || p.cps != 1) return false;
  const long blocks = ((n_queries * p.nsplit + 7) / 8) * 8 * p.nhg;  // as launched
  return blocks <= compute_units();
}

size_t mqa_workspace_bytes(long n_queries, int nh, int c, int k, bool bf16) {
  if (n_queries <= 0) return 0;
  const Plan p = plan(n_queries, nh, c, k, bf16);
  if (p.nsplit == 1) return 0;
  return ws_add(ws_align(ws_bytes(n_queries, p.nsplit, (uint64_t)nh * c, sizeof(float))),
                ws_align(ws_bytes(n_queries, p.nsplit, (uint64_t)nh * 2, sizeof(float))));
}

hipError_t launch_mqa(csa_dtype dt, long n_queries, int nh, int c, int k, float scale,
                      const void* q, const void* C, const int32_t* q_seq,
                      const int64_t* kv_offset, const int32_t* idx, void* o, float* lse,
                      void* workspace, hipStream_t s, const TileSelect* sel) {
  if (n_queries == 0) return hipSuccess;
  const Plan p = plan(n_queries, nh, c, k, dt == CSA_BF16);
  if (sel && !mqa_tile_selects(n_queries, nh, c, k, dt == CSA_BF16)) return hipErrorInvalidValue;
  float* part_o = (float*)workspace;
  float* part_ml =
      p.nsplit == 1 ? nullptr
                    : (float*)((char*)workspace + align256((size_t)n_queries * p.nsplit * nh * c * sizeof(float)));
  if (dt == CSA_F32)
    return pick<float>(n_queries, nh, c, k, scale, q, C, q_seq, kv_offset, idx, o, lse, part_o, part_ml, sel, s);
  return pick<bf16_t>(n_queries, nh, c, k, scale, q, C, q_seq, kv_offset, idx, o, lse, part_o, part_ml, sel, s);
}

}  // namespace csa
