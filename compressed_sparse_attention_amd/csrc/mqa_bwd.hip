// Backward of the shared key-value MQA, eq 11 of "Compressed Sparse
// Attention" (section "Shared Key-Value MQA").  For query r, head h and its
// selected rows C_j (each both key and value), with P = softmax_j(scale q.C_j)
// recomputed from the forward's log-sum-exp and o the forward output:
//
//   dP_hj = dO_h . C_j,   D_h = dO_h . o_h,   dS_hj = P_hj (dP_hj - D_h),
//   dq_h  = scale sum_j dS_hj C_j,
//   dC_j  = sum_h P_hj dO_h + scale sum_h dS_hj q_h      (value + key paths).
//
// The key gradient of one compressed row collects a share from every query
// that selected it.  Global fp32 atomics for that scatter (n * k * c of them)
// would run about ten times longer than all of the arithmetic, so each
// query's shares are written as bf16 rows of a workspace instead (one
// 1 KiB row per (query, slot)), and the rows are summed per compressed entry
// afterwards: a counting sort of the (query, slot) pairs by entry, then a
// segmented sum over the sorted pairs.
//
// Main kernel: one workgroup of 8 waves per (query, 64-head group), c = 512,
// bf16.  q and dO stay resident for the whole sweep in the two layouts the
// products need: dims as the contraction axis for the scores (q and dO
// fragments in registers) and heads as the contraction axis for the key
// gradient (q^T fragments in registers, dO^T read from a swizzled LDS copy);
// dq accumulates in registers.  The selection is walked in chunks of 32 slots
// whose rows are gathered straight into LDS (asm-issued global_load_lds, one
// chunk ahead, double buffered; each chunk waits for its rows once).  Per chunk:
//   A. S^T and dP^T [32 keys x 16 heads] per wave, the 512 dims split in two
//      halves between wave pairs (partial sums exchanged through LDS);
//   B. P and dS (the softmax is the forward's: exp(scale q.C - lse));
//   C. dq^T += C_sel^T dS^T  (dims x heads, contraction over the 32 keys);
//   D. dC_sel^T = [dO; q]^T [P; scale dS]  (dims x keys, contraction over
//      the 128 head slots), stored as the chunk's 32 bf16 share rows at the
//      top of the next chunk (so that the stores drain during a whole chunk).
#include "common.hpp"
#include "internal.hpp"

namespace csa {
namespace {

// s_waitcnt vmcnt(1): every vector memory operation of this wave except the
// newest one has completed (the counter drains in issue order).
__device__ __forceinline__ void wait_vm_all_but_one() { __builtin_amdgcn_s_waitcnt(0x0F71); }

constexpr int kBwdCD = 512;             // c
constexpr int kBwdHeads = 64;           // heads per workgroup
constexpr int kBwdChunk = 32;           // selection slots per chunk
constexpr int kBwdPitch = kBwdCD + 8;   // padded LDS row of gathered rows / staged q, dO (a 32-byte
                                        // stagger would read faster but leaves no room in 160 KiB of LDS)
constexpr int kBwdWPitch = 128 + 8;     // row of [P | scale dS] for one key
constexpr int kBwdSPitch = kBwdChunk + 8;  // row of dS for one head (32 keys)

struct BwdLoop {
  bf16_t C[2][kBwdChunk * kBwdPitch];
  f32x4 xch[4][2][2][64];  // partial S / dP exchange: [head tile][key tile][S | dP][lane], 16 bytes per lane
  bf16_t W[kBwdChunk * kBwdWPitch];
  bf16_t dS[kBwdHeads * kBwdSPitch];
};
union BwdSmem {
  bf16_t X[kBwdHeads * kBwdPitch];  // prologue: q, then dO, of the 64 heads
  BwdLoop loop;
};

__device__ __forceinline__ void store4_bf16(bf16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(pack_bf16x2(a, b), pack_bf16x2(c, d));
}

// dO of the 64 heads stays in LDS for the whole sweep in the swizzled
// 512-column row layout of swz512_at (no padding).  (A rotation of each row
// by two chunks reads fragments faster in isolation but made this kernel
// 4% slower.)

__global__ __launch_bounds__(512) void mqa_bwd_kernel(int nh, int k, int nhg, float scale, const bf16_t* __restrict__ q,
                                                      const bf16_t* __restrict__ C, const int32_t* __restrict__ q_seq,
                                                      const int64_t* __restrict__ kv_off,
                                                      const int32_t* __restrict__ idx, const bf16_t* __restrict__ o,
                                                      const float* __restrict__ lse, const bf16_t* __restrict__ dO,
                                                      bf16_t* __restrict__ dq, bf16_t* __restrict__ part, long q0,
                                                      long nqc) {
  constexpr int CD = kBwdCD, P = kBwdPitch, KC = kBwdChunk;
  __shared__ __attribute__((aligned(16))) BwdSmem sm;
  __shared__ __attribute__((aligned(16))) bf16_t s_dO[kBwdHeads * kBwdCD];
  __shared__ float s_D[kBwdHeads], s_lse2[kBwdHeads];
  __shared__ __attribute__((aligned(16))) int32_t s_ids[3][KC];  // slot ids of chunks ch - 1, ch, ch + 1 (by ch mod 3)
  __shared__ int s_ext[2][8];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: selects on it stay scalar
  const int g = lane >> 4, c16 = lane & 15;
  const long rl = blockIdx.x / nhg;  // query within this call's chunk of queries
  const int hg = (int)(blockIdx.x - rl * nhg);
  const long r = q0 + rl;
  const int h0 = hg * kBwdHeads;
  const int NT = min(4, (nh - h0 + 15) / 16);  // live 16-head tiles
  const int seq = q_seq ? q_seq[r] : 0;
  const long off = kv_off ? kv_off[seq] : 0;
  const bf16_t* Cb = C + off * CD;
  const float scale_log2 = scale * kLog2e;

  // ---- prologue: q and dO into registers (through LDS), D and lse per head.
  // Every load of the query's state goes out first, together (the slot ids
  // for the chunk count, q, dO and o): one memory round trip, not three.
  const int ht = wave & 3, half = wave >> 2;  // phase A: head tile, dims half
  Frag<bf16_t> qB[8], dB[8];                  // [16 heads of tile ht] x [256 dims of half], by 32-dim step
  Frag<bf16_t> xA[4][2];                      // [16 dims] x [32 heads] of q^T: the wave's dims tiles (dO^T: from LDS)
  const int id0 = idx[r * k + (tid < k ? tid : 0)];
  u32x4 vq[8], vd[8], vo[8];                  // piece tid + 512 i: head 8i + wave, dims 8 lane .. 8 lane + 7
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int head = 8 * i + wave;
    const bool live = h0 + head < nh;
    const long base = ((long)r * nh + h0 + head) * CD + 8 * lane;
    vq[i] = load16_clamped(q + base, live, q);
    vd[i] = load16_clamped(dO + base, live, dO);
    vo[i] = load16_clamped(o + base, live, o);
  }
  issue_fence();

  // Chunks to walk: when the valid slots form a prefix (the selector pads
  // with -1 at the end), chunks past it are skipped.
  int first_bad = 0x7FFFFFFF, last_good = -1;
  if (tid < k) {
    if (id0 < 0) first_bad = tid; else last_good = tid;
  }
  for (int sl = tid + 512; sl < k; sl += 512) {
    const int id = idx[r * k + sl];
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

  float dsum[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int head = 8 * i + wave;
    const bool live = h0 + head < nh;
    *reinterpret_cast<u32x4*>(&sm.X[head * P + 8 * lane]) = live ? vq[i] : u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(&s_dO[swz512_at(head, 8 * lane)]) = live ? vd[i] : u32x4{0u, 0u, 0u, 0u};
    dsum[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      dsum[i] = fmaf(__uint_as_float(vd[i][j] << 16), __uint_as_float(vo[i][j] << 16), dsum[i]);
      dsum[i] = fmaf(__uint_as_float(vd[i][j] & 0xFFFF0000u), __uint_as_float(vo[i][j] & 0xFFFF0000u), dsum[i]);
    }
    dsum[i] = live ? dsum[i] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float x = dsum[i];
#pragma unroll
    for (int sh = 1; sh < 64; sh <<= 1) x += __shfl_xor(x, sh);
    if (lane == 0) s_D[8 * i + wave] = x;
  }
  if (tid < kBwdHeads)
    s_lse2[tid] = h0 + tid < nh ? lse[(long)r * nh + h0 + tid] * kLog2e : INFINITY;  // dead heads: P = 0
  __syncthreads();
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) qB[kk].load(&sm.X[(16 * ht + c16) * P + 256 * half + 32 * kk + 8 * g]);
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) xA[dt][h2] = frag_ct<bf16_t>(sm.X, P, 32 * h2, 64 * wave + 16 * dt, lane);
#pragma unroll
  for (int kk = 0; kk < 8; ++kk) dB[kk].load(&s_dO[swz512_at(16 * ht + c16, 256 * half + 32 * kk + 8 * g)]);
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    first_bad = min(first_bad, s_ext[0][w]);
    last_good = max(last_good, s_ext[1][w]);
  }
  __syncthreads();  // q's staging area is the loop's row buffer
  const int nch = last_good < first_bad ? (last_good + KC) / KC : (k + KC - 1) / KC;

  // Gather of chunk ch into buffer b: wave w brings slots 4w .. 4w+3, one
  // 1 KiB row per instruction (lane l's 16 bytes land at row offset 16 l).
  // The slot ids come from `ids` (lane j < 4: slot 4w + j of the chunk),
  // loaded one chunk ahead so that no gather waits for its own id.
  // (always one load instruction: the id load is the newest vector memory
  // operation of a chunk, which the wait at the top of the next chunk counts
  // on).  The raw value is kept as loaded (slots past k are masked when the
  // ids are used) so that nothing waits for the load where it is issued.
  auto load_ids = [&](int ch) -> int {
    const int sl = min(ch, nch - 1) * KC + 4 * wave + (lane & 3);
    return idx[r * k + min(sl, k - 1)];
  };
  auto gather = [&](int ch, int raw) {
    const int ids = ch * KC + 4 * wave + (lane & 3) < k ? raw : -1;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int id = __builtin_amdgcn_readlane(ids, j);
      const bf16_t* row = id >= 0 ? Cb + (long)id * CD : q;  // -1: finite filler, weight 0
      const uint32_t base = (uint32_t)(size_t)(lds_char*)&sm.loop.C[ch & 1][(4 * wave + j) * P];
      gather_row_lds(row + 8 * lane, __builtin_amdgcn_readfirstlane(base));
    }
    if (lane < 4) s_ids[ch % 3][4 * wave + lane] = ids;
  };

  // D: the key-gradient shares of chunk pc (from its [P | scale dS] rows in
  // LDS), 16 keys at a time, stored as bf16 rows of the workspace.
  auto shares = [&](int pc) {
    const int* ids = s_ids[pc % 3];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x4 acc[4];
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        Frag<bf16_t> b;
        b.load(&sm.loop.W[(16 * kt + c16) * kBwdWPitch + 32 * kk + 8 * g]);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          if (kk < 2) mma(acc[dt], frag_ct_swz512(s_dO, 32 * kk, 64 * wave + 16 * dt, lane), b);
          else mma(acc[dt], xA[dt][kk - 2], b);
        }
      }
      if (ids[16 * kt + c16] >= 0) {
        const int slot = pc * KC + 16 * kt + c16;
        bf16_t* dst = part + (((long)hg * nqc + rl) * k + slot) * CD + 64 * wave + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) store4_bf16(dst + 16 * dt, acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
      }
    }
  };

  f32x4 acc_dq[4][4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc_dq[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  int ids_next = 0;
  if (nch > 0) {
    const int ids0 = load_ids(0);
    gather(0, ids0);
    ids_next = load_ids(1);
  }
  // Chunk ch starts by issuing the gather of chunk ch + 1, then computes and
  // stores the shares of chunk ch - 1: those writes then have a whole chunk of
  // work to drain before the next wait for this wave's memory operations (the
  // gathers share that counter), and the id load of chunk ch + 2 comes last.
  for (int ch = 0; ch < nch; ++ch) {
    const int cur = ch & 1, sid = ch % 3;
    // this wave's gathers of chunk ch and the share stores issued after them
    // have completed; only the id load issued last may be pending
    wait_vm_all_but_one();
    lds_barrier();
    if (ch + 1 < nch) gather(ch + 1, ids_next);
    // the two waves of a SIMD (w, w + 4) take the share products and phase
    // A in opposite orders, so their LDS and MFMA use interleave
    if (ch > 0 && half == 0) shares(ch - 1);
    if (ch + 1 < nch) ids_next = load_ids(ch + 2);
    const bf16_t* Cs = sm.loop.C[cur];

    // ---- A: partial S^T, dP^T over this wave's 256 dims, both key tiles
    f32x4 as[2], ad[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      as[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
      ad[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        Frag<bf16_t> a;
        a.load(&Cs[(16 * kt + c16) * P + 256 * half + 32 * kk + 8 * g]);
        mma(as[kt], a, qB[kk]);
        mma(ad[kt], a, dB[kk]);
      }
    }
    // the partner wave (same head tile, other half) finishes key tile 1 - half
    {
      sm.loop.xch[ht][1 - half][0][lane] = half ? as[0] : as[1];
      sm.loop.xch[ht][1 - half][1][lane] = half ? ad[0] : ad[1];
    }
    if (ch > 0 && half == 1) shares(ch - 1);
    lds_barrier();
    // ---- B: P and dS for key tile `half`, heads of tile ht
    {
      const f32x4 xs = sm.loop.xch[ht][half][0][lane], xd = sm.loop.xch[ht][half][1][lane];
      const int hl = 16 * ht + c16;
      const float l2 = s_lse2[hl], Dh = s_D[hl];
      const int4 ids4 = *reinterpret_cast<const int4*>(&s_ids[sid][16 * half + 4 * g]);  // this lane's 4 keys
      float dsv[4];
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int key = 16 * half + 4 * g + rr;
        const float sv = (half ? as[1][rr] : as[0][rr]) + xs[rr];
        const float dp = (half ? ad[1][rr] : ad[0][rr]) + xd[rr];
        const float p = (rr == 0 ? ids4.x : rr == 1 ? ids4.y : rr == 2 ? ids4.z : ids4.w) >= 0 ? exp2_fast(sv * scale_log2 - l2) : 0.f;
        dsv[rr] = p * (dp - Dh);
        sm.loop.W[key * kBwdWPitch + hl] = f2bf(p);
        sm.loop.W[key * kBwdWPitch + 64 + hl] = f2bf(scale * dsv[rr]);
      }
      store4_bf16(&sm.loop.dS[hl * kBwdSPitch + 16 * half + 4 * g], dsv[0], dsv[1], dsv[2], dsv[3]);
    }
    lds_barrier();
    // ---- C: dq^T += C_sel^T dS^T  (wave's 64 dims x 64 heads, 32 keys)
    {
      Frag<bf16_t> bs[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) bs[nt].load(&sm.loop.dS[(16 * nt + c16) * kBwdSPitch + 8 * g]);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const Frag<bf16_t> a = frag_ct<bf16_t>(Cs, P, 0, 64 * wave + 16 * dt, lane);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
          if (nt < NT) mma(acc_dq[dt][nt], a, bs[nt]);
      }
    }
  }

  if (nch > 0) {
    __syncthreads();  // the last chunk's [P | scale dS] rows are complete
    shares(nch - 1);
  }

  // ---- dq = scale * acc  (lane: head 16 nt + c16, dims 4g .. 4g+3 of each tile)
#pragma unroll
  for (int nt = 0; nt < 4; ++nt) {
    const int head = h0 + 16 * nt + c16;
    if (nt < NT && head < nh) {
      bf16_t* dst = dq + ((long)r * nh + head) * CD + 64 * wave + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
        store4_bf16(dst + 16 * dt, scale * acc_dq[dt][nt][0], scale * acc_dq[dt][nt][1], scale * acc_dq[dt][nt][2],
                    scale * acc_dq[dt][nt][3]);
    }
  }
}

// ---------------------------------------------------------------------------
// Sum of the share rows per compressed entry.
// ---------------------------------------------------------------------------
__device__ __forceinline__ long entry_of(int r, int id, const int32_t* q_seq, const int64_t* kv_off) {
  return (kv_off ? kv_off[q_seq ? q_seq[r] : 0] : 0) + id;
}

// cnt[e] = number of (query, slot) pairs of queries q0 .. q0+nqc-1 that select entry e
__global__ __launch_bounds__(256) void pair_count_kernel(long nqc, int k, long q0, long rows,
                                                         const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ q_seq,
                                                         const int64_t* __restrict__ kv_off, int32_t* __restrict__ cnt) {
  const long p = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= nqc * k) return;
  const long r = q0 + p / k;
  const int id = idx[q0 * k + p];
  if (id < 0) return;
  const long e = entry_of((int)r, id, q_seq, kv_off);
  if (e < rows) atomicAdd(&cnt[e], 1);
}

// start[e] = sum_{e' < e} cnt[e'] (e = 0 .. rows; start[rows] = number of pairs), cursor = start
__global__ __launch_bounds__(1024) void pair_scan_kernel(long rows, const int32_t* __restrict__ cnt,
                                                         int32_t* __restrict__ start, int32_t* __restrict__ cursor) {
  __shared__ int32_t s_part[1024];
  const int t = threadIdx.x;
  const long per = (rows + 1023) / 1024;
  const long lo = t * per, hi = min(rows, lo + per);
  int32_t sum = 0;
  for (long e = lo; e < hi; ++e) sum += cnt[e];
  s_part[t] = sum;
  __syncthreads();
  for (int d = 1; d < 1024; d <<= 1) {  // inclusive scan of the per-thread sums
    const int32_t v = t >= d ? s_part[t - d] : 0;
    __syncthreads();
    s_part[t] += v;
    __syncthreads();
  }
  int32_t run = s_part[t] - sum;
  for (long e = lo; e < hi; ++e) {
    start[e] = run;
    cursor[e] = run;
    run += cnt[e];
  }
  if (t == 1023) start[rows] = s_part[1023];
}

// pairs grouped by entry: pair[pos] = local query * k + slot, pkey[pos] = entry
__global__ __launch_bounds__(256) void pair_fill_kernel(long nqc, int k, long q0, long rows,
                                                        const int32_t* __restrict__ idx,
                                                        const int32_t* __restrict__ q_seq,
                                                        const int64_t* __restrict__ kv_off,
                                                        int32_t* __restrict__ cursor, int32_t* __restrict__ pair,
                                                        int32_t* __restrict__ pkey) {
  const long p = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (p >= nqc * k) return;
  const long r = q0 + p / k;
  const int id = idx[q0 * k + p];
  if (id < 0) return;
  const long e = entry_of((int)r, id, q_seq, kv_off);
  if (e >= rows) return;
  const int pos = atomicAdd(&cursor[e], 1);
  pair[pos] = (int32_t)p;
  pkey[pos] = (int32_t)e;
}

// The same two steps with the counting done in LDS first (entries < kLdsRows):
// a workgroup histograms kPairsPerWG pairs in LDS and adds each nonzero bin
// to the global count once, so a popular entry (early blocks are selected
// by almost every query) takes one global atomic per workgroup instead of
// one per query.  The fill reserves each bin's run in the entry's list with
// one global atomic and hands out positions inside it with LDS atomics.
constexpr int kLdsRows = 16384;
constexpr int kPairsPerWG = 32768;

template <bool FILL>
__global__ __launch_bounds__(1024) void pair_bins_kernel(long nqc, int k, long q0, long rows,
                                                         const int32_t* __restrict__ idx,
                                                         const int32_t* __restrict__ q_seq,
                                                         const int64_t* __restrict__ kv_off,
                                                         int32_t* __restrict__ cnt_or_cursor,
                                                         int32_t* __restrict__ pair, int32_t* __restrict__ pkey) {
  __shared__ int32_t s_bin[kLdsRows];
  const int t = threadIdx.x;
  const long total = nqc * k;
  const long p0 = (long)blockIdx.x * kPairsPerWG, p1 = min(total, p0 + kPairsPerWG);
  for (long e = t; e < rows; e += 1024) s_bin[e] = 0;
  __syncthreads();
  for (long p = p0 + t; p < p1; p += 1024) {
    const int id = idx[q0 * k + p];
    if (id < 0) continue;
    const long e = entry_of((int)(q0 + p / k), id, q_seq, kv_off);
    if (e < rows) atomicAdd(&s_bin[e], 1);
  }
  __syncthreads();
  for (long e = t; e < rows; e += 1024) {
    const int c = s_bin[e];
    if (c == 0) continue;
    const int base = atomicAdd(&cnt_or_cursor[e], c);
    if (FILL) s_bin[e] = base;
  }
  if (!FILL) return;
  __syncthreads();
  for (long p = p0 + t; p < p1; p += 1024) {
    const int id = idx[q0 * k + p];
    if (id < 0) continue;
    const long e = entry_of((int)(q0 + p / k), id, q_seq, kv_off);
    if (e >= rows) continue;
    const int pos = atomicAdd(&s_bin[e], 1);
    pair[pos] = (int32_t)p;
    pkey[pos] = (int32_t)e;
  }
}

// One wave per segment of kSegPairs consecutive sorted pairs: lane l sums
// dims 8l .. 8l+7 of the share rows of each entry in the segment (over all
// head groups) and adds the sum into dC (fp32) when the entry changes, so an
// entry gets one atomic add per segment it spans.
constexpr int kSegPairs = 512;
constexpr int kSegBatch = 8;

__global__ __launch_bounds__(256) void share_reduce_kernel(int k, int nhg, long nqc, const int32_t* __restrict__ start,
                                                           long rows, const int32_t* __restrict__ pair,
                                                           const int32_t* __restrict__ pkey,
                                                           const bf16_t* __restrict__ part, float* __restrict__ dC) {
  const int lane = threadIdx.x & 63;
  const long seg = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long total = start[rows];
  const long p0 = seg * kSegPairs;
  if (p0 >= total) return;
  const long p1 = min(total, p0 + kSegPairs);
  const long hstride = nqc * k * kBwdCD;
  float acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = 0.f;
  int cur = pkey[p0];
  auto flush = [&](int e) {
    float* d = dC + (long)e * kBwdCD + 8 * lane;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      unsafeAtomicAdd(d + j, acc[j]);
      acc[j] = 0.f;
    }
  };
  for (long p = p0; p < p1; p += kSegBatch) {
    u32x4 v[kSegBatch];
    int key[kSegBatch];
#pragma unroll
    for (int u = 0; u < kSegBatch; ++u) {
      const long pp = min(p + u, p1 - 1);
      key[u] = pkey[pp];
      v[u] = *reinterpret_cast<const u32x4*>(part + (long)pair[pp] * kBwdCD + 8 * lane);
    }
#pragma unroll
    for (int u = 0; u < kSegBatch; ++u) {
      if (p + u >= p1) break;
      if (key[u] != cur) {
        flush(cur);
        cur = key[u];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[2 * j] += __uint_as_float(v[u][j] << 16);
        acc[2 * j + 1] += __uint_as_float(v[u][j] & 0xFFFF0000u);
      }
      for (int h = 1; h < nhg; ++h) {  // the other head groups' shares of the same pair
        const u32x4 w = *reinterpret_cast<const u32x4*>(part + h * hstride + (long)pair[p + u] * kBwdCD + 8 * lane);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] += __uint_as_float(w[j] << 16);
          acc[2 * j + 1] += __uint_as_float(w[j] & 0xFFFF0000u);
        }
      }
    }
  }
  flush(cur);
}

__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* __restrict__ p, long n) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x) p[i] = 0u;
}

constexpr long kMaxPairsPerPass = 2L << 20;  // share rows held at once (2 GiB of bf16 at c = 512)

struct BwdLayout {
  long qc;  // queries per pass
  size_t part, cnt, start, cursor, pair, pkey, total;
};


BwdLayout bwd_layout(long nq, int nh, int k, long rows) {
  BwdLayout L;
  const long nhg = (nh + kBwdHeads - 1) / kBwdHeads;
  L.qc = std::max(1L, std::min(nq, kMaxPairsPerPass / ((long)k * nhg)));
  const size_t pairs = ws_bytes(L.qc, k);
  const size_t row_words = ws_align(ws_bytes(rows + 1, sizeof(int32_t)));
  L.part = 0;
  L.cnt = ws_align(ws_bytes(pairs, nhg, kBwdCD, sizeof(bf16_t)));
  L.start = ws_add(L.cnt, row_words);
  L.cursor = ws_add(L.start, row_words);
  L.pair = ws_add(L.cursor, row_words);
  L.pkey = ws_add(L.pair, ws_align(ws_bytes(pairs, sizeof(int32_t))));
  L.total = ws_add(L.pkey, ws_align(ws_bytes(pairs, sizeof(int32_t))));
  return L;
}

hipError_t zero_words(void* p, long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const long blocks = std::min(4096L, (n + 255) / 256);
  return launch("mqa_bwd_zero", zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint32_t*)p, n);
}

}  // namespace

size_t mqa_backward_workspace_bytes(long n_queries, int nh, int k, long rows) {
  if (n_queries <= 0) return 0;
  return bwd_layout(n_queries, nh, k, rows).total;
}

hipError_t launch_mqa_backward(long nq, int nh, int k, float scale, const void* q, const void* C, long rows,
                               const int32_t* q_seq, const int64_t* kv_off, const int32_t* idx, const void* o,
                               const float* lse, const void* dO, void* dq, float* dC, void* workspace,
                               hipStream_t s) {
  hipError_t e = zero_words(dC, rows * kBwdCD, s);
  if (e != hipSuccess || nq == 0) return e;
  const BwdLayout L = bwd_layout(nq, nh, k, rows);
  char* ws = (char*)workspace;
  bf16_t* part = (bf16_t*)(ws + L.part);
  int32_t* cnt = (int32_t*)(ws + L.cnt);
  int32_t* start = (int32_t*)(ws + L.start);
  int32_t* cursor = (int32_t*)(ws + L.cursor);
  int32_t* pair = (int32_t*)(ws + L.pair);
  int32_t* pkey = (int32_t*)(ws + L.pkey);
  const int nhg = (nh + kBwdHeads - 1) / kBwdHeads;
  for (long q0 = 0; q0 < nq; q0 += L.qc) {
    const long nqc = std::min(L.qc, nq - q0);
    e = launch("mqa_bwd", mqa_bwd_kernel, dim3((unsigned)(nqc * nhg)), dim3(512), 0, s, nh, k, nhg, scale,
               (const bf16_t*)q, (const bf16_t*)C, q_seq, kv_off, idx, (const bf16_t*)o, lse, (const bf16_t*)dO,
               (bf16_t*)dq, part, q0, nqc);
    if (e != hipSuccess) return e;
    if (rows == 0) continue;
    e = zero_words(cnt, rows, s);
    if (e != hipSuccess) return e;
    const bool lds_bins = rows <= kLdsRows;
    const unsigned pblocks = (unsigned)((nqc * k + 255) / 256);
    const unsigned bblocks = (unsigned)((nqc * k + kPairsPerWG - 1) / kPairsPerWG);
    e = lds_bins ? launch("mqa_bwd_sort", pair_bins_kernel<false>, dim3(bblocks), dim3(1024), 0, s, nqc, k, q0, rows,
                          idx, q_seq, kv_off, cnt, (int32_t*)nullptr, (int32_t*)nullptr)
                 : launch("mqa_bwd_sort", pair_count_kernel, dim3(pblocks), dim3(256), 0, s, nqc, k, q0, rows, idx,
                          q_seq, kv_off, cnt);
    if (e != hipSuccess) return e;
    e = launch("mqa_bwd_sort", pair_scan_kernel, dim3(1), dim3(1024), 0, s, rows, (const int32_t*)cnt, start, cursor);
    if (e != hipSuccess) return e;
    e = lds_bins ? launch("mqa_bwd_sort", pair_bins_kernel<true>, dim3(bblocks), dim3(1024), 0, s, nqc, k, q0, rows,
                          idx, q_seq, kv_off, cursor, pair, pkey)
                 : launch("mqa_bwd_sort", pair_fill_kernel, dim3(pblocks), dim3(256), 0, s, nqc, k, q0, rows, idx,
                          q_seq, kv_off, cursor, pair, pkey);
    if (e != hipSuccess) return e;
    const long segs = (nqc * k + kSegPairs - 1) / kSegPairs;
    e = launch("mqa_bwd_reduce", share_reduce_kernel, dim3((unsigned)((segs + 3) / 4)), dim3(256), 0, s, k, nhg, nqc,
               (const int32_t*)start, rows, (const int32_t*)pair, (const int32_t*)pkey, (const bf16_t*)part, dC);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace csa
