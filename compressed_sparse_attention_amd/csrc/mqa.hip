// Shared key-value MQA, eq 11 of "Compressed Sparse Attention" (section
// "Shared Key-Value MQA"): every selected compressed entry C_s is both the key
// and the value of all n_h query heads of its token,
//
//   o[r, h] = sum_s softmax_s(scale * q[r, h] . C_s) C_s.
//
// A workgroup owns one query, one group of up to 64 heads and a contiguous
// range of its selection slots, which it walks in chunks of kKS slots with an
// online softmax.  Per chunk it gathers the kKS selected rows of C^Comp ONCE
// into LDS and serves every head of the group from there (one read of a
// selected entry for all heads: the point of a shared key-value MQA):
//   * S^T = C_sel . q^T on MFMA, keys as M (rows read from LDS with 16-byte
//     reads), heads as N (query fragments straight from global memory).  The
//     accumulator holds one head per lane column, so the per-head max and sum
//     over keys are in-lane plus two cross-lane steps;
//   * P = exp2(S*scale*log2e - running max) goes to LDS as [head][key], with
//     each head's rescale factor for the running output;
//   * O^T = C_sel^T . P^T on MFMA, output dims as M split across the 4 waves,
//     heads as N.  The C^T operand is read from the same LDS rows with 2-byte
//     reads (8 per fragment); P^T is one 16-byte read.
// With one split per query the workgroup normalises and writes o and lse
// itself.  Short batches (decode) split the slots across workgroups to fill
// the GPU; each split then writes its unnormalised output and (max, sum) per
// head, and the combine kernel merges the splits by log-sum-exp.
#include "common.hpp"
#include "internal.hpp"

namespace csa {
namespace {

constexpr int kKS = 32;  // selection slots per split
constexpr int kHG = 64;  // heads per pass (4 waves x 16)

template <typename T> __device__ __forceinline__ void frag_set(Frag<T>& f, int j, T v);
template <> __device__ __forceinline__ void frag_set<bf16_t>(Frag<bf16_t>& f, int j, bf16_t v) {
  f.v[j] = __builtin_bit_cast(__bf16, v);
}
template <> __device__ __forceinline__ void frag_set<float>(Frag<float>& f, int j, float v) {
  f.f[j] = v;
}

template <typename T> __device__ __forceinline__ void store4(T* p, const float* v);
template <> __device__ __forceinline__ void store4<float>(float* p, const float* v) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}
template <> __device__ __forceinline__ void store4<bf16_t>(bf16_t* p, const float* v) {
  uint2 u;
  u.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
  u.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
  *reinterpret_cast<uint2*>(p) = u;
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
  constexpr int VEC = 16 / sizeof(T);
  constexpr int CPITCH = CD + VEC;
  constexpr int PPITCH = kKS + VEC;
  constexpr int CHUNKS = CD / VEC;
  __shared__ __attribute__((aligned(16))) T Cs[kKS * CPITCH];
  __shared__ __attribute__((aligned(16))) T Ps[kHG * PPITCH];
  __shared__ int32_t s_rows[kKS];
  __shared__ float s_alpha[kHG];
  __shared__ float s_l[kHG];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
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

  f32x4 acc_o[DTW][4];
#pragma unroll
  for (int dt = 0; dt < DTW; ++dt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc_o[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int ch = 0; ch < cps; ++ch) {
    const int slot0 = (j * cps + ch) * kKS;
    if (slot0 >= k) break;  // uniform across the workgroup
    if (tid < kKS) {
      const int slot = slot0 + tid;
      s_rows[tid] = slot < k ? idx[r * k + slot] : -1;
    }
    __syncthreads();
    for (int v = tid; v < kKS * CHUNKS; v += 256) {
      const int key = v / CHUNKS;
      const int cc = (v - key * CHUNKS) * VEC;
      const int id = s_rows[key];
      u32x4 val = {0u, 0u, 0u, 0u};
      if (id >= 0) val = *reinterpret_cast<const u32x4*>(C + (off + id) * CD + cc);
      *reinterpret_cast<u32x4*>(&Cs[key * CPITCH + cc]) = val;
    }
    __syncthreads();

    if (qwave) {
      f32x4 acc[kKS / 16];
#pragma unroll
      for (int mt = 0; mt < kKS / 16; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const T* qrow = q + (r * nh + qhead) * CD + 8 * g;
#pragma unroll 4
      for (int kk = 0; kk < CD / 32; ++kk) {
        Frag<T> bq;
        if (qhead < nh)
          bq.load(qrow + 32 * kk);
        else
          bq.zero();
#pragma unroll
        for (int mt = 0; mt < kKS / 16; ++mt) {
          Frag<T> ac;
          ac.load(&Cs[(16 * mt + c16) * CPITCH + 32 * kk + 8 * g]);
          mma(acc[mt], ac, bq);
        }
      }
      float x[kKS / 16][4];
      float cm = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < kKS / 16; ++mt)
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
      for (int mt = 0; mt < kKS / 16; ++mt)
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
    for (int kk = 0; kk < kKS / 32; ++kk) {
      Frag<T> bp[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)
        if (nt < NT) bp[nt].load(&Ps[(16 * nt + c16) * PPITCH + 32 * kk + 8 * g]);
#pragma unroll
      for (int dt = 0; dt < DTW; ++dt) {
        Frag<T> ac;
        const int dim = (wave * DTW + dt) * 16 + c16;
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) frag_set<T>(ac, jj, Cs[(32 * kk + 8 * g + jj) * CPITCH + dim]);
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

template <typename T>
__global__ __launch_bounds__(256) void mqa_combine_kernel(long nrows, int nh, int c, int nsplit,
                                                          const float* __restrict__ part_o,
                                                          const float* __restrict__ part_ml,
                                                          T* __restrict__ o, float* __restrict__ lse) {
  const int groups = c / 4;
  const long gid = (long)blockIdx.x * 256 + threadIdx.x;
  const long rh = gid / groups;
  if (rh >= nrows * nh) return;
  const int d4 = (int)(gid - rh * groups) * 4;
  const long r = rh / nh;
  const int h = (int)(rh - r * nh);
  float M = -INFINITY;
  for (int j = 0; j < nsplit; ++j) M = fmaxf(M, part_ml[((r * nsplit + j) * nh + h) * 2]);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  float L = 0.f;
  if (M != -INFINITY) {
    for (int j = 0; j < nsplit; ++j) {
      const long b = (r * nsplit + j) * nh + h;
      const float mj = part_ml[b * 2];
      if (mj == -INFINITY) continue;
      const float wgt = exp2_fast(mj - M);
      L = fmaf(part_ml[b * 2 + 1], wgt, L);
      const float4 po = *reinterpret_cast<const float4*>(part_o + b * c + d4);
      acc[0] = fmaf(wgt, po.x, acc[0]);
      acc[1] = fmaf(wgt, po.y, acc[1]);
      acc[2] = fmaf(wgt, po.z, acc[2]);
      acc[3] = fmaf(wgt, po.w, acc[3]);
    }
  }
  const float inv = (M == -INFINITY) ? 0.f : 1.f / L;
  T* dst = o + rh * c + d4;
#pragma unroll
  for (int q = 0; q < 4; ++q) dst[q] = from_f32<T>(acc[q] * inv);
  if (d4 == 0 && lse) lse[rh] = (M == -INFINITY) ? -INFINITY : (M + log2f(L)) * 0.6931471805599453f;
}

struct Plan {
  int nhg, nchunks, nsplit, cps;
};

// Splits of the selection per (query, head group): enough workgroups to cover
// the GPU twice over when the batch alone does not.
Plan plan(long nq, int nh, int k) {
  Plan p;
  p.nhg = (nh + kHG - 1) / kHG;
  p.nchunks = (k + kKS - 1) / kKS;
  const long base = nq * p.nhg;
  const long target = 512;
  long ns = base >= target ? 1 : (target + base - 1) / base;
  if (ns > p.nchunks) ns = p.nchunks;
  p.cps = (int)((p.nchunks + ns - 1) / ns);
  p.nsplit = (p.nchunks + p.cps - 1) / p.cps;
  return p;
}

template <typename T, int DTW>
hipError_t run(long nq, int nh, int k, float scale, const void* q, const void* C,
               const int32_t* q_seq, const int64_t* kv_off, const int32_t* idx, void* o,
               float* lse, float* part_o, float* part_ml, hipStream_t s) {
  const Plan p = plan(nq, nh, k);
  {
    TimedScope t("mqa", s);
    hipLaunchKernelGGL((mqa_kernel<T, DTW>), dim3((unsigned)(nq * p.nhg * p.nsplit)), dim3(256), 0, s,
                       nh, k, p.nhg, p.nsplit, p.cps, scale * kLog2e, (const T*)q, (const T*)C, q_seq,
                       kv_off, idx, (T*)o, lse, part_o, part_ml);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.nsplit == 1) return e;
  const long threads = nq * nh * (64 * DTW / 4);
  {
    TimedScope t("mqa_combine", s);
    hipLaunchKernelGGL((mqa_combine_kernel<T>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       s, nq, nh, 64 * DTW, p.nsplit, part_o, part_ml, (T*)o, lse);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t pick(long nq, int nh, int c, int k, float scale, const void* q, const void* C,
                const int32_t* q_seq, const int64_t* kv_off, const int32_t* idx, void* o, float* lse,
                float* part_o, float* part_ml, hipStream_t s) {
  switch (c / 64) {
    case 1: return run<T, 1>(nq, nh, k, scale, q, C, q_seq, kv_off, idx, o, lse, part_o, part_ml, s);
    case 2: return run<T, 2>(nq, nh, k, scale, q, C, q_seq, kv_off, idx, o, lse, part_o, part_ml, s);
    case 4: return run<T, 4>(nq, nh, k, scale, q, C, q_seq, kv_off, idx, o, lse, part_o, part_ml, s);
    case 8: return run<T, 8>(nq, nh, k, scale, q, C, q_seq, kv_off, idx, o, lse, part_o, part_ml, s);
    case 16: return run<T, 16>(nq, nh, k, scale, q, C, q_seq, kv_off, idx, o, lse, part_o, part_ml, s);
    default: return hipErrorInvalidValue;
  }
}

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

bool mqa_supported_c(int c) { return c == 64 || c == 128 || c == 256 || c == 512 || c == 1024; }

size_t mqa_workspace_bytes(long n_queries, int nh, int c, int k) {
  const Plan p = plan(n_queries, nh, k);
  if (p.nsplit == 1) return 0;
  return align256((size_t)n_queries * p.nsplit * nh * c * sizeof(float)) +
         align256((size_t)n_queries * p.nsplit * nh * 2 * sizeof(float));
}

hipError_t launch_mqa(csa_dtype dt, long n_queries, int nh, int c, int k, float scale,
                      const void* q, const void* C, const int32_t* q_seq,
                      const int64_t* kv_offset, const int32_t* idx, void* o, float* lse,
                      void* workspace, hipStream_t s) {
  if (n_queries == 0) return hipSuccess;
  const Plan p = plan(n_queries, nh, k);
  float* part_o = (float*)workspace;
  float* part_ml =
      p.nsplit == 1 ? nullptr
                    : (float*)((char*)workspace + align256((size_t)n_queries * p.nsplit * nh * c * sizeof(float)));
  if (dt == CSA_F32)
    return pick<float>(n_queries, nh, c, k, scale, q, C, q_seq, kv_offset, idx, o, lse, part_o, part_ml, s);
  return pick<bf16_t>(n_queries, nh, c, k, scale, q, C, q_seq, kv_offset, idx, o, lse, part_o, part_ml, s);
}

}  // namespace csa
