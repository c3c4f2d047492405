// Shared key-value MQA, eq 11 of "Compressed Sparse Attention" (section
// "Shared Key-Value MQA"): every selected compressed entry C_s is both the key
// and the value of all n_h query heads of its token,
//
//   o[r, h] = sum_s softmax_s(scale * q[r, h] . C_s) C_s.
//
// Split kernel: a workgroup takes one query and kKS consecutive slots of its
// selection.  It gathers those kKS rows of C^Comp ONCE into LDS and serves
// all heads from there (the defining property of MQA here: one read of a
// selected entry for every head).  Per 64-head group:
//   * S^T = C_sel . q^T on MFMA, keys as M (rows read from LDS with 16-byte
//     reads), heads as N (query fragments straight from global memory).  The
//     accumulator holds one head per lane column, so the per-head max and sum
//     over keys are in-lane plus two cross-lane steps;
//   * P = exp2(S*scale*log2e - max) goes to LDS as [head][key];
//   * O^T = C_sel^T . P^T on MFMA, output dims as M split across the 4 waves,
//     heads as N.  The C^T operand is read from the same LDS rows with 2-byte
//     reads (8 per fragment); P^T is one 16-byte read.
// The split writes unnormalised partial outputs plus (max, sum) per head; the
// combine kernel merges splits by log-sum-exp and normalises.
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

template <typename T, int DTW>
__global__ __launch_bounds__(256) void mqa_split_kernel(int nh, int k, int nsplit, float scale_log2,
                                                        const T* __restrict__ q,
                                                        const T* __restrict__ C,
                                                        const int32_t* __restrict__ q_seq,
                                                        const int64_t* __restrict__ kv_off,
                                                        const int32_t* __restrict__ idx,
                                                        float* __restrict__ part_o,
                                                        float* __restrict__ part_ml) {
  constexpr int CD = 64 * DTW;  // head dim c
  constexpr int VEC = 16 / sizeof(T);
  constexpr int CPITCH = CD + VEC;
  constexpr int PPITCH = kKS + VEC;
  constexpr int CHUNKS = CD / VEC;
  __shared__ __attribute__((aligned(16))) T Cs[kKS * CPITCH];
  __shared__ __attribute__((aligned(16))) T Ps[kHG * PPITCH];
  __shared__ int32_t s_rows[kKS];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int g = lane >> 4, c16 = lane & 15;
  const long r = blockIdx.x / nsplit;
  const int j = blockIdx.x - (int)(r * nsplit);
  const int seq = q_seq ? q_seq[r] : 0;
  const long off = kv_off ? kv_off[seq] : 0;

  if (tid < kKS) {
    const int slot = j * kKS + tid;
    s_rows[tid] = slot < k ? idx[r * k + slot] : -1;
  }
  __syncthreads();
  for (int v = tid; v < kKS * CHUNKS; v += 256) {
    const int key = v / CHUNKS;
    const int ch = (v - key * CHUNKS) * VEC;
    const int id = s_rows[key];
    u32x4 val = {0u, 0u, 0u, 0u};
    if (id >= 0) val = *reinterpret_cast<const u32x4*>(C + (off + id) * CD + ch);
    *reinterpret_cast<u32x4*>(&Cs[key * CPITCH + ch]) = val;
  }
  __syncthreads();

  const long pbase = (r * nsplit + j) * (long)nh;
  for (int h0 = 0; h0 < nh; h0 += kHG) {
    const int hbase = h0 + 16 * wave;
    if (hbase < nh) {
      const int head = hbase + c16;
      f32x4 acc[kKS / 16];
#pragma unroll
      for (int mt = 0; mt < kKS / 16; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const T* qrow = q + (r * nh + head) * CD + 8 * g;
#pragma unroll 4
      for (int kk = 0; kk < CD / 32; ++kk) {
        Frag<T> bq;
        if (head < nh)
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
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < kKS / 16; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int key = 16 * mt + 4 * g + rr;
          x[mt][rr] = s_rows[key] >= 0 ? acc[mt][rr] * scale_log2 : -INFINITY;
          mx = fmaxf(mx, x[mt][rr]);
        }
      mx = wave_max_xor_16_32(mx);
      float sum = 0.f;
#pragma unroll
      for (int mt = 0; mt < kKS / 16; ++mt)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const float p = (mx == -INFINITY) ? 0.f : exp2_fast(x[mt][rr] - mx);
          sum += p;
          Ps[(16 * wave + c16) * PPITCH + 16 * mt + 4 * g + rr] = from_f32<T>(p);
        }
      sum = wave_sum_xor_16_32(sum);
      if (g == 0 && head < nh) {
        part_ml[(pbase + head) * 2] = mx;
        part_ml[(pbase + head) * 2 + 1] = sum;
      }
    }
    __syncthreads();

    const int NT = min(4, (nh - h0 + 15) / 16);
    f32x4 o[DTW][4];
#pragma unroll
    for (int dt = 0; dt < DTW; ++dt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) o[dt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
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
          if (nt < NT) mma(o[dt][nt], ac, bp[nt]);
      }
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int head = h0 + 16 * nt + c16;
      if (nt < NT && head < nh) {
#pragma unroll
        for (int dt = 0; dt < DTW; ++dt) {
          float* dst = part_o + (pbase + head) * CD + (wave * DTW + dt) * 16 + 4 * g;
          *reinterpret_cast<float4*>(dst) = make_float4(o[dt][nt][0], o[dt][nt][1], o[dt][nt][2], o[dt][nt][3]);
        }
      }
    }
    __syncthreads();
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

template <typename T, int DTW>
hipError_t run(long nq, int nh, int k, float scale, const void* q, const void* C,
               const int32_t* q_seq, const int64_t* kv_off, const int32_t* idx, void* o,
               float* lse, float* part_o, float* part_ml, hipStream_t s) {
  const int nsplit = (k + kKS - 1) / kKS;
  {
    TimedScope t("mqa_split", s);
    hipLaunchKernelGGL((mqa_split_kernel<T, DTW>), dim3((unsigned)(nq * nsplit)), dim3(256), 0, s,
                       nh, k, nsplit, scale * kLog2e, (const T*)q, (const T*)C, q_seq, kv_off, idx,
                       part_o, part_ml);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long threads = nq * nh * (64 * DTW / 4);
  {
    TimedScope t("mqa_combine", s);
    hipLaunchKernelGGL((mqa_combine_kernel<T>), dim3((unsigned)((threads + 255) / 256)), dim3(256), 0,
                       s, nq, nh, 64 * DTW, nsplit, part_o, part_ml, (T*)o, lse);
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
  const long nsplit = (k + kKS - 1) / kKS;
  return align256((size_t)n_queries * nsplit * nh * c * sizeof(float)) +
         align256((size_t)n_queries * nsplit * nh * 2 * sizeof(float));
}

hipError_t launch_mqa(csa_dtype dt, long n_queries, int nh, int c, int k, float scale,
                      const void* q, const void* C, const int32_t* q_seq,
                      const int64_t* kv_offset, const int32_t* idx, void* o, float* lse,
                      void* workspace, hipStream_t s) {
  if (n_queries == 0) return hipSuccess;
  const long nsplit = (k + kKS - 1) / kKS;
  float* part_o = (float*)workspace;
  float* part_ml = (float*)((char*)workspace + align256((size_t)n_queries * nsplit * nh * c * sizeof(float)));
  if (dt == CSA_F32)
    return pick<float>(n_queries, nh, c, k, scale, q, C, q_seq, kv_offset, idx, o, lse, part_o, part_ml, s);
  return pick<bf16_t>(n_queries, nh, c, k, scale, q, C, q_seq, kv_offset, idx, o, lse, part_o, part_ml, s);
}

}  // namespace csa
