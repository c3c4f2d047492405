// Softmax-gated overlapping compression, eqs 3-4 of "Compressed Sparse
// Attention" (section "Compressed Key-Value Entries"), for one sequence, for
// several packed sequences (each compressed on its own, blocks never span two
// sequences), and the decode-time append.
//
// One thread owns one block i and V adjacent channels.  It streams the 2m
// (logit, value) pairs of its block -- rows m*i .. m*i+m-1 of Z^a/C^a and,
// for i > 0, rows m*(i-1) .. m*i-1 of Z^b/C^b -- through an online softmax
// held in registers (running max, denominator and weighted sum, one exp per
// pair), so any m works and nothing is staged.  Adjacent threads own
// adjacent channel groups, so each row is read as one contiguous run.  Every
// projected row is read exactly twice overall (once as an a-row, once as a
// b-row of the next block), which is the minimum the overlap allows.
#include "common.hpp"
#include "internal.hpp"

namespace csa {
namespace {

template <typename T, int V> struct Vec;
template <> struct Vec<bf16_t, 8> {
  static __device__ __forceinline__ void load(const bf16_t* p, float* o) {
    const u32x4 u = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(u[i] << 16);
      o[2 * i + 1] = __uint_as_float(u[i] & 0xFFFF0000u);
    }
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* v) {
    u32x4 u;
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = (uint32_t)f2bf(v[2 * i]) | ((uint32_t)f2bf(v[2 * i + 1]) << 16);
    *reinterpret_cast<u32x4*>(p) = u;
  }
};
template <> struct Vec<bf16_t, 4> {
  static __device__ __forceinline__ void load(const bf16_t* p, float* o) {
    const uint2 u = *reinterpret_cast<const uint2*>(p);
    o[0] = __uint_as_float(u.x << 16);
    o[1] = __uint_as_float(u.x & 0xFFFF0000u);
    o[2] = __uint_as_float(u.y << 16);
    o[3] = __uint_as_float(u.y & 0xFFFF0000u);
  }
  static __device__ __forceinline__ void store(bf16_t* p, const float* v) {
    uint2 u;
    u.x = (uint32_t)f2bf(v[0]) | ((uint32_t)f2bf(v[1]) << 16);
    u.y = (uint32_t)f2bf(v[2]) | ((uint32_t)f2bf(v[3]) << 16);
    *reinterpret_cast<uint2*>(p) = u;
  }
};
template <> struct Vec<float, 4> {
  static __device__ __forceinline__ void load(const float* p, float* o) {
    const float4 u = *reinterpret_cast<const float4*>(p);
    o[0] = u.x; o[1] = u.y; o[2] = u.z; o[3] = u.w;
  }
  static __device__ __forceinline__ void store(float* p, const float* v) {
    *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  }
};

template <typename T, int V>
__global__ __launch_bounds__(256) void compress_kernel(long nblk, int m, int c,
                                                       const T* __restrict__ Ca,
                                                       const T* __restrict__ Cb,
                                                       const T* __restrict__ Za,
                                                       const T* __restrict__ Zb, long ld,
                                                       const T* __restrict__ Ba,
                                                       const T* __restrict__ Bb, T* __restrict__ out,
                                                       long ldo, int nseq, const int64_t* __restrict__ cu,
                                                       const int64_t* __restrict__ boff) {
  const int groups = c / V;
  const long gid = (long)blockIdx.x * blockDim.x + threadIdx.x;
  const long i = gid / groups;  // output row
  if (i >= nblk) return;
  const int ch = (int)(gid - i * groups) * V;
  // Several sequences (cu set): output row i is block il of the sequence b
  // with boff[b] <= i < boff[b+1]; that sequence's tokens start at row cu[b]
  // of the projections, and its block 0 has no b-terms.
  long il = i, rbase = 0;
  if (cu != nullptr) {
    int lo = 0, hi = nseq - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (boff[mid] <= i) lo = mid; else hi = mid - 1;
    }
    il = i - boff[lo];
    rbase = cu[lo];
  }

  float mx[V], den[V], acc[V];
  // Online softmax over the 2m pairs; logits are carried in log2 units.
  auto absorb = [&](const T* zrow, const T* crow, const T* brow, bool first) {
    float z[V], v[V], b[V];
    Vec<T, V>::load(zrow, z);
    Vec<T, V>::load(crow, v);
    Vec<T, V>::load(brow, b);
#pragma unroll
    for (int q = 0; q < V; ++q) {
      const float l = (z[q] + b[q]) * kLog2e;
      if (first) {
        mx[q] = l;
        den[q] = 1.f;
        acc[q] = v[q];
      } else {
        const float d = l - mx[q];
        const float e = exp2_fast(-fabsf(d));
        const bool up = d > 0.f;
        acc[q] = up ? fmaf(acc[q], e, v[q]) : fmaf(e, v[q], acc[q]);
        den[q] = up ? fmaf(den[q], e, 1.f) : den[q] + e;
        mx[q] = up ? l : mx[q];
      }
    }
  };

  for (int r = 0; r < m; ++r) {
    const long row = rbase + il * m + r;
    absorb(Za + row * ld + ch, Ca + row * ld + ch, Ba + (long)r * c + ch, r == 0);
  }
  if (il > 0) {
    for (int r = 0; r < m; ++r) {
      const long row = rbase + (il - 1) * m + r;
      absorb(Zb + row * ld + ch, Cb + row * ld + ch, Bb + (long)r * c + ch, false);
    }
  }
  float res[V];
#pragma unroll
  for (int q = 0; q < V; ++q) res[q] = acc[q] / den[q];
  Vec<T, V>::store(out + i * ldo + ch, res);
}

// ---------------------------------------------------------------------------
// Decode-time append: one new token per sequence.  Workgroup b stores the new
// projected row [C^a | C^b | Z^a | Z^b] of sequence b in its 2m-row ring (slot
// t mod 2m) and, when the token completes block i = floor(t/m), compresses
// block i from the ring (a-terms: block i's rows, b-terms: block i-1's rows,
// absent for i = 0) into row kv_offset[b] + i of the compressed cache; each
// thread owns V channels of it.
// ---------------------------------------------------------------------------
template <typename T, int V>
__global__ __launch_bounds__(256) void compress_append_kernel(int m, int c, const T* __restrict__ rows, long ld_new,
                                                              T* __restrict__ ring, const T* __restrict__ Ba,
                                                              const T* __restrict__ Bb,
                                                              const int64_t* __restrict__ t_new,
                                                              const int64_t* __restrict__ kv_off,
                                                              T* __restrict__ out, long ldo) {
  const long b = blockIdx.x;
  const long t = t_new[b];
  const int W4 = 4 * c;  // ring row: C^a | C^b | Z^a | Z^b
  T* rb = ring + b * (long)(2 * m) * W4;
  const T* src = rows + b * ld_new;
  T* dst = rb + (t % (2 * m)) * W4;
  for (int e = threadIdx.x * V; e < W4; e += blockDim.x * V) {
    float v[V];
    Vec<T, V>::load(src + e, v);
    Vec<T, V>::store(dst + e, v);
  }
  if (t % m != m - 1) return;  // the token does not complete a block (uniform)
  __syncthreads();             // the new row is in the ring for every thread
  const long i = t / m;
  for (int ch = threadIdx.x * V; ch < c; ch += blockDim.x * V) {
    float mx[V], den[V], acc[V];
    auto absorb = [&](const T* rrow, const T* brow, int zoff, int coff, bool first) {
      float z[V], v[V], bb[V];
      Vec<T, V>::load(rrow + zoff + ch, z);
      Vec<T, V>::load(rrow + coff + ch, v);
      Vec<T, V>::load(brow, bb);
#pragma unroll
      for (int q = 0; q < V; ++q) {
        const float l = (z[q] + bb[q]) * kLog2e;
        if (first) {
          mx[q] = l;
          den[q] = 1.f;
          acc[q] = v[q];
        } else {
          const float d = l - mx[q];
          const float e = exp2_fast(-fabsf(d));
          const bool up = d > 0.f;
          acc[q] = up ? fmaf(acc[q], e, v[q]) : fmaf(e, v[q], acc[q]);
          den[q] = up ? fmaf(den[q], e, 1.f) : den[q] + e;
          mx[q] = up ? l : mx[q];
        }
      }
    };
    for (int r = 0; r < m; ++r)  // block i: C^a (offset 0), Z^a (offset 2c)
      absorb(rb + ((i * m + r) % (2 * m)) * W4, Ba + (long)r * c + ch, 2 * c, 0, r == 0);
    if (i > 0)
      for (int r = 0; r < m; ++r)  // block i-1: C^b (offset c), Z^b (offset 3c)
        absorb(rb + (((i - 1) * m + r) % (2 * m)) * W4, Bb + (long)r * c + ch, 3 * c, c, false);
    float res[V];
#pragma unroll
    for (int q = 0; q < V; ++q) res[q] = acc[q] / den[q];
    Vec<T, V>::store(out + (kv_off[b] + i) * ldo + ch, res);
  }
}

template <typename T, int V>
hipError_t run(long nblk, int m, int c, const void* Ca, const void* Cb, const void* Za,
               const void* Zb, long ld, const void* Ba, const void* Bb, void* out, long ldo,
               int nseq, const int64_t* cu, const int64_t* boff, hipStream_t s) {
  const long threads = nblk * (c / V);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  return launch("compress", compress_kernel<T, V>, dim3(blocks), dim3(256), 0, s, nblk, m, c, (const T*)Ca,
                (const T*)Cb, (const T*)Za, (const T*)Zb, ld, (const T*)Ba, (const T*)Bb, (T*)out, ldo, nseq, cu,
                boff);
}

hipError_t dispatch(csa_dtype dt, long nblk, int m, int c, const void* Ca, const void* Cb, const void* Za,
                    const void* Zb, long ld_in, const void* Ba, const void* Bb, void* out, long ld_out, int nseq,
                    const int64_t* cu, const int64_t* boff, hipStream_t s) {
  if (nblk == 0) return hipSuccess;
  if (dt == CSA_F32)
    return run<float, 4>(nblk, m, c, Ca, Cb, Za, Zb, ld_in, Ba, Bb, out, ld_out, nseq, cu, boff, s);
  if (c % 8 == 0 && ld_in % 8 == 0 && ld_out % 8 == 0)
    return run<bf16_t, 8>(nblk, m, c, Ca, Cb, Za, Zb, ld_in, Ba, Bb, out, ld_out, nseq, cu, boff, s);
  return run<bf16_t, 4>(nblk, m, c, Ca, Cb, Za, Zb, ld_in, Ba, Bb, out, ld_out, nseq, cu, boff, s);
}

}  // namespace

hipError_t launch_compress(csa_dtype dt, long n, int m, int c, const void* Ca, const void* Cb,
                           const void* Za, const void* Zb, long ld_in, const void* Ba,
                           const void* Bb, void* out, long ld_out, hipStream_t s) {
  return dispatch(dt, n / m, m, c, Ca, Cb, Za, Zb, ld_in, Ba, Bb, out, ld_out, 0, nullptr, nullptr, s);
}

hipError_t launch_compress_varlen(csa_dtype dt, long nseq, int m, int c, const void* Ca, const void* Cb,
                                  const void* Za, const void* Zb, long ld_in, const void* Ba, const void* Bb,
                                  const int64_t* cu, const int64_t* boff, long nblk, void* out, long ld_out,
                                  hipStream_t s) {
  if (nseq == 0) return hipSuccess;
  return dispatch(dt, nblk, m, c, Ca, Cb, Za, Zb, ld_in, Ba, Bb, out, ld_out, (int)nseq, cu, boff, s);
}

hipError_t launch_compress_append(csa_dtype dt, long B, int m, int c, const void* rows, long ld_new, void* ring,
                                  const void* Ba, const void* Bb, const int64_t* t_new, const int64_t* kv_off,
                                  void* out, long ld_out, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const dim3 grid((unsigned)B);
  if (dt == CSA_F32)
    return launch("compress_append", compress_append_kernel<float, 4>, grid, dim3(256), 0, s, m, c,
                  (const float*)rows, ld_new, (float*)ring, (const float*)Ba, (const float*)Bb, t_new, kv_off,
                  (float*)out, ld_out);
  if (c % 8 == 0 && ld_new % 8 == 0 && ld_out % 8 == 0)
    return launch("compress_append", compress_append_kernel<bf16_t, 8>, grid, dim3(256), 0, s, m, c,
                  (const bf16_t*)rows, ld_new, (bf16_t*)ring, (const bf16_t*)Ba, (const bf16_t*)Bb, t_new, kv_off,
                  (bf16_t*)out, ld_out);
  return launch("compress_append", compress_append_kernel<bf16_t, 4>, grid, dim3(256), 0, s, m, c,
                (const bf16_t*)rows, ld_new, (bf16_t*)ring, (const bf16_t*)Ba, (const bf16_t*)Bb, t_new, kv_off,
                (bf16_t*)out, ld_out);
}

}  // namespace csa
