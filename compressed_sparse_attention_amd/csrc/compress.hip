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

#include <algorithm>

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
template <typename T>
struct AppendArgs {
  int c;
  const T* rows;
  long ld_new;
  T* ring;
  const T* Ba;
  const T* Bb;
  T* out;
  long ldo;
};

template <typename T, int V>
__device__ __forceinline__ void append_one(int m, const AppendArgs<T>& p, long b, const int64_t* __restrict__ t_new,
                                           const int64_t* __restrict__ kv_off) {
  const int c = p.c;
  const T* __restrict__ rows = p.rows;
  const long ld_new = p.ld_new;
  T* __restrict__ ring = p.ring;
  const T* __restrict__ Ba = p.Ba;
  const T* __restrict__ Bb = p.Bb;
  T* __restrict__ out = p.out;
  const long ldo = p.ldo;
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
__global__ __launch_bounds__(256) void compress_append_kernel(int m, AppendArgs<T> p, const int64_t* __restrict__ t_new,
                                                              const int64_t* __restrict__ kv_off) {
  append_one<T, V>(m, p, blockIdx.x, t_new, kv_off);
}

// Two caches of the same sequences (the main and the indexer cache) in one
// launch: workgroups below B append to the first, the others to the second.
template <typename T, int V>
__global__ __launch_bounds__(256) void compress_append_pair_kernel(int m, long B, AppendArgs<T> p1, AppendArgs<T> p2,
                                                                   const int64_t* __restrict__ t_new,
                                                                   const int64_t* __restrict__ kv_off) {
  const long b = blockIdx.x;
  if (b < B)
    append_one<T, V>(m, p1, b, t_new, kv_off);
  else
    append_one<T, V>(m, p2, b - B, t_new, kv_off);
}

// ---------------------------------------------------------------------------
// Backward of eqs 3-4.  For block i and channel j, with S_r the softmax
// weights of the 2m pairs (v_r, l_r) and out = sum_r S_r v_r:
//
//   dv_r = S_r * dout,   dl_r = S_r * dout * (v_r - out),
//
// and the logit l_r = Z_r + B_r passes dl_r to both Z_r and B_r.  A projected
// row is an a-row of exactly one block and a b-row of exactly one other, so
// each element of dC^a, dZ^a (from its own block) and dC^b, dZ^b (from the
// next block) is written once, by the thread that owns that block: no
// accumulation.  The bias gradients sum dl over all blocks: each workgroup
// adds its blocks' terms in LDS and writes one partial row set, and a second
// kernel sums the partials in a fixed order (deterministic).
//
// Thread mapping: lane l of every wave owns channels V*(64*blockIdx.x + l)
// .. +V-1 (one contiguous run per row for the wave); the 8 waves of a
// workgroup take the blocks of its range in turn.  The extra block index N
// (one past the last block) stands for the rows no block reads: the a-rows
// past N*m and the b-rows past (N-1)*m get zero gradients.
// ---------------------------------------------------------------------------
constexpr int kBwdWaves = 8;
constexpr int kBwdRowGroup = 8;  // rows loaded together: all 2m rows of a block when m <= 4

// V elements of a row as loaded (bf16 kept packed), converted on use.
template <typename T, int V> struct Raw {
  static constexpr int W = V * (int)sizeof(T) / 4;
  uint32_t w[W];
  __device__ __forceinline__ void load(const T* p) {
    if constexpr (W == 4) {
      const u32x4 u = *reinterpret_cast<const u32x4*>(p);
      w[0] = u[0]; w[1] = u[1]; w[2] = u[2]; w[3] = u[3];
    } else {
      const uint2 u = *reinterpret_cast<const uint2*>(p);
      w[0] = u.x; w[1] = u.y;
    }
  }
  __device__ __forceinline__ float at(int q) const {
    if constexpr (sizeof(T) == 4) return __uint_as_float(w[q]);
    else return __uint_as_float((q & 1) ? (w[q >> 1] & 0xFFFF0000u) : (w[q >> 1] << 16));
  }
};

template <typename T, int V>
__global__ __launch_bounds__(64 * kBwdWaves) void compress_bwd_kernel(
    long N, long n, int m, int c, const T* __restrict__ Ca, const T* __restrict__ Cb, const T* __restrict__ Za,
    const T* __restrict__ Zb, long ld, const T* __restrict__ Ba, const T* __restrict__ Bb,
    const float* __restrict__ dC, long ldd, T* __restrict__ dCa, T* __restrict__ dCb, T* __restrict__ dZa,
    T* __restrict__ dZb, long ldo, long bpw, float* __restrict__ part, int nseq, const int64_t* __restrict__ cu,
    const int64_t* __restrict__ boff) {
  extern __shared__ float s_db[];  // [2m][64 V]: bias-gradient sums of this workgroup's blocks
  constexpr int G = kBwdRowGroup;
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = 64 * V;
  const int ch = (blockIdx.x * 64 + lane) * V;
  const bool live = ch < c;
  for (int e = tid; e < 2 * m * W; e += 64 * kBwdWaves) s_db[e] = 0.f;
  __syncthreads();

  // Units 0 .. N-1 are the blocks; then one tail unit per sequence (one in all
  // without cu) writes zeros to the rows that no block reads.
  const long units = N + (cu != nullptr ? nseq : 1);
  const long i0 = (long)blockIdx.y * bpw, i1 = min(i0 + bpw, units);
  for (long i = i0 + wave; live && i < i1; i += kBwdWaves) {
    long il = i, rbase = 0;  // block index within its sequence, the sequence's first token row
    if (i >= N) {
      long len = n;
      if (cu != nullptr) {
        rbase = cu[i - N];
        len = cu[i - N + 1] - rbase;
      }
      const long nb = len / m, end = rbase + len;
      const float zero[V] = {};
      for (long row = rbase + nb * m; row < end; ++row) {
        Vec<T, V>::store(dCa + row * ldo + ch, zero);
        Vec<T, V>::store(dZa + row * ldo + ch, zero);
      }
      for (long row = rbase + (nb > 0 ? (nb - 1) * m : 0); row < end; ++row) {
        Vec<T, V>::store(dCb + row * ldo + ch, zero);
        Vec<T, V>::store(dZb + row * ldo + ch, zero);
      }
      continue;
    }
    if (cu != nullptr) {  // block i is block il of the sequence b with boff[b] <= i < boff[b+1]
      int lo = 0, hi = nseq - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (boff[mid] <= i) lo = mid; else hi = mid - 1;
      }
      il = i - boff[lo];
      rbase = cu[lo];
    }
    // Pair p < m is a-row p of block i; pair m + r is b-row r (a row of block i-1).
    const int npairs = il > 0 ? 2 * m : m;
    auto row_of = [&](int p) -> long { return rbase + (p < m ? il * m + p : (il - 1) * m + (p - m)); };
    Raw<T, V> z[G], v[G], b[G];
    auto load_group = [&](int p0) {
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int p = min(p0 + u, npairs - 1);  // past the end: a repeat, never used
        const long row = row_of(p);
        const bool is_a = p < m;
        z[u].load((is_a ? Za : Zb) + row * ld + ch);
        v[u].load((is_a ? Ca : Cb) + row * ld + ch);
        b[u].load((is_a ? Ba : Bb) + (long)(is_a ? p : p - m) * c + ch);
      }
    };
    // pass 1: max (log2 units), denominator and weighted sum, as the forward
    float mx[V], den[V], acc[V];
    for (int p0 = 0; p0 < npairs; p0 += G) {
      load_group(p0);
#pragma unroll
      for (int u = 0; u < G; ++u) {
        if (p0 + u >= npairs) break;
#pragma unroll
        for (int q = 0; q < V; ++q) {
          const float l = (z[u].at(q) + b[u].at(q)) * kLog2e;
          const float x = v[u].at(q);
          if (p0 + u == 0) {
            mx[q] = l;
            den[q] = 1.f;
            acc[q] = x;
          } else {
            const float d = l - mx[q];
            const float e = exp2_fast(-fabsf(d));
            const bool up = d > 0.f;
            acc[q] = up ? fmaf(acc[q], e, x) : fmaf(e, x, acc[q]);
            den[q] = up ? fmaf(den[q], e, 1.f) : den[q] + e;
            mx[q] = up ? l : mx[q];
          }
        }
      }
    }
    float out[V], inv[V], dout[V];
    Vec<float, 4>::load(dC + i * ldd + ch, dout);
    if constexpr (V == 8) Vec<float, 4>::load(dC + i * ldd + ch + 4, dout + 4);
#pragma unroll
    for (int q = 0; q < V; ++q) {
      inv[q] = 1.f / den[q];
      out[q] = acc[q] * inv[q];
    }
    // pass 2: per-pair gradients (rows re-read only when 2m > G)
    for (int p0 = 0; p0 < npairs; p0 += G) {
      if (npairs > G) load_group(p0);
#pragma unroll
      for (int u = 0; u < G; ++u) {
        const int p = p0 + u;
        if (p >= npairs) break;
        float gv[V], gl[V];
#pragma unroll
        for (int q = 0; q < V; ++q) {
          const float S = exp2_fast((z[u].at(q) + b[u].at(q)) * kLog2e - mx[q]) * inv[q];
          gv[q] = S * dout[q];
          gl[q] = gv[q] * (v[u].at(q) - out[q]);
        }
        const long row = row_of(p);
        const bool is_a = p < m;
        Vec<T, V>::store((is_a ? dCa : dCb) + row * ldo + ch, gv);
        Vec<T, V>::store((is_a ? dZa : dZb) + row * ldo + ch, gl);
        float* sb = s_db + (long)p * W + lane * V;
#pragma unroll
        for (int q = 0; q < V; ++q) atomicAdd(sb + q, gl[q]);
      }
    }
  }
  __syncthreads();
  // this workgroup's partial bias gradients: part[blockIdx.y][p][ch], p < 2m
  for (int e = tid; e < 2 * m * 64; e += 64 * kBwdWaves) {
    const int p = e >> 6, l = e & 63;
    const int cc = (blockIdx.x * 64 + l) * V;
    if (cc < c) {
      float* dst = part + ((long)blockIdx.y * 2 * m + p) * c + cc;
#pragma unroll
      for (int q = 0; q < V; ++q) dst[q] = s_db[p * W + l * V + q];
    }
  }
}

// dBa[r][j] = sum_y part[y][r][j], dBb[r][j] = sum_y part[y][m + r][j], the
// partials summed in a fixed order: 16 slices of y per column, then the
// slices in index order.
__global__ __launch_bounds__(1024) void compress_bias_reduce_kernel(long ny, int m, int c,
                                                                    const float* __restrict__ part,
                                                                    float* __restrict__ dBa,
                                                                    float* __restrict__ dBb) {
  __shared__ float s_sum[16][64];
  const int col_l = threadIdx.x & 63, slice = threadIdx.x >> 6;
  const long col = (long)blockIdx.x * 64 + col_l;  // over 2m * c
  const long ncol = 2L * m * c;
  float sum = 0.f;
  if (col < ncol)
    for (long y = slice; y < ny; y += 16) sum += part[y * ncol + col];
  s_sum[slice][col_l] = sum;
  __syncthreads();
  if (slice == 0 && col < ncol) {
    float t = 0.f;
#pragma unroll
    for (int s = 0; s < 16; ++s) t += s_sum[s][col_l];
    const long p = col / c, j = col - p * c;
    if (p < m) dBa[p * c + j] = t; else dBb[(p - m) * c + j] = t;
  }
}

// Workgroup rows of the backward grid and blocks per workgroup row.
void compress_bwd_grid(long units, long* ny, long* bpw) {
  const long want = 256;
  *bpw = std::max(1L, (units + want - 1) / want);
  *ny = std::max(1L, (units + *bpw - 1) / *bpw);  // one row even with no units: it writes the zero partials
}

// Backward units: the blocks, then one tail unit per sequence (a single
// sequence when cu is null).
long compress_bwd_units(long n, int m, long nseq, long nblk, bool varlen) { return varlen ? nblk + nseq : n / m + 1; }

template <typename T, int V>
hipError_t run_bwd(long n, long nblk, int m, int c, const void* Ca, const void* Cb, const void* Za, const void* Zb,
                   long ld, const void* Ba, const void* Bb, const float* dC, long ldd, void* dCa, void* dCb,
                   void* dZa, void* dZb, long ldo, float* dBa, float* dBb, float* part, int nseq, const int64_t* cu,
                   const int64_t* boff, hipStream_t s) {
  long ny, bpw;
  compress_bwd_grid(compress_bwd_units(n, m, nseq, nblk, cu != nullptr), &ny, &bpw);
  const dim3 grid((unsigned)((c / V + 63) / 64), (unsigned)ny);
  const uint32_t lds = (uint32_t)(2 * m * 64 * V * sizeof(float));
  hipError_t e = launch("compress_bwd", compress_bwd_kernel<T, V>, grid, dim3(64 * kBwdWaves), lds, s, nblk, n, m,
                        c, (const T*)Ca, (const T*)Cb, (const T*)Za, (const T*)Zb, ld, (const T*)Ba, (const T*)Bb,
                        dC, ldd, (T*)dCa, (T*)dCb, (T*)dZa, (T*)dZb, ldo, bpw, part, nseq, cu, boff);
  if (e != hipSuccess) return e;
  const long ncol = 2L * m * c;
  return launch("compress_bias_reduce", compress_bias_reduce_kernel, dim3((unsigned)((ncol + 63) / 64)),
                dim3(1024), 0, s, ny, m, c, (const float*)part, dBa, dBb);
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

size_t compress_backward_workspace_bytes(long n, int m, int c, long nseq, long nblk, bool varlen) {
  long ny, bpw;
  compress_bwd_grid(compress_bwd_units(n, m, nseq, nblk, varlen), &ny, &bpw);
  return ws_bytes(ny, 2 * m, c, sizeof(float));
}

namespace {
hipError_t dispatch_bwd(csa_dtype dt, long n, long nblk, int m, int c, const void* Ca, const void* Cb,
                        const void* Za, const void* Zb, long ld_in, const void* Ba, const void* Bb,
                        const float* dCcomp, long ld_dc, void* dCa, void* dCb, void* dZa, void* dZb, long ld_out,
                        float* dBa, float* dBb, void* workspace, int nseq, const int64_t* cu, const int64_t* boff,
                        hipStream_t s) {
  float* part = (float*)workspace;
  if (dt == CSA_F32)
    return run_bwd<float, 4>(n, nblk, m, c, Ca, Cb, Za, Zb, ld_in, Ba, Bb, dCcomp, ld_dc, dCa, dCb, dZa, dZb, ld_out,
                             dBa, dBb, part, nseq, cu, boff, s);
  if (c % 8 == 0 && ld_in % 8 == 0 && ld_out % 8 == 0)
    return run_bwd<bf16_t, 8>(n, nblk, m, c, Ca, Cb, Za, Zb, ld_in, Ba, Bb, dCcomp, ld_dc, dCa, dCb, dZa, dZb,
                              ld_out, dBa, dBb, part, nseq, cu, boff, s);
  return run_bwd<bf16_t, 4>(n, nblk, m, c, Ca, Cb, Za, Zb, ld_in, Ba, Bb, dCcomp, ld_dc, dCa, dCb, dZa, dZb, ld_out,
                            dBa, dBb, part, nseq, cu, boff, s);
}
}  // namespace

hipError_t launch_compress_backward(csa_dtype dt, long n, int m, int c, const void* Ca, const void* Cb,
                                    const void* Za, const void* Zb, long ld_in, const void* Ba, const void* Bb,
                                    const float* dCcomp, long ld_dc, void* dCa, void* dCb, void* dZa, void* dZb,
                                    long ld_out, float* dBa, float* dBb, void* workspace, hipStream_t s) {
  return dispatch_bwd(dt, n, n / m, m, c, Ca, Cb, Za, Zb, ld_in, Ba, Bb, dCcomp, ld_dc, dCa, dCb, dZa, dZb, ld_out,
                      dBa, dBb, workspace, 0, nullptr, nullptr, s);
}

hipError_t launch_compress_backward_varlen(csa_dtype dt, long nseq, long nblk, int m, int c, const void* Ca,
                                           const void* Cb, const void* Za, const void* Zb, long ld_in,
                                           const void* Ba, const void* Bb, const int64_t* cu, const int64_t* boff,
                                           const float* dCcomp, long ld_dc, void* dCa, void* dCb, void* dZa,
                                           void* dZb, long ld_out, float* dBa, float* dBb, void* workspace,
                                           hipStream_t s) {
  return dispatch_bwd(dt, 0, nblk, m, c, Ca, Cb, Za, Zb, ld_in, Ba, Bb, dCcomp, ld_dc, dCa, dCb, dZa, dZb, ld_out,
                      dBa, dBb, workspace, (int)nseq, cu, boff, s);
}

hipError_t launch_compress_append(csa_dtype dt, long B, int m, int c, const void* rows, long ld_new, void* ring,
                                  const void* Ba, const void* Bb, const int64_t* t_new, const int64_t* kv_off,
                                  void* out, long ld_out, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const dim3 grid((unsigned)B);
  if (dt == CSA_F32)
    return launch("compress_append", compress_append_kernel<float, 4>, grid, dim3(256), 0, s, m,
                  AppendArgs<float>{c, (const float*)rows, ld_new, (float*)ring, (const float*)Ba, (const float*)Bb,
                                    (float*)out, ld_out},
                  t_new, kv_off);
  const AppendArgs<bf16_t> p{c, (const bf16_t*)rows, ld_new, (bf16_t*)ring, (const bf16_t*)Ba, (const bf16_t*)Bb,
                             (bf16_t*)out, ld_out};
  if (c % 8 == 0 && ld_new % 8 == 0 && ld_out % 8 == 0)
    return launch("compress_append", compress_append_kernel<bf16_t, 8>, grid, dim3(256), 0, s, m, p, t_new, kv_off);
  return launch("compress_append", compress_append_kernel<bf16_t, 4>, grid, dim3(256), 0, s, m, p, t_new, kv_off);
}

hipError_t launch_compress_append_pair(csa_dtype dt, long B, int m, const int64_t* t_new, const int64_t* kv_off,
                                       const AppendCache& a, const AppendCache& b, hipStream_t s) {
  if (B == 0) return hipSuccess;
  const dim3 grid((unsigned)(2 * B));
  if (dt == CSA_F32) {
    const AppendArgs<float> p1{a.c, (const float*)a.rows, a.ld_new, (float*)a.ring, (const float*)a.Ba,
                               (const float*)a.Bb, (float*)a.out, a.ld_out};
    const AppendArgs<float> p2{b.c, (const float*)b.rows, b.ld_new, (float*)b.ring, (const float*)b.Ba,
                               (const float*)b.Bb, (float*)b.out, b.ld_out};
    return launch("compress_append", compress_append_pair_kernel<float, 4>, grid, dim3(256), 0, s, m, B, p1, p2,
                  t_new, kv_off);
  }
  const AppendArgs<bf16_t> p1{a.c, (const bf16_t*)a.rows, a.ld_new, (bf16_t*)a.ring, (const bf16_t*)a.Ba,
                              (const bf16_t*)a.Bb, (bf16_t*)a.out, a.ld_out};
  const AppendArgs<bf16_t> p2{b.c, (const bf16_t*)b.rows, b.ld_new, (bf16_t*)b.ring, (const bf16_t*)b.Ba,
                              (const bf16_t*)b.Bb, (bf16_t*)b.out, b.ld_out};
  auto v8 = [](const AppendCache& x) { return x.c % 8 == 0 && x.ld_new % 8 == 0 && x.ld_out % 8 == 0; };
  if (v8(a) && v8(b))
    return launch("compress_append", compress_append_pair_kernel<bf16_t, 8>, grid, dim3(256), 0, s, m, B, p1, p2,
                  t_new, kv_off);
  return launch("compress_append", compress_append_pair_kernel<bf16_t, 4>, grid, dim3(256), 0, s, m, B, p1, p2,
                t_new, kv_off);
}

}  // namespace csa
