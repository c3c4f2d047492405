// Shared device helpers for the CSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef uint16_t bf16_t;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// fp32 -> bf16, round to nearest, ties to even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// Two fp32 -> two bf16 packed in one word (a in the low half), one instruction.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf2f(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f2bf(v); }

// 2^x on the hardware exp unit.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// max(x, 0) as one v_med3_f32 (median of x, 0 and a finite bound far above any
// score; an infinite bound would be folded back into a NaN-quieting max pair).
__device__ __forceinline__ float relu(float x) { return __builtin_amdgcn_fmed3f(x, 0.f, 3.0e38f); }

// Keeps the instruction scheduler from moving anything across this point.
// Placed right after a batch of load issues so the compiler cannot sink part
// of the batch below the first use of its data (which would make the wave pay
// two memory latencies instead of one).
__device__ __forceinline__ void issue_fence() { __builtin_amdgcn_sched_barrier(0); }

// Cross-workgroup hand-off without cache maintenance.  Data that one
// workgroup publishes for another one of the same launch is written with
// st_agent (write-through to the device-coherent level) and read with
// ld_agent (which bypasses possibly stale cache lines), so no cache-wide
// write-back or invalidate is needed.  Before a workgroup announces its data
// (an atomic), every thread waits for its own stores with wait_stores()
// and the workgroup meets at a barrier.
template <typename T>
__device__ __forceinline__ void st_agent(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ T ld_agent(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// s_waitcnt vmcnt(0): this thread's loads and stores have completed.
__device__ __forceinline__ void wait_stores() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Workgroup barrier for LDS traffic only: this wave's LDS operations have
// completed; its vector memory operations may still be in flight.  (The
// compiler drains every counter before a plain s_barrier on this target, so
// a prefetch issued just before __syncthreads() would be waited for there.)
// Loads whose results are consumed later are still waited for by the
// compiler at their first use.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Guarded 16-byte load without control flow: loads from p, or from
// `fallback` (any readable address holding finite input values) when !pred.
// The value loaded for !pred is NOT zeroed: every caller discards or masks
// those lanes' results (zero head weight, -inf logit, unwritten output).
// Neither a branch around the load (the compiler then waits for all loads in
// flight where the branches merge) nor a select on the loaded value (it ties
// each load to the next through the shared condition register) is used, so
// a batch of these loads stays in flight together.
__device__ __forceinline__ u32x4 load16_clamped(const void* p, bool pred, const void* fallback) {
  return *reinterpret_cast<const u32x4*>(pred ? p : fallback);
}

// ---------------------------------------------------------------------------
// MFMA fragments.
//
// Every contraction here uses 16x16 output tiles.  A fragment holds, for one
// lane, 8 values along the contraction axis of one row (A) or one column (B):
// lane l covers row/column (l % 16) and contraction slots 8*(l/16) .. +7 of a
// 32-wide step.  For bf16 that is exactly the operand of
// v_mfma_f32_16x16x32_bf16; for fp32 the same 32-wide step is issued as eight
// v_mfma_f32_16x16x4_f32, the j-th taking slot 8*(l/16)+j.  Because a
// contraction only needs A and B to agree on which slot holds which k, callers
// are free to map slots to k in any consistent way (several kernels map them
// so that a lane reads one contiguous run of memory).
//
// Accumulator (both types): lane l holds D[4*(l/16) + r][l % 16], r = 0..3.
// ---------------------------------------------------------------------------
template <typename T> struct Frag;

template <> struct Frag<bf16_t> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const bf16x8*>(p); }
  // see load16_clamped
  __device__ __forceinline__ void load_clamped(const bf16_t* p, bool pred, const void* fallback) {
    v = __builtin_bit_cast(bf16x8, load16_clamped(p, pred, fallback));
  }
  __device__ __forceinline__ void zero() {
    u32x4 z = {0u, 0u, 0u, 0u};
    v = __builtin_bit_cast(bf16x8, z);
  }
};

template <> struct Frag<float> {
  float f[8];
  __device__ __forceinline__ void load(const float* p) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
  }
  __device__ __forceinline__ void zero() {
#pragma unroll
    for (int j = 0; j < 8; ++j) f[j] = 0.f;
  }
  // see load16_clamped (fallback must hold at least 8 readable floats)
  __device__ __forceinline__ void load_clamped(const float* p, bool pred, const void* fallback) {
    load(pred ? p : reinterpret_cast<const float*>(fallback));
  }
};

__device__ __forceinline__ void mma(f32x4& acc, const Frag<bf16_t>& a, const Frag<bf16_t>& b) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a.v, b.v, acc, 0, 0, 0);
}

__device__ __forceinline__ void mma(f32x4& acc, const Frag<float>& a, const Frag<float>& b) {
#pragma unroll
  for (int j = 0; j < 8; ++j) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(a.f[j], b.f[j], acc, 0, 0, 0);
}

template <typename T> __device__ __forceinline__ void frag_set(Frag<T>& f, int j, T v);
template <> __device__ __forceinline__ void frag_set<bf16_t>(Frag<bf16_t>& f, int j, bf16_t v) {
  f.v[j] = __builtin_bit_cast(__bf16, v);
}
template <> __device__ __forceinline__ void frag_set<float>(Frag<float>& f, int j, float v) {
  f.f[j] = v;
}

// Transposed operand fragment from row-major LDS rows (pitch `pitch`
// elements): fragment row j = column dim0 + j, contraction slots = rows
// key0 + 8g .. key0 + 8g + 7 (g = lane / 16).  Used for C_sel^T in the
// attention products and for q^T / dO^T in their gradients.  bf16 uses two
// transposing LDS reads (ds_read_b64_tr_b16): within each 16-lane group, lane
// s points at 4 consecutive columns dim0 + 4(s%4) of row key0 + 8g + s/4 (+4),
// and lane j receives column dim0 + j of those four rows.  fp32 reads the 8
// values one by one.
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ Frag<T> frag_ct(const T* Cs, int pitch, int key0, int dim0, int lane) {
  Frag<T> f;
  const int g = lane >> 4, s = lane & 15;
  if constexpr (sizeof(T) == 2) {
    typedef __attribute__((address_space(3))) bf16x4 lds4;
    const T* p0 = Cs + (key0 + 8 * g + (s >> 2)) * pitch + dim0 + 4 * (s & 3);
    const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)p0);
    const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)(p0 + 4 * pitch));
    f.v = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) frag_set<T>(f, jj, Cs[(key0 + 8 * g + jj) * pitch + dim0 + (lane & 15)]);
  }
  return f;
}

// Rows of 512 bf16 in LDS without padding: 16-byte chunk j of row h is stored
// at position j ^ f(h).  f is a
// bijection on the low four bits that sends 16 consecutive rows to 16
// distinct positions (16-lane reads of one chunk from 16 rows: all banks
// distinct) and keeps f(h) >> 1 distinct over any 4 aligned consecutive rows
// (the transposing reads of 4 rows x 2 adjacent chunks: 8 distinct positions).
__device__ __forceinline__ int swz512_at(int row, int col) {
  const int f = ((row & 3) << 1) | ((row >> 2) & 1) | (((row >> 3) & 1) << 3);
  return row * 512 + ((((col >> 3) ^ f)) << 3) + (col & 7);
}

// frag_ct over swizzled 512-column rows: fragment row j = column dim0 + j,
// contraction slots = rows row0 + 8g .. row0 + 8g + 7.
__device__ __forceinline__ Frag<bf16_t> frag_ct_swz512(const bf16_t* D, int row0, int dim0, int lane) {
  typedef __attribute__((address_space(3))) bf16x4 lds4;
  const int g = lane >> 4, s = lane & 15;
  const int row = row0 + 8 * g + (s >> 2), col = dim0 + 4 * (s & 3);
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)(D + swz512_at(row, col)));
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds4*)(D + swz512_at(row + 4, col)));
  Frag<bf16_t> f;
  f.v = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return f;
}

typedef __attribute__((address_space(3))) char lds_char;

// Row gather straight into LDS: lane l's 16 bytes at `src` land at LDS byte
// offset `lds_base` + 16 l (global_load_lds_dwordx4; m0 holds the base).
// Issued from asm so that the compiler does not treat every later LDS read
// as a possible reader of these writes (it would wait for the whole gather
// right after issuing it); the kernel waits for them itself, with vmcnt, at
// the top of the next chunk.  No vector register is written, so nothing is
// left for the compiler to misread as already loaded.  m0 is a register the
// compiler reserves (it may hold a live value across this statement), so the
// block saves it in an SGPR and puts it back after the load has been issued
// (the load reads m0 at issue; s_nop 0 is the one wait state an m0 write needs
// before an LDS-DMA load reads it).
__device__ __forceinline__ void gather_row_lds(const void* src, uint32_t lds_base) {
  uint32_t saved_m0;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved_m0)
      : "v"(src), "s"(lds_base)
      : "memory");
}

// Order-preserving map of an fp32 score to uint32 (larger score -> larger key);
// -0.0 is mapped like +0.0 so the two compare equal.
__device__ __forceinline__ uint32_t score_key(float s) {
  uint32_t u = __float_as_uint(s);
  if (u == 0x80000000u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive prefix sum over the 64 lanes of a wave (all lanes active), built
// from DPP moves: shifts by 1, 2, 4, 8 inside each 16-lane row, then the
// last lane of row 0 is added to row 1 (and of row 2 to row 3), then the last
// lane of row 1 to rows 2 and 3.  Lanes without a source add 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  int v = (int)x;
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return (uint32_t)v;
}

// Value of lane 63 (a uniform result).
__device__ __forceinline__ uint32_t wave_last(uint32_t x) { return (uint32_t)__builtin_amdgcn_readlane((int)x, 63); }

// Sum (max) over the four lanes l, l^16, l^32, l^48.  v_permlane16_swap /
// v_permlane32_swap exchange 16-lane rows (32-lane halves) between two
// registers; with both operands equal, the two results of lane l hold x[l]
// and x[l ^ 16] (x[l ^ 32]) in some order, so their sum (max) is the pair's.
// Both lanes of a pair compute the same value (addition is commutative).
__device__ __forceinline__ float wave_sum_xor_16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float wave_max_xor_16_32(float v) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

}  // namespace csa
