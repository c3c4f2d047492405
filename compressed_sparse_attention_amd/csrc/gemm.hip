// Projection GEMM: Y[M,N] = X[M,K] . W[K,N], with W supplied transposed (Wt[N,K]).
//
// Eqs 1, 2, 5, 6, 7 and 10 of "Compressed Sparse Attention" are all
// row-vector projections of this form.  Both operands are K-contiguous, so
// each 16x16x32 MFMA operand is one 16-byte LDS read per lane.
//
// Tiling: 128x128 output tile per 256-thread workgroup (4 waves in 2x2, each
// 64x64 = 4x4 MFMA tiles), K staged through LDS in 128-byte slabs, double
// buffered: the next slab is fetched into registers while the current one
// feeds the MFMAs.  Rows are padded by 16 bytes so the 16 lanes reading one
// column of fragments hit distinct LDS banks.
#include "common.hpp"
#include "internal.hpp"

namespace csa {
namespace {

constexpr int kBM = 128;
constexpr int kBN = 128;

template <typename TI, typename TO>
__global__ __launch_bounds__(256) void gemm_nt_kernel(int M, int N, int K, const TI* __restrict__ X,
                                                      long ldx, const TI* __restrict__ W, long ldw,
                                                      TO* __restrict__ Y, long ldy) {
  constexpr int VEC = 16 / sizeof(TI);      // elements per 16-byte load
  constexpr int BK = 128 / sizeof(TI);      // elements per 128-byte slab row
  constexpr int PITCH = BK + VEC;           // padded LDS row (elements)
  constexpr int CHUNKS = BK / VEC;          // 16-byte chunks per slab row
  constexpr int ROWS_PER_PASS = 256 / CHUNKS;
  constexpr int PASSES = kBM / ROWS_PER_PASS;
  constexpr int KSTEPS = BK / 32;

  __shared__ __attribute__((aligned(16))) TI As[2][kBM * PITCH];
  __shared__ __attribute__((aligned(16))) TI Bs[2][kBN * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 4, c16 = lane & 15;
  const long m0 = (long)blockIdx.y * kBM;
  const long n0 = (long)blockIdx.x * kBN;

  const int lrow = tid / CHUNKS;
  const int lcol = (tid % CHUNKS) * VEC;

  u32x4 ra[PASSES], rb[PASSES];
  const int KT = (K + BK - 1) / BK;
  auto fetch = [&](int kt) {
    const long k = (long)kt * BK + lcol;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const long row = m0 + lrow + p * ROWS_PER_PASS;
      const long col = n0 + lrow + p * ROWS_PER_PASS;
      // out-of-range rows/columns load filler that only reaches unwritten outputs
      ra[p] = load16_clamped(X + row * ldx + k, row < M && k < K, X);
      rb[p] = load16_clamped(W + col * ldw + k, col < N && k < K, W);
    }
    if (kt == KT - 1 && (K % BK) != 0) {  // the K tail must contribute zeros (uniform branch)
#pragma unroll
      for (int p = 0; p < PASSES; ++p) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        if (k >= K) rb[p] = z;
      }
    }
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const int row = lrow + p * ROWS_PER_PASS;
      *reinterpret_cast<u32x4*>(&As[buf][row * PITCH + lcol]) = ra[p];
      *reinterpret_cast<u32x4*>(&Bs[buf][row * PITCH + lcol]) = rb[p];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  fetch(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) fetch(kt + 1);
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      Frag<TI> af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i].load(&As[cur][(wm * 64 + i * 16 + c16) * PITCH + ks * 32 + 8 * g]);
        bfr[i].load(&Bs[cur][(wn * 64 + i * 16 + c16) * PITCH + ks * 32 + 8 * g]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) mma(acc[i][j], af[i], bfr[j]);
    }
    if (kt + 1 < KT) stash(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long col = n0 + wn * 64 + j * 16 + c16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const long row = m0 + wm * 64 + i * 16 + 4 * g + r;
        if (row < M && col < N) Y[row * ldy + col] = from_f32<TO>(acc[i][j][r]);
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm(csa_dtype in_dt, csa_dtype out_dt, long M, long N, long K, const void* X,
                       long ldx, const void* W, long ldw, void* Y, long ldy, hipStream_t s) {
  dim3 grid((unsigned)((N + kBN - 1) / kBN), (unsigned)((M + kBM - 1) / kBM));
  if (in_dt == CSA_F32)
    return launch("gemm", gemm_nt_kernel<float, float>, grid, dim3(256), 0, s, (int)M, (int)N, (int)K,
                  (const float*)X, ldx, (const float*)W, ldw, (float*)Y, ldy);
  if (out_dt == CSA_BF16)
    return launch("gemm", gemm_nt_kernel<bf16_t, bf16_t>, grid, dim3(256), 0, s, (int)M, (int)N, (int)K,
                  (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, (bf16_t*)Y, ldy);
  return launch("gemm", gemm_nt_kernel<bf16_t, float>, grid, dim3(256), 0, s, (int)M, (int)N, (int)K,
                (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, (float*)Y, ldy);
}

}  // namespace csa
