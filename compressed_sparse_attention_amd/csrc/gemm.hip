// Projection GEMM: Y[M,N] = X[M,K] . W[K,N], with W supplied transposed (Wt[N,K]).
//
// Eqs 1, 2, 5, 6, 7 and 10 of "Compressed Sparse Attention" are all
// row-vector projections of this form.  Both operands are K-contiguous, so
// each 16x16x32 MFMA operand is one 16-byte LDS read per lane.
//
// Kernels: gemm_smallm and its wide form (below) for bf16 with M <= 16 (the
// wide form, 64 columns per workgroup over all of K with X staged in LDS, for
// a short K and many columns), gemm256 and its copy-pipelined form
// gemm256_dma (K a multiple of 64) (below) for bf16 operands with
// M, N >= 256, and the general gemm_nt (fp32 too, any shape): 128x128 output
// tile per 256-thread
// workgroup (4 waves in 2x2, each 64x64 = 4x4 MFMA tiles), K staged through
// LDS in 128-byte slabs, double buffered: the next slab is fetched into
// registers while the current one feeds the MFMAs.  LDS rows are padded by
// 16 bytes so the 16 lanes reading one column of fragments hit distinct banks.
#include "common.hpp"
#include "internal.hpp"

namespace csa {
namespace {

// Four consecutive outputs (16-byte aligned for fp32, 8-byte for bf16).
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

constexpr int kBM = 128;
constexpr int kBN = 128;

template <typename TI, typename TO>
__global__ __launch_bounds__(256) void gemm_nt_kernel(int M, int N, int K, const TI* __restrict__ X,
                                                      long ldx, const TI* __restrict__ W, long ldw,
                                                      TO* __restrict__ Y, long ldy) {
  constexpr int VEC = 16 / sizeof(TI);      // elements per 16-byte load
  constexpr int BK = 128 / sizeof(TI);      // elements per 128-byte slab row
  constexpr int PITCH = BK + 2 * VEC;       // padded LDS row: rows 32 bytes apart, conflict-free fragment reads
  constexpr int CHUNKS = BK / VEC;          // 16-byte chunks per slab row
  constexpr int ROWS_PER_PASS = 256 / CHUNKS;
  constexpr int PASSES = kBM / ROWS_PER_PASS;
  constexpr int KSTEPS = BK / 32;

  __shared__ __attribute__((aligned(16))) TI As[2][kBM * PITCH];
  __shared__ __attribute__((aligned(16))) TI Bs[2][kBN * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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

// ---------------------------------------------------------------------------
// Large bf16 projections: 256x256 output tile per 512-thread workgroup.
//
// Eight waves (two per SIMD, so one can issue MFMAs while the other waits on
// LDS or on its slab loads), each owning a 128x64 strip of 8x4 MFMA tiles:
// a 32-deep k-step reads 12 fragments from LDS for 32 MFMAs, against 8 for
// 16 in the 128x128 kernel above (whose 64x64 wave tiles keep LDS at its read
// bandwidth).  K is staged in 64-element slabs, double buffered through
// registers.  Workgroups are dealt to the eight XCDs round-robin; each XCD
// gets a contiguous run of the tile sequence, walked in groups of kG2Group
// tile rows, so the workgroups resident on one XCD share operand strips in
// its L2.  Measured alternatives: four waves of 128x128 (one per SIMD, with
// the next k-step's fragments prefetched) and 32x32x16 MFMAs were slower.
// ---------------------------------------------------------------------------
constexpr int kG2M = 256;
constexpr int kG2N = 256;
constexpr int kG2K = 64;               // elements per slab row (128 bytes)
// LDS slab rows are unpadded; 16-byte chunk c of row r is stored at chunk
// c ^ ((r >> 1) & 7), so the 16 lanes of a fragment read (16 rows, one chunk)
// and of a staging store (2 rows x 8 chunks) each hit 16 distinct 4-bank groups.
__device__ __forceinline__ int g2_swz(int row, int chunk) { return row * kG2K + ((chunk ^ ((row >> 1) & 7)) << 3); }
constexpr int kG2Group = 4;            // tile rows per group in the walk order

template <typename TO>
__global__ __launch_bounds__(512) void gemm256_kernel(int M, int N, int K, const bf16_t* __restrict__ X, long ldx,
                                                        const bf16_t* __restrict__ W, long ldw, TO* __restrict__ Y,
                                                        long ldy, int tiles_m, int tiles_n, int per_xcd) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][kG2M * kG2K];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][kG2N * kG2K];

  const int seq = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (seq >= tiles_m * tiles_n) return;
  const int in_group = kG2Group * tiles_n;
  const int first_m = (seq / in_group) * kG2Group;
  const int gsize = min(kG2Group, tiles_m - first_m);
  const int r = seq % in_group;
  const long m0 = (long)(first_m + r % gsize) * kG2M;
  const long n0 = (long)(r / gsize) * kG2N;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves: 128 rows x 64 columns each
  if (wave >= 4) __builtin_amdgcn_s_setprio(1);  // the later wave of each SIMD issues first
  const int g = lane >> 4, c16 = lane & 15;
  const int lrow = tid >> 3;          // 0..63
  const int lcol = (tid & 7) * 8;
  constexpr int PASSES = kG2M / 64;   // 4 rows per thread per operand

  u32x4 ra[PASSES], rb[PASSES];
  const int KT = (K + kG2K - 1) / kG2K;
  auto fetch = [&](int kt) {
    const long k = (long)kt * kG2K + lcol;
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      const long row = m0 + lrow + 64 * p;
      const long col = n0 + lrow + 64 * p;
      ra[p] = load16_clamped(X + row * ldx + k, row < M && k < K, X);
      rb[p] = load16_clamped(W + col * ldw + k, col < N && k < K, W);
    }
    if (kt == KT - 1 && (K % kG2K) != 0) {
#pragma unroll
      for (int p = 0; p < PASSES; ++p)
        if (k >= K) rb[p] = u32x4{0u, 0u, 0u, 0u};
    }
    issue_fence();
  };
  auto stash = [&](int buf) {
#pragma unroll
    for (int p = 0; p < PASSES; ++p) {
      *reinterpret_cast<u32x4*>(&As[buf][g2_swz(lrow + 64 * p, tid & 7)]) = ra[p];
      *reinterpret_cast<u32x4*>(&Bs[buf][g2_swz(lrow + 64 * p, tid & 7)]) = rb[p];
    }
  };

  // acc[j][i] = (W tile j) x (X tile i)^T: lane (g, c16) holds output row
  // m = ... + 16 i + c16 and the four consecutive columns n = ... + 16 j + 4 g
  // .. +3, so the epilogue writes 4 adjacent outputs per store.
  f32x4 acc[4][8];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

  fetch(0);
  stash(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) fetch(kt + 1);
#pragma unroll
    for (int ks = 0; ks < kG2K / 32; ++ks) {
      Frag<bf16_t> fa[8], fb[4];
      // rows wm*128 + 16 i + c16 (A) and wn*64 + 16 j + c16 (B), chunk 4 ks + g
      const bf16_t* Ab = &As[cur][g2_swz(wm * 128 + c16, 4 * ks + g)];
      const bf16_t* Bb = &Bs[cur][g2_swz(wn * 64 + c16, 4 * ks + g)];
#pragma unroll
      for (int j = 0; j < 4; ++j) fb[j].load(Bb + j * 16 * kG2K);
#pragma unroll
      for (int i = 0; i < 8; ++i) fa[i].load(Ab + i * 16 * kG2K);
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int i = 0; i < 8; ++i) mma(acc[j][i], fb[j], fa[i]);
    }
    if (kt + 1 < KT) stash(cur ^ 1);
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const long row = m0 + wm * 128 + i * 16 + c16;
    if (row >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const long col = n0 + wn * 64 + j * 16 + 4 * g;
      if (col < N) {
        float v[4] = {acc[j][i][0], acc[j][i][1], acc[j][i][2], acc[j][i][3]};
        store4<TO>(Y + row * ldy + col, v);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The same 256x256 tile and wave layout for K a multiple of 64, with the
// operands brought in by direct global-to-LDS copies (global_load_lds, no
// VGPR staging) into a ring of kDmaStages 32-deep stages, and each wave's
// fragments for stage kt+1 read from LDS while its MFMAs on stage kt run.
//
// Per stage a workgroup's LDS traffic is 96 KiB of fragment reads and 32 KiB
// of copies for 8 x 32 MFMAs, about 125 bytes per clock at full MFMA rate,
// against ~140 bytes per clock measured for 16-byte LDS reads from eight
// waves; the ring, the prefetch and spreading the copies and reads over the
// MFMAs recover part of what the barrier-synchronised register staging left
// idle (W_H at 32768x4096x4096 1.04 -> 0.94 ms, W_UQ at 32768x32768x1536
// 3.55 -> 3.18 ms).
// bf16 outputs are staged through LDS and written as 512-byte row segments
// (the MFMA layout alone gives 32-byte pieces of 16 rows per store).
//
// Copy layout: wave w copies 16-row blocks 2w and 2w+1 of both operands per
// stage; lane l lands at byte 16 l of its block, i.e. row l/4 and stored
// chunk l%4, which holds the row's source chunk (l%4) ^ ((l/8)%4).  Rows r
// and r+1 share the XOR term, and pairs of rows differ: measured on this
// GPU, that reads a fragment (16 rows x 4 chunks of 16 bytes) at the full LDS
// rate, where the term ((l/16)%4) took about 1.6 times as long.
// The copies are asm (the compiler does not track them): each wave waits
// for its own with an explicit vmcnt, then the workgroup meets at a barrier.
// ---------------------------------------------------------------------------
constexpr int kDmaStages = 3;
constexpr int kDmaK = 32;  // k per stage

template <int N>
__device__ __forceinline__ void wait_vm_n() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// LDS wait the compiler can see (it then knows earlier LDS reads are done,
// instead of waiting for the next batch at the first use), then a barrier
// with no wait for vector memory.
__device__ __forceinline__ void lds_wait_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
  asm volatile("s_barrier" ::: "memory");
}

template <typename TO>
__global__ __launch_bounds__(512) void gemm256_dma_kernel(int M, int N, int K, const bf16_t* __restrict__ X,
                                                            long ldx, const bf16_t* __restrict__ W, long ldw,
                                                            TO* __restrict__ Y, long ldy, int tiles_m, int tiles_n,
                                                            int per_xcd) {
  constexpr int S = kDmaStages;
  constexpr int STAGE = 2 * 256 * kDmaK;  // elements: the A block, then the B block
  constexpr int OP = kG2N + 8;            // pitch of the staged output tile
  constexpr int SM = S * STAGE > kG2M * OP ? S * STAGE : kG2M * OP;
  __shared__ __attribute__((aligned(16))) bf16_t smem[SM];

  const int seq = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if (seq >= tiles_m * tiles_n) return;
  const int in_group = kG2Group * tiles_n;
  const int first_m = (seq / in_group) * kG2Group;
  const int gsize = min(kG2Group, tiles_m - first_m);
  const int r = seq % in_group;
  const long m0 = (long)(first_m + r % gsize) * kG2M;
  const long n0 = (long)(r / gsize) * kG2N;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves: 128 rows x 64 columns each
  if (wave >= 4) __builtin_amdgcn_s_setprio(1);  // the later wave of each SIMD issues first
  const int g = lane >> 4, c16 = lane & 15;
  const int KT = K / kDmaK;  // even

  // copy sources: rows past M or N repeat the last row (their outputs are not written)
  const int rl = lane >> 2;
  const int schunk = (lane & 3) ^ ((lane >> 3) & 3);
  const bf16_t* src[2][2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const long ra = m0 + 16 * (2 * wave + j) + rl;
    const long rb = n0 + 16 * (2 * wave + j) + rl;
    src[0][j] = X + (ra < M ? ra : M - 1) * ldx + schunk * 8;
    src[1][j] = W + (rb < N ? rb : N - 1) * ldw + schunk * 8;
  }
  const uint32_t lds0 = (uint32_t)(size_t)(lds_char*)smem;
  auto issue = [&](int kt) {  // four 1 KiB copies per wave
    const int buf = kt % S;
#pragma unroll
    for (int op = 0; op < 2; ++op)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const uint32_t dst = lds0 + 2u * (uint32_t)(buf * STAGE + op * 256 * kDmaK + (2 * wave + j) * 16 * kDmaK);
        gather_row_lds(src[op][j] + (long)kt * kDmaK, __builtin_amdgcn_readfirstlane(dst));
      }
  };
  auto wait_later = [&](int later) {  // this wave's copies, but for `later` stages, have landed
    if (later >= 2) wait_vm_n<8>();
    else if (later == 1) wait_vm_n<4>();
    else wait_vm_n<0>();
  };
  // fragment rows: A wm*128 + 16 i + c16, B wn*64 + 16 j + c16; their chunk
  // g is stored at g ^ ((row / 2) % 4) = g ^ ((c16 / 2) % 4)
  const int fchunk = (g ^ ((c16 >> 1) & 3)) * 8;
  auto read_frags = [&](int kt, Frag<bf16_t>(&fa)[8], Frag<bf16_t>(&fb)[4]) {
    const bf16_t* As = smem + (kt % S) * STAGE;
    const bf16_t* Bs = As + 256 * kDmaK;
#pragma unroll
    for (int j = 0; j < 4; ++j) fb[j].load(Bs + (wn * 64 + 16 * j + c16) * kDmaK + fchunk);
#pragma unroll
    for (int i = 0; i < 8; ++i) fa[i].load(As + (wm * 128 + 16 * i + c16) * kDmaK + fchunk);
  };

  // acc[j][i] = (W tile j) x (X tile i)^T, as in gemm256_kernel
  f32x4 acc[4][8];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

#pragma unroll
  for (int st = 0; st < S; ++st)
    if (st < KT) issue(st);
  Frag<bf16_t> fa0[8], fb0[4], fa1[8], fb1[4];
  wait_later(min(S - 1, KT - 1));
  lds_wait_barrier();
  read_frags(0, fa0, fb0);
  // Step kt: stage kt's fragments are in registers.  Once stage kt+1 has
  // landed for every wave (which also means stage kt's buffer is no longer
  // read), stage kt+S is copied into that buffer and stage kt+1's fragments
  // are read while stage kt's MFMAs run.  On the last step the read is of a
  // stale buffer and unused: a branch around it would make the compiler wait
  // for those reads before the MFMAs.
  //
  // The copy and the reads are spread over the MFMAs, one copy and three
  // fragment reads before each group of 8 MFMAs: issued all at once after the
  // barrier, they held both waves of a SIMD (which leave the barrier
  // together) off the MFMA pipe (measured 6-8% slower).  Fences keep the
  // scheduler from regrouping them.
  auto step = [&](int kt, Frag<bf16_t>(&fa)[8], Frag<bf16_t>(&fb)[4], Frag<bf16_t>(&na)[8],
                  Frag<bf16_t>(&nb)[4]) {
    wait_later(min(S - 2, KT - 2 - kt));
    lds_wait_barrier();
    const bool more = kt + S < KT;
    const int buf = (kt + S) % S;
    const bf16_t* As = smem + ((kt + 1) % S) * STAGE;
    const bf16_t* Bs = As + 256 * kDmaK;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (more) {  // copy j of stage kt+S: operand j / 2, this wave's block j % 2
        const int op = j >> 1, jj = j & 1;
        const uint32_t dst = lds0 + 2u * (uint32_t)(buf * STAGE + op * 256 * kDmaK + (2 * wave + jj) * 16 * kDmaK);
        gather_row_lds(src[op][jj] + (long)(kt + S) * kDmaK, __builtin_amdgcn_readfirstlane(dst));
      }
      nb[j].load(Bs + (wn * 64 + 16 * j + c16) * kDmaK + fchunk);
      na[2 * j].load(As + (wm * 128 + 16 * (2 * j) + c16) * kDmaK + fchunk);
      na[2 * j + 1].load(As + (wm * 128 + 16 * (2 * j + 1) + c16) * kDmaK + fchunk);
      issue_fence();
#pragma unroll
      for (int i = 0; i < 8; ++i) mma(acc[j][i], fb[j], fa[i]);
      issue_fence();
    }
  };
  for (int kt = 0; kt < KT; kt += 2) {
    step(kt, fa0, fb0, fa1, fb1);
    step(kt + 1, fa1, fb1, fa0, fb0);
  }

  if constexpr (sizeof(TO) == 2) {
    lds_wait_barrier();  // every wave's last fragment reads are done before the tile is staged over them
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = wm * 128 + i * 16 + c16;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float v[4] = {acc[j][i][0], acc[j][i][1], acc[j][i][2], acc[j][i][3]};
        store4<bf16_t>(&smem[row * OP + wn * 64 + j * 16 + 4 * g], v);
      }
    }
    lds_wait_barrier();
    // 32 lanes per row, 16 bytes each; N % 4 == 0, so a half chunk is all in or all out
#pragma unroll 4
    for (int it = 0; it < kG2M / 16; ++it) {
      const int row = it * 16 + (tid >> 5), ch = (tid & 31) * 8;
      const long grow = m0 + row, gcol = n0 + ch;
      const u32x4 v = *reinterpret_cast<const u32x4*>(&smem[row * OP + ch]);
      if (grow < M) {
        if (gcol + 8 <= N) {
          *reinterpret_cast<u32x4*>(Y + grow * ldy + gcol) = v;
        } else if (gcol < N) {
          *reinterpret_cast<uint2*>(Y + grow * ldy + gcol) = make_uint2(v[0], v[1]);
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const long row = m0 + wm * 128 + i * 16 + c16;
      if (row >= M) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const long col = n0 + wn * 64 + j * 16 + 4 * g;
        if (col < N) {
          float v[4] = {acc[j][i][0], acc[j][i][1], acc[j][i][2], acc[j][i][3]};
          store4<TO>(Y + row * ldy + col, v);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Few rows (M <= 16: one decode token per sequence): the weights are the
// traffic.  A 256-thread workgroup owns 16 output columns over all of K; its
// four waves split K and stream their share of the 16 weight rows straight
// from HBM into MFMA operands (the rows of X, read from L2, are the other
// operand; rows past M produce outputs that are not written), DEPTH 128-deep
// super-steps in flight per wave.  Within a super-step the k-slots of the
// MFMA operands are permuted the same way on both sides (a contraction does
// not depend on the order of k): load kk of lane group g takes
// k = 32 kk + 8 g .. +7, so the four groups of one load read 64 contiguous
// bytes of each row (measured on cold 100 MB weights: 10% faster than each
// lane reading 64 contiguous bytes over its four loads).  The four partial
// 16x16 tiles are summed through LDS.
// ---------------------------------------------------------------------------
constexpr int kSmN = 16;        // output columns per workgroup
constexpr int kSmSuper = 128;   // k per super-step

// One workgroup's 16 columns n0 .. n0 + 15 (s_part: the waves' partial tiles).
template <typename TO, int DEPTH>
__device__ __forceinline__ void smallm_tile(int M, int N, int K, const bf16_t* __restrict__ X, long ldx,
                                            const bf16_t* __restrict__ W, long ldw, TO* __restrict__ Y, long ldy,
                                            long n0, float (*s_part)[256]) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int nsup = (K + kSmSuper - 1) / kSmSuper;
  const int s0 = (wave * nsup) / 4, s1 = ((wave + 1) * nsup) / 4;  // this wave's super-steps
  const long wrow = n0 + c16 < N ? n0 + c16 : 0;  // rows past N / M read row 0: their outputs are not written
  const long xrow = c16 < M ? c16 : 0;
  const bf16_t* Wr = W + wrow * ldw + 8 * g;
  const bf16_t* Xr = X + xrow * ldx + 8 * g;

  Frag<bf16_t> wb[DEPTH][4], xb[DEPTH][4];
  // Loads of super-step ss into slot.  Super-steps past this wave's range are
  // not fetched (a uniform branch; filler loads there would all hit one
  // address); pieces past K read the start of the lane's own rows (never used).
  auto issue = [&](int ss, int slot) {
    if (ss >= s1) return;
    const long k = (long)ss * kSmSuper;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bool ok = k + 32 * kk + 8 * g < K;  // K % 8 == 0: a piece is all in or all out
      wb[slot][kk].load_clamped(Wr + k + 32 * kk, ok, Wr);
      xb[slot][kk].load_clamped(Xr + k + 32 * kk, ok, Xr);
    }
  };
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  auto compute = [&](int ss, int slot) {
    if (ss == nsup - 1 && (K % kSmSuper) != 0) {  // the K tail contributes zeros (uniform branch)
      const long k = (long)ss * kSmSuper;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        if (k + 32 * kk + 8 * g >= K) xb[slot][kk].zero();
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) mma(acc, xb[slot][kk], wb[slot][kk]);
  };
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) issue(s0 + d, d);
  issue_fence();
  for (int ss = s0; ss < s1; ss += DEPTH) {
#pragma unroll
    for (int d = 0; d < DEPTH; ++d) {
      if (ss + d < s1) compute(ss + d, d);
      issue(ss + d + DEPTH, d);
      issue_fence();
    }
  }
  // acc[r] = partial of Y[4 g + r][n0 + c16]
  if (wave > 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s_part[wave - 1][lane * 4 + r] = acc[r];
  }
  __syncthreads();
  if (wave == 0) {
    const long col = n0 + c16;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float v = acc[r] + s_part[0][lane * 4 + r] + s_part[1][lane * 4 + r] + s_part[2][lane * 4 + r];
      const int row = 4 * g + r;
      if (row < M && col < N) Y[row * ldy + col] = from_f32<TO>(v);
    }
  }
}

template <typename TO, int DEPTH>
__global__ __launch_bounds__(256) void gemm_smallm_kernel(int M, int N, int K, const bf16_t* __restrict__ X, long ldx,
                                                          const bf16_t* __restrict__ W, long ldw, TO* __restrict__ Y,
                                                          long ldy) {
  __shared__ float s_part[3][256];
  smallm_tile<TO, DEPTH>(M, N, K, X, ldx, W, ldw, Y, ldy, (long)blockIdx.x * kSmN, s_part);
}

// Two few-row products of the same X in one launch: workgroups below nb1
// take Y1 = X W1, the rest Y2 = X W2 (a uniform branch per workgroup).  A
// small product (a few workgroups, latency-bound on its own) then runs in the
// shadow of the large one instead of costing a launch of its own.
template <typename TO1, typename TO2, int DEPTH>
__global__ __launch_bounds__(256) void gemm_smallm_pair_kernel(int M, int K, const bf16_t* __restrict__ X, long ldx,
                                                               int nb1, int N1, const bf16_t* __restrict__ W1,
                                                               long ldw1, TO1* __restrict__ Y1, long ldy1, int N2,
                                                               const bf16_t* __restrict__ W2, long ldw2,
                                                               TO2* __restrict__ Y2, long ldy2) {
  __shared__ float s_part[3][256];
  const int b = (int)blockIdx.x;
  if (b < nb1)
    smallm_tile<TO1, DEPTH>(M, N1, K, X, ldx, W1, ldw1, Y1, ldy1, (long)b * kSmN, s_part);
  else
    smallm_tile<TO2, DEPTH>(M, N2, K, X, ldx, W2, ldw2, Y2, ldy2, (long)(b - nb1) * kSmN, s_part);
}

// ---------------------------------------------------------------------------
// Few rows with a short K (M <= 16, K <= kWideMaxK): the products of the
// decode-time query side (eqs 6 and 10, K = d_c).  A 256-thread workgroup owns
// 64 output columns; each wave owns 16 of them over ALL of K, so no partial
// sums cross waves.  The few rows of X (all of K) are staged once in LDS, and
// each wave streams its 16 weight rows through a rolling window of
// kWideDepth 128-deep super-steps: a slot is refilled as soon as its MFMAs
// are issued, so a wave computes while its later weights stream in (the
// pattern of the decode indexer sweep).  The k-slots are permuted as in
// smallm_tile (load kk of lane group g takes k = 32 kk + 8 g .. +7 of the
// super-step, on both operands).
// ---------------------------------------------------------------------------
constexpr int kWideN = 64;        // output columns per workgroup
constexpr int kWideMaxK = 1920;  // keeps the X stage within 64 KiB of LDS
constexpr int kWideDepth = 4;     // super-steps in flight per wave

// LDS bytes of one workgroup: 16 rows of X over K rounded up to a super-step,
// rows staggered by 32 bytes (conflict-free 16-byte fragment reads).
inline uint32_t wide_lds_bytes(long K) {
  const long kp = (K + kSmSuper - 1) / kSmSuper * kSmSuper;
  return (uint32_t)(16 * (kp + 16) * sizeof(bf16_t));
}

template <typename TO>
__device__ __forceinline__ void smallm_wide_tile(int M, int N, int K, const bf16_t* __restrict__ X, long ldx,
                                                 const bf16_t* __restrict__ W, long ldw, TO* __restrict__ Y,
                                                 long ldy, long n0, bf16_t* __restrict__ s_x) {
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, c16 = lane & 15;
  const int nsup = (K + kSmSuper - 1) / kSmSuper;
  const int XP = nsup * kSmSuper + 16;  // LDS pitch of an X row
  const long col = n0 + 16 * wave + c16;
  const bf16_t* Wr = W + (col < N ? col : 0) * ldw + 8 * g;  // columns past N read row 0: not written

  Frag<bf16_t> wb[kWideDepth][4];
  // pieces past K read the start of the lane's own row (X is zero there)
  auto issue = [&](int ss, int slot) {
    if (ss >= nsup) return;  // uniform
    const long k = (long)ss * kSmSuper;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) wb[slot][kk].load_clamped(Wr + k + 32 * kk, k + 32 * kk + 8 * g < K, Wr);
  };
#pragma unroll
  for (int d = 0; d < kWideDepth; ++d) issue(d, d);
  issue_fence();

  // X rows 0..15 over k < nsup * 128 into LDS; rows past M and pieces past K
  // are zero (K % 8 == 0: a piece is all in or all out)
  const int pieces = nsup * (kSmSuper / 8);
  for (int p = tid; p < 16 * pieces; p += 256) {
    const int row = p / pieces, kc = (p - row * pieces) * 8;
    const bool ok = row < M && kc < K;
    u32x4 v = load16_clamped(X + (long)row * ldx + kc, ok, X);
    if (!ok) v = u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(&s_x[row * XP + kc]) = v;
  }
  __syncthreads();

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const bf16_t* xr = s_x + c16 * XP + 8 * g;
  for (int ss = 0; ss < nsup; ss += kWideDepth) {
#pragma unroll
    for (int d = 0; d < kWideDepth; ++d) {
      if (ss + d < nsup) {  // uniform
        Frag<bf16_t> xf[4];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) xf[kk].load(xr + (ss + d) * kSmSuper + 32 * kk);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) mma(acc, xf[kk], wb[d][kk]);
      }
      issue(ss + d + kWideDepth, d);
      issue_fence();
    }
  }
  // acc[r] = Y[4 g + r][col]
  if (col < N) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * g + r;
      if (row < M) Y[row * ldy + col] = from_f32<TO>(acc[r]);
    }
  }
}

template <typename TO>
__global__ __launch_bounds__(256) void gemm_smallm_wide_kernel(int M, int N, int K, const bf16_t* __restrict__ X,
                                                               long ldx, const bf16_t* __restrict__ W, long ldw,
                                                               TO* __restrict__ Y, long ldy) {
  extern __shared__ __attribute__((aligned(16))) bf16_t s_x_dyn[];
  smallm_wide_tile<TO>(M, N, K, X, ldx, W, ldw, Y, ldy, (long)blockIdx.x * kWideN, s_x_dyn);
}

// Two such products of the same X in one launch (workgroups below nb1 take
// Y1 = X W1, the rest Y2 = X W2).
template <typename TO1, typename TO2>
__global__ __launch_bounds__(256) void gemm_smallm_wide_pair_kernel(int M, int K, const bf16_t* __restrict__ X,
                                                                    long ldx, int nb1, int N1,
                                                                    const bf16_t* __restrict__ W1, long ldw1,
                                                                    TO1* __restrict__ Y1, long ldy1, int N2,
                                                                    const bf16_t* __restrict__ W2, long ldw2,
                                                                    TO2* __restrict__ Y2, long ldy2) {
  extern __shared__ __attribute__((aligned(16))) bf16_t s_x_dyn[];
  const int b = (int)blockIdx.x;
  if (b < nb1)
    smallm_wide_tile<TO1>(M, N1, K, X, ldx, W1, ldw1, Y1, ldy1, (long)b * kWideN, s_x_dyn);
  else
    smallm_wide_tile<TO2>(M, N2, K, X, ldx, W2, ldw2, Y2, ldy2, (long)(b - nb1) * kWideN, s_x_dyn);
}

// ---------------------------------------------------------------------------
// dst[c][r] = src[r][c] for r < R, c < C, and dst[c][r] = 0 for R <= r < Rp
// (the padded tail of each destination row).  64 x 64 tiles through LDS with
// 16-byte loads and stores; requires C, Rp, the leading dimensions and both
// pointers to be multiples of 16 bytes.
// ---------------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(long R, long C, long Rp, const T* __restrict__ src, long lds,
                                                        T* __restrict__ dst, long ldd) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int PR = 64 / VEC;             // 16-byte pieces per 64-element row
  constexpr int PITCH = 64 + VEC;          // padded LDS row
  __shared__ __attribute__((aligned(16))) T tile[64 * PITCH];
  const long r0 = (long)blockIdx.y * 64, c0 = (long)blockIdx.x * 64;
  for (int p = threadIdx.x; p < 64 * PR; p += 256) {
    const int r = p / PR, ch = (p % PR) * VEC;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (r0 + r < R && c0 + ch < C) v = *reinterpret_cast<const u32x4*>(src + (r0 + r) * lds + c0 + ch);
    *reinterpret_cast<u32x4*>(&tile[r * PITCH + ch]) = v;
  }
  __syncthreads();
  for (int p = threadIdx.x; p < 64 * PR; p += 256) {
    const int cc = p / PR, rc = (p % PR) * VEC;
    if (c0 + cc >= C || r0 + rc >= Rp) continue;
    T v[VEC];
#pragma unroll
    for (int j = 0; j < VEC; ++j) v[j] = tile[(rc + j) * PITCH + cc];
    *reinterpret_cast<u32x4*>(dst + (c0 + cc) * ldd + r0 + rc) = *reinterpret_cast<const u32x4*>(v);
  }
}

}  // namespace

hipError_t launch_gemm(csa_dtype in_dt, csa_dtype out_dt, long M, long N, long K, const void* X,
                       long ldx, const void* W, long ldw, void* Y, long ldy, hipStream_t s) {
  if (in_dt == CSA_BF16 && M <= 16 && K <= kWideMaxK && N >= 256L * kWideN) {  // enough 64-column workgroups
    const dim3 gw((unsigned)((N + kWideN - 1) / kWideN));
    if (out_dt == CSA_BF16)
      return launch("gemm_smallm", gemm_smallm_wide_kernel<bf16_t>, gw, dim3(256), wide_lds_bytes(K), s, (int)M,
                    (int)N, (int)K, (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, (bf16_t*)Y, ldy);
    return launch("gemm_smallm", gemm_smallm_wide_kernel<float>, gw, dim3(256), wide_lds_bytes(K), s, (int)M, (int)N,
                  (int)K, (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, (float*)Y, ldy);
  }
  if (in_dt == CSA_BF16 && M <= 16) {
    // all of a wave's super-steps in flight when K is short (measured: up to
    // 8% faster at K = 1536), two otherwise
    const dim3 grid1((unsigned)((N + kSmN - 1) / kSmN));
    const bool deep = K <= 2048;
    if (out_dt == CSA_BF16)
      return deep ? launch("gemm_smallm", gemm_smallm_kernel<bf16_t, 4>, grid1, dim3(256), 0, s, (int)M, (int)N,
                           (int)K, (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, (bf16_t*)Y, ldy)
                  : launch("gemm_smallm", gemm_smallm_kernel<bf16_t, 2>, grid1, dim3(256), 0, s, (int)M, (int)N,
                           (int)K, (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, (bf16_t*)Y, ldy);
    return deep ? launch("gemm_smallm", gemm_smallm_kernel<float, 4>, grid1, dim3(256), 0, s, (int)M, (int)N, (int)K,
                         (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, (float*)Y, ldy)
                : launch("gemm_smallm", gemm_smallm_kernel<float, 2>, grid1, dim3(256), 0, s, (int)M, (int)N, (int)K,
                         (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, (float*)Y, ldy);
  }
  if (in_dt == CSA_BF16 && M >= kG2M && N >= kG2N && N % 4 == 0) {
    const int tm = (int)((M + kG2M - 1) / kG2M), tn = (int)((N + kG2N - 1) / kG2N);
    const int per_xcd = (tm * tn + 7) / 8;
    const dim3 grid2((unsigned)(8 * per_xcd));
    if (K % (2 * kDmaK) == 0) {  // rows are 16-byte aligned (checked by csa_project)
      if (out_dt == CSA_BF16)
        return launch("gemm", gemm256_dma_kernel<bf16_t>, grid2, dim3(512), 0, s, (int)M, (int)N, (int)K,
                      (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, (bf16_t*)Y, ldy, tm, tn, per_xcd);
      return launch("gemm", gemm256_dma_kernel<float>, grid2, dim3(512), 0, s, (int)M, (int)N, (int)K,
                    (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, (float*)Y, ldy, tm, tn, per_xcd);
    }
    if (out_dt == CSA_BF16)
      return launch("gemm", gemm256_kernel<bf16_t>, grid2, dim3(512), 0, s, (int)M, (int)N, (int)K,
                    (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, (bf16_t*)Y, ldy, tm, tn, per_xcd);
    return launch("gemm", gemm256_kernel<float>, grid2, dim3(512), 0, s, (int)M, (int)N, (int)K,
                  (const bf16_t*)X, ldx, (const bf16_t*)W, ldw, (float*)Y, ldy, tm, tn, per_xcd);
  }
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

hipError_t launch_transpose(csa_dtype dt, long R, long C, long Rp, const void* src, long lds, void* dst, long ldd,
                            hipStream_t s) {
  if (R == 0 && Rp == 0) return hipSuccess;
  const dim3 grid((unsigned)((C + 63) / 64), (unsigned)((Rp + 63) / 64));
  if (dt == CSA_F32)
    return launch("transpose", transpose_kernel<float>, grid, dim3(256), 0, s, R, C, Rp, (const float*)src, lds,
                  (float*)dst, ldd);
  return launch("transpose", transpose_kernel<bf16_t>, grid, dim3(256), 0, s, R, C, Rp, (const bf16_t*)src, lds,
                (bf16_t*)dst, ldd);
}

namespace {
template <typename TO1, typename TO2>
hipError_t launch_pair_typed(long M, long K, const void* X, long ldx, long N1, const void* W1, long ldw1, void* Y1,
                             long ldy1, long N2, const void* W2, long ldw2, void* Y2, long ldy2, hipStream_t s) {
  if (K <= kWideMaxK && N1 + N2 >= 256L * kWideN) {  // enough 64-column workgroups to fill the chip
    const int nw1 = (int)((N1 + kWideN - 1) / kWideN), nw2 = (int)((N2 + kWideN - 1) / kWideN);
    return launch("gemm_smallm", gemm_smallm_wide_pair_kernel<TO1, TO2>, dim3((unsigned)(nw1 + nw2)), dim3(256),
                  wide_lds_bytes(K), s, (int)M, (int)K, (const bf16_t*)X, ldx, nw1, (int)N1, (const bf16_t*)W1,
                  ldw1, (TO1*)Y1, ldy1, (int)N2, (const bf16_t*)W2, ldw2, (TO2*)Y2, ldy2);
  }
  const int nb1 = (int)((N1 + kSmN - 1) / kSmN), nb2 = (int)((N2 + kSmN - 1) / kSmN);
  const dim3 grid((unsigned)(nb1 + nb2));
  // super-step depth as for one product of this K
  if (K <= 2048)
    return launch("gemm_smallm", gemm_smallm_pair_kernel<TO1, TO2, 4>, grid, dim3(256), 0, s, (int)M, (int)K,
                  (const bf16_t*)X, ldx, nb1, (int)N1, (const bf16_t*)W1, ldw1, (TO1*)Y1, ldy1, (int)N2,
                  (const bf16_t*)W2, ldw2, (TO2*)Y2, ldy2);
  return launch("gemm_smallm", gemm_smallm_pair_kernel<TO1, TO2, 2>, grid, dim3(256), 0, s, (int)M, (int)K,
                (const bf16_t*)X, ldx, nb1, (int)N1, (const bf16_t*)W1, ldw1, (TO1*)Y1, ldy1, (int)N2,
                (const bf16_t*)W2, ldw2, (TO2*)Y2, ldy2);
}
}  // namespace

hipError_t launch_gemm_pair(csa_dtype in_dt, long M, long K, const void* X, long ldx, csa_dtype out1, long N1,
                            const void* W1, long ldw1, void* Y1, long ldy1, csa_dtype out2, long N2, const void* W2,
                            long ldw2, void* Y2, long ldy2, hipStream_t s) {
  if (in_dt == CSA_BF16 && M <= 16) {
    if (out1 == CSA_BF16 && out2 == CSA_BF16)
      return launch_pair_typed<bf16_t, bf16_t>(M, K, X, ldx, N1, W1, ldw1, Y1, ldy1, N2, W2, ldw2, Y2, ldy2, s);
    if (out1 == CSA_BF16)
      return launch_pair_typed<bf16_t, float>(M, K, X, ldx, N1, W1, ldw1, Y1, ldy1, N2, W2, ldw2, Y2, ldy2, s);
    if (out2 == CSA_BF16)
      return launch_pair_typed<float, bf16_t>(M, K, X, ldx, N1, W1, ldw1, Y1, ldy1, N2, W2, ldw2, Y2, ldy2, s);
    return launch_pair_typed<float, float>(M, K, X, ldx, N1, W1, ldw1, Y1, ldy1, N2, W2, ldw2, Y2, ldy2, s);
  }
  // many rows: each product fills the chip on its own
  const hipError_t e = launch_gemm(in_dt, out1, M, N1, K, X, ldx, W1, ldw1, Y1, ldy1, s);
  if (e != hipSuccess) return e;
  return launch_gemm(in_dt, out2, M, N2, K, X, ldx, W2, ldw2, Y2, ldy2, s);
}

}  // namespace csa
