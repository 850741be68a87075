// gemm_bf16.hip -- bf16 MFMA GEMM for the two projections of the block-MHSA
// sub-layer on gfx950:
//
//   qkv_proj:           C[M][Nc] = A[M][K] . W[Nc][K]^T              (Nc = 3d)
//   out_proj+residual:  C[M][Nc] = R[M][Nc] + A[M][K] . W[Nc][K]^T   (Nc = d)
//
// Both operands are K-contiguous (activations row-major, weights in the
// nn.Linear [out][in] layout), which is exactly what the MFMA operand layout
// wants: each lane feeds 8 consecutive k values of one row.
//
// Design (one workgroup = 256 threads = 4 waves, one wave per SIMD):
//   * macro tile 256 x BN (BN = 256 or 128), K step 64, waves in a 2 x 2 grid,
//     wave tile 128 x BN/2 built from v_mfma_f32_32x32x16_bf16.
//   * A and W tiles are staged in LDS with 16-byte global->LDS direct copies
//     (no VGPR round trip), double buffered: 2 x (32 KB + BN*128 B).
//   * LDS rows are 128 B (64 bf16); the eight 16-byte chunks of row r are
//     stored XOR-swizzled by (r & 7) so the fragment reads of 8 consecutive
//     lanes hit 8 distinct bank groups.
//   * the MFMA is issued with the weight fragment as its first operand, so
//     the accumulator is the transposed tile: each lane ends up holding 4
//     consecutive output columns of one row -> 8-byte bf16 stores.
//   * fp32 accumulate, residual added in fp32, one RNE rounding to bf16.
//   * workgroup ids are remapped so that each of the 8 XCDs (which get ids
//     round-robin) works on a contiguous range of tiles: the 12 (or 4/8)
//     column tiles of a 256-row activation panel then share one L2.
//   * rows >= M are clamped on load and masked on store, so M is arbitrary.
//     K must be a multiple of 64 and Nc a multiple of 4.
#include "gs_device.hpp"

namespace gs {

constexpr int GEMM_BM = 256;
constexpr int GEMM_THREADS = 256;

// LDS tile geometry for a K step of BK bf16: a row is BK*2 bytes = BK/8
// chunks of 16 bytes.  gfx950 serves a 16-byte-per-lane LDS read 16 lanes at
// a time from a 256-byte window of banks; the fragment reads below touch 16
// consecutive rows at one logical chunk, so the physical chunk of row r is the
// logical one XOR-ed with (r / rows_per_window) mod chunks_per_row: the 16
// rows then land on 16 distinct 16-byte bank slots.
template <int BK>
struct TileGeom {
  static constexpr int CPR = BK / 8;                 // 16-byte chunks per row
  static constexpr int RPW = 256 / (BK * 2);         // rows per 256-byte bank window
  static constexpr int ROWS_PER_COPY = 1024 / (BK * 2);  // rows one wave copy fills
  __device__ static __forceinline__ int swz(int r) { return (r / RPW) % CPR; }
};

// Issue the 16-byte LDS-direct copies of one [ROWS x BK] bf16 tile (ROWS rows
// starting at global row row0, k columns k0..k0+BK-1).  Each wave instruction
// fills ROWS_PER_COPY consecutive LDS rows (1 KB); rows past row_limit are
// clamped (their results are never stored).
template <int ROWS, int BK>
__device__ __forceinline__ void stage_tile(const bf16* __restrict__ src, int row0, int row_limit,
                                           int ld, int k0, GS_LDS bf16* dst, int wave, int lane) {
  using G = TileGeom<BK>;
  constexpr int INSTR = ROWS / G::ROWS_PER_COPY / 4;  // per wave
#pragma unroll
  for (int j = 0; j < INSTR; ++j) {
    const int r0 = (j * 4 + wave) * G::ROWS_PER_COPY;  // first LDS row of this copy
    const int r = r0 + lane / G::CPR;                  // LDS row this lane fills
    const int p = lane % G::CPR;                       // physical chunk in the row
    const int c = p ^ G::swz(r);                       // logical chunk stored there
    int gr = row0 + r;
    gr = gr < row_limit ? gr : row_limit - 1;
    copy16_to_lds(src + (size_t)gr * ld + k0 + c * 8, dst + r0 * BK);
  }
}

// vmcnt(N) with lgkmcnt/expcnt at max (gfx9 s_waitcnt encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// C[M][Nc] = (R +) A[M][K] . W[Nc][K]^T.  Tile 256 x BN, K step BK, NST-stage
// LDS ring (copies for K steps kt+1..kt+NST-1 are in flight while kt is multiplied).
template <int BN, int BK, int NST, bool RESID>
__global__ __launch_bounds__(GEMM_THREADS, 1) void gemm_bf16_nt_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ W, const bf16* R, bf16* C,
    int M, int Nc, int K) {
  using G = TileGeom<BK>;
  constexpr int WN = BN / 2;   // wave tile columns
  constexpr int TI = 4;        // 32-row MFMA tiles per wave (128 rows)
  constexpr int TJ = WN / 32;  // 32-col MFMA tiles per wave
  constexpr int KK = BK / 16;  // MFMA k chunks per K step
  constexpr int A_ELEMS = GEMM_BM * BK, B_ELEMS = BN * BK;
  // copies per stage per wave (the vmcnt unit)
  constexpr int LPS = GEMM_BM / G::ROWS_PER_COPY / 4 + BN / G::ROWS_PER_COPY / 4;
  static_assert(KK % 2 == 0, "register double buffer assumes an even chunk count");
  __shared__ __attribute__((aligned(1024))) bf16 smem[NST * (A_ELEMS + B_ELEMS)];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // tile id remap: the 8 XCDs receive workgroup ids round-robin; give each
  // XCD a contiguous range of tiles (column tiles of a row panel share its L2)
  const int mt_count = (M + GEMM_BM - 1) / GEMM_BM;
  const int nt_count = Nc / BN + (Nc % BN ? 1 : 0);
  const int T = mt_count * nt_count;
  const int b = blockIdx.x;
  const int full = (T / 8) * 8;
  const int t = b < full ? (b & 7) * (T / 8) + (b >> 3) : b;
  const int m0 = (t / nt_count) * GEMM_BM;
  const int n0 = (t % nt_count) * BN;

  auto sA = [&](int st) { return (GS_LDS bf16*)&smem[st * (A_ELEMS + B_ELEMS)]; };
  auto sB = [&](int st) { return (GS_LDS bf16*)&smem[st * (A_ELEMS + B_ELEMS) + A_ELEMS]; };
  auto issue = [&](int kt) {
    const int st = kt % NST;
    stage_tile<GEMM_BM, BK>(A, m0, M, K, kt * BK, sA(st), wave, lane);
    stage_tile<BN, BK>(W, n0, Nc, K, kt * BK, sB(st), wave, lane);
  };

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int KT = K / BK;
  const int frag_row = lane & 31;
  const int half = lane >> 5;

  // fragments of one 16-wide k chunk (A rows = activations, W rows = weights)
  auto load_frags = [&](int st, int kk, bf16x8* af, bf16x8* bfr) {
    const GS_LDS bf16* as = sA(st);
    const GS_LDS bf16* bs = sB(st);
    const int c = kk * 2 + half;
#pragma unroll
    for (int i = 0; i < TI; ++i) {
      const int r = wm * 128 + i * 32 + frag_row;
      af[i] = *(const GS_LDS bf16x8*)(as + r * BK + (c ^ G::swz(r)) * 8);
    }
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int r = wn * WN + j * 32 + frag_row;
      bfr[j] = *(const GS_LDS bf16x8*)(bs + r * BK + (c ^ G::swz(r)) * 8);
    }
  };

  // prologue: fill all NST stages (K steps 0..NST-1), wait for step 0.
  // Invariant in the loop: while step kt is multiplied, steps kt+1..kt+NST-1
  // are in flight; after step kt's last reads, its stage is refilled with
  // step kt+NST.
#pragma unroll
  for (int s = 0; s < NST; ++s)
    if (s < KT) issue(s);
  if (KT >= NST) wait_vmcnt<LPS * (NST - 1)>(); else wait_vmem();
  __syncthreads();

  // Registers hold two k chunks: while chunk kk's MFMAs run, chunk kk+1's LDS
  // reads are in flight.  The stage barrier sits before the last chunk's
  // MFMAs, so the next step's first chunk is read under them, and the freed
  // stage is refilled right after the barrier.
  bf16x8 af[2][TI], bfr[2][TJ];
  load_frags(0, 0, af[0], bfr[0]);
  for (int kt = 0; kt < KT; ++kt) {
    const int st = kt % NST;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int p = kk & 1;
      wait_lds();  // chunk kk is in registers; all reads of this stage so far are done
      if (kk + 1 < KK) {
        load_frags(st, kk + 1, af[p ^ 1], bfr[p ^ 1]);
      } else if (kt + 1 < KT) {
        // step kt+1 must have landed: after its copies only steps kt+2..kt+NST-1 may be pending
        if (kt + NST - 1 < KT) wait_vmcnt<LPS * (NST - 2)>(); else wait_vmem();
        __syncthreads();                    // all waves are done reading stage st
        if (kt + NST < KT) issue(kt + NST);  // refill the freed stage
        load_frags((kt + 1) % NST, 0, af[p ^ 1], bfr[p ^ 1]);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[p][j], af[p][i], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // epilogue: acc[i][j] is the transposed 32x32 tile; register e holds
  // column m = lane%32 and row n = (e/4)*8 + (lane/32)*4 + e%4.
#pragma unroll
  for (int i = 0; i < TI; ++i) {
    const int m = m0 + wm * 128 + i * 32 + (lane & 31);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int n = n0 + wn * WN + j * 32 + g * 8 + half * 4;
        if (n >= Nc) continue;
        float v0 = acc[i][j][g * 4 + 0], v1 = acc[i][j][g * 4 + 1];
        float v2 = acc[i][j][g * 4 + 2], v3 = acc[i][j][g * 4 + 3];
        const size_t off = (size_t)m * Nc + n;
        if constexpr (RESID) {
          const bf16x4 r = *(const bf16x4*)(R + off);
          v0 += to_f32(r[0]); v1 += to_f32(r[1]); v2 += to_f32(r[2]); v3 += to_f32(r[3]);
        }
        bf16x4 o;
        o[0] = to_bf16(v0); o[1] = to_bf16(v1); o[2] = to_bf16(v2); o[3] = to_bf16(v3);
        *(bf16x4*)(C + off) = o;
      }
    }
  }
}

// Host-side launchers ------------------------------------------------------

static inline int gemm_grid(int M, int Nc, int BN) {
  return ((M + GEMM_BM - 1) / GEMM_BM) * (Nc / BN + (Nc % BN ? 1 : 0));
}

hipError_t launch_qkv_proj_bf16(const void* x, const void* wqkv, void* qkv, int M, int d,
                                hipStream_t stream) {
  const int Nc = 3 * d;
  hipLaunchKernelGGL((gemm_bf16_nt_kernel<256, 64, 2, false>), dim3(gemm_grid(M, Nc, 256)),
                     dim3(GEMM_THREADS), 0, stream, (const bf16*)x, (const bf16*)wqkv,
                     (const bf16*)nullptr, (bf16*)qkv, M, Nc, d);
  return hipGetLastError();
}

hipError_t launch_out_proj_bf16(const void* o, const void* wo, const void* x, void* out, int M,
                                int d, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_bf16_nt_kernel<128, 64, 2, true>), dim3(gemm_grid(M, d, 128)),
                     dim3(GEMM_THREADS), 0, stream, (const bf16*)o, (const bf16*)wo,
                     (const bf16*)x, (bf16*)out, M, d, d);
  return hipGetLastError();
}

}  // namespace gs
