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
constexpr int GEMM_BK = 64;
constexpr int GEMM_THREADS = 256;

// Issue the 16-byte LDS-direct copies of one [ROWS x 64] bf16 tile.
// Each wave instruction fills 8 consecutive LDS rows (1 KB).
template <int ROWS>
__device__ __forceinline__ void stage_tile(const bf16* __restrict__ src, int row0, int row_limit,
                                           int ld, int k0, GS_LDS bf16* dst, int wave, int lane) {
  constexpr int INSTR = ROWS / 8 / 4;  // per wave
#pragma unroll
  for (int j = 0; j < INSTR; ++j) {
    const int r0 = (j * 4 + wave) * 8;        // first LDS row of this instruction
    const int r = r0 + (lane >> 3);           // LDS row this lane fills
    const int p = lane & 7;                   // physical 16-byte chunk in the row
    const int c = p ^ (r & 7);                // logical chunk stored there
    int gr = row0 + r;
    gr = gr < row_limit ? gr : row_limit - 1;  // clamp rows past the end
    const bf16* g = src + (size_t)gr * ld + k0 + c * 8;
    copy16_to_lds(g, dst + r0 * GEMM_BK);
  }
}

template <int BN, bool RESID>
__global__ __launch_bounds__(GEMM_THREADS, 1) void gemm_bf16_nt_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ W, const bf16* R, bf16* C,
    int M, int Nc, int K) {
  constexpr int WN = BN / 2;   // wave tile columns
  constexpr int TI = 4;        // 32-row MFMA tiles per wave (128 rows)
  constexpr int TJ = WN / 32;  // 32-col MFMA tiles per wave
  __shared__ __attribute__((aligned(1024))) bf16 As[2][GEMM_BM * GEMM_BK];
  __shared__ __attribute__((aligned(1024))) bf16 Bs[2][BN * GEMM_BK];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // tile id remap: contiguous ranges of tiles per XCD
  const int mt_count = (M + GEMM_BM - 1) / GEMM_BM;
  const int nt_count = Nc / BN + (Nc % BN ? 1 : 0);
  const int T = mt_count * nt_count;
  const int b = blockIdx.x;
  const int full = (T / 8) * 8;
  const int t = b < full ? (b & 7) * (T / 8) + (b >> 3) : b;
  const int m0 = (t / nt_count) * GEMM_BM;
  const int n0 = (t % nt_count) * BN;

  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int KT = K / GEMM_BK;
  GS_LDS bf16* as0 = (GS_LDS bf16*)&As[0][0];
  GS_LDS bf16* as1 = (GS_LDS bf16*)&As[1][0];
  GS_LDS bf16* bs0 = (GS_LDS bf16*)&Bs[0][0];
  GS_LDS bf16* bs1 = (GS_LDS bf16*)&Bs[1][0];

  // fragment read offsets (in bf16 elements) inside a stage
  const int frag_row = lane & 31;
  const int half = lane >> 5;

  // fragments of one 16-wide k chunk: A rows (activations) and W rows (weights)
  auto load_frags = [&](const GS_LDS bf16* as, const GS_LDS bf16* bs, int kk, bf16x8* af,
                        bf16x8* bfr) {
    const int phys = ((kk * 2 + half) ^ (frag_row & 7)) * 8;
#pragma unroll
    for (int i = 0; i < TI; ++i)
      af[i] = *(const GS_LDS bf16x8*)(as + (wm * 128 + i * 32 + frag_row) * GEMM_BK + phys);
#pragma unroll
    for (int j = 0; j < TJ; ++j)
      bfr[j] = *(const GS_LDS bf16x8*)(bs + (wn * WN + j * 32 + frag_row) * GEMM_BK + phys);
  };

  stage_tile<GEMM_BM>(A, m0, M, K, 0, as0, wave, lane);
  stage_tile<BN>(W, n0, Nc, K, 0, bs0, wave, lane);
  wait_vmem();
  __syncthreads();

  // Software pipeline.  Registers hold two k chunks: while the 16 MFMAs of
  // chunk kk run, the LDS reads of chunk kk+1 are in flight.  The stage
  // barrier sits in the last chunk, so the first chunk of the next stage is
  // read while the last chunk of this one is multiplied.
  bf16x8 af[2][TI], bfr[2][TJ];
  load_frags(as0, bs0, 0, af[0], bfr[0]);
  constexpr int KK = GEMM_BK / 16;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) {
      stage_tile<GEMM_BM>(A, m0, M, K, (kt + 1) * GEMM_BK, cur ? as0 : as1, wave, lane);
      stage_tile<BN>(W, n0, Nc, K, (kt + 1) * GEMM_BK, cur ? bs0 : bs1, wave, lane);
    }
    const GS_LDS bf16* as = cur ? as1 : as0;
    const GS_LDS bf16* bs = cur ? bs1 : bs0;
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int p = kk & 1;  // KK is even: chunk parity is the same in every stage
      wait_lds();            // chunk kk is in registers
      if (kk + 1 < KK) {
        load_frags(as, bs, kk + 1, af[p ^ 1], bfr[p ^ 1]);
      } else {
        wait_vmem();         // next stage landed (this wave's copies) ...
        __syncthreads();     // ... and everyone's; everyone is done with this stage
        if (kt + 1 < KT) load_frags(cur ? as0 : as1, cur ? bs0 : bs1, 0, af[p ^ 1], bfr[p ^ 1]);
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
  hipLaunchKernelGGL((gemm_bf16_nt_kernel<256, false>), dim3(gemm_grid(M, Nc, 256)),
                     dim3(GEMM_THREADS), 0, stream, (const bf16*)x, (const bf16*)wqkv,
                     (const bf16*)nullptr, (bf16*)qkv, M, Nc, d);
  return hipGetLastError();
}

hipError_t launch_out_proj_bf16(const void* o, const void* wo, const void* x, void* out, int M,
                                int d, hipStream_t stream) {
  hipLaunchKernelGGL((gemm_bf16_nt_kernel<128, true>), dim3(gemm_grid(M, d, 128)),
                     dim3(GEMM_THREADS), 0, stream, (const bf16*)o, (const bf16*)wo,
                     (const bf16*)x, (bf16*)out, M, d, d);
  return hipGetLastError();
}

}  // namespace gs
