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
// Design (one workgroup = 256 threads = 4 waves, one wave per SIMD, one
// workgroup per CU, persistent):
//   * output tiles of BM x BN (256 x 192 for the projection, 256 x 128 for
//     out_proj; 64..256 x 128 for one round of small tiles after the
//     two-wave kernel's whole rounds), waves in a 2 x 2 grid, wave tile
//     BM/2 x BN/2 of v_mfma_f32_32x32x16_bf16 with fp32 accumulators in AGPRs.
//   * one flat stream of K steps (of BK = 32) over all of the workgroup's tiles
//     flows through an NST-stage LDS ring filled by 16-byte global->LDS
//     direct copies.  The copies run NST-1 steps ahead of the math and cross
//     tile boundaries, so the memory pipe never drains between tiles.  Each
//     wave counts its vector-memory operations and waits only for the step it
//     is about to read.
//   * the epilogue does not stall the math: a cross-lane swap
//     (v_permlane32_swap) joins lane l's and lane l+32's 4-column halves of
//     the transposed accumulator tile into whole 16-byte row pieces.  The
//     first EARLY pieces are stored at once; the rest stay in registers and
//     are stored during the first SPLIT steps of the next tile, a few per
//     step, under its MFMAs.
//   * out_proj: the residual is prefetched a few steps before the end of the
//     tile in the same 16-byte-piece layout and added in fp32 before the one
//     RNE rounding.
//   * tile order (more tiles than workgroups): the 8 XCDs receive workgroup
//     ids round-robin; each XCD owns a contiguous range of BM-row panels and
//     walks them in groups of 8 panels, panel fastest, so the 32 tiles one
//     XCD runs at a time share 8 activation panels and 4 weight slices in its
//     L2.  With at most one tile per workgroup, tile = workgroup id.
//   * rows >= M of A are read as row M-1; their results are never stored.
//     The output and the residual go through buffer resources that end at
//     row M of the tile, so the hardware drops the stores of rows >= M and
//     their residual reads return zero (a stored copy of row M-1 would race
//     with C == R in place).  Requires K % BK == 0 and Nc % BN == 0.
//   * side job: a launch of fewer tiles than CUs (the round of small tiles
//     after the two-wave kernel's whole rounds) can take one more workgroup
//     that builds the attention's work-unit table instead of taking tiles,
//     on a CU that would otherwise idle; the tiles are dealt over the other
//     workgroups.
#include "attn_units.hpp"
#include "gs_device.hpp"

namespace gs {

constexpr int GEMM_BM = 256;
constexpr int GEMM_THREADS = 256;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// LDS tile geometry for a K step of BK bf16: a row is BK*2 bytes = BK/8
// chunks of 16 bytes.  A 16-byte-per-lane LDS read is served 16 lanes at a
// time from a 256-byte window of banks; the fragment reads touch 16
// consecutive rows at one logical chunk, so the physical chunk of row r is the
// logical one XOR-ed with (r / rows_per_window) mod chunks_per_row: the 16
// rows then land on 16 distinct 16-byte bank slots.
template <int BK>
struct TileGeom {
  static constexpr int CPR = BK / 8;                     // 16-byte chunks per row
  static constexpr int RPW = 256 / (BK * 2);             // rows per 256-byte bank window
  static constexpr int ROWS_PER_COPY = 1024 / (BK * 2);  // rows one wave copy fills
  __device__ static __forceinline__ int swz(int r) { return (r / RPW) % CPR; }
};

// LDS-direct copies of one [ROWS x BK] bf16 operand tile per K step.  Each
// wave instruction fills ROWS_PER_COPY consecutive LDS rows (1 KB).  The
// per-lane byte offsets from the tile's first row are computed once per tile
// (32-bit, so a copy address is a uniform 64-bit base plus one VGPR); rows at
// or past row_limit read row row_limit-1.  Without CLAMP (every row valid)
// one offset serves all of the wave's copies.
template <int ROWS, int BK, bool CLAMP>
struct TileCopy {
  using G = TileGeom<BK>;
  static constexpr int INSTR = ROWS / G::ROWS_PER_COPY / 4;  // per wave
  static constexpr int NOFF = CLAMP ? INSTR : 1;
  // consecutive copies of a wave are 4*ROWS_PER_COPY rows apart: same swizzle
  static_assert((4 * G::ROWS_PER_COPY / G::RPW) % G::CPR == 0, "one offset per wave needs equal swizzles");
  unsigned off[NOFF];

  __device__ __forceinline__ void init(int row0, int row_limit, int ld, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < NOFF; ++j) {
      const int r = (j * 4 + wave) * G::ROWS_PER_COPY + lane / G::CPR;  // LDS row this lane fills
      const int c = (lane % G::CPR) ^ G::swz(r);  // logical chunk stored at physical chunk lane%CPR
      int gr = row0 + r;
      if (CLAMP) gr = gr < row_limit ? gr : row_limit - 1;
      off[j] = (unsigned)((gr - row0) * ld + c * 8) * 2u;
    }
  }
  // copy j of the wave (j < INSTR); tile: first element of the tile's first
  // row at this K step (uniform)
  __device__ __forceinline__ void issue_one(int j, const bf16* tile, int ld, GS_LDS bf16* dst,
                                            int wave) const {
    const char* base = (const char*)tile + (CLAMP ? 0 : (size_t)j * 4 * G::ROWS_PER_COPY * ld * 2);
    copy16_to_lds(base + (CLAMP ? off[j] : off[0]), dst + (j * 4 + wave) * G::ROWS_PER_COPY * BK);
  }
};

template <int N>
struct IntC {
  static constexpr int value = N;
};

// vmcnt(n) (gfx9 encoding, expcnt and lgkmcnt at max), n rounded down to a
// multiple of 4 and capped at 60: only ever waits longer.
#define GS_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))
__device__ __forceinline__ void gemm_wait_vmcnt_le(int n) {
  switch (n >= 60 ? 15 : (n < 0 ? 0 : n >> 2)) {
    case 0: GS_VMCNT(0); break;    case 1: GS_VMCNT(4); break;
    case 2: GS_VMCNT(8); break;    case 3: GS_VMCNT(12); break;
    case 4: GS_VMCNT(16); break;   case 5: GS_VMCNT(20); break;
    case 6: GS_VMCNT(24); break;   case 7: GS_VMCNT(28); break;
    case 8: GS_VMCNT(32); break;   case 9: GS_VMCNT(36); break;
    case 10: GS_VMCNT(40); break;  case 11: GS_VMCNT(44); break;
    case 12: GS_VMCNT(48); break;  case 13: GS_VMCNT(52); break;
    case 14: GS_VMCNT(56); break;  default: GS_VMCNT(60); break;
  }
}
#undef GS_VMCNT

// Workgroup barrier without the memory fence __syncthreads() adds (the fence
// would wait for every outstanding store and LDS-direct copy).  LDS ordering
// is kept by the explicit waits around it; the empty asm statements keep the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void gemm_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(unsigned, bf16x2_t{to_bf16(a), to_bf16(b)});
}

// v_permlane32_swap: x's lanes 32..63 trade places with y's lanes 0..31.
__device__ __forceinline__ void swap_lo_hi(unsigned& x, unsigned& y) {
  const auto s = __builtin_amdgcn_permlane32_swap(x, y, false, false);
  x = s[0];
  y = s[1];
}

template <int BM, int BN, int BK, int NST, bool DEFER, int EARLY, int SPLIT, bool RESID>
__global__ __launch_bounds__(GEMM_THREADS, 1) void gemm_bf16_nt_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ W, const bf16* R, bf16* C,
    int M, int Nc, int K, UnitTableJob job) {
  using G = TileGeom<BK>;
  using CopyA = TileCopy<BM, BK, true>;        // activation rows: the last panel is ragged
  using CopyB = TileCopy<BN, BK, false>;       // weight rows: Nc % BN == 0
  constexpr int WM = BM / 2;   // wave tile rows
  constexpr int WN = BN / 2;   // wave tile columns
  constexpr int TI = WM / 32;  // 32-row MFMA tiles per wave
  constexpr int TJ = WN / 32;  // 32-col MFMA tiles per wave
  constexpr int KK = BK / 16;  // MFMA k chunks per K step
  constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;
  static_assert(BM % 64 == 0 && BM <= 256, "row tile");
  constexpr int STAGE = A_ELEMS + B_ELEMS;
  constexpr int LPS = CopyA::INSTR + CopyB::INSTR;  // copies per step per wave
  constexpr int NOUT = TI * TJ * 2;                 // 16-byte output pieces per lane per tile
  constexpr int SPS = (NOUT - EARLY) / SPLIT;       // pieces stored per early step of the next tile
  constexpr int RPRE = 3;                           // residual prefetched this many steps ahead
  static_assert(KK % 2 == 0, "register double buffer assumes an even chunk count");
  static_assert((NOUT - EARLY) % SPLIT == 0, "stores spread evenly over the early steps");
  __shared__ __attribute__((aligned(1024))) bf16 smem[NST * STAGE];
  static_assert(NST * STAGE * 2 >= UNIT_TABLE_LDS_INTS * 4, "LDS for the side job");

  // With a job, the grid's last workgroup builds the attention's work-unit
  // table instead of taking tiles (a launch of fewer tiles than CUs runs it
  // on a CU that would otherwise idle).  Only the projection's launch
  // carries one; the residual instantiations leave the code out (inlined
  // there, it slowed out_proj's small-tile launch by about 15 %).
  if constexpr (!RESID) {
    if (job.table && blockIdx.x == gridDim.x - 1) {
      build_unit_table(job, (int*)smem);
      return;
    }
  }

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int frag_row = lane & 31;
  const int half = lane >> 5;

  const int mt_count = (M + BM - 1) / BM;
  const int nt_count = Nc / BN;
  const int KT = K / BK;

  // ---- tile order ----
  // k-th tile of this workgroup as (panel, column tile), or panel = -1.
  const int Gs = gridDim.x - (job.table ? 1 : 0);
  // (else: plain round-robin over tiles)
  const bool by_xcd = (Gs & 7) == 0 && mt_count >= 8 && (long long)mt_count * nt_count > Gs;
  const int xcd = blockIdx.x & 7;
  const int p_lo = by_xcd ? (int)(((long long)xcd * mt_count) >> 3) : 0;
  const int p_hi = by_xcd ? (int)(((long long)(xcd + 1) * mt_count) >> 3) : mt_count;
  const int slot0 = by_xcd ? (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  const int per = by_xcd ? (Gs >> 3) : Gs;
  const int x_tiles = (p_hi - p_lo) * nt_count;
  // One tile per workgroup (a round of small tiles): workgroup ids reach the
  // XCDs round-robin, so the tiles of ids x, x + 8, ... share XCD x's L2.
  // The order below gives each XCD whole groups of 8 panels (all column
  // tiles of a few panels); when that makes an XCD read more rows of the
  // operands than all panels of an eighth of the column tiles, the XCD takes
  // the latter instead (the projection's 565 leftover rows: 9 panels of 64
  // rows against 24 weight slices of 128).
  const bool col_split = !by_xcd && (nt_count & 7) == 0 && (Gs & 7) == 0 &&
                         (long long)mt_count * nt_count <= Gs &&
                         mt_count * BM + (nt_count >> 3) * BN <
                             ((mt_count + 7) >> 3) * BM + nt_count * BN;
  auto tile_of = [&](int k, int& panel, int& col) __attribute__((always_inline)) {
    const int u = slot0 + k * per;
    if (u >= x_tiles) {
      panel = -1;
      col = 0;
      return;
    }
    if (col_split) {
      const int slot = u >> 3;
      col = (u & 7) * (nt_count >> 3) + slot / mt_count;
      panel = slot - (slot / mt_count) * mt_count;
      return;
    }
    const int grp = u / (8 * nt_count);
    const int v = u - grp * 8 * nt_count;
    const int gp = min(8, p_hi - p_lo - grp * 8);
    col = v / gp;
    panel = p_lo + grp * 8 + (v - col * gp);
  };

  auto stage_a = [&](int st) { return (GS_LDS bf16*)&smem[st * STAGE]; };
  auto stage_b = [&](int st) { return (GS_LDS bf16*)&smem[st * STAGE + A_ELEMS]; };

  // ---- copy side: the next (tile, step) to issue ----
  int ops = 0;         // vector-memory ops this wave has issued
  // Steps in the ring ahead of the one being computed.  Without DEFER a
  // stage is refilled as soon as it is freed (in the last chunk of a step);
  // with DEFER its copies are spread over all chunks of the following step,
  // so one stage is always being refilled and NST-1 are ready or in flight.
  constexpr int DEPTH = DEFER ? NST - 1 : NST;
  int mark[DEPTH];     // ops right after the copies of each of the next DEPTH steps
  int is_k = 0, is_step = 0, is_panel, is_col, is_slot = 0;
  tile_of(0, is_panel, is_col);
  if (is_panel < 0) return;  // uniform: no work for this workgroup
  CopyA cpA;
  CopyB cpB;
  const bf16* tA = nullptr;
  const bf16* tB = nullptr;
  auto set_issue_tile = [&]() __attribute__((always_inline)) {
    tA = A + (size_t)is_panel * BM * K;
    tB = W + (size_t)is_col * BN * K;
    cpA.init(is_panel * BM, M, K, wave, lane);
    cpB.init(is_col * BN, Nc, K, wave, lane);
  };
  set_issue_tile();
  // copy j (< LPS) of the step being issued: activation rows first
  auto copy_one = [&](int j) __attribute__((always_inline)) {
    if (j < CopyA::INSTR)
      cpA.issue_one(j, tA + is_step * BK, K, stage_a(is_slot), wave);
    else
      cpB.issue_one(j - CopyA::INSTR, tB + is_step * BK, K, stage_b(is_slot), wave);
  };
  // after all LPS copies of a step (the caller counts them in ops)
  auto advance_issue = [&]() __attribute__((always_inline)) {
    is_slot = is_slot + 1 == NST ? 0 : is_slot + 1;
    if (++is_step == KT) {
      is_step = 0;
      tile_of(++is_k, is_panel, is_col);
      if (is_panel >= 0) set_issue_tile();
    }
  };

  // ---- compute side ----
  int k = 0, panel, col;
  tile_of(0, panel, col);
  int cm_slot = 0;  // ring slot of the step being computed

  // fragments of one 16-wide k chunk.  Fragment rows are (multiple of 32) +
  // lane%32, and 32-row shifts keep the swizzle, so an address is a per-lane
  // chunk offset plus a compile-time row offset.
  static_assert((32 / G::RPW) % G::CPR == 0, "swizzle must repeat every 32 rows");
  auto load_frags = [&](int st, int kk, bf16x8* af, bf16x8* bfr) __attribute__((always_inline)) {
    const int lo = frag_row * BK + ((kk * 2 + half) ^ G::swz(frag_row)) * 8;
    const GS_LDS bf16* as = stage_a(st) + wm * WM * BK + lo;
    const GS_LDS bf16* bs = stage_b(st) + wn * WN * BK + lo;
#pragma unroll
    for (int i = 0; i < TI; ++i) af[i] = *(const GS_LDS bf16x8*)(as + i * 32 * BK);
#pragma unroll
    for (int j = 0; j < TJ; ++j) bfr[j] = *(const GS_LDS bf16x8*)(bs + j * 32 * BK);
  };

  // ---- output pieces ----
  // Piece q = (i*TJ + j)*2 + gp of a lane: row wm*WM + i*32 + lane%32 of the
  // tile, columns wn*WN + j*32 + (2*gp + lane/32)*8 .. +7.  Its byte offset
  // from the tile's origin is row_off[i] + a column constant.  Pieces below
  // EARLY are stored as soon as they are formed; vals[q - EARLY] holds the
  // others until the next tile's early steps.
  u32x4_t vals[NOUT > EARLY ? NOUT - EARLY : 1];
  u32x4_t rres[RESID ? NOUT : 1];
  unsigned row_off[TI];        // for the tile whose pieces vals holds
  __amdgpu_buffer_rsrc_t out_rs = buffer_rsrc(C, 0);  // that tile's rows below M
  bool have_out = false;
  int mark_r = 0;
  auto piece_col_bytes = [&](int q) { return ((q / 2 % TJ) * 32 + (q % 2) * 16) * 2; };
  // offsets of a lane's rows from the tile's origin (rows >= M included)
  auto tile_row_offsets = [&](unsigned* ro) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < TI; ++i)
      ro[i] = (unsigned)((wm * WM + i * 32 + frag_row) * Nc + wn * WN + half * 8) * 2u;
  };
  // bytes from the tile's origin (m0, n0) to the end of its last row below M
  auto tile_bytes = [&](int m0, int n0) __attribute__((always_inline)) {
    return (unsigned)(min(M - m0, BM) * Nc - n0) * 2u;
  };
  auto store_piece = [&](int q) __attribute__((always_inline)) {
    __builtin_amdgcn_raw_buffer_store_b128(vals[q - EARLY], out_rs,
                                           row_off[q / (2 * TJ)] + piece_col_bytes(q), 0, 0);
  };
  auto store_pieces = [&](int q0, int nq) __attribute__((always_inline)) {
#pragma unroll
    for (int q = q0; q < q0 + nq; ++q) store_piece(q);
    ops += nq;
  };
  auto load_residual = [&](int m0, int n0) __attribute__((always_inline)) {
    if constexpr (RESID) {
      unsigned ro[TI];
      tile_row_offsets(ro);
      const auto res_rs = buffer_rsrc(R + (size_t)m0 * Nc + n0, tile_bytes(m0, n0));
#pragma unroll
      for (int q = 0; q < NOUT; ++q)
        rres[q] = __builtin_amdgcn_raw_buffer_load_b128(res_rs, ro[q / (2 * TJ)] + piece_col_bytes(q),
                                                        0, 0);
      ops += NOUT;
      mark_r = ops;
    }
  };

  // ---- prologue: the first DEPTH steps ----
#pragma unroll
  for (int s = 0; s < DEPTH; ++s) {
    if (is_panel >= 0) {
#pragma unroll
      for (int j = 0; j < LPS; ++j) copy_one(j);
      advance_issue();
      ops += LPS;
    }
    mark[s] = ops;
  }
  gemm_wait_vmcnt_le(__builtin_amdgcn_readfirstlane(ops - mark[0]));
  gemm_barrier();

  bf16x8 af[2][TI], bfr[2][TJ];
  load_frags(cm_slot, 0, af[0], bfr[0]);

  f32x16 acc[TI][TJ];
  for (;;) {
    const int m0 = __builtin_amdgcn_readfirstlane(panel * BM);
    const int n0 = __builtin_amdgcn_readfirstlane(col * BN);
    const int rstep = KT > RPRE ? KT - RPRE : 0;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

    // One K step of KK chunks.  Registers hold two k chunks: chunk kk's
    // MFMAs run while chunk kk+1's fragments are read.  The stage barrier
    // sits before the last chunk, whose MFMAs then also cover the next step's
    // first fragment reads, the refill of the freed stage (NST steps ahead)
    // and NS of the previous tile's output pieces.  Those side instructions
    // are interleaved one or two per MFMA, so their issue hides under the
    // matrix pipe instead of stalling it.
    auto step = [&](int kt, auto ns_tag, int q0, bool st_active) __attribute__((always_inline)) {
      constexpr int NS = decltype(ns_tag)::value;  // output pieces stored in this step
      constexpr int NM = TI * TJ, NR = TI + TJ;
      if (kt == rstep) load_residual(m0, n0);
      // DEFER: the stage freed in the previous step is refilled during this one
      bool do_issue = DEFER && is_panel >= 0;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int p = kk & 1;
        const bool last = kk == KK - 1;
        wait_lds();  // chunk kk's fragments are in registers
        int nslot = cm_slot;
        if (last) {
          // the next step landed (this wave's copies), then for everyone;
          // everyone is done reading this step's stage
          gemm_wait_vmcnt_le(__builtin_amdgcn_readfirstlane(ops - mark[1]));
          gemm_barrier();
          if (!DEFER) do_issue = is_panel >= 0;
          nslot = cm_slot + 1 == NST ? 0 : cm_slot + 1;
        }
        const int nkk = last ? 0 : kk + 1;
        const int lo = frag_row * BK + ((nkk * 2 + half) ^ G::swz(frag_row)) * 8;
        const GS_LDS bf16* as = stage_a(nslot) + wm * WM * BK + lo;
        const GS_LDS bf16* bs = stage_b(nslot) + wn * WN * BK + lo;
        // side instructions of this chunk: fragment reads, copies c0..c1-1,
        // output pieces s0..s1-1
        const int c0 = DEFER ? kk * LPS / KK : 0;
        const int c1 = DEFER ? (kk + 1) * LPS / KK : (last ? LPS : 0);
        const int s0 = kk * NS / KK, s1 = (kk + 1) * NS / KK;
        const int nside = NR + (c1 - c0) + (s1 - s0);
#pragma unroll
        for (int n = 0; n < NM; ++n) {
          acc[n / TJ][n % TJ] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              bfr[p][n % TJ], af[p][n / TJ], acc[n / TJ][n % TJ], 0, 0, 0);
#pragma unroll
          for (int si = n * nside / NM; si < (n + 1) * nside / NM; ++si) {
            if (si < TI) {
              af[p ^ 1][si] = *(const GS_LDS bf16x8*)(as + si * 32 * BK);
            } else if (si < NR) {
              bfr[p ^ 1][si - TI] = *(const GS_LDS bf16x8*)(bs + (si - TI) * 32 * BK);
            } else if (si < NR + (c1 - c0)) {
              if (do_issue) copy_one(c0 + si - NR);
            } else if (st_active) {
              store_piece(q0 + s0 + si - NR - (c1 - c0));
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        if (last) {
          // In issue order, this step's copies end before the pieces of its
          // last chunk: the mark goes there.
          if (do_issue) {
            advance_issue();
            ops += LPS;
          }
          if (st_active) ops += s0;
#pragma unroll
          for (int i = 0; i < DEPTH - 1; ++i) mark[i] = mark[i + 1];
          mark[DEPTH - 1] = ops;
          if (st_active) ops += NS - s0;
          cm_slot = nslot;
        }
      }
    };

    // early steps: the previous tile's pieces leave, SPS per step
#pragma unroll
    for (int s = 0; s < SPLIT; ++s) {
      if (s < KT) {
        step(s, IntC<SPS>{}, EARLY + s * SPS, have_out);
      } else if (have_out) {
        store_pieces(EARLY + s * SPS, SPS);
      }
    }
    for (int kt = SPLIT; kt < KT; ++kt) step(kt, IntC<0>{}, 0, false);

    // ---- epilogue: accumulators -> 16-byte row pieces ----
    // acc[i][j] is the transposed 32x32 tile: register g*4+e holds row
    // lane%32 and column g*8 + (lane/32)*4 + e.  For column groups g = 2gp
    // and 2gp+1, the swap leaves lane l (< 32) with all 8 columns of group
    // 2gp and lane l+32 with all 8 of group 2gp+1.
    if constexpr (RESID) gemm_wait_vmcnt_le(__builtin_amdgcn_readfirstlane(ops - mark_r));
    tile_row_offsets(row_off);
    out_rs = buffer_rsrc(C + (size_t)m0 * Nc + n0, tile_bytes(m0, n0));
    have_out = true;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
      for (int j = 0; j < TJ; ++j)
#pragma unroll
        for (int gp = 0; gp < 2; ++gp) {
          const f32x16& a = acc[i][j];
          const int q = (i * TJ + j) * 2 + gp;
          u32x4_t piece;
          if constexpr (RESID) {
            // swap fp32 values, add the residual piece, round once
            unsigned x[4], y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // (element values first: bit-casting a vector-element lvalue
              // directly reads the wrong bytes)
              const float fx = a[gp * 8 + e], fy = a[gp * 8 + 4 + e];
              x[e] = __builtin_bit_cast(unsigned, fx);
              y[e] = __builtin_bit_cast(unsigned, fy);
              swap_lo_hi(x[e], y[e]);
            }
            // columns 0..3 of the piece are x[0..3], columns 4..7 are y[0..3]
            const u32x4_t r = rres[q];
            unsigned w[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const unsigned rv = r[e];  // bf16 pair: columns 2e, 2e+1 of the piece
              const float r0 = __builtin_bit_cast(float, rv << 16);
              const float r1 = __builtin_bit_cast(float, rv & 0xFFFF0000u);
              const float v0 = __builtin_bit_cast(float, e < 2 ? x[2 * e] : y[2 * e - 4]);
              const float v1 = __builtin_bit_cast(float, e < 2 ? x[2 * e + 1] : y[2 * e - 3]);
              w[e] = pack_bf16x2(v0 + r0, v1 + r1);
            }
            piece = u32x4_t{w[0], w[1], w[2], w[3]};
          } else {
            unsigned x0 = pack_bf16x2(a[gp * 8 + 0], a[gp * 8 + 1]);
            unsigned x1 = pack_bf16x2(a[gp * 8 + 2], a[gp * 8 + 3]);
            unsigned y0 = pack_bf16x2(a[gp * 8 + 4], a[gp * 8 + 5]);
            unsigned y1 = pack_bf16x2(a[gp * 8 + 6], a[gp * 8 + 7]);
            swap_lo_hi(x0, y0);
            swap_lo_hi(x1, y1);
            piece = u32x4_t{x0, x1, y0, y1};
          }
          if (q < EARLY) {
            __builtin_amdgcn_raw_buffer_store_b128(piece, out_rs, row_off[i] + piece_col_bytes(q),
                                                   0, 0);
            ++ops;
          } else {
            vals[q - EARLY] = piece;
          }
          // one piece at a time: keeps the accumulator reads from being
          // hoisted into a register-hungry batch
          __builtin_amdgcn_sched_barrier(0);
        }

    tile_of(++k, panel, col);
    if (panel < 0) break;
  }
  // the last tile's pieces
  store_pieces(EARLY, NOUT - EARLY);
  wait_vmem();
}

// Host-side launchers ------------------------------------------------------

static int g_gemm_cus = 0;

static int gemm_persistent_grid(int tiles) {
  if (g_gemm_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_gemm_cus = n;
  }
  return tiles < g_gemm_cus ? tiles : g_gemm_cus;
}

hipError_t launch_qkv_proj_bf16_pp(const void* x, const void* wqkv, void* qkv, int M, int d,
                                   hipStream_t stream, const UnitTableJob* job, bool* job_done);

// job (optional): a unit-table build to run in a spare workgroup of the
// launch; *job_done tells whether it was enqueued (else the caller runs it).
hipError_t launch_qkv_proj_bf16(const void* x, const void* wqkv, void* qkv, int M, int d,
                                hipStream_t stream, const UnitTableJob* job, bool* job_done) {
  if (job_done) *job_done = false;
  // 3d is a multiple of 256 when d is (two waves per SIMD, 256 x 256 tiles);
  // otherwise 3d = 384 * (d / 128) is a multiple of 192
  if ((3 * d) % 256 == 0)
    return launch_qkv_proj_bf16_pp(x, wqkv, qkv, M, d, stream, job, job_done);
  const int Nc = 3 * d;
  const int mt = (M + GEMM_BM - 1) / GEMM_BM;
  hipLaunchKernelGGL((gemm_bf16_nt_kernel<GEMM_BM, 192, 64, 2, false, 0, 12, false>), dim3(gemm_persistent_grid(mt * (Nc / 192))),
                     dim3(GEMM_THREADS), 0, stream, (const bf16*)x, (const bf16*)wqkv,
                     (const bf16*)nullptr, (bf16*)qkv, M, Nc, d, UnitTableJob{});
  return hipGetLastError();
}

hipError_t launch_out_proj_bf16_pp(const void* o, const void* wo, const void* x, void* out, int M,
                                   int d, hipStream_t stream);

hipError_t launch_out_proj_bf16(const void* o, const void* wo, const void* x, void* out, int M,
                                int d, hipStream_t stream) {
  if (d % 256 == 0) return launch_out_proj_bf16_pp(o, wo, x, out, M, d, stream);
  const int mt = (M + GEMM_BM - 1) / GEMM_BM;
  hipLaunchKernelGGL((gemm_bf16_nt_kernel<GEMM_BM, 128, 64, 3, false, 0, 8, true>), dim3(gemm_persistent_grid(mt * (d / 128))),
                     dim3(GEMM_THREADS), 0, stream, (const bf16*)o, (const bf16*)wo,
                     (const bf16*)x, (bf16*)out, M, d, d, UnitTableJob{});
  return hipGetLastError();
}

// One round of small tiles: C[rows][Nc] (+ R) for the rows left after a
// persistent launch's whole rounds of large tiles.  Tiles are BM x 128 with
// BM the smallest of 64, 128, 192, 256 whose tiles all fit on the CUs at
// once, so every CU takes at most one small tile instead of a few CUs taking
// a whole round of large ones.  Returns that BM, or 0 if even 256-row tiles
// would need a second round (the caller then keeps one launch).
int gemm_tail_tile_rows(int rows, int Nc) {
  const int cus = gemm_persistent_grid(1 << 30);
  if (rows <= 0 || Nc % 128 != 0) return 0;
  for (int bm = 64; bm <= 256; bm += 64)
    if ((long long)((rows + bm - 1) / bm) * (Nc / 128) <= cus) return bm;
  return 0;
}

template <int BM, bool RESID>
static void launch_tail(const bf16* A, const bf16* W, const bf16* R, bf16* C, int rows, int Nc,
                        int K, hipStream_t stream, const UnitTableJob* job) {
  const int tiles = (rows + BM - 1) / BM * (Nc / 128);
  hipLaunchKernelGGL((gemm_bf16_nt_kernel<BM, 128, 64, 3, false, 0, 4, RESID>),
                     dim3(tiles + (job ? 1 : 0)), dim3(GEMM_THREADS), 0, stream, A, W, R, C, rows,
                     Nc, K, job ? *job : UnitTableJob{});
}

// bm: gemm_tail_tile_rows(rows, Nc); requires K % 64 == 0.  job (optional):
// a unit-table build for one more workgroup of the launch.
hipError_t launch_gemm_tail_bf16(const void* A, const void* W, const void* R, void* C, int rows,
                                 int Nc, int K, int bm, hipStream_t stream,
                                 const UnitTableJob* job) {
  const bf16 *a = (const bf16*)A, *w = (const bf16*)W, *r = (const bf16*)R;
  bf16* c = (bf16*)C;
  switch (bm * 2 + (R != nullptr)) {
    case 128: launch_tail<64, false>(a, w, r, c, rows, Nc, K, stream, job); break;
    case 129: launch_tail<64, true>(a, w, r, c, rows, Nc, K, stream, job); break;
    case 256: launch_tail<128, false>(a, w, r, c, rows, Nc, K, stream, job); break;
    case 257: launch_tail<128, true>(a, w, r, c, rows, Nc, K, stream, job); break;
    case 384: launch_tail<192, false>(a, w, r, c, rows, Nc, K, stream, job); break;
    case 385: launch_tail<192, true>(a, w, r, c, rows, Nc, K, stream, job); break;
    case 512: launch_tail<256, false>(a, w, r, c, rows, Nc, K, stream, job); break;
    case 513: launch_tail<256, true>(a, w, r, c, rows, Nc, K, stream, job); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gs
