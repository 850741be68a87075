// gemm_pp_bf16.hip -- bf16 MFMA GEMM for the projections of the block-MHSA
// sub-layer on gfx950, two waves per SIMD in alternating roles:
//
//   qkv_proj:           C[M][Nc] = A[M][K] . W[Nc][K]^T              (Nc = 3d)
//   out_proj+residual:  C[M][Nc] = R[M][Nc] + A[M][K] . W[Nc][K]^T   (Nc = d)
//
// Both operands are K-contiguous (activations row-major, weights in the
// nn.Linear [out][in] layout): each lane feeds 8 consecutive k values of one
// row to v_mfma_f32_32x32x16_bf16.
//
// Design (one workgroup = 8 waves, one per CU, persistent):
//   * output tiles of 256 x BN; wave w owns the 128 x BN/4 sub-tile
//     (w & 1, w >> 1) with fp32 accumulators in registers.
//   * waves w and w + 4 share a SIMD and belong to different groups (w >> 2).
//     Time is cut into phases separated by workgroup barriers; in each phase
//     one group issues the matrix products of a half stage back to back while
//     the other group reads its fragments of the next half stage from LDS,
//     issues its share of the global->LDS copies of the next stage and (at a
//     tile boundary) writes the finished tile.  The matrix pipe of every SIMD
//     thus always has one wave feeding it.
//   * one flat stream of K stages (64 wide: each row piece is one whole
//     128-byte cache line) over all of the workgroup's tiles flows through a
//     2-stage LDS ring (64 KB per stage) filled by 16-byte global->LDS direct
//     copies, one stage ahead and across tile boundaries.  A phase covers half
//     a stage (32 k).  Each wave waits only for its own copies and the
//     barrier makes them visible to all.
//   * output: a cross-lane swap (v_permlane32_swap) joins lane l's and lane
//     l+32's 4-column halves of the transposed accumulator tile into 16-byte
//     row pieces.  Each wave then transposes its pieces through 8 KB of LDS
//     (the 32 KB the ring leaves free, one area per wave of a group; the two
//     groups use them in different phases), so that each store writes 8
//     whole 128-byte rows: stores of 32 rows x 32 bytes, the MFMA layout,
//     cost qkv_proj about 2.5 % and out_proj about 4 % more.  These
//     whole-row stores are non-temporal, so the output does not push the
//     operand slices out of L2.  out_proj transposes the fp32 sums (32 rows
//     at a time), loads the residual in the same whole-row layout and adds
//     it in fp32 before the one RNE rounding.
//   * tile order: all tiles are ordered in groups of 8 panels (256-row
//     strips), panel fastest within a group.  The 8 XCDs receive workgroup
//     ids round-robin; each XCD owns one eighth of that order (a contiguous
//     range, so its share differs from the others' by at most one tile) and
//     its workgroups take its tiles in turn, so the tiles one XCD runs at a
//     time share a few activation panels and weight slices in its L2.
//   * rows >= M of A are read as row M-1; their results are never stored.
//     The output and the residual go through buffer resources that end at
//     row M of the tile, so the hardware drops the stores of rows >= M and
//     their residual reads return zero.  (Letting such a row store a copy of
//     row M-1 would race with C == R in place: another wave may already have
//     written row M-1 when the copy reads its residual.)
//   * row tables (the padded-bucket path, whose valid rows are scattered
//     over the buckets): row r of the product is row rows[r] of A (without
//     a residual: the copies read A's rows through the table) or of R and C
//     (with one: the epilogue reads the residual and stores the output at
//     per-row offsets, past the buffers' end for rows >= M).  A template
//     parameter: without it the kernel is unchanged.
//     Requires K % 64 == 0 and Nc % BN == 0.
#include "attn_units.hpp"
#include "gs_device.hpp"

namespace gs {

namespace pp {

constexpr int BM = 256;
constexpr int BK = 64;           // K width of a ring stage
constexpr int kCachePolicyNT = 2;  // buffer-store cache policy bit: non-temporal
constexpr int NST = 2;           // ring stages
constexpr int WAVES = 8;
constexpr int THREADS = WAVES * 64;

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// LDS rows are BK = 64 bf16 = 128 B = 8 chunks of 16 B; a 16-byte read is
// served from a 256-byte window of banks (2 rows).  Fragment reads touch 16
// consecutive rows at one logical chunk, so chunk c of row r is stored at
// physical chunk c ^ ((r / 2) mod 8): those rows then hit 16 distinct slots.
__device__ __forceinline__ int swz(int r) { return (r >> 1) & 7; }

// Row tables are read through the constant address space, so that a
// wave-uniform address becomes a scalar load (counted in lgkmcnt, apart from
// the vector-memory count that paces the copies).
#define GS_CONST __attribute__((address_space(4)))
typedef int int8v __attribute__((ext_vector_type(8)));
// e[i] for a per-lane i in 0..7 (a select chain: no dynamic vector index)
__device__ __forceinline__ int pick8(int8v e, int i) {
  int v = e[0];
  v = i == 1 ? e[1] : v;
  v = i == 2 ? e[2] : v;
  v = i == 3 ? e[3] : v;
  v = i == 4 ? e[4] : v;
  v = i == 5 ? e[5] : v;
  v = i == 6 ? e[6] : v;
  v = i == 7 ? e[7] : v;
  return v;
}

// Global->LDS copies of one [ROWS x BK] operand tile per stage by 8 waves:
// copy j of wave w fills LDS rows (j*8 + w)*8 ... +7 (1 KB); lane i writes
// row + i/8 at physical chunk i%8.  Per-lane byte offsets from the tile's
// first row are set once per tile (32-bit: the address is a uniform base plus
// one VGPR).  With CLAMP, rows at or past row_limit read row row_limit-1.
template <int ROWS, bool CLAMP>
struct Copy {
  static constexpr int INSTR = ROWS / 64;  // per wave per stage
  static constexpr int NOFF = CLAMP ? INSTR : 1;
  unsigned off[NOFF];

  __device__ __forceinline__ void init(int row0, int row_limit, int ld, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < NOFF; ++j) {
      const int r = (j * 8 + wave) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      int gr = row0 + r;
      if (CLAMP) gr = gr < row_limit ? gr : row_limit - 1;
      off[j] = (unsigned)((gr - row0) * ld + c * 8) * 2u;
    }
  }
  // Rows through a table (row r of the product is row rows[r] of the
  // operand; rows at or past row_limit read row last_src): offsets from the
  // operand's first row.  The entries of one copy's 8 rows come by one
  // scalar load.
  __device__ __forceinline__ void init_rows(int row0, int row_limit, int ld, int wave, int lane,
                                            const GS_CONST int* rows, int last_src) {
#pragma unroll
    for (int j = 0; j < NOFF; ++j) {
      const int rb = row0 + (j * 8 + wave) * 8;  // uniform
      const int r = (j * 8 + wave) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ swz(r);
      int src = pick8(*(const GS_CONST int8v*)(rows + rb), lane >> 3);
      if (rb + (lane >> 3) >= row_limit) src = last_src;
      off[j] = (unsigned)(src * ld + c * 8) * 2u;
    }
  }
  // copy j of this wave; tile: the tile's first row at this K step (uniform)
  __device__ __forceinline__ void issue(int j, const bf16* tile, int ld, GS_LDS bf16* dst,
                                        int wave) const {
    // (copies j and j+1 are 64 rows apart: the same swizzle, one offset)
    const char* base = (const char*)tile + (CLAMP ? 0 : (size_t)j * 64 * ld * 2);
    copy16_to_lds(base + (CLAMP ? off[j] : off[0]), dst + (j * 8 + wave) * 8 * BK);
  }
};

// vmcnt(n) (gfx9 encoding, expcnt and lgkmcnt at max)
#define PP_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))
// waits until at most n vector-memory ops of this wave are in flight, n
// rounded down to a multiple of 4 (only ever waits longer)
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  switch (n >= 60 ? 15 : (n < 0 ? 0 : n >> 2)) {
    case 0: PP_VMCNT(0); break;    case 1: PP_VMCNT(4); break;
    case 2: PP_VMCNT(8); break;    case 3: PP_VMCNT(12); break;
    case 4: PP_VMCNT(16); break;   case 5: PP_VMCNT(20); break;
    case 6: PP_VMCNT(24); break;   case 7: PP_VMCNT(28); break;
    case 8: PP_VMCNT(32); break;   case 9: PP_VMCNT(36); break;
    case 10: PP_VMCNT(40); break;  case 11: PP_VMCNT(44); break;
    case 12: PP_VMCNT(48); break;  case 13: PP_VMCNT(52); break;
    case 14: PP_VMCNT(56); break;  default: PP_VMCNT(60); break;
  }
}

// Workgroup barrier without the memory fence __syncthreads() adds (the fence
// would wait for every outstanding store and LDS-direct copy).  LDS ordering
// is kept by the explicit waits before it; the empty asm statements keep the
// compiler from moving memory accesses across it, the scheduling barriers
// any other instruction (a matrix product must stay in its phase).
__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
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

}  // namespace pp

// KK: 16-wide k chunks per phase (a stage of 64 k takes 4 / KK phases per
// group).  m_dev: if not null, the row count is read from device memory
// instead of M (M then only bounds the grid), for row counts that exist only
// on the device.
template <int BN, bool RESID, int KK, bool ROWS = false>
__global__ __launch_bounds__(pp::THREADS, 1) void gemm_pp_bf16_kernel(
    const bf16* __restrict__ A, const bf16* __restrict__ W, const bf16* R, bf16* C, int M,
    int Nc, int K, const int* __restrict__ m_dev, const int* __restrict__ rows_table) {
  using namespace pp;
  const int m_cap = M;  // rows the buffers hold (the row count's bound)
  if (m_dev) M = __builtin_amdgcn_readfirstlane(*m_dev);
  // ROWS: a row table maps row r of the product to row rows[r] of A (without
  // a residual) or of R and C (with one); rows at or past M read row
  // rows[M - 1] of A, and their residual reads and stores are dropped.
  const GS_CONST int* rows = (const GS_CONST int*)rows_table;
  int last_src = 0;
  if constexpr (ROWS) {
    if (M > 0) last_src = rows[M - 1];
  }
  using CopyA = Copy<BM, true>;   // activation rows: the last panel is ragged
  using CopyB = Copy<BN, false>;  // weight rows: Nc % BN == 0
  constexpr int WN = BN / 4;      // wave tile columns
  constexpr int TI = 4;           // 32-row MFMA tiles per wave (128 rows)
  constexpr int TJ = WN / 32;     // 32-column MFMA tiles per wave
  constexpr int NSUB = 4 / KK;    // load/product phase pairs per stage
  constexpr int A_ELEMS = BM * BK;
  constexpr int STAGE = (BM + BN) * BK;
  constexpr int LPS = CopyA::INSTR + CopyB::INSTR;  // copies per wave per stage
  constexpr int NOUT = TI * TJ * 2;                 // 16-byte output pieces per lane per tile
  static_assert(BN % 128 == 0 || BN == 384, "tile width");
  static_assert((KK == 1 || KK == 2) && WN % 32 == 0, "phase and tile shape");
  static_assert(WN == 64, "the output transpose writes 128-byte wave rows");
  // 8 KB per wave of a group after the ring, for the transpose of finished
  // pieces into whole output rows
  constexpr int XT_ELEMS = 4 * 4096;
  __shared__ __attribute__((aligned(1024))) bf16 smem[NST * STAGE + XT_ELEMS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int grp = wave >> 2;  // waves w and w+4 share a SIMD: different groups
  const int wm = wave & 1, wn = wave >> 1;
  const int frag_row = lane & 31;
  const int half = lane >> 5;

  const int mt_count = (M + BM - 1) / BM;
  const int nt_count = Nc / BN;
  const int KT = K / BK;  // stages per tile

  // ---- tile order ----
  // k-th tile of this workgroup as (panel, column tile), or panel = -1.
  const int Gs = gridDim.x;
  const bool by_xcd = (Gs & 7) == 0 && mt_count >= 8;  // else: plain round-robin over tiles
  const int xcd = blockIdx.x & 7;
  const long long all_tiles = (long long)mt_count * nt_count;
  const int t_lo = by_xcd ? (int)((xcd * all_tiles) >> 3) : 0;
  const int t_hi = by_xcd ? (int)(((xcd + 1) * all_tiles) >> 3) : (int)all_tiles;
  const int slot0 = by_xcd ? (int)(blockIdx.x >> 3) : (int)blockIdx.x;
  const int per = by_xcd ? (Gs >> 3) : Gs;
  const int x_tiles = t_hi - t_lo;
  auto tile_of = [&](int k, int& panel, int& col) __attribute__((always_inline)) {
    const int u = slot0 + k * per;
    if (u >= x_tiles) {
      panel = -1;
      col = 0;
      return;
    }
    const int g = t_lo + u;
    const int grp8 = g / (8 * nt_count);
    const int v = g - grp8 * 8 * nt_count;
    const int gp = min(8, mt_count - grp8 * 8);
    col = v / gp;
    panel = grp8 * 8 + (v - col * gp);
  };

  auto stage_a = [&](int st) { return (GS_LDS bf16*)&smem[st * STAGE]; };
  auto stage_b = [&](int st) { return (GS_LDS bf16*)&smem[st * STAGE + A_ELEMS]; };

  // ---- copy side: the next (tile, stage) to issue ----
  // Every stage issues LPS copies per wave.  Past the end of the stream the
  // copy side keeps re-reading its last stage into the freed slot (never
  // read), so the number of operations between two waits never changes.
  int ops = 0;  // vector-memory ops this wave has issued
  int is_k = 0, is_step = 0, is_panel, is_col, is_slot = 0;
  tile_of(0, is_panel, is_col);
  if (is_panel < 0) return;  // uniform: no work for this workgroup
  CopyA cpA;
  CopyB cpB;
  const bf16* tA = nullptr;
  const bf16* tB = nullptr;
  auto set_issue_tile = [&]() __attribute__((always_inline)) {
    if constexpr (ROWS && !RESID) {
      tA = A;
      tB = W + (size_t)is_col * BN * K;
      cpA.init_rows(is_panel * BM, M, K, wave, lane, rows, last_src);
    } else {
      tA = A + (size_t)is_panel * BM * K;
      tB = W + (size_t)is_col * BN * K;
      cpA.init(is_panel * BM, M, K, wave, lane);
    }
    cpB.init(is_col * BN, Nc, K, wave, lane);
  };
  set_issue_tile();
  // copies c0 .. c1-1 of the stage being issued (activation rows first); the
  // last batch of a stage moves the cursor on
  auto issue_copies = [&](int c0, int c1) __attribute__((always_inline)) {
#pragma unroll
    for (int c = c0; c < c1; ++c) {
      if (c < CopyA::INSTR)
        cpA.issue(c, tA + is_step * BK, K, stage_a(is_slot), wave);
      else
        cpB.issue(c - CopyA::INSTR, tB + is_step * BK, K, stage_b(is_slot), wave);
    }
    ops += c1 - c0;
    if (c1 == LPS) {
      is_slot ^= 1;
      if (is_step + 1 < KT) {
        ++is_step;
      } else {
        int np, nc;
        tile_of(is_k + 1, np, nc);
        if (np >= 0) {  // (else: stay on the last stage)
          ++is_k;
          is_step = 0;
          is_panel = np;
          is_col = nc;
          set_issue_tile();
        }
      }
    }
  };

  // ---- fragments of sub-step u of a stage (k chunks u*KK .. u*KK+KK-1) ----
  // Fragment rows are (multiple of 32) + lane%32, and 32-row shifts keep the
  // swizzle, so an address is a per-lane chunk offset plus a compile-time row
  // offset.
  bf16x8 af[KK][TI], bfr[KK][TJ];
  auto read_frags = [&](int st, int u) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
      const int lo = frag_row * BK + (((u * KK + kk) * 2 + half) ^ swz(frag_row)) * 8;
      const GS_LDS bf16* as = stage_a(st) + wm * 128 * BK + lo;
      const GS_LDS bf16* bs = stage_b(st) + wn * WN * BK + lo;
#pragma unroll
      for (int i = 0; i < TI; ++i) af[kk][i] = *(const GS_LDS bf16x8*)(as + i * 32 * BK);
#pragma unroll
      for (int j = 0; j < TJ; ++j) bfr[kk][j] = *(const GS_LDS bf16x8*)(bs + j * 32 * BK);
    }
  };

  f32x16 acc[TI][TJ];
  // the products of a half stage; the first of a tile starts from zero
  auto compute = [&](bool first) __attribute__((always_inline)) {
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              bfr[kk][j], af[kk][i], (first && kk == 0) ? f32x16{} : acc[i][j], 0, 0, 0);
  };

  // ---- output ----
  // acc[i][j] is the transposed 32x32 tile: register g*4+e holds row lane%32
  // and column g*8 + (lane/32)*4 + e.  For column groups g = 2gp and 2gp+1,
  // the swap leaves lane l (< 32) with all 8 columns of group 2gp and lane
  // l+32 with all 8 of group 2gp+1: piece (i, j, gp) of a lane is row
  // wm*128 + i*32 + lane%32, columns wn*WN + j*32 + gp*16 + (lane/32)*8 .. +7.
  // With a row table and a residual: one byte offset per access k (row
  // 8k + lane / 8 of this wave's 128 rows of the finished tile) from the
  // start of R and C, past the buffers' end for rows >= M.  The table
  // entries come by vector loads at the start of the tile-boundary phase,
  // before its copies, so that waiting for them never waits for the copies
  // (scalar loads would each need 8 SGPRs and run one after another).
  constexpr bool SCATTER = ROWS && RESID;
  unsigned roff[SCATTER ? NOUT : 1];
  auto load_rows = [&](int m0, int n0) __attribute__((always_inline)) {
    if constexpr (SCATTER) {
      int src[NOUT];
#pragma unroll
      for (int k = 0; k < NOUT; ++k) src[k] = rows_table[m0 + wm * 128 + 8 * k + (lane >> 3)];
#pragma unroll
      for (int k = 0; k < NOUT; ++k)
        roff[k] = m0 + wm * 128 + 8 * k + (lane >> 3) < M
                      ? (unsigned)(src[k] * Nc + n0 + wn * WN + (lane & 7) * 8) * 2u
                      : 0xFFFFFFF0u;
    }
  };
  auto store_tile = [&](int m0, int n0) __attribute__((always_inline)) {
    m0 = __builtin_amdgcn_readfirstlane(m0);
    n0 = __builtin_amdgcn_readfirstlane(n0);
    // bytes from the tile's origin to the end of its last row below M
    const unsigned tile_bytes = (unsigned)(min(M - m0, BM) * Nc - n0) * 2u;
    // Whole-row addressing: 16-byte piece lane % 8 of row 8k + lane / 8 of
    // the wave's 128 rows; one per-lane offset, the row step in the uniform
    // soffset.  Each access covers 8 whole 128-byte rows.
    const unsigned st_base =
        (unsigned)((wm * 128 + (lane >> 3)) * Nc + wn * WN + (lane & 7) * 8) * 2u;
    // the output (and residual) through buffers over the tile's rows below
    // M, or over all M_cap rows of C (and R) with a row table
    auto rows_rsrc = [&](const bf16* base) __attribute__((always_inline)) {
      if constexpr (SCATTER)
        return buffer_rsrc(base, (unsigned)((size_t)m_cap * Nc * 2));
      else
        return buffer_rsrc(base + (size_t)m0 * Nc + n0, tile_bytes);
    };
    const auto out_rs = rows_rsrc(C);
    // the residual rows, all loaded first (the fragments are dead here)
    u32x4_t rres[RESID ? NOUT : 1];
    if constexpr (RESID) {
      const auto res_rs = rows_rsrc(R);
      if constexpr (SCATTER) {
#pragma unroll
        for (int k = 0; k < NOUT; ++k)
          rres[k] = __builtin_amdgcn_raw_buffer_load_b128(res_rs, roff[k], 0, 0);
      } else {
#pragma unroll
        for (int k = 0; k < NOUT; ++k)
          rres[k] = __builtin_amdgcn_raw_buffer_load_b128(res_rs, st_base, k * 8 * Nc * 2, 0);
      }
    }
    // The wave transposes its pieces through its own 8 KB LDS area: it reads
    // only what it wrote itself (LDS keeps one wave's accesses in order), and
    // the other group uses the area only after the next barrier.  The
    // stores are non-temporal (cache policy nt): a round of tiles writes as
    // much output per XCD as its L2 holds, and with the default policy those
    // lines pushed out the operand slices the next tiles read.
    GS_LDS u32x4_t* xt = (GS_LDS u32x4_t*)&smem[NST * STAGE] + (wave & 3) * 512;
    if constexpr (!RESID) {
      // bf16, 64 rows at a time: rows of 8 pieces, piece c of row r at
      // c ^ (r mod 8), so the 32 rows a write touches and the 8 pieces a
      // read takes hit distinct banks.
#pragma unroll
      for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
          for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int gp = 0; gp < 2; ++gp) {
              const f32x16& a = acc[h * 2 + ii][j];
              unsigned x0 = pack_bf16x2(a[gp * 8 + 0], a[gp * 8 + 1]);
              unsigned x1 = pack_bf16x2(a[gp * 8 + 2], a[gp * 8 + 3]);
              unsigned y0 = pack_bf16x2(a[gp * 8 + 4], a[gp * 8 + 5]);
              unsigned y1 = pack_bf16x2(a[gp * 8 + 6], a[gp * 8 + 7]);
              swap_lo_hi(x0, y0);
              swap_lo_hi(x1, y1);
              const int r = ii * 32 + frag_row;
              const int c8 = j * 4 + gp * 2 + half;
              xt[r * 8 + (c8 ^ (r & 7))] = u32x4_t{x0, x1, y0, y1};
            }
#pragma unroll
        for (int s = 0; s < 8; ++s) {
          const int r = s * 8 + (lane >> 3);
          const int c8 = lane & 7;
          const u32x4_t v = xt[r * 8 + (c8 ^ (r & 7))];
          __builtin_amdgcn_raw_buffer_store_b128(v, out_rs, st_base, (h * 64 + s * 8) * Nc * 2,
                                                 kCachePolicyNT);
        }
      }
    } else {
      // fp32, 32 rows at a time (the residual is added to the unrounded
      // sums): rows of 16 four-column chunks, chunk c of row r at
      // c ^ (r mod 16), so the 16 rows of a write and the 2 x 8 chunks of a
      // read hit distinct banks.
#pragma unroll
      for (int i = 0; i < TI; ++i) {
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
          for (int gp = 0; gp < 2; ++gp) {
            const f32x16& a = acc[i][j];
            unsigned x[4], y[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              // (through float copies: clang lowers a bit cast of a vector
              // element as a read of element 0)
              const float fx = a[gp * 8 + e], fy = a[gp * 8 + 4 + e];
              x[e] = __builtin_bit_cast(unsigned, fx);
              y[e] = __builtin_bit_cast(unsigned, fy);
              swap_lo_hi(x[e], y[e]);
            }
            // columns 0..3 of the piece are x[0..3] (chunk c), 4..7 are y[0..3]
            const int r = frag_row;
            const int c = (j * 4 + gp * 2 + half) * 2;
            xt[r * 16 + (c ^ (r & 15))] = u32x4_t{x[0], x[1], x[2], x[3]};
            xt[r * 16 + ((c + 1) ^ (r & 15))] = u32x4_t{y[0], y[1], y[2], y[3]};
          }
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int r = s * 8 + (lane >> 3);
          const int c = (lane & 7) * 2;
          const u32x4_t lo = xt[r * 16 + (c ^ (r & 15))];
          const u32x4_t hi = xt[r * 16 + ((c + 1) ^ (r & 15))];
          const u32x4_t rv = rres[i * 4 + s];
          // the 8 sums as plain words (columns 0..7 of the piece)
          const unsigned v[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          unsigned w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            // bf16 pair of the residual: columns 2e, 2e+1 of the piece
            const unsigned re = rv[e];
            const float r0 = __builtin_bit_cast(float, re << 16);
            const float r1 = __builtin_bit_cast(float, re & 0xFFFF0000u);
            const float v0 = __builtin_bit_cast(float, v[2 * e]);
            const float v1 = __builtin_bit_cast(float, v[2 * e + 1]);
            w[e] = pack_bf16x2(v0 + r0, v1 + r1);
          }
          const u32x4_t piece = u32x4_t{w[0], w[1], w[2], w[3]};
          if constexpr (SCATTER)
            __builtin_amdgcn_raw_buffer_store_b128(piece, out_rs, roff[i * 4 + s], 0,
                                                   kCachePolicyNT);
          else
            __builtin_amdgcn_raw_buffer_store_b128(piece, out_rs, st_base,
                                                   (i * 32 + s * 8) * Nc * 2, kCachePolicyNT);
        }
      }
    }
    ops += NOUT + (RESID ? NOUT : 0);
  };

  // ---- phases ----
  // Sub-step q (counted over the whole stream) belongs to stage S = q / NSUB,
  // which lives in ring slot S % 2.  Group g reads its fragments of q in
  // phase 2q + g - 1 and runs its products in phase 2q + g, so stage S is
  // read in phases 2 NSUB S - 1 .. 2 NSUB (S + 1) - 2.  Stage S + 1 goes to
  // the slot of stage S - 1, last read in phase 2 NSUB S - 2; a wave issues
  // its copies of it in its load phases of the first NSUB - 1 sub-steps of S
  // and waits for them at the end of its last load phase of S, before the
  // first read of S + 1.
  issue_copies(0, LPS);  // stage 0
  wait_vmem();
  barrier();
  if (grp == 1) barrier();  // group 1 starts one phase later

  int rd_slot = 0;
  int mark = 0;  // ops right after this wave's copies of the next stage
  int k = 0, panel, col;
  tile_of(0, panel, col);
  int m0p = 0, n0p = 0;
  bool have_prev = false;
  // one stage of the tile; FIRST: its products start from zero and the
  // previous tile's output leaves in the first load phase (after that
  // phase's copies)
  auto run_stage = [&](bool first) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < NSUB; ++u) {
      if (SCATTER && u == 0 && first && have_prev) load_rows(m0p, n0p);
      if (u < NSUB - 1) {
        constexpr int NB = NSUB - 1;
        issue_copies(u * LPS / NB, (u + 1) * LPS / NB);
        if (u == NB - 1) mark = ops;
      }
      if (u == 0 && first && have_prev) store_tile(m0p, n0p);
      read_frags(rd_slot, u);
      wait_lds();
      if (u == NSUB - 1)  // the next stage has landed (this wave's copies)
        wait_vmcnt_le(__builtin_amdgcn_readfirstlane(ops - mark));
      barrier();
      compute(first && u == 0);
      barrier();
    }
    rd_slot ^= 1;
  };
  for (;;) {
    run_stage(true);
    for (int kt = 1; kt < KT; ++kt) run_stage(false);
    m0p = panel * BM;
    n0p = col * BN;
    have_prev = true;
    tile_of(++k, panel, col);
    if (panel < 0) break;
  }
  load_rows(m0p, n0p);
  store_tile(m0p, n0p);
  if (grp == 0) barrier();  // as many barriers as group 1
  wait_vmem();
}
#undef PP_VMCNT

// Host-side launchers ------------------------------------------------------

static int g_pp_cus = 0;

static int pp_persistent_grid(int tiles) {
  if (g_pp_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_pp_cus = n;
  }
  return tiles < g_pp_cus ? tiles : g_pp_cus;
}

int gemm_tail_tile_rows(int rows, int Nc);
hipError_t launch_gemm_tail_bf16(const void* A, const void* W, const void* R, void* C, int rows,
                                 int Nc, int K, int bm, hipStream_t stream,
                                 const UnitTableJob* job);

// Load balance: 256 x 256 tiles over the CUs leave a partial last round,
// which a few CUs would run while the others wait.  The panels (256-row
// strips) that fill whole rounds run as the persistent launch; the rows
// after them run as a second launch of one round of small tiles (BM x 128,
// BM chosen so that every tile has a CU of its own), if such a round can
// hold them.  Returns the first row of that second part (M when one launch
// is kept, 0 when the small tiles take all rows) and its row tile in
// *tail_bm.  For M = 55093 on 256 CUs: the projection (12 tiles per panel)
// runs 213 panels in 10 rounds, then 565 rows as 216 tiles of 64 x 128;
// out_proj (4 tiles per panel) runs 192 panels in 3 rounds, then 6144 rows
// as 256 tiles of 192 x 128.  With fewer 256 x 256 tiles than CUs (a short
// batch) the round of small tiles takes every row when it fits: for
// M = 800 the projection runs 168 tiles of 128 x 128 instead of 48 large
// ones, out_proj 104 tiles of 64 x 128 instead of 16.
static int pp_split_rows(int M, int Nc, int* tail_bm) {
  const int tiles_per_panel = Nc / 256;
  const int mt = (M + pp::BM - 1) / pp::BM;
  const int cus = pp_persistent_grid(1 << 30);
  const long long tiles = (long long)mt * tiles_per_panel;
  const long long rounds = tiles / cus;
  *tail_bm = 0;
  if (rounds < 1) {
    const int bm = gemm_tail_tile_rows(M, Nc);
    if (bm == 0) return M;
    *tail_bm = bm;
    return 0;
  }
  if (tiles % cus == 0) return M;
  const int main_panels = (int)(rounds * cus / tiles_per_panel);
  const int rest = M - main_panels * pp::BM;
  if (rest <= 0) return M;
  const int bm = gemm_tail_tile_rows(rest, Nc);
  if (bm == 0) return M;
  *tail_bm = bm;
  return main_panels * pp::BM;
}

// m_dev (optional): the row count on the device, at most M; one launch then.
// job (optional): a unit-table build, run by one more workgroup of the
// small-tile launch if there is one (*job_done then set).
template <bool RESID>
static hipError_t pp_launch(const bf16* A, const bf16* W, const bf16* R, bf16* C, int M, int Nc,
                            int K, hipStream_t stream, const int* m_dev = nullptr,
                            const UnitTableJob* job = nullptr, bool* job_done = nullptr) {
  auto launch = [&](int rows, const int* md) {
    const int mt = (rows + pp::BM - 1) / pp::BM;
    hipLaunchKernelGGL((gemm_pp_bf16_kernel<256, RESID, 2>),
                       dim3(pp_persistent_grid(mt * (Nc / 256))), dim3(pp::THREADS), 0, stream, A,
                       W, R, C, rows, Nc, K, md, nullptr);
  };
  if (m_dev) {
    launch(M, m_dev);
    return hipGetLastError();
  }
  int tail_bm = 0;
  const int m1 = pp_split_rows(M, Nc, &tail_bm);
  hipError_t e = hipSuccess;
  if (m1 > 0) {
    launch(m1, nullptr);
    e = hipGetLastError();
  }
  if (e != hipSuccess || m1 == M) return e;
  const size_t a_off = (size_t)m1 * K, c_off = (size_t)m1 * Nc;
  e = launch_gemm_tail_bf16(A + a_off, W, RESID ? R + c_off : nullptr, C + c_off, M - m1, Nc, K,
                            tail_bm, stream, job);
  if (e == hipSuccess && job && job_done) *job_done = true;
  return e;
}

// Through a row table (row r of the product is row rows[r] of the operand
// named below), with the row count m_dev on the device, at most M: one
// launch.  Without R: C[r] = A[rows[r]] . W^T.  With R: C[rows[r]] =
// R[rows[r]] + A[r] . W^T (M rows of R and C then lie anywhere among M_cap).
// rows needs ceil(M / 256) * 256 readable entries, 32-byte aligned; byte
// offsets into A (without R) or into R and C (with R) must fit 32 bits:
// M_cap * Nc * 2 (with R) or M_cap * K * 2 (without) below 2^32 - 16.
hipError_t launch_gemm_nt_bf16_pp_rows(const void* A, const void* W, const void* R, void* C,
                                       int M, int M_cap, int Nc, int K, const int* m_dev,
                                       const int* rows, hipStream_t stream) {
  const int mt = (M + pp::BM - 1) / pp::BM;
  const dim3 grid(pp_persistent_grid(mt * (Nc / 256)));
  if (R)
    hipLaunchKernelGGL((gemm_pp_bf16_kernel<256, true, 2, true>), grid, dim3(pp::THREADS), 0,
                       stream, (const bf16*)A, (const bf16*)W, (const bf16*)R, (bf16*)C, M_cap,
                       Nc, K, m_dev, rows);
  else
    hipLaunchKernelGGL((gemm_pp_bf16_kernel<256, false, 2, true>), grid, dim3(pp::THREADS), 0,
                       stream, (const bf16*)A, (const bf16*)W, (const bf16*)nullptr, (bf16*)C,
                       M_cap, Nc, K, m_dev, rows);
  return hipGetLastError();
}

hipError_t launch_qkv_proj_bf16_pp(const void* x, const void* wqkv, void* qkv, int M, int d,
                                   hipStream_t stream, const UnitTableJob* job, bool* job_done) {
  // 3d = 384 * heads is a multiple of 256 for an even head count
  return pp_launch<false>((const bf16*)x, (const bf16*)wqkv, nullptr, (bf16*)qkv, M, 3 * d, d,
                          stream, nullptr, job, job_done);
}

hipError_t launch_out_proj_bf16_pp(const void* o, const void* wo, const void* x, void* out, int M,
                                   int d, hipStream_t stream) {
  return pp_launch<true>((const bf16*)o, (const bf16*)wo, (const bf16*)x, (bf16*)out, M, d, d,
                         stream);
}

// C[M][Nc] = A[M][K] . W[Nc][K]^T (+ R[M][Nc] when R is not null), for any
// Nc % 256 == 0 and K % 64 == 0 (the window cross-attention's projections).
// m_dev (optional): rows counted on the device (at most M).
hipError_t launch_gemm_nt_bf16_pp(const void* A, const void* W, const void* R, void* C, int M,
                                  int Nc, int K, hipStream_t stream, const int* m_dev) {
  if (R)
    return pp_launch<true>((const bf16*)A, (const bf16*)W, (const bf16*)R, (bf16*)C, M, Nc, K,
                           stream, m_dev);
  return pp_launch<false>((const bf16*)A, (const bf16*)W, nullptr, (bf16*)C, M, Nc, K, stream,
                          m_dev);
}

}  // namespace gs
