// attn_bf16.hip -- block-local bidirectional attention on gfx950 (bf16 in/out,
// fp32 softmax and accumulation).
//
// For every block (<= B consecutive rows of one sequence; blocks restart at
// each cu_seqlens boundary, the last one is partial) and head h:
//   O_h = softmax(Q_h K_h^T / sqrt(128)) V_h
// reading Q|K|V from the projection output qkv[N][3d] and writing O[N][d].
//
// Work item = (unit, head), unit = (block, group of up to 256 query rows),
// taken from a unit table built on the device from cu_seqlens, sorted by cost
// (read here with scalar loads).
//
// Persistent workgroups, one per CU (8 waves), each taking one item per round
// in snake order over the sorted table.  All operands stream through one LDS ring of NST
// stages of 16 KB filled by 16-byte global->LDS direct copies: an item
// contributes its query stages (64 rows each), then its key chunks (32 K
// rows + 32 V rows).  Copies run NST-1 stages ahead of the math, across item
// boundaries, so the memory pipe does not drain between items.  Each wave
// counts its own vector-memory operations, so the wait before a stage allows
// exactly the operations issued after that stage's copies (later copies and
// O stores) to stay in flight.
//
// Math per wave (32 query rows = two 16-row tiles), v_mfma_f32_16x16x32_bf16:
//   * S^T = K Q^T: the K rows of the two 16-key tiles of a chunk are permuted
//     so that a lane's scores for both tiles are 8 consecutive keys -- the P^T
//     operand layout of the PV product; P never leaves registers;
//   * O^T += V^T P^T: the V^T operand is read straight from the row-major V
//     rows with the transposing LDS read ds_read_b64_tr_b16 (per 16-lane
//     group, lane j receives element j%4 of the 8-byte pieces addressed by
//     lanes j/4 + 4s, s = 0..3);
//   * online softmax in base 2 with fp32 running max and sum; the max is
//     reduced across the 4 lane groups holding one query, the sum at the end;
//     P is rounded to bf16 (RNE) for the MFMA and the sum uses the rounded
//     values; O = acc / sum is rounded once to bf16;
//   * rows past the block end are copied from its last row (finite data),
//     keys past it are masked to -inf, and key tiles or query tiles lying
//     wholly past the end are skipped.
#include "attn_units.hpp"

namespace gs {

constexpr int ATT_THREADS = 512;
constexpr int ATT_WAVES = ATT_THREADS / 64;
constexpr int ATT_QG = 256;          // query rows per unit (8 waves x 32)
constexpr int ATT_QS = 64;           // query rows per query stage
constexpr int ATT_KC = 32;           // keys per key chunk
constexpr int DH = 128;
constexpr int ATT_NST = 8;           // ring stages
constexpr int STAGE_ELEMS = 8192;    // 16 KB: 64 rows of 128 bf16
constexpr int COPIES = 2;            // 16-byte copies per lane per stage

// LDS rows are 128 bf16 = 256 B = 16 chunks of 16 B, one full window of the
// 64 four-byte banks; chunk c of row r is stored at physical chunk c ^ swz(r)
// so that each read below touches distinct banks:
//   Q rows: 16 consecutive rows read at one chunk              -> r & 15
//   K rows: the 16 permuted keys of an MFMA tile at one chunk,
//           keys {g*8 + i (+4) : g, i = 0..3}                   -> (k&3) | ((k>>3)&3)<<2
//   V rows: a transposing read takes a chunk pair of 8 keys
//           {g*8 + i : g = 0,1; i = 0..3} per half-wave          -> pair ^ ((k&3) | ((k>>3)&1)<<2)
__device__ __forceinline__ int swz_q(int r) { return r & 15; }
__device__ __forceinline__ int swz_k(int k) { return (k & 3) | (((k >> 3) & 3) << 2); }
__device__ __forceinline__ int swz_v(int k) { return ((k & 3) | (((k >> 3) & 1) << 2)) << 1; }

// Chunk-relative key that row r of 16-key MFMA tile kt feeds.
__device__ __forceinline__ int perm_key(int kt, int r) {
  return (kt >> 1) * 32 + (r >> 2) * 8 + (kt & 1) * 4 + (r & 3);
}

// Four transposing LDS reads (ds_read_b64_tr_b16) and a wait for them, in one
// asm block, so the results are complete when it ends.  (Through the builtin,
// the compiler makes every such read wait for all in-flight global->LDS
// copies, which would drain the ring; ordering against those copies is
// enforced by the explicit waits and barriers of the stream loop.)
__device__ __forceinline__ void lds_read_tr_x4(const GS_LDS bf16* const* p, bf16x8* out) {
  typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
  unsigned long long r[4];
  unsigned a[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = (unsigned)(uintptr_t)p[i];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %4\n\t"
      "ds_read_b64_tr_b16 %1, %5\n\t"
      "ds_read_b64_tr_b16 %2, %6\n\t"
      "ds_read_b64_tr_b16 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3])
      : "memory");
  out[0] = __builtin_bit_cast(bf16x8, u64x2{r[0], r[1]});
  out[1] = __builtin_bit_cast(bf16x8, u64x2{r[2], r[3]});
}

// Max / sum of a value over the lane pairs (l, l^32) and (l, l^16), with the
// gfx950 cross-lane swaps (VALU, no LDS round trip).  Each swap leaves, in
// every lane, the lane's own value and its partner's in the two results.
__device__ __forceinline__ float xmax_lanes32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xmax_lanes16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xsum_lanes32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xsum_lanes16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// The softmax reference max moves only when a row max exceeds it by more than
// this many doublings (P stays <= 2^8, well inside bf16 and fp32 range).
constexpr float LAZY_RESCALE = 8.f;

// Workgroup barrier without a memory fence.  A fence would make every wave
// wait for all of its outstanding global->LDS copies and global stores; the
// stream loop instead waits explicitly for exactly the copies it needs.  This
// wave's own LDS reads are complete before it arrives (wait_lds), and the
// empty asm with a memory clobber keeps the compiler from moving memory
// accesses across the barrier.
__device__ __forceinline__ void stream_barrier() {
  wait_lds();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Wait until at most n of this wave's vector-memory operations are pending
// (n rounded down to even and capped at 30, which only waits longer).
#define GS_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  switch (n >= 30 ? 15 : (n < 0 ? 0 : n >> 1)) {
    case 0: GS_VMCNT(0); break;    case 1: GS_VMCNT(2); break;
    case 2: GS_VMCNT(4); break;    case 3: GS_VMCNT(6); break;
    case 4: GS_VMCNT(8); break;    case 5: GS_VMCNT(10); break;
    case 6: GS_VMCNT(12); break;   case 7: GS_VMCNT(14); break;
    case 8: GS_VMCNT(16); break;   case 9: GS_VMCNT(18); break;
    case 10: GS_VMCNT(20); break;  case 11: GS_VMCNT(22); break;
    case 12: GS_VMCNT(24); break;  case 13: GS_VMCNT(26); break;
    case 14: GS_VMCNT(28); break;  default: GS_VMCNT(30); break;
  }
}
#undef GS_VMCNT

// Position in a workgroup's stream of stages.  Items are taken in snake
// order over the cost-sorted unit table: round r gives this workgroup the
// item at position r*G + w (even r) or r*G + G-1-w (odd r).
struct Cursor {
  int r;       // round
  int v;       // work item (unit position * heads + head)
  bool valid;  // false past the workgroup's last item
  int row0, L, q0, qn, h;
  int s;       // stage index inside the item
  int nq, ns;  // query stages, all stages
};

__device__ __forceinline__ void cursor_load(Cursor& c, const int4* __restrict__ table, int items,
                                            int heads) {
  c.v = c.r * (int)gridDim.x + ((c.r & 1) ? (int)gridDim.x - 1 - (int)blockIdx.x : (int)blockIdx.x);
  c.valid = c.v < items;
  c.s = 0;
  if (c.valid) {
    const int u = c.v / heads;
    const int4 e = table[1 + u];  // wave-uniform address: scalar load
    c.h = c.v - u * heads;
    c.row0 = e.x; c.L = e.y; c.q0 = e.z; c.qn = e.w;
    c.nq = (c.qn + ATT_QS - 1) / ATT_QS;
    c.ns = c.nq + (c.L + ATT_KC - 1) / ATT_KC;
  }
}

__device__ __forceinline__ void cursor_next(Cursor& c, const int4* __restrict__ table, int items,
                                            int heads) {
  if (++c.s == c.ns) {
    ++c.r;
    cursor_load(c, table, items, heads);
  }
}

__global__ __launch_bounds__(ATT_THREADS, 1) void block_attn_bf16_kernel(
    const bf16* __restrict__ qkv, const int4* __restrict__ table, int heads, int d,
    float scale_log2, bf16* __restrict__ O) {
  __shared__ __attribute__((aligned(1024))) bf16 ring[ATT_NST * STAGE_ELEMS];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int ld = 3 * d;
  const int g4 = lane >> 4;   // lane group
  const int l16 = lane & 15;
  const int items = table[0].x * heads;

  // Vector-memory ops this wave has issued, and that count right after the
  // copies of stream positions p .. p+NST-2 (a shift register, no indexing).
  int ops = 0;
  int mark[ATT_NST - 1];
#pragma unroll
  for (int i = 0; i < ATT_NST - 1; ++i) mark[i] = 0;

  // ---- copies of one stage into ring slot `slot` --------------------------
  // 16 KB = 16 wave copies of 1 KB (4 rows of 256 B); wave w does copies w and
  // w+8; lane -> row r0 + lane/16, physical chunk lane%16.
  auto issue = [&](const Cursor& c, int slot) __attribute__((always_inline)) {
    GS_LDS bf16* dst = (GS_LDS bf16*)&ring[slot * STAGE_ELEMS];
    const int pc = lane & 15;
    if (c.s < c.nq) {  // query stage: 64 rows
      const int q0 = c.q0 + c.s * ATT_QS;
      const int qlast = c.q0 + c.qn - 1;
#pragma unroll
      for (int j = 0; j < COPIES; ++j) {
        const int r0 = (j * ATT_WAVES + wave) * 4;
        const int rr = r0 + (lane >> 4);
        int q = q0 + rr;
        q = q <= qlast ? q : qlast;
        const int lc = pc ^ swz_q(rr);
        copy16_to_lds(qkv + (size_t)(c.row0 + q) * ld + c.h * DH + lc * 8, dst + r0 * DH);
      }
    } else {           // key chunk: 32 K rows (copy 0) then 32 V rows (copy 1)
      const int k0 = (c.s - c.nq) * ATT_KC;
#pragma unroll
      for (int j = 0; j < COPIES; ++j) {
        const bool isv = j == 1;
        const int r0 = (j * ATT_WAVES + wave) * 4;
        const int kr = (r0 + (lane >> 4)) & (ATT_KC - 1);
        int key = k0 + kr;
        key = key < c.L ? key : c.L - 1;
        const int lc = pc ^ (isv ? swz_v(kr) : swz_k(kr));
        copy16_to_lds(qkv + (size_t)(c.row0 + key) * ld + (isv ? 2 * d : d) + c.h * DH + lc * 8,
                      dst + r0 * DH);
      }
    }
    ops += COPIES;
  };

  // ---- stream -------------------------------------------------------------------
  // Copies run AHEAD = NST-2 stages ahead: the slot of the previous stage stays
  // resident for one more iteration, because its PV product is done then.
  constexpr int AHEAD = ATT_NST - 2;
  Cursor comp, iss;
  comp.r = 0;
  cursor_load(comp, table, items, heads);
  if (!comp.valid) return;  // uniform over the workgroup
  iss = comp;
#pragma unroll
  for (int s = 0; s < AHEAD; ++s) {
    if (iss.valid) {
      issue(iss, s);
      cursor_next(iss, table, items, heads);
    }
    mark[s] = ops;
  }

  // per-wave query state: rows 32*wave + 16*tt + lane%16 of the current item
  bf16x8 qf[2][4];
  f32x4 oacc[2][8];
  // Running row sums of P, kept by the matrix unit: lsum[tt] += 1 * P^T, so
  // each of the four values of a lane holds the sum for query lane%16.
  f32x4 lsum[2];
  // reference max per query in log2 units, and the raw score above which it
  // has to move: thr = (mref + LAZY_RESCALE) / scale_log2
  float mref[2] = {0.f, 0.f}, thr[2] = {INFINITY, INFINITY};
  bool tval[2] = {false, false};
  bool fresh = false;         // the next key chunk is its item's first
  bf16x8 pprev[2];            // P of the previous key chunk; its PV product is pending
  bool pend = false;
  int pslot = 0;
  bool fin = false;           // the pending chunk was its item's last: store O after its PV
  bool fval0 = false, fval1 = false;
  // (wave-uniform) first O row of this wave's query tiles in that item, its
  // head, and the item's rows from that first row on
  int fin_row = 0, fin_h = 0, fin_n = 0;
  const float inv_scale_log2 = 1.f / scale_log2;
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (bf16)1.f;

  // Per-lane LDS byte offsets inside a stage (the slot base is added per stage).
  //   K: row perm_key(kt, lane%16) at chunk kc*4 + lane/16; tile kt = 1 is 4
  //      rows (1 KB) further on with the same swizzle.
  //   V: rows g4*8 + r*4 + lane%16/4 at dh (quarter*2+q)*16 + 4*(lane%16%4);
  //      r = 1 is 4 rows further on with the same swizzle.
  unsigned koff[4], voff[8];
  {
    const int kr = perm_key(0, l16);
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) koff[kc] = (unsigned)(kr * DH + ((kc * 4 + g4) ^ swz_k(kr)) * 8) * 2u;
    const int vr = g4 * 8 + (l16 >> 2);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int e0 = j * 16 + 4 * (l16 & 3);
      voff[j] = (unsigned)(ATT_KC * DH + vr * DH + (((e0 >> 3) ^ swz_v(vr)) * 8) + (e0 & 7)) * 2u;
    }
  }
  const unsigned ring_base = (unsigned)(uintptr_t)(GS_LDS bf16*)ring;

  // O^T += V^T P^T and lsum += 1 P^T for the pending chunk.  The V^T fragment
  // (16 dh x 32 keys) of dh tile dt is two transposing reads; four reads per
  // asm block.
  auto pv_pending = [&]() __attribute__((always_inline)) {
    const unsigned vb = ring_base + (unsigned)pslot * (STAGE_ELEMS * 2);
#pragma unroll
    for (int quarter = 0; quarter < 4; ++quarter) {
      const GS_LDS bf16* va[4];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int r = 0; r < 2; ++r)
          va[q * 2 + r] = (const GS_LDS bf16*)(uintptr_t)(vb + voff[quarter * 2 + q] + r * (4 * DH * 2));
      bf16x8 vf[2];
      lds_read_tr_x4(va, vf);
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int dt = quarter * 2 + q;
        oacc[0][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[q], pprev[0], oacc[0][dt], 0, 0, 0);
        if (tval[1])
          oacc[1][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[q], pprev[1], oacc[1][dt], 0, 0, 0);
      }
    }
    lsum[0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pprev[0], lsum[0], 0, 0, 0);
    if (tval[1]) lsum[1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pprev[1], lsum[1], 0, 0, 0);
  };
  // normalise and store the finished item's O (8 stores per valid tile)
  auto store_fin = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      if (tt == 0 ? !fval0 : !fval1) continue;
      const float inv = 1.f / lsum[tt][0];
      if (tt * 16 + l16 < fin_n) {
        bf16* op = O + (size_t)(fin_row + tt * 16 + l16) * d + fin_h * DH + g4 * 4;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
          bf16x4 o;
          o[0] = to_bf16(oacc[tt][dt][0] * inv);
          o[1] = to_bf16(oacc[tt][dt][1] * inv);
          o[2] = to_bf16(oacc[tt][dt][2] * inv);
          o[3] = to_bf16(oacc[tt][dt][3] * inv);
          *(bf16x4*)(op + dt * 16) = o;
        }
      }
      ops += 8;  // issued: lane l16 = 0 of a valid tile is in range
    }
  };

  for (int p = 0; comp.valid; ++p) {
    const int slot = p & (ATT_NST - 1);
    // this stage's copies (and everything before them) have landed
    wait_vmcnt_le(__builtin_amdgcn_readfirstlane(ops - mark[0]));
    stream_barrier();  // everyone's landed; everyone is done with stage p-2
    if (iss.valid) {
      issue(iss, (p + AHEAD) & (ATT_NST - 1));  // refill the slot of stage p-2
      cursor_next(iss, table, items, heads);
    }
#pragma unroll
    for (int i = 0; i < AHEAD - 1; ++i) mark[i] = mark[i + 1];
    mark[AHEAD - 1] = ops;  // position p+AHEAD (if issued; otherwise never waited for)
    const unsigned sb = ring_base + (unsigned)slot * (STAGE_ELEMS * 2);
    const GS_LDS bf16* st = (const GS_LDS bf16*)&ring[slot * STAGE_ELEMS];
    const bool kstage = comp.s >= comp.nq;
    const bool work = kstage && tval[0];

    // ---- S^T = K Q^T for this chunk (32 keys) ----
    // Tile kt row r feeds key perm_key(kt, r), so a lane holds keys
    // g4*8 + kt*4 + i.  Tile 1 holds keys {4..7, 12..15, 20..23, 28..31}: it
    // has a valid key iff kvalid > 4.
    const int kvalid = min(ATT_KC, comp.L - (comp.s - comp.nq) * ATT_KC);
    f32x4 s[2][2];
    if (work) {
      const bool two = kvalid > 4;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        s[0][kt] = s[1][kt] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (kt == 0 || two) {
          bf16x8 kf[4];
#pragma unroll
          for (int kc = 0; kc < 4; ++kc)
            kf[kc] = *(const GS_LDS bf16x8*)(uintptr_t)(sb + koff[kc] + kt * (4 * DH * 2));
#pragma unroll
          for (int kc = 0; kc < 4; ++kc)
            s[0][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kc], qf[0][kc], s[0][kt], 0, 0, 0);
          if (tval[1]) {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc)
              s[1][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kc], qf[1][kc], s[1][kt], 0, 0, 0);
          }
        }
      }
    }

    // ---- the previous chunk's PV product (its V rows are still resident) and,
    // if that chunk finished an item, the item's output ----
    if (pend) {
      pv_pending();
      pend = false;
    }
    if (fin) {
      store_fin();
      fin = false;
    }

    if (!kstage) {
      // ---- query stage: the waves owning these 64 rows load their tiles ----
      const int wfirst = comp.s * (ATT_QS / 32);  // 2 waves per query stage
      if (comp.s == 0) {
        tval[0] = tval[1] = false;
        fresh = true;
      }
      if (wave >= wfirst && wave < wfirst + ATT_QS / 32) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          const int rr = (wave - wfirst) * 32 + tt * 16 + l16;
          tval[tt] = (wave * 32 + tt * 16) < comp.qn;
#pragma unroll
          for (int kc = 0; kc < 4; ++kc) {
            const int lc = kc * 4 + g4;
            qf[tt][kc] = *(const GS_LDS bf16x8*)(st + rr * DH + (lc ^ swz_q(rr)) * 8);
          }
        }
      }
    } else if (work) {
      // ---- softmax of this chunk ----
      if (kvalid < ATT_KC) {  // masked keys (a block's partial last chunk) get -inf
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (g4 * 8 + kt * 4 + i >= kvalid) s[tt][kt][i] = -INFINITY;
      }
      // this lane's max raw score per query tile
      float lmax[2];
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
        lmax[tt] = fmaxf(fmaxf(fmaxf(s[tt][0][0], s[tt][0][1]), fmaxf(s[tt][0][2], s[tt][0][3])),
                         fmaxf(fmaxf(s[tt][1][0], s[tt][1][1]), fmaxf(s[tt][1][2], s[tt][1][3])));
      // Lazy rescaling: the reference max only moves when some score exceeds
      // it by more than 2^LAZY_RESCALE (the previous chunk's PV is already in
      // O), so P <= 2^LAZY_RESCALE and the common case needs no cross-lane
      // reduction and leaves O alone.  An item's first chunk sets it.
      const bool grow = (lmax[0] > thr[0]) | (lmax[1] > thr[1]);
      if (fresh || __builtin_amdgcn_ballot_w64(grow) != 0) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          // the chunk's row max over the 4 lane groups of a query
          const float cmax = xmax_lanes16(xmax_lanes32(lmax[tt])) * scale_log2;
          const float mnew = fresh ? cmax : fmaxf(mref[tt], cmax);
          const float alpha = __builtin_amdgcn_exp2f(mref[tt] - mnew);
          mref[tt] = mnew;
          thr[tt] = (mnew + LAZY_RESCALE) * inv_scale_log2;
          if (fresh) {  // the accumulators still hold the previous item's values
            lsum[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) oacc[tt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
          } else {
            lsum[tt] *= alpha;
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) oacc[tt][dt] *= alpha;
          }
        }
        fresh = false;
      }
      // P = exp2(s*scale - mref), rounded to bf16, in the PV operand layout
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            pprev[tt][kt * 4 + i] =
                to_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(s[tt][kt][i], scale_log2, -mref[tt])));
      pend = true;
      pslot = slot;
      if (comp.s == comp.ns - 1) {  // the item is done once this chunk's PV is in
        fin = true;
        fval0 = tval[0];
        fval1 = tval[1];
        fin_row = comp.row0 + comp.q0 + wave * 32;
        fin_h = comp.h;
        fin_n = comp.qn - wave * 32;
      }
    }
    cursor_next(comp, table, items, heads);
  }
  // the stream's last chunk
  if (pend) pv_pending();
  if (fin) store_fin();
}

static int g_num_cus = 0;

int attn_bf16_table_entries(long long N) { return (int)(N + 1); }

hipError_t launch_block_attn_bf16(const void* qkv, const int* cu, int S, long long N, int d,
                                  int heads, int B, void* o, void* table, hipStream_t stream) {
  if (g_num_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_num_cus = n;
  }
  build_unit_table_kernel<ATT_QG, ATT_QS, ATT_KC><<<dim3(1), dim3(1024), 0, stream>>>(cu, S, B, (int4*)table);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long items = (long long)attn_unit_bound(N, S, B, ATT_QG) * heads;
  const int grid = items < g_num_cus ? (int)items : g_num_cus;
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)DH);
  hipLaunchKernelGGL(block_attn_bf16_kernel, dim3(grid), dim3(ATT_THREADS), 0, stream,
                     (const bf16*)qkv, (const int4*)table, heads, d, scale_log2, (bf16*)o);
  return hipGetLastError();
}

}  // namespace gs
