// attn_bf16.hip -- block-local bidirectional attention on gfx950 (bf16 in/out,
// fp32 softmax and accumulation).
//
// For every block (<= B consecutive rows of one sequence; blocks restart at
// each cu_seqlens boundary, the last one is partial) and head h:
//   O_h = softmax(Q_h K_h^T / sqrt(128)) V_h
// reading Q|K|V from the projection output qkv[N][3d] and writing O[N][d].
//
// Work item = (unit, head), unit = (block, group of up to 224 query rows),
// taken from a unit table built on the device from cu_seqlens and sorted by
// cost (a math wave reads the entry of the item after next with a vector load one
// item ahead).  Persistent workgroups, one per CU, each
// take one item per round in snake order over the sorted table.
//
// A workgroup is 7 math waves (32 query rows each) and one copy wave:
//   * the copy wave streams the K|V rows of its items, 32 keys per stage,
//     through an LDS ring of 8 stages of 16 KB with 16-byte global->LDS direct
//     copies, 3 stages ahead and across item boundaries, and waits for each
//     stage's copies before the stage's workgroup barrier; the math waves
//     never issue ring copies (a copy issued behind a saturated memory pipe
//     holds its wave for hundreds of cycles);
//   * a math wave loads the Q fragments of its rows of the next item into a
//     second register set with plain global loads while the current item
//     runs.
//
// Math per math wave and key chunk, v_mfma_f32_16x16x32_bf16:
//   * S^T = K Q^T: the K rows of the two 16-key tiles of a chunk are permuted
//     so that a lane's scores for both tiles are 8 consecutive keys -- the P^T
//     operand layout of the PV product; P never leaves registers;
//   * O^T += V^T P^T: the V^T operand is read straight from the row-major V
//     rows with the transposing LDS read ds_read_b64_tr_b16; the row sums of
//     P come from the same product with an all-ones operand;
//   * softmax in base 2 against a per-row reference set at the item's first
//     chunk (an integer: the ceiling of that chunk's row max); later scores
//     may exceed it: P then carries an exact power-of-two factor, rounds to
//     bf16 as it would against the true max, and cancels in O = acc / sum.
//     When a chunk's scores run more than 2^32 above a row's reference, the
//     reference rises to that chunk's ceiling and the accumulated O, sum and
//     pending P are scaled by the exact power of two between the two (rare
//     at unit-variance logits, common in deep unnormalised stacks).  An item
//     whose row sums or accumulators still end non-finite is flagged and
//     recomputed exactly at the end of the kernel;
//   * P is rounded to bf16 (RNE) for the MFMA and the sums use the rounded
//     values; O = acc / sum is rounded once to bf16;
//   * rows past the block end are copies of its last row (finite data) and
//     keys past it are masked to -inf.
#include <type_traits>

#include "attn_units.hpp"

namespace gs {

constexpr int ATT_WAVES = 8;         // 7 math waves and one copy wave
constexpr int ATT_PRODUCER = ATT_WAVES - 1;
constexpr int ATT_THREADS = ATT_WAVES * 64;
constexpr int ATT_QT = 2;            // 16-row query tiles per math wave
constexpr int ATT_QW = 16 * ATT_QT;  // query rows per math wave
constexpr int ATT_QG = ATT_PRODUCER * ATT_QW;  // query rows per unit (7 waves x 32)
constexpr int ATT_KC = 32;           // keys per key chunk
constexpr float ATT_HEADROOM = 32.f;  // log2 margin of a score over its row's reference
constexpr int DH = 128;
constexpr int ATT_NST = 8;           // ring stages
constexpr int ATT_AHEAD = 3;         // copies run this many stages ahead (<= 63 in flight)
constexpr int STAGE_ELEMS = 8192;    // 16 KB: 64 rows of 128 bf16
constexpr int COPIES = 16;           // 1 KB wave copies per stage, all by the copy wave

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

// The V^T operands of one key chunk: sixteen transposing LDS reads
// (ds_read_b64_tr_b16) and a wait for them, in one asm block, so the results
// are complete when it ends.  Fragment dt is the pair of reads at a[dt] and
// a[dt] + 1 KB (the second group of four V rows).  (Through the builtin, the
// compiler makes every such read wait for all in-flight global->LDS copies,
// which would drain the ring; ordering against those copies is enforced by
// the explicit waits and barriers of the stream loop.)
__device__ __forceinline__ void lds_read_vt_chunk(const unsigned* a, bf16x8* out) {
  typedef unsigned long long u64x2 __attribute__((ext_vector_type(2)));
  unsigned long long r[16];
  asm volatile(
      "ds_read_b64_tr_b16 %0, %16\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:1024\n\t"
      "ds_read_b64_tr_b16 %2, %17\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:1024\n\t"
      "ds_read_b64_tr_b16 %4, %18\n\t"
      "ds_read_b64_tr_b16 %5, %18 offset:1024\n\t"
      "ds_read_b64_tr_b16 %6, %19\n\t"
      "ds_read_b64_tr_b16 %7, %19 offset:1024\n\t"
      "ds_read_b64_tr_b16 %8, %20\n\t"
      "ds_read_b64_tr_b16 %9, %20 offset:1024\n\t"
      "ds_read_b64_tr_b16 %10, %21\n\t"
      "ds_read_b64_tr_b16 %11, %21 offset:1024\n\t"
      "ds_read_b64_tr_b16 %12, %22\n\t"
      "ds_read_b64_tr_b16 %13, %22 offset:1024\n\t"
      "ds_read_b64_tr_b16 %14, %23\n\t"
      "ds_read_b64_tr_b16 %15, %23 offset:1024\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]), "=&v"(r[14]), "=&v"(r[15])
      : "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(a[4]), "v"(a[5]), "v"(a[6]), "v"(a[7])
      : "memory");
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) out[dt] = __builtin_bit_cast(bf16x8, u64x2{r[2 * dt], r[2 * dt + 1]});
}

// Scores of two query tiles against the two 16-key tiles of a chunk:
// s[t][kt] = sum over kc of K[kt][kc] Q[t][kc] (16x16x32 bf16 products, four
// chained per tile, interleaved so that dependent products are four apart),
// with the results in VGPRs for the VALU softmax that reads them.  (Left to
// the compiler, every product of a kernel that may use more than 256
// registers gets an AGPR destination, and each score would be moved out
// again.)  The chains accumulate in place; the wait states at the end cover
// a VALU read or write of a result right after the block (XDL write, then
// VALU access of the same VGPRs: 4 passes + 4 on gfx950).
__device__ __forceinline__ void score_tiles2(const bf16x8 (*k)[4], const bf16x8* q0, const bf16x8* q1,
                                             f32x4& s00, f32x4& s01, f32x4& s10, f32x4& s11) {
  asm volatile(
      "v_mfma_f32_16x16x32_bf16 %0, %4, %12, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %8, %12, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %4, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %8, %16, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %5, %13, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %9, %13, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %5, %17, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %9, %17, %3\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %6, %14, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %10, %14, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %6, %18, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %10, %18, %3\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %7, %15, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %11, %15, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %2, %7, %19, %2\n\t"
      "v_mfma_f32_16x16x32_bf16 %3, %11, %19, %3\n\t"
      "s_nop 7\n\t"
      "s_nop 7\n\t"
      "s_nop 3"
      : "=&v"(s00), "=&v"(s01), "=&v"(s10), "=&v"(s11)
      : "v"(k[0][0]), "v"(k[0][1]), "v"(k[0][2]), "v"(k[0][3]), "v"(k[1][0]), "v"(k[1][1]),
        "v"(k[1][2]), "v"(k[1][3]), "v"(q0[0]), "v"(q0[1]), "v"(q0[2]), "v"(q0[3]), "v"(q1[0]),
        "v"(q1[1]), "v"(q1[2]), "v"(q1[3]));
}

// One query tile against the two 16-key tiles of a chunk (as score_tiles2).
__device__ __forceinline__ void score_tiles1(const bf16x8 (*k)[4], const bf16x8* q0, f32x4& s00, f32x4& s01) {
  asm volatile(
      "v_mfma_f32_16x16x32_bf16 %0, %2, %10, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %6, %10, 0\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %3, %11, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %7, %11, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %4, %12, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %8, %12, %1\n\t"
      "v_mfma_f32_16x16x32_bf16 %0, %5, %13, %0\n\t"
      "v_mfma_f32_16x16x32_bf16 %1, %9, %13, %1\n\t"
      "s_nop 7\n\t"
      "s_nop 7\n\t"
      "s_nop 3"
      : "=&v"(s00), "=&v"(s01)
      : "v"(k[0][0]), "v"(k[0][1]), "v"(k[0][2]), "v"(k[0][3]), "v"(k[1][0]), "v"(k[1][1]),
        "v"(k[1][2]), "v"(k[1][3]), "v"(q0[0]), "v"(q0[1]), "v"(q0[2]), "v"(q0[3]));
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
// (n rounded down to even and capped at 62, which only waits longer).
#define GS_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))
__device__ __forceinline__ void wait_vmcnt_le(int n) {
  switch (n >= 62 ? 31 : (n < 0 ? 0 : n >> 1)) {
    case 0: GS_VMCNT(0); break;
    case 1: GS_VMCNT(2); break;
    case 2: GS_VMCNT(4); break;
    case 3: GS_VMCNT(6); break;
    case 4: GS_VMCNT(8); break;
    case 5: GS_VMCNT(10); break;
    case 6: GS_VMCNT(12); break;
    case 7: GS_VMCNT(14); break;
    case 8: GS_VMCNT(16); break;
    case 9: GS_VMCNT(18); break;
    case 10: GS_VMCNT(20); break;
    case 11: GS_VMCNT(22); break;
    case 12: GS_VMCNT(24); break;
    case 13: GS_VMCNT(26); break;
    case 14: GS_VMCNT(28); break;
    case 15: GS_VMCNT(30); break;
    case 16: GS_VMCNT(32); break;
    case 17: GS_VMCNT(34); break;
    case 18: GS_VMCNT(36); break;
    case 19: GS_VMCNT(38); break;
    case 20: GS_VMCNT(40); break;
    case 21: GS_VMCNT(42); break;
    case 22: GS_VMCNT(44); break;
    case 23: GS_VMCNT(46); break;
    case 24: GS_VMCNT(48); break;
    case 25: GS_VMCNT(50); break;
    case 26: GS_VMCNT(52); break;
    case 27: GS_VMCNT(54); break;
    case 28: GS_VMCNT(56); break;
    case 29: GS_VMCNT(58); break;
    case 30: GS_VMCNT(60); break;
    default: GS_VMCNT(62); break;
  }
}
#undef GS_VMCNT

// Position in a workgroup's stream of stages.  Items are dealt in snake
// order over the cost-sorted unit table: round r gives workgroup w the item
// at position r*G + w (even r) or r*G + G-1-w (odd r).  Odd workgroups run
// their items in the reverse order: each workgroup keeps the same items and
// the same total, but half of them then start with their cheapest items, so
// item ends (each workgroup stores 56 KB of O there) do not fall on all CUs
// at once.  Workgroups w and w + 8 sit on the same XCD and, in a round, run
// the same head of consecutive units (the query groups of one long block
// share its K|V in that XCD's L2); both run in the same direction.
struct Cursor {
  int r;       // round
  int v;       // work item (unit position * heads + head)
  bool valid;  // false past the workgroup's last item
  int row0, L, q0, qn, h;
  int s;       // key chunk inside the item
  int ns;      // key chunks of the item
};

__device__ __forceinline__ void cursor_index(Cursor& c, int items) {
  const int G = (int)gridDim.x, w = (int)blockIdx.x;
  int r = c.r;
  if (w & 1) {  // reversed: this workgroup's rounds counted from its last
    const int rl = items / G;                          // the last, partial round
    const int sl = (rl & 1) ? G - 1 - w : w;           // this workgroup's slot in it
    const int R = rl + (rl * G + sl < items ? 1 : 0);  // this workgroup's item count
    r = R - 1 - r;
  }
  c.v = r < 0 ? items : r * G + ((r & 1) ? G - 1 - w : w);
  c.valid = c.v < items;
  c.s = 0;
}

// The item's fields from its unit's table entry e.
__device__ __forceinline__ void cursor_fill(Cursor& c, int4 e, int heads) {
  c.h = c.v - (c.v / heads) * heads;
  c.row0 = e.x; c.L = e.y; c.q0 = e.z; c.qn = e.w;
  c.ns = (c.L + ATT_KC - 1) / ATT_KC;
}

__device__ __forceinline__ void cursor_load(Cursor& c, const int4* __restrict__ table, int items,
                                            int heads) {
  cursor_index(c, items);
  if (c.valid) cursor_fill(c, table[1 + c.v / heads], heads);  // uniform address: scalar load
}

__device__ __forceinline__ void cursor_next(Cursor& c, const int4* __restrict__ table, int items,
                                            int heads) {
  if (++c.s == c.ns) {
    ++c.r;
    cursor_load(c, table, items, heads);
  }
}

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(unsigned, bf16x2{to_bf16(a), to_bf16(b)});
}

// v_permlane16_swap: x's odd 16-lane groups trade places with y's even ones.
__device__ __forceinline__ void swap_row_pairs(unsigned& x, unsigned& y) {
  const auto s = __builtin_amdgcn_permlane16_swap(x, y, false, false);
  x = s[0];
  y = s[1];
}

// Exact attention for one item (unit u of the table, head h) whose row sums
// or accumulators overflowed against its reference (a chunk's scores ran
// about 100 doublings or more above it within one chunk of the reference's
// last rise; never seen with logits of ordinary size).  Two passes over the keys per query row: the row
// max, then P with the rounding of the fast path (reference = ceil of the row
// max in log2 units, P rounded to bf16, the sum taken over the rounded values)
// and O = sum_j P_j V_j / sum_j P_j, rounded once to bf16.  Each rounded P is
// scaled by 2^-ceil(log2 L) before the sums (exact, and it cancels in the
// ratio): P <= 1 then keeps both sums within the largest |V| and within 1, so
// V anywhere in the fp32 range cannot overflow them.  Waves w0, w0 + nw, ...
// of the calling waves take one query row each; pbuf holds 64 floats per
// calling wave.
__device__ __forceinline__ float exact_dot(const bf16* __restrict__ a, const bf16* __restrict__ b) {
  float acc = 0.f;
#pragma unroll 4
  for (int t = 0; t < DH; t += 8) {
    const bf16x8 x = *(const bf16x8*)(a + t);
    const bf16x8 y = *(const bf16x8*)(b + t);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc = __builtin_fmaf(to_f32(x[i]), to_f32(y[i]), acc);
  }
  return acc;
}

__device__ void exact_item(const bf16* __restrict__ qkv, int4 e, int h, int d, float scale_log2,
                           bf16* __restrict__ O, int w0, int nw, float* pbuf) {
  const int lane = threadIdx.x & 63;
  const int ld = 3 * d;
  const int row0 = e.x, L = e.y, q0 = e.z, qn = e.w;
  const bf16* kbase = qkv + (size_t)row0 * ld + d + h * DH;
  const bf16* vbase = qkv + (size_t)row0 * ld + 2 * d + h * DH;
  const int lg = L > 1 ? 32 - __builtin_clz((unsigned)(L - 1)) : 0;  // ceil(log2 L)
  const float pscale = __builtin_bit_cast(float, (unsigned)(127 - lg) << 23);  // 2^-lg
  for (int i = w0; i < qn; i += nw) {
    const bf16* q = qkv + (size_t)(row0 + q0 + i) * ld + h * DH;
    float mx = -INFINITY;
    for (int j = lane; j < L; j += 64) mx = fmaxf(mx, exact_dot(q, kbase + (size_t)j * ld));
    for (int off = 32; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
    const float mref = __builtin_ceilf(mx * scale_log2);
    float o0 = 0.f, o1 = 0.f, psum = 0.f;  // this lane's dims 2*lane, 2*lane + 1
    for (int j0 = 0; j0 < L; j0 += 64) {
      const int j = j0 + lane;
      float pj = 0.f;
      if (j < L)
        pj = to_f32(to_bf16(__builtin_amdgcn_exp2f(
                 __builtin_fmaf(exact_dot(q, kbase + (size_t)j * ld), scale_log2, -mref)))) *
             pscale;
      psum += pj;
      pbuf[lane] = pj;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int jn = min(64, L - j0);
      for (int t = 0; t < jn; ++t) {
        const float pt = pbuf[t];
        const bf16* v = vbase + (size_t)(j0 + t) * ld + 2 * lane;
        o0 = __builtin_fmaf(pt, to_f32(v[0]), o0);
        o1 = __builtin_fmaf(pt, to_f32(v[1]), o1);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    for (int off = 32; off > 0; off >>= 1) psum += __shfl_xor(psum, off);
    const float inv = 1.f / psum;
    bf16* op = O + (size_t)(row0 + q0 + i) * d + h * DH + 2 * lane;
    op[0] = to_bf16(o0 * inv);
    op[1] = to_bf16(o1 * inv);
  }
}

// Items a workgroup flagged are listed in LDS (up to this many; beyond that
// every item of the workgroup is checked against the flag words).
constexpr int ATT_FLIST = 64;

__global__ __launch_bounds__(ATT_THREADS, 1) void block_attn_bf16_kernel(
    const bf16* __restrict__ qkv, int4* __restrict__ table, unsigned long long* __restrict__ ovf,
    int heads, int d, float scale_log2, bf16* __restrict__ O) {
  __shared__ __attribute__((aligned(1024))) bf16 ring[ATT_NST * STAGE_ELEMS];
  __shared__ int flist[1 + ATT_FLIST];          // count, then flagged item ids
  __shared__ float pbuf[ATT_PRODUCER][64];      // the exact path's P, per math wave

  const int lane = threadIdx.x & 63;
  if (threadIdx.x == 0) flist[0] = 0;  // (ordered before any use by the first barrier)
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

  // ---- copies of one stage into ring slot `slot` (the copy wave) ----------
  // 16 KB = 16 wave copies of 1 KB (4 rows of 256 B); lane -> row r0 +
  // lane/16, physical chunk lane%16.  In a key stage rows 0..31 are the
  // chunk's K rows and rows 32..63 its V rows.
  // Addresses are a workgroup-uniform base (the block's first row in the
  // part and head being copied) plus a 32-bit byte offset per lane, the form
  // the copy instruction takes with the base in SGPRs (cheaper to issue than
  // a 64-bit address per lane).
  // Lane byte offsets of the 16 copies of a chunk relative to its first K
  // (copies 0..7) or V (copies 8..15) row, for chunks wholly inside the
  // block: the same for every chunk (set up by the copy wave only).
  unsigned koff_c[COPIES / 2], voff_c[COPIES / 2];
  auto issue = [&](const Cursor& c, int slot) __attribute__((always_inline)) {
    GS_LDS bf16* dst = (GS_LDS bf16*)&ring[slot * STAGE_ELEMS];
    const int k0 = __builtin_amdgcn_readfirstlane(c.s * ATT_KC);
    const int brow = __builtin_amdgcn_readfirstlane(c.row0);
    const int hcol = __builtin_amdgcn_readfirstlane(c.h * DH);
    const char* kb = (const char*)(qkv + (size_t)brow * ld + d + hcol);
    const char* vb = kb + (size_t)d * 2;
    if (k0 + ATT_KC <= c.L) {  // a full chunk: uniform base + fixed lane offsets
      const size_t c0 = (size_t)k0 * ld * 2;
      // (the empty asm keeps each offset a 32-bit value at its use, so the copy
      // takes the SGPR-base form)
#pragma unroll
      for (int j = 0; j < COPIES / 2; ++j) {
        unsigned o = koff_c[j];
        asm volatile("" : "+v"(o));
        copy16_to_lds(kb + c0 + o, dst + j * 4 * DH);
      }
#pragma unroll
      for (int j = 0; j < COPIES / 2; ++j) {
        unsigned o = voff_c[j];
        asm volatile("" : "+v"(o));
        copy16_to_lds(vb + c0 + o, dst + (ATT_KC + j * 4) * DH);
      }
    } else {  // the block's partial last chunk: keys past its end repeat its last row
      // (the chunk's first key goes into the 64-bit base: key * ld can pass
      // 2^31 in a long block, the distance from k0 cannot)
      const int pc = lane & 15;
      const size_t c0 = (size_t)k0 * ld * 2;
#pragma unroll
      for (int j = 0; j < COPIES; ++j) {
        const int r0 = j * 4;
        const bool isv = r0 >= ATT_KC;
        const int kr = (r0 + (lane >> 4)) & (ATT_KC - 1);
        int key = k0 + kr;
        key = key < c.L ? key : c.L - 1;
        const int lc = pc ^ (isv ? swz_v(kr) : swz_k(kr));
        copy16_to_lds((isv ? vb : kb) + c0 + (unsigned)((key - k0) * ld + lc * 8) * 2u,
                      dst + r0 * DH);
      }
    }
    ops += COPIES;
  };

  // ---- stream -------------------------------------------------------------------
  // The copy wave runs AHEAD stages ahead of the math waves; at the start of
  // stage p it has waited for stage p's copies and then refills the slot of
  // stage p - (NST - AHEAD) (the math waves read the slots of p and p-1).
  constexpr int AHEAD = ATT_AHEAD;
  const bool producer = wave == ATT_PRODUCER;
  Cursor comp, iss;
  comp.r = 0;
  cursor_load(comp, table, items, heads);
  if (!comp.valid) return;  // uniform over the workgroup
  if (producer) {
    // ---- the copy wave: one barrier per stream position, like the math waves
#pragma unroll
    for (int j = 0; j < COPIES / 2; ++j) {
      const int kr = j * 4 + (lane >> 4);
      koff_c[j] = (unsigned)(kr * ld + ((lane & 15) ^ swz_k(kr)) * 8) * 2u;
      voff_c[j] = (unsigned)(kr * ld + ((lane & 15) ^ swz_v(kr)) * 8) * 2u;
    }
    iss = comp;
#pragma unroll
    for (int s = 0; s < AHEAD; ++s) {
      if (iss.valid) {
        issue(iss, s);
        cursor_next(iss, table, items, heads);
      }
      mark[s] = ops;
    }
    for (int p = 0; comp.valid; ++p) {
      wait_vmcnt_le(__builtin_amdgcn_readfirstlane(ops - mark[0]));  // stage p has landed
      stream_barrier();  // ... for everyone; everyone is done with stage p-2
      if (iss.valid) {
        issue(iss, (p + AHEAD) & (ATT_NST - 1));
        cursor_next(iss, table, items, heads);
      }
#pragma unroll
      for (int i = 0; i < AHEAD - 1; ++i) mark[i] = mark[i + 1];
      mark[AHEAD - 1] = ops;  // position p+AHEAD (if issued; otherwise never waited for)
      cursor_next(comp, table, items, heads);
    }
    stream_barrier();  // the math waves' closing barrier (every copy it issued has landed)
    return;
  }

  // Row slot of a math wave: its 32 rows of an item are rslot*32 ... The wave
  // that shares its SIMD with the copy wave (wave 3) takes the last slot, which
  // a 200-frame block leaves mostly empty (and then runs one query tile).
  const int rslot = wave == 3 ? ATT_PRODUCER - 1 : (wave > 3 ? wave - 1 : wave);

  // ---- query rows: a math wave loads the fragments of its rows of the next
  // item straight from global memory while the current item runs, and moves
  // them to its working set at the end of the current item's last product,
  // before that item's output stores (the wait for the loads then never
  // waits for stores).  The loads are unconditional -- rows past the unit
  // read its last row -- so that no copy of an older value, with a wait for
  // every load in flight, lands on the item boundary. ----
  bf16x8 qnext[ATT_QT][4];
  auto load_q = [&](const Cursor& c) __attribute__((always_inline)) {
    const int qlast = c.qn - 1;
    const bf16* blk = qkv + (size_t)(c.row0 + c.q0) * ld + c.h * DH + g4 * 8;
#pragma unroll
    for (int tt = 0; tt < ATT_QT; ++tt) {
      int r = rslot * ATT_QW + tt * 16 + l16;
      r = r <= qlast ? r : qlast;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) qnext[tt][kc] = *(const bf16x8*)(blk + (size_t)r * ld + kc * 32);
    }
  };
  // ---- per-wave query state: rows ATT_QW*rslot + 16*tt + lane%16 of the item ----
  // Working set <- the loaded fragments.  The empty asm makes the working set
  // a value of its own, defined at this point: a plain copy would turn into a
  // register copy at the end of the loop, after the stores, with its wait,
  // and the loads' registers would carry their pending state into the loop.
  bf16x8 qf[ATT_QT][4];
  auto take_q = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int tt = 0; tt < ATT_QT; ++tt)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) asm volatile("" : "=v"(qf[tt][kc]) : "0"(qnext[tt][kc]));
  };
  load_q(comp);
  take_q();

  // ---- items ahead: the next item's cursor, and the table entry of the one
  // after it, loaded with a vector load at the start of an item (an address
  // the compiler sees as per-lane) and read out at the point above, so that
  // no scalar-load latency falls on the item boundary ----
  Cursor nxt;
  nxt.r = comp.r + 1;
  cursor_load(nxt, table, items, heads);
  int vzero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(vzero));
  int4 epre;
  int e2x = 0, e2y = 0, e2z = 0, e2w = 0;  // the entry after the next item's (uniform)
  // working set <- next item's Q; entry after next -> SGPRs
  auto take_next = [&]() __attribute__((always_inline)) {
    take_q();
    e2x = __builtin_amdgcn_readfirstlane(epre.x);
    e2y = __builtin_amdgcn_readfirstlane(epre.y);
    e2z = __builtin_amdgcn_readfirstlane(epre.z);
    e2w = __builtin_amdgcn_readfirstlane(epre.w);
  };
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (bf16)1.f;

  // Per-lane LDS byte offsets inside a stage (the slot base is added per stage).
  //   K: row perm_key(kt, lane%16) at chunk kc*4 + lane/16; tile kt = 1 is 4
  //      rows (1 KB) further on with the same swizzle.
  //   V: rows g4*8 + r*4 + lane%16/4 at dh dt*16 + 4*(lane%16%4); r = 1 is 4
  //      rows (1 KB) further on with the same swizzle.
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
  constexpr unsigned STAGE_BYTES = STAGE_ELEMS * 2;

  // Start of stream position p (the copy wave has waited for its copies).
  int p = 0;
  auto stage_begin = [&]() __attribute__((always_inline)) {
    stream_barrier();  // stage p has landed; everyone is done with stage p-2
  };

  // V^T fragments of the chunk in ring slot `sl` (16 dh x 32 keys per dh tile).
  auto read_vt = [&](int sl, bf16x8* vf) __attribute__((always_inline)) {
    const unsigned vb = ring_base + (unsigned)sl * STAGE_BYTES;
    unsigned va[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) va[dt] = vb + voff[dt];
    lds_read_vt_chunk(va, vf);
  };
  // S^T = K Q^T for the chunk in slot `sl`: tile kt row r feeds key
  // perm_key(kt, r), so a lane holds keys g4*8 + kt*4 + i of its query.
  auto scores = [&](auto qtc, int sl, f32x4 (*s)[2]) __attribute__((always_inline)) {
    constexpr int QT = decltype(qtc)::value;
    const unsigned sb = ring_base + (unsigned)sl * STAGE_BYTES;
    bf16x8 kf[2][4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int kc = 0; kc < 4; ++kc)
        kf[kt][kc] = *(const GS_LDS bf16x8*)(uintptr_t)(sb + koff[kc] + kt * (4 * DH * 2));
    if constexpr (QT == 2)
      score_tiles2(kf, qf[0], qf[1], s[0][0], s[0][1], s[1][0], s[1][1]);
    else
      score_tiles1(kf, qf[0], s[0][0], s[0][1]);
  };
  // Masks keys past the block end (a block's partial last chunk).
  auto mask = [&](auto qtc, f32x4 (*s)[2], int kvalid) __attribute__((always_inline)) {
    constexpr int QT = decltype(qtc)::value;
    if (kvalid < ATT_KC) {
#pragma unroll
      for (int tt = 0; tt < QT; ++tt)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (g4 * 8 + kt * 4 + i >= kvalid) s[tt][kt][i] = -INFINITY;
    }
  };
  // ... and returns this lane's max raw score per query tile.
  auto mask_max = [&](auto qtc, f32x4 (*s)[2], int kvalid, float* lmax) __attribute__((always_inline)) {
    constexpr int QT = decltype(qtc)::value;
    mask(qtc, s, kvalid);
#pragma unroll
    for (int tt = 0; tt < QT; ++tt)
      lmax[tt] = fmaxf(fmaxf(fmaxf(s[tt][0][0], s[tt][0][1]), fmaxf(s[tt][0][2], s[tt][0][3])),
                       fmaxf(fmaxf(s[tt][1][0], s[tt][1][1]), fmaxf(s[tt][1][2], s[tt][1][3])));
  };
  // P = exp2(s*scale - mref), rounded to bf16, in the PV operand layout
  auto probs = [&](auto qtc, f32x4 (*s)[2], const float* mref, bf16x8* pn) __attribute__((always_inline)) {
    constexpr int QT = decltype(qtc)::value;
#pragma unroll
    for (int tt = 0; tt < QT; ++tt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          pn[tt][kt * 4 + i] =
              to_bf16(__builtin_amdgcn_exp2f(__builtin_fmaf(s[tt][kt][i], scale_log2, -mref[tt])));
  };

  // ---- items ----
  for (; comp.valid; ) {
    const int nk = comp.ns;
    const int nval = min(ATT_QW, comp.qn - rslot * ATT_QW);  // this wave's query rows
    const int row0 = comp.row0, L = comp.L, q0 = comp.q0, h = comp.h;
    const int uidx = comp.v / heads;  // the unit's position in the table
    // ---- loads for the items ahead: the entry after next, the next item's Q ----
    {
      Cursor t;
      t.r = nxt.r + 1;
      cursor_index(t, items);
      epre = table[1 + (t.valid ? t.v / heads : 0) + vzero];  // (unconditional, as for Q)
    }
    load_q(nxt.valid ? nxt : comp);
    if (nval <= 0) {  // no rows for this wave: only keep the stream going
      for (int kc = 0; kc < nk; ++kc, ++p) stage_begin();
      take_next();
    } else {
      // one or two query tiles (a wave with at most 16 rows skips the second)
      auto run_item = [&](auto qtc) __attribute__((always_inline)) {
        constexpr int QT = decltype(qtc)::value;
        f32x4 oacc[QT][8];
        f32x4 lsum[QT];  // P row sums: lsum[tt] += 1 * P^T (4 copies per lane)
        // Reference max per query: an integer in log2 units, set at the item's
        // first chunk to ceil(that chunk's row max) and raised when a later
        // chunk runs far above it.  Later scores may exceed it: with an
        // integer reference P differs from P against the true row max by an
        // exact power of two, so it rounds to bf16 the same way and the factor
        // cancels in acc / sum, unless something overflows (checked at the end
        // of the item).
        float mref[QT];
        float sthr[QT];    // raw score above which a row's reference rises
        bf16x8 pprev[QT];  // P of the previous chunk, whose PV product is pending
        int pslot;
        // ---- first key chunk: sets the reference, no PV product yet ----
        {
          stage_begin();
          const int sl = p & (ATT_NST - 1);
          f32x4 s[QT][2];
          scores(qtc, sl, s);
          float lmax[QT];
          mask_max(qtc, s, min(ATT_KC, L), lmax);
#pragma unroll
          for (int tt = 0; tt < QT; ++tt) {
            // the chunk's row max over the 4 lane groups of a query
            mref[tt] = __builtin_ceilf(xmax_lanes16(xmax_lanes32(lmax[tt])) * scale_log2);
            sthr[tt] = (mref[tt] + ATT_HEADROOM) / scale_log2;
            lsum[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int dt = 0; dt < 8; ++dt) oacc[tt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          probs(qtc, s, mref, pprev);
          pslot = sl;
          ++p;
        }
        // ---- further key chunks ----
        for (int kc = 1; kc < nk; ++kc, ++p) {
          stage_begin();
          const int sl = p & (ATT_NST - 1);
          f32x4 s[QT][2];
          scores(qtc, sl, s);
          __builtin_amdgcn_sched_barrier(0);
          // V^T of the previous chunk, read while the S products run
          bf16x8 vf[8];
          read_vt(pslot, vf);
          __builtin_amdgcn_sched_barrier(0);
          mask(qtc, s, min(ATT_KC, L - kc * ATT_KC));
          // Lazy rescale: when a row's scores run more than 2^ATT_HEADROOM
          // above its reference, the reference rises to this chunk's
          // ceiling and everything accumulated against the old one (O, the
          // row sum and the pending P) is scaled by the exact power of two
          // between them.  Rare for unit-variance inputs; frequent in deep
          // stacks without normalisation, whose logits grow layer by layer.
          // The test compares the raw scores with a threshold kept per row.
          {
            unsigned grow = 0;  // (bitwise: no short-circuit branches)
#pragma unroll
            for (int tt = 0; tt < QT; ++tt) {
              const float lm =
                  fmaxf(fmaxf(fmaxf(s[tt][0][0], s[tt][0][1]), fmaxf(s[tt][0][2], s[tt][0][3])),
                        fmaxf(fmaxf(s[tt][1][0], s[tt][1][1]), fmaxf(s[tt][1][2], s[tt][1][3])));
              grow |= (unsigned)(lm > sthr[tt]);
            }
            if (__builtin_amdgcn_ballot_w64(grow != 0) != 0) {  // (wave-uniform, rare)
              float lmax[QT];
              mask_max(qtc, s, ATT_KC, lmax);  // (masked keys are -inf already)
#pragma unroll
              for (int tt = 0; tt < QT; ++tt) {
                const float mnew = __builtin_ceilf(xmax_lanes16(xmax_lanes32(lmax[tt])) * scale_log2);
                const float m2 = fmaxf(mref[tt], mnew);
                const float f = __builtin_ldexpf(1.0f, (int)(mref[tt] - m2));
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) oacc[tt][dt] *= f;
                lsum[tt] *= f;
#pragma unroll
                for (int j = 0; j < 8; ++j) pprev[tt][j] = to_bf16(to_f32(pprev[tt][j]) * f);
                mref[tt] = m2;
                sthr[tt] = (m2 + ATT_HEADROOM) / scale_log2;
              }
            }
          }
          // P of this chunk and the previous chunk's PV product
          bf16x8 pn[QT];
          probs(qtc, s, mref, pn);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int tt = 0; tt < QT; ++tt)
              oacc[tt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pprev[tt], oacc[tt][dt], 0, 0, 0);
#pragma unroll
          for (int tt = 0; tt < QT; ++tt)
            lsum[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pprev[tt], lsum[tt], 0, 0, 0);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int tt = 0; tt < QT; ++tt) pprev[tt] = pn[tt];
          pslot = sl;
        }
        // ---- the last chunk's PV product and the item's output ----
        {
          bf16x8 vf[8];
          read_vt(pslot, vf);
#pragma unroll
          for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int tt = 0; tt < QT; ++tt)
              oacc[tt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf[dt], pprev[tt], oacc[tt][dt], 0, 0, 0);
#pragma unroll
          for (int tt = 0; tt < QT; ++tt)
            lsum[tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pprev[tt], lsum[tt], 0, 0, 0);
          take_next();
          // Overflow: a non-finite row sum or accumulator (inf or NaN: all
          // exponent bits set) flags the item for the exact recomputation.
          {
            // (whole vectors are reinterpreted: clang lowers a bit cast of
            // one vector element as a read of element 0)
            unsigned big = 0;
#pragma unroll
            for (int tt = 0; tt < QT; ++tt) {
              big = max(big, __builtin_bit_cast(u32x4, lsum[tt]).x & 0x7fffffffu);
#pragma unroll
              for (int dt = 0; dt < 8; ++dt) {
                const u32x4 u = __builtin_bit_cast(u32x4, oacc[tt][dt]) & 0x7fffffffu;
                big = max(big, max(max(u.x, u.y), max(u.z, u.w)));
              }
            }
            if (__builtin_amdgcn_ballot_w64(big >= 0x7f800000u) != 0 && lane == 0) {
              atomicOr(&ovf[uidx], 1ull << h);
              const int pos = atomicAdd(&flist[0], 1);
              if (pos < ATT_FLIST) flist[1 + pos] = comp.v;
            }
          }
          // O rows, 16 bytes per lane: lane (g4, l16) holds dh dt*16 + 4*g4 ..
          // +3 of its row.  For a pair of tiles dt, dt+1, v_permlane16_swap
          // trades the odd lane groups' dt values for the even groups' dt+1
          // values, so an even group g4 ends with dh dt*16 + 4*g4 .. +7 and an
          // odd group with dh (dt+1)*16 + 4*(g4-1) .. +7: piece k = dt/2 of
          // the lane's row, 16-byte chunk 4k + sg of the row's 16, with
          // sg = (g4 & 1) * 2 + g4 / 2.
          // Stores then write whole 128-byte row halves: lanes l16 and l16^8
          // trade pieces (DPP row_ror:8), so that store (H, b) gives lane
          // (g4, l16) chunk 8H + 4 (l16 / 8) + sg of row (l16 mod 8) + 8b,
          // i.e. 8 rows x 128 bytes per instruction instead of 16 x 64.
          const int orow = row0 + q0 + rslot * ATT_QW;
          const int hb = l16 >> 3;
          const int sg = (g4 & 1) * 2 + (g4 >> 1);
#pragma unroll
          for (int tt = 0; tt < QT; ++tt) {
            if (tt * 16 >= nval) continue;  // wave-uniform
            const float inv = 1.f / lsum[tt][0];
            u32x4 pc[4];
#pragma unroll
            for (int dt = 0; dt < 8; dt += 2) {
              unsigned x0 = pack_bf16x2(oacc[tt][dt][0] * inv, oacc[tt][dt][1] * inv);
              unsigned x1 = pack_bf16x2(oacc[tt][dt][2] * inv, oacc[tt][dt][3] * inv);
              unsigned y0 = pack_bf16x2(oacc[tt][dt + 1][0] * inv, oacc[tt][dt + 1][1] * inv);
              unsigned y1 = pack_bf16x2(oacc[tt][dt + 1][2] * inv, oacc[tt][dt + 1][3] * inv);
              swap_row_pairs(x0, y0);
              swap_row_pairs(x1, y1);
              pc[dt >> 1] = u32x4{x0, x1, y0, y1};
            }
#pragma unroll
            for (int H = 0; H < 2; ++H) {
              // the piece the partner l16^8 stores: 2H + 1 from the lower
              // half, 2H from the upper
              const u32x4 send = hb ? pc[2 * H] : pc[2 * H + 1];
              u32x4 recv;
#pragma unroll
              for (int e = 0; e < 4; ++e)
                recv[e] = (unsigned)__builtin_amdgcn_update_dpp(0, (int)send[e], 0x128, 0xf, 0xf, false);
#pragma unroll
              for (int b = 0; b < 2; ++b) {
                const u32x4 v = hb == b ? pc[2 * H + b] : recv;
                const int rr = tt * 16 + (l16 & 7) + 8 * b;
                if (rr < nval)
                  *(u32x4*)(O + (size_t)(orow + rr) * d + h * DH + (8 * H + 4 * hb + sg) * 8) = v;
              }
            }
          }
        }
    
      };
      if (nval > 16)
        run_item(std::integral_constant<int, 2>{});
      else
        run_item(std::integral_constant<int, 1>{});
    }
    comp = nxt;  // (the compute cursor only moves item by item)
    nxt.r = comp.r + 1;
    cursor_index(nxt, items);
    if (nxt.valid) cursor_fill(nxt, int4{e2x, e2y, e2z, e2w}, heads);
  }
  // ---- items whose scores outran their reference: recompute them exactly ----
  wait_vmcnt_le(0);  // this wave's O stores are done before anyone overwrites them
  stream_barrier();
  const int nflag = flist[0];
  if (nflag == 0) return;
  // Each flagged item's bit is cleared again once it is recomputed, so every
  // launch starts with clear flag words even when it reuses the unit table of
  // an earlier launch (only this workgroup touches the bits of its items;
  // other heads of a unit are other bits).
  if (nflag <= ATT_FLIST) {
    for (int i = 0; i < nflag; ++i) {
      const int v = flist[1 + i];
      const int u = v / heads;
      exact_item(qkv, table[1 + u], v - u * heads, d, scale_log2, O, wave, ATT_PRODUCER, pbuf[wave]);
    }
    if ((int)threadIdx.x < nflag) {
      const int v = flist[1 + threadIdx.x];
      const int u = v / heads;
      atomicAnd(&ovf[u], ~(1ull << (v - u * heads)));
    }
  } else {  // more than the list holds: check every item of this workgroup
    Cursor c;
    c.r = 0;
    for (cursor_load(c, table, items, heads); c.valid; ++c.r, cursor_load(c, table, items, heads)) {
      const int u = c.v / heads;
      if ((__atomic_load_n(&ovf[u], __ATOMIC_RELAXED) >> c.h) & 1) {
        exact_item(qkv, table[1 + u], c.h, d, scale_log2, O, wave, ATT_PRODUCER, pbuf[wave]);
        if (threadIdx.x == 0) atomicAnd(&ovf[u], ~(1ull << c.h));
      }
    }
  }
}

// The unit table as a kernel of its own (one workgroup).
__global__ __launch_bounds__(1024) void build_unit_table_kernel(UnitTableJob j) {
  __shared__ int lds[UNIT_TABLE_LDS_INTS];
  build_unit_table(j, lds);
}

static int g_num_cus = 0;

static int attn_cus() {
  if (g_num_cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    g_num_cus = n;
  }
  return g_num_cus;
}

int attn_bf16_table_entries(long long N) { return (int)(N + 1); }

// Query rows per unit.  A unit normally takes ATT_QG = 224 rows, all 7 math
// waves, two to a SIMD on three of the SIMDs.  When a batch is so short that
// units of 96 rows still give every item a CU of its own (an 800-frame
// sequence: 4 blocks x 8 heads = 32 items of 224 rows, or 96 items of 96,
// 96 and 8 rows), its blocks are cut into 96-row units: three times the
// items on otherwise idle CUs, each with the math waves of query slots 0-2,
// which sit on SIMDs 0-2, one per SIMD, so that no two share a matrix pipe
// (slot 3 would share SIMD 0).  Each 32-row group of queries still runs
// whole on one wave (96 = 3 x 32), so the results are the same bits.  A
// function of the host's sizes only: the table's builder and the attention
// launch agree on it.
static int attn_bf16_qg(long long N, int S, int B, int heads) {
  constexpr int QG_SHORT = 3 * ATT_QW;
  static_assert(QG_SHORT % ATT_QW == 0 && QG_SHORT < ATT_QG, "short-batch unit");
  const long long items = (long long)attn_unit_bound(N, S, B, QG_SHORT) * heads;
  return items <= attn_cus() ? QG_SHORT : ATT_QG;
}

// The unit-table build of a launch over these spans, for another launch to
// run in a spare workgroup (the table in the workspace `table`, then,
// 256-byte aligned, one overflow flag word per unit).
UnitTableJob attn_bf16_table_job(SeqSpans sp, int S, long long N, int B, int heads, void* table) {
  unsigned long long* ovf =
      (unsigned long long*)((char*)table + ((16 * (N + 1) + 255) / 256) * 256);
  return UnitTableJob{sp, S, B, attn_bf16_qg(N, S, B, heads), ATT_KC, (int4*)table, ovf};
}

// build_table = false: `table` already holds the unit table of these spans
// (from an earlier launch), and its flag words are clear (every launch clears
// the bits it sets).
hipError_t launch_block_attn_bf16(const void* qkv, SeqSpans sp, int S, long long N, int d,
                                  int heads, int B, void* o, void* table, hipStream_t stream,
                                  bool build_table) {
  const UnitTableJob job = attn_bf16_table_job(sp, S, N, B, heads, table);
  unsigned long long* ovf = job.flags;
  if (build_table) {
    hipLaunchKernelGGL(build_unit_table_kernel, dim3(1), dim3(1024), 0, stream, job);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const long long units = attn_unit_bound(N, S, B, job.qg);
  const long long items = units * heads;
  const int grid = items < attn_cus() ? (int)items : attn_cus();
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)DH);
  hipLaunchKernelGGL(block_attn_bf16_kernel, dim3(grid), dim3(ATT_THREADS), 0, stream,
                     (const bf16*)qkv, (int4*)table, ovf, heads, d, scale_log2, (bf16*)o);
  return hipGetLastError();
}

}  // namespace gs
