// attn_units.hpp -- work units of the block-attention kernels.
//
// A block is a run of at most B consecutive rows of one sequence; blocks
// restart at every sequence start and the last block of a sequence holds the
// remainder.  A work unit is one block, or a group of at most QG query rows
// of a block when B > QG.  Units are numbered sequence by sequence, block by
// block, and are located on the device from the sequence spans alone.
#pragma once

#include "gs_device.hpp"

namespace gs {

// Where sequence s lives: packed (rows cu[s] .. cu[s+1]-1 of a cu_seqlens
// array) or padded (rows s*T .. s*T + len[s] - 1 of fixed buckets of T rows,
// the rest of the bucket being padding; a length outside [0, T] is clamped).
struct SeqSpans {
  const int* p;  // cu_seqlens [S+1] (stride 0) or lengths [S] (stride T > 0)
  int stride;
  __device__ __forceinline__ int start(int s) const { return stride ? s * stride : p[s]; }
  __device__ __forceinline__ int len(int s) const {
    if (!stride) return p[s + 1] - p[s];
    const int l = p[s];
    return l < 0 ? 0 : (l > stride ? stride : l);
  }
};

struct AttnUnit {
  int row0;   // first row of the block
  int L;      // block length (keys)
  int q0;     // first query row of the unit (block-relative)
  int qn;     // number of query rows
};

// Units of one sequence of `len` rows: full blocks need upb = ceil(B/QG)
// units each, the last block ceil(tail/QG).
template <int QG>
__device__ __forceinline__ int units_of_seq(int len, int B, int upb) {
  if (len <= 0) return 0;
  const int nb = (len - 1) / B + 1;
  const int tail = len - (nb - 1) * B;
  return (nb - 1) * upb + (tail + QG - 1) / QG;
}

// Wave-level search for unit u (every lane gets the result).  Sequences are
// scanned 64 at a time with a wave prefix sum.  False if u is past the end.
template <int QG>
__device__ bool find_unit(SeqSpans sp, int S, int B, int u, AttnUnit& out) {
  const int lane = threadIdx.x & 63;
  const int upb = (B - 1) / QG + 1;
  int base = 0;
  for (int c0 = 0; c0 < S; c0 += 64) {
    const int s = c0 + lane;
    int len = 0;
    if (s < S) len = sp.len(s);
    const int units = units_of_seq<QG>(len, B, upb);
    int incl = units;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const int total = __shfl(incl, 63);
    if (u < base + total) {
      const bool mine = units > 0 && (base + incl - units) <= u && u < base + incl;
      const unsigned long long m = __ballot(mine);
      const int src = __ffsll((long long)m) - 1;
      const int seq = c0 + src;
      const int v = u - (base + __shfl(incl - units, src));
      const int slen = __shfl(len, src);
      const int nb = (slen - 1) / B + 1;
      int j = v / upb;
      if (j > nb - 1) j = nb - 1;
      const int g = v - j * upb;
      out.row0 = sp.start(seq) + j * B;
      out.L = (j < nb - 1) ? B : slen - (nb - 1) * B;
      out.q0 = g * QG;
      out.qn = min(QG, out.L - out.q0);
      return true;
    }
    base += total;
  }
  return false;
}

// Unit table for kernels that read their units with scalar loads.
// table[0] = {number of units, 0, 0, 0};
// table[1 + i] = {row0, L, q0, qn} of the i-th
// unit in order of decreasing cost, the cost being the number of key chunks
// of kc keys a unit takes, ceil(L/kc) (capped at 1023; the order of units of
// equal cost is unspecified).  With the costliest units first, a
// persistent kernel that deals them out in a snake order (round r hands
// position r*G + w to workgroup w for even r, to G-1-w for odd r) keeps its
// workgroups within about one unit of each other.
// Every unit holds at least one row, so N + 1 entries always suffice.  If
// `flags` is not null, flags[i] is cleared for every unit i.
struct UnitTableJob {
  SeqSpans sp;
  int S, B;
  int qg, kc;                       // query rows per unit, keys per chunk
  int4* table;                      // null: nothing to build
  unsigned long long* flags;
};

constexpr int UNIT_BINS = 1024;
constexpr int UNIT_TABLE_LDS_INTS = UNIT_BINS + 16;

// A counting sort over the cost, by one workgroup (blockDim.x a multiple of
// 64 that divides 1024; every thread calls it): a count pass and a
// placement pass over the sequences, blockDim.x sequences at a time.  The
// units of a sequence come in two runs of equal cost (those of its full
// blocks, those of its last block), each counted and placed with one LDS
// atomic.  lds: UNIT_TABLE_LDS_INTS ints.  Not inlined: inside a GEMM
// kernel (the side job of its small-tile launch) the inlined builder
// slowed the GEMM's own code.
static __device__ __attribute__((noinline)) void build_unit_table(UnitTableJob j,
                                                                  int* lds) {
  int* next = lds;                  // per cost bin: count, then next free position
  int* wsum = lds + UNIT_BINS;      // per wave: the count of its threads' bins
  const int T = blockDim.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int per = UNIT_BINS / T;    // bins per thread in the scan
  const int upb = (j.B - 1) / j.qg + 1;
  auto bin_of = [&](int L) {  // bin 0 holds the costliest units
    const int cost = (L + j.kc - 1) / j.kc;
    return UNIT_BINS - 1 - min(cost, UNIT_BINS - 1);
  };
  auto put = [&](int pos, int row0, int L, int g) {
    j.table[1 + pos] = make_int4(row0, L, g * j.qg, min(j.qg, L - g * j.qg));
    if (j.flags) j.flags[pos] = 0;
  };
  for (int b = tid; b < UNIT_BINS; b += T) next[b] = 0;
  __syncthreads();
  for (int pass = 0; pass < 2; ++pass) {
    for (int c0 = 0; c0 < j.S; c0 += T) {
      const int s = c0 + tid;
      const int len = s < j.S ? j.sp.len(s) : 0;
      if (len > 0) {
        const int nb = (len - 1) / j.B + 1;
        const int tail = len - (nb - 1) * j.B;
        const int nfull = (nb - 1) * upb;      // units of the full blocks
        const int ntail = (tail - 1) / j.qg + 1;  // units of the last block
        if (pass == 0) {
          if (nfull) atomicAdd(&next[bin_of(j.B)], nfull);
          atomicAdd(&next[bin_of(tail)], ntail);
        } else {
          const int start = j.sp.start(s);
          if (nfull) {
            const int pos = atomicAdd(&next[bin_of(j.B)], nfull);
            for (int v = 0; v < nfull; ++v) {
              const int blk = v / upb;
              put(pos + v, start + blk * j.B, j.B, v - blk * upb);
            }
          }
          const int pos = atomicAdd(&next[bin_of(tail)], ntail);
          for (int g = 0; g < ntail; ++g) put(pos + g, start + (nb - 1) * j.B, tail, g);
        }
      }
    }
    __syncthreads();
    if (pass == 0) {  // counts -> first position of each bin (exclusive scan)
      int sum = 0;
      for (int i = 0; i < per; ++i) sum += next[tid * per + i];
      int incl = sum;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      if (lane == 63) wsum[wave] = incl;
      __syncthreads();
      int run = incl - sum;
      for (int w = 0; w < wave; ++w) run += wsum[w];
      for (int i = 0; i < per; ++i) {
        const int c = next[tid * per + i];
        next[tid * per + i] = run;
        run += c;
      }
      if (tid == T - 1) j.table[0] = make_int4(run, 0, 0, 0);
      __syncthreads();
    }
  }
}

// Upper bound on the number of units of N rows in S sequences:
// sum_s ceil(len_s/B) <= N/B + S, plus N/QG more query groups when B > QG.
inline int attn_unit_bound(long long N, int S, int B, int QG) {
  long long b = N / B + S;
  if (B > QG) b += N / QG;
  return (int)b;
}

}  // namespace gs
