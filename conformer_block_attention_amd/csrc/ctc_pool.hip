// ctc_pool.hip -- the BPE head's posterior-weighted pooling and CTC greedy
// decoding of its pooled argmax.
//
// Pooling (IBM model card, "Model Architecture" (1): windows of 4 frames
// weighted by 1 - blank probability of a middle layer; stride 2 from the
// ONNX export's 211 positions for a 422-frame clip): position j of a
// sequence pools frames s*j .. min(s*j + window, T) - 1 and scores class c
// as sum_t w_t * logit[t][c], w_t = 1 - blank_prob[t], frames in order, each
// product and partial sum rounded to fp32 (no fused multiply-add, so the
// argmax is reproducible on any IEEE host).  Decoding (Q4 export README,
// "Inference note (NAR decode)"): per position the argmax class (ties to the
// lowest index), consecutive repeats merged, blank 0 dropped, token =
// class - 1.
//
// Kernels:
//   * position table: one workgroup finds each sequence's first position
//     (a prefix sum of ceil(len / stride) over cu_seqlens), then one thread
//     per position finds its sequence by binary search and writes (first
//     frame, frames, sequence);
//   * pooled argmax (HBM-bound: it reads the [N][C] logits once): one
//     workgroup per PA_POS consecutive positions; thread i scores classes
//     8i + 2048k .. +7 (16-byte loads of bf16 logits) for each of its
//     positions, keeps a running (max, index) per position, and the
//     workgroup reduces them at the end.  With window 4 and stride 2 and
//     positions of one sequence, each frame is loaded once by the workgroup
//     and serves the two windows that hold it; the two frames neighbouring
//     groups share come from L2 for the second (groups in order on one XCD);
//   * decode: one wave per sequence, 64 positions at a time, ballot and
//     prefix count to compact the kept tokens.
#include "gs_device.hpp"

namespace gs {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int PA_THREADS = 256;
constexpr int PA_POS = 4;       // positions per workgroup
constexpr int PA_MAXWIN = 8;    // frames per pooling window

// pos_cu[s] = first position of sequence s, pos_cu[S] = the number of
// positions the sequences make.  (The table of positions, {first frame,
// frames, sequence, 0} in order, with frames 0 for entries from that count
// up to P, is filled by the next kernel.)
__global__ __launch_bounds__(1024) void build_position_table_kernel(const int* __restrict__ cu,
                                                                   int S, int stride,
                                                                   int* __restrict__ pos_cu) {
  __shared__ int scan[1024];
  __shared__ int base;
  const int tid = threadIdx.x;
  if (tid == 0) base = 0;
  __syncthreads();
  for (int c0 = 0; c0 < S; c0 += 1024) {
    const int s = c0 + tid;
    const int len = s < S ? cu[s + 1] - cu[s] : 0;
    const int n = len > 0 ? (len + stride - 1) / stride : 0;
    scan[tid] = n;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int y = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += y;
      __syncthreads();
    }
    const int first = base + scan[tid] - n;
    if (s < S) pos_cu[s] = first;
    __syncthreads();
    if (tid == 1023) base += scan[1023];
    __syncthreads();
  }
  if (tid == 0) pos_cu[S] = base;
}

// table[p] for every position p < P: its sequence by binary search in
// pos_cu, then its first frame and frame count.
__global__ __launch_bounds__(256) void fill_position_table_kernel(
    const int* __restrict__ cu, const int* __restrict__ pos_cu, int S, int window, int stride,
    int P, int4* __restrict__ table) {
  const int p = blockIdx.x * 256 + threadIdx.x;
  if (p >= P) return;
  if (p >= pos_cu[S]) {  // past the positions the sequences make
    table[p] = make_int4(0, 0, 0, 0);
    return;
  }
  int lo = 0, hi = S - 1;  // the last s with pos_cu[s] <= p (sequences without positions skipped)
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (pos_cu[mid] <= p) lo = mid; else hi = mid - 1;
  }
  const int j = p - pos_cu[lo];
  const int start = cu[lo], len = cu[lo + 1] - start;
  table[p] = make_int4(start + j * stride, min(window, len - j * stride), lo, 0);
}

__device__ __forceinline__ bool better(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// logits [N][ld] bf16 (ld % 8 == 0, ld >= C), blank_prob [N] fp32.
__global__ __launch_bounds__(PA_THREADS) void pooled_argmax_kernel(
    const bf16* __restrict__ logits, long long ld, const float* __restrict__ blank_prob,
    const int4* __restrict__ table, int P, int C, int stride, int window,
    int* __restrict__ argmax) {
  // every product and sum rounded on its own (the argmax must not depend on
  // contraction into fused multiply-adds)
#pragma clang fp contract(off)
  __shared__ float sv[PA_POS][PA_THREADS / 64];
  __shared__ int si[PA_POS][PA_THREADS / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Neighbouring groups of positions share frames (window 4, stride 2: the
  // last two frames of one group are the first two of the next).  Workgroup
  // ids reach the 8 XCDs round-robin, so consecutive groups are dealt to
  // the workgroups of one XCD (wg, wg + 8, ...), which run at about the same
  // time and find the shared frames in that XCD's L2.
  const int G = (int)gridDim.x, wg = (int)blockIdx.x, G8 = G & ~7;
  const int group = wg < G8 ? (wg & 7) * (G8 >> 3) + (wg >> 3) : wg;
  const int p0 = group * PA_POS;
  int t0[PA_POS], nt[PA_POS];
  float w[PA_POS][PA_MAXWIN];
#pragma unroll
  for (int r = 0; r < PA_POS; ++r) {
    const int p = p0 + r < P ? p0 + r : P - 1;  // (repeats of the last position are not stored)
    const int4 e = table[p];
    t0[r] = e.x;
    nt[r] = e.y;
#pragma unroll
    for (int f = 0; f < PA_MAXWIN; ++f)
      w[r][f] = f < nt[r] ? 1.0f - blank_prob[e.x + f] : 0.f;
  }
  float bv[PA_POS];
  int bi[PA_POS];
#pragma unroll
  for (int r = 0; r < PA_POS; ++r) {
    bv[r] = -INFINITY;
    bi[r] = 0x7fffffff;
  }
  // the scores of position r for classes c0 .. c0+7 from its frames' 16-byte
  // pieces (frames in order), folded into the running maximum
  auto score = [&](int r, int c0, auto piece) __attribute__((always_inline)) {
    float acc[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] = 0.f;
#pragma unroll
    for (int f = 0; f < PA_MAXWIN; ++f) {
      if (f < nt[r]) {
        const u32x4_t u = piece(r, f);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float lo = __builtin_bit_cast(float, u[e] << 16);
          const float hi = __builtin_bit_cast(float, u[e] & 0xFFFF0000u);
          acc[2 * e] = acc[2 * e] + w[r][f] * lo;
          acc[2 * e + 1] = acc[2 * e + 1] + w[r][f] * hi;
        }
      }
    }
#pragma unroll
    for (int k = 0; k < 8; ++k)
      if (c0 + k < C && acc[k] > bv[r]) {  // classes rise within a thread: '>' keeps the first
        bv[r] = acc[k];
        bi[r] = c0 + k;
      }
  };
  // Window 4, stride 2, the workgroup's positions consecutive in one
  // sequence: their windows cover 2 (PA_POS - 1) + 4 consecutive frames, each
  // loaded once and shared by the two positions whose windows hold it.
  constexpr int FROWS = 2 * (PA_POS - 1) + 4;
  bool shared_rows = stride == 2 && window == 4;
#pragma unroll
  for (int r = 1; r < PA_POS; ++r) shared_rows = shared_rows && t0[r] == t0[0] + 2 * r;
  if (shared_rows) {
    const int nrows = 2 * (PA_POS - 1) + nt[PA_POS - 1];  // frames the last window reaches
    for (int c0 = 8 * tid; c0 < C; c0 += 8 * PA_THREADS) {
      u32x4_t u[FROWS];
#pragma unroll
      for (int i = 0; i < FROWS; ++i)
        u[i] = i < nrows ? *(const u32x4_t*)(logits + (size_t)(t0[0] + i) * ld + c0)
                         : u32x4_t{0u, 0u, 0u, 0u};
#pragma unroll
      for (int r = 0; r < PA_POS; ++r)
        score(r, c0, [&](int rr, int f) { return u[2 * rr + f < FROWS ? 2 * rr + f : 0]; });
    }
  } else {
    for (int c0 = 8 * tid; c0 < C; c0 += 8 * PA_THREADS) {
#pragma unroll
      for (int r = 0; r < PA_POS; ++r)
        score(r, c0, [&](int rr, int f) {
          return *(const u32x4_t*)(logits + (size_t)(t0[rr] + f) * ld + c0);
        });
    }
  }
  // reduce (max, lowest index) over the wave, then over the waves
#pragma unroll
  for (int r = 0; r < PA_POS; ++r) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv[r], off);
      const int oi = __shfl_xor(bi[r], off);
      if (better(ov, oi, bv[r], bi[r])) {
        bv[r] = ov;
        bi[r] = oi;
      }
    }
    if (lane == 0) {
      sv[r][wave] = bv[r];
      si[r][wave] = bi[r];
    }
  }
  __syncthreads();
  if (tid < PA_POS && p0 + tid < P) {
    float v = sv[tid][0];
    int i = si[tid][0];
    for (int q = 1; q < PA_THREADS / 64; ++q)
      if (better(sv[tid][q], si[tid][q], v, i)) {
        v = sv[tid][q];
        i = si[tid][q];
      }
    // a position with no frames (past the sequences' count) or only
    // non-finite scores: class 0
    argmax[p0 + tid] = i == 0x7fffffff ? 0 : i;
  }
}

// tokens of sequence s at tokens[pos_cu[s] ..], their number in counts[s]
// (positions at or past P, when P is below the sequences' count, are left out)
__global__ __launch_bounds__(256) void ctc_collapse_kernel(const int* __restrict__ argmax,
                                                           const int* __restrict__ pos_cu, int S,
                                                           int P, int* __restrict__ tokens,
                                                           int* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (s >= S) return;
  const int a = min(pos_cu[s], P), b = min(pos_cu[s + 1], P);
  int n = 0;
  for (int j0 = a; j0 < b; j0 += 64) {
    const int j = j0 + lane;
    int c = 0;
    bool keep = false;
    if (j < b) {
      c = argmax[j];
      keep = c != 0 && (j == a || c != argmax[j - 1]);
    }
    const unsigned long long m = __ballot(keep);
    const int rank = __popcll(m & ((1ull << lane) - 1ull));
    if (keep) tokens[a + n + rank] = c - 1;
    n += __popcll(m);
  }
  if (lane == 0) counts[s] = n;
}

hipError_t launch_bpe_pool_ctc(const void* logits, long long ld, const float* blank_prob,
                               const int* cu, int S, int C, int P, int window, int stride,
                               int* argmax, int* tokens, int* counts, void* workspace,
                               hipStream_t stream) {
  int4* table = (int4*)workspace;
  int* pos_cu = (int*)(table + (P > 0 ? P : 1));
  build_position_table_kernel<<<dim3(1), dim3(1024), 0, stream>>>(cu, S, stride, pos_cu);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (P > 0) {
    hipLaunchKernelGGL(fill_position_table_kernel, dim3((P + 255) / 256), dim3(256), 0, stream, cu,
                       (const int*)pos_cu, S, window, stride, P, table);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (P > 0) {
    hipLaunchKernelGGL(pooled_argmax_kernel, dim3((P + PA_POS - 1) / PA_POS), dim3(PA_THREADS), 0,
                       stream, (const bf16*)logits, ld, blank_prob, (const int4*)table, P, C,
                       stride, window, argmax);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(ctc_collapse_kernel, dim3((S + 3) / 4), dim3(256), 0, stream, argmax, pos_cu,
                     S, P, tokens, counts);
  return hipGetLastError();
}

}  // namespace gs
