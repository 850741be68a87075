// window_xattn.hip -- the attention step of the window cross-attention in the
// Q-Former projector (IBM model card, "Model Architecture" (2): each 15-frame
// window of the concatenated encoder states is reduced to 3 queries by
// cross-attention).
//
//   o[w][i][h] = softmax_l(q[w][i][h] . k[l][h] / sqrt(dh)) v[l][h],
//   l over the frames of window w, for the nq query rows i of the window.
//
// Windows are runs of `window` frames from each sequence's first frame, the
// last one holding the remainder; a small kernel lists them (first row,
// frames) on the device from cu_seqlens.
//
// Design: the work is tiny per window (3 queries x 15 keys x 128) and the
// step is bound by reading K|V once, so there is no matrix-core tiling.  A
// group of 16 lanes runs one (window, head), each lane owning 8 of the 128
// head dimensions, and a wave runs four of them (consecutive heads of one
// window, so their K|V pieces are adjacent).  A key's K and V rows of the
// head are 256-byte contiguous pieces (one 16-byte load per lane each); a
// group loads a chunk of 8 keys at once, forms each score as a lane partial
// plus a butterfly sum over its 16 lanes, and keeps an online softmax
// (running max, sum and fp32 accumulators) across chunks.  The output row is
// divided by its sum and rounded once to bf16.
#include "gs_device.hpp"

namespace gs {

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

constexpr int WX_DH = 128;
constexpr int WX_MAXQ = 4;      // query rows per window
constexpr int WX_CHUNK = 8;     // keys loaded together
constexpr int WX_WAVES = 4;     // waves (items) per workgroup

// table[w] = {first row, frames} for the windows the sequences make, in
// sequence order; entries from that count up to W hold {0, 0};
// count[0] = that count.  One workgroup of 1024 threads, 1024 sequences at a
// time with a workgroup prefix sum of their window counts.
__global__ __launch_bounds__(1024) void build_window_table_kernel(const int* __restrict__ cu,
                                                                 int S, int window, int W,
                                                                 int2* __restrict__ table,
                                                                 int* __restrict__ count) {
  __shared__ int scan[1024];
  __shared__ int base;
  const int tid = threadIdx.x;
  if (tid == 0) base = 0;
  __syncthreads();
  for (int c0 = 0; c0 < S; c0 += 1024) {
    const int s = c0 + tid;
    const int start = s < S ? cu[s] : 0;
    const int len = s < S ? cu[s + 1] - start : 0;
    const int n = len > 0 ? (len + window - 1) / window : 0;
    scan[tid] = n;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
      const int y = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += y;
      __syncthreads();
    }
    const int first = base + scan[tid] - n;
    for (int j = 0; j < n; ++j) {
      const int w = first + j;
      if (w < W) table[w] = make_int2(start + j * window, min(window, len - j * window));
    }
    __syncthreads();
    if (tid == 1023) base += scan[1023];
    __syncthreads();
  }
  for (int w = base + tid; w < W; w += 1024) table[w] = make_int2(0, 0);
  if (tid == 0) count[0] = base;
}

// sum over the 16 lanes of a lane group (lanes 16g .. 16g+15)
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  return v;
}

__device__ __forceinline__ void unpack8(const u32x4_t& u, float* f) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    f[2 * e] = __builtin_bit_cast(float, u[e] << 16);
    f[2 * e + 1] = __builtin_bit_cast(float, u[e] & 0xFFFF0000u);
  }
}

// kv [N][2 dq] (K columns then V columns), q and o [W * nq][dq].  A wave
// runs four items (window, head) = consecutive values of w * heads + h, one
// per group of 16 lanes; lane j of a group owns dimensions 8j .. 8j+7.
__global__ __launch_bounds__(WX_WAVES * 64) void window_attn_bf16_kernel(
    const bf16* __restrict__ kv, const bf16* __restrict__ q, const int2* __restrict__ table,
    int W, int nq, int heads, int dq, float scale_log2, bf16* __restrict__ o) {
  const int lane = threadIdx.x & 63;
  const long long items = (long long)W * heads;
  const long long it0 = ((long long)blockIdx.x * WX_WAVES + (threadIdx.x >> 6)) * 4;
  if (it0 >= items) return;  // (uniform per wave)
  long long it = it0 + (lane >> 4);
  const bool live = it < items;
  if (!live) it = items - 1;  // idle groups repeat the last item and store nothing
  const int w = (int)(it / heads), h = (int)(it - (long long)w * heads);
  const int2 e = table[w];
  const int col = h * WX_DH + 8 * (lane & 15);
  const size_t ldkv = 2 * (size_t)dq;
  int lmax = e.y;  // keys of the longest window among the wave's items
#pragma unroll
  for (int off = 16; off <= 32; off <<= 1) lmax = max(lmax, __shfl_xor(lmax, off));

  float qv[WX_MAXQ][8], m[WX_MAXQ], l[WX_MAXQ], acc[WX_MAXQ][8];
#pragma unroll
  for (int i = 0; i < WX_MAXQ; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) qv[i][t] = acc[i][t] = 0.f;
    if (i < nq) {
      const u32x4_t u = *(const u32x4_t*)(q + ((size_t)w * nq + i) * dq + col);
      unpack8(u, qv[i]);
      // logits in log2 units: fold 1/sqrt(dh) * log2(e) into q
#pragma unroll
      for (int t = 0; t < 8; ++t) qv[i][t] *= scale_log2;
    }
  }
  for (int k0 = 0; k0 < lmax; k0 += WX_CHUNK) {
    const int nk = min(WX_CHUNK, e.y - k0);  // this group's keys in the chunk (may be <= 0)
    u32x4_t kr[WX_CHUNK], vr[WX_CHUNK];
#pragma unroll
    for (int j = 0; j < WX_CHUNK; ++j) {
      // rows past this group's window repeat its last row (never used)
      const int r = e.y > 0 ? e.x + min(k0 + j, e.y - 1) : 0;
      const bf16* row = kv + (size_t)r * ldkv + col;
      kr[j] = *(const u32x4_t*)row;
      vr[j] = *(const u32x4_t*)(row + dq);
    }
#pragma unroll
    for (int i = 0; i < WX_MAXQ; ++i) {
      if (i >= nq) break;
      float sc[WX_CHUNK];
      float cmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < WX_CHUNK; ++j) {
        float kf[8];
        unpack8(kr[j], kf);
        float part = 0.f;
#pragma unroll
        for (int t = 0; t < 8; ++t) part += qv[i][t] * kf[t];
        sc[j] = group_sum(part);  // every group takes part in every shuffle
        if (j >= nk) sc[j] = -INFINITY;
        cmax = fmaxf(cmax, sc[j]);
      }
      const float mn = fmaxf(m[i], cmax);
      // all keys of this chunk masked (and none before): nothing to add
      const float alpha = mn == -INFINITY ? 1.f : exp2f(m[i] - mn);
      float ps = 0.f, pv[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) pv[t] = 0.f;
#pragma unroll
      for (int j = 0; j < WX_CHUNK; ++j) {
        const float p = sc[j] == -INFINITY ? 0.f : exp2f(sc[j] - mn);
        float vf[8];
        unpack8(vr[j], vf);
        ps += p;
#pragma unroll
        for (int t = 0; t < 8; ++t) pv[t] += p * vf[t];
      }
      l[i] = l[i] * alpha + ps;
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[i][t] = acc[i][t] * alpha + pv[t];
      m[i] = mn;
    }
  }
  if (!live) return;
#pragma unroll
  for (int i = 0; i < WX_MAXQ; ++i) {
    if (i >= nq) break;
    const float inv = l[i] > 0.f ? 1.f / l[i] : 0.f;  // a window with no frames gives zeros
    u32x4_t u;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const unsigned short a = __builtin_bit_cast(unsigned short, to_bf16(acc[i][2 * t] * inv));
      const unsigned short b = __builtin_bit_cast(unsigned short, to_bf16(acc[i][2 * t + 1] * inv));
      u[t] = (unsigned)a | ((unsigned)b << 16);
    }
    *(u32x4_t*)(o + ((size_t)w * nq + i) * dq + col) = u;
  }
}

// The table (table: W entries of 8 bytes, then one int for the count) and
// the attention step.
hipError_t launch_window_attn_bf16(const void* kv, const void* q, const int* cu, int S, int W,
                                   int nq, int heads, int dq, int window, void* table,
                                   void* o, hipStream_t stream) {
  int* count = (int*)((int2*)table + W);
  build_window_table_kernel<<<dim3(1), dim3(1024), 0, stream>>>(cu, S, window, W, (int2*)table,
                                                               count);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const long long items = (long long)W * heads;
  if (items == 0) return hipSuccess;
  const long long blocks = (items + 4 * WX_WAVES - 1) / (4 * WX_WAVES);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)WX_DH);
  hipLaunchKernelGGL(window_attn_bf16_kernel, dim3((unsigned)blocks), dim3(WX_WAVES * 64), 0,
                     stream, (const bf16*)kv, (const bf16*)q, (const int2*)table, W, nq, heads,
                     dq, scale_log2, (bf16*)o);
  return hipGetLastError();
}

}  // namespace gs
