// attn_f32.hip -- block-local bidirectional attention, IEEE fp32 throughout
// (fp32 workloads).  Same blocks as the bf16 kernel, with
// v_mfma_f32_16x16x4_f32:
//   * workgroup = 4 waves = one unit of up to 16 query rows of one block and
//     one head, Q^T in every wave's registers;
//   * the block's keys in chunks of 32, dealt to the waves round-robin (wave
//     w takes chunks w, w + 4, ...), each wave staging its chunk's K and V
//     rows in its own LDS area as [key][dh] (padded rows);
//   * per wave: S^T = K Q^T (a lane holds 4 consecutive keys of one query),
//     an online softmax in base 2 over its chunks, O^T += V^T P^T with P fed
//     straight from registers;
//   * the four partial results (row max, row sum, O) merge through LDS:
//     O = sum_w 2^(m_w - M) O_w / sum_w 2^(m_w - M) l_w, M = max_w m_w;
//   * keys past the block end are clamped to the block's last row and masked.
// Splitting the keys over the waves keeps each wave's chain of products to a
// quarter of the block: a short fp32 batch (one 422-frame clip: 28 units x 8
// heads) then fills the chip with short workgroups.
#include "attn_units.hpp"

namespace gs {

constexpr int AF_THREADS = 256;
constexpr int AF_WAVES = AF_THREADS / 64;
constexpr int AF_QG = 16;
constexpr int AF_KC = 32;
constexpr int AF_DH = 128;
constexpr int AF_LD = AF_DH + 4;   // padded LDS row (floats)
constexpr int AF_WAVE_FLOATS = 2 * AF_KC * AF_LD;  // one wave's K and V chunk

__global__ __launch_bounds__(AF_THREADS) void block_attn_f32_kernel(
    const float* __restrict__ qkv, SeqSpans sp, int S, int B, int d, float scale_log2,
    float* __restrict__ O) {
  __shared__ float lds[AF_WAVES * AF_WAVE_FLOATS];

  AttnUnit U;
  if (!find_unit<AF_QG>(sp, S, B, blockIdx.x, U)) return;
  const int h = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g4 = lane >> 4;
  const int ld = 3 * d;
  const float* Qg = qkv + h * AF_DH;
  const float* Kg = qkv + d + h * AF_DH;
  const float* Vg = qkv + 2 * d + h * AF_DH;
  const int L = U.L;
  float* Ks = lds + wave * AF_WAVE_FLOATS;
  float* Vs = Ks + AF_KC * AF_LD;

  // Q^T operand: lane holds query (lane&15) at dh = 4s + g4, s = 0..31
  const int qrow = U.q0 + (lane & 15);
  const bool qvalid = (lane & 15) < U.qn;
  const int qc = qrow < L ? qrow : L - 1;
  float qf[32];
  {
    const float* qp = Qg + (size_t)(U.row0 + qc) * ld + g4;
#pragma unroll
    for (int s = 0; s < 32; ++s) qf[s] = qp[4 * s];
  }

  f32x4 oacc[8];
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) oacc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrun = -INFINITY, lrun = 0.f;

  const int nchunks = (L + AF_KC - 1) / AF_KC;
  for (int c = wave; c < nchunks; c += AF_WAVES) {
    // this wave's area is free: its reads of the previous chunk were issued
    // before these writes, and one wave's LDS accesses complete in order
    // 32 keys x 128 floats for K and V: 1024 float4 each, 16 per lane
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int idx = j * 64 + lane;
      const int kr = idx >> 5, c4 = (idx & 31) * 4;
      int key = c * AF_KC + kr;
      key = key < L ? key : L - 1;
      const size_t g = (size_t)(U.row0 + key) * ld + c4;
      *(float4*)&Ks[kr * AF_LD + c4] = *(const float4*)(Kg + g);
      *(float4*)&Vs[kr * AF_LD + c4] = *(const float4*)(Vg + g);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    float p[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      f32x4 a = {0.f, 0.f, 0.f, 0.f};
      const float* kp = &Ks[(kt * 16 + (lane & 15)) * AF_LD + g4];
#pragma unroll
      for (int s = 0; s < 32; ++s) a = __builtin_amdgcn_mfma_f32_16x16x4f32(kp[4 * s], qf[s], a, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = c * AF_KC + kt * 16 + g4 * 4 + i;
        const float v = key < L ? a[i] * scale_log2 : -INFINITY;
        p[kt][i] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(mrun, mx);
    const float alpha = exp2f(mrun - mnew);
    mrun = mnew;
    float psum = 0.f;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[kt][i] = exp2f(p[kt][i] - mnew);
        psum += p[kt][i];
      }
    lrun = lrun * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt] *= alpha;

    // O^T[dh][q] += sum_k V[k][dh] P[q][k]; MFMA step (kt, i) contracts keys kt*16 + g*4 + i
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* vp = &Vs[(kt * 16 + g4 * 4 + i) * AF_LD + (lane & 15)];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vp[dt * 16], p[kt][i], oacc[dt], 0, 0, 0);
      }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }

  // row sum of this wave's part (lanes l, l^16, l^32, l^48 hold one query)
  float l = lrun;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);

  // merge the four waves' parts: each wave's (max, sum, O^T) per lane
  __syncthreads();  // every wave is done with its K|V area
  float* part = lds + wave * (64 * 34);
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) part[(dt * 4 + e) * 64 + lane] = oacc[dt][e];
  part[32 * 64 + lane] = mrun;
  part[33 * 64 + lane] = l;
  __syncthreads();
  if (wave != 0) return;
  float m[AF_WAVES], f[AF_WAVES];
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < AF_WAVES; ++w) {
    m[w] = lds[w * (64 * 34) + 32 * 64 + lane];
    M = fmaxf(M, m[w]);
  }
  float lt = 0.f;
#pragma unroll
  for (int w = 0; w < AF_WAVES; ++w) {
    // a wave without chunks (a block of fewer than 4 chunks) has m = -inf,
    // sum 0 and O 0: its factor is 0
    f[w] = m[w] == -INFINITY ? 0.f : exp2f(m[w] - M);
    lt += f[w] * lds[w * (64 * 34) + 33 * 64 + lane];
  }
  if (!qvalid) return;
  const float inv = 1.f / lt;
  float* op = O + (size_t)(U.row0 + qrow) * d + h * AF_DH + g4 * 4;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt) {
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < AF_WAVES; ++w) acc += f[w] * lds[w * (64 * 34) + (dt * 4 + e) * 64 + lane];
      v[e] = acc * inv;
    }
    *(float4*)(op + dt * 16) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

hipError_t launch_block_attn_f32(const void* qkv, SeqSpans sp, int S, long long N, int d,
                                 int heads, int B, void* o, hipStream_t stream) {
  const int units = attn_unit_bound(N, S, B, AF_QG);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)AF_DH);
  hipLaunchKernelGGL(block_attn_f32_kernel, dim3(units, heads), dim3(AF_THREADS), 0, stream,
                     (const float*)qkv, sp, S, B, d, scale_log2, (float*)o);
  return hipGetLastError();
}

}  // namespace gs
