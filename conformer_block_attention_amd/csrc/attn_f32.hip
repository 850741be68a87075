// attn_f32.hip -- block-local bidirectional attention, IEEE fp32 throughout
// (fp32 workloads).  Same blocks and work units as the bf16 kernel, with
// v_mfma_f32_16x16x4_f32:
//   * workgroup = 4 waves = one unit of up to 64 query rows of one block and
//     one head; each wave owns one 16-row query tile, Q^T in registers;
//   * keys in chunks of 64 staged in LDS as [key][dh] (padded rows) for both
//     K and V;
//   * S^T = K Q^T (lane holds 4 consecutive keys of one query), online softmax
//     in base 2, then O^T += V^T P^T with P fed straight from registers;
//   * keys past the block end are clamped to the block's last row and masked.
#include "attn_units.hpp"

namespace gs {

constexpr int AF_THREADS = 256;
constexpr int AF_QG = 64;
constexpr int AF_KC = 64;
constexpr int AF_DH = 128;
constexpr int AF_LD = AF_DH + 4;   // padded LDS row (floats)

__global__ __launch_bounds__(AF_THREADS) void block_attn_f32_kernel(
    const float* __restrict__ qkv, SeqSpans sp, int S, int B, int d, float scale_log2,
    float* __restrict__ O) {
  __shared__ float Ks[AF_KC * AF_LD];
  __shared__ float Vs[AF_KC * AF_LD];

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

  // Q^T operand: lane holds query (lane&15) at dh = 4s + g4, s = 0..31
  const int qrow = U.q0 + wave * 16 + (lane & 15);
  const bool qvalid = (wave * 16 < U.qn) && qrow < L;
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
  for (int c = 0; c < nchunks; ++c) {
    __syncthreads();  // previous chunk fully consumed
    // 64 keys x 128 floats for K and V: 2048 float4 each, 8 per thread
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int idx = j * AF_THREADS + tid;
      const int kr = idx >> 5, c4 = (idx & 31) * 4;
      int key = c * AF_KC + kr;
      key = key < L ? key : L - 1;
      const size_t g = (size_t)(U.row0 + key) * ld + c4;
      *(float4*)&Ks[kr * AF_LD + c4] = *(const float4*)(Kg + g);
      *(float4*)&Vs[kr * AF_LD + c4] = *(const float4*)(Vg + g);
    }
    __syncthreads();

    float p[4][4];
    float mx = -INFINITY;
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
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
    for (int kt = 0; kt < 4; ++kt)
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
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* vp = &Vs[(kt * 16 + g4 * 4 + i) * AF_LD + (lane & 15)];
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x4f32(vp[dt * 16], p[kt][i], oacc[dt], 0, 0, 0);
      }
  }

  float l = lrun;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  if (!qvalid) return;
  const float inv = 1.f / l;
  float* op = O + (size_t)(U.row0 + qrow) * d + h * AF_DH + g4 * 4;
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
    *(float4*)(op + dt * 16) = make_float4(oacc[dt][0] * inv, oacc[dt][1] * inv,
                                           oacc[dt][2] * inv, oacc[dt][3] * inv);
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
