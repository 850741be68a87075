// gemm_f32.hip -- IEEE fp32 GEMM for the projections (fp32 workloads):
//   C[M][Nc] = (R[M][Nc] +) A[M][K] . W[Nc][K]^T
// on v_mfma_f32_16x16x4_f32 (fp32 products and sums, no reduced-precision
// inputs).  Macro tile 64 x 64, K step 32, 4 waves each 32 x 32 (2 x 2 MFMA
// tiles).  Tiles are staged k-major in LDS ([k][row], padded) so that one MFMA
// operand read is 16 consecutive rows of one k.  The weight fragment is the
// first MFMA operand, so each lane holds 4 consecutive output columns.
// K must be a multiple of 32 and Nc a multiple of 4; M is arbitrary.
#include "gs_device.hpp"

namespace gs {

constexpr int F32_BM = 64, F32_BN = 64, F32_BK = 32, F32_PAD = 4;
constexpr int F32_PF = 2;  // K steps whose loads are in flight

template <bool RESID>
__global__ __launch_bounds__(256) void gemm_f32_nt_kernel(const float* __restrict__ A,
                                                          const float* __restrict__ W,
                                                          const float* R, float* C, int M,
                                                          int Nc, int K) {
  __shared__ float As[F32_BK][F32_BM + F32_PAD];
  __shared__ float Bs[F32_BK][F32_BN + F32_PAD];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int m0 = blockIdx.x * F32_BM, n0 = blockIdx.y * F32_BN;

  // loader: thread -> row tid/4, k (tid%4)*4 .. +3 and 16 further on
  const int lr = tid >> 2, lk = (tid & 3) * 4;
  int ar = m0 + lr; ar = ar < M ? ar : M - 1;
  int br = n0 + lr; br = br < Nc ? br : Nc - 1;

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // The loads of a K step are issued F32_PF steps before the step stages
  // them in LDS, so a workgroup alone on its CU (a short batch) does not
  // wait for each step's loads in turn.
  const float* ap = A + (size_t)ar * K + lk;
  const float* wp = W + (size_t)br * K + lk;
  const int ksteps = K / F32_BK;
  float4 a[F32_PF][2], w[F32_PF][2];
  auto load = [&](int p, int s) __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      a[p][h] = *(const float4*)(ap + s * F32_BK + h * 16);
      w[p][h] = *(const float4*)(wp + s * F32_BK + h * 16);
    }
  };
#pragma unroll
  for (int p = 0; p < F32_PF; ++p)
    if (p < ksteps) load(p, p);
  for (int s0 = 0; s0 < ksteps; s0 += F32_PF) {
#pragma unroll
    for (int p = 0; p < F32_PF; ++p) {
      const int s = s0 + p;
      if (s >= ksteps) break;
      float4 ca[2], cw[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        ca[h] = a[p][h];
        cw[h] = w[p][h];
      }
      if (s + F32_PF < ksteps) load(p, s + F32_PF);
      __syncthreads();
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int k = lk + h * 16;
        As[k + 0][lr] = ca[h].x; As[k + 1][lr] = ca[h].y; As[k + 2][lr] = ca[h].z; As[k + 3][lr] = ca[h].w;
        Bs[k + 0][lr] = cw[h].x; Bs[k + 1][lr] = cw[h].y; Bs[k + 2][lr] = cw[h].z; Bs[k + 3][lr] = cw[h].w;
      }
      __syncthreads();
#pragma unroll
      for (int ks = 0; ks < F32_BK / 4; ++ks) {
        const int k = ks * 4 + (lane >> 4);
        float af[2], bf[2];
#pragma unroll
        for (int i = 0; i < 2; ++i) af[i] = As[k][wm * 32 + i * 16 + (lane & 15)];
#pragma unroll
        for (int j = 0; j < 2; ++j) bf[j] = Bs[k][wn * 32 + j * 16 + (lane & 15)];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(bf[j], af[i], acc[i][j], 0, 0, 0);
      }
    }
  }

  // acc[i][j][e]: column m = lane%16, row n = (lane/16)*4 + e of the transposed tile
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + wm * 32 + i * 16 + (lane & 15);
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 32 + j * 16 + (lane >> 4) * 4;
      if (n >= Nc) continue;
      float4 v = make_float4(acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]);
      const size_t off = (size_t)m * Nc + n;
      if constexpr (RESID) {
        const float4 r = *(const float4*)(R + off);
        v.x += r.x; v.y += r.y; v.z += r.z; v.w += r.w;
      }
      *(float4*)(C + off) = v;
    }
  }
}

hipError_t launch_qkv_proj_f32(const void* x, const void* wqkv, void* qkv, int M, int d,
                               hipStream_t stream) {
  const int Nc = 3 * d;
  dim3 grid((M + F32_BM - 1) / F32_BM, (Nc + F32_BN - 1) / F32_BN);
  hipLaunchKernelGGL(gemm_f32_nt_kernel<false>, grid, dim3(256), 0, stream, (const float*)x,
                     (const float*)wqkv, (const float*)nullptr, (float*)qkv, M, Nc, d);
  return hipGetLastError();
}

hipError_t launch_out_proj_f32(const void* o, const void* wo, const void* x, void* out, int M,
                               int d, hipStream_t stream) {
  dim3 grid((M + F32_BM - 1) / F32_BM, (d + F32_BN - 1) / F32_BN);
  hipLaunchKernelGGL(gemm_f32_nt_kernel<true>, grid, dim3(256), 0, stream, (const float*)o,
                     (const float*)wo, (const float*)x, (float*)out, M, d, d);
  return hipGetLastError();
}

}  // namespace gs
