// attn_bf16.hip -- block-local bidirectional attention on gfx950 (bf16 in/out,
// fp32 softmax and accumulation).
//
// For every block (<= B consecutive rows of one sequence; blocks restart at
// each cu_seqlens boundary, the last one is partial) and head h:
//   O_h = softmax(Q_h K_h^T / sqrt(128)) V_h
// reading Q|K|V from the projection output qkv[N][3d] and writing O[N][d].
//
// Work unit = (block, group of up to 256 query rows); grid = units x heads.
// Units are found on the device from cu_seqlens (no host round trip): each
// wave scans the per-sequence unit counts with a wave prefix sum.  The grid is
// an upper bound; surplus workgroups exit at once.
//
// Per workgroup (8 waves, 512 threads):
//   * each wave owns up to two 16-row query tiles (Q stays in registers as the
//     MFMA B operand);
//   * keys stream through LDS in chunks of 64, double buffered: K as
//     [key][dh] (LDS-direct 16-byte copies) and V transposed to [dh][key]
//     (through registers), so both MFMA operands are read as 16-byte rows;
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16.  The K rows
//     of each 16-key MFMA tile are permuted so that a lane's scores for two
//     adjacent tiles are 8 consecutive keys -- exactly the P^T operand layout
//     of the PV product; P never leaves registers;
//   * online softmax in base 2 with fp32 running max and sum; the max is
//     reduced across the 4 lane groups holding the same query, the sum only
//     at the end.  P is rounded to bf16 (RNE) for the MFMA and the sum uses
//     the rounded values; O = acc / sum is rounded once to bf16.
//   * keys past the block end are read from the block's last row (finite
//     data) and masked to -inf, so no read leaves the block.
#include "attn_units.hpp"

namespace gs {

constexpr int ATT_THREADS = 512;
constexpr int ATT_WAVES = ATT_THREADS / 64;
constexpr int ATT_QG = 256;   // query rows per workgroup
constexpr int ATT_KC = 64;    // keys per LDS chunk
constexpr int DH = 128;

// LDS layouts (bf16 elements):
//   Ks [64 keys][128 dh]  row = 256 B = 16 chunks of 16 B; chunk c of key k is
//                         stored at physical chunk c ^ fk(k)
//   Vt [128 dh][64 keys]  row = 128 B = 8 chunks; chunk c of row e is stored at
//                         c ^ fv(e)
// fk spreads the 8 keys {0..3, 8..11} (+4, +32) that 8 consecutive lanes read;
// fv spreads both the 8 consecutive rows the MFMA reads and the rows 4 apart
// the transposing writes touch.
__device__ __forceinline__ int fk(int k) { return (k & 3) | (((k >> 3) & 1) << 2); }
__device__ __forceinline__ int fv(int e) { return (e ^ (e >> 2)) & 7; }

// Key row (chunk-relative) that row r of 16-key MFMA tile ks feeds: the tile
// pair (ks/2) covers 32 keys; tile parity selects the upper/lower 4 of each 8.
__device__ __forceinline__ int perm_key(int ks, int r) {
  return (ks >> 1) * 32 + (r >> 2) * 8 + (ks & 1) * 4 + (r & 3);
}

__global__ __launch_bounds__(ATT_THREADS, 1) void block_attn_bf16_kernel(
    const bf16* __restrict__ qkv, const int* __restrict__ cu, int S, int B, int d,
    float scale_log2, bf16* __restrict__ O) {
  __shared__ __attribute__((aligned(1024))) bf16 Ks[2][ATT_KC * DH];
  __shared__ __attribute__((aligned(1024))) bf16 Vt[2][DH * ATT_KC];

  AttnUnit U;
  if (!find_unit<ATT_QG>(cu, S, B, blockIdx.x, U)) return;  // uniform over the workgroup
  const int h = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int ld = 3 * d;
  const bf16* Qg = qkv + h * DH;
  const bf16* Kg = qkv + d + h * DH;
  const bf16* Vg = qkv + 2 * d + h * DH;
  const int L = U.L;
  const int nchunks = (L + ATT_KC - 1) / ATT_KC;

  // --- chunk staging -------------------------------------------------------
  // K: 64 rows x 16 chunks = 1024 copies of 16 B; one wave instruction fills
  // 4 key rows (1 KB); 16 instructions, 2 per wave.
  auto stage_k = [&](int c, int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int k0 = (j * ATT_WAVES + wave) * 4;   // first key row of this instruction
      const int kr = k0 + (lane >> 4);
      const int pc = lane & 15;                     // physical chunk
      const int lc = pc ^ fk(kr);                   // logical chunk stored there
      int key = c * ATT_KC + kr;
      key = key < L ? key : L - 1;
      const bf16* g = Kg + (size_t)(U.row0 + key) * ld + lc * 8;
      copy16_to_lds(g, (GS_LDS bf16*)&Ks[buf][k0 * DH]);
    }
  };
  // V: thread -> 4 keys (kg*4..+3) x 4 dh (dg*4..+3); 8-byte loads, then four
  // 8-byte LDS writes of the transposed 4x4 block.
  const int vkg = threadIdx.x >> 5;   // 0..15
  const int vdg = threadIdx.x & 31;   // 0..31
  auto load_v = [&](int c, uint2* r) {
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      int key = c * ATT_KC + vkg * 4 + kk;
      key = key < L ? key : L - 1;
      r[kk] = *(const uint2*)(Vg + (size_t)(U.row0 + key) * ld + vdg * 4);
    }
  };
  auto store_vt = [&](const uint2* r, int buf) {
    // r[kk] holds dh (vdg*4 + 0..3) of key vkg*4+kk as 4 packed bf16
#pragma unroll
    for (int dd = 0; dd < 4; ++dd) {
      const int e = vdg * 4 + dd;
      uint32_t lo, hi;  // keys 0,1 and 2,3 of this dh
      const int sh = (dd & 1) * 16;
      const uint32_t w0 = (dd < 2) ? r[0].x : r[0].y;
      const uint32_t w1 = (dd < 2) ? r[1].x : r[1].y;
      const uint32_t w2 = (dd < 2) ? r[2].x : r[2].y;
      const uint32_t w3 = (dd < 2) ? r[3].x : r[3].y;
      lo = ((w0 >> sh) & 0xFFFFu) | (((w1 >> sh) & 0xFFFFu) << 16);
      hi = ((w2 >> sh) & 0xFFFFu) | (((w3 >> sh) & 0xFFFFu) << 16);
      const int lchunk = vkg >> 1;                  // 8 keys per 16-byte chunk
      const int pchunk = lchunk ^ fv(e);
      GS_LDS u32x2* dst = (GS_LDS u32x2*)((GS_LDS bf16*)&Vt[buf][0] + e * ATT_KC + pchunk * 8 +
                                          (vkg & 1) * 4);
      *dst = u32x2{lo, hi};
    }
  };

  // --- queries of this wave -------------------------------------------------
  // tile t = wave + 8*tt covers block-relative rows q0 + 16t .. +15
  const int ntiles = (U.qn + 15) >> 4;
  bool tvalid[2];
  bf16x8 qf[2][4];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int t = wave + ATT_WAVES * tt;
    tvalid[tt] = t < ntiles;
    int q = U.q0 + t * 16 + (lane & 15);
    q = q < L ? q : L - 1;
    const bf16* qp = Qg + (size_t)(U.row0 + q) * ld + (lane >> 4) * 8;
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) qf[tt][kc] = *(const bf16x8*)(qp + kc * 32);
  }

  f32x4 oacc[2][8];
  float mrun[2], lrun[2];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    mrun[tt] = -INFINITY;
    lrun[tt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[tt][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // prologue: chunk 0
  {
    uint2 vr[4];
    stage_k(0, 0);
    load_v(0, vr);
    store_vt(vr, 0);
  }
  wait_vmem();
  __syncthreads();

  const int g4 = lane >> 4;       // lane group: keys g4*8.. of each 32-key pair
  for (int c = 0; c < nchunks; ++c) {
    const int buf = c & 1;
    uint2 vr[4];
    const bool more = c + 1 < nchunks;
    if (more) {
      stage_k(c + 1, buf ^ 1);
      load_v(c + 1, vr);
    }
    const GS_LDS bf16* ks = (const GS_LDS bf16*)&Ks[buf][0];
    const GS_LDS bf16* vt = (const GS_LDS bf16*)&Vt[buf][0];

    // S^T tiles for both query tiles: s[tt][ks] holds keys
    //   c*64 + (ks/2)*32 + g4*8 + (ks&1)*4 + i,  i = 0..3, for query lane&15
    f32x4 s[2][4];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int kr = perm_key(kt, lane & 15);
      bf16x8 kf[4];
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const int lc = kc * 4 + g4;
        kf[kc] = *(const GS_LDS bf16x8*)(ks + kr * DH + (lc ^ fk(kr)) * 8);
      }
#pragma unroll
      for (int tt = 0; tt < 2; ++tt) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[kc], qf[tt][kc], a, 0, 0, 0);
        s[tt][kt] = a;
      }
    }

    // online softmax (base 2) and P in the PV operand layout
    bf16x8 pf[2][2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = c * ATT_KC + (kt >> 1) * 32 + g4 * 8 + (kt & 1) * 4 + i;
          float v = s[tt][kt][i] * scale_log2;
          v = key < L ? v : -INFINITY;
          s[tt][kt][i] = v;
          mx = fmaxf(mx, v);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mnew = fmaxf(mrun[tt], mx);
      const float alpha = exp2f(mrun[tt] - mnew);
      mrun[tt] = mnew;
      float psum = 0.f;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bf16 pb = to_bf16(exp2f(s[tt][kt][i] - mnew));
          psum += to_f32(pb);
          pf[tt][kt >> 1][(kt & 1) * 4 + i] = pb;
        }
      lrun[tt] = lrun[tt] * alpha + psum;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oacc[tt][dt] *= alpha;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int e = dt * 16 + (lane & 15);
        const int lc = pr * 4 + g4;
        const bf16x8 vf = *(const GS_LDS bf16x8*)(vt + e * ATT_KC + (lc ^ fv(e)) * 8);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
          oacc[tt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[tt][pr], oacc[tt][dt], 0, 0, 0);
      }
    }

    if (more) store_vt(vr, buf ^ 1);
    wait_vmem();
    __syncthreads();
  }

  // normalise and store: oacc[tt][dt][i] is O[query lane&15][dh dt*16 + g4*4 + i]
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    if (!tvalid[tt]) continue;
    float l = lrun[tt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const float inv = 1.f / l;
    const int t = wave + ATT_WAVES * tt;
    const int q = U.q0 + t * 16 + (lane & 15);
    if (q >= L) continue;
    bf16* op = O + (size_t)(U.row0 + q) * d + h * DH + g4 * 4;
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
}

hipError_t launch_block_attn_bf16(const void* qkv, const int* cu, int S, long long N, int d,
                                  int heads, int B, void* o, hipStream_t stream) {
  const int units = attn_unit_bound(N, S, B, ATT_QG);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)DH);
  hipLaunchKernelGGL(block_attn_bf16_kernel, dim3(units, heads), dim3(ATT_THREADS), 0, stream,
                     (const bf16*)qkv, cu, S, B, d, scale_log2, (bf16*)o);
  return hipGetLastError();
}

}  // namespace gs
