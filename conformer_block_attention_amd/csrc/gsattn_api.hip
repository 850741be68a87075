// gsattn_api.hip -- the C ABI of libgsattn (declared in include/gsattn.h):
// host-side argument checks, workspace layout and kernel launches.
//
// Every check happens before anything is enqueued; on failure the call
// returns a status and a thread-local detail string and leaves the stream
// untouched.  Nothing here allocates device memory.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "gsattn.h"
#include "attn_units.hpp"

namespace gs {
hipError_t launch_qkv_proj_bf16(const void* x, const void* wqkv, void* qkv, int M, int d,
                                hipStream_t stream, const UnitTableJob* job = nullptr,
                                bool* job_done = nullptr);
UnitTableJob attn_bf16_table_job(SeqSpans sp, int S, long long N, int B, int heads,
                                  void* table);
hipError_t launch_out_proj_bf16(const void* o, const void* wo, const void* x, void* out, int M,
                                int d, hipStream_t stream);
hipError_t launch_block_attn_bf16(const void* qkv, SeqSpans sp, int S, long long N, int d,
                                  int heads, int B, void* o, void* table, hipStream_t stream,
                                  bool build_table = true);
hipError_t launch_qkv_proj_f32(const void* x, const void* wqkv, void* qkv, int M, int d,
                               hipStream_t stream);
hipError_t launch_bpe_pool_ctc(const void* logits, long long ld, const float* blank_prob,
                               const int* cu, int S, int C, int P, int window, int stride,
                               int* argmax, int* tokens, int* counts, void* workspace,
                               hipStream_t stream);
hipError_t launch_gemm_nt_bf16_pp(const void* A, const void* W, const void* R, void* C, int M,
                                  int Nc, int K, hipStream_t stream, const int* m_dev = nullptr);
hipError_t launch_gemm_nt_bf16_pp_rows(const void* A, const void* W, const void* R, void* C,
                                       int M, int M_cap, int Nc, int K, const int* m_dev,
                                       const int* rows, hipStream_t stream);
hipError_t launch_window_attn_bf16(const void* kv, const void* q, const int* cu, int S, int W,
                                   int nq, int heads, int dq, int window, void* table,
                                   void* o, hipStream_t stream);
hipError_t launch_out_proj_f32(const void* o, const void* wo, const void* x, void* out, int M,
                               int d, hipStream_t stream);
hipError_t launch_block_attn_f32(const void* qkv, SeqSpans sp, int S, long long N, int d,
                                 int heads, int B, void* o, hipStream_t stream);

// Validates cu_seqlens on the device: flag[0] = 0 if cu[0] == 0, cu is
// non-decreasing and cu[S] == N; 1 otherwise.  One workgroup.
__global__ void check_cu_kernel(const int* cu, int S, long long N, int* flag) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = (cu[0] != 0) || ((long long)cu[S] != N);
  __syncthreads();
  for (int s = threadIdx.x; s < S; s += blockDim.x)
    if (cu[s + 1] < cu[s]) atomicOr(&bad, 1);
  __syncthreads();
  if (threadIdx.x == 0) flag[0] = bad;
}

// Validates padded lengths: flag[0] = 1 if some len[s] is outside [0, T].
__global__ void check_lengths_kernel(const int* len, int S, int T, int* flag) {
  __shared__ int bad;
  if (threadIdx.x == 0) bad = 0;
  __syncthreads();
  for (int s = threadIdx.x; s < S; s += blockDim.x)
    if (len[s] < 0 || len[s] > T) atomicOr(&bad, 1);
  __syncthreads();
  if (threadIdx.x == 0) flag[0] = bad;
}

// Zeroes the padding rows len[b] .. T-1 of every bucket b of o [S*T][d]
// (their attention output), ZP_ROWS rows of a bucket per workgroup, in
// 16-byte pieces: grid (ceil(T / ZP_ROWS), S).
constexpr int ZP_ROWS = 16;
__global__ __launch_bounds__(256) void zero_pad_rows_kernel(const int* len, int T, int pieces,
                                                            uint4* o) {
  const int b = blockIdx.y;
  int l = len[b];
  l = l < 0 ? 0 : (l > T ? T : l);
  const int t0 = blockIdx.x * ZP_ROWS;
  const int t1 = min(t0 + ZP_ROWS, T);
  for (int t = max(t0, l); t < t1; ++t) {
    uint4* row = o + ((size_t)b * T + t) * pieces;
    for (int i = threadIdx.x; i < pieces; i += blockDim.x) row[i] = make_uint4(0u, 0u, 0u, 0u);
  }
}
// cu[0] = 0, cu[b + 1] = cu[b] + (len[b] clamped to [0, T]).  One workgroup.
__global__ __launch_bounds__(1024) void lengths_prefix_kernel(const int* __restrict__ len, int S,
                                                             int T, int* __restrict__ cu) {
  __shared__ int scan[1024];
  __shared__ int base;
  const int tid = threadIdx.x;
  if (tid == 0) base = 0;
  __syncthreads();
  for (int c0 = 0; c0 < S; c0 += 1024) {
    const int b = c0 + tid;
    int l = b < S ? len[b] : 0;
    l = l < 0 ? 0 : (l > T ? T : l);
    scan[tid] = l;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const int y = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += y;
      __syncthreads();
    }
    if (b < S) cu[b + 1] = base + scan[tid];
    __syncthreads();
    if (tid == 1023) base += scan[1023];
    __syncthreads();
  }
  if (tid == 0) cu[0] = 0;
}

// Row copies of the padded-bucket path: ZP_ROWS rows of one bucket per
// workgroup, viewed as one run of nrows * pieces 16-byte pieces.  Each
// thread issues ZP_PER loads before its stores, so a workgroup keeps
// ZP_PER * 256 pieces (32 KB) in flight instead of one 2 KB row.
constexpr int ZP_PER = 8;
typedef unsigned int zp_u32x4 __attribute__((ext_vector_type(4)));
template <class SrcRow, class DstRow>
__device__ __forceinline__ void copy_row_run(int nrows, int pieces, SrcRow src_row,
                                             DstRow dst_row) {
  const int total = nrows * pieces;
  for (int p0 = 0; p0 < total; p0 += ZP_PER * 256) {
    zp_u32x4 v[ZP_PER];
#pragma unroll
    for (int k = 0; k < ZP_PER; ++k) {
      const int p = p0 + k * 256 + (int)threadIdx.x;
      const int r = p / pieces;
      v[k] = zp_u32x4{0u, 0u, 0u, 0u};
      if (p < total && dst_row(r)) v[k] = *(const zp_u32x4*)(src_row(r) + (p - r * pieces));
    }
#pragma unroll
    for (int k = 0; k < ZP_PER; ++k) {
      const int p = p0 + k * 256 + (int)threadIdx.x;
      const int r = p / pieces;
      if (p < total) {
        uint4* d = dst_row(r);
        if (d) *(zp_u32x4*)(d + (p - r * pieces)) = v[k];
      }
    }
  }
}

// Valid rows of the buckets, packed: xp[cu[b] + t] = x[b*T + t], t < len[b].
// Grid (ceil(T / ZP_ROWS), S); rows of `pieces` 16-byte pieces.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint4* __restrict__ x,
                                                          const int* __restrict__ len,
                                                          const int* __restrict__ cu, int T,
                                                          int pieces, uint4* __restrict__ xp) {
  const int b = blockIdx.y;
  int l = len[b];
  l = l < 0 ? 0 : (l > T ? T : l);
  const int t0 = blockIdx.x * ZP_ROWS;
  const int n = min(ZP_ROWS, l - t0);
  if (n <= 0) return;
  const uint4* src = x + ((size_t)b * T + t0) * pieces;
  uint4* dst = xp + ((size_t)cu[b] + t0) * pieces;
  copy_row_run(
      n, pieces, [=](int r) { return src + (size_t)r * pieces; },
      [=](int r) { return dst + (size_t)r * pieces; });
}

// out[b*T + t] = outp[cu[b] + t] for t < len[b], x[b*T + t] for padding rows.
__global__ __launch_bounds__(256) void scatter_rows_kernel(const uint4* __restrict__ outp,
                                                           const uint4* x,
                                                           const int* __restrict__ len,
                                                           const int* __restrict__ cu, int T,
                                                           int pieces, uint4* out) {
  const int b = blockIdx.y;
  int l = len[b];
  l = l < 0 ? 0 : (l > T ? T : l);
  const int t0 = blockIdx.x * ZP_ROWS;
  const int n = min(ZP_ROWS, T - t0);
  if (n <= 0) return;
  const size_t row0 = (size_t)b * T + t0;
  const uint4* valid = outp + ((size_t)cu[b] + t0) * pieces;
  const bool in_place = x == out;
  copy_row_run(
      n, pieces,
      [=](int r) { return t0 + r < l ? valid + (size_t)r * pieces : x + (row0 + r) * pieces; },
      // (in place, a padding row already holds x)
      [=](int r) { return t0 + r < l || !in_place ? out + (row0 + r) * pieces : nullptr; });
}

// The row table of the padded path: rows[cu[b] + t] = b*T + t for the valid
// rows t < len[b] of bucket b (packed row -> padded row).  Grid
// (ceil(T / 256), S + 1): the first workgroup of the last row of the grid
// builds the attention's work-unit table (job) meanwhile.
__global__ __launch_bounds__(256) void padded_rows_table_kernel(const int* __restrict__ len,
                                                                const int* __restrict__ cu,
                                                                int T, int* __restrict__ rows,
                                                                UnitTableJob job) {
  if (blockIdx.y == gridDim.y - 1) {
    __shared__ int lds[UNIT_TABLE_LDS_INTS];
    if (blockIdx.x == 0) build_unit_table(job, lds);
    return;
  }
  const int b = blockIdx.y;
  int l = len[b];
  l = l < 0 ? 0 : (l > T ? T : l);
  const int t = blockIdx.x * 256 + (int)threadIdx.x;
  if (t < l) rows[cu[b] + t] = b * T + t;
}

// out[b*T + t] = x[b*T + t] for the padding rows t >= len[b] (out != x).
__global__ __launch_bounds__(256) void copy_padding_rows_kernel(const uint4* __restrict__ x,
                                                                const int* __restrict__ len,
                                                                int T, int pieces,
                                                                uint4* __restrict__ out) {
  const int b = blockIdx.y;
  int l = len[b];
  l = l < 0 ? 0 : (l > T ? T : l);
  const int t0 = max((int)blockIdx.x * ZP_ROWS, l);
  const int n = min((int)blockIdx.x * ZP_ROWS + ZP_ROWS, T) - t0;
  if (n <= 0) return;
  const size_t row0 = (size_t)b * T + t0;
  copy_row_run(
      n, pieces, [=](int r) { return x + (row0 + r) * pieces; },
      [=](int r) { return out + (row0 + r) * pieces; });
}
}  // namespace gs

// Workspace of gs_block_mhsa_fwd_noalloc: one copy per GPU, held until the
// process ends.  Host code never uses this name as an address (on the host
// it only stands for the symbol): scratch_of_current_device() looks up each
// device's copy with hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[GS_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kDh = 128;
constexpr int kMaxD = 8192;
constexpr size_t kAlign = 256;

thread_local char g_detail[512] = "";

gs_status fail(gs_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof(g_detail), fmt, ap);
  va_end(ap);
  return s;
}

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

size_t elem_size(gs_dtype t) { return t == GS_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool debug_checks() {
  const char* e = getenv("GSATTN_DEBUG_CHECKS");
  return e && e[0] == '1';
}

gs_status check_dtype(gs_dtype t) {
  if (t != GS_F32 && t != GS_BF16) return fail(GS_ERR_INVALID_ARGUMENT, "unknown dtype %d", (int)t);
  return GS_OK;
}

gs_status check_dims(int64_t N, int32_t d) {
  if (N < 0) return fail(GS_ERR_INVALID_ARGUMENT, "total_frames %lld < 0", (long long)N);
  if (N >= (int64_t)1 << 31)
    return fail(GS_ERR_UNSUPPORTED, "total_frames %lld >= 2^31", (long long)N);
  if (d < 1) return fail(GS_ERR_INVALID_ARGUMENT, "d_model %d < 1", d);
  if (d % kDh != 0 || d > kMaxD)
    return fail(GS_ERR_UNSUPPORTED, "d_model %d: the kernels need a multiple of 128, at most %d",
                d, kMaxD);
  if ((__int128)N * 3 * d >= ((__int128)1 << 62))
    return fail(GS_ERR_UNSUPPORTED, "N * 3d overflows");
  return GS_OK;
}

gs_status check_heads(int32_t d, int32_t heads) {
  if (heads < 1) return fail(GS_ERR_INVALID_ARGUMENT, "heads %d < 1", heads);
  if (d % heads != 0)
    return fail(GS_ERR_INVALID_ARGUMENT, "d_model %d is not divisible by heads %d", d, heads);
  if (d / heads != kDh)
    return fail(GS_ERR_UNSUPPORTED, "head dim %d: the kernels implement dh = 128", d / heads);
  return GS_OK;
}

gs_status check_ptr(const void* p, const char* name) {
  if (!p) return fail(GS_ERR_INVALID_ARGUMENT, "%s is NULL", name);
  if (!aligned16(p)) return fail(GS_ERR_INVALID_ARGUMENT, "%s is not 16-byte aligned", name);
  return GS_OK;
}

gs_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return GS_OK;
  return fail(GS_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define GS_TRY(expr)             \
  do {                           \
    gs_status _s = (expr);       \
    if (_s != GS_OK) return _s;  \
  } while (0)

// Runs the device check of cu_seqlens when GSATTN_DEBUG_CHECKS=1.  Needs one
// int of device scratch.
gs_status debug_check_cu(const int32_t* cu, int32_t S, int64_t N, int* dflag, hipStream_t st) {
  if (!debug_checks()) return GS_OK;
  hipLaunchKernelGGL(gs::check_cu_kernel, dim3(1), dim3(256), 0, st, (const int*)cu, (int)S,
                     (long long)N, dflag);
  GS_TRY(hip_status(hipGetLastError(), "cu_seqlens check launch"));
  int flag = 1;
  GS_TRY(hip_status(hipMemcpyAsync(&flag, dflag, sizeof(int), hipMemcpyDeviceToHost, st),
                    "cu_seqlens check copy"));
  GS_TRY(hip_status(hipStreamSynchronize(st), "cu_seqlens check sync"));
  if (flag) return fail(GS_ERR_INVALID_ARGUMENT, "cu_seqlens is not a valid offset array");
  return GS_OK;
}

gs_status debug_check_lengths(const int32_t* len, int32_t S, int32_t T, int* dflag,
                              hipStream_t st) {
  if (!debug_checks()) return GS_OK;
  hipLaunchKernelGGL(gs::check_lengths_kernel, dim3(1), dim3(256), 0, st, (const int*)len, (int)S,
                     (int)T, dflag);
  GS_TRY(hip_status(hipGetLastError(), "lengths check launch"));
  int flag = 1;
  GS_TRY(hip_status(hipMemcpyAsync(&flag, dflag, sizeof(int), hipMemcpyDeviceToHost, st),
                    "lengths check copy"));
  GS_TRY(hip_status(hipStreamSynchronize(st), "lengths check sync"));
  if (flag) return fail(GS_ERR_INVALID_ARGUMENT, "a length is outside [0, bucket_frames]");
  return GS_OK;
}

// The attention step over sequences given as spans (packed or padded).
gs_status attn_spans(const void* qkv, gs::SeqSpans sp, int32_t S, int64_t N, int32_t d,
                     int32_t heads, int32_t B, gs_dtype dtype, void* o, void* table,
                     hipStream_t stream, bool build_table = true) {
  hipError_t e = dtype == GS_BF16
                     ? gs::launch_block_attn_bf16(qkv, sp, S, N, d, heads, B, o, table, stream,
                                                  build_table)
                     : gs::launch_block_attn_f32(qkv, sp, S, N, d, heads, B, o, stream);
  return hip_status(e, "block_attn launch");
}

// Checks shared by the whole-sub-layer entry points; on success the
// workspace pieces are set.
struct FwdPlan {
  int64_t N;
  int32_t d;
  void* qkv;
  void* o;
  char* table;
  size_t table_bytes;
  int* dflag;
};

gs_status plan_fwd(const void* x, const void* Wqkv, const void* Wo, int32_t block_frames,
                   int32_t heads, void* out, const gs_mhsa_desc* desc, FwdPlan& p) {
  if (!desc) return fail(GS_ERR_INVALID_ARGUMENT, "desc is NULL");
  GS_TRY(check_dtype(desc->dtype));
  const int64_t N = desc->total_frames;
  const int32_t d = desc->d_model;
  GS_TRY(check_dims(N, d));
  GS_TRY(check_heads(d, heads));
  if (desc->num_seqs < 1) return fail(GS_ERR_INVALID_ARGUMENT, "num_seqs %d < 1", desc->num_seqs);
  if (block_frames < 1) return fail(GS_ERR_INVALID_ARGUMENT, "block_frames %d < 1", block_frames);
  p.N = N;
  p.d = d;
  if (N == 0) return GS_OK;
  GS_TRY(check_ptr(x, "x"));
  GS_TRY(check_ptr(Wqkv, "Wqkv"));
  GS_TRY(check_ptr(Wo, "Wo"));
  GS_TRY(check_ptr(out, "out"));
  const size_t e = elem_size(desc->dtype);
  const size_t xbytes = (size_t)N * d * e;
  if (out != x) {
    const char* a = (const char*)x;
    const char* b = (const char*)out;
    if (a < b + xbytes && b < a + xbytes)
      return fail(GS_ERR_INVALID_ARGUMENT, "out partially overlaps x");
  }
  const size_t need = gs_block_mhsa_workspace_bytes(N, d, desc->dtype);
  if (!desc->workspace) return fail(GS_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (((uintptr_t)desc->workspace & (kAlign - 1)) != 0)
    return fail(GS_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  if (desc->workspace_bytes < need)
    return fail(GS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed",
                desc->workspace_bytes, need);
  char* ws = (char*)desc->workspace;
  p.qkv = ws;
  p.o = ws + align_up((size_t)N * 3 * d * e);
  p.table = (char*)p.o + align_up((size_t)N * d * e);
  p.table_bytes = gs_block_attn_workspace_bytes(N);
  p.dflag = (int*)(p.table + p.table_bytes);
  return GS_OK;
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

gs_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  GS_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(GS_ERR_UNSUPPORTED, "device %d: the static scratch serves devices 0..%d", dev,
                kMaxDevices - 1);
  std::call_once(g_scratch_once[dev], [dev] {
    void* p = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = p;
  });
  GS_TRY(hip_status(g_scratch_err[dev], "hipGetSymbolAddress(scratch)"));
  if (!g_scratch_ptr[dev]) return fail(GS_ERR_HIP, "hipGetSymbolAddress(scratch) gave NULL");
  *ptr = g_scratch_ptr[dev];
  return GS_OK;
}

gs_status record(const gs_mhsa_desc* desc, int i, hipStream_t st) {
  if (!desc->kernel_events) return GS_OK;
  return hip_status(hipEventRecord(desc->kernel_events[i], st), "hipEventRecord");
}

}  // namespace

extern "C" {

int32_t gs_version(void) { return 10000; }

const char* gs_status_string(gs_status s) {
  switch (s) {
    case GS_OK: return "GS_OK";
    case GS_ERR_INVALID_ARGUMENT: return "GS_ERR_INVALID_ARGUMENT";
    case GS_ERR_UNSUPPORTED: return "GS_ERR_UNSUPPORTED";
    case GS_ERR_WORKSPACE_TOO_SMALL: return "GS_ERR_WORKSPACE_TOO_SMALL";
    case GS_ERR_HIP: return "GS_ERR_HIP";
  }
  return "unknown gs_status";
}

const char* gs_last_error_detail(void) { return g_detail; }

size_t gs_block_attn_workspace_bytes(int64_t total_frames) {
  if (total_frames < 0) return 0;
  // work-unit table: a header and at most one 16-byte entry per row; then one
  // 8-byte word per unit flagging heads for the exact fallback
  return align_up(16 * ((size_t)total_frames + 1)) + align_up(8 * ((size_t)total_frames + 1));
}

size_t gs_block_mhsa_workspace_bytes(int64_t total_frames, int32_t d_model, gs_dtype dtype) {
  if (total_frames < 0 || d_model < 1 || (dtype != GS_F32 && dtype != GS_BF16)) return 0;
  const size_t e = elem_size(dtype);
  const size_t n = (size_t)total_frames, d = (size_t)d_model;
  // Q|K|V [N][3d], O [N][d], the attention step's unit table, a debug flag slot
  return align_up(n * 3 * d * e) + align_up(n * d * e) + gs_block_attn_workspace_bytes(total_frames) +
         kAlign;
}

gs_status gs_qkv_proj(const void* x, const void* Wqkv, void* qkv, int64_t total_frames,
                      int32_t d_model, gs_dtype dtype, hipStream_t stream) {
  GS_TRY(check_dtype(dtype));
  GS_TRY(check_dims(total_frames, d_model));
  if (total_frames == 0) return GS_OK;
  GS_TRY(check_ptr(x, "x"));
  GS_TRY(check_ptr(Wqkv, "Wqkv"));
  GS_TRY(check_ptr(qkv, "qkv"));
  const int M = (int)total_frames;
  hipError_t e = dtype == GS_BF16 ? gs::launch_qkv_proj_bf16(x, Wqkv, qkv, M, d_model, stream)
                                  : gs::launch_qkv_proj_f32(x, Wqkv, qkv, M, d_model, stream);
  return hip_status(e, "qkv_proj launch");
}

gs_status gs_block_attn(const void* qkv, const int32_t* cu_seqlens, int32_t num_seqs,
                        int64_t total_frames, int32_t d_model, int32_t heads,
                        int32_t block_frames, gs_dtype dtype, void* o, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  GS_TRY(check_dtype(dtype));
  GS_TRY(check_dims(total_frames, d_model));
  GS_TRY(check_heads(d_model, heads));
  if (num_seqs < 1) return fail(GS_ERR_INVALID_ARGUMENT, "num_seqs %d < 1", num_seqs);
  if (block_frames < 1) return fail(GS_ERR_INVALID_ARGUMENT, "block_frames %d < 1", block_frames);
  if (!cu_seqlens) return fail(GS_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL");
  if (total_frames == 0) return GS_OK;
  GS_TRY(check_ptr(qkv, "qkv"));
  GS_TRY(check_ptr(o, "o"));
  if (!workspace) return fail(GS_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (((uintptr_t)workspace & (kAlign - 1)) != 0)
    return fail(GS_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  const size_t need = gs_block_attn_workspace_bytes(total_frames);
  if (workspace_bytes < need)
    return fail(GS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  return attn_spans(qkv, gs::SeqSpans{cu_seqlens, 0}, num_seqs, total_frames, d_model, heads,
                    block_frames, dtype, o, workspace, stream);
}

gs_status gs_out_proj_residual(const void* o, const void* Wo, const void* x, void* out,
                               int64_t total_frames, int32_t d_model, gs_dtype dtype,
                               hipStream_t stream) {
  GS_TRY(check_dtype(dtype));
  GS_TRY(check_dims(total_frames, d_model));
  if (total_frames == 0) return GS_OK;
  GS_TRY(check_ptr(o, "o"));
  GS_TRY(check_ptr(Wo, "Wo"));
  GS_TRY(check_ptr(x, "x"));
  GS_TRY(check_ptr(out, "out"));
  const int M = (int)total_frames;
  hipError_t e = dtype == GS_BF16 ? gs::launch_out_proj_bf16(o, Wo, x, out, M, d_model, stream)
                                  : gs::launch_out_proj_f32(o, Wo, x, out, M, d_model, stream);
  return hip_status(e, "out_proj launch");
}

gs_status gs_block_mhsa_fwd(const void* x, const int32_t* cu_seqlens, const void* Wqkv,
                            const void* Wo, int32_t block_frames, int32_t heads, void* out,
                            hipStream_t stream, const gs_mhsa_desc* desc) {
  FwdPlan p{};
  GS_TRY(plan_fwd(x, Wqkv, Wo, block_frames, heads, out, desc, p));
  if (!cu_seqlens) return fail(GS_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL");
  if (p.N == 0) return GS_OK;
  GS_TRY(debug_check_cu(cu_seqlens, desc->num_seqs, p.N, p.dflag, stream));

  if (desc->flags & ~GS_FWD_REUSE_UNIT_TABLE)
    return fail(GS_ERR_INVALID_ARGUMENT, "unknown flags 0x%x", desc->flags);
  const bool build_table = !(desc->flags & GS_FWD_REUSE_UNIT_TABLE);

  GS_TRY(record(desc, 0, stream));
  bool table_built = false;
  if (desc->dtype == GS_BF16 && build_table) {
    // the projection's small-tile launch, if it has one, builds the
    // attention's unit table in a workgroup of its own
    const gs::UnitTableJob job = gs::attn_bf16_table_job(gs::SeqSpans{cu_seqlens, 0},
                                                         desc->num_seqs, p.N, block_frames,
                                                         heads, p.table);
    GS_TRY(hip_status(gs::launch_qkv_proj_bf16(x, Wqkv, p.qkv, (int)p.N, p.d, stream, &job,
                                               &table_built),
                      "qkv_proj launch"));
  } else {
    GS_TRY(gs_qkv_proj(x, Wqkv, p.qkv, p.N, p.d, desc->dtype, stream));
  }
  GS_TRY(record(desc, 1, stream));
  GS_TRY(attn_spans(p.qkv, gs::SeqSpans{cu_seqlens, 0}, desc->num_seqs, p.N, p.d, heads,
                    block_frames, desc->dtype, p.o, p.table, stream,
                    build_table && !table_built));
  GS_TRY(record(desc, 2, stream));
  GS_TRY(gs_out_proj_residual(p.o, Wo, x, out, p.N, p.d, desc->dtype, stream));
  GS_TRY(record(desc, 3, stream));
  return GS_OK;
}

gs_status gs_block_mhsa_fwd_noalloc(const void* x, const int32_t* cu_seqlens, const void* Wqkv,
                                    const void* Wo, int32_t block_frames, int32_t heads,
                                    void* out, hipStream_t stream, int32_t num_seqs,
                                    int64_t total_frames, int32_t d_model, gs_dtype dtype) {
  GS_TRY(check_dtype(dtype));
  GS_TRY(check_dims(total_frames, d_model));
  const size_t need = gs_block_mhsa_workspace_bytes(total_frames, d_model, dtype);
  if (need > GS_NOALLOC_SCRATCH_BYTES)
    return fail(GS_ERR_UNSUPPORTED,
                "%lld frames at d_model %d need %zu bytes of workspace; the static scratch "
                "holds %zu",
                (long long)total_frames, d_model, need, (size_t)GS_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  GS_TRY(scratch_of_current_device(&ws));
  const gs_mhsa_desc desc{num_seqs, total_frames, d_model, dtype, ws, GS_NOALLOC_SCRATCH_BYTES,
                          nullptr, 0u};
  return gs_block_mhsa_fwd(x, cu_seqlens, Wqkv, Wo, block_frames, heads, out, stream, &desc);
}

// The bf16 padded path moves valid rows through a row table when byte
// offsets into x and out fit the projection kernels' 32-bit offsets; larger
// inputs pack the valid rows into the workspace instead.
static bool padded_rows_by_table(int64_t rows, int32_t d_model) {
  return (uint64_t)rows * (uint64_t)d_model * 2 < 0xFFFFFFF0ull;
}

size_t gs_block_mhsa_padded_workspace_bytes(int32_t num_seqs, int32_t bucket_frames,
                                            int32_t d_model, gs_dtype dtype) {
  if (num_seqs < 1 || bucket_frames < 1) return 0;
  const int64_t rows = (int64_t)num_seqs * bucket_frames;
  const size_t base = gs_block_mhsa_workspace_bytes(rows, d_model, dtype);
  if (base == 0) return 0;
  // the buckets' offsets, and either the row table (a 256-row panel of slack)
  // or the valid rows packed (input and output)
  const size_t offsets = align_up(4 * ((size_t)num_seqs + 1));
  if (padded_rows_by_table(rows, d_model)) return base + offsets + align_up(4 * ((size_t)rows + 256));
  const size_t packed = align_up((size_t)rows * d_model * elem_size(dtype));
  return base + 2 * packed + offsets;
}

gs_status gs_block_mhsa_fwd_padded(const void* x, const int32_t* lengths, int32_t bucket_frames,
                                   const void* Wqkv, const void* Wo, int32_t block_frames,
                                   int32_t heads, void* out, hipStream_t stream,
                                   const gs_mhsa_desc* desc) {
  FwdPlan p{};
  GS_TRY(plan_fwd(x, Wqkv, Wo, block_frames, heads, out, desc, p));
  if (desc && p.N > 0 && bucket_frames >= 1 && desc->num_seqs >= 1) {
    const size_t need = gs_block_mhsa_padded_workspace_bytes(desc->num_seqs, bucket_frames, p.d,
                                                             desc->dtype);
    if (desc->workspace_bytes < need)
      return fail(GS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed",
                  desc->workspace_bytes, need);
  }
  if (!lengths) return fail(GS_ERR_INVALID_ARGUMENT, "lengths is NULL");
  if (bucket_frames < 1) return fail(GS_ERR_INVALID_ARGUMENT, "bucket_frames %d < 1", bucket_frames);
  if ((int64_t)desc->num_seqs * bucket_frames != p.N)
    return fail(GS_ERR_INVALID_ARGUMENT, "total_frames %lld != num_seqs %d * bucket_frames %d",
                (long long)p.N, desc->num_seqs, bucket_frames);
  if (p.N == 0) return GS_OK;
  GS_TRY(debug_check_lengths(lengths, desc->num_seqs, bucket_frames, p.dflag, stream));
  const size_t e = elem_size(desc->dtype);
  const dim3 rows_grid((bucket_frames + gs::ZP_ROWS - 1) / gs::ZP_ROWS, desc->num_seqs);
  const int pieces = (int)((size_t)p.d * e / 16);

  if (desc->dtype == GS_BF16 && p.d % 256 == 0 && padded_rows_by_table(p.N, p.d)) {
    // Compact through a row table: the projection reads the valid rows of x
    // straight from their buckets, the attention runs on the packed Q|K|V,
    // out_proj reads the residual from x and writes each valid row to its
    // bucket, and the padding rows are copied from x (none in place).  The
    // row count exists only on the device.
    char* ws = (char*)desc->workspace + gs_block_mhsa_workspace_bytes(p.N, p.d, desc->dtype);
    const int S = desc->num_seqs;
    int* cu = (int*)ws;
    int* rows = (int*)(ws + align_up(4 * ((size_t)S + 1)));
    GS_TRY(record(desc, 0, stream));
    hipLaunchKernelGGL(gs::lengths_prefix_kernel, dim3(1), dim3(1024), 0, stream,
                       (const int*)lengths, S, (int)bucket_frames, cu);
    // (the attention's unit table is built in the same launch)
    const gs::UnitTableJob job = gs::attn_bf16_table_job(gs::SeqSpans{cu, 0}, S, p.N,
                                                         block_frames, heads, p.table);
    hipLaunchKernelGGL(gs::padded_rows_table_kernel, dim3((bucket_frames + 255) / 256, S + 1),
                       dim3(256), 0, stream, (const int*)lengths, (const int*)cu,
                       (int)bucket_frames, rows, job);
    GS_TRY(hip_status(hipGetLastError(), "row table launch"));
    GS_TRY(hip_status(gs::launch_gemm_nt_bf16_pp_rows(x, Wqkv, nullptr, p.qkv, (int)p.N, (int)p.N,
                                                      3 * p.d, p.d, cu + S, rows, stream),
                      "qkv_proj launch"));
    GS_TRY(record(desc, 1, stream));
    GS_TRY(attn_spans(p.qkv, gs::SeqSpans{cu, 0}, S, p.N, p.d, heads, block_frames, desc->dtype,
                      p.o, p.table, stream, false));
    GS_TRY(record(desc, 2, stream));
    GS_TRY(hip_status(gs::launch_gemm_nt_bf16_pp_rows(p.o, Wo, x, out, (int)p.N, (int)p.N, p.d,
                                                      p.d, cu + S, rows, stream),
                      "out_proj launch"));
    if (out != x) {
      hipLaunchKernelGGL(gs::copy_padding_rows_kernel, rows_grid, dim3(256), 0, stream,
                         (const uint4*)x, (const int*)lengths, (int)bucket_frames, pieces,
                         (uint4*)out);
      GS_TRY(hip_status(hipGetLastError(), "padding rows launch"));
    }
    GS_TRY(record(desc, 3, stream));
    return GS_OK;
  }

  if (desc->dtype == GS_BF16 && p.d % 256 == 0) {
    // Inputs too large for the row table's 32-bit offsets: pack the valid
    // rows, run the packed sub-layer on them with the row count taken on the
    // device, and unpack (padding rows copy x).
    char* ws = (char*)desc->workspace + gs_block_mhsa_workspace_bytes(p.N, p.d, desc->dtype);
    const size_t packed = align_up((size_t)p.N * p.d * e);
    void* xp = ws;
    void* outp = ws + packed;
    int* cu = (int*)(ws + 2 * packed);
    const int S = desc->num_seqs;
    GS_TRY(record(desc, 0, stream));
    hipLaunchKernelGGL(gs::lengths_prefix_kernel, dim3(1), dim3(1024), 0, stream,
                       (const int*)lengths, S, (int)bucket_frames, cu);
    hipLaunchKernelGGL(gs::gather_rows_kernel, rows_grid, dim3(256), 0, stream, (const uint4*)x,
                       (const int*)lengths, (const int*)cu, (int)bucket_frames, pieces,
                       (uint4*)xp);
    GS_TRY(hip_status(hipGetLastError(), "row packing launch"));
    GS_TRY(hip_status(gs::launch_gemm_nt_bf16_pp(xp, Wqkv, nullptr, p.qkv, (int)p.N, 3 * p.d, p.d,
                                                 stream, cu + S),
                      "qkv_proj launch"));
    GS_TRY(record(desc, 1, stream));
    GS_TRY(attn_spans(p.qkv, gs::SeqSpans{cu, 0}, S, p.N, p.d, heads, block_frames, desc->dtype,
                      p.o, p.table, stream));
    GS_TRY(record(desc, 2, stream));
    GS_TRY(hip_status(gs::launch_gemm_nt_bf16_pp(p.o, Wo, xp, outp, (int)p.N, p.d, p.d, stream,
                                                 cu + S),
                      "out_proj launch"));
    hipLaunchKernelGGL(gs::scatter_rows_kernel, rows_grid, dim3(256), 0, stream,
                       (const uint4*)outp, (const uint4*)x, (const int*)lengths, (const int*)cu,
                       (int)bucket_frames, pieces, (uint4*)out);
    GS_TRY(hip_status(hipGetLastError(), "row unpacking launch"));
    GS_TRY(record(desc, 3, stream));
    return GS_OK;
  }

  GS_TRY(record(desc, 0, stream));
  GS_TRY(gs_qkv_proj(x, Wqkv, p.qkv, p.N, p.d, desc->dtype, stream));
  GS_TRY(record(desc, 1, stream));
  GS_TRY(attn_spans(p.qkv, gs::SeqSpans{lengths, bucket_frames}, desc->num_seqs, p.N, p.d, heads,
                    block_frames, desc->dtype, p.o, p.table, stream));
  hipLaunchKernelGGL(gs::zero_pad_rows_kernel, rows_grid, dim3(256), 0, stream,
                     (const int*)lengths, (int)bucket_frames, pieces, (uint4*)p.o);
  GS_TRY(hip_status(hipGetLastError(), "padding rows launch"));
  GS_TRY(record(desc, 2, stream));
  GS_TRY(gs_out_proj_residual(p.o, Wo, x, out, p.N, p.d, desc->dtype, stream));
  GS_TRY(record(desc, 3, stream));
  return GS_OK;
}

size_t gs_window_xattn_workspace_bytes(int64_t total_frames, int32_t d_q, int32_t num_windows,
                                       int32_t queries) {
  if (total_frames < 0 || d_q < 1 || num_windows < 0 || queries < 1) return 0;
  const size_t n = (size_t)total_frames, dq = (size_t)d_q;
  const size_t rows = (size_t)num_windows * queries;
  // K|V, Q, O, the window table (8 bytes per window and a count), a debug slot
  return align_up(n * 2 * dq * 2) + 2 * align_up(rows * dq * 2) +
         align_up(8 * (size_t)num_windows + 4) + kAlign;
}

gs_status gs_window_xattn_fwd(const void* hcat, const int32_t* cu_seqlens, const void* xq,
                              const void* Wq, const void* Wkv, const void* Wo,
                              int32_t window_frames, int32_t heads, void* out,
                              hipStream_t stream, const gs_xattn_desc* desc) {
  if (!desc) return fail(GS_ERR_INVALID_ARGUMENT, "desc is NULL");
  GS_TRY(check_dtype(desc->dtype));
  if (desc->dtype != GS_BF16)
    return fail(GS_ERR_UNSUPPORTED, "window cross-attention is implemented for bf16 only");
  const int64_t N = desc->total_frames;
  const int32_t F = desc->feat_dim, dq = desc->d_q, W = desc->num_windows, nq = desc->queries;
  if (desc->num_seqs < 1) return fail(GS_ERR_INVALID_ARGUMENT, "num_seqs %d < 1", desc->num_seqs);
  if (N < 0) return fail(GS_ERR_INVALID_ARGUMENT, "total_frames %lld < 0", (long long)N);
  if (W < 0) return fail(GS_ERR_INVALID_ARGUMENT, "num_windows %d < 0", W);
  if (nq < 1 || nq > 4) return fail(GS_ERR_UNSUPPORTED, "queries %d: 1 to 4 are implemented", nq);
  if (window_frames < 1) return fail(GS_ERR_INVALID_ARGUMENT, "window_frames %d < 1", window_frames);
  if (F < 1 || dq < 1) return fail(GS_ERR_INVALID_ARGUMENT, "feat_dim %d or d_q %d < 1", F, dq);
  if (heads < 1 || dq % heads != 0)
    return fail(GS_ERR_INVALID_ARGUMENT, "d_q %d is not a multiple of heads %d", dq, heads);
  if (dq / heads != kDh) return fail(GS_ERR_UNSUPPORTED, "head dim %d: dh = 128 is implemented", dq / heads);
  if (dq % 256 != 0 || dq > kMaxD || F % 64 != 0 || F > 4 * kMaxD)
    return fail(GS_ERR_UNSUPPORTED, "d_q %d (multiple of 256, at most %d) or feat_dim %d "
                "(multiple of 64, at most %d)", dq, kMaxD, F, 4 * kMaxD);
  if (N >= (int64_t)1 << 31 || (int64_t)W * nq >= (int64_t)1 << 31 ||
      (__int128)N * 2 * dq >= ((__int128)1 << 62))
    return fail(GS_ERR_UNSUPPORTED, "sizes exceed the 32-bit row counts of the kernels");
  if (!cu_seqlens) return fail(GS_ERR_INVALID_ARGUMENT, "cu_seqlens is NULL");
  if (W == 0) return GS_OK;
  GS_TRY(check_ptr(xq, "xq"));
  GS_TRY(check_ptr(Wq, "Wq"));
  GS_TRY(check_ptr(Wkv, "Wkv"));
  GS_TRY(check_ptr(Wo, "Wo"));
  GS_TRY(check_ptr(out, "out"));
  if (N > 0) GS_TRY(check_ptr(hcat, "hcat"));
  const size_t rows = (size_t)W * nq;
  const size_t qbytes = rows * dq * 2;
  if (out != xq) {
    const char* a = (const char*)xq;
    const char* b = (const char*)out;
    if (a < b + qbytes && b < a + qbytes)
      return fail(GS_ERR_INVALID_ARGUMENT, "out partially overlaps xq");
  }
  const size_t need = gs_window_xattn_workspace_bytes(N, dq, W, nq);
  if (!desc->workspace) return fail(GS_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (((uintptr_t)desc->workspace & (kAlign - 1)) != 0)
    return fail(GS_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  if (desc->workspace_bytes < need)
    return fail(GS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed",
                desc->workspace_bytes, need);
  char* ws = (char*)desc->workspace;
  void* kv = ws;
  void* q = ws + align_up((size_t)N * 2 * dq * 2);
  void* o = (char*)q + align_up(qbytes);
  char* table = (char*)o + align_up(qbytes);
  int* dflag = (int*)(table + align_up(8 * (size_t)W + 4));
  if (debug_checks()) {
    if (N > 0) GS_TRY(debug_check_cu(cu_seqlens, desc->num_seqs, N, dflag, stream));
    // the window count the sequences make
    GS_TRY(hip_status(gs::launch_window_attn_bf16(kv, q, cu_seqlens, desc->num_seqs, 0, nq, heads,
                                                  dq, window_frames, table, o, stream),
                      "window table launch"));
    int count = -1;
    GS_TRY(hip_status(hipMemcpyAsync(&count, table, sizeof(int), hipMemcpyDeviceToHost, stream),
                      "window count copy"));
    GS_TRY(hip_status(hipStreamSynchronize(stream), "window count sync"));
    if (count != W)
      return fail(GS_ERR_INVALID_ARGUMENT, "num_windows %d, the sequences make %d", W, count);
  }

  auto rec = [&](int i) -> gs_status {
    if (!desc->kernel_events) return GS_OK;
    return hip_status(hipEventRecord(desc->kernel_events[i], stream), "hipEventRecord");
  };
  GS_TRY(rec(0));
  if (N > 0)
    GS_TRY(hip_status(gs::launch_gemm_nt_bf16_pp(hcat, Wkv, nullptr, kv, (int)N, 2 * dq, F, stream),
                      "K|V projection launch"));
  GS_TRY(hip_status(gs::launch_gemm_nt_bf16_pp(xq, Wq, nullptr, q, (int)rows, dq, dq, stream),
                    "Q projection launch"));
  GS_TRY(rec(1));
  GS_TRY(hip_status(gs::launch_window_attn_bf16(kv, q, cu_seqlens, desc->num_seqs, W, nq, heads,
                                                dq, window_frames, table, o, stream),
                    "window attention launch"));
  GS_TRY(rec(2));
  GS_TRY(hip_status(gs::launch_gemm_nt_bf16_pp(o, Wo, xq, out, (int)rows, dq, dq, stream),
                    "output projection launch"));
  GS_TRY(rec(3));
  return GS_OK;
}

size_t gs_bpe_ctc_workspace_bytes(int32_t num_seqs, int32_t num_positions) {
  if (num_seqs < 1 || num_positions < 0) return 0;
  // position table (16 bytes per position, at least one), first positions [S+1]
  return align_up(16 * ((size_t)(num_positions > 0 ? num_positions : 1)) +
                  4 * ((size_t)num_seqs + 1));
}

gs_status gs_bpe_pool_ctc_greedy(const void* logits, int64_t ld, const float* blank_prob,
                                 const int32_t* cu_seqlens, int32_t num_seqs,
                                 int64_t total_frames, int32_t num_classes, int32_t window,
                                 int32_t stride, int32_t num_positions, int32_t* argmax,
                                 int32_t* tokens, int32_t* token_counts, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  if (num_seqs < 1) return fail(GS_ERR_INVALID_ARGUMENT, "num_seqs %d < 1", num_seqs);
  if (total_frames < 0) return fail(GS_ERR_INVALID_ARGUMENT, "total_frames < 0");
  if (total_frames >= (int64_t)1 << 31) return fail(GS_ERR_UNSUPPORTED, "total_frames >= 2^31");
  if (num_classes < 1) return fail(GS_ERR_INVALID_ARGUMENT, "num_classes %d < 1", num_classes);
  if (ld < num_classes || ld % 8 != 0)
    return fail(GS_ERR_INVALID_ARGUMENT, "ld %lld: at least num_classes and a multiple of 8",
                (long long)ld);
  if (window < 1 || window > 8) return fail(GS_ERR_UNSUPPORTED, "window %d: 1 to 8", window);
  if (stride < 1) return fail(GS_ERR_INVALID_ARGUMENT, "stride %d < 1", stride);
  if (num_positions < 0) return fail(GS_ERR_INVALID_ARGUMENT, "num_positions < 0");
  if (!cu_seqlens || !token_counts)
    return fail(GS_ERR_INVALID_ARGUMENT, "cu_seqlens or token_counts is NULL");
  if (num_positions > 0) {
    if (!argmax || !tokens) return fail(GS_ERR_INVALID_ARGUMENT, "argmax or tokens is NULL");
    GS_TRY(check_ptr(logits, "logits"));
    if (!blank_prob) return fail(GS_ERR_INVALID_ARGUMENT, "blank_prob is NULL");
  }
  if (!workspace) return fail(GS_ERR_INVALID_ARGUMENT, "workspace is NULL");
  if (((uintptr_t)workspace & (kAlign - 1)) != 0)
    return fail(GS_ERR_INVALID_ARGUMENT, "workspace is not 256-byte aligned");
  const size_t need = gs_bpe_ctc_workspace_bytes(num_seqs, num_positions);
  if (workspace_bytes < need)
    return fail(GS_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes,
                need);
  return hip_status(gs::launch_bpe_pool_ctc(logits, ld, blank_prob, cu_seqlens, num_seqs,
                                            num_classes, num_positions, window, stride, argmax,
                                            tokens, token_counts, workspace, stream),
                    "pooling / decoding launch");
}

}  // extern "C"
