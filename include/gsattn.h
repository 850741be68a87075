/*
 * gsattn.h -- C ABI of libgsattn: the block-local multi-head self-attention
 * sub-layer of the Granite-Speech-4.1-2B-NAR conformer encoder on AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (IBM model card, "Model Architecture" (1) CTC Speech Encoder:
 * every conformer layer uses block attention with 4-second audio blocks; the
 * card's usage section runs it with sequence packing and non-causal,
 * i.e. bidirectional, attention):
 *
 *   given packed rows x[N][d] of S sequences delimited by cu_seqlens[S+1],
 *     qkv = x . Wqkv^T                           (Wqkv [3d][d], rows Q|K|V)
 *     for every block of at most B consecutive rows of one sequence
 *       (blocks restart at each sequence's first row, the last block of a
 *        sequence holds the remainder) and every head h (dh = d / heads):
 *       O_h = softmax(Q_h K_h^T / sqrt(dh)) V_h  (no mask inside the block)
 *     out = x + O . Wo^T                         (Wo [d][d], O in head order)
 *
 * No bias, normalisation or positional term belongs to this sub-layer.
 *
 * Conventions shared by every entry point:
 *   - All pointers named x, Wqkv, Wo, out, qkv, o, workspace, cu_seqlens are
 *     DEVICE pointers, owned by the caller; the library allocates nothing.
 *   - Row-major, densely packed.  Weights use the nn.Linear [out][in] layout;
 *     inside Wqkv rows 0..d-1 are Q, d..2d-1 are K, 2d..3d-1 are V, and head
 *     h owns rows h*dh..h*dh+dh-1 of each.  O columns are head-concatenated.
 *   - dtype GS_BF16: x, weights, out and intermediates are bfloat16, all sums
 *     accumulate in fp32, every fp32->bf16 conversion rounds to nearest even.
 *     GS_F32: everything IEEE fp32.
 *   - Every device pointer must be 16-byte aligned.
 *   - Supported on the GPU: dh == 128 (d = 128 * heads), d_model <= 8192,
 *     total_frames < 2^31.  Other shapes return GS_ERR_UNSUPPORTED.
 *   - Work is enqueued on `stream` and the call returns without waiting;
 *     device faults surface at the caller's next synchronisation.
 *   - Argument errors are detected on the host before anything is enqueued,
 *     so a non-OK status means no device work was issued (except GS_ERR_HIP,
 *     reported when a launch itself fails).
 *   - cu_seqlens (int32, S+1 entries) must satisfy cu[0] = 0, cu[s] <= cu[s+1],
 *     cu[S] = total_frames.  It lives on the device and is not read by the
 *     host; violating it is undefined behaviour unless the environment
 *     variable GSATTN_DEBUG_CHECKS=1 is set, which validates it on the device
 *     (with a stream synchronisation) before launching.
 */
#ifndef GSATTN_H
#define GSATTN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GS_OK = 0,
  GS_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, misaligned pointer, bad cu_seqlens */
  GS_ERR_UNSUPPORTED = 2,        /* valid, but not a shape the GPU kernels implement */
  GS_ERR_WORKSPACE_TOO_SMALL = 3,
  GS_ERR_HIP = 4                 /* a HIP runtime call or kernel launch failed */
} gs_status;

typedef enum { GS_F32 = 0, GS_BF16 = 1 } gs_dtype;

/* Sizes and scratch for gs_block_mhsa_fwd. */
typedef struct {
  int32_t num_seqs;        /* S >= 1; cu_seqlens has S+1 entries */
  int64_t total_frames;    /* N = cu_seqlens[S] >= 0 (N == 0 is a no-op) */
  int32_t d_model;         /* d */
  gs_dtype dtype;
  void* workspace;         /* device scratch, >= gs_block_mhsa_workspace_bytes() bytes,
                              256-byte aligned; holds Q|K|V [N][3d], O [N][d] and the
                              attention step's work-unit table; contents on entry are
                              ignored, contents on return are unspecified */
  size_t workspace_bytes;
  /* Optional (may be NULL): four events the library records on `stream`
     before the projection, after it, after the attention and after the
     output projection, for per-step timing (each event between two
     kernels adds an idle gap of a few microseconds on the GPU). */
  hipEvent_t* kernel_events;
  /* 0, or GS_FWD_REUSE_UNIT_TABLE (gs_block_mhsa_fwd only, bf16): the
     workspace already holds the attention work-unit table that an earlier
     call on this stream built from the same cu_seqlens values, num_seqs,
     total_frames, d_model, heads and block_frames, with this workspace, and
     nothing has written the workspace since except such calls (a stack of
     layers over one packed batch); the table is then not rebuilt.  With
     anything else in the workspace the result is undefined. */
  uint32_t flags;
} gs_mhsa_desc;

#define GS_FWD_REUSE_UNIT_TABLE 1u

/* Bytes of workspace gs_block_mhsa_fwd needs for these sizes (0 on bad input). */
size_t gs_block_mhsa_workspace_bytes(int64_t total_frames, int32_t d_model, gs_dtype dtype);

/*
 * The whole sub-layer: out = x + BlockMHSA(x).
 *   x          [N][d]    input rows (packed sequences)
 *   cu_seqlens [S+1]     int32 sequence offsets (device)
 *   Wqkv       [3d][d]   projection weights
 *   Wo         [d][d]    output projection weights
 *   block_frames          B >= 1; B >= the longest sequence gives full attention
 *   heads                 number of heads, d % heads == 0
 *   out        [N][d]    result; may equal x (in place); any other overlap is invalid
 *   stream               HIP stream to enqueue on (0 = null stream)
 *   desc                 sizes, dtype, workspace (see gs_mhsa_desc)
 * Three steps run in stream order, each one or two kernel launches: the
 * projection, the block attention (with the build of its work-unit table
 * from cu_seqlens, done in a spare workgroup of the projection's second
 * launch when it has one, else by a kernel of its own), and the output
 * projection with the residual.  Only kernels are enqueued (no memset, no
 * host synchronisation unless GSATTN_DEBUG_CHECKS=1), so the call can be
 * captured in a HIP graph.
 */
gs_status gs_block_mhsa_fwd(const void* x, const int32_t* cu_seqlens, const void* Wqkv,
                            const void* Wo, int32_t block_frames, int32_t heads, void* out,
                            hipStream_t stream, const gs_mhsa_desc* desc);

/*
 * gs_block_mhsa_fwd without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The arguments are those of
 * gs_block_mhsa_fwd with the descriptor's sizes passed directly; the
 * workspace is a static device array of GS_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, held until the process ends.  The call itself
 * allocates nothing (no hipMalloc, hipFree or allocating library routine).
 *   - The scratch of the current device (hipGetDevice) is used; `stream`
 *     must belong to that device.  Its address is looked up once per device
 *     on the first call there.
 *   - Sizes whose workspace (gs_block_mhsa_workspace_bytes) exceeds
 *     GS_NOALLOC_SCRATCH_BYTES return GS_ERR_UNSUPPORTED before anything is
 *     enqueued: at d_model 1024 that is up to 8 168 bf16 frames (4 089 fp32).
 *   - Every call on one GPU shares that GPU's scratch and leaves its
 *     contents behind; calls on one GPU that overlap in time (other streams,
 *     other threads) race and must be serialised by the caller.
 * Results are bit for bit those of gs_block_mhsa_fwd with its own workspace.
 */
#define GS_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)

gs_status gs_block_mhsa_fwd_noalloc(const void* x, const int32_t* cu_seqlens, const void* Wqkv,
                                    const void* Wo, int32_t block_frames, int32_t heads,
                                    void* out, hipStream_t stream, int32_t num_seqs,
                                    int64_t total_frames, int32_t d_model, gs_dtype dtype);

/*
 * The whole sub-layer on fixed-length padded buckets instead of packed
 * sequences (the fixed [1, 800, features] encoder bucket of the portable
 * INT4 export, README "What Changed" item 4; how its padding is treated is
 * not stated there, so this reading is used):
 *   x        [S][T][d]  S buckets of T = bucket_frames rows; in bucket b the
 *                       first lengths[b] rows are the sequence, the rest is
 *                       padding (any finite values)
 *   lengths  [S]        int32 valid rows per bucket, 0 <= lengths[b] <= T
 *                       (device; values outside are clamped, or rejected
 *                       under GSATTN_DEBUG_CHECKS=1)
 *   bucket_frames       T >= 1; desc->num_seqs = S, desc->total_frames = S*T
 *   Wqkv, Wo, block_frames, heads, out, stream: as gs_block_mhsa_fwd.
 * Blocks restart at each bucket's first row and never include padding rows,
 * so the valid rows of `out` equal those of gs_block_mhsa_fwd on the same
 * sequences packed.  Padding rows are neither queries nor keys: their
 * attention output is zero, so out = x there (up to the sign of zero).  For
 * bf16 with d a multiple of 256 the valid rows run packed, with their count
 * and a packed-to-padded row table built on the device: the Q|K|V
 * projection reads them from their buckets, the attention runs on the
 * packed Q|K|V, and out_proj reads the residual from x and writes each
 * valid row into its bucket; padding rows are then copied from x (nothing
 * to copy when out == x).  When S*T*d*2 bytes reach 4 GiB (beyond the
 * projections' 32-bit offsets) the valid rows are packed into the
 * workspace and unpacked instead.  Other dtypes and widths run the
 * projections over all S*T rows and zero O's padding rows.  out may equal
 * x.  The workspace is gs_block_mhsa_padded_workspace_bytes(S, T, d, dtype)
 * bytes.
 */
size_t gs_block_mhsa_padded_workspace_bytes(int32_t num_seqs, int32_t bucket_frames,
                                            int32_t d_model, gs_dtype dtype);

gs_status gs_block_mhsa_fwd_padded(const void* x, const int32_t* lengths, int32_t bucket_frames,
                                   const void* Wqkv, const void* Wo, int32_t block_frames,
                                   int32_t heads, void* out, hipStream_t stream,
                                   const gs_mhsa_desc* desc);

/*
 * Step 1 alone: qkv[N][3d] = x[N][d] . Wqkv[3d][d]^T (fp32 accumulate).
 */
gs_status gs_qkv_proj(const void* x, const void* Wqkv, void* qkv, int64_t total_frames,
                      int32_t d_model, gs_dtype dtype, hipStream_t stream);

/* Bytes of workspace gs_block_attn needs for total_frames rows (0 on bad input). */
size_t gs_block_attn_workspace_bytes(int64_t total_frames);

/*
 * Step 2 alone: o[N][d] from qkv[N][3d] (layout as produced by gs_qkv_proj):
 * per block and head, softmax(Q K^T / sqrt(dh)) V, keys limited to the block.
 *   workspace  device scratch of >= gs_block_attn_workspace_bytes(N) bytes,
 *              256-byte aligned (the table of work units built from cu_seqlens
 *              and, for bf16, one word per unit marking the heads whose logits
 *              ran so far above those of the unit's first 32 keys that they go
 *              to an exact two-pass recomputation); calls that share a
 *              workspace must not overlap in time.
 */
gs_status gs_block_attn(const void* qkv, const int32_t* cu_seqlens, int32_t num_seqs,
                        int64_t total_frames, int32_t d_model, int32_t heads,
                        int32_t block_frames, gs_dtype dtype, void* o, void* workspace,
                        size_t workspace_bytes, hipStream_t stream);

/*
 * Step 3 alone: out[N][d] = x[N][d] + o[N][d] . Wo[d][d]^T (fp32 accumulate and
 * add, one rounding).  out may equal x.
 */
gs_status gs_out_proj_residual(const void* o, const void* Wo, const void* x, void* out,
                               int64_t total_frames, int32_t d_model, gs_dtype dtype,
                               hipStream_t stream);

/*
 * Window cross-attention of the Q-Former projector (IBM model card, "Model
 * Architecture" (2) Q-Former Projector: each 15-frame window of the
 * concatenated states of encoder layers 4, 8, 12, 16 is reduced to 3 queries
 * by cross-attention).  The pages give no widths, head count or bias terms;
 * this entry point computes, for every window w of every sequence (runs of
 * window_frames rows from the sequence's first row, the last one holding the
 * remainder) and each of its nq query rows i:
 *   q = xq[w][i] . Wq^T;  k_l | v_l = hcat[l] . Wkv^T for the window's rows l
 *   o = per head (dh = 128): softmax_l(q . k_l / sqrt(dh)) v_l
 *   out[w][i] = xq[w][i] + o . Wo^T
 * bf16 storage, fp32 accumulation, every fp32->bf16 conversion rounds to
 * nearest even.  Device pointers, caller-owned, 16-byte aligned:
 *   hcat  [N][F]          frames (F = feat_dim, e.g. 4 x 1024 for four layers)
 *   cu_seqlens [S+1]      int32 sequence offsets into hcat (as gs_block_mhsa_fwd)
 *   xq    [W][nq][dq]     query states per window
 *   Wq    [dq][dq], Wkv [2 dq][F] (K rows then V rows), Wo [dq][dq]
 *   out   [W][nq][dq]     may equal xq; any other overlap is invalid
 * W = num_windows must equal sum_s ceil(len_s / window_frames) (checked on
 * the device, with a synchronisation, only under GSATTN_DEBUG_CHECKS=1;
 * otherwise windows past the sequences' count get o = 0).  Supported: bf16,
 * dq % 256 == 0 with dq / heads == 128, F % 64 == 0, 1 <= nq <= 4,
 * window_frames >= 1.  Kernel events (if given): before the projections of
 * K|V and Q, after them, after the attention step, after the output
 * projection.
 */
typedef struct {
  int32_t num_seqs;        /* S >= 1 */
  int64_t total_frames;    /* N = cu_seqlens[S] */
  int32_t feat_dim;        /* F */
  int32_t d_q;             /* dq */
  int32_t num_windows;     /* W */
  int32_t queries;         /* nq */
  gs_dtype dtype;          /* GS_BF16 */
  void* workspace;         /* >= gs_window_xattn_workspace_bytes() bytes, 256-byte aligned */
  size_t workspace_bytes;
  hipEvent_t* kernel_events;  /* NULL or four events */
} gs_xattn_desc;

/* Bytes of workspace gs_window_xattn_fwd needs (0 on bad input): K|V
   [N][2 dq], Q and O [W*nq][dq], the window table. */
size_t gs_window_xattn_workspace_bytes(int64_t total_frames, int32_t d_q, int32_t num_windows,
                                       int32_t queries);

gs_status gs_window_xattn_fwd(const void* hcat, const int32_t* cu_seqlens, const void* xq,
                              const void* Wq, const void* Wkv, const void* Wo,
                              int32_t window_frames, int32_t heads, void* out,
                              hipStream_t stream, const gs_xattn_desc* desc);

/*
 * The BPE head's posterior-weighted pooling and CTC greedy decoding (IBM
 * model card, "Model Architecture" (1): the BPE head pools windows of 4
 * frames weighted by 1 - blank probability; ONNX export README, "Parity":
 * 211 positions for 422 frames, i.e. stride 2; Q4 export README,
 * "Inference note (NAR decode)": 100353 classes, blank 0, argmax, merge
 * repeats, drop blanks, token = class - 1).  For each sequence of T frames,
 * position j = 0 .. ceil(T / stride) - 1 pools frames stride*j ..
 * min(stride*j + window, T) - 1; class c scores sum_t w_t * logit[t][c] with
 * w_t = 1 - blank_prob[t], frames in order, every product and partial sum
 * rounded to fp32 without fused multiply-add (the positive normaliser
 * 1 / sum w_t changes no argmax and is left out).  argmax[p] = the best
 * class of position p (ties to the lowest index); then per sequence the kept
 * classes (not blank, not equal to the previous position's) minus one are
 * written to tokens[first position of the sequence ...] and their number to
 * token_counts[s].
 *   logits       [N][ld] bf16, ld >= num_classes, ld % 8 == 0 (16-byte rows)
 *   blank_prob   [N] fp32
 *   cu_seqlens   [S+1] int32 (device), as for gs_block_mhsa_fwd
 *   num_positions P = sum_s ceil(len_s / stride) (a smaller P drops the
 *                positions past it; a larger one gets class 0 there)
 *   argmax, tokens [P] int32, token_counts [S] int32 (device outputs)
 *   workspace    >= gs_bpe_ctc_workspace_bytes(S, P) bytes, 256-byte aligned
 * Supported: 1 <= window <= 8, 1 <= stride.
 */
size_t gs_bpe_ctc_workspace_bytes(int32_t num_seqs, int32_t num_positions);

gs_status gs_bpe_pool_ctc_greedy(const void* logits, int64_t ld, const float* blank_prob,
                                 const int32_t* cu_seqlens, int32_t num_seqs,
                                 int64_t total_frames, int32_t num_classes, int32_t window,
                                 int32_t stride, int32_t num_positions, int32_t* argmax,
                                 int32_t* tokens, int32_t* token_counts, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/* Static text for a status code. */
const char* gs_status_string(gs_status s);

/* Thread-local detail for the last non-OK status returned on this thread. */
const char* gs_last_error_detail(void);

/* Library version as major*10000 + minor*100 + patch. */
int32_t gs_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GSATTN_H */
