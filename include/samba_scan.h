/*
 * samba_scan.h -- C ABI of the MI355X (gfx950) selective state-space scan.
 *
 * The operation (page "SAMBA混合注意力状态空间模型", metaphor-xennon.pages.dev,
 * section 数学框架 -> Mamba层): a diagonal linear recurrence per channel,
 *     h_t = Ā_t h_{t-1} + B̄_t x_t,   y_t = C_t h_t   (readout after the update),
 * with B_t, C_t and Δ_t chosen from the input.  The pages leave Ā, B̄ and τ_Δ
 * undefined; this library uses the Mamba reading, stated once here:
 *     Δ      = softplus(dt_raw + dt_bias[d])
 *     Ā[n]   = exp(Δ * A[d][n])          A diagonal, negative real (not checked)
 *     B̄x[n]  = Δ * B_t[n] * x_t
 *     y      = (sum_n C_t[n] h[n] + D[d] * x_t) * silu(z_t)
 * State size: 16 per channel (same page, section 实现细节 -> 模型配置).
 * Arithmetic is fp32 (state, discretisation, readout); x, dt, z, B, C are bf16
 * or fp32; y is written as bf16 (round to nearest even) or fp32.
 *
 * Layout (all row-major, contiguous, token-major):
 *     x, dt, z, y   [tokens][dim]        tokens = batch * seqlen (rows of batch b
 *                                        are tokens b*seqlen .. b*seqlen+seqlen-1)
 *     B, C          [tokens][16]         one vector per token, shared by all channels
 *     A             [dim][16]  fp32      D, dt_bias  [dim] fp32
 *     h0, h_last    [nseq][dim][16] fp32 (nseq = batch, or the cu_seqlens count)
 *     state (step)  [batch][dim][16] fp32
 *
 * Ownership: every pointer (except the args struct itself) is a DEVICE pointer
 * owned by the caller.  The library allocates no device memory, keeps no
 * pointers after a call returns, and caches only per-device properties.
 *
 * Asynchrony: calls validate on the host, then enqueue kernels on `stream`
 * (a hipStream_t passed as void*; NULL = the default stream) and return.
 * Results are valid once the caller synchronises that stream.  Calls on one
 * stream run in order; calls on different streams must not share outputs.
 *
 * Errors: all validation happens before anything is enqueued; on any error
 * nothing is enqueued and no output is touched.  A failed launch returns
 * SAMBA_ERR_HIP.  Faults inside a kernel surface at the caller's next
 * synchronisation.  No C++ exception crosses this interface.
 */
#ifndef SAMBA_SCAN_H
#define SAMBA_SCAN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SAMBA_SCAN_ABI_VERSION 13
#define SAMBA_DSTATE 16

typedef enum {
  SAMBA_OK = 0,
  SAMBA_ERR_NULL_ARG = 1,      /* a required pointer is NULL */
  SAMBA_ERR_BAD_SHAPE = 2,     /* negative / inconsistent sizes, or varlen with batch != 1 */
  SAMBA_ERR_BAD_DTYPE = 3,     /* in_dtype / y_dtype not a samba_dtype value */
  SAMBA_ERR_MISALIGNED = 4,    /* a pointer violates its alignment rule (below) */
  SAMBA_ERR_ALIASING = 5,      /* an output overlaps an input it must not overlap */
  SAMBA_ERR_UNSUPPORTED = 6,   /* dstate != 16, or time_slices not 0/1/2/4/8/16 */
  SAMBA_ERR_BAD_STRUCT = 7,    /* struct_size does not match this header */
  SAMBA_ERR_HIP = 8,           /* the HIP runtime refused the launch */
  SAMBA_ERR_WORKSPACE = 9      /* workspace NULL or too small (backward, SSD prefill, chunked GLA) */
} samba_status;

typedef enum { SAMBA_F32 = 0, SAMBA_BF16 = 1 } samba_dtype;

/*
 * Prefill: scan every sequence from its carry-in h0 (zeros if NULL) over its
 * tokens, write y for every token and, if h_last is not NULL, each sequence's
 * final state.  "Unlimited streaming" (page 2 abstract; hackernoon page,
 * abstract and §1) is served by chaining calls: pass one call's h_last as the
 * next call's h0; the result equals one call over the concatenated tokens.
 *
 * Sequences: without cu_seqlens, `batch` rows of `seqlen` tokens each.  With
 * cu_seqlens (device int32 [nseq+1], cu[0] = 0, ascending, cu[nseq] =
 * seqlen), batch must be 1 and the `seqlen` tokens hold nseq packed
 * sequences; each restarts from its own h0 row and writes its own h_last row.
 * Out-of-range or descending offsets are clamped into [0, seqlen] on the
 * device (memory-safe; results for such input are unspecified).
 *
 * Sizes: 1 <= dim < 2^24 (SAMBA_ERR_BAD_SHAPE otherwise: the kernels address
 * a lane's elements within a slice of token rows with 32-bit byte offsets).
 * Pointers: x, dt, z, B, C, y may be NULL only when there are no tokens.
 * Alignment: B, C, A, h0, h_last 16 bytes; x, dt, z, y, D, dt_bias their
 * element size.  h_last may equal h0 exactly (in-place carry); any other
 * overlap of an output (y, h_last) with an input is SAMBA_ERR_ALIASING.
 * time_slices: 0 lets the library choose how many waves split each time chunk
 * of one channel tile (1, 2, 4, 8 or 16); other values force it (testing and
 * tuning; results agree to fp32 rounding, and are bitwise reproducible for a
 * given choice).
 * lanes_per_channel: 0 lets the library choose how many lanes share one
 * channel's 16 states in a time-split launch: 4 (16-channel tiles) or 8
 * (8-channel tiles: twice the workgroups, for few sequences); other values
 * force it.  8 needs time_slices 0 or >= 2 and no h_ckpt (else
 * SAMBA_ERR_UNSUPPORTED); h_ckpt always runs the 4-lane kernel.
 *
 * h_ckpt (optional output, fp32, 16-byte aligned): the state before every 8th
 * token of each sequence, for a later samba_scan_bwd of the same inputs (a
 * training forward keeps them instead of the backward recomputing them).  A
 * call with h_ckpt runs the 4-lane kernel: y and h_last equal, bit for bit,
 * those of the same call without h_ckpt and lanes_per_channel = 4.  The
 * state before token 8j of sequence s (first token row start_s) is slot
 * floor(start_s / 8) + s + j of an array [slots][dim][16], slots = tokens / 8 +
 * nseq + 1 (samba_scan_ckpt_bytes); slots no sequence uses are not written.
 * It must not overlap any other argument.
 */
typedef struct {
  uint32_t struct_size;        /* = sizeof(samba_scan_fwd_args) */
  int32_t batch, seqlen, dim, dstate;
  const int32_t* cu_seqlens;   /* optional, device */
  int32_t nseq;                /* number of packed sequences when cu_seqlens != NULL */
  int32_t in_dtype, y_dtype;   /* samba_dtype */
  int32_t time_slices;         /* 0 = automatic */
  const void *x, *dt, *z;
  const void *B, *C;
  const float *A, *D, *dt_bias;
  const float* h0;             /* optional */
  float* h_last;               /* optional */
  void* y;
  float* h_ckpt;               /* optional: states every 8 tokens, for the backward */
  int32_t lanes_per_channel;   /* 0 = automatic; 4 or 8 force the kernel (see above) */
} samba_scan_fwd_args;

/*
 * Decode: one token for each of `batch` sequences (page 1, section 推理效率:
 * the per-token constant-time state update of generation).  The state is read
 * and written IN PLACE; y gets one value per (sequence, channel).
 * Alignment: state, B, C, A 16 bytes; others their element size.  y must not
 * overlap state or any input.
 */
typedef struct {
  uint32_t struct_size;        /* = sizeof(samba_scan_step_args) */
  int32_t batch, dim, dstate;
  int32_t in_dtype, y_dtype;
  float* state;                /* [batch][dim][16], in place */
  const void *x, *dt, *z;      /* [batch][dim] */
  const void *B, *C;           /* [batch][16] */
  const float *A, *D, *dt_bias;
  void* y;                     /* [batch][dim] */
} samba_scan_step_args;

/*
 * Backward of the prefill: gradients of every input of samba_scan_fwd for the
 * loss sum(dy * y) + sum(dh_last * h_last), i.e. the reverse-mode derivative
 * of the operation above (the pages train Samba with this scan: page 1,
 * section 实现细节 -> 训练配置; hackernoon page, §2.1.2).  Per token t of a
 * sequence and channel d, with v = dt_raw + dt_bias, Δ = softplus(v) and
 * r = sum_n C_t[n] h_t[n] + D x_t:
 *     g_t[n]  = dr_t C_t[n] + Ā_{t+1}[n] g_{t+1}[n]   adjoint of h_t (dh_last after the last token)
 *     dr_t    = dy_t silu(z_t);       dz_t = dy_t r_t silu'(z_t)
 *     dx_t    = dr_t D + Δ_t sum_n g_t[n] B_t[n]
 *     ddt_t   = sigmoid(v) sum_n g_t[n] (A[n] Ā_t[n] h_{t-1}[n] + B_t[n] x_t)
 *     dB_t[n] = sum_d g_t[n] Δ_t x_t,   dC_t[n] = sum_d dr_t h_t[n]
 *     dA[d][n] = sum g_t[n] Δ_t Ā_t[n] h_{t-1}[n],  dD[d] = sum dr_t x_t,  ddt_bias[d] = sum ddt_t
 *     dh0[n]  = Ā_first[n] g_first[n]   (dh_last for an empty sequence)
 * The forward states are recomputed inside the call from x, dt, B and h0, or,
 * when h_ckpt is given, from those checkpoints: the h_ckpt a samba_scan_fwd
 * call wrote for the same x, dt, B, h0 and sequences (with time_slices 0 on
 * both sides the two routes give bitwise the same gradients).
 *
 * Shapes and dtypes: x, dt, z, B, C, cu_seqlens, A, D, dt_bias, h0 exactly as
 * for samba_scan_fwd (in_dtype; also 1 <= dim < 2^24).  dy [tokens][dim] and the outputs dx, ddt, dz
 * [tokens][dim] have in_dtype too.  dB, dC [tokens][16], dA [dim][16], dD,
 * ddt_bias [dim] are fp32 and are overwritten (not accumulated).  dh_last
 * (input) and dh0 (output) are fp32 [nseq][dim][16] and optional (NULL:
 * zeros / not written).  Alignment: as for the forward, plus dB, dC, dA,
 * dh_last, dh0 16 bytes, dy/dx/ddt/dz their element size, workspace 256
 * bytes.  No output may overlap an input or another output.
 *
 * Workspace: caller-owned device memory of at least
 * samba_scan_bwd_workspace_size() bytes (checkpointed states every 8 tokens
 * unless h_ckpt is given, per-tile partial sums of dB and dC, per-sequence
 * partial sums of dA, dD and ddt_bias).  Calls that overlap in time must use different workspaces.
 * time_slices: 0 = automatic, else 1, 2, 4 or 8 waves per time chunk of a
 * channel tile (results agree to fp32 rounding; bitwise reproducible for a
 * given choice).
 */
typedef struct {
  uint32_t struct_size;        /* = sizeof(samba_scan_bwd_args) */
  int32_t batch, seqlen, dim, dstate;
  const int32_t* cu_seqlens;   /* optional, device */
  int32_t nseq;
  int32_t in_dtype;            /* x, dt, z, B, C, dy, dx, ddt, dz */
  int32_t time_slices;         /* 0 = automatic */
  const void *x, *dt, *z;
  const void *B, *C;
  const float *A, *D, *dt_bias;
  const float* h0;             /* optional */
  const void* dy;
  const float* dh_last;        /* optional */
  const float* h_ckpt;         /* optional: checkpoints from samba_scan_fwd (see there) */
  void *dx, *ddt, *dz;
  float *dB, *dC;
  float *dA, *dD, *ddt_bias;
  float* dh0;                  /* optional */
  void* workspace;
  size_t workspace_bytes;
} samba_scan_bwd_args;

/* Host-only: bytes of the h_ckpt array for these sizes (nseq = batch without cu_seqlens):
 * (batch * seqlen / 8 + nseq + 1) * dim * 16 * 4; dim must satisfy the prefill's bound. */
samba_status samba_scan_ckpt_bytes(int32_t batch, int32_t seqlen, int32_t nseq, int32_t dim, size_t* bytes);

/* Host-only: bytes of workspace samba_scan_bwd needs for these sizes and for whether h_ckpt is given
 * (no other pointer is examined). */
samba_status samba_scan_bwd_workspace_size(const samba_scan_bwd_args* args, size_t* bytes);

/* Enqueue the backward.  See samba_scan_bwd_args. */
samba_status samba_scan_bwd(const samba_scan_bwd_args* args, void* stream);

/*
 * Selection projections (page "SAMBA混合注意力状态空间模型", 数学框架 -> Mamba层:
 * B_t = Linear_B(x_t), C_t = Linear_C(x_t), and Linear_Δ(x_t) inside τ_Δ): the
 * three linear maps that produce the scan's dt, B and C from its input x, as
 * one bf16 GEMM on the matrix cores with fp32 accumulation.
 *     out[t][j] = sum_k x[t][k] * W[j][k],  j < dim + 2*dstate
 *     dt[t][j] = out[t][j] (j < dim);  B[t][n] = out[t][dim + n];  C[t][n] = out[t][dim + dstate + n]
 * W [dim + 2*dstate][dim] holds the maps as rows (one output feature per row,
 * as a linear layer stores its weight): Linear_Δ (dim rows, full rank), then
 * Linear_B, then Linear_C.  No bias (τ_Δ's bias is dt_bias of the scan).
 * x [tokens][dim] and W are bf16 (in_dtype must be SAMBA_BF16), 16-byte
 * aligned, dim a multiple of 8 and below 2^22; dt [tokens][dim], B and C [tokens][dstate]
 * are written in out_dtype (bf16 round to nearest even, or fp32), aligned to
 * their element size, and must not overlap x, W or each other.  The outputs
 * feed samba_scan_fwd / samba_scan_bwd directly (same layouts).  bf16
 * results go out as 16-byte chunks where dt (and B, C with dstate a multiple
 * of 8) are 16-byte aligned, element by element otherwise; the result is the
 * same either way.
 */
typedef struct {
  uint32_t struct_size;        /* = sizeof(samba_proj_args) */
  int32_t tokens, dim, dstate;
  int32_t in_dtype, out_dtype;
  const void* x;               /* [tokens][dim] bf16 */
  const void* W;               /* [dim + 2*dstate][dim] bf16 */
  void *dt, *B, *C;            /* [tokens][dim], [tokens][dstate], [tokens][dstate] */
} samba_proj_args;

/* Enqueue the selection projections.  See samba_proj_args. */
samba_status samba_proj(const samba_proj_args* args, void* stream);

/*
 * Grouped prefill: samba_scan_fwd generalised to ngroups (B, C) vectors per
 * token and to state sizes 16, 32, 64, 128 or 256 (the pages' selection is
 * the case ngroups = 1, dstate = 16; same recurrence, discretisation, skip
 * and gate).  Channel d reads group d / (dim / ngroups): contiguous blocks of
 * channels share a group.  B, C are [tokens][ngroups][dstate] in in_dtype;
 * A [dim][dstate]; h0, h_last [nseq][dim][dstate] fp32; everything else as
 * for samba_scan_fwd (batched rows or cu_seqlens, optional h0 / h_last, h_last
 * may equal h0 exactly).  Constraints: dim divisible by ngroups and each
 * group's dim / ngroups channels a multiple of 256 / dstate (a wave's
 * channels share a group); per sequence tokens * dim * 4 < 2^32.  Alignment:
 * B, C, A, h0, h_last 16 bytes; others their element size.  No time slicing:
 * parallelism comes from sequences x channels x dstate / 4 lanes.
 */
typedef struct {
  uint32_t struct_size;        /* = sizeof(samba_scan_groups_args) */
  int32_t batch, seqlen, dim, dstate, ngroups;
  const int32_t* cu_seqlens;   /* optional, device */
  int32_t nseq;
  int32_t in_dtype, y_dtype;
  const void *x, *dt, *z;      /* [tokens][dim] */
  const void *B, *C;           /* [tokens][ngroups][dstate] */
  const float *A, *D, *dt_bias;
  const float* h0;             /* optional */
  float* h_last;               /* optional */
  void* y;
} samba_scan_groups_args;

/* Enqueue a grouped prefill.  See samba_scan_groups_args. */
samba_status samba_scan_fwd_groups(const samba_scan_groups_args* args, void* stream);

/*
 * Grouped decode step: samba_scan_step with ngroups (B, C) vectors per token
 * ([batch][ngroups][dstate]) and 16, 32, 64, 128 or 256 states; state
 * [batch][dim][dstate] fp32 read and written in place; dim divisible by
 * ngroups.  Alignment: state and A 16 bytes, others their element size; y
 * must not overlap the state or any input.
 */
typedef struct {
  uint32_t struct_size;        /* = sizeof(samba_scan_step_groups_args) */
  int32_t batch, dim, dstate, ngroups;
  int32_t in_dtype, y_dtype;
  float* state;                /* [batch][dim][dstate], in place */
  const void *x, *dt, *z;      /* [batch][dim] */
  const void *B, *C;           /* [batch][ngroups][dstate] */
  const float *A, *D, *dt_bias;
  void* y;                     /* [batch][dim] */
} samba_scan_step_groups_args;

/* Enqueue one grouped decode step.  See samba_scan_step_groups_args. */
samba_status samba_scan_step_groups(const samba_scan_step_groups_args* args, void* stream);

/* Enqueue a prefill scan.  See samba_scan_fwd_args. */
samba_status samba_scan_fwd(const samba_scan_fwd_args* args, void* stream);

/* Enqueue one decode step.  See samba_scan_step_args. */
samba_status samba_scan_step(const samba_scan_step_args* args, void* stream);

/*
 * Host-only: validate `args` and report the launch the library would make on
 * the current device (time slices per channel tile, workgroups, threads per
 * workgroup, lanes per channel).  Enqueues nothing.  Any of the out pointers
 * may be NULL.
 */
samba_status samba_scan_fwd_plan(const samba_scan_fwd_args* args, int32_t* time_slices,
                                 int32_t* workgroups, int32_t* threads_per_workgroup,
                                 int32_t* lanes_per_channel);

/* Static, human-readable name of a status code ("unknown status" otherwise). */
const char* samba_status_string(int status);

/* SAMBA_SCAN_ABI_VERSION of the built library. */
int samba_scan_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SAMBA_SCAN_H */
