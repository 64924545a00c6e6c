/*
 * samba_ssd.h -- C ABI of the MI355X (gfx950) state-space duality layer: the
 * Mamba-2 form that page "SAMBA混合注意力状态空间模型" (metaphor-xennon.pages.dev)
 * compares Samba with (与其他混合架构对比 and 设计哲学对比: SSD, 状态空间对偶).
 * The pages name the form and give no formula; this library takes its usual
 * definition, in the conventions of samba_scan.h:
 *     Δ_t = softplus(dt[t][h] + dt_bias[h]),  a_t = exp(Δ_t A[h])    (A[h] < 0)
 *     H_t = a_t H_{t-1} + Δ_t x_t B_tᵀ          (H: head_dim x dstate per head)
 *     y_t = (H_t C_t + D[h] x_t) * silu(z_t)     (no gate when z is NULL)
 * i.e. a scalar decay per head (instead of the diagonal A[d][n] of the
 * selective scan) and a matrix state per head; the (B, C) of group g serve
 * heads g*heads/ngroups .. (g+1)*heads/ngroups - 1.  With a scalar decay the
 * prefill is computed in chunks of 64 tokens as dense products on the matrix
 * cores: inside a chunk y = (L ∘ C Bᵀ) x with the decay mask L, across chunks
 * through the carried state.
 *
 * Layout: x, z, y [tokens][heads][head_dim]; dt [tokens][heads]; B, C
 * [tokens][ngroups][dstate]; A, D, dt_bias fp32 [heads]; h0, h_last fp32
 * [nseq][heads][head_dim][dstate].  Tokens: batch * seqlen rows (sequence b
 * in rows b*seqlen ..), or packed sequences given by cu_seqlens as for
 * samba_scan_fwd (out-of-range offsets clamped on the device).
 * Types: x, dt, z, B, C bf16; y bf16 (round to nearest even) or fp32; the
 * state fp32.  Arithmetic: bf16 products with fp32 accumulation, where every
 * operand that is not an input (the masked C Bᵀ, the state, the decay-weighted
 * x) enters as a pair of bf16 values whose sum carries 16 significant bits.
 * Supported: head_dim 64, dstate 64 or 128, heads a multiple of ngroups.
 * Alignment: x, B, C, h0, h_last 16 bytes; z 8; y 8 (bf16) or 16 (fp32);
 * dt 2; A, D, dt_bias 4.  y and h_last must not overlap any input, except
 * h_last == h0 exactly (the final state written in place over the initial).
 *
 * Workspace: none by default.  The products C Bᵀ of each chunk are formed by
 * the prefill kernel itself (cb_mode below).  With cb_mode
 * SAMBA_SSD_CB_PREPASS a first kernel writes them, once per (chunk, group),
 * into a caller-owned device workspace of samba_ssd_workspace_size() bytes
 * (256-byte aligned; 12 KiB per chunk slot and group, about 3 MiB for
 * 4 x 4096 tokens and one group), which the prefill kernel then reads.  Calls
 * that overlap in time must use different workspaces; the workspace may not
 * overlap any input or output (SAMBA_ERR_ALIASING); NULL or too small is
 * SAMBA_ERR_WORKSPACE.  Without a workspace (size 0) the pointer is ignored.
 *
 * Ownership, asynchrony and errors as for samba_scan.h: device pointers owned
 * by the caller, nothing allocated or kept, validation before anything is
 * enqueued, kernels enqueued on `stream` (hipStream_t as void*, NULL = the
 * default stream), status codes from samba_status.
 */
#ifndef SAMBA_SSD_H
#define SAMBA_SSD_H

#include "samba_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  uint32_t struct_size;        /* = sizeof(samba_ssd_args) */
  int32_t batch, seqlen;
  int32_t heads, head_dim, dstate, ngroups;
  const int32_t* cu_seqlens;   /* optional, device int32 [nseq + 1] (batch must be 1) */
  int32_t nseq;
  int32_t y_dtype;             /* samba_dtype of y */
  const void* x;               /* bf16 [tokens][heads][head_dim] */
  const void* dt;              /* bf16 [tokens][heads] */
  const void* z;               /* bf16 [tokens][heads][head_dim], optional */
  const void *B, *C;           /* bf16 [tokens][ngroups][dstate] */
  const float *A, *D, *dt_bias;  /* [heads] */
  const float* h0;             /* optional [nseq][heads][head_dim][dstate] */
  float* h_last;               /* optional, same shape */
  void* y;                     /* [tokens][heads][head_dim] */
  void* workspace;             /* device, samba_ssd_workspace_size() bytes */
  size_t workspace_bytes;
  int32_t cb_mode;             /* samba_ssd_cb_mode: where C Bᵀ is formed (0 = the library chooses) */
} samba_ssd_args;

/* Where the products C Bᵀ are formed.  SAMBA_SSD_CB_PREPASS: a first kernel writes them once per (chunk,
 * group) into the workspace and the prefill reads them back (shared by the heads of a group).
 * SAMBA_SSD_CB_IN_KERNEL: the prefill kernel's helper waves form each chunk's tiles on the matrix cores
 * from B and C as they stream by (per head; no workspace: samba_ssd_workspace_size() is 0).  Both give
 * bit for bit the same results.  SAMBA_SSD_CB_AUTO takes the in-kernel form.  Other values:
 * SAMBA_ERR_UNSUPPORTED. */
enum samba_ssd_cb_mode { SAMBA_SSD_CB_AUTO = 0, SAMBA_SSD_CB_PREPASS = 1, SAMBA_SSD_CB_IN_KERNEL = 2 };

/* Host-only: bytes of workspace samba_ssd_fwd needs for these sizes (0 when
 * there are no tokens); validates the sizes like samba_ssd_fwd. */
samba_status samba_ssd_workspace_size(const samba_ssd_args* args, size_t* bytes);

samba_status samba_ssd_fwd(const samba_ssd_args* args, void* stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): samba_ssd_fwd with the C Bᵀ tiles of the pre-pass form
 * (SAMBA_SSD_CB_PREPASS) in a static scratch array of SAMBA_SSD_SCRATCH_BYTES that the library holds on
 * each GPU it runs on (until the process ends), instead of a caller workspace; the default form needs no
 * scratch and the call then only enqueues the prefill.  Same arguments, results bit for bit those of
 * samba_ssd_fwd; args->workspace and workspace_bytes are ignored.  A pre-pass call whose
 * samba_ssd_workspace_size() exceeds SAMBA_SSD_SCRATCH_BYTES
 * (16 MiB: 1365 chunk slots x groups of 12 KiB, e.g. 87,360 tokens with one group) is refused with
 * SAMBA_ERR_WORKSPACE before anything is enqueued.  The call allocates nothing: on its first use on a
 * device it looks up that device's copy of the array (SAMBA_ERR_HIP if that fails).  Every call on one
 * GPU shares that GPU's array: calls that overlap in time on one GPU (other streams, other host threads)
 * race and must be serialised by the caller.  The array needs no clearing: each call writes every tile it
 * reads before reading it.
 */
#define SAMBA_SSD_SCRATCH_BYTES (16u << 20)
samba_status samba_ssd_fwd_noalloc(const samba_ssd_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAMBA_SSD_H */
