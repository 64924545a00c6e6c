/*
 * samba_gla.h -- C ABI of the MI355X (gfx950) gated linear attention layer,
 * which the hackernoon page "Microsoft's Samba Model Redefines Long-Context
 * Learning for AI" (§2) names, with Multi-Scale Retention, as a substitute
 * for the Mamba layer.  The page gives no formula; this library computes the
 * GLA paper's recurrence, per head h, with a decay per key dimension that
 * depends on the token:
 *     S_t[n][p] = exp(gk[t][h][n]) S_{t-1}[n][p] + k[t][h][n] v[t][h][p]
 *     o[t][h][p] = sum_n q[t][h][n] S_t[n][p]
 * gk is the log of the decay (<= 0; the gate's projection and any 1/sqrt(d)
 * scaling of q are the caller's).  The output normalisation and gate that
 * follow in the GLA layer are separate layers.
 *
 * Layout: q, k, gk [tokens][heads][dstate] (dstate = the key size N);
 * v, o [tokens][heads][head_dim] (head_dim = the value size P); h0, h_last
 * fp32 [nseq][heads][head_dim][dstate] (the state stored value-major).
 * Tokens: batch * seqlen rows, or packed sequences given by cu_seqlens as for
 * samba_scan_fwd.  q, k, v, gk share in_dtype (bf16 or fp32); o is y_dtype;
 * the state and all arithmetic are fp32.  Supported: dstate 16, 32, 64, 128
 * or 256, head_dim a multiple of 16 (32 at dstate 32, 64 at dstate 16), heads * head_dim * 4 * tokens
 * of a sequence below 2^32.  Alignment: h0, h_last 16 bytes; q, k, gk 16
 * bytes; v, o their element size.  o and h_last must not overlap any input,
 * except h_last == h0 exactly (the final state written in place).
 *
 * Two forms.  bf16 inputs with dstate 128 or 256 and head_dim a multiple of
 * 32 run the chunked form (the GLA paper's, §3 and §4.2): 64-token chunks
 * whose inter-chunk, intra-chunk and state products run on the matrix cores,
 * with every operand that is not an input as a bf16 hi + lo pair (16
 * significant bits; outputs within a few 1e-6 of the recurrence's scale).
 * Each call first writes, per (64-token chunk slot, head), the decayed q and
 * k, the chunk's decay and its intra-chunk matrix into a caller-owned device
 * workspace of samba_gla_workspace_size() bytes (256-byte aligned; 145 KiB
 * per slot and head at dstate 256; slots as for the SSD layer: nch per
 * batched sequence, tokens / 64 + nseq in all when packed), which the chunk
 * kernel then reads.  Calls that overlap in time need different workspaces;
 * it may not overlap any input or output (SAMBA_ERR_ALIASING); NULL or too
 * small is SAMBA_ERR_WORKSPACE.  For these calls v must also be 16-byte
 * aligned and o 8-byte (bf16) or 16-byte (fp32) aligned.  The other shapes
 * run the recurrence in fp32 (a diagonal scan per (head, value column), the
 * key dimension split over dstate / 4 lanes) and need no workspace.
 * Ownership, asynchrony and errors as for samba_scan.h.
 */
#ifndef SAMBA_GLA_H
#define SAMBA_GLA_H

#include "samba_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  uint32_t struct_size;        /* = sizeof(samba_gla_args) */
  int32_t batch, seqlen;
  int32_t heads, head_dim, dstate;
  const int32_t* cu_seqlens;   /* optional, device int32 [nseq + 1] (batch must be 1) */
  int32_t nseq;
  int32_t in_dtype, y_dtype;   /* samba_dtype values */
  const void *q, *k, *gk;      /* [tokens][heads][dstate] */
  const void* v;               /* [tokens][heads][head_dim] */
  const float* h0;             /* optional [nseq][heads][head_dim][dstate] */
  float* h_last;               /* optional, same shape */
  void* o;                     /* [tokens][heads][head_dim] */
  void* workspace;             /* device, samba_gla_workspace_size() bytes (chunked form only) */
  size_t workspace_bytes;
} samba_gla_args;

/* Host-only: bytes of workspace samba_gla_fwd needs for these sizes (0 for the
 * recurrent form, and when there are no tokens); validates like samba_gla_fwd. */
samba_status samba_gla_workspace_size(const samba_gla_args* args, size_t* bytes);

samba_status samba_gla_fwd(const samba_gla_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAMBA_GLA_H */
