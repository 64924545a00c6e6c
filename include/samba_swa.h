/*
 * samba_swa.h -- C ABI of the MI355X (gfx950) sliding-window attention layer
 * of the Samba hybrid (the layers between the Mamba layers).
 *
 * The operation: page "SAMBA混合注意力状态空间模型" (metaphor-xennon.pages.dev),
 * section 数学框架 -> 滑动窗口注意力: softmax(Q K^T / sqrt(d_k) + M) V with the
 * window mask M; the hackernoon page, §2.1.2: a window of w = 2048 tokens
 * sliding over the sequence, RoPE relative positions applied inside it.  The
 * mask as printed on the first page is inverted; this library reads it as:
 *     query i of a sequence sees keys j of the same sequence with
 *     i - window <= j <= i                         (causal, window + 1 keys)
 * and one key/value head per query head (the pages give no grouping).
 * Scale 1/sqrt(head_dim).  Window sizes by model size: 512 / 1024 / 2048
 * (page 1, 实现细节 -> 模型配置, with 16 or 24 heads).
 *
 * RoPE reading (the pages name RoPE, not its form): rotate-half pairs; for a
 * token at position p and c < head_dim / 2,
 *     x'[c]              = x[c] cos[p][c] - x[c + head_dim/2] sin[p][c]
 *     x'[c + head_dim/2] = x[c + head_dim/2] cos[p][c] + x[c] sin[p][c]
 * with caller-supplied fp32 tables cos, sin [npos][head_dim / 2] (the usual
 * choice is the angle p * base^(-2c / head_dim)).  Rotating q and k by their
 * own positions makes every score depend on relative position only.
 *
 * Layout: q, k, v, o are token-major [tokens][heads][head_dim] (one row of
 * heads * head_dim per token; tokens = batch * seqlen, sequence b in rows
 * b*seqlen .. b*seqlen+seqlen-1, or packed sequences given by cu_seqlens as
 * for samba_scan_fwd).  q, k, v are bf16; o is bf16 (round to nearest even) or
 * fp32.  Arithmetic: bf16 products on the matrix cores with fp32
 * accumulation; softmax in fp32 (the probabilities enter the P.V product as
 * bf16).
 *
 * Ownership, asynchrony and errors as for samba_scan.h: device pointers owned
 * by the caller, nothing allocated or kept, validation before anything is
 * enqueued, kernels enqueued on `stream` (hipStream_t as void*, NULL = the
 * default stream), status codes from samba_status.
 */
#ifndef SAMBA_SWA_H
#define SAMBA_SWA_H

#include "samba_scan.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * RoPE: rotate q and k (either may be NULL, with its output) by each token's
 * position, out of place or in place (q_out == q_in exactly; any other
 * overlap is SAMBA_ERR_ALIASING).  Positions: the token's index inside its
 * sequence, plus pos0[s] for sequence s when pos0 (device int32 [nseq]) is
 * given; a decode step is a batch of one-token sequences with pos0 = the
 * tokens' positions.  Positions outside [0, npos) are clamped into the table
 * (memory-safe; results for such input are unspecified).  head_dim a multiple
 * of 16 up to 4096, heads * head_dim at most 2^20; q/k 16-byte aligned;
 * tables 16-byte aligned.
 */
typedef struct {
  uint32_t struct_size;        /* = sizeof(samba_rope_args) */
  int32_t batch, seqlen, heads, head_dim;
  const int32_t* cu_seqlens;   /* optional, device, as for samba_scan_fwd (batch must be 1) */
  int32_t nseq;
  const int32_t* pos0;         /* optional, device [nseq]: position of each sequence's first token */
  const float *cos, *sin;      /* [npos][head_dim / 2] fp32 */
  int32_t npos;
  const void* q_in;            /* bf16 [tokens][heads][head_dim], optional */
  const void* k_in;            /* bf16 [tokens][heads][head_dim], optional */
  void* q_out;                 /* required with q_in */
  void* k_out;                 /* required with k_in */
} samba_rope_args;

samba_status samba_rope(const samba_rope_args* args, void* stream);

/*
 * Prefill: o = sliding-window attention of (q, k, v) over every sequence, q
 * and k already rotated (samba_rope).  head_dim 128.  window >= 0 (0: each
 * token sees only itself).  q, k, v 16-byte aligned; o its element size; o
 * must not overlap q, k or v.  Sequences as for samba_scan_fwd (cu_seqlens
 * out-of-range values are clamped on the device).
 */
typedef struct {
  uint32_t struct_size;        /* = sizeof(samba_swa_fwd_args) */
  int32_t batch, seqlen, heads, head_dim;
  const int32_t* cu_seqlens;   /* optional, device */
  int32_t nseq;
  int32_t window;
  int32_t out_dtype;           /* samba_dtype of o */
  const void *q, *k, *v;       /* bf16 [tokens][heads][head_dim] */
  void* o;                     /* [tokens][heads][head_dim] */
} samba_swa_fwd_args;

samba_status samba_swa_fwd(const samba_swa_fwd_args* args, void* stream);

/*
 * Decode step (page 1, section 推理效率: one new token per sequence attends to
 * its window through a cache of keys and values): for each of `batch`
 * sequences the new token at position pos[b] (device int32 [batch], >= 0)
 * has q, k, v rows [batch][heads][head_dim] (q and k rotated at pos[b]).
 * The call writes k and v into the cache slot pos[b] % cache_len, then
 * attends over the keys at positions max(0, pos[b] - window) .. pos[b], read
 * from slots p % cache_len of k_cache, v_cache [batch][heads][cache_len]
 * [head_dim] (bf16, in place).  cache_len >= window + 1; slots of positions
 * before pos[b] must hold what earlier steps (or the caller) wrote for them.
 * head_dim 128; q, k, v, caches 16-byte aligned; o [batch][heads][head_dim]
 * (out_dtype) must not overlap anything else; negative pos[b] reads as 0.
 */
typedef struct {
  uint32_t struct_size;        /* = sizeof(samba_swa_decode_args) */
  int32_t batch, heads, head_dim;
  int32_t window, cache_len;
  int32_t out_dtype;
  const int32_t* pos;          /* device [batch] */
  const void *q, *k, *v;       /* bf16 [batch][heads][head_dim] */
  void *k_cache, *v_cache;     /* bf16 [batch][heads][cache_len][head_dim] */
  void* o;                     /* [batch][heads][head_dim] */
} samba_swa_decode_args;

samba_status samba_swa_decode(const samba_swa_decode_args* args, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAMBA_SWA_H */
