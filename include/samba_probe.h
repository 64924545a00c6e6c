/* samba_probe.h -- issue-rate probes of the gfx950 vector ALU (measurement only; not part of the scan).
 *
 * The selective scan's prefill (page "SAMBA混合注意力状态空间模型", 数学框架 -> Mamba层) is bound by plain
 * vector arithmetic: exponentials for Ā = exp(ΔA) and fp32 multiplies / fused multiply-adds.  These probes
 * measure the issue rate of exactly those instruction forms on the device, so that the prefill's ALU
 * roofline rests on a measured ceiling.  Built into libsamba_probe.so with the scan library's flags.
 *
 * samba_probe_alu(kind, blocks, iters, out, stream)
 *   Enqueues one launch of `blocks` workgroups of 256 threads on `stream` (a hipStream_t as void*; NULL =
 *   the default stream).  Every thread runs `iters` rounds of samba_probe_instructions_per_round(kind)
 *   independent instructions of the named form and writes one float to out[block * 256 + thread]; `out`
 *   is a caller-owned DEVICE buffer of at least blocks * 256 floats.  The value written has no meaning.
 *   Returns 0 when enqueued, 1 for a bad argument (nothing enqueued), 2 when the launch failed.
 *   Instructions executed = blocks * 256 / 64 waves * iters * instructions_per_round (per wave, one
 *   wave-wide instruction counts once; lane operations are 64 times that).
 */
#ifndef SAMBA_PROBE_H
#define SAMBA_PROBE_H

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SAMBA_PROBE_FMAC_VOP2 = 0,     /* v_fmac_f32 (two VGPR sources, addend in the destination) */
  SAMBA_PROBE_FMA_VOP3 = 1,      /* v_fma_f32 with three VGPR sources */
  SAMBA_PROBE_MUL_VOP2 = 2,      /* v_mul_f32 */
  SAMBA_PROBE_FMAC_SGPR = 3,     /* v_fmac_f32 with a scalar-register multiplicand */
  SAMBA_PROBE_EXP = 4,           /* v_exp_f32 (2^x) */
  SAMBA_PROBE_LOG = 5,           /* v_log_f32 (log2 x) */
  SAMBA_PROBE_RCP = 6,           /* v_rcp_f32 */
  SAMBA_PROBE_DPP = 7,           /* v_add_f32 with a DPP quad permutation */
  SAMBA_PROBE_MIX_4FMAC_1EXP = 8 /* 2 v_fmac + 2 v_mul per v_exp: the scan's per-state mix */
};

int samba_probe_instructions_per_round(int kind);
int samba_probe_alu(int kind, int blocks, int iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SAMBA_PROBE_H */
