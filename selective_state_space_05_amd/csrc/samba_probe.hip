// samba_probe.hip -- issue-rate probes of the gfx950 vector ALU forms the scan kernels are built from.
//
// The prefill of the selective scan is bound by plain vector arithmetic: per (token, channel) 16
// exponentials for Ā = exp(ΔA) and about 75 fp32 multiplies and fused multiply-adds (page
// "SAMBA混合注意力状态空间模型", 数学框架 -> Mamba层, with the Mamba discretisation the library adopts).
// Its roofline therefore needs the chip's measured issue rate of exactly those instruction forms, built
// with the library's own flags (packed fp32 forms disabled).  Each probe kernel runs a fixed number of
// rounds of independent instructions of one form (or a fixed mix) in every lane; the rate follows from
// the instruction count and the launch time the caller measures.  The instructions are written as inline
// assembly so that the form is exactly the one named (two-operand VOP2 with the addend in the
// destination, three-VGPR VOP3, a scalar-register operand, DPP, the transcendentals); they touch no
// memory.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "samba_probe.h"

namespace {

constexpr int kChains = 16;  // independent destinations per lane: enough to hide the dependent latency

template <int KIND>
__global__ __launch_bounds__(256) void alu_probe_kernel(int iters, float seed, float* out) {
  float acc[kChains], src[kChains], tmp[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) {
    acc[i] = seed * static_cast<float>(i + 1) + static_cast<float>(threadIdx.x) * 1e-7f;
    src[i] = 0.25f + 0.01f * static_cast<float>(i);
    tmp[i] = 0.f;
  }
  const float a = seed * 0.5f, b = 0.999f;
  for (int it = 0; it < iters; ++it) {
    // each statement form is issued for all chains in turn, so that consecutive instructions are
    // independent (no back-to-back dependence, which would add wait states)
    if constexpr (KIND == SAMBA_PROBE_FMAC_VOP2) {
#pragma unroll
      for (int i = 0; i < kChains; ++i) asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(acc[i]) : "v"(a), "v"(src[i]));
    } else if constexpr (KIND == SAMBA_PROBE_FMA_VOP3) {
      // ping-pong between two destinations: three distinct VGPR sources, no register moves
#pragma unroll
      for (int i = 0; i < kChains; ++i)
        asm volatile("v_fma_f32 %0, %1, %2, %3" : "=&v"(tmp[i]) : "v"(acc[i]), "v"(b), "v"(src[i]));
#pragma unroll
      for (int i = 0; i < kChains; ++i)
        asm volatile("v_fma_f32 %0, %1, %2, %3" : "=&v"(acc[i]) : "v"(tmp[i]), "v"(b), "v"(src[i]));
    } else if constexpr (KIND == SAMBA_PROBE_MUL_VOP2) {
#pragma unroll
      for (int i = 0; i < kChains; ++i) asm volatile("v_mul_f32_e32 %0, %1, %0" : "+v"(acc[i]) : "v"(b));
    } else if constexpr (KIND == SAMBA_PROBE_FMAC_SGPR) {
#pragma unroll
      for (int i = 0; i < kChains; ++i) asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(acc[i]) : "s"(seed), "v"(src[i]));  // kernel argument: an SGPR
    } else if constexpr (KIND == SAMBA_PROBE_EXP) {
#pragma unroll
      for (int i = 0; i < kChains; ++i) asm volatile("v_exp_f32_e32 %0, %1" : "=v"(acc[i]) : "v"(src[i]));
    } else if constexpr (KIND == SAMBA_PROBE_LOG) {
#pragma unroll
      for (int i = 0; i < kChains; ++i) asm volatile("v_log_f32_e32 %0, %1" : "=v"(acc[i]) : "v"(src[i]));
    } else if constexpr (KIND == SAMBA_PROBE_RCP) {
#pragma unroll
      for (int i = 0; i < kChains; ++i) asm volatile("v_rcp_f32_e32 %0, %1" : "=v"(acc[i]) : "v"(src[i]));
    } else if constexpr (KIND == SAMBA_PROBE_DPP) {
#pragma unroll
      for (int i = 0; i < kChains; ++i)
        asm volatile("v_add_f32_dpp %0, %1, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf"
                     : "+v"(acc[i]) : "v"(src[i]));
    } else if constexpr (KIND == SAMBA_PROBE_MIX_4FMAC_1EXP) {
      // the scan's per-state ratio: four two-operand multiply / fma forms per exponential
#pragma unroll
      for (int i = 0; i < kChains; ++i) asm volatile("v_mul_f32_e32 %0, %1, %2" : "=v"(tmp[i]) : "v"(a), "v"(src[i]));
#pragma unroll
      for (int i = 0; i < kChains; ++i) asm volatile("v_exp_f32_e32 %0, %1" : "=v"(src[i]) : "v"(tmp[i]));
#pragma unroll
      for (int i = 0; i < kChains; ++i) asm volatile("v_mul_f32_e32 %0, %1, %2" : "=v"(tmp[i]) : "v"(b), "v"(acc[i]));
#pragma unroll
      for (int i = 0; i < kChains; ++i) asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(tmp[i]) : "v"(a), "v"(src[i]));
#pragma unroll
      for (int i = 0; i < kChains; ++i) asm volatile("v_fmac_f32_e32 %0, %1, %2" : "+v"(acc[i]) : "v"(b), "v"(tmp[i]));
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kChains; ++i) s += acc[i] + src[i] + tmp[i];
  out[blockIdx.x * blockDim.x + threadIdx.x] = s;
}

template <int KIND>
hipError_t launch(int blocks, int iters, float* out, hipStream_t s) {
  hipLaunchKernelGGL(alu_probe_kernel<KIND>, dim3(blocks), dim3(256), 0, s, iters, 1.0001f, out);
  return hipGetLastError();
}

}  // namespace

extern "C" {

int samba_probe_instructions_per_round(int kind) {
  switch (kind) {
    case SAMBA_PROBE_FMA_VOP3:
      return 2 * kChains;
    case SAMBA_PROBE_FMAC_VOP2: case SAMBA_PROBE_MUL_VOP2:
    case SAMBA_PROBE_FMAC_SGPR: case SAMBA_PROBE_EXP: case SAMBA_PROBE_LOG: case SAMBA_PROBE_RCP:
    case SAMBA_PROBE_DPP:
      return kChains;
    case SAMBA_PROBE_MIX_4FMAC_1EXP:
      return 5 * kChains;
    default:
      return 0;
  }
}

int samba_probe_alu(int kind, int blocks, int iters, float* out, void* stream) {
  if (blocks < 1 || iters < 1 || !out) return 1;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (kind) {
    case SAMBA_PROBE_FMAC_VOP2: e = launch<SAMBA_PROBE_FMAC_VOP2>(blocks, iters, out, s); break;
    case SAMBA_PROBE_FMA_VOP3: e = launch<SAMBA_PROBE_FMA_VOP3>(blocks, iters, out, s); break;
    case SAMBA_PROBE_MUL_VOP2: e = launch<SAMBA_PROBE_MUL_VOP2>(blocks, iters, out, s); break;
    case SAMBA_PROBE_FMAC_SGPR: e = launch<SAMBA_PROBE_FMAC_SGPR>(blocks, iters, out, s); break;
    case SAMBA_PROBE_EXP: e = launch<SAMBA_PROBE_EXP>(blocks, iters, out, s); break;
    case SAMBA_PROBE_LOG: e = launch<SAMBA_PROBE_LOG>(blocks, iters, out, s); break;
    case SAMBA_PROBE_RCP: e = launch<SAMBA_PROBE_RCP>(blocks, iters, out, s); break;
    case SAMBA_PROBE_DPP: e = launch<SAMBA_PROBE_DPP>(blocks, iters, out, s); break;
    case SAMBA_PROBE_MIX_4FMAC_1EXP: e = launch<SAMBA_PROBE_MIX_4FMAC_1EXP>(blocks, iters, out, s); break;
    default: return 1;
  }
  return e == hipSuccess ? 0 : 2;
}

}  // extern "C"
