// samba_scan_fwd_ilp.hip -- a second copy of the selective scan's prefill kernel (samba_scan_fwd.h) for the
// launch plans of inference calls (no checkpoints) where it runs faster: one wave per (sequence, 16-channel
// tile) with four tiles per workgroup, and 4, 8 or 16 waves splitting each time chunk.
//
// The build compiles this file alone with LLVM's max-ILP machine scheduler (-amdgpu-sched-strategy=max-ilp).
// The scheduler only orders instructions; every arithmetic operation is the same, so y and h_last are
// bitwise those of samba_scan.hip's copy (this copy is also built without the checkpoint branches, which an
// inference launch never takes, and stores y without a branch).  Measured on MI355X in alternating rounds:
// the 16384-token launch at D 4096 (16 slices) 2.6-4 % faster, 8 slices 1 %, the sequential kernel 1-5 %;
// 4 slices (B4 L4096 D4096) 2.7 % faster with the branch-free stores (the scheduler alone was not).  With
// checkpoint writes, and for the backward, grouped, SSD and 8-lane kernels the default scheduler measured
// faster, so those stay in samba_scan.hip.
#include "samba_scan_fwd.h"

namespace samba_fwd {

namespace {

template <typename Tin, typename Tout>
hipError_t launch_typed(int W, dim3 grid, dim3 block, const FwdParams& p, hipStream_t st) {
  switch (W) {
    case 1: hipLaunchKernelGGL((scan_fwd_kernel<Tin, Tout, 1, 4, 16, false, true>), grid, block, 0, st, p); break;
    case 4: hipLaunchKernelGGL((scan_fwd_kernel<Tin, Tout, 4, 1, 8, false, true>), grid, block, 0, st, p); break;
    case 8: hipLaunchKernelGGL((scan_fwd_kernel<Tin, Tout, 8, 1, 8, false, true>), grid, block, 0, st, p); break;
    case 16: hipLaunchKernelGGL((scan_fwd_kernel<Tin, Tout, 16, 1, 8, false, true>), grid, block, 0, st, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_ilp(bool in_bf16, bool out_bf16, int W, dim3 grid, dim3 block, const FwdParams& p,
                          hipStream_t st) {
  if (in_bf16) return out_bf16 ? launch_typed<uint16_t, uint16_t>(W, grid, block, p, st)
                               : launch_typed<uint16_t, float>(W, grid, block, p, st);
  return out_bf16 ? launch_typed<float, uint16_t>(W, grid, block, p, st)
                  : launch_typed<float, float>(W, grid, block, p, st);
}

}  // namespace samba_fwd
