// samba_scan_groups.hip -- gfx950 (MI355X) prefill of the selective scan with several (B, C) groups per
// token and state sizes 16 .. 256 (the generalisation of the single selection vector and the 16 states
// of page "SAMBA混合注意力状态空间模型", 数学框架 -> Mamba层 / 实现细节 -> 模型配置).  Same recurrence,
// discretisation, skip and gate as samba_scan_fwd (the Mamba reading stated in samba_scan.h); channel d
// reads the (B, C) of group d / (dim / ngroups).
//
// Work decomposition: a channel's N states are split over N / 4 lanes (4 states per lane), so a wave
// covers 256 / N channels, all of one group (the host checks that a group's channels are a multiple of
// that).  Tokens advance 8 at a time:
//   * the wave stages the chunk's B and C rows of its group into LDS as fp32 (one contiguous run per
//     lane) and the per-token scalars are computed once per (token, channel) by one lane of the channel
//     (softplus, Δx, published to LDS; gate and skip kept for the output);
//   * every lane then runs the 8 state updates of its 4 states with Δ, Δx, B, C from LDS, and the
//     channel's partial readouts are summed over its N / 4 lanes by a butterfly (DPP within a 16-lane row,
//     the lane-16 and lane-32 swaps across rows for 128 and 256 states: no LDS round trip per token);
//   * the lane that computed a token's scalars forms and stores its output.
// The next chunk's loads are issued before the current chunk's arithmetic.  No state crosses waves: no
// workspace and no workgroup barrier (each wave has its own LDS region).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "samba_scan.h"

namespace {

using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw (untyped, unswizzled) buffer
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kTK = 8;                   // tokens per chunk
constexpr int kWaves = 4;                // waves per workgroup

__device__ __forceinline__ rsrc_t rsrc_bytes(const void* base, int64_t bytes) {
  const uint32_t b = bytes <= 0 ? 0u : (bytes >= 0xffffffffLL ? 0xffffffffu : static_cast<uint32_t>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(b),
                                          kRsrcWord3);
}

__device__ __forceinline__ float widen(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
__device__ __forceinline__ float widen(float v) { return v; }

__device__ __forceinline__ void ld_elem(rsrc_t r, uint32_t off, uint16_t& v) {
  v = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ void ld_elem(rsrc_t r, uint32_t off, float& v) {
  v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
__device__ __forceinline__ void st_elem(rsrc_t r, uint32_t off, float v, float*) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
__device__ __forceinline__ void st_elem(rsrc_t r, uint32_t off, float v, uint16_t*) {
  __builtin_amdgcn_raw_buffer_store_b16(__builtin_bit_cast(uint16_t, static_cast<__bf16>(v)), r, off, 0, 0);
}

// NW 32-bit words from a buffer, in 16-, 8- or 4-byte pieces.
template <int NW>
__device__ __forceinline__ void ld_words(rsrc_t r, uint32_t off, uint32_t (&w)[NW]) {
  if constexpr (NW >= 4) {
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16u * i, 0, 0);
      w[4 * i] = v[0]; w[4 * i + 1] = v[1]; w[4 * i + 2] = v[2]; w[4 * i + 3] = v[3];
    }
  } else if constexpr (NW == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    w[0] = v[0]; w[1] = v[1];
  } else {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  }
}

// softplus(v) = log(1 + e^v): log2 of 1 + e with the rounding of 1 + e undone to first order when e < 1
// (small Δ keep full relative accuracy); v > 20 returns v.
__device__ __forceinline__ float softplus_f32(float v) {
  const float e = __builtin_amdgcn_exp2f(v * kLog2e);
  const float u = 1.0f + e;
  const float lost = e - (u - 1.0f);
  const float r = fmaf(__builtin_amdgcn_logf(u), kLn2, e < 1.0f ? lost * (2.0f - u) : 0.0f);
  return v > 20.0f ? v : r;
}
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
// sum over the LPC consecutive lanes of a channel, in every one of them.  Each step adds the partner
// group's partial sum: after the quad steps a lane's 8-lane partner quad is its mirror in the half row,
// its 16-lane partner half the mirror in the row; across rows the permlane swaps give every lane both
// halves of a 32- or 64-lane group.
template <int LPC>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (LPC >= 8) v += dpp<0x141>(v);   // row_half_mirror
  if constexpr (LPC >= 16) v += dpp<0x140>(v);  // row_mirror
  if constexpr (LPC >= 32) {
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  if constexpr (LPC >= 64) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  return v;
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct GParams {
  const void *x, *dt, *z, *B, *C;
  const float *A, *Dskip, *bias, *h0;
  float* h_last;
  void* y;
  const int32_t* cu;
  int32_t nseq, seqlen, dim, ngroups, total;
  int32_t ntiles;   // channel tiles (4 waves' channels) per sequence; the grid is ntiles x nseq
};

// Block index -> logical index such that consecutive logical blocks land on the same XCD (the dispatcher
// deals blocks round-robin over the 8 XCDs).  A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7, xcd = bid & 7, slot = bid >> 3;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

template <typename Tin, typename Tout, int N>
__global__ __launch_bounds__(64 * kWaves) void scan_groups_kernel(GParams p) {
  constexpr int LPC = N / 4;              // lanes per channel
  constexpr int CPW = 64 / LPC;           // channels per wave
  constexpr int VPL = kTK * N / 64;       // B (and C) elements each lane stages per chunk
  constexpr int ES = sizeof(Tin);
  constexpr int NW = (VPL * ES + 3) / 4;  // 32-bit words per lane per tensor per chunk
  constexpr int IPL = (kTK * CPW + 63) / 64;   // (token, channel) items per lane per chunk: 2 at N = 16
  static_assert(VPL * ES >= 4, "staging runs of at least one word");
  __shared__ __attribute__((aligned(16))) float s_bc[kWaves][2][kTK][N];
  __shared__ __attribute__((aligned(16))) float s_du[kWaves][2][CPW][kTK];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // (channel tile, sequence) of this workgroup: consecutive tiles of a sequence on one XCD, so that its L2
  // assembles whole lines of x, dt, z and y from the few bytes per token each wave touches
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int s = logical / p.ntiles;
  const int tile = logical - s * p.ntiles;
  const int ch0 = (tile * kWaves + wave) * CPW;
  if (ch0 >= p.dim) return;               // a whole wave past the last channel
  int64_t t0;
  int32_t len;
  if (p.cu) {
    int32_t a = p.cu[s], e = p.cu[s + 1];
    a = a < 0 ? 0 : (a > p.total ? p.total : a);
    e = e < a ? a : (e > p.total ? p.total : e);
    t0 = a;
    len = e - a;
  } else {
    t0 = static_cast<int64_t>(s) * p.seqlen;
    len = p.seqlen;
  }
  const int g = ch0 / (p.dim / p.ngroups);
  const int sub = lane % LPC, cw = lane / LPC;
  const int d = ch0 + cw;

  // this lane's 4 states
  float a2[4], h[4];
  {
    const float4 av = reinterpret_cast<const float4*>(p.A + static_cast<int64_t>(d) * N)[sub];
    a2[0] = av.x * kLog2e; a2[1] = av.y * kLog2e; a2[2] = av.z * kLog2e; a2[3] = av.w * kLog2e;
    if (p.h0) {
      const float4 hv = reinterpret_cast<const float4*>(p.h0 + (static_cast<int64_t>(s) * p.dim + d) * N)[sub];
      h[0] = hv.x; h[1] = hv.y; h[2] = hv.z; h[3] = hv.w;
    } else {
      h[0] = h[1] = h[2] = h[3] = 0.f;
    }
  }
  // (token, channel) items of this lane: item i = lane + 64 k -> token i / CPW, channel i % CPW of the wave
  int it_j[IPL], it_c[IPL];
  float it_bias[IPL], it_dsk[IPL];
#pragma unroll
  for (int k = 0; k < IPL; ++k) {
    const int i = lane + 64 * k;
    it_j[k] = i / CPW;
    it_c[k] = i % CPW;
    it_bias[k] = p.bias[ch0 + it_c[k]];
    it_dsk[k] = p.Dskip[ch0 + it_c[k]];
  }
  const uint32_t row_bytes = static_cast<uint32_t>(p.dim) * ES;
  const uint32_t bc_row = static_cast<uint32_t>(p.ngroups) * N * ES;
  const int e0 = lane * VPL;               // staging run: token e0 / N, states e0 % N .. + VPL
  const int st_j = e0 / N, st_n = e0 % N;

  // chunk loads into registers
  Tin xv[IPL], dv[IPL], zv[IPL];
  uint32_t bw[NW], cwd[NW];
  auto load_chunk = [&](int c0) {
    const int64_t tok = t0 + c0;
    const int rows = len - c0;
    const int64_t remain = static_cast<int64_t>(rows < kTK ? rows : kTK);
    const rsrc_t rx = rsrc_bytes(static_cast<const Tin*>(p.x) + tok * p.dim, remain * row_bytes);
    const rsrc_t rd = rsrc_bytes(static_cast<const Tin*>(p.dt) + tok * p.dim, remain * row_bytes);
    const rsrc_t rz = rsrc_bytes(static_cast<const Tin*>(p.z) + tok * p.dim, remain * row_bytes);
#pragma unroll
    for (int k = 0; k < IPL; ++k) {
      const uint32_t off = static_cast<uint32_t>(it_j[k]) * row_bytes + static_cast<uint32_t>(ch0 + it_c[k]) * ES;
      ld_elem(rx, off, xv[k]);
      ld_elem(rd, off, dv[k]);
      ld_elem(rz, off, zv[k]);
    }
    const int64_t bbase = (tok * p.ngroups + g) * N;
    const rsrc_t rb = rsrc_bytes(static_cast<const Tin*>(p.B) + bbase, remain * bc_row);
    const rsrc_t rc = rsrc_bytes(static_cast<const Tin*>(p.C) + bbase, remain * bc_row);
    const uint32_t boff = static_cast<uint32_t>(st_j) * bc_row + static_cast<uint32_t>(st_n) * ES;
    ld_words<NW>(rb, boff, bw);
    ld_words<NW>(rc, boff, cwd);
  };
  auto widen_word = [&](const uint32_t (&w)[NW], int i) -> float {
    if constexpr (ES == 2) return (i & 1) ? __uint_as_float(w[i >> 1] & 0xffff0000u) : __uint_as_float(w[i >> 1] << 16);
    else return __uint_as_float(w[i]);
  };

  const rsrc_t ry = rsrc_bytes(static_cast<Tout*>(p.y) + t0 * p.dim, static_cast<int64_t>(len) * p.dim *
                                                                      static_cast<int64_t>(sizeof(Tout)));
  if (len > 0) load_chunk(0);
  for (int c0 = 0; c0 < len; c0 += kTK) {
    // publish this chunk: B, C rows (fp32) and the per-token Δ, Δx of every (token, channel)
    float* sb = &s_bc[wave][0][st_j][st_n];
    float* sc = &s_bc[wave][1][st_j][st_n];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      sb[i] = widen_word(bw, i);
      sc[i] = widen_word(cwd, i);
    }
    float gate[IPL], skip[IPL];
#pragma unroll
    for (int k = 0; k < IPL; ++k) {
      const bool ok = c0 + it_j[k] < len;     // tokens past the end leave the state alone
      const float delta = ok ? softplus_f32(widen(dv[k]) + it_bias[k]) : 0.f;
      const float xf = widen(xv[k]);
      if (it_j[k] < kTK) {
        s_du[wave][0][it_c[k]][it_j[k]] = delta;
        s_du[wave][1][it_c[k]][it_j[k]] = delta * xf;
      }
      gate[k] = silu_f32(widen(zv[k]));
      skip[k] = it_dsk[k] * xf;
    }
    wave_sync();
    if (c0 + kTK < len) load_chunk(c0 + kTK);
    // the chunk's 8 state updates of this lane's 4 states, readouts summed over the channel's lanes
    float dl[kTK], uu[kTK], r[kTK];
    {
      const float4* pd = reinterpret_cast<const float4*>(&s_du[wave][0][cw][0]);
      const float4* pu = reinterpret_cast<const float4*>(&s_du[wave][1][cw][0]);
      const float4 d0 = pd[0], d1 = pd[1], u0 = pu[0], u1 = pu[1];
      dl[0] = d0.x; dl[1] = d0.y; dl[2] = d0.z; dl[3] = d0.w; dl[4] = d1.x; dl[5] = d1.y; dl[6] = d1.z; dl[7] = d1.w;
      uu[0] = u0.x; uu[1] = u0.y; uu[2] = u0.z; uu[3] = u0.w; uu[4] = u1.x; uu[5] = u1.y; uu[6] = u1.z; uu[7] = u1.w;
    }
#pragma unroll
    for (int j = 0; j < kTK; ++j) {
      const float4 b4 = reinterpret_cast<const float4*>(&s_bc[wave][0][j][0])[sub];
      const float4 c4 = reinterpret_cast<const float4*>(&s_bc[wave][1][j][0])[sub];
      const float bb[4] = {b4.x, b4.y, b4.z, b4.w}, cc[4] = {c4.x, c4.y, c4.z, c4.w};
      float pr = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        h[i] = fmaf(__builtin_amdgcn_exp2f(dl[j] * a2[i]), h[i], uu[j] * bb[i]);
        pr = fmaf(cc[i], h[i], pr);
      }
      r[j] = group_sum<LPC>(pr);
    }
    // readouts to the item lanes through LDS (lane sub 0 of each channel writes the channel's 8 sums)
    wave_sync();
    if (sub == 0) {
      float4* pr = reinterpret_cast<float4*>(&s_du[wave][0][cw][0]);
      pr[0] = make_float4(r[0], r[1], r[2], r[3]);
      pr[1] = make_float4(r[4], r[5], r[6], r[7]);
    }
    wave_sync();
#pragma unroll
    for (int k = 0; k < IPL; ++k) {
      if (it_j[k] < kTK && c0 + it_j[k] < len && ch0 + it_c[k] < p.dim) {
        const float yv = (s_du[wave][0][it_c[k]][it_j[k]] + skip[k]) * gate[k];
        st_elem(ry, (static_cast<uint32_t>(c0 + it_j[k]) * p.dim + static_cast<uint32_t>(ch0 + it_c[k])) *
                        static_cast<uint32_t>(sizeof(Tout)),
                yv, static_cast<Tout*>(nullptr));
      }
    }
    wave_sync();   // the next chunk overwrites this wave's LDS
  }
  if (p.h_last) {
    reinterpret_cast<float4*>(p.h_last + (static_cast<int64_t>(s) * p.dim + d) * N)[sub] =
        make_float4(h[0], h[1], h[2], h[3]);
  }
}

// ---------------------------------------------------------------------------
// Grouped decode step: one token per sequence, state [batch][dim][N] read and written in place.  Lanes as
// in the prefill (N/4 per channel, 4 states each); the per-token scalars are recomputed by each of the
// channel's lanes (the step streams the state: N * 8 bytes per channel against ~20 issue slots of scalars).
// ---------------------------------------------------------------------------
struct SParams {
  float* state;
  const void *x, *dt, *z, *B, *C;
  const float *A, *Dskip, *bias;
  void* y;
  int32_t batch, dim, ngroups;
};

template <typename Tin, typename Tout, int N>
__global__ __launch_bounds__(256) void step_groups_kernel(SParams p) {
  constexpr int LPC = N / 4, CPB = 256 / LPC;   // lanes per channel, channels per workgroup
  const int64_t item = static_cast<int64_t>(blockIdx.x) * CPB + threadIdx.x / LPC;   // (sequence, channel)
  const int sub = threadIdx.x % LPC;
  const int64_t total = static_cast<int64_t>(p.batch) * p.dim;
  const bool live = item < total;
  const int64_t it = live ? item : total - 1;   // dead lanes mirror the last item (reads only)
  const int b = static_cast<int>(it / p.dim), d = static_cast<int>(it - static_cast<int64_t>(b) * p.dim);
  const int g = d / (p.dim / p.ngroups);
  const float xv = widen(static_cast<const Tin*>(p.x)[it]);
  const float delta = softplus_f32(widen(static_cast<const Tin*>(p.dt)[it]) + p.bias[d]);
  const float zv = widen(static_cast<const Tin*>(p.z)[it]);
  const int64_t bc = (static_cast<int64_t>(b) * p.ngroups + g) * N + 4 * sub;
  float bb[4], cc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    bb[i] = widen(static_cast<const Tin*>(p.B)[bc + i]);
    cc[i] = widen(static_cast<const Tin*>(p.C)[bc + i]);
  }
  const float4 av = reinterpret_cast<const float4*>(p.A + static_cast<int64_t>(d) * N)[sub];
  float4* sp = reinterpret_cast<float4*>(p.state + it * N) + sub;
  const float4 hv = *sp;
  const float a[4] = {av.x, av.y, av.z, av.w};
  float h[4] = {hv.x, hv.y, hv.z, hv.w};
  const float u = delta * xv;
  float pr = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    h[i] = fmaf(__builtin_amdgcn_exp2f(delta * a[i] * kLog2e), h[i], u * bb[i]);
    pr = fmaf(cc[i], h[i], pr);
  }
  const float r = group_sum<LPC>(pr);
  if (live) {
    *sp = make_float4(h[0], h[1], h[2], h[3]);
    if (sub == 0) {
      const float yv = (r + p.Dskip[d] * xv) * silu_f32(zv);
      if constexpr (sizeof(Tout) == 2)
        static_cast<uint16_t*>(p.y)[it] = __builtin_bit_cast(uint16_t, static_cast<__bf16>(yv));
      else
        static_cast<float*>(p.y)[it] = yv;
    }
  }
}

template <typename Tin, typename Tout>
hipError_t launch_step_groups(const SParams& p, int dstate, hipStream_t s) {
  const int64_t lanes = static_cast<int64_t>(p.batch) * p.dim * (dstate / 4);
  const dim3 grid(static_cast<uint32_t>((lanes + 255) / 256)), block(256);
  switch (dstate) {
    case 16: hipLaunchKernelGGL((step_groups_kernel<Tin, Tout, 16>), grid, block, 0, s, p); break;
    case 32: hipLaunchKernelGGL((step_groups_kernel<Tin, Tout, 32>), grid, block, 0, s, p); break;
    case 64: hipLaunchKernelGGL((step_groups_kernel<Tin, Tout, 64>), grid, block, 0, s, p); break;
    case 128: hipLaunchKernelGGL((step_groups_kernel<Tin, Tout, 128>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((step_groups_kernel<Tin, Tout, 256>), grid, block, 0, s, p); break;
  }
  return hipGetLastError();
}

bool aligned(const void* q, uintptr_t a) { return (reinterpret_cast<uintptr_t>(q) & (a - 1)) == 0; }
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

template <typename Tin, typename Tout>
hipError_t launch_groups(const GParams& p, int dstate, dim3 grid, hipStream_t s) {
  const dim3 block(64 * kWaves);
  switch (dstate) {
    case 16: hipLaunchKernelGGL((scan_groups_kernel<Tin, Tout, 16>), grid, block, 0, s, p); break;
    case 32: hipLaunchKernelGGL((scan_groups_kernel<Tin, Tout, 32>), grid, block, 0, s, p); break;
    case 64: hipLaunchKernelGGL((scan_groups_kernel<Tin, Tout, 64>), grid, block, 0, s, p); break;
    case 128: hipLaunchKernelGGL((scan_groups_kernel<Tin, Tout, 128>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((scan_groups_kernel<Tin, Tout, 256>), grid, block, 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

extern "C" samba_status samba_scan_fwd_groups(const samba_scan_groups_args* a, void* stream) {
  if (!a) return SAMBA_ERR_NULL_ARG;
  if (a->struct_size != sizeof(samba_scan_groups_args)) return SAMBA_ERR_BAD_STRUCT;
  if (a->batch < 0 || a->seqlen < 0 || a->dim < 1 || a->ngroups < 1 || a->nseq < 0) return SAMBA_ERR_BAD_SHAPE;
  const int N = a->dstate;
  if (N != 16 && N != 32 && N != 64 && N != 128 && N != 256) return SAMBA_ERR_UNSUPPORTED;
  if (a->in_dtype != SAMBA_F32 && a->in_dtype != SAMBA_BF16) return SAMBA_ERR_BAD_DTYPE;
  if (a->y_dtype != SAMBA_F32 && a->y_dtype != SAMBA_BF16) return SAMBA_ERR_BAD_DTYPE;
  // a group's channels must fill whole waves (256 / N channels each)
  if (a->dim % a->ngroups != 0 || (a->dim / a->ngroups) % (256 / N) != 0) return SAMBA_ERR_BAD_SHAPE;
  int64_t nseq;
  if (a->cu_seqlens) {
    if (a->batch != 1 || a->nseq < 1) return SAMBA_ERR_BAD_SHAPE;
    nseq = a->nseq;
  } else {
    nseq = a->batch;
  }
  const int64_t tokens = static_cast<int64_t>(a->batch) * a->seqlen;
  if (nseq == 0) return SAMBA_OK;
  if (static_cast<int64_t>(a->dim) * a->ngroups * N > (int64_t{1} << 28)) return SAMBA_ERR_BAD_SHAPE;
  if (static_cast<int64_t>(a->seqlen) * a->dim * 4 >= (int64_t{1} << 32)) return SAMBA_ERR_BAD_SHAPE;
  if (!a->A || !a->D || !a->dt_bias) return SAMBA_ERR_NULL_ARG;
  if (tokens > 0 && (!a->x || !a->dt || !a->z || !a->B || !a->C || !a->y)) return SAMBA_ERR_NULL_ARG;
  const size_t ie = a->in_dtype == SAMBA_BF16 ? 2 : 4, oe = a->y_dtype == SAMBA_BF16 ? 2 : 4;
  if (!aligned(a->x, ie) || !aligned(a->dt, ie) || !aligned(a->z, ie) || !aligned(a->y, oe) ||
      !aligned(a->B, 16) || !aligned(a->C, 16) || !aligned(a->A, 16) || !aligned(a->h0, 16) ||
      !aligned(a->h_last, 16) || !aligned(a->D, 4) || !aligned(a->dt_bias, 4))
    return SAMBA_ERR_MISALIGNED;
  const size_t td = static_cast<size_t>(tokens) * a->dim;
  const size_t tbc = static_cast<size_t>(tokens) * a->ngroups * N;
  const size_t st = static_cast<size_t>(nseq) * a->dim * N * 4;
  const void* ins[11] = {a->x, a->dt, a->z, a->B, a->C, a->A, a->D, a->dt_bias, a->h0, a->cu_seqlens, nullptr};
  const size_t in_sz[11] = {td * ie, td * ie, td * ie, tbc * ie, tbc * ie, static_cast<size_t>(a->dim) * N * 4,
                            static_cast<size_t>(a->dim) * 4, static_cast<size_t>(a->dim) * 4, st,
                            a->cu_seqlens ? (static_cast<size_t>(nseq) + 1) * 4 : 0, 0};
  for (int k = 0; k < 10; ++k) {
    if (overlap(a->y, td * oe, ins[k], in_sz[k])) return SAMBA_ERR_ALIASING;
    if (a->h_last && !(k == 8 && a->h_last == a->h0) && overlap(a->h_last, st, ins[k], in_sz[k]))
      return SAMBA_ERR_ALIASING;
  }
  if (overlap(a->y, td * oe, a->h_last, st)) return SAMBA_ERR_ALIASING;

  GParams p{};
  p.x = a->x; p.dt = a->dt; p.z = a->z; p.B = a->B; p.C = a->C;
  p.A = a->A; p.Dskip = a->D; p.bias = a->dt_bias; p.h0 = a->h0; p.h_last = a->h_last; p.y = a->y;
  p.cu = a->cu_seqlens;
  p.nseq = static_cast<int32_t>(nseq);
  p.seqlen = a->seqlen;
  p.dim = a->dim;
  p.ngroups = a->ngroups;
  p.total = a->seqlen;
  const int cpb = kWaves * (256 / N);
  p.ntiles = (a->dim + cpb - 1) / cpb;
  if (static_cast<int64_t>(p.ntiles) * nseq > 0x7fffffff) return SAMBA_ERR_BAD_SHAPE;
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.ntiles) * nseq));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (a->in_dtype == SAMBA_BF16)
    e = a->y_dtype == SAMBA_BF16 ? launch_groups<uint16_t, uint16_t>(p, N, grid, s)
                                 : launch_groups<uint16_t, float>(p, N, grid, s);
  else
    e = a->y_dtype == SAMBA_BF16 ? launch_groups<float, uint16_t>(p, N, grid, s)
                                 : launch_groups<float, float>(p, N, grid, s);
  return e == hipSuccess ? SAMBA_OK : SAMBA_ERR_HIP;
}

extern "C" samba_status samba_scan_step_groups(const samba_scan_step_groups_args* a, void* stream) {
  if (!a) return SAMBA_ERR_NULL_ARG;
  if (a->struct_size != sizeof(samba_scan_step_groups_args)) return SAMBA_ERR_BAD_STRUCT;
  if (a->batch < 0 || a->dim < 1 || a->ngroups < 1) return SAMBA_ERR_BAD_SHAPE;
  const int N = a->dstate;
  if (N != 16 && N != 32 && N != 64 && N != 128 && N != 256) return SAMBA_ERR_UNSUPPORTED;
  if (a->in_dtype != SAMBA_F32 && a->in_dtype != SAMBA_BF16) return SAMBA_ERR_BAD_DTYPE;
  if (a->y_dtype != SAMBA_F32 && a->y_dtype != SAMBA_BF16) return SAMBA_ERR_BAD_DTYPE;
  if (a->dim % a->ngroups != 0) return SAMBA_ERR_BAD_SHAPE;
  if (static_cast<int64_t>(a->batch) * a->dim * (N / 4) > (int64_t{1} << 38)) return SAMBA_ERR_BAD_SHAPE;
  if (a->batch == 0) return SAMBA_OK;
  if (!a->state || !a->x || !a->dt || !a->z || !a->B || !a->C || !a->A || !a->D || !a->dt_bias || !a->y)
    return SAMBA_ERR_NULL_ARG;
  const size_t ie = a->in_dtype == SAMBA_BF16 ? 2 : 4, oe = a->y_dtype == SAMBA_BF16 ? 2 : 4;
  if (!aligned(a->state, 16) || !aligned(a->A, 16) || !aligned(a->x, ie) || !aligned(a->dt, ie) ||
      !aligned(a->z, ie) || !aligned(a->B, ie) || !aligned(a->C, ie) || !aligned(a->y, oe) || !aligned(a->D, 4) ||
      !aligned(a->dt_bias, 4))
    return SAMBA_ERR_MISALIGNED;
  const size_t bd = static_cast<size_t>(a->batch) * a->dim;
  const size_t bc = static_cast<size_t>(a->batch) * a->ngroups * N;
  const size_t st = bd * N * 4;
  const void* ins[8] = {a->x, a->dt, a->z, a->B, a->C, a->A, a->D, a->dt_bias};
  const size_t in_sz[8] = {bd * ie, bd * ie, bd * ie, bc * ie, bc * ie, static_cast<size_t>(a->dim) * N * 4,
                           static_cast<size_t>(a->dim) * 4, static_cast<size_t>(a->dim) * 4};
  for (int k = 0; k < 8; ++k)
    if (overlap(a->state, st, ins[k], in_sz[k]) || overlap(a->y, bd * oe, ins[k], in_sz[k])) return SAMBA_ERR_ALIASING;
  if (overlap(a->y, bd * oe, a->state, st)) return SAMBA_ERR_ALIASING;
  SParams p{};
  p.state = a->state;
  p.x = a->x; p.dt = a->dt; p.z = a->z; p.B = a->B; p.C = a->C;
  p.A = a->A; p.Dskip = a->D; p.bias = a->dt_bias; p.y = a->y;
  p.batch = a->batch; p.dim = a->dim; p.ngroups = a->ngroups;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (a->in_dtype == SAMBA_BF16)
    e = a->y_dtype == SAMBA_BF16 ? launch_step_groups<uint16_t, uint16_t>(p, N, s)
                                 : launch_step_groups<uint16_t, float>(p, N, s);
  else
    e = a->y_dtype == SAMBA_BF16 ? launch_step_groups<float, uint16_t>(p, N, s)
                                 : launch_step_groups<float, float>(p, N, s);
  return e == hipSuccess ? SAMBA_OK : SAMBA_ERR_HIP;
}
