// samba_scan.hip -- gfx950 (MI355X) kernels and the C ABI of the selective scan.
//
// Operation: page "SAMBA混合注意力状态空间模型" (metaphor-xennon.pages.dev),
// section 数学框架 -> Mamba层: h_t = Ā_t h_{t-1} + B̄_t x_t, y_t = C_t h_t with
// B_t, C_t, Δ_t chosen from the input.  Ā = exp(ΔA), B̄x = ΔBx, Δ = softplus(dt +
// bias), y = (C.h + D x) silu(z) is the Mamba reading this library adopts (the
// pages leave those maps undefined).  State size 16 (same page, 实现细节 ->
// 模型配置).  Prefill is the page's forward(prompt); the decode step is its
// per-token constant-time state update (section 推理效率).
//
// Work decomposition (both kernels): a channel's 16 states are split over a
// quad of 4 lanes (4 states per lane), so a wave covers 16 channels.  B_t and
// C_t are shared by all channels; they are staged once per wave into LDS as
// fp32, so the per-lane work is only the recurrence itself.  The per-token
// scalar work of a channel (softplus, skip, gate, conversions, load and store)
// is spread over the quad: lane g of a quad owns tokens t with t % 4 == g of
// each group of four, and shares Δ and Δx with its quad through LDS.  The four
// lanes' partial readouts are summed with a transposed quad reduction in
// registers (DPP quad permutes) so that each lane ends with the finished y of
// its own token.
//
// Prefill parallelism: (sequence x 16-channel tile) workgroups; when that is
// too few to fill 256 CUs, W waves of a workgroup split each time chunk of
// W*8 tokens into W slices of 8 tokens.  Each wave runs its slice from a zero state,
// keeping every Ā and B̄x it computed in registers and publishing the slice's
// (product of Ā, local end state) pair through LDS; after one barrier each
// wave folds its predecessors' pairs into its carry-in and replays the slice
// from the registers (two FMAs per state and token, no second exp).  The
// carry-ins come from up to four fold waves between two barriers; the chunk
// carry stays in the fold threads' registers.  With very few (sequence, tile)
// pairs a variant with 8 lanes per channel (8-channel tiles) doubles the
// workgroups.  No state crosses workgroups, so no workspace and no
// inter-workgroup synchronisation is needed.
#include <hip/hip_runtime.h>

#include <stdint.h>
#include <string.h>

#include <atomic>
#include <type_traits>

#include "samba_scan.h"

#include "samba_scan_fwd.h"

namespace {

// Prefill and backward kernels address a lane's elements inside a slice (up to 16 token rows of x, dt, z, y,
// and a channel's 16-state checkpoint row) with 32-bit byte offsets of at most 64 * dim; this bound keeps
// them below 2^30.
constexpr int32_t kMaxDim = 1 << 24;
#ifndef SAMBA_STEP_QPT
#define SAMBA_STEP_QPT 4
#endif
constexpr int kStepQPT = SAMBA_STEP_QPT;  // quads per thread of the decode step on large batches

// ---------------------------------------------------------------------------
// Prefill, time-sliced, eight lanes per channel.  Lane (c, g) of a wave owns
// states 2g and 2g+1 of channel c, so a wave covers 8 channels and the
// workgroup an 8-channel tile; each wave's slice is 16 tokens, which keeps the
// same 2 x 16 x 2 replay registers per lane as the quad variant's 8 tokens x
// 4 states.  Halving the channels per workgroup doubles the workgroups: with
// one or few sequences that fills twice the CUs, or puts two independent
// workgroups on each CU, so one workgroup's barriers and LDS round trips are
// covered by the other's work.  Per lane the scalar work is the same two
// tokens per slice (g and g + 8).  No checkpoint variant.
// ---------------------------------------------------------------------------
constexpr int kCPW8 = 8;      // channels per wave (and per tile)
constexpr int kK8 = 16;       // tokens per slice
constexpr int kDuRow8 = kK8 / 2 + 1;  // float4 per channel row of the (Δ, Δx) pairs: 8 used + 1 (bank spread)

template <typename Tin>
struct RawSlice8 {
  static constexpr int kWords = static_cast<int>(sizeof(Tin));  // 4 B (and 4 C) values per lane, as words
  Tin x[2], dt[2], z[2];
  uint32_t bw[kWords], cw[kWords];
};

// Sum over the 8 lanes of each octet (two quad exchanges, then each half-row's mirror image)
__device__ __forceinline__ float octet_allsum(float v) {
  v += qperm<kQXor1>(v);
  v += qperm<kQXor2>(v);
  v += __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xF, 0xF, true));  // row_half_mirror
  return v;
}

template <typename Tin>
__device__ __forceinline__ void widen4(const uint32_t (&w)[RawSlice8<Tin>::kWords], float4& v) {
  if constexpr (sizeof(Tin) == 2) {
    v = make_float4(bf_lo(w[0]), bf_hi(w[0]), bf_lo(w[1]), bf_hi(w[1]));
  } else {
    v = make_float4(__uint_as_float(w[0]), __uint_as_float(w[1]), __uint_as_float(w[2]), __uint_as_float(w[3]));
  }
}

template <typename Tin, typename Tout, int W>
__global__ __launch_bounds__(64 * W, 4) void scan_split8_kernel(FwdParams p) {   // (<= 128 VGPRs)
  static_assert(W >= 2 && W <= 16, "time slices");
  constexpr int K = kK8;
  __shared__ float4 s_bc[W][2][K * kN / 4];        // B, C rows [K][16] of each wave's slice (fp32)
  __shared__ float4 s_du[W][kCPW8][kDuRow8];       // (Δ, Δx) of each channel's K tokens, two tokens per float4
  __shared__ float2 s_agg[W][2][64];               // slice (P, H) pairs of the current chunk
  __shared__ float2 s_cin[W][64];                  // each slice's carry-in, from the fold waves

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int logical = xcd_remap(blockIdx.x, p.nblocks);
  const int s = logical / p.ngroups;
  const int tile = logical - s * p.ngroups;
  const int lane = threadIdx.x & 63, g = lane & 7, c = lane >> 3;
  const int d = tile * kCPW8 + c;
  const bool dvalid = d < p.dim;
  const int dc = dvalid ? d : p.dim - 1;
  int64_t start, end;
  if (p.cu) {
    int64_t a = p.cu[s], b = p.cu[s + 1];
    a = a < 0 ? 0 : (a > p.total_tokens ? p.total_tokens : a);
    b = b < a ? a : (b > p.total_tokens ? p.total_tokens : b);
    start = a;
    end = b;
  } else {
    start = static_cast<int64_t>(s) * p.seqlen;
    end = start + p.seqlen;
  }
  float A2[2];
  {
    const float2 a2 = reinterpret_cast<const float2*>(p.A + static_cast<int64_t>(dc) * kN)[g];
    A2[0] = a2.x * kLog2e;
    A2[1] = a2.y * kLog2e;
  }
  const float dsk = p.Dskip[dc], bias = p.bias[dc];
  const uint32_t dim = static_cast<uint32_t>(p.dim);
  uint32_t in_off[2], out_off[2];  // byte offsets of tokens g and g + 8 of this lane's channel from a slice's first row
  {
    const uint32_t e0 = static_cast<uint32_t>(g) * dim + static_cast<uint32_t>(d);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      in_off[j] = (e0 + static_cast<uint32_t>(j) * 8u * dim) * static_cast<uint32_t>(sizeof(Tin));
      out_off[j] = (e0 + static_cast<uint32_t>(j) * 8u * dim) * static_cast<uint32_t>(sizeof(Tout));
    }
  }
  const uint32_t bc_off = static_cast<uint32_t>(lane) * 4u * static_cast<uint32_t>(sizeof(Tin));  // 4 of the slice's K x 16 values
  Tout* const yout = static_cast<Tout*>(p.y);

  const int ntok = static_cast<int>(end - start);   // 32-bit loop bookkeeping (a sequence is < 2^31 tokens)
  constexpr int chunk = W * K;
  const int nchunks = (ntok + chunk - 1) / chunk;
  const int my0 = wave * K;

  // Carry fold: the chunk's 64 lanes x 2 states = 128 chains, one per thread of the first two waves
  // (chain k is float k of a [64 lanes][2 states] row); the chunk carry stays in that thread's register.
  const bool folder = wave < 2;
  auto chain_off = [&]() -> int64_t {
    const int k = wave * 64 + lane;
    const int cl = k >> 1;
    const int dch = tile * kCPW8 + (cl >> 3);
    return (folder && dch < p.dim) ? (static_cast<int64_t>(s) * p.dim + dch) * kN + 2 * (cl & 7) + (k & 1) : -1;
  };
  float carry;
  {
    const int64_t off = chain_off();
    carry = (off >= 0 && p.h0) ? p.h0[off] : 0.f;
  }

  auto load8 = [&](int64_t t0, int rem, RawSlice8<Tin>& r) {
    const int64_t row0 = t0 * p.dim;
    const rsrc_t rx = make_rsrc_rows(static_cast<const Tin*>(p.x) + row0, rem, dim);
    const rsrc_t rd = make_rsrc_rows(static_cast<const Tin*>(p.dt) + row0, rem, dim);
    const rsrc_t rz = make_rsrc_rows(static_cast<const Tin*>(p.z) + row0, rem, dim);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bload(rx, in_off[j], r.x[j]);
      bload(rd, in_off[j], r.dt[j]);
      bload(rz, in_off[j], r.z[j]);
    }
    const rsrc_t rb = make_rsrc_rows(static_cast<const Tin*>(p.B) + t0 * kN, rem, kN);
    const rsrc_t rc = make_rsrc_rows(static_cast<const Tin*>(p.C) + t0 * kN, rem, kN);
    bload_words(rb, bc_off, r.bw);
    bload_words(rc, bc_off, r.cw);
  };

  const float2* sB2 = reinterpret_cast<const float2*>(s_bc[wave][0]);
  const float2* sC2 = reinterpret_cast<const float2*>(s_bc[wave][1]);

  auto chunk_step = [&](int ci, const RawSlice8<Tin>& cur, RawSlice8<Tin>& nxt) {
    const int i0 = my0 + ci * chunk;
    const int64_t t0 = start + i0;
    const int nv = ntok - i0 <= 0 ? 0 : (ntok - i0 < K ? ntok - i0 : K);
    load8(t0 + chunk, ntok - i0 - chunk, nxt);   // this wave's slice of the next chunk
    {
      float4 v;
      widen4<Tin>(cur.bw, v);
      s_bc[wave][0][lane] = v;
      widen4<Tin>(cur.cw, v);
      s_bc[wave][1][lane] = v;
    }
    float xv[2], zv[2], dl[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const bool ok = dvalid && (g + 8 * j) < nv;
      xv[j] = widen(cur.x[j]);
      zv[j] = widen(cur.z[j]);
      const float delta = softplus_f32(widen(cur.dt[j]) + bias);
      dl[j] = ok ? delta : 0.0f;
      reinterpret_cast<float2*>(s_du[wave][c])[g + 8 * j] = make_float2(dl[j], ok ? delta * xv[j] : 0.0f);
    }
    wave_lds_sync();

    // phase 1: local scan of the slice from zero; keep Ā and B̄x in registers
    float ak[K][2], bk[K][2];
    float H[2];
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 4) {
      const float4 du01 = s_du[wave][c][k0 / 2], du23 = s_du[wave][c][k0 / 2 + 1];
      const float dq[4] = {du01.x, du01.z, du23.x, du23.z};
      const float uq[4] = {du01.y, du01.w, du23.y, du23.w};
      float2 bq[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) bq[r] = sB2[(k0 + r) * 8 + g];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int k = k0 + r;
        ak[k][0] = __builtin_amdgcn_exp2f(dq[r] * A2[0]);
        ak[k][1] = __builtin_amdgcn_exp2f(dq[r] * A2[1]);
        bk[k][0] = uq[r] * bq[r].x;
        bk[k][1] = uq[r] * bq[r].y;
#pragma unroll
        for (int i = 0; i < 2; ++i) H[i] = (k == 0) ? bk[0][i] : fmaf(ak[k][i], H[i], bk[k][i]);
      }
    }
    // product of the slice's Ā = exp(A * sum of the slice's Δ)
    const float sd = octet_allsum(dl[0] + dl[1]);
    s_agg[wave][0][lane] = make_float2(__builtin_amdgcn_exp2f(A2[0] * sd), __builtin_amdgcn_exp2f(A2[1] * sd));
    s_agg[wave][1][lane] = make_float2(H[0], H[1]);
    __syncthreads();

    // fold: every slice's carry-in (all four slices of a group read first, then one FMA per slice)
    if (folder) {
      const float* aggf = reinterpret_cast<const float*>(s_agg);
      float* cinf = reinterpret_cast<float*>(s_cin);
      const int k = wave * 64 + lane;
      float cc = carry;
#pragma unroll
      for (int g0 = 0; g0 < W; g0 += 4) {
        constexpr int G = W < 4 ? W : 4;
        float Pv[G], Hv[G];
#pragma unroll
        for (int u = 0; u < G; ++u) {
          Pv[u] = aggf[((g0 + u) * 2 + 0) * 128 + k];
          Hv[u] = aggf[((g0 + u) * 2 + 1) * 128 + k];
        }
#pragma unroll
        for (int u = 0; u < G; ++u) {
          cinf[(g0 + u) * 128 + k] = cc;
          cc = fmaf(Pv[u], cc, Hv[u]);
        }
      }
      carry = cc;
    }
    __syncthreads();

    // phase 3: replay the slice from its carry-in, read out, gate, store
    float h[2];
    {
      const float2 cr = s_cin[wave][lane];
      h[0] = cr.x;
      h[1] = cr.y;
    }
    const rsrc_t ry = make_rsrc_rows(yout + t0 * p.dim, ntok - i0, dim);
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      float pr[8];
      float2 cq[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) cq[q] = sC2[(8 * jj + q) * 8 + g];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int k = 8 * jj + q;
#pragma unroll
        for (int i = 0; i < 2; ++i) h[i] = fmaf(ak[k][i], h[i], bk[k][i]);
        pr[q] = fmaf(cq[q].y, h[1], cq[q].x * h[0]);
      }
      // transposed sum over the octet (a half row) by a reduce-scatter on DPP: lane g keeps the tokens
      // whose index matches it in bit 2, then bit 1, then bit 0, adding its partner's share each time (the
      // partner 7 - g across the half row, then g ^ 2, then g ^ 1); lane g ends with token g's sum
      const bool b2 = (g & 4) != 0, b1 = (g & 2) != 0, b0 = (g & 1) != 0;
      float s4[4], s2[2];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float keep = b2 ? pr[k + 4] : pr[k], send = b2 ? pr[k] : pr[k + 4];
        s4[k] = keep + qperm<0x141>(send);   // row_half_mirror
      }
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const float keep = b1 ? s4[k + 2] : s4[k], send = b1 ? s4[k] : s4[k + 2];
        s2[k] = keep + qperm<kQXor2>(send);
      }
      const float yraw = (b0 ? s2[1] : s2[0]) + qperm<kQXor1>(b0 ? s2[0] : s2[1]);
      if (g + 8 * jj < nv) {
        const float yv = (yraw + dsk * xv[jj]) * silu_f32(zv[jj]);
        if (dvalid) bstore(ry, out_off[jj], yv, static_cast<Tout*>(nullptr));
      }
    }
    wave_lds_sync();
  };

  RawSlice8<Tin> ra, rb;
  load8(start + my0, ntok - my0, ra);
  for (int ci = 0; ci < nchunks; ci += 2) {
    chunk_step(ci, ra, rb);
    if (ci + 1 < nchunks) chunk_step(ci + 1, rb, ra);
  }
  // the state leaving the sequence is the fold's carry after the last chunk
  if (p.h_last) {
    const int64_t off = chain_off();
    if (off >= 0) p.h_last[off] = carry;
  }
}

// ---------------------------------------------------------------------------
// Backward (gradients of the prefill).  Per sequence and channel the adjoint
// g_t = dr_t C_t + Ā_{t+1} g_{t+1} runs from the last token to the first, and
// every gradient term of token t needs g_t together with the forward states
// h_{t-1}, h_t.  Decomposition (same lanes as the forward: a quad of lanes per
// channel, 4 states per lane, 16 channels per wave):
//   * the forward states are recomputed from checkpoints (the state before
//     every 8th token, written by the forward kernel's checkpoint variant);
//   * a workgroup owns one (sequence, 16-channel tile); its W waves split each
//     time chunk of 8W tokens into slices of 8, and chunks run from the end of
//     the sequence to its start;
//   * each wave recomputes its slice forward from its checkpoint, keeping Ā_t
//     and h_t in registers, and in the same sweep forms the slice's adjoint
//     transfer pair (P = product of Ā, Ĝ = sum_t (prod_{r<=t} Ā_r) dr_t C_t):
//     Ĝ is the adjoint leaving the slice's start when none enters its end;
//   * after one barrier each wave folds the later slices' pairs into the
//     adjoint entering the chunk, then runs the reverse sweep, where every
//     gradient term is formed; the leftmost wave's result is the adjoint
//     entering the previous chunk (LDS, double buffered);
//   * dB_t and dC_t are sums over all channels: each wave sums its 16 channels
//     through LDS and writes one partial row per token and tile; dA, dD and
//     ddt_bias are summed over the sequence in registers and written per
//     sequence; a final kernel adds the partials in a fixed order (no atomics,
//     bitwise reproducible).
// ---------------------------------------------------------------------------
constexpr int kBK = 8;      // tokens per backward slice = checkpoint interval
constexpr int kParW = 20;   // per-sequence partial row: dA[16], dD, ddt_bias, 2 pad (16-byte rows)

struct BwdParams {
  const void *x, *dt, *z, *B, *C, *dy;
  const float *A, *Dskip, *bias;
  const float* dh_last;
  const float* ckpt;      // [slots][dim][16]
  void *dx, *ddt, *dz;
  float* dbc;             // [ntiles][total_tokens][32]: per-tile dB (0..15) and dC (16..31)
  float* dpar;            // [nseq][dim][kParW]
  float* dh0;
  const int32_t* cu;
  int64_t total_tokens;
  int32_t seqlen, dim, ntiles, nblocks;
};

template <typename T, int W>
__global__ __launch_bounds__(64 * W, 3) void scan_bwd_kernel(BwdParams p) {   // (3 waves per SIMD: <= 168 VGPRs)
  constexpr int K = kBK;
  // LDS, per wave (7.1 KiB) plus 2 KiB per workgroup: 30.5 KiB for 4 waves.
  __shared__ float4 s_bc[W][2][K * kN / 4];   // B, C rows of the slice (fp32)
  __shared__ float4 s_sc[W][K][kCPW + 1];     // per token and channel: (Δ, Δx, dr, 0), masked (rows padded:
                                              // the four tokens of a lane quad land on different banks)
  __shared__ float4 s_tok[W][K / 4][64];      // this lane's tokens: (x, dy, sigmoid(v), silu'(z))
  __shared__ float4 s_agg[W][2][64];          // slice (P, Ĝ); after the last chunk: per-wave parameter sums
  __shared__ float4 s_carry[2][64];           // adjoint entering a chunk from the right, double buffered

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int logical = xcd_remap(blockIdx.x, p.nblocks);
  const int s = logical / p.ntiles;
  const int tile = logical - s * p.ntiles;
  const int lane = threadIdx.x & 63, g = lane & 3, c = lane >> 2;
  const int d = tile * kCPW + c;
  const bool dvalid = d < p.dim;
  const int dc = dvalid ? d : p.dim - 1;
  int64_t start, end;
  if (p.cu) {
    int64_t a = p.cu[s], b = p.cu[s + 1];
    a = a < 0 ? 0 : (a > p.total_tokens ? p.total_tokens : a);
    b = b < a ? a : (b > p.total_tokens ? p.total_tokens : b);
    start = a;
    end = b;
  } else {
    start = static_cast<int64_t>(s) * p.seqlen;
    end = start + p.seqlen;
  }
  const int ntok = static_cast<int>(end - start);
  float A2[kSPL];   // A * log2(e); the dΔ sum is taken against A2 and rescaled by ln 2 per token
  {
    const float4 a4 = reinterpret_cast<const float4*>(p.A + static_cast<int64_t>(dc) * kN)[g];
    A2[0] = a4.x * kLog2e; A2[1] = a4.y * kLog2e; A2[2] = a4.z * kLog2e; A2[3] = a4.w * kLog2e;
  }
  const float dsk = p.Dskip[dc], bias = p.bias[dc];
  const uint32_t dim = static_cast<uint32_t>(p.dim);
  uint32_t in_off[K / 4];
#pragma unroll
  for (int j = 0; j < K / 4; ++j)
    in_off[j] = ((static_cast<uint32_t>(4 * j + g)) * dim + static_cast<uint32_t>(d)) * static_cast<uint32_t>(sizeof(T));
  const int bc_lds = (lane >> 3) * kN + (lane & 7) * 2;   // 2 of the 8 x 16 B (and C) values per lane
  const uint32_t bc_off = static_cast<uint32_t>(bc_lds) * static_cast<uint32_t>(sizeof(T));
  const uint32_t ck_off = (static_cast<uint32_t>(dc) * kN + 4u * static_cast<uint32_t>(g)) * 4u;
  float* sB = reinterpret_cast<float*>(s_bc[wave][0]);
  float* sC = reinterpret_cast<float*>(s_bc[wave][1]);
  const float4* sB4 = s_bc[wave][0];
  const float4* sC4 = s_bc[wave][1];

  // adjoint entering the sequence's last token from the right: dh_last
  float gh[kSPL] = {0.f, 0.f, 0.f, 0.f};
  if (p.dh_last) {
    const float4 v = reinterpret_cast<const float4*>(p.dh_last + (static_cast<int64_t>(s) * p.dim + dc) * kN)[g];
    gh[0] = v.x; gh[1] = v.y; gh[2] = v.z; gh[3] = v.w;
  }
  if (wave == 0) s_carry[1][lane] = make_float4(gh[0], gh[1], gh[2], gh[3]);

  constexpr int chunk = W * K;
  const int nchunks = (ntok + chunk - 1) / chunk;
  float dAacc[kSPL] = {0.f, 0.f, 0.f, 0.f};
  float dDacc = 0.f, dbacc = 0.f;

  // ---- loads of one slice: this lane's tokens of x, dt, z, dy; the slice's B, C; the checkpoint.  They are
  // issued one chunk ahead (the loop's iteration `it` loads iteration it + 1's slice), so that their latency
  // hides behind a whole chunk of work.  Past the first chunk of the sequence (it >= nchunks) every resource
  // is empty and based at the tensor's start: the loads read 0 and touch no memory.
  struct BwdRaw {
    T xr[K / 4], dtr[K / 4], zr[K / 4], dyr[K / 4];
    uint32_t bw[RawSlice<T, K>::kWords], cw[RawSlice<T, K>::kWords];
    uint32_t hk[kSPL];
  };
  auto load_slice = [&](int it_l, BwdRaw& r) {
    const bool live = it_l < nchunks;
    const int i0l = (nchunks - 1 - it_l) * chunk + wave * K;
    const int reml = live ? ntok - i0l : 0;
    const int64_t t0l = live ? start + i0l : 0;
    const int64_t row0l = t0l * p.dim;
    const rsrc_t rx = make_rsrc_rows(static_cast<const T*>(p.x) + row0l, reml, dim);
    const rsrc_t rd = make_rsrc_rows(static_cast<const T*>(p.dt) + row0l, reml, dim);
    const rsrc_t rz = make_rsrc_rows(static_cast<const T*>(p.z) + row0l, reml, dim);
    const rsrc_t ry = make_rsrc_rows(static_cast<const T*>(p.dy) + row0l, reml, dim);
#pragma unroll
    for (int j = 0; j < K / 4; ++j) {
      bload(rx, in_off[j], r.xr[j]);
      bload(rd, in_off[j], r.dtr[j]);
      bload(rz, in_off[j], r.zr[j]);
      bload(ry, in_off[j], r.dyr[j]);
    }
    const rsrc_t rb = make_rsrc_rows(static_cast<const T*>(p.B) + t0l * kN, reml, kN);
    const rsrc_t rc = make_rsrc_rows(static_cast<const T*>(p.C) + t0l * kN, reml, kN);
    bload_words(rb, bc_off, r.bw);
    bload_words(rc, bc_off, r.cw);
    // checkpoint row of this slice (an empty resource past the sequence end: reads give 0)
    const rsrc_t rk = make_rsrc_rows(live ? p.ckpt + ckpt_slot(start, s, i0l >> 3) * p.dim * kN : p.ckpt,
                                     reml > 0 ? 1 : 0, dim * kN);
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(rk, ck_off, 0, 0);
    r.hk[0] = v[0]; r.hk[1] = v[1]; r.hk[2] = v[2]; r.hk[3] = v[3];
  };
  // one chunk of the sweep; `cur` holds its loaded slice, and it loads the next chunk's slice into `nxt` (the
  // loop runs the body twice per step with the two register sets swapped, so no copy waits for the loads)
  auto chunk_body = [&](int it, const BwdRaw& cur, BwdRaw& nxt) {
    const int ci = nchunks - 1 - it;
    const int buf = it & 1;
    const int i0 = ci * chunk + wave * K;
    const int rem = ntok - i0;
    const int nv = rem <= 0 ? 0 : (rem < K ? rem : K);
    const int64_t t0 = start + i0;
    const int64_t row0 = t0 * p.dim;

    load_slice(it + 1, nxt);
    const T(&xr)[K / 4] = cur.xr;
    const T(&dtr)[K / 4] = cur.dtr;
    const T(&zr)[K / 4] = cur.zr;
    const T(&dyr)[K / 4] = cur.dyr;
    const uint32_t(&bw)[RawSlice<T, K>::kWords] = cur.bw;
    const uint32_t(&cw)[RawSlice<T, K>::kWords] = cur.cw;
    float hs[kSPL] = {__uint_as_float(cur.hk[0]), __uint_as_float(cur.hk[1]), __uint_as_float(cur.hk[2]),
                      __uint_as_float(cur.hk[3])};
    {
      float v[K / 4];
      widen_words<T, K>(bw, v);
      lds_put<K / 4>(sB + bc_lds, v);
      widen_words<T, K>(cw, v);
      lds_put<K / 4>(sC + bc_lds, v);
    }
    // ---- per-token scalars of this lane's tokens (4j + g), parked in LDS until the outputs
#pragma unroll
    for (int j = 0; j < K / 4; ++j) {
      const bool ok = dvalid && (4 * j + g) < nv;
      const float xv = widen(xr[j]), zv = widen(zr[j]), dyv = widen(dyr[j]);
      const float v = widen(dtr[j]) + bias;
      const float delta = softplus_f32(v);
      const float sz = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-zv * kLog2e));
      const float sigv = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-v * kLog2e));
      s_tok[wave][j][lane] = make_float4(xv, dyv, sigv, sz * fmaf(zv, 1.0f - sz, 1.0f));
      s_sc[wave][4 * j + g][c] = make_float4(ok ? delta : 0.0f, ok ? delta * xv : 0.0f, ok ? dyv * zv * sz : 0.0f, 0.0f);
    }
    wave_lds_sync();

    // ---- forward recompute of the slice; adjoint transfer pair (P, Ĝ).  Ā_t and h_t of the
    // second half of the slice stay in registers; the first half is recomputed (same operations,
    // same order, so bit for bit the same values) after the second half's reverse sweep: half the
    // replay registers, so four waves fit a SIMD.
    constexpr int H = K / 2;
    float ak[H][kSPL], hk[H][kSPL];   // tokens H..K-1 during the first reverse half, 0..H-1 after
    float hmid[kSPL];                 // state after token H-1
    float P[kSPL], G[kSPL];
    float rr[K / 4];
    auto fwd_token = [&](int k, const float (&prev)[kSPL], float (&a)[kSPL], float (&h)[kSPL], float4& cv_out) {
      const float4 sc = s_sc[wave][k][c];
      const float4 bv = sB4[k * 4 + g];
      cv_out = sC4[k * 4 + g];
      const float bb[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
      for (int i = 0; i < kSPL; ++i) {
        a[i] = __builtin_amdgcn_exp2f(sc.x * A2[i]);
        h[i] = fmaf(a[i], prev[i], sc.y * bb[i]);
      }
      return sc;
    };
    {
      float hcur[kSPL] = {hs[0], hs[1], hs[2], hs[3]};
#pragma unroll
      for (int jj = 0; jj < K / 4; ++jj) {
        float pr[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int k = 4 * jj + q;
          float a[kSPL], h[kSPL];
          float4 cv;
          const float4 sc = fwd_token(k, hcur, a, h, cv);
          const float cc[4] = {cv.x, cv.y, cv.z, cv.w};
          float acc = 0.f;
#pragma unroll
          for (int i = 0; i < kSPL; ++i) {
            P[i] = (k == 0) ? a[i] : P[i] * a[i];
            const float drc = sc.z * cc[i];
            G[i] = (k == 0) ? P[i] * drc : fmaf(P[i], drc, G[i]);
            acc = fmaf(cc[i], h[i], acc);
            hcur[i] = h[i];
            if (k >= H) { ak[k - H][i] = a[i]; hk[k - H][i] = h[i]; }
            if (k == H - 1) hmid[i] = h[i];
          }
          pr[q] = acc;
        }
        rr[jj] = quad_transpose_sum(pr[0], pr[1], pr[2], pr[3], g);
      }
    }
    __syncthreads();  // every wave has finished reading the previous chunk's pairs
    s_agg[wave][0][lane] = make_float4(P[0], P[1], P[2], P[3]);
    s_agg[wave][1][lane] = make_float4(G[0], G[1], G[2], G[3]);
    __syncthreads();

    // ---- adjoint entering this slice's end: fold the later slices into the chunk's incoming adjoint
    {
      const float4 v = s_carry[buf ^ 1][lane];
      gh[0] = v.x; gh[1] = v.y; gh[2] = v.z; gh[3] = v.w;
    }
    for (int w2 = W - 1; w2 > wave; --w2) {
      const float4 P2 = s_agg[w2][0][lane];
      const float4 G2 = s_agg[w2][1][lane];
      gh[0] = fmaf(P2.x, gh[0], G2.x);
      gh[1] = fmaf(P2.y, gh[1], G2.y);
      gh[2] = fmaf(P2.z, gh[2], G2.z);
      gh[3] = fmaf(P2.w, gh[3], G2.w);
    }

    // ---- reverse sweep: every gradient term
    const int prow = rem < 0 ? 0 : rem;
    const rsrc_t rbc = make_rsrc_rows(p.dbc + (static_cast<int64_t>(tile) * p.total_tokens + t0) * 32, prow, 32u);
    // after the channel reduction below, lanes with channel bits 2..3 clear write outputs 16 (lane bit 5) +
    // 4 g + 2 (lane bit 4) + 0..1 of the token's row (kind dB / dC, then the state)
    const bool dbc_writer = (lane & 12) == 0;
    const uint32_t dbc_off = static_cast<uint32_t>(16 * (lane >> 5) + 4 * g + 2 * ((lane >> 4) & 1)) * 4u;
    float sau_t[K / 4], sgb_t[K / 4];
    // one token k of the reverse sweep, with Ā_k, h_{k-1} and h_k; returns its (Σ g A2 Ā h_{k-1}, Σ g B) partials
    auto rev_token = [&](int k, const float (&a)[kSPL], const float (&hprev)[kSPL], const float (&hc)[kSPL],
                         float& sa, float& sb) {
      const float4 sc = s_sc[wave][k][c];
      const float4 bv = sB4[k * 4 + g], cv = sC4[k * 4 + g];
      const float bb[4] = {bv.x, bv.y, bv.z, bv.w};
      const float cc[4] = {cv.x, cv.y, cv.z, cv.w};
      float db[4], dcv[4];
      sa = 0.f;
      sb = 0.f;
#pragma unroll
      for (int i = 0; i < kSPL; ++i) {
        const float gi = fmaf(sc.z, cc[i], gh[i]);
        const float gu = gi * (a[i] * hprev[i]);
        dAacc[i] = fmaf(gu, sc.x, dAacc[i]);
        sa = fmaf(gu, A2[i], sa);
        sb = fmaf(gi, bb[i], sb);
        db[i] = gi * sc.y;
        dcv[i] = sc.z * hc[i];
        gh[i] = a[i] * gi;
      }
      // this token's dB / dC summed over the wave's 16 channels (lane bits 2..5), in registers: a
      // reduce-scatter over bit 5 (the lower half keeps dB, the upper dC) and bit 4 (states 0, 1 of the
      // lane's four, or 2, 3), then rotations within each row of 16 lanes add over bits 2 and 3
      float u[4], w[2];
#pragma unroll
      for (int i = 0; i < 4; ++i) u[i] = swap32_sum(db[i], dcv[i]);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        w[i] = swap16_sum(u[i], u[i + 2]);
        w[i] += row_ror<4>(w[i]);
        w[i] += row_ror<8>(w[i]);
      }
      if (dbc_writer) {
        const u32x2_t wv = {__float_as_uint(w[0]), __float_as_uint(w[1])};
        __builtin_amdgcn_raw_buffer_store_b64(wv, rbc, static_cast<uint32_t>(k * 32 * 4) + dbc_off, 0, 0);
      }
    };
    static_assert(H == 4, "one quad group per half");
    // second half (tokens K-1 .. H) from the registers
    {
      float sau[4], sgb[4];
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        const int k = H + q;
        float hp[kSPL];
#pragma unroll
        for (int i = 0; i < kSPL; ++i) hp[i] = (q == 0) ? hmid[i] : hk[q - 1][i];
        rev_token(k, ak[q], hp, hk[q], sau[q], sgb[q]);
      }
      sau_t[1] = quad_transpose_sum(sau[0], sau[1], sau[2], sau[3], g);
      sgb_t[1] = quad_transpose_sum(sgb[0], sgb[1], sgb[2], sgb[3], g);
    }
    // first half (tokens H-1 .. 0): recompute from the checkpoint, then reverse
    {
      float hcur[kSPL] = {hs[0], hs[1], hs[2], hs[3]};
#pragma unroll
      for (int k = 0; k < H; ++k) {
        float4 cv;
        fwd_token(k, hcur, ak[k], hk[k], cv);
#pragma unroll
        for (int i = 0; i < kSPL; ++i) hcur[i] = hk[k][i];
      }
      float sau[4], sgb[4];
#pragma unroll
      for (int q = 3; q >= 0; --q) {
        float hp[kSPL];
#pragma unroll
        for (int i = 0; i < kSPL; ++i) hp[i] = (q == 0) ? hs[i] : hk[q - 1][i];
        rev_token(q, ak[q], hp, hk[q], sau[q], sgb[q]);
      }
      sau_t[0] = quad_transpose_sum(sau[0], sau[1], sau[2], sau[3], g);
      sgb_t[0] = quad_transpose_sum(sgb[0], sgb[1], sgb[2], sgb[3], g);
    }

    // ---- per-token outputs of this lane's tokens
    {
      const rsrc_t ox = make_rsrc_rows(static_cast<T*>(p.dx) + row0, rem, dim);
      const rsrc_t od = make_rsrc_rows(static_cast<T*>(p.ddt) + row0, rem, dim);
      const rsrc_t oz = make_rsrc_rows(static_cast<T*>(p.dz) + row0, rem, dim);
#pragma unroll
      for (int j = 0; j < K / 4; ++j) {
        const bool ok = dvalid && (4 * j + g) < nv;
        const float4 tk = s_tok[wave][j][lane];           // x, dy, sigmoid(v), silu'(z)
        const float4 sc = s_sc[wave][4 * j + g][c];       // Δ, Δx, dr (masked)
        const float r = fmaf(dsk, tk.x, rr[j]);
        const float dzv = tk.y * r * tk.w;
        const float dxv = fmaf(sc.z, dsk, sc.x * sgb_t[j]);
        const float ddtv = fmaf(sgb_t[j], tk.x, sau_t[j] * kLn2) * tk.z;
        if (ok) {
          dDacc = fmaf(sc.z, tk.x, dDacc);
          dbacc += ddtv;
          bstore(ox, in_off[j], dxv, static_cast<T*>(nullptr));
          bstore(od, in_off[j], ddtv, static_cast<T*>(nullptr));
          bstore(oz, in_off[j], dzv, static_cast<T*>(nullptr));
        }
      }
    }
    if (wave == 0) s_carry[buf][lane] = make_float4(gh[0], gh[1], gh[2], gh[3]);
    wave_lds_sync();
    };
  BwdRaw ra, rb;
  load_slice(0, ra);
  for (int it = 0; it < nchunks; it += 2) {
    chunk_body(it, ra, rb);
    if (it + 1 < nchunks) chunk_body(it + 1, rb, ra);
  }

  // ---- end of the sequence: dh0 (wave 0 holds the adjoint leaving the first token), parameter partials
  if (wave == 0 && p.dh0 && dvalid)
    reinterpret_cast<float4*>(p.dh0 + (static_cast<int64_t>(s) * p.dim + d) * kN)[g] =
        make_float4(gh[0], gh[1], gh[2], gh[3]);
  dDacc = quad_allsum(dDacc);
  dbacc = quad_allsum(dbacc);
  __syncthreads();  // the last chunk's folds are done with s_agg
  s_agg[wave][0][lane] = make_float4(dAacc[0], dAacc[1], dAacc[2], dAacc[3]);
  s_agg[wave][1][lane] = make_float4(dDacc, dbacc, 0.f, 0.f);
  __syncthreads();
  if (wave == 0 && dvalid) {
    float4 a = s_agg[0][0][lane];
    float4 b = s_agg[0][1][lane];
#pragma unroll
    for (int w2 = 1; w2 < W; ++w2) {
      const float4 a2 = s_agg[w2][0][lane];
      const float4 b2 = s_agg[w2][1][lane];
      a.x += a2.x; a.y += a2.y; a.z += a2.z; a.w += a2.w;
      b.x += b2.x; b.y += b2.y;
    }
    float* row = p.dpar + (static_cast<int64_t>(s) * p.dim + d) * kParW;
    reinterpret_cast<float4*>(row)[g] = a;
    if (g == 0) { row[16] = b.x; row[17] = b.y; }
  }
}

// dB, dC: sum of the per-tile partial rows; dA, dD, ddt_bias: sum of the
// per-sequence partial rows.  One thread per output element, fixed order.
__global__ __launch_bounds__(256) void scan_bwd_finish_kernel(const float* dbc, const float* dpar, float* dB, float* dC,
                                                              float* dA, float* dD, float* dbias, int64_t total_tokens,
                                                              int32_t ntiles, int32_t nseq, int32_t dim) {
  const int64_t idx = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t n4 = total_tokens * 8;   // 4 consecutive outputs of one row per thread (16-byte loads)
  if (idx < n4) {
    const float4* src = reinterpret_cast<const float4*>(dbc) + idx;
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll 8
    for (int t = 0; t < ntiles; ++t) {   // (each output still sums its tiles in order 0, 1, ..)
      const float4 v = src[static_cast<int64_t>(t) * n4];
      acc.x += v.x; acc.y += v.y; acc.z += v.z; acc.w += v.w;
    }
    const int64_t row = idx >> 3;
    const int o = 4 * static_cast<int>(idx & 7);
    float4* dst = reinterpret_cast<float4*>((o < 16 ? dB : dC) + row * 16 + (o & 15));
    *dst = acc;
    return;
  }
  const int64_t i2 = idx - n4;
  if (i2 >= static_cast<int64_t>(dim) * 18) return;
  const int64_t dd = i2 / 18;
  const int q = static_cast<int>(i2 - dd * 18);
  float acc = 0.f;
  for (int s2 = 0; s2 < nseq; ++s2) acc += dpar[(static_cast<int64_t>(s2) * dim + dd) * kParW + q];
  if (q < 16) dA[dd * 16 + q] = acc;
  else if (q == 16) dD[dd] = acc;
  else dbias[dd] = acc;
}

// ---------------------------------------------------------------------------
// Decode step: one token per sequence; lane = (sequence, channel, state quarter).
// ---------------------------------------------------------------------------
struct StepParams {
  float* state;
  const void *x, *dt, *z, *B, *C;
  const float *A, *Dskip, *bias;
  void* y;
  int32_t batch;
  int32_t dim;
};

template <typename Tin>
__device__ __forceinline__ void load4(const Tin* p, int64_t i, float (&v)[4]);
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t* p, int64_t i, float (&v)[4]) {
  const uint2 w = *reinterpret_cast<const uint2*>(p + i);
  v[0] = bf_lo(w.x); v[1] = bf_hi(w.x); v[2] = bf_lo(w.y); v[3] = bf_hi(w.y);
}
template <>
__device__ __forceinline__ void load4<float>(const float* p, int64_t i, float (&v)[4]) {
  const float4 w = *reinterpret_cast<const float4*>(p + i);
  v[0] = w.x; v[1] = w.y; v[2] = w.z; v[3] = w.w;
}

// A workgroup of 256 threads = 64 channel quads covers channels
// [64*bx, 64*bx+64) for QPT consecutive sequences [QPT*by, QPT*by+QPT): each
// thread loads its channel's A, dt_bias and D once and reuses them for all its
// sequences; each round of a wave touches 1 KB of contiguous state.  All
// rounds' loads are issued before any compute.
template <typename Tin, typename Tout, int QPT>
__global__ __launch_bounds__(256) void scan_step_kernel(StepParams p) {
  const int g = threadIdx.x & 3;
  const int d = blockIdx.x * 64 + (threadIdx.x >> 2);
  const bool dvalid = d < p.dim;
  const int dc = dvalid ? d : p.dim - 1;
  const int64_t b0 = static_cast<int64_t>(blockIdx.y) * QPT;
  const float4 a4 = reinterpret_cast<const float4*>(p.A + static_cast<int64_t>(dc) * kN)[g];
  const float bias = p.bias[dc];
  const float dsk = p.Dskip[dc];
  float4 h4[QPT];
  float xv[QPT], dr[QPT], zv[QPT], Bv[QPT][4], Cv[QPT][4];
  int64_t qs[QPT];
  bool valid[QPT];
#pragma unroll
  for (int r = 0; r < QPT; ++r) {
    const int64_t b = b0 + r;
    valid[r] = dvalid && b < p.batch;
    const int64_t bc = b < p.batch ? b : p.batch - 1;
    qs[r] = bc * p.dim + dc;
    h4[r] = reinterpret_cast<const float4*>(p.state + qs[r] * kN)[g];
    // per-step inputs and y are touched once: non-temporal, so they do not
    // displace the state (which stays cache-resident from step to step)
    xv[r] = widen(__builtin_nontemporal_load(static_cast<const Tin*>(p.x) + qs[r]));
    dr[r] = widen(__builtin_nontemporal_load(static_cast<const Tin*>(p.dt) + qs[r]));
    zv[r] = widen(__builtin_nontemporal_load(static_cast<const Tin*>(p.z) + qs[r]));
    load4<Tin>(static_cast<const Tin*>(p.B), bc * kN + 4 * g, Bv[r]);
    load4<Tin>(static_cast<const Tin*>(p.C), bc * kN + 4 * g, Cv[r]);
  }
  const float A2[4] = {a4.x * kLog2e, a4.y * kLog2e, a4.z * kLog2e, a4.w * kLog2e};
#pragma unroll
  for (int r = 0; r < QPT; ++r) {
    const float delta = softplus_f32(dr[r] + bias);
    const float u = delta * xv[r];
    float h[4] = {h4[r].x, h4[r].y, h4[r].z, h4[r].w};
    float pr = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = fmaf(__builtin_amdgcn_exp2f(delta * A2[i]), h[i], u * Bv[r][i]);
      pr = fmaf(Cv[r][i], h[i], pr);
    }
    pr = quad_allsum(pr);
    if (valid[r]) {
      reinterpret_cast<float4*>(p.state + qs[r] * kN)[g] = make_float4(h[0], h[1], h[2], h[3]);
      if (g == 0) {
        const float yv = (pr + dsk * xv[r]) * silu_f32(zv[r]);
        if constexpr (sizeof(Tout) == 2) __builtin_nontemporal_store(f32_to_bf16(yv), static_cast<uint16_t*>(p.y) + qs[r]);
        else __builtin_nontemporal_store(yv, static_cast<float*>(p.y) + qs[r]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Selection projections: [dt_raw | B | C] = x W^T, one bf16 GEMM on the matrix
// cores (v_mfma_f32_32x32x16_bf16, fp32 accumulation).  x [T][dim] and W
// [dim + 2N][dim] are both K-contiguous.  A workgroup computes a 256 x 256
// output tile with WM x WN waves, each owning a block of 32 x 32 MFMA tiles.
// Operand tiles go from memory straight into LDS (buffer_load_dwordx4 ... lds:
// the 64 lanes of a wave fill 1 KiB of LDS, lane l at byte 16 l), so no VGPRs
// hold prefetched data; K advances BK per step through a ring of S stages.
// The LDS image of a 256 x BK operand tile is row-major with 2 BK bytes per
// row, its 16-byte chunks permuted per row (logical chunk c of row r sits at
// position c ^ swz(r)) so that fragment reads are free of bank conflicts.  The
// compiler does not track these LDS writes, so the waits are explicit: before
// step s each wave waits for its own loads of stage s (vmcnt), then a barrier
// publishes every wave's loads and frees the buffer that step s - 1 read,
// which the loads of stage s + S - 1 then refill.  Inside a step the fragments
// of the next 16-wide K slice are read while the MFMAs of this one run.
// Out-of-range rows, and chunks past the K tail, read as zero (the resource
// bounds, and an offset past them).  A wave whose output columns lie beyond
// the last one skips their MFMAs (the ragged last column tile).  bf16 results
// leave through LDS as 16-byte row chunks, fp32 results element-wise.  Tiles
// are ordered in groups of 8 row tiles so that workgroups running together on
// one XCD share their A and B tiles in L2.  Operand layouts (checked on the
// device): lane l holds A[l % 32][8 (l / 32) + 0..7] and B[8 (l / 32) +
// 0..7][l % 32]; result element e of lane l is D[8 (e / 4) + 4 (l / 32) + e %
// 4][l % 32].
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kPGroup = 8;          // row tiles per ordering group

struct ProjParams {
  const uint16_t* x;    // [T][dim]
  const uint16_t* W;    // [nout][dim]
  void *dt, *B, *C;
  int32_t T, dim, dstate, nout, mtiles, ntiles, nblocks;
  int32_t vec_dt, vec_bc;  // bf16 results may leave as 16-byte chunks (alignment, dstate % 8 == 0)
};

template <typename Tout>
__device__ __forceinline__ void proj_store(const ProjParams& p, int t, int j, float v) {
  if (t >= p.T || j >= p.nout) return;
  if (j < p.dim) st_out(static_cast<Tout*>(p.dt), static_cast<int64_t>(t) * p.dim + j, v);
  else if (j < p.dim + p.dstate) st_out(static_cast<Tout*>(p.B), static_cast<int64_t>(t) * p.dstate + (j - p.dim), v);
  else st_out(static_cast<Tout*>(p.C), static_cast<int64_t>(t) * p.dstate + (j - p.dim - p.dstate), v);
}

// Tile configuration (build-time): K step, ring stages, waves per tile (WM x WN).  Measured on
// 16384 x 4096 -> 4128: 64 / 2 / 2 x 4 at 0.48-0.51 ms, against 32 / 4 / 2 x 4 (0.53-0.56), 64 / 2 / 2 x 2
// (0.53-0.57) and 32 / 4 / 2 x 2 (0.55-0.59).
#ifndef SAMBA_PROJ_BK
#define SAMBA_PROJ_BK 64
#endif
#ifndef SAMBA_PROJ_STAGES
#define SAMBA_PROJ_STAGES 2
#endif
#ifndef SAMBA_PROJ_WM
#define SAMBA_PROJ_WM 2
#endif
#ifndef SAMBA_PROJ_WN
#define SAMBA_PROJ_WN 4
#endif
constexpr int kDBK = SAMBA_PROJ_BK, kDS = SAMBA_PROJ_STAGES, kDWM = SAMBA_PROJ_WM, kDWN = SAMBA_PROJ_WN;

// Chunk permutation of tile row r.  gfx950's LDS serves a 16-byte-per-lane read to 16 lanes per cycle
// over 64 banks (256 bytes), and the 16 lanes of a fragment read are 16 consecutive rows: with 128-byte
// rows, rows r and r + 8 must land in different 16-byte bank groups as well as rows r .. r + 7.
template <int BK>
__device__ __forceinline__ int proj_swz(int r) { return BK == 64 ? ((r & 7) ^ ((r >> 3) & 1)) : ((r >> 2) & 3); }

// s_waitcnt on the vector-memory counter only (gfx9 encoding: vmcnt in bits 3:0 and 15:14)
template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (15 << 8));
}

// one wave-wide 16-byte-per-lane load from a buffer resource straight into LDS at `lds` + 16 lane
__device__ __forceinline__ void dma16(rsrc_t r, void* lds, uint32_t voff, int soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
}

template <typename Tout, int BK, int S, int WM, int WN>
__global__ __launch_bounds__(64 * WM * WN) void proj_dma_kernel(ProjParams p) {
  constexpr int kW = WM * WN;
  constexpr int BM = 256, BN = 256;
  constexpr int RM = BM / WM, RN = BN / WN;   // a wave's output block
  constexpr int TM = RM / 32, TN = RN / 32;   // MFMA tiles per wave
  constexpr int kRowB = BK * 2;               // bytes per LDS tile row
  constexpr int kCh = BK / 8;                 // 16-byte chunks per row
  constexpr int kRPL = 64 / kCh;              // rows filled by one wave load
  constexpr int kTileB = BM * kRowB;
  constexpr int kStageB = 2 * kTileB;
  constexpr int kLPT = BM / kRPL / kW;        // loads per wave per operand tile
  constexpr int kL = 2 * kLPT;                // loads per wave per stage
  constexpr int kEpRow = RN * 2 + 16;         // bf16 epilogue staging row (padded)
  constexpr int kEpB = RM * kEpRow;
  constexpr int kLdsB = (S * kStageB > kW * kEpB) ? S * kStageB : kW * kEpB;
  static_assert(kLPT * kRPL * kW == BM && BM == BN, "loads per wave");
  static_assert(S >= 2 && (S - 2) * kL < 64, "stages");
  __shared__ __attribute__((aligned(1024))) unsigned char smem[kLdsB];

  const int logical = xcd_remap(blockIdx.x, p.nblocks);
  const int per_group = kPGroup * p.ntiles;
  const int grp = logical / per_group;
  const int first_m = grp * kPGroup;
  const int gm = (p.mtiles - first_m) < kPGroup ? (p.mtiles - first_m) : kPGroup;
  const int within = logical - grp * per_group;
  const int m0 = (first_m + within % gm) * BM, n0 = (within / gm) * BN;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int wm = wave / WN, wn = wave % WN;

  const uint32_t row_bytes = static_cast<uint32_t>(p.dim) * 2u;
  const rsrc_t rx = make_rsrc_rows(p.x + static_cast<int64_t>(m0) * p.dim, p.T - m0 < BM ? p.T - m0 : BM,
                                   static_cast<uint32_t>(p.dim));
  const rsrc_t rw = make_rsrc_rows(p.W + static_cast<int64_t>(n0) * p.dim, p.nout - n0 < BN ? p.nout - n0 : BN,
                                   static_cast<uint32_t>(p.dim));
  // this lane's share of a wave load: row rl of the 1 KiB block, physical chunk pc holding logical chunk lc
  static_assert(kW % 2 == 0, "the row parity of 8-row blocks is the wave's");
  const int rl = lane / kCh, pc = lane % kCh;
  const int lc = pc ^ proj_swz<BK>(kRPL * wave + rl);
  const uint32_t vlane = static_cast<uint32_t>(rl) * row_bytes + static_cast<uint32_t>(lc) * 16u;
  uint32_t voff[kLPT];   // load q of this wave fills rows kRPL (wave + kW q) ..
#pragma unroll
  for (int q = 0; q < kLPT; ++q) voff[q] = vlane + static_cast<uint32_t>(kRPL * (wave + kW * q)) * row_bytes;

  // issue the loads of the stage at K offset k0 into ring slot `slot`; chunks at or past dim get an offset
  // past the resource (read as zero): only the last stage of a ragged K has any
  auto load_stage = [&](int k0, int slot) {
    const uint32_t kill = (k0 + 8 * lc < p.dim) ? 0u : 0x80000000u;
    unsigned char* base = smem + slot * kStageB;
#pragma unroll
    for (int q = 0; q < kLPT; ++q) {
      const int blk = (wave + kW * q) * 1024;
      dma16(rx, base + blk, voff[q] | kill, k0 * 2);
      dma16(rw, base + kTileB + blk, voff[q] | kill, k0 * 2);
    }
  };

  // fragment offsets within a stage: A rows wm RM + 32 i + lane % 32, B rows wn RN + 32 j + lane % 32,
  // logical chunk 2 kk + lane / 32 of each
  const int fr = lane & 31, fh = lane >> 5;
  int aoff[BK / 16], boff[BK / 16];
#pragma unroll
  for (int kk = 0; kk < BK / 16; ++kk) {
    const int ph = ((2 * kk + fh) ^ proj_swz<BK>(fr)) * 16;
    aoff[kk] = (wm * RM + fr) * kRowB + ph;
    boff[kk] = kTileB + (wn * RN + fr) * kRowB + ph;
  }

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  const int nk = (p.dim + BK - 1) / BK;
  // MFMA tiles of this wave that hold output columns (wave-uniform)
  const int live = p.nout - (n0 + wn * RN);
  const int jm = live <= 0 ? 0 : (live >= RN ? TN : (live + 31) / 32);

  auto main_loop = [&](auto jm_c) {
    constexpr int JM = decltype(jm_c)::value;
    constexpr int KK = BK / 16;
#pragma unroll
    for (int st = 0; st < S - 1; ++st)
      if (st < nk) load_stage(st * BK, st);
    for (int ks = 0; ks < nk; ++ks) {
      if (ks + S - 2 < nk) wait_vmcnt<(S - 2) * kL>();
      else wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      const int nxt = ks + S - 1;
      if (nxt < nk) load_stage(nxt * BK, nxt % S);
      const unsigned char* base = smem + (ks % S) * kStageB;
      // fragments of slice kk + 1 are read while the MFMAs of slice kk run
      bf16x8_t a[2][TM], b[2][TN > 0 ? TN : 1];
      auto rd = [&](int kk, int sl) {
#pragma unroll
        for (int i = 0; i < TM; ++i) a[sl][i] = *reinterpret_cast<const bf16x8_t*>(base + aoff[kk] + 32 * i * kRowB);
#pragma unroll
        for (int j = 0; j < JM; ++j) b[sl][j] = *reinterpret_cast<const bf16x8_t*>(base + boff[kk] + 32 * j * kRowB);
      };
      if constexpr (JM > 0) {
        rd(0, 0);
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
          if (kk + 1 < KK) rd(kk + 1, (kk + 1) & 1);
#pragma unroll
          for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int j = 0; j < JM; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[kk & 1][i], b[kk & 1][j], acc[i][j], 0, 0, 0);
        }
        // issue order: the ring loads, slice 0's fragments, then per slice one fragment read of the next
        // slice after every few MFMAs
        constexpr int kRd = TM + JM, kMf = TM * JM;
        constexpr int kPer = kMf / kRd > 0 ? kMf / kRd : 1;
        __builtin_amdgcn_sched_group_barrier(0x020, 2 * kLPT, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, kRd, 0);
#pragma unroll
        for (int kk = 0; kk + 1 < KK; ++kk) {
#pragma unroll
          for (int r = 0; r < kRd; ++r) {
            __builtin_amdgcn_sched_group_barrier(0x008, kPer, 0);
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
          }
          if constexpr (kMf > kPer * kRd) __builtin_amdgcn_sched_group_barrier(0x008, kMf - kPer * kRd, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, kMf, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  if (jm == TN) main_loop(std::integral_constant<int, TN>());
  else if (jm == 0) main_loop(std::integral_constant<int, 0>());
  else if (jm == 1) main_loop(std::integral_constant<int, 1>());
  else if (jm == 2) main_loop(std::integral_constant<int, (TN > 2 ? 2 : TN)>());
  else main_loop(std::integral_constant<int, (TN > 3 ? 3 : TN)>());

  // element e of lane l: row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32 of its 32 x 32 tile
  if constexpr (sizeof(Tout) == 4) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = wm * RM + 32 * i + 8 * (e >> 2) + 4 * fh + (e & 3);
          const int n = wn * RN + 32 * j + fr;
          proj_store<Tout>(p, m0 + m, n0 + n, acc[i][j][e]);
        }
  } else {
    __syncthreads();  // every wave is done reading the operand ring
    unsigned char* ep = smem + wave * kEpB;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int m = 32 * i + 8 * (e >> 2) + 4 * fh + (e & 3);
          const int n = 32 * j + fr;
          *reinterpret_cast<uint16_t*>(ep + m * kEpRow + n * 2) = f32_to_bf16(acc[i][j][e]);
        }
    wave_lds_sync();
    // read back 16-byte row chunks: RN / 8 chunks per row, 64 lanes per pass
    constexpr int kCPR = RN / 8;
    constexpr int kRPP = 64 / kCPR;
    const int cr = lane / kCPR, cc = lane % kCPR;
#pragma unroll 4
    for (int r0 = 0; r0 < RM; r0 += kRPP) {
      const int m = m0 + wm * RM + r0 + cr;
      const int n = n0 + wn * RN + 8 * cc;
      const uint4 v = *reinterpret_cast<const uint4*>(ep + (r0 + cr) * kEpRow + cc * 16);
      if (m >= p.T || n >= p.nout) continue;
      uint16_t* dst = nullptr;   // a 16-byte aligned destination for the whole chunk, when there is one
      if (n < p.dim) {
        if (p.vec_dt) dst = static_cast<uint16_t*>(p.dt) + static_cast<int64_t>(m) * p.dim + n;
      } else if (p.vec_bc) {
        const int cb = n - p.dim;
        dst = cb < p.dstate ? static_cast<uint16_t*>(p.B) + static_cast<int64_t>(m) * p.dstate + cb
                            : static_cast<uint16_t*>(p.C) + static_cast<int64_t>(m) * p.dstate + (cb - p.dstate);
      }
      if (dst) {
        *reinterpret_cast<uint4*>(dst) = v;
      } else {
        const uint32_t w4[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const uint16_t bits = static_cast<uint16_t>(u & 1 ? (w4[u >> 1] >> 16) : (w4[u >> 1] & 0xffffu));
          const int j = n + u;
          if (j >= p.nout) break;
          if (j < p.dim) static_cast<uint16_t*>(p.dt)[static_cast<int64_t>(m) * p.dim + j] = bits;
          else if (j < p.dim + p.dstate) static_cast<uint16_t*>(p.B)[static_cast<int64_t>(m) * p.dstate + (j - p.dim)] = bits;
          else static_cast<uint16_t*>(p.C)[static_cast<int64_t>(m) * p.dstate + (j - p.dim - p.dstate)] = bits;
        }
      }
    }
  }
}


// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64) {
    const int v = cache[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

size_t esize(int32_t dt) { return dt == SAMBA_BF16 ? 2 : 4; }

// Bytes of a checkpoint array: slots = tokens / 8 + nseq + 1 (see ckpt_slot), dim x 16 fp32 each.
size_t ckpt_bytes(int64_t tokens, int64_t nseq, int64_t dim) {
  return static_cast<size_t>(tokens / 8 + nseq + 1) * static_cast<size_t>(dim) * kN * 4;
}
bool dtype_ok(int32_t dt) { return dt == SAMBA_F32 || dt == SAMBA_BF16; }

// Tokens per wave slice.  Time-sliced variants keep 2*K*4 replay values per
// lane in registers: K = 8 stays within 128 VGPRs (four waves per SIMD); 16
// would halve the occupancy.  The sequential variant keeps no replay
// registers and takes 16.
int slice_tokens(int W) { return W >= 2 ? 8 : 16; }

struct FwdPlan {
  int W, tpw, lanes, threads, grid;   // lanes: per channel, 4 (scan_fwd_kernel) or 8 (scan_split8_kernel)
  int64_t nseq;
  FwdParams prm;
};

// Waves per time chunk.  Enough (sequence, tile) waves for two per SIMD:
// plain sequential scan.  Otherwise aim at four waves per SIMD by splitting
// time, but never into slices that the average sequence cannot fill.
int choose_time_slices(int64_t nseq, int64_t ntiles, int64_t tokens, int wmax, int (*slice)(int)) {
  const int64_t cus = device_cu_count();
  const int64_t base = nseq * ntiles;
  const int64_t avg_len = nseq > 0 ? tokens / nseq : 0;
  int W = 1;
  if (base < cus * 8) {
    while (W < wmax && base * W < cus * 16 && static_cast<int64_t>(W) * 2 * slice(W * 2) <= avg_len) W *= 2;
  }
  return W;
}

int slice_tokens8(int) { return kK8; }

// lanes: 0 (choose), 4 or 8 lanes per channel; ckpt: checkpoints requested (the 8-lane kernel has none).
// Automatic choice: the quad kernel's plan, unless it splits time and its (sequence, 16-channel tile)
// workgroups would leave at least half of the CUs idle; then 8-channel tiles double the workgroups at the
// same work per (token, channel).  (With one 16-wave workgroup per CU already, two 8-channel workgroups
// per CU measured slower than the 4-lane kernel: its instructions per (token, channel) are the same, its
// memory rows half as wide.)
samba_status make_fwd_plan(const void* x, const void* dt, const void* z, const void* B, const void* C, const float* A,
                           const float* D, const float* bias, const float* h0, const int32_t* cu, int64_t nseq,
                           int32_t batch, int32_t seqlen, int32_t dim, int ts, int lanes, bool ckpt, FwdPlan* plan) {
  const int64_t tokens = static_cast<int64_t>(batch) * seqlen;
  const int ntiles16 = (dim + kCPW - 1) / kCPW, ntiles8 = (dim + kCPW8 - 1) / kCPW8;
  if (lanes == 0) {
    lanes = 4;
    const int Wq = ts ? ts : choose_time_slices(nseq, ntiles16, tokens, 16, slice_tokens);
    const int W8 = ts ? ts : choose_time_slices(nseq, ntiles8, tokens, 16, slice_tokens8);
    if (!ckpt && Wq >= 2 && W8 >= 2 && 2 * nseq * ntiles16 <= device_cu_count()) lanes = 8;
  }
  if (lanes == 8 && (ckpt || ts == 1)) return SAMBA_ERR_UNSUPPORTED;
  const int ntiles = lanes == 8 ? ntiles8 : ntiles16;
  int W = ts;
  if (!W) {
    W = lanes == 8 ? choose_time_slices(nseq, ntiles, tokens, 16, slice_tokens8)
                   : choose_time_slices(nseq, ntiles, tokens, 16, slice_tokens);
    if (lanes == 8 && W < 2) W = 2;   // (forced 8 lanes on a sequence too short to split: two slices)
  }
  const int tpw = (W == 1) ? 4 : 1;
  const int ngroups = (ntiles + tpw - 1) / tpw;
  FwdParams& p = plan->prm;
  p = FwdParams{};
  p.x = x; p.dt = dt; p.z = z; p.B = B; p.C = C;
  p.A = A; p.Dskip = D; p.bias = bias;
  p.h0 = h0;
  p.cu = cu;
  p.total_tokens = tokens;
  p.seqlen = seqlen;
  p.dim = dim;
  p.ntiles = ntiles;
  p.tiles_per_wg = tpw;
  p.ngroups = ngroups;
  const int64_t nblocks = nseq * ngroups;
  if (nblocks > 0x7fffffff) return SAMBA_ERR_BAD_SHAPE;
  p.nblocks = static_cast<int32_t>(nblocks);
  plan->W = W;
  plan->tpw = tpw;
  plan->lanes = lanes;
  plan->threads = 64 * W * tpw;
  plan->grid = static_cast<int>(nblocks);
  plan->nseq = nseq;
  return SAMBA_OK;
}

samba_status validate_fwd(const samba_scan_fwd_args* a, FwdPlan* plan) {
  if (!a) return SAMBA_ERR_NULL_ARG;
  if (a->struct_size != sizeof(samba_scan_fwd_args)) return SAMBA_ERR_BAD_STRUCT;
  if (a->dstate != kN) return SAMBA_ERR_UNSUPPORTED;
  if (!dtype_ok(a->in_dtype) || !dtype_ok(a->y_dtype)) return SAMBA_ERR_BAD_DTYPE;
  if (a->batch < 0 || a->seqlen < 0 || a->dim < 1 || a->dim >= kMaxDim) return SAMBA_ERR_BAD_SHAPE;
  const int ts = a->time_slices;
  if (!(ts == 0 || ts == 1 || ts == 2 || ts == 4 || ts == 8 || ts == 16)) return SAMBA_ERR_UNSUPPORTED;
  const int lanes = a->lanes_per_channel;
  if (!(lanes == 0 || lanes == 4 || lanes == 8)) return SAMBA_ERR_UNSUPPORTED;
  if (lanes == 8 && (ts == 1 || a->h_ckpt)) return SAMBA_ERR_UNSUPPORTED;
  int64_t nseq = a->batch;
  if (a->cu_seqlens) {
    if (a->batch != 1 || a->nseq < 1) return SAMBA_ERR_BAD_SHAPE;
    nseq = a->nseq;
    if (!aligned(a->cu_seqlens, 4)) return SAMBA_ERR_MISALIGNED;
  }
  const int64_t tokens = static_cast<int64_t>(a->batch) * a->seqlen;
  if (!a->A || !a->D || !a->dt_bias) return SAMBA_ERR_NULL_ARG;
  if (tokens > 0 && (!a->x || !a->dt || !a->z || !a->B || !a->C || !a->y)) return SAMBA_ERR_NULL_ARG;
  const size_t ei = esize(a->in_dtype), eo = esize(a->y_dtype);
  if (!aligned(a->x, ei) || !aligned(a->dt, ei) || !aligned(a->z, ei) || !aligned(a->y, eo)) return SAMBA_ERR_MISALIGNED;
  if (!aligned(a->B, 16) || !aligned(a->C, 16) || !aligned(a->A, 16) || !aligned(a->h0, 16) ||
      !aligned(a->h_last, 16) || !aligned(a->h_ckpt, 16) || !aligned(a->D, 4) || !aligned(a->dt_bias, 4))
    return SAMBA_ERR_MISALIGNED;
  // outputs must not overlap inputs (h_last == h0 exactly is allowed: in-place carry)
  const size_t n_td = static_cast<size_t>(tokens) * a->dim;
  const size_t n_state = static_cast<size_t>(nseq) * a->dim * kN * 4;
  const void* ins[] = {a->x, a->dt, a->z, a->B, a->C, a->A, a->D, a->dt_bias, a->h0, a->cu_seqlens};
  const size_t insz[] = {n_td * ei, n_td * ei, n_td * ei, static_cast<size_t>(tokens) * kN * ei,
                         static_cast<size_t>(tokens) * kN * ei, static_cast<size_t>(a->dim) * kN * 4,
                         static_cast<size_t>(a->dim) * 4, static_cast<size_t>(a->dim) * 4, n_state,
                         a->cu_seqlens ? static_cast<size_t>(nseq + 1) * 4 : 0};
  for (int i = 0; i < 10; ++i) {
    if (overlap(a->y, n_td * eo, ins[i], insz[i])) return SAMBA_ERR_ALIASING;
    if (i != 8 && overlap(a->h_last, n_state, ins[i], insz[i])) return SAMBA_ERR_ALIASING;
  }
  if (a->h_last && a->h0 && a->h_last != a->h0 && overlap(a->h_last, n_state, a->h0, n_state))
    return SAMBA_ERR_ALIASING;
  if (overlap(a->y, n_td * eo, a->h_last, n_state)) return SAMBA_ERR_ALIASING;
  if (a->h_ckpt) {
    const size_t n_ck = ckpt_bytes(tokens, nseq, a->dim);
    for (int i = 0; i < 10; ++i)
      if (overlap(a->h_ckpt, n_ck, ins[i], insz[i])) return SAMBA_ERR_ALIASING;
    if (overlap(a->h_ckpt, n_ck, a->y, n_td * eo) || overlap(a->h_ckpt, n_ck, a->h_last, n_state))
      return SAMBA_ERR_ALIASING;
  }

  if (!plan) return SAMBA_OK;
  return make_fwd_plan(a->x, a->dt, a->z, a->B, a->C, a->A, a->D, a->dt_bias, a->h0, a->cu_seqlens, nseq,
                       a->batch, a->seqlen, a->dim, ts, lanes, a->h_ckpt != nullptr, plan);
}

template <typename Tin, typename Tout>
hipError_t launch_fwd(const FwdPlan& pl, hipStream_t st) {
  const dim3 grid(pl.grid), block(pl.threads);
  if (pl.lanes == 8) {
    switch (pl.W) {
      case 2: hipLaunchKernelGGL((scan_split8_kernel<Tin, Tout, 2>), grid, block, 0, st, pl.prm); break;
      case 4: hipLaunchKernelGGL((scan_split8_kernel<Tin, Tout, 4>), grid, block, 0, st, pl.prm); break;
      case 8: hipLaunchKernelGGL((scan_split8_kernel<Tin, Tout, 8>), grid, block, 0, st, pl.prm); break;
      default: hipLaunchKernelGGL((scan_split8_kernel<Tin, Tout, 16>), grid, block, 0, st, pl.prm); break;
    }
    return hipGetLastError();
  }
  if (pl.prm.ckpt == nullptr && (pl.W == 1 || pl.W == 4 || pl.W == 8 || pl.W == 16))   // the copy in samba_scan_fwd_ilp.hip
    return samba_fwd::launch_fwd_ilp(sizeof(Tin) == 2, sizeof(Tout) == 2, pl.W, grid, block, pl.prm, st);
  switch (pl.W) {
    case 1: hipLaunchKernelGGL((scan_fwd_kernel<Tin, Tout, 1, 4, 16>), grid, block, 0, st, pl.prm); break;
    case 2: hipLaunchKernelGGL((scan_fwd_kernel<Tin, Tout, 2, 1, 8>), grid, block, 0, st, pl.prm); break;
    case 4: hipLaunchKernelGGL((scan_fwd_kernel<Tin, Tout, 4, 1, 8>), grid, block, 0, st, pl.prm); break;
    case 8: hipLaunchKernelGGL((scan_fwd_kernel<Tin, Tout, 8, 1, 8>), grid, block, 0, st, pl.prm); break;
    default: hipLaunchKernelGGL((scan_fwd_kernel<Tin, Tout, 16, 1, 8>), grid, block, 0, st, pl.prm); break;
  }
  return hipGetLastError();
}

template <typename Tin>
hipError_t launch_ckpt(const FwdPlan& pl, hipStream_t st) {
  const dim3 grid(pl.grid), block(pl.threads);
  switch (pl.W) {
    case 1: hipLaunchKernelGGL((scan_fwd_kernel<Tin, float, 1, 4, 16, true>), grid, block, 0, st, pl.prm); break;
    case 2: hipLaunchKernelGGL((scan_fwd_kernel<Tin, float, 2, 1, 8, true>), grid, block, 0, st, pl.prm); break;
    case 4: hipLaunchKernelGGL((scan_fwd_kernel<Tin, float, 4, 1, 8, true>), grid, block, 0, st, pl.prm); break;
    case 8: hipLaunchKernelGGL((scan_fwd_kernel<Tin, float, 8, 1, 8, true>), grid, block, 0, st, pl.prm); break;
    default: hipLaunchKernelGGL((scan_fwd_kernel<Tin, float, 16, 1, 8, true>), grid, block, 0, st, pl.prm); break;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// backward host side
// ---------------------------------------------------------------------------
struct BwdPlan {
  int W;                    // backward waves per workgroup
  int64_t nseq, tokens;
  int ntiles;
  size_t off_dbc, off_dpar, bytes;  // workspace layout: checkpoints at 0, then dB/dC partials, then parameter partials
  FwdPlan ck;               // checkpoint pass
  BwdParams prm;
};

size_t round256(size_t v) { return (v + 255) & ~static_cast<size_t>(255); }

int bwd_slice(int) { return kBK; }

samba_status bwd_layout(int64_t nseq, int64_t tokens, int32_t dim, bool own_ckpt, BwdPlan* pl) {
  const int64_t ntiles = (dim + kCPW - 1) / kCPW;
  const size_t ck = own_ckpt ? round256(ckpt_bytes(tokens, nseq, dim)) : 0;
  const size_t dbc = round256(static_cast<size_t>(ntiles) * tokens * 32 * 4);
  const size_t dpar = round256(static_cast<size_t>(nseq) * dim * kParW * 4);
  pl->nseq = nseq;
  pl->tokens = tokens;
  pl->ntiles = static_cast<int>(ntiles);
  pl->off_dbc = ck;
  pl->off_dpar = ck + dbc;
  pl->bytes = ck + dbc + dpar;
  return SAMBA_OK;
}

samba_status bwd_shape(const samba_scan_bwd_args* a, int64_t* nseq) {
  if (!a) return SAMBA_ERR_NULL_ARG;
  if (a->struct_size != sizeof(samba_scan_bwd_args)) return SAMBA_ERR_BAD_STRUCT;
  if (a->dstate != kN) return SAMBA_ERR_UNSUPPORTED;
  if (!dtype_ok(a->in_dtype)) return SAMBA_ERR_BAD_DTYPE;
  if (a->batch < 0 || a->seqlen < 0 || a->dim < 1 || a->dim >= kMaxDim) return SAMBA_ERR_BAD_SHAPE;
  const int ts = a->time_slices;
  if (!(ts == 0 || ts == 1 || ts == 2 || ts == 4 || ts == 8)) return SAMBA_ERR_UNSUPPORTED;
  *nseq = a->batch;
  if (a->cu_seqlens) {
    if (a->batch != 1 || a->nseq < 1) return SAMBA_ERR_BAD_SHAPE;
    *nseq = a->nseq;
  }
  return SAMBA_OK;
}

samba_status validate_bwd(const samba_scan_bwd_args* a, BwdPlan* plan) {
  int64_t nseq = 0;
  samba_status st = bwd_shape(a, &nseq);
  if (st != SAMBA_OK) return st;
  if (a->cu_seqlens && !aligned(a->cu_seqlens, 4)) return SAMBA_ERR_MISALIGNED;
  const int64_t tokens = static_cast<int64_t>(a->batch) * a->seqlen;
  if (!a->A || !a->D || !a->dt_bias || !a->dA || !a->dD || !a->ddt_bias) return SAMBA_ERR_NULL_ARG;
  if (tokens > 0 && (!a->x || !a->dt || !a->z || !a->B || !a->C || !a->dy || !a->dx || !a->ddt || !a->dz ||
                     !a->dB || !a->dC))
    return SAMBA_ERR_NULL_ARG;
  const size_t ei = esize(a->in_dtype);
  const void* elem[] = {a->x, a->dt, a->z, a->dy, a->dx, a->ddt, a->dz};
  for (const void* q : elem)
    if (!aligned(q, ei)) return SAMBA_ERR_MISALIGNED;
  const void* a16[] = {a->B, a->C, a->A, a->h0, a->dh_last, a->h_ckpt, a->dB, a->dC, a->dA, a->dh0};
  for (const void* q : a16)
    if (!aligned(q, 16)) return SAMBA_ERR_MISALIGNED;
  const void* a4[] = {a->D, a->dt_bias, a->dD, a->ddt_bias};
  for (const void* q : a4)
    if (!aligned(q, 4)) return SAMBA_ERR_MISALIGNED;
  BwdPlan local;
  BwdPlan* pl = plan ? plan : &local;
  bwd_layout(nseq, tokens, a->dim, a->h_ckpt == nullptr, pl);
  if (!a->workspace || a->workspace_bytes < pl->bytes) return SAMBA_ERR_WORKSPACE;
  if (!aligned(a->workspace, 256)) return SAMBA_ERR_WORKSPACE;
  // no output may overlap an input or another output
  const size_t n_td = static_cast<size_t>(tokens) * a->dim, n_tn = static_cast<size_t>(tokens) * kN;
  const size_t n_dn = static_cast<size_t>(a->dim) * kN * 4, n_d = static_cast<size_t>(a->dim) * 4;
  const size_t n_state = static_cast<size_t>(nseq) * a->dim * kN * 4;
  const void* ins[] = {a->x, a->dt, a->z, a->B, a->C, a->A, a->D, a->dt_bias, a->h0, a->dy, a->dh_last, a->cu_seqlens,
                       a->h_ckpt};
  const size_t insz[] = {n_td * ei, n_td * ei, n_td * ei, n_tn * ei, n_tn * ei, n_dn, n_d, n_d, n_state, n_td * ei,
                         n_state, a->cu_seqlens ? static_cast<size_t>(nseq + 1) * 4 : 0,
                         a->h_ckpt ? ckpt_bytes(tokens, nseq, a->dim) : 0};
  const void* outs[] = {a->dx, a->ddt, a->dz, a->dB, a->dC, a->dA, a->dD, a->ddt_bias, a->dh0, a->workspace};
  const size_t outsz[] = {n_td * ei, n_td * ei, n_td * ei, n_tn * 4, n_tn * 4, n_dn, n_d, n_d, n_state, pl->bytes};
  for (int i = 0; i < 10; ++i) {
    for (int j = 0; j < 13; ++j)
      if (overlap(outs[i], outsz[i], ins[j], insz[j])) return SAMBA_ERR_ALIASING;
    for (int j = i + 1; j < 10; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return SAMBA_ERR_ALIASING;
  }
  if (!plan) return SAMBA_OK;

  // checkpoint pass: the forward kernel's checkpoint variant, its own launch plan
  st = make_fwd_plan(a->x, a->dt, a->z, a->B, a->C, a->A, a->D, a->dt_bias, a->h0, a->cu_seqlens, nseq, a->batch,
                     a->seqlen, a->dim, 0, 4, true, &pl->ck);
  if (st != SAMBA_OK) return st;
  char* ws = static_cast<char*>(a->workspace);
  float* ckpt = a->h_ckpt ? const_cast<float*>(a->h_ckpt) : reinterpret_cast<float*>(ws);
  pl->ck.prm.ckpt = ckpt;
  const int ts = a->time_slices;
  pl->W = ts ? ts : choose_time_slices(nseq, pl->ntiles, tokens, 8, bwd_slice);
  const int64_t nblocks = nseq * pl->ntiles;
  if (nblocks > 0x7fffffff) return SAMBA_ERR_BAD_SHAPE;
  BwdParams& p = pl->prm;
  p = BwdParams{};
  p.x = a->x; p.dt = a->dt; p.z = a->z; p.B = a->B; p.C = a->C; p.dy = a->dy;
  p.A = a->A; p.Dskip = a->D; p.bias = a->dt_bias;
  p.dh_last = a->dh_last;
  p.ckpt = ckpt;
  p.dx = a->dx; p.ddt = a->ddt; p.dz = a->dz;
  p.dbc = reinterpret_cast<float*>(ws + pl->off_dbc);
  p.dpar = reinterpret_cast<float*>(ws + pl->off_dpar);
  p.dh0 = a->dh0;
  p.cu = a->cu_seqlens;
  p.total_tokens = tokens;
  p.seqlen = a->seqlen;
  p.dim = a->dim;
  p.ntiles = pl->ntiles;
  p.nblocks = static_cast<int32_t>(nblocks);
  return SAMBA_OK;
}

template <typename T>
hipError_t launch_bwd_kernel(const BwdPlan& pl, hipStream_t st) {
  const dim3 grid(pl.prm.nblocks), block(64 * pl.W);
  switch (pl.W) {
    case 1: hipLaunchKernelGGL((scan_bwd_kernel<T, 1>), grid, block, 0, st, pl.prm); break;
    case 2: hipLaunchKernelGGL((scan_bwd_kernel<T, 2>), grid, block, 0, st, pl.prm); break;
    case 4: hipLaunchKernelGGL((scan_bwd_kernel<T, 4>), grid, block, 0, st, pl.prm); break;
    default: hipLaunchKernelGGL((scan_bwd_kernel<T, 8>), grid, block, 0, st, pl.prm); break;
  }
  return hipGetLastError();
}

samba_status validate_step(const samba_scan_step_args* a) {
  if (!a) return SAMBA_ERR_NULL_ARG;
  if (a->struct_size != sizeof(samba_scan_step_args)) return SAMBA_ERR_BAD_STRUCT;
  if (a->dstate != kN) return SAMBA_ERR_UNSUPPORTED;
  if (!dtype_ok(a->in_dtype) || !dtype_ok(a->y_dtype)) return SAMBA_ERR_BAD_DTYPE;
  if (a->batch < 0 || a->dim < 1) return SAMBA_ERR_BAD_SHAPE;
  if (!a->A || !a->D || !a->dt_bias) return SAMBA_ERR_NULL_ARG;
  if (a->batch > 0 && (!a->state || !a->x || !a->dt || !a->z || !a->B || !a->C || !a->y)) return SAMBA_ERR_NULL_ARG;
  const size_t ei = esize(a->in_dtype), eo = esize(a->y_dtype);
  if (!aligned(a->state, 16) || !aligned(a->B, 16) || !aligned(a->C, 16) || !aligned(a->A, 16) ||
      !aligned(a->x, ei) || !aligned(a->dt, ei) || !aligned(a->z, ei) || !aligned(a->y, eo) ||
      !aligned(a->D, 4) || !aligned(a->dt_bias, 4))
    return SAMBA_ERR_MISALIGNED;
  const size_t nbd = static_cast<size_t>(a->batch) * a->dim;
  const size_t n_state = nbd * kN * 4;
  const void* ins[] = {a->x, a->dt, a->z, a->B, a->C, a->A, a->D, a->dt_bias};
  const size_t insz[] = {nbd * ei, nbd * ei, nbd * ei, static_cast<size_t>(a->batch) * kN * ei,
                         static_cast<size_t>(a->batch) * kN * ei, static_cast<size_t>(a->dim) * kN * 4,
                         static_cast<size_t>(a->dim) * 4, static_cast<size_t>(a->dim) * 4};
  for (int i = 0; i < 8; ++i) {
    if (overlap(a->y, nbd * eo, ins[i], insz[i])) return SAMBA_ERR_ALIASING;
    if (overlap(a->state, n_state, ins[i], insz[i])) return SAMBA_ERR_ALIASING;
  }
  if (overlap(a->y, nbd * eo, a->state, n_state)) return SAMBA_ERR_ALIASING;
  return SAMBA_OK;
}

}  // namespace

extern "C" {

samba_status samba_scan_fwd(const samba_scan_fwd_args* args, void* stream) {
  FwdPlan pl;
  const samba_status st = validate_fwd(args, &pl);
  if (st != SAMBA_OK) return st;
  pl.prm.h_last = args->h_last;
  pl.prm.y = args->y;
  pl.prm.ckpt = args->h_ckpt;
  if (pl.grid == 0) return SAMBA_OK;  // no sequences
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (args->in_dtype == SAMBA_BF16)
    e = (args->y_dtype == SAMBA_BF16) ? launch_fwd<uint16_t, uint16_t>(pl, s) : launch_fwd<uint16_t, float>(pl, s);
  else
    e = (args->y_dtype == SAMBA_BF16) ? launch_fwd<float, uint16_t>(pl, s) : launch_fwd<float, float>(pl, s);
  return e == hipSuccess ? SAMBA_OK : SAMBA_ERR_HIP;
}

samba_status samba_scan_fwd_plan(const samba_scan_fwd_args* args, int32_t* time_slices, int32_t* workgroups,
                                 int32_t* threads_per_workgroup, int32_t* lanes_per_channel) {
  FwdPlan pl;
  const samba_status st = validate_fwd(args, &pl);
  if (st != SAMBA_OK) return st;
  if (lanes_per_channel) *lanes_per_channel = pl.lanes;
  if (time_slices) *time_slices = pl.W;
  if (workgroups) *workgroups = pl.grid;
  if (threads_per_workgroup) *threads_per_workgroup = pl.threads;
  return SAMBA_OK;
}

samba_status samba_scan_bwd_workspace_size(const samba_scan_bwd_args* args, size_t* bytes) {
  int64_t nseq = 0;
  const samba_status st = bwd_shape(args, &nseq);
  if (st != SAMBA_OK) return st;
  if (!bytes) return SAMBA_ERR_NULL_ARG;
  BwdPlan pl;
  bwd_layout(nseq, static_cast<int64_t>(args->batch) * args->seqlen, args->dim, args->h_ckpt == nullptr, &pl);
  *bytes = pl.bytes;
  return SAMBA_OK;
}

samba_status samba_scan_ckpt_bytes(int32_t batch, int32_t seqlen, int32_t nseq, int32_t dim, size_t* bytes) {
  if (!bytes) return SAMBA_ERR_NULL_ARG;
  if (batch < 0 || seqlen < 0 || nseq < 0 || dim < 1 || dim >= kMaxDim) return SAMBA_ERR_BAD_SHAPE;
  *bytes = ckpt_bytes(static_cast<int64_t>(batch) * seqlen, nseq, dim);
  return SAMBA_OK;
}

samba_status samba_scan_bwd(const samba_scan_bwd_args* args, void* stream) {
  BwdPlan pl;
  const samba_status st = validate_bwd(args, &pl);
  if (st != SAMBA_OK) return st;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool bf = args->in_dtype == SAMBA_BF16;
  if (pl.prm.nblocks > 0) {
    if (pl.tokens > 0 && !args->h_ckpt) {
      const hipError_t e = bf ? launch_ckpt<uint16_t>(pl.ck, s) : launch_ckpt<float>(pl.ck, s);
      if (e != hipSuccess) return SAMBA_ERR_HIP;
    }
    const hipError_t e = bf ? launch_bwd_kernel<uint16_t>(pl, s) : launch_bwd_kernel<float>(pl, s);
    if (e != hipSuccess) return SAMBA_ERR_HIP;
  }
  const int64_t nout = pl.tokens * 8 + static_cast<int64_t>(args->dim) * 18;
  const int64_t blocks = (nout + 255) / 256;
  if (blocks > 0x7fffffff) return SAMBA_ERR_BAD_SHAPE;
  hipLaunchKernelGGL(scan_bwd_finish_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s, pl.prm.dbc,
                     pl.prm.dpar, args->dB, args->dC, args->dA, args->dD, args->ddt_bias, pl.tokens, pl.ntiles,
                     static_cast<int32_t>(pl.nseq), args->dim);
  return hipGetLastError() == hipSuccess ? SAMBA_OK : SAMBA_ERR_HIP;
}

samba_status samba_proj(const samba_proj_args* a, void* stream) {
  if (!a) return SAMBA_ERR_NULL_ARG;
  if (a->struct_size != sizeof(samba_proj_args)) return SAMBA_ERR_BAD_STRUCT;
  if (a->in_dtype != SAMBA_BF16 || !dtype_ok(a->out_dtype)) return SAMBA_ERR_BAD_DTYPE;
  if (a->tokens < 0 || a->dim < 8 || a->dstate < 1) return SAMBA_ERR_BAD_SHAPE;
  // dim % 8: 16-byte operand chunks; dim < 2^22: byte offsets within a 256-row tile stay below 2^31
  if (a->dim % 8 != 0 || a->dim >= (1 << 22)) return SAMBA_ERR_BAD_SHAPE;
  const int64_t nout = static_cast<int64_t>(a->dim) + 2 * static_cast<int64_t>(a->dstate);
  if (nout > 0x7fffffff) return SAMBA_ERR_BAD_SHAPE;
  if (!a->W) return SAMBA_ERR_NULL_ARG;
  if (a->tokens > 0 && (!a->x || !a->dt || !a->B || !a->C)) return SAMBA_ERR_NULL_ARG;
  const size_t eo = esize(a->out_dtype);
  if (!aligned(a->x, 16) || !aligned(a->W, 16) || !aligned(a->dt, eo) || !aligned(a->B, eo) || !aligned(a->C, eo))
    return SAMBA_ERR_MISALIGNED;
  const size_t T = static_cast<size_t>(a->tokens), dim = static_cast<size_t>(a->dim), n = static_cast<size_t>(a->dstate);
  const void* outs[] = {a->dt, a->B, a->C};
  const size_t outsz[] = {T * dim * eo, T * n * eo, T * n * eo};
  const void* ins[] = {a->x, a->W};
  const size_t insz[] = {T * dim * 2, static_cast<size_t>(nout) * dim * 2};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 2; ++j)
      if (overlap(outs[i], outsz[i], ins[j], insz[j])) return SAMBA_ERR_ALIASING;
    for (int j = i + 1; j < 3; ++j)
      if (overlap(outs[i], outsz[i], outs[j], outsz[j])) return SAMBA_ERR_ALIASING;
  }
  if (a->tokens == 0) return SAMBA_OK;
  ProjParams p;
  p.x = static_cast<const uint16_t*>(a->x);
  p.W = static_cast<const uint16_t*>(a->W);
  p.dt = a->dt; p.B = a->B; p.C = a->C;
  p.T = a->tokens; p.dim = a->dim; p.dstate = a->dstate; p.nout = static_cast<int32_t>(nout);
  p.mtiles = (a->tokens + 255) / 256;
  p.ntiles = static_cast<int32_t>((nout + 255) / 256);
  const int64_t nblocks = static_cast<int64_t>(p.mtiles) * p.ntiles;
  if (nblocks > 0x7fffffff) return SAMBA_ERR_BAD_SHAPE;
  p.nblocks = static_cast<int32_t>(nblocks);
  p.vec_dt = aligned(a->dt, 16);
  p.vec_bc = a->dstate % 8 == 0 && aligned(a->B, 16) && aligned(a->C, 16);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 block(64 * kDWM * kDWN);
  if (a->out_dtype == SAMBA_BF16)
    hipLaunchKernelGGL((proj_dma_kernel<uint16_t, kDBK, kDS, kDWM, kDWN>), dim3(p.nblocks), block, 0, s, p);
  else
    hipLaunchKernelGGL((proj_dma_kernel<float, kDBK, kDS, kDWM, kDWN>), dim3(p.nblocks), block, 0, s, p);
  return hipGetLastError() == hipSuccess ? SAMBA_OK : SAMBA_ERR_HIP;
}

samba_status samba_scan_step(const samba_scan_step_args* args, void* stream) {
  const samba_status st = validate_step(args);
  if (st != SAMBA_OK) return st;
  const int64_t nquads = static_cast<int64_t>(args->batch) * args->dim;
  if (nquads == 0) return SAMBA_OK;
  // sequences per thread: more than one once the batch is large enough to
  // keep every CU busy (A, dt_bias and D are then loaded once per channel)
  const int qpt = (args->batch >= 2 * kStepQPT &&
                   static_cast<int64_t>((args->dim + 63) / 64) * (args->batch / kStepQPT) >= device_cu_count() * 2)
                      ? kStepQPT : 1;
  const int64_t gx = (args->dim + 63) / 64, gy = (static_cast<int64_t>(args->batch) + qpt - 1) / qpt;
  if (gy > 65535) return SAMBA_ERR_BAD_SHAPE;
  StepParams p;
  p.state = args->state;
  p.x = args->x; p.dt = args->dt; p.z = args->z; p.B = args->B; p.C = args->C;
  p.A = args->A; p.Dskip = args->D; p.bias = args->dt_bias;
  p.y = args->y;
  p.batch = args->batch;
  p.dim = args->dim;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const dim3 grid(static_cast<unsigned>(gx), static_cast<unsigned>(gy)), block(256);
  const bool bi = args->in_dtype == SAMBA_BF16, bo = args->y_dtype == SAMBA_BF16;
  if (qpt == 1) {
    if (bi) { if (bo) hipLaunchKernelGGL((scan_step_kernel<uint16_t, uint16_t, 1>), grid, block, 0, s, p);
              else hipLaunchKernelGGL((scan_step_kernel<uint16_t, float, 1>), grid, block, 0, s, p); }
    else { if (bo) hipLaunchKernelGGL((scan_step_kernel<float, uint16_t, 1>), grid, block, 0, s, p);
           else hipLaunchKernelGGL((scan_step_kernel<float, float, 1>), grid, block, 0, s, p); }
  } else {
    if (bi) { if (bo) hipLaunchKernelGGL((scan_step_kernel<uint16_t, uint16_t, kStepQPT>), grid, block, 0, s, p);
              else hipLaunchKernelGGL((scan_step_kernel<uint16_t, float, kStepQPT>), grid, block, 0, s, p); }
    else { if (bo) hipLaunchKernelGGL((scan_step_kernel<float, uint16_t, kStepQPT>), grid, block, 0, s, p);
           else hipLaunchKernelGGL((scan_step_kernel<float, float, kStepQPT>), grid, block, 0, s, p); }
  }
  return hipGetLastError() == hipSuccess ? SAMBA_OK : SAMBA_ERR_HIP;
}

const char* samba_status_string(int status) {
  switch (status) {
    case SAMBA_OK: return "ok";
    case SAMBA_ERR_NULL_ARG: return "a required pointer is NULL";
    case SAMBA_ERR_BAD_SHAPE: return "invalid or inconsistent sizes";
    case SAMBA_ERR_BAD_DTYPE: return "unsupported dtype code";
    case SAMBA_ERR_MISALIGNED: return "pointer misaligned";
    case SAMBA_ERR_ALIASING: return "an output overlaps an input";
    case SAMBA_ERR_UNSUPPORTED: return "unsupported configuration (dstate must be 16; time_slices 0/1/2/4/8/16)";
    case SAMBA_ERR_BAD_STRUCT: return "argument struct size mismatch (header/library version skew)";
    case SAMBA_ERR_HIP: return "HIP runtime error at launch";
    case SAMBA_ERR_WORKSPACE:
      return "workspace NULL, too small or not 256-byte aligned (no-allocation entry: needs more than its static "
             "scratch)";
    default: return "unknown status";
  }
}

int samba_scan_abi_version(void) { return SAMBA_SCAN_ABI_VERSION; }

}  // extern "C"
