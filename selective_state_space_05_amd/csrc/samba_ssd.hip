// samba_ssd.hip -- gfx950 (MI355X) prefill of the state-space duality layer (the Mamba-2 form that page
// "SAMBA混合注意力状态空间模型" compares Samba with, 与其他混合架构对比): a scalar decay per head and a
// head_dim x dstate state per head, so that a chunk of tokens is a handful of dense products.
//
// One workgroup (4 waves) owns one (sequence, head) and walks its tokens in chunks of Q = 64, the fp32
// state carried in registers from chunk to chunk.  With la_t = log2e * A * sum_{r<=t} Δ_r inside the chunk,
// w_s = 2^(la_end - la_s) Δ_s and the entering state H (P x N):
//   (a) Sᵀ[s][t] = sum_n B[s][n] C[t][n]                       MFMA, K = N
//   (b) Mᵀ[s][t] = Sᵀ[s][t] 2^(la_t - la_s) Δ_s  (s <= t, else 0), + D on the diagonal (the skip)
//   (c) Yᵀ[p][t] = sum_s X[s][p] Mᵀ[s][t]                      MFMA, K = Q
//   (d)         + 2^(la_t) sum_n H[p][n] C[t][n]               MFMA, K = N
//   (e) Hᵀ[n][p] = 2^(la_end) Hᵀ[n][p] + sum_s B[s][n] (w_s X[s][p])     MFMA, K = Q
//   y[t][p] = Yᵀ[p][t] * silu(z[t][p])
// The operands built here rather than read (M, H, w X) are split into bf16 hi + lo pairs, two MFMAs each:
// one bf16 rounding of them alone costs about 2e-3 of the output's scale, the pair about 1e-6.
//
// Wave roles (32x32 tiles, v_mfma_f32_32x32x16_bf16): wave w holds p-tile a = w & 1 of the state and its
// n-tiles of half hb = w >> 1, and finishes the output tile (p-tile a, t-tile hb).  Products are laid out
// so that one product's accumulators are the next one's operand without a trip through LDS:
//   * Sᵀ's accumulator rows s are the contraction index of (c): a lane's 8 elements of a 16-wide step
//     are s = 16kk + 8(j/4) + 4hi + j%4, and X is read from LDS in that order;
//   * the state lives as Hᵀ accumulators (lane = column p), which are (d)'s A operand in the same way,
//     with C read in the matching n order.
// (d) over a wave's half of the states leaves partial sums for both t-tiles; the half for the other
// t-tile goes to the partner wave through LDS.  Chunk inputs are loaded one chunk ahead into registers and
// staged into LDS (C and B row-major, B and X transposed); Δ, la and w are computed by wave 0.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "samba_ssd.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
using rsrc_t = __amdgpu_buffer_rsrc_t;

constexpr int kRsrcWord3 = 0x00020000;   // raw (untyped, unswizzled) buffer
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kQ = 64;                   // tokens per chunk
constexpr int kP = 64;                   // head size
constexpr int kTRow = kQ + 8;            // row stride (bf16) of the transposed tiles in LDS

__device__ __forceinline__ rsrc_t rsrc_bytes(const void* base, int64_t bytes) {
  const uint32_t b = bytes <= 0 ? 0u : (bytes >= 0xffffffffLL ? 0xffffffffu : static_cast<uint32_t>(bytes));
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(b),
                                          kRsrcWord3);
}
__device__ __forceinline__ uint4 ld16(rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ float widen(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }

// softplus(v) = log(1 + e^v), with the rounding of 1 + e undone to first order when e < 1 (small Δ keep
// full relative accuracy); v > 20 returns v.
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

// Consecutive logical blocks land on the same XCD (the dispatcher deals blocks round-robin over 8 XCDs),
// so the heads of one sequence, which read the same B and C, share an L2.  A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7, xcd = bid & 7, slot = bid >> 3;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// 16-bit halves: (low of a, low of b) and (high of a, high of b)
__device__ __forceinline__ uint32_t lows(uint32_t a, uint32_t b) { return (a & 0xffffu) | (b << 16); }
__device__ __forceinline__ uint32_t highs(uint32_t a, uint32_t b) { return (a >> 16) | (b & 0xffff0000u); }
__device__ __forceinline__ uint32_t word(const uint4& v, int k) {
  return k == 0 ? v.x : (k == 1 ? v.y : (k == 2 ? v.z : v.w));
}

// two 4-element runs of a bf16 row as one 8-element operand
__device__ __forceinline__ bf16x8_t cat4(const uint16_t* p0, const uint16_t* p1) {
  const bf16x4_t u = *reinterpret_cast<const bf16x4_t*>(p0);
  const bf16x4_t v = *reinterpret_cast<const bf16x4_t*>(p1);
  return __builtin_shufflevector(u, v, 0, 1, 2, 3, 4, 5, 6, 7);
}

// the 8 accumulator elements e0 .. e0 + 7 as a bf16 hi + lo pair
__device__ __forceinline__ void split8(const f32x16_t& acc, int e0, bf16x8_t& hi, bf16x8_t& lo) {
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float v = acc[e0 + j];
    const __bf16 h = static_cast<__bf16>(v);
    hi[j] = h;
    lo[j] = static_cast<__bf16>(v - static_cast<float>(h));
  }
}

struct SsdParams {
  const void *x, *dt, *z, *B, *C;
  const float *A, *Dskip, *bias, *h0;
  float* h_last;
  void* y;
  const int32_t* cu;
  int32_t nseq, seqlen, heads, ngroups, total;
};

template <int N>
struct Smem {
  static constexpr int kRow = N + 8;                // row stride (bf16) of the row-major tiles
  uint16_t c[kQ * kRow];                            // C [t][n]
  uint16_t b[kQ * kRow];                            // B [s][n]
  uint16_t bt[N * kTRow];                           // B transposed [n][s]
  uint16_t xt[kP * kTRow];                          // X transposed [p][s]
  float dl[kQ], la[kQ], w[kQ];                      // Δ_s, la_s (log2 units), w_s
  float4 xch[4][4][64];                             // (d) partial sums for the partner wave
};

// The chunk loop of one wave; HB (the wave's state half and output t-tile) is a template argument so that
// every register array is indexed by constants.
template <typename Tout, int N, bool kGate, int HB>
__device__ __forceinline__ void ssd_wave(const SsdParams& p, Smem<N>& sm, int s, int h, int64_t t0, int32_t len) {
  constexpr int kRow = Smem<N>::kRow;
  constexpr int NTW = N / 64;             // state n-tiles per wave
  constexpr int NPR = N / 8;              // 16-byte pieces per B / C row
  constexpr int RPL = N / 32;             // B rows per lane (transposed staging), C pieces per lane
  const int tid = threadIdx.x;
  const int lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int a = wave & 1;
  const int H = p.heads;
  const int g = h / (H / p.ngroups);
  const int p_own = 32 * a + l32;         // this lane's column of the state and of Yᵀ

  const float A2 = p.A[h] * kLog2e;
  const float Dh = p.Dskip[h];
  const float bias = p.bias[h];

  // per-(sequence, head) views; rows past the sequence read as 0 and are not written
  const uint32_t rowx = static_cast<uint32_t>(H) * kP * 2;          // bytes per token of x, z (bf16)
  const uint32_t rowbc = static_cast<uint32_t>(p.ngroups) * N * 2;  // bytes per token of B, C
  const int64_t hx = static_cast<int64_t>(h) * kP;
  const rsrc_t rx = rsrc_bytes(static_cast<const uint16_t*>(p.x) + t0 * H * kP + hx,
                               (static_cast<int64_t>(len) * H * kP - hx) * 2);
  const rsrc_t rz = kGate ? rsrc_bytes(static_cast<const uint16_t*>(p.z) + t0 * H * kP + hx,
                                       (static_cast<int64_t>(len) * H * kP - hx) * 2)
                          : rsrc_bytes(nullptr, 0);
  const rsrc_t ry = rsrc_bytes(static_cast<Tout*>(p.y) + t0 * H * kP + hx,
                               (static_cast<int64_t>(len) * H * kP - hx) * static_cast<int64_t>(sizeof(Tout)));
  const rsrc_t rdt = rsrc_bytes(static_cast<const uint16_t*>(p.dt) + t0 * H + h,
                                (static_cast<int64_t>(len) * H - h) * 2);
  const int64_t gb = static_cast<int64_t>(g) * N;
  const int64_t bcb = (static_cast<int64_t>(len) * p.ngroups * N - gb) * 2;
  const rsrc_t rb = rsrc_bytes(static_cast<const uint16_t*>(p.B) + t0 * p.ngroups * N + gb, bcb);
  const rsrc_t rc = rsrc_bytes(static_cast<const uint16_t*>(p.C) + t0 * p.ngroups * N + gb, bcb);

  // the state: NTW accumulator tiles Hᵀ[n][p], n-tile HB * NTW + i; element e is
  // n = 32 nt + 8 (e / 4) + 4 hi + e % 4, p = p_own
  f32x16_t hst[NTW];
  const int64_t st_off = ((static_cast<int64_t>(s) * H + h) * kP + p_own) * N;
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    const int nt = HB * NTW + i;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (p.h0) v = *reinterpret_cast<const float4*>(p.h0 + st_off + 32 * nt + 8 * q + 4 * hi);
      hst[i][4 * q] = v.x; hst[i][4 * q + 1] = v.y; hst[i][4 * q + 2] = v.z; hst[i][4 * q + 3] = v.w;
    }
  }

  // staging assignment: C pieces (row-major), B rows (RPL consecutive rows, one 8-column run), X rows
  const int bcol = 8 * (tid % NPR), brow = RPL * (tid / NPR);
  const int xcol = 8 * (tid % 8), xrow = 2 * (tid / 8);
  uint4 cr[RPL], br[RPL], xr[2];
  uint16_t dtr = 0;
  auto load_chunk = [&](int c0) {
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int id = i * 256 + tid;
      cr[i] = ld16(rc, static_cast<uint32_t>(c0 + id / NPR) * rowbc + (id % NPR) * 16);
      br[i] = ld16(rb, static_cast<uint32_t>(c0 + brow + i) * rowbc + bcol * 2);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) xr[i] = ld16(rx, static_cast<uint32_t>(c0 + xrow + i) * rowx + xcol * 2);
    if (wave == 0) dtr = __builtin_amdgcn_raw_buffer_load_b16(rdt, static_cast<uint32_t>(c0 + lane) * H * 2, 0, 0);
  };

  const int nchunks = (len + kQ - 1) / kQ;
  if (nchunks > 0) load_chunk(0);
  for (int c = 0; c < nchunks; ++c) {
    const int c0 = c * kQ;
    __syncthreads();   // every wave is done with the previous chunk's LDS
#pragma unroll
    for (int i = 0; i < RPL; ++i) {
      const int id = i * 256 + tid;
      *reinterpret_cast<uint4*>(&sm.c[(id / NPR) * kRow + (id % NPR) * 8]) = cr[i];
      *reinterpret_cast<uint4*>(&sm.b[(brow + i) * kRow + bcol]) = br[i];
    }
    // B transposed: column n = bcol + j, rows brow .. brow + RPL - 1
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      uint32_t v[RPL / 2];
#pragma unroll
      for (int r = 0; r < RPL / 2; ++r) {
        const uint32_t w0 = word(br[2 * r], j / 2), w1 = word(br[2 * r + 1], j / 2);
        v[r] = (j & 1) ? highs(w0, w1) : lows(w0, w1);
      }
      uint16_t* dst = &sm.bt[(bcol + j) * kTRow + brow];
      if constexpr (RPL == 4) *reinterpret_cast<u32x2_t*>(dst) = u32x2_t{v[0], v[1]};
      else *reinterpret_cast<uint32_t*>(dst) = v[0];
    }
    // X transposed: column p = xcol + j, rows xrow, xrow + 1
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w0 = word(xr[0], j / 2), w1 = word(xr[1], j / 2);
      *reinterpret_cast<uint32_t*>(&sm.xt[(xcol + j) * kTRow + xrow]) = (j & 1) ? highs(w0, w1) : lows(w0, w1);
    }
    if (wave == 0) {
      // Δ, la (inclusive prefix sum of Δ A log2e over the chunk) and w = 2^(la_end - la) Δ; tokens past the
      // sequence get Δ = 0 (no decay, no input)
      const float dlt = c0 + lane < len ? softplus_f32(widen(dtr) + bias) : 0.0f;
      float la = dlt * A2;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float v = __shfl_up(la, off, 64);
        la = lane >= off ? la + v : la;
      }
      const float la_end = __shfl(la, 63, 64);
      sm.dl[lane] = dlt;
      sm.la[lane] = la;
      sm.w[lane] = __builtin_amdgcn_exp2f(la_end - la) * dlt;
    }
    __syncthreads();
    if (c + 1 < nchunks) load_chunk(c0 + kQ);

    // z of this chunk for the output tile (p-tile a, t-tile HB): 4 runs of 4 columns
    u32x2_t zr[4];
    const int t_own = 32 * HB + l32;
    if constexpr (kGate) {
#pragma unroll
      for (int q = 0; q < 4; ++q)
        zr[q] = __builtin_amdgcn_raw_buffer_load_b64(rz, static_cast<uint32_t>(c0 + t_own) * rowx +
                                                             (32 * a + 8 * q + 4 * hi) * 2, 0, 0);
    }

    // (d) partial sums over this wave's states, both t-tiles, from the entering state
    f32x16_t yo[2];
    yo[0] = f32x16_t{};
    yo[1] = f32x16_t{};
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      const int nt = HB * NTW + i;
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8_t hh, hl;
        split8(hst[i], 8 * kk, hh, hl);
        const int n0 = 32 * nt + 16 * kk + 4 * hi;
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          const uint16_t* row = &sm.c[(32 * tb + l32) * kRow];
          const bf16x8_t cop = cat4(row + n0, row + n0 + 8);
          yo[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hh, cop, yo[tb], 0, 0, 0);
          yo[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hl, cop, yo[tb], 0, 0, 0);
        }
      }
    }
    // the other t-tile's partial goes to the partner wave (same p-tile, other state half)
#pragma unroll
    for (int q = 0; q < 4; ++q)
      sm.xch[wave][q][lane] = make_float4(yo[1 - HB][4 * q], yo[1 - HB][4 * q + 1], yo[1 - HB][4 * q + 2],
                                          yo[1 - HB][4 * q + 3]);

    // (a) Sᵀ tiles (s-tile si, t-tile HB) for si <= HB, then (b) M as bf16 hi + lo operands
    f32x16_t sacc[HB + 1];
#pragma unroll
    for (int si = 0; si <= HB; ++si) sacc[si] = f32x16_t{};
#pragma unroll
    for (int kk = 0; kk < N / 16; ++kk) {
      const bf16x8_t cop = *reinterpret_cast<const bf16x8_t*>(&sm.c[t_own * kRow + 16 * kk + 8 * hi]);
#pragma unroll
      for (int si = 0; si <= HB; ++si) {
        const bf16x8_t bop = *reinterpret_cast<const bf16x8_t*>(&sm.b[(32 * si + l32) * kRow + 16 * kk + 8 * hi]);
        sacc[si] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bop, cop, sacc[si], 0, 0, 0);
      }
    }
    const float la_t = sm.la[t_own];
    f32x16_t yd = f32x16_t{};
#pragma unroll
    for (int si = 0; si <= HB; ++si) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int s0 = 32 * si + 8 * q + 4 * hi;
        const float4 las = *reinterpret_cast<const float4*>(&sm.la[s0]);
        const float4 dls = *reinterpret_cast<const float4*>(&sm.dl[s0]);
        const float lv[4] = {las.x, las.y, las.z, las.w}, dv[4] = {dls.x, dls.y, dls.z, dls.w};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sv = s0 + r;
          float m = sv <= t_own ? sacc[si][4 * q + r] * __builtin_amdgcn_exp2f(la_t - lv[r]) * dv[r] : 0.0f;
          m += sv == t_own ? Dh : 0.0f;
          sacc[si][4 * q + r] = m;
        }
      }
      // (c) Yᵀ += X M over this s-tile (X read in the accumulator's s order)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8_t mh, ml;
        split8(sacc[si], 8 * kk, mh, ml);
        const uint16_t* row = &sm.xt[p_own * kTRow + 32 * si + 16 * kk + 4 * hi];
        const bf16x8_t xop = cat4(row, row + 8);
        yd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xop, mh, yd, 0, 0, 0);
        yd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xop, ml, yd, 0, 0, 0);
      }
    }

    // (e) the state update: Hᵀ = 2^(la_end) Hᵀ + Bᵀ (w X), w X as a bf16 hi + lo pair
    const float decay = __builtin_amdgcn_exp2f(sm.la[kQ - 1]);
#pragma unroll
    for (int i = 0; i < NTW; ++i) hst[i] *= decay;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int s0 = 16 * kk + 8 * hi;
      const bf16x8_t xv = *reinterpret_cast<const bf16x8_t*>(&sm.xt[p_own * kTRow + s0]);
      const float4 w0 = *reinterpret_cast<const float4*>(&sm.w[s0]);
      const float4 w1 = *reinterpret_cast<const float4*>(&sm.w[s0 + 4]);
      const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
      bf16x8_t xh, xl;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float v = static_cast<float>(xv[j]) * wv[j];
        const __bf16 hv = static_cast<__bf16>(v);
        xh[j] = hv;
        xl[j] = static_cast<__bf16>(v - static_cast<float>(hv));
      }
#pragma unroll
      for (int i = 0; i < NTW; ++i) {
        const int nt = HB * NTW + i;
        const bf16x8_t bop = *reinterpret_cast<const bf16x8_t*>(&sm.bt[(32 * nt + l32) * kTRow + s0]);
        hst[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bop, xh, hst[i], 0, 0, 0);
        hst[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bop, xl, hst[i], 0, 0, 0);
      }
    }

    __syncthreads();   // the partner's partial sums are in LDS
    const float eo = __builtin_amdgcn_exp2f(la_t);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 o = sm.xch[wave ^ 2][q][lane];
      const float ov[4] = {o.x, o.y, o.z, o.w};
      float yv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) yv[r] = fmaf(eo, yo[HB][4 * q + r] + ov[r], yd[4 * q + r]);
      if constexpr (kGate) {
        const uint32_t zw[2] = {zr[q][0], zr[q][1]};
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const uint32_t zb = (r & 1) ? (zw[r / 2] & 0xffff0000u) : (zw[r / 2] << 16);
          yv[r] *= silu_f32(__uint_as_float(zb));
        }
      }
      const uint32_t off = static_cast<uint32_t>(c0 + t_own) * H * kP * sizeof(Tout) +
                           (32 * a + 8 * q + 4 * hi) * sizeof(Tout);
      if constexpr (sizeof(Tout) == 2) {
        const u32x2_t v = {static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(yv[0]))) |
                               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(yv[1]))) << 16),
                           static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(yv[2]))) |
                               (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(yv[3]))) << 16)};
        __builtin_amdgcn_raw_buffer_store_b64(v, ry, off, 0, 0);
      } else {
        const u32x4_t v = {__float_as_uint(yv[0]), __float_as_uint(yv[1]), __float_as_uint(yv[2]),
                           __float_as_uint(yv[3])};
        __builtin_amdgcn_raw_buffer_store_b128(v, ry, off, 0, 0);
      }
    }
  }

  if (p.h_last) {
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      const int nt = HB * NTW + i;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(p.h_last + st_off + 32 * nt + 8 * q + 4 * hi) =
            make_float4(hst[i][4 * q], hst[i][4 * q + 1], hst[i][4 * q + 2], hst[i][4 * q + 3]);
    }
  }
}

template <typename Tout, int N, bool kGate>
__global__ __launch_bounds__(256, 1) void ssd_fwd_kernel(SsdParams p) {
  __shared__ __attribute__((aligned(16))) Smem<N> sm;
  const int nblk = static_cast<int>(gridDim.x);
  const int logical = xcd_remap(static_cast<int>(blockIdx.x), nblk);
  const int s = logical / p.heads;
  const int h = logical - s * p.heads;
  int64_t t0;
  int32_t len;
  if (p.cu) {
    int32_t b = p.cu[s], e = p.cu[s + 1];
    b = b < 0 ? 0 : (b > p.total ? p.total : b);
    e = e < b ? b : (e > p.total ? p.total : e);
    t0 = b;
    len = e - b;
  } else {
    t0 = static_cast<int64_t>(s) * p.seqlen;
    len = p.seqlen;
  }
  const int hb = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 7);
  if (hb == 0) ssd_wave<Tout, N, kGate, 0>(p, sm, s, h, t0, len);
  else ssd_wave<Tout, N, kGate, 1>(p, sm, s, h, t0, len);
}

bool aligned(const void* q, uintptr_t a) { return (reinterpret_cast<uintptr_t>(q) & (a - 1)) == 0; }
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

template <typename Tout, int N>
hipError_t launch_ssd(const SsdParams& p, bool gate, dim3 grid, hipStream_t s) {
  const dim3 block(256);
  if (gate) hipLaunchKernelGGL((ssd_fwd_kernel<Tout, N, true>), grid, block, 0, s, p);
  else hipLaunchKernelGGL((ssd_fwd_kernel<Tout, N, false>), grid, block, 0, s, p);
  return hipGetLastError();
}

}  // namespace

extern "C" samba_status samba_ssd_fwd(const samba_ssd_args* a, void* stream) {
  if (!a) return SAMBA_ERR_NULL_ARG;
  if (a->struct_size != sizeof(samba_ssd_args)) return SAMBA_ERR_BAD_STRUCT;
  if (a->batch < 0 || a->seqlen < 0 || a->heads < 1 || a->ngroups < 1 || a->nseq < 0) return SAMBA_ERR_BAD_SHAPE;
  if (a->head_dim != kP || (a->dstate != 64 && a->dstate != 128)) return SAMBA_ERR_UNSUPPORTED;
  if (a->heads % a->ngroups != 0) return SAMBA_ERR_BAD_SHAPE;
  if (a->y_dtype != SAMBA_F32 && a->y_dtype != SAMBA_BF16) return SAMBA_ERR_BAD_DTYPE;
  int64_t nseq;
  if (a->cu_seqlens) {
    if (a->batch != 1 || a->nseq < 1) return SAMBA_ERR_BAD_SHAPE;
    nseq = a->nseq;
  } else {
    nseq = a->batch;
  }
  const int64_t tokens = static_cast<int64_t>(a->batch) * a->seqlen;
  if (nseq == 0) return SAMBA_OK;
  const int N = a->dstate;
  // 32-bit buffer offsets: a sequence's rows of y (fp32) and of B / C
  if (tokens * a->heads * kP * 4 >= (int64_t{1} << 32)) return SAMBA_ERR_BAD_SHAPE;
  if (tokens * a->ngroups * N * 2 >= (int64_t{1} << 32)) return SAMBA_ERR_BAD_SHAPE;
  if (nseq * a->heads > 0x7fffffff) return SAMBA_ERR_BAD_SHAPE;
  if (!a->A || !a->D || !a->dt_bias) return SAMBA_ERR_NULL_ARG;
  if (tokens > 0 && (!a->x || !a->dt || !a->B || !a->C || !a->y)) return SAMBA_ERR_NULL_ARG;
  const size_t oe = a->y_dtype == SAMBA_BF16 ? 2 : 4;
  if (!aligned(a->x, 16) || !aligned(a->B, 16) || !aligned(a->C, 16) || !aligned(a->h0, 16) ||
      !aligned(a->h_last, 16) || !aligned(a->z, 8) || !aligned(a->y, 4 * oe) || !aligned(a->dt, 2) ||
      !aligned(a->A, 4) || !aligned(a->D, 4) || !aligned(a->dt_bias, 4))
    return SAMBA_ERR_MISALIGNED;
  const size_t thp = static_cast<size_t>(tokens) * a->heads * kP;
  const size_t tbc = static_cast<size_t>(tokens) * a->ngroups * N * 2;
  const size_t st = static_cast<size_t>(nseq) * a->heads * kP * N * 4;
  const size_t hv = static_cast<size_t>(a->heads) * 4;
  const void* ins[11] = {a->x, a->dt, a->z, a->B, a->C, a->A, a->D, a->dt_bias, a->h0, a->cu_seqlens, nullptr};
  const size_t in_sz[11] = {thp * 2, static_cast<size_t>(tokens) * a->heads * 2, thp * 2, tbc, tbc, hv, hv, hv, st,
                            a->cu_seqlens ? (static_cast<size_t>(nseq) + 1) * 4 : 0, 0};
  for (int k = 0; k < 10; ++k) {
    if (overlap(a->y, thp * oe, ins[k], in_sz[k])) return SAMBA_ERR_ALIASING;
    if (a->h_last && !(k == 8 && a->h_last == a->h0) && overlap(a->h_last, st, ins[k], in_sz[k]))
      return SAMBA_ERR_ALIASING;
  }
  if (overlap(a->y, thp * oe, a->h_last, st)) return SAMBA_ERR_ALIASING;

  SsdParams p{};
  p.x = a->x; p.dt = a->dt; p.z = a->z; p.B = a->B; p.C = a->C;
  p.A = a->A; p.Dskip = a->D; p.bias = a->dt_bias; p.h0 = a->h0; p.h_last = a->h_last; p.y = a->y;
  p.cu = a->cu_seqlens;
  p.nseq = static_cast<int32_t>(nseq);
  p.seqlen = a->seqlen;
  p.heads = a->heads;
  p.ngroups = a->ngroups;
  p.total = a->seqlen;
  const dim3 grid(static_cast<uint32_t>(nseq * a->heads));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool gate = a->z != nullptr;
  hipError_t e;
  if (a->y_dtype == SAMBA_BF16)
    e = N == 64 ? launch_ssd<uint16_t, 64>(p, gate, grid, s) : launch_ssd<uint16_t, 128>(p, gate, grid, s);
  else
    e = N == 64 ? launch_ssd<float, 64>(p, gate, grid, s) : launch_ssd<float, 128>(p, gate, grid, s);
  return e == hipSuccess ? SAMBA_OK : SAMBA_ERR_HIP;
}
