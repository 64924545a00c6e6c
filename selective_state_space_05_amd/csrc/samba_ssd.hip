// samba_ssd.hip -- gfx950 (MI355X) prefill of the state-space duality layer (the Mamba-2 form that page
// "SAMBA混合注意力状态空间模型" compares Samba with, 与其他混合架构对比): a scalar decay per head and a
// head_dim x dstate state per head, so that a chunk of tokens is a handful of dense products.
//
// ssd_fwd_kernel: one workgroup (8 waves) per (sequence, head) walks the tokens in chunks of Q = 64, the
// fp32 state carried in registers from chunk to chunk.  The three nonzero 32x32 tiles of Sᵀ = B Cᵀ of each
// chunk are formed by the kernel's helper waves from B and C staged row-major in LDS (the default), or, in
// the pre-pass form, by ssd_cb_kernel once per (chunk, group) (the (B, C) of a group serve every head of
// the group) into the caller's workspace, each tile stored as the accumulator image its consumer loads (16
// floats per lane).  Both forms run the same MFMA sequence: bit for bit the same tiles.
// With la_t = log2e * A * sum_{r<=t} Δ_r inside the chunk, w_s = 2^(la_end - la_s) Δ_s and the entering
// state H (P x N), per chunk:
//   (b) Mᵀ[s][t] = Sᵀ[s][t] 2^(la_t - la_s) Δ_s  (s <= t, else 0), + D on the diagonal (the skip)
//   (c) Yᵀ[p][t] = sum_s X[s][p] Mᵀ[s][t]                      MFMA, K = Q
//   (d)         + 2^(la_t) sum_n H[p][n] C[t][n]               MFMA, K = N
//   (e) Hᵀ[n][p] = 2^(la_end) Hᵀ[n][p] + sum_s B[s][n] (w_s X[s][p])     MFMA, K = Q
//   y[t][p] = Yᵀ[p][t] * silu(z[t][p])
// The operands built here rather than read (M, H, w X) are split into bf16 hi + lo pairs, two MFMAs each:
// one bf16 rounding of them alone costs about 2e-3 of the output's scale, the pair about 1e-6.
//
// Roles (32x32 tiles, v_mfma_f32_32x32x16_bf16, two waves per SIMD):
//   * state waves 0 .. 3: wave k holds p-tile a = k & 1 of the state for half hb = k >> 1 of the n-tiles
//     as Hᵀ accumulators and finishes the output tile (p-tile a, t-tile hb): the partner's partial sums,
//     the gate (z loaded one chunk ahead in the wave's own layout) and the store.  Products are laid out so
//     that one product's accumulators are the next one's operand: Sᵀ's accumulator rows s are the
//     contraction index of (c) (a lane's 8 elements of a 16-wide step are s = 16kk + 8(j/4) + 4hi + j%4,
//     and X is read from LDS in that order), and the Hᵀ accumulators (lane = column p) are (d)'s A operand
//     the same way, with C read in the matching n order.  (d) over a wave's half of the states gives
//     partial sums for both t-tiles; the other t-tile's goes to the partner wave through LDS;
//   * helper waves 4 .. 7 load C, B, X and Δ through a ring of two register sets (every load instruction
//     reads whole 128-byte row segments) and stage them into LDS (C row-major; B and X transposed into
//     tiles whose 16-byte token groups are permuted by row, so that both the transposing stores and the
//     state waves' operand reads are free of bank conflicts); helper 0 computes Δ, la and w with a DPP
//     prefix sum, and three helpers build the chunk's masked M tiles (in the default form between the two
//     barriers of the chunk before, once every helper has staged B and C, each from its own Sᵀ tile formed
//     on the matrix cores).
//     (z and y in the state waves' layout are 8-byte pieces of 32 rows per instruction; staging y through
//     LDS for whole-line stores by the helpers measured no faster.)
// The inputs are staged in two alternating LDS buffers, so the helpers fill chunk c + 1's while the state
// waves compute chunk c: two barriers per chunk (partial sums exchanged; chunk done and next one staged).
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <mutex>
#include <type_traits>

#include "samba_ssd.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
using rsrc_t = __amdgpu_buffer_rsrc_t;

constexpr int kRsrcWord3 = 0x00020000;   // raw (untyped, unswizzled) buffer
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kQ = 64;                   // tokens per chunk
constexpr int kP = 64;                   // head size
constexpr int kTRow = kQ + 8;            // row stride (bf16) of the transposed tiles in LDS
// a buffer offset past every resource here (a sequence's rows of any tensor span less than 2^31 bytes):
// accesses at it read 0 and write nothing
constexpr uint32_t kNowhere = 0x80000000u;

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

// Position (bf16 units) of token s in row `row` of a transposed tile (B as [n][s], X as [p][s]): the row's
// eight 16-byte groups of tokens are XOR-permuted by bits 4-5 of the row index.  The helpers write a token pair
// of eight rows per lane group (their loads read whole rows of B and X), the state waves read eight tokens of
// one row per lane (consecutive rows across lanes); with the permutation both are free of bank conflicts on
// the 64 four-byte banks, and a group stays whole, so the operand reads stay single 16-byte reads.
__device__ __forceinline__ int tpos(int row, int s) {
  return row * kTRow + 8 * ((s >> 3) ^ (2 * ((row >> 4) & 3))) + (s & 7);
}

// two 4-element runs of a bf16 row as one 8-element operand
__device__ __forceinline__ bf16x8_t cat4(const uint16_t* p0, const uint16_t* p1) {
  const bf16x4_t u = *reinterpret_cast<const bf16x4_t*>(p0);
  const bf16x4_t v = *reinterpret_cast<const bf16x4_t*>(p1);
  return __builtin_shufflevector(u, v, 0, 1, 2, 3, 4, 5, 6, 7);
}

// a and b rounded to bf16 (to nearest even) by one paired conversion, a in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
// bf16 hi + lo of a and b: hi = bf16(v), lo = bf16(v - hi), each a packed pair (one conversion per pair)
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}

// the 8 accumulator elements e0 .. e0 + 7 as a bf16 hi + lo pair
__device__ __forceinline__ void split8(const f32x16_t& acc, int e0, bf16x8_t& hi, bf16x8_t& lo) {
  uint32_t h[4], l[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) split2(acc[e0 + 2 * j], acc[e0 + 2 * j + 1], h[j], l[j]);
  hi = __builtin_bit_cast(bf16x8_t, u32x4_t{h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(bf16x8_t, u32x4_t{l[0], l[1], l[2], l[3]});
}

struct SsdParams {
  const void *x, *dt, *z, *B, *C;
  const float *A, *Dskip, *bias, *h0;
  float* h_last;
  void* y;
  float* ws;                                        // Sᵀ tile images [slot][group][3][64][16]
  const int32_t* cu;
  int32_t nseq, seqlen, heads, ngroups, total, nch;   // nch: chunks per batched sequence
};

constexpr int kWaves = 8;                // 4 state waves + 4 helper waves
constexpr int kThreads = 64 * kWaves;
constexpr int kTileFloats = 64 * 16;     // one 32x32 accumulator image
constexpr bool kCbInAuto = true;         // SAMBA_SSD_CB_AUTO: C Bᵀ inside the prefill kernel

__device__ __forceinline__ int32_t cu_at(const int32_t* cu, int s, int32_t total) {
  const int32_t v = cu[s];
  return v < 0 ? 0 : (v > total ? total : v);
}
// (first token, length) of sequence s and the workspace slot of its first chunk: batched sequences own nch
// slots each; packed sequence s owns slots (cu[s] >> 6) + s .. (these ranges never overlap and all lie below
// (total >> 6) + nseq)
struct SeqInfo {
  int64_t t0;
  int32_t len, slot0;
};
__device__ __forceinline__ SeqInfo seq_info(const SsdParams& p, int s) {
  SeqInfo r;
  if (p.cu) {
    const int32_t b = cu_at(p.cu, s, p.total), e0 = cu_at(p.cu, s + 1, p.total);
    const int32_t e = e0 < b ? b : e0;
    r.t0 = b;
    r.len = e - b;
    r.slot0 = (b >> 6) + s;
  } else {
    r.t0 = static_cast<int64_t>(s) * p.seqlen;
    r.len = p.seqlen;
    r.slot0 = s * p.nch;
  }
  return r;
}

// Sᵀ tiles (s-tile, t-tile) = (0, 0), (0, 1), (1, 1) of one (chunk, group): one wave per tile, operands read
// straight from B and C (rows past the sequence read as 0).  Block b is (slot b / G, group b % G); slots of
// no chunk (between packed sequences) return at once.
template <int N>
__global__ __launch_bounds__(192) void ssd_cb_kernel(SsdParams p) {
  const int G = p.ngroups;
  const int slot = static_cast<int>(blockIdx.x) / G, g = static_cast<int>(blockIdx.x) - slot * G;
  int s, c;
  if (p.cu) {
    // the last sequence whose first slot is <= slot (first slots ascend with s)
    int lo = 0, hi = p.nseq;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((cu_at(p.cu, mid, p.total) >> 6) + mid <= slot) lo = mid;
      else hi = mid;
    }
    s = lo;
  } else {
    s = slot / p.nch;
  }
  const SeqInfo si = seq_info(p, s);
  c = slot - si.slot0;
  if (c < 0 || c * kQ >= si.len) return;
  const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
  const int tile = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int m_si = tile == 2 ? 1 : 0, m_tb = tile == 0 ? 0 : 1;
  const uint32_t rowbc = static_cast<uint32_t>(G) * N * 2;
  const int64_t gb = static_cast<int64_t>(g) * N;
  const int64_t bcb = (static_cast<int64_t>(si.len) * G * N - gb) * 2;
  const rsrc_t rb = rsrc_bytes(static_cast<const uint16_t*>(p.B) + si.t0 * G * N + gb, bcb);
  const rsrc_t rc = rsrc_bytes(static_cast<const uint16_t*>(p.C) + si.t0 * G * N + gb, bcb);
  const uint32_t ob = static_cast<uint32_t>(c * kQ + 32 * m_si + l32) * rowbc + 16 * hi;
  const uint32_t oc = static_cast<uint32_t>(c * kQ + 32 * m_tb + l32) * rowbc + 16 * hi;
  uint4 bv[N / 16], cv[N / 16];
#pragma unroll
  for (int kk = 0; kk < N / 16; ++kk) {
    bv[kk] = ld16(rb, ob + 32 * kk);
    cv[kk] = ld16(rc, oc + 32 * kk);
  }
  f32x16_t acc = f32x16_t{};
#pragma unroll
  for (int kk = 0; kk < N / 16; ++kk)
    acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, bv[kk]),
                                                  __builtin_bit_cast(bf16x8_t, cv[kk]), acc, 0, 0, 0);
  float4* dst = reinterpret_cast<float4*>(p.ws + ((static_cast<int64_t>(slot) * G + g) * 3 + tile) * kTileFloats) +
                lane * 4;
#pragma unroll
  for (int q = 0; q < 4; ++q) dst[q] = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
}

// One chunk's staged inputs and its M tiles; two of them alternate between consecutive chunks.
template <int N>
struct Stage {
  static constexpr int kRow = N + 8;                // row stride (bf16) of C
  uint16_t c[kQ * kRow];                            // C [t][n]
  uint16_t bt[N * kTRow];                           // B transposed [n][s]
  uint16_t xt[kP * kTRow];                          // X transposed [p][s]
  bf16x8_t m[3][2][2][64];                          // M tiles (0,0), (0,1), (1,1): [tile][kk][hi/lo][lane]
  float dl[kQ], la[kQ], w[kQ];                      // Δ_s, la_s (log2 units), w_s
};
template <int N>
struct Smem {
  Stage<N> st[2];                                   // chunk c uses st[c & 1]
  uint16_t brm[kQ * Stage<N>::kRow];                // B [s][n] of the chunk being prepared (C Bᵀ in kernel)
  float4 xch[4][4][64];                             // (d) partial sums for the partner wave
  float hs[4][2][kQ];                               // (pre-pass form) each helper's own la, Δ of its chunk
};

// Per-workgroup views of one (sequence, head): rows past the sequence read as 0 and are not written.
struct Ctx {
  rsrc_t rx, rz, ry, rdt, rb, rc;
  uint32_t rowx, rowbc;                             // bytes per token of x (bf16) and of B, C
  int64_t st_off0;                                  // offset of this (sequence, head)'s state
  const float* ws;                                  // this group's first chunk's tiles
  int64_t ws_stride;                                // floats from one chunk's tiles to the next's
  int32_t len, H;
  float A2, Dh, bias;
};

template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_or0(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, true));
}
// inclusive prefix sum over the 64 lanes: shifts within rows of 16, then the row totals carried forward
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += dpp_or0<0x111, 0xF>(v);   // row_shr:1
  v += dpp_or0<0x112, 0xF>(v);   // row_shr:2
  v += dpp_or0<0x114, 0xF>(v);   // row_shr:4
  v += dpp_or0<0x118, 0xF>(v);   // row_shr:8
  v += dpp_or0<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v += dpp_or0<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}

__device__ __forceinline__ float uniform(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Helper waves (h = 0 .. 3).  While the state waves compute chunk c, the helpers
//   1. stage chunk c + 1 (loaded two chunks earlier into a ring of two register sets) into its LDS stage:
//      C as row-major pieces, B and X transposed (each lane holds a 16-byte piece of two consecutive rows
//      and stores token pairs; eight lanes read one 128-byte row segment, so the loads are whole cache
//      lines, and the transposed rows are permuted by tpos so the stores are free of bank conflicts); helper
//      0 computes Δ, la and w of the chunk with a DPP prefix sum and publishes them (in the pre-pass form
//      helpers 1 .. 2 compute their own copy for step 2, which comes before the barrier);
//   2. helpers 0 .. 2 turn the chunk's Sᵀ tile h into M = Sᵀ 2^(la_t - la_s) Δ_s (s <= t), + D on the
//      diagonal, published as bf16 hi + lo operand images.  In the pre-pass form the tile was loaded from
//      the workspace two chunks earlier and M is built right away; by default (kCbIn) every helper also
//      stages B row-major, and after the next barrier (once all of B and C are staged) helpers 0 .. 2 form
//      their tiles on the matrix cores from LDS and build M;
//   3. load chunk c + 3 (and, in the pre-pass form, its workspace tile).
template <int N, bool kCbIn>
__device__ __forceinline__ void helper_wave(const Ctx& cx, Smem<N>& sm) {
  constexpr int kRow = Stage<N>::kRow;
  constexpr int NPR = N / 8;              // 16-byte pieces per C row
  constexpr int PC = N / 32;              // C pieces per helper thread
  constexpr int NB = N / 64;              // B passes (16-byte pieces pc + 8 i of a row)
  const int t = static_cast<int>(threadIdx.x) - 256;
  const int lane = t & 63, l32 = lane & 31, hi = lane >> 5;
  const int hw = __builtin_amdgcn_readfirstlane(t >> 6);   // helper index
  // B and X loads: token pair rr (rows 2 rr, 2 rr + 1), 16-byte piece pc; one load instruction reads eight whole
  // 128-byte row segments
  const int rr = 8 * hw + (lane >> 3), pc = lane & 7;
  // M tile of this helper: (s-tile, t-tile) = (0, 0), (0, 1), (1, 1); helper 3 has none
  const int m_si = hw == 2 ? 1 : 0, m_tb = hw == 0 ? 0 : 1;
  const int tile = hw < 3 ? hw : 2;       // (helper 3 loads a tile it does not use: no branch around loads)
  struct Set {
    uint4 cr[PC], br[NB][2], xr[2];
    uint16_t dtr;
  } set[2];
  f32x16_t sring[2];                      // Sᵀ tiles two chunks ahead (from the workspace)
  const int nchunks = (cx.len + kQ - 1) / kQ;
  auto load = [&](auto kset, int c) {
    Set& st = set[decltype(kset)::value];
    const int c0 = c * kQ;
#pragma unroll
    for (int i = 0; i < PC; ++i) {
      const int id = i * 256 + t;
      st.cr[i] = ld16(cx.rc, static_cast<uint32_t>(c0 + id / NPR) * cx.rowbc + (id % NPR) * 16);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int k = 0; k < 2; ++k)
        st.br[i][k] = ld16(cx.rb, static_cast<uint32_t>(c0 + 2 * rr + k) * cx.rowbc + (pc + 8 * i) * 16);
#pragma unroll
    for (int k = 0; k < 2; ++k)
      st.xr[k] = ld16(cx.rx, static_cast<uint32_t>(c0 + 2 * rr + k) * cx.rowx + pc * 16);
    // Δ: with C Bᵀ formed here only helper 0 needs it (the others read its la and Δ from the stage after the
    // next barrier) and the others read one row
    const int dtok = (kCbIn && hw != 0) ? 0 : lane;
    st.dtr = __builtin_amdgcn_raw_buffer_load_b16(cx.rdt, static_cast<uint32_t>(c0 + dtok) * cx.H * 2, 0, 0);
    if constexpr (!kCbIn) {
      // the chunk's Sᵀ tile (the last chunk's past the sequence: a padding chunk's M is the skip alone)
      const int cs = c < nchunks ? c : nchunks - 1;
      const float4* q = reinterpret_cast<const float4*>(cx.ws + cs * cx.ws_stride + tile * kTileFloats) + lane * 4;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const float4 v = q[k];
        sring[decltype(kset)::value][4 * k] = v.x;
        sring[decltype(kset)::value][4 * k + 1] = v.y;
        sring[decltype(kset)::value][4 * k + 2] = v.z;
        sring[decltype(kset)::value][4 * k + 3] = v.w;
      }
    }
  };
  // M = Sᵀ 2^(la_t - la_s) Δ_s (s <= t), + D on the diagonal, from the helper's Sᵀ tile and the chunk's la
  // and Δ, published as bf16 hi + lo operand images.  The la and Δ values are read into
  // registers first (before the product that feeds M, when it is formed here) and the causal mask is a
  // select, so that no LDS read waits inside the mask.
  struct Decay {
    float la_t;
    float4 las[4], dls[4];
  };
  // (la and Δ: helper 0's, in the stage, when C Bᵀ is formed after the barrier; the helper's own otherwise)
  auto load_decay = [&](const Stage<N>& g) {
    const float* la = kCbIn ? g.la : sm.hs[hw][0];
    const float* dl = kCbIn ? g.dl : sm.hs[hw][1];
    Decay d;
    d.la_t = la[32 * m_tb + l32];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int s0 = 32 * m_si + 8 * q + 4 * hi;
      d.las[q] = *reinterpret_cast<const float4*>(&la[s0]);
      d.dls[q] = *reinterpret_cast<const float4*>(&dl[s0]);
    }
    return d;
  };
  auto build_m = [&](Stage<N>& g, f32x16_t m, const Decay& d) {
    const int t_own = 32 * m_tb + l32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int s0 = 32 * m_si + 8 * q + 4 * hi;
      const float lv[4] = {d.las[q].x, d.las[q].y, d.las[q].z, d.las[q].w};
      const float dv[4] = {d.dls[q].x, d.dls[q].y, d.dls[q].z, d.dls[q].w};
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int sv = s0 + rr;
        const float e = __builtin_amdgcn_exp2f(d.la_t - lv[rr]);   // (> 1 above the diagonal: masked)
        float v = sv <= t_own ? m[4 * q + rr] * e * dv[rr] : 0.0f;
        v += sv == t_own ? cx.Dh : 0.0f;
        m[4 * q + rr] = v;
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8_t mh, ml;
      split8(m, 8 * kk, mh, ml);
      g.m[hw][kk][0][lane] = mh;
      g.m[hw][kk][1][lane] = ml;
    }
  };
  auto prepare = [&](auto kset, int c) {
    constexpr int K = decltype(kset)::value;
    const Set& st = set[K];
    Stage<N>& g = sm.st[K];
    const int c0 = c * kQ;
#pragma unroll
    for (int i = 0; i < PC; ++i) {
      const int id = i * 256 + t;
      *reinterpret_cast<uint4*>(&g.c[(id / NPR) * kRow + (id % NPR) * 8]) = st.cr[i];
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const uint32_t w0 = word(st.br[i][0], j / 2), w1 = word(st.br[i][1], j / 2);
        *reinterpret_cast<uint32_t*>(&g.bt[tpos(8 * (pc + 8 * i) + j, 2 * rr)]) = (j & 1) ? highs(w0, w1) : lows(w0, w1);
      }
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t w0 = word(st.xr[0], j / 2), w1 = word(st.xr[1], j / 2);
      *reinterpret_cast<uint32_t*>(&g.xt[tpos(8 * pc + j, 2 * rr)]) = (j & 1) ? highs(w0, w1) : lows(w0, w1);
    }
    // Δ, la (inclusive prefix sum of Δ A log2e) and w = 2^(la_end - la) Δ; tokens past the sequence get
    // Δ = 0 (no decay, no input)
    float dlt = 0.0f, l = 0.0f;
    if (!kCbIn || hw == 0) {
      dlt = c0 + lane < cx.len ? softplus_f32(widen(st.dtr) + cx.bias) : 0.0f;
      l = wave_prefix_sum(dlt * cx.A2);
    }
    if (hw == 0) {
      const float l_end = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), 63));
      g.dl[lane] = dlt;
      g.la[lane] = l;
      g.w[lane] = __builtin_amdgcn_exp2f(l_end - l) * dlt;
    }
    if constexpr (kCbIn) {
      // B row-major as well, for the C Bᵀ tile that the helpers form after the next barrier
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int k = 0; k < 2; ++k)
          *reinterpret_cast<uint4*>(&sm.brm[(2 * rr + k) * kRow + 8 * (pc + 8 * i)]) = st.br[i][k];
    }
    if constexpr (!kCbIn) {
      if (hw < 3) {
        sm.hs[hw][0][lane] = l;
        sm.hs[hw][1][lane] = dlt;
        wave_sync();
        build_m(g, sring[K], load_decay(g));
      }
    }
  };
  // C Bᵀ formed here: the helper's tile of chunk c from B and C row-major in LDS (staged by all helpers
  // before the last barrier), the same MFMA sequence as the pre-pass kernel (bit for bit the same tile;
  // rows past the sequence were staged as 0: a padding chunk's M is the skip alone)
  auto form_m = [&](auto kset) {
    Stage<N>& g = sm.st[decltype(kset)::value];
    if (hw < 3) {
      const Decay d = load_decay(g);
      bf16x8_t bo[N / 16], co[N / 16];
#pragma unroll
      for (int kk = 0; kk < N / 16; ++kk) {
        bo[kk] = *reinterpret_cast<const bf16x8_t*>(&sm.brm[(32 * m_si + l32) * kRow + 8 * hi + 16 * kk]);
        co[kk] = *reinterpret_cast<const bf16x8_t*>(&g.c[(32 * m_tb + l32) * kRow + 8 * hi + 16 * kk]);
      }
      f32x16_t m = f32x16_t{};
#pragma unroll
      for (int kk = 0; kk < N / 16; ++kk) m = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bo[kk], co[kk], m, 0, 0, 0);
      build_m(g, m, d);
    }
  };
  // An even number of chunks (the state waves pad the same way; a chunk past the sequence reads zeros and
  // changes nothing), and no load or store behind a data-dependent branch inside the loop, so that the
  // compiler's wait counts keep the other register set's loads in flight.
  const int npad = (nchunks + 1) & ~1;
  // With C Bᵀ formed here, the M tiles of chunk c + 1 are built between the two barriers of chunk c (after
  // every helper has staged B and C of chunk c + 1, before the state waves need them), and those of chunk 0
  // behind one more barrier.
  if (nchunks > 0) {
    load(std::integral_constant<int, 0>{}, 0);
    load(std::integral_constant<int, 1>{}, 1);
    prepare(std::integral_constant<int, 0>{}, 0);
    load(std::integral_constant<int, 0>{}, 2);
  }
  if constexpr (kCbIn) {
    __syncthreads();   // chunk 0's B and C staged
    if (nchunks > 0) form_m(std::integral_constant<int, 0>{});
  }
  __syncthreads();   // chunk 0 staged
  auto body = [&](auto knext, int c) {
    prepare(knext, c + 1);
    load(knext, c + 3);
    __syncthreads();   // X1: the state waves' partial sums
    if constexpr (kCbIn) form_m(knext);
    __syncthreads();   // X2: chunk c computed, chunk c + 1 prepared
  };
  for (int c = 0; c < npad; c += 2) {
    body(std::integral_constant<int, 1>{}, c);
    body(std::integral_constant<int, 0>{}, c + 1);
  }
}

// State wave k (0 .. 3): p-tile a = k & 1, n-tiles of half HB = k >> 1 (element e of tile nt: n = 32 nt +
// 8 (e / 4) + 4 hi + e % 4, p = 32 a + lane % 32); finishes the output tile (a, HB): sums it with the
// partner's partial sums, applies the gate (z loaded one chunk ahead) and stores it.
template <typename Tout, int N, int HB, bool kGate, bool kCbIn>
__device__ __forceinline__ void state_wave(const Ctx& cx, Smem<N>& sm, const float* h0, float* h_last) {
  constexpr int NTW = N / 64;
  constexpr int kRow = Stage<N>::kRow;
  const int lane = threadIdx.x & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  const int a = wave & 1;
  const int p_own = 32 * a + l32;
  const int t_own = 32 * HB + l32;
  const int64_t st_off = cx.st_off0 + static_cast<int64_t>(p_own) * N;

  f32x16_t hst[NTW];
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    const int nt = HB * NTW + i;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (h0) v = *reinterpret_cast<const float4*>(h0 + st_off + 32 * nt + 8 * q + 4 * hi);
      hst[i][4 * q] = v.x; hst[i][4 * q + 1] = v.y; hst[i][4 * q + 2] = v.z; hst[i][4 * q + 3] = v.w;
    }
  }
  // an even number of chunks, as the helper waves run (a padding chunk has Δ = 0 and x = 0: it leaves the
  // state alone and its output goes past the sequence)
  const int npad = ((cx.len + kQ - 1) / kQ + 1) & ~1;
  if constexpr (kCbIn) __syncthreads();   // chunk 0's B and C staged (the helpers then form its M)
  __syncthreads();   // chunk 0 staged

  // z and y pieces of this lane: token t_own, channels 32 a + 8 q + 4 hi + 0..3 (q = 0..3); z of the next
  // chunk is loaded while this one computes (register set kbuf ^ 1)
  uint2 zr0[4], zr1[4];
  auto load_z = [&](int c, uint2 (&zr)[4]) {
    if constexpr (kGate) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const auto v = __builtin_amdgcn_raw_buffer_load_b64(
            cx.rz, static_cast<uint32_t>(c * kQ + t_own) * cx.rowx + (32 * a + 8 * q + 4 * hi) * 2, 0, 0);
        zr[q] = make_uint2(v[0], v[1]);
      }
    }
  };
  const uint32_t rowy = static_cast<uint32_t>(cx.H) * kP * sizeof(Tout);
  load_z(0, zr0);
  int cc = 0;   // the chunk being computed
  auto chunk = [&](auto kbuf) {
    constexpr int KB = decltype(kbuf)::value;
    const Stage<N>& g = sm.st[KB];
    if constexpr (KB == 0) load_z(cc + 1, zr1);
    else load_z(cc + 1, zr0);
    // operands of (d): C in the state accumulators' n order, both t-tiles; of (c): X in M's s order
    bf16x8_t cop[2][NTW][2], xop[HB + 1][2];
#pragma unroll
    for (int tb = 0; tb < 2; ++tb)
#pragma unroll
      for (int i = 0; i < NTW; ++i)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const uint16_t* row = &g.c[(32 * tb + l32) * kRow + 32 * (HB * NTW + i) + 16 * kk + 4 * hi];
          cop[tb][i][kk] = cat4(row, row + 8);
        }
#pragma unroll
    for (int si = 0; si <= HB; ++si)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int s = 32 * si + 16 * kk + 4 * hi;
        xop[si][kk] = cat4(&g.xt[tpos(p_own, s)], &g.xt[tpos(p_own, s + 8)]);
      }
    const float la_t = g.la[t_own];
    const float decay = __builtin_amdgcn_exp2f(g.la[kQ - 1]);

    // (d) partial sums over this wave's states, both t-tiles, from the entering state
    f32x16_t yo[2];
    yo[0] = f32x16_t{};
    yo[1] = f32x16_t{};
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        bf16x8_t hh, hl;
        split8(hst[i], 8 * kk, hh, hl);
#pragma unroll
        for (int tb = 0; tb < 2; ++tb) {
          yo[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hh, cop[tb][i][kk], yo[tb], 0, 0, 0);
          yo[tb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(hl, cop[tb][i][kk], yo[tb], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q)
      sm.xch[wave][q][lane] = make_float4(yo[1 - HB][4 * q], yo[1 - HB][4 * q + 1], yo[1 - HB][4 * q + 2],
                                          yo[1 - HB][4 * q + 3]);

    // (c) Yᵀ = X M over the s-tiles up to HB, M from the helpers' images
    f32x16_t yd = f32x16_t{};
#pragma unroll
    for (int si = 0; si <= HB; ++si)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        yd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xop[si][kk], g.m[si + HB][kk][0][lane], yd, 0, 0, 0);
        yd = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xop[si][kk], g.m[si + HB][kk][1][lane], yd, 0, 0, 0);
      }

    // (e) Hᵀ = 2^(la_end) Hᵀ + Bᵀ (w X), w X as a bf16 hi + lo pair.  It reads only this chunk's stage,
    // which stays valid until the second barrier.  Before the first barrier, except without a gate when the
    // helpers form the M tiles between the two: the ungated epilogue is short, and the state waves would
    // wait there for the helpers instead.
    auto update_state = [&]() {
#pragma unroll
      for (int i = 0; i < NTW; ++i) hst[i] *= decay;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int s0 = 16 * kk + 8 * hi;
        const bf16x8_t xv = *reinterpret_cast<const bf16x8_t*>(&g.xt[tpos(p_own, s0)]);
        const float4 w0 = *reinterpret_cast<const float4*>(&g.w[s0]);
        const float4 w1 = *reinterpret_cast<const float4*>(&g.w[s0 + 4]);
        const float wv[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        uint32_t xhw[4], xlw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j)
          split2(static_cast<float>(xv[2 * j]) * wv[2 * j], static_cast<float>(xv[2 * j + 1]) * wv[2 * j + 1], xhw[j],
                 xlw[j]);
        const bf16x8_t xh = __builtin_bit_cast(bf16x8_t, u32x4_t{xhw[0], xhw[1], xhw[2], xhw[3]});
        const bf16x8_t xl = __builtin_bit_cast(bf16x8_t, u32x4_t{xlw[0], xlw[1], xlw[2], xlw[3]});
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
          const bf16x8_t bop = *reinterpret_cast<const bf16x8_t*>(&g.bt[tpos(32 * (HB * NTW + i) + l32, s0)]);
          hst[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bop, xh, hst[i], 0, 0, 0);
          hst[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bop, xl, hst[i], 0, 0, 0);
        }
      }
    };
    constexpr bool kLate = !kGate && kCbIn;
    if constexpr (!kLate) update_state();

    __syncthreads();   // X1: the partner's partial sums are in LDS
    const float eo = __builtin_amdgcn_exp2f(la_t);
    const uint2* zr = KB == 0 ? zr0 : zr1;
    // (the stores of a padding chunk past the sequence fall outside the output resource)
    const uint32_t yrow = static_cast<uint32_t>(cc * kQ + t_own) * rowy;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float4 o = sm.xch[wave ^ 2][q][lane];
      float v[4] = {fmaf(eo, yo[HB][4 * q] + o.x, yd[4 * q]), fmaf(eo, yo[HB][4 * q + 1] + o.y, yd[4 * q + 1]),
                    fmaf(eo, yo[HB][4 * q + 2] + o.z, yd[4 * q + 2]), fmaf(eo, yo[HB][4 * q + 3] + o.w, yd[4 * q + 3])};
      if constexpr (kGate) {
        const uint32_t zw[2] = {zr[q].x, zr[q].y};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          v[j] *= silu_f32(__uint_as_float((j & 1) ? (zw[j >> 1] & 0xffff0000u) : (zw[j >> 1] << 16)));
      }
      const uint32_t off = yrow + (32 * a + 8 * q + 4 * hi) * static_cast<uint32_t>(sizeof(Tout));
      if constexpr (sizeof(Tout) == 2) {
        const u32x2_t w = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        __builtin_amdgcn_raw_buffer_store_b64(w, cx.ry, off, 0, 0);
      } else {
        const u32x4_t w = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
        __builtin_amdgcn_raw_buffer_store_b128(w, cx.ry, off, 0, 0);
      }
    }
    if constexpr (kLate) update_state();
    ++cc;
    __syncthreads();   // X2: chunk computed, the next chunk prepared
  };
  for (int c = 0; c < npad; c += 2) {
    chunk(std::integral_constant<int, 0>{});
    chunk(std::integral_constant<int, 1>{});
  }

  if (h_last) {
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
      const int nt = HB * NTW + i;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        *reinterpret_cast<float4*>(h_last + st_off + 32 * nt + 8 * q + 4 * hi) =
            make_float4(hst[i][4 * q], hst[i][4 * q + 1], hst[i][4 * q + 2], hst[i][4 * q + 3]);
    }
  }
}

// A state wave of the value tile that its workgroup leaves to the other one (kSplit): it only takes part in
// the barriers, as many as a computing state wave does.
template <bool kCbIn>
__device__ __forceinline__ void idle_state_wave(const Ctx& cx) {
  const int npad = ((cx.len + kQ - 1) / kQ + 1) & ~1;
  if constexpr (kCbIn) __syncthreads();   // chunk 0's B and C staged
  __syncthreads();   // chunk 0 staged
  for (int c = 0; c < npad; ++c) {
    __syncthreads();   // X1
    __syncthreads();   // X2
  }
}

// kSplit: the head's two 32-column value tiles go to two workgroups (when one workgroup per (sequence, head)
// would leave at least half of the CUs idle); both stage the chunk and build M, and each runs the state
// waves of its own tile.
template <typename Tout, int N, bool kGate, bool kSplit, bool kCbIn>
__global__ __launch_bounds__(kThreads, 1) void ssd_fwd_kernel(SsdParams p) {
  __shared__ __attribute__((aligned(16))) Smem<N> sm;
  const int nblk = static_cast<int>(gridDim.x);
  const int logical = xcd_remap(static_cast<int>(blockIdx.x), nblk);
  const int sh = kSplit ? (logical >> 1) : logical;   // (the two halves of a head are neighbours: same XCD)
  const int pa = kSplit ? (logical & 1) : 0;
  // (sequence, head) and the head's parameters through readfirstlane: scalar loads.  A per-lane load issued
  // before the chunk loop leaves the compiler unsure whether it is still in flight inside the loop, and it
  // then waits for every outstanding load (prefetches included) at each use.
  const int s = __builtin_amdgcn_readfirstlane(sh / p.heads);
  const int h = __builtin_amdgcn_readfirstlane(sh - s * p.heads);
  const SeqInfo si = seq_info(p, s);
  const int H = p.heads;
  const int G = p.ngroups;
  const int g = h / (H / G);
  Ctx cx;
  cx.len = si.len;
  cx.H = H;
  cx.A2 = uniform(p.A[h] * kLog2e);
  cx.Dh = uniform(p.Dskip[h]);
  cx.bias = uniform(p.bias[h]);
  cx.rowx = static_cast<uint32_t>(H) * kP * 2;
  cx.rowbc = static_cast<uint32_t>(G) * N * 2;
  const int64_t t0 = si.t0;
  const int64_t hx = static_cast<int64_t>(h) * kP;
  const int64_t xb = (static_cast<int64_t>(si.len) * H * kP - hx);
  cx.rx = rsrc_bytes(static_cast<const uint16_t*>(p.x) + t0 * H * kP + hx, xb * 2);
  cx.rz = kGate ? rsrc_bytes(static_cast<const uint16_t*>(p.z) + t0 * H * kP + hx, xb * 2) : rsrc_bytes(nullptr, 0);
  cx.ry = rsrc_bytes(static_cast<Tout*>(p.y) + t0 * H * kP + hx, xb * static_cast<int64_t>(sizeof(Tout)));
  cx.rdt = rsrc_bytes(static_cast<const uint16_t*>(p.dt) + t0 * H + h, (static_cast<int64_t>(si.len) * H - h) * 2);
  const int64_t gb = static_cast<int64_t>(g) * N;
  const int64_t bcb = (static_cast<int64_t>(si.len) * G * N - gb) * 2;
  cx.rb = rsrc_bytes(static_cast<const uint16_t*>(p.B) + t0 * G * N + gb, bcb);
  cx.rc = rsrc_bytes(static_cast<const uint16_t*>(p.C) + t0 * G * N + gb, bcb);
  cx.st_off0 = (static_cast<int64_t>(s) * H + h) * kP * N;
  cx.ws_stride = static_cast<int64_t>(G) * 3 * kTileFloats;
  cx.ws = kCbIn ? nullptr : p.ws + (static_cast<int64_t>(si.slot0) * G + g) * 3 * kTileFloats;

  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
  if (wave >= 4) helper_wave<N, kCbIn>(cx, sm);
  else if (kSplit && (wave & 1) != pa) idle_state_wave<kCbIn>(cx);
  else if (wave >= 2) state_wave<Tout, N, 1, kGate, kCbIn>(cx, sm, p.h0, p.h_last);
  else state_wave<Tout, N, 0, kGate, kCbIn>(cx, sm, p.h0, p.h_last);
}

bool aligned(const void* q, uintptr_t a) { return (reinterpret_cast<uintptr_t>(q) & (a - 1)) == 0; }
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

template <typename Tout, int N, bool kCbIn>
void launch_fwd(const SsdParams& p, bool gate, bool split, int64_t nblocks, hipStream_t s) {
  const dim3 grid(static_cast<uint32_t>(split ? 2 * nblocks : nblocks)), block(kThreads);
  if (gate) {
    if (split) hipLaunchKernelGGL((ssd_fwd_kernel<Tout, N, true, true, kCbIn>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((ssd_fwd_kernel<Tout, N, true, false, kCbIn>), grid, block, 0, s, p);
  } else {
    if (split) hipLaunchKernelGGL((ssd_fwd_kernel<Tout, N, false, true, kCbIn>), grid, block, 0, s, p);
    else hipLaunchKernelGGL((ssd_fwd_kernel<Tout, N, false, false, kCbIn>), grid, block, 0, s, p);
  }
}

// cb_in: C Bᵀ formed inside the prefill kernel (no pre-pass, no workspace)
template <typename Tout, int N>
hipError_t launch_ssd(const SsdParams& p, bool gate, bool split, bool cb_in, int64_t nslots, int64_t nblocks,
                      hipStream_t s) {
  if (cb_in) {
    launch_fwd<Tout, N, true>(p, gate, split, nblocks, s);
  } else {
    if (nslots > 0)
      hipLaunchKernelGGL((ssd_cb_kernel<N>), dim3(static_cast<uint32_t>(nslots * p.ngroups)), dim3(192), 0, s, p);
    launch_fwd<Tout, N, false>(p, gate, split, nblocks, s);
  }
  return hipGetLastError();
}

// compute units of the current device (256 when the runtime cannot tell)
int ssd_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return 256;
  }
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

// sequences, chunk slots and workspace bytes of a validated call
struct Plan {
  int64_t nseq, tokens, nch, nslots;
  bool cb_in;        // C Bᵀ inside the prefill kernel
  size_t ws_bytes;
};
samba_status plan_ssd(const samba_ssd_args* a, Plan* pl) {
  if (!a) return SAMBA_ERR_NULL_ARG;
  if (a->struct_size != sizeof(samba_ssd_args)) return SAMBA_ERR_BAD_STRUCT;
  if (a->batch < 0 || a->seqlen < 0 || a->heads < 1 || a->ngroups < 1 || a->nseq < 0) return SAMBA_ERR_BAD_SHAPE;
  if (a->head_dim != kP || (a->dstate != 64 && a->dstate != 128)) return SAMBA_ERR_UNSUPPORTED;
  if (a->heads % a->ngroups != 0) return SAMBA_ERR_BAD_SHAPE;
  if (a->y_dtype != SAMBA_F32 && a->y_dtype != SAMBA_BF16) return SAMBA_ERR_BAD_DTYPE;
  if (a->cu_seqlens) {
    if (a->batch != 1 || a->nseq < 1) return SAMBA_ERR_BAD_SHAPE;
    pl->nseq = a->nseq;
  } else {
    pl->nseq = a->batch;
  }
  pl->tokens = static_cast<int64_t>(a->batch) * a->seqlen;
  pl->nch = (static_cast<int64_t>(a->seqlen) + kQ - 1) / kQ;
  pl->nslots = a->cu_seqlens ? (pl->tokens >> 6) + pl->nseq : pl->nseq * pl->nch;
  const int N = a->dstate;
  // 32-bit buffer offsets: the kernels address up to two chunks past a sequence's end (reads of zeros,
  // dropped writes), so a sequence's rows of y (fp32) and of B / C stay below 2^31 bytes and 128 rows below
  // 2^31 bytes more, which keeps every such offset below 2^32 and kNowhere past every sequence
  if (a->heads > 65536) return SAMBA_ERR_BAD_SHAPE;
  if (pl->tokens * a->heads * kP * 4 >= (int64_t{1} << 31)) return SAMBA_ERR_BAD_SHAPE;
  if (pl->tokens * a->ngroups * N * 2 >= (int64_t{1} << 31)) return SAMBA_ERR_BAD_SHAPE;
  if (pl->nseq * a->heads > 0x7fffffff || pl->nslots * a->ngroups > 0x7fffffff) return SAMBA_ERR_BAD_SHAPE;
  if (a->cb_mode != SAMBA_SSD_CB_AUTO && a->cb_mode != SAMBA_SSD_CB_PREPASS && a->cb_mode != SAMBA_SSD_CB_IN_KERNEL)
    return SAMBA_ERR_UNSUPPORTED;
  pl->cb_in = a->cb_mode == SAMBA_SSD_CB_IN_KERNEL || (a->cb_mode == SAMBA_SSD_CB_AUTO && kCbInAuto);
  pl->ws_bytes = pl->tokens > 0 && !pl->cb_in ? static_cast<size_t>(pl->nslots) * a->ngroups * 3 * kTileFloats * 4 : 0;
  return SAMBA_OK;
}

}  // namespace

extern "C" samba_status samba_ssd_workspace_size(const samba_ssd_args* a, size_t* bytes) {
  if (!bytes) return SAMBA_ERR_NULL_ARG;
  Plan pl;
  const samba_status st = plan_ssd(a, &pl);
  if (st != SAMBA_OK) return st;
  *bytes = pl.nseq == 0 ? 0 : pl.ws_bytes;
  return SAMBA_OK;
}

namespace {

// Scratch of the no-allocation entry point: a file-scope device array, one copy per GPU, holding the
// C Bᵀ tiles that the pre-pass form of samba_ssd_fwd writes into the caller's workspace.  Host code never
// passes the array's name to a kernel (on the host it is a stand-in, not a device address): it uses the
// address that hipGetSymbolAddress returned for the device, kept per device below.
constexpr size_t kSsdScratchBytes = SAMBA_SSD_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kSsdScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
std::mutex g_scratch_mu;

// The scratch array's device address on the current device, looked up once per device (with that device
// current) and kept; nullptr if the lookup fails.
void* scratch_address() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_addr[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) {
      (void)hipGetLastError();
      return nullptr;
    }
    g_scratch_addr[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

// The prefill with the C Bᵀ tiles in `ws` (ws_bytes usable), which is either the caller's workspace
// (samba_ssd_fwd) or this device's scratch array (samba_ssd_fwd_noalloc).
samba_status ssd_fwd_impl(const samba_ssd_args* a, void* ws, size_t ws_bytes, bool caller_ws, void* stream) {
  Plan pl;
  const samba_status st0 = plan_ssd(a, &pl);
  if (st0 != SAMBA_OK) return st0;
  if (pl.nseq == 0) return SAMBA_OK;
  const int N = a->dstate;
  const int64_t tokens = pl.tokens;
  if (!a->A || !a->D || !a->dt_bias) return SAMBA_ERR_NULL_ARG;
  if (tokens > 0 && (!a->x || !a->dt || !a->B || !a->C || !a->y)) return SAMBA_ERR_NULL_ARG;
  const size_t oe = a->y_dtype == SAMBA_BF16 ? 2 : 4;
  if (!aligned(a->x, 16) || !aligned(a->B, 16) || !aligned(a->C, 16) || !aligned(a->h0, 16) ||
      !aligned(a->h_last, 16) || !aligned(a->z, 8) || !aligned(a->y, 4 * oe) || !aligned(a->dt, 2) ||
      !aligned(a->A, 4) || !aligned(a->D, 4) || !aligned(a->dt_bias, 4))
    return SAMBA_ERR_MISALIGNED;
  if (pl.ws_bytes > 0 && (!ws || ws_bytes < pl.ws_bytes || !aligned(ws, 256))) return SAMBA_ERR_WORKSPACE;
  const size_t thp = static_cast<size_t>(tokens) * a->heads * kP;
  const size_t tbc = static_cast<size_t>(tokens) * a->ngroups * N * 2;
  const size_t st = static_cast<size_t>(pl.nseq) * a->heads * kP * N * 4;
  const size_t hv = static_cast<size_t>(a->heads) * 4;
  const void* ins[11] = {a->x, a->dt, a->z, a->B, a->C, a->A, a->D, a->dt_bias, a->h0, a->cu_seqlens, nullptr};
  const size_t in_sz[11] = {thp * 2, static_cast<size_t>(tokens) * a->heads * 2, thp * 2, tbc, tbc, hv, hv, hv, st,
                            a->cu_seqlens ? (static_cast<size_t>(pl.nseq) + 1) * 4 : 0, 0};
  for (int k = 0; k < 10; ++k) {
    if (overlap(a->y, thp * oe, ins[k], in_sz[k])) return SAMBA_ERR_ALIASING;
    if (a->h_last && !(k == 8 && a->h_last == a->h0) && overlap(a->h_last, st, ins[k], in_sz[k]))
      return SAMBA_ERR_ALIASING;
    if (caller_ws && overlap(ws, pl.ws_bytes, ins[k], in_sz[k])) return SAMBA_ERR_ALIASING;
  }
  if (overlap(a->y, thp * oe, a->h_last, st)) return SAMBA_ERR_ALIASING;
  if (caller_ws && (overlap(ws, pl.ws_bytes, a->y, thp * oe) || overlap(ws, pl.ws_bytes, a->h_last, st)))
    return SAMBA_ERR_ALIASING;

  SsdParams p{};
  p.x = a->x; p.dt = a->dt; p.z = a->z; p.B = a->B; p.C = a->C;
  p.A = a->A; p.Dskip = a->D; p.bias = a->dt_bias; p.h0 = a->h0; p.h_last = a->h_last; p.y = a->y;
  p.ws = static_cast<float*>(ws);
  p.cu = a->cu_seqlens;
  p.nseq = static_cast<int32_t>(pl.nseq);
  p.seqlen = a->seqlen;
  p.heads = a->heads;
  p.ngroups = a->ngroups;
  p.total = a->seqlen;
  p.nch = static_cast<int32_t>(pl.nch);
  const hipStream_t s = static_cast<hipStream_t>(stream);
  const bool gate = a->z != nullptr;
  const int64_t nblocks = pl.nseq * a->heads;
  const int64_t nslots = tokens > 0 ? pl.nslots : 0;
  // value columns over two workgroups per head when that still fits the CUs in one round
  const bool split = nblocks > 0 && 2 * nblocks <= ssd_cu_count();
  hipError_t e;
  // (no tokens: no chunk, no workspace read; every sequence's h_last is its h0, or zero)
  if (a->y_dtype == SAMBA_BF16) {
    e = N == 64 ? launch_ssd<uint16_t, 64>(p, gate, split, pl.cb_in, nslots, nblocks, s)
                : launch_ssd<uint16_t, 128>(p, gate, split, pl.cb_in, nslots, nblocks, s);
  } else {
    e = N == 64 ? launch_ssd<float, 64>(p, gate, split, pl.cb_in, nslots, nblocks, s)
                : launch_ssd<float, 128>(p, gate, split, pl.cb_in, nslots, nblocks, s);
  }
  return e == hipSuccess ? SAMBA_OK : SAMBA_ERR_HIP;
}

}  // namespace

extern "C" samba_status samba_ssd_fwd(const samba_ssd_args* a, void* stream) {
  if (!a) return SAMBA_ERR_NULL_ARG;
  return ssd_fwd_impl(a, a->workspace, a->workspace_bytes, true, stream);
}

extern "C" samba_status samba_ssd_fwd_noalloc(const samba_ssd_args* a, void* stream) {
  Plan pl;
  const samba_status st = plan_ssd(a, &pl);
  if (st != SAMBA_OK) return st;
  if (pl.nseq == 0) return SAMBA_OK;
  if (pl.ws_bytes > kSsdScratchBytes) return SAMBA_ERR_WORKSPACE;   // beyond the static scratch: refused
  void* ws = nullptr;
  if (pl.ws_bytes > 0) {
    ws = scratch_address();
    if (!ws) return SAMBA_ERR_HIP;
  }
  return ssd_fwd_impl(a, ws, kSsdScratchBytes, false, stream);
}
