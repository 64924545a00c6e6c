// samba_gla.hip -- gfx950 (MI355X) gated linear attention (the GLA layer that the hackernoon page "Microsoft's
// Samba Model Redefines Long-Context Learning for AI", §2, names as a substitute for the Mamba layer): per
// head, S_t = diag(exp(gk_t)) S_{t-1} + k_tᵀ v_t, o_t = q_t S_t.  Two forms: the chunked form on the matrix
// cores (bf16 inputs, 128 or 256 keys, values a multiple of 32; see the chunked-form section below) and the
// recurrence (every other shape), which follows.
//
// The recurrence is a diagonal scan per (head, value column) over the key dimension.  A lane holds 4 keys of
// C value columns (N / 4 lanes cover the keys; C = N / 64 from 64 keys up, so a wave covers 4 columns and a
// workgroup of 4 waves 16 columns of one head), and tokens advance 16 at a time (8 below 64 keys).  The
// workgroup stages the chunk's k, q and the decay exp(gk) (once per (token, key)) and its columns' v into
// LDS, shared by its 4 waves; every lane runs the chunk's updates of its C x 4 states (one multiply and one
// FMA each) and keeps its partial readouts, C x kT of them; those are reduced over the N / 4 lanes of the
// keys by one reduce-scatter per chunk (v_permlane32_swap and v_permlane16_swap, then LDS swizzles and DPP),
// after which each lane holds the sum of exactly one (column, token).  Two barriers per chunk, no workspace;
// LDS 49 KiB at 256 keys, so three workgroups fit a CU.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <type_traits>

#include "samba_gla.h"

namespace {

using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // raw (untyped, unswizzled) buffer
constexpr float kLog2e = 1.4426950408889634f;
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

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
// the value of lane l ^ 4 (within rows of 16 lanes), from two row rotations (a rotation right by r gives lane
// l the value of lane l - r mod 16): no LDS round trip
__device__ __forceinline__ float xor4(float v, bool bit4) {
  const float from_below = dpp<0x124>(v), from_above = dpp<0x12C>(v);   // row_ror:4 (l - 4), row_ror:12 (l + 4)
  return bit4 ? from_below : from_above;
}
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

struct GlaParams {
  const void *q, *k, *gk, *v;
  const float* h0;
  float* h_last;
  void* o;
  const int32_t* cu;
  int32_t nseq, seqlen, heads, head_dim, dim, total;
  int32_t ntiles;   // channel tiles (4 waves' channels) per sequence; the grid is ntiles x nseq
};

// Block index -> logical index such that consecutive logical blocks land on the same XCD (the dispatcher
// deals blocks round-robin over the 8 XCDs).  A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7, xcd = bid & 7, slot = bid >> 3;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// one exchange step of the reduce-scatter: lanes whose bit M is set keep the upper half of each pair and
// receive the partner's upper half; the others keep the lower half
template <int M>
__device__ __forceinline__ float rs_step(float lo, float hi, bool upper) {
  if constexpr (M == 32) {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  } else if constexpr (M == 16) {
    const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
    return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  } else {
    const float send = upper ? lo : hi, keep = upper ? hi : lo;
    float got;
    if constexpr (M == 8) got = dpp<0x128>(send);        // row_ror:8 (lane l - 8 mod 16 = l ^ 8)
    else if constexpr (M == 4) got = xor4(send, upper);
    else if constexpr (M == 2) got = dpp<0x4E>(send);   // quad_perm [2,3,0,1]
    else got = dpp<0xB1>(send);                         // quad_perm [1,0,3,2]
    return keep + got;
  }
}

// The K partial sums of every lane, reduced over groups of LPC consecutive lanes: afterwards lane l holds
// K / LPC sums, those of partial indices r + (K / LPC) (l % LPC), r < K / LPC.
template <int LPC, int K>
__device__ __forceinline__ void reduce_scatter(float (&v)[K], int lane) {
  if constexpr (LPC > 1) {
    constexpr int M = LPC / 2, H = K / 2;
    const bool upper = (lane & M) != 0;
#pragma unroll
    for (int k = 0; k < H; ++k) v[k] = rs_step<M>(v[k], v[k + H], upper);
    float (&w)[H] = *reinterpret_cast<float (*)[H]>(&v[0]);
    reduce_scatter<M, H>(w, lane);
  }
}

// Chunk and lane shape per key size N: a lane holds 4 keys of C value columns; tokens advance kT at a time so
// that the C x kT partial readouts of a lane reduce to whole sums over the N / 4 lanes of the keys.
template <int N>
struct GlaShape {
  static constexpr int kT = N >= 64 ? 16 : 8;            // tokens per chunk
  static constexpr int LPC = N / 4;                      // lanes per column group
  static constexpr int GPW = 64 / LPC;                   // column groups per wave
  static constexpr int C = N >= 64 ? N / 64 : 1;         // value columns per lane
  static constexpr int CPW = GPW * C;                    // value columns per wave: 4 (8 at N = 32, 16 at 16)
  static constexpr int CPB = CPW * kWaves;               // value columns per workgroup
  static constexpr int K = C * kT;                       // partial readouts per lane per chunk
  static constexpr int R = K / LPC;                      // sums per lane after the reduction
  static constexpr int VPT = kT * N / 256 > 2 ? kT * N / 256 : 2;   // k, q, gk elements a staging thread moves
  static constexpr int NST = kT * N / VPT;               // staging threads
  static constexpr int VV = kT * CPB / 256;              // v elements per thread
  static_assert(K % LPC == 0 && R >= 1 && VV >= 1 && NST % 64 == 0, "chunk shape");
};

template <typename Tin, typename Tout, int N>
__global__ __launch_bounds__(64 * kWaves) void gla_fwd_kernel(GlaParams p) {
  using S = GlaShape<N>;
  constexpr int kT = S::kT, LPC = S::LPC, C = S::C, CPW = S::CPW, CPB = S::CPB, K = S::K, R = S::R;
  constexpr int VPT = S::VPT, NST = S::NST, VV = S::VV;
  constexpr int ES = sizeof(Tin);
  constexpr int NW = (VPT * ES + 3) / 4;  // 32-bit words per staging thread per tensor per chunk
  static_assert(VPT * ES >= 4, "staging runs of at least one word");
  // the chunk's k, q and decay exp(gk) of the workgroup's head, and v of its columns, shared by its 4 waves
  __shared__ __attribute__((aligned(16))) float s_kqd[3][kT][N];
  __shared__ __attribute__((aligned(16))) float s_v[kT][CPB];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int logical = xcd_remap(blockIdx.x, gridDim.x);
  const int s = logical / p.ntiles;
  const int tile = logical - s * p.ntiles;
  const int colb = tile * CPB;            // the workgroup's first column (head_dim is a multiple of CPB)
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
  const int hd = colb / p.head_dim;
  const int sub = lane % LPC, grp = lane / LPC;
  const int cw0 = wave * CPW + grp * C;   // this lane's first column inside the workgroup
  const int col0 = colb + cw0;

  // this lane's states S[4 sub + i][column col0 + c]
  float h[C][4];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    if (p.h0) {
      const float4 hv =
          reinterpret_cast<const float4*>(p.h0 + (static_cast<int64_t>(s) * p.dim + col0 + c) * N)[sub];
      h[c][0] = hv.x; h[c][1] = hv.y; h[c][2] = hv.z; h[c][3] = hv.w;
    } else {
      h[c][0] = h[c][1] = h[c][2] = h[c][3] = 0.f;
    }
  }
  const uint32_t row_bytes = static_cast<uint32_t>(p.dim) * ES;
  const uint32_t kq_row = static_cast<uint32_t>(p.heads) * N * ES;
  const bool stager = tid < NST;          // whole waves (NST is a multiple of 64)
  const int e0 = tid * VPT;               // staging run: token e0 / N, keys e0 % N .. + VPT
  const int st_j = e0 / N, st_n = e0 % N;

  // chunk loads into registers (rows past the sequence read as 0: k = v = 0 and decay exp(0) = 1 leave the
  // state alone)
  Tin vv[VV];
  uint32_t kw[NW], qw[NW], gw[NW];
  auto load_chunk = [&](int c0) {
    const int64_t tok = t0 + c0;
    const int rows = len - c0;
    const int64_t remain = static_cast<int64_t>(rows < kT ? rows : kT);
    const rsrc_t rv = rsrc_bytes(static_cast<const Tin*>(p.v) + tok * p.dim, remain * row_bytes);
#pragma unroll
    for (int k = 0; k < VV; ++k) {
      const int i = tid + 256 * k;         // token i / CPB, column i % CPB of the workgroup
      ld_elem(rv, static_cast<uint32_t>(i / CPB) * row_bytes + static_cast<uint32_t>(colb + i % CPB) * ES, vv[k]);
    }
    if (stager) {
      const int64_t kbase = (tok * p.heads + hd) * N;
      const rsrc_t rk = rsrc_bytes(static_cast<const Tin*>(p.k) + kbase, remain * kq_row);
      const rsrc_t rq = rsrc_bytes(static_cast<const Tin*>(p.q) + kbase, remain * kq_row);
      const rsrc_t rg = rsrc_bytes(static_cast<const Tin*>(p.gk) + kbase, remain * kq_row);
      const uint32_t koff = static_cast<uint32_t>(st_j) * kq_row + static_cast<uint32_t>(st_n) * ES;
      ld_words<NW>(rk, koff, kw);
      ld_words<NW>(rq, koff, qw);
      ld_words<NW>(rg, koff, gw);
    }
  };
  auto widen_word = [&](const uint32_t (&w)[NW], int i) -> float {
    if constexpr (ES == 2) return (i & 1) ? __uint_as_float(w[i >> 1] & 0xffff0000u) : __uint_as_float(w[i >> 1] << 16);
    else return __uint_as_float(w[i]);
  };

  const rsrc_t ro = rsrc_bytes(static_cast<Tout*>(p.o) + t0 * p.dim, static_cast<int64_t>(len) * p.dim *
                                                                      static_cast<int64_t>(sizeof(Tout)));
  if (len > 0) load_chunk(0);
  for (int c0 = 0; c0 < len; c0 += kT) {
    // publish this chunk: k, q and the decay exp(gk) (once per (token, key)), and v
    if (stager) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        s_kqd[0][st_j][st_n + i] = widen_word(kw, i);
        s_kqd[1][st_j][st_n + i] = widen_word(qw, i);
        s_kqd[2][st_j][st_n + i] = __builtin_amdgcn_exp2f(widen_word(gw, i) * kLog2e);
      }
    }
#pragma unroll
    for (int k = 0; k < VV; ++k) {
      const int i = tid + 256 * k;
      s_v[i / CPB][i % CPB] = widen(vv[k]);
    }
    __syncthreads();   // chunk staged
    if (c0 + kT < len) load_chunk(c0 + kT);
    // the chunk's kT updates of this lane's C x 4 states; partial readouts over its 4 keys
    float part[K];
#pragma unroll
    for (int j = 0; j < kT; ++j) {
      const float4 k4 = reinterpret_cast<const float4*>(&s_kqd[0][j][0])[sub];
      const float4 q4 = reinterpret_cast<const float4*>(&s_kqd[1][j][0])[sub];
      const float4 d4 = reinterpret_cast<const float4*>(&s_kqd[2][j][0])[sub];
      const float kk[4] = {k4.x, k4.y, k4.z, k4.w}, qq[4] = {q4.x, q4.y, q4.z, q4.w};
      const float dd[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const float vc = s_v[j][cw0 + c];
        float pr = 0.f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          h[c][i] = fmaf(dd[i], h[c][i], vc * kk[i]);
          pr = fmaf(qq[i], h[c][i], pr);
        }
        part[c * kT + j] = pr;
      }
    }
    __syncthreads();   // every wave is done with the chunk's LDS
    // sums over the group's LPC lanes: lane l keeps partial indices r + R (l % LPC) = (column, token)
    reduce_scatter<LPC, K>(part, lane);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int idx = r + R * sub;
      const int c = idx / kT, j = idx % kT;
      st_elem(ro, (static_cast<uint32_t>(c0 + j) * p.dim + static_cast<uint32_t>(col0 + c)) *
                      static_cast<uint32_t>(sizeof(Tout)),
              part[r], static_cast<Tout*>(nullptr));
    }
  }
  if (p.h_last) {
#pragma unroll
    for (int c = 0; c < C; ++c)
      reinterpret_cast<float4*>(p.h_last + (static_cast<int64_t>(s) * p.dim + col0 + c) * N)[sub] =
          make_float4(h[c][0], h[c][1], h[c][2], h[c][3]);
  }
}

// ---------------------------------------------------------------------------
// Chunked form (the GLA paper's hardware-efficient form, §3 and §4.2 of "Gated Linear Attention
// Transformers with Hardware-Efficient Training"), for bf16 inputs, 128 or 256 keys and a multiple of 32
// values.  A chunk holds 64 tokens; with b_t the inclusive cumulative sum of gk over the chunk's tokens and
// S0 the state entering the chunk,
//     o_t  = (q_t ⊙ e^{b_t}) S0 + Σ_{s ≤ t} A_ts v_s,   A_ts = Σ_n q_tn k_sn e^{b_tn − b_sn}
//     S64  = diag(e^{b_64}) S0 + Σ_s (k_s ⊙ e^{b_64 − b_s})ᵀ v_s
// where every exponent is ≤ 0 (no overflow, whatever the gates).  A prep kernel computes, once per
// (chunk, head), the scaled q and k, e^{b_64}, and A exactly (pairwise exponents), into a workspace; the
// chunk kernel then runs the three products on the matrix cores for one head and 32 value columns: each of
// its N / 32 waves keeps a 32-key x 32-value tile of S as an MFMA accumulator, its partial outputs over its
// keys are summed through LDS, and the tile is updated in place.  Operands that are not inputs (scaled q
// and k, A, S) enter as bf16 hi + lo pairs (16 significant bits); v is exact in bf16.  S used as the B
// operand straight from its accumulator registers fixes the key order of the contraction (inside each
// 16-key group, keys 4..7 and 8..11 trade places); the scaled q is stored in that order.
// ---------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
constexpr int kCQ = 64;        // tokens per chunk
constexpr int kVtRow = 72;     // LDS row of the transposed v tile (bf16): 64 tokens + 8 (16 rows on distinct banks)

// Workspace of one (chunk slot, head), in MFMA operand fragments: a fragment is the 16 bytes each of the 64
// lanes of a wave feeds one MFMA, stored lane after lane (1 KiB), so that a wave loads it whole and in order.
// Scaled q: fragment (token tile tt, wave w, 16-key slice kk, hi/lo) holds rows 32 tt + l % 32, contraction
// positions 32 w + 16 kk + 8 (l / 32) + 0..7.  Scaled kᵀ: (w, 16-token slice kk, hi/lo) holds keys
// 32 w + l % 32, tokens 16 kk + 8 (l / 32) + 0..7.  A: (tt, kk, hi/lo) holds rows 32 tt + l % 32, tokens
// 16 kk + 8 (l / 32) + 0..7 (zero above the diagonal).  Then e^{b_64} [N] in fp32.
template <int N>
struct ChunkWs {
  static constexpr int NW = N / 32;
  static constexpr int kQs = 0, kKt = 8 * NW * 1024, kAm = 16 * NW * 1024, kG = kAm + 16 * 1024;
  static constexpr int kBytes = kG + 4 * N;
  static_assert(kBytes % 256 == 0, "256-byte slots");
  __device__ static constexpr int qs(int tt, int w, int kk, int pl) { return kQs + (((tt * NW + w) * 2 + kk) * 2 + pl) * 1024; }
  __device__ static constexpr int kt(int w, int kk, int pl) { return kKt + ((w * 4 + kk) * 2 + pl) * 1024; }
  __device__ static constexpr int am(int tt, int kk, int pl) { return kAm + ((tt * 4 + kk) * 2 + pl) * 1024; }
};

struct GlaChunkParams {
  const uint16_t *q, *k, *gk, *v;
  const float* h0;
  float* h_last;
  void* o;
  const int32_t* cu;
  unsigned char* ws;
  int32_t nseq, seqlen, heads, head_dim, total, nch, vtiles, nblocks;
};

__device__ __forceinline__ int32_t cu_at(const int32_t* cu, int s, int32_t total) {
  const int32_t v = cu[s];
  return v < 0 ? 0 : (v > total ? total : v);
}
struct ChunkSeq {
  int64_t t0;
  int32_t len, slot0;
};
// (first token, length) of sequence s and the workspace slot of its first chunk: batched sequences own nch
// slots each; packed sequence s owns slots (cu[s] >> 6) + s .. (never overlapping, all below (total >> 6) + nseq)
__device__ __forceinline__ ChunkSeq chunk_seq(const GlaChunkParams& p, int s) {
  ChunkSeq r;
  if (p.cu) {
    const int32_t b = cu_at(p.cu, s, p.total), e0 = cu_at(p.cu, s + 1, p.total);
    r.t0 = b;
    r.len = (e0 < b ? b : e0) - b;
    r.slot0 = (b >> 6) + s;
  } else {
    r.t0 = static_cast<int64_t>(s) * p.seqlen;
    r.len = p.seqlen;
    r.slot0 = s * p.nch;
  }
  return r;
}

__device__ __forceinline__ float bf16f(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
// a and b rounded to bf16 (to nearest even) by one paired conversion, a in the low half
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
// a and b as hi + lo bf16 (hi = v rounded, lo = the remainder rounded), each a packed pair
__device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack_bf16x2(a, b);
  lo = pack_bf16x2(a - __uint_as_float(hi << 16), b - __uint_as_float(hi & 0xffff0000u));
}
// v[0 .. 7] as hi + lo bf16, element j in half j % 2 of word j / 2
__device__ __forceinline__ void hilo8(const float (&v)[8], uint4& h, uint4& l) {
  uint32_t hw[4], lw[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) split2(v[2 * j], v[2 * j + 1], hw[j], lw[j]);
  h = make_uint4(hw[0], hw[1], hw[2], hw[3]);
  l = make_uint4(lw[0], lw[1], lw[2], lw[3]);
}
// key at contraction position p of a 16-key group (and back: the map is its own inverse)
__device__ __forceinline__ int swap23(int p) { return (p & ~12) | ((p & 4) << 1) | ((p & 8) >> 1); }

// the 8 accumulator elements e0 .. e0 + 7 as a bf16 hi + lo pair
__device__ __forceinline__ void split8(const f32x16_t& acc, int e0, bf16x8_t& hi, bf16x8_t& lo) {
  const float v[8] = {acc[e0], acc[e0 + 1], acc[e0 + 2], acc[e0 + 3], acc[e0 + 4], acc[e0 + 5], acc[e0 + 6], acc[e0 + 7]};
  uint4 h, l;
  hilo8(v, h, l);
  hi = __builtin_bit_cast(bf16x8_t, h);
  lo = __builtin_bit_cast(bf16x8_t, l);
}
__device__ __forceinline__ bf16x8_t ldop(const unsigned char* p) { return *reinterpret_cast<const bf16x8_t*>(p); }
__device__ __forceinline__ f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Largest decay span (in e-folds) across which A is formed from factors e^{b_t − m} and e^{m − b_s}; a
// 32-token half of a chunk whose gates sum to more than this falls back to the exact pairwise form.
constexpr float kSpanMax = 64.f;

// Prep kernel: block = (slot, head), 8 waves; slots between packed sequences return at once.  The keys go
// through in passes of 128 (one for N = 128, two for N = 256), which keeps the LDS footprint near 80 KiB so
// that two blocks share a CU.  Per pass:
//   * b = inclusive cumulative sum of gk over the chunk's 64 tokens (tokens past the sequence add 0);
//   * scaled q and kᵀ and e^{b_64}, elementwise, straight into their workspace fragments;
//   * the pass's keys' share of A in 32 x 32 tiles (GLA paper, §4.2, secondary chunking): with m the decay at
//     the start of a token half, A_ts = Σ_n (q_tn e^{b_tn − m_n}) (k_sn e^{m_n − b_sn}).  The block below the
//     diagonal (queries in the second half, keys in the first) takes m = b_31, where both factors are ≤ 1;
//     the two diagonal blocks take m at their half's start, where the key factor is ≤ e^{span of the half}:
//     one wave and 24 MFMAs (bf16 hi + lo factors) per tile and pass, accumulated across the passes.  For a
//     diagonal block whose half spans more than kSpanMax for some key of the pass, that pass's terms are
//     taken exactly instead, Σ_n q_tn k_sn e^{b_tn − b_sn} term by term (A is a sum over keys, so each pass
//     may take either form).
template <int N>
__global__ __launch_bounds__(512) void gla_prep_kernel(GlaChunkParams p) {
  constexpr int kT = 512;
  constexpr int KP = 128;        // keys per pass
  constexpr int NP = N / KP;     // passes
  static_assert(N % KP == 0, "whole passes");
  using W = ChunkWs<N>;
  constexpr int kQR = KP + 8;    // LDS row strides (padded so that 16 consecutive rows hit distinct banks)
  constexpr int kBR = KP + 4;
  constexpr int kAR = 33;
  __shared__ __attribute__((aligned(16))) uint16_t sQ[kCQ * kQR];
  __shared__ __attribute__((aligned(16))) uint16_t sK[kCQ * kQR];
  __shared__ __attribute__((aligned(16))) float sB[kCQ * kBR];
  __shared__ float sA[3][32 * kAR];   // A tiles (0,0), (1,0), (1,1) as [query][key token]
  __shared__ int sWide[2];            // half h spans more than kSpanMax for some key of the pass
  const int slot = static_cast<int>(blockIdx.x) / p.heads, h = static_cast<int>(blockIdx.x) - slot * p.heads;
  int s;
  if (p.cu) {
    int lo = 0, hi = p.nseq;   // the last sequence whose first slot is <= slot
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((cu_at(p.cu, mid, p.total) >> 6) + mid <= slot) lo = mid;
      else hi = mid;
    }
    s = lo;
  } else {
    s = slot / p.nch;
  }
  const ChunkSeq cs = chunk_seq(p, s);
  const int c = slot - cs.slot0;
  if (c < 0 || c * kCQ >= cs.len) return;
  const int nv = (cs.len - c * kCQ) < kCQ ? cs.len - c * kCQ : kCQ;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const uint32_t rowb = static_cast<uint32_t>(p.heads) * N * 2;
  const int64_t e0 = (cs.t0 + static_cast<int64_t>(c) * kCQ) * p.heads * N + static_cast<int64_t>(h) * N;
  const int64_t bytes = static_cast<int64_t>(nv - 1) * rowb + N * 2;   // rows past the chunk's tokens read 0
  const rsrc_t rq = rsrc_bytes(p.q + e0, bytes), rk = rsrc_bytes(p.k + e0, bytes), rg = rsrc_bytes(p.gk + e0, bytes);
  unsigned char* ws = p.ws + (static_cast<int64_t>(slot) * p.heads + h) * W::kBytes;
  // A tiles on the matrix cores: wave 0 → (0,0) with m = 0, wave 1 → (1,0) and wave 2 → (1,1) with m = b_31
  const int tt = wave == 0 ? 0 : 1, sb = wave == 2 ? 1 : 0;
  const bool ref31 = wave != 0;
  const int diag = wave == 0 ? 0 : 1;   // the half of a diagonal tile (waves 0 and 2)
  const int tq = 32 * tt + l32, tk = 32 * sb + l32;
  f32x16_t acc = f32x16_t{};
  float ex[2][2] = {{0.f, 0.f}, {0.f, 0.f}};   // exact diagonal terms of wide passes: [half][item]
  bool wide_any[2] = {false, false};
  for (int ps = 0; ps < NP; ++ps) {
    const int nb = KP * ps;   // first key of the pass
    if (ps > 0) __syncthreads();   // the previous pass is done with LDS
    if (tid < 2) sWide[tid] = 0;
    // q, k and gk rows (gk widened to fp32 in place of b)
#pragma unroll 2
    for (int i = tid; i < kCQ * KP / 8; i += kT) {
      const int t = i / (KP / 8), c8 = i - t * (KP / 8);
      const uint32_t off = static_cast<uint32_t>(t) * rowb + 2u * nb + 16u * c8;
      const auto a = __builtin_amdgcn_raw_buffer_load_b128(rq, off, 0, 0);
      const auto b = __builtin_amdgcn_raw_buffer_load_b128(rk, off, 0, 0);
      const auto g = __builtin_amdgcn_raw_buffer_load_b128(rg, off, 0, 0);
      *reinterpret_cast<uint4*>(&sQ[t * kQR + 8 * c8]) = make_uint4(a[0], a[1], a[2], a[3]);
      *reinterpret_cast<uint4*>(&sK[t * kQR + 8 * c8]) = make_uint4(b[0], b[1], b[2], b[3]);
      float* gb = &sB[t * kBR + 8 * c8];
      *reinterpret_cast<float4*>(gb) = make_float4(__uint_as_float(g[0] << 16), __uint_as_float(g[0] & 0xffff0000u),
                                                   __uint_as_float(g[1] << 16), __uint_as_float(g[1] & 0xffff0000u));
      *reinterpret_cast<float4*>(gb + 4) = make_float4(__uint_as_float(g[2] << 16), __uint_as_float(g[2] & 0xffff0000u),
                                                       __uint_as_float(g[3] << 16), __uint_as_float(g[3] & 0xffff0000u));
    }
    __syncthreads();
    // inclusive cumulative sum over the tokens, in place: two threads per key (tokens 0..31 and 32..63), then
    // the second adds the first's total
    const int cn = tid % KP, ch = tid / KP;
    if (tid < 2 * KP) {
      float run = 0.f;
#pragma unroll 8
      for (int t = 32 * ch; t < 32 * ch + 32; ++t) {
        run += sB[t * kBR + cn];
        sB[t * kBR + cn] = run;
      }
    }
    __syncthreads();
    if (tid < 2 * KP && ch == 1) {
      const float b31 = sB[31 * kBR + cn];
#pragma unroll 8
      for (int t = 32; t < kCQ; ++t) sB[t * kBR + cn] += b31;
    }
    __syncthreads();
    for (int n = tid; n < KP; n += kT) {
      const float b31 = sB[31 * kBR + n], b63 = sB[(kCQ - 1) * kBR + n];
      reinterpret_cast<float*>(ws + W::kG)[nb + n] = __builtin_amdgcn_exp2f(b63 * kLog2e);
      if (-b31 > kSpanMax) sWide[0] = 1;
      if (b31 - b63 > kSpanMax) sWide[1] = 1;
    }
    // q ⊙ e^{b_t} at contraction positions: 8 positions per item
    for (int i = tid; i < kCQ * KP / 8; i += kT) {
      const int t = i / (KP / 8), p8 = i - t * (KP / 8);
      const int pg = p8 + nb / 8;   // position group among all N keys
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int n = (p8 & ~1) * 8 + swap23(8 * (p8 & 1) + j);
        v[j] = bf16f(sQ[t * kQR + n]) * __builtin_amdgcn_exp2f(sB[t * kBR + n] * kLog2e);
      }
      uint4 hq, lq;
      hilo8(v, hq, lq);
      const int ln = 16 * (32 * (p8 & 1) + (t & 31));
      *reinterpret_cast<uint4*>(ws + W::qs(t >> 5, pg >> 2, (pg >> 1) & 1, 0) + ln) = hq;
      *reinterpret_cast<uint4*>(ws + W::qs(t >> 5, pg >> 2, (pg >> 1) & 1, 1) + ln) = lq;
    }
    // (k ⊙ e^{b_64 − b_s})ᵀ: 8 tokens of one key per item
    for (int i = tid; i < KP * kCQ / 8; i += kT) {
      const int n = i % KP, tb = i / KP;
      const int ng = nb + n;
      const float be = sB[(kCQ - 1) * kBR + n];
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int t = 8 * tb + j;
        v[j] = bf16f(sK[t * kQR + n]) * __builtin_amdgcn_exp2f((be - sB[t * kBR + n]) * kLog2e);
      }
      uint4 hk, lk;
      hilo8(v, hk, lk);
      const int ln = 16 * (32 * (tb & 1) + (ng & 31));
      *reinterpret_cast<uint4*>(ws + W::kt(ng >> 5, tb >> 1, 0) + ln) = hk;
      *reinterpret_cast<uint4*>(ws + W::kt(ng >> 5, tb >> 1, 1) + ln) = lk;
    }
    __syncthreads();   // the pass's span flags
    const bool w0 = sWide[0] != 0, w1 = sWide[1] != 0;   // (block-uniform)
    wide_any[0] = wide_any[0] || w0;
    wide_any[1] = wide_any[1] || w1;
    if (wave < 3 && !(wave != 1 && (diag == 0 ? w0 : w1))) {
      for (int kk = 0; kk < KP / 16; ++kk) {
        const int n0 = 16 * kk + 8 * hl;
        float xs[8], ys[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int n = n0 + j;
          const float m = ref31 ? sB[31 * kBR + n] : 0.f;
          xs[j] = bf16f(sQ[tq * kQR + n]) * __builtin_amdgcn_exp2f((sB[tq * kBR + n] - m) * kLog2e);
          ys[j] = bf16f(sK[tk * kQR + n]) * __builtin_amdgcn_exp2f((m - sB[tk * kBR + n]) * kLog2e);
        }
        uint4 xh, xl, yh, yl;
        hilo8(xs, xh, xl);
        hilo8(ys, yh, yl);
        const bf16x8_t ah = __builtin_bit_cast(bf16x8_t, xh), al = __builtin_bit_cast(bf16x8_t, xl);
        const bf16x8_t bh = __builtin_bit_cast(bf16x8_t, yh), bl = __builtin_bit_cast(bf16x8_t, yl);
        acc = mfma(ah, bh, acc);
        acc = mfma(ah, bl, acc);
        acc = mfma(al, bh, acc);
      }
    }
    // a diagonal tile whose half spans too much in this pass: its exact terms
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      if (!(hf == 0 ? w0 : w1)) continue;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int i = tid + kT * r;
        const int tl = i >> 5, sl = i & 31;
        if (sl > tl) continue;
        const int t = 32 * hf + tl, sj = 32 * hf + sl;
        float a = 0.f;
        for (int n = 0; n < KP; ++n)
          a = fmaf(bf16f(sQ[t * kQR + n]) * bf16f(sK[sj * kQR + n]),
                   __builtin_amdgcn_exp2f((sB[t * kBR + n] - sB[sj * kBR + n]) * kLog2e), a);
        ex[hf][r] += a;
      }
    }
  }
  if (wave < 3) {
#pragma unroll
    for (int e = 0; e < 16; ++e) sA[wave][(8 * (e >> 2) + 4 * hl + (e & 3)) * kAR + l32] = acc[e];
  }
  __syncthreads();
  // add the exact terms of the wide passes (each item belongs to one thread)
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    if (!wide_any[hf]) continue;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const int i = tid + kT * r;
      const int tl = i >> 5, sl = i & 31;
      if (sl <= tl) sA[2 * hf][tl * kAR + sl] += ex[hf][r];
    }
  }
  __syncthreads();
  // A fragments: item (tt, kk, lane) holds row 32 tt + l % 32, key tokens 16 kk + 8 (l / 32) + 0..7
  for (int i = tid; i < 2 * 4 * 64; i += kT) {
    const int ln = i & 63, kk = (i >> 6) & 3, ft = i >> 8;
    const int tl = ln & 31, s0 = 16 * kk + 8 * (ln >> 5);
    const int fb = s0 >> 5;
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int sl = (s0 & 31) + j;
      float a = 0.f;
      if (ft == 1 && fb == 0) a = sA[1][tl * kAR + sl];
      else if (ft == fb && sl <= tl) a = sA[2 * ft][tl * kAR + sl];
      v[j] = a;
    }
    uint4 ha, la;
    hilo8(v, ha, la);
    *reinterpret_cast<uint4*>(ws + W::am(ft, kk, 0) + 16 * ln) = ha;
    *reinterpret_cast<uint4*>(ws + W::am(ft, kk, 1) + 16 * ln) = la;
  }
}

// Chunk kernel: block = (sequence, head, 32-column value tile), N / 32 waves; wave w keeps keys 32 w ..
// 32 w + 31 of the state and adds a share of the intra-chunk product (its (token tile, 16-token slice)
// pairs of A V).  The next chunk's operands are loaded into registers while this chunk computes, and the
// next chunk's v is loaded here and written to LDS at the end.  MFMA lane layouts: lane l holds
// A[l % 32][8 (l / 32) + 0..7] and B[8 (l / 32) + 0..7][l % 32]; result element e of lane l is
// D[8 (e / 4) + 4 (l / 32) + e % 4][l % 32].
template <int N>
struct ChunkOps {                      // operands of the output products (loaded one chunk ahead)
  static constexpr int NW = N / 32;
  static constexpr int kAV = 8 / NW;   // (token tile, slice) pairs of A V per wave
  bf16x8_t qh[2][2], ql[2][2];         // scaled q: [token tile][16-key slice]
  bf16x8_t ah[kAV], al[kAV];           // A
};
struct ChunkKt {                       // operands of the state update (loaded at the chunk's start)
  bf16x8_t kh[4], kl[4];               // scaled kᵀ: [16-token slice]
};

template <typename Tout, int N>
__global__ __launch_bounds__(64 * (N / 32)) void gla_chunk_kernel(GlaChunkParams p) {
  using W = ChunkWs<N>;
  using Ops = ChunkOps<N>;
  constexpr int NW = N / 32;
  constexpr int kThreads = 64 * NW;
  constexpr int kVE = kCQ * 32 / kThreads;      // v elements of a chunk per thread (8 or 4)
  __shared__ __attribute__((aligned(16))) uint16_t sVt[2][32 * kVtRow];   // the chunk's v, [value][token]
  __shared__ __attribute__((aligned(16))) float sO[2][NW][kCQ * 32];      // partial outputs, [token][value]
  __shared__ __attribute__((aligned(16))) float sG[2][N];                  // the chunk's e^{b_64}
  const int logical = xcd_remap(blockIdx.x, p.nblocks);
  const int vt = logical % p.vtiles, sh = logical / p.vtiles;
  const int h = sh % p.heads, s = sh / p.heads;
  const ChunkSeq cs = chunk_seq(p, s);
  const int nch = (cs.len + kCQ - 1) / kCQ;
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hi = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int v0 = vt * 32;
  const int64_t state0 = ((static_cast<int64_t>(s) * p.heads + h) * p.head_dim + v0 + l32) * N + 32 * wave + 4 * hi;

  f32x16_t S;
  if (p.h0) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 v = *reinterpret_cast<const float4*>(p.h0 + state0 + 8 * j);
      S[4 * j] = v.x; S[4 * j + 1] = v.y; S[4 * j + 2] = v.z; S[4 * j + 3] = v.w;
    }
  } else {
    S = f32x16_t{};
  }

  const uint32_t rowv = static_cast<uint32_t>(p.heads) * p.head_dim * 2;
  const int64_t vbase = cs.t0 * p.heads * p.head_dim + static_cast<int64_t>(h) * p.head_dim + v0;
  const int64_t vbytes = cs.len > 0 ? (static_cast<int64_t>(cs.len - 1) * p.heads * p.head_dim + 32) * 2 : 0;
  const rsrc_t rv = rsrc_bytes(p.v + vbase, vbytes);
  // this thread's piece of a chunk's v: token tid / (32 / kVE), columns kVE (tid % (32 / kVE)) .. + kVE - 1
  const int vtok = tid / (32 / kVE), vcol = kVE * (tid % (32 / kVE));
  using VPiece = std::conditional_t<kVE == 8, uint4, uint2>;
  auto load_v = [&](int c, VPiece& w) {
    const uint32_t off = static_cast<uint32_t>(c * kCQ + vtok) * rowv + 2u * vcol;
    if constexpr (kVE == 8) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(rv, off, 0, 0);
      w = make_uint4(x[0], x[1], x[2], x[3]);
    } else {
      const auto x = __builtin_amdgcn_raw_buffer_load_b64(rv, off, 0, 0);
      w = make_uint2(x[0], x[1]);
    }
  };
  auto put_v = [&](int buf, const VPiece& w) {   // written transposed
    uint32_t ws4[kVE / 2];
    if constexpr (kVE == 8) {
      ws4[0] = w.x; ws4[1] = w.y; ws4[2] = w.z; ws4[3] = w.w;
    } else {
      ws4[0] = w.x; ws4[1] = w.y;
    }
#pragma unroll
    for (int j = 0; j < kVE / 2; ++j) {
      sVt[buf][(vcol + 2 * j) * kVtRow + vtok] = static_cast<uint16_t>(ws4[j] & 0xffffu);
      sVt[buf][(vcol + 2 * j + 1) * kVtRow + vtok] = static_cast<uint16_t>(ws4[j] >> 16);
    }
  };
  auto load_ops = [&](int c, Ops& f) {
    const unsigned char* ws = p.ws + (static_cast<int64_t>(cs.slot0 + c) * p.heads + h) * W::kBytes;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        f.qh[tt][kk] = ldop(ws + W::qs(tt, wave, kk, 0) + 16 * lane);
        f.ql[tt][kk] = ldop(ws + W::qs(tt, wave, kk, 1) + 16 * lane);
      }
#pragma unroll
    for (int u = 0; u < Ops::kAV; ++u) {
      const int pr = Ops::kAV * wave + u, tt = pr >> 2, kk = pr & 3;
      f.ah[u] = ldop(ws + W::am(tt, kk, 0) + 16 * lane);
      f.al[u] = ldop(ws + W::am(tt, kk, 1) + 16 * lane);
    }
  };
  auto load_kt = [&](int c, ChunkKt& f) {
    const unsigned char* ws = p.ws + (static_cast<int64_t>(cs.slot0 + c) * p.heads + h) * W::kBytes;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      f.kh[kk] = ldop(ws + W::kt(wave, kk, 0) + 16 * lane);
      f.kl[kk] = ldop(ws + W::kt(wave, kk, 1) + 16 * lane);
    }
  };
  // the chunk's e^{b_64}: 16 bytes for each of the first N / 4 threads, staged through LDS like v
  auto load_g = [&](int c, float4& g4) {
    const unsigned char* ws = p.ws + (static_cast<int64_t>(cs.slot0 + c) * p.heads + h) * W::kBytes;
    g4 = reinterpret_cast<const float4*>(ws + W::kG)[tid < N / 4 ? tid : 0];
  };
  auto put_g = [&](int buf, const float4& g4) {
    if (tid < N / 4) reinterpret_cast<float4*>(sG[buf])[tid] = g4;   // (the other threads hold copies)
  };

  // v and e^{b_64} travel two chunks ahead (registers, then LDS), the operands one chunk ahead (registers)
  Ops cur, nxt;
  VPiece vw0, vw1;   // register sets 0 and 1 (named, so that they stay in registers)
  float4 gw0, gw1;
  if (nch > 0) {
    load_v(0, vw0);
    load_g(0, gw0);
    const int c1 = nch > 1 ? 1 : 0;
    load_v(c1, vw1);
    load_g(c1, gw1);
    load_ops(0, cur);
    put_v(0, vw0);
    put_g(0, gw0);
  }
  // one chunk; the parity of c (which LDS buffer and register set) is a compile-time constant
  // TTc: the token tile of this wave's share of A V (waves 0 .. NW / 2 - 1 take tile 0): a compile-time
  // constant, so that the accumulator it feeds is chosen without selects
  // chunk c's outputs: the sum of the waves' partials in buffer ob, rounded and stored
  auto reduce_store = [&](int c, int ob) {
    const int nv = (cs.len - c * kCQ) < kCQ ? cs.len - c * kCQ : kCQ;
    for (int i = tid; i < kCQ * 8; i += kThreads) {
      const int t = i >> 3, q4 = i & 7;
      if (t >= nv) continue;
      float4 a = *reinterpret_cast<const float4*>(&sO[ob][0][t * 32 + 4 * q4]);
#pragma unroll
      for (int w = 1; w < NW; ++w) {
        const float4 b = *reinterpret_cast<const float4*>(&sO[ob][w][t * 32 + 4 * q4]);
        a.x += b.x; a.y += b.y; a.z += b.z; a.w += b.w;
      }
      const int64_t oe = (cs.t0 + static_cast<int64_t>(c) * kCQ + t) * p.heads * p.head_dim +
                         static_cast<int64_t>(h) * p.head_dim + v0 + 4 * q4;
      if constexpr (sizeof(Tout) == 2) {
        const uint2 w2 = make_uint2(pack_bf16x2(a.x, a.y), pack_bf16x2(a.z, a.w));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.o) + oe) = w2;
      } else {
        *reinterpret_cast<float4*>(static_cast<float*>(p.o) + oe) = a;
      }
    }
  };
  // One barrier per chunk: at the top of chunk c, its v and e^{b_64} are staged and every wave's partial
  // outputs of chunk c - 1 are in LDS; they are summed and stored during chunk c, and their buffer is
  // written again only in chunk c + 1, after the next barrier.
  auto step = [&](int c, auto bufc, auto ttc) {
    constexpr int buf = decltype(bufc)::value;
    constexpr int TTc = decltype(ttc)::value;
    __syncthreads();
    // next chunk's v and operands (the last chunk reloads its own: no branch around the loads)
    const int cn = c + 1 < nch ? c + 1 : c, cnn = c + 2 < nch ? c + 2 : cn;
    // issue order = wait order: this chunk's kᵀ (needed first of these), then chunk c + 2's v and e^{b_64}
    // (register set buf; chunk c + 1's are in set buf ^ 1), then chunk c + 1's output operands
    ChunkKt kt;
    load_kt(c, kt);
    VPiece& vw_mine = buf ? vw1 : vw0;
    float4& gw_mine = buf ? gw1 : gw0;
    VPiece& vw_next = buf ? vw0 : vw1;
    float4& gw_next = buf ? gw0 : gw1;
    load_v(cnn, vw_mine);
    load_g(cnn, gw_mine);
    load_ops(cn, nxt);
    bf16x8_t vf[4];
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) vf[kk] = *reinterpret_cast<const bf16x8_t*>(&sVt[buf][l32 * kVtRow + 16 * kk + 8 * hi]);
    bf16x8_t sh2[2], sl2[2];
    split8(S, 0, sh2[0], sl2[0]);
    split8(S, 8, sh2[1], sl2[1]);
    // partial o over this wave's keys, (q ⊙ e^b) S0, plus its share of A V
    f32x16_t op[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      op[tt] = f32x16_t{};
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        op[tt] = mfma(cur.qh[tt][kk], sh2[kk], op[tt]);
        op[tt] = mfma(cur.qh[tt][kk], sl2[kk], op[tt]);
        op[tt] = mfma(cur.ql[tt][kk], sh2[kk], op[tt]);
      }
    }
#pragma unroll
    for (int u = 0; u < Ops::kAV; ++u) {
      const int kk = (Ops::kAV * wave + u) & 3;   // (its v fragment read again: kk is not a constant)
      const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(&sVt[buf][l32 * kVtRow + 16 * kk + 8 * hi]);
      op[TTc] = mfma(cur.ah[u], va, op[TTc]);
      op[TTc] = mfma(cur.al[u], va, op[TTc]);
    }
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 16; ++e) sO[buf][wave][(32 * tt + 8 * (e >> 2) + 4 * hi + (e & 3)) * 32 + l32] = op[tt][e];
    if (c > 0) reduce_store(c - 1, buf ^ 1);
    // state: S ← diag(e^{b_64}) S + (k ⊙ e^{b_64 − b})ᵀ V
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float4 g4 = reinterpret_cast<const float4*>(sG[buf])[8 * wave + 2 * j + hi];
      S[4 * j] *= g4.x; S[4 * j + 1] *= g4.y; S[4 * j + 2] *= g4.z; S[4 * j + 3] *= g4.w;
    }
    {   // (two accumulation chains: slices 0, 2 into S, 1, 3 into T)
      f32x16_t T = f32x16_t{};
#pragma unroll
      for (int kk = 0; kk < 4; kk += 2) {
        S = mfma(kt.kh[kk], vf[kk], S);
        T = mfma(kt.kh[kk + 1], vf[kk + 1], T);
        S = mfma(kt.kl[kk], vf[kk], S);
        T = mfma(kt.kl[kk + 1], vf[kk + 1], T);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) S[e] += T[e];
    }
    put_v(buf ^ 1, vw_next);   // (chunk c + 1's buffers were last read in chunk c - 1)
    put_g(buf ^ 1, gw_next);
    cur = nxt;
  };
  auto run = [&](auto ttc) {
    for (int c = 0; c < nch; c += 2) {
      step(c, std::integral_constant<int, 0>(), ttc);
      if (c + 1 < nch) step(c + 1, std::integral_constant<int, 1>(), ttc);
    }
  };
  // (both halves of the workgroup run the same barriers)
  if (wave < NW / 2) run(std::integral_constant<int, 0>());
  else run(std::integral_constant<int, 1>());
  if (nch > 0) {
    __syncthreads();
    reduce_store(nch - 1, (nch - 1) & 1);
  }
  if (p.h_last) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      *reinterpret_cast<float4*>(p.h_last + state0 + 8 * j) = make_float4(S[4 * j], S[4 * j + 1], S[4 * j + 2], S[4 * j + 3]);
  }
}

bool aligned(const void* q, uintptr_t a) { return (reinterpret_cast<uintptr_t>(q) & (a - 1)) == 0; }
bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

template <typename Tin, typename Tout>
hipError_t launch_gla(const GlaParams& p, int dstate, dim3 grid, hipStream_t s) {
  const dim3 block(64 * kWaves);
  switch (dstate) {
    case 16: hipLaunchKernelGGL((gla_fwd_kernel<Tin, Tout, 16>), grid, block, 0, s, p); break;
    case 32: hipLaunchKernelGGL((gla_fwd_kernel<Tin, Tout, 32>), grid, block, 0, s, p); break;
    case 64: hipLaunchKernelGGL((gla_fwd_kernel<Tin, Tout, 64>), grid, block, 0, s, p); break;
    case 128: hipLaunchKernelGGL((gla_fwd_kernel<Tin, Tout, 128>), grid, block, 0, s, p); break;
    default: hipLaunchKernelGGL((gla_fwd_kernel<Tin, Tout, 256>), grid, block, 0, s, p); break;
  }
  return hipGetLastError();
}

}  // namespace

namespace {

struct GlaPlan {
  int64_t nseq, tokens, nch, nslots;
  bool chunked;
  size_t ws_bytes;
};

int64_t chunk_ws_bytes(int N) { return N == 256 ? ChunkWs<256>::kBytes : ChunkWs<128>::kBytes; }

samba_status plan_gla(const samba_gla_args* a, GlaPlan* pl) {
  if (!a) return SAMBA_ERR_NULL_ARG;
  if (a->struct_size != sizeof(samba_gla_args)) return SAMBA_ERR_BAD_STRUCT;
  if (a->batch < 0 || a->seqlen < 0 || a->heads < 1 || a->head_dim < 1 || a->nseq < 0) return SAMBA_ERR_BAD_SHAPE;
  const int N = a->dstate;
  if (N != 16 && N != 32 && N != 64 && N != 128 && N != 256) return SAMBA_ERR_UNSUPPORTED;
  if (a->in_dtype != SAMBA_F32 && a->in_dtype != SAMBA_BF16) return SAMBA_ERR_BAD_DTYPE;
  if (a->y_dtype != SAMBA_F32 && a->y_dtype != SAMBA_BF16) return SAMBA_ERR_BAD_DTYPE;
  // a workgroup's value columns (16; 32 at dstate 32, 64 at dstate 16) share a head
  const int cpb = N == 16 ? 64 : (N == 32 ? 32 : 16);
  if (a->head_dim % cpb != 0) return SAMBA_ERR_BAD_SHAPE;
  if (a->cu_seqlens) {
    if (a->batch != 1 || a->nseq < 1) return SAMBA_ERR_BAD_SHAPE;
    pl->nseq = a->nseq;
  } else {
    pl->nseq = a->batch;
  }
  pl->tokens = static_cast<int64_t>(a->batch) * a->seqlen;
  const int64_t dim = static_cast<int64_t>(a->heads) * a->head_dim;
  if (dim * N > (int64_t{1} << 28)) return SAMBA_ERR_BAD_SHAPE;
  // 32-bit offsets inside a sequence's rows
  if (static_cast<int64_t>(a->seqlen) * dim * 4 >= (int64_t{1} << 32)) return SAMBA_ERR_BAD_SHAPE;
  if (static_cast<int64_t>(a->seqlen) * a->heads * N * 4 >= (int64_t{1} << 32)) return SAMBA_ERR_BAD_SHAPE;
  // the chunked form: bf16 inputs, 128 or 256 keys, 32-column value tiles
  pl->chunked = a->in_dtype == SAMBA_BF16 && (N == 128 || N == 256) && a->head_dim % 32 == 0;
  pl->nch = (static_cast<int64_t>(a->seqlen) + kCQ - 1) / kCQ;
  pl->nslots = a->cu_seqlens ? (pl->tokens >> 6) + pl->nseq : pl->nseq * pl->nch;
  if (pl->nslots * a->heads > 0x7fffffff || pl->nseq * a->heads * (a->head_dim / 32 + 1) > 0x7fffffff)
    return SAMBA_ERR_BAD_SHAPE;
  pl->ws_bytes = pl->chunked && pl->tokens > 0 ? static_cast<size_t>(pl->nslots) * a->heads * chunk_ws_bytes(N) : 0;
  return SAMBA_OK;
}

template <typename Tout>
hipError_t launch_chunked(const GlaChunkParams& p, int N, int64_t nslots, hipStream_t s) {
  // (no tokens: no prep, and the chunk kernel only carries h0 to h_last)
  if (N == 256) {
    if (nslots > 0)
      hipLaunchKernelGGL((gla_prep_kernel<256>), dim3(static_cast<uint32_t>(nslots * p.heads)), dim3(512), 0, s, p);
    hipLaunchKernelGGL((gla_chunk_kernel<Tout, 256>), dim3(static_cast<uint32_t>(p.nblocks)), dim3(64 * 8), 0, s, p);
  } else {
    if (nslots > 0)
      hipLaunchKernelGGL((gla_prep_kernel<128>), dim3(static_cast<uint32_t>(nslots * p.heads)), dim3(512), 0, s, p);
    hipLaunchKernelGGL((gla_chunk_kernel<Tout, 128>), dim3(static_cast<uint32_t>(p.nblocks)), dim3(64 * 4), 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace

extern "C" samba_status samba_gla_workspace_size(const samba_gla_args* a, size_t* bytes) {
  if (!bytes) return SAMBA_ERR_NULL_ARG;
  GlaPlan pl;
  const samba_status st = plan_gla(a, &pl);
  if (st != SAMBA_OK) return st;
  *bytes = pl.ws_bytes;
  return SAMBA_OK;
}

extern "C" samba_status samba_gla_fwd(const samba_gla_args* a, void* stream) {
  GlaPlan pl;
  const samba_status st = plan_gla(a, &pl);
  if (st != SAMBA_OK) return st;
  const int N = a->dstate;
  const int64_t nseq = pl.nseq, tokens = pl.tokens;
  if (nseq == 0) return SAMBA_OK;
  const int64_t dim = static_cast<int64_t>(a->heads) * a->head_dim;
  if (tokens > 0 && (!a->q || !a->k || !a->gk || !a->v || !a->o)) return SAMBA_ERR_NULL_ARG;
  const size_t ie = a->in_dtype == SAMBA_BF16 ? 2 : 4, oe = a->y_dtype == SAMBA_BF16 ? 2 : 4;
  if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->gk, 16) || !aligned(a->v, ie) || !aligned(a->o, oe) ||
      !aligned(a->h0, 16) || !aligned(a->h_last, 16))
    return SAMBA_ERR_MISALIGNED;
  // the chunked form reads v in 16-byte pieces and writes o in 4-element pieces
  if (pl.chunked && (!aligned(a->v, 16) || !aligned(a->o, a->y_dtype == SAMBA_BF16 ? 8 : 16))) return SAMBA_ERR_MISALIGNED;
  const size_t tv = static_cast<size_t>(tokens) * dim;
  const size_t tk = static_cast<size_t>(tokens) * a->heads * N * ie;
  const size_t stb = static_cast<size_t>(nseq) * dim * N * 4;
  const void* ins[7] = {a->q, a->k, a->gk, a->v, a->h0, a->cu_seqlens, nullptr};
  const size_t in_sz[7] = {tk, tk, tk, tv * ie, stb, a->cu_seqlens ? (static_cast<size_t>(nseq) + 1) * 4 : 0, 0};
  for (int k = 0; k < 6; ++k) {
    if (overlap(a->o, tv * oe, ins[k], in_sz[k])) return SAMBA_ERR_ALIASING;
    if (a->h_last && !(k == 4 && a->h_last == a->h0) && overlap(a->h_last, stb, ins[k], in_sz[k]))
      return SAMBA_ERR_ALIASING;
  }
  if (overlap(a->o, tv * oe, a->h_last, stb)) return SAMBA_ERR_ALIASING;
  if (pl.ws_bytes > 0) {
    if (!a->workspace || a->workspace_bytes < pl.ws_bytes) return SAMBA_ERR_WORKSPACE;
    if (!aligned(a->workspace, 256)) return SAMBA_ERR_MISALIGNED;
    for (int k = 0; k < 6; ++k)
      if (overlap(a->workspace, pl.ws_bytes, ins[k], in_sz[k])) return SAMBA_ERR_ALIASING;
    if (overlap(a->workspace, pl.ws_bytes, a->o, tv * oe) || overlap(a->workspace, pl.ws_bytes, a->h_last, stb))
      return SAMBA_ERR_ALIASING;
  }
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (pl.chunked) {
    GlaChunkParams p{};
    p.q = static_cast<const uint16_t*>(a->q); p.k = static_cast<const uint16_t*>(a->k);
    p.gk = static_cast<const uint16_t*>(a->gk); p.v = static_cast<const uint16_t*>(a->v);
    p.h0 = a->h0; p.h_last = a->h_last; p.o = a->o;
    p.cu = a->cu_seqlens;
    p.ws = static_cast<unsigned char*>(a->workspace);
    p.nseq = static_cast<int32_t>(nseq);
    p.seqlen = a->seqlen;
    p.heads = a->heads;
    p.head_dim = a->head_dim;
    p.total = a->seqlen;
    p.nch = static_cast<int32_t>(pl.nch);
    p.vtiles = a->head_dim / 32;
    p.nblocks = static_cast<int32_t>(nseq * a->heads * p.vtiles);
    const int64_t nslots = tokens > 0 ? pl.nslots : 0;
    e = a->y_dtype == SAMBA_BF16 ? launch_chunked<uint16_t>(p, N, nslots, s) : launch_chunked<float>(p, N, nslots, s);
    return e == hipSuccess ? SAMBA_OK : SAMBA_ERR_HIP;
  }
  GlaParams p{};
  p.q = a->q; p.k = a->k; p.gk = a->gk; p.v = a->v;
  p.h0 = a->h0; p.h_last = a->h_last; p.o = a->o;
  p.cu = a->cu_seqlens;
  p.nseq = static_cast<int32_t>(nseq);
  p.seqlen = a->seqlen;
  p.heads = a->heads;
  p.head_dim = a->head_dim;
  p.dim = static_cast<int32_t>(dim);
  p.total = a->seqlen;
  const int cpb = N == 16 ? 64 : (N == 32 ? 32 : 16);
  p.ntiles = static_cast<int32_t>((dim + cpb - 1) / cpb);
  if (static_cast<int64_t>(p.ntiles) * nseq > 0x7fffffff) return SAMBA_ERR_BAD_SHAPE;
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.ntiles) * nseq));
  if (a->in_dtype == SAMBA_BF16)
    e = a->y_dtype == SAMBA_BF16 ? launch_gla<uint16_t, uint16_t>(p, N, grid, s) : launch_gla<uint16_t, float>(p, N, grid, s);
  else
    e = a->y_dtype == SAMBA_BF16 ? launch_gla<float, uint16_t>(p, N, grid, s) : launch_gla<float, float>(p, N, grid, s);
  return e == hipSuccess ? SAMBA_OK : SAMBA_ERR_HIP;
}
