// samba_gla.hip -- gfx950 (MI355X) gated linear attention (the GLA layer that the hackernoon page "Microsoft's
// Samba Model Redefines Long-Context Learning for AI", §2, names as a substitute for the Mamba layer), computed
// as its recurrence: per head, S_t = diag(exp(gk_t)) S_{t-1} + k_tᵀ v_t, o_t = q_t S_t.
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
// XOR-k exchange within 32 lanes (k < 32) through the LDS swizzle unit (bit mode: and 0x1f, xor k)
template <int K>
__device__ __forceinline__ float swz_xor(float v) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x1f | (K << 10)));
}
// sum over the LPC consecutive lanes of a channel, in every one of them
template <int LPC>
__device__ __forceinline__ float group_sum(float v) {
  v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
  if constexpr (LPC >= 8) v += swz_xor<4>(v);
  if constexpr (LPC >= 16) v += swz_xor<8>(v);
  if constexpr (LPC >= 32) v += swz_xor<16>(v);
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
    if constexpr (M == 8 || M == 4) got = swz_xor<M>(send);
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

extern "C" samba_status samba_gla_fwd(const samba_gla_args* a, void* stream) {
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
  int64_t nseq;
  if (a->cu_seqlens) {
    if (a->batch != 1 || a->nseq < 1) return SAMBA_ERR_BAD_SHAPE;
    nseq = a->nseq;
  } else {
    nseq = a->batch;
  }
  const int64_t tokens = static_cast<int64_t>(a->batch) * a->seqlen;
  if (nseq == 0) return SAMBA_OK;
  const int64_t dim = static_cast<int64_t>(a->heads) * a->head_dim;
  if (dim * N > (int64_t{1} << 28)) return SAMBA_ERR_BAD_SHAPE;
  // 32-bit offsets inside a sequence's rows
  if (static_cast<int64_t>(a->seqlen) * dim * 4 >= (int64_t{1} << 32)) return SAMBA_ERR_BAD_SHAPE;
  if (static_cast<int64_t>(a->seqlen) * a->heads * N * 4 >= (int64_t{1} << 32)) return SAMBA_ERR_BAD_SHAPE;
  if (tokens > 0 && (!a->q || !a->k || !a->gk || !a->v || !a->o)) return SAMBA_ERR_NULL_ARG;
  const size_t ie = a->in_dtype == SAMBA_BF16 ? 2 : 4, oe = a->y_dtype == SAMBA_BF16 ? 2 : 4;
  if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->gk, 16) || !aligned(a->v, ie) || !aligned(a->o, oe) ||
      !aligned(a->h0, 16) || !aligned(a->h_last, 16))
    return SAMBA_ERR_MISALIGNED;
  const size_t tv = static_cast<size_t>(tokens) * dim;
  const size_t tk = static_cast<size_t>(tokens) * a->heads * N * ie;
  const size_t st = static_cast<size_t>(nseq) * dim * N * 4;
  const void* ins[7] = {a->q, a->k, a->gk, a->v, a->h0, a->cu_seqlens, nullptr};
  const size_t in_sz[7] = {tk, tk, tk, tv * ie, st, a->cu_seqlens ? (static_cast<size_t>(nseq) + 1) * 4 : 0, 0};
  for (int k = 0; k < 6; ++k) {
    if (overlap(a->o, tv * oe, ins[k], in_sz[k])) return SAMBA_ERR_ALIASING;
    if (a->h_last && !(k == 4 && a->h_last == a->h0) && overlap(a->h_last, st, ins[k], in_sz[k]))
      return SAMBA_ERR_ALIASING;
  }
  if (overlap(a->o, tv * oe, a->h_last, st)) return SAMBA_ERR_ALIASING;

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
  p.ntiles = static_cast<int32_t>((dim + cpb - 1) / cpb);
  if (static_cast<int64_t>(p.ntiles) * nseq > 0x7fffffff) return SAMBA_ERR_BAD_SHAPE;
  const dim3 grid(static_cast<uint32_t>(static_cast<int64_t>(p.ntiles) * nseq));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (a->in_dtype == SAMBA_BF16)
    e = a->y_dtype == SAMBA_BF16 ? launch_gla<uint16_t, uint16_t>(p, N, grid, s) : launch_gla<uint16_t, float>(p, N, grid, s);
  else
    e = a->y_dtype == SAMBA_BF16 ? launch_gla<float, uint16_t>(p, N, grid, s) : launch_gla<float, float>(p, N, grid, s);
  return e == hipSuccess ? SAMBA_OK : SAMBA_ERR_HIP;
}
