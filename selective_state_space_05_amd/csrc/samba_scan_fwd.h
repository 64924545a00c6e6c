// samba_scan_fwd.h -- device code of the selective scan's prefill kernel (scan_fwd_kernel, 4 lanes per
// channel) and of the helpers the library's other scan kernels share with it.  What the kernel computes and
// how the work is split are described at the top of samba_scan.hip.
//
// Two translation units include this header: samba_scan.hip (every kernel and the C ABI) and
// samba_scan_fwd_ilp.hip, which holds a second copy of the prefill kernels that inference calls (no
// checkpoints) launch at 1, 8 or 16 time slices, compiled with another instruction scheduler.  Both copies
// are built from the same source, so their results are bitwise the same.
#pragma once

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace samba_fwd {

struct FwdParams {
  const void *x, *dt, *z, *B, *C;
  const float *A, *Dskip, *bias;
  const float* h0;
  float* h_last;
  void* y;
  float* ckpt;           // checkpoint variant: state before every 8th token of each sequence
  const int32_t* cu;
  int64_t total_tokens;
  int32_t seqlen;        // tokens per sequence when cu == nullptr
  int32_t dim;
  int32_t ntiles;        // ceil(dim / 16)
  int32_t tiles_per_wg;  // waves of one workgroup that take consecutive tiles (W == 1 only)
  int32_t ngroups;       // ceil(ntiles / tiles_per_wg)
  int32_t nblocks;       // nseq * ngroups
};

// Launches scan_fwd_kernel<Tin, Tout, W, TPW, K> (no checkpoint variant) for W = 1 (TPW 4, K 16), 4, 8 or 16
// (TPW 1, K 8) from the copy compiled in samba_scan_fwd_ilp.hip; in_bf16 / out_bf16 select Tin / Tout
// (bf16 or fp32).  Returns hipErrorInvalidValue for any other W, else the launch status.
__attribute__((visibility("hidden"))) hipError_t launch_fwd_ilp(bool in_bf16, bool out_bf16, int W, dim3 grid,
                                                                dim3 block, const FwdParams& p, hipStream_t st);

}  // namespace samba_fwd

namespace {

constexpr int kN = 16;         // states per channel
constexpr int kSPL = 4;        // states per lane
constexpr int kCPW = 16;       // channels per wave
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
// Byte offset that every slice-sized y resource ends before (a slice is at most 16 rows of dim < 2^24 fp32
// values, < 2^30 bytes): a lane past the last channel stores there, and the hardware drops the store.
constexpr uint32_t kDropOffset = 0x40000000u;

// ---------------------------------------------------------------------------
// element access and conversion
// ---------------------------------------------------------------------------
__device__ __forceinline__ float ld_in(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float ld_in(const uint16_t* p, int64_t i) {
  return __uint_as_float(static_cast<uint32_t>(p[i]) << 16);
}
__device__ __forceinline__ float widen(uint16_t v) { return __uint_as_float(static_cast<uint32_t>(v) << 16); }
__device__ __forceinline__ float widen(float v) { return v; }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (the gfx950 conversion instruction)
__device__ __forceinline__ uint16_t f32_to_bf16(float v) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(v)); }
__device__ __forceinline__ void st_out(float* p, int64_t i, float v) { p[i] = v; }
__device__ __forceinline__ void st_out(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16(v); }

// ---------------------------------------------------------------------------
// scalar maps
// ---------------------------------------------------------------------------
// softplus(v) = log(1 + e^v) with e = e^v and u = fl(1 + e).  log(1 + e) =
// log(u) + log((1 + e) / u), and (1 + e) - u = e - (u - 1) exactly when e < 1
// (u - 1 is then exact), so the rounding of u is undone by the first-order term
// (e - (u - 1)) / u, with 1/u taken as 2 - u (error (u-1)^2 relative to a term
// already below one ulp).  For e >= 1 the rounding of u costs at most 2^-24
// relative and is left alone; v > 20 returns v (the remainder is below fp32
// resolution).  Full relative accuracy for the small Δ this map produces, with
// two transcendental instructions (exp2, log2).
__device__ __forceinline__ float softplus_f32(float v) {
  const float e = __builtin_amdgcn_exp2f(v * kLog2e);
  const float u = 1.0f + e;
  const float lost = e - (u - 1.0f);
  const float inv_u = (e < 1.0f) ? (2.0f - u) : 0.0f;
  const float r = fmaf(__builtin_amdgcn_logf(u), kLn2, lost * inv_u);
  return (v > 20.0f) ? v : r;
}

// silu(z) = z / (1 + e^{-z})
__device__ __forceinline__ float silu_f32(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-z * kLog2e));
}

// ---------------------------------------------------------------------------
// quad (4-lane) exchanges through DPP quad_perm
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ float qperm(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
constexpr int kQXor1 = 0xB1;  // [1,0,3,2]
constexpr int kQXor2 = 0x4E;  // [2,3,0,1]
// Lane g holds partial sums p[0..3] for the four tokens of a group; returns, on
// lane g, the quad's total for token g.  Register-only version: two exchange
// rounds of a transposed butterfly (6 selects, 3 DPP adds), no LDS traffic.
__device__ __forceinline__ float quad_transpose_sum(float p0, float p1, float p2, float p3, int g) {
  const bool hi = (g & 2) != 0;
  const float k0 = hi ? p2 : p0, s0 = hi ? p0 : p2;
  const float k1 = hi ? p3 : p1, s1 = hi ? p1 : p3;
  const float r0 = k0 + qperm<kQXor2>(s0);
  const float r1 = k1 + qperm<kQXor2>(s1);
  const bool odd = (g & 1) != 0;
  const float k = odd ? r1 : r0, s = odd ? r0 : r1;
  return k + qperm<kQXor1>(s);
}

__device__ __forceinline__ float quad_allsum(float v) {
  v += qperm<kQXor1>(v);
  v += qperm<kQXor2>(v);
  return v;
}

// rotation by N lanes within each row of 16 lanes
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x120 + N, 0xF, 0xF, true));
}
// reduce-scatter steps: lanes 0..31 get lo + lo of the lane 32 above, lanes 32..63 hi + hi of the lane 32
// below; likewise over rows of 16 (even rows keep lo, odd rows hi)
__device__ __forceinline__ float swap32_sum(float lo, float hi) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}
__device__ __forceinline__ float swap16_sum(float lo, float hi) {
  const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(hi), false, false);
  return __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------------------
// buffer access: a wave-uniform resource (base, byte count) in SGPRs plus a
// 32-bit per-lane byte offset.  Reads at or beyond the byte count return 0 and
// writes there are dropped, so a resource that ends at the current sequence's
// last token makes ragged tails free of per-lane predicates.
// ---------------------------------------------------------------------------
using rsrc_t = __amdgpu_buffer_rsrc_t;
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped, unswizzled) buffer

template <typename T>
__device__ __forceinline__ rsrc_t make_rsrc_bytes(const T* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<T*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                          kRsrcWord3);
}
// Resource over `rows` rows of `row_elems` elements; rows <= 0 gives an empty
// resource, and byte counts beyond 32 bits saturate (offsets stay 32-bit).
// 32-bit arithmetic throughout, so the wave-uniform values stay in SGPRs.
template <typename T>
__device__ __forceinline__ rsrc_t make_rsrc_rows(const T* base, int rows, uint32_t row_elems) {
  const uint32_t row_bytes = row_elems * static_cast<uint32_t>(sizeof(T));
  const uint32_t max_rows = 0xffffffffu / row_bytes;
  const uint32_t bytes = rows <= 0 ? 0u
                         : (static_cast<uint32_t>(rows) >= max_rows ? 0xffffffffu : static_cast<uint32_t>(rows) * row_bytes);
  return make_rsrc_bytes(base, bytes);
}
__device__ __forceinline__ void bload(rsrc_t r, uint32_t off, uint16_t& v) {
  v = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 0);
}
__device__ __forceinline__ void bload(rsrc_t r, uint32_t off, float& v) {
  v = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0));
}
template <int NW>
__device__ __forceinline__ void bload_words(rsrc_t r, uint32_t off, uint32_t (&w)[NW]) {
  static_assert(NW == 1 || NW == 2 || NW == 4, "4, 8 or 16 bytes");
  if constexpr (NW == 1) {
    w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
  } else if constexpr (NW == 2) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    w[0] = v[0]; w[1] = v[1];
  } else {
    const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
    w[0] = v[0]; w[1] = v[1]; w[2] = v[2]; w[3] = v[3];
  }
}
__device__ __forceinline__ void bstore(rsrc_t r, uint32_t off, float v, float*) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, 0);
}
__device__ __forceinline__ void bstore(rsrc_t r, uint32_t off, float v, uint16_t*) {
  __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, off, 0, 0);
}

// Block index -> logical index so that consecutive logical blocks (adjacent
// channel tiles, which share 128-byte lines of x, dt, z, y) land on the same
// XCD, given that the dispatcher deals blocks round-robin over the 8 XCDs.
// A bijection on [0, n) whatever the dispatch order is.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7, xcd = bid & 7, slot = bid >> 3;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

using samba_fwd::FwdParams;

// ---------------------------------------------------------------------------
// One slice = K consecutive tokens (K = 8 or 16) of a 16-channel tile.
// Lane g of a quad owns tokens 4j+g (j < K/4) for x, dt, z, y.  B and C rows
// of the slice (K x 16 values each) are spread over the wave, E = K/4 values of
// each per lane, and widened once into fp32 LDS rows (stage_bc).
// ---------------------------------------------------------------------------
template <typename Tin, int K>
struct RawSlice {
  static constexpr int kE = K / 4;                                            // B (and C) values per lane
  static constexpr int kWords = kE * static_cast<int>(sizeof(Tin)) / 4;       // as 32-bit words
  Tin x[K / 4], dt[K / 4], z[K / 4];
  uint32_t bw[kWords], cw[kWords];
};

template <typename Tin, typename Tout, int K>
struct LaneCtx {
  int lane, g, c, d;
  bool dvalid;
  int64_t start, end;
  float A2[kSPL];
  float dsk, bias;
  float hinit[kSPL];
  uint32_t in_off[K / 4];   // byte offsets of this lane's x/dt/z elements from a slice's first row
  uint32_t out_off[K / 4];  // same for y (kDropOffset for a lane past the last channel: its stores are dropped)
  uint32_t bc_off;          // byte offset of this lane's B/C values from a slice's first row
  int bc_lds;               // float index of those values in an LDS [K][16] tile
};

// Issue the loads of the slice starting at token row t0 (all buffer loads); rem = tokens of the sequence
// from t0 on (wave-uniform, 32-bit: a sequence is < 2^31 tokens; 0 or less past its end).
template <typename Tin, typename Tout, int K>
__device__ __forceinline__ void load_raw(const FwdParams& p, const LaneCtx<Tin, Tout, K>& L, int64_t t0, int rem,
                                         RawSlice<Tin, K>& r) {
  const int64_t row0 = t0 * p.dim;
  const uint32_t dim = static_cast<uint32_t>(p.dim);
  const rsrc_t rx = make_rsrc_rows(static_cast<const Tin*>(p.x) + row0, rem, dim);
  const rsrc_t rd = make_rsrc_rows(static_cast<const Tin*>(p.dt) + row0, rem, dim);
  const rsrc_t rz = make_rsrc_rows(static_cast<const Tin*>(p.z) + row0, rem, dim);
#pragma unroll
  for (int j = 0; j < K / 4; ++j) {
    bload(rx, L.in_off[j], r.x[j]);
    bload(rd, L.in_off[j], r.dt[j]);
    bload(rz, L.in_off[j], r.z[j]);
  }
  const rsrc_t rb = make_rsrc_rows(static_cast<const Tin*>(p.B) + t0 * kN, rem, kN);
  const rsrc_t rc = make_rsrc_rows(static_cast<const Tin*>(p.C) + t0 * kN, rem, kN);
  bload_words(rb, L.bc_off, r.bw);
  bload_words(rc, L.bc_off, r.cw);
}

template <typename Tin, int K>
__device__ __forceinline__ void widen_words(const uint32_t (&w)[RawSlice<Tin, K>::kWords], float (&v)[K / 4]) {
  if constexpr (sizeof(Tin) == 2) {
#pragma unroll
    for (int i = 0; i < RawSlice<Tin, K>::kWords; ++i) {
      v[2 * i] = bf_lo(w[i]);
      v[2 * i + 1] = bf_hi(w[i]);
    }
  } else {
#pragma unroll
    for (int i = 0; i < K / 4; ++i) v[i] = __uint_as_float(w[i]);
  }
}

template <int E>
__device__ __forceinline__ void lds_put(float* dst, const float (&v)[E]) {
  if constexpr (E == 2) {
    *reinterpret_cast<float2*>(dst) = make_float2(v[0], v[1]);
  } else {
    *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
  }
}

template <typename Tin, typename Tout, int K>
__device__ __forceinline__ void stage_bc(const RawSlice<Tin, K>& r, const LaneCtx<Tin, Tout, K>& L, float* sB,
                                         float* sC) {
  float v[K / 4];
  widen_words<Tin, K>(r.bw, v);
  lds_put<K / 4>(sB + L.bc_lds, v);
  widen_words<Tin, K>(r.cw, v);
  lds_put<K / 4>(sC + L.bc_lds, v);
}

// Widen a slice's own tokens and discretise: Δ = softplus(dt + bias), u = Δ x.
template <typename Tin, typename Tout, int K>
__device__ __forceinline__ void decode_raw(const RawSlice<Tin, K>& r, const LaneCtx<Tin, Tout, K>& L, int nv,
                                           float (&xv)[K / 4], float (&zv)[K / 4], float (&dl)[K / 4],
                                           float (&uu)[K / 4]) {
#pragma unroll
  for (int j = 0; j < K / 4; ++j) {
    const bool ok = L.dvalid && (4 * j + L.g) < nv;
    const float xr = widen(r.x[j]);
    xv[j] = xr;
    zv[j] = widen(r.z[j]);
    // computed on every lane and then masked: branching would not skip any work
    const float delta = softplus_f32(widen(r.dt[j]) + L.bias);
    dl[j] = ok ? delta : 0.0f;
    uu[j] = ok ? delta * xr : 0.0f;
  }
}

// Share each lane's (Δ, Δx) with its quad through LDS: lane g of channel c
// writes token 4j+g's pair; every lane of the quad then reads the four pairs of
// group j with two 16-byte reads (no cross-lane VALU work).
template <int K>
__device__ __forceinline__ void publish_du(float4 (*du)[kCPW][2], int c, int g, const float (&dl)[K / 4],
                                           const float (&uu)[K / 4]) {
#pragma unroll
  for (int j = 0; j < K / 4; ++j)
    reinterpret_cast<float2*>(du[j][c])[g] = make_float2(dl[j], uu[j]);
}
__device__ __forceinline__ void fetch_du(const float4 (*du)[kCPW][2], int j, int c, float (&dk)[4], float (&uk)[4]) {
  const float4 a = du[j][c][0], b = du[j][c][1];
  dk[0] = a.x; uk[0] = a.y; dk[1] = a.z; uk[1] = a.w;
  dk[2] = b.x; uk[2] = b.y; dk[3] = b.z; uk[3] = b.w;
}

template <int K>
__device__ __forceinline__ int slice_len(int64_t rem) {
  return rem <= 0 ? 0 : (rem < K ? static_cast<int>(rem) : K);
}

// y of token 4j+g: skip, gate, round, store.  No branch: tokens past the sequence end are outside ry (which
// covers the slice's valid rows only) and lanes past the last channel store at kDropOffset; the hardware
// drops both.  With no branch around the stores the count of memory operations in flight is fixed, so the
// next slice's wait for its own loads need not wait for these stores as well.
template <typename Tin, typename Tout, int K>
__device__ __forceinline__ void store_y(const LaneCtx<Tin, Tout, K>& L, rsrc_t ry, int j, float yraw, float xr,
                                        float zr) {
  const float yv = (yraw + L.dsk * xr) * silu_f32(zr);
  bstore(ry, L.out_off[j], yv, static_cast<Tout*>(nullptr));
}

// Checkpoint slot of the state before token 8*j of the sequence that starts
// at token row `start` and is the s-th one: (start / 8) + s + j.  Distinct
// sequences never share a slot, and all slots fit in tokens / 8 + nseq + 1.
__device__ __forceinline__ int64_t ckpt_slot(int64_t start, int s, int j) { return (start >> 3) + s + j; }

// ---------------------------------------------------------------------------
// Prefill kernel.  W = waves splitting each time chunk (1 = plain sequential
// scan); TPW = channel tiles per workgroup (W == 1 only); K = tokens per wave
// slice (8 or 16).  kCkpt: instead of y, write the state before every 8th
// token of each sequence to p.ckpt (the backward's recomputation points).
// kNoCkpt: the launch never passes p.ckpt (inference), so its checks compile out.
// ---------------------------------------------------------------------------
template <typename Tin, typename Tout, int W, int TPW, int K, bool kCkpt = false, bool kNoCkpt = false>
__global__ __launch_bounds__(64 * W * TPW, 4) void scan_fwd_kernel(FwdParams p) {   // (4 waves per SIMD: <= 128 VGPRs)
  static_assert(W == 1 || TPW == 1, "time slices and tile packing are exclusive");
  static_assert(K == 8 || K == 16, "slice length");
  constexpr int kWaves = W * TPW;
  __shared__ float4 s_bc[kWaves][2][K * kN / 4];                   // per-wave staged B, C (fp32)
  __shared__ float4 s_du[kWaves][K / 4][kCPW][2];                  // per-wave (Δ, Δx) of each group's 4 tokens
  __shared__ float4 s_agg[(W > 1) ? W : 1][2][64];                // slice (P, H) pairs of the current chunk
  __shared__ float4 s_cin[(W > 1) ? W : 1][64];                    // each slice's carry-in, from the fold waves

  // wave index, declared wave-uniform so that everything derived from it lives in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int logical = xcd_remap(blockIdx.x, p.nblocks);
  const int s = logical / p.ngroups;
  const int grp = logical - s * p.ngroups;
  const int tile = (W == 1) ? grp * TPW + wave : grp;
  if (W == 1 && tile >= p.ntiles) return;  // whole wave idle (no barriers in the W == 1 path)

  LaneCtx<Tin, Tout, K> L;
  L.lane = threadIdx.x & 63;
  L.g = L.lane & 3;
  L.c = L.lane >> 2;
  L.d = tile * kCPW + L.c;
  L.dvalid = L.d < p.dim;
  {
    const uint32_t dim = static_cast<uint32_t>(p.dim);
    const uint32_t e0 = static_cast<uint32_t>(L.g) * dim + static_cast<uint32_t>(L.d);
#pragma unroll
    for (int j = 0; j < K / 4; ++j) {
      L.in_off[j] = (e0 + static_cast<uint32_t>(j) * 4u * dim) * static_cast<uint32_t>(sizeof(Tin));
      L.out_off[j] = L.dvalid ? (e0 + static_cast<uint32_t>(j) * 4u * dim) * static_cast<uint32_t>(sizeof(Tout))
                              : kDropOffset;
    }
    constexpr int E = K / 4, lanes_per_row = kN / E;
    L.bc_lds = (L.lane / lanes_per_row) * kN + (L.lane % lanes_per_row) * E;
    L.bc_off = static_cast<uint32_t>(L.bc_lds) * static_cast<uint32_t>(sizeof(Tin));
  }
  const int dc = L.dvalid ? L.d : p.dim - 1;
  if (p.cu) {
    int64_t a = p.cu[s], b = p.cu[s + 1];
    a = a < 0 ? 0 : (a > p.total_tokens ? p.total_tokens : a);
    b = b < a ? a : (b > p.total_tokens ? p.total_tokens : b);
    L.start = a;
    L.end = b;
  } else {
    L.start = static_cast<int64_t>(s) * p.seqlen;
    L.end = L.start + p.seqlen;
  }
  {
    const float4 a4 = reinterpret_cast<const float4*>(p.A + static_cast<int64_t>(dc) * kN)[L.g];
    L.A2[0] = a4.x * kLog2e;
    L.A2[1] = a4.y * kLog2e;
    L.A2[2] = a4.z * kLog2e;
    L.A2[3] = a4.w * kLog2e;
  }
  L.dsk = p.Dskip[dc];
  L.bias = p.bias[dc];
  if (p.h0) {
    const float4 h4 = reinterpret_cast<const float4*>(p.h0 + (static_cast<int64_t>(s) * p.dim + dc) * kN)[L.g];
    L.hinit[0] = h4.x; L.hinit[1] = h4.y; L.hinit[2] = h4.z; L.hinit[3] = h4.w;
  } else {
    L.hinit[0] = L.hinit[1] = L.hinit[2] = L.hinit[3] = 0.f;
  }

  float* sB = reinterpret_cast<float*>(s_bc[wave][0]);
  float* sC = reinterpret_cast<float*>(s_bc[wave][1]);
  const float4* sB4 = s_bc[wave][0];
  const float4* sC4 = s_bc[wave][1];
  float h[kSPL] = {L.hinit[0], L.hinit[1], L.hinit[2], L.hinit[3]};
  Tout* const yout = static_cast<Tout*>(p.y);
  // checkpoint of the state before token i (a multiple of 8) of this sequence
  auto put_ckpt = [&](int i, const float (&hv)[kSPL]) {
    if (L.dvalid)
      reinterpret_cast<float4*>(p.ckpt + (ckpt_slot(L.start, s, i >> 3) * p.dim + L.d) * kN)[L.g] =
          make_float4(hv[0], hv[1], hv[2], hv[3]);
  };

  if constexpr (W == 1) {
    // ---------------- sequential scan over the whole sequence ----------------
    // One slice of K tokens per step; the next slice's loads are issued first
    // (into the other register set: the loop body is instantiated twice).
    // Loop bookkeeping stays in 32-bit scalars (a sequence is < 2^31 tokens):
    // 64-bit compares would go through VGPRs and force waits on in-flight loads.
    const int ntok = static_cast<int>(L.end - L.start);
    auto step = [&](int i0, const RawSlice<Tin, K>& cur, RawSlice<Tin, K>& nxt) {
      const int64_t t0 = L.start + i0;
      const int nv = ntok - i0 < K ? ntok - i0 : K;
      load_raw<Tin, Tout, K>(p, L, t0 + K, ntok - i0 - K, nxt);
      stage_bc<Tin, Tout, K>(cur, L, sB, sC);
      float xv[K / 4], zv[K / 4], dl[K / 4], uu[K / 4];
      decode_raw<Tin, Tout, K>(cur, L, nv, xv, zv, dl, uu);
      publish_du<K>(s_du[wave], L.c, L.g, dl, uu);
      // y of this slice only (the checkpoint variant writes none: an empty resource); nv rows are at most
      // 16 * dim * 4 bytes < 2^30 (dim < 2^24), so a lane past the last channel stores beyond the resource
      const rsrc_t ry = make_rsrc_rows(kCkpt ? yout : yout + t0 * p.dim, kCkpt ? 0 : __builtin_amdgcn_readfirstlane(nv),
                                       static_cast<uint32_t>(p.dim));
      if (kCkpt || (!kNoCkpt && p.ckpt)) put_ckpt(i0, h);
      wave_lds_sync();
#pragma unroll
      for (int j = 0; j < K / 4; ++j) {
        // (groups past the sequence end run on with Δ = 0, which leaves the state exactly as it is)
        if constexpr (K == 16) {
          if ((kCkpt || (!kNoCkpt && p.ckpt)) && j == 2 && nv > 8) put_ckpt(i0 + 8, h);
        }
        float4 bv[4], cv[4];
        float dk[4], uk[4];
        fetch_du(s_du[wave], j, L.c, dk, uk);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          bv[q] = sB4[(4 * j + q) * 4 + L.g];
          cv[q] = sC4[(4 * j + q) * 4 + L.g];
        }
        float pr[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          h[0] = fmaf(__builtin_amdgcn_exp2f(dk[q] * L.A2[0]), h[0], uk[q] * bv[q].x);
          h[1] = fmaf(__builtin_amdgcn_exp2f(dk[q] * L.A2[1]), h[1], uk[q] * bv[q].y);
          h[2] = fmaf(__builtin_amdgcn_exp2f(dk[q] * L.A2[2]), h[2], uk[q] * bv[q].z);
          h[3] = fmaf(__builtin_amdgcn_exp2f(dk[q] * L.A2[3]), h[3], uk[q] * bv[q].w);
          pr[q] = fmaf(cv[q].w, h[3], fmaf(cv[q].z, h[2], fmaf(cv[q].y, h[1], cv[q].x * h[0])));
        }
        if constexpr (!kCkpt) {
          // stored without a branch, as in the time-split path below
          const float yraw = quad_transpose_sum(pr[0], pr[1], pr[2], pr[3], L.g);
          store_y<Tin, Tout, K>(L, ry, j, yraw, xv[j], zv[j]);
        }
      }
      wave_lds_sync();
    };
    RawSlice<Tin, K> ra, rb;
    load_raw<Tin, Tout, K>(p, L, L.start, ntok, ra);
    for (int i0 = 0; i0 < ntok; i0 += 2 * K) {
      step(i0, ra, rb);
      if (i0 + K < ntok) step(i0 + K, rb, ra);
    }
    if (p.h_last && L.dvalid)
      reinterpret_cast<float4*>(p.h_last + (static_cast<int64_t>(s) * p.dim + L.d) * kN)[L.g] =
          make_float4(h[0], h[1], h[2], h[3]);
  } else {
    // ---------------- time-sliced scan: W waves per chunk of W*K tokens ----------------
    // 32-bit loop bookkeeping (see the sequential path)
    const int ntok = static_cast<int>(L.end - L.start);
    constexpr int chunk = W * K;
    const int nchunks = (ntok + chunk - 1) / chunk;
    const int my0 = wave * K;  // this wave's slice in chunk 0, relative to the sequence start

    // Carry fold.  The chunk's 64 lanes x 4 states = 256 independent chains are shared out over the first
    // kFoldWaves waves (one per SIMD where W >= 4): thread t of fold wave f owns the kChainsPerThread chains
    // k = (f * kChainsPerThread + q) * 64 + t, i.e. float k of a [64 lanes][4 states] row, so that a fold
    // wave's LDS accesses are contiguous.  Each chain keeps the running carry (the state entering the
    // chunk) in a register: it starts as h0 and after every chunk becomes the state leaving it.
    constexpr int kFoldWaves = W < 4 ? W : 4;
    constexpr int kChainsPerThread = 4 / kFoldWaves;
    constexpr int kFoldGroup = 4;   // slices whose (P, H) are read together: bounds the fold's extra registers
    const bool folder = wave < kFoldWaves;
    // element of h0 / h_last [nseq][dim][16] of chain q of this thread, or -1 (not a fold thread, or past
    // the last channel)
    auto chain_off = [&](int q) -> int64_t {
      const int k = (wave * kChainsPerThread + q) * 64 + L.lane;   // float index in a [64][4] row
      const int cl = k >> 2, st = 4 * (cl & 3) + (k & 3);           // lane of the row, state of the chain
      const int dch = tile * kCPW + (cl >> 2);
      return (folder && dch < p.dim) ? (static_cast<int64_t>(s) * p.dim + dch) * kN + st : -1;
    };
    float carry[kChainsPerThread];
#pragma unroll
    for (int q = 0; q < kChainsPerThread; ++q) {
      const int64_t off = chain_off(q);
      carry[q] = (off >= 0 && p.h0) ? p.h0[off] : 0.f;
    }

    auto chunk_step = [&](int ci, const RawSlice<Tin, K>& cur, RawSlice<Tin, K>& nxt) {
      const int i0 = my0 + ci * chunk;
      const int64_t t0 = L.start + i0;
      const int nv = ntok - i0 <= 0 ? 0 : (ntok - i0 < K ? ntok - i0 : K);
      load_raw<Tin, Tout, K>(p, L, t0 + chunk, ntok - i0 - chunk, nxt);  // prefetch this wave's slice of the next chunk
      stage_bc<Tin, Tout, K>(cur, L, sB, sC);
      float xv[K / 4], zv[K / 4], dl[K / 4], uu[K / 4];
      decode_raw<Tin, Tout, K>(cur, L, nv, xv, zv, dl, uu);
      publish_du<K>(s_du[wave], L.c, L.g, dl, uu);
      wave_lds_sync();

      // phase 1: local scan of the slice from zero; keep Ā and B̄x in registers
      float ak[K][kSPL], bk[K][kSPL];
      float H[kSPL];
      float4 bq[4];
      float dq[4], uq[4];
#pragma unroll
      for (int k = 0; k < K; ++k) {
        const int j = k >> 2, q = k & 3;
        if (q == 0) {
          fetch_du(s_du[wave], j, L.c, dq, uq);
#pragma unroll
          for (int r = 0; r < 4; ++r) bq[r] = sB4[(k + r) * 4 + L.g];  // the group's B rows, read together
        }
        const float dk = dq[q];
        const float uk = uq[q];
        const float4 bv = bq[q];
        ak[k][0] = __builtin_amdgcn_exp2f(dk * L.A2[0]);
        ak[k][1] = __builtin_amdgcn_exp2f(dk * L.A2[1]);
        ak[k][2] = __builtin_amdgcn_exp2f(dk * L.A2[2]);
        ak[k][3] = __builtin_amdgcn_exp2f(dk * L.A2[3]);
        bk[k][0] = uk * bv.x;
        bk[k][1] = uk * bv.y;
        bk[k][2] = uk * bv.z;
        bk[k][3] = uk * bv.w;
#pragma unroll
        for (int i = 0; i < kSPL; ++i) H[i] = (k == 0) ? bk[0][i] : fmaf(ak[k][i], H[i], bk[k][i]);  // from a zero state
      }
      // product of the slice's Ā = exp(A * sum of the slice's Δ)
      float sd = 0.f;
#pragma unroll
      for (int j = 0; j < K / 4; ++j) sd += dl[j];
      sd = quad_allsum(sd);
      s_agg[wave][0][L.lane] = make_float4(__builtin_amdgcn_exp2f(L.A2[0] * sd), __builtin_amdgcn_exp2f(L.A2[1] * sd),
                                           __builtin_amdgcn_exp2f(L.A2[2] * sd), __builtin_amdgcn_exp2f(L.A2[3] * sd));
      s_agg[wave][1][L.lane] = make_float4(H[0], H[1], H[2], H[3]);
      __syncthreads();

      // fold: every slice's carry-in, from the chunk carry through the slices before it (all reads issued
      // first, then one dependent FMA per slice); the result of the last slice is the next chunk's carry
      if (folder) {
        const float* aggf = reinterpret_cast<const float*>(s_agg);
        float* cinf = reinterpret_cast<float*>(s_cin);
#pragma unroll
        for (int q = 0; q < kChainsPerThread; ++q) {
          const int k = (wave * kChainsPerThread + q) * 64 + L.lane;
          float c = carry[q];
#pragma unroll
          for (int g0 = 0; g0 < W; g0 += kFoldGroup) {
            constexpr int G = W < kFoldGroup ? W : kFoldGroup;
            float Pv[G], Hv[G];
#pragma unroll
            for (int u = 0; u < G; ++u) {
              Pv[u] = aggf[((g0 + u) * 2 + 0) * 256 + k];
              Hv[u] = aggf[((g0 + u) * 2 + 1) * 256 + k];
            }
#pragma unroll
            for (int u = 0; u < G; ++u) {
              cinf[(g0 + u) * 256 + k] = c;
              c = fmaf(Pv[u], c, Hv[u]);
            }
          }
          carry[q] = c;
        }
      }
      __syncthreads();

      // phase 3: replay the slice from its carry-in, read out, gate, store
      float hin[kSPL];
      {
        const float4 cr = s_cin[wave][L.lane];
        hin[0] = cr.x; hin[1] = cr.y; hin[2] = cr.z; hin[3] = cr.w;
      }
      // The inference copy (kNoCkpt) stores y without a branch (store_y): its resource covers this slice's
      // valid rows only (nv is wave-uniform).  The other copy keeps the branches, with which it compiles
      // without spills.
      const rsrc_t ry = make_rsrc_rows(kCkpt ? yout : yout + t0 * p.dim,
                                       kCkpt ? 0 : (kNoCkpt ? __builtin_amdgcn_readfirstlane(nv) : ntok - i0),
                                       static_cast<uint32_t>(p.dim));
      if (kCkpt || (!kNoCkpt && p.ckpt)) {
        if (nv > 0) put_ckpt(i0, hin);
      }
#pragma unroll
      for (int i = 0; i < kSPL; ++i) h[i] = hin[i];
#pragma unroll
      for (int j = 0; j < K / 4; ++j) {
        if constexpr (K == 16) {
          if ((kCkpt || (!kNoCkpt && p.ckpt)) && j == 2 && nv > 8) put_ckpt(i0 + 8, h);
        }
        float pr[4];
        float4 cq[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) cq[q] = sC4[(4 * j + q) * 4 + L.g];  // the group's C rows, read together
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int k = 4 * j + q;
          const float4 cv = cq[q];
#pragma unroll
          for (int i = 0; i < kSPL; ++i) h[i] = fmaf(ak[k][i], h[i], bk[k][i]);
          pr[q] = fmaf(cv.w, h[3], fmaf(cv.z, h[2], fmaf(cv.y, h[1], cv.x * h[0])));
        }
        if constexpr (kNoCkpt) {
          const float yraw = quad_transpose_sum(pr[0], pr[1], pr[2], pr[3], L.g);
          store_y<Tin, Tout, K>(L, ry, j, yraw, xv[j], zv[j]);
        } else if constexpr (!kCkpt) {
          if (4 * j < nv) {
            const float yraw = quad_transpose_sum(pr[0], pr[1], pr[2], pr[3], L.g);
            const float yv = (yraw + L.dsk * xv[j]) * silu_f32(zv[j]);
            if (L.dvalid) bstore(ry, L.out_off[j], yv, static_cast<Tout*>(nullptr));
          }
        }
      }
      wave_lds_sync();
    };

    RawSlice<Tin, K> ra, rb;
    load_raw<Tin, Tout, K>(p, L, L.start + my0, ntok - my0, ra);
    for (int ci = 0; ci < nchunks; ci += 2) {
      chunk_step(ci, ra, rb);
      if (ci + 1 < nchunks) chunk_step(ci + 1, rb, ra);
    }
    // the state leaving the sequence is the fold's carry after the last chunk (also for a chained call's
    // next h0, so that chunk-aligned chained calls reproduce a single pass bit for bit)
    if (p.h_last) {
#pragma unroll
      for (int q = 0; q < kChainsPerThread; ++q) {
        const int64_t off = chain_off(q);
        if (off >= 0) p.h_last[off] = carry[q];
      }
    }
  }
}

}  // namespace
