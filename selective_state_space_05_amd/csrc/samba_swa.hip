// samba_swa.hip -- gfx950 (MI355X) kernels and C ABI of the sliding-window
// attention layer of the Samba hybrid: RoPE, prefill attention, decode step.
//
// Operation: page "SAMBA混合注意力状态空间模型", section 数学框架 ->
// 滑动窗口注意力 (softmax of the scaled scores plus the window mask, times V)
// and the hackernoon page, §2.1.2 (window w = 2048, RoPE inside the window).
// Query i sees keys i - window .. i of its own sequence (the mask printed on
// the first page is inverted; this is its causal reading).
//
// Prefill design (FlashAttention-2's online softmax, laid out for CDNA4's
// 64-wide waves and v_mfma_f32_32x32x16_bf16):
//   * a workgroup of 8 waves owns 256 consecutive queries of one head; each
//     wave owns 32 of them and keeps their rotated q (32 x 128 bf16) in
//     registers for the whole key loop;
//   * keys advance 64 at a time through double-buffered LDS tiles (K as
//     [key][hd], V transposed as [hd][key]), half the waves staging K and half V;
//   * scores are formed transposed, S^T = K Q^T, so that every lane holds one
//     query's scores for 16 of each 32 keys: the row maximum is a reduction
//     inside the lane plus one exchange with the lane 32 away, and the running
//     sum needs no exchange at all until the end;
//   * the output is accumulated transposed as well, O^T += V^T P^T, with the
//     probabilities taken straight from the score registers; the key order
//     inside a 16-key chunk is permuted (middle two groups of four swapped) to
//     match the score layout, and V^T is written to LDS in that order;
//   * LDS rows are unpadded and XOR-swizzled at 16-byte granularity so that
//     both the staging writes and the fragment reads spread over the banks;
//   * a wave skips the tiles its 32 queries cannot see, and masks only the
//     tiles that cross the diagonal or the window's far edge.
// Operand layouts of the 32x32x16 MFMA (checked on the device): lane l holds
// A[l % 32][8 (l / 32) + 0..7] and B[8 (l / 32) + 0..7][l % 32]; result
// element e of lane l is D[8 (e / 4) + 4 (l / 32) + e % 4][l % 32].
//
// Decode design: one workgroup per (sequence, head); 16 groups of 16 lanes
// stream the window's keys from the cache (a key row per group per step,
// 16 bytes per lane), each group keeping its own online-softmax state; the
// groups are merged through LDS at the end.  HBM-bound: every cached key and
// value row of the window is read once.
#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "samba_swa.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
using rsrc_t = __amdgpu_buffer_rsrc_t;

constexpr int kRsrcWord3 = 0x00020000;  // raw (untyped, unswizzled) buffer
constexpr float kLog2e = 1.4426950408889634f;
constexpr int kHD = 128;                // head size served by the attention kernels
constexpr int kQB = 256;                // queries per prefill workgroup (8 waves of 32)
constexpr int kQBShift = 8;             // log2(kQB)
constexpr int kSwaThreads = 512;
constexpr int kKB = 64;                 // keys per prefill tile
constexpr int kKRow = kHD + 8;          // K tile row stride in LDS (bf16): 16 rows cover all banks
constexpr float kRescale = 8.0f;        // exp2 units a score may exceed the softmax reference by

// Resource over `rows` rows of row_bytes; rows <= 0 gives an empty resource (loads return 0, stores are
// dropped), byte counts beyond 32 bits saturate.
__device__ __forceinline__ rsrc_t rsrc_rows(const void* base, int rows, uint32_t row_bytes) {
  const uint32_t max_rows = 0xffffffffu / row_bytes;
  const uint32_t bytes = rows <= 0 ? 0u
                         : (static_cast<uint32_t>(rows) >= max_rows ? 0xffffffffu : static_cast<uint32_t>(rows) * row_bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                          kRsrcWord3);
}

__device__ __forceinline__ uint4 ld16(rsrc_t r, uint32_t off) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
__device__ __forceinline__ void st16(rsrc_t r, uint32_t off, uint4 v) {
  const u32x4_t w = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(w, r, off, 0, 0);
}
// same with a wave-uniform part of the offset in the instruction's scalar offset
__device__ __forceinline__ uint4 ld16s(rsrc_t r, uint32_t voff, uint32_t soff) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Consecutive logical blocks land on the same XCD (the dispatcher deals blocks round-robin over 8 XCDs),
// so query blocks that share keys share an L2.  A bijection on [0, n).
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int q = n >> 3, r = n & 7, xcd = bid & 7, slot = bid >> 3;
  return (xcd < r) ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(lo))) |
         (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, static_cast<__bf16>(hi))) << 16);
}

__device__ __forceinline__ int32_t cu_at(const int32_t* cu, int s, int32_t total) {
  const int32_t v = cu[s];
  return v < 0 ? 0 : (v > total ? total : v);
}

// Packed block numbering for sequences given by offsets: sequence s owns the blocks first(s) ..
// first(s) + ceil(len_s / 2^shift) - 1 with first(s) = (cu[s] >> shift) + s.  These ranges never overlap
// and all lie below (total >> shift) + nseq.  Returns the largest s with first(s) <= b (a wave-wide search,
// 64 candidates per round); for offsets that are not ascending the answer is some s (callers clamp).
__device__ int seq_of_block(const int32_t* cu, int nseq, int b, int shift, int32_t total) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = nseq;
  while (hi - lo > 1) {
    const int step = (hi - lo + 63) / 64;
    const int s = lo + lane * step;
    const bool ok = s < hi && (cu_at(cu, s, total) >> shift) + s <= b;
    const uint64_t m = __builtin_amdgcn_ballot_w64(ok);
    const int k = m ? 63 - __builtin_clzll(m) : 0;
    lo += k * step;
    hi = (lo + step < hi) ? lo + step : hi;
  }
  return lo;
}

// (first token row, length, block index inside the sequence) of packed block `b`.
struct SeqBlock {
  int64_t t0;
  int32_t len, j;
};
__device__ __forceinline__ SeqBlock locate(const int32_t* cu, int nseq, int32_t total, int32_t seqlen, int per_seq,
                                           int b, int shift) {
  SeqBlock r;
  if (cu) {
    const int s = seq_of_block(cu, nseq, b, shift, total);
    const int32_t a = cu_at(cu, s, total), e = cu_at(cu, s + 1, total);
    r.t0 = a;
    r.len = e > a ? e - a : 0;
    r.j = b - ((a >> shift) + s);
  } else {
    const int s = b / per_seq;
    r.j = b - s * per_seq;
    r.t0 = static_cast<int64_t>(s) * seqlen;
    r.len = seqlen;
  }
  return r;
}

// ---------------------------------------------------------------------------
// RoPE
// ---------------------------------------------------------------------------
struct RopeParams {
  const uint16_t *qi, *ki;
  uint16_t *qo, *ko;
  const float *cs, *sn;
  const int32_t *cu, *pos0;
  int32_t nseq, seqlen, heads, hd, npos, per_seq, total;
  int32_t shift;   // log2 of the tokens per workgroup
  int32_t groups;  // head groups per token (threads per token = groups x head_dim / 16)
};

// Rotate 8 pairs (x[c..c+7], x[c+half..c+half+7]) held as bf16 words a (first half) and b (second half).
__device__ __forceinline__ void rope8(uint4& a, uint4& b, const float (&c)[8], const float (&s)[8]) {
  uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float x0 = bf_lo(aw[w]), x1 = bf_hi(aw[w]), y0 = bf_lo(bw[w]), y1 = bf_hi(bw[w]);
    const int i = 2 * w;
    aw[w] = pack_bf16(fmaf(x0, c[i], -y0 * s[i]), fmaf(x1, c[i + 1], -y1 * s[i + 1]));
    bw[w] = pack_bf16(fmaf(y0, c[i], x0 * s[i]), fmaf(y1, c[i + 1], x1 * s[i + 1]));
  }
  a = make_uint4(aw[0], aw[1], aw[2], aw[3]);
  b = make_uint4(bw[0], bw[1], bw[2], bw[3]);
}

constexpr int kRopeGroups = 8;   // head groups per token (thread (token, group, chunk)), fewer for head_dim > 512
constexpr int kRopeBatch = 4;    // heads of a group loaded together before any store

// One workgroup per 2^shift tokens of one sequence; thread (token, head group g, chunk c of 8 rotation
// pairs) reads the token's table entries once and rotates chunk c of heads g, g + G, g + 2G, ... of q and k.
// Every access goes through a buffer resource over the workgroup's token rows, and accesses that do not
// exist (a head past the last, a token past the sequence's end) get an out-of-range offset: loads return
// zeros and stores are dropped, so the code has no branches, and all loads of a batch of heads are issued
// before its stores (in-place calls alias input and output, so the compiler could not reorder them).
template <bool kQ, bool kK>
__global__ __launch_bounds__(256) void rope_kernel(RopeParams p) {
  const SeqBlock sb = locate(p.cu, p.nseq, p.total, p.seqlen, p.per_seq, blockIdx.x, p.shift);
  const int tpb = 1 << p.shift;
  if (sb.j < 0 || sb.j * tpb >= sb.len) return;
  const int first = sb.j * tpb;
  const int ntok = (sb.len - first) < tpb ? sb.len - first : tpb;
  const int half = p.hd >> 1, cph = half >> 3;
  const int t = static_cast<int>(threadIdx.x);
  const int cc = t % cph, g = (t / cph) % p.groups, tl = t / (cph * p.groups);
  const bool live = tl < ntok;
  int32_t pos = first + (live ? tl : 0);
  if (p.pos0) {
    const int s = p.cu ? seq_of_block(p.cu, p.nseq, blockIdx.x, p.shift, p.total)
                       : static_cast<int>(blockIdx.x) / p.per_seq;
    pos += p.pos0[s];
  }
  pos = pos < 0 ? 0 : (pos >= p.npos ? p.npos - 1 : pos);
  float c[8], s[8];
  {
    const float4* tc = reinterpret_cast<const float4*>(p.cs + static_cast<int64_t>(pos) * half + 8 * cc);
    const float4* ts = reinterpret_cast<const float4*>(p.sn + static_cast<int64_t>(pos) * half + 8 * cc);
    const float4 c0 = tc[0], c1 = tc[1], s0 = ts[0], s1 = ts[1];
    c[0] = c0.x; c[1] = c0.y; c[2] = c0.z; c[3] = c0.w; c[4] = c1.x; c[5] = c1.y; c[6] = c1.z; c[7] = c1.w;
    s[0] = s0.x; s[1] = s0.y; s[2] = s0.z; s[3] = s0.w; s[4] = s1.x; s[5] = s1.y; s[6] = s1.z; s[7] = s1.w;
  }
  const int64_t blk = (sb.t0 + first) * p.heads * p.hd;   // first element of the workgroup's rows
  const uint32_t row_bytes = static_cast<uint32_t>(p.heads) * p.hd * 2u;
  // (a tensor that is not rotated gets an empty resource over the other one's rows; it is never used)
  const uint16_t* qi = kQ ? p.qi : p.ki;
  uint16_t* qo = kQ ? p.qo : p.ko;
  const uint16_t* ki = kK ? p.ki : p.qi;
  uint16_t* ko = kK ? p.ko : p.qo;
  const rsrc_t rqi = rsrc_rows(qi + blk, kQ ? ntok : 0, row_bytes), rqo = rsrc_rows(qo + blk, kQ ? ntok : 0, row_bytes);
  const rsrc_t rki = rsrc_rows(ki + blk, kK ? ntok : 0, row_bytes), rko = rsrc_rows(ko + blk, kK ? ntok : 0, row_bytes);
  // beyond any resource (a workgroup's rows span at most 32 x 2 MiB), also after adding the half-row step:
  // loads read zeros, stores are dropped
  constexpr uint32_t kNowhere = 0x80000000u;
  const uint32_t base = live ? static_cast<uint32_t>(tl) * row_bytes + 16u * cc : kNowhere;
  const uint32_t hstep = static_cast<uint32_t>(p.hd) * 2u, hb = static_cast<uint32_t>(half) * 2u;
  for (int h0 = g; h0 < p.heads; h0 += p.groups * kRopeBatch) {
    uint32_t off[kRopeBatch];
    uint4 qa[kRopeBatch], qb[kRopeBatch], ka[kRopeBatch], kb[kRopeBatch];
#pragma unroll
    for (int u = 0; u < kRopeBatch; ++u) {
      const int h = h0 + p.groups * u;
      off[u] = (h < p.heads && live) ? base + static_cast<uint32_t>(h) * hstep : kNowhere;
      if constexpr (kQ) {
        qa[u] = ld16(rqi, off[u]);
        qb[u] = ld16(rqi, off[u] + hb);
      }
      if constexpr (kK) {
        ka[u] = ld16(rki, off[u]);
        kb[u] = ld16(rki, off[u] + hb);
      }
    }
#pragma unroll
    for (int u = 0; u < kRopeBatch; ++u) {
      if constexpr (kQ) {
        rope8(qa[u], qb[u], c, s);
        st16(rqo, off[u], qa[u]);
        st16(rqo, off[u] + hb, qb[u]);
      }
      if constexpr (kK) {
        rope8(ka[u], kb[u], c, s);
        st16(rko, off[u], ka[u]);
        st16(rko, off[u] + hb, kb[u]);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill attention
// ---------------------------------------------------------------------------
struct SwaParams {
  const uint16_t *q, *k, *v;
  void* o;
  const int32_t* cu;
  int32_t nseq, seqlen, heads, window;
  int32_t per_seq;   // query blocks per sequence without offsets
  int32_t nqb;       // query blocks per head (grid = nqb * heads)
  int32_t total;     // tokens
  float c;           // log2(e) / sqrt(head size): scores enter exp2 scaled by it
};

// V^T row swizzle: the 16-byte group g of row r is stored at g ^ vswz(r), vswz(r) = (r ^ (r >> 3)) & 7.
// Rows written by one staging instruction differ in r >> 3, rows read by one fragment load in r & 7; both
// spread over the banks.  (The addresses below are this map in closed form.)
// slot of key k inside a 64-key tile: bits 2 and 3 swapped (the score layout's key order)
__device__ __forceinline__ int key_slot(int k) { return (k & ~12) | ((k & 4) << 1) | ((k & 8) >> 1); }

template <typename Tout>
__global__ __launch_bounds__(kSwaThreads, 1) void swa_fwd_kernel(SwaParams p) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kKB * kKRow];  // [key][hd], rows padded to 272 bytes
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][kHD * kKB];   // [hd][slot], group g at g ^ vswz(hd)
  const int logical = xcd_remap(blockIdx.x, p.nqb * p.heads);
  const int head = logical / p.nqb;
  const SeqBlock sb = locate(p.cu, p.nseq, p.total, p.seqlen, p.per_seq, logical - head * p.nqb, kQBShift);
  if (sb.j < 0 || sb.j * kQB >= sb.len) return;   // the whole workgroup leaves together
  const int len = sb.len;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, ql = lane & 31;
  const uint32_t row_bytes = static_cast<uint32_t>(p.heads) * kHD * 2u;
  const int64_t head_off = static_cast<int64_t>(head) * kHD;

  const int qfirst = sb.j * kQB;
  const int qlast = ((len - qfirst) < kQB ? len : qfirst + kQB) - 1;
  const int kt_lo = (qfirst - p.window > 0 ? qfirst - p.window : 0) / kKB;
  const int kt_hi = qlast / kKB;

  // this wave's queries
  const int q_lo = qfirst + 32 * wave;
  const bool wave_live = q_lo < len;
  const int q_hi = wave_live ? ((len - q_lo) < 32 ? len - 1 : q_lo + 31) : q_lo;
  const int qp = q_lo + ql;   // this lane's query
  // q fragments as stored (bf16): the scale log2(e) / sqrt(head size) is applied to the fp32 scores
  bf16x8_t qf[8];
  {
    const rsrc_t rq = rsrc_rows(p.q + (sb.t0 + q_lo) * p.heads * kHD + head_off, wave_live ? q_hi - q_lo + 1 : 0,
                                row_bytes);
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      qf[jj] = __builtin_bit_cast(bf16x8_t, ld16(rq, static_cast<uint32_t>(ql) * row_bytes + (16 * jj + 8 * hf) * 2));
  }

  // staging: waves 4..7 load K (rows sr + 16 r, 16-byte group sg), waves 0..3 load V (keys 4 sr .. 4 sr + 3,
  // hd 8 sg .. 8 sg + 7), four 16-byte pieces per thread either way
  const bool stage_k = wave >= 4;
  const int st = stage_k ? tid - 256 : tid;
  const int sr = st >> 4, sg = st & 15;
  uint4 sv0[4], sv1[4];   // two register sets: the tile after next is loaded while the next one is stored
  // one offset register; the row steps go in the instruction's scalar offset
  const uint32_t g_off = (stage_k ? static_cast<uint32_t>(sr) : static_cast<uint32_t>(4 * sr)) * row_bytes + sg * 16;
  const uint32_t g_step = stage_k ? 16u * row_bytes : row_bytes;
  auto gload = [&](int kt, uint4 (&sv)[4]) {
    const int64_t tok = sb.t0 + static_cast<int64_t>(kt) * kKB;
    const int rows = (len - kt * kKB) < kKB ? len - kt * kKB : kKB;
    const rsrc_t rs = rsrc_rows((stage_k ? p.k : p.v) + tok * p.heads * kHD + head_off, rows, row_bytes);
#pragma unroll
    for (int i = 0; i < 4; ++i) sv[i] = ld16s(rs, g_off, static_cast<uint32_t>(i) * g_step);
  };
  // V^T element (row 8 sg + d, slot s) of this thread's keys: row (8 sg + d) * 64, group (s >> 3) ^ vswz(row)
  // with vswz(8 sg + d) = (sg ^ d) & 7.  As 8 sg * 64 has no bits in 3..5, the address is vbase ^ (d << 3)
  // plus d * 64: one XOR per row, the rest an immediate offset (no per-row address registers).
  const int vslot = key_slot(4 * sr);
  const int vbase = 8 * sg * kKB + ((((vslot >> 3) ^ sg) & 7) << 3) + (vslot & 7);
  auto lstore = [&](auto bufc, const uint4 (&sv)[4]) {
    constexpr int buf = decltype(bufc)::value;
    if (stage_k) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = sr + 16 * r;
        *reinterpret_cast<uint4*>(&sK[buf][row * kKRow + 8 * sg]) = sv[r];
      }
    } else {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const int w = d >> 1;
        const uint32_t a0 = (&sv[0].x)[w], a1 = (&sv[1].x)[w], a2 = (&sv[2].x)[w], a3 = (&sv[3].x)[w];
        // bf16 number d of keys 4 sr + 0..3, packed in key order (byte select: low or high halves)
        constexpr uint32_t kLoHalves = 0x05040100u, kHiHalves = 0x07060302u;
        const uint32_t sel = (d & 1) ? kHiHalves : kLoHalves;
        uint2 pk;
        pk.x = __builtin_amdgcn_perm(a1, a0, sel);
        pk.y = __builtin_amdgcn_perm(a3, a2, sel);
        *reinterpret_cast<uint2*>(&sV[buf][(vbase ^ (d << 3)) + d * kKB]) = pk;
      }
    }
  };

  // fragment addresses (elements) of this lane.  K rows are padded: affine in the 16-column chunk.  V^T row
  // 32 hb + ql, slot group 2 cc + hf, is stored at group (2 cc + hf) ^ vswz(32 hb + ql), and vswz(32 hb + ql)
  // = z ^ 4 (hb & 1) with z = (ql ^ (ql >> 3)) & 7; as ql * 64 has no bits in 3..5 the address is
  // vtbase ^ ((2 cc ^ 4 (hb & 1)) << 3) plus hb * 32 * 64.
  const int kbase = ql * kKRow + 8 * hf;
  const int vtbase = ql * kKB + ((hf ^ ((ql ^ (ql >> 3)) & 7)) << 3);

  f32x16_t acc[4];
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[hb][e] = 0.f;
  // Softmax reference per lane (exp2 units): the scores of a tile are formed relative to it (scaled score
  // minus m_ref, one fp32 fma each), and it is moved only when a score exceeds it by more than kRescale (or
  // before the lane has seen any key), so the rescaling of the output is rare.  Any reference gives the same
  // result once the output is divided by the sum; keeping the maximum within 2^kRescale of it bounds the
  // probabilities by 2^kRescale and keeps the largest one >= 1.
  float m_ref = -INFINITY, l_run = 0.f;
  float mneg = 0.f;   // -m_ref, or 0 before the first key
  const float sc = p.c;

  auto compute = [&](auto bufc, int kt, bool need_mask) {
    constexpr int buf = decltype(bufc)::value;
    const uint16_t* K = sK[buf];
    const uint16_t* Vt = sV[buf];
    f32x16_t s0, s1;
#pragma unroll
    for (int e = 0; e < 16; ++e) s0[e] = s1[e] = 0.f;
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const bf16x8_t a0 = *reinterpret_cast<const bf16x8_t*>(K + kbase + 16 * jj);
      const bf16x8_t a1 = *reinterpret_cast<const bf16x8_t*>(K + kbase + 32 * kKRow + 16 * jj);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, qf[jj], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, qf[jj], s1, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {   // exp2 units, relative to the reference
      s0[e] = fmaf(s0[e], sc, mneg);
      s1[e] = fmaf(s1[e], sc, mneg);
    }
    if (need_mask) {   // visible iff 0 <= query - key <= window
      // (the tile's first key through readfirstlane: an opaque value, so that the compiler does not keep 32
      // per-element induction variables alive across the loop for this rarely taken branch)
      const int dq = qp - __builtin_amdgcn_readfirstlane(kt * kKB) - 4 * hf;
      const uint32_t w = static_cast<uint32_t>(p.window);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int off = 8 * (e >> 2) + (e & 3);
        s0[e] = static_cast<uint32_t>(dq - off) <= w ? s0[e] : -INFINITY;
        s1[e] = static_cast<uint32_t>(dq - off - 32) <= w ? s1[e] : -INFINITY;
      }
    }
    // largest score above the reference, as the integer maximum of the bit patterns: exact whenever some
    // score is positive, and <= 0 as a float otherwise (all that the test below needs)
    int im = __float_as_int(s0[0]);
#pragma unroll
    for (int e = 1; e < 16; ++e) im = max(im, __float_as_int(s0[e]));
#pragma unroll
    for (int e = 0; e < 16; ++e) im = max(im, __float_as_int(s1[e]));
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(im), static_cast<uint32_t>(im), false,
                                                       false);
      im = max(static_cast<int>(sw[0]), static_cast<int>(sw[1]));
    }
    const bool move = (m_ref == -INFINITY) || (__int_as_float(im) > kRescale);
    if (__builtin_amdgcn_ballot_w64(move)) {
      // exact online-softmax step for the whole wave: new reference = running maximum
      float mx = fmaxf(s0[0], s1[0]);
#pragma unroll
      for (int e = 1; e < 16; ++e) mx = fmaxf(mx, fmaxf(s0[e], s1[e]));
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      const float ref = (m_ref == -INFINITY) ? 0.f : m_ref;   // what the scores are relative to
      const float m_new = fmaxf(m_ref, mx + ref);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - m_use);   // 0 before the first key
      const float delta = ref - m_use;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s0[e] += delta;
        s1[e] += delta;
      }
      mneg = -m_use;
      l_run *= alpha;
#pragma unroll
      for (int hb = 0; hb < 4; ++hb)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[hb][e] *= alpha;
      m_ref = m_new;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      s0[e] = __builtin_amdgcn_exp2f(s0[e]);
      s1[e] = __builtin_amdgcn_exp2f(s1[e]);
    }
    bf16x8_t pf[4];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      pf[0][i] = static_cast<__bf16>(s0[i]);
      pf[1][i] = static_cast<__bf16>(s0[8 + i]);
      pf[2][i] = static_cast<__bf16>(s1[i]);
      pf[3][i] = static_cast<__bf16>(s1[8 + i]);
    }
    // the denominator sums the same bf16 probabilities the P.V product weighs the values with, so the output
    // stays a convex combination of the values (a dominant key returns its value exactly)
    {
      float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const u32x4_t w = __builtin_bit_cast(u32x4_t, pf[i]);
#pragma unroll
        for (int j = 0; j < 4; ++j) rs[j] += bf_lo(w[j]) + bf_hi(w[j]);
      }
      l_run += (rs[0] + rs[1]) + (rs[2] + rs[3]);
    }
#pragma unroll
    for (int hb = 0; hb < 4; ++hb)
#pragma unroll
      for (int cc = 0; cc < 4; ++cc) {
        const bf16x8_t a =
            *reinterpret_cast<const bf16x8_t*>(Vt + hb * 32 * kKB + (vtbase ^ (((2 * cc) ^ (4 * (hb & 1))) << 3)));
        acc[hb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[cc], acc[hb], 0, 0, 0);
      }
  };

  // one tile: prefetch the next into registers, compute from LDS buffer `buf`, stage the next into the other
  // buffer.  Two tiles per loop trip so that the buffer (and every LDS address) is a compile-time constant.
  // Tile kt (LDS buffer buf, the parity of kt - kt_lo): register set buf ^ 1 holds tile kt + 1 (loaded one
  // tile earlier), and set buf takes tile kt + 2 (the last tile is reloaded past the end: no branch around
  // the loads); compute from LDS, then store tile kt + 1 into the other buffer.
  auto tile = [&](auto bufc, int kt) {
    constexpr int buf = decltype(bufc)::value;
    const int k2 = kt + 2 <= kt_hi ? kt + 2 : kt_hi;
    if constexpr (buf == 0) gload(k2, sv0);
    else gload(k2, sv1);
    const int k_first = kt * kKB, k_last = k_first + kKB - 1;
    if (wave_live && k_first <= q_hi && k_last >= q_lo - p.window)
      compute(bufc, kt, k_last > q_lo || k_first < q_hi - p.window);
    if (kt < kt_hi) {
      if constexpr (buf == 0) lstore(std::integral_constant<int, 1>{}, sv1);
      else lstore(std::integral_constant<int, 0>{}, sv0);
    }
    __syncthreads();
  };
  gload(kt_lo, sv0);
  gload(kt_lo + 1 <= kt_hi ? kt_lo + 1 : kt_hi, sv1);
  lstore(std::integral_constant<int, 0>{}, sv0);
  __syncthreads();
  for (int kt = kt_lo; kt <= kt_hi; kt += 2) {
    tile(std::integral_constant<int, 0>{}, kt);
    if (kt + 1 <= kt_hi) tile(std::integral_constant<int, 1>{}, kt + 1);
  }

  if (!wave_live) return;
  float lt;
  {
    const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l_run), __float_as_uint(l_run), false, false);
    lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  }
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  constexpr uint32_t esz = sizeof(Tout);
  const uint32_t orow = static_cast<uint32_t>(p.heads) * kHD * esz;
  const rsrc_t ro = rsrc_rows(static_cast<Tout*>(p.o) + (sb.t0 + q_lo) * p.heads * kHD + head_off, q_hi - q_lo + 1,
                              orow);
#pragma unroll
  for (int hb = 0; hb < 4; ++hb)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const uint32_t off = static_cast<uint32_t>(ql) * orow + (32 * hb + 8 * g + 4 * hf) * esz;
      const float v0 = acc[hb][4 * g] * inv, v1 = acc[hb][4 * g + 1] * inv, v2 = acc[hb][4 * g + 2] * inv,
                  v3 = acc[hb][4 * g + 3] * inv;
      if constexpr (esz == 2) {
        const u32x2_t w = {pack_bf16(v0, v1), pack_bf16(v2, v3)};
        __builtin_amdgcn_raw_buffer_store_b64(w, ro, off, 0, 0);
      } else {
        const u32x4_t w = {__float_as_uint(v0), __float_as_uint(v1), __float_as_uint(v2), __float_as_uint(v3)};
        __builtin_amdgcn_raw_buffer_store_b128(w, ro, off, 0, 0);
      }
    }
}

// ---------------------------------------------------------------------------
// Decode step
// ---------------------------------------------------------------------------
struct DecParams {
  const uint16_t *q, *k, *v;
  uint16_t *kc, *vc;
  void* o;
  const int32_t* pos;
  int32_t heads, window, cache_len, step;   // step = 16 % cache_len
  float c;
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
// sum over the 16 lanes of a DPP row, in every lane of the row
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dpp<0x124>(v);   // row_ror 4
  v += dpp<0x128>(v);   // row_ror 8
  return v;
}

__device__ __forceinline__ float dot8(const float (&q)[8], uint4 w) {
  float d = q[0] * bf_lo(w.x);
  d = fmaf(q[1], bf_hi(w.x), d);
  d = fmaf(q[2], bf_lo(w.y), d);
  d = fmaf(q[3], bf_hi(w.y), d);
  d = fmaf(q[4], bf_lo(w.z), d);
  d = fmaf(q[5], bf_hi(w.z), d);
  d = fmaf(q[6], bf_lo(w.w), d);
  d = fmaf(q[7], bf_hi(w.w), d);
  return d;
}
__device__ __forceinline__ void axpy8(float (&a)[8], float p, uint4 w) {
  a[0] = fmaf(p, bf_lo(w.x), a[0]);
  a[1] = fmaf(p, bf_hi(w.x), a[1]);
  a[2] = fmaf(p, bf_lo(w.y), a[2]);
  a[3] = fmaf(p, bf_hi(w.y), a[3]);
  a[4] = fmaf(p, bf_lo(w.z), a[4]);
  a[5] = fmaf(p, bf_hi(w.z), a[5]);
  a[6] = fmaf(p, bf_lo(w.w), a[6]);
  a[7] = fmaf(p, bf_hi(w.w), a[7]);
}

constexpr int kDecGroups = 16;   // 16-lane groups per workgroup
constexpr int kDecBatch = 8;     // keys per group per step

// One workgroup of 256 threads per (sequence, head): blockIdx.x = b * heads + h.
template <typename Tout>
__global__ __launch_bounds__(256) void swa_decode_kernel(DecParams p) {
  __shared__ float s_acc[kDecGroups][kHD];
  __shared__ float s_ml[kDecGroups][2];
  const int bh = blockIdx.x;
  const int b = bh / p.heads;
  const int tid = threadIdx.x, gi = tid >> 4, li = tid & 15;
  int32_t pos = p.pos[b];
  pos = pos < 0 ? 0 : pos;
  const int32_t lo = (pos - p.window > 0) ? pos - p.window : 0;
  const int64_t row = static_cast<int64_t>(bh) * kHD + 8 * li;
  const uint4 qw = *reinterpret_cast<const uint4*>(p.q + row);
  const float qv[8] = {bf_lo(qw.x), bf_hi(qw.x), bf_lo(qw.y), bf_hi(qw.y),
                       bf_lo(qw.z), bf_hi(qw.z), bf_lo(qw.w), bf_hi(qw.w)};
  const uint4 kn = *reinterpret_cast<const uint4*>(p.k + row);
  const uint4 vn = *reinterpret_cast<const uint4*>(p.v + row);
  const int64_t cache_base = static_cast<int64_t>(bh) * p.cache_len * kHD;
  const int32_t new_slot = pos % p.cache_len;
  if (gi == 0) *reinterpret_cast<uint4*>(p.kc + cache_base + static_cast<int64_t>(new_slot) * kHD + 8 * li) = kn;
  if (gi == 1) *reinterpret_cast<uint4*>(p.vc + cache_base + static_cast<int64_t>(new_slot) * kHD + 8 * li) = vn;

  // group 0 starts from the new token itself; the others from nothing
  float m, l, acc[8];
  {
    const float s = row16_sum(dot8(qv, kn)) * p.c;
    if (gi == 0) {
      m = s;
      l = 1.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
      axpy8(acc, 1.f, vn);
    } else {
      m = -INFINITY;
      l = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
  }
  // cached keys lo .. pos - 1: group gi takes lo + gi + 16 n
  const rsrc_t rk = rsrc_rows(p.kc + cache_base, p.cache_len, kHD * 2);
  const rsrc_t rv = rsrc_rows(p.vc + cache_base, p.cache_len, kHD * 2);
  const int32_t nkeys = pos - lo;
  int32_t slot = (lo + gi) % p.cache_len;
  for (int32_t base = 0; base < nkeys; base += kDecGroups * kDecBatch) {
    uint4 kw[kDecBatch], vw[kDecBatch];
    bool valid[kDecBatch];
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) {
      valid[u] = base + gi + kDecGroups * u < nkeys;
      const uint32_t off = static_cast<uint32_t>(slot) * (kHD * 2) + li * 16;
      kw[u] = ld16(rk, off);
      vw[u] = ld16(rv, off);
      slot += p.step;
      slot = slot >= p.cache_len ? slot - p.cache_len : slot;
    }
    float s[kDecBatch];
    float mb = -INFINITY;
#pragma unroll
    for (int u = 0; u < kDecBatch; ++u) {
      const float d = row16_sum(dot8(qv, kw[u])) * p.c;
      s[u] = valid[u] ? d : -INFINITY;
      mb = fmaxf(mb, s[u]);
    }
    const float m_new = fmaxf(m, mb);
    if (m_new != -INFINITY) {   // uniform within the group
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] *= alpha;
#pragma unroll
      for (int u = 0; u < kDecBatch; ++u) {
        const float pu = __builtin_amdgcn_exp2f(s[u] - m_new);
        l += pu;
        axpy8(acc, pu, vw[u]);
      }
      m = m_new;
    }
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) s_acc[gi][8 * li + i] = acc[i];
  if (li == 0) {
    s_ml[gi][0] = m;
    s_ml[gi][1] = l;
  }
  __syncthreads();
  if (tid < kHD) {
    float M = -INFINITY;
#pragma unroll
    for (int g = 0; g < kDecGroups; ++g) M = fmaxf(M, s_ml[g][0]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int g = 0; g < kDecGroups; ++g) {
      const float w = s_ml[g][0] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_ml[g][0] - M);
      num = fmaf(w, s_acc[g][tid], num);
      den = fmaf(w, s_ml[g][1], den);
    }
    const float out = num / den;
    if constexpr (sizeof(Tout) == 2)
      static_cast<uint16_t*>(p.o)[static_cast<int64_t>(bh) * kHD + tid] =
          __builtin_bit_cast(uint16_t, static_cast<__bf16>(out));
    else
      static_cast<float*>(p.o)[static_cast<int64_t>(bh) * kHD + tid] = out;
  }
}

// ---------------------------------------------------------------------------
// host side
// ---------------------------------------------------------------------------
bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, size_t na, const void* b, size_t nb) {
  if (!a || !b || na == 0 || nb == 0) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

bool dtype_ok(int32_t dt) { return dt == SAMBA_F32 || dt == SAMBA_BF16; }

// Common shape rules of a token batch: sizes >= 0, offsets only with batch 1.
samba_status token_shape(int32_t batch, int32_t seqlen, const int32_t* cu, int32_t nseq, int64_t* nblocks_seq,
                         int shift, int32_t* per_seq) {
  if (batch < 0 || seqlen < 0 || nseq < 0) return SAMBA_ERR_BAD_SHAPE;
  const int64_t blk = int64_t{1} << shift;
  if (cu) {
    if (batch != 1 || nseq < 1) return SAMBA_ERR_BAD_SHAPE;
    *per_seq = 0;
    *nblocks_seq = nseq == 0 ? 0 : (static_cast<int64_t>(seqlen) >> shift) + nseq;
  } else {
    *per_seq = static_cast<int32_t>((seqlen + blk - 1) / blk);
    *nblocks_seq = static_cast<int64_t>(batch) * *per_seq;
  }
  return SAMBA_OK;
}

}  // namespace

extern "C" {

samba_status samba_rope(const samba_rope_args* a, void* stream) {
  if (!a) return SAMBA_ERR_NULL_ARG;
  if (a->struct_size != sizeof(samba_rope_args)) return SAMBA_ERR_BAD_STRUCT;
  RopeParams p{};
  int64_t nblk = 0;
  if (a->heads < 1 || a->head_dim < 16 || a->head_dim % 16 != 0 || a->head_dim > 4096 || a->npos < 1 ||
      static_cast<int64_t>(a->heads) * a->head_dim > (1 << 20))
    return SAMBA_ERR_BAD_SHAPE;
  // head groups: 8, or as many as fit 256 threads for one token (head_dim > 512); tokens per workgroup: the
  // largest power of two whose threads fit 256
  const int cph = a->head_dim / 16;
  p.groups = cph * kRopeGroups <= 256 ? kRopeGroups : 256 / cph;
  int shift = 0;
  while ((2 << shift) * p.groups * cph <= 256) ++shift;
  p.shift = shift;
  samba_status st = token_shape(a->batch, a->seqlen, a->cu_seqlens, a->nseq, &nblk, shift, &p.per_seq);
  if (st != SAMBA_OK) return st;
  const int64_t tokens = static_cast<int64_t>(a->batch) * a->seqlen;
  const size_t bytes = static_cast<size_t>(tokens) * a->heads * a->head_dim * 2;
  if (nblk == 0 || tokens == 0) return SAMBA_OK;
  if (!a->cos || !a->sin) return SAMBA_ERR_NULL_ARG;
  if ((a->q_in && !a->q_out) || (a->k_in && !a->k_out) || (!a->q_in && a->q_out) || (!a->k_in && a->k_out))
    return SAMBA_ERR_NULL_ARG;
  if (!aligned(a->q_in, 16) || !aligned(a->k_in, 16) || !aligned(a->q_out, 16) || !aligned(a->k_out, 16) ||
      !aligned(a->cos, 16) || !aligned(a->sin, 16))
    return SAMBA_ERR_MISALIGNED;
  const size_t tbytes = static_cast<size_t>(a->npos) * (a->head_dim / 2) * 4;
  const void* outs[2] = {a->q_out, a->k_out};
  const void* ins[2] = {a->q_in, a->k_in};
  for (int i = 0; i < 2; ++i) {
    if (!outs[i]) continue;
    if (overlap(outs[i], bytes, a->cos, tbytes) || overlap(outs[i], bytes, a->sin, tbytes)) return SAMBA_ERR_ALIASING;
    if (a->cu_seqlens && overlap(outs[i], bytes, a->cu_seqlens, (static_cast<size_t>(a->nseq) + 1) * 4))
      return SAMBA_ERR_ALIASING;
    if (a->pos0 && overlap(outs[i], bytes, a->pos0, static_cast<size_t>(a->nseq > 0 ? a->nseq : a->batch) * 4))
      return SAMBA_ERR_ALIASING;
    for (int k = 0; k < 2; ++k)
      if (ins[k] && overlap(outs[i], bytes, ins[k], bytes) && !(k == i && outs[i] == ins[k])) return SAMBA_ERR_ALIASING;
    if (i == 0 && outs[1] && overlap(outs[0], bytes, outs[1], bytes)) return SAMBA_ERR_ALIASING;
  }
  if (nblk > 0x7fffffff) return SAMBA_ERR_BAD_SHAPE;
  p.qi = static_cast<const uint16_t*>(a->q_in);
  p.ki = static_cast<const uint16_t*>(a->k_in);
  p.qo = static_cast<uint16_t*>(a->q_out);
  p.ko = static_cast<uint16_t*>(a->k_out);
  p.cs = a->cos;
  p.sn = a->sin;
  p.cu = a->cu_seqlens;
  p.pos0 = a->pos0;
  p.nseq = a->nseq;
  p.seqlen = a->seqlen;
  p.heads = a->heads;
  p.hd = a->head_dim;
  p.npos = a->npos;
  p.total = a->seqlen;
  if (!p.qi && !p.ki) return SAMBA_OK;
  const dim3 grid(static_cast<uint32_t>(nblk));
  const hipStream_t sm = static_cast<hipStream_t>(stream);
  if (p.qi && p.ki) hipLaunchKernelGGL((rope_kernel<true, true>), grid, dim3(256), 0, sm, p);
  else if (p.qi) hipLaunchKernelGGL((rope_kernel<true, false>), grid, dim3(256), 0, sm, p);
  else hipLaunchKernelGGL((rope_kernel<false, true>), grid, dim3(256), 0, sm, p);
  return hipGetLastError() == hipSuccess ? SAMBA_OK : SAMBA_ERR_HIP;
}

samba_status samba_swa_fwd(const samba_swa_fwd_args* a, void* stream) {
  if (!a) return SAMBA_ERR_NULL_ARG;
  if (a->struct_size != sizeof(samba_swa_fwd_args)) return SAMBA_ERR_BAD_STRUCT;
  SwaParams p{};
  int64_t nqb = 0;
  samba_status st = token_shape(a->batch, a->seqlen, a->cu_seqlens, a->nseq, &nqb, kQBShift, &p.per_seq);
  if (st != SAMBA_OK) return st;
  if (a->heads < 1 || a->heads > 4096 || a->window < 0) return SAMBA_ERR_BAD_SHAPE;
  if (a->head_dim != kHD) return SAMBA_ERR_UNSUPPORTED;
  if (!dtype_ok(a->out_dtype)) return SAMBA_ERR_BAD_DTYPE;
  const int64_t tokens = static_cast<int64_t>(a->batch) * a->seqlen;
  if (nqb == 0 || tokens == 0) return SAMBA_OK;
  if (!a->q || !a->k || !a->v || !a->o) return SAMBA_ERR_NULL_ARG;
  if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->o, a->out_dtype == SAMBA_BF16 ? 2 : 4))
    return SAMBA_ERR_MISALIGNED;
  const size_t in_bytes = static_cast<size_t>(tokens) * a->heads * kHD * 2;
  const size_t out_bytes = in_bytes / 2 * (a->out_dtype == SAMBA_BF16 ? 2 : 4);
  if (overlap(a->o, out_bytes, a->q, in_bytes) || overlap(a->o, out_bytes, a->k, in_bytes) ||
      overlap(a->o, out_bytes, a->v, in_bytes) ||
      (a->cu_seqlens && overlap(a->o, out_bytes, a->cu_seqlens, (static_cast<size_t>(a->nseq) + 1) * 4)))
    return SAMBA_ERR_ALIASING;
  if (nqb * a->heads > 0x7fffffff) return SAMBA_ERR_BAD_SHAPE;
  p.q = static_cast<const uint16_t*>(a->q);
  p.k = static_cast<const uint16_t*>(a->k);
  p.v = static_cast<const uint16_t*>(a->v);
  p.o = a->o;
  p.cu = a->cu_seqlens;
  p.nseq = a->nseq;
  p.seqlen = a->seqlen;
  p.heads = a->heads;
  p.window = a->window;
  p.nqb = static_cast<int32_t>(nqb);
  p.total = a->seqlen;
  p.c = kLog2e / sqrtf(static_cast<float>(kHD));
  const dim3 grid(static_cast<uint32_t>(nqb * a->heads));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (a->out_dtype == SAMBA_BF16) hipLaunchKernelGGL(swa_fwd_kernel<uint16_t>, grid, dim3(kSwaThreads), 0, s, p);
  else hipLaunchKernelGGL(swa_fwd_kernel<float>, grid, dim3(kSwaThreads), 0, s, p);
  return hipGetLastError() == hipSuccess ? SAMBA_OK : SAMBA_ERR_HIP;
}

samba_status samba_swa_decode(const samba_swa_decode_args* a, void* stream) {
  if (!a) return SAMBA_ERR_NULL_ARG;
  if (a->struct_size != sizeof(samba_swa_decode_args)) return SAMBA_ERR_BAD_STRUCT;
  if (a->batch < 0 || a->heads < 1 || a->window < 0 || a->cache_len < 1) return SAMBA_ERR_BAD_SHAPE;
  if (a->head_dim != kHD) return SAMBA_ERR_UNSUPPORTED;
  if (a->cache_len < static_cast<int64_t>(a->window) + 1 || a->cache_len > (1 << 24)) return SAMBA_ERR_BAD_SHAPE;
  if (!dtype_ok(a->out_dtype)) return SAMBA_ERR_BAD_DTYPE;
  if (a->batch == 0) return SAMBA_OK;
  if (!a->pos || !a->q || !a->k || !a->v || !a->k_cache || !a->v_cache || !a->o) return SAMBA_ERR_NULL_ARG;
  if (!aligned(a->q, 16) || !aligned(a->k, 16) || !aligned(a->v, 16) || !aligned(a->k_cache, 16) ||
      !aligned(a->v_cache, 16) || !aligned(a->pos, 4) || !aligned(a->o, a->out_dtype == SAMBA_BF16 ? 2 : 4))
    return SAMBA_ERR_MISALIGNED;
  const int64_t bh = static_cast<int64_t>(a->batch) * a->heads;
  if (bh > 0x7fffffff) return SAMBA_ERR_BAD_SHAPE;
  const size_t row_bytes = static_cast<size_t>(bh) * kHD * 2;
  const size_t cache_bytes = row_bytes * static_cast<size_t>(a->cache_len);
  const size_t out_bytes = static_cast<size_t>(bh) * kHD * (a->out_dtype == SAMBA_BF16 ? 2 : 4);
  const size_t pos_bytes = static_cast<size_t>(a->batch) * 4;
  const void* ins[4] = {a->q, a->k, a->v, a->pos};
  const size_t in_sz[4] = {row_bytes, row_bytes, row_bytes, pos_bytes};
  const void* outs[3] = {a->o, a->k_cache, a->v_cache};
  const size_t out_sz[3] = {out_bytes, cache_bytes, cache_bytes};
  for (int i = 0; i < 3; ++i) {
    for (int k = 0; k < 4; ++k)
      if (overlap(outs[i], out_sz[i], ins[k], in_sz[k])) return SAMBA_ERR_ALIASING;
    for (int k = i + 1; k < 3; ++k)
      if (overlap(outs[i], out_sz[i], outs[k], out_sz[k])) return SAMBA_ERR_ALIASING;
  }
  DecParams p{};
  p.q = static_cast<const uint16_t*>(a->q);
  p.k = static_cast<const uint16_t*>(a->k);
  p.v = static_cast<const uint16_t*>(a->v);
  p.kc = static_cast<uint16_t*>(a->k_cache);
  p.vc = static_cast<uint16_t*>(a->v_cache);
  p.o = a->o;
  p.pos = a->pos;
  p.heads = a->heads;
  p.window = a->window;
  p.cache_len = a->cache_len;
  p.step = 16 % a->cache_len;
  p.c = kLog2e / sqrtf(static_cast<float>(kHD));
  const hipStream_t s = static_cast<hipStream_t>(stream);
  if (a->out_dtype == SAMBA_BF16) hipLaunchKernelGGL(swa_decode_kernel<uint16_t>, dim3(static_cast<uint32_t>(bh)), dim3(256), 0, s, p);
  else hipLaunchKernelGGL(swa_decode_kernel<float>, dim3(static_cast<uint32_t>(bh)), dim3(256), 0, s, p);
  return hipGetLastError() == hipSuccess ? SAMBA_OK : SAMBA_ERR_HIP;
}

}  // extern "C"
