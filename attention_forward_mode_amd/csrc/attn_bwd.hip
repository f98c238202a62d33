// attn_bwd.hip -- reverse-mode derivative (backward pass) of softmax attention
// for gfx950, bf16 inputs: FlashAttention-2's gradients of a loss through O.
//
// Per (b, h), with S = s Q K^T, P = row-softmax(S) = exp(S - lse), O = P V and
// the incoming gradient gO (of the loss with respect to O):
//   gV = P^T gO,  gP = gO V^T,  gS = P * (gP - D),  D_i = sum_j P_ij gP_ij = <gO_i, O_i>,
//   gQ = s gS K,  gK = s gS^T Q.
// (rCM record LIT-783 in the Anthology of the SOTA: the student is trained
// through the attention output, "Key takeaways", "JVP at production scale".)
//
// Kernels per call, all on one stream:
//  0. range_stats (range.hpp), twice: per (b, h) the largest finite |Q|, |gO|
//     and |K|, from which the packs take per-slice powers of two 2^eQ, 2^eG,
//     2^eK that put Q^T, gO^T and K^T into fp16's upper range.
//  1. pack_q: per 64 queries, a tile image of Q and gO rows (bf16, padded),
//     Q^T 2^eQ and gO^T 2^eG (fp16, [d][64 queries] in matrix-core operand
//     order), and per query lse (+inf past Nq) and D = <gO_i, O_i> (fp32, from
//     O); the slice's largest |gO_i| and |D_i| go to its header.
//  2. pack_k: per 64 keys, a tile image of K and V rows (bf16) and K^T 2^eK
//     (fp16); the slice's largest |v_j| goes to its header.
//  3. bwd_kv: one workgroup = 8 waves x 32 keys (K, V fragments held in
//     registers); it streams the query tiles (direct-to-LDS copies, double
//     buffered) and per 32-query block forms S = Q K^T and gP = gO V^T (bf16
//     MFMA), P = exp(S - lse), gS 2^t = P 2^t (gP - D) (rounded to fp16
//     pairs), and accumulates gV^T += gO^T P and gK^T += Q^T gS (fp16 MFMA).
//  4. bwd_q: one workgroup = 8 waves x 32 queries (Q, gO fragments held in
//     registers); it streams the key tiles and per 32-key block forms
//     S^T = K Q^T, gP^T = V gO^T, P^T, gS^T 2^t, and accumulates
//     gQ^T += K^T gS^T.
// The tangent-free analogue of the forward's s P dS scaling: with P <= 1,
// |gS_ij| <= |gO_i| |v_j| + |D_i| (Cauchy-Schwarz), and each wave takes t
// from that bound over its keys (bwd_kv) or its queries (bwd_q) so that gS 2^t
// stays below 4000; the stores undo 2^t and the image exponents exactly.
// Every access to global memory is a buffer access range-checked against its
// tensor (or one (b, h) slice of the workspace).  Products: 8 (bwd_kv) + 6
// (bwd_q) Nq x Nk x d contractions' worth of flops, S and gP formed twice.
#include "cdna4.hpp"
#include "launch.hpp"
#include "range.hpp"

namespace ajvp {
namespace bwd_path {

constexpr int kTile = 64;            // keys or queries per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRows = 32 * kWaves;   // keys (bwd_kv) or queries (bwd_q) per workgroup
constexpr int kPackThreads = 256;
constexpr int kDmaBytes = 1024;
constexpr uint32_t kXcds = 8;

// A tile image: NR row tiles (bf16, [64][d], rows padded by 16 bytes), NT
// transposed tiles (fp16, [d][64], positions in operand order, rows padded),
// and kExtra bytes of per-row data, rounded up to 8 KiB.
template <int D, int NR, int NT, int kExtra>
struct Img {
  static constexpr int kRRow = D * 2 + 16;
  static constexpr int kTRow = kTile * 2 + 16;
  static constexpr int kRTile = kTile * kRRow;
  static constexpr int kTTile = D * kTRow;
  static constexpr int kOffT = NR * kRTile;
  static constexpr int kOffX = kOffT + NT * kTTile;
  static constexpr int kUsed = kOffX + kExtra;
  static constexpr int kRound = kThreads * 16;
  static constexpr int kBytes = (kUsed + kRound - 1) / kRound * kRound;
  static constexpr int kDmaPerWave = kBytes / (kWaves * kDmaBytes);
  static constexpr int kKS = D / 16;
  static constexpr int kCB = D / 32;
};
// query image: Q, gO rows; Q^T, gO^T; lse and D in accumulator-row order
template <int D>
using QImg = Img<D, 2, 2, 2 * kTile * 4>;
// key image: K, V rows; K^T
template <int D>
using KImg = Img<D, 2, 1, 0>;
static_assert(QImg<128>::kBytes == 73728 && KImg<128>::kBytes == 57344, "image sizes");

// Row (0..63) of a 64-row tile held at operand position `pos` of a transposed
// row: positions 16G + 8g + e hold the rows that the accumulator of lane half
// g puts in slots 8t + e of block G/2, t = G%2.
__device__ inline int packed_row(int pos) {
  const int G = pos >> 4, g = (pos >> 3) & 1, e = pos & 7;
  return 16 * G + (e < 4 ? 4 * g + e : 8 + 4 * g + (e - 4));
}
// Accumulator slot r of lane half g holds row 8(r/4) + 4g + r%4 of its block.
__device__ __attribute__((always_inline)) inline int slot_row(int r, int g) {
  return 8 * (r >> 2) + 4 * g + (r & 3);
}

// Bytes of one (b, h) slice of the query-side (kQuery) or key-side workspace:
// its tile images, then the header of range.hpp.  Query side: record =
// {eQ, eG}, norm maxima = {max_i |gO_i|, max_i |D_i|}; key side: record =
// {eK}, norm maxima = {max_j |v_j|, 0}.
template <int D, bool kQuery>
__host__ __device__ constexpr uint32_t slice_bytes(int ntiles) {
  using G = Img<D, 2, kQuery ? 2 : 1, kQuery ? 2 * kTile * 4 : 0>;
  return (uint32_t)ntiles * G::kBytes + kHdrBytes;
}

// One tile image (blockIdx.x = tile, blockIdx.y = (b, h)).  Rows past N are
// zero; with kQuery, the extras are lse (+inf past N) and D = <gO_i, O_i>,
// 32 floats per 32-row block in slot order (lane half g, slot r at 16 g + r).
// The transposed tiles hold t0 2^e0 and t1 2^e1 in fp16, e0, e1 from the
// range pass's maxima of t0, t1 (which every wave reduces itself); the
// workgroup of tile 0 writes them to the slice header, and every tile raises
// the header's maxima of |r1 row| and (kQuery) |D| to its own.
template <int D, bool kQuery>
__device__ __attribute__((always_inline)) inline void pack_body(
    const uint16_t* __restrict__ r0, const uint16_t* __restrict__ r1,
    const uint16_t* __restrict__ t0, const uint16_t* __restrict__ t1,
    const float* __restrict__ o, const float* __restrict__ lse, char* __restrict__ ws, int N,
    int ntiles, uint32_t in_bytes) {
  using G = Img<D, 2, kQuery ? 2 : 1, kQuery ? 2 * kTile * 4 : 0>;
  constexpr int NT = kQuery ? 2 : 1;
  __shared__ _Float16 sv[NT][kTile][D + 2];
  __shared__ float sd[kTile];
  __shared__ double sn[kTile];
  const int tile = blockIdx.x;
  const uint32_t bh = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const auto rr0 = make_rsrc(r0, in_bytes);
  const auto rr1 = make_rsrc(r1, in_bytes);
  const auto rt0 = make_rsrc(t0, in_bytes);
  const auto rt1 = make_rsrc(t1, kQuery ? in_bytes : 0u);
  const uint32_t slice = slice_bytes<D, kQuery>(ntiles);
  const uint32_t hdr = (uint32_t)ntiles * G::kBytes;
  const auto rws = make_rsrc(ws + (size_t)bh * slice, slice);
  const int row0 = tile * kTile;
  const uint32_t img = (uint32_t)tile * G::kBytes;
  constexpr int kC = D / 8;
  constexpr u32x4 kZero = {0u, 0u, 0u, 0u};
  uint32_t m0, m1;
  slice_maxima(rws, hdr, ntiles, lane, m0, m1);
  const int e0 = fp16_exponent(m0), e1 = kQuery ? fp16_exponent(m1) : 0;
  constexpr int kRChunks = kTile * (kC + 1);
  for (int c = threadIdx.x; c < 2 * kRChunks; c += kPackThreads) {
    const int t = c / kRChunks, rem = c % kRChunks, r = rem / (kC + 1), col = rem % (kC + 1);
    u32x4 x = kZero;
    if (col < kC && row0 + r < N)
      x = buf_load16(t == 0 ? rr0 : rr1, ((bh * (uint32_t)N + row0 + r) * D + 8 * col) * 2);
    buf_store16(rws, img + t * G::kRTile + r * G::kRRow + col * 16, x);
  }
  constexpr int kIn = kTile * kC;
  for (int c = threadIdx.x; c < NT * kIn; c += kPackThreads) {
    const int t = c / kIn, rem = c % kIn, r = rem / kC, col = (rem % kC) * 8;
    const int e_t = t == 0 ? e0 : e1;
    u32x4 x = kZero;
    if (row0 + r < N)
      x = buf_load16(t == 0 ? rt0 : rt1, ((bh * (uint32_t)N + row0 + r) * D + col) * 2);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t bits = (x[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      sv[t][r][col + e] = (_Float16)__builtin_amdgcn_ldexpf(__builtin_bit_cast(float, bits << 16), e_t);
    }
  }
  {
    // Per row of r1 (gO or V), four threads: the squared norm (fp64) and, with
    // kQuery, D_i = <gO_i, O_i> (fp32 sums of bf16 gO times fp32 O).
    static_assert(kTile * 4 == kPackThreads, "one row quarter per thread");
    const auto ro = make_rsrc(o, kQuery ? in_bytes * 2 : 0u);
    const int r = threadIdx.x / 4, part = threadIdx.x % 4;
    float acc = 0.f;
    double ss = 0.0;
    if (row0 + r < N) {
      for (int j = part * (D / 4); j < (part + 1) * (D / 4); j += 4) {
        const uint32_t e = (bh * (uint32_t)N + row0 + r) * D + j;
        const u32x2 gw = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rr1, (int)(e * 2), 0, 0));
        f32x4 ov = {0.f, 0.f, 0.f, 0.f};
        if constexpr (kQuery) ov = __builtin_bit_cast(f32x4, buf_load16(ro, e * 4));
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t bits = (gw[q >> 1] >> (16 * (q & 1))) & 0xffffu;
          const float gv = __builtin_bit_cast(float, bits << 16);
          if constexpr (kQuery) acc += gv * ov[q];
          ss = __builtin_fma((double)gv, (double)gv, ss);
        }
      }
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    if (part == 0) {
      sd[r] = acc;
      sn[r] = ss;
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    // the tile's largest row norm of r1 and |D| (NaN rows left out: fmax)
    double nmax = sn[threadIdx.x];
    float dmax = __builtin_fabsf(sd[threadIdx.x]);
    nmax = wave_max_f64(nmax);
    dmax = wave_max_f32(dmax);
    if (threadIdx.x == 0) {
      raise_norms(ws + (size_t)bh * slice + hdr, tile, round_up_f32(__builtin_sqrt(nmax)),
                  kQuery ? dmax : 0.f);
      if (tile == 0)
        buf_store16(rws, hdr + kHdrRecord, u32x4{(uint32_t)e0, (uint32_t)e1, 0u, 0u});
    }
  }
  for (int c = threadIdx.x; c < NT * D * 9; c += kPackThreads) {
    const int t = c / (D * 9), rem = c % (D * 9), col = rem / 9, p = rem % 9;
    u32x4 x = kZero;
    if (p < 8) {
      f16x8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = sv[t][packed_row(8 * p + e)][col];
      x = __builtin_bit_cast(u32x4, h);
    }
    buf_store16(rws, img + G::kOffT + t * G::kTTile + col * G::kTRow + p * 16, x);
  }
  if constexpr (kQuery) {
    // extras: [block b][lse log2 e | D][lane half g][slot r]
    const auto rl = make_rsrc(lse, in_bytes / D * 2);
    for (int c = threadIdx.x; c < 2 * kTile; c += kPackThreads) {
      const int which = c / kTile, rem = c % kTile;       // 0: lse, 1: D
      const int b = rem / 32, g = (rem / 16) % 2, r = rem % 16;
      const int row = 32 * b + slot_row(r, g);
      float val;
      if (which == 0)
        val = row0 + row < N ? buf_load4f(rl, (bh * (uint32_t)N + row0 + row) * 4) * kLog2e
                             : INFINITY;
      else
        val = sd[row];
      buf_store4(rws, img + G::kOffX + (b * 2 + which) * 128 + (g * 16 + r) * 4, val);
    }
  }
  for (int off = G::kUsed + threadIdx.x * 16; off < G::kBytes; off += kPackThreads * 16)
    buf_store16(rws, img + off, kZero);
}

template <int D, bool kQuery>
__global__ __launch_bounds__(kPackThreads) void pack_kernel(
    const uint16_t* __restrict__ r0, const uint16_t* __restrict__ r1,
    const uint16_t* __restrict__ t0, const uint16_t* __restrict__ t1,
    const float* __restrict__ o, const float* __restrict__ lse, char* __restrict__ ws, int N,
    int ntiles, uint32_t in_bytes) {
  pack_body<D, kQuery>(r0, r1, t0, t1, o, lse, ws, N, ntiles, in_bytes);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Copy of tile image t into a stage: this wave's kPer consecutive KiB, lane l
// moving bytes 16 l .. 16 l + 15 of each (LDS address = the wave-uniform stage
// pointer + 16 l; global = image offset + 16 l).
template <int kPer, int kBytes>
__device__ __attribute__((always_inline)) inline void copy_image(__amdgpu_buffer_rsrc_t rimg,
                                                                 char* stage, uint32_t wave_part,
                                                                 int lane, int t) {
#pragma unroll
  for (int j = 0; j < kPer; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rimg, (lds_ptr_t)(stage + wave_part + j * kDmaBytes),
                                             16, lane * 16,
                                             (uint32_t)t * kBytes + wave_part + j * kDmaBytes, 0, 0);
}

// Linear workgroup id -> (tile, slice): XCD x (id % 8) is given the x-th
// contiguous range of the work list ordered by (slice, tile).
__device__ __attribute__((always_inline)) inline void work_item(int ntile, int& tile,
                                                                uint32_t& bh) {
  const uint32_t wg = blockIdx.x, nwg = gridDim.x;
  const uint32_t xcd = wg % kXcds, slot = wg / kXcds, per = nwg / kXcds, extra = nwg % kXcds;
  const uint32_t w = xcd < extra ? xcd * (per + 1) + slot
                                 : extra * (per + 1) + (xcd - extra) * per + slot;
  tile = (int)(w % (uint32_t)ntile);
  bh = w / (uint32_t)ntile;
}

struct Sizes {
  uint32_t q_bytes, k_bytes, oq_bytes, ok_bytes;  // bf16 inputs, fp32 outputs
};

// Fragments of 32 rows of a [N, D] bf16 tensor as the B operand (lane: row
// l32, d-slice g); rows past N read zero.
template <int D>
__device__ __attribute__((always_inline)) inline void load_frags(__amdgpu_buffer_rsrc_t r,
                                                                 uint32_t row_off, bool ok,
                                                                 int g, u32x4* f) {
  const uint32_t base = ok ? row_off : 0x80000000u;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) f[ks] = buf_load16(r, base + (16 * ks + 8 * g) * 2);
}

// Store a [D][32] accumulator (4 blocks of 32x32; lane: column l32) as rows
// of a [N, D] fp32 tensor, times mul 2^-e (the accumulators hold their sums
// scaled by 2^e; the power of two is applied exactly, after the multiply).
template <int D>
__device__ __attribute__((always_inline)) inline void store_rows(__amdgpu_buffer_rsrc_t r,
                                                                 uint32_t row_elem,
                                                                 const f32x16* acc, int g,
                                                                 float mul, int e) {
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int c0 = 32 * cb + 8 * qq + 4 * g;
      f32x4 v;
#pragma unroll
      for (int k = 0; k < 4; ++k) v[k] = __builtin_amdgcn_ldexpf(acc[cb][4 * qq + k] * mul, -e);
      buf_store16(r, (row_elem + c0) * 4, __builtin_bit_cast(u32x4, v));
    }
}

// The wave's exponent t for gS 2^t from per-lane bounds of |gS| (rows or keys
// whose bound is not finite hold Inf or NaN inputs and do not take part),
// capped so that the operand scaled by 2^t (norm `norm` per lane) stays
// finite in bf16.
__device__ __attribute__((always_inline)) inline int gs_exponent(double bound, double norm) {
  const int t = product_exponent(wave_max_f64(__builtin_isfinite(bound) ? bound : 0.0));
  const int cap = cap_exponent(wave_max_f64(__builtin_isfinite(norm) ? norm : 0.0));
  return __builtin_amdgcn_readfirstlane(t < cap ? t : cap);
}

// The row norm of 32 rows held as B-operand fragments (lane: row l32, d-slice
// g), in fp64, in every lane of the row.
template <int D>
__device__ __attribute__((always_inline)) inline double frag_row_norm(const u32x4* f) {
  double ss = 0.0;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) ss += sumsq8(f[ks]);
  return __builtin_sqrt(halves_sum_f64(ss));
}

// ---- bwd_kv: gK, gV for 256 keys per workgroup --------------------------------
template <int D, bool kMaskQ>
__device__ __attribute__((always_inline)) inline void kv_block(
    const char* stage, int qb, const u32x4* kf, const u32x4* vf, int l32, int g,
    f32x16* gk, f32x16* gv, float c_log2, float gs_mul) {
  using G = QImg<D>;
  const char* sQ = stage;
  const char* sGO = stage + G::kRTile;
  const char* sQT = stage + G::kOffT;
  const char* sGOT = sQT + G::kTTile;
  const char* sX = stage + G::kOffX + qb * 256 + g * 64;  // lse log2 e at +0, D at +128
  const int rowoff = (32 * qb + l32) * G::kRRow + 16 * g;
  // S = Q K^T, gP = gO V^T (rows: query, columns: this wave's keys)
  f32x16 s, gp;
#pragma unroll
  for (int ks = 0; ks < G::kKS; ++ks) {
    const u32x4 qa = lds_load16(sQ + rowoff + 32 * ks);
    const u32x4 ga = lds_load16(sGO + rowoff + 32 * ks);
    s = mma_bf16(qa, kf[ks], ks == 0 ? f32x16{} : s);
    gp = mma_bf16(ga, vf[ks], ks == 0 ? f32x16{} : gp);
    __builtin_amdgcn_sched_barrier(0);
  }
  // P = 2^(S c - lse log2 e) (queries past Nq have lse = +inf, so P = 0 there),
  // gS 2^t = P (gP 2^t - D 2^t), gP 2^t from the wave's V fragments scaled by
  // 2^t; both rounded to fp16 pairs straight into B operands.
  u32x4 pb[2], sb[2];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const f32x4 l4 = __builtin_bit_cast(f32x4, lds_load16(sX + 16 * q4));
    const f32x4 d4 = __builtin_bit_cast(f32x4, lds_load16(sX + 128 + 16 * q4));
    float pp[4], gs[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int r = 4 * q4 + e;
      pp[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, -l4[e]));
      gs[e] = pp[e] * __builtin_fmaf(-d4[e], gs_mul, gp[r]);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int q = 2 * q4 + e;
      pb[q >> 2][q & 3] = pack_f16x2(pp[2 * e], pp[2 * e + 1]);
      sb[q >> 2][q & 3] = pack_f16x2(gs[2 * e], gs[2 * e + 1]);
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // gV^T += gO^T P, gK^T += Q^T gS
  constexpr int kSteps = 2 * G::kCB;
  auto toff = [&](int step) {
    const int t = step / G::kCB, cb = step % G::kCB;
    return (32 * cb + l32) * G::kTRow + 16 * g + 16 * (4 * qb + 2 * t);
  };
#pragma unroll
  for (int step = 0; step < kSteps; ++step) {
    const int t = step / G::kCB, cb = step % G::kCB;
    const u32x4 go_t = lds_load16(sGOT + toff(step));
    const u32x4 q_t = lds_load16(sQT + toff(step));
    gv[cb] = mma_f16(go_t, pb[t], gv[cb]);
    gk[cb] = mma_f16(q_t, sb[t], gk[cb]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One query tile: the copy of the next tile image into `next` goes first, then
// both 32-query blocks from `cur`.  The stage pointers are restrict-qualified
// (disjoint halves of the LDS), so reads of `cur` need not wait for the copy.
template <int D>
__device__ __attribute__((always_inline)) inline void kv_tile(
    char* __restrict__ next, const char* __restrict__ cur, __amdgpu_buffer_rsrc_t rimg,
    uint32_t wave_part, int lane, int t_next, bool copy, const u32x4* kf, const u32x4* vf,
    int l32, int g, f32x16* gk, f32x16* gv, float c_log2, float gs_mul) {
  using G = QImg<D>;
  if (copy) copy_image<G::kDmaPerWave, G::kBytes>(rimg, next, wave_part, lane, t_next);
  kv_block<D, false>(cur, 0, kf, vf, l32, g, gk, gv, c_log2, gs_mul);
  kv_block<D, false>(cur, 1, kf, vf, l32, g, gk, gv, c_log2, gs_mul);
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_kv_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const char* __restrict__ qimg, float* __restrict__ gk, float* __restrict__ gv, int Nq,
    int Nk, int nqtiles, int nktile, int nsplit, Sizes sz, float scale, float c_log2) {
  using G = QImg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * G::kBytes];
  // work item: key tile kt of slice bh, over query tiles [t0, t1) of split
  // `split`; with several splits the outputs are partial sums, one array each
  int tile;
  uint32_t bh;
  work_item(nktile * nsplit, tile, bh);
  const int kt = tile % nktile, split = tile / nktile;
  const int t0 = split * nqtiles / nsplit, t1 = (split + 1) * nqtiles / nsplit;
  const size_t part = (size_t)split * (sz.ok_bytes / 4);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int key = kt * kRows + wave * 32 + l32;
  const bool key_ok = key < Nk;
  const uint32_t slice = slice_bytes<D, true>(nqtiles);
  const uint32_t hdr = (uint32_t)nqtiles * G::kBytes;
  const auto rimg = make_rsrc(qimg + (size_t)bh * slice, slice);
  const uint32_t wave_part = (uint32_t)wave * G::kDmaPerWave * kDmaBytes;
  copy_image<G::kDmaPerWave, G::kBytes>(rimg, smem, wave_part, lane, t0);
  u32x4 kf[G::kKS], vf[G::kKS];
  const uint32_t krow = (bh * (uint32_t)Nk + key) * D * 2;
  load_frags<D>(make_rsrc(k, sz.k_bytes), krow, key_ok, g, kf);
  load_frags<D>(make_rsrc(v, sz.k_bytes), krow, key_ok, g, vf);
  // the query side's exponents eQ (Q^T) and eG (gO^T) and maxima of |gO_i|,
  // |D_i|; t from |gS_ij| <= max|gO_i| |v_j| + max|D_i| over this wave's keys
  const u32x4 rec = buf_load16(rimg, hdr + kHdrRecord);
  float mg, md;
  slice_norms(rimg, hdr, nqtiles, lane, mg, md);
  const int eq = __builtin_amdgcn_readfirstlane((int)rec[0]);
  const int eg = __builtin_amdgcn_readfirstlane((int)rec[1]);
  const double vn = frag_row_norm<D>(vf);
  const int t = gs_exponent((double)mg * vn + (double)md, vn);
  const float gs_mul = __builtin_amdgcn_ldexpf(1.0f, t);
#pragma unroll
  for (int ks = 0; ks < G::kKS; ++ks) vf[ks] = scale_bf16x8(vf[ks], t);
  f32x16 acc_k[G::kCB], acc_v[G::kCB];
#pragma unroll
  for (int cb = 0; cb < G::kCB; ++cb) {
    acc_k[cb] = f32x16{};
    acc_v[cb] = f32x16{};
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // the copy into the other stage starts once every wave has left the tile
  // that last read it (the barrier at the end of each tile)
  for (int qt = t0; qt < t1; ++qt) {
    const int i = qt - t0;
    kv_tile<D>(smem + ((i + 1) & 1) * G::kBytes, smem + (i & 1) * G::kBytes, rimg, wave_part,
               lane, qt + 1, qt + 1 < t1, kf, vf, l32, g, acc_k, acc_v, c_log2, gs_mul);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  if (key_ok) {
    const uint32_t row = (bh * (uint32_t)Nk + key) * D;
    store_rows<D>(make_rsrc(gk + part, sz.ok_bytes), row, acc_k, g, scale, eq + t);
    store_rows<D>(make_rsrc(gv + part, sz.ok_bytes), row, acc_v, g, 1.0f, eg);
  }
}

// ---- bwd_q: gQ for 256 queries per workgroup --------------------------------
template <int D, bool kMaskK, typename Issue>
__device__ __attribute__((always_inline)) inline void q_block(
    const char* stage, int kb, const u32x4* qf, const u32x4* gof, int l32, int g, f32x16* gq,
    float c_log2, float lse2, float dq, int key0, int Nk, Issue issue) {
  using G = KImg<D>;
  const char* sK = stage;
  const char* sV = stage + G::kRTile;
  const char* sKT = stage + G::kOffT;
  const int rowoff = (32 * kb + l32) * G::kRRow + 16 * g;
  // S^T = K Q^T, gP^T = V gO^T (rows: key, columns: this wave's queries)
  f32x16 s, gp;
#pragma unroll
  for (int ks = 0; ks < G::kKS; ++ks) {
    issue(ks);
    const u32x4 ka = lds_load16(sK + rowoff + 32 * ks);
    const u32x4 va = lds_load16(sV + rowoff + 32 * ks);
    s = mma_bf16(ka, qf[ks], ks == 0 ? f32x16{} : s);
    gp = mma_bf16(va, gof[ks], ks == 0 ? f32x16{} : gp);
    __builtin_amdgcn_sched_barrier(0);
  }
  // gS^T 2^t = P^T (gP^T 2^t - D 2^t), P^T = 2^(S^T c - lse log2 e), gP^T 2^t
  // from the wave's gO fragments scaled by 2^t; keys past Nk: 0
  u32x4 sb[2];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    float gs[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 2 * q + e;
      float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, -lse2));
      if (kMaskK && key0 + slot_row(r, g) >= Nk) p = 0.f;
      gs[e] = p * (gp[r] - dq);
    }
    sb[q >> 2][q & 3] = pack_f16x2(gs[0], gs[1]);
  }
  __builtin_amdgcn_sched_barrier(0);
  // gQ^T += K^T gS^T, each K^T fragment read one step ahead
  constexpr int kSteps = 2 * G::kCB;
  auto koff = [&](int step) {
    const int t = step / G::kCB, cb = step % G::kCB;
    return (32 * cb + l32) * G::kTRow + 16 * g + 16 * (4 * kb + 2 * t);
  };
  u32x4 ktp[2];
  ktp[0] = lds_load16(sKT + koff(0));
#pragma unroll
  for (int step = 0; step < kSteps; ++step) {
    const int t = step / G::kCB, cb = step % G::kCB;
    if (step + 1 < kSteps) ktp[(step + 1) & 1] = lds_load16(sKT + koff(step + 1));
    gq[cb] = mma_f16(ktp[step & 1], sb[t], gq[cb]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D>
__device__ __attribute__((always_inline)) inline void q_tile(
    char* __restrict__ next, const char* __restrict__ cur, __amdgpu_buffer_rsrc_t rimg,
    uint32_t wave_part, int lane, int t_next, const u32x4* qf, const u32x4* gof, int l32, int g,
    f32x16* gq, float c_log2, float lse2, float dq, int Nk) {
  using G = KImg<D>;
  // the copy of the next tile, one instruction per step of block 0's S^T
  // (not all at once: same-box A/B, backward of video_1p3b -0.8%)
  auto one = [&](int j) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rimg, (lds_ptr_t)(next + wave_part + j * kDmaBytes), 16, lane * 16,
        (uint32_t)t_next * G::kBytes + wave_part + j * kDmaBytes, 0, 0);
  };
  q_block<D, false>(cur, 0, qf, gof, l32, g, gq, c_log2, lse2, dq, 0, Nk, [&](int slot) {
    if (slot < G::kDmaPerWave) one(slot);
  });
  q_block<D, false>(cur, 1, qf, gof, l32, g, gq, c_log2, lse2, dq, 0, Nk, [](int) {});
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_q_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ go,
    const float* __restrict__ lse, const char* __restrict__ qimg, const char* __restrict__ kimg,
    float* __restrict__ gq, int Nq, int Nk, int nqtiles, int nktiles, int nqtile, int nsplit,
    Sizes sz, float scale, float c_log2) {
  using G = KImg<D>;
  using GQ = QImg<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * G::kBytes];
  // work item: query tile qt of slice bh, over key tiles [k0, k1) of split
  // `split` (partial sums, one array per split, when there are several)
  int tile;
  uint32_t bh;
  work_item(nqtile * nsplit, tile, bh);
  const int qt = tile % nqtile, split = tile / nqtile;
  const int k0 = split * nktiles / nsplit, k1 = (split + 1) * nktiles / nsplit;
  const size_t part = (size_t)split * (sz.oq_bytes / 4);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int row = qt * kRows + wave * 32 + l32;
  const bool row_ok = row < Nq;
  const uint32_t slice = slice_bytes<D, false>(nktiles);
  const uint32_t khdr = (uint32_t)nktiles * G::kBytes;
  const auto rimg = make_rsrc(kimg + (size_t)bh * slice, slice);
  const uint32_t wave_part = (uint32_t)wave * G::kDmaPerWave * kDmaBytes;
  copy_image<G::kDmaPerWave, G::kBytes>(rimg, smem, wave_part, lane, k0);
  u32x4 qf[G::kKS], gof[G::kKS];
  const uint32_t qrow = (bh * (uint32_t)Nq + row) * D * 2;
  load_frags<D>(make_rsrc(q, sz.q_bytes), qrow, row_ok, g, qf);
  load_frags<D>(make_rsrc(go, sz.q_bytes), qrow, row_ok, g, gof);
  // this row's lse and D, from the query image's extras (written by pack_q)
  float lse2 = 0.f, dq = 0.f;
  {
    const uint32_t qslice = slice_bytes<D, true>(nqtiles);
    const auto rq = make_rsrc(qimg + (size_t)bh * qslice, qslice);
    const int in_tile = row % kTile, blk = in_tile / 32, r32 = in_tile % 32;
    // slot of row r32 within its block: r32 = 8(r/4) + 4 gg + r%4
    const int gg = (r32 >> 2) & 1, r = ((r32 >> 3) << 2) | (r32 & 3);
    const uint32_t x = (uint32_t)(row / kTile) * GQ::kBytes + GQ::kOffX + blk * 256 + (gg * 16 + r) * 4;
    lse2 = buf_load4f(rq, x);
    dq = buf_load4f(rq, x + 128);
  }
  // the key side's exponent eK (K^T) and max |v_j|; t from
  // |gS_ij| <= |gO_i| max|v_j| + |D_i| over this wave's rows
  const int ek = __builtin_amdgcn_readfirstlane((int)buf_load16(rimg, khdr + kHdrRecord)[0]);
  float mv, unused;
  slice_norms(rimg, khdr, nktiles, lane, mv, unused);
  const double gn = frag_row_norm<D>(gof);
  const int t = gs_exponent(gn * (double)mv + __builtin_fabs((double)dq), gn);
#pragma unroll
  for (int ks = 0; ks < G::kKS; ++ks) gof[ks] = scale_bf16x8(gof[ks], t);
  dq = __builtin_amdgcn_ldexpf(dq, t);  // D_i 2^t
  f32x16 acc[G::kCB];
#pragma unroll
  for (int cb = 0; cb < G::kCB; ++cb) acc[cb] = f32x16{};
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int kLast = k1 - 1;
  for (int kt = k0; kt < kLast; ++kt) {
    const int i = kt - k0;
    q_tile<D>(smem + ((i + 1) & 1) * G::kBytes, smem + (i & 1) * G::kBytes, rimg, wave_part,
              lane, kt + 1, qf, gof, l32, g, acc, c_log2, lse2, dq, Nk);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  {
    // keys past Nk exist only in the last tile of the last split
    const char* cur = smem + ((kLast - k0) & 1) * G::kBytes;
    const int kl = kLast * kTile;
    if (k1 == nktiles) {
      q_block<D, true>(cur, 0, qf, gof, l32, g, acc, c_log2, lse2, dq, kl, Nk, [](int) {});
      q_block<D, true>(cur, 1, qf, gof, l32, g, acc, c_log2, lse2, dq, kl + 32, Nk, [](int) {});
    } else {
      q_block<D, false>(cur, 0, qf, gof, l32, g, acc, c_log2, lse2, dq, kl, Nk, [](int) {});
      q_block<D, false>(cur, 1, qf, gof, l32, g, acc, c_log2, lse2, dq, kl + 32, Nk, [](int) {});
    }
  }
  if (row_ok)
    store_rows<D>(make_rsrc(gq + part, sz.oq_bytes), (bh * (uint32_t)Nq + row) * D, acc, g,
                  scale, ek + t);
}

// out[i] = sum_s parts[s n + i], i < n (n a multiple of 4); fp32
__global__ __launch_bounds__(256) void sum_parts_kernel(const float* __restrict__ parts,
                                                        float* __restrict__ out, int nsplit,
                                                        uint32_t n) {
  const auto rp = make_rsrc(parts, (uint32_t)((size_t)nsplit * n * 4));
  const auto ro = make_rsrc(out, n * 4);
  for (uint32_t i = (blockIdx.x * 256 + threadIdx.x) * 4; i < n; i += gridDim.x * 256 * 4) {
    f32x4 acc = __builtin_bit_cast(f32x4, buf_load16(rp, i * 4));
    for (int s = 1; s < nsplit; ++s)
      acc += __builtin_bit_cast(f32x4, buf_load16(rp, ((uint32_t)s * n + i) * 4));
    buf_store16(ro, i * 4, __builtin_bit_cast(u32x4, acc));
  }
}

// Splits of the query range (gK, gV kernel) and of the key range (gQ kernel):
// enough workgroups for two rounds over 256 CUs, partial arrays under 2^31 B.
constexpr int kTargetGroups = 512;
inline int pick_split(int groups, int tiles, size_t part_bytes) {
  int n = (kTargetGroups + groups - 1) / groups;
  n = n < 1 ? 1 : (n > tiles ? tiles : n);
  while (n > 1 && (size_t)n * part_bytes >= ((size_t)1 << 31)) --n;
  return n;
}
struct Plan {
  int nqt, nkt, nkw, nqw, split_kv, split_q;
  size_t qimg, kimg, pkv, pq;  // bytes of each workspace part
};
template <int D>
Plan plan(int B, int H, int Nq, int Nk) {
  Plan p;
  const size_t bh = (size_t)B * H;
  p.nqt = (Nq + kTile - 1) / kTile;
  p.nkt = (Nk + kTile - 1) / kTile;
  p.nkw = (Nk + kRows - 1) / kRows;
  p.nqw = (Nq + kRows - 1) / kRows;
  const size_t kbytes = bh * Nk * D * 4, qbytes = bh * Nq * D * 4;
  p.split_kv = pick_split(p.nkw * (int)bh, p.nqt, kbytes);
  p.split_q = pick_split(p.nqw * (int)bh, p.nkt, qbytes);
  p.qimg = bh * slice_bytes<D, true>(p.nqt);
  p.kimg = bh * slice_bytes<D, false>(p.nkt);
  p.pkv = p.split_kv > 1 ? 2 * (size_t)p.split_kv * kbytes : 0;
  p.pq = p.split_q > 1 ? (size_t)p.split_q * qbytes : 0;
  return p;
}

template <int D>
hipError_t launch_d(const void* q, const void* k, const void* v, const float* o, const void* go,
                    const float* lse, float* gq, float* gk, float* gv, int B, int H, int Nq,
                    int Nk, float scale, char* ws, hipStream_t stream) {
  const int bh = B * H;
  const Plan p = plan<D>(B, H, Nq, Nk);
  const int nqt = p.nqt, nkt = p.nkt;
  char* qimg = ws;
  char* kimg = qimg + p.qimg;
  float* pkv = reinterpret_cast<float*>(kimg + p.kimg);
  float* pq = reinterpret_cast<float*>(kimg + p.kimg + p.pkv);
  const uint32_t qb = (uint32_t)((size_t)bh * Nq * D * 2), kb = (uint32_t)((size_t)bh * Nk * D * 2);
  hipError_t e = launch_range_stats<D>(q, go, qimg, bh, Nq, slice_bytes<D, true>(nqt),
                                       (uint32_t)nqt * QImg<D>::kBytes, stream);
  if (e != hipSuccess) return e;
  e = launch_range_stats<D>(k, nullptr, kimg, bh, Nk, slice_bytes<D, false>(nkt),
                            (uint32_t)nkt * KImg<D>::kBytes, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((pack_kernel<D, true>), dim3(nqt, bh), dim3(kPackThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(go),
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(go), o, lse,
                     qimg, Nq, nqt, qb);
  hipLaunchKernelGGL((pack_kernel<D, false>), dim3(nkt, bh), dim3(kPackThreads), 0, stream,
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<const uint16_t*>(k), nullptr, nullptr, nullptr, kimg, Nk, nkt,
                     kb);
  Sizes sz;
  sz.q_bytes = qb;
  sz.k_bytes = kb;
  sz.oq_bytes = (uint32_t)((size_t)bh * Nq * D * 4);
  sz.ok_bytes = (uint32_t)((size_t)bh * Nk * D * 4);
  const size_t nk_elems = (size_t)bh * Nk * D;
  float* ok = p.split_kv > 1 ? pkv : gk;
  float* ov = p.split_kv > 1 ? pkv + (size_t)p.split_kv * nk_elems : gv;
  float* oq = p.split_q > 1 ? pq : gq;
  hipLaunchKernelGGL((bwd_kv_kernel<D>), dim3(p.nkw * bh * p.split_kv), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), qimg, ok,
                     ov, Nq, Nk, nqt, p.nkw, p.split_kv, sz, scale, scale * kLog2e);
  hipLaunchKernelGGL((bwd_q_kernel<D>), dim3(p.nqw * bh * p.split_q), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(go), lse, qimg,
                     kimg, oq, Nq, Nk, nqt, nkt, p.nqw, p.split_q, sz, scale, scale * kLog2e);
  auto sum = [&](const float* parts, float* out, int n, size_t elems) {
    const size_t want = (elems / 4 + 255) / 256;
    hipLaunchKernelGGL(sum_parts_kernel, dim3((unsigned)(want < 4096 ? want : 4096)), dim3(256),
                       0, stream, parts, out, n, (uint32_t)elems);
  };
  if (p.split_kv > 1) {
    sum(ok, gk, p.split_kv, nk_elems);
    sum(ov, gv, p.split_kv, nk_elems);
  }
  if (p.split_q > 1) sum(oq, gq, p.split_q, (size_t)bh * Nq * D);
  return hipGetLastError();
}

}  // namespace bwd_path

size_t bwd_workspace_bytes(int B, int H, int Nq, int Nk, int d) {
  using namespace bwd_path;
  const Plan p = d == 128 ? plan<128>(B, H, Nq, Nk) : plan<64>(B, H, Nq, Nk);
  return p.qimg + p.kimg + p.pkv + p.pq;
}

hipError_t launch_bwd(const void* q, const void* k, const void* v, const float* o, const void* go,
                      const float* lse, float* gq, float* gk, float* gv, int B, int H, int Nq,
                      int Nk, int d, float scale, void* ws, hipStream_t stream) {
  char* w = static_cast<char*>(ws);
  return d == 128 ? bwd_path::launch_d<128>(q, k, v, o, go, lse, gq, gk, gv, B, H, Nq, Nk, scale,
                                            w, stream)
                  : bwd_path::launch_d<64>(q, k, v, o, go, lse, gq, gk, gv, B, H, Nq, Nk, scale,
                                           w, stream);
}

}  // namespace ajvp
