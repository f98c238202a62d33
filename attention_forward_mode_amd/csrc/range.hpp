// range.hpp -- power-of-two scalings that keep the fp16 operands of the
// matrix-core products inside fp16's range (gfx950 device helpers).
//
// The second contraction of the forward pass (P and s P dS against V and dV)
// and the products of the backward pass run on fp16 operands, which hold 11
// significant bits but only magnitudes from 2^-24 to 65504; bf16 inputs span
// 2^-133 .. 3.4e38.  Multiplying an operand by a power of two is exact in
// binary floating point (short of overflow and underflow), so each operand
// family is scaled by 2^e into fp16's upper range and the result is scaled
// back by 2^-e in fp32: the products, sums and roundings in between are those
// of the unscaled values, moved by whole binades.
//   - a tensor of the inputs (V, dV; Q, gO, K in the backward pass) gets one
//     exponent per (b, h) slice from its largest finite magnitude, found by a
//     reduction pass before the pack;
//   - a per-element product formed in the kernel (s P dS; the backward's
//     softmax gradient) gets its exponent from an upper bound of its
//     magnitude (Cauchy-Schwarz on row norms) computed before the key loop.
// Non-finite inputs are left out of the maxima, so they stay Inf or NaN in
// fp16 and propagate through the products as they would unscaled.
#pragma once

#include "cdna4.hpp"

namespace ajvp {

// Largest finite |x| among the eight bf16 values of a 16-byte chunk, as bf16
// magnitude bits (the bit patterns of non-negative bf16 values order like
// their values; exponent field 0xff = Inf or NaN is left out).
__device__ inline uint32_t finite_absmax8(u32x4 x) {
  uint32_t m = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = x[w] & 0x7fffu, hi = (x[w] >> 16) & 0x7fffu;
    m = lo < 0x7f80u && lo > m ? lo : m;
    m = hi < 0x7f80u && hi > m ? hi : m;
  }
  return m;
}

// The exponent e that puts a largest magnitude given as bf16 bits into
// [2^14, 2^15) after multiplying by 2^e (below fp16's 65504, so every scaled
// value of the tensor converts without overflow); 0 when the tensor is zero.
__device__ inline int fp16_exponent(uint32_t absbits) {
  if (absbits == 0) return 0;
  int e;
  __builtin_frexpf(__builtin_bit_cast(float, absbits << 16), &e);  // max = f 2^e, f in [0.5, 1)
  return 15 - e;
}

// Bound on |s P dS| or |gS| after scaling, with P <= 2^4 (the forward pass's
// lazy rescale keeps p <= 16): 16 * 4000 = 64000 < 65504, the largest fp16.
constexpr double kProdSafe = 4000.0;

// The largest t with bound * 2^t <= kProdSafe, clamped to [-150, 100] (a bound
// of 0 or NaN gives 0, an infinite one -150).
__device__ inline int product_exponent(double bound) {
  if (!(bound > 0.0)) return 0;
  if (bound > 1.0e300) return -150;
  int e;
  __builtin_frexp(kProdSafe / bound, &e);  // = f 2^e, f in [0.5, 1): floor(log2) = e - 1
  const int t = e - 1;
  return t < -150 ? -150 : (t > 100 ? 100 : t);
}

// Sum of squares of the eight bf16 values of a 16-byte chunk, in fp64 (exact
// products; no overflow for any finite bf16).
__device__ inline double sumsq8(u32x4 x) {
  double s = 0.0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const double lo = (double)__builtin_bit_cast(float, x[w] << 16);
    const double hi = (double)__builtin_bit_cast(float, x[w] & 0xffff0000u);
    s = __builtin_fma(lo, lo, s);
    s = __builtin_fma(hi, hi, s);
  }
  return s;
}

// fp64 value of lane l and lane l ^ 32 summed, in every lane.
__device__ inline double halves_sum_f64(double x) {
  const uint64_t u = __builtin_bit_cast(uint64_t, x);
  const uint32_t lo = (uint32_t)u, hi = (uint32_t)(u >> 32);
  const auto a = __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
  const double x0 = __builtin_bit_cast(double, ((uint64_t)(uint32_t)b[0] << 32) | (uint32_t)a[0]);
  const double x1 = __builtin_bit_cast(double, ((uint64_t)(uint32_t)b[1] << 32) | (uint32_t)a[1]);
  return x0 + x1;
}

// Reductions over the 64 lanes of a wave, leaving the result in every lane,
// without a trip through LDS: two quad permutations and two rotations of each
// 16-lane row (DPP) combine a row, then the swaps of rows 0 <-> 1, 2 <-> 3
// (v_permlane16_swap) and of the two halves (v_permlane32_swap) combine the
// rows.  Each swap of x with itself hands every lane its own value and that of
// its partner lane (l ^ 16, l ^ 32), in either order, so the operation must be
// commutative.  Every lane of the wave must be active.
template <int kCtrl>
__device__ inline uint32_t dpp_word(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, kCtrl, 0xf, 0xf, false);
}
template <typename T>
struct LaneWords {  // T as 32-bit words (T of 4 or 8 bytes)
  static constexpr int kN = sizeof(T) / 4;
  uint32_t w[kN];
};
template <typename T, typename Op>
__device__ inline T wave_allreduce(T x, Op op) {
  using W = LaneWords<T>;
  auto step = [&](auto move) {
    W a = __builtin_bit_cast(W, x), b;
#pragma unroll
    for (int i = 0; i < W::kN; ++i) b.w[i] = move(a.w[i]);
    x = op(x, __builtin_bit_cast(T, b));
  };
  step([](uint32_t v) { return dpp_word<0xB1>(v); });   // quad_perm [1,0,3,2]: lane ^ 1
  step([](uint32_t v) { return dpp_word<0x4E>(v); });   // quad_perm [2,3,0,1]: lane ^ 2
  step([](uint32_t v) { return dpp_word<0x124>(v); });  // row_ror:4
  step([](uint32_t v) { return dpp_word<0x128>(v); });  // row_ror:8
  auto swap = [&](auto perm) {
    W a = __builtin_bit_cast(W, x), p, q;
#pragma unroll
    for (int i = 0; i < W::kN; ++i) {
      const auto r = perm(a.w[i]);
      p.w[i] = (uint32_t)r[0];
      q.w[i] = (uint32_t)r[1];
    }
    x = op(__builtin_bit_cast(T, p), __builtin_bit_cast(T, q));
  };
  swap([](uint32_t v) { return __builtin_amdgcn_permlane16_swap(v, v, false, false); });
  swap([](uint32_t v) { return __builtin_amdgcn_permlane32_swap(v, v, false, false); });
  return x;
}

// Maximum over the 64 lanes of a wave (NaN lanes are ignored: fmax).
__device__ inline double wave_max_f64(double x) {
  return wave_allreduce(x, [](double a, double b) { return __builtin_fmax(a, b); });
}
__device__ inline uint32_t wave_max_u32(uint32_t x) {
  return wave_allreduce(x, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}
__device__ inline float wave_max_f32(float x) {
  return wave_allreduce(x, [](float a, float b) { return __builtin_fmaxf(a, b); });
}

// Eight bf16 values times 2^t (exact while the results stay normal; rounded
// to nearest even below that).
__device__ inline u32x4 scale_bf16x8(u32x4 x, int t) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t v = x[w];
    const float lo = __builtin_amdgcn_ldexpf(__builtin_bit_cast(float, v << 16), t);
    const float hi = __builtin_amdgcn_ldexpf(__builtin_bit_cast(float, v & 0xffff0000u), t);
    const uint32_t blo = __builtin_bit_cast(uint16_t, (__bf16)lo);
    const uint32_t bhi = __builtin_bit_cast(uint16_t, (__bf16)hi);
    r[w] = blo | (bhi << 16);
  }
  return r;
}

// The largest t with x 2^t <= 2^120 (x > 0 finite; otherwise 1000, no limit):
// a cap on a scaling exponent that keeps bf16 values and their sums finite.
__device__ inline int cap_exponent(double x) {
  if (!(x > 0.0) || !__builtin_isfinite(x)) return 1000;
  int e;
  __builtin_frexp(x, &e);  // x = f 2^e, f in [0.5, 1): x 2^(120 - e) < 2^120
  return 120 - e;
}

// fp32 value not below the fp64 x (x >= 0): rounded to nearest, then raised by
// 2^-20 relative, more than the rounding can have taken off.
__device__ inline float round_up_f32(double x) { return (float)(x * (1.0 + 0x1p-20)); }

// ---- the per-slice header of a packed workspace -------------------------------
// Each (b, h) slice of a packed workspace (tile images of 64 rows of one
// side, keys or queries) ends with a header of kHdrBytes:
//   +kHdrRecord  the slice's fp16 exponents (int, up to four) and flags
//   +kHdrStats   the range pass's partial maxima, per chunk of rows: uint max
//                finite |x| and |y| as bf16 magnitude bits
//   +kHdrNorms   kNormSlots pairs of fp32 maxima of row norms (rounded up):
//                the pack's workgroup of tile i raises pair i % kNormSlots with
//                integer atomics (the bit patterns of non-negative floats
//                order like their values; spreading the tiles over slots keeps
//                the atomics on one address few), after the range pass has
//                zeroed them; a consumer takes the maximum over the slots
constexpr int kHdrRecord = 0;
constexpr int kHdrStats = 256;
constexpr int kStatChunks = 64;
constexpr int kHdrNorms = 1024;
constexpr int kNormSlots = 64;
constexpr int kHdrBytes = 2048;
static_assert(kHdrStats + 8 * kStatChunks <= kHdrNorms &&
                  kHdrNorms + 8 * kNormSlots <= kHdrBytes,
              "header layout");
constexpr int kStatThreads = 256;

__host__ __device__ constexpr int stat_chunks(int ntiles) {
  return ntiles < kStatChunks ? ntiles : kStatChunks;
}

// Largest finite |x| and |y| (y NULL: 0) over one chunk of rows (blockIdx.x;
// the ntiles 64-row tiles are cut into stat_chunks(ntiles) contiguous chunks)
// of slice blockIdx.y of [slices, N, D] bf16 tensors of in_bytes bytes,
// written to the header of that slice (at ws + slice * slice_bytes + hdr).
// Chunk 0 also zeroes the header's norm words.
template <int D>
__global__ __launch_bounds__(kStatThreads) void range_stats_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ y, char* __restrict__ ws,
    int N, int ntiles, uint32_t in_bytes, uint32_t slice_bytes, uint32_t hdr) {
  const int nch = stat_chunks(ntiles), c = blockIdx.x;
  const uint32_t bh = blockIdx.y;
  const int tpc = (ntiles + nch - 1) / nch;
  const int r0 = c * tpc * 64, r1 = r0 + tpc * 64 < N ? r0 + tpc * 64 : N;
  const auto rws = make_rsrc(ws + (size_t)bh * slice_bytes, slice_bytes);
  const auto rx = make_rsrc(x, in_bytes);
  const auto ry = make_rsrc(y, y != nullptr ? in_bytes : 0u);
  uint32_t mx = 0, my = 0;
  if (r1 > r0) {
    const uint32_t base = (bh * (uint32_t)N + r0) * D * 2, n = (uint32_t)(r1 - r0) * D * 2;
    constexpr uint32_t kStep = kStatThreads * 16;
    uint32_t off = threadIdx.x * 16;
    for (; off + 3 * kStep < n; off += 4 * kStep) {  // four loads in flight per tensor
      u32x4 a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = buf_load16(rx, base + off + u * kStep);
        b[u] = buf_load16(ry, base + off + u * kStep);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t ma = finite_absmax8(a[u]), mb = finite_absmax8(b[u]);
        mx = ma > mx ? ma : mx;
        my = mb > my ? mb : my;
      }
    }
    for (; off < n; off += kStep) {
      const uint32_t ma = finite_absmax8(buf_load16(rx, base + off));
      const uint32_t mb = finite_absmax8(buf_load16(ry, base + off));
      mx = ma > mx ? ma : mx;
      my = mb > my ? mb : my;
    }
  }
  mx = wave_max_u32(mx);
  my = wave_max_u32(my);
  __shared__ uint32_t sm[2][kStatThreads / 64];
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    sm[0][w] = mx;
    sm[1][w] = my;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int i = 1; i < kStatThreads / 64; ++i) {
      mx = sm[0][i] > mx ? sm[0][i] : mx;
      my = sm[1][i] > my ? sm[1][i] : my;
    }
    buf_store8(rws, hdr + kHdrStats + 8 * c, u32x2{mx, my});
  }
  // the norm slots the pack raises with atomics start at 0
  if (c == 0 && threadIdx.x < kNormSlots)
    buf_store8(rws, hdr + kHdrNorms + 8 * threadIdx.x, u32x2{0u, 0u});
}

template <int D>
inline hipError_t launch_range_stats(const void* x, const void* y, void* ws, int slices, int N,
                                     uint32_t slice_bytes, uint32_t hdr, hipStream_t stream) {
  const int ntiles = (N + 63) / 64;
  hipLaunchKernelGGL((range_stats_kernel<D>), dim3(stat_chunks(ntiles), slices),
                     dim3(kStatThreads), 0, stream, static_cast<const uint16_t*>(x),
                     static_cast<const uint16_t*>(y), static_cast<char*>(ws), N, ntiles,
                     (uint32_t)((size_t)slices * N * D * 2), slice_bytes, hdr);
  return hipGetLastError();
}

// Raise norm slot tile % kNormSlots of the slice header at `hdr_ptr` to
// (a, b) (non-negative fp32, as bits).
__device__ inline void raise_norms(char* hdr_ptr, int tile, float a, float b) {
  uint32_t* slot = reinterpret_cast<uint32_t*>(hdr_ptr + kHdrNorms) + 2 * (tile % kNormSlots);
  atomicMax(slot, __builtin_bit_cast(uint32_t, a));
  atomicMax(slot + 1, __builtin_bit_cast(uint32_t, b));
}

// This lane's norm slot of a slice (lane < the slot count; 0 elsewhere): the
// loads of slice_norms, to be reduced over the wave later.
__device__ inline void slice_norm_slots(__amdgpu_buffer_rsrc_t rws, uint32_t hdr, int ntiles,
                                        int lane, float& a, float& b) {
  a = 0.f;
  b = 0.f;
  if (lane < (ntiles < kNormSlots ? ntiles : kNormSlots)) {
    const int o = (int)(hdr + kHdrNorms + 8 * lane);
    a = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rws, o, 0, 0));
    b = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rws, o + 4, 0, 0));
  }
}

// The two norm maxima of a slice (over its slots), in every lane of a wave.
__device__ inline void slice_norms(__amdgpu_buffer_rsrc_t rws, uint32_t hdr, int ntiles,
                                   int lane, float& a, float& b) {
  slice_norm_slots(rws, hdr, ntiles, lane, a, b);
  a = wave_max_f32(a);
  b = wave_max_f32(b);
}

// The range pass's maxima of one slice, reduced by one wave from its partial
// maxima: every lane returns max |x| and max |y| as bf16 magnitude bits.
__device__ inline void slice_maxima(__amdgpu_buffer_rsrc_t rws, uint32_t hdr, int ntiles,
                                    int lane, uint32_t& mx, uint32_t& my) {
  mx = 0;
  my = 0;
  if (lane < stat_chunks(ntiles)) {
    const int o = (int)(hdr + kHdrStats + 8 * lane);
    mx = __builtin_amdgcn_raw_buffer_load_b32(rws, o, 0, 0);
    my = __builtin_amdgcn_raw_buffer_load_b32(rws, o + 4, 0, 0);
  }
  mx = wave_max_u32(mx);
  my = wave_max_u32(my);
}

}  // namespace ajvp
