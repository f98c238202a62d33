// attn_jvp_f32.hip -- fused attention forward + JVP for gfx950, fp32 throughout.
//
// Same operation as the bf16 path (rCM record LIT-783 in the Anthology of the
// SOTA, "Key takeaways", "JVP at production scale", paper §3.2 / App. C), kept
// in fp32 end to end: it is the precision reference the pages motivate (the
// record's second takeaway, Fig. 11: a tangent computed in BF16 is far less
// accurate than an output computed in BF16).  Structure: one workgroup = 4 waves x 32 query rows; 32-key
// tiles of K, dK, V, dV copied straight into LDS (double buffered, one tile
// ahead); fp32 MFMA 32x32x2 for S^T = K Q^T, dS^T = dK Q^T + K dQ^T,
// A^T += V^T P^T and G^T += V^T (s P dS)^T + dV^T P^T; online softmax per lane.
#include "cdna4.hpp"
#include "launch.hpp"

namespace ajvp {
namespace f32_path {

constexpr int kBC = 32;        // keys per tile
constexpr int kThreads = 256;  // 4 waves
constexpr int kRowsPerWave = 32;
constexpr int kBR = 128;
constexpr float kTau = 4.0f;   // lazy-rescale headroom, log2 units

template <int D>
struct GeoF {
  static constexpr int kTileBytes = kBC * D * 4;       // one fp32 tile
  static constexpr int kStageBytes = 4 * kTileBytes;   // K | dK | V | dV
  static constexpr int kQ4 = D / 8;                    // float4 operand chunks per lane
  static constexpr int kCB = D / 32;
  static constexpr int kRowChunks = D / 4;             // 16-byte chunks per row
};

__device__ inline f32x16 mma_f32(float a, float b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

template <int D>
struct RowStateF {
  f32x16 accA[GeoF<D>::kCB];
  f32x16 accG[GeoF<D>::kCB];
  float m, l, u;
};

// Tiles are stored row-major [32 keys][D] with 16-byte chunk c of row r at
// chunk position c ^ (r & 7): conflict-free for both read patterns below.
template <int D>
__device__ inline int swz(int r, int chunk) {
  return r * D * 4 + ((chunk ^ (r & 7)) << 4);
}

template <int D, bool kMask>
__device__ __attribute__((always_inline)) inline void jvp_tile_f32(
    RowStateF<D>& st, const char* stage, const f32x4* qf, const f32x4* dqf, int l32, int g,
    int key0, int Nk, float c_log2, float scale) {
  using G = GeoF<D>;
  const char* sK = stage;
  const char* sdK = stage + G::kTileBytes;
  const char* sV = stage + 2 * G::kTileBytes;
  const char* sdV = stage + 3 * G::kTileBytes;

  // S^T, dS^T: contraction slot (j, e, half g) <-> d = 8j + 4g + e.
  // S is accumulated in fp32 over chunks of 32 d-values and the chunk sums are
  // added in fp64: a logit rounded to fp32 carries an absolute error of
  // 2^-24 |S|, which for large logits (outlier rows) moves p by more than the
  // fp32 path's error budget.  The exponent argument is formed from the fp64
  // sum.  dS stays a single fp32 chain (its rounding enters dO only linearly).
  constexpr int kChunkJ = 4;  // 4 x 8 = 32 d-values per fp32 chunk
  double s64[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) s64[r] = 0.0;
  f32x16 ds = f32x16{};
#pragma unroll
  for (int j0 = 0; j0 < G::kQ4; j0 += kChunkJ) {
    f32x16 s = f32x16{};
#pragma unroll
    for (int j = j0; j < j0 + kChunkJ; ++j) {
      const int off = swz<D>(l32, 2 * j + g);
      const f32x4 a = *reinterpret_cast<const f32x4*>(sK + off);
      const f32x4 da = *reinterpret_cast<const f32x4*>(sdK + off);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s = mma_f32(a[e], qf[j][e], s);
        ds = mma_f32(a[e], dqf[j][e], ds);
        ds = mma_f32(da[e], qf[j][e], ds);
      }
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) s64[r] += (double)s[r];
    __builtin_amdgcn_sched_barrier(0);
  }
  auto masked = [&](int r) { return kMask && key0 + 8 * (r >> 2) + 4 * g + (r & 3) >= Nk; };
  if constexpr (kMask) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (masked(r)) s64[r] = -INFINITY;
  }

  float mx = (float)s64[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, (float)s64[r]);
  mx = fmaxf(mx, swap_halves(mx));
  const float mt = mx * c_log2;
  const float m_new = (mt > st.m + kTau) ? mt : st.m;
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
  st.m = m_new;

  const double c64 = (double)scale * 1.4426950408889634;
  float p[16], pd[16], lsum = 0.f, usum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    p[r] = __builtin_amdgcn_exp2f((float)__builtin_fma(s64[r], c64, -(double)m_new));
    if (masked(r)) p[r] = 0.f;
    lsum += p[r];
    const float t = p[r] * ds[r];
    usum += t;
    pd[r] = t * scale;
  }
  st.l = st.l * alpha + lsum;
  st.u = st.u * alpha + usum;
  if (wave_any(alpha != 1.0f)) {
#pragma unroll
    for (int cb = 0; cb < G::kCB; ++cb) {
      st.accA[cb] *= alpha;
      st.accG[cb] *= alpha;
    }
  }

  // Second contraction over keys: step r uses key 8(r/4) + 4g + r%4, which is
  // the key this lane's accumulator slot r holds.
#pragma unroll
  for (int cb = 0; cb < G::kCB; ++cb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = 8 * (r >> 2) + 4 * g + (r & 3);
      const int c = 32 * cb + l32;
      const int off = swz<D>(key, c >> 2) + ((c & 3) << 2);
      const float a = *reinterpret_cast<const float*>(sV + off);
      const float da = *reinterpret_cast<const float*>(sdV + off);
      st.accA[cb] = mma_f32(a, p[r], st.accA[cb]);
      st.accG[cb] = mma_f32(a, pd[r], st.accG[cb]);
      st.accG[cb] = mma_f32(da, p[r], st.accG[cb]);
      // Keep the scheduler from hoisting every LDS read of the tile at once
      // (that alone would exceed the register file next to the fp32 operands).
      if ((r & 3) == 3) __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// One tile: the copy of the next tile into `next` is issued first, then the
// tile in `cur` is computed.  The stage pointers are restrict-qualified
// (disjoint halves of the LDS), so the compiler does not make the LDS reads
// of `cur` wait for the copy into `next`.
template <int D, typename Copy>
__device__ __attribute__((always_inline)) inline void f32_tile_step(
    char* __restrict__ next, const char* __restrict__ cur, Copy copy, RowStateF<D>& st,
    const f32x4* qf, const f32x4* dqf, int l32, int g, int key0, int Nk, float c_log2,
    float scale) {
  copy(next);
  jvp_tile_f32<D, false>(st, cur, qf, dqf, l32, g, key0, Nk, c_log2, scale);
}

// Sizes of the whole tensors (bytes); every global access is checked against
// them by its buffer descriptor.
struct ExtentsF {
  uint32_t q_bytes, k_bytes, o_bytes, lse_bytes;
};

template <int D>
__device__ __attribute__((always_inline)) inline void attn_jvp_f32_body(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ tq, const float* __restrict__ tk, const float* __restrict__ tv,
    float* __restrict__ o, float* __restrict__ to, float* __restrict__ lse, int Nq, int Nk,
    int ntiles, ExtentsF ext, float scale, float c_log2) {
  using G = GeoF<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * G::kStageBytes];

  // Work item: blockIdx.x = 128-row query tile, blockIdx.y = (b, h) slice.
  const int qt = blockIdx.x;
  const uint32_t bh = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int row = qt * kBR + wave * kRowsPerWave + l32;
  const bool row_ok = row < Nq;

  const auto rq = make_rsrc(q, ext.q_bytes);
  const auto rtq = make_rsrc(tq, ext.q_bytes);
  // Rows past Nq get an offset past the tensor, which the descriptor reads as 0.
  f32x4 qf[G::kQ4], dqf[G::kQ4];
  const uint32_t qrow = row_ok ? (bh * (uint32_t)Nq + row) * D * 4 : 0x80000000u;
#pragma unroll
  for (int j = 0; j < G::kQ4; ++j) {
    const uint32_t off = qrow + (8 * j + 4 * g) * 4;
    qf[j] = __builtin_bit_cast(f32x4, buf_load16(rq, off));
    dqf[j] = __builtin_bit_cast(f32x4, buf_load16(rtq, off));
  }
  // A negative scale s: s Q K^T = |s| (-Q) K^T and s dS = |s| dS of (-Q, -dQ),
  // so negating the Q and dQ fragments (exact) and working with |s| keeps every
  // scaled logit and tangent term, while the running max is taken over the
  // logits as they are.
  if (scale < 0.f) {
#pragma unroll
    for (int j = 0; j < G::kQ4; ++j) {
      qf[j] = -qf[j];
      dqf[j] = -dqf[j];
    }
    scale = -scale;
    c_log2 = -c_log2;
  }

  // Direct-to-LDS copies of the next 32-key tile (no staging registers): wave
  // w copies tensor w (K, dK, V, dV), kChunks 1 KiB loads, load n writing
  // the stage's 16-byte chunks 64 n + lane of that tensor.  The XOR swizzle
  // is applied on the global side: LDS chunk c holds row r = c / kRowChunks,
  // column chunk (c % kRowChunks) ^ (r & 7).  Rows past Nk get an offset past
  // the tensor, which the descriptor reads as zeros.
  constexpr int kChunks = G::kTileBytes / 16 / 64;  // loads per wave and tile
  typedef __attribute__((address_space(3))) void* lds_ptr_t;
  const float* const srcs[4] = {k, tk, v, tv};
  const auto rsrc = make_rsrc(srcs[wave], ext.k_bytes);
  const uint32_t kslice = bh * (uint32_t)Nk * D * 4;
  auto copy_tile = [&](char* stage, int kt) {
#pragma unroll
    for (int n = 0; n < kChunks; ++n) {
      const int c = 64 * n + lane, r = c / G::kRowChunks, pos = c % G::kRowChunks;
      const int key = kt * kBC + r;
      const uint32_t off = key < Nk ? kslice + (uint32_t)(key * D * 4 + ((pos ^ (r & 7)) << 4))
                                    : 0x80000000u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (lds_ptr_t)(stage + wave * G::kTileBytes + n * 1024), 16, off, 0, 0, 0);
    }
  };

  RowStateF<D> st;
#pragma unroll
  for (int cb = 0; cb < G::kCB; ++cb) {
    st.accA[cb] = f32x16{};
    st.accG[cb] = f32x16{};
  }
  st.m = -INFINITY;
  st.l = 0.f;
  st.u = 0.f;

  copy_tile(smem, 0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  for (int kt = 0; kt < ntiles - 1; ++kt) {
    f32_tile_step<D>(smem + ((kt + 1) & 1) * G::kStageBytes, smem + (kt & 1) * G::kStageBytes,
                     [&](char* next) { copy_tile(next, kt + 1); }, st, qf, dqf, l32, g,
                     kt * kBC, Nk, c_log2, scale);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  }
  {
    const int kt = ntiles - 1;  // peeled: keys past Nk are masked
    jvp_tile_f32<D, true>(st, smem + (kt & 1) * G::kStageBytes, qf, dqf, l32, g, kt * kBC, Nk,
                          c_log2, scale);
  }

  const float l = st.l + swap_halves(st.l);
  const float u = st.u + swap_halves(st.u);
  const float inv_l = 1.0f / l;
  const float mu = u * scale * inv_l;
  if (row_ok) {
    const auto ro = make_rsrc(o, ext.o_bytes);
    const auto rto = make_rsrc(to, ext.o_bytes);
    const uint32_t orow = (bh * (uint32_t)Nq + row) * D * 4;
#pragma unroll
    for (int cb = 0; cb < G::kCB; ++cb)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int c0 = 32 * cb + 8 * qq + 4 * g;
        f32x4 ov, tv4;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = st.accA[cb][4 * qq + e] * inv_l;
          ov[e] = a;
          tv4[e] = st.accG[cb][4 * qq + e] * inv_l - mu * a;
        }
        buf_store16(ro, orow + c0 * 4, __builtin_bit_cast(u32x4, ov));
        buf_store16(rto, orow + c0 * 4, __builtin_bit_cast(u32x4, tv4));
      }
    if (lse != nullptr && g == 0) {
      const auto rl = make_rsrc(lse, ext.lse_bytes);
      buf_store4(rl, (bh * (uint32_t)Nq + row) * 4, (st.m + __log2f(l)) * kLn2);
    }
  }
}

#define AJVP_F32_KERNEL(D)                                                                     \
  __global__ __launch_bounds__(kThreads, 1) void attn_jvp_f32_d##D(                             \
      const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,    \
      const float* __restrict__ tq, const float* __restrict__ tk, const float* __restrict__ tv, \
      float* __restrict__ o, float* __restrict__ to, float* __restrict__ lse, int Nq, int Nk,   \
      int ntiles, ExtentsF ext, float scale, float c_log2) {                                    \
    attn_jvp_f32_body<D>(q, k, v, tq, tk, tv, o, to, lse, Nq, Nk, ntiles, ext, scale, c_log2);  \
  }
AJVP_F32_KERNEL(64)
AJVP_F32_KERNEL(128)
#undef AJVP_F32_KERNEL

template <int D>
hipError_t launch_f32_d(const float* q, const float* k, const float* v, const float* tq,
                        const float* tk, const float* tv, float* o, float* to, float* lse, int B,
                        int H, int Nq, int Nk, float scale, hipStream_t stream) {
  const int ntiles = (Nk + kBC - 1) / kBC;
  const int nqt = (Nq + kBR - 1) / kBR;
  const int bh = B * H;
  ExtentsF ext;
  ext.q_bytes = (uint32_t)((size_t)bh * Nq * D * 4);
  ext.k_bytes = (uint32_t)((size_t)bh * Nk * D * 4);
  ext.o_bytes = ext.q_bytes;
  ext.lse_bytes = (uint32_t)((size_t)bh * Nq * 4);
  hipLaunchKernelGGL((D == 128 ? attn_jvp_f32_d128 : attn_jvp_f32_d64), dim3(nqt, bh),
                     dim3(kThreads), 0, stream, q, k, v, tq, tk, tv, o, to, lse, Nq, Nk, ntiles,
                     ext, scale, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace f32_path
using namespace f32_path;

hipError_t launch_f32(const float* q, const float* k, const float* v, const float* tq,
                      const float* tk, const float* tv, float* o, float* to, float* lse, int B,
                      int H, int Nq, int Nk, int d, float scale, hipStream_t stream) {
  if (d == 128) return launch_f32_d<128>(q, k, v, tq, tk, tv, o, to, lse, B, H, Nq, Nk, scale, stream);
  return launch_f32_d<64>(q, k, v, tq, tk, tv, o, to, lse, B, H, Nq, Nk, scale, stream);
}

}  // namespace ajvp
