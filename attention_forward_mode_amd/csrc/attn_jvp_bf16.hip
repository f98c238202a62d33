// attn_jvp_bf16.hip -- fused attention forward + JVP for gfx950, bf16 inputs.
//
// The operation (rCM record LIT-783 in the Anthology of the SOTA, "Key
// takeaways", "JVP at production scale", paper §3.2 / App. C: the
// FlashAttention-2 forward fused with its directional derivative in a single
// sweep over key tiles):
//   O = softmax(s Q K^T) V,  dO = (P * (dS - mu)) V + P dV,
//   dS = s (dQ K^T + Q dK^T),  mu = rowsum(P * dS),  lse = ln rowsum exp(s Q K^T),
//   and mu is also the tangent of lse.
//
// Three kernels per call:
//  1. range_stats (range.hpp): per (b, h) the largest finite |V| and |dV|
//     (partial maxima over chunks of keys), from which the pack takes the
//     power-of-two exponents that scale V and dV into fp16's upper range.
//  2. pack_kv: K, dK, V, dV -> one "tile image" per 64 keys in the workspace,
//     byte for byte the LDS layout the fused kernel computes from: K and dK
//     (bf16), then V^T 2^eV and dV^T 2^edV (fp16), each stored as the sequence
//     of matrix-core operand fragments the waves read (1 KiB per fragment, lane
//     l at bytes 16 l .. 16 l + 15), zero past Nk; and the slice's largest key
//     norms |k_j|, |dk_j|.  HBM bound, about 1% of the fused kernel's time at
//     N = 32760 together with the stats.  fp16 instead of bf16 for the
//     second contraction keeps P and P*dS at 11 significant bits.
//  3. attn_jvp_bf16: one workgroup = 8 waves x 32 query rows of one (b, h),
//     two waves per SIMD.  Per 64-key tile the waves copy the next tile image
//     from the workspace straight into LDS (buffer loads with the LDS-direct
//     bit, 1 KiB per instruction, no registers in between; double buffered),
//     then per wave and 32-key block
//        S^T  = K Q^T            (bf16 MFMA 32x32x16, Q held in registers)
//        dS^T = dK Q^T + K dQ^T  (same K fragments reused)
//     online softmax in the accumulator layout (each lane owns one query row,
//     so row state is per lane), and
//        A^T += V^T P^T,  G^T += V^T (s P dS)^T + dV^T P^T  (fp16 MFMA)
//     with P, s*P*dS rounded to fp16.  s*P*dS is formed as P dS (s 2^t): each
//     wave takes t from a bound of |s dS| over its rows (|s| (|dq_i| max|k_j|
//     + |q_i| max|dk_j|)), so that it stays below 4000 and |s P dS 2^t| below
//     64000; G then holds 2^(eV + t) times its value (dV is packed at
//     2^(eV + t) when the head's t fits every wave; a wave whose bound needs a
//     smaller t scales its dV^T fragments by the difference instead).  The
//     epilogue forms O = A 2^-eV / l, mu = u 2^-t / l (u = rowsum s P dS 2^t),
//     dO = G 2^-(eV + t) / l - mu O and lse.
//  While one wave of a SIMD runs its softmax on the vector ALU, the other
//  keeps the matrix core busy; every wave fits in 256 registers (128
//  accumulators, 64 for the Q and dQ operands, 64 for the rest).
//  The running max is only raised when a block's max exceeds it by more than
//  kTau (log2 units): results are exact either way, p stays <= 2^kTau, and the
//  accumulator rescale is skipped on most blocks.
//
// Two modes share that body:
//  kFull    the JVP along (dQ, dK, dV); a NULL tangent reads as zeros;
//  kFrozen  the JVP with dK = dV = 0 (e.g. frozen text keys of cross-attention):
//           the products with dK and dV and their tiles are left out (4 of the
//           6 contractions remain).
// The forward pass alone (O, lse: 2 contractions) has a kernel of its own
// (attn_fwd_bf16_kernel, 64 rows per wave).  Outputs O and dO are written in
// fp32 or bf16 (round to nearest even).  Both kernels can also run a range of
// key tiles per work item and write partial states (split-KV for few query
// rows), which the merge kernel of attn_jvp_merge.hip combines.
#include <cmath>
#include <cstdlib>

#include "cdna4.hpp"
#include "launch.hpp"
#include "range.hpp"

namespace ajvp {
namespace bf16_path {

constexpr int kBC = 64;             // keys per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kRowsPerWave = 32;
constexpr int kBR = kWaves * kRowsPerWave;  // query rows per workgroup
constexpr int kPackThreads = 256;
constexpr float kTau = 4.0f;        // lazy-rescale headroom, log2 units
constexpr int kDmaBytes = 1024;     // one LDS-direct load: 64 lanes x 16 bytes
constexpr uint32_t kXcds = 8;       // accelerator dies (each with its own L2) on MI355X

enum : int { kFull = 0, kFrozen = 1 };
template <int kMode>
struct Mode {
  static constexpr bool kKV = kMode == kFull;  // dK and dV take part
};

// Tile image of 64 keys: K | dK | V^T | dV^T (without dK and dV when kKV is
// false), each part a sequence of 1 KiB operand fragments in the order the
// waves read them: a wave's 16-byte read is lane l at fragment base + 16 l,
// consecutive lanes on consecutive bytes (no bank conflicts, no padding), and
// every address is the per-lane 16 l plus a constant.
//   K, dK:     fragment kb * kKS + ks = keys 32 kb + (l % 32), d 16 ks + 8 (l / 32) .. +8
//   V^T, dV^T: fragment (2 kb + t) kCB + cb = d 32 cb + (l % 32), keys at packed
//              positions 8 (4 kb + 2 t + l / 32) .. +8 (packed_key)
template <int D, bool kKV>
struct Geo {
  static constexpr int kKTile = kBC * D * 2;              // K, dK: 64 keys x D bf16
  static constexpr int kVTile = D * kBC * 2;              // V^T, dV^T: D x 64 keys fp16
  static constexpr int kNT = kKV ? 2 : 1;                 // tiles per kind
  static constexpr int kOffdK = kKTile;
  static constexpr int kOffV = kNT * kKTile;
  static constexpr int kOffdV = kOffV + kVTile;
  static constexpr int kImgUsed = kNT * (kKTile + kVTile);
  static constexpr int kRound = kThreads * 16;            // 8 KiB
  static constexpr int kImgBytes = (kImgUsed + kRound - 1) / kRound * kRound;
  static constexpr int kDmaPerWave = kImgBytes / (kWaves * kDmaBytes);
  static constexpr int kKS = D / 16;                      // contraction steps over d
  static constexpr int kCB = D / 32;                      // 32-column output blocks
};
static_assert(Geo<128, true>::kImgBytes == 65536 && Geo<64, true>::kImgBytes == 32768 &&
                  Geo<128, false>::kImgBytes == 32768 && Geo<64, false>::kImgBytes == 16384 &&
                  Geo<128, true>::kImgUsed == Geo<128, true>::kImgBytes,
              "tile image sizes");

// One (b, h) slice of the workspace: the ntiles tile images, then the header
// of range.hpp (kHdrBytes): record = {int eV, int edV, uint flags}, the range
// pass's partial maxima of |V| and |dV|, norm slots = {max |k_j|, max |dk_j|}.
constexpr uint32_t kDvZero = 1u;  // flags: dV has no finite nonzero value (or no dV at all)

// How a wave forms its tangent products (chosen per wave, see WaveScale).
enum : int { kPathFast = 0, kPathScaleDV = 1, kPathSepU = 2 };
template <int D, bool kKV>
__host__ __device__ constexpr uint32_t slice_bytes(int ntiles) {
  return (uint32_t)ntiles * Geo<D, kKV>::kImgBytes + kHdrBytes;
}

// Key held at position `pos` (0..63) of a packed V^T row.  Positions
// 16G + 8g + e hold the keys that the S^T accumulator of lane half g puts in
// slots 8t + e of block G/2, t = G%2: keys 16G + 4g + e (e < 4) and
// 16G + 8 + 4g + (e - 4) (e >= 4).
__device__ inline int packed_key(int pos) {
  const int G = pos >> 4, g = (pos >> 3) & 1, e = pos & 7;
  return 16 * G + (e < 4 ? 4 * g + e : 8 + 4 * g + (e - 4));
}

// One tile image: blockIdx.x = 64-key tile, blockIdx.y = (b, h) slice.  A NULL
// dk or dv gets an empty descriptor, so its part of the image is zero.  V and
// dV are written as fp16(v 2^eV), fp16(dv 2^edV) with the slice's exponents
// (fp16_exponent of range_stats' maxima, which every wave reduces itself);
// the workgroup of tile 0 writes them to the slice header, and every tile
// raises the slice's largest key norms to its own.
template <int D, bool kKV>
__device__ __attribute__((always_inline)) inline void pack_kv_body(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dk, const uint16_t* __restrict__ dv, char* __restrict__ ws,
    int Nk, int ntiles, uint32_t kv_bytes) {
  using G = Geo<D, kKV>;
  constexpr int kT = G::kNT;
  __shared__ _Float16 sv[kT][kBC][D + 2];
  __shared__ double snorm[2][kPackThreads / 64];
  const int tile = blockIdx.x;
  const uint32_t bh = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Every global access goes through a buffer descriptor spanning the whole
  // tensor: an offset outside it is dropped (stores) or reads zero (loads).
  const auto rk = make_rsrc(k, kv_bytes);
  const auto rdk = make_rsrc(dk, dk != nullptr ? kv_bytes : 0u);
  const auto rv = make_rsrc(v, kv_bytes);
  const auto rdv = make_rsrc(dv, dv != nullptr ? kv_bytes : 0u);
  // the workspace descriptor spans this (b, h) slice's images and header only
  const uint32_t sb = slice_bytes<D, kKV>(ntiles);
  const uint32_t hdr = (uint32_t)ntiles * G::kImgBytes;
  const auto rws = make_rsrc(ws + (size_t)bh * sb, sb);
  const int key0 = tile * kBC;
  const uint32_t img = (uint32_t)tile * G::kImgBytes;
  constexpr int kChunksPerRow = D / 8;  // 16-byte chunks of one input row
  constexpr u32x4 kZero = {0u, 0u, 0u, 0u};

  // the slice's exponents, from the partial maxima of range_stats
  uint32_t mv, mdv;
  slice_maxima(rws, hdr, ntiles, lane, mv, mdv);
  const int ev = fp16_exponent(mv);
  const int edv = kKV ? fp16_exponent(mdv) : 0;

  // The inputs are read here for the last time (non-temporal loads: same-box
  // A/B, the range pass and pack of video_1p3b 0.184 -> 0.177 ms).
  // K, dK: 16-byte chunk col of key row r goes to lane (r % 32) + 32 (col % 2)
  // of fragment (r / 32) kKS + col / 2; keys >= Nk are zero.  Each key's sum
  // of squares (fp64) is summed over the kChunksPerRow consecutive lanes that
  // hold its row; the tile's largest goes to the header.
  constexpr int kKChunks = kBC * kChunksPerRow;
  static_assert(kKChunks % kPackThreads == 0, "one tensor per pass of the loop");
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    double kss = 0.0;
    if (t < kT) {
      for (int c = threadIdx.x; c < kKChunks; c += kPackThreads) {
        const int r = c / kChunksPerRow, col = c % kChunksPerRow;
        const int key = key0 + r;
        u32x4 x = kZero;
        if (key < Nk)
          x = buf_load16_nt(t == 0 ? rk : rdk, ((bh * (uint32_t)Nk + key) * D + 8 * col) * 2);
        const int frag = (r >> 5) * G::kKS + (col >> 1), ln = (r & 31) + 32 * (col & 1);
        buf_store16(rws, img + t * G::kOffdK + frag * kDmaBytes + ln * 16, x);
        double ss = sumsq8(x);
#pragma unroll
        for (int m = 1; m < kChunksPerRow; m <<= 1) ss += __shfl_xor(ss, m);
        kss = __builtin_fmax(kss, ss);
      }
    }
    kss = wave_max_f64(kss);
    if (lane == 0) snorm[t][wave] = kss;
  }
  // V, dV: scaled to fp16 in LDS, then written transposed as operand fragments.
  constexpr int kIn = kBC * kChunksPerRow;
  for (int c = threadIdx.x; c < kT * kIn; c += kPackThreads) {
    const int t = c / kIn, rem = c % kIn, r = rem / kChunksPerRow, col = (rem % kChunksPerRow) * 8;
    const int key = key0 + r;
    const int e_t = t == 0 ? ev : edv;
    u32x4 x = kZero;
    if (key < Nk) x = buf_load16_nt(t == 0 ? rv : rdv, ((bh * (uint32_t)Nk + key) * D + col) * 2);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t bits = (x[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      sv[t][r][col + e] = (_Float16)__builtin_amdgcn_ldexpf(__builtin_bit_cast(float, bits << 16), e_t);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double nk = snorm[0][0], ndk = snorm[1][0];
    for (int i = 1; i < kPackThreads / 64; ++i) {
      nk = __builtin_fmax(nk, snorm[0][i]);
      ndk = __builtin_fmax(ndk, snorm[1][i]);
    }
    const float fk = round_up_f32(__builtin_sqrt(nk));
    const float fdk = kKV ? round_up_f32(__builtin_sqrt(ndk)) : 0.f;
    raise_norms(ws + (size_t)bh * sb + hdr, tile, fk, fdk);
    if (tile == 0) {
      const uint32_t flags = (!kKV || mdv == 0) ? kDvZero : 0u;
      buf_store16(rws, hdr + kHdrRecord, u32x4{(uint32_t)ev, (uint32_t)edv, flags, 0u});
    }
  }
  constexpr int kVChunks = G::kVTile / 16;  // = 64 lanes x fragments
  for (int c = threadIdx.x; c < kT * kVChunks; c += kPackThreads) {
    const int t = c / kVChunks, rem = c % kVChunks, frag = rem >> 6, ln = rem & 63;
    const int kb = frag / (2 * G::kCB), tt = (frag / G::kCB) & 1, cb = frag % G::kCB;
    const int col = 32 * cb + (ln & 31), p = 4 * kb + 2 * tt + (ln >> 5);
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = sv[t][packed_key(8 * p + e)][col];
    buf_store16(rws, img + G::kOffV + t * G::kVTile + frag * kDmaBytes + ln * 16,
                __builtin_bit_cast(u32x4, h));
  }
  // the image's tail beyond its tiles
  for (int o = G::kImgUsed + threadIdx.x * 16; o < G::kImgBytes; o += kPackThreads * 16)
    buf_store16(rws, img + o, kZero);
}

template <int D>
struct RowState {
  f32x16 accA[D / 32];  // A^T = sum p v      (rows: output column, cols: query)
  f32x16 accG[D / 32];  // G^T = sum p (s dS v + dv)
  float m;              // running max of s*log2e*S (log2 units), per query row
  float l;              // this lane's half of sum p         (of the fp16-rounded p)
  float u;              // this lane's half of sum s p dS    (of the fp16-rounded values)
};

// Slot r of lane half g holds key 8(r/4) + 4g + r%4 of its 32-key block.
__device__ __attribute__((always_inline)) inline int slot_key(int r, int g) {
  return 8 * (r >> 2) + 4 * g + (r & 3);
}

// One 32-key block for this wave's 32 query rows, in two phases so that a
// caller can put other work between them: qk_phase forms S^T and dS^T from
// the K and dK fragments at kbase, dkbase; sm_pv_phase runs the softmax on
// them and adds the block's P V products with the V^T and dV^T fragments at
// vbase, dvbase (fragment f of a part at base + f KiB, the tile image's
// layout).  kMask: the block may hold keys >= Nk, which get p = 0 and
// contribute nothing to u.  kPath (see WaveScale): kPathScaleDV multiplies
// the dV^T fragments by dv_mul (two equal fp16 powers of two) after their
// read, for a wave whose tangent exponent is below the one dV was packed for;
// kPathSepU sums u from s P dS at its own power of two 2^tu (dv_mul then holds
// the float s 2^tu), for a wave whose s P dS would sit far below fp16's range
// at the exponent dV sets.  `scale` is s 2^t, the wave's scale of s P dS.
// issue(slot) is called at the start of each step (slots 0..kKS-1: the S/dS
// steps, then kKS.. the P V steps).
// Online-softmax order: the accumulators hold sums normalised to the running
// max m; a raised max rescales them by alpha = 2^(m_old - m_new) before this
// block's P V is added.
template <int D, int kMode, typename Issue>
__device__ __attribute__((always_inline)) inline void qk_phase(
    f32x16& s, f32x16& ds, const char* kbase, const char* dkbase, const u32x4* qf,
    const u32x4* dqf, int lane16, Issue issue) {
  using M = Mode<kMode>;
  using G = Geo<D, M::kKV>;
  // S^T and dS^T (rows: key, columns: this wave's queries).  The K and dK
  // fragments are read at their own step (the other wave on the SIMD covers
  // the LDS latency); scheduling barriers keep the compiler from hoisting
  // reads, and their registers, across steps.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < G::kKS; ++ks) {
    issue(ks);
    const u32x4 kf = lds_load16(kbase + lane16 + ks * kDmaBytes);
    u32x4 dkf;
    if constexpr (M::kKV) dkf = lds_load16(dkbase + lane16 + ks * kDmaBytes);
    s = mma_bf16(kf, qf[ks], ks == 0 ? f32x16{} : s);
    ds = mma_bf16(kf, dqf[ks], ks == 0 ? f32x16{} : ds);
    if constexpr (M::kKV) ds = mma_bf16(dkf, qf[ks], ds);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D, int kMode, bool kMask, int kPath, typename Issue>
__device__ __attribute__((always_inline)) inline void sm_pv_phase(
    RowState<D>& st, f32x16 s, f32x16 ds, const char* vbase, const char* dvbase, int lane16,
    int g, int key0, int Nk, float c_log2, float scale, uint32_t dv_mul, Issue issue) {
  using M = Mode<kMode>;
  using G = Geo<D, M::kKV>;
  // running max (NaN-propagating maximum, combined across the half-waves)
  if constexpr (kMask) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (key0 + slot_key(r, g) >= Nk) s[r] = -INFINITY;
  }
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, s[r]);
  mx = halves_max(mx);
  const float mt = mx * c_log2;
  const float m_new = (mt > st.m + kTau) ? mt : st.m;
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
  st.m = m_new;

  // P and s*P*dS, rounded to fp16 in pairs straight into the B operands of the
  // second contraction; l and u sum exactly those rounded values (one dot
  // instruction per pair), so the weights of the normalisation are the ones
  // the matrix cores multiply: O is an exact convex combination of V's rows
  // and sum_j (p_j s dS_j - mu p_j) cancels as it must.
  u32x4 p[2], pd[2];
  float lsum = 0.f, usum = 0.f;
  const float su = __builtin_bit_cast(float, dv_mul);  // kPathSepU: s 2^tu
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    float pp[2], pdd[2], pdu[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int r = 2 * q + e;
      pp[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, -m_new));
      // keys past Nk: p = 0 (their K and dK rows are zero, so dS is 0 there
      // unless the row's own Q or dQ is not finite)
      if (kMask && key0 + slot_key(r, g) >= Nk) pp[e] = 0.f;
      pdd[e] = pp[e] * ds[r] * scale;
      if constexpr (kPath == kPathSepU) pdu[e] = pp[e] * ds[r] * su;
    }
    const uint32_t hp = pack_f16x2(pp[0], pp[1]);
    p[q >> 2][q & 3] = hp;
    lsum = add_f16x2(hp, lsum);
    const uint32_t hd = pack_f16x2(pdd[0], pdd[1]);
    pd[q >> 2][q & 3] = hd;
    if constexpr (kPath == kPathSepU)
      usum = add_f16x2(pack_f16x2(pdu[0], pdu[1]), usum);
    else
      usum = add_f16x2(hd, usum);
  }
  st.l = st.l * alpha + lsum;
  st.u = st.u * alpha + usum;
  // Pin the sums here (empty asm: a register constraint only); left alone, the
  // compiler sinks them into the next block and keeps P alive until then.
  asm volatile("" : "+v"(st.l), "+v"(st.u));
  if (wave_any(alpha != 1.0f)) {
#pragma unroll
    for (int cb = 0; cb < G::kCB; ++cb) {
      st.accA[cb] *= alpha;
      st.accG[cb] *= alpha;
    }
  }

  __builtin_amdgcn_sched_barrier(0);

  // A^T += V^T P^T, G^T += V^T (s P dS)^T + dV^T P^T; step = (t, cb), its
  // V^T and dV^T fragments read one step ahead (S and dS are dead by now, so
  // the prefetch registers come free)
  constexpr int kSteps = 2 * G::kCB;
  auto voff = [&](int step) {  // fragment t kCB + cb of the block, step = t kCB + cb
    return lane16 + step * kDmaBytes;
  };
  u32x4 vf[2], dvf[2];
  vf[0] = lds_load16(vbase + voff(0));
  if constexpr (M::kKV) dvf[0] = lds_load16(dvbase + voff(0));
#pragma unroll
  for (int step = 0; step < kSteps; ++step) {
    const int t = step / G::kCB, cb = step % G::kCB;
    issue(G::kKS + step);
    if (step + 1 < kSteps) {
      vf[(step + 1) & 1] = lds_load16(vbase + voff(step + 1));
      if constexpr (M::kKV) dvf[(step + 1) & 1] = lds_load16(dvbase + voff(step + 1));
    }
    st.accA[cb] = mma_f16(vf[step & 1], p[t], st.accA[cb]);
    st.accG[cb] = mma_f16(vf[step & 1], pd[t], st.accG[cb]);
    if constexpr (M::kKV) {
      u32x4 dvx = dvf[step & 1];
      if constexpr (kPath == kPathScaleDV) dvx = mul_f16x8(dvx, dv_mul);
      st.accG[cb] = mma_f16(dvx, p[t], st.accG[cb]);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// One 32-key block whose K, dK, V^T and dV^T fragments start at the four
// given LDS addresses (fragment f of a part at its base + f KiB): both phases
// back to back.
template <int D, int kMode, bool kMask, int kPath, typename Issue>
__device__ __attribute__((always_inline)) inline void jvp_block_at(
    RowState<D>& st, const char* kp, const char* dkp, const char* vp, const char* dvp,
    const u32x4* qf, const u32x4* dqf, int l32, int g, int key0, int Nk, float c_log2,
    float scale, uint32_t dv_mul, Issue issue) {
  const int lane16 = 16 * l32 + 512 * g;  // this lane's 16 bytes of a fragment
  f32x16 s, ds;
  qk_phase<D, kMode>(s, ds, kp, dkp, qf, dqf, lane16, issue);
  sm_pv_phase<D, kMode, kMask, kPath>(st, s, ds, vp, dvp, lane16, g, key0, Nk, c_log2, scale,
                                         dv_mul, issue);
}

// Block `kb` of the 64-key tile image in `stage`.
template <int D, int kMode, bool kMask, int kPath, typename Issue>
__device__ __attribute__((always_inline)) inline void jvp_block(
    RowState<D>& st, const char* stage, int kb, const u32x4* qf, const u32x4* dqf, int l32,
    int g, int key0, int Nk, float c_log2, float scale, uint32_t dv_mul, Issue issue) {
  using G = Geo<D, Mode<kMode>::kKV>;
  const int kf0 = kb * G::kKS * kDmaBytes, vf0 = 2 * kb * G::kCB * kDmaBytes;
  jvp_block_at<D, kMode, kMask, kPath>(st, stage + kf0, stage + G::kOffdK + kf0,
                                          stage + G::kOffV + vf0, stage + G::kOffdV + vf0, qf,
                                          dqf, l32, g, key0, Nk, c_log2, scale, dv_mul, issue);
}

// One full tile: the copy of the next tile image into `next` is spread over
// the first steps of the first block (copy instruction j at step j, so the
// copy queue holds one load per wave at a time), while both 32-key blocks are
// computed from `cur`.  The two stage pointers are restrict-qualified (they
// name disjoint halves of the LDS), which tells the compiler that reads of
// `cur` need not wait for the copy into `next`.
template <int D, int kMode, int kPath, typename Copy>
__device__ __attribute__((always_inline)) inline void tile_step(
    char* __restrict__ next, const char* __restrict__ cur, Copy copy, RowState<D>& st,
    const u32x4* qf, const u32x4* dqf, int l32, int g, int Nk, float c_log2, float scale,
    uint32_t dv_mul) {
  using G = Geo<D, Mode<kMode>::kKV>;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
    jvp_block<D, kMode, false, kPath>(st, cur, kb, qf, dqf, l32, g, 0, Nk, c_log2, scale,
                                         dv_mul, [&](int slot) {
                                           if (kb == 0 && slot < G::kDmaPerWave) copy(next, slot);
                                         });
}

// Sizes of the whole tensors (bytes) the kernel may touch; each global access
// is checked against them by the buffer descriptor.
struct Extents {
  uint32_t q_bytes, o_bytes, lse_bytes;
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Four consecutive outputs of one row: 16 bytes of fp32, or 8 bytes of bf16.
// The stores carry the non-temporal hint: outputs are written once and not
// read again by this kernel, so they should not push the tile images out of
// L2 (same-box A/B: text_cross 0.336 -> 0.298 ms, image_dit 0.670 -> 0.650).
template <bool kBf16>
__device__ __attribute__((always_inline)) inline void store4(__amdgpu_buffer_rsrc_t r,
                                                             uint32_t elem, f32x4 x) {
  constexpr int kNonTemporal = 2;  // the nt cache-policy bit of a buffer store
  if constexpr (kBf16) {
    bf16x4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = (__bf16)x[e];
    __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, h), r, (int)(elem * 2), 0,
                                          kNonTemporal);
  } else {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, (int)(elem * 4), 0,
                                           kNonTemporal);
  }
}

// Row-ordered output stores.  A wave's accumulators hold, for query row l32
// of its 32 (lanes l32 and l32 + 32), the columns 32 cb + 8 qq + 4 g + e; a
// store straight from them writes 32 bytes into each of 32 rows per
// instruction.  Each 32-column block instead passes through the wave's own
// stage of 32 rows x kRowPitch floats in LDS and is read back by rows, so one
// store instruction writes 8 whole rows of the block (128 bytes each in fp32:
// a whole cache line).  The 4 floats of padding per row put the rows' first
// words in different banks.  The stage is the wave's alone and a wave's LDS
// operations complete in the order it issues them, so the block's reads see
// its writes and the next block's writes come after them without a barrier.
constexpr int kRowPitch = 36;                    // floats per staged row
constexpr int kStageBytes = 32 * kRowPitch * 4;  // one wave's stage
template <int D, bool kOutBf16, typename Val>
__device__ __attribute__((always_inline)) inline void store_rows(float* stage,
                                                                 __amdgpu_buffer_rsrc_t r,
                                                                 uint32_t elem0, int nrows,
                                                                 int l32, int g, Val val) {
  const int rr = (l32 >> 3) + 4 * g, cc = 4 * (l32 & 7);  // lane = l32 + 32 g reads row rr
#pragma unroll
  for (int cb = 0; cb < D / 32; ++cb) {
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = val(cb, 4 * qq + e);
      *reinterpret_cast<f32x4*>(stage + l32 * kRowPitch + 8 * qq + 4 * g) = v;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rw = 8 * i + rr;
      const f32x4 x = *reinterpret_cast<const f32x4*>(stage + rw * kRowPitch + cc);
      if (rw < nrows) store4<kOutBf16>(r, elem0 + (uint32_t)rw * D + 32 * cb + cc, x);
    }
    // one block's values in flight at a time (the scheduler would otherwise
    // hoist every block's reads and run out of registers)
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Epilogue of one wave: O = A 2^-ea / l, mu = u 2^-eu / l,
// dO = G 2^-eg / l - mu O, lse and tlse = mu for this lane's query row of
// output slice obh (rows past Nq are not stored).  The accumulators hold A,
// G and u scaled by 2^ea, 2^eg and 2^eu (the fp16 exponents of V and of the
// tangent terms); multiplying 1/l by a power of two is exact.  O and dO go
// out through the wave's LDS stage (store_rows); every wave of the workgroup
// must be done reading the tile stages the stage overlaps.
template <int D, bool kOutBf16>
__device__ __attribute__((always_inline)) inline void jvp_epilogue(
    const RowState<D>& st, float* stage, uint32_t obh, int row, int Nq, int l32, int g, void* o,
    void* to, float* lse, float* tlse, const Extents& ext, int ea, int eg, int eu) {
  const float l = halves_sum(st.l);
  const float inv_l = 1.0f / l;
  const float fa = __builtin_amdgcn_ldexpf(inv_l, -ea), fg = __builtin_amdgcn_ldexpf(inv_l, -eg);
  const float mu = halves_sum(st.u) * __builtin_amdgcn_ldexpf(inv_l, -eu);
  const int row0 = row - l32;  // the wave's first row
  const uint32_t elem0 = (obh * (uint32_t)Nq + row0) * D;
  store_rows<D, kOutBf16>(stage, make_rsrc(o, ext.o_bytes), elem0, Nq - row0, l32, g,
                          [&](int cb, int i) { return st.accA[cb][i] * fa; });
  store_rows<D, kOutBf16>(stage, make_rsrc(to, ext.o_bytes), elem0, Nq - row0, l32, g,
                          [&](int cb, int i) {
                            const float a = st.accA[cb][i] * fa;
                            return st.accG[cb][i] * fg - mu * a;
                          });
  if (row < Nq && g == 0) {
    const uint32_t off = (obh * (uint32_t)Nq + row) * 4;
    if (lse != nullptr)
      buf_store4(make_rsrc(lse, ext.lse_bytes), off, (st.m + __log2f(l)) * kLn2);
    if (tlse != nullptr) buf_store4(make_rsrc(tlse, ext.lse_bytes), off, mu);
  }
}

template <bool B>
struct Flag {
  static constexpr bool value = B;
};
template <int N>
struct IntC {
  static constexpr int value = N;
};

// A wave's fp16 exponents: eV of the slice (header record), and the tangent
// exponent t of s P dS, from the bound |s dS_ij| <= |s| (|dq_i| Mk + |q_i| Mdk)
// (Cauchy-Schwarz) over the wave's rows i (row norms from its Q and dQ
// fragments; see sumsq_f32) and all keys of the slice (Mk, Mdk: the largest
// key norms, from the header).
// With dV present, t is the slice's edV - eV (dV was packed at 2^(eV + t))
// unless the bound needs a smaller one; then the path is kPathScaleDV and
// dv_mul = 2^(t - edV + eV) rescales the dV^T fragments.  If instead the bound
// is far below the range that t leaves to s P dS (bound 2^t < 1, so every
// s P dS 2^t is under 16 and may sit among fp16's subnormals), the products
// keep t (their part of dO is then below dV's by more than fp32 resolves) but
// u, the sum behind mu and the tangent of lse, is taken from s P dS 2^tu with
// tu from the bound (kPathSepU; dv_mul carries the float s 2^tu).  Without dV
// (frozen keys, or dV = 0) any t is consistent and the bound alone sets it.
struct WaveScale {
  int ev, t;
  int eu;           // exponent of u: t, or tu on kPathSepU
  float s_t;        // scale 2^t
  uint32_t dv_mul;  // kPathScaleDV: two fp16 copies of 2^(t - edV + eV); kPathSepU: s 2^tu
  int path;         // kPathFast, kPathScaleDV or kPathSepU (wave-uniform)
};

// A negative scale s: s Q K^T = |s| (-Q) K^T and s (dQ K^T + Q dK^T) =
// |s| ((-dQ) K^T + (-Q) dK^T), so flipping the sign bits of the Q and dQ
// fragments (exact in bf16) and working with |s| from here on gives every
// scaled logit and tangent term unchanged, while the running max of the
// online softmax is taken over the logits as they are (max_j s S_ij, not
// s max_j S_ij).
template <int D>
__device__ __attribute__((always_inline)) inline void flip_negative_scale(
    u32x4* qf, u32x4* dqf, float& scale, float& c_log2) {
  if (scale < 0.f) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      qf[ks] ^= 0x80008000u;
      dqf[ks] ^= 0x80008000u;
    }
    scale = -scale;
    c_log2 = -c_log2;
  }
}

// What wave_scale reads from the slice header: the record and this lane's
// norm slot.  Loaded apart from the rest so that a kernel can issue the loads
// before its Q and dQ loads and have them arrive together.
struct ScaleLoads {
  u32x4 rec;
  float mk, mdk;  // this lane's norm slot (reduced over the wave in wave_scale)
};
__device__ __attribute__((always_inline)) inline ScaleLoads scale_loads(
    __amdgpu_buffer_rsrc_t rimg, uint32_t hdr, int ntiles, int lane) {
  ScaleLoads sl;
  sl.rec = buf_load16(rimg, hdr + kHdrRecord);
  slice_norm_slots(rimg, hdr, ntiles, lane, sl.mk, sl.mdk);
  return sl;
}

// Squares of the 64 bf16 values of a lane's D / 16 fragments, summed in fp32
// by v_dot2 (each product exact): the sum and the OR of the values' bits.
template <int D>
__device__ __attribute__((always_inline)) inline float sumsq_f32(const u32x4* f, uint32_t& bits) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  float s = 0.f;
  bits = 0;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const bf16x2 x = __builtin_bit_cast(bf16x2, f[ks][w]);
      s = __builtin_amdgcn_fdot2_f32_bf16(x, x, s, false);
      bits |= f[ks][w];
    }
  return s;
}

// fp32 sum of squares that stands for the exact one: no term overflowed (sum
// at most 2^100) and the terms lost to underflow (each below 2^-126, at most
// 64) are under 2^-20 of it (sum at least 2^-100), or every value is zero.
__device__ inline bool sumsq_f32_usable(float s, uint32_t bits) {
  return (s >= 0x1p-100f && s <= 0x1p100f) || (bits & 0x7fff7fffu) == 0;
}

template <int D, bool kKV>
__device__ __attribute__((always_inline)) inline WaveScale wave_scale(
    const ScaleLoads& sl, const u32x4* qf, const u32x4* dqf, float scale) {
  const u32x4 rec = sl.rec;
  const float mk = wave_max_f32(sl.mk), mdk = wave_max_f32(sl.mdk);
  // Row norms: the fp32 sums of squares when every lane's are usable as they
  // are (the bound needs far less than fp32's precision), else fp64 sums.
  uint32_t bq = 0, bdq;
  const float fdq = sumsq_f32<D>(dqf, bdq);
  const float fq = kKV ? sumsq_f32<D>(qf, bq) : 0.f;
  double nq = 0.0, ndq = 0.0;
  if (!wave_any(!(sumsq_f32_usable(fdq, bdq) && sumsq_f32_usable(fq, bq)))) {
    ndq = fdq;
    nq = fq;
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      if constexpr (kKV) nq += sumsq8(qf[ks]);
      ndq += sumsq8(dqf[ks]);
    }
  }
  double b = __builtin_sqrt(halves_sum_f64(ndq)) * (double)mk;
  if constexpr (kKV) b += __builtin_sqrt(halves_sum_f64(nq)) * (double)mdk;
  b *= __builtin_fabs((double)scale);
  // A row (or key) with an Inf or NaN gives a non-finite bound; its outputs
  // are non-finite whatever t is, so it does not take part in the wave's choice.
  b = wave_max_f64(__builtin_isfinite(b) ? b : 0.0);
  const int ev = __builtin_amdgcn_readfirstlane((int)rec[0]);
  const int edv = __builtin_amdgcn_readfirstlane((int)rec[1]);
  const uint32_t flags = __builtin_amdgcn_readfirstlane(rec[2]);
  WaveScale w;
  w.ev = ev;
  w.path = kPathFast;
  w.dv_mul = 0x3c003c00u;  // 1.0, 1.0
  int t, tu;
  if (!kKV || (flags & kDvZero)) {
    t = product_exponent(b);
    tu = t;
  } else {
    const int th = edv - ev;
    const double bh = __builtin_ldexp(b, th);
    const bool slow = bh > kProdSafe;  // false for NaN
    t = slow ? product_exponent(b) : th;
    tu = product_exponent(b);
    w.path = __builtin_amdgcn_readfirstlane(slow ? kPathScaleDV : bh < 1.0 ? kPathSepU : kPathFast);
    if (w.path == kPathSepU) {
      w.dv_mul = __builtin_bit_cast(uint32_t, __builtin_amdgcn_ldexpf(scale, tu));
    } else {
      const _Float16 m = (_Float16)__builtin_amdgcn_ldexpf(1.0f, t - th);
      w.dv_mul = (uint32_t)__builtin_bit_cast(uint16_t, m) * 0x10001u;
    }
  }
  w.t = __builtin_amdgcn_readfirstlane(t);
  w.eu = __builtin_amdgcn_readfirstlane(w.path == kPathSepU ? tu : t);
  w.dv_mul = __builtin_amdgcn_readfirstlane(w.dv_mul);
  w.s_t = __builtin_bit_cast(
      float, __builtin_amdgcn_readfirstlane(
                 __builtin_bit_cast(int, __builtin_amdgcn_ldexpf(scale, w.t))));
  return w;
}

// o, to: [B, H, Nq, D] in fp32 (kOutBf16 false) or bf16; lse, tlse: [B, H, Nq]
// fp32, each may be NULL.  Two waves per SIMD (256 registers each).
// Split-KV: with nsplit > 1 the key tiles are cut into ranges of tps tiles;
// split s computes the state over its range alone and writes it as (b, h)
// slice s * nbh + bh of o, to, lse and tlse (partial results that the merge
// kernel combines).  nsplit = 1, tps = ntiles is the plain pass.
template <int D, int kMode, bool kOutBf16>
__global__ __launch_bounds__(kThreads, 2) void attn_jvp_bf16_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ tq,
    const char* __restrict__ img, void* __restrict__ o, void* __restrict__ to,
    float* __restrict__ lse, float* __restrict__ tlse, int Nq, int Nk, int ntiles, int nqt,
    int nbh, int tps, Extents ext, float scale, float c_log2) {
  using M = Mode<kMode>;
  using G = Geo<D, M::kKV>;
  __shared__ __attribute__((aligned(1024)))
  char smem[2 * G::kImgBytes > kWaves * kStageBytes ? 2 * G::kImgBytes : kWaves * kStageBytes];

  // Work item (query tile qt of kBR rows, (b, h) slice bh, key split) from
  // the linear workgroup id: the dispatcher deals workgroups to the 8 XCDs in
  // turn (id % 8), so XCD x is given the x-th contiguous range of the work
  // list ordered by (split, bh, qt).  The row tiles of one head then run on
  // one XCD and share its L2, which holds the head's tile images once instead
  // of once per XCD.  Any XCD count still gives a bijection (only locality
  // changes).
  const uint32_t wg = blockIdx.x, nwg = gridDim.x;
  const uint32_t xcd = wg % kXcds, slot = wg / kXcds, per = nwg / kXcds, extra = nwg % kXcds;
  const uint32_t work = xcd < extra ? xcd * (per + 1) + slot
                                    : extra * (per + 1) + (xcd - extra) * per + slot;
  const int qt = (int)(work % (uint32_t)nqt);
  const uint32_t obh = work / (uint32_t)nqt;  // output slice: split * nbh + bh
  const uint32_t bh = obh % (uint32_t)nbh;
  const int t0 = (int)(obh / (uint32_t)nbh) * tps;
  const int t1 = t0 + tps < ntiles ? t0 + tps : ntiles;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int row = qt * kBR + wave * kRowsPerWave + l32;
  const bool row_ok = row < Nq;

  // Buffer descriptors over whole tensors (see Extents); a NULL tq reads zeros.
  const auto rq = make_rsrc(q, ext.q_bytes);
  const auto rtq = make_rsrc(tq, tq != nullptr ? ext.q_bytes : 0u);
  // the workspace descriptor spans this (b, h) slice's tile images and header
  const uint32_t sb = slice_bytes<D, M::kKV>(ntiles);
  const auto rimg = make_rsrc(img + (size_t)bh * sb, sb);
  const uint32_t hdr = (uint32_t)ntiles * G::kImgBytes;

  // Copy of tile image kt into a stage: this wave's kDmaPerWave consecutive
  // KiB, lane l moving bytes 16 l .. 16 l + 15 of each (LDS address = the
  // wave-uniform stage pointer + 16 l; global = image offset + 16 l).
  const uint32_t wave_part = (uint32_t)wave * G::kDmaPerWave * kDmaBytes;
  auto copy_one = [&](int kt, char* stage, int j) {
    const uint32_t src = (uint32_t)kt * G::kImgBytes + wave_part + j * kDmaBytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rimg, (lds_ptr_t)(stage + wave_part + j * kDmaBytes),
                                             16, lane * 16, src, 0, 0);
  };
#pragma unroll
  for (int j = 0; j < G::kDmaPerWave; ++j) copy_one(t0, smem, j);

  // Q and dQ fragments: the B operand of S^T = K Q^T (lane: row l32, d-slice g).
  // Rows past Nq get an offset past the tensor, which the descriptor reads as 0.
  const ScaleLoads sl = scale_loads(rimg, hdr, ntiles, lane);
  u32x4 qf[G::kKS], dqf[G::kKS];
  const uint32_t qrow = row_ok ? (bh * (uint32_t)Nq + row) * D * 2 : 0x80000000u;
#pragma unroll
  for (int ks = 0; ks < G::kKS; ++ks) {
    const uint32_t off = qrow + (16 * ks + 8 * g) * 2;
    qf[ks] = buf_load16(rq, off);
    dqf[ks] = buf_load16(rtq, off);
  }

  flip_negative_scale<D>(qf, dqf, scale, c_log2);
  const WaveScale sc = wave_scale<D, M::kKV>(sl, qf, dqf, scale);

  RowState<D> st;
#pragma unroll
  for (int cb = 0; cb < G::kCB; ++cb) {
    st.accA[cb] = f32x16{};
    st.accG[cb] = f32x16{};
  }
  st.m = -INFINITY;
  st.l = 0.f;
  st.u = 0.f;

  // Tile kt is computed from stage (kt - t0) % 2 while tile kt + 1 is copied
  // into the other stage; the wait for the copies and the barrier at the end
  // of each tile make tile kt + 1 visible to every wave and retire every read
  // of the stage the next copy overwrites.  Both forms of the loop (with and
  // without the dV^T rescale) run the same barriers.
  const int kLast = t1 - 1;
  auto finish_tile = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  auto key_loop = [&](auto path) {
    constexpr int kS = decltype(path)::value;
    finish_tile();
    for (int kt = t0; kt < kLast; ++kt) {
      const int cs = (kt - t0) & 1;
      tile_step<D, kMode, kS>(smem + (cs ^ 1) * G::kImgBytes, smem + cs * G::kImgBytes,
                              [&](char* next, int j) { copy_one(kt + 1, next, j); }, st, qf, dqf,
                              l32, g, Nk, c_log2, sc.s_t, sc.dv_mul);
      finish_tile();
    }
    // last tile of the range: keys past Nk are masked (the tile image holds
    // zeros there; in a range that ends before the last tile nothing is masked)
    const char* cur = smem + ((kLast - t0) & 1) * G::kImgBytes;
    const int kl = kLast * kBC;
    auto none = [](int) {};
    jvp_block<D, kMode, true, kS>(st, cur, 0, qf, dqf, l32, g, kl, Nk, c_log2, sc.s_t,
                                  sc.dv_mul, none);
    jvp_block<D, kMode, true, kS>(st, cur, 1, qf, dqf, l32, g, kl + 32, Nk, c_log2, sc.s_t,
                                  sc.dv_mul, none);
  };
  if (M::kKV && sc.path == kPathScaleDV)
    key_loop(IntC<M::kKV ? kPathScaleDV : kPathFast>{});
  else if (M::kKV && sc.path == kPathSepU)
    key_loop(IntC<M::kKV ? kPathSepU : kPathFast>{});
  else
    key_loop(IntC<kPathFast>{});

  __syncthreads();  // the output stages overlap the tile stages
  jvp_epilogue<D, kOutBf16>(st, reinterpret_cast<float*>(smem + wave * kStageBytes), obh, row,
                            Nq, l32, g, o, to, lse, tlse, ext, sc.ev, sc.ev + sc.t, sc.eu);
}

// ---- short key ranges: 128-row workgroups, two per CU ----
// With few key tiles per work item (cross-attention to a short text, or a
// short split-KV range) the 256-row kernel spends a large share of its time
// loading Q, dQ and storing O, dO, and with one workgroup per CU nothing runs
// beside those memory phases.  Here a workgroup holds 4 waves (128 rows), so
// two fit on a CU (registers: 2 x 4 waves x 256 = two waves per SIMD, as
// before) and one computes while the other loads, stores or waits.  The key
// range is streamed in 32-key halves of the tile images: the half-stage holds
// one block's K, dK, V^T and dV^T fragments (32 KiB at d = 128 with the
// tangents), and two half-stages alternate, so the copy of the next block
// runs under the products of the current one (LDS: 2 x 64 KiB per CU at
// d = 128).  Per row the arithmetic is that of the 256-row kernel (same
// blocks, same key order), so the results are the same bit for bit.
constexpr int kShortWaves = 4;
constexpr int kShortThreads = 64 * kShortWaves;
constexpr int kShortBR = kShortWaves * kRowsPerWave;  // query rows per workgroup
// Work items of at most this many key tiles take the short kernel.  Measured
// at H = 12, Nq = 32760 against the 256-row kernel: 64 keys 146 vs 171 us, 256
// keys 220 vs 245, 512 keys 337 vs 369, 1024 keys 551 vs 567; 2048 keys 1034
// vs 1021 and B H = 32, N = 4096 750 vs 701 (there the doubled tile stream per
// row costs more than the overlap gains).
constexpr int kShortMaxTiles = 16;

// One 32-key block of a tile image as the short kernel stages it: its K, dK,
// V^T, dV^T parts (kF fragments each; K and dK blocks are kKS fragments, V^T
// and dV^T blocks 2 kCB, both D / 16) back to back.  Fragment i of block kb of
// tile kt comes from image offset kt img + (i / kF) kPart + kb kF KiB + (i % kF)
// KiB, since every part of the image spans the same kPart bytes.
template <int D, bool kKV>
struct HalfGeo {
  using G = Geo<D, kKV>;
  static constexpr int kF = D / 16;
  static constexpr int kPart = G::kKTile;
  static constexpr int kParts = 2 * G::kNT;
  static constexpr int kBytes = kParts * kF * kDmaBytes;
  static constexpr int kPerWave = kBytes / (kShortWaves * kDmaBytes);
  static_assert(G::kKTile == G::kVTile && G::kOffV == G::kNT * kPart && 2 * G::kCB == kF &&
                    G::kKS == kF && kPerWave * kShortWaves * kDmaBytes == kBytes,
                "half-stage layout");
};

// One block of the short kernel: computed from half-stage `cur` while
// copy(next, slot) fills the other half-stage over the block's first steps.
// As in tile_step, the two restrict-qualified pointers name disjoint halves of
// the LDS, so reads of `cur` need not wait for the copy into `next`.
template <int D, int kMode, bool kMask, int kPath, typename Copy>
__device__ __attribute__((always_inline)) inline void short_block(
    char* __restrict__ next, const char* __restrict__ cur, Copy copy, RowState<D>& st,
    const u32x4* qf, const u32x4* dqf, int l32, int g, int key0, int Nk, float c_log2,
    float scale, uint32_t dv_mul) {
  using M = Mode<kMode>;
  using G = Geo<D, M::kKV>;
  using HG = HalfGeo<D, M::kKV>;
  const char* dkp = cur + (M::kKV ? HG::kF * kDmaBytes : 0);
  const char* vp = cur + G::kNT * HG::kF * kDmaBytes;
  const char* dvp = vp + (M::kKV ? HG::kF * kDmaBytes : 0);
  jvp_block_at<D, kMode, kMask, kPath>(st, cur, dkp, vp, dvp, qf, dqf, l32, g, key0, Nk,
                                          c_log2, scale, dv_mul, [&](int slot) {
                                            if (slot < HG::kPerWave) copy(next, slot);
                                          });
}

template <int D, int kMode, bool kOutBf16>
__global__ __launch_bounds__(kShortThreads, 2) void attn_jvp_bf16_short_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ tq,
    const char* __restrict__ img, void* __restrict__ o, void* __restrict__ to,
    float* __restrict__ lse, float* __restrict__ tlse, int Nq, int Nk, int ntiles, int nqt,
    int nbh, int tps, Extents ext, float scale, float c_log2) {
  using M = Mode<kMode>;
  using G = Geo<D, M::kKV>;
  using HG = HalfGeo<D, M::kKV>;
  __shared__ __attribute__((aligned(1024)))
  char smem[2 * HG::kBytes > kShortWaves * kStageBytes ? 2 * HG::kBytes
                                                       : kShortWaves * kStageBytes];

  // work item: as in attn_jvp_bf16_kernel, with row tiles of kShortBR rows
  const uint32_t wg = blockIdx.x, nwg = gridDim.x;
  const uint32_t xcd = wg % kXcds, slot = wg / kXcds, per = nwg / kXcds, extra = nwg % kXcds;
  const uint32_t work = xcd < extra ? xcd * (per + 1) + slot
                                    : extra * (per + 1) + (xcd - extra) * per + slot;
  const int qt = (int)(work % (uint32_t)nqt);
  const uint32_t obh = work / (uint32_t)nqt;
  const uint32_t bh = obh % (uint32_t)nbh;
  const int t0 = (int)(obh / (uint32_t)nbh) * tps;
  const int t1 = t0 + tps < ntiles ? t0 + tps : ntiles;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int row = qt * kShortBR + wave * kRowsPerWave + l32;
  const bool row_ok = row < Nq;

  const auto rq = make_rsrc(q, ext.q_bytes);
  const auto rtq = make_rsrc(tq, tq != nullptr ? ext.q_bytes : 0u);
  const uint32_t sb = slice_bytes<D, M::kKV>(ntiles);
  const auto rimg = make_rsrc(img + (size_t)bh * sb, sb);
  const uint32_t hdr = (uint32_t)ntiles * G::kImgBytes;

  // Copy of block h of the range (tile t0 + h / 2, block h % 2) into a
  // half-stage: this wave's kPerWave consecutive fragments of it, 1 KiB per
  // instruction, lane l moving bytes 16 l .. 16 l + 15.
  auto copy_half = [&](int h, char* stage, int j) {
    const int i = wave * HG::kPerWave + j;
    const uint32_t src = (uint32_t)(t0 + (h >> 1)) * G::kImgBytes + (i / HG::kF) * HG::kPart +
                         ((h & 1) * HG::kF + i % HG::kF) * kDmaBytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rimg, (lds_ptr_t)(stage + i * kDmaBytes), 16,
                                             lane * 16, src, 0, 0);
  };
#pragma unroll
  for (int j = 0; j < HG::kPerWave; ++j) copy_half(0, smem, j);

  const ScaleLoads sl = scale_loads(rimg, hdr, ntiles, lane);
  u32x4 qf[G::kKS], dqf[G::kKS];
  const uint32_t qrow = row_ok ? (bh * (uint32_t)Nq + row) * D * 2 : 0x80000000u;
#pragma unroll
  for (int ks = 0; ks < G::kKS; ++ks) {
    const uint32_t off = qrow + (16 * ks + 8 * g) * 2;
    qf[ks] = buf_load16(rq, off);
    dqf[ks] = buf_load16(rtq, off);
  }

  flip_negative_scale<D>(qf, dqf, scale, c_log2);
  const WaveScale sc = wave_scale<D, M::kKV>(sl, qf, dqf, scale);

  RowState<D> st;
#pragma unroll
  for (int cb = 0; cb < G::kCB; ++cb) {
    st.accA[cb] = f32x16{};
    st.accG[cb] = f32x16{};
  }
  st.m = -INFINITY;
  st.l = 0.f;
  st.u = 0.f;

  // Block h: wait for its copy (every wave's share) and make it visible; the
  // same barrier retires every read of block h - 1, whose half-stage the copy
  // of block h + 1 (issued over the first steps of block h) overwrites.  The
  // two blocks of the last tile are masked (keys >= Nk).  Both forms of the
  // loop (with and without the dV^T rescale) run the same barriers.
  const int nh = 2 * (t1 - t0);
  auto block_ready = [&]() {
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  auto block = [&](int h, auto mask, auto path, bool copy_next) {
    constexpr bool kMk = decltype(mask)::value;
    constexpr int kS = decltype(path)::value;
    short_block<D, kMode, kMk, kS>(
        smem + ((h + 1) & 1) * HG::kBytes, smem + (h & 1) * HG::kBytes,
        [&](char* next, int j) {
          if (copy_next) copy_half(h + 1, next, j);
        },
        st, qf, dqf, l32, g, (t0 + (h >> 1)) * kBC + 32 * (h & 1), Nk, c_log2, sc.s_t,
        sc.dv_mul);
  };
  auto key_loop = [&](auto path) {
    int h = 0;
    for (; h < nh - 2; ++h) {
      block_ready();
      block(h, Flag<false>{}, path, true);
    }
    block_ready();
    block(h, Flag<true>{}, path, true);
    block_ready();
    block(h + 1, Flag<true>{}, path, false);
  };
  if (M::kKV && sc.path == kPathScaleDV)
    key_loop(IntC<M::kKV ? kPathScaleDV : kPathFast>{});
  else if (M::kKV && sc.path == kPathSepU)
    key_loop(IntC<M::kKV ? kPathSepU : kPathFast>{});
  else
    key_loop(IntC<kPathFast>{});

  __syncthreads();  // the output stages overlap the tile stages
  jvp_epilogue<D, kOutBf16>(st, reinterpret_cast<float*>(smem + wave * kStageBytes), obh, row,
                            Nq, l32, g, o, to, lse, tlse, ext, sc.ev, sc.ev + sc.t, sc.eu);
}

// ---- forward attention alone (O, lse) ----
// RB = 2: each wave holds 64 query rows (two 32-row blocks), so every K and
// V^T fragment it reads from LDS feeds two matrix products, and a workgroup of
// 8 waves covers 512 rows per pass over the key tiles: half the LDS reads and
// half the tile-image stream per row of a 32-row wave.  Registers: 128
// accumulators, 64 for the Q fragments, 32 for the two S blocks; two waves per
// SIMD.  RB = 1 (32 rows per wave, 256 per workgroup, 128 registers, four
// waves per SIMD and two workgroups per CU) is used when its 256-row tiles
// fit the chip one per CU.
template <int RB>
constexpr int fwd_rows() { return kWaves * 32 * RB; }  // query rows per workgroup
// The 64-row form runs its two wave groups a phase apart (fwd_tile_lagged).
constexpr bool kFwdLag = true;

template <int D, int RB>
struct FwdState {
  f32x16 acc[RB][D / 32];  // A^T = sum p v per row block (rows: output column)
  float m[RB];             // running max, log2 units
  float l[RB];             // this lane's half of sum p (of the fp16-rounded p)
};

// One 32-key block for the wave's RB row blocks; same arithmetic as the
// tangent-free part of jvp_block (online softmax with the lazy rescale, P
// rounded to fp16 for the second product, l summed from those values).
// S^T of one 32-key block for the wave's RB row blocks (K fragments from the
// stage, Q fragments from registers); issue(ks) runs at step ks.
template <int D, int RB, typename Issue>
__device__ __attribute__((always_inline)) inline void fwd_scores(f32x16 (&s)[RB], const char* stage,
                                                                 int kb, const u32x4 (*qf)[D / 16],
                                                                 int l32, int g, Issue issue) {
  using G = Geo<D, false>;
  const char* sK = stage;
  const int lane16 = 16 * l32 + 512 * g;
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int ks = 0; ks < G::kKS; ++ks) {
    issue(ks);
    const u32x4 kf = lds_load16(sK + lane16 + (kb * G::kKS + ks) * kDmaBytes);
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
      s[rb] = mma_bf16(kf, qf[rb][ks], ks == 0 ? f32x16{} : s[rb]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The online softmax of a block from its S^T, with the lazy rescale of the
// accumulators: P rounded to fp16 pairs in the B-operand layout of the
// second product, l summed from those values.
template <int D, int RB, bool kMask>
__device__ __attribute__((always_inline)) inline void fwd_softmax(FwdState<D, RB>& st,
                                                                  f32x16 (&s)[RB],
                                                                  u32x4 (&p)[RB][2], int g,
                                                                  int key0, int Nk,
                                                                  float c_log2) {
  using G = Geo<D, false>;
  float alpha[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    if constexpr (kMask) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (key0 + slot_key(r, g) >= Nk) s[rb][r] = -INFINITY;
    }
    float mx = s[rb][0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = __builtin_elementwise_maximum(mx, s[rb][r]);
    mx = halves_max(mx);
    const float mt = mx * c_log2;
    const float m_new = (mt > st.m[rb] + kTau) ? mt : st.m[rb];
    alpha[rb] = __builtin_amdgcn_exp2f(st.m[rb] - m_new);
    st.m[rb] = m_new;
    float lsum = 0.f;
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      float pp[2];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int r = 2 * q + e;
        pp[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[rb][r], c_log2, -m_new));
        if (kMask && key0 + slot_key(r, g) >= Nk) pp[e] = 0.f;
      }
      const uint32_t hp = pack_f16x2(pp[0], pp[1]);
      p[rb][q >> 2][q & 3] = hp;
      lsum = add_f16x2(hp, lsum);
    }
    st.l[rb] = st.l[rb] * alpha[rb] + lsum;
  }
  // pin the sums here (an empty asm with register constraints only)
  bool moved = false;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    asm volatile("" : "+v"(st.l[rb]));
    moved = moved || alpha[rb] != 1.0f;
  }
  if (wave_any(moved)) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int cb = 0; cb < G::kCB; ++cb) st.acc[rb][cb] *= alpha[rb];
  }
  __builtin_amdgcn_sched_barrier(0);
}

// A^T += V^T P^T for a block; issue(kKS + step) runs at step `step`.
template <int D, int RB, typename Issue>
__device__ __attribute__((always_inline)) inline void fwd_pv(FwdState<D, RB>& st,
                                                             const u32x4 (&p)[RB][2],
                                                             const char* stage, int kb, int l32,
                                                             int g, Issue issue) {
  using G = Geo<D, false>;
  const char* sV = stage + G::kOffV;
  const int lane16 = 16 * l32 + 512 * g;
  // step = (t, cb) reads fragment
  // (2 kb + t) kCB + cb, one step ahead with two row blocks (the one-block
  // instance, held to 128 registers, reads it at its step)
  constexpr int kSteps = 2 * G::kCB;
  constexpr bool kPf = RB > 1;
  auto voff = [&](int step) { return lane16 + (2 * kb * G::kCB + step) * kDmaBytes; };
  u32x4 vfp[2];
  if constexpr (kPf) vfp[0] = lds_load16(sV + voff(0));
#pragma unroll
  for (int step = 0; step < kSteps; ++step) {
    const int t = step / G::kCB, cb = step % G::kCB;
    issue(G::kKS + step);
    if constexpr (kPf) {
      if (step + 1 < kSteps) vfp[(step + 1) & 1] = lds_load16(sV + voff(step + 1));
    } else {
      vfp[step & 1] = lds_load16(sV + voff(step));
    }
    const u32x4 vf = vfp[step & 1];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) st.acc[rb][cb] = mma_f16(vf, p[rb][t], st.acc[rb][cb]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int D, int RB, bool kMask, typename Issue>
__device__ __attribute__((always_inline)) inline void fwd_finish(FwdState<D, RB>& st,
                                                                 f32x16 (&s)[RB], const char* stage,
                                                                 int kb, int l32, int g, int key0,
                                                                 int Nk, float c_log2,
                                                                 Issue issue) {
  u32x4 p[RB][2];
  fwd_softmax<D, RB, kMask>(st, s, p, g, key0, Nk, c_log2);
  fwd_pv<D, RB>(st, p, stage, kb, l32, g, issue);
}

template <int D, int RB, bool kMask, typename Issue>
__device__ __attribute__((always_inline)) inline void fwd_block(
    FwdState<D, RB>& st, const char* stage, int kb, const u32x4 (*qf)[D / 16], int l32, int g,
    int key0, int Nk, float c_log2, Issue issue) {
  f32x16 s[RB];
  fwd_scores<D, RB>(s, stage, kb, qf, l32, g, issue);
  fwd_finish<D, RB, kMask>(st, s, stage, kb, l32, g, key0, Nk, c_log2, issue);
}

template <int D, int RB, typename Copy>
__device__ __attribute__((always_inline)) inline void fwd_tile(
    char* __restrict__ next, const char* __restrict__ cur, Copy copy, FwdState<D, RB>& st,
    const u32x4 (*qf)[D / 16], int l32, int g, int Nk, float c_log2) {
  using G = Geo<D, false>;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
    fwd_block<D, RB, false>(st, cur, kb, qf, l32, g, 0, Nk, c_log2, [&](int slot) {
      if (kb == 0 && slot < G::kDmaPerWave) copy(next, slot);
    });
}

// One tile of the lagged schedule of the 64-row form.  Waves 0-3 run blocks 0
// and 1 of the tile (scores, softmax, products); waves 4-7, which share their
// SIMDs, run a phase behind: they first run the products of block 1 of the
// previous tile from its P (kept in pl), then block 0, then the scores and
// softmax of block 1, whose products they carry into the next tile.  So while
// one wave of a SIMD is in its softmax the other is mostly in matrix
// products, which a shared per-tile barrier would otherwise keep in step.
// Three stages rotate: the tile's own, the previous one (still read by waves
// 4-7) and the next one (copied during block 0's scores); all three are
// distinct, so the restrict-qualified pointers hold.
template <int D, bool kLag, bool kMask, typename Copy>
__device__ __attribute__((always_inline)) inline void fwd_tile_lagged(
    const char* __restrict__ prev, const char* __restrict__ cur, char* __restrict__ next,
    Copy copy, bool has_prev, FwdState<D, 2>& st, u32x4 (&pl)[2][2],
    const u32x4 (*qf)[D / 16], int l32, int g, int key0, int Nk, float c_log2) {
  using G = Geo<D, false>;
  auto none = [](int) {};
  if (kLag && has_prev) fwd_pv<D, 2>(st, pl, prev, 1, l32, g, none);
  f32x16 s[2];
  fwd_scores<D, 2>(s, cur, 0, qf, l32, g, [&](int slot) {
    if (slot < G::kDmaPerWave) copy(next, slot);
  });
  fwd_finish<D, 2, kMask>(st, s, cur, 0, l32, g, key0, Nk, c_log2, none);
  fwd_scores<D, 2>(s, cur, 1, qf, l32, g, none);
  if constexpr (!kLag)
    fwd_finish<D, 2, kMask>(st, s, cur, 1, l32, g, key0 + 32, Nk, c_log2, none);
  else
    fwd_softmax<D, 2, kMask>(st, s, pl, g, key0 + 32, Nk, c_log2);
}

// o: [B, H, Nq, D] fp32 or bf16; lse: [B, H, Nq] fp32 or NULL.  Tile images
// hold K and V^T only (the layout of the frozen-key mode).
template <int D, int RB, bool kOutBf16>
__global__ __launch_bounds__(kThreads, RB == 2 ? 2 : 4) void attn_fwd_bf16_kernel(
    const uint16_t* __restrict__ q, const char* __restrict__ img, void* __restrict__ o,
    float* __restrict__ lse, int Nq, int Nk, int ntiles, int nqt, int nbh, int tps, Extents ext,
    float c_log2) {
  using G = Geo<D, false>;
  constexpr int kStages = RB == 2 && kFwdLag ? 3 : 2;
  __shared__ __attribute__((aligned(1024)))
  char smem[kStages * G::kImgBytes > kWaves * kStageBytes ? kStages * G::kImgBytes
                                                          : kWaves * kStageBytes];
  // XCD-aware work order and key-tile ranges, as in attn_jvp_bf16_kernel
  const uint32_t wg = blockIdx.x, nwg = gridDim.x;
  const uint32_t xcd = wg % kXcds, slot = wg / kXcds, per = nwg / kXcds, extra = nwg % kXcds;
  const uint32_t work = xcd < extra ? xcd * (per + 1) + slot
                                    : extra * (per + 1) + (xcd - extra) * per + slot;
  const int qt = (int)(work % (uint32_t)nqt);
  const uint32_t obh = work / (uint32_t)nqt;  // output slice: split * nbh + bh
  const uint32_t bh = obh % (uint32_t)nbh;
  const int t0 = (int)(obh / (uint32_t)nbh) * tps;
  const int t1 = t0 + tps < ntiles ? t0 + tps : ntiles;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;
  const int row0 = qt * fwd_rows<RB>() + wave * 32 * RB + l32;  // block rb: row0 + 32 rb

  const auto rq = make_rsrc(q, ext.q_bytes);
  const uint32_t sb = slice_bytes<D, false>(ntiles);
  const auto rimg = make_rsrc(img + (size_t)bh * sb, sb);
  // V's fp16 exponent (slice header): the accumulators hold A 2^eV
  const u32x4 rec = buf_load16(rimg, (uint32_t)ntiles * G::kImgBytes + kHdrRecord);
  const uint32_t wave_part = (uint32_t)wave * G::kDmaPerWave * kDmaBytes;
  auto copy_one = [&](int kt, char* stage, int j) {
    const uint32_t src = (uint32_t)kt * G::kImgBytes + wave_part + j * kDmaBytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rimg, (lds_ptr_t)(stage + wave_part + j * kDmaBytes),
                                             16, lane * 16, src, 0, 0);
  };
#pragma unroll
  for (int j = 0; j < G::kDmaPerWave; ++j) copy_one(t0, smem, j);

  // Q fragments of the row blocks (rows past Nq read as 0 through the descriptor)
  u32x4 qf[RB][G::kKS];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = row0 + 32 * rb;
    const uint32_t qrow = row < Nq ? (bh * (uint32_t)Nq + row) * D * 2 : 0x80000000u;
#pragma unroll
    for (int ks = 0; ks < G::kKS; ++ks) qf[rb][ks] = buf_load16(rq, qrow + (16 * ks + 8 * g) * 2);
  }
  // a negative scale: the logits from -Q with |s| (see flip_negative_scale)
  if (c_log2 < 0.f) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb)
#pragma unroll
      for (int ks = 0; ks < G::kKS; ++ks) qf[rb][ks] ^= 0x80008000u;
    c_log2 = -c_log2;
  }

  FwdState<D, RB> st;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int cb = 0; cb < G::kCB; ++cb) st.acc[rb][cb] = f32x16{};
    st.m[rb] = -INFINITY;
    st.l[rb] = 0.f;
  }

  const int kLast = t1 - 1;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const int ev = __builtin_amdgcn_readfirstlane((int)rec[0]);  // in a scalar register
  if constexpr (RB == 2 && kFwdLag) {
    // waves 4-7 run a phase behind waves 0-3 (fwd_tile_lagged); both groups
    // pass the same barriers
    auto stg = [&](int i) { return smem + i * G::kImgBytes; };
    auto lagged = [&](auto lagc) {
      constexpr bool kL = decltype(lagc)::value;
      u32x4 pl[2][2];
      int cs = 0;  // stage of tile kt; the previous tile's is (cs + 2) % 3, the next one's (cs + 1) % 3
      for (int kt = t0; kt < kLast; ++kt) {
        const int ns = cs == 2 ? 0 : cs + 1, ps = cs == 0 ? 2 : cs - 1;
        fwd_tile_lagged<D, kL, false>(stg(ps), stg(cs), stg(ns),
                                      [&](char* next, int j) { copy_one(kt + 1, next, j); },
                                      kt > t0, st, pl, qf, l32, g, kt * kBC, Nk, c_log2);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        cs = ns;
      }
      // last tile of the range (keys past Nk masked), nothing left to copy
      const int ns = cs == 2 ? 0 : cs + 1, ps = cs == 0 ? 2 : cs - 1;
      const int kl = kLast * kBC;
      fwd_tile_lagged<D, kL, true>(stg(ps), stg(cs), stg(ns), [](char*, int) {}, kLast > t0, st,
                                   pl, qf, l32, g, kl, Nk, c_log2);
      if constexpr (kL) fwd_pv<D, 2>(st, pl, stg(cs), 1, l32, g, [](int) {});
    };
    if (wave >= kWaves / 2)
      lagged(Flag<true>{});
    else
      lagged(Flag<false>{});
  } else {
    for (int kt = t0; kt < kLast; ++kt) {
      const int sc = (kt - t0) & 1;
      fwd_tile<D, RB>(smem + (sc ^ 1) * G::kImgBytes, smem + sc * G::kImgBytes,
                      [&](char* next, int j) { copy_one(kt + 1, next, j); }, st, qf, l32, g, Nk,
                      c_log2);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    }
    const char* cur = smem + ((kLast - t0) & 1) * G::kImgBytes;
    const int kl = kLast * kBC;
    auto none = [](int) {};
    fwd_block<D, RB, true>(st, cur, 0, qf, l32, g, kl, Nk, c_log2, none);
    fwd_block<D, RB, true>(st, cur, 1, qf, l32, g, kl + 32, Nk, c_log2, none);
  }

  __syncthreads();  // the output stages overlap the tile stages
  const auto ro = make_rsrc(o, ext.o_bytes);
  float* stage = reinterpret_cast<float*>(smem + wave * kStageBytes);
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int row = row0 + 32 * rb, first = row - l32;
    const float l = halves_sum(st.l[rb]);
    const float inv_l = __builtin_amdgcn_ldexpf(1.0f / l, -ev);
    store_rows<D, kOutBf16>(stage, ro, (obh * (uint32_t)Nq + first) * D, Nq - first, l32, g,
                            [&](int cb, int i) { return st.acc[rb][cb][i] * inv_l; });
    if (row < Nq && g == 0 && lse != nullptr)
      buf_store4(make_rsrc(lse, ext.lse_bytes), (obh * (uint32_t)Nq + row) * 4,
                 (st.m[rb] + __log2f(l)) * kLn2);
  }
}

template <int D, bool kKV>
__global__ __launch_bounds__(kPackThreads) void pack_kv_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dk, const uint16_t* __restrict__ dv, char* __restrict__ ws,
    int Nk, int ntiles, uint32_t kv_bytes) {
  pack_kv_body<D, kKV>(k, v, dk, dv, ws, Nk, ntiles, kv_bytes);
}

template <int D, bool kKV>
hipError_t launch_pack_d(const void* k, const void* v, const void* tk, const void* tv, int B,
                         int H, int Nk, void* ws, hipStream_t stream) {
  const int ntiles = (Nk + kBC - 1) / kBC;
  const int bh = B * H;
  const uint32_t kv_bytes = (uint32_t)((size_t)bh * Nk * D * 2);
  const hipError_t e = launch_range_stats<D>(v, kKV ? tv : nullptr, ws, bh, Nk,
                                             slice_bytes<D, kKV>(ntiles),
                                             (uint32_t)ntiles * Geo<D, kKV>::kImgBytes, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((pack_kv_kernel<D, kKV>), dim3(ntiles, bh), dim3(kPackThreads), 0, stream,
                     static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v),
                     static_cast<const uint16_t*>(tk), static_cast<const uint16_t*>(tv),
                     static_cast<char*>(ws), Nk, ntiles, kv_bytes);
  return hipGetLastError();
}

// ATTN_JVP_TILE in the environment (read on every call) overrides the choice
// of kernel form, for tuning sweeps and for the tests that compare the forms:
// 128 or 256 query rows per workgroup of the JVP kernels (the short-key and
// the 256-row kernel), 256 or 512 of the forward kernel (one or two 32-row
// blocks per wave).  Every form computes each row with the same products in
// the same order, so the results do not change.
int tile_override() {
  const char* e = std::getenv("ATTN_JVP_TILE");
  return e != nullptr ? std::atoi(e) : 0;
}

template <int D, int kMode, bool kOutBf16>
hipError_t launch_main_d(const void* q, const void* tq, const void* ws, void* o, void* to,
                         float* lse, float* tlse, int B, int H, int Nq, int Nk, float scale,
                         int nsplit, hipStream_t stream) {
  const int ntiles = (Nk + kBC - 1) / kBC;
  const int bh = B * H;
  const int tps = (ntiles + nsplit - 1) / nsplit;
  const int ns = (ntiles + tps - 1) / tps;  // no empty range
  Extents ext;
  ext.q_bytes = (uint32_t)((size_t)bh * Nq * D * 2);
  ext.o_bytes = (uint32_t)((size_t)ns * bh * Nq * D * (kOutBf16 ? 2 : 4));
  ext.lse_bytes = (uint32_t)((size_t)ns * bh * Nq * 4);
  const int tile = tile_override();
  if (tile == kShortBR || (tile != kBR && tps <= kShortMaxTiles)) {
    const int nqt = (Nq + kShortBR - 1) / kShortBR;
    hipLaunchKernelGGL((attn_jvp_bf16_short_kernel<D, kMode, kOutBf16>), dim3(nqt * bh * ns),
                       dim3(kShortThreads), 0, stream, static_cast<const uint16_t*>(q),
                       static_cast<const uint16_t*>(tq), static_cast<const char*>(ws), o, to,
                       lse, tlse, Nq, Nk, ntiles, nqt, bh, tps, ext, scale, scale * kLog2e);
    return hipGetLastError();
  }
  const int nqt = (Nq + kBR - 1) / kBR;
  hipLaunchKernelGGL((attn_jvp_bf16_kernel<D, kMode, kOutBf16>), dim3(nqt * bh * ns),
                     dim3(kThreads), 0, stream, static_cast<const uint16_t*>(q),
                     static_cast<const uint16_t*>(tq), static_cast<const char*>(ws), o, to, lse,
                     tlse, Nq, Nk, ntiles, nqt, bh, tps, ext, scale, scale * kLog2e);
  return hipGetLastError();
}

template <int kMode>
hipError_t launch_main(const void* q, const void* tq, const void* ws, void* o, void* to,
                       float* lse, float* tlse, int B, int H, int Nq, int Nk, int d, float scale,
                       bool out_bf16, hipStream_t stream, int nsplit = 1) {
  if (d == 128)
    return out_bf16 ? launch_main_d<128, kMode, true>(q, tq, ws, o, to, lse, tlse, B, H, Nq, Nk,
                                                      scale, nsplit, stream)
                    : launch_main_d<128, kMode, false>(q, tq, ws, o, to, lse, tlse, B, H, Nq, Nk,
                                                       scale, nsplit, stream);
  return out_bf16 ? launch_main_d<64, kMode, true>(q, tq, ws, o, to, lse, tlse, B, H, Nq, Nk,
                                                   scale, nsplit, stream)
                  : launch_main_d<64, kMode, false>(q, tq, ws, o, to, lse, tlse, B, H, Nq, Nk,
                                                    scale, nsplit, stream);
}

hipError_t launch_pack(bool kv_tangents, const void* k, const void* v, const void* tk,
                       const void* tv, int B, int H, int Nk, int d, void* ws,
                       hipStream_t stream) {
  if (kv_tangents)
    return d == 128 ? launch_pack_d<128, true>(k, v, tk, tv, B, H, Nk, ws, stream)
                    : launch_pack_d<64, true>(k, v, tk, tv, B, H, Nk, ws, stream);
  return d == 128 ? launch_pack_d<128, false>(k, v, nullptr, nullptr, B, H, Nk, ws, stream)
                  : launch_pack_d<64, false>(k, v, nullptr, nullptr, B, H, Nk, ws, stream);
}

}  // namespace bf16_path
using namespace bf16_path;

size_t bf16_workspace_bytes(int B, int H, int Nk, int d) {
  // tile images and header of every slice, in the full (dK, dV) layout; the
  // modes without dK, dV lay out smaller slices in the same space
  const size_t ntiles = ((size_t)Nk + kBC - 1) / kBC;
  const size_t img = d == 128 ? Geo<128, true>::kImgBytes : Geo<64, true>::kImgBytes;
  return (size_t)B * H * (ntiles * img + kHdrBytes);
}

hipError_t launch_pack_kv(const void* k, const void* v, const void* tk, const void* tv, int B,
                          int H, int Nk, int d, void* ws, hipStream_t stream) {
  return launch_pack(true, k, v, tk, tv, B, H, Nk, d, ws, stream);
}

hipError_t launch_bf16_packed(const void* q, const void* tq, const void* ws, float* o,
                              float* to, float* lse, int B, int H, int Nq, int Nk, int d,
                              float scale, hipStream_t stream) {
  return launch_main<kFull>(q, tq, ws, o, to, lse, nullptr, B, H, Nq, Nk, d, scale, false,
                            stream);
}

hipError_t launch_bf16(const void* q, const void* k, const void* v, const void* tq,
                       const void* tk, const void* tv, float* o, float* to, float* lse, int B,
                       int H, int Nq, int Nk, int d, float scale, void* ws, hipStream_t stream) {
  const hipError_t e = launch_pack_kv(k, v, tk, tv, B, H, Nk, d, ws, stream);
  if (e != hipSuccess) return e;
  return launch_bf16_packed(q, tq, ws, o, to, lse, B, H, Nq, Nk, d, scale, stream);
}

hipError_t launch_bf16_ex(const void* q, const void* k, const void* v, const void* tq,
                          const void* tk, const void* tv, void* o, void* to, float* lse,
                          float* tlse, int B, int H, int Nq, int Nk, int d, float scale,
                          bool out_bf16, void* ws, hipStream_t stream) {
  // dK = dV = 0: the frozen-key mode leaves their products and tiles out
  const bool kv = tk != nullptr || tv != nullptr;
  hipError_t e = launch_pack(kv, k, v, tk, tv, B, H, Nk, d, ws, stream);
  if (e != hipSuccess) return e;
  return kv ? launch_main<kFull>(q, tq, ws, o, to, lse, tlse, B, H, Nq, Nk, d, scale, out_bf16,
                                 stream)
            : launch_main<kFrozen>(q, tq, ws, o, to, lse, tlse, B, H, Nq, Nk, d, scale, out_bf16,
                                   stream);
}

template <int D, int RB, bool kOutBf16>
hipError_t launch_fwd_rb(const void* q, const void* ws, void* o, float* lse, int B, int H, int Nq,
                         int Nk, float scale, int ns, hipStream_t stream) {
  const int ntiles = (Nk + kBC - 1) / kBC;
  const int nqt = (Nq + fwd_rows<RB>() - 1) / fwd_rows<RB>();
  const int bh = B * H;
  const int tps = (ntiles + ns - 1) / ns;
  ns = (ntiles + tps - 1) / tps;
  Extents ext;
  ext.q_bytes = (uint32_t)((size_t)bh * Nq * D * 2);
  ext.o_bytes = (uint32_t)((size_t)ns * bh * Nq * D * (kOutBf16 ? 2 : 4));
  ext.lse_bytes = (uint32_t)((size_t)ns * bh * Nq * 4);
  hipLaunchKernelGGL((attn_fwd_bf16_kernel<D, RB, kOutBf16>), dim3(nqt * bh * ns), dim3(kThreads),
                     0, stream, static_cast<const uint16_t*>(q), static_cast<const char*>(ws), o,
                     lse, Nq, Nk, ntiles, nqt, bh, tps, ext, scale * kLog2e);
  return hipGetLastError();
}

// 512-row workgroups, unless even the 256-row ones fit the chip's 256 CUs
// one per CU (then twice as many CUs work; measured at Nk = 32760, H = 12:
// Nq = 4096 1446 -> 994 us, Nq = 8192 with 512 rows 1534 us vs 1730) or a
// work item has at most kShortMaxTiles key tiles.  ns key-tile ranges (1: the
// plain pass).
template <int D, bool kOutBf16>
hipError_t launch_fwd_d(const void* q, const void* ws, void* o, float* lse, int B, int H, int Nq,
                        int Nk, float scale, int ns, hipStream_t stream) {
  const long tiles256 = (long)(Nq + fwd_rows<1>() - 1) / fwd_rows<1>() * B * H * ns;
  const int ntiles = (Nk + kBC - 1) / kBC, tps = (ntiles + ns - 1) / ns;
  // few key tiles per work item: two workgroups per CU overlap one's query
  // and output traffic with the other's products, as in the short-key JVP
  // kernel (H = 12, Nq = 32760: 512 keys 148 vs 164 us, 1024 keys 231 vs 244;
  // 2048 keys 402 vs 395)
  const int tile = tile_override();
  if (tile == fwd_rows<2>() || (tile != fwd_rows<1>() && tiles256 > 256 && tps > kShortMaxTiles))
    return launch_fwd_rb<D, 2, kOutBf16>(q, ws, o, lse, B, H, Nq, Nk, scale, ns, stream);
  return launch_fwd_rb<D, 1, kOutBf16>(q, ws, o, lse, B, H, Nq, Nk, scale, ns, stream);
}

hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int Nq, int Nk, int d, float scale, bool out_bf16, void* ws,
                      hipStream_t stream) {
  hipError_t e = launch_pack(false, k, v, nullptr, nullptr, B, H, Nk, d, ws, stream);
  if (e != hipSuccess) return e;
  if (d == 128)
    return out_bf16 ? launch_fwd_d<128, true>(q, ws, o, lse, B, H, Nq, Nk, scale, 1, stream)
                    : launch_fwd_d<128, false>(q, ws, o, lse, B, H, Nq, Nk, scale, 1, stream);
  return out_bf16 ? launch_fwd_d<64, true>(q, ws, o, lse, B, H, Nq, Nk, scale, 1, stream)
                  : launch_fwd_d<64, false>(q, ws, o, lse, B, H, Nq, Nk, scale, 1, stream);
}


// ---- split-KV: key-tile ranges on separate workgroups, then the merge ----
// Ranges of whole 64-key tiles: the number actually used is
// ceil(ntiles / ceil(ntiles / nsplit)) (no empty range).
namespace {
constexpr int kSplitMinTiles = 4;        // at least 256 keys per range
constexpr int kSplitMaxParts = 1024;     // the merge kernel's limit
constexpr int kSplitCUs = 256;           // one workgroup per compute unit at a time
// HBM bytes moved in the time of one 64-key tile step of a workgroup
// (~5 TB/s x ~4.7 us): the unit in which a range's partial state is priced
constexpr double kSplitTileBytes = 24e6;
inline size_t align256(size_t n) { return (n + 255) / 256 * 256; }
inline int ranges_used(int ntiles, int n) {
  const int tps = (ntiles + n - 1) / n;
  return (ntiles + tps - 1) / tps;
}
}  // namespace

// The automatic count (nsplit = 0) minimises a model of the time in units of
// one tile step: rounds of workgroups (items of `rows` query rows x ranges
// over 256 compute units) times tiles per range, plus, per extra range, the
// partial O, dO, lse, mu written and read back by the merge.  A count is taken
// only if it is at least 5% below the best smaller one.  rows: 256 for the
// JVP kernel, 512 for the forward one.
int splitkv_count(int B, int H, int Nq, int Nk, int d, int nsplit, int rows) {
  const int ntiles = (Nk + kBC - 1) / kBC;
  if (nsplit == 0) {
    const double items = (double)((Nq + rows - 1) / rows) * B * H;
    const double state = (double)B * H * Nq * (2.0 * d + 2.0) * 4.0 * 2.0 / kSplitTileBytes;
    double best = std::ceil(items / kSplitCUs) * ntiles;
    nsplit = 1;
    const int cap = ntiles / kSplitMinTiles < kSplitMaxParts ? ntiles / kSplitMinTiles
                                                              : kSplitMaxParts;
    for (int n = 2; n <= cap; ++n) {
      const int used = ranges_used(ntiles, n);
      const int tps = (ntiles + n - 1) / n;
      const double cost = std::ceil(items * used / kSplitCUs) * tps + state * used;
      if (cost < 0.95 * best) {
        best = cost;
        nsplit = n;
      }
    }
  }
  if (nsplit > ntiles) nsplit = ntiles;
  if (nsplit > kSplitMaxParts) nsplit = kSplitMaxParts;
  if (nsplit < 1) nsplit = 1;
  // partial O and dO arrays each stay under 2^31 bytes
  const size_t per = (size_t)B * H * Nq * d * 4;
  while (nsplit > 1 && (size_t)ranges_used(ntiles, nsplit) * per >= ((size_t)1 << 31)) --nsplit;
  return ranges_used(ntiles, nsplit);
}

// Workspace for either kernel's count (the forward one may choose more ranges).
size_t splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int nsplit) {
  const int a = splitkv_count(B, H, Nq, Nk, d, nsplit, kBR);
  const int b = splitkv_count(B, H, Nq, Nk, d, nsplit, fwd_rows<2>());
  const int ns = a > b ? a : b;
  size_t n = align256(bf16_workspace_bytes(B, H, Nk, d));
  if (ns > 1) {
    const size_t rows = (size_t)ns * B * H * Nq;
    n += 2 * align256(rows * d * 4) + 2 * align256(rows * 4);
  }
  return n;
}

hipError_t launch_bf16_splitkv(const void* q, const void* k, const void* v, const void* tq,
                               const void* tk, const void* tv, float* o, float* to, float* lse,
                               float* tlse, int B, int H, int Nq, int Nk, int d, float scale,
                               int nsplit, void* ws, hipStream_t stream) {
  const int ns = splitkv_count(B, H, Nq, Nk, d, nsplit, kBR);
  const bool kv = tk != nullptr || tv != nullptr;
  hipError_t e = launch_pack(kv, k, v, tk, tv, B, H, Nk, d, ws, stream);
  if (e != hipSuccess) return e;
  auto fused = [&](float* mo, float* mto, float* ml, float* mtl, int n) {
    return kv ? launch_main<kFull>(q, tq, ws, mo, mto, ml, mtl, B, H, Nq, Nk, d, scale, false,
                                   stream, n)
              : launch_main<kFrozen>(q, tq, ws, mo, mto, ml, mtl, B, H, Nq, Nk, d, scale, false,
                                     stream, n);
  };
  if (ns == 1) return fused(o, to, lse, tlse, 1);
  char* p = static_cast<char*>(ws) + align256(bf16_workspace_bytes(B, H, Nk, d));
  const size_t rows = (size_t)ns * B * H * Nq;
  float* o_p = reinterpret_cast<float*>(p);
  float* to_p = reinterpret_cast<float*>(p + align256(rows * d * 4));
  float* lse_p = reinterpret_cast<float*>(p + 2 * align256(rows * d * 4));
  float* mu_p = reinterpret_cast<float*>(p + 2 * align256(rows * d * 4) + align256(rows * 4));
  e = fused(o_p, to_p, lse_p, mu_p, ns);
  if (e != hipSuccess) return e;
  return launch_merge(lse_p, o_p, to_p, mu_p, ns, B * H * Nq, d, lse, o, to, tlse, stream);
}

// Forward alone with key-tile ranges: partial O and lse in the workspace
// (after the tile images, laid out as for the JVP's split), then the merge.
hipError_t launch_fwd_splitkv(const void* q, const void* k, const void* v, float* o, float* lse,
                              int B, int H, int Nq, int Nk, int d, float scale, int nsplit,
                              void* ws, hipStream_t stream) {
  const int ns = splitkv_count(B, H, Nq, Nk, d, nsplit, fwd_rows<2>());
  hipError_t e = launch_pack(false, k, v, nullptr, nullptr, B, H, Nk, d, ws, stream);
  if (e != hipSuccess) return e;
  auto fwd = [&](float* mo, float* ml, int n) {
    return d == 128 ? launch_fwd_d<128, false>(q, ws, mo, ml, B, H, Nq, Nk, scale, n, stream)
                    : launch_fwd_d<64, false>(q, ws, mo, ml, B, H, Nq, Nk, scale, n, stream);
  };
  if (ns == 1) return fwd(o, lse, 1);
  char* p = static_cast<char*>(ws) + align256(bf16_workspace_bytes(B, H, Nk, d));
  const size_t rows = (size_t)ns * B * H * Nq;
  float* o_p = reinterpret_cast<float*>(p);
  float* lse_p = reinterpret_cast<float*>(p + 2 * align256(rows * d * 4));
  e = fwd(o_p, lse_p, ns);
  if (e != hipSuccess) return e;
  return launch_merge(lse_p, o_p, nullptr, nullptr, ns, B * H * Nq, d, lse, o, nullptr, nullptr,
                      stream);
}

}  // namespace ajvp
