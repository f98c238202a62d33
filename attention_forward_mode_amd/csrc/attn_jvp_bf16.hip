// attn_jvp_bf16.hip -- fused attention forward + JVP for gfx950, bf16 inputs.
//
// The operation (rCM record LIT-783 in the Anthology of the SOTA, "Key
// takeaways", "JVP at production scale", paper §3.2 / App. C: FlashAttention-2
// and its Jacobian-vector product in one tiled pass):
//   O = softmax(s Q K^T) V,  dO = (P * (dS - mu)) V + P dV,
//   dS = s (dQ K^T + Q dK^T),  mu = rowsum(P * dS),  lse = ln rowsum exp(s Q K^T).
//
// Two kernels per call:
//  1. pack_v: V and dV -> fp16, transposed to [d][64 keys] tiles in matrix-core
//     operand order, zero-padded past Nk.  HBM
//     bound, ~1% of the fused kernel's time at N = 32760.  fp16 instead of bf16
//     for the second contraction keeps P and P*dS at 11 significant bits.
//  2. attn_jvp_bf16: one workgroup = 4 waves x 32 query rows of one (b, h).
//     Per 64-key tile: stage K, dK (bf16) and the packed V^T, dV^T (fp16) in
//     LDS through registers (double buffered, loads one tile ahead), then
//     per wave and 32-key block
//        S^T  = K Q^T            (bf16 MFMA 32x32x16, Q held in registers)
//        dS^T = dK Q^T + K dQ^T  (same K fragments reused)
//     online softmax in the accumulator layout (each lane owns one query row,
//     so row state is per lane), and
//        A^T += V^T P^T,  G^T += V^T (s P dS)^T + dV^T P^T  (fp16 MFMA)
//     with P, s*P*dS rounded to fp16.  The epilogue forms O = A / l,
//     mu = u / l (u = rowsum s P dS), dO = G / l - mu O and lse.
//  The running max is only raised when a tile's max exceeds it by more than
//  kTau (log2 units): results are exact either way, p stays <= 2^kTau, and the
//  accumulator rescale is skipped on most tiles.
#include "cdna4.hpp"
#include "launch.hpp"

namespace ajvp {
namespace bf16_path {

constexpr int kBC = 64;             // keys per tile
constexpr int kThreads = 256;       // 4 waves
constexpr int kRowsPerWave = 32;
constexpr int kBR = 128;            // query rows per workgroup
constexpr float kTau = 4.0f;        // lazy-rescale headroom, log2 units

template <int D>
struct Geo {
  static constexpr int kTileBytes = kBC * D * 2;          // one tile of K (bf16) or V^T (fp16)
  static constexpr int kPackTileBytes = 2 * kTileBytes;   // V^T | dV^T in the workspace
  // LDS rows are padded by 16 bytes: the 8 rows that one phase of a 16-byte
  // matrix-operand read touches then start 16 bytes apart modulo the bank
  // width, so the reads are conflict-free, and every address is a per-lane
  // base plus a constant.
  static constexpr int kKRow = D * 2 + 16;                // K, dK: 64 key rows
  static constexpr int kVRow = kBC * 2 + 16;              // V^T, dV^T: D rows of 64 keys
  static constexpr int kKTile = kBC * kKRow;
  static constexpr int kVTile = D * kVRow;
  static constexpr int kStageBytes = 2 * kKTile + 2 * kVTile;  // K | dK | V^T | dV^T
  static constexpr int kKS = D / 16;                      // contraction steps over d
  static constexpr int kCB = D / 32;                      // 32-column output blocks
};

// Key held at position `pos` (0..63) of a packed V^T row.  Positions
// 16G + 8g + e hold the keys that the S^T accumulator of lane half g puts in
// slots 8t + e of block G/2, t = G%2: keys 16G + 4g + e (e < 4) and
// 16G + 8 + 4g + (e - 4) (e >= 4).
__device__ inline int packed_key(int pos) {
  const int G = pos >> 4, g = (pos >> 3) & 1, e = pos & 7;
  return 16 * G + (e < 4 ? 4 * g + e : 8 + 4 * g + (e - 4));
}

template <int D>
__device__ __attribute__((always_inline)) inline void pack_v_body(const uint16_t* __restrict__ v,
                                                                  const uint16_t* __restrict__ dv,
                                                                  char* __restrict__ ws, int Nk,
                                                                  int ntiles, uint32_t v_bytes,
                                                                  uint32_t ws_bytes) {
  using G = Geo<D>;
  __shared__ _Float16 sv[2][kBC][D + 2];
  const int tile = blockIdx.x;                 // 64-key tile
  const uint32_t bh = blockIdx.y;              // (b, h) slice
  // Every global access goes through a buffer descriptor spanning the whole
  // tensor: an offset outside it is dropped (stores) or reads zero (loads).
  const auto rv = make_rsrc(v, v_bytes);
  const auto rdv = make_rsrc(dv, v_bytes);
  const auto rws = make_rsrc(ws, ws_bytes);
  const int key0 = tile * kBC;
  constexpr int kIn = kBC * D / 8;  // 16-byte input chunks per tensor
  for (int c = threadIdx.x; c < 2 * kIn; c += kThreads) {
    const int t = c / kIn, rem = c % kIn, r = rem / (D / 8), col = (rem % (D / 8)) * 8;
    const int key = key0 + r;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (key < Nk) {
      const uint32_t off = ((bh * (uint32_t)Nk + key) * D + col) * 2;
      x = buf_load16(t == 0 ? rv : rdv, off);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t bits = (x[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      sv[t][r][col + e] = (_Float16)__builtin_bit_cast(float, bits << 16);
    }
  }
  __syncthreads();
  const uint32_t out = (bh * (uint32_t)ntiles + tile) * G::kPackTileBytes;
  for (int c = threadIdx.x; c < 2 * D * 8; c += kThreads) {
    const int t = c / (D * 8), rem = c % (D * 8), col = rem / 8, p = rem % 8;
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = sv[t][packed_key(8 * p + e)][col];
    buf_store16(rws, out + t * G::kTileBytes + col * 128 + p * 16, __builtin_bit_cast(u32x4, h));
  }
}

template <int D>
struct RowState {
  f32x16 accA[Geo<D>::kCB];  // A^T = sum p v      (rows: output column, cols: query)
  f32x16 accG[Geo<D>::kCB];  // G^T = sum p (s dS v + dv)
  float m;                   // running max of s*log2e*S (log2 units), per query row
  float alpha;               // 2^(m_prev - m) of the latest max update
  float l;                   // this lane's half of sum p         (of the fp16-rounded p)
  float u;                   // this lane's half of sum s p dS    (of the fp16-rounded values)
};

// S^T and dS^T of one 32-key block (rows: key, columns: this wave's queries).
struct SBlock {
  f32x16 s, ds;
};

// Operands of the second contraction for one block: P and s*P*dS in fp16.
struct PBlock {
  u32x4 p[2], pd[2];
};

// Slot r of lane half g holds key 8(r/4) + 4g + r%4 of its 32-key block.
__device__ __attribute__((always_inline)) inline int slot_key(int r, int g) {
  return 8 * (r >> 2) + 4 * g + (r & 3);
}

// ---- the per-block pipeline ----
// Block j of the key sequence passes through two scheduling regions:
//   R1(j): S/dS of block j on the matrix cores, while the vector ALU turns
//          block j-1 into P, s*P*dS (fp16) and its row sums;
//   R2(j): P V of block j-1 on the matrix cores, while the vector ALU finds
//          the max of block j's S and the new running max / rescale factor;
//   then the accumulators are rescaled (rare, see kTau).
// Both regions are written as slots of one matrix-core instruction plus a
// share of vector work, separated by scheduling barriers, so the two units
// run side by side within one wave.  Operand fragments are read from LDS two
// slots-of-three ahead of their use.
// Online-softmax order: P V of block j-1 (normalised to m_{j-1}) is added
// before the rescale by alpha_j = 2^(m_{j-1} - m_j), and P of block j is
// formed with m_j, so the accumulators always hold sums normalised to the
// current m.

// R1.  kQK: form S/dS of block `kb` of `stage` into `snew`.  kEW: finish block
// `sold` (max already applied to st.m): P, s*P*dS -> `pb`, and l, u updated
// with the rescale factor of that block.  kMask: `sold` lies in the last tile
// (keys >= Nk get p = 0 and contribute nothing to u).  Each pair of results is
// rounded to fp16 as soon as it exists, and l, u sum exactly those rounded
// values (one dot instruction per pair): the weights that the normalisation
// uses are the ones the matrix cores multiply, so O is an exact convex
// combination of V's rows and sum_j (p_j dS_j - mu p_j) cancels as it must.
template <int D, bool kQK, bool kEW, bool kMask>
__device__ __attribute__((always_inline)) inline void region1(
    RowState<D>& st, const char* stage, int kb, const u32x4* qf, const u32x4* dqf, int l32,
    int g, SBlock& snew, const SBlock& sold, int key0_old, int Nk, float c_log2, float scale,
    PBlock& pb) {
  using G = Geo<D>;
  constexpr int kSlots = 3 * G::kKS;
  constexpr int kPairSlots = kSlots - 1;  // element pairs spread over these slots
  const char* sK = stage;
  const char* sdK = stage + G::kKTile;
  const int rowoff = (32 * kb + l32) * G::kKRow + 16 * g;
  u32x4 ka[3], kda[3];
  if constexpr (kQK) {
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      ka[ks] = lds_load16(sK + rowoff + 32 * ks);
      kda[ks] = lds_load16(sdK + rowoff + 32 * ks);
    }
  }
  float lsum = 0.f, usum = 0.f;
  const float m = st.m;
#pragma unroll
  for (int i = 0; i < kSlots; ++i) {
    if constexpr (kQK) {
      const int ks = i / 3, w = i % 3;
      if (w == 0 && ks + 2 < G::kKS) {
        ka[(ks + 2) % 3] = lds_load16(sK + rowoff + 32 * (ks + 2));
        kda[(ks + 2) % 3] = lds_load16(sdK + rowoff + 32 * (ks + 2));
      }
      if (w == 0) snew.s = mma_bf16(ka[ks % 3], qf[ks], ks == 0 ? f32x16{} : snew.s);
      if (w == 1) snew.ds = mma_bf16(ka[ks % 3], dqf[ks], ks == 0 ? f32x16{} : snew.ds);
      if (w == 2) snew.ds = mma_bf16(kda[ks % 3], qf[ks], snew.ds);
    }
    if constexpr (kEW) {
#pragma unroll
      for (int q = i * 8 / kPairSlots; q < (i + 1) * 8 / kPairSlots && q < 8; ++q) {
        float pp[2], pdd[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const int r = 2 * q + e;
          pp[e] = __builtin_amdgcn_exp2f(__builtin_fmaf(sold.s[r], c_log2, -m));
          pdd[e] = pp[e] * sold.ds[r] * scale;
          if (kMask && key0_old + slot_key(r, g) >= Nk) {
            pp[e] = 0.f;
            pdd[e] = 0.f;
          }
        }
        const uint32_t hp = pack_f16x2(pp[0], pp[1]);
        const uint32_t hd = pack_f16x2(pdd[0], pdd[1]);
        pb.p[q >> 2][q & 3] = hp;
        pb.pd[q >> 2][q & 3] = hd;
        lsum = add_f16x2(hp, lsum);
        usum = add_f16x2(hd, usum);
      }
      if (i == kSlots - 1) {
        st.l = st.l * st.alpha + lsum;
        st.u = st.u * st.alpha + usum;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// R2.  kPV: A^T += V^T P^T, G^T += V^T (s P dS)^T + dV^T P^T for block `kb` of
// `stage` with operands `pb`.  kMax: running-max update from block `snew`
// (kMask: its keys >= Nk are left out), then the rescale.
template <int D, bool kPV, bool kMax, bool kMask>
__device__ __attribute__((always_inline)) inline void region2(
    RowState<D>& st, const char* stage, int kb, const PBlock& pb, int l32, int g,
    SBlock& snew, int key0_new, int Nk, float c_log2) {
  using G = Geo<D>;
  constexpr int kSteps = 2 * G::kCB;  // (cb, t) pairs, three products each
  constexpr int kSlots = 3 * kSteps;
  const char* sV = stage + 2 * G::kKTile;
  const char* sdV = sV + G::kVTile;
  auto voff = [&](int step) {  // step = 2 cb + t
    return ((32 * (step >> 1) + l32) * G::kVRow + 16 * g) + 16 * (4 * kb + 2 * (step & 1));
  };
  u32x4 va[3], vda[3];
  if constexpr (kPV) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      va[k] = lds_load16(sV + voff(k));
      vda[k] = lds_load16(sdV + voff(k));
    }
  }
  if constexpr (kMax && kMask) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (key0_new + slot_key(r, g) >= Nk) snew.s[r] = -INFINITY;
  }
  float mx = -INFINITY;
#pragma unroll
  for (int i = 0; i < kSlots; ++i) {
    if constexpr (kPV) {
      const int step = i / 3, w = i % 3, cb = step >> 1, t = step & 1;
      if (w == 0 && step + 2 < kSteps) {
        va[(step + 2) % 3] = lds_load16(sV + voff(step + 2));
        vda[(step + 2) % 3] = lds_load16(sdV + voff(step + 2));
      }
      if (w == 0) st.accA[cb] = mma_f16(va[step % 3], pb.p[t], st.accA[cb]);
      if (w == 1) st.accG[cb] = mma_f16(va[step % 3], pb.pd[t], st.accG[cb]);
      if (w == 2) st.accG[cb] = mma_f16(vda[step % 3], pb.p[t], st.accG[cb]);
    }
    if constexpr (kMax) {
      // two elements per slot over the first eight slots, then the combine.
      // NaN-propagating maximum: one v_maximum3 per slot, no canonicalisation.
      if (i < 8)
        mx = __builtin_elementwise_maximum(__builtin_elementwise_maximum(mx, snew.s[2 * i]),
                                           snew.s[2 * i + 1]);
      if (i == 8) {
        mx = halves_max(mx);
        const float mt = mx * c_log2;
        const float m_new = (mt > st.m + kTau) ? mt : st.m;
        st.alpha = __builtin_amdgcn_exp2f(st.m - m_new);
        st.m = m_new;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (kMax) {
    if (wave_any(st.alpha != 1.0f)) {
      // One 16-register block at a time, so this rare path needs few
      // temporaries and does not raise the main path's register pressure.
#pragma unroll
      for (int cb = 0; cb < G::kCB; ++cb) {
        st.accA[cb] *= st.alpha;
        __builtin_amdgcn_sched_barrier(0);
        st.accG[cb] *= st.alpha;
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
}

// Sizes of the whole tensors (bytes) the kernel may touch; each global access
// is checked against them by the buffer descriptor.
struct Extents {
  uint32_t q_bytes, k_bytes, ws_bytes, o_bytes, lse_bytes;
};

template <int D>
__device__ __attribute__((always_inline)) inline void attn_jvp_bf16_body(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ tq, const uint16_t* __restrict__ tk,
    const char* __restrict__ vpack, float* __restrict__ o, float* __restrict__ to,
    float* __restrict__ lse, int Nq, int Nk, int ntiles, Extents ext, float scale,
    float c_log2) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * G::kStageBytes];

  // Work item: blockIdx.x = 128-row query tile, blockIdx.y = (b, h) slice.
  const int qt = blockIdx.x;
  const uint32_t bh = blockIdx.y;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, g = lane >> 5;
  const int row = qt * kBR + wave * kRowsPerWave + l32;
  const bool row_ok = row < Nq;

  // Buffer descriptors over whole tensors (see Extents).
  const auto rq = make_rsrc(q, ext.q_bytes);
  const auto rtq = make_rsrc(tq, ext.q_bytes);
  const auto rk = make_rsrc(k, ext.k_bytes);
  const auto rtk = make_rsrc(tk, ext.k_bytes);
  const auto rv = make_rsrc(vpack, ext.ws_bytes);
  const auto ro = make_rsrc(o, ext.o_bytes);
  const auto rto = make_rsrc(to, ext.o_bytes);

  // Q and dQ fragments: the B operand of S^T = K Q^T (lane: row l32, d-slice g).
  // Rows past Nq get an offset past the tensor, which the descriptor reads as 0.
  u32x4 qf[G::kKS], dqf[G::kKS];
  const uint32_t qrow = row_ok ? (bh * (uint32_t)Nq + row) * D * 2 : 0x80000000u;
#pragma unroll
  for (int ks = 0; ks < G::kKS; ++ks) {
    const uint32_t off = qrow + (16 * ks + 8 * g) * 2;
    qf[ks] = buf_load16(rq, off);
    dqf[ks] = buf_load16(rtq, off);
  }
  // The Q/dQ fragments are only ever matrix-core operands, which may come
  // from accumulation registers: keep them there and leave the vector
  // registers to the softmax.  (Empty asm: a register-class constraint only.)
#pragma unroll
  for (int ks = 0; ks < G::kKS; ++ks) asm volatile("" : "+a"(qf[ks]), "+a"(dqf[ks]));

  // Staging through registers, one tensor pair at a time: each thread loads
  // kChunks 16-byte chunks of K|dK (or of the packed V^T|dV^T tile) into stg
  // and later writes them to LDS.  Chunk n of thread tid is chunk tid + 256 n
  // of the tile pair: its row advances by a constant per n, so the per-lane
  // part of every offset is fixed and the rest is a constant or wave-uniform.
  // Key rows past Nk in the last tile hold whatever the descriptor returns;
  // they are masked in the compute.
  constexpr int kChunks = G::kTileBytes * 2 / 16 / kThreads;  // per pair of tensors
  constexpr int kChunksPerTensor = kChunks / 2;
  constexpr int kKRowsPerN = kThreads / (D / 8);   // K rows advanced per chunk step
  constexpr int kVRowsPerN = kThreads / 8;         // V^T rows advanced per chunk step
  const uint32_t kslice = bh * (uint32_t)Nk * D * 2;
  const uint32_t vslice = bh * (uint32_t)ntiles * G::kPackTileBytes;
  const uint32_t k_lane = (uint32_t)tid * 16;  // global: row tid/(D/8), chunk tid%(D/8)
  const int k_lds = (tid / (D / 8)) * G::kKRow + (tid % (D / 8)) * 16;
  const int v_lds = (tid / 8) * G::kVRow + (tid % 8) * 16;
  u32x4 stg[kChunks];
  auto load_k = [&](int kt) {
    const uint32_t kbase = kslice + (uint32_t)kt * kBC * D * 2;
#pragma unroll
    for (int n = 0; n < kChunks; ++n)
      stg[n] = buf_load16(n < kChunksPerTensor ? rk : rtk, k_lane,
                          kbase + (uint32_t)(n % kChunksPerTensor) * kThreads * 16);
  };
  auto load_v = [&](int kt) {
    const uint32_t vbase = vslice + (uint32_t)kt * G::kPackTileBytes;
#pragma unroll
    for (int n = 0; n < kChunks; ++n)
      stg[n] = buf_load16(rv, k_lane, vbase + (uint32_t)n * kThreads * 16);
  };
  auto store_k = [&](char* sb) {
#pragma unroll
    for (int n = 0; n < kChunks; ++n)
      lds_store16(sb + k_lds + (n / kChunksPerTensor) * G::kKTile +
                      (n % kChunksPerTensor) * kKRowsPerN * G::kKRow,
                  stg[n]);
  };
  // The V^T and dV^T tiles are D rows each, so row r >= D of the pair is row
  // r - D of dV^T, which starts kVTile bytes after V^T: one formula covers both.
  auto store_v = [&](char* sb) {
#pragma unroll
    for (int n = 0; n < kChunks; ++n)
      lds_store16(sb + 2 * G::kKTile + v_lds + n * kVRowsPerN * G::kVRow, stg[n]);
  };

  RowState<D> st;
#pragma unroll
  for (int cb = 0; cb < G::kCB; ++cb) {
    st.accA[cb] = f32x16{};
    st.accG[cb] = f32x16{};
  }
  st.m = -INFINITY;
  st.alpha = 1.f;
  st.l = 0.f;
  st.u = 0.f;

  // Blocks j = 0 .. 2*ntiles-1 (block j is half j % 2 of tile j / 2) run
  // through region1 / region2 (R1(j), R2(j)) as described above.  K|dK(t) and
  // V|dV(t) live in LDS buffer t % 2; K(t) is read in R1 of blocks 2t, 2t+1
  // and V(t) in R2 of blocks 2t+1, 2t+2.  Per tile kt, with a barrier after
  // each block:
  //   K|dK(kt+1) -> LDS, V|dV(kt+1) loads issued   (K|dK(kt-1) last read in block 2kt-1)
  //   block 2kt,   barrier
  //   V|dV(kt+1) -> LDS, K|dK(kt+2) loads issued   (V|dV(kt-1) last read in block 2kt)
  //   block 2kt+1, barrier
  // so K|dK(kt+1) is visible from block 2kt+1 on and V|dV(kt+1) from 2kt+2 on.
  SBlock sa, sb;  // S/dS of the even / odd block
  PBlock pb;      // P, s*P*dS of the block whose P V is next
  const int kLast = ntiles - 1;
  const int key_last = kLast * kBC;
  auto stage = [&](int t) { return smem + (t & 1) * G::kStageBytes; };
  load_k(0);
  store_k(smem);
  load_v(0);
  store_v(smem);
  load_k(1);  // past the last tile the descriptors read zeros or unused data
  __syncthreads();
  if (ntiles == 1) {
    region1<D, true, false, false>(st, smem, 0, qf, dqf, l32, g, sa, sb, 0, Nk, c_log2, scale, pb);
    region2<D, false, true, true>(st, smem, 0, pb, l32, g, sa, 0, Nk, c_log2);
    region1<D, true, true, true>(st, smem, 1, qf, dqf, l32, g, sb, sa, 0, Nk, c_log2, scale, pb);
    region2<D, true, true, true>(st, smem, 0, pb, l32, g, sb, 32, Nk, c_log2);
    region1<D, false, true, true>(st, smem, 0, qf, dqf, l32, g, sa, sb, 32, Nk, c_log2, scale, pb);
    region2<D, true, false, false>(st, smem, 1, pb, l32, g, sb, 0, Nk, c_log2);
  } else {
    // tile 0
    store_k(stage(1));
    load_v(1);
    region1<D, true, false, false>(st, smem, 0, qf, dqf, l32, g, sa, sb, 0, Nk, c_log2, scale, pb);
    region2<D, false, true, false>(st, smem, 0, pb, l32, g, sa, 0, Nk, c_log2);
    __syncthreads();
    store_v(stage(1));
    load_k(2);
    region1<D, true, true, false>(st, smem, 1, qf, dqf, l32, g, sb, sa, 0, Nk, c_log2, scale, pb);
    region2<D, true, true, false>(st, smem, 0, pb, l32, g, sb, 0, Nk, c_log2);
    __syncthreads();
    // tiles 1 .. ntiles-2
    for (int kt = 1; kt < kLast; ++kt) {
      store_k(stage(kt + 1));
      load_v(kt + 1);
      region1<D, true, true, false>(st, stage(kt), 0, qf, dqf, l32, g, sa, sb, 0, Nk, c_log2,
                                    scale, pb);
      region2<D, true, true, false>(st, stage(kt - 1), 1, pb, l32, g, sa, 0, Nk, c_log2);
      __syncthreads();
      store_v(stage(kt + 1));
      load_k(kt + 2);
      region1<D, true, true, false>(st, stage(kt), 1, qf, dqf, l32, g, sb, sa, 0, Nk, c_log2,
                                    scale, pb);
      region2<D, true, true, false>(st, stage(kt), 0, pb, l32, g, sb, 0, Nk, c_log2);
      __syncthreads();
    }
    // last tile: keys past Nk are masked (the tile is complete in LDS already)
    region1<D, true, true, false>(st, stage(kLast), 0, qf, dqf, l32, g, sa, sb, 0, Nk, c_log2,
                                  scale, pb);
    region2<D, true, true, true>(st, stage(kLast - 1), 1, pb, l32, g, sa, key_last, Nk, c_log2);
    region1<D, true, true, true>(st, stage(kLast), 1, qf, dqf, l32, g, sb, sa, key_last, Nk,
                                 c_log2, scale, pb);
    region2<D, true, true, true>(st, stage(kLast), 0, pb, l32, g, sb, key_last + 32, Nk, c_log2);
    region1<D, false, true, true>(st, stage(kLast), 0, qf, dqf, l32, g, sa, sb, key_last + 32, Nk,
                                  c_log2, scale, pb);
    region2<D, true, false, false>(st, stage(kLast), 1, pb, l32, g, sb, 0, Nk, c_log2);
  }

  // ---- epilogue: O = A / l, mu = u / l, dO = G / l - mu O, lse ----
  const float l = halves_sum(st.l);
  const float u = halves_sum(st.u);
  const float inv_l = 1.0f / l;
  const float mu = u * inv_l;
  if (row_ok) {
    const uint32_t orow = (bh * (uint32_t)Nq + row) * D * 4;
#pragma unroll
    for (int cb = 0; cb < G::kCB; ++cb)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int c0 = 32 * cb + 8 * qq + 4 * g;
        f32x4 ov, tv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float a = st.accA[cb][4 * qq + e] * inv_l;
          ov[e] = a;
          tv[e] = st.accG[cb][4 * qq + e] * inv_l - mu * a;
        }
        buf_store16(ro, orow + c0 * 4, __builtin_bit_cast(u32x4, ov));
        buf_store16(rto, orow + c0 * 4, __builtin_bit_cast(u32x4, tv));
      }
    if (lse != nullptr && g == 0) {
      const auto rl = make_rsrc(lse, ext.lse_bytes);
      buf_store4(rl, (bh * (uint32_t)Nq + row) * 4, (st.m + __log2f(l)) * kLn2);
    }
  }
}

#define AJVP_BF16_KERNEL(D)                                                                 \
  __global__ __launch_bounds__(kThreads, 1) void attn_jvp_bf16_d##D(                         \
      const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,                        \
      const uint16_t* __restrict__ tq, const uint16_t* __restrict__ tk,                      \
      const char* __restrict__ vpack, float* __restrict__ o, float* __restrict__ to,         \
      float* __restrict__ lse, int Nq, int Nk, int ntiles, Extents ext, float scale,         \
      float c_log2) {                                                                         \
    attn_jvp_bf16_body<D>(q, k, tq, tk, vpack, o, to, lse, Nq, Nk, ntiles, ext, scale, c_log2); \
  }                                                                                           \
  __global__ __launch_bounds__(kThreads) void pack_v_d##D(                                   \
      const uint16_t* __restrict__ v, const uint16_t* __restrict__ dv, char* __restrict__ ws, \
      int Nk, int ntiles, uint32_t v_bytes, uint32_t ws_bytes) {                              \
    pack_v_body<D>(v, dv, ws, Nk, ntiles, v_bytes, ws_bytes);                                 \
  }
AJVP_BF16_KERNEL(64)
AJVP_BF16_KERNEL(128)
#undef AJVP_BF16_KERNEL

template <int D>
struct Kernels;
template <>
struct Kernels<64> {
  static constexpr auto main = attn_jvp_bf16_d64;
  static constexpr auto pack = pack_v_d64;
};
template <>
struct Kernels<128> {
  static constexpr auto main = attn_jvp_bf16_d128;
  static constexpr auto pack = pack_v_d128;
};

template <int D>
hipError_t launch_pack_d(const void* v, const void* tv, int B, int H, int Nk, void* ws,
                         hipStream_t stream) {
  const int ntiles = (Nk + kBC - 1) / kBC;
  const int bh = B * H;
  const uint32_t v_bytes = (uint32_t)((size_t)bh * Nk * D * 2);
  const uint32_t ws_bytes = (uint32_t)bf16_workspace_bytes(B, H, Nk, D);
  hipLaunchKernelGGL(Kernels<D>::pack, dim3(ntiles, bh), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(v), static_cast<const uint16_t*>(tv),
                     static_cast<char*>(ws), Nk, ntiles, v_bytes, ws_bytes);
  return hipGetLastError();
}

template <int D>
hipError_t launch_main_d(const void* q, const void* k, const void* tq, const void* tk,
                         const void* ws, float* o, float* to, float* lse, int B, int H, int Nq,
                         int Nk, float scale, hipStream_t stream) {
  const int ntiles = (Nk + kBC - 1) / kBC;
  const int nqt = (Nq + kBR - 1) / kBR;
  const int bh = B * H;
  Extents ext;
  ext.q_bytes = (uint32_t)((size_t)bh * Nq * D * 2);
  ext.k_bytes = (uint32_t)((size_t)bh * Nk * D * 2);
  ext.ws_bytes = (uint32_t)bf16_workspace_bytes(B, H, Nk, D);
  ext.o_bytes = (uint32_t)((size_t)bh * Nq * D * 4);
  ext.lse_bytes = (uint32_t)((size_t)bh * Nq * 4);
  hipLaunchKernelGGL(Kernels<D>::main, dim3(nqt, bh), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(tq), static_cast<const uint16_t*>(tk),
                     static_cast<const char*>(ws), o, to, lse, Nq, Nk, ntiles, ext, scale,
                     scale * kLog2e);
  return hipGetLastError();
}

}  // namespace bf16_path
using namespace bf16_path;

size_t bf16_workspace_bytes(int B, int H, int Nk, int d) {
  const size_t ntiles = ((size_t)Nk + kBC - 1) / kBC;
  return (size_t)B * H * ntiles * 2 * kBC * (size_t)d * 2;
}

hipError_t launch_pack_v(const void* v, const void* tv, int B, int H, int Nk, int d, void* ws,
                         hipStream_t stream) {
  return d == 128 ? launch_pack_d<128>(v, tv, B, H, Nk, ws, stream)
                  : launch_pack_d<64>(v, tv, B, H, Nk, ws, stream);
}

hipError_t launch_bf16_packed(const void* q, const void* k, const void* tq, const void* tk,
                              const void* ws, float* o, float* to, float* lse, int B, int H,
                              int Nq, int Nk, int d, float scale, hipStream_t stream) {
  return d == 128 ? launch_main_d<128>(q, k, tq, tk, ws, o, to, lse, B, H, Nq, Nk, scale, stream)
                  : launch_main_d<64>(q, k, tq, tk, ws, o, to, lse, B, H, Nq, Nk, scale, stream);
}

hipError_t launch_bf16(const void* q, const void* k, const void* v, const void* tq,
                       const void* tk, const void* tv, float* o, float* to, float* lse, int B,
                       int H, int Nq, int Nk, int d, float scale, void* ws, hipStream_t stream) {
  const hipError_t e = launch_pack_v(v, tv, B, H, Nk, d, ws, stream);
  if (e != hipSuccess) return e;
  return launch_bf16_packed(q, k, tq, tk, ws, o, to, lse, B, H, Nq, Nk, d, scale, stream);
}

}  // namespace ajvp
