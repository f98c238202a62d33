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
//     mu = s u / l (u = rowsum P dS), dO = G / l - mu O and lse.
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
  float l;                   // this lane's half of sum p
  float u;                   // this lane's half of sum p * dS_raw
};

// ---- one 32-key block of a staged tile, in four pieces ----
// The main loop software-pipelines them: the S/dS products of block j+1 (matrix
// cores) are issued in the same scheduling region as the softmax of block j
// (vector ALU), so the two units overlap within one wave.

// S^T = K Q^T and dS^T = dK Q^T + K dQ^T for keys 32kb..32kb+31 of the staged
// tile (rows: key, columns: this wave's 32 queries).
template <int D>
__device__ __attribute__((always_inline)) inline void qk_block(const char* stage, int kb,
                                                               const u32x4* qf, const u32x4* dqf,
                                                               int l32, int g, f32x16& s,
                                                               f32x16& ds) {
  using G = Geo<D>;
  const char* sK = stage;
  const char* sdK = stage + G::kKTile;
  const int rowoff = (32 * kb + l32) * G::kKRow + 16 * g;
  s = f32x16{};
  ds = f32x16{};
#pragma unroll
  for (int ks = 0; ks < G::kKS; ++ks) {
    const int off = rowoff + 32 * ks;
    const u32x4 a = lds_load16(sK + off);
    const u32x4 da = lds_load16(sdK + off);
    s = mma_bf16(a, qf[ks], s);
    ds = mma_bf16(a, dqf[ks], ds);
    ds = mma_bf16(da, qf[ks], ds);
  }
}

// Keys at or past Nk (last tile only) leave the max and get p = 0, dS = 0,
// whatever their staged rows hold.  Slot r of lane half g holds key
// key0 + 8(r/4) + 4g + r%4.
__device__ __attribute__((always_inline)) inline void mask_block(f32x16& s, f32x16& ds, int key0,
                                                                 int Nk, int g) {
#pragma unroll
  for (int r = 0; r < 16; ++r)
    if (key0 + 8 * (r >> 2) + 4 * g + (r & 3) >= Nk) {
      s[r] = -INFINITY;
      ds[r] = 0.f;
    }
}

// Operands of the second contraction for one block: P and s*P*dS in fp16.
struct PBlock {
  u32x4 p[2], pd[2];
};

// Online softmax in the accumulator layout: each lane owns one query row and
// half of the block's keys (the other half is in lane l ^ 32).  Updates m, l, u
// and returns the factor alpha by which the accumulators must be rescaled
// before this block's products are added.  kMask: keys >= Nk (already -inf in
// s) get p = 0 explicitly, which also covers scale = 0 (-inf * 0 is NaN).
template <int D, bool kMask>
__device__ __attribute__((always_inline)) inline float softmax_block(RowState<D>& st,
                                                                     const f32x16& s,
                                                                     const f32x16& ds,
                                                                     float c_log2, float scale,
                                                                     int key0, int Nk, int g,
                                                                     PBlock& pb) {
  float mx = s[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
  mx = fmaxf(mx, swap_halves(mx));
  const float mt = mx * c_log2;
  const float m_new = (mt > st.m + kTau) ? mt : st.m;
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
  st.m = m_new;
  float p[16], pd[16], lsum = 0.f, usum = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], c_log2, -m_new));
    if (kMask && key0 + 8 * (r >> 2) + 4 * g + (r & 3) >= Nk) p[r] = 0.f;
    lsum += p[r];
    const float t = p[r] * ds[r];
    usum += t;
    pd[r] = t * scale;
  }
  pb.p[0] = pack_f16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
  pb.p[1] = pack_f16x8(p[8], p[9], p[10], p[11], p[12], p[13], p[14], p[15]);
  pb.pd[0] = pack_f16x8(pd[0], pd[1], pd[2], pd[3], pd[4], pd[5], pd[6], pd[7]);
  pb.pd[1] = pack_f16x8(pd[8], pd[9], pd[10], pd[11], pd[12], pd[13], pd[14], pd[15]);
  st.l = st.l * alpha + lsum;
  st.u = st.u * alpha + usum;
  return alpha;
}

// The running max moved (rare with the kTau headroom): rescale A and G.  One
// 16-register block at a time (scheduling barriers in between), so this rare
// path needs few temporaries and does not raise the register pressure of the
// main path.
template <int D>
__device__ __attribute__((always_inline)) inline void rescale(RowState<D>& st, float alpha) {
  if (wave_any(alpha != 1.0f)) {
#pragma unroll
    for (int cb = 0; cb < Geo<D>::kCB; ++cb) {
      st.accA[cb] *= alpha;
      __builtin_amdgcn_sched_barrier(0);
      st.accG[cb] *= alpha;
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// A^T += V^T P^T ; G^T += V^T (s P dS)^T + dV^T P^T for keys 32kb.. of the tile.
template <int D>
__device__ __attribute__((always_inline)) inline void pv_block(RowState<D>& st, const char* stage,
                                                               int kb, const PBlock& pb, int l32,
                                                               int g) {
  using G = Geo<D>;
  const char* sV = stage + 2 * G::kKTile;
  const char* sdV = sV + G::kVTile;
#pragma unroll
  for (int cb = 0; cb < G::kCB; ++cb) {
    const int vrow = (32 * cb + l32) * G::kVRow + 16 * g;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int off = vrow + 16 * (4 * kb + 2 * t);
      const u32x4 a = lds_load16(sV + off);
      const u32x4 da = lds_load16(sdV + off);
      st.accA[cb] = mma_f16(a, pb.p[t], st.accA[cb]);
      st.accG[cb] = mma_f16(a, pb.pd[t], st.accG[cb]);
      st.accG[cb] = mma_f16(da, pb.p[t], st.accG[cb]);
    }
  }
}

// Keeps the softmax outputs of a block in registers at this point, so the
// compiler does not sink their computation past the rescale branch into the
// next region.  Emits no instruction.
__device__ __attribute__((always_inline)) inline void pin(PBlock& pb) {
  asm volatile("" : "+v"(pb.p[0]), "+v"(pb.p[1]), "+v"(pb.pd[0]), "+v"(pb.pd[1]));
}

// One pipeline region for block j of the key sequence: S/dS of block j, then
// the products P V of block j-1 (kPrev; operands `prev` from the previous
// region), which are independent of block j's softmax, so the scheduler can
// keep the matrix cores busy with them while the vector ALU runs the softmax.
// kMask: block j lies in the last tile (keys >= Nk masked).  The accumulators
// are rescaled by block j's alpha after P V of block j-1 has been added and
// before that of block j is, as the online update requires.
template <int D, bool kPrev, bool kMask>
__device__ __attribute__((always_inline)) inline void region(
    RowState<D>& st, const char* stage_cur, int kb_cur, const char* stage_prev, int kb_prev,
    const u32x4* qf, const u32x4* dqf, int l32, int g, const PBlock& prev, PBlock& cur, int Nk,
    int key0, float c_log2, float scale) {
  f32x16 s, ds;
  qk_block<D>(stage_cur, kb_cur, qf, dqf, l32, g, s, ds);
  if constexpr (kPrev) pv_block<D>(st, stage_prev, kb_prev, prev, l32, g);
  if constexpr (kMask) mask_block(s, ds, key0, Nk, g);
  const float alpha = softmax_block<D, kMask>(st, s, ds, c_log2, scale, key0, Nk, g, cur);
  pin(cur);
  rescale<D>(st, alpha);
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
  st.l = 0.f;
  st.u = 0.f;

  // Software pipeline over 32-key blocks j = 0 .. 2*ntiles-1 (block j is half
  // j % 2 of tile j / 2): region j forms S/dS and the softmax of block j and
  // the products P V of block j-1.  K|dK(t) and V|dV(t) live in LDS buffer
  // t % 2; K(t) is read in regions 2t, 2t+1 and V(t) in regions 2t+1, 2t+2.
  // Per tile kt, with barrier B_j after region j:
  //   K|dK(kt+1) -> LDS, V|dV(kt+1) loads issued   (K|dK(kt-1) last read in region 2kt-1)
  //   region 2kt,   B_2kt
  //   V|dV(kt+1) -> LDS, K|dK(kt+2) loads issued   (V|dV(kt-1) last read in region 2kt)
  //   region 2kt+1, B_2kt+1
  // so K|dK(kt+1) is visible from region 2kt+1 on and V|dV(kt+1) from 2kt+2 on.
  PBlock pa, pb;  // softmax outputs of the even / odd block
  const int kLast = ntiles - 1;
  auto stage = [&](int t) { return smem + (t & 1) * G::kStageBytes; };
  load_k(0);
  store_k(smem);
  load_v(0);
  store_v(smem);
  load_k(1);  // past the last tile the descriptors read zeros or unused data
  __syncthreads();
  if (ntiles == 1) {
    region<D, false, true>(st, smem, 0, nullptr, 0, qf, dqf, l32, g, pb, pa, Nk, 0, c_log2, scale);
    region<D, true, true>(st, smem, 1, smem, 0, qf, dqf, l32, g, pa, pb, Nk, 32, c_log2, scale);
  } else {
    // tile 0
    store_k(stage(1));
    load_v(1);
    region<D, false, false>(st, smem, 0, nullptr, 0, qf, dqf, l32, g, pb, pa, Nk, 0, c_log2, scale);
    __syncthreads();
    store_v(stage(1));
    load_k(2);
    region<D, true, false>(st, smem, 1, smem, 0, qf, dqf, l32, g, pa, pb, Nk, 0, c_log2, scale);
    __syncthreads();
    // tiles 1 .. ntiles-2
    for (int kt = 1; kt < kLast; ++kt) {
      store_k(stage(kt + 1));
      load_v(kt + 1);
      region<D, true, false>(st, stage(kt), 0, stage(kt - 1), 1, qf, dqf, l32, g, pb, pa, Nk, 0,
                             c_log2, scale);
      __syncthreads();
      store_v(stage(kt + 1));
      load_k(kt + 2);
      region<D, true, false>(st, stage(kt), 1, stage(kt), 0, qf, dqf, l32, g, pa, pb, Nk, 0,
                             c_log2, scale);
      __syncthreads();
    }
    // last tile: keys past Nk are masked
    region<D, true, true>(st, stage(kLast), 0, stage(kLast - 1), 1, qf, dqf, l32, g, pb, pa, Nk,
                          kLast * kBC, c_log2, scale);
    region<D, true, true>(st, stage(kLast), 1, stage(kLast), 0, qf, dqf, l32, g, pa, pb, Nk,
                          kLast * kBC + 32, c_log2, scale);
  }
  pv_block<D>(st, stage(kLast), 1, pb, l32, g);

  // ---- epilogue: O = A / l, mu = s u / l, dO = G / l - mu O, lse ----
  const float l = st.l + swap_halves(st.l);
  const float u = st.u + swap_halves(st.u);
  const float inv_l = 1.0f / l;
  const float mu = u * scale * inv_l;
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
