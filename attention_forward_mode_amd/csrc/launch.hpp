// launch.hpp -- host-side launchers of the gfx950 attention-JVP kernels.
// Called only by the C ABI (attn_jvp_api.cpp) after it has validated every
// argument; each returns the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace ajvp {

// Workspace bytes of the bf16 path: one LDS tile image (K, dK, V^T, dV^T) per
// (b, h) and 64-key tile.
size_t bf16_workspace_bytes(int B, int H, int Nk, int d);

hipError_t launch_bf16(const void* q, const void* k, const void* v, const void* tq,
                       const void* tk, const void* tv, float* o, float* to, float* lse,
                       int B, int H, int Nq, int Nk, int d, float scale, void* workspace,
                       hipStream_t stream);

// The two phases of launch_bf16: K, V, dK, dV -> tile images in the
// workspace, then the fused kernel reading them.
hipError_t launch_pack_kv(const void* k, const void* v, const void* tk, const void* tv, int B,
                          int H, int Nk, int d, void* workspace, hipStream_t stream);
hipError_t launch_bf16_packed(const void* q, const void* tq, const void* workspace, float* o,
                              float* to, float* lse, int B, int H, int Nq, int Nk, int d,
                              float scale, hipStream_t stream);

// Extended JVP: tq, tk, tv may be NULL (zero tangents; with tk = tv = NULL the
// frozen-key mode skips their products), tlse (the tangent of lse) and lse may
// be NULL, o and to are fp32 or (out_bf16) bf16.
hipError_t launch_bf16_ex(const void* q, const void* k, const void* v, const void* tq,
                          const void* tk, const void* tv, void* o, void* to, float* lse,
                          float* tlse, int B, int H, int Nq, int Nk, int d, float scale,
                          bool out_bf16, void* workspace, hipStream_t stream);

// Split-KV: the key tiles cut into ranges that run on separate workgroups
// (nsplit ranges, 0 = chosen from the sizes), partial states merged.
int splitkv_count(int B, int H, int Nq, int Nk, int d, int nsplit, int rows);
size_t splitkv_workspace_bytes(int B, int H, int Nq, int Nk, int d, int nsplit);
hipError_t launch_bf16_splitkv(const void* q, const void* k, const void* v, const void* tq,
                               const void* tk, const void* tv, float* o, float* to, float* lse,
                               float* tlse, int B, int H, int Nq, int Nk, int d, float scale,
                               int nsplit, void* ws, hipStream_t stream);

// Forward attention alone with key-tile ranges (fp32 O), merged.
hipError_t launch_fwd_splitkv(const void* q, const void* k, const void* v, float* o, float* lse,
                              int B, int H, int Nq, int Nk, int d, float scale, int nsplit,
                              void* ws, hipStream_t stream);

// Forward attention alone (O, lse).
hipError_t launch_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                      int H, int Nq, int Nk, int d, float scale, bool out_bf16, void* workspace,
                      hipStream_t stream);

// Merge of P partial results over disjoint key subsets (rows R, head dim d;
// R * d * 4 under 2^31 bytes).  Part p starts `stride` rows after part p - 1
// (0: stride R, the parts back to back).
hipError_t launch_merge(const float* lse_p, const float* o_p, const float* to_p,
                        const float* tlse_p, int P, int R, int d, float* lse, float* o,
                        float* to, float* tlse, hipStream_t stream, int64_t stride = 0);

// Backward pass (gradients of a loss through O): workspace bytes and launch.
size_t bwd_workspace_bytes(int B, int H, int Nq, int Nk, int d);
hipError_t launch_bwd(const void* q, const void* k, const void* v, const float* o, const void* go,
                      const float* lse, float* gq, float* gk, float* gv, int B, int H, int Nq,
                      int Nk, int d, float scale, void* workspace, hipStream_t stream);

// The device buffer of attn_jvp_fwd_noalloc (attn_jvp_noalloc.hip): its size,
// and its address on the current device (looked up once per device).
size_t scratch_bytes();
hipError_t scratch_buffer(void** out);

hipError_t launch_f32(const float* q, const float* k, const float* v, const float* tq,
                      const float* tk, const float* tv, float* o, float* to, float* lse,
                      int B, int H, int Nq, int Nk, int d, float scale, hipStream_t stream);

}  // namespace ajvp
