// Internal host-side launch interface between the C ABI (abi.cpp) and the
// kernel translation units. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nc {

enum Dtype { kBF16 = 0, kF32 = 1 };

// ---- prefill input stage: k' = RMSNorm(RoPE(k)) in k's layout and type, and
// ---- the (cos, sin) table [T][D/2] of positions pos_offset + t for q. With
// ---- vc non-null, kp and vc are (B, Tk, Hkv, D) caches: k' and a copy of v
// ---- go to their rows row0 .. row0 + T - 1; with ve non-null the copy is
// ---- v + vgate * ve (vgate (B, T, Hkv), one value per row).
size_t attn_prep_table_bytes(int T, int D, Dtype dt);
size_t attn_prep_k_bytes(int B, int T, int Hkv, int D, Dtype dt);
hipError_t launch_attn_prep(const void* k, void* kp, void* tabq, int B, int T, int Hkv, int D,
                            double rope_base, int pos_offset, const void* v, void* vc, int Tk,
                            int row0, const void* ve, const void* vgate, Dtype dt,
                            hipStream_t stream);

// the (cos, sin) table of positions pos_offset .. pos_offset + T - 1 alone,
// in the layout and type of attn_prep's (attn_prep_table_bytes(T, D, dt))
hipError_t launch_rope_table(void* tab, int T, int D, double rope_base, int pos_offset, Dtype dt,
                             hipStream_t stream);

hipError_t launch_rope_qknorm(const void* q, const void* k, void* q_out, void* k_out, int B,
                              int T, int H, int Hkv, int D, double rope_base, int pos_offset,
                              Dtype dt, hipStream_t stream);

// attention from raw q (rotated/normalised in the kernel with tabq), k' and v;
// kp and v hold Tk key rows per sequence, query row t sits at key row kofs + t.
// part (part_bytes, at least attn_core_part_bytes) holds the partial rows of a
// launch whose key tiles are cut into slices; with part_bytes 0 there is none.
// lse, when not null, receives ln of each output row's softmax denominator
// (fp32, one per row of o: the row log-sum-exp of the scaled scores).
size_t attn_core_part_bytes(int B, int T, int H, int Hkv, int D, int Tk, Dtype dt);
hipError_t launch_attn_core(const void* q, const void* kp, const void* v, void* o, int B, int T,
                            int H, int Hkv, int D, int window, const void* tabq, int Tk, int kofs,
                            void* part, size_t part_bytes, Dtype dt, hipStream_t stream,
                            float* lse = nullptr);

size_t decode_workspace_bytes(int B, int Tmax, int H, int Hkv, int D, int window, int Lp);
// ve_new (B, Hkv, D) and ve_gate (B, Hkv), or both null: v_new + ve_gate * ve_new
// is appended and used in place of v_new
hipError_t launch_attn_decode(const void* q, const void* k_new, const void* v_new, void* k_cache,
                              void* v_cache, const int32_t* seqlens, void* o, int B, int Tmax,
                              int H, int Hkv, int D, int window, double rope_base, Dtype dt,
                              void* ws, hipStream_t stream, const void* ve_new = nullptr,
                              const void* ve_gate = nullptr);
// decode over a shared (Lp, Hkv, D) prompt cache and per-sequence caches of
// Tgen rows holding positions Lp ..
hipError_t launch_attn_decode_shared(const void* q, const void* k_new, const void* v_new,
                                     const void* k_prompt, const void* v_prompt, int Lp,
                                     void* k_cache, void* v_cache, const int32_t* seqlens, void* o,
                                     int B, int Tgen, int H, int Hkv, int D, int window,
                                     double rope_base, Dtype dt, void* ws, hipStream_t stream,
                                     const void* ve_new = nullptr, const void* ve_gate = nullptr);

// ---- backward: gradients with respect to the raw q, k, v from dO and the
// ---- forward's o and row log-sum-exp; ws of attn_bwd_workspace_bytes
size_t attn_bwd_workspace_bytes(int B, int T, int H, int Hkv, int D, Dtype dt);
hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                           int T, int H, int Hkv, int D, int window, double rope_base,
                           int pos_offset, Dtype dt, void* ws, hipStream_t stream);

// ---- the static per-device scratch of the entry point that allocates
// ---- nothing: its size, and its address on the current device (looked up
// ---- once per device)
size_t scratch_capacity();
hipError_t scratch_address(void** out);

// ---- fused bias-free q, k, v projection of x (B*T, C) with the RoPE and
// ---- QK-norm epilogue on q and k; tab: launch_rope_table's table for T, D
hipError_t launch_qkv_rope_qknorm(const void* x, const void* wq, const void* wk, const void* wv,
                                  void* q, void* k, void* v, const void* tab, int B, int T, int C,
                                  int H, int Hkv, int D, Dtype dt, hipStream_t stream);

}  // namespace nc
