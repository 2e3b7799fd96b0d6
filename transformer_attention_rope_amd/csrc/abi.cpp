// C ABI of the attention-block library: host-side validation, workspace
// sizing and kernel dispatch. Every check runs before the first HIP call, so
// argument errors are reported without touching the device.
#include "nc_attn.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>

#include "launch.hpp"

namespace {

thread_local char g_err[512] = "";

nc_status fail(nc_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

nc_status ok() {
  g_err[0] = '\0';
  return NC_OK;
}

nc_status hip_fail(hipError_t e, const char* what) {
  return fail(NC_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

nc_status check_common(int B, int T, int H, int Hkv, int D, nc_dtype dt, const char* tname) {
  if (dt != NC_BF16 && dt != NC_F32) return fail(NC_ERR_INVALID, "dtype %d is not NC_BF16 or NC_F32", (int)dt);
  if (B < 1 || T < 1 || H < 1 || Hkv < 1 || D < 1)
    return fail(NC_ERR_INVALID, "sizes must be >= 1 (B=%d %s=%d H=%d Hkv=%d D=%d)", B, tname, T, H, Hkv, D);
  if (H % Hkv != 0) return fail(NC_ERR_INVALID, "H=%d is not a multiple of Hkv=%d", H, Hkv);
  if (D != 32 && D != 64 && D != 128) return fail(NC_ERR_UNSUPPORTED, "head dim D=%d not in {32, 64, 128}", D);
  // every element index must fit comfortably in 63 bits and every row index in 31
  const long long rows_q = (long long)B * T * H;
  const long long rows_k = (long long)B * T * Hkv;
  if (rows_q > 0x7fffffffLL || rows_k > 0x7fffffffLL)
    return fail(NC_ERR_INVALID, "B*%s*H=%lld rows exceed 2^31-1", tname, rows_q);
  return NC_OK;
}

nc_status check_rope(double rope_base, int pos_offset, int T) {
  if (!std::isfinite(rope_base) || !(rope_base > 0.0))
    return fail(NC_ERR_INVALID, "rope_base must be finite and > 0 (got %g)", rope_base);
  if (pos_offset < 0) return fail(NC_ERR_INVALID, "pos_offset must be >= 0 (got %d)", pos_offset);
  if ((long long)pos_offset + T > (1LL << 30))
    return fail(NC_ERR_INVALID, "pos_offset + T = %lld exceeds 2^30", (long long)pos_offset + T);
  return NC_OK;
}

// one sequence's K or V must be addressable with 32-bit byte offsets
nc_status check_seq_bytes(int T, int Hkv, int D, nc_dtype dt) {
  const long long bytes = (long long)T * Hkv * D * (dt == NC_BF16 ? 2 : 4);
  if (bytes >= (1LL << 32))
    return fail(NC_ERR_UNSUPPORTED, "T*Hkv*D*elem = %lld bytes per sequence reaches 2^32", bytes);
  return NC_OK;
}

// the value-embedding pair: both NULL (no gate) or both valid
nc_status check_ve(const void* ve, const void* gate, nc_dtype dt) {
  if ((ve == nullptr) != (gate == nullptr))
    return fail(NC_ERR_INVALID, "ve and ve_gate must both be NULL or both be given");
  if (ve == nullptr) return NC_OK;
  if (!aligned16(ve)) return fail(NC_ERR_INVALID, "ve is not 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(gate) & (dt == NC_BF16 ? 1u : 3u)) != 0)
    return fail(NC_ERR_INVALID, "ve_gate is not aligned to its element size");
  return NC_OK;
}

nc_status check_ptrs(const char* names[], const void* ptrs[], int n) {
  for (int i = 0; i < n; ++i) {
    if (ptrs[i] == nullptr) return fail(NC_ERR_INVALID, "%s is NULL", names[i]);
    if (!aligned16(ptrs[i])) return fail(NC_ERR_INVALID, "%s is not 16-byte aligned", names[i]);
  }
  return NC_OK;
}

}  // namespace

extern "C" {

int nc_abi_version(void) { return NC_ABI_VERSION; }

const char* nc_status_string(nc_status s) {
  switch (s) {
    case NC_OK: return "NC_OK";
    case NC_ERR_INVALID: return "NC_ERR_INVALID: invalid argument";
    case NC_ERR_UNSUPPORTED: return "NC_ERR_UNSUPPORTED: unsupported shape";
    case NC_ERR_HIP: return "NC_ERR_HIP: HIP runtime error";
    default: return "unknown nc_status";
  }
}

const char* nc_last_error(void) { return g_err; }

// ------------------------------------------------------------ rope_qknorm
size_t nc_rope_qknorm_workspace_bytes(int T, int D, int pos_offset) {
  (void)T;
  (void)D;
  (void)pos_offset;
  return 0;
}

nc_status nc_rope_qknorm(const void* q, const void* k, void* q_out, void* k_out, int B, int T,
                         int H, int Hkv, int D, double rope_base, int pos_offset, nc_dtype dt,
                         void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  nc_status s = check_common(B, T, H, Hkv, D, dt, "T");
  if (s != NC_OK) return s;
  if ((s = check_rope(rope_base, pos_offset, T)) != NC_OK) return s;
  const char* names[] = {"q", "k", "q_out", "k_out"};
  const void* ptrs[] = {q, k, q_out, k_out};
  if ((s = check_ptrs(names, ptrs, 4)) != NC_OK) return s;
  hipError_t e = nc::launch_rope_qknorm(q, k, q_out, k_out, B, T, H, Hkv, D, rope_base, pos_offset,
                                        dt == NC_BF16 ? nc::kBF16 : nc::kF32, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "rope_qknorm launch");
  return ok();
}

// ------------------------------------------------------ qkv_rope_qknorm
size_t nc_qkv_rope_qknorm_workspace_bytes(int T, int D, nc_dtype dtype) {
  if (T < 1 || (D != 32 && D != 64 && D != 128) || (dtype != NC_BF16 && dtype != NC_F32)) return 0;
  return round_up(nc::attn_prep_table_bytes(T, D, dtype == NC_F32 ? nc::kF32 : nc::kBF16));
}

nc_status nc_qkv_rope_qknorm(const void* x, const void* w_q, const void* w_k, const void* w_v,
                             void* q_out, void* k_out, void* v_out, int B, int T, int C, int H,
                             int Hkv, int D, double rope_base, int pos_offset, nc_dtype dt,
                             void* ws, size_t ws_bytes, void* stream) {
  nc_status s = check_common(B, T, H, Hkv, D, dt, "T");
  if (s != NC_OK) return s;
  if (C < 1) return fail(NC_ERR_INVALID, "C must be >= 1 (got %d)", C);
  if (C % 64 != 0) return fail(NC_ERR_UNSUPPORTED, "C=%d is not a multiple of 64", C);
  if (C > (1 << 20)) return fail(NC_ERR_UNSUPPORTED, "C=%d exceeds 2^20", C);
  if ((s = check_rope(rope_base, pos_offset, T)) != NC_OK) return s;
  const char* names[] = {"x", "w_q", "w_k", "w_v", "q_out", "k_out", "v_out"};
  const void* ptrs[] = {x, w_q, w_k, w_v, q_out, k_out, v_out};
  if ((s = check_ptrs(names, ptrs, 7)) != NC_OK) return s;
  const size_t need = nc_qkv_rope_qknorm_workspace_bytes(T, D, dt);
  if (ws == nullptr) return fail(NC_ERR_INVALID, "ws is NULL");
  if (!aligned16(ws)) return fail(NC_ERR_INVALID, "ws is not 16-byte aligned");
  if (ws_bytes < need)
    return fail(NC_ERR_INVALID, "workspace of %zu bytes is below the required %zu", ws_bytes, need);
  const nc::Dtype d = dt == NC_F32 ? nc::kF32 : nc::kBF16;
  hipError_t e = nc::launch_rope_table(ws, T, D, rope_base, pos_offset, d, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "rope table launch");
  e = nc::launch_qkv_rope_qknorm(x, w_q, w_k, w_v, q_out, k_out, v_out, ws, B, T, C, H, Hkv, D, d,
                                 (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "qkv launch");
  return ok();
}

// ---------------------------------------------------------------- attn_fwd
// Workspace: the (cos, sin) table of the T positions (fp16 pairs for bf16,
// fp32 pairs for fp32), then k', then room for the partial rows of a launch
// cut into key-tile slices (bf16 launches too small to fill the device).
namespace {
nc::Dtype to_dt(nc_dtype dt) { return dt == NC_F32 ? nc::kF32 : nc::kBF16; }
size_t prep_table_bytes(int T, int D, nc_dtype dt) {
  return round_up(nc::attn_prep_table_bytes(T, D, to_dt(dt)));
}
size_t prep_k_bytes(int B, int T, int Hkv, int D, nc_dtype dt) {
  return round_up(nc::attn_prep_k_bytes(B, T, Hkv, D, dt == NC_F32 ? nc::kF32 : nc::kBF16));
}
size_t part_bytes(int B, int T, int H, int Hkv, int D, int Tk, nc_dtype dt) {
  return nc::attn_core_part_bytes(B, T, H, Hkv, D, Tk, to_dt(dt));
}
nc_status check_fwd_sizes(int B, int T, int H, int Hkv, int D, nc_dtype dt) {
  nc_status s = check_common(B, T, H, Hkv, D, dt, "T");
  if (s != NC_OK) return s;
  if ((long long)T * (D / 2) > 0x7fffffffLL)
    return fail(NC_ERR_INVALID, "T=%d too long for the RoPE table", T);
  return check_seq_bytes(T, Hkv, D, dt);
}
nc_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (ws == nullptr) return fail(NC_ERR_INVALID, "ws is NULL");
  if (!aligned16(ws)) return fail(NC_ERR_INVALID, "ws is not 16-byte aligned");
  if (ws_bytes < need)
    return fail(NC_ERR_INVALID, "workspace of %zu bytes is below the required %zu", ws_bytes, need);
  return NC_OK;
}
}  // namespace

size_t nc_attn_fwd_workspace_bytes(int B, int T, int H, int Hkv, int D, int pos_offset,
                                   nc_dtype dtype) {
  (void)H;
  (void)pos_offset;
  if (B < 1 || T < 1 || Hkv < 1 || D < 2 || (dtype != NC_BF16 && dtype != NC_F32)) return 0;
  return prep_table_bytes(T, D, dtype) + prep_k_bytes(B, T, Hkv, D, dtype) +
         round_up(part_bytes(B, T, H, Hkv, D, T, dtype));
}

nc_status nc_attn_prep(const void* k, int B, int T, int Hkv, int D, double rope_base,
                       int pos_offset, nc_dtype dt, void* ws, size_t ws_bytes, void* stream) {
  nc_status s = check_fwd_sizes(B, T, Hkv, Hkv, D, dt);
  if (s != NC_OK) return s;
  if ((s = check_rope(rope_base, pos_offset, T)) != NC_OK) return s;
  const char* names[] = {"k"};
  const void* ptrs[] = {k};
  if ((s = check_ptrs(names, ptrs, 1)) != NC_OK) return s;
  if ((s = check_ws(ws, ws_bytes, prep_table_bytes(T, D, dt) + prep_k_bytes(B, T, Hkv, D, dt))) != NC_OK)
    return s;
  hipError_t e = nc::launch_attn_prep(k, (char*)ws + prep_table_bytes(T, D, dt), ws, B, T, Hkv, D,
                                      rope_base, pos_offset, nullptr, nullptr, T, 0, nullptr, nullptr,
                                      to_dt(dt), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attn_prep launch");
  return ok();
}

nc_status nc_attn_core(const void* q, const void* v, void* o, int B, int T, int H, int Hkv, int D,
                       int window, nc_dtype dt, void* ws, size_t ws_bytes, void* stream) {
  nc_status s = check_fwd_sizes(B, T, H, Hkv, D, dt);
  if (s != NC_OK) return s;
  if (window < 1) return fail(NC_ERR_INVALID, "window must be >= 1 (got %d)", window);
  const char* names[] = {"q", "v", "o"};
  const void* ptrs[] = {q, v, o};
  if ((s = check_ptrs(names, ptrs, 3)) != NC_OK) return s;
  if ((s = check_ws(ws, ws_bytes, nc_attn_fwd_workspace_bytes(B, T, H, Hkv, D, 0, dt))) != NC_OK)
    return s;
  const size_t front = prep_table_bytes(T, D, dt) + prep_k_bytes(B, T, Hkv, D, dt);
  hipError_t e = nc::launch_attn_core(q, (const char*)ws + prep_table_bytes(T, D, dt), v, o, B, T, H,
                                      Hkv, D, window, ws, T, 0, (char*)ws + front,
                                      part_bytes(B, T, H, Hkv, D, T, dt), to_dt(dt), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attn_core launch");
  return ok();
}

nc_status nc_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int T, int H,
                      int Hkv, int D, int window, double rope_base, int pos_offset, nc_dtype dt,
                      void* ws, size_t ws_bytes, void* stream) {
  nc_status s = check_fwd_sizes(B, T, H, Hkv, D, dt);
  if (s != NC_OK) return s;
  if (window < 1) return fail(NC_ERR_INVALID, "window must be >= 1 (got %d)", window);
  if ((s = check_rope(rope_base, pos_offset, T)) != NC_OK) return s;
  const char* names[] = {"q", "k", "v", "o"};
  const void* ptrs[] = {q, k, v, o};
  if ((s = check_ptrs(names, ptrs, 4)) != NC_OK) return s;
  if ((s = check_ws(ws, ws_bytes, nc_attn_fwd_workspace_bytes(B, T, H, Hkv, D, pos_offset, dt))) != NC_OK)
    return s;
  if ((s = nc_attn_prep(k, B, T, Hkv, D, rope_base, pos_offset, dt, ws, ws_bytes, stream)) != NC_OK)
    return s;
  return nc_attn_core(q, v, o, B, T, H, Hkv, D, window, dt, ws, ws_bytes, stream);
}

size_t nc_attn_fwd_normed_workspace_bytes(int B, int T, int H, int Hkv, int D, nc_dtype dtype) {
  if (B < 1 || T < 1 || H < 1 || Hkv < 1 || D < 2 || (dtype != NC_BF16 && dtype != NC_F32)) return 0;
  const size_t n = part_bytes(B, T, H, Hkv, D, T, dtype);
  return n ? round_up(n) : 0;
}

nc_status nc_attn_fwd_normed(const void* q, const void* k, const void* v, void* o, int B, int T,
                             int H, int Hkv, int D, int window, nc_dtype dt, void* ws,
                             size_t ws_bytes, void* stream) {
  nc_status s = check_fwd_sizes(B, T, H, Hkv, D, dt);
  if (s != NC_OK) return s;
  if (window < 1) return fail(NC_ERR_INVALID, "window must be >= 1 (got %d)", window);
  const char* names[] = {"q", "k", "v", "o"};
  const void* ptrs[] = {q, k, v, o};
  if ((s = check_ptrs(names, ptrs, 4)) != NC_OK) return s;
  const size_t need = nc_attn_fwd_normed_workspace_bytes(B, T, H, Hkv, D, dt);
  if (need > 0 && (s = check_ws(ws, ws_bytes, need)) != NC_OK) return s;
  // no table: the kernel takes the q rows as rotated and normalised
  hipError_t e = nc::launch_attn_core(q, k, v, o, B, T, H, Hkv, D, window, nullptr, T, 0,
                                      need > 0 ? ws : nullptr, need, to_dt(dt), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attn_core launch");
  return ok();
}

nc_status nc_attn_fwd_lse(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                          int T, int H, int Hkv, int D, int window, double rope_base, int pos_offset,
                          nc_dtype dt, void* ws, size_t ws_bytes, void* stream) {
  nc_status s = check_fwd_sizes(B, T, H, Hkv, D, dt);
  if (s != NC_OK) return s;
  if (window < 1) return fail(NC_ERR_INVALID, "window must be >= 1 (got %d)", window);
  if ((s = check_rope(rope_base, pos_offset, T)) != NC_OK) return s;
  const char* names[] = {"q", "k", "v", "o"};
  const void* ptrs[] = {q, k, v, o};
  if ((s = check_ptrs(names, ptrs, 4)) != NC_OK) return s;
  if (lse == nullptr) return fail(NC_ERR_INVALID, "lse is NULL");
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return fail(NC_ERR_INVALID, "lse is not 4-byte aligned");
  if ((s = check_ws(ws, ws_bytes, nc_attn_fwd_workspace_bytes(B, T, H, Hkv, D, pos_offset, dt))) != NC_OK)
    return s;
  if ((s = nc_attn_prep(k, B, T, Hkv, D, rope_base, pos_offset, dt, ws, ws_bytes, stream)) != NC_OK)
    return s;
  const size_t front = prep_table_bytes(T, D, dt) + prep_k_bytes(B, T, Hkv, D, dt);
  hipError_t e = nc::launch_attn_core(q, (const char*)ws + prep_table_bytes(T, D, dt), v, o, B, T, H,
                                      Hkv, D, window, ws, T, 0, (char*)ws + front,
                                      part_bytes(B, T, H, Hkv, D, T, dt), to_dt(dt),
                                      (hipStream_t)stream, lse);
  if (e != hipSuccess) return hip_fail(e, "attn_core launch");
  return ok();
}

nc_status nc_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, int B, int T,
                              int H, int Hkv, int D, int window, double rope_base, int pos_offset,
                              nc_dtype dt, void* stream) {
  nc_status s = check_fwd_sizes(B, T, H, Hkv, D, dt);
  if (s != NC_OK) return s;
  const size_t need = nc_attn_fwd_workspace_bytes(B, T, H, Hkv, D, pos_offset, dt);
  if (need > nc::scratch_capacity())
    return fail(NC_ERR_INVALID, "the call needs %zu bytes of scratch, beyond the library's static %zu",
                need, nc::scratch_capacity());
  if (window < 1) return fail(NC_ERR_INVALID, "window must be >= 1 (got %d)", window);
  if ((s = check_rope(rope_base, pos_offset, T)) != NC_OK) return s;
  const char* names[] = {"q", "k", "v", "o"};
  const void* ptrs[] = {q, k, v, o};
  if ((s = check_ptrs(names, ptrs, 4)) != NC_OK) return s;
  void* ws = nullptr;
  hipError_t e = nc::scratch_address(&ws);
  if (e != hipSuccess) return hip_fail(e, "scratch address");
  return nc_attn_fwd(q, k, v, o, B, T, H, Hkv, D, window, rope_base, pos_offset, dt, ws,
                     nc::scratch_capacity(), stream);
}

// ---------------------------------------------------------------- attn_bwd
size_t nc_attn_bwd_workspace_bytes(int B, int T, int H, int Hkv, int D, nc_dtype dtype) {
  if (B < 1 || T < 1 || H < 1 || Hkv < 1 || H % Hkv != 0 || (D != 32 && D != 64 && D != 128) ||
      (dtype != NC_BF16 && dtype != NC_F32))
    return 0;
  return nc::attn_bwd_workspace_bytes(B, T, H, Hkv, D, to_dt(dtype));
}

nc_status nc_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                      const float* lse, void* dq, void* dk, void* dv, int B, int T, int H, int Hkv,
                      int D, int window, double rope_base, int pos_offset, nc_dtype dt, void* ws,
                      size_t ws_bytes, void* stream) {
  nc_status s = check_fwd_sizes(B, T, H, Hkv, D, dt);
  if (s != NC_OK) return s;
  if (window < 1) return fail(NC_ERR_INVALID, "window must be >= 1 (got %d)", window);
  if ((s = check_rope(rope_base, pos_offset, T)) != NC_OK) return s;
  if ((s = check_seq_bytes(T, H, D, dt)) != NC_OK) return s;  // q, o, dout rows: 32-bit offsets
  const char* names[] = {"q", "k", "v", "o", "dout", "dq", "dk", "dv"};
  const void* ptrs[] = {q, k, v, o, dout, dq, dk, dv};
  if ((s = check_ptrs(names, ptrs, 8)) != NC_OK) return s;
  if (lse == nullptr) return fail(NC_ERR_INVALID, "lse is NULL");
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0) return fail(NC_ERR_INVALID, "lse is not 4-byte aligned");
  if ((s = check_ws(ws, ws_bytes, nc_attn_bwd_workspace_bytes(B, T, H, Hkv, D, dt))) != NC_OK) return s;
  hipError_t e = nc::launch_attn_bwd(q, k, v, o, dout, lse, dq, dk, dv, B, T, H, Hkv, D, window,
                                     rope_base, pos_offset, to_dt(dt), ws, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attn_bwd launch");
  return ok();
}

// ------------------------------------------------------------- attn_prefill
// Workspace: the (cos, sin) table of the chunk's T positions, then room for
// partial rows as in attn_fwd; k' and v go straight to the caches.
size_t nc_attn_prefill_workspace_bytes(int B, int T, int Tmax, int H, int Hkv, int D,
                                       nc_dtype dtype) {
  if (B < 1 || T < 1 || Tmax < T || H < 1 || Hkv < 1 || D < 2 ||
      (dtype != NC_BF16 && dtype != NC_F32))
    return 0;
  return prep_table_bytes(T, D, dtype) + round_up(part_bytes(B, T, H, Hkv, D, Tmax, dtype));
}

nc_status nc_attn_prefill(const void* q, const void* k, const void* v, const void* ve,
                          const void* ve_gate, void* k_cache, void* v_cache, void* o, int B, int T,
                          int Tmax, int H, int Hkv, int D, int window, double rope_base,
                          int pos_offset, nc_dtype dt, void* ws, size_t ws_bytes, void* stream) {
  nc_status s = check_fwd_sizes(B, T, H, Hkv, D, dt);
  if (s != NC_OK) return s;
  if (Tmax < 1) return fail(NC_ERR_INVALID, "Tmax must be >= 1 (got %d)", Tmax);
  if ((long long)B * Tmax * Hkv > 0x7fffffffLL)
    return fail(NC_ERR_INVALID, "B*Tmax*Hkv=%lld cache rows exceed 2^31-1", (long long)B * Tmax * Hkv);
  if (window < 1) return fail(NC_ERR_INVALID, "window must be >= 1 (got %d)", window);
  if ((s = check_rope(rope_base, pos_offset, T)) != NC_OK) return s;
  if ((long long)pos_offset + T > Tmax)
    return fail(NC_ERR_INVALID, "pos_offset + T = %lld exceeds Tmax=%d", (long long)pos_offset + T, Tmax);
  if ((s = check_seq_bytes(Tmax, Hkv, D, dt)) != NC_OK) return s;
  const char* names[] = {"q", "k", "v", "k_cache", "v_cache", "o"};
  const void* ptrs[] = {q, k, v, k_cache, v_cache, o};
  if ((s = check_ptrs(names, ptrs, 6)) != NC_OK) return s;
  if ((s = check_ws(ws, ws_bytes, nc_attn_prefill_workspace_bytes(B, T, Tmax, H, Hkv, D, dt))) != NC_OK)
    return s;
  if ((s = check_ve(ve, ve_gate, dt)) != NC_OK) return s;
  hipError_t e = nc::launch_attn_prep(k, k_cache, ws, B, T, Hkv, D, rope_base, pos_offset, v,
                                      v_cache, Tmax, pos_offset, ve, ve_gate, to_dt(dt),
                                      (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attn_prep launch");
  e = nc::launch_attn_core(q, k_cache, v_cache, o, B, T, H, Hkv, D, window, ws, Tmax, pos_offset,
                           (char*)ws + prep_table_bytes(T, D, dt),
                           part_bytes(B, T, H, Hkv, D, Tmax, dt), to_dt(dt), (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "attn_core launch");
  return ok();
}

// -------------------------------------------------------------- attn_decode
size_t nc_attn_decode_workspace_bytes(int B, int Tmax, int H, int Hkv, int D, int window) {
  if (B < 1 || Tmax < 1 || H < 1 || Hkv < 1 || H % Hkv != 0 || window < 1) return 0;
  const size_t n = nc::decode_workspace_bytes(B, Tmax, H, Hkv, D, window, 0);
  return n ? round_up(n) : 0;
}

nc_status nc_attn_decode(const void* q, const void* k_new, const void* v_new, const void* ve_new,
                         const void* ve_gate, void* k_cache, void* v_cache, const int32_t* seqlens,
                         void* o, int B, int Tmax, int H, int Hkv, int D, int window,
                         double rope_base, nc_dtype dt, void* ws, size_t ws_bytes, void* stream) {
  nc_status s = check_common(B, Tmax, H, Hkv, D, dt, "Tmax");
  if (s != NC_OK) return s;
  if (H / Hkv > 64) return fail(NC_ERR_UNSUPPORTED, "H/Hkv=%d query heads per K/V head exceed 64", H / Hkv);
  if (window < 1) return fail(NC_ERR_INVALID, "window must be >= 1 (got %d)", window);
  if ((s = check_rope(rope_base, 0, Tmax)) != NC_OK) return s;
  const char* names[] = {"q", "k_new", "v_new", "k_cache", "v_cache", "o"};
  const void* ptrs[] = {q, k_new, v_new, k_cache, v_cache, o};
  if ((s = check_ptrs(names, ptrs, 6)) != NC_OK) return s;
  if (seqlens == nullptr) return fail(NC_ERR_INVALID, "seqlens is NULL");
  if ((reinterpret_cast<uintptr_t>(seqlens) & 3u) != 0)
    return fail(NC_ERR_INVALID, "seqlens is not 4-byte aligned");
  if ((s = check_ve(ve_new, ve_gate, dt)) != NC_OK) return s;
  const size_t need = nc_attn_decode_workspace_bytes(B, Tmax, H, Hkv, D, window);
  if (need > 0) {
    if (ws == nullptr) return fail(NC_ERR_INVALID, "ws is NULL but %zu bytes are required", need);
    if (!aligned16(ws)) return fail(NC_ERR_INVALID, "ws is not 16-byte aligned");
    if (ws_bytes < need)
      return fail(NC_ERR_INVALID, "workspace of %zu bytes is below the required %zu", ws_bytes, need);
  }
  hipError_t e = nc::launch_attn_decode(q, k_new, v_new, k_cache, v_cache, seqlens, o, B, Tmax, H,
                                        Hkv, D, window, rope_base,
                                        dt == NC_BF16 ? nc::kBF16 : nc::kF32, ws,
                                        (hipStream_t)stream, ve_new, ve_gate);
  if (e != hipSuccess) return hip_fail(e, "attn_decode launch");
  return ok();
}

// ------------------------------------------------- attn_decode_shared
size_t nc_attn_decode_shared_workspace_bytes(int B, int Lp, int Tgen, int H, int Hkv, int D,
                                             int window) {
  if (B < 1 || Lp < 1 || Tgen < 1 || H < 1 || Hkv < 1 || H % Hkv != 0 || window < 1 ||
      (long long)Lp + Tgen > (1LL << 30))
    return 0;
  const size_t n = nc::decode_workspace_bytes(B, Lp + Tgen, H, Hkv, D, window, Lp);
  return n ? round_up(n) : 0;
}

nc_status nc_attn_decode_shared(const void* q, const void* k_new, const void* v_new,
                                const void* ve_new, const void* ve_gate,
                                const void* k_prompt, const void* v_prompt, int Lp, void* k_cache,
                                void* v_cache, const int32_t* seqlens, void* o, int B, int Tgen,
                                int H, int Hkv, int D, int window, double rope_base, nc_dtype dt,
                                void* ws, size_t ws_bytes, void* stream) {
  nc_status s = check_common(B, Tgen, H, Hkv, D, dt, "Tgen");
  if (s != NC_OK) return s;
  if (Lp < 1) return fail(NC_ERR_INVALID, "Lp must be >= 1 (got %d)", Lp);
  if (H / Hkv > 64) return fail(NC_ERR_UNSUPPORTED, "H/Hkv=%d query heads per K/V head exceed 64", H / Hkv);
  if (window < 1) return fail(NC_ERR_INVALID, "window must be >= 1 (got %d)", window);
  if ((s = check_rope(rope_base, Lp, Tgen)) != NC_OK) return s;
  if ((s = check_seq_bytes(Lp, Hkv, D, dt)) != NC_OK) return s;
  if ((s = check_seq_bytes(Tgen, Hkv, D, dt)) != NC_OK) return s;
  const char* names[] = {"q", "k_new", "v_new", "k_prompt", "v_prompt", "k_cache", "v_cache", "o"};
  const void* ptrs[] = {q, k_new, v_new, k_prompt, v_prompt, k_cache, v_cache, o};
  if ((s = check_ptrs(names, ptrs, 8)) != NC_OK) return s;
  if (seqlens == nullptr) return fail(NC_ERR_INVALID, "seqlens is NULL");
  if ((reinterpret_cast<uintptr_t>(seqlens) & 3u) != 0)
    return fail(NC_ERR_INVALID, "seqlens is not 4-byte aligned");
  if ((s = check_ve(ve_new, ve_gate, dt)) != NC_OK) return s;
  const size_t need = nc_attn_decode_shared_workspace_bytes(B, Lp, Tgen, H, Hkv, D, window);
  if (need > 0) {
    if (ws == nullptr) return fail(NC_ERR_INVALID, "ws is NULL but %zu bytes are required", need);
    if (!aligned16(ws)) return fail(NC_ERR_INVALID, "ws is not 16-byte aligned");
    if (ws_bytes < need)
      return fail(NC_ERR_INVALID, "workspace of %zu bytes is below the required %zu", ws_bytes, need);
  }
  hipError_t e = nc::launch_attn_decode_shared(q, k_new, v_new, k_prompt, v_prompt, Lp, k_cache,
                                               v_cache, seqlens, o, B, Tgen, H, Hkv, D, window,
                                               rope_base, to_dt(dt), ws, (hipStream_t)stream,
                                               ve_new, ve_gate);
  if (e != hipSuccess) return hip_fail(e, "attn_decode_shared launch");
  return ok();
}

}  // extern "C"
