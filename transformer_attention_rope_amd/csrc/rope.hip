// RoPE + parameter-free QK RMSNorm kernels for gfx950.
//
// What is computed ("从文本到聊天模型" (onehacker.top) §5.6: q and k are rotated
// by position; "Nanochat与nanoGPT对比：关键升级" (lzwjava.github.io) §1 table:
// RMSNorm without learnable parameters applied to q and k after RoPE):
//   x'[2i]   = x[2i] cos(p th_i) - x[2i+1] sin(p th_i)
//   x'[2i+1] = x[2i] sin(p th_i) + x[2i+1] cos(p th_i),  th_i = base^(-2i/D)
//   y = x' / sqrt(mean(x'^2) + 1e-6)
// Angles are formed and reduced in fp64 so that large positions keep full
// fp32 accuracy in cos/sin; the rotation and the norm run in fp32.
#include "device_common.hpp"
#include "launch.hpp"

#include <algorithm>
#include <cmath>

namespace nc {

// ------------------------------------------------------- attention prep
// Input stage of the prefill forward: k' = RMSNorm(RoPE(k)) for every key row,
// written once (the attention kernel revisits each key tile for several query
// tiles and only copies it), and the (cos, sin) table of every position for
// the rotation of q rows:
//   tabq[t][i] = (cos, sin)(p * theta_i),  p = pos_offset + t,  i < D/2,
// as two fp16 halves of one 32-bit word for bf16 rows (round to nearest:
// at most 2^-11 relative, a quarter of the bf16 rounding of the rotated q),
// as two fp32 values for fp32 rows.
// One workgroup per (position t, block of RB key rows of that position), where
// the rows of a position are its B*Hkv (sequence, head) pairs and RB rows hold
// 256*PREP_CPT 16-byte chunks. Each thread issues its (up to PREP_CPT) loads
// first; meanwhile the first D/2 threads form the position's angles in fp64
// (theta_i = base^(-2i/D) as exp2(-(2i/D) log2 base), then a two-constant
// Cody-Waite reduction modulo 2*pi) and evaluate them with sincosf on
// [-pi, pi]. The rotation and the norm of the rows run in fp32; the CPR
// 16-byte chunks of a row sit in consecutive lanes and reduce their sum of
// squares across lanes. k' keeps k's layout (B, T, Hkv, D) and element type.
// With CACHE the k' rows go to rows row0 + t of a (B, Tk, Hkv, D) cache
// instead, and the v rows of the same (sequence, position, head) are copied
// to the same rows of the value cache, so the chunk's keys and values are in
// the cache before the attention kernel reads them there. With ve non-null
// the value rows written are v' = v + gate * ve (value embedding; one gate
// per row, i.e. per (sequence, position, head)), formed in fp32 and rounded
// once to the element type.
// Where a position's rows fill at most half a workgroup (the d12 layer: 48 k
// rows of 16 chunks against 96 per workgroup), one workgroup takes pp
// consecutive positions whole, so the angle computation and the barrier are
// paid once per pp positions.
// (cos, sin) of p * theta_i, theta_i = base^(-2i/D): the angle is formed in
// fp64 (theta as exp2(-(2i/D) log2 base)), reduced modulo 2*pi with a
// two-constant Cody-Waite step, and evaluated with sincosf on [-pi, pi].
__device__ __forceinline__ float2 rope_cs_theta(long long p, double theta) {
  const double a = (double)p * theta;
  const double kq = rint(a * 0.15915494309189535);  // a / (2 pi)
  double r = fma(-kq, 6.283185307179586, a);        // 2 pi, high part
  r = fma(-kq, 2.4492935982947064e-16, r);          // 2 pi, low part
  float sn, c;
  sincosf((float)r, &sn, &c);
  return make_float2(c, sn);
}
__device__ __forceinline__ float2 rope_cs(long long p, int i, int D, double log2_base) {
  return rope_cs_theta(p, exp2(-(double)i / (D / 2) * log2_base));
}

constexpr int PREP_CPT = 6;  // 16-byte chunks per thread
constexpr int PREP_MAXPP = 8;  // positions per workgroup at most

template <int D, typename Elem, int CPT = PREP_CPT>
constexpr int prep_rows_per_block() {
  return 256 * CPT / (D / (sizeof(Elem) == 2 ? 8 : 4));
}
constexpr int ROPE_CPT = 6;  // chunks per thread of rope_qknorm_kernel (96 d12 rows per workgroup)

template <int D, typename Elem, bool CACHE>
__global__ void __launch_bounds__(256) attn_prep_kernel(const Elem* __restrict__ k,
                                                         Elem* __restrict__ kp,
                                                         void* __restrict__ tabq, int T,
                                                         int Hkv, int rows, double log2_base,
                                                         int pos_offset, int nrb, int pp,
                                                         const Elem* __restrict__ v,
                                                         Elem* __restrict__ vc, int Tk, int row0,
                                                         const Elem* __restrict__ ve,
                                                         const Elem* __restrict__ vgate) {
  constexpr bool kBf = sizeof(Elem) == 2;
  constexpr int EPC = kBf ? 8 : 4;  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;      // chunks per row
  constexpr int RB = prep_rows_per_block<D, Elem>();
  static_assert(64 % CPR == 0, "a row's chunks stay inside one wave");
  __shared__ float2 cs[PREP_MAXPP][D / 2];

  // positions t0 .. t0+npos-1 whole (pp > 1), or rows r0 .. r0+RB-1 of position t0
  const int t0 = pp > 1 ? (int)blockIdx.x * pp : (int)blockIdx.x / nrb;
  const int r0 = pp > 1 ? 0 : ((int)blockIdx.x - t0 * nrb) * RB;
  const int npos = pp > 1 ? min(pp, T - t0) : 1;
  const int total = (pp > 1 ? npos * rows : min(RB, rows - r0)) * CPR;  // whole rows only
  const int tid = threadIdx.x;

  u32x4_t w[PREP_CPT];
  u32x4_t wv[CACHE ? PREP_CPT : 1];
  u32x4_t wve[CACHE ? PREP_CPT : 1];
  float gt[CACHE ? PREP_CPT : 1];
  size_t off[PREP_CPT];   // element offset of the chunk in k (and v)
  size_t doff[PREP_CPT];  // and in the destination of k'
  int tls[PREP_CPT];      // the chunk's position, t0 + tls
#pragma unroll
  for (int p = 0; p < PREP_CPT; ++p) {
    const int ci = p * 256 + tid;
    const int lr = ci / CPR;  // row within the workgroup
    const int tl = pp > 1 ? lr / rows : 0;
    const int row = pp > 1 ? lr - tl * rows : r0 + lr;
    const int t = t0 + tl;
    tls[p] = ci < total ? tl : 0;  // idle chunks still read a (valid) table row
    const int cc = ci % CPR;
    const int bb = row / Hkv, g = row - bb * Hkv;
    off[p] = (((size_t)bb * T + t) * Hkv + g) * D + (size_t)cc * EPC;
    doff[p] = CACHE ? (((size_t)bb * Tk + row0 + t) * Hkv + g) * D + (size_t)cc * EPC : off[p];
    if (ci < total) {
      w[p] = ld16_nt(k + off[p]);
      if constexpr (CACHE) {
        wv[p] = ld16_nt(v + off[p]);
        if (ve != nullptr) {
          wve[p] = ld16_nt(ve + off[p]);
          const Elem gr = vgate[((size_t)bb * T + t) * Hkv + g];
          if constexpr (kBf) gt[p] = __uint_as_float((uint32_t)gr << 16);
          else gt[p] = gr;
        }
      }
    }
  }

  for (int idx = tid; idx < npos * (D / 2); idx += 256) {
    const int tl = idx / (D / 2), i = idx - tl * (D / 2);
    const int t = t0 + tl;
    const float2 csv = rope_cs((long long)pos_offset + t, i, D, log2_base);
    const float c = csv.x, sn = csv.y;
    cs[tl][i] = csv;
    if (r0 == 0) {
      if constexpr (kBf)
        reinterpret_cast<uint32_t*>(tabq)[(size_t)t * (D / 2) + i] = pack_h2(c, sn);
      else
        reinterpret_cast<float2*>(tabq)[(size_t)t * (D / 2) + i] = make_float2(c, sn);
    }
  }
  __syncthreads();

#pragma unroll
  for (int p = 0; p < PREP_CPT; ++p) {
    const int ci = p * 256 + tid;
    if (p * 256 >= total) break;  // uniform across the workgroup
    const bool ok = ci < total;   // uniform across the CPR lanes of a row
    const int cc = ci % CPR;
    float x[EPC];
    if constexpr (kBf) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        x[2 * m] = ok ? bf_lo(w[p][m]) : 0.f;
        x[2 * m + 1] = ok ? bf_hi(w[p][m]) : 0.f;
      }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) x[m] = ok ? __uint_as_float(w[p][m]) : 0.f;
    }
    float ss = 0.f;
#pragma unroll
    for (int m = 0; m < EPC / 2; ++m) {
      const float2 r = cs[tls[p]][cc * (EPC / 2) + m];
      const float xe = x[2 * m], xo = x[2 * m + 1];
      const float ye = xe * r.x - xo * r.y;
      const float yo = xe * r.y + xo * r.x;
      x[2 * m] = ye;
      x[2 * m + 1] = yo;
      ss += ye * ye + yo * yo;
    }
    ss = group_sum<CPR>(ss);
    const float inv = 1.0f / sqrtf(ss * (1.0f / D) + kEps);
    if (ok) {
      u32x4_t o;
      if constexpr (kBf) {
#pragma unroll
        for (int m = 0; m < 4; ++m) o[m] = pack_bf2(x[2 * m] * inv, x[2 * m + 1] * inv);
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) o[m] = __float_as_uint(x[m] * inv);
      }
      // a plain store: k' is read again at once by the attention kernel, and
      // the last-level cache then serves it (the d12 step 69.0 -> 66.8 us
      // against the non-temporal store)
      st16(kp + doff[p], o);
      if constexpr (CACHE) {
        u32x4_t vo = wv[p];
        if (ve != nullptr) {
          const float gg = gt[p];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            if constexpr (kBf)
              vo[m] = pack_bf2(bf_lo(wv[p][m]) + gg * bf_lo(wve[p][m]), bf_hi(wv[p][m]) + gg * bf_hi(wve[p][m]));
            else
              vo[m] = __float_as_uint(__uint_as_float(wv[p][m]) + gg * __uint_as_float(wve[p][m]));
          }
        }
        st16_nt(vc + doff[p], vo);
      }
    }
  }
}

size_t attn_prep_table_bytes(int T, int D, Dtype dt) {
  return (size_t)T * (size_t)(D / 2) * (dt == kF32 ? sizeof(float2) : sizeof(uint32_t));
}
size_t attn_prep_k_bytes(int B, int T, int Hkv, int D, Dtype dt) {
  return (size_t)B * T * Hkv * D * (dt == kF32 ? 4 : 2);
}

template <int D, typename Elem>
static hipError_t attn_prep_launch(const void* k, void* kp, void* tabq, int B, int T, int Hkv,
                                   double rope_base, int pos_offset, const void* v, void* vc,
                                   int Tk, int row0, const void* ve, const void* vgate,
                                   hipStream_t stream) {
  constexpr int RB = prep_rows_per_block<D, Elem>();
  const long long rows = (long long)B * Hkv;
  if (rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int pp = 2 * rows <= RB ? (int)std::min<long long>(PREP_MAXPP, RB / rows) : 1;
  const int nrb = pp > 1 ? 1 : (int)((rows + RB - 1) / RB);
  const long long nblk = pp > 1 ? ((long long)T + pp - 1) / pp : (long long)T * nrb;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (vc != nullptr)
    hipLaunchKernelGGL((attn_prep_kernel<D, Elem, true>), dim3((unsigned)nblk), dim3(256), 0,
                       stream, (const Elem*)k, (Elem*)kp, tabq, T, Hkv, (int)rows,
                       std::log2(rope_base), pos_offset, nrb, pp, (const Elem*)v, (Elem*)vc, Tk, row0,
                       (const Elem*)ve, (const Elem*)vgate);
  else
    hipLaunchKernelGGL((attn_prep_kernel<D, Elem, false>), dim3((unsigned)nblk), dim3(256), 0,
                       stream, (const Elem*)k, (Elem*)kp, tabq, T, Hkv, (int)rows,
                       std::log2(rope_base), pos_offset, nrb, pp, (const Elem*)nullptr,
                       (Elem*)nullptr, T, 0, (const Elem*)nullptr, (const Elem*)nullptr);
  return hipGetLastError();
}

template <int D>
static hipError_t attn_prep_d(const void* k, void* kp, void* tabq, int B, int T, int Hkv,
                              double rope_base, int pos_offset, const void* v, void* vc, int Tk,
                              int row0, const void* ve, const void* vgate, Dtype dt,
                              hipStream_t stream) {
  if (dt == kBF16)
    return attn_prep_launch<D, uint16_t>(k, kp, tabq, B, T, Hkv, rope_base, pos_offset, v, vc, Tk,
                                         row0, ve, vgate, stream);
  return attn_prep_launch<D, float>(k, kp, tabq, B, T, Hkv, rope_base, pos_offset, v, vc, Tk, row0,
                                    ve, vgate, stream);
}

hipError_t launch_attn_prep(const void* k, void* kp, void* tabq, int B, int T, int Hkv, int D,
                            double rope_base, int pos_offset, const void* v, void* vc, int Tk,
                            int row0, const void* ve, const void* vgate, Dtype dt,
                            hipStream_t stream) {
  switch (D) {
    case 32: return attn_prep_d<32>(k, kp, tabq, B, T, Hkv, rope_base, pos_offset, v, vc, Tk, row0, ve, vgate, dt, stream);
    case 64: return attn_prep_d<64>(k, kp, tabq, B, T, Hkv, rope_base, pos_offset, v, vc, Tk, row0, ve, vgate, dt, stream);
    case 128: return attn_prep_d<128>(k, kp, tabq, B, T, Hkv, rope_base, pos_offset, v, vc, Tk, row0, ve, vgate, dt, stream);
    default: return hipErrorInvalidValue;
  }
}

// --------------------------------------------------------- rope + qknorm
// Same structure as the input stage above. One workgroup per (position t,
// block of RB rows of that position), where the rows of a position are its
// B*(H + Hkv) (sequence, q head or k head) pairs. Each thread issues its (up
// to ROPE_CPT) 16-byte loads first; meanwhile the first D/2 threads form the
// angles (fp64, exp2 of the scaled log2 base, two-constant Cody-Waite
// reduction modulo 2*pi, sincosf on [-pi, pi]). The CPR chunks of a row sit
// in consecutive lanes and reduce their sum of squares across lanes.
// In-place use (out == in) is safe: each thread writes back exactly the
// chunks it read.
template <int D, typename Elem>
__global__ void __launch_bounds__(256) rope_qknorm_kernel(const Elem* q, const Elem* k,  // may alias
                                                           Elem* q_out, Elem* k_out, int T, int H,
                                                           int Hkv, int rows, double log2_base,
                                                           int pos_offset, int nrb) {
  constexpr bool kBf = sizeof(Elem) == 2;
  constexpr int EPC = kBf ? 8 : 4;  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;      // chunks per row
  constexpr int RB = prep_rows_per_block<D, Elem, ROPE_CPT>();
  static_assert(64 % CPR == 0, "a row's chunks stay inside one wave");
  __shared__ float2 cs[D / 2];

  const int t = (int)blockIdx.x / nrb;
  const int r0 = ((int)blockIdx.x - t * nrb) * RB;
  const int total = min(RB, rows - r0) * CPR;  // whole rows only
  const int tid = threadIdx.x;
  const int R = H + Hkv;

  u32x4_t w[ROPE_CPT];
  size_t off[ROPE_CPT];
  bool isq[ROPE_CPT];
#pragma unroll
  for (int p = 0; p < ROPE_CPT; ++p) {
    const int ci = p * 256 + tid;
    const int row = r0 + ci / CPR;
    const int cc = ci % CPR;
    const int bb = row / R, rr = row - bb * R;
    isq[p] = rr < H;
    off[p] = isq[p] ? (((size_t)bb * T + t) * H + rr) * D + (size_t)cc * EPC
                    : (((size_t)bb * T + t) * Hkv + (rr - H)) * D + (size_t)cc * EPC;
    if (ci < total) w[p] = ld16(isq[p] ? q + off[p] : k + off[p]);
  }

  if (tid < D / 2) cs[tid] = rope_cs((long long)pos_offset + t, tid, D, log2_base);
  __syncthreads();

#pragma unroll
  for (int p = 0; p < ROPE_CPT; ++p) {
    const int ci = p * 256 + tid;
    if (p * 256 >= total) break;  // uniform across the workgroup
    const bool ok = ci < total;   // uniform across the CPR lanes of a row
    const int cc = ci % CPR;
    float x[EPC];
    if constexpr (kBf) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        x[2 * m] = ok ? bf_lo(w[p][m]) : 0.f;
        x[2 * m + 1] = ok ? bf_hi(w[p][m]) : 0.f;
      }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) x[m] = ok ? __uint_as_float(w[p][m]) : 0.f;
    }
    float ss = 0.f;
#pragma unroll
    for (int m = 0; m < EPC / 2; ++m) {
      const float2 r = cs[cc * (EPC / 2) + m];
      const float xe = x[2 * m], xo = x[2 * m + 1];
      const float ye = xe * r.x - xo * r.y;
      const float yo = xe * r.y + xo * r.x;
      x[2 * m] = ye;
      x[2 * m + 1] = yo;
      ss += ye * ye + yo * yo;
    }
    ss = group_sum<CPR>(ss);
    const float inv = 1.0f / sqrtf(ss * (1.0f / D) + kEps);
    if (ok) {
      u32x4_t o;
      if constexpr (kBf) {
#pragma unroll
        for (int m = 0; m < 4; ++m) o[m] = pack_bf2(x[2 * m] * inv, x[2 * m + 1] * inv);
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) o[m] = __float_as_uint(x[m] * inv);
      }
      st16_nt(isq[p] ? q_out + off[p] : k_out + off[p], o);
    }
  }
}

template <int D, typename Elem>
static hipError_t rope_qknorm_launch(const void* q, const void* k, void* q_out, void* k_out, int B,
                                     int T, int H, int Hkv, double rope_base, int pos_offset,
                                     hipStream_t stream) {
  constexpr int RB = prep_rows_per_block<D, Elem, ROPE_CPT>();
  const long long rows = (long long)B * (H + Hkv);
  if (rows > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int nrb = (int)((rows + RB - 1) / RB);
  const long long nblk = (long long)T * nrb;
  if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((rope_qknorm_kernel<D, Elem>), dim3((unsigned)nblk), dim3(256), 0, stream,
                     (const Elem*)q, (const Elem*)k, (Elem*)q_out, (Elem*)k_out, T, H, Hkv,
                     (int)rows, std::log2(rope_base), pos_offset, nrb);
  return hipGetLastError();
}

template <int D>
static hipError_t rope_qknorm_d(const void* q, const void* k, void* q_out, void* k_out, int B,
                                int T, int H, int Hkv, double rope_base, int pos_offset, Dtype dt,
                                hipStream_t stream) {
  if (dt == kBF16)
    return rope_qknorm_launch<D, uint16_t>(q, k, q_out, k_out, B, T, H, Hkv, rope_base, pos_offset,
                                           stream);
  return rope_qknorm_launch<D, float>(q, k, q_out, k_out, B, T, H, Hkv, rope_base, pos_offset,
                                      stream);
}

// The (cos, sin) table alone: tab[t][i] of positions pos_offset + t, t < T,
// i < D/2, fp16 pairs in 32 bits (bf16) or float2 (fp32), as the input stage
// writes it. A thread takes one frequency i and kTabPos consecutive
// positions, so theta_i (an fp64 exp2) is formed once per kTabPos entries;
// the lanes of a wave write consecutive i of one position.
constexpr int kTabPos = 8;
template <bool kBf>
__global__ void __launch_bounds__(256) rope_table_kernel(void* __restrict__ tab, int T, int D,
                                                          double log2_base, int pos_offset) {
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;
  const int half = D / 2;
  if (idx >= (long long)((T + kTabPos - 1) / kTabPos) * half) return;
  const int i = (int)(idx % half), t0 = (int)(idx / half) * kTabPos;
  const double theta = exp2(-(double)i / half * log2_base);
  for (int t = t0; t < min(T, t0 + kTabPos); ++t) {
    const float2 c = rope_cs_theta((long long)pos_offset + t, theta);
    if constexpr (kBf) reinterpret_cast<uint32_t*>(tab)[(size_t)t * half + i] = pack_h2(c.x, c.y);
    else reinterpret_cast<float2*>(tab)[(size_t)t * half + i] = c;
  }
}

hipError_t launch_rope_table(void* tab, int T, int D, double rope_base, int pos_offset, Dtype dt,
                             hipStream_t stream) {
  const long long n = (long long)((T + kTabPos - 1) / kTabPos) * (D / 2);
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (dt == kBF16)
    hipLaunchKernelGGL(rope_table_kernel<true>, dim3(grid), dim3(256), 0, stream, tab, T, D,
                       std::log2(rope_base), pos_offset);
  else
    hipLaunchKernelGGL(rope_table_kernel<false>, dim3(grid), dim3(256), 0, stream, tab, T, D,
                       std::log2(rope_base), pos_offset);
  return hipGetLastError();
}

hipError_t launch_rope_qknorm(const void* q, const void* k, void* q_out, void* k_out, int B,
                              int T, int H, int Hkv, int D, double rope_base, int pos_offset,
                              Dtype dt, hipStream_t stream) {
  switch (D) {
    case 32: return rope_qknorm_d<32>(q, k, q_out, k_out, B, T, H, Hkv, rope_base, pos_offset, dt, stream);
    case 64: return rope_qknorm_d<64>(q, k, q_out, k_out, B, T, H, Hkv, rope_base, pos_offset, dt, stream);
    case 128: return rope_qknorm_d<128>(q, k, q_out, k_out, B, T, H, Hkv, rope_base, pos_offset, dt, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nc
