// Attention backward for gfx950: gradients of the block forward (RoPE, then
// parameter-free RMSNorm on q and k, then GQA softmax attention over the
// causal sliding-window band) with respect to the RAW q, k, v, given dO and
// the forward's row log-sum-exp.
//
// A training step runs the forward, backpropagates the loss and steps the
// optimizer ("从文本到聊天模型" (onehacker.top), §6.5); the attention kernel
// that serves training does both passes ("Nanochat与nanoGPT对比：关键升级"
// (lzwjava.github.io), §1 table, Flash Attention row). The pages give no
// backward formulas; this is the chain rule through the forward of §5.4-5.6
// and the §1 table (QK-norm after RoPE, GQA, window):
//   P = exp(q'k'^T/sqrt(D) - lse) on the band,  Delta_i = dO_i . o_i,
//   dV_g += P^T dO,  dP = dO V^T,  dS = P (dP - Delta),
//   dq' = dS k'/sqrt(D),  dk'_g += dS^T q'/sqrt(D),
//   RMSNorm y = x r:  dx = r (dy - y mean(dy y));  RoPE: rotate back by -p theta.
//
// Design (bf16 path):
//  * A prep pass forms, once per row, what the two main kernels stream:
//    q's = q' log2(e)/sqrt(D) in bf16 (row-major, the same rounding as the
//    forward's q operand), transposed copies of q's, dO and k' ([d][t]
//    tiles of 32 positions, permuted within 16 so that one 16-byte read is
//    the MFMA operand matching the order in which a score accumulator hands
//    over its rows), Delta = dO.o and lse*log2(e) per row. k' and the
//    (cos, sin) table come from the forward's input stage (attn_prep_kernel).
//  * Kernel A (dK, dV): a workgroup owns 128 keys of one (sequence, K/V
//    head), 32 per wave, K' and V held in registers as MFMA B operands, and
//    walks the 32-position query tiles of every query head of the group that
//    can see its keys. Per tile and wave: S = Q K'^T and dP = dO V^T (the
//    lane holds one key, 16 queries), P and dS in registers, then
//    dV^T += dO^T P and dK^T += Q^T dS with the transposed tiles as A
//    operands. dK and dV sum over the group's heads in registers: no atomics.
//  * Kernel B (dQ): a workgroup owns 128 positions of one query head, q's
//    and dO held as B operands, and walks the 32-key tiles of its band:
//    S^T = K' Q^T and dP^T = V dO^T (the lane holds one query), then
//    dQ^T += K'^T dS^T with the transposed k' tile as A operand.
//  * Tiles move from memory to LDS with 16-byte buffer-to-LDS copies (no
//    registers), double-buffered, one barrier per tile; row tiles are XOR-
//    swizzled so the row-strided fragment reads spread over all LDS banks.
//  * Both epilogues finish the chain in registers: a lane holds half of one
//    key's (query's) row, so the RMSNorm backward needs one cross-lane sum,
//    and the RoPE backward rotates the in-lane pairs back.
//
// fp32 path: exact fp32 arithmetic on the vector ALUs, one thread per key
// row (dK, dV) or query row (dQ), not a performance path.
#include <utility>

#include "device_common.hpp"
#include "launch.hpp"

namespace nc {

struct BwdArgs {
  const void* q;        // raw q (B, T, H, D)
  const void* k;        // raw k (B, T, Hkv, D)
  const void* v;        // (B, T, Hkv, D)
  const void* o;        // forward output (B, T, H, D)
  const void* dout;     // dL/do (B, T, H, D)
  const float* lse;     // forward row log-sum-exp (B, T, H)
  const void* tab;      // (cos, sin) of positions pos_offset + t: [T][D/2]
  const void* kp;       // k' = norm(rope(k)) (B, T, Hkv, D)
  uint16_t* kpt;        // bf16: k'^T tiles [B][Hkv][D][Tp], positions permuted
  void* qs;             // bf16: q' log2e/sqrt(D) (B, T, H, D); fp32: q' (B, T, H, D)
  uint16_t* qst;        // bf16: q's^T [B][H][D][Tp]
  uint16_t* dot;        // bf16: dO^T [B][H][D][Tp]
  float* stats;         // per (b, h, 32-position tile) 64 floats: lse * log2(e) of
                        // the 32 positions (+inf past T), then dO . o (0 past T)
  void* dq;             // outputs, raw-input gradients, the inputs' type
  void* dk;
  void* dv;
  int B, T, H, Hkv, G, W, Tp;
  float qscale;         // log2(e) / sqrt(D)
};

// Position held by slot s (0..31) of a transposed tile. The accumulator of
// v_mfma_f32_32x32x16_bf16 gives lane-half hf of k-step s2 the rows
// 16 s2 + 4 hf + {0,1,2,3, 8,9,10,11}; slots 16 s2 + 8 hf .. + 7 hold those
// 8 positions in that order, so the matching operand is one 16-byte read.
__device__ __forceinline__ int tr_pos(int s) {
  return (s & 16) | (((s >> 3) & 1) << 2) | (((s >> 2) & 1) << 3) | (s & 3);
}

template <int D>
struct BwCfg {
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int KS = D / 16;                  // MFMA k-steps over D
  static constexpr int DB = D / 32;                  // 32-row blocks of D
  static constexpr int KSW = D >= 128 ? 1 : 128 / D; // rows per 256-byte bank span
  static constexpr int ROWT = 32 * D;                // bf16 elements of a 32-row tile
  static constexpr int TRT = D * 32;                 // bf16 elements of a transposed tile
  static constexpr int RCOPY = 32 * CPR / 64;        // 1 KB copies per row tile
  static constexpr int TCOPY = D * 4 / 64;           // 1 KB copies per transposed tile
};

// LDS chunk of logical chunk c of row r in a swizzled row tile, and of
// logical chunk c of row d in a transposed tile (4 chunks per row).
template <int D>
__device__ __forceinline__ int row_chunk(int r, int c) {
  using C = BwCfg<D>;
  return r * C::CPR + (c ^ ((r / C::KSW) % C::CPR));
}
__device__ __forceinline__ int tr_chunk(int d, int c) { return d * 4 + (c ^ ((d >> 2) & 3)); }

__device__ __forceinline__ void wg_sync() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0): this wave's copies have landed
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// The RMSNorm and RoPE backward of one row held by a lane pair (lanes n and
// n + 32): g[db][r] is the gradient with respect to the normalised row at
// dims 32 db + 8 (r / 4) + 4 hf + r % 4; xrow is the raw row (bf16), tab the
// position's (cos, sin) fp16 pairs. Writes the raw-input gradient (bf16).
template <int D>
__device__ __forceinline__ void norm_rope_bwd_store(float (&g)[D / 32][16], const uint16_t* xrow,
                                                    const uint32_t* tab, uint16_t* out, int hf,
                                                    bool valid) {
  constexpr int DB = D / 32;
  float x[DB][16];
  float ss = 0.f;
  uint32_t cs[DB][4][2];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = db * 32 + 8 * r4 + 4 * hf;
      const u32x2_t w = valid ? *reinterpret_cast<const u32x2_t*>(xrow + d) : u32x2_t{0u, 0u};
      const u32x2_t t = valid ? *reinterpret_cast<const u32x2_t*>(tab + d / 2) : u32x2_t{0u, 0u};
      cs[db][r4][0] = t[0];
      cs[db][r4][1] = t[1];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const float xe = bf_lo(w[m]), xo = bf_hi(w[m]);
        const float c = h_lo(t[m]), s = h_hi(t[m]);
        const float ye = xe * c - xo * s, yo = xe * s + xo * c;
        x[db][4 * r4 + 2 * m] = ye;
        x[db][4 * r4 + 2 * m + 1] = yo;
        ss += ye * ye + yo * yo;
      }
    }
  ss = sum_halves(ss);
  const float rn = rsq(ss * (1.0f / D) + kEps);
  float dot = 0.f;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dot += g[db][r] * x[db][r];
  dot = sum_halves(dot) * rn;  // sum of g * y, y = x rn
  const float proj = dot * (1.0f / D) * rn;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      uint32_t w[2];
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const int i = 4 * r4 + 2 * m;
        // dx = rn (g - y mean(g y)) = rn g - x rn^2 mean(g y)
        const float de = rn * g[db][i] - proj * rn * x[db][i];
        const float dd = rn * g[db][i + 1] - proj * rn * x[db][i + 1];
        const float c = h_lo(cs[db][r4][m]), s = h_hi(cs[db][r4][m]);
        w[m] = pack_bf2(de * c + dd * s, -de * s + dd * c);
      }
      if (valid) st8(out + db * 32 + 8 * r4 + 4 * hf, u32x2_t{w[0], w[1]});
    }
}

// =====================================================================
// prep (bf16): q side per (b, h, 32 positions), k side per (b, g, 32 keys)
// =====================================================================
template <int D>
__global__ void __launch_bounds__(256) attn_bwd_prep_bf16_kernel(BwdArgs p) {
  using C = BwCfg<D>;
  constexpr int LD = D + 8;  // LDS row stride (bf16)
  __shared__ __attribute__((aligned(16))) uint16_t t0s[32 * LD];
  __shared__ __attribute__((aligned(16))) uint16_t t1s[32 * LD];
  const int tid = threadIdx.x;
  const int ntile = p.Tp / 32;
  const int nq = p.B * p.H * ntile;
  int blk = blockIdx.x;
  const bool qside = blk < nq;
  if (!qside) blk -= nq;
  const int tile = blk % ntile;
  const int bh = blk / ntile;          // b * H + h, or b * Hkv + g
  const int nh = qside ? p.H : p.Hkv;
  const int b = bh / nh, h = bh % nh;
  const int t0 = tile * 32;

  const uint16_t* src = (const uint16_t*)(qside ? p.q : p.kp);
  const uint32_t* tab = (const uint32_t*)p.tab;
#pragma unroll
  for (int pass = 0; pass < (32 * C::CPR + 255) / 256; ++pass) {
    const int e = pass * 256 + tid;
    if (e >= 32 * C::CPR) break;  // (D = 32: waves 2 and 3 idle, whole rows per wave)
    const int r = e / C::CPR, c = e % C::CPR;
    const int t = t0 + r;
    const bool valid = t < p.T;
    const size_t row = ((size_t)b * p.T + t) * nh + h;
    if (qside) {
      u32x4_t qw = valid ? ld16((const uint16_t*)p.q + row * D + c * 8) : u32x4_t{0u, 0u, 0u, 0u};
      u32x4_t tq = valid ? ld16(tab + (size_t)t * (D / 2) + c * 4) : u32x4_t{0u, 0u, 0u, 0u};
      u32x4_t dw = valid ? ld16((const uint16_t*)p.dout + row * D + c * 8) : u32x4_t{0u, 0u, 0u, 0u};
      u32x4_t ow = valid ? ld16((const uint16_t*)p.o + row * D + c * 8) : u32x4_t{0u, 0u, 0u, 0u};
      float xr[8];
      float ss = 0.f, dl = 0.f;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float xe = bf_lo(qw[m]), xo = bf_hi(qw[m]);
        const float cc = h_lo(tq[m]), sn = h_hi(tq[m]);
        const float ye = xe * cc - xo * sn, yo = xe * sn + xo * cc;
        xr[2 * m] = ye;
        xr[2 * m + 1] = yo;
        ss += ye * ye + yo * yo;
        dl += bf_lo(dw[m]) * bf_lo(ow[m]) + bf_hi(dw[m]) * bf_hi(ow[m]);
      }
      ss = dpp_group_sum<C::CPR>(ss);
      dl = dpp_group_sum<C::CPR>(dl);
      const float sc = p.qscale * rsq(ss * (1.0f / D) + kEps);
      u32x4_t w;
#pragma unroll
      for (int m = 0; m < 4; ++m) w[m] = pack_bf2(xr[2 * m] * sc, xr[2 * m + 1] * sc);
      if (valid) st16((uint16_t*)p.qs + row * D + c * 8, w);
      st16(t0s + r * LD + c * 8, w);
      st16(t1s + r * LD + c * 8, dw);
      if (c == 0) {
        float* st = p.stats + ((size_t)bh * ntile + tile) * 64;
        st[r] = valid ? p.lse[row] * kLog2e : __builtin_inff();
        st[32 + r] = valid ? dl : 0.f;
      }
    } else {
      u32x4_t kw = valid ? ld16(src + row * D + c * 8) : u32x4_t{0u, 0u, 0u, 0u};
      st16(t0s + r * LD + c * 8, kw);
    }
  }
  __syncthreads();
  // transposed tiles: row d holds the 32 positions in slot order
  const int ntr = qside ? 2 : 1;
  for (int which = 0; which < ntr; ++which) {
    const uint16_t* ts = which == 0 ? t0s : t1s;
    uint16_t* dst = qside ? (which == 0 ? p.qst : p.dot) : p.kpt;
#pragma unroll
    for (int pass = 0; pass < (D * 4 + 255) / 256; ++pass) {
      const int e = pass * 256 + tid;
      if (e >= D * 4) break;
      const int d = e >> 2, j = e & 3;
      uint32_t w[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int pa = tr_pos(8 * j + 2 * m), pb = tr_pos(8 * j + 2 * m + 1);
        w[m] = (uint32_t)ts[pa * LD + d] | ((uint32_t)ts[pb * LD + d] << 16);
      }
      st16(dst + ((size_t)bh * D + d) * p.Tp + t0 + 8 * j, u32x4_t{w[0], w[1], w[2], w[3]});
    }
  }
}

// Calls f(std::integral_constant<int, i>) for i = 0 .. N-1, expanded at
// compile time.
template <typename F, int... I>
__device__ __forceinline__ void bw_static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void bw_static_for(F&& f) {
  bw_static_for_impl(f, std::make_integer_sequence<int, N>{});
}
template <int I>
using bw_ic = std::integral_constant<int, I>;

// =====================================================================
// kernel A (bf16): dK, dV per (b, g, 128 keys)
// =====================================================================
// A step covers 64 query positions of one head as two 32-position sub-tiles,
// whose score products are issued before either softmax: one sub-tile's
// vector work then runs under the other's MFMAs (one wave per SIMD at
// D = 128 leaves nothing else to hide it).
template <int D>
struct BwACfg {
  using C = BwCfg<D>;
  static constexpr int ROWT = 64 * D;             // bf16 elements of a 64-row tile
  static constexpr int TRT = D * 64;              // of a transposed tile [D][64]
  static constexpr int RCOPY = 64 * C::CPR / 64;  // 1 KB copies per row tile
  static constexpr int TCOPY = D * 8 / 64;        // per transposed tile
  static constexpr int STAGE = 2 * ROWT + 2 * TRT + 512;  // + stats: 2 x (lse2[32], delta[32])
};
// LDS chunk of logical chunk c (0..7) of row d of a [D][64] transposed tile
__device__ __forceinline__ int tr64_chunk(int d, int c) { return d * 8 + (c ^ ((d >> 1) & 7)); }

template <int D>
__global__ void __launch_bounds__(256, D == 128 ? 1 : 2) attn_bwd_kv_bf16_kernel(BwdArgs p) {
  using C = BwCfg<D>;
  using A = BwACfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * A::STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hf = lane >> 5;

  const int per = p.B * p.Hkv;
  const int kb = (int)blockIdx.x / per;  // lower key blocks have more queries: first
  const int bg = (int)blockIdx.x % per;
  const int b = bg / p.Hkv, g = bg % p.Hkv;
  const int j0 = kb * 128 + wave * 32;  // this wave's first key
  const int key = j0 + n;

  // stationary K' and V fragments: B operand (col = key, k = dims 16 s + 8 hf ..)
  const uint32_t kvrow = (uint32_t)p.Hkv * D * 2;
  const size_t kv_base = ((size_t)b * p.T * p.Hkv + g) * D;
  const uint32_t kv_rec = (uint32_t)(((size_t)(p.T - 1) * p.Hkv) * D * 2 + D * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc((const uint16_t*)p.kp + kv_base, kv_rec);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc((const uint16_t*)p.v + kv_base, kv_rec);
  bf16x8_t kf[C::KS], vf[C::KS];
#pragma unroll
  for (int s = 0; s < C::KS; ++s) {
    const uint32_t off = (uint32_t)key * kvrow + (16 * s + 8 * hf) * 2;
    kf[s] = __builtin_bit_cast(bf16x8_t, bload16(rk, key < p.T ? off : 0xF0000000u, 0));
    vf[s] = __builtin_bit_cast(bf16x8_t, bload16(rv, key < p.T ? off : 0xF0000000u, 0));
  }

  f32x16_t dva[C::DB], dka[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dva[db][r] = 0.f;
      dka[db][r] = 0.f;
    }

  // query positions that see this workgroup's keys [kb*128, kb*128 + 127]:
  // from kb*128 (a multiple of 64) to min(T, kb*128 + 127 + W) - 1, in steps of 64
  const int q_lo = kb * 128;
  const int q_hi = min(p.T - 1, kb * 128 + 127 + p.W - 1);
  const int nq = (q_hi - q_lo) / 64 + 1;
  const int nsteps = p.G * nq;

  const uint32_t qrow = (uint32_t)p.H * D * 2;
  auto issue = [&](int step, int buf) __attribute__((always_inline)) {
    const int hh = g * p.G + step / nq;
    const int t0 = q_lo + (step % nq) * 64;
    uint16_t* st = smem + buf * A::STAGE;
    // row tiles: positions t0 .. t0 + 63 of head hh; past T reads zeros
    const size_t rbase = (((size_t)b * p.T + t0) * p.H + hh) * D;
    const uint32_t rrec = (uint32_t)((p.T - t0) * (size_t)qrow);
    const __amdgpu_buffer_rsrc_t rq = make_rsrc((const uint16_t*)p.qs + rbase, rrec);
    const __amdgpu_buffer_rsrc_t rd = make_rsrc((const uint16_t*)p.dout + rbase, rrec);
    // transposed tiles: t0 + 64 <= Tp (a multiple of 64), padded with zeros
    const size_t tbase = ((size_t)b * p.H + hh) * D * p.Tp + t0;
    const __amdgpu_buffer_rsrc_t rqt = make_rsrc(p.qst + tbase, 0x7fffffff);
    const __amdgpu_buffer_rsrc_t rdt = make_rsrc(p.dot + tbase, 0x7fffffff);
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(p.stats + (((size_t)b * p.H + hh) * (p.Tp / 32) + t0 / 32) * 64, 512);
    constexpr int NI = 2 * A::RCOPY + 2 * A::TCOPY + 1;
#pragma unroll
    for (int f = 0; f < NI; ++f) {
      if (f % 4 != wave) continue;
      if (f < 2 * A::RCOPY) {
        const int ff = f % A::RCOPY;
        const int e = ff * 64 + lane;
        const int r = e / C::CPR, c = e % C::CPR;
        const uint32_t off = (uint32_t)r * qrow + (uint32_t)((c ^ ((r / C::KSW) % C::CPR)) * 16);
        lds_copy16(f < A::RCOPY ? rq : rd, st + (f < A::RCOPY ? 0 : A::ROWT) + ff * 512, off);
      } else if (f < 2 * A::RCOPY + 2 * A::TCOPY) {
        const int f2 = f - 2 * A::RCOPY;
        const int ff = f2 % A::TCOPY;
        const int e = ff * 64 + lane;
        const int d = e >> 3, c = e & 7;
        const uint32_t off = (uint32_t)d * p.Tp * 2 + (uint32_t)((c ^ ((d >> 1) & 7)) * 16);
        lds_copy16(f2 < A::TCOPY ? rqt : rdt,
                   st + 2 * A::ROWT + (f2 < A::TCOPY ? 0 : A::TRT) + ff * 512, off);
      } else {
        // lanes 0..31: the 2 x 64 stats floats of the two sub-tiles; the rest read nothing
        lds_copy16(rs, st + 2 * A::ROWT + 2 * A::TRT, lane < 32 ? lane * 16 : 0xF0000000u);
      }
    }
  };

  // A-operand fragment reads: row tile (row 32 u + n) and transposed tile
  // (row 32 db + n, sub-tile u's slots 32 u + 16 s2 + 8 hf ..)
  auto rowfrag = [&](const uint16_t* t, int u, int s) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8_t*>(t + row_chunk<D>(32 * u + n, 2 * s + hf) * 8);
  };
  auto trfrag = [&](const uint16_t* t, int db, int u, int s2) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8_t*>(t + tr64_chunk(db * 32 + n, 4 * u + 2 * s2 + hf) * 8);
  };

  issue(0, 0);
  wg_sync();
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    if (step + 1 < nsteps) issue(step + 1, buf ^ 1);
    const int t0 = q_lo + (step % nq) * 64;
    const uint16_t* st = smem + buf * A::STAGE;
    const uint16_t* qt = st;
    const uint16_t* dt = st + A::ROWT;
    const uint16_t* qtt = st + 2 * A::ROWT;
    const uint16_t* dtt = st + 2 * A::ROWT + A::TRT;
    const float* stat = reinterpret_cast<const float*>(st + 2 * A::ROWT + 2 * A::TRT);
    // Every product runs on every step (a conditional update of the dK, dV
    // accumulators makes the compiler copy all of them between register
    // files); sub-tiles the wave cannot see are masked to zero below.
    //
    // The step is written out as its NM MFMAs in a fixed order, with a
    // scheduling barrier after each: the scores S, dP of sub-tile 0, those of
    // sub-tile 1, then dV, dK of sub-tile 0 and of sub-tile 1. MFMA m takes
    // fragment m, read from LDS LA MFMAs earlier, so no MFMA waits on its own
    // read. The softmax of sub-tile 0 (8 units) sits between the score MFMAs
    // of sub-tile 1, that of sub-tile 1 between the dV, dK MFMAs of sub-tile
    // 0: vector work that no nearby MFMA depends on, issued while the matrix
    // unit is busy.
    constexpr int NSU = 2 * C::KS;   // score MFMAs per sub-tile (S and dP per k-step)
    constexpr int NGU = 4 * C::DB;   // dV, dK MFMAs per sub-tile
    constexpr int NM = 2 * NSU + 2 * NGU;
    constexpr int LA = D == 128 ? 8 : 3;  // fragment look-ahead in MFMAs
    f32x4_t l2v[2][4], dlv[2][4];
    int lo[2];
    unsigned span[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      // register r holds query tq = t0 + 32 u + 8 (r / 4) + 4 hf + r % 4 against key `key`:
      // visible iff 0 <= tq - key < W and tq < T, i.e. e = 8 (r / 4) + r % 4 lies in
      // [key - base, min(key - base + W, T - base)), base = t0 + 32 u + 4 hf
      const int base = t0 + 32 * u + 4 * hf;
      lo[u] = key - base;
      const int hi = min(lo[u] + p.W, p.T - base);
      span[u] = hi > lo[u] ? (unsigned)(hi - lo[u]) : 0u;  // empty past T
    }
    // the sub-tile's lse and delta, read a few MFMAs before its softmax
    auto load_stats = [&](int u) __attribute__((always_inline)) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        l2v[u][r4] = *reinterpret_cast<const f32x4_t*>(stat + 64 * u + 8 * r4 + 4 * hf);
        dlv[u][r4] = *reinterpret_cast<const f32x4_t*>(stat + 64 * u + 32 + 8 * r4 + 4 * hf);
      }
    };
    f32x16_t sa[2], pa[2];
#pragma unroll
    for (int u = 0; u < 2; ++u)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sa[u][r] = 0.f;
        pa[u][r] = 0.f;
      }
    uint32_t pw[2][4][2], sw[2][4][2];
    // fragment of MFMA m
    auto frag = [&](auto mc) __attribute__((always_inline)) -> bf16x8_t {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < 2 * NSU) {
        constexpr int u = m / NSU, s = (m % NSU) / 2;
        return rowfrag((m & 1) ? dt : qt, u, s);
      } else {
        constexpr int mm = m - 2 * NSU, u = mm / NGU, r = mm % NGU;
        constexpr int s2 = r / (2 * C::DB), db = (r % (2 * C::DB)) / 2;
        return trfrag((r & 1) ? qtt : dtt, db, u, s2);
      }
    };
    auto mfma = [&](auto mc, const bf16x8_t& a) __attribute__((always_inline)) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m < 2 * NSU) {
        constexpr int u = m / NSU, s = (m % NSU) / 2;
        if constexpr (m & 1) pa[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[s], pa[u], 0, 0, 0);
        else sa[u] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[s], sa[u], 0, 0, 0);
      } else {
        constexpr int mm = m - 2 * NSU, u = mm / NGU, r = mm % NGU;
        constexpr int s2 = r / (2 * C::DB), db = (r % (2 * C::DB)) / 2;
        // k-step s2 of sub-tile u takes registers 8 s2 .. 8 s2 + 7
        if constexpr (r & 1) {
          const bf16x8_t bs = __builtin_bit_cast(
              bf16x8_t, u32x4_t{sw[u][2 * s2][0], sw[u][2 * s2][1], sw[u][2 * s2 + 1][0], sw[u][2 * s2 + 1][1]});
          dka[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bs, dka[db], 0, 0, 0);
        } else {
          const bf16x8_t bp = __builtin_bit_cast(
              bf16x8_t, u32x4_t{pw[u][2 * s2][0], pw[u][2 * s2][1], pw[u][2 * s2 + 1][0], pw[u][2 * s2 + 1][1]});
          dva[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bp, dva[db], 0, 0, 0);
        }
      }
    };
    // softmax unit k of sub-tile u: registers 4 r4 + 2 h, 4 r4 + 2 h + 1 (r4 = k / 2, h = k % 2)
    auto unit = [&](int u, int k) __attribute__((always_inline)) {
      const int r4 = k >> 1, h = k & 1;
      float pv[2], sv[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int i = 2 * h + j, r = 4 * r4 + i;
        const bool vis = (unsigned)(8 * r4 + i - lo[u]) < span[u];
        const float pr = vis ? fast_exp2(sa[u][r] - l2v[u][r4][i]) : 0.f;
        pv[j] = pr;
        sv[j] = pr * (pa[u][r] - dlv[u][r4][i]);
      }
      pw[u][r4][h] = pack_bf2(pv[0], pv[1]);
      sw[u][r4][h] = pack_bf2(sv[0], sv[1]);
    };
    bf16x8_t fr[NM];
    bw_static_for<LA>([&](auto jc) { fr[decltype(jc)::value] = frag(jc); });
    __builtin_amdgcn_sched_barrier(0);
    bw_static_for<NM>([&](auto mc) {
      constexpr int m = decltype(mc)::value;
      if constexpr (m + LA < NM) fr[m + LA] = frag(bw_ic<m + LA>{});
      mfma(mc, fr[m]);
      if constexpr (m == NSU - 3) load_stats(0);
      if constexpr (m == 2 * NSU - 3) load_stats(1);
      // sub-tile 0's units after score MFMAs NSU+1 .. 2 NSU-1, sub-tile 1's
      // after dV, dK MFMAs 2 NSU+1 .. 2 NSU+NGU-1
      bw_static_for<8>([&](auto kc) {
        constexpr int k = decltype(kc)::value;
        if constexpr (m == NSU + 1 + k * (NSU - 1) / 8) unit(0, k);
        if constexpr (m == 2 * NSU + 1 + k * (NGU - 1) / 8) unit(1, k);
      });
      __builtin_amdgcn_sched_barrier(0);
    });
    wg_sync();
  }

  // ---- epilogue: the lane holds key `key`, dims 32 db + 8 (r/4) + 4 hf + r%4
  const bool kvalid = key < p.T;
  const size_t orow = (((size_t)b * p.T + (kvalid ? key : 0)) * p.Hkv + g) * D;
  uint16_t* dvo = (uint16_t*)p.dv + orow;
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const u32x2_t w = {pack_bf2(dva[db][4 * r4], dva[db][4 * r4 + 1]),
                         pack_bf2(dva[db][4 * r4 + 2], dva[db][4 * r4 + 3])};
      if (kvalid) st8(dvo + db * 32 + 8 * r4 + 4 * hf, w);
    }
  // dk' = (sum dS q's) / log2(e): q's carries the factor log2(e)/sqrt(D)
  float gk[C::DB][16];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) gk[db][r] = dka[db][r] * kLn2;
  norm_rope_bwd_store<D>(gk, (const uint16_t*)p.k + orow,
                         (const uint32_t*)p.tab + (size_t)(kvalid ? key : 0) * (D / 2),
                         (uint16_t*)p.dk + orow, hf, kvalid);
}

// =====================================================================
// kernel B (bf16): dQ per (b, h, 128 positions)
// =====================================================================
template <int D>
__global__ void __launch_bounds__(256, 2) attn_bwd_q_bf16_kernel(BwdArgs p) {
  using C = BwCfg<D>;
  constexpr int STAGE = 2 * C::ROWT + C::TRT;  // K' rows, V rows, K'^T
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n = lane & 31, hf = lane >> 5;

  const int nqb = (p.T + 127) / 128;
  const int per = p.B * p.H;
  const int qb = nqb - 1 - (int)blockIdx.x / per;  // later positions have more keys: first
  const int bh = (int)blockIdx.x % per;
  const int b = bh / p.H, h = bh % p.H;
  const int g = h / p.G;
  const int tw0 = qb * 128 + wave * 32;  // this wave's first position
  const int t = tw0 + n;
  const bool tvalid = t < p.T;

  // stationary q's and dO fragments: B operand (col = position, k = dims)
  const uint32_t qrow = (uint32_t)p.H * D * 2;
  const size_t qbase = ((size_t)b * p.T * p.H + h) * D;
  const uint32_t q_rec = (uint32_t)(((size_t)(p.T - 1) * p.H) * D * 2 + D * 2);
  const __amdgpu_buffer_rsrc_t rq = make_rsrc((const uint16_t*)p.qs + qbase, q_rec);
  const __amdgpu_buffer_rsrc_t rd = make_rsrc((const uint16_t*)p.dout + qbase, q_rec);
  bf16x8_t qf[C::KS], df[C::KS];
#pragma unroll
  for (int s = 0; s < C::KS; ++s) {
    const uint32_t off = tvalid ? (uint32_t)t * qrow + (16 * s + 8 * hf) * 2 : 0xF0000000u;
    qf[s] = __builtin_bit_cast(bf16x8_t, bload16(rq, off, 0));
    df[s] = __builtin_bit_cast(bf16x8_t, bload16(rd, off, 0));
  }
  const int tc = tvalid ? t : 0;
  const float* sts = p.stats + (((size_t)b * p.H + h) * (p.Tp / 32) + tc / 32) * 64 + (tc & 31);
  const float l2 = sts[0], dlt = sts[32];

  f32x16_t dqa[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqa[db][r] = 0.f;

  const int q_last = min(qb * 128 + 127, p.T - 1);
  const int kt_lo = max(0, qb * 128 - p.W + 1) / 32;
  const int kt_hi = q_last / 32;
  const int nsteps = kt_hi - kt_lo + 1;

  const uint32_t kvrow = (uint32_t)p.Hkv * D * 2;
  auto issue = [&](int step, int buf) __attribute__((always_inline)) {
    const int k0 = (kt_lo + step) * 32;
    uint16_t* st = smem + buf * STAGE;
    const size_t rbase = (((size_t)b * p.T + k0) * p.Hkv + g) * D;
    const uint32_t rrec = (uint32_t)((p.T - k0) * (size_t)kvrow);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc((const uint16_t*)p.kp + rbase, rrec);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc((const uint16_t*)p.v + rbase, rrec);
    const __amdgpu_buffer_rsrc_t rkt =
        make_rsrc(p.kpt + ((size_t)b * p.Hkv + g) * D * p.Tp + k0, 0x7fffffff);
    constexpr int NI = 2 * C::RCOPY + C::TCOPY;
#pragma unroll
    for (int f = 0; f < NI; ++f) {
      if (f % 4 != wave) continue;
      if (f < 2 * C::RCOPY) {
        const int ff = f % C::RCOPY;
        const int e = ff * 64 + lane;
        const int r = e / C::CPR, c = e % C::CPR;
        const uint32_t off = (uint32_t)r * kvrow + (uint32_t)((c ^ ((r / C::KSW) % C::CPR)) * 16);
        lds_copy16(f < C::RCOPY ? rk : rv, st + (f < C::RCOPY ? 0 : C::ROWT) + ff * 512, off);
      } else {
        const int ff = f - 2 * C::RCOPY;
        const int e = ff * 64 + lane;
        const int d = e >> 2, c = e & 3;
        const uint32_t off = (uint32_t)d * p.Tp * 2 + (uint32_t)((c ^ ((d >> 2) & 3)) * 16);
        lds_copy16(rkt, st + 2 * C::ROWT + ff * 512, off);
      }
    }
  };
  auto rowfrag = [&](const uint16_t* tl, int s) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8_t*>(tl + row_chunk<D>(n, 2 * s + hf) * 8);
  };
  auto trfrag = [&](const uint16_t* tl, int db, int s2) __attribute__((always_inline)) {
    return *reinterpret_cast<const bf16x8_t*>(tl + tr_chunk(db * 32 + n, 2 * s2 + hf) * 8);
  };

  issue(0, 0);
  wg_sync();
  const int tw1 = min(tw0 + 31, p.T - 1);
  for (int step = 0; step < nsteps; ++step) {
    const int buf = step & 1;
    if (step + 1 < nsteps) issue(step + 1, buf ^ 1);
    const int k0 = (kt_lo + step) * 32;
    const bool any = tw0 < p.T && k0 <= tw1 && tw0 - (k0 + 31) < p.W;
    if (any) {
      const uint16_t* st = smem + buf * STAGE;
      f32x16_t sa, pa;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sa[r] = 0.f;
        pa[r] = 0.f;
      }
#pragma unroll
      for (int s = 0; s < C::KS; ++s) {
        sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rowfrag(st, s), qf[s], sa, 0, 0, 0);
        pa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(rowfrag(st + C::ROWT, s), df[s], pa, 0, 0, 0);
      }
      // rows: key k0 + 8 (r / 4) + 4 hf + r % 4; the lane's column: position t
      const bool full = k0 + 31 <= tw0 && tw1 - k0 < p.W && tw0 + 31 < p.T;
      uint32_t sw[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        float sv[2];
#pragma unroll
        for (int m = 0; m < 2; ++m) {
          const int r = 2 * i + m;
          float pr = fast_exp2(sa[r] - l2);
          if (!full) {
            const int kk = k0 + 8 * (r >> 2) + 4 * hf + (r & 3);
            const int dl2 = t - kk;
            if (!(dl2 >= 0 && dl2 < p.W && tvalid)) pr = 0.f;
          }
          sv[m] = pr * (pa[r] - dlt);
        }
        sw[i] = pack_bf2(sv[0], sv[1]);
      }
      const uint16_t* ktt = st + 2 * C::ROWT;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8_t bs =
            __builtin_bit_cast(bf16x8_t, u32x4_t{sw[4 * s2], sw[4 * s2 + 1], sw[4 * s2 + 2], sw[4 * s2 + 3]});
#pragma unroll
        for (int db = 0; db < C::DB; ++db)
          dqa[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(trfrag(ktt, db, s2), bs, dqa[db], 0, 0, 0);
      }
    }
    wg_sync();
  }

  // ---- epilogue: dq' = (sum dS k') / sqrt(D), then RMSNorm and RoPE backward
  const float isd = __builtin_amdgcn_rsqf((float)D);
  float gq[C::DB][16];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) gq[db][r] = dqa[db][r] * isd;
  const size_t orow = (((size_t)b * p.T + (tvalid ? t : 0)) * p.H + h) * D;
  norm_rope_bwd_store<D>(gq, (const uint16_t*)p.q + orow,
                         (const uint32_t*)p.tab + (size_t)(tvalid ? t : 0) * (D / 2),
                         (uint16_t*)p.dq + orow, hf, tvalid);
}

// =====================================================================
// fp32 path: exact arithmetic on the vector ALUs
// =====================================================================
// q' (unscaled), lse * log2(e) and dO . o per (b, t, h) row
template <int D>
__global__ void __launch_bounds__(128) attn_bwd_prep_f32_kernel(BwdArgs p) {
  const long long row = (long long)blockIdx.x * 128 + threadIdx.x;
  if (row >= (long long)p.B * p.T * p.H) return;
  const int h = (int)(row % p.H);
  const long long bt = row / p.H;
  const int t = (int)(bt % p.T), b = (int)(bt / p.T);
  const float* qr = (const float*)p.q + row * D;
  const float2* tr = (const float2*)p.tab + (size_t)t * (D / 2);
  float ss = 0.f;
#pragma unroll 4
  for (int i = 0; i < D / 2; ++i) {
    const float2 cs = tr[i];
    const float xe = qr[2 * i], xo = qr[2 * i + 1];
    const float ye = xe * cs.x - xo * cs.y, yo = xe * cs.y + xo * cs.x;
    ss += ye * ye + yo * yo;
  }
  const float rn = 1.0f / sqrtf(ss * (1.0f / D) + kEps);
  float* qo = (float*)p.qs + row * D;
#pragma unroll 4
  for (int i = 0; i < D / 2; ++i) {
    const float2 cs = tr[i];
    const float xe = qr[2 * i], xo = qr[2 * i + 1];
    qo[2 * i] = (xe * cs.x - xo * cs.y) * rn;
    qo[2 * i + 1] = (xe * cs.y + xo * cs.x) * rn;
  }
  const float* dr = (const float*)p.dout + row * D;
  const float* orw = (const float*)p.o + row * D;
  float dl = 0.f;
  for (int d = 0; d < D; ++d) dl += dr[d] * orw[d];
  float* st = p.stats + (((size_t)b * p.H + h) * (p.Tp / 32) + t / 32) * 64 + (t & 31);
  st[0] = p.lse[row] * kLog2e;
  st[32] = dl;
}

// RMSNorm + RoPE backward of one fp32 row: g (gradient w.r.t. the normalised
// row, overwritten), x the raw row, tab the position's (cos, sin) pairs.
template <int D>
__device__ __forceinline__ void norm_rope_bwd_row_f32(float (&g)[D], const float* x, const float2* tr,
                                                      float* out) {
  float ss = 0.f, dot = 0.f;
  for (int i = 0; i < D / 2; ++i) {
    const float2 cs = tr[i];
    const float ye = x[2 * i] * cs.x - x[2 * i + 1] * cs.y, yo = x[2 * i] * cs.y + x[2 * i + 1] * cs.x;
    ss += ye * ye + yo * yo;
    dot += g[2 * i] * ye + g[2 * i + 1] * yo;
  }
  const float rn = 1.0f / sqrtf(ss * (1.0f / D) + kEps);
  const float proj = dot * rn * (1.0f / D) * rn;  // mean(g y) rn
  for (int i = 0; i < D / 2; ++i) {
    const float2 cs = tr[i];
    const float ye = x[2 * i] * cs.x - x[2 * i + 1] * cs.y, yo = x[2 * i] * cs.y + x[2 * i + 1] * cs.x;
    const float de = rn * g[2 * i] - proj * rn * ye;
    const float dd = rn * g[2 * i + 1] - proj * rn * yo;
    out[2 * i] = de * cs.x + dd * cs.y;
    out[2 * i + 1] = -de * cs.y + dd * cs.x;
  }
}

// dK, dV: one thread per (b, key, g)
template <int D>
__global__ void __launch_bounds__(64) attn_bwd_kv_f32_kernel(BwdArgs p) {
  const long long id = (long long)blockIdx.x * 64 + threadIdx.x;
  if (id >= (long long)p.B * p.T * p.Hkv) return;
  const int g = (int)(id % p.Hkv);
  const long long bj = id / p.Hkv;
  const int j = (int)(bj % p.T), b = (int)(bj / p.T);
  const float* kr = (const float*)p.kp + id * D;
  const float* vr = (const float*)p.v + id * D;
  float dv[D], dk[D];
  for (int d = 0; d < D; ++d) {
    dv[d] = 0.f;
    dk[d] = 0.f;
  }
  const int i1 = min(p.T - 1, j + p.W - 1);
  for (int hh = g * p.G; hh < (g + 1) * p.G; ++hh) {
    const float* sb = p.stats + ((size_t)b * p.H + hh) * (p.Tp / 32) * 64;
    for (int i = j; i <= i1; ++i) {
      const size_t qrow = ((size_t)b * p.T + i) * p.H + hh;
      const float* qn = (const float*)p.qs + qrow * D;
      const float* dr = (const float*)p.dout + qrow * D;
      float s = 0.f, dp = 0.f;
      for (int d = 0; d < D; ++d) {
        s += qn[d] * kr[d];
        dp += dr[d] * vr[d];
      }
      const float* st = sb + (i / 32) * 64 + (i & 31);
      const float pr = exp2f(s * p.qscale - st[0]);
      const float ds = pr * (dp - st[32]);
      for (int d = 0; d < D; ++d) {
        dv[d] += pr * dr[d];
        dk[d] += ds * qn[d];
      }
    }
  }
  const float isd = 1.0f / sqrtf((float)D);
  for (int d = 0; d < D; ++d) dk[d] *= isd;
  float* dvo = (float*)p.dv + id * D;
  for (int d = 0; d < D; ++d) dvo[d] = dv[d];
  norm_rope_bwd_row_f32<D>(dk, (const float*)p.k + id * D, (const float2*)p.tab + (size_t)j * (D / 2),
                           (float*)p.dk + id * D);
}

// dQ: one thread per (b, t, h)
template <int D>
__global__ void __launch_bounds__(64) attn_bwd_q_f32_kernel(BwdArgs p) {
  const long long row = (long long)blockIdx.x * 64 + threadIdx.x;
  if (row >= (long long)p.B * p.T * p.H) return;
  const int h = (int)(row % p.H);
  const long long bt = row / p.H;
  const int t = (int)(bt % p.T), b = (int)(bt / p.T);
  const int g = h / p.G;
  const float* qn = (const float*)p.qs + row * D;
  const float* dr = (const float*)p.dout + row * D;
  const float* st = p.stats + (((size_t)b * p.H + h) * (p.Tp / 32) + t / 32) * 64 + (t & 31);
  const float l2 = st[0], dlt = st[32];
  float dq[D];
  for (int d = 0; d < D; ++d) dq[d] = 0.f;
  for (int j = max(0, t - p.W + 1); j <= t; ++j) {
    const size_t kr = (((size_t)b * p.T + j) * p.Hkv + g) * D;
    const float* kp = (const float*)p.kp + kr;
    const float* vp = (const float*)p.v + kr;
    float s = 0.f, dp = 0.f;
    for (int d = 0; d < D; ++d) {
      s += qn[d] * kp[d];
      dp += dr[d] * vp[d];
    }
    const float ds = exp2f(s * p.qscale - l2) * (dp - dlt);
    for (int d = 0; d < D; ++d) dq[d] += ds * kp[d];
  }
  const float isd = 1.0f / sqrtf((float)D);
  for (int d = 0; d < D; ++d) dq[d] *= isd;
  norm_rope_bwd_row_f32<D>(dq, (const float*)p.q + row * D, (const float2*)p.tab + (size_t)t * (D / 2),
                           (float*)p.dq + row * D);
}

// =====================================================================
// launch
// =====================================================================
static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

// Workspace carve-up, in order: table, k', then (bf16) k'^T, q's, q's^T,
// dO^T or (fp32) q'; then the per-tile stats.
struct BwdWs {
  size_t tab, kp, kpt, qs, qst, dot, stats, total;
};
static BwdWs bwd_ws(int B, int T, int H, int Hkv, int D, Dtype dt) {
  const size_t el = dt == kBF16 ? 2 : 4;
  const size_t Tp = (size_t)(T + 63) / 64 * 64;
  BwdWs w{};
  size_t o = 0;
  w.tab = o;
  o += al256(attn_prep_table_bytes(T, D, dt));
  w.kp = o;
  o += al256(attn_prep_k_bytes(B, T, Hkv, D, dt));
  if (dt == kBF16) {
    w.kpt = o;
    o += al256((size_t)B * Hkv * D * Tp * 2);
  }
  w.qs = o;
  o += al256((size_t)B * T * H * D * el);
  if (dt == kBF16) {
    w.qst = o;
    o += al256((size_t)B * H * D * Tp * 2);
    w.dot = o;
    o += al256((size_t)B * H * D * Tp * 2);
  }
  w.stats = o;
  o += al256((size_t)B * H * Tp * 2 * 4);
  w.total = o;
  return w;
}

size_t attn_bwd_workspace_bytes(int B, int T, int H, int Hkv, int D, Dtype dt) {
  return bwd_ws(B, T, H, Hkv, D, dt).total;
}

template <int D>
static hipError_t attn_bwd_d(BwdArgs a, Dtype dt, hipStream_t stream) {
  a.qscale = kLog2e / sqrtf((float)D);
  if (dt == kBF16) {
    const long long ntile = a.Tp / 32;
    const long long nblk = ((long long)a.B * a.H + (long long)a.B * a.Hkv) * ntile;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(attn_bwd_prep_bf16_kernel<D>, dim3((unsigned)nblk), dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const long long nb = (a.T + 127) / 128;
    hipLaunchKernelGGL(attn_bwd_kv_bf16_kernel<D>, dim3((unsigned)(nb * a.B * a.Hkv)), dim3(256), 0,
                       stream, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(attn_bwd_q_bf16_kernel<D>, dim3((unsigned)(nb * a.B * a.H)), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
  }
  const long long rows = (long long)a.B * a.T * a.H;
  hipLaunchKernelGGL(attn_bwd_prep_f32_kernel<D>, dim3((unsigned)((rows + 127) / 128)), dim3(128), 0,
                     stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const long long krows = (long long)a.B * a.T * a.Hkv;
  hipLaunchKernelGGL(attn_bwd_kv_f32_kernel<D>, dim3((unsigned)((krows + 63) / 64)), dim3(64), 0, stream,
                     a);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_q_f32_kernel<D>, dim3((unsigned)((rows + 63) / 64)), dim3(64), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_bwd(const void* q, const void* k, const void* v, const void* o,
                           const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                           int T, int H, int Hkv, int D, int window, double rope_base,
                           int pos_offset, Dtype dt, void* ws, hipStream_t stream) {
  const BwdWs w = bwd_ws(B, T, H, Hkv, D, dt);
  char* base = (char*)ws;
  // k' and the (cos, sin) table: the forward's input stage
  hipError_t e = launch_attn_prep(k, base + w.kp, base + w.tab, B, T, Hkv, D, rope_base, pos_offset,
                                  nullptr, nullptr, T, 0, nullptr, nullptr, dt, stream);
  if (e != hipSuccess) return e;
  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.dout = dout;
  a.lse = lse;
  a.tab = base + w.tab;
  a.kp = base + w.kp;
  a.kpt = dt == kBF16 ? (uint16_t*)(base + w.kpt) : nullptr;
  a.qs = base + w.qs;
  a.qst = dt == kBF16 ? (uint16_t*)(base + w.qst) : nullptr;
  a.dot = dt == kBF16 ? (uint16_t*)(base + w.dot) : nullptr;
  a.stats = (float*)(base + w.stats);
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  a.B = B;
  a.T = T;
  a.H = H;
  a.Hkv = Hkv;
  a.G = H / Hkv;
  a.W = window;
  a.Tp = (T + 63) / 64 * 64;
  switch (D) {
    case 32: return attn_bwd_d<32>(a, dt, stream);
    case 64: return attn_bwd_d<64>(a, dt, stream);
    case 128: return attn_bwd_d<128>(a, dt, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nc
