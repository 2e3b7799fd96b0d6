// Prefill attention forward for gfx950: RoPE + QK-norm fused into the Q/K
// loads, GQA, causal sliding-window band, online softmax, bf16 MFMA.
//
// What is computed ("从文本到聊天模型" (onehacker.top) §5.4 score = Q K^T,
// softmax, weighted sum of V; §5.5 causal mask; §5.6 RoPE;
// "Nanochat与nanoGPT对比：关键升级" (lzwjava.github.io) §1 table and notes:
// QK-norm after RoPE, GQA, sliding window):
//   o[b,t,h] = sum_j P[t,j] v[b,j,g],  g = h / (H/Hkv),
//   P[t,:]   = softmax_j( q'[t].k'[j] / sqrt(D) ) over 0 <= t - j < W,
//   q', k'   = RMSNorm(RoPE(q)), RMSNorm(RoPE(k)) at positions pos_offset + t.
//
// Design (bf16 path):
//  * A workgroup of 4 waves owns 128 query columns: hpw query heads of one
//    K/V group times 128/hpw consecutive positions, so a K/V tile staged in
//    LDS serves every head of the group. Each wave owns 32 columns.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_bf16:
//    the K tile is the A operand (LDS), the rotated, normalised, pre-scaled Q
//    is the B operand (registers, loaded once). In the accumulator layout a
//    lane then holds 16 keys of ONE query column, so the softmax needs no
//    cross-lane work per tile, and the accumulator registers feed the P.V
//    product directly as its B operand (O^T = V^T P^T).
//  * Softmax without a running maximum: after QK-norm |q'|, |k'| <= sqrt(D),
//    hence |q'.k'/sqrt(D)| <= sqrt(D) and, in the log2 domain used here,
//    |s| <= sqrt(D)*log2(e) (16.3 at D=128). 2^s then lies in
//    [2^-16.3, 2^16.3] and the row sum below T * 2^16.3, far inside the fp32
//    and bf16 ranges, so the numerators need no max subtraction and the
//    output accumulators are never rescaled. The normalisation by the row
//    sum cancels any common factor, so the result equals the textbook
//    max-subtracted softmax up to rounding.
//  * V is transposed into LDS (V^T[d][key]) with keys permuted so that each
//    MFMA A-operand fetch is one 16-byte LDS read matching the key order the
//    score accumulator hands over.
//  * Key tiles entirely outside the band are never visited; tiles entirely
//    inside skip the mask. Heaviest query tiles are dispatched first.
//
// fp32 path: exact fp32 arithmetic on the vector ALUs (one thread per query
// column), same band, same softmax without a running maximum.
#include "device_common.hpp"
#include "launch.hpp"

#include <type_traits>

namespace nc {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  const float2* tabq;  // [T][D/2] (cos, sin) fp32 for positions pos_offset + t
  const uint2* tabk;   // [T][D/2] bf16 pairs {(cos, -sin), (sin, cos)}
  int B, T, H, Hkv, W;
  int G;         // H / Hkv
  int hpw_log2;  // log2(query heads per workgroup)
  int ngroups;   // H / hpw
  int nqt;       // query tiles per (b, head group)
  int bp_log2;   // log2(positions per workgroup)
  float qscale;  // log2(e) / sqrt(D): folded into q'
};

// =====================================================================
// bf16 MFMA kernel
// =====================================================================
template <int D>
struct BfCfg {
  static constexpr int NW = 8;          // waves per workgroup
  static constexpr int NT = 64 * NW;    // threads per workgroup
  static constexpr int NC = 32 * NW;    // query columns per workgroup
  static constexpr int BN = 64;         // keys per tile
  static constexpr int KS = D / 16;     // MFMA k-steps of Q.K^T
  static constexpr int DB = D / 32;     // 32-row blocks of O^T
  static constexpr int RB = BN / 32;    // 32-key blocks per tile
  static constexpr int PS = BN / 16;    // MFMA k-steps of P.V
  static constexpr int KLD = D + 8;     // LDS row stride of K (bf16), +16 B against bank conflicts
  static constexpr int VLD = BN + 8;    // LDS row stride of V^T (bf16)
  static constexpr int CPR = D / 8;     // 16-byte chunks per K row
  static constexpr int KCH = BN * CPR;  // K chunks per tile
  static constexpr int NKP = (KCH + NT - 1) / NT;  // K chunks per thread
  static constexpr int NMB = (BN / 4) * (D / 4);   // 4-key x 4-dim V micro-blocks per tile
  static constexpr int KBUF = BN * KLD; // bf16 elements per K buffer
  static constexpr int VBUF = D * VLD;  // bf16 elements per V^T buffer
};

// Position of key kk (0..BN-1) inside a V^T row. The score accumulator of
// v_mfma_f32_32x32x16_bf16 gives lane-half hf the keys
// 8*(r/4) + 4*hf + r%4 (r = register 0..15) of a 32-key block; registers
// 8s..8s+7 form the P operand of k-step s. Placing those 8 keys next to each
// other makes the matching V^T operand a single 16-byte read.
__device__ __forceinline__ int vt_pos(int kk) {
  const int blk16 = kk >> 4, w = kk & 15;
  return (blk16 << 4) | (((w >> 2) & 1) << 3) | ((w >> 3) << 2) | (w & 3);
}

// Instruction order of a full tile for D = 128 and D = 64. Step m issues
// one MFMA -- the score MFMAs S0[0..KS), S1[0..KS) of the two 32-key blocks,
// then the P.V MFMAs of block 0 and of block 1 -- followed by up to two
// slices of vector work that do not depend on it:
//   0..4*NKP-1   RoPE + RMSNorm of the next tile's K chunk id/4, part id%4
//   100, 101     transposition of the next tile's V micro-block, half 0/1
//   200+8*rb+i   2^S of score registers 2i, 2i+1 of block rb, packed into
//                the P operand, and their contribution to the row sum
// A block's exponentials start two MFMAs after its last score MFMA, and
// each P.V MFMA comes after the four slices that produce its P operand.
template <int D>
struct FullSched;
template <>
struct FullSched<128> {
  static constexpr int NM = 32;
  static constexpr short v[NM][2] = {
      {0, -1},   {1, -1},   {2, -1},   {3, -1},   {4, -1},   {5, -1},   {6, -1},   {7, -1},
      {100, -1}, {101, -1}, {200, -1}, {201, -1}, {202, -1}, {203, -1}, {204, -1}, {205, -1},
      {206, -1}, {207, -1}, {208, -1}, {209, -1}, {210, -1}, {211, -1}, {212, -1}, {213, -1},
      {214, -1}, {215, -1}, {-1, -1},  {-1, -1},  {-1, -1},  {-1, -1},  {-1, -1},  {-1, -1}};
};
template <>
struct FullSched<32> {  // not used: D = 32 tiles run the generic order
  static constexpr int NM = 8;
  static constexpr short v[NM][2] = {{-1, -1}, {-1, -1}, {-1, -1}, {-1, -1},
                                     {-1, -1}, {-1, -1}, {-1, -1}, {-1, -1}};
};
template <>
struct FullSched<64> {
  static constexpr int NM = 16;
  static constexpr short v[NM][2] = {
      {0, -1},    {1, -1},    {2, -1},    {3, -1},    {100, -1},  {101, -1}, {200, 201}, {202, 203},
      {204, 205}, {206, 207}, {208, 209}, {210, 211}, {212, 213}, {214, 215}, {-1, -1},  {-1, -1}};
};

template <int D>
__global__ void __launch_bounds__(BfCfg<D>::NT, 1) attn_fwd_bf16_kernel(FwdArgs p) {
  using C = BfCfg<D>;
  __shared__ __attribute__((aligned(16))) uint16_t Ks[2 * C::KBUF];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[2 * C::VBUF];

  const uint16_t* __restrict__ qg = (const uint16_t*)p.q;
  uint16_t* __restrict__ og = (uint16_t*)p.o;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int n = lane & 31, hf = lane >> 5;

  // ---- work item: heaviest (latest) query tiles first
  const int per_qt = p.B * p.ngroups;
  const int qt = p.nqt - 1 - (int)blockIdx.x / per_qt;
  const int rem = (int)blockIdx.x % per_qt;
  const int b = rem / p.ngroups, grp = rem - (rem / p.ngroups) * p.ngroups;
  const int hpw = 1 << p.hpw_log2;
  const int q0 = qt << p.bp_log2;
  const int q_last = min(q0 + (1 << p.bp_log2), p.T) - 1;
  const int g = (grp * hpw) / p.G;

  // ---- this lane's query column
  const int col = wave * 32 + n;
  const int t = q0 + (col >> p.hpw_log2);
  const int h = grp * hpw + (col & (hpw - 1));
  const bool tvalid = t < p.T;
  const int tc = tvalid ? t : p.T - 1;

  // ---- Q: load, RoPE (fp32 table), RMSNorm, fold log2(e)/sqrt(D), pack as
  // ---- the MFMA B operand (lane-half hf holds dims 16s + 8hf .. +7)
  bf16x8_t bq[C::KS];
  {
    const uint16_t* qrow = qg + (((size_t)b * p.T + tc) * p.H + h) * D;
    const float2* trow = p.tabq + (size_t)tc * (D / 2);
    float x[C::KS][8];
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const int d0 = 16 * s + 8 * hf;
      const u32x4_t w = ld16(qrow + d0);
      const f32x4_t c01 = *reinterpret_cast<const f32x4_t*>(trow + d0 / 2);
      const f32x4_t c23 = *reinterpret_cast<const f32x4_t*>(trow + d0 / 2 + 2);
      const float cs[8] = {c01[0], c01[1], c01[2], c01[3], c23[0], c23[1], c23[2], c23[3]};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float xe = bf_lo(w[m]), xo = bf_hi(w[m]);
        const float c = cs[2 * m], sn = cs[2 * m + 1];
        const float ye = xe * c - xo * sn, yo = xe * sn + xo * c;
        x[s][2 * m] = ye;
        x[s][2 * m + 1] = yo;
        ss += ye * ye + yo * yo;
      }
    }
    ss = sum_halves(ss);
    const float sc = p.qscale * rsq(ss * (1.0f / D) + kEps);
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      u32x4_t w;
#pragma unroll
      for (int m = 0; m < 4; ++m) w[m] = pack_bf2(x[s][2 * m] * sc, x[s][2 * m + 1] * sc);
      bq[s] = __builtin_bit_cast(bf16x8_t, w);
    }
  }

  // ---- key-tile range of the band [max(0, q0 - W + 1), q_last]
  const int k_first = max(0, q0 - p.W + 1);
  const int kt0 = k_first / C::BN, kt1 = q_last / C::BN;

  // ---- staging: buffer resources whose ranges end at token T (reads past
  // ---- the tail return zeros), per-thread byte offsets, per-tile SGPR offsets
  const uint32_t row_bytes = (uint32_t)p.Hkv * D * 2;
  const size_t kv_base = ((size_t)b * p.T * p.Hkv + g) * D;
  const uint32_t kv_records = (uint32_t)(((size_t)p.T * p.Hkv - g) * D * 2);
  const char* kseq = (const char*)((const uint16_t*)p.k + kv_base);
  const char* vseq = (const char*)((const uint16_t*)p.v + kv_base);
  const uint32_t tab_row = (D / 2) * 8;
  const uint32_t tab_records = (uint32_t)p.T * tab_row;

  uint32_t k_voff[C::NKP], t_voff[C::NKP], k_lds[C::NKP];
  bool k_act[C::NKP];
#pragma unroll
  for (int j = 0; j < C::NKP; ++j) {
    const int idx = tid + C::NT * j;
    const int kr = idx / C::CPR, kc = idx % C::CPR;
    k_act[j] = idx < C::KCH;
    k_voff[j] = (uint32_t)kr * row_bytes + kc * 16;
    t_voff[j] = (uint32_t)kr * (D / 2) * 8 + kc * 32;
    k_lds[j] = kr * C::KLD + kc * 8;
  }
  const bool v_act = tid < C::NMB;
  const int vgp = tid & 15, vd = tid >> 4;  // V micro-block: keys 4*vgp.., dims 4*vd..
  const uint32_t v_voff = (uint32_t)(4 * vgp) * row_bytes + vd * 8;
  const int v_lds = (4 * vd) * C::VLD + vt_pos(4 * vgp);

  u32x4_t kw[C::NKP], kt_[C::NKP][2];
  u32x2_t vw[4];

  // Resources rebased on the tile's first key: rows past token T (and only
  // those) fall beyond num_records and read as zero.
  auto gload = [&](int kt) {
    // a tile past the sequence (staged but never used) gets empty ranges
    const uint32_t so = (uint32_t)kt * C::BN * row_bytes;
    const uint32_t st = (uint32_t)kt * C::BN * tab_row;
    const uint32_t nk = __builtin_amdgcn_readfirstlane(so < kv_records ? kv_records - so : 0u);
    const uint32_t nt = __builtin_amdgcn_readfirstlane(st < tab_records ? tab_records - st : 0u);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kseq + so, nk);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vseq + so, nk);
    const __amdgpu_buffer_rsrc_t rt = make_rsrc((const char*)p.tabk + st, nt);
#pragma unroll
    for (int j = 0; j < C::NKP; ++j) {
      if (C::NKP * C::NT == C::KCH || k_act[j]) {
        kw[j] = bload16(rk, k_voff[j], 0);
        kt_[j][0] = bload16(rt, t_voff[j], 0);
        kt_[j][1] = bload16(rt, t_voff[j] + 16, 0);
      }
    }
    if (C::NMB >= C::NT || v_act) {
#pragma unroll
      for (int r = 0; r < 4; ++r) vw[r] = bload8(rv, v_voff + r * row_bytes, 0);
    }
  };

  // RoPE + RMSNorm of the staged K chunks (bf16 pair dot products against the
  // (cos,-sin)/(sin,cos) table), and the V micro-block transposed into V^T.
  auto stage = [&](int buf) {
    uint16_t* kb = Ks + buf * C::KBUF;
    uint16_t* vb = Vt + buf * C::VBUF;
#pragma unroll
    for (int j = 0; j < C::NKP; ++j) {
      if (C::NKP * C::NT == C::KCH || k_act[j]) {
        float ss = dot2bf(kw[j][0], kw[j][0], 0.f);
        ss = dot2bf(kw[j][1], kw[j][1], ss);
        ss = dot2bf(kw[j][2], kw[j][2], ss);
        ss = dot2bf(kw[j][3], kw[j][3], ss);  // a rotation keeps the sum of squares
        ss = dpp_group_sum<C::CPR>(ss);
        const float inv = rsq(ss * (1.0f / D) + kEps);
        u32x4_t w;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const u32x4_t& tt = kt_[j][m >> 1];
          const float xe = dot2bf(kw[j][m], tt[2 * (m & 1)], 0.f);
          const float xo = dot2bf(kw[j][m], tt[2 * (m & 1) + 1], 0.f);
          w[m] = pack_bf2(xe * inv, xo * inv);
        }
        st16(kb + k_lds[j], w);
      }
    }
    if (C::NMB >= C::NT || v_act) {
      // rows 4vd..4vd+3 of V^T, 4 consecutive (permuted) key slots each
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        const uint32_t a0 = vw[0][m], a1 = vw[1][m], a2 = vw[2][m], a3 = vw[3][m];
        const u32x2_t lo = {(a0 & 0xffffu) | (a1 << 16), (a2 & 0xffffu) | (a3 << 16)};
        const u32x2_t hi = {(a0 >> 16) | (a1 & 0xffff0000u), (a2 >> 16) | (a3 & 0xffff0000u)};
        st8(vb + v_lds + (2 * m) * C::VLD, lo);
        st8(vb + v_lds + (2 * m + 1) * C::VLD, hi);
      }
    }
  };

  f32x16_t oacc[C::DB];
#pragma unroll
  for (int db = 0; db < C::DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float lsum = 0.f;

  // Positions covered by this wave (its 32 columns): [tw0, tw1].
  const int tw0 = q0 + ((wave * 32) >> p.hpw_log2);
  const int tw1 = min(q0 + ((wave * 32 + 31) >> p.hpw_log2), p.T - 1);
  constexpr uint32_t kOnes = 0x3F803F80u;  // bf16 pair (1, 1)

  // Scores of one 32-key block: S^T = K Q^T (MFMA, log2 domain).
  auto scores = [&](const uint16_t* kb, int rb) {
    f32x16_t acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
    for (int s = 0; s < C::KS; ++s) {
      const bf16x8_t a =
          *reinterpret_cast<const bf16x8_t*>(kb + (rb * 32 + n) * C::KLD + 16 * s + 8 * hf);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[s], acc, 0, 0, 0);
    }
    return acc;
  };
  // Softmax numerators 2^S packed as the two bf16 P operands of the block,
  // their sum accumulated with bf16 pair dot products (the same rounded
  // values the P.V product uses), then O^T += V^T P^T.
  auto accumulate = [&](const uint16_t* vb, int rb, const f32x16_t& sc) {
    bf16x8_t pb[2];
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      u32x4_t w;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        w[m] = pack_bf2(fast_exp2(sc[8 * s2 + 2 * m]), fast_exp2(sc[8 * s2 + 2 * m + 1]));
        lsum = dot2bf(w[m], kOnes, lsum);
      }
      pb[s2] = __builtin_bit_cast(bf16x8_t, w);
    }
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
            vb + (db * 32 + n) * C::VLD + 16 * (2 * rb + s2) + 8 * hf);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[s2], oacc[db], 0, 0, 0);
      }
    }
  };

  // Tile entirely inside the band for every column of the workgroup.
  auto compute_full = [&](int buf) {
    const uint16_t* kb = Ks + buf * C::KBUF;
    const uint16_t* vb = Vt + buf * C::VBUF;
    f32x16_t sc[C::RB];
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) sc[rb] = scores(kb, rb);
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) accumulate(vb, rb, sc[rb]);
  };

  // Tile crossing the band edge: per wave and 32-key block, skip blocks the
  // wave cannot see at all, mask blocks it sees in part.
  auto compute_edge = [&](int buf, int kt) {
    const uint16_t* kb = Ks + buf * C::KBUF;
    const uint16_t* vb = Vt + buf * C::VBUF;
    // key of register r in block rb is kt*BN + rb*32 + 8*(r/4) + 4*hf + r%4
    const int dl0 = t - kt * C::BN - 4 * hf;
#pragma unroll
    for (int rb = 0; rb < C::RB; ++rb) {
      const int kb0 = kt * C::BN + rb * 32;
      const bool none = kb0 > tw1 || tw0 - (kb0 + 31) >= p.W;
      if (none) continue;
      f32x16_t sc = scores(kb, rb);
      const bool all = kb0 + 31 <= tw0 && tw1 - kb0 < p.W;
      if (!all) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int dl = dl0 - (rb * 32 + 8 * (r >> 2) + (r & 3));
          sc[r] = ((unsigned)dl < (unsigned)p.W) ? sc[r] : -INFINITY;  // 2^-inf = 0
        }
      }
      accumulate(vb, rb, sc);
    }
  };

  // Full tile in a fixed instruction order (FullSched): compute tile `buf`
  // while the next tile's K and V, already in registers, are rotated,
  // normalised and transposed between the MFMAs, then written to the other
  // buffer. LDS fragments are read three MFMAs ahead.
  auto tile_full_sched = [&](int buf) {
    using SCH = FullSched<D>;
    constexpr int NS = C::KS, NP = 2 * C::DB, NM = 2 * NS + 2 * NP, LA = 8;
    static_assert(SCH::NM == NM, "schedule length");
    const uint16_t* kb = Ks + buf * C::KBUF;
    const uint16_t* vb = Vt + buf * C::VBUF;
    f32x16_t sacc[2];
    u32x4_t pbu[2][2];
    float kss[C::NKP], kinv[C::NKP];
    u32x4_t kout[C::NKP];
    u32x2_t vlo[2], vhi[2];
    bf16x8_t fr[LA + 1];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sacc[0][r] = 0.f;
      sacc[1][r] = 0.f;
    }
    auto frag = [&](int m) -> bf16x8_t {
      if (m < 2 * NS) {
        const int rb = m / NS, s = m % NS;
        return *reinterpret_cast<const bf16x8_t*>(kb + (rb * 32 + n) * C::KLD + 16 * s + 8 * hf);
      }
      const int idx = m - 2 * NS, rb = idx / NP, i = idx % NP;
      const int db = i % C::DB, s2 = i / C::DB;
      return *reinterpret_cast<const bf16x8_t*>(vb + (db * 32 + n) * C::VLD + 16 * (2 * rb + s2) +
                                                8 * hf);
    };
    auto slice = [&](int id) {
      if (id < 0) return;
      if (id < 100) {
        const int j = id >> 2, part = id & 3;
        if (part == 0) {
          float ss = dot2bf(kw[j][0], kw[j][0], 0.f);
          ss = dot2bf(kw[j][1], kw[j][1], ss);
          ss = dot2bf(kw[j][2], kw[j][2], ss);
          kss[j] = dot2bf(kw[j][3], kw[j][3], ss);  // a rotation keeps the sum of squares
          pin(kss[j]);
        } else if (part == 1) {
          kinv[j] = rsq(dpp_group_sum<C::CPR>(kss[j]) * (1.0f / D) + kEps);
          pin(kinv[j]);
        } else {
#pragma unroll
          for (int mm = 0; mm < 2; ++mm) {
            const int m = 2 * (part - 2) + mm;
            const u32x4_t& tt = kt_[j][m >> 1];
            const float xe = dot2bf(kw[j][m], tt[2 * (m & 1)], 0.f);
            const float xo = dot2bf(kw[j][m], tt[2 * (m & 1) + 1], 0.f);
            uint32_t w = pack_bf2(xe * kinv[j], xo * kinv[j]);
            pin(w);
            kout[j][m] = w;
          }
        }
      } else if (id < 200) {
        const int m = id - 100;
        const uint32_t a0 = vw[0][m], a1 = vw[1][m], a2 = vw[2][m], a3 = vw[3][m];
        uint32_t l0 = (a0 & 0xffffu) | (a1 << 16), l1 = (a2 & 0xffffu) | (a3 << 16);
        uint32_t h0 = (a0 >> 16) | (a1 & 0xffff0000u), h1 = (a2 >> 16) | (a3 & 0xffff0000u);
        pin(l0);
        pin(l1);
        pin(h0);
        pin(h1);
        vlo[m] = u32x2_t{l0, l1};
        vhi[m] = u32x2_t{h0, h1};
      } else {
        const int rb = (id - 200) >> 3, i = (id - 200) & 7;
        const uint32_t w = pack_bf2(fast_exp2(sacc[rb][2 * i]), fast_exp2(sacc[rb][2 * i + 1]));
        lsum = dot2bf(w, kOnes, lsum);
        pbu[rb][i >> 2][i & 3] = w;
      }
    };
#pragma unroll
    for (int m = 0; m < LA; ++m) fr[m] = frag(m);
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      if (m + LA < NM) fr[(m + LA) % (LA + 1)] = frag(m + LA);
      const bf16x8_t a = fr[m % (LA + 1)];
      if (m < 2 * NS) {
        const int rb = m / NS, s = m % NS;
        sacc[rb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bq[s], sacc[rb], 0, 0, 0);
      } else {
        const int idx = m - 2 * NS, rb = idx / NP, i = idx % NP;
        const int db = i % C::DB, s2 = i / C::DB;
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            a, __builtin_bit_cast(bf16x8_t, pbu[rb][s2]), oacc[db], 0, 0, 0);
      }
      slice(SCH::v[m][0]);
      slice(SCH::v[m][1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the next tile's K' and V^T into the other buffer
    uint16_t* kbw = Ks + (buf ^ 1) * C::KBUF;
    uint16_t* vbw = Vt + (buf ^ 1) * C::VBUF;
#pragma unroll
    for (int j = 0; j < C::NKP; ++j) st16(kbw + k_lds[j], kout[j]);
    if (C::NMB >= C::NT || v_act) {
#pragma unroll
      for (int m = 0; m < 2; ++m) {
        st8(vbw + v_lds + (2 * m) * C::VLD, vlo[m]);
        st8(vbw + v_lds + (2 * m + 1) * C::VLD, vhi[m]);
      }
    }
  };

  // ---- double-buffered main loop: tile kt is computed from one LDS buffer
  // ---- while tile kt+1 is rotated/normalised into the other and tile kt+2
  // ---- is in flight from memory; one barrier per tile. Staging runs
  // ---- unconditionally (past kt1 it reads zeros). The band splits into
  // ---- leading window-edge tiles, full tiles and trailing diagonal tiles;
  // ---- each range runs its own loop so every loop body is straight-line.
  gload(kt0);
  stage(0);
  gload(kt0 + 1);
  __syncthreads();
  auto run = [&](int ka, int kb_, bool edge) {
    for (int kt = ka; kt <= kb_; ++kt) {
      const int cur = (kt - kt0) & 1;
      if constexpr (D >= 64) {
        if (edge) {
          compute_edge(cur, kt);
          stage(cur ^ 1);
        } else {
          tile_full_sched(cur);
        }
      } else {
        if (edge) compute_edge(cur, kt); else compute_full(cur);
        stage(cur ^ 1);
      }
      gload(kt + 2);
      __syncthreads();
    }
  };
  // full tiles: j0 + BN - 1 <= q0 (every key at or before every query) and
  // q_last - j0 < W (every key inside every query's window)
  const int ktA = max(kt0, (q_last - p.W + 1 + C::BN - 1 >= 0) ? (q_last - p.W + C::BN) / C::BN : 0);
  const int ktB = min(kt1, (q0 + 1) / C::BN - 1);
  if (ktA <= ktB) {
    run(kt0, ktA - 1, true);
    run(ktA, ktB, false);
    run(ktB + 1, kt1, true);
  } else {
    run(kt0, kt1, true);
  }

  // ---- epilogue: normalise by the row sum and store bf16 (B, T, H, D)
  lsum = sum_halves(lsum);
  const float inv_l = 1.0f / lsum;
  if (tvalid) {
    uint16_t* orow = og + (((size_t)b * p.T + t) * p.H + h) * D;
#pragma unroll
    for (int db = 0; db < C::DB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = db * 32 + 8 * r4 + 4 * hf;
        const u32x2_t w = {pack_bf2(oacc[db][4 * r4] * inv_l, oacc[db][4 * r4 + 1] * inv_l),
                           pack_bf2(oacc[db][4 * r4 + 2] * inv_l, oacc[db][4 * r4 + 3] * inv_l)};
        st8(orow + d, w);
      }
    }
  }
}

// =====================================================================
// fp32 kernel: one thread per query column, fp32 FMAs, K'/V tiles in LDS.
// =====================================================================
template <int D>
__global__ void __launch_bounds__(128) attn_fwd_f32_kernel(FwdArgs p) {
  constexpr int NT = 128, BN = 32;
  __shared__ float Kf[BN][D + 1];
  __shared__ float Vf[BN][D + 1];

  const float* __restrict__ qg = (const float*)p.q;
  const float* __restrict__ kg = (const float*)p.k;
  const float* __restrict__ vg = (const float*)p.v;
  float* __restrict__ og = (float*)p.o;

  const int tid = threadIdx.x;
  const int per_qt = p.B * p.H;
  const int qt = p.nqt - 1 - (int)blockIdx.x / per_qt;
  const int rem = (int)blockIdx.x % per_qt;
  const int b = rem / p.H, h = rem - (rem / p.H) * p.H;
  const int g = h / p.G;
  const int q0 = qt * NT;
  const int q_last = min(q0 + NT, p.T) - 1;
  const int t = q0 + tid;
  const bool tvalid = t < p.T;
  const int tc = tvalid ? t : p.T - 1;

  float qv[D];
  {
    const float* qrow = qg + (((size_t)b * p.T + tc) * p.H + h) * D;
    const float2* trow = p.tabq + (size_t)tc * (D / 2);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < D / 2; ++i) {
      const float2 cs = trow[i];
      const float xe = qrow[2 * i], xo = qrow[2 * i + 1];
      const float ye = xe * cs.x - xo * cs.y, yo = xe * cs.y + xo * cs.x;
      qv[2 * i] = ye;
      qv[2 * i + 1] = yo;
      ss += ye * ye + yo * yo;
    }
    const float sc = p.qscale / sqrtf(ss * (1.0f / D) + kEps);
#pragma unroll
    for (int d = 0; d < D; ++d) qv[d] *= sc;
  }

  float acc[D];
#pragma unroll
  for (int d = 0; d < D; ++d) acc[d] = 0.f;
  float lsum = 0.f;

  const int k_first = max(0, q0 - p.W + 1);
  const size_t kv_row = (size_t)p.Hkv * D;
  for (int j0 = (k_first / BN) * BN; j0 <= q_last; j0 += BN) {
    __syncthreads();
    // stage K' (rotated + normalised) and V: 4 threads per key row
    {
      const int r = tid >> 2, part = tid & 3;
      const int key = j0 + r;
      float y[D / 4];
      float ss = 0.f;
      if (key < p.T) {
        const float* krow = kg + ((size_t)b * p.T + key) * kv_row + (size_t)g * D + part * (D / 4);
        const float2* trow = p.tabq + (size_t)key * (D / 2) + part * (D / 8);
#pragma unroll
        for (int i = 0; i < D / 8; ++i) {
          const float2 cs = trow[i];
          const float xe = krow[2 * i], xo = krow[2 * i + 1];
          y[2 * i] = xe * cs.x - xo * cs.y;
          y[2 * i + 1] = xe * cs.y + xo * cs.x;
          ss += y[2 * i] * y[2 * i] + y[2 * i + 1] * y[2 * i + 1];
        }
      } else {
#pragma unroll
        for (int i = 0; i < D / 4; ++i) y[i] = 0.f;
      }
      ss = group_sum<4>(ss);
      const float inv = 1.0f / sqrtf(ss * (1.0f / D) + kEps);
#pragma unroll
      for (int i = 0; i < D / 4; ++i) Kf[r][part * (D / 4) + i] = y[i] * inv;
      if (key < p.T) {
        const float* vrow = vg + ((size_t)b * p.T + key) * kv_row + (size_t)g * D + part * (D / 4);
#pragma unroll
        for (int i = 0; i < D / 4; ++i) Vf[r][part * (D / 4) + i] = vrow[i];
      } else {
#pragma unroll
        for (int i = 0; i < D / 4; ++i) Vf[r][part * (D / 4) + i] = 0.f;
      }
    }
    __syncthreads();
#pragma unroll 1
    for (int jj = 0; jj < BN; ++jj) {
      const int key = j0 + jj;
      const int dl = t - key;
      if (dl < 0 || dl >= p.W) continue;
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < D; ++d) s += qv[d] * Kf[jj][d];
      const float e = exp2f(s);
      lsum += e;
#pragma unroll
      for (int d = 0; d < D; ++d) acc[d] += e * Vf[jj][d];
    }
  }
  if (tvalid) {
    float* orow = og + (((size_t)b * p.T + t) * p.H + h) * D;
    const float inv_l = 1.0f / lsum;
#pragma unroll
    for (int d = 0; d < D; ++d) orow[d] = acc[d] * inv_l;
  }
}

// =====================================================================
// launch
// =====================================================================
static int ilog2(int x) {
  int r = 0;
  while ((1 << (r + 1)) <= x) ++r;
  return r;
}

template <int D>
static hipError_t attn_fwd_d(FwdArgs a, Dtype dt, hipStream_t stream) {
  a.qscale = kLog2e / sqrtf((float)D);
  if (dt == kBF16) {
    // heads per workgroup: largest power of two dividing G, at most 32
    int hpw = 1;
    while (hpw < 32 && (a.G % (hpw * 2)) == 0) hpw *= 2;
    a.hpw_log2 = ilog2(hpw);
    a.ngroups = a.H / hpw;
    a.bp_log2 = ilog2(BfCfg<D>::NC / hpw);
    a.nqt = (a.T + (1 << a.bp_log2) - 1) >> a.bp_log2;
    const long long grid = (long long)a.nqt * a.B * a.ngroups;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<D>, dim3((unsigned)grid), dim3(BfCfg<D>::NT), 0, stream,
                       a);
  } else {
    a.hpw_log2 = 0;
    a.ngroups = a.H;
    a.bp_log2 = 7;
    a.nqt = (a.T + 127) / 128;
    const long long grid = (long long)a.nqt * a.B * a.H;
    if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(attn_fwd_f32_kernel<D>, dim3((unsigned)grid), dim3(128), 0, stream, a);
  }
  return hipGetLastError();
}

hipError_t launch_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int T,
                           int H, int Hkv, int D, int window, const void* tab, Dtype dt,
                           hipStream_t stream) {
  FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.tabq = (const float2*)tab;
  a.tabk = (const uint2*)((const char*)tab + rope_table_half_bytes(T, D));
  a.B = B;
  a.T = T;
  a.H = H;
  a.Hkv = Hkv;
  a.W = window;
  a.G = H / Hkv;
  switch (D) {
    case 32: return attn_fwd_d<32>(a, dt, stream);
    case 64: return attn_fwd_d<64>(a, dt, stream);
    case 128: return attn_fwd_d<128>(a, dt, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace nc
