// One-token decode step over a contiguous per-layer KV cache, split over the
// key range ("split-KV"), for gfx950.
//
// What is computed ("从文本到聊天模型" (onehacker.top) §10.2-10.4: compute the
// new token's q, k, v, append k and v to the cache, then let q attend to every
// cached key; §10.3: one cache per layer of shape (batch, seq, heads, dim);
// "Nanochat与nanoGPT对比：关键升级" (lzwjava.github.io) §1 table: QK-norm after
// RoPE, GQA, sliding window):
//   L = seqlens[b] (counts the new token), p = L - 1,
//   k_cache[b, p] = RMSNorm(RoPE(k_new[b], p)),  v_cache[b, p] = v_new[b],
//   o[b, h] = softmax_j( q'.k_j / sqrt(D) ) v_j  over j in [max(0, L-W), L-1],
//   q' = RMSNorm(RoPE(q[b, h], p)).
//
// Design: decode reads every visible K/V row once, so it is bound by HBM.
// A workgroup owns (sequence b, K/V head g, up to GP query heads of g, a chunk
// of C consecutive keys). CPR lanes stream one 16-byte piece of a K row and of
// a V row per key, so a wave reads whole rows with unit-stride loads (with the
// non-temporal hint: each row is read once); each lane group takes U keys per
// iteration, with loads up to two iterations ahead, and rescales its running
// softmax state once per U keys (the scores of cache rows are not assumed
// bounded, so this path keeps a running maximum). Partial (max, sum,
// unnormalised output) states are merged across lanes with DPP/shuffles and
// across waves in LDS. A sequence whose visible range fits one chunk writes
// its output directly; otherwise each chunk stores its state in the
// workspace and a second small kernel merges the states (the kernel boundary
// makes every chunk's state visible across the chip's L2 caches at once,
// which a per-workgroup device-scope release would pay for many times). The
// chunk holding key L-1 writes the appended row and uses it from LDS, so no
// workgroup waits on another's write.
//
// Shared prompt (SH, nc_attn_decode_shared; the same page, §10.6: the prompt
// is prefilled once and several samples generate from its cache): positions
// 0 .. Lp-1 are read from one (Lp, Hkv, D) cache shared by all sequences,
// position p >= Lp from row p - Lp of the sequence's own cache. A chunk lies
// wholly in one of the two caches when the range is cut at Lp (long prompt
// parts, which then run in parallel with the own part), or runs as two
// segments in one workgroup (prompt rows first, one softmax state). Prompt
// rows are loaded with the temporal hint and the workgroups are ordered
// head-major per XCD, so each XCD's L2 serves the prompt rows of a few heads
// to every sequence. Without SH the kernel is the one described above.
//
// Value embedding ("Nanochat与nanoGPT对比：关键升级" §1 notes, value residual):
// with ve_new given, the appended value is v_new + ve_gate * ve_new, formed in
// fp32 and rounded once.
#include "device_common.hpp"
#include "launch.hpp"

#include <algorithm>
#include <cmath>

namespace nc {

struct DecArgs {
  const void* q;
  const void* k_new;
  const void* v_new;
  void* k_cache;        // (B, Tgen, Hkv, D): row r holds position Lp + r
  void* v_cache;
  const void* k_prompt;  // (Lp, Hkv, D): positions 0 .. Lp-1, shared by all sequences
  const void* v_prompt;
  const void* ve_new;    // (B, Hkv, D) value embedding of the new token, or null
  const void* ve_gate;   // (B, Hkv): the appended value is v_new + ve_gate * ve_new
  const int32_t* seqlens;
  void* o;
  float* part;  // [B][H][nsplit][D + 2]: unnormalised o (D), max, sum
  int B, Tmax, H, Hkv, G, W;  // Tmax = Lp + Tgen: the longest sequence
  int Lp;       // shared prompt rows (0: none; every position in the sequence's cache)
  int Tgen;     // rows per sequence cache
  int nwg;      // workgroups with an item (the shared-prompt launch pads the grid to a multiple of 8)
  int cut;      // shared prompt: 1 cuts every range at the prompt's end; 0 lets a chunk span
                // both caches (run as two segments in one workgroup)
  int Cp;       // keys per chunk of a cut prompt part (= C otherwise)
  int C;        // keys per chunk (multiple of the keys per workgroup step)
  int nsplit;   // chunks per (b, g) upper bound = ceil(min(Tmax, W) / C)
  int ngh;      // head groups per K/V head = ceil(G / GP)
  int ncu;      // compute units of the device
  int order;    // 1: workgroups take (b, g, head group) items by visible length (below)
  double log2_base;  // log2(rope_base)
};

// Largest batch for which workgroups rank the sequences by length themselves.
constexpr int kDecRankMaxB = 512;

template <typename Elem>
struct ElemTraits;
template <>
struct ElemTraits<uint16_t> {
  static constexpr int EPC = 8;
  __device__ static void unpack(const u32x4_t& w, float* x) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      x[2 * m] = bf_lo(w[m]);
      x[2 * m + 1] = bf_hi(w[m]);
    }
  }
  __device__ static float to_f(uint16_t x) { return __uint_as_float((uint32_t)x << 16); }
  __device__ static uint16_t from_f(float x) { return (uint16_t)(pack_bf2(x, 0.f) & 0xffffu); }
};
template <>
struct ElemTraits<float> {
  static constexpr int EPC = 4;
  __device__ static void unpack(const u32x4_t& w, float* x) {
#pragma unroll
    for (int m = 0; m < 4; ++m) x[m] = __uint_as_float(w[m]);
  }
  __device__ static float to_f(float x) { return x; }
  __device__ static float from_f(float x) { return x; }
};

__device__ __forceinline__ int clamp_len(int L, int Lp, int Tmax) {
  return L < Lp + 1 ? Lp + 1 : (L > Tmax ? Tmax : L);
}

// Chunks of the visible keys [lo, L): those of the shared prompt [lo, Lp)
// first, then those of the sequence's own rows [max(lo, Lp), L), C keys each,
// so that no chunk spans both caches. Returns the chunk count and, for chunk
// c, its key range [ks0, ks1). With Lp = 0 these are C-key chunks from lo.
__device__ __forceinline__ int dec_chunks(int L, int lo, int Lp, int Cp, int C, int c, int& ks0,
                                          int& ks1) {
  const int ea = min(L, Lp);                             // end of the prompt part
  const int na = lo < ea ? (ea - lo + Cp - 1) / Cp : 0;  // its chunks, Cp keys each
  const int sb = max(lo, Lp);                          // start of the own part
  const int nb = (L - sb + C - 1) / C;
  if (c < na) {
    ks0 = lo + c * Cp;
    ks1 = min(ks0 + Cp, ea);
  } else {
    ks0 = sb + (c - na) * C;
    ks1 = min(ks0 + C, L);
  }
  return na + nb;
}

// Sum over groups of `width` consecutive lanes, width a power of two <= 64.
template <int width>
__device__ __forceinline__ float lane_group_sum(float x) {
  if constexpr (width <= 16) {
    return dpp_group_sum<width>(x);
  } else {
    x = dpp_group_sum<16>(x);
#pragma unroll
    for (int off = 16; off < width; off <<= 1) x += __shfl_xor(x, off, 64);
    return x;
  }
}

// Merge softmax states (m, l, acc) of two disjoint key sets.
__device__ __forceinline__ float merge_scale(float m, float mn) {
  return m == -INFINITY ? 0.f : fast_exp2(m - mn);
}

// Keys per lane group per iteration, and register sets of K/V rows in flight
// (the loads of iteration it + NBUF - 1 go out while iteration it is
// consumed; the loop below is written for 2 and 3 sets): three, except with
// 8 query heads per workgroup, where the third set would take the kernel past
// 256 registers and so to one wave per SIMD.
constexpr int kDecU = 4;
template <int GP>
constexpr int dec_bufs() { return GP <= 4 ? 3 : 2; }

// SH: a shared prompt cache holds positions 0 .. Lp-1 (nc_attn_decode_shared);
// without it Lp = 0 and every position is in the sequence's own cache.
template <int D, int GP, typename Elem, bool SH>
__global__ void __launch_bounds__(256) attn_decode_kernel(DecArgs a) {
  using TR = ElemTraits<Elem>;
  constexpr int EPC = TR::EPC;
  constexpr int CPR = D / EPC;        // lanes per key row
  constexpr int KPW = 64 / CPR;       // keys per wave per step
  constexpr int U = kDecU;            // keys per lane group per iteration
  constexpr int NBUF = dec_bufs<GP>();  // register sets: loads run NBUF-1 iterations ahead
  static_assert(NBUF == 2 || NBUF == 3, "register sets in flight");
  constexpr int KPI = 4 * KPW * U;    // keys per workgroup iteration

  __shared__ float qs[GP][D];         // q' * log2(e)/sqrt(D)
  __shared__ float knew_s[D];         // appended key (rounded to the cache type)
  __shared__ float vnew_s[D];
  __shared__ float2 cs[D / 2];
  __shared__ float red_m[4][GP], red_l[4][GP];
  __shared__ float red_o[4][GP][D];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  int split = (int)blockIdx.x % a.nsplit;
  int rest = (int)blockIdx.x / a.nsplit;
  int hg = rest % a.ngh;
  int bg = rest / a.ngh;
  const int Lp = SH ? a.Lp : 0;
  const int Tgen = SH ? a.Tgen : a.Tmax;
  if constexpr (SH) {
    // Shared prompt: workgroup i runs on XCD i % 8. Each XCD takes a
    // contiguous run of the items ordered head-major, (g, b, head group,
    // chunk), so that it reads the prompt rows of at most two or three K/V
    // heads, which then stay in its L2 for all the sequences. The grid is
    // 8 * per_x workgroups, so (i % 8, i / 8) -> lin is one-to-one onto
    // [0, 8 * per_x); those past the nwg items have nothing to do.
    const int per_x = (int)gridDim.x >> 3;
    const int lin = ((int)blockIdx.x & 7) * per_x + ((int)blockIdx.x >> 3);
    if (lin >= a.nwg) return;
    split = lin % a.nsplit;
    const int item = lin / a.nsplit;  // (g * B + b) * ngh + hg
    hg = item % a.ngh;
    const int gb = item / a.ngh;
    bg = (gb % a.B) * a.Hkv + gb / a.B;
  }
  __shared__ int s_len[kDecRankMaxB];  // clamped lengths (ranked placement only)
  if (a.order) {
    // Unsplit ranges (nsplit == 1): workgroup i takes the item of rank i (by
    // the sequence's visible length, longest first, ties by index) while
    // i < ncu, then rank nitems-1-(i-ncu). Workgroups i and i+ncu are placed
    // on the same compute unit, which caps the pair's streaming rate, so the
    // longest ranges share a unit with the shortest and every unit gets a
    // similar number of bytes.
    __shared__ int s_b;
    const int per_b = a.Hkv * a.ngh;
    const int nitems = a.B * per_b;
    const int i = (int)blockIdx.x;
    const int r = i < a.ncu ? i : nitems - 1 - (i - a.ncu);
    const int br = r / per_b;
    for (int t = tid; t < a.B; t += 256) s_len[t] = clamp_len(a.seqlens[t], Lp, a.Tmax);
    __syncthreads();
    for (int t = tid; t < a.B; t += 256) {
      const int lt = min(s_len[t], a.W);  // visible keys
      int rk = 0;
      for (int u = 0; u < a.B; ++u) {
        const int lu = min(s_len[u], a.W);
        rk += (lu > lt || (lu == lt && u < t)) ? 1 : 0;
      }
      if (rk == br) s_b = t;
    }
    __syncthreads();
    const int within = r - br * per_b;
    hg = within % a.ngh;
    bg = s_b * a.Hkv + within / a.ngh;
  }
  const int g = bg % a.Hkv, b = bg / a.Hkv;

  const int h0 = g * a.G + hg * GP;
  const int nh = min(GP, a.G - hg * GP);
  const Elem* qg = (const Elem*)a.q;

  // ---- the rows this wave rotates (q heads, then the appended k row, one
  // ---- wave per row, one (even, odd) pair per lane; D/2 <= 64) and v_new:
  // ---- loaded first, before the sequence length, so that their latency
  // ---- overlaps that load, the K/V loads and the angles (every chunk of the
  // ---- sequence loads the appended row; the one that owns it uses it)
  constexpr int MAXR = (GP + 1 + 3) / 4;  // rows per wave
  float rx[MAXR][2];
  Elem vn0 = Elem(0), vn1 = Elem(0);
#pragma unroll
  for (int j = 0; j < MAXR; ++j) {
    const int r = wave + 4 * j;
    rx[j][0] = rx[j][1] = 0.f;
    if (r <= nh && lane < D / 2) {
      const bool is_k = r == nh;
      const Elem* src = is_k ? (const Elem*)a.k_new + ((size_t)b * a.Hkv + g) * D
                             : qg + ((size_t)b * a.H + h0 + r) * D;
      rx[j][0] = TR::to_f(src[2 * lane]);
      rx[j][1] = TR::to_f(src[2 * lane + 1]);
      if (is_k) {
        const Elem* vsrc = (const Elem*)a.v_new + ((size_t)b * a.Hkv + g) * D;
        vn0 = vsrc[2 * lane];
        vn1 = vsrc[2 * lane + 1];
        if (a.ve_new != nullptr) {  // value embedding: v_new + gate * ve_new, rounded once
          const Elem* esrc = (const Elem*)a.ve_new + ((size_t)b * a.Hkv + g) * D;
          const float gg = TR::to_f(((const Elem*)a.ve_gate)[(size_t)b * a.Hkv + g]);
          vn0 = TR::from_f(TR::to_f(vn0) + gg * TR::to_f(esrc[2 * lane]));
          vn1 = TR::from_f(TR::to_f(vn1) + gg * TR::to_f(esrc[2 * lane + 1]));
        }
      }
    }
  }

  // theta_i = base^(-2i/D) of this lane's pair, formed while the length loads
  const double theta = tid < D / 2 ? exp2(-(double)tid / (D / 2) * a.log2_base) : 0.0;
  const int L = a.order ? s_len[b] : clamp_len(a.seqlens[b], Lp, a.Tmax);
  const int pos = L - 1;
  const int lo = L > a.W ? L - a.W : 0;
  int ks0, ks1;
  const int nch = dec_chunks(L, lo, SH && a.cut ? Lp : 0, SH ? a.Cp : a.C, a.C, split, ks0, ks1);
  if (split >= nch) return;
  const bool owns_new = ks1 == L;
  const int nrows = nh + (owns_new ? 1 : 0);
  const float qscale = kLog2e / sqrtf((float)D);
  // The chunk's keys as one or two segments [sk0, sk1): with a shared prompt
  // and no cut, a chunk spanning the prompt's end runs its prompt rows first,
  // then (second segment) the sequence's own rows, with one softmax state.
  const bool two_seg = SH && ks0 < Lp && ks1 > Lp;
  int sk0 = ks0, sk1 = two_seg ? Lp : ks1;
  bool in_prompt = SH && ks0 < Lp;  // the segment's rows are the shared prompt's

  Elem* kc = (Elem*)a.k_cache;
  Elem* vc = (Elem*)a.v_cache;

  // ---- the chunk's K/V rows as buffer loads relative to key ks0; rows past
  // ---- ks1 (the chunk end) read as zero and are masked out of the softmax.
  // ---- The first iterations' loads are issued before the RoPE prologue so
  // ---- that their latency overlaps it; later ones run NBUF-1 iterations
  // ---- ahead of their use, in NBUF register sets.
  const int cc = lane % CPR;        // 16-byte piece within the row
  const int kl = lane / CPR;        // key slot within the wave
  const uint32_t row_bytes = (uint32_t)a.Hkv * D * sizeof(Elem);
  auto seg_rsrc = [&](const void* kbase, const void* vbase, __amdgpu_buffer_rsrc_t& rk_,
                      __amdgpu_buffer_rsrc_t& rv_) __attribute__((always_inline)) {
    const size_t base_el = in_prompt ? ((size_t)sk0 * a.Hkv + g) * D
                                     : (((size_t)b * Tgen + (sk0 - Lp)) * a.Hkv + g) * D;
    const uint32_t nrec = (uint32_t)(sk1 - sk0) * row_bytes;  // the segment's keys only
    rk_ = make_rsrc((const Elem*)kbase + base_el, nrec);
    rv_ = make_rsrc((const Elem*)vbase + base_el, nrec);
  };
  __amdgpu_buffer_rsrc_t rk, rv;
  seg_rsrc(in_prompt ? a.k_prompt : (const void*)kc, in_prompt ? a.v_prompt : (const void*)vc, rk, rv);
  const int slot = wave * KPW + kl;   // key slot within a workgroup step
  u32x4_t kw[NBUF][U], vw[NBUF][U];
  // the sequence's own rows are read once (non-temporal); the shared prompt's
  // rows are read by every sequence and stay cached
  auto issue = [&](int it, int set) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t off = (uint32_t)(it * KPI + u * 4 * KPW + slot) * row_bytes + cc * 16;
      if (SH && in_prompt) {
        kw[set][u] = bload16(rk, off, 0);
        vw[set][u] = bload16(rv, off, 0);
      } else {
        kw[set][u] = bload16_nt(rk, off, 0);
        vw[set][u] = bload16_nt(rv, off, 0);
      }
    }
  };
  issue(0, 0);
  if constexpr (NBUF == 3) issue(1, 1);  // rows past the chunk read as zero

  // ---- cos/sin at position pos: the angle is formed and reduced modulo
  // ---- 2*pi in fp64, then evaluated in fp32 on [-pi, pi]
  if (tid < D / 2) {
    const double ang = (double)pos * theta;
    const double kq = rint(ang * 0.15915494309189535);
    double r = fma(-kq, 6.283185307179586, ang);
    r = fma(-kq, 2.4492935982947064e-16, r);
    float sn, c;
    sincosf((float)r, &sn, &c);
    cs[tid] = make_float2(c, sn);
  }
  __syncthreads();

  // ---- q' for the nh heads, and the appended row if this chunk owns it
#pragma unroll
  for (int j = 0; j < MAXR; ++j) {
    const int r = wave + 4 * j;
    if (r >= nrows) break;  // uniform across the wave
    const bool is_k = r == nh;
    const int i = lane;  // pair index
    float ye = 0.f, yo = 0.f;
    if (i < D / 2) {
      const float xe = rx[j][0], xo = rx[j][1];
      const float2 c = cs[i];
      ye = xe * c.x - xo * c.y;
      yo = xe * c.y + xo * c.x;
    }
    const float ss = group_sum<64>(ye * ye + yo * yo);
    const float inv = 1.0f / sqrtf(ss * (1.0f / D) + kEps);
    if (i < D / 2) {
      if (is_k) {
        const Elem ke = TR::from_f(ye * inv), ko = TR::from_f(yo * inv);
        knew_s[2 * i] = TR::to_f(ke);
        knew_s[2 * i + 1] = TR::to_f(ko);
        Elem* dst = kc + (((size_t)b * Tgen + (pos - Lp)) * a.Hkv + g) * D;
        dst[2 * i] = ke;
        dst[2 * i + 1] = ko;
        Elem* vdst = vc + (((size_t)b * Tgen + (pos - Lp)) * a.Hkv + g) * D;
        const Elem v0 = vn0, v1 = vn1;
        vdst[2 * i] = v0;
        vdst[2 * i + 1] = v1;
        vnew_s[2 * i] = TR::to_f(v0);
        vnew_s[2 * i + 1] = TR::to_f(v1);
      } else {
        qs[r][2 * i] = ye * inv * qscale;
        qs[r][2 * i + 1] = yo * inv * qscale;
      }
    }
  }
  __syncthreads();

  float qv[GP][EPC];
#pragma unroll
  for (int i = 0; i < GP; ++i)
#pragma unroll
    for (int e = 0; e < EPC; ++e) qv[i][e] = i < nh ? qs[i][cc * EPC + e] : 0.f;

  float m[GP], l[GP], acc[GP][EPC];
#pragma unroll
  for (int i = 0; i < GP; ++i) {
    m[i] = -INFINITY;
    l[i] = 0.f;
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[i][e] = 0.f;
  }

  auto consume = [&](int it, int set) __attribute__((always_inline)) {
    float kx[U][EPC], vx[U][EPC];
    bool live[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int key = sk0 + it * KPI + u * 4 * KPW + slot;
      live[u] = key < sk1;
      if (key == pos) {  // the appended row, from LDS (its cache row may not be written yet)
#pragma unroll
        for (int e = 0; e < EPC; ++e) {
          kx[u][e] = knew_s[cc * EPC + e];
          vx[u][e] = vnew_s[cc * EPC + e];
        }
      } else {
        TR::unpack(kw[set][u], kx[u]);
        TR::unpack(vw[set][u], vx[u]);
      }
    }
#pragma unroll
    for (int i = 0; i < GP; ++i) {
      if (i >= nh) break;
      float sc[U];
      float mx = m[i];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float s = 0.f;
#pragma unroll
        for (int e = 0; e < EPC; ++e) s += qv[i][e] * kx[u][e];
        s = lane_group_sum<CPR>(s);
        sc[u] = live[u] ? s : -INFINITY;
        mx = fmaxf(mx, sc[u]);
      }
      if (mx == -INFINITY) continue;  // no live key for this lane group yet
      const float alpha = merge_scale(m[i], mx);
      float ps = 0.f, pe[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        pe[u] = fast_exp2(sc[u] - mx);  // 2^-inf = 0 for dead slots
        ps += pe[u];
      }
      l[i] = l[i] * alpha + ps;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        float t = acc[i][e] * alpha;
#pragma unroll
        for (int u = 0; u < U; ++u) t += pe[u] * vx[u][e];
        acc[i][e] = t;
      }
      m[i] = mx;
    }
  };

  // bf16 rows: packed math. q' as bf16 pairs (the rounding the prefill MFMAs
  // use too): a key's score is four v_dot2_f32_bf16 per lane on the raw
  // 16-byte piece; the weights of two keys are packed as a bf16 pair, and
  // one v_perm_b32 plus one dot2 per dimension adds both keys' V to the fp32
  // accumulator; the row sum takes the same rounded weights. Half the vector
  // instructions of the widening path, which bounds the loop.
  constexpr bool kPacked = EPC == 8;
  uint32_t qv2[GP][kPacked ? 4 : 1];
  if constexpr (kPacked) {
#pragma unroll
    for (int i = 0; i < GP; ++i)
#pragma unroll
      for (int mm = 0; mm < 4; ++mm) qv2[i][mm] = pack_bf2(qv[i][2 * mm], qv[i][2 * mm + 1]);
  }
  // the iteration that holds key pos (only in the chunk that owns it)
  int it_pos = owns_new && pos < sk1 ? (pos - sk0) / KPI : -1;
  auto consume_packed = [&](int it, int set, auto) __attribute__((always_inline)) {  // generic: only built for bf16
    static_assert(U % 2 == 0, "keys are paired");
    u32x4_t kq[U], vq[U];
    bool live[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      live[u] = sk0 + it * KPI + u * 4 * KPW + slot < sk1;
      kq[u] = kw[set][u];
      vq[u] = vw[set][u];
    }
    if (it == it_pos) {  // the appended row, from LDS (its cache row may not be written yet)
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (sk0 + it * KPI + u * 4 * KPW + slot == pos) {
#pragma unroll
          for (int mm = 0; mm < 4; ++mm) {
            kq[u][mm] = pack_bf2(knew_s[cc * 8 + 2 * mm], knew_s[cc * 8 + 2 * mm + 1]);
            vq[u][mm] = pack_bf2(vnew_s[cc * 8 + 2 * mm], vnew_s[cc * 8 + 2 * mm + 1]);
          }
        }
    }
#pragma unroll
    for (int i = 0; i < GP; ++i) {
      if (i >= nh) break;
      float sc[U];
      float mx = m[i];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        float sd = 0.f;
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) sd = dot2bf(kq[u][mm], qv2[i][mm], sd);
        sd = lane_group_sum<CPR>(sd);
        sc[u] = live[u] ? sd : -INFINITY;
        mx = fmaxf(mx, sc[u]);
      }
      if (mx == -INFINITY) continue;  // no live key for this lane group yet
      const float alpha = merge_scale(m[i], mx);
      uint32_t pp[U / 2];
#pragma unroll
      for (int u2 = 0; u2 < U / 2; ++u2)  // 2^-inf = 0 for dead slots
        pp[u2] = pack_bf2(fast_exp2(sc[2 * u2] - mx), fast_exp2(sc[2 * u2 + 1] - mx));
      float li = l[i] * alpha;
#pragma unroll
      for (int u2 = 0; u2 < U / 2; ++u2) li = dot2bf(pp[u2], 0x3F803F80u, li);  // (1, 1)
      l[i] = li;
#pragma unroll
      for (int e = 0; e < EPC; ++e) acc[i][e] *= alpha;
#pragma unroll
      for (int u2 = 0; u2 < U / 2; ++u2)
#pragma unroll
        for (int mm = 0; mm < 4; ++mm) {
          const uint32_t va = vq[2 * u2][mm], vb = vq[2 * u2 + 1][mm];
          // (key 2u2, key 2u2+1) of dims 2mm and 2mm+1
          const uint32_t lo = __builtin_amdgcn_perm(vb, va, 0x05040100u);
          const uint32_t hi = __builtin_amdgcn_perm(vb, va, 0x07060302u);
          acc[i][2 * mm] = dot2bf(lo, pp[u2], acc[i][2 * mm]);
          acc[i][2 * mm + 1] = dot2bf(hi, pp[u2], acc[i][2 * mm + 1]);
        }
      m[i] = mx;
    }
  };
  auto step = [&](int it, int set) __attribute__((always_inline)) {
    if constexpr (kPacked) consume_packed(it, set, 0); else consume(it, set);
  };

  auto run_segment = [&]() __attribute__((always_inline)) {
  const int niter = (sk1 - sk0 + KPI - 1) / KPI;
  if constexpr (NBUF == 2) {
    for (int it = 0; it < niter; it += 2) {
      if (it + 1 < niter) issue(it + 1, 1);
      step(it, 0);
      if (it + 1 >= niter) break;
      if (it + 2 < niter) issue(it + 2, 0);
      step(it + 1, 1);
    }
  } else {
    for (int it = 0; it < niter; it += 3) {
      if (it + 2 < niter) issue(it + 2, 2);
      step(it, 0);
      if (it + 1 >= niter) break;
      if (it + 3 < niter) issue(it + 3, 0);
      step(it + 1, 1);
      if (it + 2 >= niter) break;
      if (it + 4 < niter) issue(it + 4, 1);
      step(it + 2, 2);
    }
  }
  };
  run_segment();
  if constexpr (SH) {
    if (two_seg) {  // the sequence's own rows: a fresh pipeline on their cache
      sk0 = Lp;
      sk1 = ks1;
      in_prompt = false;
      seg_rsrc(kc, vc, rk, rv);
      it_pos = owns_new ? (pos - sk0) / KPI : -1;
      issue(0, 0);
      if constexpr (NBUF == 3) issue(1, 1);
      run_segment();
    }
  }

  // ---- merge the key slots of a wave (lanes kl differ by multiples of CPR)
#pragma unroll
  for (int off = CPR; off < 64; off <<= 1) {
#pragma unroll
    for (int i = 0; i < GP; ++i) {
      const float mo = __shfl_xor(m[i], off, 64);
      const float lo_ = __shfl_xor(l[i], off, 64);
      const float mn = fmaxf(m[i], mo);
      const float a0 = merge_scale(m[i], mn), a1 = merge_scale(mo, mn);
      l[i] = l[i] * a0 + lo_ * a1;
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const float ao = __shfl_xor(acc[i][e], off, 64);
        acc[i][e] = acc[i][e] * a0 + ao * a1;
      }
      m[i] = mn;
    }
  }
  if (kl == 0) {
#pragma unroll
    for (int i = 0; i < GP; ++i) {
      if (cc == 0) {
        red_m[wave][i] = m[i];
        red_l[wave][i] = l[i];
      }
#pragma unroll
      for (int e = 0; e < EPC; ++e) red_o[wave][i][cc * EPC + e] = acc[i][e];
    }
  }
  __syncthreads();

  // ---- merge the 4 waves; write the output, or this chunk's state
  const bool single = nch == 1;
  for (int idx = tid; idx < nh * D; idx += 256) {
    const int i = idx / D, d = idx - (idx / D) * D;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w) mx = fmaxf(mx, red_m[w][i]);
    float lsum = 0.f, osum = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = merge_scale(red_m[w][i], mx);
      lsum += red_l[w][i] * sc;
      osum += red_o[w][i][d] * sc;
    }
    const int h = h0 + i;
    if (single) {
      ((Elem*)a.o)[((size_t)b * a.H + h) * D + d] = TR::from_f(osum / lsum);
    } else {
      float* pp = a.part + (((size_t)b * a.H + h) * a.nsplit + split) * (D + 2);
      pp[d] = osum;
      if (d == 0) {
        pp[D] = mx;
        pp[D + 1] = lsum;
      }
    }
  }
}

// One wave per (b, h) whose visible range spans more than one chunk: merge
// the chunk states in one pass (running maximum), lanes over the head dim.
template <int D, typename Elem>
__global__ void __launch_bounds__(256) attn_decode_combine_kernel(DecArgs a) {
  const int wid = ((int)blockIdx.x * 256 + (int)threadIdx.x) >> 6;
  const int lane = threadIdx.x & 63;
  if (wid >= a.B * a.H) return;
  const int b = wid / a.H, h = wid - (wid / a.H) * a.H;
  const int L = clamp_len(a.seqlens[b], a.Lp, a.Tmax);
  const int lo = L > a.W ? L - a.W : 0;
  int ks0, ks1;
  const int nch = dec_chunks(L, lo, a.cut ? a.Lp : 0, a.cut ? a.Cp : a.C, a.C, 0, ks0, ks1);
  if (nch <= 1) return;
  constexpr int PER = (D + 63) / 64;
  constexpr int NB = 8;  // chunk states loaded per batch
  const float* pp = a.part + ((size_t)b * a.H + h) * a.nsplit * (D + 2);
  float mx = -INFINITY, lsum = 0.f, o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
  for (int s0 = 0; s0 < nch; s0 += NB) {
    float ms[NB], ls[NB], os[NB][PER];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const bool ok = s0 + j < nch;
      const float* ps = pp + (ok ? s0 + j : 0) * (D + 2);
      ms[j] = ok ? ps[D] : -INFINITY;
      ls[j] = ok ? ps[D + 1] : 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int d = e * 64 + lane;
        os[j][e] = (ok && d < D) ? ps[d] : 0.f;
      }
    }
    float mn = mx;
#pragma unroll
    for (int j = 0; j < NB; ++j) mn = fmaxf(mn, ms[j]);
    const float a0 = merge_scale(mx, mn);
    lsum *= a0;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] *= a0;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float aj = merge_scale(ms[j], mn);
      lsum += ls[j] * aj;
#pragma unroll
      for (int e = 0; e < PER; ++e) o[e] += os[j][e] * aj;
    }
    mx = mn;
  }
  const float inv = 1.0f / lsum;
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int d = e * 64 + lane;
    if (d < D) ((Elem*)a.o)[((size_t)b * a.H + h) * D + d] = ElemTraits<Elem>::from_f(o[e] * inv);
  }
}

// ---------------------------------------------------------------- host side
static int decode_gp(int G) { return G <= 1 ? 1 : (G <= 2 ? 2 : (G <= 4 ? 4 : 8)); }

static int decode_kpi(int D, bool bf16) {
  const int cpr = D / (bf16 ? 8 : 4);
  return 4 * (64 / cpr) * kDecU;  // waves * keys per wave step * keys per lane group
}

static int decode_chunk(int B, int Tmax, int H, int Hkv, int D, int W) {
  // Each workgroup pays a fixed start-up (RoPE of q, first load latency) and
  // a split range pays a merge pass, so a visible range is split only when
  // there are fewer (b, K/V head, head group) workgroups than compute units;
  // then chunks are sized for about 1024 workgroups, at least two workgroup
  // iterations each so that the loads run ahead of their use.
  const int G = H / Hkv;
  const int ngh = (G + decode_gp(G) - 1) / decode_gp(G);
  const int kpi = decode_kpi(D, true);
  const long long span = (long long)(W < Tmax ? W : Tmax);
  const long long whole = (span + kpi - 1) / kpi * kpi;
  const long long nbg = (long long)B * Hkv * ngh;
  if (nbg >= 256) return (int)whole;
  long long c = 2 * kpi;
  while (c < whole && nbg * ((span + c - 1) / c) > 1024) c <<= 1;
  return (int)(c < whole ? c : whole);
}

// Compute units of the current device, queried once per device.
static int device_cu_count() {
  static int cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cached[dev] = n;
  }
  return cached[dev];
}

static int decode_nsplit(int Tmax, int W, int C) {
  const int span = W < Tmax ? W : Tmax;
  return (span + C - 1) / C;
}

// A cut prompt part is run in this many chunks, next to the sequence's own
// chunks (measured, 64 samples of a 1536-token d12 prompt at W = 2048:
// 38.2 us in one chunk, 35.7 in two, 37.2 in three, 39.6 in four).
constexpr int kDecCutPromptChunks = 2;

// A shared prompt adds at most kDecCutPromptChunks chunks (its cut part).
size_t decode_workspace_bytes(int B, int Tmax, int H, int Hkv, int D, int window, int Lp) {
  const int C = decode_chunk(B, Tmax, H, Hkv, D, window);
  const int ns = decode_nsplit(Tmax, window, C) + (Lp > 0 ? kDecCutPromptChunks : 0);
  if (ns <= 1) return 0;
  return (size_t)B * H * ns * (D + 2) * sizeof(float);
}

template <int D, int GP, typename Elem>
static void launch_decode_gp(bool sh, long long grid, const DecArgs& a, hipStream_t stream) {
  if (sh)
    hipLaunchKernelGGL((attn_decode_kernel<D, GP, Elem, true>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_decode_kernel<D, GP, Elem, false>), dim3((unsigned)grid), dim3(256), 0, stream, a);
}

template <int D, typename Elem>
static hipError_t decode_d(DecArgs a, hipStream_t stream) {
  const int GP = decode_gp(a.G);
  a.ngh = (a.G + GP - 1) / GP;
  a.nwg = (int)std::min<long long>((long long)a.B * a.Hkv * a.ngh * a.nsplit, 0x7fffffffLL);
  const long long grid = a.Lp > 0 ? ((long long)a.B * a.Hkv * a.ngh * a.nsplit + 7) / 8 * 8
                                  : (long long)a.B * a.Hkv * a.ngh * a.nsplit;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const bool sh = a.Lp > 0;
  switch (GP) {
    case 1: launch_decode_gp<D, 1, Elem>(sh, grid, a, stream); break;
    case 2: launch_decode_gp<D, 2, Elem>(sh, grid, a, stream); break;
    case 4: launch_decode_gp<D, 4, Elem>(sh, grid, a, stream); break;
    default: launch_decode_gp<D, 8, Elem>(sh, grid, a, stream); break;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.nsplit <= 1) return e;
  const long long waves = (long long)a.B * a.H;
  hipLaunchKernelGGL((attn_decode_combine_kernel<D, Elem>), dim3((unsigned)((waves + 3) / 4)),
                     dim3(256), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_attn_decode_shared(const void* q, const void* k_new, const void* v_new,
                                     const void* k_prompt, const void* v_prompt, int Lp,
                                     void* k_cache, void* v_cache, const int32_t* seqlens, void* o,
                                     int B, int Tgen, int H, int Hkv, int D, int window,
                                     double rope_base, Dtype dt, void* ws, hipStream_t stream,
                                     const void* ve_new, const void* ve_gate) {
  DecArgs a{};
  a.ve_new = ve_new;
  a.ve_gate = ve_gate;
  const int Tmax = Lp + Tgen;
  a.q = q;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_prompt = k_prompt;
  a.v_prompt = v_prompt;
  a.Lp = Lp;
  a.Tgen = Tgen;
  a.seqlens = seqlens;
  a.o = o;
  a.B = B;
  a.Tmax = Tmax;
  a.H = H;
  a.Hkv = Hkv;
  a.G = H / Hkv;
  a.W = window;
  a.C = decode_chunk(B, Tmax, H, Hkv, D, window);
  // Cut at the prompt's end where a sequence can see 1024 or more prompt rows:
  // the prompt part then runs in parallel with the own part (measured, 64
  // samples of a 1536-token prompt at W = 2048: 37.9 us cut). Shorter prompt
  // parts run as the first segment of the same workgroup, with no merge pass.
  a.cut = (Lp > 0 && std::min(window, Lp) >= 1024) ? 1 : 0;
  a.Cp = a.C;
  int npc = 0;  // chunks of a cut prompt part
  if (a.cut) {
    npc = kDecCutPromptChunks;
    const int kpi = decode_kpi(D, dt == kBF16);
    const int span_p = std::min(window, Lp);
    a.Cp = std::max(kpi, ((span_p + npc - 1) / npc + kpi - 1) / kpi * kpi);
    npc = (span_p + a.Cp - 1) / a.Cp;
  }
  a.nsplit = decode_nsplit(Tmax, window, a.C) + (a.cut ? npc : 0);
  a.log2_base = std::log2(rope_base);
  a.part = (float*)ws;
  a.ncu = device_cu_count();
  // Ranking costs each workgroup one more dependent round trip; it pays where
  // visible lengths can differ by more than a few hundred keys.
  const int span = window < Tmax ? window : Tmax;
  // (not with a shared prompt, whose workgroups take their items head-major per XCD)
  a.order = (Lp == 0 && a.nsplit == 1 && B <= kDecRankMaxB && a.ncu > 0 && span >= 1024) ? 1 : 0;
  const bool bf = dt == kBF16;
  switch (D) {
    case 32: return bf ? decode_d<32, uint16_t>(a, stream) : decode_d<32, float>(a, stream);
    case 64: return bf ? decode_d<64, uint16_t>(a, stream) : decode_d<64, float>(a, stream);
    case 128: return bf ? decode_d<128, uint16_t>(a, stream) : decode_d<128, float>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn_decode(const void* q, const void* k_new, const void* v_new, void* k_cache,
                              void* v_cache, const int32_t* seqlens, void* o, int B, int Tmax,
                              int H, int Hkv, int D, int window, double rope_base, Dtype dt,
                              void* ws, hipStream_t stream, const void* ve_new,
                              const void* ve_gate) {
  return launch_attn_decode_shared(q, k_new, v_new, nullptr, nullptr, 0, k_cache, v_cache, seqlens,
                                   o, B, Tmax, H, Hkv, D, window, rope_base, dt, ws, stream, ve_new,
                                   ve_gate);
}

}  // namespace nc
